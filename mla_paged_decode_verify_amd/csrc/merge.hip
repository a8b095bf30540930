// Segment merge and shard (LSE) merge.
//
// Segment merge: vLLM PR #51705 digest (prhub), Implementation breakdown item 4
// and the merge_mla_segments_triton snippet -- base-2 per-segment max / exp2
// sum / unnormalised output are folded into one output and a natural-log LSE
// (ln 2 * (max + log2 sum)); which segments are active is derived from each
// row's real length and the same tiles_per_segment partition the attention
// kernel used. Shard merge: same digest, Motivation (rank-local partials go
// through the DCP attention merge) and SGLang PR #34432 report, review item 4
// (natural-log LSE, so the combine uses exp/log).
//
// One wave per (row, head) pair. The wave first works on the per-segment
// statistics with one lane per (shard, segment) -- per-shard maxima, sums and
// LSEs, the weight of every segment inside its shard and of every shard in the
// result -- through a small LDS area; then each lane owns 8 consecutive latent
// dims and streams the partial outputs, all shards' loads in flight at once.
// Every per-shard output is rounded to bf16 first, as it would be when a shard
// sends it to the others. Pairs whose W * (nseg + 2) values do not fit the LDS
// area take a sequential path over shards.
#include "internal.h"

namespace mla {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309f;
constexpr int kMergeWaves = 4;
constexpr int kStatSlots = 1024;            // floats of LDS per wave

// Request owning row rho: the largest i with q_start[i] <= rho, by a 64-way
// search (each round, every lane tests one candidate boundary).
__device__ inline int find_request(const int32_t* q_start, int N, int rho, int lane) {
  int lo = 0, n = N;                        // answer in [lo, lo + n)
  while (n > 1) {
    const int step = (n + 63) / 64;
    const int cand = lo + lane * step;
    const bool le = cand < lo + n && q_start[cand] <= rho;
    const int cnt = __builtin_popcountll(__builtin_amdgcn_ballot_w64(le));
    if (cnt == 0) return lo;                // malformed q_start; caught below
    lo += (cnt - 1) * step;
    n = min(step, N - lo);
  }
  return lo;
}

__device__ inline float bf16_round(float x) { return (float)(__bf16)x; }

__device__ inline uint32_t pack2_bf16(float a, float b) {
  __bf16 x = (__bf16)a, y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) |
         ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

__device__ inline float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Number of segments of shard r that hold tokens of row rho: the attention
// kernel splits the group's longest row Lg into segments of `span` tokens.
__device__ inline int active_segments(const MergeArgs& a, int r, int rho, int last) {
  const int seg_tokens = a.nseg * a.page_size;
  const int Lg = a.row_lens[(int64_t)r * a.R + last];
  const int L = a.row_lens[(int64_t)r * a.R + rho];
  const int span = (Lg + seg_tokens - 1) / seg_tokens * a.page_size;
  const int nact = span > 0 ? (L + span - 1) / span : 0;
  return min(nact, a.nseg);
}

__device__ inline void store_out(const MergeArgs& a, int64_t pair, int lane, const float (&v)[8],
                                 float lse) {
  const uint4 w = make_uint4(pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3]),
                             pack2_bf16(v[4], v[5]), pack2_bf16(v[6], v[7]));
  *reinterpret_cast<uint4*>(a.out + pair * kVDim + 8 * lane) = w;
  if (lane == 0) a.lse[pair] = lse;
}

__device__ inline void store_shard(const MergeArgs& a, int r, int rho, int h, int lane,
                                   const float (&o)[8], float lse_r) {
  const int64_t e = ((int64_t)r * a.R + rho) * a.H + h;
  if (a.shard_out != nullptr) {
    const uint4 w = make_uint4(pack2_bf16(o[0], o[1]), pack2_bf16(o[2], o[3]),
                               pack2_bf16(o[4], o[5]), pack2_bf16(o[6], o[7]));
    *reinterpret_cast<uint4*>(a.shard_out + e * kVDim + 8 * lane) = w;
  }
  if (a.shard_lse != nullptr && lane == 0) a.shard_lse[e] = lse_r;
}

// Accumulate 8 dims of one partial output with weight c.
__device__ inline void axpy8(float (&acc)[8], float c, const float* src) {
  const float4 x = reinterpret_cast<const float4*>(src)[0];
  const float4 y = reinterpret_cast<const float4*>(src)[1];
  acc[0] += c * x.x; acc[1] += c * x.y; acc[2] += c * x.z; acc[3] += c * x.w;
  acc[4] += c * y.x; acc[5] += c * y.y; acc[6] += c * y.z; acc[7] += c * y.w;
}

__global__ void __launch_bounds__(64 * kMergeWaves) merge_kernel(MergeArgs a) {
  __shared__ float stat[kMergeWaves][kStatSlots];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t pair = (int64_t)blockIdx.x * kMergeWaves + wave;
  if (pair >= (int64_t)a.R * a.H) return;
  const int rho = (int)(pair / a.H);
  const int h = (int)(pair % a.H);
  const int i = find_request(a.q_start, a.N, rho, lane);
  const int last = a.q_start[i + 1] - 1;
  if (a.q_start[i] > rho || last < rho || last >= a.R) return;  // malformed q_start
  const int W = a.W, nseg = a.nseg;
  float* sl = stat[wave];                   // [W] shard LSEs
  float* sw = sl + W;                       // [W] shard weights
  float* sc = sw + W;                       // [W * nseg] segment weights inside a shard
  const bool fast = W * (nseg + 2) <= kStatSlots;

  float res[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) res[k] = 0.f;
  float lse_out = kNegInf;

  if (fast) {
    // ---- per shard (one lane each): maximum, sum, LSE and segment weights
    float gm = kNegInf;                     // largest LSE of this lane's shards
    for (int r = lane; r < W; r += 64) {
      const int nact = active_segments(a, r, rho, last);
      const int64_t base = (((int64_t)r * a.R + rho) * a.H + h) * nseg;
      float M = kNegInf;
      for (int s = 0; s < nact; ++s) M = fmaxf(M, a.segm_max[base + s]);
      float E = 0.f;
      for (int s = 0; s < nact; ++s) {
        const float sc_s = __builtin_amdgcn_exp2f(a.segm_max[base + s] - M);
        sc[r * nseg + s] = sc_s;
        E += a.segm_expsum[base + s] * sc_s;
      }
      for (int s = nact; s < nseg; ++s) sc[r * nseg + s] = 0.f;
      float l = kNegInf;
      if (M != kNegInf && E > 0.f) {
        const float inv = 1.f / E;
        for (int s = 0; s < nact; ++s) sc[r * nseg + s] *= inv;
        l = kLn2 * (M + __log2f(E));
      } else {
        for (int s = 0; s < nact; ++s) sc[r * nseg + s] = 0.f;
      }
      gm = fmaxf(gm, l);
      sl[r] = l;
    }
    // ---- shard weights: exp(lse_r - G) / sum, G the largest LSE
    const float G = wave_max(gm);
    if (G != kNegInf) {
      float part = 0.f;
      for (int r = lane; r < W; r += 64) {
        const float wr = sl[r] == kNegInf ? 0.f : __expf(sl[r] - G);
        sw[r] = wr;
        part += wr;
      }
      const float total = wave_sum(part);
      lse_out = G + __logf(total);
      const float inv = 1.f / total;
      for (int r = lane; r < W; r += 64) sw[r] *= inv;
    } else {
      for (int r = lane; r < W; r += 64) sw[r] = 0.f;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- outputs: each lane's 8 dims, shard by shard (bf16 per shard); the
    // unrolled loop keeps several shards' loads in flight
#pragma unroll 8
    for (int r = 0; r < W; ++r) {
      const int64_t base = (((int64_t)r * a.R + rho) * a.H + h) * nseg;
      float o[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] = 0.f;
      const float* src = a.segm_out + base * kVDim + 8 * lane;
#pragma unroll 4
      for (int s = 0; s < nseg; ++s) {
        const float c = sc[r * nseg + s];   // 0 for segments without tokens
        if (c != 0.f) axpy8(o, c, src + (int64_t)s * kVDim);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] = bf16_round(o[k]);
      const float wr = sw[r];
#pragma unroll
      for (int k = 0; k < 8; ++k) res[k] += wr * o[k];
      if (a.shard_out != nullptr || a.shard_lse != nullptr) store_shard(a, r, rho, h, lane, o, sl[r]);
    }
    store_out(a, pair, lane, res, lse_out);
    return;
  }

  // ---- sequential path: shards folded in online
  float gmax = kNegInf, gsum = 0.f;
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.f;
  for (int r = 0; r < W; ++r) {
    const int nact = active_segments(a, r, rho, last);
    const int64_t base = (((int64_t)r * a.R + rho) * a.H + h) * nseg;
    float M = kNegInf;
    for (int s = 0; s < nact; ++s) M = fmaxf(M, a.segm_max[base + s]);
    float o[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] = 0.f;
    float lse_r = kNegInf;
    if (M != kNegInf) {
      float E = 0.f;
      for (int s = 0; s < nact; ++s) {
        const float c = __builtin_amdgcn_exp2f(a.segm_max[base + s] - M);
        E += a.segm_expsum[base + s] * c;
        axpy8(o, c, a.segm_out + (base + s) * kVDim + 8 * lane);
      }
      const float inv = 1.f / E;
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] = bf16_round(o[k] * inv);
      lse_r = kLn2 * (M + __log2f(E));
    }
    store_shard(a, r, rho, h, lane, o, lse_r);
    if (lse_r == kNegInf) continue;          // empty shard contributes nothing
    if (lse_r > gmax) {
      const float f = __expf(gmax - lse_r);  // gmax = -inf gives 0
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] *= f;
      gsum *= f;
      gmax = lse_r;
    }
    const float wgt = __expf(lse_r - gmax);
    gsum += wgt;
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] += wgt * o[k];
  }
  if (gmax != kNegInf) {
    const float inv = 1.f / gsum;
#pragma unroll
    for (int k = 0; k < 8; ++k) res[k] = acc[k] * inv;
    lse_out = gmax + __logf(gsum);
  }
  store_out(a, pair, lane, res, lse_out);
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  const int64_t pairs = (int64_t)a.R * a.H;
  if (pairs <= 0) return hipSuccess;
  merge_kernel<<<(unsigned)((pairs + kMergeWaves - 1) / kMergeWaves), 64 * kMergeWaves, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
