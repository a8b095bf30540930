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
// One wave per (row, head) pair, in three rounds of global loads: (1) every
// segment's maximum and sum, this row's length per shard, and the search for
// the row's request; (2) the length of the request's last row per shard,
// which fixes the segment partition; (3) the partial outputs, each lane owning
// 8 consecutive latent dims, several segments in flight at once. Statistics go
// through a small LDS area: per-shard maxima, sums and LSEs, the weight of
// every segment inside its shard and of every shard in the result. All shards
// live on this device, so the per-shard outputs stay in fp32 between the two
// merges; only the optional shard_out copy is rounded to bf16. Pairs whose
// 2 W (nseg + 1) values do not fit the LDS area take a sequential path over
// shards.
#include "internal.h"

namespace mla {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309f;
constexpr int kMergeWaves = 4;
constexpr int kStatSlots = 1024;            // floats of LDS per wave

// Request owning row rho and its last row: i with q_start[i] <= rho <
// q_start[i + 1]. Coarse rounds narrow the range 64 candidates at a time; in
// the final round lanes 0..n hold q_start[lo .. lo + n], so q_start[i + 1]
// comes from a lane instead of another load. Returns -1 for a malformed
// q_start.
__device__ inline int find_request(const int32_t* q_start, int N, int rho, int lane, int& last) {
  int lo = 0, n = N;                        // answer in [lo, lo + n)
  while (n > 63) {
    const int step = (n + 63) / 64;
    const int cand = lo + lane * step;
    const bool le = cand < lo + n && q_start[cand] <= rho;
    const int cnt = __builtin_popcountll(__builtin_amdgcn_ballot_w64(le));
    if (cnt == 0) return -1;
    lo += (cnt - 1) * step;
    n = min(step, N - lo);
  }
  const int qv = lane <= n ? q_start[lo + lane] : 0x7FFFFFFF;
  const int cnt = __builtin_popcountll(__builtin_amdgcn_ballot_w64(qv <= rho));
  if (cnt == 0 || cnt > n) return -1;
  const int first = __builtin_amdgcn_readlane(qv, cnt - 1);
  const int next = __builtin_amdgcn_readlane(qv, cnt);
  if (first > rho || next <= rho) return -1;  // not non-decreasing
  last = next - 1;
  return lo + cnt - 1;
}

__device__ inline uint32_t pack2_bf16(float a, float b) {
  __bf16 x = (__bf16)a, y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) |
         ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// Maximum that keeps a NaN (fmaxf drops it): partials of rows the attention
// grid did not cover are NaN, and must reach out and lse as NaN.
__device__ inline float max_keep_nan(float m, float x) {
  return (m != m || x != x) ? __builtin_nanf("") : fmaxf(m, x);
}

__device__ inline float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = max_keep_nan(x, __shfl_xor(x, o));
  return x;
}
__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Segments of a row of length L that hold tokens, in a group whose last row
// has length Lg: the attention kernel cut the group into segments of `span`
// tokens and wrote the partials of every segment that starts before Lg, for
// every row of the group. A row is never read past Lg (a well-formed plan has
// L <= Lg, the last row being the longest), so exactly the segments the
// attention wrote are read, whatever the row lengths hold.
__device__ inline int active_segments(int Lg, int L, int nseg, int page_size) {
  const int seg_tokens = nseg * page_size;
  const int span = (int)(((int64_t)Lg + seg_tokens - 1) / seg_tokens * page_size);
  const int nact = span > 0 ? (min(L, Lg) + span - 1) / span : 0;
  return min(nact, nseg);
}

__device__ inline void store_out8(uint16_t* out, float* lse, int64_t pair, int lane,
                                  const float (&v)[8], float l) {
  const uint4 w = make_uint4(pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3]),
                             pack2_bf16(v[4], v[5]), pack2_bf16(v[6], v[7]));
  *reinterpret_cast<uint4*>(out + pair * kVDim + 8 * lane) = w;
  if (lane == 0) lse[pair] = l;
}
__device__ inline void store_out(const MergeArgs& a, int64_t pair, int lane, const float (&v)[8],
                                 float lse) {
  store_out8(a.out, a.lse, pair, lane, v, lse);
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

// o += c * (8 dims of one partial output); c == 0 marks a segment without
// tokens, whose memory may never have been written, so its values are
// discarded rather than multiplied.
__device__ inline void axpy8(float (&o)[8], float c, const float* src) {
  const float4 x = reinterpret_cast<const float4*>(src)[0];
  const float4 y = reinterpret_cast<const float4*>(src)[1];
  const bool on = c != 0.f;
  o[0] += on ? c * x.x : 0.f; o[1] += on ? c * x.y : 0.f;
  o[2] += on ? c * x.z : 0.f; o[3] += on ? c * x.w : 0.f;
  o[4] += on ? c * y.x : 0.f; o[5] += on ? c * y.y : 0.f;
  o[6] += on ? c * y.z : 0.f; o[7] += on ? c * y.w : 0.f;
}

__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__global__ void __launch_bounds__(64 * kMergeWaves) merge_kernel(MergeArgs a) {
  __shared__ float stat[kMergeWaves][kStatSlots];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t pair = (int64_t)blockIdx.x * kMergeWaves + wave;
  if (pair >= (int64_t)a.R * a.H) return;
  const int rho = (int)(pair / a.H);
  const int h = (int)(pair % a.H);
  const int W = a.W, nseg = a.nseg, F = W * nseg;
  // partial index e = r * rstride + pbase + s
  const int64_t rstride = (int64_t)a.R * a.H * nseg;
  const int64_t pbase = ((int64_t)rho * a.H + h) * nseg;

  float res[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) res[k] = 0.f;
  float lse_out = kNegInf;

  if (2 * (F + W) <= kStatSlots) {
    float* sm = stat[wave];                 // [F] segment maxima
    float* sc = sm + F;                     // [F] segment sums, then segment weights
    float* sl = sc + F;                     // [W] shard LSEs
    float* sw = sl + W;                     // [W] shard weights
    // ---- first round of loads: all that does not depend on the request
    // (every segment's statistics, whether it holds tokens or not; this row's
    // length in the first 64 shards), in flight together with the search
    for (int f = lane; f < F; f += 64) {
      const int r = f / nseg, s = f - r * nseg;
      sm[f] = a.segm_max[r * rstride + pbase + s];
      sc[f] = a.segm_expsum[r * rstride + pbase + s];
    }
    const int L0 = lane < W ? a.row_lens[(int64_t)lane * a.R + rho] : 0;
    int last = 0;
    if (find_request(a.q_start, a.N, rho, lane, last) < 0 || last >= a.R) return;  // malformed
    wave_lds_sync();

    // ---- per shard (one lane each): active segments (second round: the
    // group's longest row), maximum, sum, LSE and segment weights
    float gm = kNegInf;                     // largest LSE of this lane's shards
    for (int r = lane; r < W; r += 64) {
      const int L = r < 64 ? L0 : a.row_lens[(int64_t)r * a.R + rho];
      const int Lg = a.row_lens[(int64_t)r * a.R + last];
      const int nact = active_segments(Lg, L, nseg, a.page_size);
      float* m = sm + r * nseg;
      float* c = sc + r * nseg;
      float M = kNegInf;
      for (int s = 0; s < nact; ++s) M = max_keep_nan(M, m[s]);
      float E = 0.f;
      if (M != kNegInf)
        for (int s = 0; s < nact; ++s) E += c[s] * __builtin_amdgcn_exp2f(m[s] - M);
      const bool live = M != kNegInf && !(E <= 0.f);   // NaN stays NaN
      const float inv = live ? 1.f / E : 0.f;
      for (int s = 0; s < nseg; ++s)
        c[s] = live && s < nact ? __builtin_amdgcn_exp2f(m[s] - M) * inv : 0.f;
      const float l = live ? kLn2 * (M + __log2f(E)) : kNegInf;
      gm = max_keep_nan(gm, l);
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
    wave_lds_sync();

    // ---- outputs (third round): each lane's 8 dims, shard by shard (fp32
    // per shard); loads are unconditional so that unrolled iterations keep
    // several segments in flight
    const float* src = a.segm_out + pbase * kVDim + 8 * lane;
    const bool want_shard = a.shard_out != nullptr || a.shard_lse != nullptr;
    auto finish_shard = [&](int r, float (&o)[8]) {
      const float wr = sw[r];
#pragma unroll
      for (int k = 0; k < 8; ++k) res[k] += wr * o[k];
      if (want_shard) store_shard(a, r, rho, h, lane, o, sl[r]);
    };
    if (nseg == 1) {
#pragma unroll 4
      for (int r = 0; r < W; ++r) {
        float o[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] = 0.f;
        axpy8(o, sc[r], src + r * rstride * kVDim);
        finish_shard(r, o);
      }
    } else {
      for (int r = 0; r < W; ++r) {
        float o[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] = 0.f;
#pragma unroll 4
        for (int s = 0; s < nseg; ++s) axpy8(o, sc[r * nseg + s], src + (r * rstride + s) * kVDim);
        finish_shard(r, o);
      }
    }
    store_out(a, pair, lane, res, lse_out);
    return;
  }

  // ---- sequential path: shards folded in online
  int last = 0;
  if (find_request(a.q_start, a.N, rho, lane, last) < 0 || last >= a.R) return;  // malformed
  float gmax = kNegInf, gsum = 0.f;
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.f;
  for (int r = 0; r < W; ++r) {
    const int nact = active_segments(a.row_lens[(int64_t)r * a.R + last],
                                     a.row_lens[(int64_t)r * a.R + rho], nseg, a.page_size);
    const int64_t base = r * rstride + pbase;
    float M = kNegInf;
    for (int s = 0; s < nact; ++s) M = max_keep_nan(M, a.segm_max[base + s]);
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
      if (!(E <= 0.f)) {                   // NaN stays NaN
        const float inv = 1.f / E;
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] *= inv;
        lse_r = kLn2 * (M + __log2f(E));
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] = 0.f;
      }
    }
    store_shard(a, r, rho, h, lane, o, lse_r);
    if (lse_r == kNegInf) continue;          // empty shard contributes nothing
    if (lse_r != lse_r) gmax = lse_r;         // NaN (an uncovered row) stays NaN
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

// Shard merge alone, from per-source bf16 outputs and natural-log LSEs (a
// source is a shard, or one (shard, segment) unit of the normalised form):
// one wave per (row, head) pair, each lane owning 8 latent dims. The weights are
// formed exactly as in merge_kernel (largest LSE G, exp(lse_r - G), wave sum,
// normalised), and the outputs are accumulated shard by shard in order, so
// both kernels give the same bits for the same per-shard results.
__global__ void __launch_bounds__(64 * kMergeWaves) shard_merge_kernel(ShardMergeArgs a) {
  __shared__ float wsh[kMergeWaves][kShardMergeMaxW];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t pair = (int64_t)blockIdx.x * kMergeWaves + wave;
  if (pair >= (int64_t)a.R * a.H) return;
  const int W = a.W;
  const int64_t rs = (int64_t)a.R * a.H;    // shard stride, in pairs
  const uint16_t* src = a.shard_out + pair * kVDim + 8 * lane;
  float res[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) res[k] = 0.f;

  if (W <= 8) {
    // Up to 8 shards: every load goes out at once, and each lane forms all the
    // weights itself. The sum of the weights follows the butterfly order of
    // wave_sum over lanes 0..W-1 (zeros elsewhere), so the bits are those of
    // the general path.
    float l[8];
    uint4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) l[j] = j < W ? a.shard_lse[j * rs + pair] : kNegInf;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < W) v[j] = *reinterpret_cast<const uint4*>(src + j * rs * kVDim);
    float G = kNegInf;
#pragma unroll
    for (int j = 0; j < 8; ++j) G = max_keep_nan(G, l[j]);
    float lse_out = kNegInf;
    float w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = 0.f;
    if (G != kNegInf) {
#pragma unroll
      for (int j = 0; j < 8; ++j) w[j] = l[j] == kNegInf ? 0.f : __expf(l[j] - G);
      const float total = ((w[0] + w[4]) + (w[2] + w[6])) + ((w[1] + w[5]) + (w[3] + w[7]));
      lse_out = G + __logf(total);
      const float inv = 1.f / total;
#pragma unroll
      for (int j = 0; j < 8; ++j) w[j] *= inv;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j >= W) break;
      const uint32_t u32[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        res[2 * k] += w[j] * __uint_as_float(u32[k] << 16);
        res[2 * k + 1] += w[j] * __uint_as_float(u32[k] & 0xFFFF0000u);
      }
    }
    store_out8(a.out, a.lse, pair, lane, res, lse_out);
    return;
  }

  float* sw = wsh[wave];

  float gm = kNegInf;
  for (int r = lane; r < W; r += 64) {
    const float l = a.shard_lse[r * rs + pair];
    sw[r] = l;
    gm = max_keep_nan(gm, l);
  }
  const float G = wave_max(gm);
  float lse_out = kNegInf;
  if (G != kNegInf) {
    float part = 0.f;
    for (int r = lane; r < W; r += 64) {
      const float wr = sw[r] == kNegInf ? 0.f : __expf(sw[r] - G);
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
  wave_lds_sync();

  for (int r0 = 0; r0 < W; r0 += 8) {
    // sources without weight (lse -inf: no token of the row) are not read
    uint4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      v[j] = (r0 + j < W && sw[r0 + j] != 0.f)
                 ? *reinterpret_cast<const uint4*>(src + (r0 + j) * rs * kVDim)
                 : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (r0 + j >= W) break;
      const float wr = sw[r0 + j];
      const uint32_t u32[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        res[2 * k] += wr * __uint_as_float(u32[k] << 16);
        res[2 * k + 1] += wr * __uint_as_float(u32[k] & 0xFFFF0000u);
      }
    }
  }
  store_out8(a.out, a.lse, pair, lane, res, lse_out);
}

}  // namespace

hipError_t launch_shard_merge(const ShardMergeArgs& a, hipStream_t s) {
  const int64_t pairs = (int64_t)a.R * a.H;
  if (pairs <= 0) return hipSuccess;
  shard_merge_kernel<<<(unsigned)((pairs + kMergeWaves - 1) / kMergeWaves), 64 * kMergeWaves, 0,
                       s>>>(a);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  const int64_t pairs = (int64_t)a.R * a.H;
  if (pairs <= 0) return hipSuccess;
  merge_kernel<<<(unsigned)((pairs + kMergeWaves - 1) / kMergeWaves), 64 * kMergeWaves, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
