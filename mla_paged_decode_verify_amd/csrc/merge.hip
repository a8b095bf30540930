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
// One wave per (row, head) pair; each lane owns 8 consecutive latent dims.
// Shards are folded in online: every per-shard output is rounded to bf16 first,
// as it would be when a shard sends it to the others.
#include "internal.h"

namespace mla {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309f;

__device__ inline int find_request(const int32_t* q_start, int N, int rho) {
  int lo = 0, hi = N - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (q_start[mid] <= rho) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ inline float bf16_round(float x) {
  return (float)(__bf16)x;
}

__device__ inline uint32_t pack2_bf16(float a, float b) {
  __bf16 x = (__bf16)a, y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) |
         ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

__global__ void __launch_bounds__(256) merge_kernel(MergeArgs a) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t pair = (int64_t)blockIdx.x * 4 + wave;
  if (pair >= (int64_t)a.R * a.H) return;
  const int rho = (int)(pair / a.H);
  const int h = (int)(pair % a.H);
  const int i = find_request(a.q_start, a.N, rho);
  const int last = a.q_start[i + 1] - 1;
  if (a.q_start[i] > rho || last < rho || last >= a.R) return;  // malformed q_start
  const int seg_tokens = a.nseg * a.page_size;

  float gmax = kNegInf, gsum = 0.f;
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.f;

  for (int r = 0; r < a.W; ++r) {
    const int Lg = a.row_lens[(int64_t)r * a.R + last];
    const int L = a.row_lens[(int64_t)r * a.R + rho];
    const int span = (Lg + seg_tokens - 1) / seg_tokens * a.page_size;
    int nact = span > 0 ? (L + span - 1) / span : 0;
    nact = min(nact, a.nseg);
    const int64_t base = (((int64_t)r * a.R + rho) * a.H + h) * a.nseg;

    float M = kNegInf;
    for (int s = 0; s < nact; ++s) M = fmaxf(M, a.segm_max[base + s]);
    float o[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] = 0.f;
    float lse_r = kNegInf;
    if (M != kNegInf) {
      float E = 0.f;
      for (int s = 0; s < nact; ++s) {
        const float sc = exp2f(a.segm_max[base + s] - M);
        E += a.segm_expsum[base + s] * sc;
        const float4* src = reinterpret_cast<const float4*>(
            a.segm_out + (base + s) * kVDim + 8 * lane);
        const float4 x = src[0], y = src[1];
        o[0] += sc * x.x; o[1] += sc * x.y; o[2] += sc * x.z; o[3] += sc * x.w;
        o[4] += sc * y.x; o[5] += sc * y.y; o[6] += sc * y.z; o[7] += sc * y.w;
      }
      const float inv = 1.f / E;
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] = bf16_round(o[k] * inv);
      lse_r = kLn2 * (M + log2f(E));
    }
    if (a.shard_out != nullptr) {
      uint4 w = make_uint4(pack2_bf16(o[0], o[1]), pack2_bf16(o[2], o[3]),
                           pack2_bf16(o[4], o[5]), pack2_bf16(o[6], o[7]));
      *reinterpret_cast<uint4*>(a.shard_out +
                                (((int64_t)r * a.R + rho) * a.H + h) * kVDim + 8 * lane) = w;
    }
    if (a.shard_lse != nullptr && lane == 0)
      a.shard_lse[((int64_t)r * a.R + rho) * a.H + h] = lse_r;
    if (lse_r == kNegInf) continue;          // empty shard contributes nothing
    if (lse_r > gmax) {
      const float f = expf(gmax - lse_r);     // gmax = -inf gives 0
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] *= f;
      gsum *= f;
      gmax = lse_r;
    }
    const float wgt = expf(lse_r - gmax);
    gsum += wgt;
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] += wgt * o[k];
  }

  float res[8];
  float lse_out = kNegInf;
  if (gmax != kNegInf) {
    const float inv = 1.f / gsum;
#pragma unroll
    for (int k = 0; k < 8; ++k) res[k] = acc[k] * inv;
    lse_out = gmax + logf(gsum);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) res[k] = 0.f;
  }
  uint4 w = make_uint4(pack2_bf16(res[0], res[1]), pack2_bf16(res[2], res[3]),
                       pack2_bf16(res[4], res[5]), pack2_bf16(res[6], res[7]));
  *reinterpret_cast<uint4*>(a.out + pair * kVDim + 8 * lane) = w;
  if (lane == 0) a.lse[pair] = lse_out;
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  const int64_t pairs = (int64_t)a.R * a.H;
  if (pairs <= 0) return hipSuccess;
  merge_kernel<<<(unsigned)((pairs + 3) / 4), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
