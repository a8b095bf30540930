// Split-K segmented MLA attention partials over a paged, round-robin sharded
// latent KV cache, for gfx950.
//
// What is computed (vLLM PR #51705 digest, Implementation breakdown items 2-4
// and the merge snippet): for every shard r, verify row rho, head h and split-K
// segment s, over the segment's local tokens that the row may see,
//   m2 = max(score * log2 e), e = sum 2^(score*log2e - m2),
//   O  = sum 2^(score*log2e - m2) * v,   score = sm_scale * <q, k> (576 dims),
// with v the 512 latent dims of the same cache entry (SGLang PR #34432 report,
// _forward_verify_dcp snippet). The partition follows the pages'
// tiles_per_segment = ceil(len / (segments * tile)) with len the group's
// longest row and tile = the sub-page size.
//
// Design (gfx950, wave64):
//  * One workgroup = 4 waves = (request i, shard r, segment s, 64-row block of
//    the request's Q_i*H (row, head) pairs). All rows of a request share the
//    shard's KV, so every KV tile is read from HBM once per row block.
//  * KV is streamed in 64-token tiles: 16-byte global loads into registers one
//    tile ahead, then a row-major bf16 tile in LDS (fp8 codes are widened to
//    bf16 exactly on the way in; the scale is folded into the score scale and
//    the output).
//  * Waves form a 2 x 2 grid: g picks 32 rows, c picks a 32-token half of the
//    tile for S^T = K Q^T (v_mfma_f32_32x32x16_bf16, Q held in registers) and a
//    256-wide half of the latent dims for O^T = V^T P^T. The S^T accumulator
//    layout is already the B-operand layout of the PV product (with a fixed
//    token permutation), so P never moves between lanes; V^T fragments come
//    straight from the row-major tile with ds_read_b64_tr_b16.
//  * Online softmax in base 2; the two token halves exchange their row maxima
//    and P fragments through LDS.
#include "internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

constexpr int kTile = 64;                 // tokens per KV tile
constexpr int kRowBytes = 1168;           // 576 bf16 + 16 pad: 8-row reads hit all banks
constexpr int kTileBytes = kTile * kRowBytes;
constexpr int kChunksPerRowBf16 = kHeadDim * 2 / 16;  // 72 x 16B per bf16 token
constexpr int kChunksPerRowFp8 = kHeadDim / 16;       // 36 x 16B per fp8 token
constexpr int kThreads = 256;
constexpr int kLoadsBf16 = kTile * kChunksPerRowBf16 / kThreads;  // 18
constexpr int kLoadsFp8 = kTile * kChunksPerRowFp8 / kThreads;    // 9
constexpr int kKSteps = kHeadDim / 16;    // 36 MFMA K-steps for QK^T
constexpr float kNegInf = -__builtin_inff();

struct __align__(16) Smem {
  unsigned char tile[kTileBytes];
  float xch[2][2][32];                 // per-row max / sum exchange [g][c][row]
  uint4 pfrag[2][2][2][64];            // P fragments [g][c][k-step][lane]
};

__device__ inline float wave_max32(float x) {  // combine lanes l and l^32
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ inline float wave_sum32(float x) { return x + __shfl_xor(x, 32); }

__device__ inline bf16x8 pack_bf16(const float* v) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)v[e];
  return r;
}

// Widen 16 e4m3fn codes (one uint4) to 16 bf16 values (two uint4). Exact:
// every e4m3fn value is a bf16 value.
__device__ inline void fp8x16_to_bf16(uint4 in, uint4& lo, uint4& hi) {
  const uint32_t w[4] = {in.x, in.y, in.z, in.w};
  uint32_t o[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    // v_cvt_pk_f32_fp8 reads the OCP e4m3fn format on gfx950.
    auto f01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], false);
    auto f23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], true);
    // f32 -> bf16 by truncation is exact for these values.
    o[2 * k] = (__float_as_uint(f01[0]) >> 16) | (__float_as_uint(f01[1]) & 0xFFFF0000u);
    o[2 * k + 1] = (__float_as_uint(f23[0]) >> 16) | (__float_as_uint(f23[1]) & 0xFFFF0000u);
  }
  lo = make_uint4(o[0], o[1], o[2], o[3]);
  hi = make_uint4(o[4], o[5], o[6], o[7]);
}

template <bool FP8>
struct TileLoader {
  static constexpr int kLoads = FP8 ? kLoadsFp8 : kLoadsBf16;
  static constexpr int kChunks = FP8 ? kChunksPerRowFp8 : kChunksPerRowBf16;
  static constexpr int kTokBytes = FP8 ? kHeadDim : kHeadDim * 2;
  uint4 reg[kLoads];

  // Issue the global loads of tile [tb, tb + 64) (tokens >= hi are skipped).
  __device__ inline void load(const AttnArgs& a, const unsigned char* pool,
                              const int32_t* pt_row, int tb, int hi, int tid) {
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int cid = tid + kThreads * j;
      const int tok = tb + cid / kChunks;
      const int col = cid % kChunks;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (tok < hi) {
        const int32_t sp = pt_row[tok >> a.page_shift];
        if (sp >= 0 && sp < a.num_subpages) {
          const int64_t t = ((int64_t)sp << a.page_shift) + (tok & (a.page_size - 1));
          v = *reinterpret_cast<const uint4*>(pool + t * kTokBytes + col * 16);
        }
      }
      reg[j] = v;
    }
  }

  // Write the loaded tile into LDS as bf16 rows; tokens >= hi become zeros.
  __device__ inline void store(unsigned char* tile, int tb, int hi, int tid) const {
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int cid = tid + kThreads * j;
      const int row = cid / kChunks;
      const int col = cid % kChunks;
      const bool ok = tb + row < hi;
      if (FP8) {
        uint4 lo, hi4;
        fp8x16_to_bf16(reg[j], lo, hi4);
        if (!ok) { lo = make_uint4(0, 0, 0, 0); hi4 = lo; }
        uint4* dst = reinterpret_cast<uint4*>(tile + row * kRowBytes + col * 32);
        dst[0] = lo;
        dst[1] = hi4;
      } else {
        uint4 v = ok ? reg[j] : make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(tile + row * kRowBytes + col * 16) = v;
      }
    }
  }
};

template <bool FP8>
__global__ void __launch_bounds__(kThreads, 1) attn_kernel(AttnArgs a) {
  __shared__ Smem sm;
  // ---- work unit of this workgroup
  int b = blockIdx.x;
  const int mb = b % a.mblocks;
  b /= a.mblocks;
  const int s = b % a.nseg;
  b /= a.nseg;
  const int r = b % a.W;
  const int i = b / a.W;

  const int qs = a.q_start[i];
  const int Q = a.q_start[i + 1] - qs;
  const int M = Q * a.H;                    // (row, head) pairs of the request
  const int m0 = mb * kAttnRows;
  if (qs < 0 || Q <= 0 || qs + Q > a.R || m0 >= M) return;
  const int last = qs + Q - 1;              // the group's longest row
  int Lg = a.row_lens[(int64_t)r * a.R + last];
  Lg = min(Lg, a.pt_width * a.page_size);
  const int span = (Lg + a.nseg * a.page_size - 1) / (a.nseg * a.page_size) * a.page_size;
  const int lo = s * span;
  const int hi = min(lo + span, Lg);
  if (lo >= hi) return;                     // segment inactive for the whole group

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = wave >> 1;                  // row group (32 rows)
  const int c = wave & 1;                   // token half (QK) / latent half (PV)
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  // ---- this lane's row and its visible length
  const int mrow = m0 + 32 * g + l32;
  const bool row_ok = mrow < M;
  int Lrow = 0;
  if (row_ok) Lrow = a.row_lens[(int64_t)r * a.R + qs + mrow / a.H];
  const int hi_row = min(hi, Lrow);

  // ---- Q fragments (B operand of S^T = K Q^T): 8 dims per K-step
  bf16x8 qf[kKSteps];
  {
    const uint16_t* qp = a.q + ((int64_t)qs * a.H + (row_ok ? mrow : 0)) * kHeadDim + 8 * hl;
#pragma unroll
    for (int k = 0; k < kKSteps; ++k) {
      uint4 v = row_ok ? *reinterpret_cast<const uint4*>(qp + 16 * k) : make_uint4(0, 0, 0, 0);
      qf[k] = __builtin_bit_cast(bf16x8, v);
    }
  }

  const unsigned char* pool =
      a.kv + (int64_t)r * a.pool_tokens * (FP8 ? kHeadDim : kHeadDim * 2);
  const int32_t* pt_row = a.page_table + ((int64_t)r * a.R + last) * a.pt_width;

  f32x16 o[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) o[n] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;

  TileLoader<FP8> ld;
  ld.load(a, pool, pt_row, lo, hi, tid);

  // LDS addresses used every tile
  const unsigned char* k_rd = sm.tile + (32 * c + l32) * kRowBytes + 16 * hl;
  const int g16 = lane >> 4, i16 = lane & 15;
  const unsigned char* v_rd =
      sm.tile + (4 * (g16 >> 1) + (i16 >> 2)) * kRowBytes +
      (256 * c + 16 * (g16 & 1) + 4 * (i16 & 3)) * 2;

  for (int tb = lo; tb < hi; tb += kTile) {
    __syncthreads();                        // previous tile fully consumed
    ld.store(sm.tile, tb, hi, tid);
    __syncthreads();
    if (tb + kTile < hi) ld.load(a, pool, pt_row, tb + kTile, hi, tid);

    // ---- S^T[32 tokens x 32 rows] for token half c
    f32x16 acc = f32x16{};
#pragma unroll
    for (int k = 0; k < kKSteps; ++k) {
      bf16x8 kf = *reinterpret_cast<const bf16x8*>(k_rd + 32 * k);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[k], acc, 0, 0, 0);
    }

    // ---- scale, mask, tile max
    float sv[16];
    float mx = kNegInf;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int tok = tb + 32 * c + 8 * (v >> 2) + 4 * hl + (v & 3);
      sv[v] = tok < hi_row ? acc[v] * a.qk_scale_log2 : kNegInf;
      mx = fmaxf(mx, sv[v]);
    }
    mx = wave_max32(mx);
    if (hl == 0) sm.xch[g][c][l32] = mx;
    __syncthreads();
    mx = fmaxf(mx, sm.xch[g][c ^ 1][l32]);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float psum = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      sv[v] = sv[v] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(sv[v] - m_use);
      psum += sv[v];
    }
    psum = wave_sum32(psum);
    l_run = l_run * alpha + psum;
    m_run = m_new;

    // ---- P fragments: this half's two K-steps; publish them for the partner
    bf16x8 pown0 = pack_bf16(sv), pown1 = pack_bf16(sv + 8);
    sm.pfrag[g][c][0][lane] = __builtin_bit_cast(uint4, pown0);
    sm.pfrag[g][c][1][lane] = __builtin_bit_cast(uint4, pown1);
#pragma unroll
    for (int n = 0; n < 8; ++n) o[n] *= alpha;
    __syncthreads();
    bf16x8 pp0 = __builtin_bit_cast(bf16x8, sm.pfrag[g][c ^ 1][0][lane]);
    bf16x8 pp1 = __builtin_bit_cast(bf16x8, sm.pfrag[g][c ^ 1][1][lane]);

    // ---- O^T[256 dims x 32 rows] += V^T[256 x 64 tokens] P^T[64 x 32]
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int half = ks >> 1;
      bf16x8 pb = (half == c) ? ((ks & 1) ? pown1 : pown0) : ((ks & 1) ? pp1 : pp0);
      const unsigned char* vk = v_rd + 16 * ks * kRowBytes;
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const unsigned char* vp = vk + 64 * n;  // 32 dims = 64 bytes per tile
        i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(vp));
        i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(vp + 8 * kRowBytes));
        i16x8 va = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
        o[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, va), pb, o[n], 0, 0, 0);
      }
    }
  }

  // ---- combine the two token halves' sums (they share m_run)
  __syncthreads();
  if (hl == 0) sm.xch[g][c][l32] = l_run;
  __syncthreads();
  const float l_tot = l_run + sm.xch[g][c ^ 1][l32];

  if (!row_ok) return;
  const int64_t e = (((int64_t)r * a.R + qs) * a.H + mrow) * a.nseg + s;
  if (c == 0 && hl == 0) {
    a.segm_max[e] = m_run;
    a.segm_expsum[e] = l_tot;
  }
  float* op = a.segm_out + e * kVDim + 256 * c + 4 * hl;
#pragma unroll
  for (int n = 0; n < 8; ++n) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      float4 v = make_float4(o[n][4 * q4] * a.v_scale, o[n][4 * q4 + 1] * a.v_scale,
                             o[n][4 * q4 + 2] * a.v_scale, o[n][4 * q4 + 3] * a.v_scale);
      *reinterpret_cast<float4*>(op + 32 * n + 8 * q4) = v;
    }
  }
}

}  // namespace

hipError_t launch_attn(const AttnArgs& a, bool fp8, hipStream_t s) {
  const int64_t blocks = (int64_t)a.N * a.W * a.nseg * a.mblocks;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (fp8)
    attn_kernel<true><<<(unsigned)blocks, kThreads, 0, s>>>(a);
  else
    attn_kernel<false><<<(unsigned)blocks, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
