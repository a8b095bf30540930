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
//    the request's Q_i*H (row, head) pairs); each wave owns 16 of those rows
//    outright, so no softmax state crosses waves. All rows of a request share
//    the shard's KV, so every KV tile is read from HBM once per row block.
//  * KV streams in 64-token tiles, double-buffered in LDS. bf16 tiles go
//    straight from HBM to LDS (global_load_lds_dwordx4: one 1 KB instruction
//    per token's latent part, one per 8 tokens' rope parts), so no registers
//    hold data in flight; the page-table entries a tile needs are fetched one
//    tile ahead so that issuing a tile never waits. fp8 codes are loaded into
//    registers one tile ahead and widened exactly to bf16 on the way into LDS
//    (the scale is folded into the score scale and the output).
//  * LDS tile layout: latent [64 tokens][512 bf16 + 16 pad] (with this row
//    stride neither the QK fragment reads nor the transposed V reads hit bank
//    conflicts; measured with the SQ_LDS_BANK_CONFLICT counter) and rope
//    [64 tokens][8 chunks of 16 B] with chunk c of token t in slot c ^ (t & 7).
//  * S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_16x16x32_bf16 with Q in
//    registers. The S^T accumulator layout is already the B-operand layout of
//    the PV product (under a fixed token permutation inside each 32-token
//    K-step), so P never moves between lanes; V^T fragments come straight from
//    the row-major tile with ds_read_b64_tr_b16.
//  * Online softmax in base 2 with a lazily refreshed reference: O and the sum
//    are rescaled only when the row maximum exceeds the reference by more than
//    8 (factor 256, harmless for bf16 P and fp32 sums); at the end they are
//    rescaled once to the true maximum, which is what is stored.
#include "internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kTile = 64;                  // tokens per KV tile
constexpr int kLatRow = 1056;              // 512 bf16 latent + 32 B pad (no bank conflicts)
constexpr int kLatBytes = kTile * kLatRow;
constexpr int kRopeRow = 128;              // 64 bf16 rope = 8 chunks of 16 B
constexpr int kRopeBytes = kTile * kRopeRow;
constexpr int kBufBytes = kLatBytes + kRopeBytes;
constexpr int kThreads = 256;
constexpr int kQSteps = kHeadDim / 32;     // 18 MFMA K-steps (32 dims) for QK^T
constexpr int kLatQSteps = kVDim / 32;     // the first 16 read the latent region
constexpr int kNTiles = kVDim / 16;        // 32 output tiles of 16 latent dims
constexpr int kTokBytesBf16 = kHeadDim * 2;
constexpr float kNegInf = -__builtin_inff();
constexpr float kRescaleSlack = 8.f;       // log2 units

// Slot permutation of the 16-byte chunks of latent row r.
__device__ __forceinline__ int lat_swz(int r) { return 0; }
// Byte offset of 16-byte chunk c (dims 8c..8c+7) of latent row r in a tile.
__device__ __forceinline__ int lat_off(int r, int c) { return r * kLatRow + ((c ^ lat_swz(r)) << 4); }

// Source of tokens outside the segment: a row of zeros, so that masked
// positions hold finite values (0 * NaN would poison the PV product).
__device__ __align__(16) unsigned char g_zero_token[kTokBytesBf16];

__device__ inline float max_over_row(float x) {  // lanes l, l^16, l^32, l^48
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ inline float sum_over_row(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
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

// Sub-page id of local token `tok` (-1 past the segment end).
__device__ inline int32_t subpage_of(const AttnArgs& a, const int32_t* pt_row, int tok, int hi) {
  return tok < hi ? pt_row[tok >> a.page_shift] : -1;
}

// Address of token `tok` with sub-page id `sp`, or the zero row when the token
// is past the segment end `hi` or sp is outside the pool.
template <int TOKB>
__device__ inline const unsigned char* token_src(const AttnArgs& a, const unsigned char* pool,
                                                 int32_t sp, int tok, int hi) {
  if (tok >= hi || sp < 0 || sp >= a.num_subpages) return g_zero_token;
  const int64_t t = ((int64_t)sp << a.page_shift) + (tok & (a.page_size - 1));
  return pool + t * TOKB;
}

// Page-table entries one wave needs to issue a bf16 tile: lane l holds the
// entry of latent token 16w + (l & 15) and of rope tokens 16w + (l >> 3) and
// 16w + 8 + (l >> 3).
// The loads are unconditional (clamped index; the consumer checks tok < hi),
// so that every fetch issues exactly three vector memory instructions and
// nothing waits for them until they are used.
__device__ inline int32_t subpage_always(const AttnArgs& a, const int32_t* pt_row, int tok,
                                         int hi) {
  return pt_row[min(tok, hi - 1) >> a.page_shift];
}
struct Bf16Pages {
  int32_t lat, rope0, rope1;
  __device__ inline void fetch(const AttnArgs& a, const int32_t* pt_row, int tb, int hi,
                               int wave, int lane) {
    lat = subpage_always(a, pt_row, tb + 16 * wave + (lane & 15), hi);
    rope0 = subpage_always(a, pt_row, tb + 16 * wave + (lane >> 3), hi);
    rope1 = subpage_always(a, pt_row, tb + 16 * wave + 8 + (lane >> 3), hi);
  }
};

// Workgroup barrier that orders LDS traffic only. __syncthreads() would also
// wait for every outstanding global load, i.e. for the prefetches this
// kernel deliberately keeps in flight across barriers.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt with vmcnt = n and no wait on the other counters (gfx9 encoding).
#define MLA_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (0x7 << 4) | (0xF << 8) | ((((n) >> 4) & 0x3) << 14))

// bf16: direct HBM -> LDS load number j (0..17) of this wave for tile
// [tb, tb + 64) into `dst`: j < 16 is the latent part of token 16w + j (one
// 1 KB instruction), j = 16, 17 the rope parts of tokens 16w + 8(j-16) + 0..7.
__device__ __forceinline__ void issue_one_bf16(const AttnArgs& a, const unsigned char* pool,
                                               const Bf16Pages& pg, int tb, int hi,
                                               unsigned char* dst, int wave, int lane, int j) {
  if (j < 16) {
    const int row = 16 * wave + j;
    const int32_t sp = __builtin_amdgcn_readlane(pg.lat, j);
    const unsigned char* src = token_src<kTokBytesBf16>(a, pool, sp, tb + row, hi);
    // slot `lane` of the row holds chunk lane ^ swz(row)
    __builtin_amdgcn_global_load_lds((const void*)(src + 16 * (lane ^ lat_swz(row))),
                                     (lds_void*)(dst + row * kLatRow), 16, 0, 0);
  } else {
    const int jj = j - 16;
    const int u = lane >> 3;                // token within the 8-token group
    const int chunk = (lane & 7) ^ u;       // slot (lane & 7) holds chunk ^ u
    const int row = 16 * wave + 8 * jj + u;
    const unsigned char* src =
        token_src<kTokBytesBf16>(a, pool, jj ? pg.rope1 : pg.rope0, tb + row, hi);
    __builtin_amdgcn_global_load_lds((const void*)(src + 2 * kVDim + 16 * chunk),
                                     (lds_void*)(dst + kLatBytes + (16 * wave + 8 * jj) * kRopeRow),
                                     16, 0, 0);
  }
}

// All 18 loads of this wave for one tile.
__device__ inline void issue_tile_bf16(const AttnArgs& a, const unsigned char* pool,
                                       const Bf16Pages& pg, int tb, int hi, unsigned char* dst,
                                       int wave, int lane) {
#pragma unroll
  for (int j = 0; j < 18; ++j) issue_one_bf16(a, pool, pg, tb, hi, dst, wave, lane, j);
}

// fp8: lane l of wave w loads chunks [9w, 9w + 9) (16 codes each) of token l.
struct Fp8Stage {
  static constexpr int kLoads = kHeadDim / 16 / 4;  // 9
  uint4 reg[kLoads];
  int32_t sp;

  __device__ inline void fetch_page(const AttnArgs& a, const int32_t* pt_row, int tb, int hi,
                                    int lane) {
    sp = subpage_always(a, pt_row, tb + lane, hi);
  }
  __device__ inline void load(const AttnArgs& a, const unsigned char* pool, int tb, int hi,
                              int wave, int lane) {
    const unsigned char* src = token_src<kHeadDim>(a, pool, sp, tb + lane, hi) + 16 * kLoads * wave;
#pragma unroll
    for (int j = 0; j < kLoads; ++j) reg[j] = *reinterpret_cast<const uint4*>(src + 16 * j);
  }
  __device__ inline void store(unsigned char* dst, int wave, int lane) const {
    const int row = lane;
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int col = kLoads * wave + j;      // 16-dim chunk
      uint4 lo, hi4;
      fp8x16_to_bf16(reg[j], lo, hi4);
      if (col < kVDim / 16) {
        *reinterpret_cast<uint4*>(dst + lat_off(row, 2 * col)) = lo;
        *reinterpret_cast<uint4*>(dst + lat_off(row, 2 * col + 1)) = hi4;
      } else {
        const int c0 = 2 * (col - kVDim / 16);
        unsigned char* rb = dst + kLatBytes + row * kRopeRow;
        *reinterpret_cast<uint4*>(rb + 16 * (c0 ^ (row & 7))) = lo;
        *reinterpret_cast<uint4*>(rb + 16 * ((c0 + 1) ^ (row & 7))) = hi4;
      }
    }
  }
};

// Exchange between the two waves of a row group goes through the tile buffer
// that is being computed on (which the direct loads provably do not target):
// row maxima in the 32-byte padding of latent rows 0..15 (never loaded or
// read otherwise), P fragments in the rope region (dead once QK^T is done).
__device__ __forceinline__ float* xmax(unsigned char* tile, int g, int c, int row) {
  const int f = (2 * g + c) * 32 + row;                // 0..127
  return reinterpret_cast<float*>(tile + (f >> 3) * kLatRow + 1024 + 4 * (f & 7));
}
__device__ __forceinline__ uint4* xpfrag(unsigned char* tile, int g, int c, int rt, int lane) {
  return reinterpret_cast<uint4*>(tile + kLatBytes) + ((2 * g + c) * 2 + rt) * 64 + lane;
}
static_assert(kLatRow - 1024 >= 32, "row padding holds 8 floats");
static_assert(kRopeBytes >= 2 * 2 * 2 * 64 * 16, "rope region holds the P fragments");

// Exchange area for the epilogue only.
struct Xchg {
  float rowsum[2][2][32];              // [g][c][32 rows]
};

// Accumulation state of one wave: 32 rows (two 16-row tiles) x 256 latent dims.
struct WaveState {
  f32x4 o[2][kNTiles / 2];  // O^T tiles: lane l holds dims 256c + 16n + 4(l/16) + 0..3
  float m_ref[2];           // reference exponent of o and l_part (row-uniform)
  float m_true[2];          // true running maximum (row-uniform)
  float l_part[2];          // this lane's share of the exp2 sum over this wave's tokens
};

// Scores, softmax and PV for one 64-token tile held in `tile` (LDS).
// Wave (g, c): rows 32g..32g+31 of the block; QK^T over tokens 32c..32c+31 of
// the tile; PV over all 64 tokens for latent dims 256c..256c+255.
// `issue(k)` is called once per QK K-step (k = 0..17), so that the loads of
// the next tile are spread over the MFMA work instead of stalling the wave.
template <class Issue>
__device__ __forceinline__ void compute_tile(unsigned char* __restrict__ tile,
                                             const bf16x8 (&qf)[2][kQSteps],
                                             WaveState& st, int tb, const int (&hi_row)[2],
                                             float qk_scale_log2, int g, int c, int lane,
                                             Issue&& issue) {
  const int r16 = lane & 15;
  const int g4 = lane >> 4;

  // ---- S^T[32 tokens x 32 rows]: per K-step two K fragments (16 tokens each),
  // each feeding both row tiles.
  f32x4 sacc[2][2] = {{f32x4{}, f32x4{}}, {f32x4{}, f32x4{}}};  // [row tile][token tile]
  auto kfrag = [&](int k, int tt) -> bf16x8 {
    const int tok = 32 * c + 16 * tt + r16;
    if (k < kLatQSteps)
      return *reinterpret_cast<const bf16x8*>(tile + lat_off(tok, 4 * k + g4));
    const int chunk = 4 * (k - kLatQSteps) + g4;
    return *reinterpret_cast<const bf16x8*>(tile + kLatBytes + tok * kRopeRow +
                                            16 * (chunk ^ (tok & 7)));
  };
  // K fragments are read two K-steps ahead of their MFMAs (a 3-slot ring);
  // the scheduling barriers keep that order.
  bf16x8 kr[3][2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    kr[k][0] = kfrag(k, 0);
    kr[k][1] = kfrag(k, 1);
  }
#pragma unroll
  for (int k = 0; k < kQSteps; ++k) {
    if (k + 2 < kQSteps) {
      kr[(k + 2) % 3][0] = kfrag(k + 2, 0);
      kr[(k + 2) % 3][1] = kfrag(k + 2, 1);
    }
    issue(k);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        sacc[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[k % 3][tt], qf[rt][k],
                                                               sacc[rt][tt], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- scale, mask, row max over this wave's 32 tokens
  float sv[2][8];
  float mx[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    mx[rt] = kNegInf;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int tok = tb + 32 * c + 16 * tt + 4 * g4 + v;
        const float x = tok < hi_row[rt] ? sacc[rt][tt][v] * qk_scale_log2 : kNegInf;
        sv[rt][4 * tt + v] = x;
        mx[rt] = fmaxf(mx[rt], x);
      }
    }
    mx[rt] = max_over_row(mx[rt]);
    if (g4 == 0) *xmax(tile, g, c, 16 * rt + r16) = mx[rt];
  }
  lds_barrier();
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    // the partner saw the other 32 tokens; both waves now hold the same tile max
    mx[rt] = fmaxf(mx[rt], *xmax(tile, g, c ^ 1, 16 * rt + r16));
    st.m_true[rt] = fmaxf(st.m_true[rt], mx[rt]);
  }

  // ---- lazily refreshed reference (identical decisions on both waves)
  const bool refresh0 = mx[0] > st.m_ref[0] + kRescaleSlack;
  const bool refresh1 = mx[1] > st.m_ref[1] + kRescaleSlack;
  if (__builtin_amdgcn_ballot_w64(refresh0 || refresh1) != 0) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const bool rf = rt ? refresh1 : refresh0;
      const float alpha = rf ? __builtin_amdgcn_exp2f(st.m_ref[rt] - mx[rt]) : 1.f;
      st.l_part[rt] *= alpha;
#pragma unroll
      for (int n = 0; n < kNTiles / 2; ++n) st.o[rt][n] *= alpha;
      st.m_ref[rt] = rf ? mx[rt] : st.m_ref[rt];
    }
  }

  // ---- P of this wave's tokens: element e of lane l is token
  // 32c + 16(e/4) + 4(l/16) + e%4; publish it for the partner.
  bf16x8 pown[2], ppart[2];  // [row tile]: this wave's tokens / the partner's
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const float m_use = st.m_ref[rt] == kNegInf ? 0.f : st.m_ref[rt];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = sv[rt][e] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(sv[rt][e] - m_use);
      st.l_part[rt] += p;
      pown[rt][e] = (__bf16)p;
    }
    *xpfrag(tile, g, c, rt, lane) = __builtin_bit_cast(uint4, pown[rt]);
  }
  lds_barrier();
  // K-step kk of the PV product covers tokens 32kk..32kk+31, i.e. half kk
  bf16x8 pf[2][2];  // [token half][row tile]
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    ppart[rt] = __builtin_bit_cast(bf16x8, *xpfrag(tile, g, c ^ 1, rt, lane));
    pf[0][rt] = c == 0 ? pown[rt] : ppart[rt];
    pf[1][rt] = c == 0 ? ppart[rt] : pown[rt];
  }

  // ---- O^T[256 dims x 32 rows] += V^T[256 x 64 tokens] P^T[64 x 32]. Lane i
  // of each 16-lane group points at dims 16n + 4(i%4) of token t0 + i/4; the
  // transposed read hands it dim 16n + i of tokens t0..t0+3.
  // Steps t = 16kk + n (K-step kk, 16-dim tile n); each step's two transposed
  // reads are issued three steps ahead of its MFMAs (a 4-slot ring).
  const int i16 = lane & 15;
  auto vread = [&](int t, i16x4& lo4, i16x4& hi4) {
    const int kk = t >> 4, n = t & 15;
    const int row = 32 * kk + 4 * g4 + (i16 >> 2);
    const int ch = 32 * c + 2 * n + ((i16 & 3) >> 1);
    const int byte = 8 * (i16 & 1);
    lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + lat_off(row, ch) + byte));
    hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(tile + lat_off(row + 16, ch) + byte));
  };
  constexpr int kPvSteps = 2 * (kNTiles / 2);
  i16x4 vr[4][2];
#pragma unroll
  for (int t = 0; t < 3; ++t) vread(t, vr[t][0], vr[t][1]);
#pragma unroll
  for (int t = 0; t < kPvSteps; ++t) {
    if (t + 3 < kPvSteps) vread(t + 3, vr[(t + 3) % 4][0], vr[(t + 3) % 4][1]);
    __builtin_amdgcn_sched_barrier(0);
    const int kk = t >> 4, n = t & 15;
    const bf16x8 va = __builtin_bit_cast(
        bf16x8, __builtin_shufflevector(vr[t % 4][0], vr[t % 4][1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
      st.o[rt][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pf[kk][rt], st.o[rt][n], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Page-table entry of the 16-token slice of wave w in tile tb, by a uniform
// (scalar) load. Valid when the sub-page size is a multiple of 16, so that a
// 16-aligned slice lies inside one sub-page.
__device__ __forceinline__ int32_t slice_page(const AttnArgs& a, const int32_t* pt_row, int tb,
                                              int hi, int wave) {
  typedef __attribute__((address_space(4))) const int32_t cint;
  const int tok = min(tb + 16 * wave, hi - 1);
  return ((cint*)pt_row)[tok >> a.page_shift];
}

// Slice-page variants of the bf16 loads (all 16 tokens of the slice in `sp`).
__device__ __forceinline__ void issue_one_slice(const AttnArgs& a, const unsigned char* pool,
                                                int32_t sp, int tb, int hi, unsigned char* dst,
                                                int wave, int lane, int j) {
  if (j < 16) {
    const int row = 16 * wave + j;
    const unsigned char* src = token_src<kTokBytesBf16>(a, pool, sp, tb + row, hi);
    __builtin_amdgcn_global_load_lds((const void*)(src + 16 * (lane ^ lat_swz(row))),
                                     (lds_void*)(dst + row * kLatRow), 16, 0, 0);
  } else {
    const int jj = j - 16;
    const int u = lane >> 3;
    const int chunk = (lane & 7) ^ u;
    const int row = 16 * wave + 8 * jj + u;
    const unsigned char* src = token_src<kTokBytesBf16>(a, pool, sp, tb + row, hi);
    __builtin_amdgcn_global_load_lds((const void*)(src + 2 * kVDim + 16 * chunk),
                                     (lds_void*)(dst + kLatBytes + (16 * wave + 8 * jj) * kRopeRow),
                                     16, 0, 0);
  }
}
// Load pipelines. kSlice: bf16 with sub-pages of >= 16 tokens -- while tile k
// is computed, tile k+1 streams HBM -> LDS one instruction per QK K-step and
// the page entries of later tiles come in by scalar loads (one per wave and
// tile: a wave's 16-token slice lies in one sub-page). kGeneric: bf16 with smaller sub-pages -- per-lane
// page entries, whole next tile issued at the start of each tile. kFp8: codes
// staged through registers and widened into LDS.
enum LoadMode { kSlice = 0, kGeneric = 1, kFp8 = 2 };

template <int MODE>
__global__ void __launch_bounds__(kThreads, 1) attn_kernel(AttnArgs a) {
  constexpr bool FP8 = MODE == kFp8;
  // Two separate arrays (not one indexed one), so that the compiler can tell
  // the buffer being read from the buffer the direct loads are filling.
  __shared__ __align__(16) unsigned char buf0[kBufBytes];
  __shared__ __align__(16) unsigned char buf1[kBufBytes];
  __shared__ Xchg xc;
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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = wave >> 1;                  // row group: 32 rows
  const int c = wave & 1;                   // token half (QK) / latent half (PV)
  const int r16 = lane & 15;
  const int g4 = lane >> 4;

  const unsigned char* pool =
      a.kv + (int64_t)r * a.pool_tokens * (FP8 ? kHeadDim : kTokBytesBf16);
  const int32_t* pt_row = a.page_table + ((int64_t)r * a.R + last) * a.pt_width;

  // ---- first tile(s) in flight before anything else
  Fp8Stage fs;
  Bf16Pages pg;
  int32_t spA = 0, spB = 0, spC = 0;        // kSlice: pages of tiles k+1, k+2, k+3
  if constexpr (MODE == kSlice) {
    const int32_t sp0 = slice_page(a, pt_row, lo, hi, wave);
    spA = slice_page(a, pt_row, lo + kTile, hi, wave);
    spB = slice_page(a, pt_row, lo + 2 * kTile, hi, wave);
#pragma unroll
    for (int j = 0; j < 18; ++j) issue_one_slice(a, pool, sp0, lo, hi, buf0, wave, lane, j);
  } else if constexpr (MODE == kGeneric) {
    pg.fetch(a, pt_row, lo, hi, wave, lane);
    issue_tile_bf16(a, pool, pg, lo, hi, buf0, wave, lane);
  } else {
    fs.fetch_page(a, pt_row, lo, hi, lane);
    fs.load(a, pool, lo, hi, wave, lane);
    fs.fetch_page(a, pt_row, lo + kTile, hi, lane);
  }

  // ---- this lane's two rows (one per 16-row tile) and their visible lengths
  int mrow[2], hi_row[2];
  bool row_ok[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    mrow[rt] = m0 + 32 * g + 16 * rt + r16;
    row_ok[rt] = mrow[rt] < M;
    const int Lrow = row_ok[rt] ? a.row_lens[(int64_t)r * a.R + qs + mrow[rt] / a.H] : 0;
    hi_row[rt] = min(hi, Lrow);
  }

  // ---- Q fragments (B operand of S^T = K Q^T): 8 dims per lane per K-step
  bf16x8 qf[2][kQSteps];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const uint16_t* qp =
        a.q + ((int64_t)qs * a.H + (row_ok[rt] ? mrow[rt] : 0)) * kHeadDim + 8 * g4;
#pragma unroll
    for (int k = 0; k < kQSteps; ++k) {
      uint4 v = row_ok[rt] ? *reinterpret_cast<const uint4*>(qp + 32 * k) : make_uint4(0, 0, 0, 0);
      qf[rt][k] = __builtin_bit_cast(bf16x8, v);
    }
  }

  WaveState st;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
    for (int n = 0; n < kNTiles / 2; ++n) st.o[rt][n] = f32x4{};
    st.m_ref[rt] = kNegInf;
    st.m_true[rt] = kNegInf;
    st.l_part[rt] = 0.f;
  }

  // One tile: make `cur` ready, start filling `nxt` with the following tile,
  // then compute on `cur`.
  auto step = [&](unsigned char* cur, unsigned char* nxt, int tb) {
    const bool more = tb + kTile < hi;
    if constexpr (MODE == kFp8) {
      // `cur` was last read two tiles ago, before the previous barrier.
      fs.store(cur, wave, lane);
      lds_barrier();
      if (more) {
        fs.load(a, pool, tb + kTile, hi, wave, lane);
        fs.fetch_page(a, pt_row, tb + 2 * kTile, hi, lane);
      }
    } else if constexpr (MODE == kGeneric) {
      __builtin_amdgcn_s_waitcnt(0);
      lds_barrier();
      if (more) {
        pg.fetch(a, pt_row, tb + kTile, hi, wave, lane);
        issue_tile_bf16(a, pool, pg, tb + kTile, hi, nxt, wave, lane);
      }
    } else {
      // This wave's loads of this tile have landed ...
      MLA_WAIT_VMCNT(0);
      lds_barrier();                        // ... for all waves; `nxt` is free
      if (more) spC = slice_page(a, pt_row, tb + 3 * kTile, hi, wave);
    }
    // kSlice: the next tile's loads go out one per QK K-step.
    auto issue = [&](int j) {
      if constexpr (MODE == kSlice) {
        if (more) {
          issue_one_slice(a, pool, spA, tb + kTile, hi, nxt, wave, lane, j);

        }
      }
    };
    compute_tile(cur, qf, st, tb, hi_row, a.qk_scale_log2, g, c, lane, issue);
    if constexpr (MODE == kSlice) {
      spA = spB;
      spB = spC;
    }
  };
  for (int tb = lo; tb < hi; tb += 2 * kTile) {
    step(buf0, buf1, tb);
    if (tb + kTile >= hi) break;
    step(buf1, buf0, tb + kTile);
  }

  // ---- sums over all 64 tokens of each tile: this wave's share + the partner's
  float l_row[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) l_row[rt] = sum_over_row(st.l_part[rt]);
  __syncthreads();                          // last use of xc.rowmax as tile maxima done
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
    if (g4 == 0) xc.rowsum[g][c][16 * rt + r16] = l_row[rt];
  __syncthreads();
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    l_row[rt] += xc.rowsum[g][c ^ 1][16 * rt + r16];
    if (!row_ok[rt]) continue;
    // move O and l from the reference exponent to the true maximum
    float fix = 1.f;
    if (st.m_true[rt] != kNegInf) fix = __builtin_amdgcn_exp2f(st.m_ref[rt] - st.m_true[rt]);
    const float vs = fix * a.v_scale;
    const int64_t e = (((int64_t)r * a.R + qs) * a.H + mrow[rt]) * a.nseg + s;
    if (c == 0 && g4 == 0) {
      a.segm_max[e] = st.m_true[rt];
      a.segm_expsum[e] = l_row[rt] * fix;
    }
    float* op = a.segm_out + e * kVDim + 256 * c + 4 * g4;
#pragma unroll
    for (int n = 0; n < kNTiles / 2; ++n) {
      *reinterpret_cast<float4*>(op + 16 * n) =
          make_float4(st.o[rt][n][0] * vs, st.o[rt][n][1] * vs, st.o[rt][n][2] * vs,
                      st.o[rt][n][3] * vs);
    }
  }
}

}  // namespace

hipError_t launch_attn(const AttnArgs& a, bool fp8, hipStream_t s) {
  const int64_t blocks = (int64_t)a.N * a.W * a.nseg * a.mblocks;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (fp8)
    attn_kernel<kFp8><<<(unsigned)blocks, kThreads, 0, s>>>(a);
  else if (a.page_size >= 16)
    attn_kernel<kSlice><<<(unsigned)blocks, kThreads, 0, s>>>(a);
  else
    attn_kernel<kGeneric><<<(unsigned)blocks, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
