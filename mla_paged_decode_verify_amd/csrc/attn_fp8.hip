// Split-K segmented MLA attention partials, fp8 KV cache (OCP e4m3fn or e5m2
// codes).
//
// The quantities computed, the work decomposition and the per-tile
// computation are those of attn_common.h, on the same double-buffered bf16
// tiles as the bf16 kernel. Specific to this kernel:
//  * The codes of the next 64-token tile (576 B per token) are fetched into
//    registers with ordinary vector loads while the current tile is computed
//    (each wave: its 16 tokens, nine 16-byte loads per lane), then widened
//    exactly to bf16 (every e4m3fn and every e5m2 value is a bf16 value) and
//    written into the other tile buffer in the latent / rope layout of
//    attn_common.h: no separate widening pass, no extra barrier, and the LDS
//    holds no staging copy of the codes.
//  * The fp8 scale is folded into the score scale and into the output.
#include "attn_common.h"

namespace mla {
namespace {

constexpr int kF8Loads = 16 * kHeadDim / 16 / 64;   // 9 16-byte loads per lane per tile
static_assert(kF8Loads * 64 * 16 == 16 * kHeadDim, "a wave's loads cover exactly 16 tokens");

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Widen 2 codes (the low or high half of a word) to 2 bf16 values with the
// gfx950 packed conversion at scale 1: e4m3fn ("fp8") or e5m2 ("bf8").
template <bool E5M2>
__device__ __forceinline__ uint32_t cvt2(uint32_t w, bool hi) {
  bf16x2_t r;
  if constexpr (E5M2) {
    r = hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, true)
           : __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, false);
  } else {
    r = hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
           : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  }
  return __builtin_bit_cast(uint32_t, r);
}
// 8 codes (two words) to 8 bf16 values (a uint4). Exact: every e4m3fn and
// every e5m2 value is a bf16 value (bf16 has more exponent and mantissa bits).
template <bool E5M2>
__device__ __forceinline__ uint4 fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  return make_uint4(cvt2<E5M2>(w0, false), cvt2<E5M2>(w0, true), cvt2<E5M2>(w1, false),
                    cvt2<E5M2>(w1, true));
}

// Sub-pages of 64 consecutive tiles for one wave: lane j holds the sub-page
// of tokens tb0 + 64 j + 16 w .. +15 (clamped to the last in-range token).
__device__ __forceinline__ int32_t f8_slice_pages(const AttnArgs& a, const int32_t* pt_row,
                                                  int tb0, int hi, int wave, int lane) {
  const int64_t tok = min((int64_t)tb0 + (int64_t)kTile * lane + 16 * wave, (int64_t)hi - 1);
  return pt_row[tok >> a.page_shift];
}

// The codes of one wave's 16 tokens of a tile (tokens tb + 16w .. + 15) in
// registers: load j of lane l is byte o = 1024 j + 16 l of the 16 tokens'
// 9216 bytes (a lane's 16 bytes never straddle two tokens: 576 = 36 * 16).
struct F8Codes {
  uint4 v[kF8Loads];
};

// Buffer-resource word 3 of the gfx9 family (gfx950 included): raw buffer
// access with no format conversion.
constexpr int kBufferRsrcWord3 = 0x00020000;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Sub-pages of 16+ tokens: the slice is contiguous in its sub-page `sp`, so
// one buffer resource covers it, its record count ending at the segment end:
// the loads of tokens past it return zeros (as the zero row would). Buffer
// loads count against vmcnt only (a flat load through a generic pointer would
// also count against lgkmcnt, and every LDS wait in the tile would then wait
// for these loads too).
__device__ __forceinline__ void load_codes_slice(F8Codes& cd, const AttnArgs& a,
                                                 const unsigned char* pool, int32_t sp, int tb,
                                                 int hi, int wave, int lane) {
  const bool ok = sp >= 0 && sp < a.num_subpages;
  const int t0 = tb + 16 * wave;
  const int nvalid = ok ? min(max(hi - t0, 0), 16) : 0;
  const unsigned char* base =
      pool + (((int64_t)(ok ? sp : 0) << a.page_shift) + (t0 & (a.page_size - 1))) * kHeadDim;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned char*>(base), (short)0, nvalid * kHeadDim, kBufferRsrcWord3);
#pragma unroll
  for (int j = 0; j < kF8Loads; ++j) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, 1024 * j + 16 * lane, 0, 0);
    cd.v[j] = make_uint4(v[0], v[1], v[2], v[3]);
  }
}
// Smaller sub-pages: one table entry per token (plain loads; tokens past the
// segment end read the zero row).
__device__ __forceinline__ void load_codes_pages(F8Codes& cd, const AttnArgs& a,
                                                 const unsigned char* pool,
                                                 const int32_t* pt_row, int tb, int hi, int wave,
                                                 int lane, const unsigned char* zero) {
#pragma unroll
  for (int j = 0; j < kF8Loads; ++j) {
    const int o = 1024 * j + 16 * lane;
    const int t = o / kHeadDim;
    const int tok = tb + 16 * wave + t;
    const int32_t sp = subpage_always(a, pt_row, tok, hi);
    const unsigned char* src = token_src<kHeadDim>(a, pool, sp, tok, hi, zero);
    cd.v[j] = *reinterpret_cast<const uint4*>(src + (o - t * kHeadDim));
  }
}

// Widen the codes of load j and write them into tile buffer `buf`: 16 codes
// = dims cpos .. cpos + 15 of one token = two 16-byte bf16 chunks.
template <bool E5M2>
__device__ __forceinline__ void write_chunk(const F8Codes& cd, int j, unsigned char* buf,
                                            int wave, int lane) {
  static_assert(kF8Loads == 9, "chunk indices 0..8");
  {
    const int o = 1024 * j + 16 * lane;
    const int t = o / kHeadDim;
    const int cpos = o - t * kHeadDim;
    const int row = 16 * wave + t;
    const uint4 w0 = fp8x8_to_bf16<E5M2>(cd.v[j].x, cd.v[j].y);
    const uint4 w1 = fp8x8_to_bf16<E5M2>(cd.v[j].z, cd.v[j].w);
    // latent: chunks cpos/8, cpos/8 + 1 of the row; rope: swizzled slots
    const int cc = (cpos - kVDim) / 8;
    const bool lat = cpos < kVDim;
    const int d0 =
        lat ? lat_off(row, cpos / 8) : kLatBytes + row * kRopeRow + 16 * (cc ^ rope_key(row));
    const int d1 =
        lat ? d0 + 16 : kLatBytes + row * kRopeRow + 16 * ((cc + 1) ^ rope_key(row));
    *reinterpret_cast<uint4*>(buf + d0) = w0;
    *reinterpret_cast<uint4*>(buf + d1) = w1;
  }
}
template <bool E5M2>
__device__ __forceinline__ void write_codes(const F8Codes& cd, unsigned char* buf, int wave,
                                            int lane) {
#pragma unroll
  for (int j = 0; j < kF8Loads; ++j) write_chunk<E5M2>(cd, j, buf, wave, lane);
}

template <bool SLICE, bool E5M2>
__global__ void __launch_bounds__(kThreads, 1) attn_fp8_kernel(AttnArgs a) {
  __shared__ __align__(16) unsigned char buf0[kBufBytes];
  __shared__ __align__(16) unsigned char buf1[kBufBytes];
  __shared__ PExchange px;
  __shared__ RowExchange rx;
  WorkUnit u = decode_head(a, blockIdx.x);
  if (!u.valid) return;
  poison_uncovered(a, u, threadIdx.x >> 6, threadIdx.x & 63);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = wave >> 1;                  // row group: 32 rows
  const int c = wave & 1;                   // token half (QK) / latent half (PV)

  const unsigned char* pool = a.kv + (int64_t)u.r * a.pool_tokens * kHeadDim;
  const unsigned char* zero = zero_row();
  const int32_t* pt_row = a.page_table + ((int64_t)u.r * a.R + u.last) * a.pt_width;

  // ---- the group's length and, for a first segment, its first sub-pages:
  // two loads in flight together, before any bulk data
  int32_t vpg = 0;                          // SLICE: sub-pages of tiles 64q .. 64q + 63
  if constexpr (SLICE) {
    if (u.s == 0 && a.pt_width > 0) vpg = first_slice_pages(a, pt_row, wave, lane);
  }
  decode_tail(a, u);
  const int lo = u.lo, hi = u.hi;
  if (lo >= hi) {                           // no token of the group to read
    store_empty(a, u, wave, lane);
    return;
  }

  // ---- Q (through the second tile buffer, as in the bf16 kernel) and the
  // first tile's codes, widened into the first buffer
  issue_q_tile(a, u, buf1, wave, lane, zero);
  F8Codes cd;
  if constexpr (SLICE) {
    if (u.s != 0) vpg = f8_slice_pages(a, pt_row, lo, hi, wave, lane);
    load_codes_slice(cd, a, pool, __builtin_amdgcn_readlane(vpg, 0), lo, hi, wave, lane);
  } else {
    load_codes_pages(cd, a, pool, pt_row, lo, hi, wave, lane, zero);
  }
  int mrow, hi_row;
  bool row_ok;
  lane_row(a, u, g, lane, mrow, hi_row, row_ok);
  const bool idle = u.m0 + 32 * g >= u.M;   // no row of this row group in the block
  WaveState st;
  state_init(st);
  write_codes<E5M2>(cd, buf0, wave, lane);
  MLA_WAIT_VMCNT(0);                        // the direct loads of Q
  lds_barrier();
  bf16x8 qf[kQSteps];
  read_q(buf1, g, lane, qf);

  // One tile (index kt from the segment start): wait until `cur` holds it,
  // fetch the next tile's codes, compute on `cur`, then widen the codes into
  // `nxt` (their loads had the whole computation to land; measured faster
  // than widening them piecewise during the PV product, 437 vs 456 us on
  // the fp8 verify workload).
  auto step = [&](const unsigned char* cur, unsigned char* nxt, int tb, int kt) {
    const bool more = tb + kTile < hi;
    lds_barrier();                          // `cur` is written; `nxt` is no longer read
    if (more) {
      if constexpr (SLICE) {
        const int nk = kt + 1;
        if ((nk & 63) == 0) vpg = f8_slice_pages(a, pt_row, lo + nk * kTile, hi, wave, lane);
        load_codes_slice(cd, a, pool, __builtin_amdgcn_readlane(vpg, nk & 63), tb + kTile, hi,
                         wave, lane);
      } else {
        load_codes_pages(cd, a, pool, pt_row, tb + kTile, hi, wave, lane, zero);
      }
    }
    if (idle)
      idle_tile([](int) {});
    else
      compute_tile(cur, &px, qf, st, tb, hi_row, a.qk_scale_log2, g, c, lane, [](int) {});
    if (more) write_codes<E5M2>(cd, nxt, wave, lane);
  };
  int kt = 0;
  for (int tb = lo; tb < hi; tb += 2 * kTile, kt += 2) {
    step(buf0, buf1, tb, kt);
    if (tb + kTile >= hi) break;
    step(buf1, buf0, tb + kTile, kt + 1);
  }

  store_partials(a, u, st, rx, g == 0 ? buf0 : buf1, mrow, row_ok, g, c, lane);
}

}  // namespace

hipError_t launch_attn_fp8(const AttnArgs& a, int64_t blocks, hipStream_t s) {
  const bool slice = a.page_size >= 16;
  if (a.e5m2) {
    if (slice) attn_fp8_kernel<true, true><<<(unsigned)blocks, kThreads, 0, s>>>(a);
    else attn_fp8_kernel<false, true><<<(unsigned)blocks, kThreads, 0, s>>>(a);
  } else {
    if (slice) attn_fp8_kernel<true, false><<<(unsigned)blocks, kThreads, 0, s>>>(a);
    else attn_fp8_kernel<false, false><<<(unsigned)blocks, kThreads, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace mla
