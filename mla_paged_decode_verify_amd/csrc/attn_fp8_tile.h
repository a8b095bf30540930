// fp8 KV tiles (OCP e4m3fn or e5m2 codes) for the attention kernels: the
// codes of a wave's 16 tokens of a 64-token tile are fetched into registers
// with ordinary vector loads, then widened exactly to bf16 (every e4m3fn and
// every e5m2 value is a bf16 value) and written into a bf16 tile buffer in
// the latent / rope layout of attn_common.h.
#pragma once

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

}  // namespace
}  // namespace mla
