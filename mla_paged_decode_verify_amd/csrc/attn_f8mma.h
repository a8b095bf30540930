// fp8 KV tiles computed on the fp8 matrix cores (gfx950
// v_mfma_scale_f32_32x32x64_f8f6f4): the KV codes go from HBM into LDS as they
// are (576 bytes per token, half a bf16 tile) and feed both products without
// being widened.
//
// The quantities are those of attn_common.h; only the operand formats differ:
//  * S^T = K Q^T with K the e4m3fn / e5m2 codes and Q as two e4m3fn terms per
//    element, Q = 2^-a (hi + 2^-4 lo), a per row such that 2^a max|q| lies in
//    [128, 256). A bf16 value has 8 significant bits and hi keeps the top 4
//    (nearest even), so the residual needs at most 4 more: lo is exact and
//    the two terms give q exactly for every element at least 2^-13 of the
//    row's largest; a smaller one's residual can fall under e4m3fn's
//    subnormal spacing, an error below 2^-21 of the row's largest. The per-row factors are
//    the B operand's block scales (E8M0) of the scaled MFMA, so both terms
//    accumulate into one fp32 accumulator.
//  * O^T += V^T P^T with V the latent codes and P as two e4m3fn terms,
//    P = hi + 2^-4 lo (P <= 256 < 448 by the lazy reference): the same
//    2^-8 relative error per weight as bf16 weights would have, except that
//    weights below about 2^-14 of the reference (which contribute less than
//    that to a row sum of at least 1) are lost to the subnormal range.
//
// MFMA operand lanes (h = l / 32), checked on the device: lane l of A holds
// row l % 32 and lane l of B column l % 32; their 32 bytes are the K-elements
// of half h, byte j of A pairing with byte j of B, so any order of the 64
// K-elements serves as long as A and B use the same one. The D layout is
// that of the 32x32 bf16 form (value j of lane l: D[8(j/4) + 4h + j%4][l%32]),
// so the accumulation state and its stores are those of attn_common.h.
//
// LDS tile: 64 tokens x 576 bytes, no padding; the 16-byte chunk c (dims
// 16c .. 16c+15) of token t sits in slot c ^ ((t >> 2) & 3), so the 16 rows
// that a K-fragment read or a transposed V read touches at once fall on
// different banks.
#pragma once

#include "attn_common.h"

namespace mla {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr int kF8Tile = kTile * kHeadDim;     // 36864 bytes
constexpr int kF8Steps = kHeadDim / 64;       // 9 K-steps of 64 dims for QK^T
constexpr int kF8Dma = 16 * kHeadDim / 1024;  // 9 direct loads per wave per tile
constexpr int kE8M0One = 127;                 // block scale 2^0
constexpr int kLoShift = 4;                   // lo terms carry the residual times 2^4
static_assert(kF8Dma * 1024 == 16 * kHeadDim, "a wave's loads cover exactly 16 tokens");
static_assert(4 * kF8Tile <= 2 * kBufBytes, "four fp8 tiles fit the two tile buffers");

__device__ __forceinline__ int f8_swz(int t) { return (t >> 2) & 3; }
// Byte offset of chunk c (dims 16c .. 16c + 15) of token t in an fp8 tile.
__device__ __forceinline__ int f8_off(int t, int c) { return t * kHeadDim + 16 * (c ^ f8_swz(t)); }

// Tile slot k of the four in the two tile buffers.
__device__ __forceinline__ unsigned char* f8_slot(unsigned char* buf0, unsigned char* buf1, int k) {
  return ((k & 2) ? buf1 : buf0) + (k & 1) * kF8Tile;
}

// Buffer-resource word 3 of the gfx9 family (gfx950 included): raw buffer
// access with no format conversion.
constexpr int kBufferRsrcWord3 = 0x00020000;

// Buffer resource of a wave's 16 tokens t0 .. t0 + 15 of a tile, which lie in
// one sub-page `sp`: its records end at the segment end `hi` (none for a
// sub-page id outside the pool), and loads past the records return zeros, so
// the tokens there come in as zero codes (+0 in both fp8 formats). All of it
// is uniform across the wave, so the resource sits in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t f8_slice_rsrc(const AttnArgs& a,
                                                                const unsigned char* pool,
                                                                int32_t sp, int t0, int hi) {
  const bool ok = sp >= 0 && sp < a.num_subpages;
  const int nvalid = ok ? min(max(hi - t0, 0), 16) : 0;
  const int64_t t = ((int64_t)(ok ? sp : 0) << a.page_shift) + (t0 & (a.page_size - 1));
  // the operands are uniform; readfirstlane tells the compiler so
  const uint64_t base = (uint64_t)(uintptr_t)(pool + t * kHeadDim);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
  const uint32_t hi32 = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
  unsigned char* p = reinterpret_cast<unsigned char*>((uintptr_t)(((uint64_t)hi32 << 32) | lo));
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0,
                                           __builtin_amdgcn_readfirstlane(nvalid * kHeadDim),
                                           kBufferRsrcWord3);
}

// Source offset, within its 16-token slice, of lane l's 16 bytes of direct
// load j (0..8): they land at byte 1024 j + 16 l of the wave's 9216 bytes of
// the tile, i.e. token t = (1024 j + 16 l) / 576 of the slice and the slot
// that holds chunk slot ^ f8_swz(t) (the same for every wave: 16 w is a
// multiple of 4).
__device__ __forceinline__ int f8_src_off(int lane, int j) {
  const int p = 1024 * j + 16 * lane;
  const int tl = p / kHeadDim;
  const int slot = (p - tl * kHeadDim) >> 4;
  return tl * kHeadDim + 16 * (slot ^ f8_swz(tl));
}

// One direct buffer -> LDS load: each lane's 16 bytes at record offset `voff`
// land at lds + 16 * lane (inline assembly for the same reason as dma16: the
// kernels order these loads themselves).
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t r, int voff,
                                          const unsigned char* lds) {
  const uint32_t base = (uint32_t)(uintptr_t)(const lds_void*)lds;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(r), "s"(base)
               : "m0");
}

// Direct load j (0..8) of this wave's 16 tokens of a tile into `dst`.
__device__ __forceinline__ void issue_f8_slice(__amdgpu_buffer_rsrc_t r, unsigned char* dst,
                                               int wave, int lane, int j) {
  dma16_buf(r, f8_src_off(lane, j), dst + 16 * kHeadDim * wave + 1024 * j);
}
// The same for sub-pages of fewer than 16 tokens: one table entry per token.
__device__ __forceinline__ void issue_f8_pages(const AttnArgs& a, const unsigned char* pool,
                                               const int32_t* pt_row, int tb, int hi,
                                               unsigned char* dst, int wave, int lane, int j,
                                               const unsigned char* zero) {
  const int p = 1024 * j + 16 * lane;
  const int tl = p / kHeadDim;
  const int slot = (p - tl * kHeadDim) >> 4;
  const int row = 16 * wave + tl;
  const int tok = tb + row;
  const int32_t sp = subpage_always(a, pt_row, tok, hi);
  const unsigned char* src = token_src<kHeadDim>(a, pool, sp, tok, hi, zero);
  dma16(src + 16 * (slot ^ f8_swz(row)), dst + 16 * kHeadDim * wave + 1024 * j);
}

// Q of this lane's row as the B operand of the QK product: K-step s holds
// dims 64s + 32h .. + 31 (byte e = dim 64s + 32h + e), as hi and lo terms,
// with the row's block scales.
struct QF8 {
  i32x8 hi[kF8Steps];
  i32x8 lo[kF8Steps];
  int sc_hi, sc_lo;
};

// Row 32g + l % 32 of the staged bf16 Q tile (attn_common.h layout): bf16
// chunk e (dims 8e .. 8e + 7) of the dims of K-step s for half h.
__device__ __forceinline__ const unsigned char* q_chunk(const unsigned char* qtile, int row, int h,
                                                       int s, int e) {
  return s < kF8Steps - 1 ? qtile + lat_off(row, 8 * s + 4 * h + e)
                          : qtile + kLatBytes + row * kRopeRow + 16 * ((4 * h + e) ^ rope_key(row));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two values to two e4m3fn codes in byte pair `sel` of `w` (nearest even).
__device__ __forceinline__ int pk_e4m3(float x, float y, int w, bool sel) {
  return sel ? __builtin_amdgcn_cvt_pk_fp8_f32(x, y, w, true)
             : __builtin_amdgcn_cvt_pk_fp8_f32(x, y, w, false);
}
__device__ __forceinline__ f32x2 unpk_e4m3(int w, bool sel) {
  return sel ? __builtin_amdgcn_cvt_pk_f32_fp8(w, true) : __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
}

// 8 values (x[0..7], already scaled) to hi and lo codes: two words each.
__device__ __forceinline__ void split8(const float (&x)[8], int& h0, int& h1, int& l0, int& l1) {
  h0 = pk_e4m3(x[0], x[1], 0, false);
  h0 = pk_e4m3(x[2], x[3], h0, true);
  h1 = pk_e4m3(x[4], x[5], 0, false);
  h1 = pk_e4m3(x[6], x[7], h1, true);
  float r[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const f32x2 b = unpk_e4m3(k < 2 ? h0 : h1, (k & 1) != 0);
    r[2 * k] = (x[2 * k] - b[0]) * (float)(1 << kLoShift);
    r[2 * k + 1] = (x[2 * k + 1] - b[1]) * (float)(1 << kLoShift);
  }
  l0 = pk_e4m3(r[0], r[1], 0, false);
  l0 = pk_e4m3(r[2], r[3], l0, true);
  l1 = pk_e4m3(r[4], r[5], 0, false);
  l1 = pk_e4m3(r[6], r[7], l1, true);
}

__device__ inline void read_q_f8(const unsigned char* qtile, int g, int lane, QF8& q) {
  const int h = lane >> 5;
  const int row = 32 * g + (lane & 31);
  // largest |q| of the row (this lane's 288 dims, then its partner lane's)
  uint32_t amax = 0;
#pragma unroll
  for (int s = 0; s < kF8Steps; ++s) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint4 w = *reinterpret_cast<const uint4*>(q_chunk(qtile, row, h, s, e));
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int k = 0; k < 4; ++k)
        amax = max(amax, max((ws[k] << 16) & 0x7FFF0000u, ws[k] & 0x7FFF0000u));
    }
  }
  {
    auto p = __builtin_amdgcn_permlane32_swap(amax, amax, false, false);
    amax = max(p[0], p[1]);
  }
  // 2^a max|q| in [2^7, 2^8): a = 7 - exponent(max|q|), kept where the scales
  // stay valid E8M0 codes (an all-zero row gets the largest a)
  const int ex = (int)(amax >> 23) - 127;
  const int a = min(max(7 - ex, -120), 100);
  q.sc_hi = kE8M0One - a;
  q.sc_lo = kE8M0One - a - kLoShift;
#pragma unroll
  for (int s = 0; s < kF8Steps; ++s) {
    int hw[8], lw[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint4 w = *reinterpret_cast<const uint4*>(q_chunk(qtile, row, h, s, e));
      float x[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                    bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = __builtin_ldexpf(x[k], a);
      split8(x, hw[2 * e], hw[2 * e + 1], lw[2 * e], lw[2 * e + 1]);
    }
    q.hi[s] = i32x8{hw[0], hw[1], hw[2], hw[3], hw[4], hw[5], hw[6], hw[7]};
    q.lo[s] = i32x8{lw[0], lw[1], lw[2], lw[3], lw[4], lw[5], lw[6], lw[7]};
  }
  // kept in accumulation registers, which the MFMAs read directly (left to
  // itself the compiler parks them there and copies them back before use)
#pragma unroll
  for (int s = 0; s < kF8Steps; ++s) asm volatile("" : "+a"(q.hi[s]), "+a"(q.lo[s]));
}

template <bool E5M2>
__device__ __forceinline__ f32x16 mfma_f8(const i32x8& a, const i32x8& b, const f32x16& c,
                                          int scale_b) {
  // A: KV codes (e4m3fn, or e5m2), B: e4m3fn terms
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, E5M2 ? 1 : 0, 0, 0, kE8M0One,
                                                          0, scale_b);
}

// K fragment (A operand of S^T = K Q^T) of K-step s: lane l reads token
// 32c + l % 32 of `tile`, dims 64s + 32h .. + 31 (two 16-byte chunks).
__device__ __forceinline__ i32x8 kfrag_f8(const unsigned char* tile, int tok, int h, int s) {
  const uint4 x0 = *reinterpret_cast<const uint4*>(tile + f8_off(tok, 4 * s + 2 * h));
  const uint4 x1 = *reinterpret_cast<const uint4*>(tile + f8_off(tok, 4 * s + 2 * h + 1));
  return i32x8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
               (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
}

// V^T fragment (A operand of O^T += V^T P^T) of output tile t: dims
// 256c + 32t + l % 32 over the 64 tokens in the B operand's order -- bytes
// 0..15 the wave's own tokens 32c + 8(j/4) + 4h + j%4, bytes 16..31 the
// partner's (32(c^1) + ...). Transposed 8-bit read r covers bytes 8r .. 8r+7:
// in each 16-lane group, lane 2k + b points at 8 dims (b: the upper 8 of the
// group's 16) of token T_k and hands out one dim of 8 tokens.
__device__ __forceinline__ i32x8 vfrag_f8(const unsigned char* tile, int c, int lane, int t) {
  const int h = lane >> 5;
  const int G = (lane >> 4) & 1;
  const int kk = (lane & 15) >> 1;
  const int b8 = lane & 1;
  i32x2 r4[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int half = r < 2 ? c : (c ^ 1);
    const int T = 32 * half + 16 * (r & 1) + 8 * (kk >> 2) + 4 * h + (kk & 3);
    r4[r] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (lds_i32x2*)(tile + f8_off(T, 16 * c + 2 * t + G) + 8 * b8));
  }
  return i32x8{r4[0][0], r4[0][1], r4[1][0], r4[1][1], r4[2][0], r4[2][1], r4[3][0], r4[3][1]};
}

// S^T[32 tokens x 32 rows] of one tile (the first of a segment): 9 K-steps,
// hi and lo terms of Q into one accumulator.
template <bool E5M2>
__device__ __forceinline__ void qk_f8(const unsigned char* __restrict__ tile, const QF8& q,
                                      f32x16& sacc, int c, int lane) {
  const int tok = 32 * c + (lane & 31), h = lane >> 5;
  sacc = f32x16{};
  i32x8 kr[2];
  kr[0] = kfrag_f8(tile, tok, h, 0);
#pragma unroll
  for (int s = 0; s < kF8Steps; ++s) {
    if (s + 1 < kF8Steps) kr[(s + 1) & 1] = kfrag_f8(tile, tok, h, s + 1);
    __builtin_amdgcn_sched_barrier(0);
    sacc = mfma_f8<E5M2>(kr[s & 1], q.hi[s], sacc, q.sc_hi);
    sacc = mfma_f8<E5M2>(kr[s & 1], q.lo[s], sacc, q.sc_lo);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One step of the tile pipeline: softmax and PV of tile `cur`, whose scores
// `sacc` the previous step computed, interleaved with the QK product of the
// next tile `nxt` (its scores replace `sacc`). The matrix cores work on the
// next tile's QK while the wave computes this tile's maxima and weights
// between its MFMAs, then on this tile's PV. On a segment's last tile `nxt`
// is any tile slot: its scores are not used. `issue(s)` is called once per
// QK K-step (s = 0..8), so that the loads of a later tile can be spread over
// the MFMA work.
template <bool E5M2, class Issue>
__device__ __forceinline__ void step_f8(const unsigned char* __restrict__ cur,
                                        const unsigned char* __restrict__ nxt, f32x16& sacc,
                                        PExchange* __restrict__ px, const QF8& q, WaveState& st,
                                        int tb, int hi_row, float qk_scale_log2, int g, int c,
                                        int lane, Issue&& issue) {
  const int h = lane >> 5;
  const int n32 = lane & 31;
  const int tok = 32 * c + n32;

  f32x16 sc = sacc;                         // this tile's scores
  float m = 0.f;
  int ph[4], pl[4];
  i32x8 bh, bl, v0;

  // ---- this tile's softmax, in pieces placed between the next tile's QK
  // MFMAs (piece i after MFMA i)
  auto piece = [&](int i) {
    if (i == 0) {
      // mask and maximum (both waves of the row group see the same tile max)
      if (__builtin_amdgcn_ballot_w64(tb + kTile > hi_row) != 0) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int t = tb + 32 * c + 8 * (j >> 2) + 4 * h + (j & 3);
          if (t >= hi_row) sc[j] = kNegInf;
        }
      }
      m = sc[0];
#pragma unroll
      for (int j = 1; j < 16; ++j) m = fmaxf(m, sc[j]);
      auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false,
                                                false);
      m = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
    } else if (i == 1) {
      if (h == 0) px->mx[g][c][n32] = m;
      v0 = vfrag_f8(cur, c, lane, 0);
    } else if (i == 3) {
      lds_barrier();
      m = fmaxf(m, px->mx[g][c ^ 1][n32]) * qk_scale_log2;
      st.m_true = fmaxf(st.m_true, m);
      // lazily refreshed reference (identical decisions on both waves)
      const bool refresh = m > st.m_ref + kRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(refresh) != 0) {
        const float alpha = refresh ? __builtin_amdgcn_exp2f(st.m_ref - m) : 1.f;
        st.l_part *= alpha;
#pragma unroll
        for (int t = 0; t < kOTiles; ++t) st.o[t] *= alpha;
        st.m_ref = refresh ? m : st.m_ref;
      }
    } else if (i >= 4 && i < 8) {
      // P of this wave's tokens as hi / lo e4m3fn terms, one word each
      const int w = i - 4;
      const float m_use = st.m_ref == kNegInf ? 0.f : st.m_ref;
      float x[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        // masked: the score is -inf and exp2(-inf) = 0 (m_use is finite)
        x[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[4 * w + k], qk_scale_log2, -m_use));
        st.l_part += x[k];
      }
      int hw = pk_e4m3(x[0], x[1], 0, false);
      hw = pk_e4m3(x[2], x[3], hw, true);
      const f32x2 b0 = unpk_e4m3(hw, false), b1 = unpk_e4m3(hw, true);
      const float f = (float)(1 << kLoShift);
      int lw = pk_e4m3((x[0] - b0[0]) * f, (x[1] - b0[1]) * f, 0, false);
      lw = pk_e4m3((x[2] - b1[0]) * f, (x[3] - b1[1]) * f, lw, true);
      asm volatile("" : "+v"(hw), "+v"(lw), "+v"(st.l_part));   // keeps the pieces apart
      ph[w] = hw;
      pl[w] = lw;
    } else if (i == 8) {
      px->p[g][c][0][lane] = make_uint4(ph[0], ph[1], ph[2], ph[3]);
      px->p[g][c][1][lane] = make_uint4(pl[0], pl[1], pl[2], pl[3]);
    } else if (i == 11) {
      lds_barrier();
      const uint4 oh = px->p[g][c ^ 1][0][lane];
      const uint4 ol = px->p[g][c ^ 1][1][lane];
      bh = i32x8{ph[0], ph[1], ph[2], ph[3], (int)oh.x, (int)oh.y, (int)oh.z, (int)oh.w};
      bl = i32x8{pl[0], pl[1], pl[2], pl[3], (int)ol.x, (int)ol.y, (int)ol.z, (int)ol.w};
    }
  };

  // ---- the next tile's S^T, with the pieces between its MFMAs
  f32x16 sn = f32x16{};
  i32x8 kr[2];
  kr[0] = kfrag_f8(nxt, tok, h, 0);
#pragma unroll
  for (int s = 0; s < kF8Steps; ++s) {
    if (s + 1 < kF8Steps) kr[(s + 1) & 1] = kfrag_f8(nxt, tok, h, s + 1);
    issue(s);
    __builtin_amdgcn_sched_barrier(0);
    sn = mfma_f8<E5M2>(kr[s & 1], q.hi[s], sn, q.sc_hi);
    // pinned here: left alone, the compiler sinks the MFMAs, whose results
    // are used only after the loop, below all the pieces
    asm volatile("" : "+v"(sn));
    __builtin_amdgcn_sched_barrier(0);
    piece(2 * s);
    __builtin_amdgcn_sched_barrier(0);
    sn = mfma_f8<E5M2>(kr[s & 1], q.lo[s], sn, q.sc_lo);
    asm volatile("" : "+v"(sn));
    __builtin_amdgcn_sched_barrier(0);
    piece(2 * s + 1);
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- O^T[256 dims x 32 rows] += V^T[256 x 64 tokens] P^T[64 x 32]
  i32x8 vr[2];
  vr[0] = v0;
#pragma unroll
  for (int t = 0; t < kOTiles; ++t) {
    if (t + 1 < kOTiles) vr[(t + 1) & 1] = vfrag_f8(cur, c, lane, t + 1);
    __builtin_amdgcn_sched_barrier(0);
    st.o[t] = mfma_f8<E5M2>(vr[t & 1], bh, st.o[t], kE8M0One);
    st.o[t] = mfma_f8<E5M2>(vr[t & 1], bl, st.o[t], kE8M0One - kLoShift);
    __builtin_amdgcn_sched_barrier(0);
  }
  sacc = sn;
}

// A tile for a wave whose row group holds no row of the block: its share of
// a later tile's loads and step_f8's two barriers.
template <class Issue>
__device__ __forceinline__ void idle_tile_f8(Issue&& issue) {
#pragma unroll
  for (int s = 0; s < kF8Steps; ++s) issue(s);
  lds_barrier();
  lds_barrier();
}

}  // namespace
}  // namespace mla
