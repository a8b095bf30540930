// Split-K segmented MLA attention partials, fp8 KV cache (OCP e4m3fn or e5m2
// codes).
//
// The quantities computed, the work decomposition and the per-tile
// computation are those of attn_common.h. Specific to this kernel:
//  * The fp8 codes of a 64-token tile (36,864 B, token-major, 576 B per
//    token) go straight from HBM to LDS with direct loads into a ring of two
//    staging tiles; each wave loads the 16 tokens 16w .. 16w + 15 with nine
//    1 KB instructions. While tile k is computed, tiles k+1 and k+2 are in
//    flight.
//  * Between two tiles the workgroup widens the next staged tile exactly to
//    bf16 into the tile buffer the shared computation reads (every e4m3fn and
//    every e5m2 value is a bf16 value), in the latent / rope layout of
//    attn_common.h.
//  * The fp8 scale is folded into the score scale and into the output.
// LDS: two staging tiles (73,728 B) + the bf16 tile buffer (75,776 B, which
// first stages Q) + the exchange areas.
#include "attn_common.h"

namespace mla {
namespace {

constexpr int kF8Tile = kTile * kHeadDim;    // 36,864 B of codes per tile
constexpr int kF8Loads = kF8Tile / 1024 / 4; // 9 direct 1 KB loads per wave per tile
static_assert(kF8Loads * 1024 == 16 * kHeadDim, "a wave's loads cover exactly 16 tokens");

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
// 8 codes (a uint2) to 8 bf16 values (a uint4). Exact: every e4m3fn and every
// e5m2 value is a bf16 value (bf16 has more exponent and mantissa bits).
template <bool E5M2>
__device__ __forceinline__ uint4 fp8x8_to_bf16(uint2 in) {
  return make_uint4(cvt2<E5M2>(in.x, false), cvt2<E5M2>(in.x, true), cvt2<E5M2>(in.y, false),
                    cvt2<E5M2>(in.y, true));
}

// Sources of one wave's 16 tokens of a tile. Sub-pages of 16+ tokens: the
// 16 tokens are contiguous in the pool (one base address, `nvalid` before the
// segment end). Smaller sub-pages: one entry per token, looked up per load.
struct F8Slice {
  const unsigned char* base;
  int nvalid;
};

// Load j (0..8) of this wave: staging bytes [9216 w + 1024 j, + 1024) of the
// tile, i.e. byte o = 1024 j + 16 l of the wave's 16 tokens in lane l (a
// lane's 16 bytes never straddle two tokens: 576 = 36 * 16).
__device__ __forceinline__ void issue_f8_slice(const F8Slice& v, const unsigned char* zero,
                                               unsigned char* stage, int wave, int lane, int j) {
  const int o = 1024 * j + 16 * lane;
  const int t = o / kHeadDim;
  const unsigned char* src = t < v.nvalid ? v.base + o : zero + (o - t * kHeadDim);
  dma16(src, stage + 16 * kHeadDim * wave + 1024 * j);
}
__device__ __forceinline__ void issue_f8_pages(const AttnArgs& a, const unsigned char* pool,
                                               const int32_t* pt_row, int tb, int hi,
                                               const unsigned char* zero, unsigned char* stage,
                                               int wave, int lane, int j) {
  const int o = 1024 * j + 16 * lane;
  const int t = o / kHeadDim;
  const int tok = tb + 16 * wave + t;
  const int32_t sp = subpage_always(a, pt_row, tok, hi);
  const unsigned char* src = token_src<kHeadDim>(a, pool, sp, tok, hi, zero);
  dma16(src + (o - t * kHeadDim), stage + 16 * kHeadDim * wave + 1024 * j);
}

// Sub-pages of 64 consecutive tiles for one wave: lane j holds the sub-page
// of tokens tb0 + 64 j + 16 w .. +15 (clamped to the last in-range token).
__device__ __forceinline__ int32_t f8_slice_pages(const AttnArgs& a, const int32_t* pt_row,
                                                  int tb0, int hi, int wave, int lane) {
  const int64_t tok = min((int64_t)tb0 + (int64_t)kTile * lane + 16 * wave, (int64_t)hi - 1);
  return pt_row[tok >> a.page_shift];
}

// Widen a staged tile into the bf16 tile buffer, 8 codes (one 16-byte bf16
// chunk h: dims 8h .. 8h + 7) per lane and pass. The 16 lanes of group G
// (G = tid / 16) take tokens 8 (G % 8) + 0..7 and the chunk pair
// 2b, 2b + 1 with b = 2i + G / 8 in pass i (i = 0..17): their 16-byte
// writes then fall on 16 distinct 4-bank groups of the latent rows (row
// stride 264 dwords) and of the swizzled rope rows, so no store conflicts;
// the 8-byte reads of the staged codes conflict at most two ways.
template <bool E5M2>
__device__ __forceinline__ void widen_tile(const unsigned char* stage, unsigned char* buf,
                                           int tid) {
  const int G = tid >> 4;
  const int tok = 8 * (G & 7) + (tid & 7);
  const int bit = (tid >> 3) & 1;
  const unsigned char* src = stage + tok * kHeadDim + 8 * bit;
  unsigned char* lat = buf + tok * kLatRow;
  unsigned char* rope = buf + kLatBytes + tok * kRopeRow;
#pragma unroll
  for (int i0 = 0; i0 < 18; i0 += 6) {
    uint2 in[6];
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      const int h0 = 2 * (2 * (i0 + i) + (G >> 3));   // even chunk of the pair
      in[i] = *reinterpret_cast<const uint2*>(src + 8 * h0);
    }
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      const int h = 2 * (2 * (i0 + i) + (G >> 3)) + bit;
      const uint4 w = fp8x8_to_bf16<E5M2>(in[i]);
      if (h < kVDim / 8)
        *reinterpret_cast<uint4*>(lat + 16 * (h ^ lat_swz(tok))) = w;
      else
        *reinterpret_cast<uint4*>(rope + 16 * ((h - kVDim / 8) ^ (tok & 7))) = w;
    }
  }
}

template <bool SLICE, bool E5M2>
__global__ void __launch_bounds__(kThreads, 1) attn_fp8_kernel(AttnArgs a) {
  __shared__ __align__(16) unsigned char stage[2 * kF8Tile];  // staging tiles 0, 1
  __shared__ __align__(16) unsigned char buf[kBufBytes];
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
  const int ntiles = (hi - lo + kTile - 1) / kTile;

  // ---- Q, staged in the tile buffer
  issue_q_tile(a, u, buf, wave, lane, zero);

  auto issue_tile = [&](int t) {
    unsigned char* st = stage + (t & 1) * kF8Tile;
    const int tb = lo + t * kTile;
    if constexpr (SLICE) {
      if ((t & 63) == 0 && (t != 0 || u.s != 0)) vpg = f8_slice_pages(a, pt_row, tb, hi, wave, lane);
      const int32_t sp = __builtin_amdgcn_readlane(vpg, t & 63);
      F8Slice v;
      const bool ok = sp >= 0 && sp < a.num_subpages;
      const int t0 = tb + 16 * wave;
      v.nvalid = ok ? min(max(hi - t0, 0), 16) : 0;
      v.base = pool + (((int64_t)(ok ? sp : 0) << a.page_shift) + (t0 & (a.page_size - 1))) *
                          kHeadDim;
#pragma unroll
      for (int j = 0; j < kF8Loads; ++j) issue_f8_slice(v, zero, st, wave, lane, j);
    } else {
#pragma unroll
      for (int j = 0; j < kF8Loads; ++j)
        issue_f8_pages(a, pool, pt_row, tb, hi, zero, st, wave, lane, j);
    }
  };

  // ---- tiles 0 and 1 in flight with Q; Q into registers; tile 0 widened
  issue_tile(0);
  if (ntiles > 1) issue_tile(1);
  int mrow, hi_row;
  bool row_ok;
  lane_row(a, u, g, lane, mrow, hi_row, row_ok);
  const bool idle = u.m0 + 32 * g >= u.M;   // no row of this row group in the block
  WaveState st;
  state_init(st);
  MLA_WAIT_VMCNT(0);
  lds_barrier();
  bf16x8 qf[kQSteps];
  read_q(buf, g, lane, qf);
  lds_barrier();                            // every wave holds its Q: the buffer is free
  widen_tile<E5M2>(stage, buf, tid);
  lds_barrier();                            // tile 0 in the buffer; staging tile 0 is free
  if (ntiles > 2) issue_tile(2);

  for (int k = 0; k < ntiles; ++k) {
    if (idle)
      idle_tile([](int) {});
    else
      compute_tile(buf, &px, qf, st, lo + k * kTile, hi_row, a.qk_scale_log2, g, c, lane,
                   [](int) {});
    if (k + 1 < ntiles) {
      // tile k + 1 has landed (this wave's later loads: tile k + 2's nine)
      if (k + 2 < ntiles) MLA_WAIT_VMCNT(kF8Loads); else MLA_WAIT_VMCNT(0);
      lds_barrier();                        // ... for every wave; the buffer is no longer read
      widen_tile<E5M2>(stage + ((k + 1) & 1) * kF8Tile, buf, tid);
      lds_barrier();                        // tile k + 1 in the buffer; its staging tile is free
      if (k + 3 < ntiles) issue_tile(k + 3);
    }
  }

  // row group 0 stages its O in the tile buffer, row group 1 in the staging tiles
  store_partials(a, u, st, rx, g == 0 ? buf : stage, mrow, row_ok, g, c, lane);
}

static_assert(2 * kF8Tile >= 32 * kStageRow, "a row group's O fits the two staging tiles");

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
