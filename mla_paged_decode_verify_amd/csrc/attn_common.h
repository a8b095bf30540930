// Shared pieces of the attention kernels (gfx950, wave64): LDS tile layout,
// sources of KV tokens in the paged pool, the direct HBM -> LDS loads of bf16
// tiles, work-unit decoding and the Q fragments.
//
// What the kernels compute (vLLM PR #51705 digest, Implementation breakdown
// items 2-4 and the merge snippet): for every shard r, verify row rho, head h
// and split-K segment s, over the segment's local tokens that the row may see,
//   m2 = max(score * log2 e), e = sum 2^(score*log2e - m2),
//   O  = sum 2^(score*log2e - m2) * v,   score = sm_scale * <q, k> (576 dims),
// with v the 512 latent dims of the same cache entry (SGLang PR #34432 report,
// _forward_verify_dcp snippet). The partition follows the pages'
// tiles_per_segment = ceil(len / (segments * tile)) with len the group's
// longest row and tile = the sub-page size.
//
// One workgroup = 4 waves = one work unit (request i, shard r, segment s,
// 64-row block of the request's Q_i*H (row, head) pairs). All rows of a
// request share the shard's KV, so a KV tile is read from HBM once per block.
// LDS tile layout (64 tokens): latent rows of 512 bf16 in 1056-byte slots,
// row r starting 16 bytes into its slot when bit 3 of r is set, and rope
// [64][8 chunks of 16 B] with chunk c of token t in slot c ^ ((t >> 1) & 7).
// So the 16 rows that a K-fragment read touches at once (16 bytes each) fall
// on 16 different groups of 4 banks -- 1056-byte rows alone map rows r and
// r + 8 to the same banks -- and the same holds for the rope chunks; the
// offsets are per row, so a lane's fragment addresses stay one base plus
// constants.
#pragma once

#include "internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
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
constexpr int kQSteps = kHeadDim / 16;     // 36 MFMA K-steps (16 dims) for QK^T
constexpr int kLatQSteps = kVDim / 16;     // the first 32 read the latent region
constexpr int kOTiles = kVDim / 2 / 32;    // 8 output tiles of 32 latent dims per wave
constexpr int kTokBytesBf16 = kHeadDim * 2;
constexpr float kNegInf = -__builtin_inff();
constexpr float kRescaleSlack = 8.f;       // log2 units
constexpr float kLn2 = 0.693147180559945309f;

// Byte offset of latent row r in a tile, and of its 16-byte chunk c (dims
// 8c..8c+7); the 16-byte shift of rows 8..15 of every 16 stays inside the
// row's 32 bytes of padding.
__device__ __forceinline__ int lat_row(int r) { return r * kLatRow + (((r >> 3) & 1) << 4); }
__device__ __forceinline__ int lat_off(int r, int c) { return lat_row(r) + (c << 4); }
// Rope chunk c of token t sits in slot c ^ rope_key(t).
__device__ __forceinline__ int rope_key(int t) { return (t >> 1) & 7; }

// Source of tokens outside the segment: a row of zeros, so that masked
// positions hold finite values (0 * NaN would poison the PV product).
__device__ __align__(16) unsigned char g_zero_token[kTokBytesBf16];

// The zero row's address, materialised once into scalar registers (left to
// itself the compiler re-derives it through the GOT, with a scalar load and a
// full lgkmcnt wait, at every use).
__device__ __forceinline__ const unsigned char* zero_row() {
  const unsigned char* z = g_zero_token;
  asm volatile("" : "+s"(z));
  return z;
}

// Address of token `tok` with sub-page id `sp`, or the zero row when the token
// is past the segment end `hi` or sp is outside the pool.
template <int TOKB>
__device__ inline const unsigned char* token_src(const AttnArgs& a, const unsigned char* pool,
                                                 int32_t sp, int tok, int hi,
                                                 const unsigned char* zero) {
  if (tok >= hi || sp < 0 || sp >= a.num_subpages) return zero;
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

// One direct HBM -> LDS load: each lane's 16 bytes at `src` land at
// lds + 16 * lane. Written as inline assembly so that the compiler does not
// track the LDS write: it cannot tell that the loads in flight target the
// other tile buffer, and would otherwise wait for them before LDS accesses
// it cannot prove disjoint. The kernels order these loads themselves
// (s_waitcnt vmcnt + barrier before a buffer is read or refilled). M0 holds
// the LDS base; one wait state separates its write from the load.
__device__ __forceinline__ void dma16(const void* src, const unsigned char* lds) {
  const uint32_t base = (uint32_t)(uintptr_t)(const lds_void*)lds;
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(base)
               : "m0");
}

// bf16: direct HBM -> LDS load number j (0..17) of this wave for tile
// [tb, tb + 64) into `dst`: j < 16 is the latent part of token 16w + j (one
// 1 KB instruction), j = 16, 17 the rope parts of tokens 16w + 8(j-16) + 0..7.
__device__ __forceinline__ void issue_one_bf16(const AttnArgs& a, const unsigned char* pool,
                                               const Bf16Pages& pg, int tb, int hi,
                                               unsigned char* dst, int wave, int lane, int j,
                                               const unsigned char* zero) {
  if (j < 16) {
    const int row = 16 * wave + j;
    const int32_t sp = __builtin_amdgcn_readlane(pg.lat, j);
    const unsigned char* src = token_src<kTokBytesBf16>(a, pool, sp, tb + row, hi, zero);
    // slot `lane` of the row holds chunk lane ^ swz(row)
    dma16(src + 16 * lane, dst + lat_row(row));
  } else {
    const int jj = j - 16;
    const int u = lane >> 3;                // token within the 8-token group
    const int row = 16 * wave + 8 * jj + u;
    const int chunk = (lane & 7) ^ rope_key(row);   // slot (lane & 7) holds chunk ^ key
    const unsigned char* src =
        token_src<kTokBytesBf16>(a, pool, jj ? pg.rope1 : pg.rope0, tb + row, hi, zero);
    dma16(src + 2 * kVDim + 16 * chunk, dst + kLatBytes + (16 * wave + 8 * jj) * kRopeRow);
  }
}

// All 18 loads of this wave for one tile.
__device__ inline void issue_tile_bf16(const AttnArgs& a, const unsigned char* pool,
                                       const Bf16Pages& pg, int tb, int hi, unsigned char* dst,
                                       int wave, int lane, const unsigned char* zero) {
#pragma unroll
  for (int j = 0; j < 18; ++j) issue_one_bf16(a, pool, pg, tb, hi, dst, wave, lane, j, zero);
}

// Slice-page variant of the bf16 loads: the 16 tokens t0 .. t0+15 of a wave's
// slice of a tile lie in one sub-page `sp`, so one base address and the count
// of tokens before the segment end describe all of them.
struct SliceSrc {
  const unsigned char* base;  // token t0
  int nvalid;                 // tokens t0 .. t0 + nvalid - 1 are read; the rest are zero rows
};
__device__ __forceinline__ SliceSrc slice_src(const AttnArgs& a, const unsigned char* pool,
                                              int32_t sp, int t0, int hi) {
  SliceSrc v;
  const bool ok = sp >= 0 && sp < a.num_subpages;
  v.nvalid = ok ? min(max(hi - t0, 0), 16) : 0;
  const int64_t t = ((int64_t)(ok ? sp : 0) << a.page_shift) + (t0 & (a.page_size - 1));
  v.base = pool + t * kTokBytesBf16;
  return v;
}
// Load j (0..17) of a wave's slice into `dst`: j < 16 is the latent part of
// token 16w + j, j = 16, 17 the rope parts of tokens 16w + 8(j-16) + 0..7.
__device__ __forceinline__ void issue_slice(const SliceSrc& v, const unsigned char* zero,
                                            unsigned char* dst, int wave, int lane, int j) {
  if (j < 16) {
    const int row = 16 * wave + j;
    const unsigned char* src = j < v.nvalid ? v.base + j * kTokBytesBf16 : zero;
    dma16(src + 16 * lane, dst + lat_row(row));
  } else {
    const int jj = j - 16;
    const int u = lane >> 3;
    const int t = 8 * jj + u;                // token within the slice
    const int chunk = (lane & 7) ^ rope_key(16 * wave + t);
    const unsigned char* src = t < v.nvalid ? v.base + t * kTokBytesBf16 : zero;
    dma16(src + 2 * kVDim + 16 * chunk, dst + kLatBytes + (16 * wave + 8 * jj) * kRopeRow);
  }
}

// Slice pages of 64 consecutive tiles for one wave: lane j holds the sub-page
// of tokens tb0 + 64 j + 16 w .. +15 (the last in-range entry past the
// segment end; tokens there are masked and read from the zero row).
__device__ __forceinline__ int32_t slice_pages(const AttnArgs& a, const int32_t* pt_row, int tb0,
                                               int hi, int wave, int lane) {
  const int64_t tok = min((int64_t)tb0 + (int64_t)kTile * lane + 16 * wave, (int64_t)hi - 1);
  return pt_row[tok >> a.page_shift];
}

// Work unit of a workgroup and the segment [lo, hi) of local tokens it covers
// (valid: the request's rows are well formed and the row block exists).
struct WorkUnit {
  int i, r, s, mb;
  int qs, Q, M, m0, last;
  int lo, hi;
  bool valid;
  bool read;                 // the segment starts before the group's end: the merge reads it
};
// Workgroups are dealt to the 8 XCDs round-robin (blockIdx % 8). Request i
// goes to XCD i % 8, and all its work units (every shard, segment and row
// block) get consecutive ids on that XCD, so they run side by side: its Q,
// and each unit's KV across row blocks, come from HBM into that XCD's L2
// once. The grid covers ceil(N / 8) * 8 requests and mblocks row blocks per
// request (see poison_uncovered for a request with more).
__device__ inline WorkUnit decode_head(const AttnArgs& a, int b) {
  WorkUnit u;
  const int slot = b >> 3;
  u.mb = slot % a.mblocks;
  int t = slot / a.mblocks;
  u.s = t % a.nseg;
  t /= a.nseg;
  u.r = t % a.W;
  u.i = (t / a.W) * 8 + (b & 7);
  u.valid = u.i < a.N;
  u.lo = u.hi = 0;
  if (!u.valid) return u;
  u.qs = a.q_start[u.i];
  u.Q = a.q_start[u.i + 1] - u.qs;
  u.M = u.Q * a.H;                          // (row, head) pairs of the request
  u.m0 = u.mb * kAttnRows;
  u.valid = !(u.qs < 0 || u.Q <= 0 || u.qs + u.Q > a.R || u.m0 >= u.M);
  u.last = u.qs + u.Q - 1;                  // the group's longest row
  return u;
}
// The unit's segment [lo, hi) from the group's longest row, its last (lo >=
// hi: the segment holds no token to read). The partition uses the row's
// length exactly as the merge does; tokens past the table row are never
// read (a well-formed plan keeps every length within it), so a segment can be
// read by the merge (`read`) and still hold no token, and then gets empty
// partials.
__device__ inline void decode_tail(const AttnArgs& a, WorkUnit& u) {
  const int Lg = a.row_lens[(int64_t)u.r * a.R + u.last];
  const int64_t seg_tokens = (int64_t)a.nseg * a.page_size;
  const int span = (int)((Lg + seg_tokens - 1) / seg_tokens * a.page_size);
  u.lo = u.s * span;
  u.read = u.lo < Lg;
  u.hi = (int)min(min((int64_t)u.lo + span, (int64_t)Lg),
                  (int64_t)a.pt_width * a.page_size);
}
// Sub-pages of the first 64 tiles of a group for one wave (lane j: the
// slice 64 j + 16 w .. +15), read before the group's length is known: the
// index is clamped to the table row instead of the segment end. A slice that
// starts before the segment end lies in one sub-page, whose entry is the same
// either way; the entries of later slices are never used. Needs a table row
// of at least one entry (pt_width >= 1).
__device__ __forceinline__ int32_t first_slice_pages(const AttnArgs& a, const int32_t* pt_row,
                                                     int wave, int lane) {
  const int64_t tok = min((int64_t)kTile * lane + 16 * wave,
                          ((int64_t)a.pt_width << a.page_shift) - 1);
  return pt_row[tok >> a.page_shift];
}

__device__ inline WorkUnit decode_unit(const AttnArgs& a, int b) {
  WorkUnit u = decode_head(a, b);
  if (u.valid) decode_tail(a, u);
  return u;
}

// Q of the block, staged in a tile buffer: block row m (the (row, head) pair
// m0 + m, one contiguous 1152-byte vector) is laid out like KV token m, so the
// QK B-operand fragments are read exactly like K fragments. The block's pairs
// are contiguous in q, so these are the same 1 KB direct loads as a KV tile:
// about half the bytes of per-wave register loads (each row group's two waves
// need the same rows) and no partial-line requests. Pairs past the request's
// last one read the zero row.
__device__ __forceinline__ void issue_q_tile(const AttnArgs& a, const WorkUnit& u,
                                             unsigned char* dst, int wave, int lane,
                                             const unsigned char* zero) {
  const unsigned char* qb =
      reinterpret_cast<const unsigned char*>(a.q + ((int64_t)u.qs * a.H + u.m0) * kHeadDim);
  auto src_of = [&](int row) -> const unsigned char* {
    return u.m0 + row < u.M ? qb + (int64_t)row * kTokBytesBf16 : zero;
  };
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int row = 16 * wave + j;
    dma16(src_of(row) + 16 * lane, dst + lat_row(row));
  }
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int uu = lane >> 3;
    const int row = 16 * wave + 8 * jj + uu;
    const int chunk = (lane & 7) ^ rope_key(row);
    dma16(src_of(row) + 2 * kVDim + 16 * chunk, dst + kLatBytes + (16 * wave + 8 * jj) * kRopeRow);
  }
}

// ---------------------------------------------------------------------------
// Per-tile computation, shared by the bf16 and fp8 kernels.
//
// Wave (g, c) of a workgroup: rows 32g..32g+31 of the block. For every 64-token
// tile it computes S^T for tokens 32c..32c+31 of the tile, and O^T for latent
// dims 256c..256c+255 over all 64 tokens, so the two waves of a row group trade
// their row maxima and their P fragments through LDS once per tile each.
//
// Both products run on v_mfma_f32_32x32x16_bf16 (a 32x32 output tile per
// instruction: more flops per issue cycle than the 16x16 forms). Operand and
// accumulator lanes of that instruction (h = l / 32):
//   A (32 x 16): lane l holds A[l % 32][8h + e], e = 0..7
//   B (16 x 32): lane l holds B[8h + e][l % 32]
//   D (32 x 32): value j of lane l is D[8 (j / 4) + 4h + j % 4][l % 32]
// So lane l owns one query row, 32g + l % 32, in both products.
//  * S^T[32 tokens x 32 rows] = K Q^T: 36 K-steps of 16 dims, Q in registers.
//    Accumulator value j is token 8 (j / 4) + 4h + j % 4 of the wave's 32.
//  * O^T[256 dims x 32 rows] += V^T P^T: 8 output tiles of 32 dims, 4 K-steps
//    of 16 tokens per tile. Values 8s..8s+7 of the S^T accumulator are tokens
//    16s + 4h + {0..3} and 16s + 8 + 4h + {0..3}: converted to bf16 they are
//    already the B operand of the wave's own K-step s, so P never moves
//    between lanes; the V^T operand takes the same token order from two
//    transposed 4-token reads (ds_read_b64_tr_b16) per instruction.
//  * The weights enter the PV product as bf16 (the operand format of the
//    matrix cores next to a bf16 V): each is rounded by at most 2^-8 of its
//    value, so the output moves by at most 2^-8 of the softmax-weighted mean
//    of |v|. (Feeding them as two bf16 terms, hi + lo, removes that but
//    doubles the PV instructions: measured 22-33 % slower.)
//
// Online softmax in base 2 with a lazily refreshed reference: O and the sum
// are rescaled only when the row maximum passes the reference by more than 8
// (P <= 256, harmless for bf16 P and fp32 sums); at the end they are rescaled
// once to the true maximum, which is what is stored. Both waves of a row
// group see the same tile maxima and so make the same decisions.

// Accumulation state of one wave: 32 rows x 256 latent dims.
struct WaveState {
  f32x16 o[kOTiles];        // O^T tiles: value j of lane l is dim 256c + 32t + 8(j/4) + 4h + j%4
  float m_ref;              // this lane's row: reference exponent of o and l_part
  float m_true;             // this lane's row: true running maximum
  float l_part;             // this lane's share of the row's exp2 sum over this wave's tokens
};

// Row maxima and P fragments handed to the partner wave, once per tile each.
struct PExchange {
  uint4 p[2][2][2][64];     // [g][c][K-step of the wave's tokens][lane]: bf16 P
  float mx[2][2][32];       // [g][c][row]: maxima over the wave's 32 tokens
};

// End-of-segment exchange of row sums between partner waves.
struct RowExchange {
  float l[2][2][32];        // [g][c][row]
};

__device__ __forceinline__ void state_init(WaveState& st) {
#pragma unroll
  for (int t = 0; t < kOTiles; ++t) st.o[t] = f32x16{};
  st.m_ref = kNegInf;
  st.m_true = kNegInf;
  st.l_part = 0.f;
}

// This lane's row (row 32g + l % 32 of the block) and the part of the segment
// it may see.
__device__ inline void lane_row(const AttnArgs& a, const WorkUnit& u, int g, int lane, int& mrow,
                                int& hi_row, bool& row_ok) {
  mrow = u.m0 + 32 * g + (lane & 31);
  row_ok = mrow < u.M;
  const int Lrow = row_ok ? a.row_lens[(int64_t)u.r * a.R + u.qs + mrow / a.H] : 0;
  hi_row = min(u.hi, Lrow);
}

// K fragment (A operand of S^T = K Q^T) of K-step k: token `tok` of the tile,
// dims 16k + 8h .. +7.
__device__ __forceinline__ bf16x8 k_fragment(const unsigned char* tile, int tok, int k, int h) {
  if (k < kLatQSteps)
    return *reinterpret_cast<const bf16x8*>(tile + lat_off(tok, 2 * k + h));
  const int chunk = 2 * (k - kLatQSteps) + h;
  return *reinterpret_cast<const bf16x8*>(tile + kLatBytes + tok * kRopeRow +
                                          16 * (chunk ^ rope_key(tok)));
}

// Q fragments (B operand of S^T = K Q^T) of this lane's row from the staged Q
// tile: dims 16k + 8h .. +7 for every K-step k. The reads are inline assembly
// that lands them in accumulation registers, where the MFMAs take them as
// operands directly (the compiler would otherwise keep them there and copy
// each one back before every use); the trailing wait is tied to every
// fragment.
__device__ __forceinline__ void read_q(const unsigned char* qtile, int g, int lane,
                                       bf16x8 (&qf)[kQSteps]) {
  const int h = lane >> 5;
  const int row = 32 * g + (lane & 31);
#pragma unroll
  for (int k = 0; k < kQSteps; ++k) {
    const unsigned char* p =
        k < kLatQSteps ? qtile + lat_off(row, 2 * k + h)
                       : qtile + kLatBytes + row * kRopeRow +
                             16 * ((2 * (k - kLatQSteps) + h) ^ rope_key(row));
    const uint32_t addr = (uint32_t)(uintptr_t)(const lds_void*)p;
    asm volatile("ds_read_b128 %0, %1" : "=a"(qf[k]) : "v"(addr));
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int k = 0; k < kQSteps; k += 6)
    asm volatile("" : "+a"(qf[k]), "+a"(qf[k + 1]), "+a"(qf[k + 2]), "+a"(qf[k + 3]),
                      "+a"(qf[k + 4]), "+a"(qf[k + 5]));
}

// Scores, softmax and PV for one 64-token tile held in `tile` (LDS).
// `issue(k)` is called once per QK K-step (k = 0..35), so that the loads of
// the next tile can be spread over the MFMA work.
template <class Issue>
__device__ __forceinline__ void compute_tile(const unsigned char* __restrict__ tile,
                                             PExchange* __restrict__ px,
                                             const bf16x8 (&qf)[kQSteps], WaveState& st, int tb,
                                             int hi_row, float qk_scale_log2, int g, int c,
                                             int lane, Issue&& issue) {
  const int h = lane >> 5;
  const int n32 = lane & 31;

  // ---- S^T[32 tokens x 32 rows]; K fragments are read kKAhead K-steps ahead
  // of their MFMAs (a ring); the scheduling barriers keep that order.
  constexpr int kKAhead = 2;
  f32x16 sacc = f32x16{};
  bf16x8 kr[kKAhead + 1];
#pragma unroll
  for (int k = 0; k < kKAhead; ++k) kr[k] = k_fragment(tile, 32 * c + n32, k, h);
#pragma unroll
  for (int k = 0; k < kQSteps; ++k) {
    if (k + kKAhead < kQSteps)
      kr[(k + kKAhead) % (kKAhead + 1)] = k_fragment(tile, 32 * c + n32, k + kKAhead, h);
    issue(k);
    __builtin_amdgcn_sched_barrier(0);
    sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[k % (kKAhead + 1)], qf[k], sacc, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- mask, maximum of this lane's 16 scores and of the other half's 16
  // (lane l ^ 32 holds the same row). Tiles that every row of the wave sees
  // whole skip the masking. The scores stay unscaled: the scale is positive,
  // so the maximum of the rounded scaled scores is the rounded scaled
  // maximum, and the scale goes into the exponent's fused multiply-add.
  if (__builtin_amdgcn_ballot_w64(tb + kTile > hi_row) != 0) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int tok = tb + 32 * c + 8 * (j >> 2) + 4 * h + (j & 3);
      if (tok >= hi_row) sacc[j] = kNegInf;
    }
  }
  float m = sacc[0];
#pragma unroll
  for (int j = 1; j < 16; ++j) m = fmaxf(m, sacc[j]);
  {
    auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    m = fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
  }
  if (h == 0) px->mx[g][c][n32] = m;

  // ---- V^T reads for the first PV steps go out before the barrier. Step t
  // covers output tile dt = t % 8 and K-step s: the wave's own tokens first
  // (s = 2c + t / 8 for t < 16), then the partner's (s = 2(c ^ 1) + (t - 16) / 8).
  // Lane i of 16-lane group (h, G) points at dims 256c + 32dt + 16G + 4(i % 4)
  // of token 16s + 4h + i / 4 (and of the token 8 further); the transposed
  // read hands it dim 256c + 32dt + 16G + i of tokens 16s + 4h + 0..3 (and
  // 16s + 8 + 4h + 0..3). Each step's reads are issued kVAhead steps ahead of
  // its MFMA (a ring).
  const int i16 = lane & 15;
  const int G = (lane >> 4) & 1;
  auto vread = [&](int t, i16x4& lo4, i16x4& hi4) {
    const int s = t < 16 ? 2 * c + (t >> 3) : 2 * (c ^ 1) + ((t - 16) >> 3);
    const int dt = t & 7;
    const int row = 16 * s + 4 * h + (i16 >> 2);
    const int ch = 32 * c + 4 * dt + 2 * G + ((i16 & 3) >> 1);
    const int byte = 8 * (i16 & 1);
    lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + lat_off(row, ch) + byte));
    hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(tile + lat_off(row + 8, ch) + byte));
  };
  constexpr int kPvSteps = 4 * kOTiles;
  constexpr int kVAhead = 3;
  i16x4 vr[kVAhead + 1][2];
#pragma unroll
  for (int t = 0; t < kVAhead; ++t) vread(t, vr[t][0], vr[t][1]);

  lds_barrier();
  // the partner saw the other 32 tokens; both waves now hold the same tile max
  m = fmaxf(m, px->mx[g][c ^ 1][n32]) * qk_scale_log2;
  st.m_true = fmaxf(st.m_true, m);

  // ---- lazily refreshed reference (identical decisions on both waves)
  const bool refresh = m > st.m_ref + kRescaleSlack;
  if (__builtin_amdgcn_ballot_w64(refresh) != 0) {
    const float alpha = refresh ? __builtin_amdgcn_exp2f(st.m_ref - m) : 1.f;
    st.l_part *= alpha;
#pragma unroll
    for (int t = 0; t < kOTiles; ++t) st.o[t] *= alpha;
    st.m_ref = refresh ? m : st.m_ref;
  }

  // ---- P of this wave's tokens (its two PV K-steps); publish it for the partner
  const float m_use = st.m_ref == kNegInf ? 0.f : st.m_ref;
  bf16x8 pown[2];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    // masked: the score is -inf and exp2(-inf) = 0 (m_use is finite)
    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[j], qk_scale_log2, -m_use));
    st.l_part += p;
    pown[j >> 3][j & 7] = (__bf16)p;
  }
  px->p[g][c][0][lane] = __builtin_bit_cast(uint4, pown[0]);
  px->p[g][c][1][lane] = __builtin_bit_cast(uint4, pown[1]);
  // The own half of the PV product needs only this wave's P: it runs while
  // the partner's P is on its way (the exchange barrier sits at step 16).
  bf16x8 ppart[2];

  // ---- O^T[256 dims x 32 rows] += V^T[256 x 64 tokens] P^T[64 x 32]
#pragma unroll
  for (int t = 0; t < kPvSteps; ++t) {
    if (t == 16) {
      lds_barrier();
      ppart[0] = __builtin_bit_cast(bf16x8, px->p[g][c ^ 1][0][lane]);
      ppart[1] = __builtin_bit_cast(bf16x8, px->p[g][c ^ 1][1][lane]);
    }
    if (t + kVAhead < kPvSteps)
      vread(t + kVAhead, vr[(t + kVAhead) % (kVAhead + 1)][0], vr[(t + kVAhead) % (kVAhead + 1)][1]);
    __builtin_amdgcn_sched_barrier(0);
    const int dt = t & 7;
    const int sl = (t >> 3) & 1;            // K-step within the wave's (or partner's) tokens
    const bf16x8 va = __builtin_bit_cast(
        bf16x8, __builtin_shufflevector(vr[t % (kVAhead + 1)][0], vr[t % (kVAhead + 1)][1], 0, 1, 2,
                                        3, 4, 5, 6, 7));
    st.o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, t < 16 ? pown[sl] : ppart[sl], st.o[dt],
                                                       0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Two fp32 values rounded (RNE) to bf16 and packed, the first in the low half.
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  const __bf16 x = (__bf16)lo, y = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) |
         ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// Normalised form (a.shard_out set): every (shard, segment) unit is one
// source of the LSE merge, source r * nseg + s; index of its (row qs of the
// unit's request, head 0) in shard_out / shard_lse [W * nseg, R, H].
__device__ __forceinline__ int64_t source_base(const AttnArgs& a, const WorkUnit& u) {
  return ((int64_t)(u.r * a.nseg + u.s) * a.R + u.qs) * a.H;
}

// A unit with no token to read: in the normalised form its rows still get
// their (empty) results, o = 0 and lse = -inf; in the split form a segment
// the merge reads gets the empty partials (maximum -inf, sum 0: the merge
// then gives it weight 0 and never touches its output), and any other
// segment nothing.
__device__ inline void store_empty(const AttnArgs& a, const WorkUnit& u, int wave, int lane) {
  const int64_t base = ((int64_t)u.r * a.R + u.qs) * a.H;
  const int64_t sbase = source_base(a, u);
  for (int k = wave; k < kAttnRows && u.m0 + k < u.M; k += 4) {
    const int64_t e = base + u.m0 + k;
    if (a.shard_out != nullptr) {
      const int64_t f = sbase + u.m0 + k;
      *reinterpret_cast<uint4*>(a.shard_out + f * kVDim + 8 * lane) = make_uint4(0, 0, 0, 0);
      if (lane == 0) a.shard_lse[f] = kNegInf;
    } else if (u.read && lane == 0) {
      a.segm_max[e * a.nseg + u.s] = kNegInf;
      a.segm_expsum[e * a.nseg + u.s] = 0.f;
    }
  }
}

// A request with more (row, head) pairs than the grid's mblocks row blocks
// cover (its Q_i above the caller's max_qlen) must not end in unwritten
// outputs: the unit of its last covered row block fills every uncovered
// pair's results for its shard and segment with NaN (written as bits, so no
// fast-math folding applies), which both merges carry into out and lse.
__device__ inline void poison_uncovered(const AttnArgs& a, const WorkUnit& u, int wave, int lane) {
  const int covered = a.mblocks * kAttnRows;
  if (u.mb != a.mblocks - 1 || u.M <= covered) return;   // uniform
  const uint32_t qnan = 0x7FC00000u;
  const int64_t base = ((int64_t)u.r * a.R + u.qs) * a.H;
  for (int m = covered + wave; m < u.M; m += 4) {
    const int64_t e = base + m;
    if (a.shard_out != nullptr) {
      const int64_t f = source_base(a, u) + m;
      *reinterpret_cast<uint4*>(a.shard_out + f * kVDim + 8 * lane) =
          make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);
      if (lane == 0) reinterpret_cast<uint32_t*>(a.shard_lse)[f] = qnan;
    } else {
      const int64_t f = e * a.nseg + u.s;
      uint32_t* o = reinterpret_cast<uint32_t*>(a.segm_out + f * kVDim) + 8 * lane;
      *reinterpret_cast<uint4*>(o) = make_uint4(qnan, qnan, qnan, qnan);
      *reinterpret_cast<uint4*>(o + 4) = make_uint4(qnan, qnan, qnan, qnan);
      if (lane == 0) {
        reinterpret_cast<uint32_t*>(a.segm_max)[f] = qnan;
        reinterpret_cast<uint32_t*>(a.segm_expsum)[f] = qnan;
      }
    }
  }
}

// A tile for a wave whose row group holds no row of the block (the last
// block of a request whose Q_i * H is not a multiple of 64 may fill only its
// first row group): the wave issues its share of the next tile's loads and
// meets compute_tile's two barriers, and leaves the LDS and the matrix cores
// to the other row group.
template <class Issue>
__device__ __forceinline__ void idle_tile(Issue&& issue) {
#pragma unroll
  for (int k = 0; k < kQSteps; ++k) issue(k);
  lds_barrier();                            // compute_tile: tile maxima published
  lds_barrier();                            // compute_tile: P fragments published
}

// End of the segment: add the partner wave's row sums and write the partials
// (maximum, sum and O relative to the maximum). O goes through LDS (`stage`:
// this row group's 32 rows, a tile buffer no longer read) so that the global
// stores write whole rows, 1 KB per instruction, instead of 16-byte pieces.
// Normalised form (a.shard_out set): the merge of a single segment is the
// normalisation, so the row's output O / sum goes out as bf16 with its
// natural-log LSE ln2 (max + log2 sum) -- in the same fp32 operations and
// order as the merge kernel applies to the partials -- as source
// r * nseg + s of the LSE merge.
constexpr int kStageRow = 4 * kVDim + 16;   // padded row of 512 fp32
constexpr int kStageRowBf16 = 2 * kVDim + 16;  // padded row of 512 bf16
static_assert(32 * kStageRow <= kBufBytes, "a row group's O fits a tile buffer");
// kLdsOnly: the barriers order LDS traffic only, for a caller that keeps
// global loads in flight across the epilogue (normalised form only).
template <bool kLdsOnly = false>
__device__ __forceinline__ void store_partials(const AttnArgs& a, const WorkUnit& u,
                                               const WaveState& st, RowExchange& rx,
                                               unsigned char* stage, int mrow, bool row_ok, int g,
                                               int c, int lane) {
  auto barrier = [] {
    if constexpr (kLdsOnly)
      lds_barrier();
    else
      __syncthreads();
  };
  const int h = lane >> 5;
  const int n32 = lane & 31;
  float l_row;
  {
    auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(st.l_part),
                                              __float_as_uint(st.l_part), false, false);
    l_row = __uint_as_float(q[0]) + __uint_as_float(q[1]);
  }
  if (h == 0) rx.l[g][c][n32] = l_row;
  barrier();                                // also: no wave reads a tile buffer any more
  const float L = l_row + rx.l[g][c ^ 1][n32];
  // move O and l from the reference exponent to the true maximum
  float fix = 1.f;
  if (st.m_true != kNegInf) fix = __builtin_amdgcn_exp2f(st.m_ref - st.m_true);
  const bool one_seg = a.shard_out != nullptr;   // uniform
  const float E = L * fix;
  const bool live = st.m_true != kNegInf && E > 0.f;
  if (row_ok && c == 0 && h == 0) {
    if (one_seg) {
      a.shard_lse[source_base(a, u) + mrow] =
          live ? kLn2 * (st.m_true + __log2f(E)) : kNegInf;
    } else {
      const int64_t e = (((int64_t)u.r * a.R + u.qs) * a.H + mrow) * a.nseg + u.s;
      a.segm_max[e] = st.m_true;
      a.segm_expsum[e] = E;
    }
  }
  const float vs = fix * a.v_scale;
  float* sp = reinterpret_cast<float*>(stage + n32 * kStageRow) + 256 * c + 4 * h;
  if (one_seg) {
    // rows staged already rounded to bf16 (half the LDS traffic of fp32)
    const float inv = live ? 1.f / E : 0.f;
    unsigned char* sb = stage + n32 * kStageRowBf16 + 2 * (256 * c + 4 * h);
#pragma unroll
    for (int t = 0; t < kOTiles; ++t) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v = (f32x4{st.o[t][4 * q], st.o[t][4 * q + 1], st.o[t][4 * q + 2],
                               st.o[t][4 * q + 3]} * vs) * inv;
        *reinterpret_cast<uint2*>(sb + 2 * (32 * t + 8 * q)) =
            make_uint2(pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3]));
      }
    }
    barrier();
    // wave (g, c) stores rows 16c .. 16c + 15 of its row group: one 1 KB
    // row of bf16 per instruction, 8 dims per lane
    // (all 16 LDS reads first, then the stores: one LDS round trip, not 16)
    const int row0 = u.m0 + 32 * g + 16 * c;
    uint4 rows[16];
#pragma unroll
    for (int k = 0; k < 16; ++k)
      rows[k] = *reinterpret_cast<const uint4*>(stage + (16 * c + k) * kStageRowBf16 + 16 * lane);
    const int64_t e0 = source_base(a, u) + row0;
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (row0 + k < u.M)
        *reinterpret_cast<uint4*>(a.shard_out + (e0 + k) * kVDim + 8 * lane) = rows[k];
    return;
  }
#pragma unroll
  for (int t = 0; t < kOTiles; ++t) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 v = {st.o[t][4 * q], st.o[t][4 * q + 1], st.o[t][4 * q + 2], st.o[t][4 * q + 3]};
      *reinterpret_cast<f32x4*>(sp + 32 * t + 8 * q) = v * vs;
    }
  }
  __syncthreads();
  // wave (g, c) stores rows 16c .. 16c + 15 of its row group, half a row a
  // go, eight rows' LDS reads in flight before their stores
  const int row0 = u.m0 + 32 * g + 16 * c;
#pragma unroll
  for (int k0 = 0; k0 < 16; k0 += 8) {
    float4 v[8][2];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const unsigned char* src = stage + (16 * c + k0 + k) * kStageRow + 16 * lane;
      v[k][0] = *reinterpret_cast<const float4*>(src);
      v[k][1] = *reinterpret_cast<const float4*>(src + 1024);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (row0 + k0 + k < u.M) {
        const int64_t e = (((int64_t)u.r * a.R + u.qs) * a.H + row0 + k0 + k) * a.nseg + u.s;
        float* dst = a.segm_out + e * kVDim + 4 * lane;
        *reinterpret_cast<float4*>(dst) = v[k][0];
        *reinterpret_cast<float4*>(dst + 256) = v[k][1];
      }
    }
  }
}

}  // namespace
}  // namespace mla
