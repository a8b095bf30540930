// Split-K segmented MLA attention partials, bf16 KV cache.
//
// The quantities computed, the work decomposition and the per-tile
// computation are those of attn_common.h. Specific to this kernel:
//  * Tiles go straight from HBM to LDS (global_load_lds_dwordx4: one 1 KB
//    instruction per token's latent part, one per 8 tokens' rope parts), so no
//    registers hold data in flight. While tile k is computed, tile k+1 streams
//    in, issued one instruction every other QK K-step; two LDS buffers
//    alternate.
//  * Page-table entries: when sub-pages hold 16+ tokens, a wave's 16-token
//    slice of a tile lies in one sub-page, so one vector load gives a wave the
//    entries of 64 tiles (one per lane), read out with v_readlane; no load of
//    a page entry sits between two tiles. Smaller sub-pages take per-token
//    entries, fetched at the start of each tile.
#include "attn_common.h"

namespace mla {
namespace {


template <bool SLICE>
__global__ void __launch_bounds__(kThreads, 1) attn_bf16_kernel(AttnArgs a) {
  // Two separate arrays (not one indexed one), so that the compiler can tell
  // the buffer being read from the buffer the direct loads are filling.
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

  const unsigned char* pool = a.kv + (int64_t)u.r * a.pool_tokens * kTokBytesBf16;
  const unsigned char* zero = zero_row();
  const int32_t* pt_row = a.page_table + ((int64_t)u.r * a.R + u.last) * a.pt_width;

  // ---- the group's length and, for a first segment, its first sub-pages:
  // two loads in flight together, before any bulk data
  int32_t vpg = 0;                          // SLICE: pages of tiles 64q .. 64q + 63
  if constexpr (SLICE) {
    if (u.s == 0 && a.pt_width > 0) vpg = first_slice_pages(a, pt_row, wave, lane);
  }
  decode_tail(a, u);
  const int lo = u.lo, hi = u.hi;
  if (lo >= hi) {                           // no token of the group to read
    store_empty(a, u, wave, lane);
    return;
  }

  // ---- Q (through the second tile buffer: free until the first step's
  // barrier, after which the next tile's loads target it), then the first tile
  issue_q_tile(a, u, buf1, wave, lane, zero);
  Bf16Pages pg;
  if constexpr (SLICE) {
    if (u.s != 0) vpg = slice_pages(a, pt_row, lo, hi, wave, lane);
    const SliceSrc v0 = slice_src(a, pool, __builtin_amdgcn_readlane(vpg, 0), lo + 16 * wave, hi);
#pragma unroll
    for (int j = 0; j < 18; ++j) issue_slice(v0, zero, buf0, wave, lane, j);
  } else {
    pg.fetch(a, pt_row, lo, hi, wave, lane);
    issue_tile_bf16(a, pool, pg, lo, hi, buf0, wave, lane, zero);
  }
  int mrow, hi_row;
  bool row_ok;
  lane_row(a, u, g, lane, mrow, hi_row, row_ok);
  const bool idle = u.m0 + 32 * g >= u.M;   // no row of this row group in the block
  WaveState st;
  state_init(st);
  MLA_WAIT_VMCNT(0);
  lds_barrier();
  bf16x8 qf[kQSteps];
  read_q(buf1, g, lane, qf);

  // One tile (index kt from the segment start): wait until `cur` holds it,
  // start filling `nxt` with the next tile, compute on `cur`.
  auto step = [&](const unsigned char* cur, unsigned char* nxt, int tb, int kt) {
    const bool more = tb + kTile < hi;
    MLA_WAIT_VMCNT(0);                      // this wave's loads of `cur` have landed ...
    lds_barrier();                          // ... for every wave; `nxt` is no longer read
    SliceSrc v{zero, 0};
    if constexpr (SLICE) {
      if (more) {
        const int nk = kt + 1;
        if ((nk & 63) == 0) vpg = slice_pages(a, pt_row, lo + nk * kTile, hi, wave, lane);
        v = slice_src(a, pool, __builtin_amdgcn_readlane(vpg, nk & 63), tb + kTile + 16 * wave, hi);
      }
    } else {
      if (more) {
        pg.fetch(a, pt_row, tb + kTile, hi, wave, lane);
        issue_tile_bf16(a, pool, pg, tb + kTile, hi, nxt, wave, lane, zero);
      }
    }
    // one load every other QK K-step: the next tile's data goes out early,
    // and its LDS writes are spread over the whole QK product, which competes
    // with them for LDS bandwidth (measured: faster than packing the loads
    // into the first half, or issuing them in the PV product)
    auto issue = [&](int j) {
      if constexpr (SLICE) {
        if (more && (j & 1) == 0) issue_slice(v, zero, nxt, wave, lane, j >> 1);
      }
    };
    if (idle)
      idle_tile(issue);
    else
      compute_tile(cur, &px, qf, st, tb, hi_row, a.qk_scale_log2, g, c, lane, issue);
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

hipError_t launch_attn(const AttnArgs& a, bool fp8, hipStream_t s) {
  const int64_t blocks = (int64_t)(a.N + 7) / 8 * 8 * a.W * a.nseg * a.mblocks;  // decode_unit
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (fp8) return launch_attn_fp8(a, blocks, s);
  if (a.page_size >= 16)
    attn_bf16_kernel<true><<<(unsigned)blocks, kThreads, 0, s>>>(a);
  else
    attn_bf16_kernel<false><<<(unsigned)blocks, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
