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
#include "attn_fp8_tile.h"

namespace mla {
namespace {

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
