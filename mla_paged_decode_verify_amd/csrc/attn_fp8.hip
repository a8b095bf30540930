// Split-K segmented MLA attention partials, fp8 KV cache (OCP e4m3fn or e5m2
// codes), on the fp8 matrix cores.
//
// The quantities computed and the work decomposition are those of
// attn_common.h; the per-tile computation is step_f8 (attn_f8mma.h): the
// codes go from HBM into LDS as they are, by direct loads, and feed the
// scaled fp8 MFMAs with Q and P as two e4m3fn terms each; each step runs the
// softmax and PV of tile k around the QK product of tile k + 1. An fp8 tile
// is half a bf16 one, so the two tile buffers hold four: tile k uses slot
// k mod 4 and the loads of tile k + 3 go out during step k. Q is staged
// (bf16) in the second buffer first and split into its terms before tiles 2
// and 3 land there. The fp8 scale is folded into the score scale and into the
// output.
#include "attn_f8mma.h"

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
  const int ntiles = (hi - lo + kTile - 1) / kTile;

  // all nine loads of this wave for tile k (slice path: k < 64)
  auto issue_all = [&](int k) {
    unsigned char* dst = f8_slot(buf0, buf1, k & 3);
    const int tb = lo + k * kTile;
    if constexpr (SLICE) {
      const __amdgpu_buffer_rsrc_t r =
          f8_slice_rsrc(a, pool, __builtin_amdgcn_readlane(vpg, k & 63), tb + 16 * wave, hi);
#pragma unroll
      for (int j = 0; j < kF8Dma; ++j) issue_f8_slice(r, dst, wave, lane, j);
    } else {
#pragma unroll
      for (int j = 0; j < kF8Dma; ++j)
        issue_f8_pages(a, pool, pt_row, tb, hi, dst, wave, lane, j, zero);
    }
  };

  // ---- Q (bf16, through the second buffer) and the first two tiles
  issue_q_tile(a, u, buf1, wave, lane, zero);
  if constexpr (SLICE) {
    if (u.s != 0) vpg = slice_pages(a, pt_row, lo, hi, wave, lane);
  }
  issue_all(0);
  if (ntiles > 1) issue_all(1);
  int mrow, hi_row;
  bool row_ok;
  lane_row(a, u, g, lane, mrow, hi_row, row_ok);
  const bool idle = u.m0 + 32 * g >= u.M;   // no row of this row group in the block
  WaveState st;
  state_init(st);
  if (ntiles > 1)
    MLA_WAIT_VMCNT(kF8Dma);                 // Q and tile 0 have landed
  else
    MLA_WAIT_VMCNT(0);
  lds_barrier();
  QF8 q;
  read_q_f8(buf1, g, lane, q);
  lds_barrier();                            // the second buffer is free for tiles 2, 3
  if (ntiles > 2) issue_all(2);
  f32x16 sacc;
  if (!idle) qk_f8<E5M2>(f8_slot(buf0, buf1, 0), q, sacc, c, lane);

  for (int k = 0; k < ntiles; ++k) {
    const int tb = lo + k * kTile;
    if (k + 2 < ntiles)
      MLA_WAIT_VMCNT(kF8Dma);               // tile k + 1 has landed (tile k + 2 may not have) ...
    else
      MLA_WAIT_VMCNT(0);
    lds_barrier();                          // ... for every wave; slot (k + 3) mod 4 is free
    const bool more3 = k + 3 < ntiles;
    unsigned char* dst = f8_slot(buf0, buf1, (k + 3) & 3);
    __amdgpu_buffer_rsrc_t rs = f8_slice_rsrc(a, pool, -1, 0, 0);
    if (more3) {
      if constexpr (SLICE) {
        const int nk = k + 3;
        if ((nk & 63) == 0) vpg = slice_pages(a, pt_row, lo + nk * kTile, hi, wave, lane);
        rs = f8_slice_rsrc(a, pool, __builtin_amdgcn_readlane(vpg, nk & 63),
                           lo + nk * kTile + 16 * wave, hi);
      } else {
        issue_all(k + 3);                   // table entries first: one wait, then the loads
      }
    }
    // one load per QK K-step (slice path)
    auto issue = [&](int s) {
      if constexpr (SLICE) {
        if (more3) issue_f8_slice(rs, dst, wave, lane, s);
      }
    };
    if (idle)
      idle_tile_f8(issue);
    else
      step_f8<E5M2>(f8_slot(buf0, buf1, k & 3), f8_slot(buf0, buf1, (k + 1) & 3), sacc, &px, q,
                    st, tb, hi_row, a.qk_scale_log2, g, c, lane, issue);
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
