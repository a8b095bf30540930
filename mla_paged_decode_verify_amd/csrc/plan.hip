// Plan kernel: rank-local row lengths and per-row sub-page tables.
//
// Row view: vLLM PR #51705 digest (prhub), Implementation breakdown item 2 and
// the _build_dcp_verify_row_view snippet -- verify row t of request i sees
// global positions [0, S_i - Q_i + t]; with round-robin interleave 1 shard r
// holds floor((w - 1 - r) / W) + 1 of the w = S_i - Q_i + 1 + t positions when
// w - 1 - r >= 0 and none otherwise. With interleave I (runs of I consecutive
// positions dealt to the shards in turn; the pages gate I > 1 off, this is a
// reading of the same layout) a window of w positions is c = w div (I W) full
// rounds plus rem = w mod (I W) positions, of which shard r gets
// clamp(rem - r I, 0, I): L = c I + clamp(rem - r I, 0, I) (for I = 1 the
// count above).
// Sub-page table: same digest, item 3 -- the physical block table expanded to
// sub-pages of page_size tokens (block b holds sub-pages b*n .. b*n + n - 1).
//
// Two-stage form: SGLang PR #34432 report, Implementation breakdown items 2-3
// and the _forward_verify_dcp snippet -- stage 1 reads each shard's part of
// the committed prefix [0, S_i - Q_i) row by row (every row of a request has
// the same local length and the same table), stage 2 attends over the dense
// causal window of the Q_i verify tokens, whose entries sit request-major in a
// separate window buffer (row t of request i sees window rows q_start[i] ..
// q_start[i] + t).
//
// One workgroup per request: it checks the request (the block ids it uses are
// checked by all threads at once), then writes the request's row lengths and
// table cells for every shard. Error bits are ORed into the caller's error
// word, which the library never clears (a sticky flag), so a valid batch
// costs no extra launch.
#include "internal.h"

namespace mla {
namespace {

constexpr int kPlanThreads = 256;

// Positions of a window of w (0 <= w < 2^31) that shard r holds. The host
// guarantees I * W <= 2^30, so 32-bit unsigned arithmetic is exact: the
// count is at most w, r * I < 2^30 and the remainder is below I * W.
__device__ __forceinline__ int32_t shard_count(int32_t w, int r, int W, int I) {
  const uint32_t cyc = (uint32_t)I * (uint32_t)W;
  const uint32_t c = (uint32_t)w / cyc;
  const int32_t rem = (int32_t)((uint32_t)w - c * cyc);
  return (int32_t)(c * (uint32_t)I) + min(max(rem - r * I, 0), I);
}
// Rows of shard r, row t of a request with window base S - Q (w = S - Q + 1 + t;
// the committed prefix w = S - Q in the two-stage form).
__device__ __forceinline__ int32_t local_len(int S, int Q, int t, int r, int W, int I,
                                             bool prefix_only) {
  const int w = prefix_only ? S - Q : S - Q + 1 + t;   // window length of row t
  return w > 0 ? shard_count(w, r, W, I) : 0;
}

// Row lengths of one request kept in LDS for its table cells.
constexpr int kPlanLdsRows = 1024;

// Sub-page ids staged in LDS per request: entry k of every table row of the
// request is the same value (sub-page k of the request's blocks), so it is
// computed once, from the block ids the validity check has already read.
constexpr int kPlanLdsPages = 4096;

__global__ void __launch_bounds__(kPlanThreads) plan_kernel(PlanArgs a) {
  __shared__ int32_t pages_lds[kPlanLdsPages];
  __shared__ int32_t len_lds[kPlanLdsRows];
  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  // the request's first 256 block ids go out with its length and rows (one
  // round trip less before the checks; entries past its blocks are unused)
  const int32_t* bt = a.block_table + (int64_t)i * a.max_blocks;
  const int32_t id0 = tid < a.max_blocks ? bt[tid] : 0;
  const int qs = a.q_start[i], qe = a.q_start[i + 1];
  const int S = a.seq_lens[i];
  const int q_end = i == 0 ? a.q_start[a.N] : a.R;   // the batch's row count (checked once)
  const int per = a.block_size / a.page_size;   // sub-pages per block

  // ---- request checks (uniform), then the block ids it uses (all threads)
  uint32_t bits = 0;
  if (qs < 0 || qe > a.R || qe - qs < 1 || S < qe - qs) bits |= MLA_PLAN_ERR_QLEN;
  if (a.win_lens != nullptr && qe - qs > a.win_width) bits |= MLA_PLAN_ERR_QLEN;
  int64_t nb = 0;
  int64_t npages = 0;                        // sub-pages of the longest local sequence
  if (S >= 0) {
    const int64_t local_max = shard_count(S, 0, a.W, a.I);   // shard 0 holds the most
    if (local_max > a.max_kv_seq_len) bits |= MLA_PLAN_ERR_BOUND;
    nb = (local_max + a.block_size - 1) / a.block_size;
    npages = (local_max + a.page_size - 1) / a.page_size;
    if (nb > a.max_blocks) {
      bits |= MLA_PLAN_ERR_BLOCKS;
      nb = 0;
    }
  }
  const bool staged = npages <= kPlanLdsPages;  // uniform
  int bad = 0;
  for (int64_t b = tid; b < nb; b += kPlanThreads) {
    const int32_t id = b == tid ? id0 : bt[b];
    bad |= (id < 0 || (int64_t)id >= a.num_blocks);
    if (staged)
      for (int j = 0; j < per && b * per + j < npages; ++j) pages_lds[b * per + j] = id * per + j;
  }
  if (__syncthreads_or(bad)) bits |= MLA_PLAN_ERR_BLOCKS;
  if (tid == 0 && a.err_flag != nullptr) {
    uint32_t all = bits;
    if (i == 0 && (qs != 0 || q_end != a.R)) all |= MLA_PLAN_ERR_ROWS;
    if (all != 0) atomicOr(a.err_flag, all);
  }
  if (i == 0 && tid == 0 && a.qo_indptr != nullptr) a.qo_indptr[a.R] = a.R;

  // ---- this request's rows (clipped to [0, R) so a bad q_start cannot write
  // outside the outputs); a request with errors gets length 0 everywhere
  const int r0 = max(qs, 0), r1 = min(qe, a.R);
  const int Q = qe - qs;
  const int nrows = r1 - r0;
  if (nrows <= 0) return;
  const int64_t rows = (int64_t)a.W * nrows;
  const bool lens_staged = rows <= kPlanLdsRows;  // uniform
  for (int idx = tid; idx < a.W * nrows; idx += kPlanThreads) {
    const int r = idx / nrows, rho = r0 + idx % nrows;
    const int32_t L = bits ? 0 : local_len(S, Q, rho - qs, r, a.W, a.I, a.prefix_only);
    a.row_lens[(int64_t)r * a.R + rho] = L;
    if (lens_staged) len_lds[idx] = L;
    if (r == 0 && a.qo_indptr != nullptr) a.qo_indptr[rho] = rho;
  }
  if (lens_staged) __syncthreads();

  // ---- two-stage form: the second stage's window of verify tokens, one
  // length and one table row per row (row t: window rows qs .. qs + t)
  if (a.win_lens != nullptr) {
    for (int idx = tid; idx < nrows * a.win_width; idx += kPlanThreads) {
      const int rho = r0 + idx / a.win_width, k = idx % a.win_width;
      const int t = rho - qs;
      if (k == 0) a.win_lens[rho] = bits ? 0 : t + 1;
      a.win_table[(int64_t)rho * a.win_width + k] = (!bits && k <= t) ? qs + k : -1;
    }
  }

  // ---- sub-page table cells (r, rho, k): page k holds local tokens
  // [kP, (k+1)P), i.e. sub-page k % per of block k / per; cells past the
  // row's last page are -1
  if (staged && lens_staged && rows * a.pt_width < 0x7FFFFFFF) {
    // 32-bit indices; row lengths and page ids come from LDS
    const uint32_t ptw = (uint32_t)a.pt_width;
    const uint32_t cells = (uint32_t)rows * ptw;
    const int shift = __builtin_ctz((unsigned)a.page_size);
    for (uint32_t idx = tid; idx < cells; idx += kPlanThreads) {
      const uint32_t row = idx / ptw;
      const int k = (int)(idx - row * ptw);
      const int r = (int)row / nrows, rho = r0 + ((int)row - r * nrows);
      const int32_t L = len_lds[row];
      const int pages = (L + a.page_size - 1) >> shift;
      a.page_table[((int64_t)r * a.R + rho) * ptw + k] = k < pages ? pages_lds[k] : -1;
    }
    return;
  }
  const int64_t cells = rows * a.pt_width;
  for (int64_t idx = tid; idx < cells; idx += kPlanThreads) {
    const int k = (int)(idx % a.pt_width);
    const int64_t row = idx / a.pt_width;
    const int r = (int)(row / nrows), rho = r0 + (int)(row % nrows);
    const int32_t L = bits ? 0 : local_len(S, Q, rho - qs, r, a.W, a.I, a.prefix_only);
    const int pages = (L + a.page_size - 1) / a.page_size;
    int32_t v = -1;
    if (k < pages) v = bt[k / per] * per + k % per;
    a.page_table[((int64_t)r * a.R + rho) * a.pt_width + k] = v;
  }
}

}  // namespace

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  plan_kernel<<<(unsigned)a.N, kPlanThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
