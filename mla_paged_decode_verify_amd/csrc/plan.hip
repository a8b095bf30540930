// Plan kernels: rank-local row lengths and per-row sub-page tables.
//
// Row view: vLLM PR #51705 digest (prhub), Implementation breakdown item 2 and
// the _build_dcp_verify_row_view snippet -- verify row t of request i sees
// global positions [0, S_i - Q_i + t]; with round-robin interleave 1 shard r
// holds floor((w - 1 - r) / W) + 1 of the w = S_i - Q_i + 1 + t positions when
// w - 1 - r >= 0 and none otherwise.
// Sub-page table: same digest, item 3 -- the physical block table expanded to
// sub-pages of page_size tokens (block b holds sub-pages b*n .. b*n + n - 1).
#include "internal.h"

namespace mla {
namespace {

// Request owning row rho: the largest i with q_start[i] <= rho.
__device__ inline int find_request(const int32_t* q_start, int N, int rho) {
  int lo = 0, hi = N - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (q_start[mid] <= rho) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Error bits of request i (0 when it is valid).
__device__ uint32_t request_errors(const PlanArgs& a, int i) {
  uint32_t bits = 0;
  const int qs = a.q_start[i], qe = a.q_start[i + 1];
  const int S = a.seq_lens[i];
  if (qs < 0 || qe > a.R || qe - qs < 1 || S < qe - qs) bits |= MLA_PLAN_ERR_QLEN;
  if (S < 0) return bits | MLA_PLAN_ERR_QLEN;
  const int64_t local_max = ((int64_t)S + a.W - 1) / a.W;
  if (local_max > a.max_kv_seq_len) bits |= MLA_PLAN_ERR_BOUND;
  const int64_t nb = (local_max + a.block_size - 1) / a.block_size;
  if (nb > a.max_blocks) {
    bits |= MLA_PLAN_ERR_BLOCKS;
  } else {
    const int32_t* bt = a.block_table + (int64_t)i * a.max_blocks;
    for (int64_t b = 0; b < nb; ++b) {
      const int32_t id = bt[b];
      if (id < 0 || (int64_t)id >= a.num_blocks) { bits |= MLA_PLAN_ERR_BLOCKS; break; }
    }
  }
  return bits;
}

__global__ void plan_clear_kernel(uint32_t* err) { *err = 0u; }

// One thread per (shard r, row rho).
__global__ void plan_rows_kernel(PlanArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)a.W * a.R) return;
  const int r = (int)(idx / a.R);
  const int rho = (int)(idx % a.R);
  const int i = find_request(a.q_start, a.N, rho);
  uint32_t bits = request_errors(a, i);
  const int qs = a.q_start[i], qe = a.q_start[i + 1];
  if (rho < qs || rho >= qe) bits |= MLA_PLAN_ERR_QLEN;
  int32_t L = 0;
  if (bits == 0) {
    const int Q = qe - qs, t = rho - qs;
    const int w = a.seq_lens[i] - Q + 1 + t;  // window length of row t
    const int d = w - 1 - r;                  // explicit guard: C division truncates
    L = d >= 0 ? d / a.W + 1 : 0;
  }
  a.row_lens[idx] = L;
  if (bits != 0 && a.err_flag != nullptr) atomicOr(a.err_flag, bits);
  if (r == 0 && a.qo_indptr != nullptr) {
    a.qo_indptr[rho] = rho;
    if (rho == a.R - 1) a.qo_indptr[a.R] = a.R;
  }
  if (idx == 0 && a.err_flag != nullptr && a.q_start[a.N] != a.R)
    atomicOr(a.err_flag, MLA_PLAN_ERR_ROWS);
}

// One thread per (shard r, row rho, table column k).
__global__ void plan_pages_kernel(PlanArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_row = a.pt_width;
  if (idx >= (int64_t)a.W * a.R * per_row) return;
  const int64_t row = idx / per_row;  // r * R + rho
  const int k = (int)(idx % per_row);
  const int rho = (int)(row % a.R);
  const int32_t L = a.row_lens[row];
  const int pages = (L + a.page_size - 1) / a.page_size;
  int32_t v = -1;
  if (k < pages) {
    const int i = find_request(a.q_start, a.N, rho);
    const int n = a.block_size / a.page_size;
    const int64_t first = (int64_t)k * a.page_size;  // first local token of page k
    const int32_t blk = a.block_table[(int64_t)i * a.max_blocks + first / a.block_size];
    v = blk * n + (int32_t)((first % a.block_size) / a.page_size);
  }
  a.page_table[idx] = v;
}

}  // namespace

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  if (a.err_flag != nullptr) {
    plan_clear_kernel<<<1, 1, 0, s>>>(a.err_flag);
  }
  const int64_t rows = (int64_t)a.W * a.R;
  plan_rows_kernel<<<(unsigned)((rows + 255) / 256), 256, 0, s>>>(a);
  const int64_t cells = rows * a.pt_width;
  if (cells > 0) plan_pages_kernel<<<(unsigned)((cells + 255) / 256), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
