// Host side of the C ABI: argument validation, then kernel launches.
// Every check runs before anything is enqueued, so a rejected call leaves the
// stream and the caller's buffers untouched.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "internal.h"

namespace {

thread_local std::string g_last_error;

mla_status_t fail(mla_status_t code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

mla_status_t ok() {
  g_last_error.clear();
  return MLA_OK;
}

mla_status_t hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int32_t subpage_size(int32_t block_size) {
  if (block_size <= 0) return -1;
  int32_t p = 1;
  int32_t rest = block_size;
  while ((rest & 1) == 0 && p < 128) {
    rest >>= 1;
    p <<= 1;
  }
  return p;
}

int log2_exact(int32_t p) {
  int k = 0;
  while ((1 << k) < p) ++k;
  return k;
}

}  // namespace

extern "C" {

int32_t mla_subpage_size(int32_t block_size) { return subpage_size(block_size); }

int32_t mla_pt_width(int32_t max_kv_seq_len, int32_t page_size) {
  if (max_kv_seq_len < 0 || page_size <= 0) return -1;
  return (int32_t)(((int64_t)max_kv_seq_len + page_size - 1) / page_size);
}

size_t mla_verify_workspace_bytes(int32_t W, int32_t R, int32_t H, int32_t nseg) {
  if (W < 1 || R < 0 || H < 1 || nseg < 1) return 0;
  const size_t cells = (size_t)W * (size_t)R * (size_t)H * (size_t)nseg;
  return cells * (mla::kVDim + 2) * sizeof(float);
}

const char* mla_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

namespace {

// Checks shared by both plan entry points; fills everything in `a` but the
// outputs. `fn` names the entry point in error messages.
mla_status_t plan_args(const char* fn, int32_t N, const int32_t* seq_lens, const int32_t* q_start,
                       int32_t R, int32_t W, int32_t interleave, const int32_t* block_table,
                       int32_t max_blocks, int64_t num_blocks, int32_t block_size,
                       int32_t page_size, int32_t max_kv_seq_len, int32_t pt_width,
                       mla::PlanArgs& a) {
  if (N < 1) return fail(MLA_ERR_INVALID, "%s: N must be >= 1 (got %d)", fn, N);
  if (R < 1) return fail(MLA_ERR_INVALID, "%s: R must be >= 1 (got %d)", fn, R);
  if (W < 1) return fail(MLA_ERR_INVALID, "%s: W must be >= 1 (got %d)", fn, W);
  if (interleave < 1 || (int64_t)interleave * W > (1 << 30))
    return fail(MLA_ERR_INVALID,
                "%s: interleave must be >= 1 with interleave * W <= 2^30 (got %d)", fn,
                interleave);
  if (block_size <= 0)
    return fail(MLA_ERR_INVALID, "%s: block_size must be > 0 (got %d)", fn, block_size);
  if (page_size != subpage_size(block_size))
    return fail(MLA_ERR_INVALID, "%s: page_size %d != sub-page size %d of block_size %d", fn,
                page_size, subpage_size(block_size), block_size);
  if (max_blocks < 1)
    return fail(MLA_ERR_INVALID, "%s: max_blocks must be >= 1 (got %d)", fn, max_blocks);
  if (num_blocks < 1) return fail(MLA_ERR_INVALID, "%s: num_blocks must be >= 1", fn);
  if (num_blocks * (int64_t)(block_size / page_size) > 0x7FFFFFFFLL)
    return fail(MLA_ERR_INVALID, "%s: too many sub-pages for int32 ids", fn);
  if (max_kv_seq_len < 0) return fail(MLA_ERR_INVALID, "%s: max_kv_seq_len must be >= 0", fn);
  if (pt_width < mla_pt_width(max_kv_seq_len, page_size) || pt_width < 0)
    return fail(MLA_ERR_INVALID, "%s: pt_width %d < ceil(max_kv_seq_len/page_size) = %d", fn,
                pt_width, mla_pt_width(max_kv_seq_len, page_size));
  if ((int64_t)W * R * (int64_t)(pt_width > 0 ? pt_width : 1) > (1LL << 40))
    return fail(MLA_ERR_INVALID, "%s: page table too large", fn);
  if (!seq_lens || !q_start || !block_table)
    return fail(MLA_ERR_INVALID, "%s: null tensor argument", fn);

  a = mla::PlanArgs{};
  a.N = N; a.R = R; a.W = W; a.I = interleave;
  a.seq_lens = seq_lens; a.q_start = q_start; a.block_table = block_table;
  a.max_blocks = max_blocks; a.num_blocks = num_blocks;
  a.block_size = block_size; a.page_size = page_size;
  a.max_kv_seq_len = max_kv_seq_len; a.pt_width = pt_width;
  return MLA_OK;
}

}  // namespace

extern "C" {

mla_status_t mla_verify_plan(int32_t N, const int32_t* seq_lens, const int32_t* q_start,
                             int32_t R, int32_t W, int32_t interleave,
                             const int32_t* block_table, int32_t max_blocks,
                             int64_t num_blocks, int32_t block_size, int32_t page_size,
                             int32_t max_kv_seq_len, int32_t pt_width, int32_t* row_lens,
                             int32_t* page_table, int32_t* qo_indptr, uint32_t* err_flag,
                             void* stream) {
  const char* fn = "mla_verify_plan";
  mla::PlanArgs a;
  const mla_status_t st = plan_args(fn, N, seq_lens, q_start, R, W, interleave, block_table,
                                    max_blocks, num_blocks, block_size, page_size,
                                    max_kv_seq_len, pt_width, a);
  if (st != MLA_OK) return st;
  if (!row_lens || (pt_width > 0 && !page_table))
    return fail(MLA_ERR_INVALID, "%s: null tensor argument", fn);
  a.row_lens = row_lens; a.page_table = page_table; a.qo_indptr = qo_indptr;
  a.err_flag = err_flag;
  return hip_status(mla::launch_plan(a, (hipStream_t)stream), "mla_verify_plan launch");
}

mla_status_t mla_verify_two_stage_plan(int32_t N, const int32_t* seq_lens,
                                       const int32_t* q_start, int32_t R, int32_t W,
                                       int32_t interleave, const int32_t* block_table,
                                       int32_t max_blocks, int64_t num_blocks,
                                       int32_t block_size, int32_t page_size,
                                       int32_t max_kv_seq_len, int32_t pt_width,
                                       int32_t max_qlen, int32_t* row_lens,
                                       int32_t* page_table, int32_t* window_table,
                                       uint32_t* err_flag, void* stream) {
  const char* fn = "mla_verify_two_stage_plan";
  mla::PlanArgs a;
  const mla_status_t st = plan_args(fn, N, seq_lens, q_start, R, W, interleave, block_table,
                                    max_blocks, num_blocks, block_size, page_size,
                                    max_kv_seq_len, pt_width, a);
  if (st != MLA_OK) return st;
  if (max_qlen < 1)
    return fail(MLA_ERR_INVALID, "%s: max_qlen must be >= 1 (got %d)", fn, max_qlen);
  if ((int64_t)R * max_qlen > (1LL << 40))
    return fail(MLA_ERR_INVALID, "%s: window table too large", fn);
  if (!row_lens || (pt_width > 0 && !page_table) || !window_table)
    return fail(MLA_ERR_INVALID, "%s: null tensor argument", fn);
  a.row_lens = row_lens; a.page_table = page_table; a.qo_indptr = nullptr;
  a.err_flag = err_flag;
  a.prefix_only = 1;
  a.win_lens = row_lens + (int64_t)W * R;   // the extra source's row of row_lens
  a.win_table = window_table;
  a.win_width = max_qlen;
  return hip_status(mla::launch_plan(a, (hipStream_t)stream),
                    "mla_verify_two_stage_plan launch");
}

}  // extern "C"

namespace {

// Checks shared by both attention entry points; fills everything in `a` but
// the outputs. `fn` names the entry point in error messages.
mla_status_t attn_args(const char* fn, const void* q, const void* kv, int64_t num_blocks,
                       int32_t block_size, int32_t page_size, mla_kv_dtype_t kv_dtype,
                       float kv_scale, float sm_scale, const int32_t* row_lens,
                       const int32_t* page_table, int32_t pt_width, const int32_t* q_start,
                       int32_t N, int32_t R, int32_t H, int32_t W, int32_t max_qlen,
                       int32_t nseg, mla::AttnArgs& a, bool& fp8) {
  if (N < 1 || R < 1 || H < 1 || W < 1)
    return fail(MLA_ERR_INVALID, "%s: N, R, H, W must be >= 1 (got %d, %d, %d, %d)", fn, N, R,
                H, W);
  if (nseg < 1) return fail(MLA_ERR_INVALID, "%s: nseg must be >= 1 (got %d)", fn, nseg);
  if (max_qlen < 1) return fail(MLA_ERR_INVALID, "%s: max_qlen must be >= 1", fn);
  if (block_size <= 0 || page_size != subpage_size(block_size))
    return fail(MLA_ERR_INVALID, "%s: page_size %d does not match block_size %d", fn,
                page_size, block_size);
  if (num_blocks < 1) return fail(MLA_ERR_INVALID, "%s: num_blocks must be >= 1", fn);
  if (pt_width < 0) return fail(MLA_ERR_INVALID, "%s: pt_width must be >= 0", fn);
  if (kv_dtype != MLA_KV_BF16 && kv_dtype != MLA_KV_FP8_E4M3 && kv_dtype != MLA_KV_FP8_E5M2)
    return fail(MLA_ERR_UNSUPPORTED, "%s: unknown kv_dtype %d", fn, (int)kv_dtype);
  fp8 = kv_dtype != MLA_KV_BF16;
  const double log2e = 1.4426950408889634;
  const float qk_scale_log2 = (float)((double)sm_scale * (fp8 ? (double)kv_scale : 1.0) * log2e);
  // the kernels take the row maximum of unscaled scores, which needs a
  // positive scale that stays positive and finite in fp32
  if (!(sm_scale > 0.f) || !std::isfinite(sm_scale) ||
      (fp8 && (!(kv_scale > 0.f) || !std::isfinite(kv_scale))) || !(qk_scale_log2 > 0.f) ||
      !std::isfinite(qk_scale_log2))
    return fail(MLA_ERR_INVALID, "%s: scales must be positive and finite", fn);
  if (!q || !kv || !row_lens || !q_start || (pt_width > 0 && !page_table))
    return fail(MLA_ERR_INVALID, "%s: null tensor argument", fn);
  if (!aligned16(q) || !aligned16(kv))
    return fail(MLA_ERR_INVALID, "%s: q and kv must be 16-byte aligned", fn);
  const int64_t mblocks = ((int64_t)max_qlen * H + mla::kAttnRows - 1) / mla::kAttnRows;
  if ((int64_t)N * W * nseg * mblocks > 0x7FFFFFFFLL)
    return fail(MLA_ERR_INVALID, "%s: grid too large", fn);

  a = mla::AttnArgs{};
  a.q = static_cast<const uint16_t*>(q);
  a.kv = static_cast<const uint8_t*>(kv);
  a.pool_tokens = num_blocks * block_size;
  a.num_subpages = num_blocks * (block_size / page_size);
  a.page_size = page_size;
  a.page_shift = log2_exact(page_size);
  a.row_lens = row_lens; a.page_table = page_table; a.pt_width = pt_width;
  a.q_start = q_start; a.N = N; a.R = R; a.H = H; a.W = W; a.nseg = nseg;
  a.mblocks = (int32_t)mblocks;
  a.qk_scale_log2 = qk_scale_log2;
  a.v_scale = fp8 ? kv_scale : 1.0f;
  a.e5m2 = kv_dtype == MLA_KV_FP8_E5M2 ? 1 : 0;
  return MLA_OK;
}

}  // namespace

extern "C" {

mla_status_t mla_verify_attn(const void* q, const void* kv, int64_t num_blocks,
                             int32_t block_size, int32_t page_size, mla_kv_dtype_t kv_dtype,
                             float kv_scale, float sm_scale, const int32_t* row_lens,
                             const int32_t* page_table, int32_t pt_width,
                             const int32_t* q_start, int32_t N, int32_t R, int32_t H,
                             int32_t W, int32_t max_qlen, int32_t nseg, float* segm_out,
                             float* segm_max, float* segm_expsum, void* stream) {
  const char* fn = "mla_verify_attn";
  mla::AttnArgs a;
  bool fp8 = false;
  const mla_status_t st = attn_args(fn, q, kv, num_blocks, block_size, page_size, kv_dtype,
                                    kv_scale, sm_scale, row_lens, page_table, pt_width, q_start,
                                    N, R, H, W, max_qlen, nseg, a, fp8);
  if (st != MLA_OK) return st;
  if (!segm_out || !segm_max || !segm_expsum)
    return fail(MLA_ERR_INVALID, "%s: null tensor argument", fn);
  if (!aligned16(segm_out))
    return fail(MLA_ERR_INVALID, "%s: segm_out must be 16-byte aligned", fn);
  a.segm_out = segm_out; a.segm_max = segm_max; a.segm_expsum = segm_expsum;
  return hip_status(mla::launch_attn(a, fp8, (hipStream_t)stream), "mla_verify_attn launch");
}

mla_status_t mla_verify_attn_shard(const void* q, const void* kv, int64_t num_blocks,
                                   int32_t block_size, int32_t page_size,
                                   mla_kv_dtype_t kv_dtype, float kv_scale, float sm_scale,
                                   const int32_t* row_lens, const int32_t* page_table,
                                   int32_t pt_width, const int32_t* q_start, int32_t N,
                                   int32_t R, int32_t H, int32_t W, int32_t max_qlen,
                                   int32_t nseg, void* shard_out, float* shard_lse,
                                   void* stream) {
  const char* fn = "mla_verify_attn_shard";
  mla::AttnArgs a;
  bool fp8 = false;
  const mla_status_t st = attn_args(fn, q, kv, num_blocks, block_size, page_size, kv_dtype,
                                    kv_scale, sm_scale, row_lens, page_table, pt_width, q_start,
                                    N, R, H, W, max_qlen, nseg, a, fp8);
  if (st != MLA_OK) return st;
  if (!shard_out || !shard_lse) return fail(MLA_ERR_INVALID, "%s: null tensor argument", fn);
  if (!aligned16(shard_out))
    return fail(MLA_ERR_INVALID, "%s: shard_out must be 16-byte aligned", fn);
  a.shard_out = static_cast<uint16_t*>(shard_out); a.shard_lse = shard_lse;
  return hip_status(mla::launch_attn(a, fp8, (hipStream_t)stream),
                    "mla_verify_attn_shard launch");
}

namespace {

// Groups of the persistent schedule, and the byte size of its counters
// (padded so that the slots start 256-byte aligned).
int64_t persist_groups(int32_t N, int32_t W, int32_t H, int32_t max_qlen) {
  const int64_t mblocks = ((int64_t)max_qlen * H + mla::kAttnRows - 1) / mla::kAttnRows;
  return (int64_t)N * W * mblocks;
}
size_t persist_counter_bytes(int64_t groups) { return ((size_t)groups * 4 + 255) / 256 * 256; }

}  // namespace

size_t mla_verify_attn_persistent_workspace_bytes(int32_t N, int32_t W, int32_t H,
                                                  int32_t max_qlen, int32_t ctas) {
  if (N < 1 || W < 1 || H < 1 || max_qlen < 1 || ctas < 0) return 0;
  if (ctas == 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
      return 0;
    ctas = cus;
  }
  return persist_counter_bytes(persist_groups(N, W, H, max_qlen)) +
         (size_t)2 * (size_t)ctas * mla::kPersistSlotBytes;
}

mla_status_t mla_verify_attn_persistent(const void* q, const void* kv, int64_t num_blocks,
                                        int32_t block_size, int32_t page_size,
                                        mla_kv_dtype_t kv_dtype, float kv_scale, float sm_scale,
                                        const int32_t* row_lens, const int32_t* page_table,
                                        int32_t pt_width, const int32_t* q_start, int32_t N,
                                        int32_t R, int32_t H, int32_t W, int32_t max_qlen,
                                        int32_t ctas, void* workspace, size_t workspace_bytes,
                                        void* shard_out, float* shard_lse, void* stream) {
  const char* fn = "mla_verify_attn_persistent";
  mla::AttnArgs a;
  bool fp8 = false;
  const mla_status_t st = attn_args(fn, q, kv, num_blocks, block_size, page_size, kv_dtype,
                                    kv_scale, sm_scale, row_lens, page_table, pt_width, q_start,
                                    N, R, H, W, max_qlen, 1, a, fp8);
  if (st != MLA_OK) return st;
  if (!shard_out || !shard_lse || !workspace)
    return fail(MLA_ERR_INVALID, "%s: null tensor argument", fn);
  if (!aligned16(shard_out))
    return fail(MLA_ERR_INVALID, "%s: shard_out must be 16-byte aligned", fn);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(MLA_ERR_INVALID, "%s: workspace must be 256-byte aligned", fn);
  if (ctas < 0 || ctas > 65536)
    return fail(MLA_ERR_INVALID, "%s: ctas must be 0 .. 65536 (got %d)", fn, ctas);
  const int64_t groups = persist_groups(N, W, H, max_qlen);
  const int64_t tiles_per_row = ((int64_t)pt_width * page_size + 63) / 64;
  if (groups > mla::kPersistMaxGroups)
    return fail(MLA_ERR_UNSUPPORTED, "%s: %lld groups (N * W * row blocks) > %d", fn,
                (long long)groups, mla::kPersistMaxGroups);
  if ((int64_t)pt_width * page_size >= (1LL << 30) || groups * tiles_per_row >= (1LL << 31))
    return fail(MLA_ERR_UNSUPPORTED, "%s: too many tiles for the schedule", fn);
  if (ctas == 0) {
    int dev = 0, cus = 0;
    const hipError_t e1 = hipGetDevice(&dev);
    if (e1 != hipSuccess) return hip_status(e1, fn);
    const hipError_t e2 = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e2 != hipSuccess) return hip_status(e2, fn);
    ctas = cus > 0 ? cus : 1;
  }
  const size_t need = persist_counter_bytes(groups) + (size_t)2 * ctas * mla::kPersistSlotBytes;
  if (workspace_bytes < need)
    return fail(MLA_ERR_INVALID, "%s: workspace of %zu bytes < %zu needed", fn, workspace_bytes,
                need);
  a.shard_out = static_cast<uint16_t*>(shard_out);
  a.shard_lse = shard_lse;
  mla::PersistArgs p{};
  p.counters = static_cast<int32_t*>(workspace);
  p.slots = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) +
                                     persist_counter_bytes(groups));
  p.ctas = ctas;
  return hip_status(mla::launch_attn_persist(a, p, fp8, (hipStream_t)stream), fn);
}

}  // extern "C"

namespace {

// Checks of the one-call attention + merge; fills `a` but the partials.
mla_status_t attn_merge_args(const char* fn, const void* q, const void* kv, int64_t num_blocks,
                             int32_t block_size, int32_t page_size, mla_kv_dtype_t kv_dtype,
                             float kv_scale, float sm_scale, const int32_t* row_lens,
                             const int32_t* page_table, int32_t pt_width,
                             const int32_t* q_start, int32_t N, int32_t R, int32_t H, int32_t W,
                             int32_t max_qlen, int32_t nseg, void* out, float* lse,
                             mla::AttnArgs& a, bool& fp8) {
  const mla_status_t st = attn_args(fn, q, kv, num_blocks, block_size, page_size, kv_dtype,
                                    kv_scale, sm_scale, row_lens, page_table, pt_width, q_start,
                                    N, R, H, W, max_qlen, nseg, a, fp8);
  if (st != MLA_OK) return st;
  if (!out || !lse) return fail(MLA_ERR_INVALID, "%s: null tensor argument", fn);
  if (!aligned16(out)) return fail(MLA_ERR_INVALID, "%s: out must be 16-byte aligned", fn);
  return MLA_OK;
}

// Attention partials into `ws` (segm_out | segm_max | segm_expsum, the
// layout of mla_verify_workspace_bytes) then the segment + shard merge.
mla_status_t attn_merge_launch(const char* fn, mla::AttnArgs& a, bool fp8, unsigned char* ws,
                               const int32_t* row_lens, const int32_t* q_start, int32_t page_size,
                               void* out, float* lse, hipStream_t stream) {
  const size_t cells = (size_t)a.W * (size_t)a.R * (size_t)a.H * (size_t)a.nseg;
  a.segm_out = reinterpret_cast<float*>(ws);
  a.segm_max = a.segm_out + cells * mla::kVDim;
  a.segm_expsum = a.segm_max + cells;
  const mla_status_t st = hip_status(mla::launch_attn(a, fp8, stream), fn);
  if (st != MLA_OK) return st;
  mla::MergeArgs m{};
  m.segm_out = a.segm_out; m.segm_max = a.segm_max; m.segm_expsum = a.segm_expsum;
  m.row_lens = row_lens; m.q_start = q_start; m.N = a.N; m.page_size = page_size;
  m.R = a.R; m.H = a.H; m.W = a.W; m.nseg = a.nseg;
  m.out = static_cast<uint16_t*>(out); m.lse = lse;
  return hip_status(mla::launch_merge(m, stream), fn);
}

}  // namespace

extern "C" {

mla_status_t mla_verify_attn_merge(const void* q, const void* kv, int64_t num_blocks,
                                   int32_t block_size, int32_t page_size,
                                   mla_kv_dtype_t kv_dtype, float kv_scale, float sm_scale,
                                   const int32_t* row_lens, const int32_t* page_table,
                                   int32_t pt_width, const int32_t* q_start, int32_t N,
                                   int32_t R, int32_t H, int32_t W, int32_t max_qlen,
                                   int32_t nseg, void* workspace, size_t workspace_bytes,
                                   void* out, float* lse, void* stream) {
  const char* fn = "mla_verify_attn_merge";
  mla::AttnArgs a;
  bool fp8 = false;
  const mla_status_t st =
      attn_merge_args(fn, q, kv, num_blocks, block_size, page_size, kv_dtype, kv_scale,
                      sm_scale, row_lens, page_table, pt_width, q_start, N, R, H, W, max_qlen,
                      nseg, out, lse, a, fp8);
  if (st != MLA_OK) return st;
  const size_t need = mla_verify_workspace_bytes(W, R, H, nseg);
  if (!workspace) return fail(MLA_ERR_INVALID, "%s: null workspace", fn);
  if (!aligned16(workspace))
    return fail(MLA_ERR_INVALID, "%s: workspace must be 16-byte aligned", fn);
  if (workspace_bytes < need)
    return fail(MLA_ERR_INVALID, "%s: workspace of %zu bytes < %zu needed", fn,
                workspace_bytes, need);
  return attn_merge_launch(fn, a, fp8, static_cast<unsigned char*>(workspace), row_lens,
                           q_start, page_size, out, lse, (hipStream_t)stream);
}

mla_status_t mla_verify_attn_merge_static(const void* q, const void* kv, int64_t num_blocks,
                                          int32_t block_size, int32_t page_size,
                                          mla_kv_dtype_t kv_dtype, float kv_scale,
                                          float sm_scale, const int32_t* row_lens,
                                          const int32_t* page_table, int32_t pt_width,
                                          const int32_t* q_start, int32_t N, int32_t R,
                                          int32_t H, int32_t W, int32_t max_qlen, int32_t nseg,
                                          void* out, float* lse, void* stream) {
  const char* fn = "mla_verify_attn_merge_static";
  mla::AttnArgs a;
  bool fp8 = false;
  const mla_status_t st =
      attn_merge_args(fn, q, kv, num_blocks, block_size, page_size, kv_dtype, kv_scale,
                      sm_scale, row_lens, page_table, pt_width, q_start, N, R, H, W, max_qlen,
                      nseg, out, lse, a, fp8);
  if (st != MLA_OK) return st;
  const size_t need = mla_verify_workspace_bytes(W, R, H, nseg);
  if (need > MLA_STATIC_SCRATCH_BYTES)
    return fail(MLA_ERR_INVALID,
                "%s: the partials need %zu bytes, more than the %llu of the static scratch "
                "array (use mla_verify_attn_merge with a workspace)",
                fn, need, (unsigned long long)MLA_STATIC_SCRATCH_BYTES);
  void* ws = nullptr;
  const hipError_t e = mla::static_scratch(&ws);
  if (e != hipSuccess)
    return fail(MLA_ERR_HIP, "%s: static scratch address: %s", fn, hipGetErrorString(e));
  return attn_merge_launch(fn, a, fp8, static_cast<unsigned char*>(ws), row_lens, q_start,
                           page_size, out, lse, (hipStream_t)stream);
}

mla_status_t mla_lse_merge(const float* segm_out, const float* segm_max,
                           const float* segm_expsum, const int32_t* row_lens,
                           const int32_t* q_start, int32_t N, int32_t page_size, int32_t R,
                           int32_t H, int32_t W, int32_t nseg, void* shard_out,
                           float* shard_lse, void* out, float* lse, void* stream) {
  if (N < 1 || R < 1 || H < 1 || W < 1)
    return fail(MLA_ERR_INVALID, "mla_lse_merge: N, R, H, W must be >= 1");
  if (nseg < 1) return fail(MLA_ERR_INVALID, "mla_lse_merge: nseg must be >= 1");
  if (page_size <= 0 || (page_size & (page_size - 1)) != 0 || page_size > 128)
    return fail(MLA_ERR_INVALID, "mla_lse_merge: page_size must be a power of two <= 128");
  if (!segm_out || !segm_max || !segm_expsum || !row_lens || !q_start || !out || !lse)
    return fail(MLA_ERR_INVALID, "mla_lse_merge: null tensor argument");
  if (!aligned16(segm_out) || !aligned16(out) || (shard_out && !aligned16(shard_out)))
    return fail(MLA_ERR_INVALID, "mla_lse_merge: segm_out, out, shard_out must be 16-byte aligned");
  mla::MergeArgs a{};
  a.segm_out = segm_out; a.segm_max = segm_max; a.segm_expsum = segm_expsum;
  a.row_lens = row_lens; a.q_start = q_start; a.N = N; a.page_size = page_size;
  a.R = R; a.H = H; a.W = W; a.nseg = nseg;
  a.shard_out = static_cast<uint16_t*>(shard_out); a.shard_lse = shard_lse;
  a.out = static_cast<uint16_t*>(out); a.lse = lse;
  return hip_status(mla::launch_merge(a, (hipStream_t)stream), "mla_lse_merge launch");
}

mla_status_t mla_shard_merge(const void* shard_out, const float* shard_lse, int32_t R,
                             int32_t H, int32_t W, void* out, float* lse, void* stream) {
  if (R < 1 || H < 1 || W < 1)
    return fail(MLA_ERR_INVALID, "mla_shard_merge: R, H, W must be >= 1 (got %d, %d, %d)", R, H,
                W);
  if (W > mla::kShardMergeMaxW)
    return fail(MLA_ERR_UNSUPPORTED, "mla_shard_merge: W %d > %d", W, mla::kShardMergeMaxW);
  if (!shard_out || !shard_lse || !out || !lse)
    return fail(MLA_ERR_INVALID, "mla_shard_merge: null tensor argument");
  if (!aligned16(shard_out) || !aligned16(out))
    return fail(MLA_ERR_INVALID, "mla_shard_merge: shard_out and out must be 16-byte aligned");
  mla::ShardMergeArgs a{};
  a.shard_out = static_cast<const uint16_t*>(shard_out); a.shard_lse = shard_lse;
  a.R = R; a.H = H; a.W = W;
  a.out = static_cast<uint16_t*>(out); a.lse = lse;
  return hip_status(mla::launch_shard_merge(a, (hipStream_t)stream), "mla_shard_merge launch");
}

}  // extern "C"
