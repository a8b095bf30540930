/*
 * mla_verify.h -- C ABI of the MI355X (gfx950) paged MLA decode / causal
 * multi-token verify path over a round-robin context-sharded KV cache.
 *
 * Sources (web pages, cited by title and section):
 *   [V51705] prhub digest of vLLM PR #51705, "ROCm AITER MLA supports causal
 *            multi-token speculative verify under DCP"
 *   [S34432] prhub report of SGLang PR #34432, "[AMD][DCP 1/N] add dcp support
 *            for aiter backend"
 *   [V51011] prhub digest of vLLM PR #51011, "fix silent wrong decode for fp8
 *            KV in ROCm AITER MLA"
 *
 * Notation. N requests; request i has S_i cached tokens (its Q_i verify tokens
 * included, all already written to the cache) and Q_i >= 1 verify rows. Rows
 * are request-major: row rho = q_start[i] + t, t in [0, Q_i), R = q_start[N].
 * W shards hold each sequence round-robin with interleave I (default 1): runs
 * of I consecutive positions are dealt to shards 0, 1, ..., W-1 in turn, so
 * global position p lives on shard (p / I) % W at local index
 * (p / (I W)) I + p % I (for I = 1: shard p % W, local index p / W). H heads. Head dim 576 = 512
 * latent + 64 rope; V is the 512 latent values of the same cache entry.
 *
 * Conventions for every call below.
 *   - Tensor arguments are DEVICE pointers to contiguous row-major arrays,
 *     allocated and owned by the caller. The library allocates no device
 *     memory at run time and keeps no state except a thread-local error
 *     string and the static scratch array of mla_verify_attn_merge_static.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; 0 = the
 *     default stream). Nothing synchronises.
 *   - Scalar arguments are validated on the host before anything is
 *     launched: a bad value returns MLA_ERR_INVALID (or MLA_ERR_UNSUPPORTED
 *     for a layout the library does not implement) and launches nothing;
 *     mla_last_error() then describes it. A failed launch returns
 *     MLA_ERR_HIP. Device data the host cannot see without a sync is checked
 *     by mla_verify_plan on the device (see err_flag).
 */
#ifndef MLA_VERIFY_H_
#define MLA_VERIFY_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID = 1,     /* bad argument; nothing was launched            */
  MLA_ERR_UNSUPPORTED = 2, /* valid but not implemented (e.g. unknown kv dtype) */
  MLA_ERR_HIP = 3          /* a HIP launch failed                           */
} mla_status_t;

typedef enum {
  MLA_KV_BF16 = 0,     /* bf16 cache entries, 1152 bytes per token           */
  MLA_KV_FP8_E4M3 = 1, /* OCP e4m3fn codes, 576 bytes per token, real value =
                          code * kv_scale (one per-tensor float scale)       */
  MLA_KV_FP8_E5M2 = 2  /* OCP e5m2 codes (the fp8_e5m2 cache dtype of the
                          [V51011] fp8 routing test grid), 576 bytes per
                          token, real value = code * kv_scale               */
} mla_kv_dtype_t;

#define MLA_HEAD_DIM 576
#define MLA_V_DIM 512

/* Device error bits ORed into *err_flag by mla_verify_plan. A request with
 * any of these problems gets row length 0 on every shard and an all -1
 * sub-page table, so later calls never read outside the caller's buffers. */
#define MLA_PLAN_ERR_QLEN 1u    /* Q_i < 1, S_i < Q_i, or q_start not monotone  */
#define MLA_PLAN_ERR_BOUND 2u   /* longest local sequence of request i (shard
                                   0's; ceil(S_i / W) for interleave 1) >
                                   max_kv_seq_len                              */
#define MLA_PLAN_ERR_BLOCKS 4u  /* request needs more than max_blocks blocks, or
                                   a block id it uses is outside [0,num_blocks) */
#define MLA_PLAN_ERR_ROWS 8u    /* q_start[N] != R                              */

/*
 * Sub-page size for a physical block size: the largest power of two that
 * divides block_size, capped at 128 ([V51705] Implementation breakdown item 3,
 * `_segmented_mla_page_size` snippet). It is the tile unit of the split-K
 * partition. Returns -1 if block_size <= 0. Host only.
 */
int32_t mla_subpage_size(int32_t block_size);

/*
 * Width of the per-row sub-page table: ceil(max_kv_seq_len / page_size).
 * max_kv_seq_len is the kernel-visible bound on any shard-local length
 * ([V51705] `AiterMLADCPVerifyMetadata.max_kv_seq_len`); a fixed configured
 * bound keeps the table shape stable between calls. Returns -1 on bad input.
 */
int32_t mla_pt_width(int32_t max_kv_seq_len, int32_t page_size);

/*
 * Bytes of the three split-K partial buffers for W shards, R rows, H heads and
 * nseg segments: segm_out (W*R*H*nseg*512 floats) + segm_max and segm_expsum
 * (W*R*H*nseg floats each). These are the per-segment output, base-2 maximum
 * and exp2 sum that the segment merge folds ([V51705] Implementation
 * breakdown item 4 and the `merge_mla_segments_triton` snippet, whose
 * segm_output / segm_max / segm_expsum arguments carry one 512-wide output and
 * two scalars per row, head and segment). Returns 0 on bad input. Host only.
 */
size_t mla_verify_workspace_bytes(int32_t W, int32_t R, int32_t H, int32_t nseg);

/*
 * Plan: rank-local row lengths and sub-page tables for every verify row on
 * every shard ([V51705] Implementation breakdown items 2-3 and the
 * `_build_dcp_verify_row_view` / `AiterMLADCPVerifyMetadata` snippets).
 * Built once per forward, shared by every layer.
 *
 *   seq_lens    [N]   int32  S_i
 *   q_start     [N+1] int32  row offsets (q_start[0] = 0, q_start[N] = R)
 *   interleave  I >= 1, with I * W <= 2^30 (else MLA_ERR_INVALID). The
 *               pages' routing accepts only I = 1 ([V51705]: the per-row
 *               window is verified only for interleave 1); I > 1 follows the
 *               placement above, under which every row's window is still a
 *               prefix of each shard's local sequence: shard r holds
 *               c I + clamp(rem - r I, 0, I) positions of a window of w, with
 *               c = w / (I W), rem = w % (I W). The bound check uses the
 *               longest local sequence, shard 0's.
 *   block_table [N, max_blocks] int32 physical block ids, one table shared by
 *               every shard's pool; local token j of request i is in block
 *               block_table[i][j / block_size] at offset j % block_size
 *   num_blocks  blocks in each shard's pool (ids must be < num_blocks)
 *   page_size   must equal mla_subpage_size(block_size) (carried explicitly,
 *               never re-derived from a cache shape: [V51705] snippet)
 *   pt_width    must be >= mla_pt_width(max_kv_seq_len, page_size)
 * Outputs (device):
 *   row_lens    [W, R] int32  L[r][rho] = #{ p < w : p % W == r } with the
 *               window w = S_i - Q_i + 1 + t (row t sees global positions
 *               [0, S_i - Q_i + t], its own token included)
 *   page_table  [W, R, pt_width] int32 sub-page ids; entry k < ceil(L/P) is
 *               block_table[i][k*P / B] * (B/P) + (k*P % B) / P, the rest -1
 *   qo_indptr   [R+1] int32 = 0..R (one query per row); may be NULL
 *   err_flag    [1] uint32, may be NULL: the MLA_PLAN_ERR_* bits of every
 *               invalid request are ORed into it. The library never clears
 *               it (sticky, like a device error flag): a caller zeroes it
 *               once and again after handling an error; it then stays 0 as
 *               long as every request of every call is valid.
 */
mla_status_t mla_verify_plan(int32_t N, const int32_t* seq_lens,
                             const int32_t* q_start, int32_t R, int32_t W,
                             int32_t interleave, const int32_t* block_table,
                             int32_t max_blocks, int64_t num_blocks,
                             int32_t block_size, int32_t page_size,
                             int32_t max_kv_seq_len, int32_t pt_width,
                             int32_t* row_lens, int32_t* page_table,
                             int32_t* qo_indptr, uint32_t* err_flag,
                             void* stream);

/*
 * Two-stage verify plan: the metadata of the SGLang decomposition of the same
 * verify result ([S34432] Implementation breakdown items 2-3 and the
 * `_forward_verify_dcp` snippet: a per-row local KV length and a per-row 2-D
 * token table for the committed prefix, read row by row, plus a dense causal
 * window over the verify tokens computed by one source, merged by LSE). Built
 * once per forward on the device; the attention and merge calls below then
 * run it unchanged:
 *   stage 1  every shard attends over its part of the request's committed
 *            prefix [0, S_i - Q_i): row_lens[r][rho] = positions of the
 *            prefix that shard r holds (the same for every row of a request),
 *            page_table[r][rho] = their sub-pages, exactly as mla_verify_plan
 *            builds them for a window of S_i - Q_i. Run mla_verify_attn with
 *            row_lens rows 0..W-1, page_table, q_start, nseg 1.
 *   stage 2  one extra source attends over the dense causal window of the
 *            request's Q_i verify tokens: row t sees verify tokens 0..t, so
 *            row_lens[W][rho] = t + 1 and window_table[rho][k] = q_start[i] + k
 *            for k <= t, else -1: the row of verify token k in a caller's
 *            window buffer [R, 576] that holds the verify tokens' cache
 *            entries request-major (as on the page). Run mla_verify_attn with
 *            kv = that buffer viewed as [1, R, 1, 576] (num_blocks R,
 *            block_size 1, page_size 1), row_lens row W, window_table as
 *            page_table (pt_width = max_qlen), q_start, W = 1, nseg 1.
 *   merge    mla_lse_merge over the W + 1 sources (row_lens [W+1, R], nseg 1).
 *
 *   N, seq_lens, q_start, R, W, interleave, block_table, max_blocks,
 *   num_blocks, block_size, page_size, max_kv_seq_len, pt_width: as for
 *              mla_verify_plan (same checks, same error codes)
 *   max_qlen   >= 1, the width of window_table; a request with Q_i above it
 *              gets MLA_PLAN_ERR_QLEN (and length 0, table -1 everywhere)
 * Outputs (device):
 *   row_lens     [W+1, R] int32 (stage-1 rows 0..W-1, stage-2 row W)
 *   page_table   [W, R, pt_width] int32
 *   window_table [R, max_qlen] int32
 *   err_flag     as for mla_verify_plan (sticky; may be NULL). An empty
 *                committed prefix (S_i = Q_i) is no error: its stage-1
 *                lengths are 0.
 */
mla_status_t mla_verify_two_stage_plan(int32_t N, const int32_t* seq_lens,
                                       const int32_t* q_start, int32_t R,
                                       int32_t W, int32_t interleave,
                                       const int32_t* block_table,
                                       int32_t max_blocks, int64_t num_blocks,
                                       int32_t block_size, int32_t page_size,
                                       int32_t max_kv_seq_len, int32_t pt_width,
                                       int32_t max_qlen, int32_t* row_lens,
                                       int32_t* page_table,
                                       int32_t* window_table,
                                       uint32_t* err_flag, void* stream);

/*
 * Split-K segmented attention partials for every (shard, row, head, segment)
 * ([V51705] Implementation breakdown item 4 and the merge snippet).
 *
 *   q          [R, H, 576] bf16 queries (RoPE already applied)
 *   kv         [W, num_blocks, block_size, 576] cache: one pool per shard,
 *              elements bf16, e4m3fn or e5m2 per kv_dtype; 16-byte aligned
 *   kv_scale   fp8 descale (real = code * kv_scale), > 0; ignored for bf16.
 *              fp8 caches run on the fp8 matrix cores: the codes against Q and
 *              the softmax weights, each as two e4m3fn terms (Q exact for a
 *              bf16 input down to 2^-13 of its row's largest, below that
 *              within 2^-21 of it; each weight within 2^-8 of itself plus
 *              2^-14)
 *   sm_scale   softmax scale applied to <q, k> (e.g. 1/sqrt(576)), > 0; the
 *              product sm_scale * kv_scale * log2(e) must be a positive
 *              finite fp32 value, else MLA_ERR_INVALID
 *   row_lens, page_table, pt_width, page_size: from mla_verify_plan
 *   q_start    [N+1] as given to the plan
 *   max_qlen   >= every Q_i: it sizes the grid (ceil(max_qlen*H/64) row
 *              blocks per request). The (row, head) pairs of a longer request
 *              past that coverage get NaN partials (NaN shard outputs and
 *              LSEs in mla_verify_attn_shard), which the merges carry into
 *              out and lse: never an unwritten or silently wrong value.
 *   nseg       segments per (request, shard) group. Partition (a reading of
 *              the pages' tiles_per_segment = ceil(len/(nseg*TILE))): with Lg
 *              the group's longest row (its last), T = ceil(Lg/(nseg*P)) and
 *              segment s covers local tokens [s*T*P, (s+1)*T*P), clipped to
 *              each row's own length.
 * Outputs (device, fp32), index e = ((r*R + rho)*H + h)*nseg + s:
 *   segm_max[e]    max over the segment of sm_scale*<q,k>*log2(e)  (base 2)
 *   segm_expsum[e] sum over the segment of 2^(score2 - segm_max[e])
 *   segm_out[e*512 + d] sum of 2^(score2 - segm_max[e]) * v[d]  (unnormalised)
 * Only segments with s*T*P < Lg are written; entries of other segments are
 * left untouched (mla_lse_merge does not read them). A row with no token in
 * a written segment gets maximum -inf and sum 0 (its segm_out entry is then
 * 0 or left untouched; the merge gives such a segment weight 0 and never
 * reads it). Local tokens past pt_width * page_size are never read (the plan
 * keeps every length within the table).
 */
mla_status_t mla_verify_attn(const void* q, const void* kv, int64_t num_blocks,
                             int32_t block_size, int32_t page_size,
                             mla_kv_dtype_t kv_dtype, float kv_scale,
                             float sm_scale, const int32_t* row_lens,
                             const int32_t* page_table, int32_t pt_width,
                             const int32_t* q_start, int32_t N, int32_t R,
                             int32_t H, int32_t W, int32_t max_qlen,
                             int32_t nseg, float* segm_out, float* segm_max,
                             float* segm_expsum, void* stream);

/*
 * Attention with each unit's result normalised, for the shard merge
 * ([V51705] Implementation breakdown item 4: the split-K segments of a
 * (request, shard) group; [S34432] report: a DCP rank hands its peers exactly
 * this pair, bf16 output plus natural-log LSE). For every shard r, segment s,
 * row and head, over the tokens of that segment of the row's window that the
 * shard holds (the partition of mla_verify_attn):
 *   o = O / e rounded to bf16,  lse = ln2 * (m2 + log2 e)
 * (o = 0, lse = -inf without a token), written as source r * nseg + s. The
 * LSE merge of all W * nseg sources (mla_shard_merge with W * nseg in place of
 * W) gives the verify result: the segment merge and the shard merge of
 * mla_lse_merge, done as one natural-log merge over (shard, segment) units,
 * with each unit's output handed over as bf16. With nseg = 1 the source is
 * the shard itself.
 *
 *   q, kv, num_blocks, block_size, page_size, kv_dtype, kv_scale, sm_scale,
 *   row_lens, page_table, pt_width, q_start, N, R, H, W, max_qlen, nseg:
 *              as for mla_verify_attn (same checks, same error codes)
 * Outputs (device, caller-allocated):
 *   shard_out  [W * nseg, R, H, 512] bf16, 16-byte aligned
 *   shard_lse  [W * nseg, R, H] fp32
 */
mla_status_t mla_verify_attn_shard(const void* q, const void* kv,
                                   int64_t num_blocks, int32_t block_size,
                                   int32_t page_size, mla_kv_dtype_t kv_dtype,
                                   float kv_scale, float sm_scale,
                                   const int32_t* row_lens,
                                   const int32_t* page_table, int32_t pt_width,
                                   const int32_t* q_start, int32_t N, int32_t R,
                                   int32_t H, int32_t W, int32_t max_qlen,
                                   int32_t nseg, void* shard_out,
                                   float* shard_lse, void* stream);

/*
 * mla_verify_attn_shard with one segment, scheduled for balance ([V51011]
 * Implementation breakdown item 3: the ASM decode path that vLLM routes to
 * runs a persistent kernel on per-launch work metadata; the schedule here is
 * this library's own). Same results layout and meaning as
 * mla_verify_attn_shard(..., nseg = 1, ...): shard_out [W, R, H, 512] bf16
 * and shard_lse [W, R, H], source r = shard r, for mla_shard_merge.
 *
 * All KV tiles of the launch -- every (request, 64-pair row block, shard)
 * group's tiles in token order, groups in that order -- are one sequence of
 * T tiles; `ctas` workgroups (one per compute unit) take contiguous ranges of
 * floor(T/ctas) or ceil(T/ctas) tiles each, so every compute unit streams for
 * about the same time whatever the spread of request lengths. A group that
 * lies in one range is finished there; a group cut between ranges is
 * finished by the piece that completes last, which combines all pieces'
 * fp32 partial states (in piece order: the result does not depend on which
 * piece comes last) and rounds once to bf16, like an uncut group. Each
 * workgroup computes the schedule itself from row_lens and q_start; no extra
 * launch and no host synchronisation.
 *
 *   q .. max_qlen: as for mla_verify_attn_shard (bf16, e4m3fn or e5m2 KV)
 *   ctas       workgroups, >= 1; 0 = the current device's compute-unit count
 *   workspace  device, 256-byte aligned, at least
 *              mla_verify_attn_persistent_workspace_bytes(N, W, H, max_qlen,
 *              ctas) bytes: per-group arrival counters, then two partial-state
 *              slots of 135168 bytes per workgroup. Its first
 *              4 * N * W * ceil(max_qlen * H / 64) bytes (the counters) must
 *              be zero before the first call; every completed call leaves them
 *              zero again, so the same workspace serves later calls (and HIP
 *              graph replays) without clearing. Calls that share a workspace
 *              must not overlap.
 *   shard_out, shard_lse: as for mla_verify_attn_shard with nseg = 1
 * Limits: at most 2048 groups (N * W * ceil(max_qlen * H / 64)),
 * pt_width * page_size < 2^30, groups times the tiles of the longest table
 * row < 2^31 (MLA_ERR_UNSUPPORTED beyond; use mla_verify_attn_shard).
 */
size_t mla_verify_attn_persistent_workspace_bytes(int32_t N, int32_t W, int32_t H,
                                                  int32_t max_qlen, int32_t ctas);
mla_status_t mla_verify_attn_persistent(const void* q, const void* kv,
                                        int64_t num_blocks, int32_t block_size,
                                        int32_t page_size, mla_kv_dtype_t kv_dtype,
                                        float kv_scale, float sm_scale,
                                        const int32_t* row_lens,
                                        const int32_t* page_table, int32_t pt_width,
                                        const int32_t* q_start, int32_t N, int32_t R,
                                        int32_t H, int32_t W, int32_t max_qlen,
                                        int32_t ctas, void* workspace,
                                        size_t workspace_bytes, void* shard_out,
                                        float* shard_lse, void* stream);

/*
 * Segment merge then shard merge ([V51705] merge snippet and Implementation
 * breakdown item 4; [S34432] review item 4 for the natural-log convention).
 * Per shard r, over its active segments (s*T*P < that row's length):
 *   M = max m2_s, E = sum e_s 2^(m2_s - M), o_r = sum O_s 2^(m2_s - M) / E,
 *   lse_r = ln2 * (M + log2 E)   (natural log; -inf and o_r = 0 if none).
 * Then across shards, with o_r kept in fp32 (every shard is on this device):
 *   lse = ln sum_r exp(lse_r), out = sum_r exp(lse_r - lse) * o_r  -> bf16.
 * Never produces NaN from empty shards or segments. A row's length is read
 * as at most its group's last row's (the segments mla_verify_attn wrote).
 *
 *   segm_*       from mla_verify_attn with the same R, H, W, nseg
 *   row_lens, q_start, N, page_size: as given to mla_verify_attn
 *   shard_out    [W, R, H, 512] bf16, may be NULL   (per-shard o_r, rounded)
 *   shard_lse    [W, R, H] fp32, may be NULL        (per-shard lse_r)
 *   out          [R, H, 512] bf16
 *   lse          [R, H] fp32, natural log, unpadded in heads
 */
mla_status_t mla_lse_merge(const float* segm_out, const float* segm_max,
                           const float* segm_expsum, const int32_t* row_lens,
                           const int32_t* q_start, int32_t N, int32_t page_size,
                           int32_t R, int32_t H, int32_t W, int32_t nseg,
                           void* shard_out, float* shard_lse, void* out,
                           float* lse, void* stream);

/*
 * Attention, segment merge and shard merge in one call ([V51705]
 * Implementation breakdown item 4 and the merge snippet; [S34432] review
 * item 4): mla_verify_attn into a caller workspace, then mla_lse_merge from
 * it, on `stream`. The same results, bit for bit, as those two calls.
 *
 *   q ... nseg   as for mla_verify_attn (same checks, same error codes)
 *   workspace    device memory of at least mla_verify_workspace_bytes(W, R,
 *                H, nseg) bytes, 16-byte aligned, laid out segm_out |
 *                segm_max | segm_expsum; its contents on entry do not
 *                matter, and on return it holds the partials
 *   out          [R, H, 512] bf16, 16-byte aligned;  lse [R, H] fp32
 */
mla_status_t mla_verify_attn_merge(const void* q, const void* kv,
                                   int64_t num_blocks, int32_t block_size,
                                   int32_t page_size, mla_kv_dtype_t kv_dtype,
                                   float kv_scale, float sm_scale,
                                   const int32_t* row_lens,
                                   const int32_t* page_table, int32_t pt_width,
                                   const int32_t* q_start, int32_t N, int32_t R,
                                   int32_t H, int32_t W, int32_t max_qlen,
                                   int32_t nseg, void* workspace,
                                   size_t workspace_bytes, void* out,
                                   float* lse, void* stream);

/* Size of the library's static scratch array (per GPU). */
#define MLA_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * mla_verify_attn_merge without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the partials go to a static scratch array
 * of MLA_STATIC_SCRATCH_BYTES (64 MiB) that the library holds on each GPU it
 * runs on until the process ends. The call allocates nothing (no hipMalloc,
 * no hipFree, no allocating library routine). Sizes whose partials exceed
 * the array (mla_verify_workspace_bytes(W, R, H, nseg) > 64 MiB) return
 * MLA_ERR_INVALID before anything is launched. Every call on one GPU shares
 * that GPU's array: calls that overlap on one GPU (on different streams, or
 * from different threads) race and must be ordered by the caller. Nothing in
 * the array needs to start at zero. Same arguments, checks and results as
 * mla_verify_attn_merge otherwise.
 */
mla_status_t mla_verify_attn_merge_static(const void* q, const void* kv,
                                          int64_t num_blocks, int32_t block_size,
                                          int32_t page_size,
                                          mla_kv_dtype_t kv_dtype, float kv_scale,
                                          float sm_scale, const int32_t* row_lens,
                                          const int32_t* page_table,
                                          int32_t pt_width, const int32_t* q_start,
                                          int32_t N, int32_t R, int32_t H, int32_t W,
                                          int32_t max_qlen, int32_t nseg, void* out,
                                          float* lse, void* stream);

/*
 * Shard merge alone ([V51705] Motivation: rank-local results combine through
 * the DCP attention merge; [S34432] review item 4: natural-log LSE), over W
 * sources (shards, or the W * nseg (shard, segment) sources of
 * mla_verify_attn_shard):
 *   lse = ln sum_r exp(lse_r),  out = sum_r exp(lse_r - lse) * o_r  -> bf16,
 * sources with lse_r = -inf ignored (their o_r is not read); out = 0 and
 * lse = -inf when every source is empty. With one source per shard it gives
 * the same bits as the shard step of mla_lse_merge would for the same bf16
 * per-shard outputs.
 *
 *   shard_out  [W, R, H, 512] bf16 (e.g. from mla_verify_attn_shard),
 *              16-byte aligned
 *   shard_lse  [W, R, H] fp32
 *   W          1 .. 1024 (MLA_ERR_UNSUPPORTED above)
 *   out        [R, H, 512] bf16, 16-byte aligned
 *   lse        [R, H] fp32
 */
mla_status_t mla_shard_merge(const void* shard_out, const float* shard_lse,
                             int32_t R, int32_t H, int32_t W, void* out,
                             float* lse, void* stream);

/* Description of the last error on the calling thread ("" if none). */
const char* mla_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_VERIFY_H_ */
