// Internal declarations shared by the host API and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_verify.h"

namespace mla {

constexpr int kHeadDim = 576;  // 512 latent + 64 rope
constexpr int kVDim = 512;

struct PlanArgs {
  int32_t N, R, W;
  int32_t I;                 // interleave: runs of I positions per shard
  const int32_t* seq_lens;
  const int32_t* q_start;
  const int32_t* block_table;
  int32_t max_blocks;
  int64_t num_blocks;
  int32_t block_size, page_size, max_kv_seq_len, pt_width;
  int32_t* row_lens;
  int32_t* page_table;
  int32_t* qo_indptr;
  uint32_t* err_flag;
  // Two-stage form (prefix_only set): every row of a request gets the
  // committed prefix S_i - Q_i as its window, and the second stage's
  // lengths [R] and window token table [R, win_width] are written too.
  int32_t prefix_only;
  int32_t* win_lens;
  int32_t* win_table;
  int32_t win_width;
};

struct AttnArgs {
  const uint16_t* q;         // [R, H, 576] bf16 bits
  const uint8_t* kv;         // [W, num_blocks, block_size, 576] elements
  int64_t pool_tokens;       // num_blocks * block_size (tokens per shard pool)
  int64_t num_subpages;      // num_blocks * block_size / page_size
  int32_t page_shift;        // log2(page_size)
  int32_t page_size;
  const int32_t* row_lens;   // [W, R]
  const int32_t* page_table; // [W, R, pt_width]
  int32_t pt_width;
  const int32_t* q_start;    // [N+1]
  int32_t N, R, H, W, nseg;
  int32_t mblocks;           // ceil(max_qlen * H / rows per workgroup)
  float qk_scale_log2;       // sm_scale * (fp8: kv_scale) * log2(e)
  float v_scale;             // fp8: kv_scale, bf16: 1
  int32_t e5m2;              // fp8 codes: 0 e4m3fn, 1 e5m2
  float* segm_out;
  float* segm_max;
  float* segm_expsum;
  // Normalised form (segm_* unused): each row's output over one (shard,
  // segment) unit, normalised and rounded to bf16, and its natural-log LSE,
  // as source r * nseg + s of the LSE merge.
  uint16_t* shard_out;       // [W * nseg, R, H, 512] bf16 bits, or null
  float* shard_lse;          // [W * nseg, R, H]
};

struct MergeArgs {
  const float* segm_out;
  const float* segm_max;
  const float* segm_expsum;
  const int32_t* row_lens;
  const int32_t* q_start;
  int32_t N, page_size, R, H, W, nseg;
  uint16_t* shard_out;  // may be null
  float* shard_lse;     // may be null
  uint16_t* out;
  float* lse;
};

struct ShardMergeArgs {
  const uint16_t* shard_out;  // [W, R, H, 512] bf16 bits
  const float* shard_lse;     // [W, R, H]
  int32_t R, H, W;
  uint16_t* out;
  float* lse;
};

// Workspace of the balanced persistent attention kernel.
struct PersistArgs {
  int32_t* counters;         // [groups]: arrivals per cut group, zero between calls
  float* slots;              // [2 * ctas] partial states of cut groups' pieces
  int32_t ctas;              // workgroups (one per compute unit)
};
// Limit of the persistent kernel's in-kernel schedule: groups (request, row
// block, shard) per launch.
constexpr int kPersistMaxGroups = 2048;
// One piece's partial state: per wave and lane 32 float4 of O and one of
// (reference exponent, running maximum, sum).
constexpr size_t kPersistSlotBytes = (size_t)4 * 33 * 64 * 16;

// Largest W the shard merge takes (its per-wave LDS area).
constexpr int kShardMergeMaxW = 1024;

// Device address of the current device's static scratch array
// (MLA_STATIC_SCRATCH_BYTES), looked up once per device.
hipError_t static_scratch(void** ptr);

hipError_t launch_plan(const PlanArgs& a, hipStream_t s);
hipError_t launch_attn(const AttnArgs& a, bool fp8, hipStream_t s);
hipError_t launch_attn_fp8(const AttnArgs& a, int64_t blocks, hipStream_t s);
hipError_t launch_attn_persist(const AttnArgs& a, const PersistArgs& p, bool fp8, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, hipStream_t s);
hipError_t launch_shard_merge(const ShardMergeArgs& a, hipStream_t s);

// Rows of one attention workgroup (two groups of 32 rows).
constexpr int kAttnRows = 64;

}  // namespace mla
