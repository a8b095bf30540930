// Split-K segmented MLA attention partials, fp8 (e4m3fn) KV cache.
//
// The quantities computed, the work decomposition and the per-tile
// computation are those of attn_common.h. Specific to this kernel: the fp8
// codes of the next tile are loaded into registers (lane l of wave w: chunks
// 9w .. 9w+8 of token l) while the current tile is computed, and are widened
// exactly to bf16 on the way into LDS; the scale is folded into the score
// scale and the output.
#include "attn_common.h"

namespace mla {
namespace {

// Widen 16 e4m3fn codes (one uint4) to 16 bf16 values (two uint4). Exact:
// every e4m3fn value is a bf16 value.
__device__ inline void fp8x16_to_bf16(uint4 in, uint4& lo, uint4& hi) {
  const uint32_t w[4] = {in.x, in.y, in.z, in.w};
  uint32_t o[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    // v_cvt_pk_f32_fp8 reads the OCP e4m3fn format on gfx950.
    auto f01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], false);
    auto f23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], true);
    // f32 -> bf16 by truncation is exact for these values.
    o[2 * k] = (__float_as_uint(f01[0]) >> 16) | (__float_as_uint(f01[1]) & 0xFFFF0000u);
    o[2 * k + 1] = (__float_as_uint(f23[0]) >> 16) | (__float_as_uint(f23[1]) & 0xFFFF0000u);
  }
  lo = make_uint4(o[0], o[1], o[2], o[3]);
  hi = make_uint4(o[4], o[5], o[6], o[7]);
}

// fp8: lane l of wave w loads chunks [9w, 9w + 9) (16 codes each) of token l.
struct Fp8Stage {
  static constexpr int kLoads = kHeadDim / 16 / 4;  // 9
  uint4 reg[kLoads];
  int32_t sp;

  __device__ inline void fetch_page(const AttnArgs& a, const int32_t* pt_row, int tb, int hi,
                                    int lane) {
    sp = subpage_always(a, pt_row, tb + lane, hi);
  }
  __device__ inline void load(const AttnArgs& a, const unsigned char* pool, int tb, int hi,
                              int wave, int lane) {
    const unsigned char* src =
        token_src<kHeadDim>(a, pool, sp, tb + lane, hi, zero_row()) + 16 * kLoads * wave;
#pragma unroll
    for (int j = 0; j < kLoads; ++j) reg[j] = *reinterpret_cast<const uint4*>(src + 16 * j);
  }
  __device__ inline void store(unsigned char* dst, int wave, int lane) const {
    const int row = lane;
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int col = kLoads * wave + j;      // 16-dim chunk
      uint4 lo, hi4;
      fp8x16_to_bf16(reg[j], lo, hi4);
      if (col < kVDim / 16) {
        *reinterpret_cast<uint4*>(dst + lat_off(row, 2 * col)) = lo;
        *reinterpret_cast<uint4*>(dst + lat_off(row, 2 * col + 1)) = hi4;
      } else {
        const int c0 = 2 * (col - kVDim / 16);
        unsigned char* rb = dst + kLatBytes + row * kRopeRow;
        *reinterpret_cast<uint4*>(rb + 16 * (c0 ^ (row & 7))) = lo;
        *reinterpret_cast<uint4*>(rb + 16 * ((c0 + 1) ^ (row & 7))) = hi4;
      }
    }
  }
};

__global__ void __launch_bounds__(kThreads, 1) attn_fp8_kernel(AttnArgs a) {
  // Two separate arrays (not one indexed one), so that the compiler can tell
  // the buffer being read from the buffer being filled.
  __shared__ __align__(16) unsigned char buf0[kBufBytes];
  __shared__ __align__(16) unsigned char buf1[kBufBytes];
  __shared__ PExchange px;
  __shared__ RowExchange rx;
  const WorkUnit u = decode_unit(a, blockIdx.x);
  if (!u.valid) return;
  const int lo = u.lo, hi = u.hi;
  if (lo >= hi) return;                     // segment inactive for the whole group

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = wave >> 1;                  // row group: 32 rows
  const int c = wave & 1;                   // token half (QK) / latent half (PV)
  const int r16 = lane & 15;

  const unsigned char* pool = a.kv + (int64_t)u.r * a.pool_tokens * kHeadDim;
  const int32_t* pt_row = a.page_table + ((int64_t)u.r * a.R + u.last) * a.pt_width;

  // ---- first tile in flight before anything else
  Fp8Stage fs;
  fs.fetch_page(a, pt_row, lo, hi, lane);
  fs.load(a, pool, lo, hi, wave, lane);
  fs.fetch_page(a, pt_row, lo + kTile, hi, lane);

  // ---- Q through the second tile buffer (first written at the second step)
  issue_q_tile(a, u, buf1, wave, lane, zero_row());
  int mrow[2], hi_row[2];
  bool row_ok[2];
  lane_rows(a, u, g, r16, mrow, hi_row, row_ok);
  WaveState st;
  state_init(st);
  MLA_WAIT_VMCNT(0);
  lds_barrier();
  bf16x8 qf[2][kQSteps];
  read_q(buf1, g, lane, qf);

  // One tile: widen the staged codes into `cur`, start loading the next tile's
  // codes, then compute on `cur` (last read two tiles ago, before the previous
  // barrier).
  auto step = [&](unsigned char* cur, int tb) {
    fs.store(cur, wave, lane);
    lds_barrier();
    if (tb + kTile < hi) {
      fs.load(a, pool, tb + kTile, hi, wave, lane);
      fs.fetch_page(a, pt_row, tb + 2 * kTile, hi, lane);
    }
    compute_tile(cur, &px, qf, st, tb, hi_row, a.qk_scale_log2, g, c, lane, [](int) {}, [] {});
  };
  for (int tb = lo; tb < hi; tb += 2 * kTile) {
    step(buf0, tb);
    if (tb + kTile >= hi) break;
    step(buf1, tb + kTile);
  }
  store_partials(a, u, st, rx, g == 0 ? buf0 : buf1, mrow, row_ok, g, c, lane);
}

}  // namespace

hipError_t launch_attn_fp8(const AttnArgs& a, int64_t blocks, hipStream_t s) {
  attn_fp8_kernel<<<(unsigned)blocks, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
