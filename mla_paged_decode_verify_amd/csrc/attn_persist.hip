// Balanced persistent attention (bf16, e4m3fn or e5m2 KV), normalised form:
// each shard's output of a row, normalised and rounded to bf16, with its
// natural-log LSE, as source r of the shard merge (the results of
// mla_verify_attn_shard with one segment).
//
// The work of a launch -- the KV tiles of every (request i, row block mb,
// shard r) group, each group's tiles in token order -- is one sequence of T
// tiles, cut into contiguous ranges of floor or ceil of T / C tiles, one per
// workgroup (C workgroups, one per compute unit). Every unit then streams for
// about the same time whatever the spread of the groups' lengths; a
// workgroup per group would end with the longest groups running alone. (The
// pages' ASM decode runs a persistent kernel on per-launch work metadata as
// well: vLLM PR #51011 digest, Implementation breakdown item 3. The split
// used here is this library's own.)
//
// Gangs: the row blocks of a request attend over the same tiles. With g the
// gcd of the requests' row-block counts, the sequence is over (request, gang
// of g row blocks, shard) and cut into C / g ranges; the g workgroups of a
// gang take the same range, one row block each, so they read each tile at
// about the same time and share it through one L2.
//
// Each workgroup computes the schedule itself when it starts: every thread
// reads the lengths of up to kRegGroups consecutive gang-groups (q_start,
// then the group's longest row length), and a workgroup-wide prefix sum over
// their tile counts gives every gang-group's first tile P. The gang-groups
// that meet the workgroup's range are its items; each item runs like one work
// unit of the unit-per-workgroup kernels (Q and the first tile loaded, the
// same tile loop and per-tile computation), so a group inside one range gets
// the unit kernels' results bit for bit.
//
// A group cut between ranges has one piece per workgroup it meets; each piece
// writes its partial state (O relative to its reference exponent, the
// reference, the running maximum and the exp2 sum, per lane in the
// accumulator layout) to a slot of its own. When all its items are done, a
// workgroup takes one device-scope release fence and adds one to each of its
// cut groups' arrival counters (vector atomics). The piece that arrives last
// (it reads pieces - 1) resets the counter, takes a device-scope acquire fence
// and combines all pieces' states in piece order -- the same operations
// whichever piece comes last, so the result does not depend on timing -- then
// stores the group's rows like a whole group. No workgroup ever waits for
// another, so every dispatch order completes.
#include "attn_f8mma.h"

namespace mla {
namespace {

constexpr int kMaxItems = 64;                              // items held at once
constexpr int kRegGroups = kPersistMaxGroups / kThreads;   // groups per thread in the scan
constexpr int kSlotVecs = 33;                              // float4 per lane and wave in a slot
static_assert(kPersistSlotBytes == (size_t)4 * kSlotVecs * 64 * 16, "slot layout");

// Items of a workgroup (group, first tile of the group in the sequence,
// readable tokens of its longest row, its request's rows [qs, qs + Q)), the
// prefix-sum scratch and the cut pieces it may have to combine.
struct Sched {
  int g[kMaxItems], P[kMaxItems], L[kMaxItems], qs[kMaxItems], Q[kMaxItems];
  int wsum[8];
  int first_rank, n;
  int lo, hi, total, v;      // this workgroup's range of tiles, the tile total, its index
  int cut[2][5];             // g, P, L, qs, Q of the first and last cut item
  int combine[2];
};

__device__ __forceinline__ int rfl(int x) { return __builtin_amdgcn_readfirstlane(x); }
// This lane's index, opaque to the optimiser: each item derives its per-lane
// addresses from it, so the compiler cannot hoist them out of the item loop
// and hold them in registers across every item's tile loop.
__device__ __forceinline__ int cold_lane() {
  int x = (int)(threadIdx.x & 63);
  asm volatile("" : "+v"(x));
  return x;
}

struct GroupId {
  int i, mb, r;
};
__device__ __forceinline__ GroupId group_id(const AttnArgs& a, int gg) {
  const int per_i = a.mblocks * a.W;
  GroupId id;
  id.i = gg / per_i;
  const int rem = gg - id.i * per_i;
  id.mb = rem / a.W;
  id.r = rem - id.mb * a.W;
  return id;
}

// A gang-group: the (request i, gang mbg, shard r) of the schedule; gang mbg
// is row blocks mbg * gang .. mbg * gang + gang - 1 of the request.
__device__ __forceinline__ GroupId gang_group_id(const AttnArgs& a, int gg, int ngang) {
  GroupId id;
  id.i = gg / (ngang * a.W);
  const int rem = gg - id.i * ngang * a.W;
  id.mb = rem / a.W;                        // the gang, not yet the row block
  id.r = rem - id.mb * a.W;
  return id;
}
// Row blocks of a request with Q rows (at most the grid's mblocks).
__device__ __forceinline__ int blocks_of(const AttnArgs& a, int Q) {
  return min((Q * a.H + kAttnRows - 1) / kAttnRows, a.mblocks);
}
__device__ __forceinline__ int gcd_int(int x, int y) {
  while (y != 0) {
    const int t = x % y;
    x = y;
    y = t;
  }
  return x;
}

__device__ __forceinline__ int tiles_of(int L) { return (L + kTile - 1) / kTile; }
// First tile of workgroup v's range, and the workgroup whose range holds tile t.
__device__ __forceinline__ int range_lo(int v, int total, int C) {
  return (int)((int64_t)v * total / C);
}
__device__ __forceinline__ int range_of(int t, int total, int C) {
  return (int)(((int64_t)(t + 1) * C - 1) / total);
}
// The pieces of a group are the workgroups whose ranges meet its tiles: walk
// them as w = range_of(t), t = range_lo(w + 1) from the group's first tile
// (with more workgroups than tiles some ranges are empty, so the workgroups
// between the first and the last piece are not all pieces).
// Slot of the piece of a group starting at tile P in workgroup w: 2w for the
// workgroup's first item, 2w + 1 for its last.
__device__ __forceinline__ int slot_of(int w, int P, int total, int Cg, int gang) {
  return 2 * w + (P > range_lo(w / gang, total, Cg) ? 1 : 0);
}

// Unit of tiles [t0, t1) of group gg.
__device__ inline WorkUnit item_unit(const AttnArgs& a, int gg, int qs, int Q, int L, int t0,
                                     int t1) {
  WorkUnit u;
  const GroupId id = group_id(a, gg);
  u.i = id.i;
  u.mb = id.mb;
  u.r = id.r;
  u.s = 0;
  u.qs = qs;
  u.Q = Q;
  u.M = Q * a.H;
  u.m0 = id.mb * kAttnRows;
  u.last = qs + Q - 1;
  u.lo = t0 * kTile;
  u.hi = (int)min((int64_t)t1 * kTile, (int64_t)L);
  u.valid = true;
  u.read = true;
  return u;
}

// Exclusive prefix sums of (x, y) over the workgroup, and their totals.
__device__ inline void scan2(int x, int y, int* wsum, int tid, int& px, int& py, int& tx,
                             int& ty) {
  const int lane = tid & 63, w = tid >> 6;
  int sx = x, sy = y;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int ox = __shfl_up(sx, d), oy = __shfl_up(sy, d);
    if (lane >= d) {
      sx += ox;
      sy += oy;
    }
  }
  if (lane == 63) {
    wsum[2 * w] = sx;
    wsum[2 * w + 1] = sy;
  }
  lds_barrier();
  px = sx - x;
  py = sy - y;
  tx = 0;
  ty = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int a = wsum[2 * k], b = wsum[2 * k + 1];
    if (k < w) {
      px += a;
      py += b;
    }
    tx += a;
    ty += b;
  }
}

// Reads every gang-group's length and fills sc with the items that meet
// tiles [pos, hi) (at most kMaxItems of them, sc.n). The first call (first
// set) also sets this workgroup's range [pos, hi): the range of its gang,
// q = v / gang, among the Cg = C / gang gang ranges (none if q >= Cg).
// Returns the tile total T.
__device__ int collect(const AttnArgs& a, Sched& sc, int G, int C, int v, int gang, bool first,
                       int& pos, int& hi, int tid) {
  const int ngang = (a.mblocks + gang - 1) / gang;
  const int k = (G + kThreads - 1) / kThreads;   // <= kRegGroups
  const int base = tid * k;
  int T[kRegGroups], L[kRegGroups], qs[kRegGroups], Q[kRegGroups];
#pragma unroll
  for (int j = 0; j < kRegGroups; ++j) {
    const int gg = base + j;
    qs[j] = 0;
    Q[j] = 0;
    if (j < k && gg < G) {
      const int i = gg / (ngang * a.W);
      qs[j] = a.q_start[i];
      Q[j] = a.q_start[i + 1] - qs[j];
    }
  }
#pragma unroll
  for (int j = 0; j < kRegGroups; ++j) {
    const int gg = base + j;
    T[j] = 0;
    L[j] = 0;
    if (j < k && gg < G) {
      const GroupId id = gang_group_id(a, gg, ngang);
      const bool ok =
          !(qs[j] < 0 || Q[j] <= 0 || qs[j] + Q[j] > a.R) && id.mb * gang < blocks_of(a, Q[j]);
      if (ok) {
        const int Lg = a.row_lens[(int64_t)id.r * a.R + qs[j] + Q[j] - 1];
        L[j] = (int)max((int64_t)0, min((int64_t)Lg, (int64_t)a.pt_width * a.page_size));
        T[j] = tiles_of(L[j]);
      }
    }
  }
  int tsum = 0, nsum = 0;
#pragma unroll
  for (int j = 0; j < kRegGroups; ++j) {
    tsum += T[j];
    nsum += T[j] > 0 ? 1 : 0;
  }
  int tpre, npre, total, ntot;
  scan2(tsum, nsum, sc.wsum, tid, tpre, npre, total, ntot);
  if (first) {
    const int Cg = C / gang, q = v / gang;
    pos = q < Cg ? range_lo(q, total, Cg) : 0;
    hi = q < Cg ? range_lo(q + 1, total, Cg) : 0;
    if (tid == 0) {
      sc.lo = pos;
      sc.hi = hi;
      sc.total = total;
      sc.v = v;
    }
  }
  {
    int P = tpre, rk = npre;
#pragma unroll
    for (int j = 0; j < kRegGroups; ++j) {
      if (T[j] > 0 && P <= pos && pos < P + T[j]) sc.first_rank = rk;
      P += T[j];
      rk += T[j] > 0 ? 1 : 0;
    }
  }
  if (tid == 0) sc.n = 0;
  lds_barrier();
  if (pos < hi) {
    const int fr = sc.first_rank;
    int P = tpre, rk = npre;
#pragma unroll
    for (int j = 0; j < kRegGroups; ++j) {
      if (T[j] > 0 && P < hi && P + T[j] > pos) {
        const int idx = rk - fr;
        if (idx < kMaxItems) {
          sc.g[idx] = base + j;
          sc.P[idx] = P;
          sc.L[idx] = L[j];
          sc.qs[idx] = qs[j];
          sc.Q[idx] = Q[j];
        }
        if (P + T[j] >= hi) sc.n = min(idx + 1, kMaxItems);
      }
      P += T[j];
      rk += T[j] > 0 ? 1 : 0;
    }
  }
  lds_barrier();
  return total;
}

// A piece's partial state into its slot: per wave and lane, the 8 O tiles as
// 32 float4 (value j of tile t at float4 4t + j / 4), then (reference
// exponent, running maximum, exp2 sum). One 1 KB store per instruction.
__device__ __forceinline__ void write_slot(float* slots, int slot, const WaveState& st, int wave,
                                           int lane) {
  float4* b = reinterpret_cast<float4*>(slots + (size_t)slot * (kPersistSlotBytes / 4)) +
              (size_t)wave * kSlotVecs * 64 + lane;
#pragma unroll
  for (int t = 0; t < kOTiles; ++t)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      b[(4 * t + q) * 64] =
          make_float4(st.o[t][4 * q], st.o[t][4 * q + 1], st.o[t][4 * q + 2], st.o[t][4 * q + 3]);
  b[32 * 64] = make_float4(st.m_ref, st.m_true, st.l_part, 0.f);
}

// The gang width: the gcd of the well-formed requests' row-block counts, so
// that every gang of that many workgroups has a row block of each request
// it meets (1 when there is no request, or when it exceeds the workgroups).
__device__ int gang_width(const AttnArgs& a, int* wsum, int tid, int C) {
  int x = 0;
  for (int i = tid; i < a.N; i += kThreads) {
    const int qs = a.q_start[i], Q = a.q_start[i + 1] - qs;
    if (!(qs < 0 || Q <= 0 || qs + Q > a.R)) x = gcd_int(x, blocks_of(a, Q));
  }
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) x = gcd_int(x, __shfl_xor(x, d));
  if ((tid & 63) == 0) wsum[tid >> 6] = x;
  lds_barrier();
  int r = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) r = gcd_int(r, wsum[w]);
  lds_barrier();                            // wsum is the scan's scratch next
  return (r < 1 || r > C) ? 1 : r;
}

// The normalised form of store_partials written straight from the
// accumulators (each lane stores its row's 4-dim runs, 8 bytes each), with no
// LDS staging: the combination of a cut group's pieces. Same fp32 operations
// as store_partials, so an uncut group would get the same results.
__device__ __forceinline__ void store_rows_direct(const AttnArgs& a, const WorkUnit& u,
                                                  const WaveState& st, RowExchange& rx, int mrow,
                                                  bool row_ok, int g, int c, int lane) {
  const int h = lane >> 5;
  const int n32 = lane & 31;
  float l_row;
  {
    auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(st.l_part),
                                              __float_as_uint(st.l_part), false, false);
    l_row = __uint_as_float(q[0]) + __uint_as_float(q[1]);
  }
  if (h == 0) rx.l[g][c][n32] = l_row;
  lds_barrier();
  const float L = l_row + rx.l[g][c ^ 1][n32];
  float fix = 1.f;
  if (st.m_true != kNegInf) fix = __builtin_amdgcn_exp2f(st.m_ref - st.m_true);
  const float E = L * fix;
  const bool live = st.m_true != kNegInf && E > 0.f;
  const int64_t e = source_base(a, u) + mrow;
  if (row_ok && c == 0 && h == 0) a.shard_lse[e] = live ? kLn2 * (st.m_true + __log2f(E)) : kNegInf;
  const float vs = fix * a.v_scale;
  const float inv = live ? 1.f / E : 0.f;
  if (row_ok) {
    uint16_t* dst = a.shard_out + e * kVDim + 256 * c + 4 * h;
#pragma unroll
    for (int t = 0; t < kOTiles; ++t) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v = (f32x4{st.o[t][4 * q], st.o[t][4 * q + 1], st.o[t][4 * q + 2],
                               st.o[t][4 * q + 3]} * vs) * inv;
        *reinterpret_cast<uint2*>(dst + 32 * t + 8 * q) =
            make_uint2(pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3]));
      }
    }
  }
}

// KV: 0 bf16, 1 e4m3fn codes, 2 e5m2 codes.
template <bool SLICE, int KV>
__global__ void __launch_bounds__(kThreads, 1) attn_persist_kernel(AttnArgs a, PersistArgs ps) {
  __shared__ __align__(16) unsigned char buf0[kBufBytes];
  __shared__ __align__(16) unsigned char buf1[kBufBytes];
  __shared__ PExchange px;
  __shared__ RowExchange rx;
  __shared__ Sched sc;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = wave >> 1;                  // row group: 32 rows
  const int c = wave & 1;                   // token half (QK) / latent half (PV)
  const int G = a.N * a.mblocks * a.W;
  const unsigned char* zero = zero_row();

  if (tid == 0) {
    sc.combine[0] = 0;
    sc.combine[1] = 0;
  }
  // Gangs: the row blocks of a request attend over the same tiles, so a gang
  // of `gang` consecutive workgroups takes one range of the sequence of
  // (request, gang of row blocks, shard) tiles, each workgroup one row block:
  // the gang's members read each tile at about the same time, through one
  // L2. Workgroups are dealt to the 8 XCDs round-robin: consecutive virtual
  // indices go to one XCD, so a gang -- and the neighbouring ranges, which
  // share requests (their Q, a cut group's slots) -- mostly share an L2.
  const int C = ps.ctas;
  const int gang = rfl(gang_width(a, sc.wsum, tid, C));
  const int ngang = (a.mblocks + gang - 1) / gang;
  const int Gs = a.N * ngang * a.W;         // gang-groups
  const int Cg = C / gang;                  // gang ranges
  {
    const int v = (C % 8 == 0) ? (int)(blockIdx.x % 8) * (C / 8) + (int)(blockIdx.x / 8)
                               : (int)blockIdx.x;
    int pos = 0, hi = 0;
    collect(a, sc, Gs, C, v, gang, true, pos, hi, tid);
  }

  // groups g = v mod C that are well formed but hold no token to read get the
  // empty result, and a request with more (row, head) pairs than the row
  // blocks cover gets NaN in the uncovered ones
  auto do_jobs = [&] {
    const int C = ps.ctas;
    for (int gg = rfl(sc.v); gg < G; gg += C) {
      const GroupId id = group_id(a, gg);
      const int qs = a.q_start[id.i];
      const int Q = a.q_start[id.i + 1] - qs;
      if (qs < 0 || Q <= 0 || qs + Q > a.R || id.mb * kAttnRows >= Q * a.H) continue;
      const int Lg = a.row_lens[(int64_t)id.r * a.R + qs + Q - 1];
      const int L = (int)max((int64_t)0, min((int64_t)Lg, (int64_t)a.pt_width * a.page_size));
      const WorkUnit ju = item_unit(a, gg, qs, Q, L, 0, 0);
      if (L == 0) store_empty(a, ju, wave, lane);
      poison_uncovered(a, ju, wave, lane);
    }
  };
  if (rfl(sc.lo) >= rfl(sc.hi)) {
    do_jobs();
    return;
  }

  int ncut = 0;                             // cut pieces written (their facts in sc.cut)
  bool first_batch = true;
  for (;;) {                                // batches of items
    const int n = rfl(sc.n);
    for (int j = 0; j < n; ++j) {           // items, each run like one work unit
      // every per-lane address of an item is derived from ln where it is used
      const int ln = cold_lane();
      const int P = rfl(sc.P[j]), L = rfl(sc.L[j]);
      const int vv = rfl(sc.v);
      const GroupId gid = gang_group_id(a, rfl(sc.g[j]), ngang);
      // this workgroup's row block of the gang: its group (i, mb, r)
      const int gg = (gid.i * a.mblocks + gid.mb * gang + vv % gang) * a.W + gid.r;
      const WorkUnit u = item_unit(a, gg, rfl(sc.qs[j]), rfl(sc.Q[j]), L,
                                   max(rfl(sc.lo) - P, 0), min(tiles_of(L), rfl(sc.hi) - P));
      const int lo = u.lo, hi = u.hi;
      const int32_t* pt_row = a.page_table + ((int64_t)u.r * a.R + u.last) * a.pt_width;
      int mrow, hi_row;
      bool row_ok;
      const bool idle = u.m0 + 32 * g >= u.M;
      WaveState st;
      bf16x8 qf[kQSteps];
      int32_t vpg = 0;

      // ---- Q through the second buffer, then the first tile into the first
      // (once every wave is done with the buffers: the last item's staged rows)
      lds_barrier();
      issue_q_tile(a, u, buf1, wave, ln, zero);
      if constexpr (KV == 0) {
        const unsigned char* pool = a.kv + (int64_t)u.r * a.pool_tokens * kTokBytesBf16;
        Bf16Pages pg;
        if constexpr (SLICE) {
          vpg = slice_pages(a, pt_row, lo, hi, wave, ln);
          const SliceSrc v0 =
              slice_src(a, pool, __builtin_amdgcn_readlane(vpg, 0), lo + 16 * wave, hi);
#pragma unroll
          for (int k = 0; k < 18; ++k) issue_slice(v0, zero, buf0, wave, ln, k);
        } else {
          pg.fetch(a, pt_row, lo, hi, wave, ln);
          issue_tile_bf16(a, pool, pg, lo, hi, buf0, wave, ln, zero);
        }
        if (first_batch && j == 0) do_jobs();
        lane_row(a, u, g, ln, mrow, hi_row, row_ok);
        state_init(st);
        MLA_WAIT_VMCNT(0);
        lds_barrier();
        read_q(buf1, g, ln, qf);

        // one tile: wait until `cur` holds it, stream the next one into `nxt`
        // during the QK product, compute on `cur`
        auto step = [&](const unsigned char* cur, unsigned char* nxt, int tb, int kt) {
          const bool more = tb + kTile < hi;
          MLA_WAIT_VMCNT(0);
          lds_barrier();
          SliceSrc v{zero, 0};
          if constexpr (SLICE) {
            if (more) {
              const int nk = kt + 1;
              if ((nk & 63) == 0) vpg = slice_pages(a, pt_row, lo + nk * kTile, hi, wave, ln);
              v = slice_src(a, pool, __builtin_amdgcn_readlane(vpg, nk & 63),
                            tb + kTile + 16 * wave, hi);
            }
          } else {
            if (more) {
              pg.fetch(a, pt_row, tb + kTile, hi, wave, ln);
              issue_tile_bf16(a, pool, pg, tb + kTile, hi, nxt, wave, ln, zero);
            }
          }
          auto issue = [&](int k) {
            if constexpr (SLICE) {
              if (more && (k & 1) == 0) issue_slice(v, zero, nxt, wave, ln, k >> 1);
            }
          };
          if (idle)
            idle_tile(issue);
          else
            compute_tile(cur, &px, qf, st, tb, hi_row, a.qk_scale_log2, g, c, ln, issue);
        };
        int kt = 0;
        for (int tb = lo; tb < hi; tb += 2 * kTile, kt += 2) {
          step(buf0, buf1, tb, kt);
          if (tb + kTile >= hi) break;
          step(buf1, buf0, tb + kTile, kt + 1);
        }
      } else {
        // fp8 codes, straight into LDS and onto the fp8 matrix cores
        // (step_f8: softmax and PV of tile k around the QK product of tile
        // k + 1): four tile slots in the two buffers, tile k + 3 loading
        // during step k; Q (staged in the second buffer) is split into its
        // e4m3fn terms before tiles 2 and 3 land there
        constexpr bool E5M2 = KV == 2;
        const unsigned char* pool = a.kv + (int64_t)u.r * a.pool_tokens * kHeadDim;
        const int ntiles = (hi - lo + kTile - 1) / kTile;
        auto issue_all = [&](int k) {       // slice path: k < 64
          unsigned char* dst = f8_slot(buf0, buf1, k & 3);
          const int tb = lo + k * kTile;
          if constexpr (SLICE) {
            const __amdgpu_buffer_rsrc_t r =
                f8_slice_rsrc(a, pool, __builtin_amdgcn_readlane(vpg, k & 63), tb + 16 * wave, hi);
#pragma unroll
            for (int jj = 0; jj < kF8Dma; ++jj) issue_f8_slice(r, dst, wave, ln, jj);
          } else {
#pragma unroll
            for (int jj = 0; jj < kF8Dma; ++jj)
              issue_f8_pages(a, pool, pt_row, tb, hi, dst, wave, ln, jj, zero);
          }
        };
        if constexpr (SLICE) vpg = slice_pages(a, pt_row, lo, hi, wave, ln);
        issue_all(0);
        if (ntiles > 1) issue_all(1);
        if (first_batch && j == 0) do_jobs();
        lane_row(a, u, g, ln, mrow, hi_row, row_ok);
        state_init(st);
        MLA_WAIT_VMCNT(0);
        lds_barrier();
        QF8 q;
        read_q_f8(buf1, g, ln, q);
        lds_barrier();                      // the second buffer is free for tiles 2, 3
        if (ntiles > 2) issue_all(2);
        f32x16 sacc;
        if (!idle) qk_f8<E5M2>(f8_slot(buf0, buf1, 0), q, sacc, c, ln);

        for (int k = 0; k < ntiles; ++k) {
          const int tb = lo + k * kTile;
          if (k + 2 < ntiles)
            MLA_WAIT_VMCNT(kF8Dma);         // tile k + 1 has landed (tile k + 2 may not have) ...
          else
            MLA_WAIT_VMCNT(0);
          lds_barrier();                    // ... for every wave; slot (k + 3) mod 4 is free
          const bool more3 = k + 3 < ntiles;
          unsigned char* dst = f8_slot(buf0, buf1, (k + 3) & 3);
          __amdgpu_buffer_rsrc_t rs = f8_slice_rsrc(a, pool, -1, 0, 0);
          if (more3) {
            if constexpr (SLICE) {
              const int nk = k + 3;
              if ((nk & 63) == 0) vpg = slice_pages(a, pt_row, lo + nk * kTile, hi, wave, ln);
              rs = f8_slice_rsrc(a, pool, __builtin_amdgcn_readlane(vpg, nk & 63),
                                 lo + nk * kTile + 16 * wave, hi);
            } else {
              issue_all(k + 3);
            }
          }
          auto issue = [&](int s) {
            if constexpr (SLICE) {
              if (more3) issue_f8_slice(rs, dst, wave, ln, s);
            }
          };
          if (idle)
            idle_tile_f8(issue);
          else
            step_f8<E5M2>(f8_slot(buf0, buf1, k & 3), f8_slot(buf0, buf1, (k + 1) & 3), sacc, &px,
                          q, st, tb, hi_row, a.qk_scale_log2, g, c, ln, issue);
        }
      }

      // ---- a whole group is stored; a cut piece writes its state to its
      // slot and counts its arrival
      if (lo == 0 && hi == L) {
        store_partials(a, u, st, rx, g == 0 ? buf0 : buf1, mrow, row_ok, g, c, ln);
        continue;
      }
      write_slot(ps.slots, slot_of(vv, P, rfl(sc.total), Cg, gang), st, wave, ln);
      if (tid == 0 && ncut < 2) {
        int* f = sc.cut[ncut];
        f[0] = gg;
        f[1] = P;
        f[2] = L;
        f[3] = u.qs;
        f[4] = u.Q;
      }
      ++ncut;
    }
    first_batch = false;
    // a batch ends with its last item; more items past it (more than
    // kMaxItems met this range) come in another batch
    const int end = rfl(sc.P[n - 1]) + tiles_of(rfl(sc.L[n - 1]));
    if (end >= rfl(sc.hi)) break;
    int pos = end, hi_v = rfl(sc.hi);
    __syncthreads();
    collect(a, sc, Gs, C, rfl(sc.v), gang, false, pos, hi_v, tid);
  }

  // ---- arrivals of this workgroup's cut pieces, counted once all its work is
  // done (one release per workgroup: every wave's slot stores have completed
  // before the barrier, and the release fence then makes this compute unit's
  // stores visible device-wide before the counters move); the pieces that
  // arrive last combine their group
  const int total = rfl(sc.total), vlane = rfl(sc.v) % gang;
  if (ncut > 0) {
    MLA_WAIT_VMCNT(0);
    __syncthreads();
  }
  if (tid == 0 && ncut > 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    for (int k = 0; k < ncut; ++k) {
      const int* f = sc.cut[k];
      const int old =
          __hip_atomic_fetch_add(ps.counters + f[0], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int end = f[1] + tiles_of(f[2]);
      int np = 0;
      for (int t = f[1]; t < end; t = range_lo(range_of(t, total, Cg) + 1, total, Cg)) ++np;
      if (old == np - 1) {
        __hip_atomic_store(ps.counters + f[0], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sc.combine[k] = 1;
      }
    }
  }
  lds_barrier();
  for (int k = 0; k < ncut; ++k) {
    if (rfl(sc.combine[k]) == 0) continue;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    const int Pc = rfl(sc.cut[k][1]), Lc = rfl(sc.cut[k][2]);
    const int T = tiles_of(Lc);
    const WorkUnit mu =
        item_unit(a, rfl(sc.cut[k][0]), rfl(sc.cut[k][3]), rfl(sc.cut[k][4]), Lc, 0, T);
    const int end = Pc + T;
    const size_t lane_off = (size_t)wave * kSlotVecs * 64 + lane;
    auto slot_ptr = [&](int w) {
      return reinterpret_cast<const float4*>(
                 ps.slots + (size_t)slot_of(w, Pc, total, Cg, gang) * (kPersistSlotBytes / 4)) +
             lane_off;
    };
    float M = kNegInf, mt = kNegInf;
    for (int t = Pc; t < end;) {
      const int qq = range_of(t, total, Cg);
      const int w = qq * gang + vlane;
      t = range_lo(qq + 1, total, Cg);
      const float4 s = slot_ptr(w)[32 * 64];
      M = fmaxf(M, s.x);
      mt = fmaxf(mt, s.y);
    }
    WaveState ms;
    state_init(ms);
    float l = 0.f;
    for (int t = Pc; t < end;) {
      const int qq = range_of(t, total, Cg);
      const int w = qq * gang + vlane;
      t = range_lo(qq + 1, total, Cg);
      const float4* b = slot_ptr(w);
      const float4 s = b[32 * 64];
      const float wgt = s.x == kNegInf ? 0.f : __builtin_amdgcn_exp2f(s.x - M);
      l = __builtin_fmaf(wgt, s.z, l);
      // one O tile's loads at a time (the accumulators take 128 registers)
#pragma unroll
      for (int t = 0; t < kOTiles; ++t) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 o = b[(4 * t + q) * 64];
          ms.o[t][4 * q] = __builtin_fmaf(wgt, o.x, ms.o[t][4 * q]);
          ms.o[t][4 * q + 1] = __builtin_fmaf(wgt, o.y, ms.o[t][4 * q + 1]);
          ms.o[t][4 * q + 2] = __builtin_fmaf(wgt, o.z, ms.o[t][4 * q + 2]);
          ms.o[t][4 * q + 3] = __builtin_fmaf(wgt, o.w, ms.o[t][4 * q + 3]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    ms.m_ref = M;
    ms.m_true = mt;
    ms.l_part = l;
    const int mrow_c = mu.m0 + 32 * g + (lane & 31);
    store_rows_direct(a, mu, ms, rx, mrow_c, mrow_c < mu.M, g, c, lane);
    lds_barrier();
  }
}

}  // namespace

hipError_t launch_attn_persist(const AttnArgs& a, const PersistArgs& p, bool fp8, hipStream_t s) {
  if (p.ctas <= 0) return hipErrorInvalidConfiguration;
  const unsigned n = (unsigned)p.ctas;
  const bool slice = a.page_size >= 16;
  if (!fp8) {
    if (slice) attn_persist_kernel<true, 0><<<n, kThreads, 0, s>>>(a, p);
    else attn_persist_kernel<false, 0><<<n, kThreads, 0, s>>>(a, p);
  } else if (!a.e5m2) {
    if (slice) attn_persist_kernel<true, 1><<<n, kThreads, 0, s>>>(a, p);
    else attn_persist_kernel<false, 1><<<n, kThreads, 0, s>>>(a, p);
  } else {
    if (slice) attn_persist_kernel<true, 2><<<n, kThreads, 0, s>>>(a, p);
    else attn_persist_kernel<false, 2><<<n, kThreads, 0, s>>>(a, p);
  }
  return hipGetLastError();
}

}  // namespace mla
