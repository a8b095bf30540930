"""Shared test utilities: cached workloads, running the HIP path, comparing
against the oracle. Test infrastructure only."""

from __future__ import annotations

import functools
import sys

import numpy as np

import oracle as orc
import workloads as wl

TOL_OUT = {"bf16": 1e-2, "fp8_e4m3": 3e-2, "fp8_e5m2": 3e-2}   # stated max-abs on out
TOL_LSE = 1e-3                                # stated max-abs on lse
# Two kinds of rounding can put an element beyond the stated bound, and only
# where they do does an element get a larger, derived one (each check prints
# how many):
#  * bf16 formats the method fixes: the output itself, and on the one-segment
#    route each shard's output handed to the shard merge. Rounding x to bf16
#    (nearest even, 8 significant bits) errs by at most half the spacing of
#    bf16 numbers at |x|: 2^(e-8) for |x| in [2^e, 2^(e+1)), i.e. at most
#    2^-8 |x|; from |x| = 4 on that alone exceeds 1e-2.
#  * the softmax weights enter the bf16 matrix cores as bf16: each weight p_j
#    moves by at most 2^-8 p_j, so a normalised output sum_j p_j v_j / sum p
#    moves by at most U_BF16 * sum_j w_j |v_j| (w the softmax weights; the
#    oracle gives that weighted mean of |v| element by element). It is small
#    for long windows (about 2^-8 * 0.8 for N(0,1) values) and only matters
#    where a few tokens carry the row.
# EPS_F32 covers the fp32 accumulation and exponentials.
U_BF16 = 2.0 ** -8
EPS_F32 = 2.0 ** -12


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=4)
def named_workload(name: str, seed: int = 0):
    return wl.make_workload(name, seed)


def run_gpu(inp, nseg=None, want_shards=False, stream=None):
    """Upload, run plan -> attn -> merge on cuda:0, return host numpy results."""
    import torch
    import mla_paged_decode_verify_amd as mla
    dev = wl.to_device(inp)
    nseg = inp["nseg"] if nseg is None else nseg
    res = mla.mla_verify_forward(dev, nseg=nseg, want_shards=want_shards, stream=stream)
    torch.cuda.synchronize()
    p = res["plan"]
    out = {
        "row_lens": p["row_lens"].cpu().numpy(),
        "page_table": p["page_table"].cpu().numpy(),
        "qo_indptr": p["qo_indptr"].cpu().numpy(),
        "err_flag": int(p["err_flag"].cpu().numpy()[0]),
        "page_size": p["page_size"],
        "out": res["out"].float().cpu().numpy().astype(np.float64),
        "lse": res["lse"].cpu().numpy().astype(np.float64),
        "segm_out": res["partials"][0].cpu().numpy(),
        "segm_max": res["partials"][1].cpu().numpy(),
        "segm_expsum": res["partials"][2].cpu().numpy(),
    }
    if want_shards:
        out["shard_out"] = res["shard_out"].float().cpu().numpy().astype(np.float64)
        out["shard_lse"] = res["shard_lse"].cpu().numpy().astype(np.float64)
    del dev, res
    return out


def oracle_plan(inp):
    return orc.plan(inp["seq_lens"], inp["q_start"], inp["W"], inp["block_table"],
                    inp["block_size"], inp["max_kv_seq_len"], inp.get("interleave", 1))


def max_err(a, b):
    """max |a - b|; equal infinities count as 0, NaN as +inf."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    d = np.abs(np.where(both_inf, 0.0, a) - np.where(both_inf, 0.0, b))
    d = np.where(np.isnan(d), np.inf, d)
    return float(np.max(d)) if d.size else 0.0


def half_ulp_bf16(x):
    """Largest error of rounding x to bf16 (nearest even): 2^(e-8) for |x| in
    [2^e, 2^(e+1)); 0 at 0."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, np.exp2(e - 8), 0.0)


def out_bound(ref, kv_dtype, absv, handoff=False):
    """Per-element bound on |out - ref|: the stated max-abs bound, unless the
    rounding terms above exceed it. absv: the softmax-weighted mean of |v| of
    each element (the same shape as ref). handoff: every merge source's output
    (a shard's, or a (shard, segment) unit's) reaches the merge as bf16; each
    source's o_s moves by at most 2^-8 |o_s|, and sum_s w_s |o_s| <= the
    weighted mean of |v| over the whole window, so that adds U_BF16 * absv
    whatever the partition into sources."""
    ref = np.asarray(ref, dtype=np.float64)
    absv = np.asarray(absv, dtype=np.float64)
    e_pre = U_BF16 * absv * (2.0 if handoff else 1.0) + EPS_F32
    return np.maximum(TOL_OUT[kv_dtype], half_ulp_bf16(np.abs(ref) + e_pre) + e_pre)


def check_out(got, ref, kv_dtype, what, absv, handoff=False):
    """Assert |got - ref| <= out_bound element by element and print the
    max-abs error, the max over elements held to the plain stated bound, and
    how many elements the derived bound covers."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if not got.size:
        return 0.0, 0
    bound = out_bound(ref, kv_dtype, absv, handoff)
    d = np.abs(got - ref)
    d = np.where(np.isnan(d), np.inf, d)
    tol = TOL_OUT[kv_dtype]
    exc = bound > tol
    plain = float(d[~exc].max()) if (~exc).any() else 0.0
    worst = float(d.max())
    say(f"  {what}: max|d|={worst:.3e} (elements held to {tol:g}: max {plain:.3e}); "
        f"{int(exc.sum())} of {d.size} elements past it by bf16 rounding"
        + (f" (max bound {float(bound.max()):.4f}, max|d| there "
           f"{float(d[exc].max()):.3e})" if exc.any() else ""))
    bad = d > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements out of bound; worst "
                           f"|d|={worst:.4g} at |ref|={float(np.abs(ref.ravel()[np.argmax(d)])):.4g}")
    return worst, int(exc.sum())


def weighted_abs_v(inp, requests=None):
    """The softmax-weighted mean of |v| for every (row, head, dim) of the given
    requests: the oracle's attention with |V| as the values (NaN elsewhere)."""
    q = orc.decode_bf16(inp["q_bits"])
    R, H = int(inp["R"]), int(inp["H"])
    out = np.full((R, H, 512), np.nan)
    for i in (range(inp["N"]) if requests is None else requests):
        qs, Q = orc.request_rows(inp["q_start"], i)
        S = int(inp["seq_lens"][i])
        K = orc.gather_request_kv(inp["kv_bits"], inp["kv_dtype"], inp["kv_scale"],
                                  inp["block_table"][i], S, int(inp["W"]),
                                  int(inp["block_size"]), int(inp.get("interleave", 1)))
        out[qs:qs + Q], _ = orc.attention_rows(q[qs:qs + Q], K, S, Q, float(inp["sm_scale"]),
                                               values=np.abs(K[:, :512]))
    return out


def compare_requests(inp, got, requests, what="out"):
    """out / lse of the given requests vs the oracle (split route: no bf16
    hand-off). Returns (max|dout|, max|dlse|)."""
    ref_out, ref_lse = orc.verify_reference(inp, requests)
    absv = weighted_abs_v(inp, requests)
    rows = np.concatenate([np.arange(inp["q_start"][i], inp["q_start"][i + 1]) for i in requests])
    eo, _ = check_out(got["out"][rows], ref_out[rows], inp["kv_dtype"], what, absv[rows])
    el = max_err(got["lse"][rows], ref_lse[rows])
    say(f"  lse: max|d|={el:.3e}")
    return eo, el


def small_spec(**kw):
    spec = dict(N=3, H=16, qlen=4, seq_range=(150, 400), block_size=64, W=3,
                kv_dtype="bf16", nseg=1)
    spec.update(kw)
    return spec


def oracle_shard_results(inp, plan, nseg, want_parts=True):
    """Per-shard (out, lse), the per-shard weighted mean of |v| and
    (want_parts) the segment partials with their weighted |v| from the
    oracle, for every request, using the oracle's own plan."""
    q = orc.decode_bf16(inp["q_bits"])
    W, R, H = inp["W"], inp["R"], inp["H"]
    so = np.zeros((W, R, H, 512))
    sa = np.zeros((W, R, H, 512))
    sl = np.full((W, R, H), -np.inf)
    parts = {}
    for i in range(inp["N"]):
        qs, Q = orc.request_rows(inp["q_start"], i)
        I = int(inp.get("interleave", 1))
        K = orc.gather_request_kv(inp["kv_bits"], inp["kv_dtype"], inp["kv_scale"],
                                  inp["block_table"][i], int(inp["seq_lens"][i]), W,
                                  inp["block_size"], I)
        for r in range(W):
            local = orc.shard_local_kv(K, W, r, I)
            Lr = plan["row_lens"][r, qs:qs + Q]
            vals = np.concatenate([local[:, :512], np.abs(local[:, :512])], axis=1)
            o, l = orc.shard_attention_rows(q[qs:qs + Q], local, Lr, inp["sm_scale"],
                                            values=vals)
            so[r, qs:qs + Q], sa[r, qs:qs + Q], sl[r, qs:qs + Q] = o[..., :512], o[..., 512:], l
            if want_parts:
                parts[(i, r)] = orc.segment_partials(q[qs:qs + Q], local, Lr, nseg,
                                                     plan["page_size"], inp["sm_scale"],
                                                     values=vals)
    return so, sl, sa, parts
