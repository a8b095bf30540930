"""Shared test utilities: cached workloads, running the HIP path, comparing
against the oracle. Test infrastructure only."""

from __future__ import annotations

import functools
import sys

import numpy as np

import oracle as orc
import workloads as wl

TOL_OUT = {"bf16": 1e-2, "fp8_e4m3": 3e-2, "fp8_e5m2": 3e-2}   # absolute floor on out
TOL_LSE = 1e-3                                # max-abs on lse
# The output is bf16 (8 significant bits) and the path rounds to bf16 three
# times: the softmax weights fed to the PV product, each shard's output as it
# is handed to the shard merge, and the final output -- each at most 2^-9
# relative. So |got - ref| <= max(floor, 2^-7 |ref|): for |ref| <= 1.28 this is
# the plain max-abs floor; above that the bf16 format's own spacing dominates.
REL_OUT = 2.0 ** -7


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
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    d = np.where(both_inf, 0.0, np.abs(a - b))
    return float(np.max(d)) if d.size else 0.0


def out_excess(got, ref, kv_dtype):
    """max over elements of |got - ref| / max(floor, 2^-7 |ref|); <= 1 passes."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if not got.size:
        return 0.0
    bound = np.maximum(TOL_OUT[kv_dtype], REL_OUT * np.abs(ref))
    return float(np.max(np.abs(got - ref) / bound))


def compare_requests(inp, got, requests):
    """Max errors of out / lse over the given requests vs the oracle."""
    ref_out, ref_lse = orc.verify_reference(inp, requests)
    rows = np.concatenate([np.arange(inp["q_start"][i], inp["q_start"][i + 1]) for i in requests])
    eo = max_err(got["out"][rows], ref_out[rows])
    el = max_err(got["lse"][rows], ref_lse[rows])
    ex = out_excess(got["out"][rows], ref_out[rows], inp["kv_dtype"])
    return eo, el, ex, ref_out, ref_lse, rows


def sample_requests(inp, k):
    """The longest, the shortest and k-2 evenly spaced other requests."""
    N = inp["N"]
    if N <= k:
        return list(range(N))
    S = inp["seq_lens"]
    pick = {int(np.argmax(S)), int(np.argmin(S))}
    for i in np.linspace(0, N - 1, k):
        pick.add(int(i))
    return sorted(pick)[:max(k, 2)]


def small_spec(**kw):
    spec = dict(N=3, H=16, qlen=4, seq_range=(150, 400), block_size=64, W=3,
                kv_dtype="bf16", nseg=1)
    spec.update(kw)
    return spec


def oracle_shard_results(inp, plan, nseg):
    """Per-shard (out, lse) and the segment partials from the oracle, for every
    request, using the oracle's own plan."""
    q = orc.decode_bf16(inp["q_bits"])
    W, R, H = inp["W"], inp["R"], inp["H"]
    so = np.zeros((W, R, H, 512))
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
            o, l = orc.shard_attention_rows(q[qs:qs + Q], local, Lr, inp["sm_scale"])
            so[r, qs:qs + Q], sl[r, qs:qs + Q] = o, l
            parts[(i, r)] = orc.segment_partials(q[qs:qs + Q], local, Lr, nseg,
                                                 plan["page_size"], inp["sm_scale"])
    return so, sl, parts
