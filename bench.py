#!/usr/bin/env python3
"""Throughput of the paged MLA verify hot path on one MI355X.

One step = plan (row lengths + sub-page tables) -> attention -> merge, over
one batch of the workload, inputs resident in HBM. Routes (--path; by default
the workload's own, measured fastest): shards -- the attention kernel runs one
workgroup per (shard, split-K segment, row block) unit, normalises each unit's
result and writes it as bf16 output + natural-log LSE, and the merge is one
LSE merge over the W * nseg units; persistent -- one workgroup per compute
unit on equal shares of all tiles (groups cut between workgroups are combined
in the kernel), then the LSE merge over the W shards; split -- fp32
segment partials, then the segment merge and the shard merge. The KV cache is
rotated over several copies (more than the 256 MB Infinity Cache holds) so
that no step re-reads the previous step's KV from cache. Timed steps launch
the three calls from Python; --graph replays a HIP graph of them instead (one
graph per KV copy; on this stack a replay costs more launch overhead than the
eager calls).
`eager_split_us` splits eager steps with events (host launch gaps included);
the attention kernel's own duration comes from back-to-back launches.
Prints one JSON line.

    python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--workload verify_dcp8]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA verify attention KV GB/s (% of HBM peak) + verify rows/sec at 1 GPU"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}   # dense, by the MFMA operand type


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="verify_dcp8")
    ap.add_argument("--nseg", type=int, default=None)
    ap.add_argument("--path", choices=["split", "shards", "persistent"], default=None,
                    help="default: the workload's route (persistent for fp8_verify_dcp4, "
                         "long_context_dcp8 and ragged_mixed, shards otherwise). shards: attn_shard (every (shard, segment) unit normalised, bf16 "
                         "+ LSE) -> shard_merge over the W * nseg units; split: attn fp32 "
                         "partials -> lse_merge (segment merge, then shard merge); "
                         "persistent: attn_persistent (one workgroup per compute unit on "
                         "equal shares of all tiles, one segment) -> shard_merge")
    ap.add_argument("--ctas", type=int, default=0,
                    help="persistent path: workgroups (0: one per compute unit)")
    ap.add_argument("--kv-copies", type=int, default=0,
                    help="KV copies to rotate over (0: enough for > 512 MB)")
    ap.add_argument("--graph", action="store_true",
                    help="replay a HIP graph of each step's three launches instead of "
                         "launching them from Python")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-shard0", action="store_true",
                    help="skip the shard-0-alone timing (every attention launch of the run "
                         "is then a full one, for profiler runs)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="before the timed steps, run a plain elementwise copy of MB MiB "
                         "(read + write) three times: the reference kernel for scaling "
                         "FETCH_SIZE / WRITE_SIZE counters in a rocprofv3 --pmc run")
    return ap.parse_args()


# sources of the attention kernel that runs a workload, by its KV dtype and path
ATTN_SOURCES = {"bf16": ["attn_common.h", "attn_bf16.hip", "internal.h"],
                "fp8": ["attn_common.h", "attn_f8mma.h", "attn_fp8.hip", "internal.h"],
                "persistent": ["attn_common.h", "attn_f8mma.h", "attn_persist.hip", "internal.h"]}
ATTN_KERNELS = {"bf16": "attn_bf16_kernel", "fp8": "attn_fp8_kernel",
                "persistent": "attn_persist_kernel"}


def attn_kind(workload, path):
    import workloads as wl
    if path == "persistent":
        return "persistent"
    return "bf16" if wl.CONFIGS[workload]["kv_dtype"] == "bf16" else "fp8"


def attn_source_hash(workload="verify_dcp8", path="shards"):
    """sha256 over the sources of the attention kernel that runs `workload`
    on `path` (to tell whether stored counter readings still describe it)."""
    import hashlib
    h = hashlib.sha256()
    for name in ATTN_SOURCES[attn_kind(workload, path)]:
        with open(os.path.join(ROOT, "mla_paged_decode_verify_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def summary_path(workload, path, what):
    """profiles/ summary of `what` (traffic, mfma) for the kernel of `path`."""
    stem = "attn_persist" if path == "persistent" else "attn"
    return os.path.join(ROOT, "profiles", f"{stem}_{workload}_{what}.txt")


def _stored(workload, path, what):
    """key: value lines of a committed counter summary, or None if there is
    none for this workload and kernel or the kernel's sources changed since."""
    fn = summary_path(workload, path, what)
    if not os.path.exists(fn):
        return None
    kv = {}
    with open(fn) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.split("(")[0].strip()] = v.split()[0] if v.split() else ""
    if (kv.get("workload") != workload
            or kv.get("source_sha256") != attn_source_hash(workload, path)
            or kv.get("path", path) != path):
        return None
    return kv


def stored_traffic(workload, path="shards"):
    """HBM bytes per attention launch (FETCH_SIZE + WRITE_SIZE, scaled) from
    the committed counter summary, or None (none, or the kernel changed)."""
    kv = _stored(workload, path, "traffic")
    try:
        return int(kv["fetch_bytes_per_launch"]) + int(kv["write_bytes_per_launch"])
    except (TypeError, KeyError, ValueError):
        return None


def stored_mfma_flops(workload, path="shards"):
    """Executed MFMA flops per attention launch ((SQ_INSTS_VALU_MFMA_MOPS_BF16 +
    SQ_INSTS_VALU_MFMA_MOPS_F8) x 512) from the committed counter summary, or
    None."""
    kv = _stored(workload, path, "mfma")
    try:
        return float(kv["executed_mfma_flops_per_launch"])
    except (TypeError, KeyError, ValueError):
        return None


def cpu_baseline(inp, target_s):
    """Time the fp64 oracle on a bounded sample: whole requests in order,
    cycling over the batch, until about target_s seconds of CPU work."""
    import oracle as orc
    import workloads as wl
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    n_req, t_total, kv_bytes, rows = 0, 0.0, 0, 0
    bpt = wl.kv_bytes_per_token(inp["kv_dtype"])
    while t_total < target_s:
        i = n_req % inp["N"]
        t0 = time.perf_counter()
        orc.verify_reference(inp, [i])
        t_total += time.perf_counter() - t0
        n_req += 1
        kv_bytes += int(inp["seq_lens"][i]) * bpt
        rows += int(inp["qlens"][i])
    return {
        "value": kv_bytes / t_total / 1e9, "unit": "GB/s", "cores": int(threads),
        "kind": "oracle",
        "sample": f"{n_req} requests ({n_req / inp['N']:.2f} passes over the {inp['N']}-request "
                  f"batch, in order; {rows} verify rows, {kv_bytes / 1e6:.1f} MB of KV) in "
                  f"{t_total:.1f} s; rows/s {rows / t_total:.3g}; host cpus {os.cpu_count()}",
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (got --gpus {args.gpus}); "
              "the path has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads as wl
    import mla_paged_decode_verify_amd as mla

    inp = wl.make_workload(args.workload, 0)
    path = args.path or inp["path"]
    nseg = (1 if path == "persistent" else inp["nseg"]) if args.nseg is None else args.nseg
    dev = wl.to_device(inp)
    kv_bytes = wl.algorithmic_kv_bytes(inp)
    flops = wl.algorithmic_flops(inp)
    kv_dev_bytes = dev["kv"].numel() * dev["kv"].element_size()
    copies = args.kv_copies or (-(-(512 << 20) // kv_dev_bytes) + 1)
    kvs = [dev["kv"]] + [dev["kv"].clone() for _ in range(copies - 1)]
    R, H, W = inp["R"], inp["H"], inp["W"]

    # preallocated outputs (the library allocates nothing)
    page_size = mla.mla_subpage_size(inp["block_size"])
    ptw = mla.mla_pt_width(inp["max_kv_seq_len"], page_size)
    i32 = dict(dtype=torch.int32, device="cuda")
    plan_bufs = dict(row_lens=torch.empty((W, R), **i32),
                     page_table=torch.empty((W, R, ptw), **i32),
                     qo_indptr=torch.empty((R + 1,), **i32), err_flag=torch.zeros((1,), **i32))
    f32 = dict(dtype=torch.float32, device="cuda")
    workspace = None
    if path == "persistent":
        if nseg != 1:
            raise SystemExit("the persistent path takes one segment")
        workspace = torch.zeros(mla.mla_verify_attn_persistent_workspace_bytes(
            inp["N"], W, H, dev["max_qlen"], args.ctas), dtype=torch.uint8, device="cuda")
    if path == "split":
        parts = (torch.empty((W, R, H, nseg, 512), **f32), torch.empty((W, R, H, nseg), **f32),
                 torch.empty((W, R, H, nseg), **f32))
    else:
        parts = (torch.empty((W * nseg, R, H, 512), dtype=torch.bfloat16, device="cuda"),
                 torch.empty((W * nseg, R, H), **f32))

    def attn(kv, row_lens, page_table, bufs):
        if path == "split":
            mla.mla_verify_attn(dev["q"], kv, row_lens, page_table, dev["q_start"],
                                page_size=page_size, max_qlen=dev["max_qlen"], nseg=nseg,
                                sm_scale=dev["sm_scale"], kv_scale=dev["kv_scale"],
                                segm_out=bufs[0], segm_max=bufs[1], segm_expsum=bufs[2])
        elif path == "persistent":
            mla.mla_verify_attn_persistent(dev["q"], kv, row_lens, page_table, dev["q_start"],
                                           page_size=page_size, max_qlen=dev["max_qlen"],
                                           sm_scale=dev["sm_scale"], kv_scale=dev["kv_scale"],
                                           ctas=args.ctas, workspace=workspace,
                                           shard_out=bufs[0], shard_lse=bufs[1])
        else:
            mla.mla_verify_attn_shard(dev["q"], kv, row_lens, page_table, dev["q_start"],
                                      page_size=page_size, max_qlen=dev["max_qlen"],
                                      sm_scale=dev["sm_scale"], kv_scale=dev["kv_scale"],
                                      nseg=nseg, shard_out=bufs[0], shard_lse=bufs[1])
    out = torch.empty((R, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((R, H), **f32)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]

    def step(k, events=None):
        e = events
        if e: e[0].record()
        plan = mla.mla_verify_plan(dev["seq_lens"], dev["q_start"], R, W, dev["block_table"],
                                   dev["num_blocks"], inp["block_size"], inp["max_kv_seq_len"],
                                   **plan_bufs)
        if e: e[1].record()
        attn(kvs[k % len(kvs)], plan["row_lens"], plan["page_table"], parts)
        if e: e[2].record()
        if path == "split":
            mla.mla_lse_merge(*parts, plan["row_lens"], dev["q_start"], page_size=page_size,
                              H=H, nseg=nseg, out=out, lse=lse)
        else:
            mla.mla_shard_merge(*parts, out=out, lse=lse)
        if e: e[3].record()

    if args.copy_calibration > 0:
        n = args.copy_calibration << 18            # float32 elements in MB MiB
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    if int(plan_bufs["err_flag"].item()) != 0:
        raise SystemExit(f"plan reported errors: {int(plan_bufs['err_flag'].item())}")
    # Per-kernel split of a step: eager steps bracketed by events.
    for k in range(args.steps):
        step(k, ev[k])
    torch.cuda.synchronize()
    plan_ms = np.mean([e[0].elapsed_time(e[1]) for e in ev])
    attn_ms = np.mean([e[1].elapsed_time(e[2]) for e in ev])
    merge_ms = np.mean([e[2].elapsed_time(e[3]) for e in ev])
    # The timed steps: the eager calls, or one HIP graph per KV copy holding
    # the step's three launches.
    graphs = []
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for c in range(len(kvs)):
                step(c)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for c in range(len(kvs)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(c)
            graphs.append(g)
        for k in range(args.warmup):
            graphs[k % len(graphs)].replay()
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        if graphs:
            graphs[k % len(graphs)].replay()
        else:
            step(k)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if int(plan_bufs["err_flag"].item()) != 0:
        raise SystemExit(f"plan reported errors: {int(plan_bufs['err_flag'].item())}")
    # The attention kernel's average launch duration: back-to-back launches on
    # the same stream (the plan is already in place), bracketed by two events.
    n_attn = 20
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record()
    for k in range(n_attn):
        attn(kvs[k % len(kvs)], plan_bufs["row_lens"], plan_bufs["page_table"], parts)
    a1.record()
    torch.cuda.synchronize()
    attn_launch_ms = a0.elapsed_time(a1) / n_attn

    # Attention + merge (the hot path without the once-per-forward plan), per
    # eager step from the step events: median and min.
    am = np.array([e[1].elapsed_time(e[3]) for e in ev]) * 1e3

    # One GPU's share in a real DCP deployment: shard 0 alone at its real
    # shape (its pool, its row lengths and page table), back to back.
    shard_us = None
    if W > 1 and not args.no_shard0:
        kv0 = [kv[0:1] for kv in kvs]
        p0 = tuple(b[0:nseg] if path != "split" else b[0:1] for b in parts)
        rl0, pt0 = plan_bufs["row_lens"][0:1], plan_bufs["page_table"][0:1]
        attn0 = lambda k: attn(kv0[k % len(kv0)], rl0, pt0, p0)
        for k in range(3):
            attn0(k)
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        for k in range(n_attn):
            attn0(k)
        s1.record()
        torch.cuda.synchronize()
        shard_us = s0.elapsed_time(s1) / n_attn * 1e3
        del p0

    # Measured copy peak: a 2 GiB elementwise copy (read + write), larger than
    # the Infinity Cache, timed with events.
    cp = torch.ones(1 << 29, dtype=torch.float32, device="cuda")
    cq = torch.empty_like(cp)
    torch.mul(cp, 1.0, out=cq)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(3):
        torch.mul(cp, 1.0, out=cq)
    c1.record()
    torch.cuda.synchronize()
    copy_gbs = 3 * 2 * cp.numel() * 4 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del cp, cq
    ms_step = wall * 1e3 / args.steps
    achieved = kv_bytes / (attn_launch_ms * 1e-3) / 1e9
    mfma_flops = stored_mfma_flops(args.workload, path)
    # bf16 KV runs on bf16 MFMAs, fp8 KV on the fp8 ones (both kernels)
    mfma_peak = MFMA_PEAK_TFLOPS["bf16" if inp["kv_dtype"] == "bf16" else "fp8"]
    res = {
        "metric": METRIC,
        "value": round(kv_bytes / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        # fp8 KV: fp8 MFMAs, KV codes against Q and P as e4m3fn term pairs
        "dtype": {"bf16": "bf16", "fp8_e4m3": "fp8e4m3",
                  "fp8_e5m2": "fp8e5m2-kv/fp8e4m3"}[inp["kv_dtype"]],
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": inp["N"], "heads": H,
                   "qlen": int(np.max(inp["qlens"])), "rows": R, "shards": W,
                   "block_size": inp["block_size"], "page_size": page_size, "nseg": nseg,
                   "kv_dtype": inp["kv_dtype"], "sum_seq_len": int(inp["seq_lens"].sum()),
                   "kv_copies": len(kvs), "path": path},
        "rows_per_s": round(R / (ms_step * 1e-3), 1),
        "hbm_frac": round(kv_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "launch": "hip_graph" if args.graph else "eager",
        "eager_split_us": {"plan": round(plan_ms * 1e3, 2), "attn": round(attn_ms * 1e3, 2),
                      "merge": round(merge_ms * 1e3, 2),
                      "attn_back_to_back": round(attn_launch_ms * 1e3, 2)},
        "attn_merge_us": {"median": round(float(np.median(am)), 2), "min": round(float(am.min()), 2),
                          "kv_gbs_median": round(kv_bytes / (float(np.median(am)) * 1e-6) / 1e9, 1)},
        "shard0_alone_attn_us": None if shard_us is None else round(shard_us, 2),
        "bytes": {"kv_algorithmic": kv_bytes, "q": R * H * 1152, "out": R * H * (1024 + 4),
                  "partials": W * R * H * nseg * ((2048 + 8) if path == "split" else (1024 + 4))},
        "t_roof_us": round(max(kv_bytes / (HBM_PEAK_GBS * 1e9), flops / 2.5e15) * 1e6, 2),
        "hbm_copy_peak_gbs": round(copy_gbs, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": stored_traffic(args.workload, path),
                     "kernel": ATTN_KERNELS[attn_kind(args.workload, path)],
                     "bytes_per_launch": kv_bytes, "flops_per_launch": flops,
                     "frac_of_copy_peak": round(achieved / copy_gbs, 4)},
        # the dense part: executed MFMA flops (from the committed counter
        # summary, null once the kernel has changed) over this run's attention time
        "mfma": None if mfma_flops is None else {
            "executed_flops_per_launch": mfma_flops,
            "achieved_tflops": round(mfma_flops / (attn_launch_ms * 1e-3) / 1e12, 1),
            "peak_tflops": mfma_peak,
            "util": round(mfma_flops / (attn_launch_ms * 1e-3) / 1e12 / mfma_peak, 4)},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
