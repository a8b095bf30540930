"""The whole path (plan -> attention -> merge) captured in a HIP graph: every
replay, with the program's own eager work and synchronisations between
replays, reproduces the eager result bit for bit (no kernel of the path uses
atomics whose order could vary, and none of them is a memset node)."""

import numpy as np
import pytest

import workloads as wl
from helpers import say, small_spec

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)
mla = pytest.importorskip("mla_paged_decode_verify_amd")


@pytest.mark.parametrize("kv_dtype,nseg", [("bf16", 1), ("bf16", 3), ("fp8_e4m3", 2)])
def test_graph_replays_match_eager(kv_dtype, nseg):
    inp = wl.make_workload(small_spec(N=4, W=2, kv_dtype=kv_dtype, nseg=nseg), seed=5)
    say(f"graph case kv={kv_dtype} nseg={nseg} S={inp['seq_lens'].tolist()}")
    dev = wl.to_device(inp)
    eager = mla.mla_verify_forward(dev, nseg=nseg)
    torch.cuda.synchronize()
    ref_out, ref_lse = eager["out"].clone(), eager["lse"].clone()
    assert torch.isfinite(ref_out.float()).all()

    plan_bufs = {k: torch.empty_like(eager["plan"][k])
                 for k in ("row_lens", "page_table", "qo_indptr")}
    plan_bufs["err_flag"] = torch.zeros_like(eager["plan"]["err_flag"])
    parts = tuple(torch.empty_like(p) for p in eager["partials"])
    out, lse = torch.empty_like(ref_out), torch.empty_like(ref_lse)

    def step():
        plan = mla.mla_verify_plan(dev["seq_lens"], dev["q_start"], dev["R"], dev["W"],
                                   dev["block_table"], dev["num_blocks"], dev["block_size"],
                                   dev["max_kv_seq_len"], **plan_bufs)
        mla.mla_verify_forward(dev, nseg=nseg, plan=plan, partials=parts, out=out, lse=lse)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep in range(4):
        # poison every output and partial, run unrelated eager work, replay
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        for p in parts:
            p.fill_(float("nan"))
        plan_bufs["row_lens"].fill_(-7)
        torch.cuda.synchronize()
        mla.mla_verify_forward(dev, nseg=nseg)
        graph.replay()
        torch.cuda.synchronize()
        say(f"  replay {rep}: max|d out|="
            f"{(out.float() - ref_out.float()).abs().max().item():.3g}")
        assert int(plan_bufs["err_flag"].item()) == 0
        assert np.array_equal(plan_bufs["row_lens"].cpu().numpy(),
                              eager["plan"]["row_lens"].cpu().numpy())
        assert torch.equal(out, ref_out)
        assert torch.equal(lse, ref_lse)


def test_graph_static_bound_replays_new_lengths():
    """Static-bound mode: the graph is captured once for fixed shapes and a
    fixed max_kv_seq_len; before each replay the requests' lengths change in
    place (every S_i between Q_i and its captured length). Each replay equals
    an eager run on the new lengths bit for bit and matches the oracle: the
    kernels read every length from device memory, so segments that lose their
    tokens are simply inactive."""
    import oracle as orc
    from helpers import TOL_LSE, check_out, max_err, weighted_abs_v

    spec = small_spec(N=4, W=3, qlen=4, seq_range=(200, 500), nseg=2)
    inp = wl.make_workload(spec, seed=9)
    dev = wl.to_device(inp)
    nseg = spec["nseg"]
    eager = mla.mla_verify_forward(dev, nseg=nseg)
    torch.cuda.synchronize()
    plan_bufs = {k: torch.empty_like(eager["plan"][k])
                 for k in ("row_lens", "page_table", "qo_indptr")}
    plan_bufs["err_flag"] = torch.zeros_like(eager["plan"]["err_flag"])
    parts = tuple(torch.empty_like(p) for p in eager["partials"])
    out, lse = torch.empty_like(eager["out"]), torch.empty_like(eager["lse"])

    def step():
        plan = mla.mla_verify_plan(dev["seq_lens"], dev["q_start"], dev["R"], dev["W"],
                                   dev["block_table"], dev["num_blocks"], dev["block_size"],
                                   dev["max_kv_seq_len"], **plan_bufs)
        mla.mla_verify_forward(dev, nseg=nseg, plan=plan, partials=parts, out=out, lse=lse)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    rng = np.random.default_rng(4)
    S0, Q = inp["seq_lens"].copy(), inp["qlens"]
    for rep in range(3):
        S = np.array([int(rng.integers(q, s + 1)) for q, s in zip(Q, S0)], dtype=np.int64)
        say(f"  replay {rep}: S={S.tolist()}")
        dev["seq_lens"].copy_(torch.from_numpy(S.astype(np.int32)).to("cuda"))
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        ref = mla.mla_verify_forward(dev, nseg=nseg)
        torch.cuda.synchronize()
        assert int(plan_bufs["err_flag"].item()) == 0
        assert torch.equal(out, ref["out"]) and torch.equal(lse, ref["lse"])
        inp_r = dict(inp, seq_lens=S)
        out_ref, lse_ref = orc.verify_reference(inp_r)
        got = out.float().cpu().numpy().astype(np.float64)
        check_out(got, out_ref, "bf16", "graph replay out", weighted_abs_v(inp_r))
        assert max_err(lse.cpu().numpy().astype(np.float64), lse_ref) <= TOL_LSE


def test_graph_one_segment_route_replays_new_lengths():
    """The one-segment route (plan -> attn_shard -> shard_merge) captured
    once; before each replay the requests' lengths change in place, down to
    S_i = Q_i, which leaves most of the 8 shards without a token (their
    units write o_r = 0, lse_r = -inf). Every replay equals an eager run of
    the same route on the new lengths bit for bit, and its per-shard results
    equal those of the split route, with outputs poisoned before each
    replay."""
    spec = small_spec(N=5, W=8, qlen=2, seq_range=(100, 900), nseg=1)
    inp = wl.make_workload(spec, seed=12)
    dev = wl.to_device(inp)
    first = mla.mla_verify_forward_shards(dev)
    torch.cuda.synchronize()
    plan_bufs = {k: torch.empty_like(first["plan"][k])
                 for k in ("row_lens", "page_table", "qo_indptr")}
    plan_bufs["err_flag"] = torch.zeros_like(first["plan"]["err_flag"])
    shards = (torch.empty_like(first["shard_out"]), torch.empty_like(first["shard_lse"]))
    out, lse = torch.empty_like(first["out"]), torch.empty_like(first["lse"])

    def step():
        plan = mla.mla_verify_plan(dev["seq_lens"], dev["q_start"], dev["R"], dev["W"],
                                   dev["block_table"], dev["num_blocks"], dev["block_size"],
                                   dev["max_kv_seq_len"], **plan_bufs)
        mla.mla_verify_forward_shards(dev, plan=plan, shards=shards, out=out, lse=lse)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    rng = np.random.default_rng(6)
    S0, Q = inp["seq_lens"].copy(), inp["qlens"]
    for rep in range(4):
        S = np.array([int(rng.integers(q, s + 1)) for q, s in zip(Q, S0)], dtype=np.int64)
        if rep == 1:
            S[:3] = Q[:3]                         # 2 tokens over 8 shards
        say(f"  replay {rep}: S={S.tolist()}")
        dev["seq_lens"].copy_(torch.from_numpy(S.astype(np.int32)).to("cuda"))
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        for b in shards:
            b.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = mla.mla_verify_forward_shards(dev)
        split = mla.mla_verify_forward(dev, nseg=1, want_shards=True)
        torch.cuda.synchronize()
        assert int(plan_bufs["err_flag"].item()) == 0
        assert torch.equal(out, ref["out"]) and torch.equal(lse, ref["lse"])
        assert torch.equal(shards[0], split["shard_out"])
        assert torch.equal(shards[1], split["shard_lse"])


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("ctas", [0, 7])
def test_graph_persistent_route_replays_new_lengths(ctas, kv_dtype):
    """The persistent route (plan -> attn_persistent -> shard_merge) captured
    once with one workspace: its arrival counters are left at zero by every
    launch, so each replay -- lengths changed in place before it, some groups
    cut between workgroups, some shards empty -- equals an eager run of the
    same route on the new lengths bit for bit."""
    spec = small_spec(N=6, W=4, qlen=3, seq_range=(100, 1500), nseg=1, kv_dtype=kv_dtype)
    inp = wl.make_workload(spec, seed=21)
    dev = wl.to_device(inp)
    nbytes = mla.mla_verify_attn_persistent_workspace_bytes(inp["N"], inp["W"], inp["H"],
                                                            dev["max_qlen"], ctas)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    first = mla.mla_verify_forward_shards(dev, persistent=True, ctas=ctas, workspace=ws)
    torch.cuda.synchronize()
    plan_bufs = {k: torch.empty_like(first["plan"][k])
                 for k in ("row_lens", "page_table", "qo_indptr")}
    plan_bufs["err_flag"] = torch.zeros_like(first["plan"]["err_flag"])
    shards = (torch.empty_like(first["shard_out"]), torch.empty_like(first["shard_lse"]))
    out, lse = torch.empty_like(first["out"]), torch.empty_like(first["lse"])

    def step():
        plan = mla.mla_verify_plan(dev["seq_lens"], dev["q_start"], dev["R"], dev["W"],
                                   dev["block_table"], dev["num_blocks"], dev["block_size"],
                                   dev["max_kv_seq_len"], **plan_bufs)
        mla.mla_verify_forward_shards(dev, plan=plan, shards=shards, out=out, lse=lse,
                                      persistent=True, ctas=ctas, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    ws2 = torch.zeros_like(ws)
    rng = np.random.default_rng(8)
    S0, Q = inp["seq_lens"].copy(), inp["qlens"]
    for rep in range(4):
        S = np.array([int(rng.integers(q, s + 1)) for q, s in zip(Q, S0)], dtype=np.int64)
        if rep == 2:
            S[:2] = Q[:2]
        say(f"  replay {rep}: S={S.tolist()}")
        dev["seq_lens"].copy_(torch.from_numpy(S.astype(np.int32)).to("cuda"))
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        for b in shards:
            b.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = mla.mla_verify_forward_shards(dev, persistent=True, ctas=ctas, workspace=ws2)
        torch.cuda.synchronize()
        assert int(plan_bufs["err_flag"].item()) == 0
        assert torch.equal(shards[0], ref["shard_out"]) and torch.equal(shards[1], ref["shard_lse"])
        assert torch.equal(out, ref["out"]) and torch.equal(lse, ref["lse"])
        groups = inp["N"] * inp["W"] * (-(-dev["max_qlen"] * inp["H"] // 64))
        assert int(ws[:4 * groups].view(torch.int32).abs().sum().item()) == 0
