"""The balanced persistent attention (mla_verify_attn_persistent) on cuda:0.

Its schedule cuts the sequence of all (request, row block, shard) groups'
tiles into equal ranges, one per workgroup; a group cut between ranges is
finished by its last piece, which combines the pieces' fp32 states. The tests
recompute that schedule here (a few lines of integer arithmetic from the
plan's row lengths) to know which groups are cut, then check:
  * groups that lie in one range: the per-shard results equal those of
    mla_verify_attn_shard (one segment) bit for bit;
  * every group, cut or not: the per-shard results against the oracle;
  * the final out / lse (after mla_shard_merge) against the oracle;
  * the arrival counters are zero again after the call, and a second call on
    the same workspace gives the same bits (the combination order does not
    depend on which piece finishes last).
Workgroup counts from 1 (one workgroup walks everything, in several batches
of items) to more workgroups than tiles (empty ranges) cover the schedule's
edge cases.
"""

import math

import numpy as np
import pytest

import oracle as orc
import workloads as wl
from helpers import (TOL_LSE, check_out, max_err, named_workload, oracle_plan,
                     oracle_shard_results, say, small_spec, weighted_abs_v)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)
mla = pytest.importorskip("mla_paged_decode_verify_amd")

SMALL_BF16 = {
    "decode_w1": small_spec(W=1, qlen=1, seq_range=(30, 300), block_size=16),
    "verify_w3_b64": small_spec(),
    "verify_w4_b16": small_spec(W=4, block_size=16, seq_range=(60, 700)),
    "verify_w2_b256_p128": small_spec(W=2, block_size=256, seq_range=(200, 900)),
    "verify_w8_b48_p16": small_spec(W=8, block_size=48, seq_range=(100, 1000), qlen=5),
    "odd_block_p1": small_spec(W=2, block_size=3, seq_range=(20, 90), qlen=2, H=4),
    "interleave2_w2": small_spec(W=2, interleave=2, qlen=5, seq_range=(60, 500)),
    "heads128_q8": small_spec(N=2, H=128, qlen=8, W=1, block_size=256, seq_range=(100, 300)),
    "heads12_q7_m84": small_spec(N=3, H=12, qlen=7, W=2, seq_range=(70, 260)),
    "ragged_q": dict(N=5, H=8, qlen_range=(1, 8), seq_range=(8, 200), block_size=32, W=3,
                     kv_dtype="bf16", nseg=1),
    # gangs of 4: row blocks {4, 8, 12} per request
    "heads128_q246": dict(N=3, H=128, qlens=[2, 4, 6], seq_lens=[300, 90, 700], block_size=64,
                          W=2, kv_dtype="bf16", nseg=1),
    # gangs of 2 with an odd max block count: {2, 4} of 4
    "heads64_q24": dict(N=4, H=64, qlens=[2, 4, 2, 4], seq_lens=[150, 400, 64, 230],
                        block_size=32, W=3, kv_dtype="bf16", nseg=1),
    "w_gt_s": dict(N=4, H=4, qlens=[1, 2, 3, 4], seq_lens=[1, 3, 5, 4], block_size=16, W=8,
                   kv_dtype="bf16", nseg=1),
    "q_equals_s": dict(N=2, H=16, qlens=[7, 1], seq_lens=[7, 1], block_size=16, W=2,
                       kv_dtype="bf16", nseg=1),
}


def schedule_model(row_lens, q_start, W, H, max_qlen, pt_width, page_size, ctas):
    """Pieces of every group (i, mb, r) under the schedule the kernel
    computes: gangs of g = gcd(row blocks of every request) workgroups (1 if
    that exceeds ctas); gang-groups (i, gang, r) in that order with
    T = ceil(min(longest row, table) / 64) tiles; gang range q of the
    ctas // g takes tiles [q T / Cg, (q + 1) T / Cg), one row block per member."""
    N = len(q_start) - 1
    mblocks = -(-max_qlen * H // 64)
    nb = [min(-(-(int(q_start[i + 1]) - int(q_start[i])) * H // 64), mblocks) for i in range(N)]
    gang = 0
    for x in nb:
        gang = math.gcd(gang, x)
    if gang < 1 or gang > ctas:
        gang = 1
    ngang = -(-mblocks // gang)
    Cg = ctas // gang
    groups, T = [], []
    for i in range(N):
        qs, qe = int(q_start[i]), int(q_start[i + 1])
        for mg in range(ngang):
            for r in range(W):
                ok = mg * gang < nb[i]
                L = min(int(row_lens[r, qe - 1]), pt_width * page_size) if ok else 0
                groups.append((i, mg, r))
                T.append(-(-L // 64))
    total = sum(T)
    pieces = {}
    P = 0
    for (i, mg, r), t in zip(groups, T):
        if t > 0:
            # gang ranges whose (non-empty) tile ranges meet tiles [P, P + t)
            n, x = 0, P
            while x < P + t:
                q = ((x + 1) * Cg - 1) // total
                x = (q + 1) * total // Cg
                n += 1
            for b in range(gang):
                pieces[(i, mg * gang + b, r)] = n
        P += t
    return pieces, total, gang


def run_persistent(inp, ctas, workspace=None, max_qlen=None):
    dev = wl.to_device(inp)
    if max_qlen is not None:
        dev["max_qlen"] = max_qlen
    W, R, H = inp["W"], inp["R"], inp["H"]
    so = torch.full((W, R, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    sl = torch.full((W, R, H), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full((R, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((R, H), float("nan"), dtype=torch.float32, device="cuda")
    res = mla.mla_verify_forward_shards(dev, shards=(so, sl), out=out, lse=lse, persistent=True,
                                        ctas=ctas, workspace=workspace)
    torch.cuda.synchronize()
    return dev, res


def _rows_of_group(inp, i, mb):
    """(row, head) pairs of row block mb of request i."""
    qs, Q = orc.request_rows(inp["q_start"], i)
    H = inp["H"]
    m = np.arange(mb * 64, min((mb + 1) * 64, Q * H))
    return qs + m // H, m % H


@pytest.mark.parametrize("ctas", [1, 3, 8, 64, 256])
@pytest.mark.parametrize("name", sorted(SMALL_BF16))
def test_persistent_small(name, ctas):
    inp = wl.make_workload(dict(SMALL_BF16[name]), seed=1)
    say(f"persistent case {name} ctas={ctas} S={inp['seq_lens'].tolist()} "
        f"Q={inp['qlens'].tolist()}")
    dev, res = run_persistent(inp, ctas)
    plan = res["plan"]
    row_lens = plan["row_lens"].cpu().numpy()
    pieces, total, gang = schedule_model(row_lens, inp["q_start"], inp["W"], inp["H"],
                                         int(np.max(inp["qlens"])), plan["page_table"].shape[2],
                                         plan["page_size"], ctas)
    ncut = sum(1 for p in pieces.values() if p > 1)
    say(f"  {total} tiles, gang {gang}, {len(pieces)} groups with tiles, {ncut} cut "
        f"(most pieces {max(pieces.values(), default=0)})")
    g_so = res["shard_out"].float().cpu().numpy().astype(np.float64)
    g_sl = res["shard_lse"].cpu().numpy().astype(np.float64)
    assert not np.any(np.isnan(g_so)) and not np.any(np.isnan(g_sl))

    # groups in one range: the bits of the one-segment unit kernel
    so1, sl1 = mla.mla_verify_attn_shard(dev["q"], dev["kv"], plan["row_lens"],
                                         plan["page_table"], dev["q_start"],
                                         page_size=plan["page_size"], max_qlen=dev["max_qlen"],
                                         sm_scale=dev["sm_scale"], nseg=1)
    torch.cuda.synchronize()
    so1 = so1.float().cpu().numpy().astype(np.float64)
    sl1 = sl1.cpu().numpy().astype(np.float64)
    for (i, mb, r), p in pieces.items():
        rows, heads = _rows_of_group(inp, i, mb)
        same = (np.array_equal(g_so[r, rows, heads], so1[r, rows, heads])
                and np.array_equal(g_sl[r, rows, heads], sl1[r, rows, heads]))
        if p == 1:
            assert same, f"uncut group {(i, mb, r)} differs from the unit kernel"

    # every group against the oracle's per-shard results, then the final merge
    so, sl, sa, _ = oracle_shard_results(inp, oracle_plan(inp), 1, want_parts=False)
    check_out(g_so, so, "bf16", "persistent per-shard", sa)
    assert max_err(g_sl, sl) <= TOL_LSE
    out_ref, lse_ref = orc.verify_reference(inp)
    g_out = res["out"].float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(g_out))
    check_out(g_out, out_ref, "bf16", "persistent out (bf16 hand-off)", weighted_abs_v(inp),
              handoff=True)
    assert max_err(res["lse"].cpu().numpy(), lse_ref) <= TOL_LSE


@pytest.mark.parametrize("ctas", [1, 2])
def test_persistent_many_items_per_workgroup(ctas):
    """40 requests on 3 shards (120 groups): one or two workgroups hold more
    items than they keep in LDS at once (64), so the schedule is read again
    for a second batch; results against the oracle and the unit kernel."""
    spec = dict(N=40, H=16, qlen=2, seq_range=(8, 200), block_size=16, W=3, kv_dtype="bf16",
                nseg=1)
    inp = wl.make_workload(spec, seed=17)
    dev, res = run_persistent(inp, ctas)
    plan = res["plan"]
    so1, sl1 = mla.mla_verify_attn_shard(dev["q"], dev["kv"], plan["row_lens"],
                                         plan["page_table"], dev["q_start"],
                                         page_size=plan["page_size"], max_qlen=dev["max_qlen"],
                                         sm_scale=dev["sm_scale"], nseg=1)
    torch.cuda.synchronize()
    g_so = res["shard_out"].float().cpu().numpy().astype(np.float64)
    assert not np.any(np.isnan(g_so))
    if ctas == 1:                            # nothing is cut: the unit kernel's bits
        assert torch.equal(res["shard_out"], so1) and torch.equal(res["shard_lse"], sl1)
    out_ref, lse_ref = orc.verify_reference(inp)
    check_out(res["out"].float().cpu().numpy().astype(np.float64), out_ref, "bf16",
              f"persistent, {ctas} workgroups, 120 groups", weighted_abs_v(inp), handoff=True)
    assert max_err(res["lse"].cpu().numpy(), lse_ref) <= TOL_LSE


@pytest.mark.parametrize("ctas", [5, 256])
def test_persistent_counters_reset_and_deterministic(ctas):
    """Two calls on one workspace: the counters are zero after each, and the
    second call's results equal the first's bit for bit."""
    inp = wl.make_workload(small_spec(N=6, W=4, qlen=4, seq_range=(100, 2000), block_size=64),
                           seed=7)
    N, W, H, Qm = inp["N"], inp["W"], inp["H"], int(np.max(inp["qlens"]))
    nbytes = mla.mla_verify_attn_persistent_workspace_bytes(N, W, H, Qm, ctas)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    groups = N * W * (-(-Qm * H // 64))
    outs = []
    for k in range(2):
        _, res = run_persistent(inp, ctas, workspace=ws)
        assert int(ws[:4 * groups].view(torch.int32).abs().sum().item()) == 0
        outs.append({n: res[n].clone() for n in ("shard_out", "shard_lse", "out", "lse")})
    for n in outs[0]:
        assert torch.equal(outs[0][n], outs[1][n])


@pytest.mark.parametrize("name", ["tiny_decode", "verify_dcp8", "long_context_dcp8",
                                  "ragged_mixed"])
def test_persistent_named_workload(name):
    """The four bf16 workloads at full size on one workgroup per compute unit,
    every request: out / lse against the oracle."""
    inp = named_workload(name)
    dev, res = run_persistent(inp, 0)
    g_out = res["out"].float().cpu().numpy().astype(np.float64)
    g_lse = res["lse"].cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(g_out)) and np.all(np.isfinite(g_lse))
    out_ref, lse_ref = orc.verify_reference(inp)
    eo, _ = check_out(g_out, out_ref, "bf16", f"{name} persistent out (bf16 hand-off)",
                      weighted_abs_v(inp), handoff=True)
    el = max_err(g_lse, lse_ref)
    say(f"persistent {name}: max|dout|={eo:.3e} max|dlse|={el:.3e}")
    assert el <= TOL_LSE


def test_persistent_understated_max_qlen_gives_nan():
    """A request with more (row, head) pairs than max_qlen's row blocks cover:
    its uncovered pairs come out NaN, the covered ones match the oracle."""
    spec = dict(N=3, H=16, qlens=[2, 9, 3], seq_lens=[50, 300, 120], block_size=16, W=3,
                kv_dtype="bf16", nseg=1)
    inp = wl.make_workload(spec, seed=3)
    _, res = run_persistent(inp, 4, max_qlen=4)
    out = res["out"].float().cpu().numpy().astype(np.float64)
    lse = res["lse"].cpu().numpy().astype(np.float64)
    covered = np.zeros((inp["R"], inp["H"]), dtype=bool)
    for i in range(inp["N"]):
        qs, Q = orc.request_rows(inp["q_start"], i)
        for t in range(Q):
            covered[qs + t, :] = [t * inp["H"] + h < 64 for h in range(inp["H"])]
    assert (~covered).sum() == 5 * 16
    assert np.all(np.isnan(out[~covered])) and np.all(np.isnan(lse[~covered]))
    out_ref, lse_ref = orc.verify_reference(inp)
    check_out(out[covered], out_ref[covered], "bf16", "persistent covered pairs",
              weighted_abs_v(inp)[covered], handoff=True)
    assert max_err(lse[covered], lse_ref[covered]) <= TOL_LSE


SMALL_FP8 = {
    "fp8_w4": small_spec(W=4, kv_dtype="fp8_e4m3", qlen=7, H=12, seq_range=(100, 600)),
    "fp8_odd_block_p4": small_spec(W=3, block_size=12, kv_dtype="fp8_e4m3", qlen=3, H=8,
                                   seq_range=(40, 300)),
    "e5m2_w4": small_spec(W=4, kv_dtype="fp8_e5m2", qlen=7, H=12, seq_range=(100, 600)),
    "fp8_q_equals_s": dict(N=2, H=12, qlens=[7, 1], seq_lens=[7, 1], block_size=16, W=2,
                           kv_dtype="fp8_e4m3", nseg=1),
}


@pytest.mark.parametrize("ctas", [1, 5, 64, 256])
@pytest.mark.parametrize("name", sorted(SMALL_FP8))
def test_persistent_fp8_small(name, ctas):
    """fp8 caches (e4m3fn, e5m2; sub-pages of 64 and of 4 tokens) on the
    persistent schedule: uncut groups equal the unit kernel's bits, every
    per-shard result and the final out / lse match the oracle."""
    inp = wl.make_workload(dict(SMALL_FP8[name]), seed=1)
    say(f"persistent fp8 case {name} ctas={ctas} S={inp['seq_lens'].tolist()}")
    dev, res = run_persistent(inp, ctas)
    plan = res["plan"]
    pieces, total, gang = schedule_model(plan["row_lens"].cpu().numpy(), inp["q_start"],
                                         inp["W"], inp["H"], int(np.max(inp["qlens"])),
                                         plan["page_table"].shape[2], plan["page_size"], ctas)
    say(f"  {total} tiles, gang {gang}, {sum(1 for p in pieces.values() if p > 1)} cut groups")
    g_so = res["shard_out"].float().cpu().numpy().astype(np.float64)
    g_sl = res["shard_lse"].cpu().numpy().astype(np.float64)
    assert not np.any(np.isnan(g_so)) and not np.any(np.isnan(g_sl))
    so1, sl1 = mla.mla_verify_attn_shard(dev["q"], dev["kv"], plan["row_lens"],
                                         plan["page_table"], dev["q_start"],
                                         page_size=plan["page_size"], max_qlen=dev["max_qlen"],
                                         sm_scale=dev["sm_scale"], kv_scale=dev["kv_scale"],
                                         nseg=1)
    torch.cuda.synchronize()
    so1 = so1.float().cpu().numpy().astype(np.float64)
    sl1 = sl1.cpu().numpy().astype(np.float64)
    for (i, mb, r), p in pieces.items():
        if p == 1:
            rows, heads = _rows_of_group(inp, i, mb)
            assert np.array_equal(g_so[r, rows, heads], so1[r, rows, heads])
            assert np.array_equal(g_sl[r, rows, heads], sl1[r, rows, heads])
    so, sl, sa, _ = oracle_shard_results(inp, oracle_plan(inp), 1, want_parts=False)
    check_out(g_so, so, inp["kv_dtype"], "persistent fp8 per-shard", sa)
    assert max_err(g_sl, sl) <= TOL_LSE
    out_ref, lse_ref = orc.verify_reference(inp)
    g_out = res["out"].float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(g_out))
    check_out(g_out, out_ref, inp["kv_dtype"], "persistent fp8 out (bf16 hand-off)",
              weighted_abs_v(inp), handoff=True)
    assert max_err(res["lse"].cpu().numpy(), lse_ref) <= TOL_LSE


def test_persistent_fp8_named_workload():
    """fp8_verify_dcp4 at full size on one workgroup per compute unit, every
    request: out / lse against the oracle."""
    inp = named_workload("fp8_verify_dcp4")
    _, res = run_persistent(inp, 0)
    g_out = res["out"].float().cpu().numpy().astype(np.float64)
    g_lse = res["lse"].cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(g_out)) and np.all(np.isfinite(g_lse))
    out_ref, lse_ref = orc.verify_reference(inp)
    eo, _ = check_out(g_out, out_ref, "fp8_e4m3", "fp8_verify_dcp4 persistent out",
                      weighted_abs_v(inp), handoff=True)
    el = max_err(g_lse, lse_ref)
    say(f"persistent fp8_verify_dcp4: max|dout|={eo:.3e} max|dlse|={el:.3e}")
    assert el <= TOL_LSE
