"""Parity of the HIP path (through the C ABI) with the fp64 oracle on cuda:0.

Plans (row lengths, sub-page tables, qo_indptr) must match bit for bit.
Outputs: max-abs 1e-2 (bf16 KV) or 3e-2 (fp8 KV) per element, except where
the bf16 roundings derived in tests/helpers.py (the bf16 output, the one-
segment route's bf16 hand-off, the bf16 softmax weights) can exceed it: there
the derived bound; each check prints how many elements that covers. LSE:
max-abs 1e-3.
"""

import math

import numpy as np
import pytest

import oracle as orc
import workloads as wl
from helpers import (EPS_F32, TOL_LSE, TOL_OUT, U_BF16, check_out, compare_requests, max_err,
                     named_workload, oracle_plan, oracle_shard_results, run_gpu, say,
                     small_spec, weighted_abs_v)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)
mla = pytest.importorskip("mla_paged_decode_verify_amd")


def _check_plan(inp, got):
    ref = oracle_plan(inp)
    assert got["err_flag"] == 0
    assert got["page_size"] == ref["page_size"]
    assert np.array_equal(got["row_lens"], ref["row_lens"])
    assert np.array_equal(got["page_table"], ref["page_table"])
    assert np.array_equal(got["qo_indptr"], ref["qo_indptr"])
    return ref


# ------------------------------------------------------------ small cases ---

SMALL = {
    "decode_w1": small_spec(W=1, qlen=1, seq_range=(30, 300), block_size=16),
    "verify_w3_b64": small_spec(),
    "verify_w4_b16": small_spec(W=4, block_size=16, seq_range=(60, 700)),
    "verify_w2_b256_p128": small_spec(W=2, block_size=256, seq_range=(200, 900)),
    "verify_w8_b48_p16": small_spec(W=8, block_size=48, seq_range=(100, 1000), qlen=5),
    "odd_block_p1": small_spec(W=2, block_size=3, seq_range=(20, 90), qlen=2, H=4),
    "fp8_w4": small_spec(W=4, kv_dtype="fp8_e4m3", qlen=7, H=12, seq_range=(100, 600)),
    # fp8 with 4-token sub-pages (per-token page lookups) and with 16-token ones
    "fp8_odd_block_p4": small_spec(W=3, block_size=12, kv_dtype="fp8_e4m3", qlen=3, H=8,
                                   seq_range=(40, 500)),
    "fp8_b48_p16": small_spec(W=2, block_size=48, kv_dtype="fp8_e4m3", qlen=5, H=12,
                              seq_range=(150, 900)),
    # e5m2 codes (the fp8_e5m2 cache dtype), 64- and 4-token sub-pages
    "e5m2_w4": small_spec(W=4, kv_dtype="fp8_e5m2", qlen=7, H=12, seq_range=(100, 600)),
    # runs of I > 1 positions per shard (interleave)
    "interleave2_w2": small_spec(W=2, interleave=2, qlen=5, seq_range=(60, 500)),
    "interleave5_w3_b16": small_spec(W=3, interleave=5, block_size=16, qlen=4,
                                     seq_range=(30, 400)),
    "e5m2_odd_block_p4": small_spec(W=3, block_size=12, kv_dtype="fp8_e5m2", qlen=2, H=8,
                                    seq_range=(40, 400)),
    "heads128_q8": small_spec(N=2, H=128, qlen=8, W=1, block_size=256, seq_range=(100, 300)),
    "heads12_q7_m84": small_spec(N=3, H=12, qlen=7, W=2, seq_range=(70, 260)),
    "ragged_q": dict(N=5, H=8, qlen_range=(1, 8), seq_range=(8, 200), block_size=32, W=3,
                     kv_dtype="bf16", nseg=1),
    "w_gt_s": dict(N=4, H=4, qlens=[1, 2, 3, 4], seq_lens=[1, 3, 5, 4],
                   block_size=16, W=8, kv_dtype="bf16", nseg=1),
    "q_equals_s": dict(N=2, H=16, qlens=[7, 1], seq_lens=[7, 1], block_size=16, W=2,
                       kv_dtype="bf16", nseg=2),
}


@pytest.mark.parametrize("name", sorted(SMALL))
@pytest.mark.parametrize("nseg", [1, 3])
def test_small_parity_all_stages(name, nseg):
    """Every stage against the oracle on inputs the oracle finishes in
    seconds: plan bit-exact, split-K partials, per-shard (out, lse), final."""
    spec = dict(SMALL[name])
    inp = wl.make_workload(spec, seed=1)
    say(f"case {name} nseg={nseg} S={inp['seq_lens'].tolist()} Q={inp['qlens'].tolist()}")
    got = run_gpu(inp, nseg=nseg, want_shards=True)
    ref = _check_plan(inp, got)
    so, sl, sa, parts = oracle_shard_results(inp, ref, nseg)
    assert np.all(np.isfinite(got["out"])) and not np.any(np.isnan(got["lse"]))
    check_out(got["shard_out"], so, inp["kv_dtype"], "shard_out", sa)
    assert max_err(got["shard_lse"], sl) <= TOL_LSE
    # split-K partials on active (row, segment) pairs (fp32: only the bf16
    # weights' bound can exceed the stated one)
    H, W, R = inp["H"], inp["W"], inp["R"]
    gm = got["segm_max"].reshape(W, R, H, nseg)
    ge = got["segm_expsum"].reshape(W, R, H, nseg)
    go = got["segm_out"].reshape(W, R, H, nseg, 512)
    for (i, r), (m2, e, Ov, act) in parts.items():
        O, Oa = Ov[..., :512], Ov[..., 512:]
        qs, Q = orc.request_rows(inp["q_start"], i)
        for t in range(Q):
            for s in np.nonzero(act[t])[0]:
                rho = qs + t
                assert max_err(gm[r, rho, :, s], m2[t, :, s]) <= 1e-3
                assert np.allclose(ge[r, rho, :, s], e[t, :, s], rtol=2e-3, atol=0)
                ref_o = O[t, :, s] / e[t, :, s, None]
                bound = np.maximum(TOL_OUT[inp["kv_dtype"]],
                                   U_BF16 * Oa[t, :, s] / e[t, :, s, None] + EPS_F32)
                assert np.all(np.abs(go[r, rho, :, s] / ge[r, rho, :, s, None] - ref_o) <= bound)
    out_ref, lse_ref = orc.verify_reference(inp)
    check_out(got["out"], out_ref, inp["kv_dtype"], "out", weighted_abs_v(inp))
    say(f"  lse: max|d|={max_err(got['lse'], lse_ref):.3e}")
    assert max_err(got["lse"], lse_ref) <= TOL_LSE


@pytest.mark.parametrize("W,B", [(1, 16), (2, 64), (3, 48), (5, 3), (8, 256), (16, 32)])
def test_plan_fuzz_bit_exact(W, B):
    for seed in range(3):
        spec = dict(N=7, H=1, qlen_range=(1, 9), seq_range=(9, 700), block_size=B, W=W,
                    kv_dtype="bf16", nseg=1)
        inp = wl.make_workload(spec, seed=seed)
        dev = wl.to_device(inp)
        p = mla.mla_verify_plan(dev["seq_lens"], dev["q_start"], dev["R"], W,
                                dev["block_table"], dev["num_blocks"], B,
                                dev["max_kv_seq_len"] + seed * 17)
        torch.cuda.synchronize()
        ref = orc.plan(inp["seq_lens"], inp["q_start"], W, inp["block_table"], B,
                       inp["max_kv_seq_len"] + seed * 17)
        assert int(p["err_flag"].item()) == 0
        assert np.array_equal(p["row_lens"].cpu().numpy(), ref["row_lens"])
        assert np.array_equal(p["page_table"].cpu().numpy(), ref["page_table"])


@pytest.mark.parametrize("W,B,I", [(2, 16, 2), (3, 48, 4), (4, 64, 3), (8, 16, 5), (2, 256, 64)])
def test_plan_interleave_bit_exact(W, B, I):
    """Row lengths and sub-page tables under interleave I against the oracle's
    brute-force ownership count."""
    for seed in range(3):
        spec = dict(N=7, H=1, qlen_range=(1, 9), seq_range=(9, 700), block_size=B, W=W,
                    interleave=I, kv_dtype="bf16", nseg=1)
        inp = wl.make_workload(spec, seed=seed)
        dev = wl.to_device(inp)
        p = mla.mla_verify_plan(dev["seq_lens"], dev["q_start"], dev["R"], W,
                                dev["block_table"], dev["num_blocks"], B,
                                dev["max_kv_seq_len"], interleave=I)
        torch.cuda.synchronize()
        ref = orc.plan(inp["seq_lens"], inp["q_start"], W, inp["block_table"], B,
                       inp["max_kv_seq_len"], I)
        assert int(p["err_flag"].item()) == 0
        assert np.array_equal(p["row_lens"].cpu().numpy(), ref["row_lens"])
        assert np.array_equal(p["page_table"].cpu().numpy(), ref["page_table"])


def _plan_raw(seq_lens, qlens, W, block_table, num_blocks, B, max_kv, R=None):
    q_start = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    t = lambda a: torch.tensor(np.asarray(a, dtype=np.int32), device="cuda")
    R = int(q_start[-1]) if R is None else R
    p = mla.mla_verify_plan(t(seq_lens), t(q_start), R, W, t(block_table), num_blocks, B, max_kv)
    torch.cuda.synchronize()
    return p


def test_plan_device_error_bits():
    bt = [[0, 1], [2, 3]]
    ok = _plan_raw([40, 30], [2, 3], 2, bt, 4, 16, 20)
    assert int(ok["err_flag"].item()) == 0
    bad_q = _plan_raw([40, 2], [2, 3], 2, bt, 4, 16, 20)          # S < Q
    assert int(bad_q["err_flag"].item()) & mla.MLA_PLAN_ERR_QLEN
    L = bad_q["row_lens"].cpu().numpy()
    assert np.all(L[:, 2:] == 0) and np.all(L[:, :2] > 0)
    assert np.all(bad_q["page_table"].cpu().numpy()[:, 2:] == -1)
    bound = _plan_raw([40, 30], [2, 3], 2, bt, 4, 16, 15)         # ceil(40/2) > 15
    assert int(bound["err_flag"].item()) & mla.MLA_PLAN_ERR_BOUND
    blk = _plan_raw([40, 30], [2, 3], 2, [[0, 9], [2, 3]], 4, 16, 20)  # id 9 >= 4
    assert int(blk["err_flag"].item()) & mla.MLA_PLAN_ERR_BLOCKS
    assert np.all(blk["row_lens"].cpu().numpy()[:, :2] == 0)
    few = _plan_raw([70, 30], [2, 3], 2, bt, 4, 16, 40)           # needs 3 blocks > 2
    assert int(few["err_flag"].item()) & mla.MLA_PLAN_ERR_BLOCKS
    rows = _plan_raw([40, 30], [2, 3], 2, bt, 4, 16, 20, R=4)     # q_start[N] != R
    assert int(rows["err_flag"].item()) & mla.MLA_PLAN_ERR_ROWS


def test_plan_error_flag_is_sticky():
    """Bits are ORed in and never cleared by the library: a valid call leaves
    an earlier error visible, and a zeroed flag stays zero over valid calls."""
    bt = [[0, 1], [2, 3]]
    t = lambda x: torch.tensor(x, dtype=torch.int32, device="cuda")
    flag = torch.zeros((1,), dtype=torch.int32, device="cuda")
    args = lambda S: (t(S), t([0, 2, 5]), 5, 2, t(bt), 4, 16, 20)
    mla.mla_verify_plan(*args([40, 30]), err_flag=flag)
    mla.mla_verify_plan(*args([40, 30]), err_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    mla.mla_verify_plan(*args([40, 2]), err_flag=flag)             # S < Q
    mla.mla_verify_plan(*args([40, 30]), err_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == mla.MLA_PLAN_ERR_QLEN


def test_zero_query_pins_every_window():
    """q = 0: every score is 0, so the final lse is ln(window) and each shard's
    lse is ln(its row length) -- one token too many or too few on any shard
    moves the lse by about 1/L, far beyond 1e-3 at these lengths."""
    spec = small_spec(N=6, W=4, qlen=5, seq_range=(5, 120), block_size=16, H=2)
    inp = wl.make_workload(spec, seed=4, q_mode="zero")
    got = run_gpu(inp, nseg=2, want_shards=True)
    ref = _check_plan(inp, got)
    for i in range(inp["N"]):
        qs, Q = orc.request_rows(inp["q_start"], i)
        for t in range(Q):
            w = inp["seq_lens"][i] - Q + 1 + t
            assert np.allclose(got["lse"][qs + t], math.log(w), atol=1e-4)
            for r in range(4):
                L = ref["row_lens"][r, qs + t]
                want = math.log(L) if L else -math.inf
                assert max_err(got["shard_lse"][r, qs + t], np.full(2, want)) <= 1e-4


def test_output_discriminates_off_by_one_window():
    """The GPU output is closer to the oracle with the pages' window than to
    the oracle with the window one position longer (the garbled snippet
    reading), on every row where those two oracles differ clearly."""
    spec = small_spec(N=6, W=2, qlen=4, seq_range=(10, 40), block_size=16, H=4)
    inp = wl.make_workload(spec, seed=2)
    got = run_gpu(inp)
    q = orc.decode_bf16(inp["q_bits"])
    checked = 0
    for i in range(inp["N"]):
        qs, Q = orc.request_rows(inp["q_start"], i)
        S = int(inp["seq_lens"][i])
        K = orc.gather_request_kv(inp["kv_bits"], "bf16", 1.0, inp["block_table"][i], S, 2, 16)
        good, _ = orc.attention_rows(q[qs:qs + Q], K, S, Q, inp["sm_scale"])
        for t in range(Q - 1):  # rows whose window can grow by one inside S
            w_bad = S - Q + 2 + t       # one position more than the pages' window
            bad, _ = orc.attention_rows(q[qs + t:qs + t + 1], K, w_bad, 1, inp["sm_scale"])
            if np.abs(good[t] - bad[0]).max() < 4 * TOL_OUT["bf16"]:
                continue
            checked += 1
            dg = np.abs(got["out"][qs + t] - good[t]).max()
            db = np.abs(got["out"][qs + t] - bad[0]).max()
            assert dg < db and dg <= TOL_OUT["bf16"]
    assert checked >= 6


def _window_oracle(q_row, K, w, sm_scale):
    """Oracle out [H, 512] and lse [H] of one row attending to positions [0, w)."""
    o, l = orc.attention_rows(q_row[None], K, w, 1, sm_scale)
    return o[0], l[0]


@pytest.mark.parametrize("name", ["tiny_decode", "tiny_decode_q4", "verify_dcp8"])
def test_every_row_discriminates_its_window(name):
    """On every row of the tiny-decode and verify workloads (and a qlen-4
    variant of the tiny one), the GPU result is closer to the oracle with the
    pages' window w = S - Q + 1 + t than to the oracle with w - 1 or w + 1
    (where w + 1 <= S), in L2 over all heads for both the LSE and the output:
    at these lengths max-abs 1e-2 alone cannot see a one-token window error."""
    spec = dict(wl.CONFIGS["tiny_decode"], qlen=4) if name == "tiny_decode_q4" else name
    inp = wl.make_workload(spec, 0)
    got = run_gpu(inp)
    q = orc.decode_bf16(inp["q_bits"])
    rows = 0
    for i in range(inp["N"]):
        qs, Q = orc.request_rows(inp["q_start"], i)
        S = int(inp["seq_lens"][i])
        K = orc.gather_request_kv(inp["kv_bits"], "bf16", 1.0, inp["block_table"][i], S,
                                  inp["W"], inp["block_size"])
        for t in range(Q):
            w = S - Q + 1 + t
            go, gl = _window_oracle(q[qs + t], K, w, inp["sm_scale"])
            dl = np.linalg.norm(got["lse"][qs + t] - gl)
            do = np.linalg.norm(got["out"][qs + t] - go)
            for wb in (w - 1, w + 1):
                if wb < 1 or wb > S:
                    continue
                bo, bl = _window_oracle(q[qs + t], K, wb, inp["sm_scale"])
                assert dl < np.linalg.norm(got["lse"][qs + t] - bl), (i, t, wb)
                assert do < np.linalg.norm(got["out"][qs + t] - bo), (i, t, wb)
            rows += 1
    say(f"{name}: {rows} rows, each closest to its own window")
    assert rows == inp["R"]


def _wrong_row_lens(inp, row_lens, kind):
    """The two wrong row views the pages reject, from the correct one:
    subtract-offset (each row = the last row's local length minus its offset
    from the last row) and committed-prefix-only (every row sees S - Q)."""
    bad = row_lens.copy()
    W = inp["W"]
    for i in range(inp["N"]):
        qs, Q = orc.request_rows(inp["q_start"], i)
        S = int(inp["seq_lens"][i])
        for t in range(Q):
            if kind == "subtract_offset":
                bad[:, qs + t] = np.maximum(row_lens[:, qs + Q - 1] - (Q - 1 - t), 0)
            else:
                bad[:, qs + t] = np.bincount(np.arange(S - Q) % W, minlength=W)[:W]
    return bad


@pytest.mark.parametrize("name", ["tiny_decode_q4", "verify_dcp8"])
@pytest.mark.parametrize("kind", ["subtract_offset", "prefix_only"])
def test_wrong_row_views_fail_the_bounds_on_the_gpu(kind, name):
    """Negative controls on the verify workload and on the tiny-decode one
    with four verify rows: the kernels run with a wrong row view (the
    correct table still covers every row) and their result must then fail
    the stated bounds against the oracle somewhere -- the parity checks
    above would catch either mistake."""
    if name == "tiny_decode_q4":
        inp = wl.make_workload(dict(wl.CONFIGS["tiny_decode"], qlen=4), 0)
    else:
        inp = named_workload(name)
    dev = wl.to_device(inp)
    plan = mla.mla_verify_plan(dev["seq_lens"], dev["q_start"], dev["R"], dev["W"],
                               dev["block_table"], dev["num_blocks"], dev["block_size"],
                               dev["max_kv_seq_len"])
    torch.cuda.synchronize()
    bad = _wrong_row_lens(inp, plan["row_lens"].cpu().numpy(), kind)
    if kind == "subtract_offset" and inp["W"] == 1:
        # one shard holds every dropped token, so the offset view is the
        # right one there: the pages' objection needs W > 1
        assert np.array_equal(bad, plan["row_lens"].cpu().numpy())
        return
    bad_dev = torch.from_numpy(bad.astype(np.int32)).to("cuda")
    parts = mla.mla_verify_attn(dev["q"], dev["kv"], bad_dev, plan["page_table"],
                                dev["q_start"], page_size=plan["page_size"],
                                max_qlen=dev["max_qlen"], nseg=1, sm_scale=dev["sm_scale"])
    out, lse, _, _ = mla.mla_lse_merge(*parts, bad_dev, dev["q_start"],
                                       page_size=plan["page_size"], H=inp["H"], nseg=1)
    torch.cuda.synchronize()
    out_ref, lse_ref = orc.verify_reference(inp)
    d = np.abs(out.float().cpu().numpy() - out_ref)
    dl = np.abs(lse.cpu().numpy() - lse_ref)
    n_out = int((d > TOL_OUT["bf16"]).sum())
    n_lse = int((dl > TOL_LSE).sum())
    say(f"{name} {kind}: {n_out}/{d.size} out elements over 1e-2 (max {d.max():.4f}), "
        f"{n_lse}/{dl.size} lse over 1e-3 (max {dl.max():.4f})")
    assert n_out > 0 and n_lse > 0


@pytest.mark.parametrize("fmt", ["fp8_e4m3", "fp8_e5m2"])
def test_fp8_every_finite_code_decodes(fmt):
    """Fill every used cache slot with codes cycling through all finite values
    of the format (254 e4m3fn codes, 248 e5m2 codes); the oracle decodes them
    from the bit definition."""
    spec = small_spec(N=2, W=2, kv_dtype=fmt, qlen=3, H=4, seq_range=(200, 300))
    inp = wl.make_workload(spec, seed=6)
    table = orc.e4m3fn_table() if fmt == "fp8_e4m3" else orc.e5m2_table()
    finite = np.array([c for c in range(256) if np.isfinite(table[c])], dtype=np.uint8)
    cache = inp["kv_bits"]
    used = cache != wl.E4M3_NAN                       # 0x7F is the canary of both formats
    cache[used] = np.resize(finite, int(used.sum()))
    inp["kv_scale"] = 1.0 / float(np.max(np.abs(table[finite])))
    got = run_gpu(inp)
    out_ref, lse_ref = orc.verify_reference(inp)
    check_out(got["out"], out_ref, fmt, "out", weighted_abs_v(inp))
    assert max_err(got["lse"], lse_ref) <= TOL_LSE


def test_side_stream_matches_default_stream():
    inp = wl.make_workload(small_spec(), seed=8)
    a = run_gpu(inp)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = run_gpu(inp, stream=s)
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["lse"], b["lse"])


# -------------------------------------------------------- named workloads ---

@pytest.mark.parametrize("name", wl.CONFIG_ORDER)
def test_named_workload_parity(name):
    """The five workloads at full size, every request: plan bit-exact; out /
    lse against the oracle; every output finite (cache slots outside any
    window hold NaN canaries)."""
    inp = named_workload(name)
    say(f"workload {name}: R={inp['R']} sum S={int(inp['seq_lens'].sum())}")
    got = run_gpu(inp)
    _check_plan(inp, got)
    assert np.all(np.isfinite(got["out"])) and np.all(np.isfinite(got["lse"]))
    eo, el = compare_requests(inp, got, list(range(inp["N"])), f"{name} out")
    say(f"workload {name}: all {inp['N']} requests max|dout|={eo:.3e} max|dlse|={el:.3e}")
    assert el <= TOL_LSE


# ------------------------------------------------- merge shapes and paths ---

MERGE_CASES = {
    # more than 511 request boundaries: the merge's request search narrows in
    # coarse rounds before its final one
    "many_requests": dict(N=600, H=2, qlen_range=(1, 2), seq_range=(2, 40), block_size=16,
                          W=2, kv_dtype="bf16", nseg=2),
    # 2 x 70 = 140 segments per pair: statistics past the 128 held in registers
    "segments_140": dict(N=2, H=2, qlen=3, seq_range=(2500, 3000), block_size=16, W=2,
                         kv_dtype="bf16", nseg=70),
    # 4 x 200 segments: too many for the LDS area, the sequential shard path
    "segments_800": dict(N=2, H=2, qlen=2, seq_range=(3000, 3600), block_size=16, W=4,
                         kv_dtype="bf16", nseg=200),
}


@pytest.mark.parametrize("name", list(MERGE_CASES))
def test_merge_paths(name):
    spec = MERGE_CASES[name]
    inp = wl.make_workload(spec, seed=11)
    say(f"merge case {name}: N={inp['N']} R={inp['R']} W={inp['W']} nseg={spec['nseg']}")
    got = run_gpu(inp, want_shards=True)
    ref = _check_plan(inp, got)
    so, sl, sa, _ = oracle_shard_results(inp, ref, spec["nseg"], want_parts=False)
    check_out(got["shard_out"], so, "bf16", "shard_out", sa)
    assert max_err(got["shard_lse"], sl) <= TOL_LSE
    out_ref, lse_ref = orc.verify_reference(inp)
    check_out(got["out"], out_ref, "bf16", "out", weighted_abs_v(inp))
    say(f"  lse: max|d|={max_err(got['lse'], lse_ref):.3e}")
    assert max_err(got["lse"], lse_ref) <= TOL_LSE


# ------------------------------------------------------ two-stage variant ---

@pytest.mark.parametrize("W,I", [(1, 1), (3, 1), (4, 2)])
def test_two_stage_verify_matches_one_stage_and_oracle(W, I):
    """The SGLang decomposition (sharded committed prefix + one-source dense
    causal window of the verify tokens, merged by LSE): the native two-stage
    plan bit for bit against the oracle's, then the result against the
    oracle's definition, its own two-stage decomposition, and the one-stage
    path. Request 0 has no committed token (S = Q)."""
    spec = dict(N=4, H=16, qlens=[5, 1, 3, 4], seq_lens=[5, 40, 233, 77], block_size=16, W=W,
                interleave=I, kv_dtype="bf16", nseg=1)
    inp = wl.make_workload(spec, seed=12, keep_logical=True)
    say(f"two-stage W={W} I={I}")
    dev = wl.to_device(inp)
    win = np.concatenate([inp["logical_kv_bits"][i][int(S) - int(Q):int(S)]
                          for i, (S, Q) in enumerate(zip(inp["seq_lens"], inp["qlens"]))])
    k_window = torch.from_numpy(win.view(np.int16)).view(torch.bfloat16).to("cuda")
    qmax = dev["max_qlen"] + 2          # a window table wider than the longest window
    plan = mla.mla_verify_two_stage_plan(dev["seq_lens"], dev["q_start"], dev["R"], W,
                                         dev["block_table"], dev["num_blocks"],
                                         dev["block_size"], dev["max_kv_seq_len"], qmax,
                                         interleave=I)
    dev2 = dict(dev, max_qlen=qmax)
    out2, lse2, flag = mla.mla_verify_two_stage(dev2, k_window, plan=plan)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    ref_plan = orc.two_stage_plan(inp["seq_lens"], inp["q_start"], W, inp["block_table"],
                                  inp["block_size"], inp["max_kv_seq_len"], qmax, I)
    assert np.array_equal(plan["row_lens"].cpu().numpy(), ref_plan["row_lens"])
    assert np.array_equal(plan["page_table"].cpu().numpy(), ref_plan["page_table"])
    assert np.array_equal(plan["window_table"].cpu().numpy(), ref_plan["window_table"])
    got_out = out2.float().cpu().numpy().astype(np.float64)
    got_lse = lse2.cpu().numpy().astype(np.float64)
    out_ref, lse_ref = orc.verify_reference(inp)
    absv = weighted_abs_v(inp)
    check_out(got_out, out_ref, "bf16", "two-stage out", absv)
    assert max_err(got_lse, lse_ref) <= TOL_LSE
    q = orc.decode_bf16(inp["q_bits"])
    for i in range(inp["N"]):
        qs, Q = orc.request_rows(inp["q_start"], i)
        K = orc.decode_bf16(inp["logical_kv_bits"][i])
        o, l = orc.two_stage_verify(q[qs:qs + Q], K, int(inp["seq_lens"][i]), Q, W,
                                    inp["sm_scale"])
        check_out(got_out[qs:qs + Q], o, "bf16", f"two-stage out, request {i}",
                  absv[qs:qs + Q])
        assert max_err(got_lse[qs:qs + Q], l) <= TOL_LSE
    one = run_gpu(inp)
    check_out(one["out"], out_ref, "bf16", "one-stage out", absv)
    assert max_err(got_lse, one["lse"]) <= TOL_LSE
    # the two-stage entry leaves the one-stage plan's checks in place: a
    # request longer than the window table is flagged, not read out of bounds
    bad = mla.mla_verify_two_stage_plan(dev["seq_lens"], dev["q_start"], dev["R"], W,
                                        dev["block_table"], dev["num_blocks"],
                                        dev["block_size"], dev["max_kv_seq_len"], 3,
                                        interleave=I)
    torch.cuda.synchronize()
    assert int(bad["err_flag"].item()) & mla.MLA_PLAN_ERR_QLEN
    L = bad["row_lens"].cpu().numpy()
    qs0, Q0 = orc.request_rows(inp["q_start"], 0)       # Q = 5 > 3
    assert np.all(L[:, qs0:qs0 + Q0] == 0)
    assert np.all(bad["window_table"].cpu().numpy()[qs0:qs0 + Q0] == -1)


# ------------------------------------------ one-segment (shard output) path ---

def _run_shards(inp, nseg=1, poison=True):
    """plan -> mla_verify_attn_shard -> mla_shard_merge, into buffers filled
    with NaN first, so that any element left unwritten fails."""
    dev = wl.to_device(inp)
    S, R, H = inp["W"] * nseg, inp["R"], inp["H"]
    fill = float("nan") if poison else 0.0
    so = torch.full((S, R, H, 512), fill, dtype=torch.bfloat16, device="cuda")
    sl = torch.full((S, R, H), fill, dtype=torch.float32, device="cuda")
    out = torch.full((R, H, 512), fill, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((R, H), fill, dtype=torch.float32, device="cuda")
    res = mla.mla_verify_forward_shards(dev, nseg=nseg, shards=(so, sl), out=out, lse=lse)
    torch.cuda.synchronize()
    return {k: res[k].cpu() for k in ("shard_out", "shard_lse", "out", "lse")}


def _oracle_sources(inp, plan, nseg):
    """The oracle's normalised (shard, segment) sources: output, LSE and
    weighted |v| of every source r * nseg + s (empty: 0, -inf, 0)."""
    W, R, H = inp["W"], inp["R"], inp["H"]
    _, _, _, parts = oracle_shard_results(inp, plan, nseg)
    so = np.zeros((W * nseg, R, H, 512))
    sa = np.zeros((W * nseg, R, H, 512))
    sl = np.full((W * nseg, R, H), -np.inf)
    for (i, r), (m2, e, Ov, act) in parts.items():
        qs, Q = orc.request_rows(inp["q_start"], i)
        for t in range(Q):
            for s_ in np.nonzero(act[t])[0]:
                src = r * nseg + s_
                so[src, qs + t] = Ov[t, :, s_, :512] / e[t, :, s_, None]
                sa[src, qs + t] = Ov[t, :, s_, 512:] / e[t, :, s_, None]
                sl[src, qs + t] = orc.LN2 * (m2[t, :, s_] + np.log2(e[t, :, s_]))
    return so, sl, sa


@pytest.mark.parametrize("nseg", [1, 3])
@pytest.mark.parametrize("name", sorted(SMALL))
def test_one_segment_path(name, nseg):
    """The normalised route (each (shard, segment) unit's output normalised
    and handed over as bf16 with its LSE, then one LSE merge over the W * nseg
    units) against the oracle's per-source and final results; its sources
    equal what the split route's merge makes of the same partials (nseg 1:
    bit for bit)."""
    spec = dict(SMALL[name])
    inp = wl.make_workload(spec, seed=1)
    say(f"normalised route case {name} nseg={nseg} S={inp['seq_lens'].tolist()} "
        f"Q={inp['qlens'].tolist()}")
    got = _run_shards(inp, nseg)
    ref_plan = oracle_plan(inp)
    so, sl, sa = _oracle_sources(inp, ref_plan, nseg)
    g_so = got["shard_out"].float().numpy().astype(np.float64)
    g_sl = got["shard_lse"].numpy().astype(np.float64)
    assert not np.any(np.isnan(g_so)) and not np.any(np.isnan(g_sl))
    check_out(g_so, so, inp["kv_dtype"], "sources", sa)
    assert max_err(g_sl, sl) <= TOL_LSE
    out_ref, lse_ref = orc.verify_reference(inp)
    g_out = got["out"].float().numpy().astype(np.float64)
    assert np.all(np.isfinite(g_out)) and not np.any(np.isnan(got["lse"].numpy()))
    check_out(g_out, out_ref, inp["kv_dtype"], "out (bf16 hand-off)", weighted_abs_v(inp),
              handoff=True)
    assert max_err(got["lse"].numpy(), lse_ref) <= TOL_LSE
    if nseg == 1:
        # the split route with one segment computes the same per-shard bits
        # (its merge then keeps them in fp32, so only its final output may differ)
        split = run_gpu(inp, nseg=1, want_shards=True)
        assert np.array_equal(g_so, split["shard_out"])
        assert np.array_equal(g_sl, split["shard_lse"])
        assert max_err(got["lse"].numpy(), split["lse"]) <= 1e-5


@pytest.mark.parametrize("name", wl.CONFIG_ORDER)
def test_one_segment_path_named_workload(name):
    """The normalised route on the five full-size workloads (their own segment
    counts), every request: out / lse against the oracle."""
    inp = named_workload(name)
    got = _run_shards(inp, inp["nseg"])
    g_out = got["out"].float().numpy().astype(np.float64)
    g_lse = got["lse"].numpy().astype(np.float64)
    assert np.all(np.isfinite(g_out)) and np.all(np.isfinite(g_lse))
    out_ref, lse_ref = orc.verify_reference(inp)
    eo, _ = check_out(g_out, out_ref, inp["kv_dtype"], f"{name} out (bf16 hand-off)",
                      weighted_abs_v(inp), handoff=True)
    el = max_err(g_lse, lse_ref)
    say(f"normalised route {name}: max|dout|={eo:.3e} max|dlse|={el:.3e}")
    assert el <= TOL_LSE


@pytest.mark.parametrize("W", [1, 5, 8, 12, 70])
def test_shard_merge_alone_matches_oracle_merge(W):
    """mla_shard_merge on given per-shard results (some shards empty: -inf)
    against the oracle's LSE merge of the same bf16 values, and an all-empty
    pair giving out 0, lse -inf (W <= 8 and the general path, which holds
    shards past 64 in a second pass)."""
    rng = np.random.default_rng(5 + W)
    R, H = 3, 4
    so = torch.tensor(rng.standard_normal((W, R, H, 512)), dtype=torch.bfloat16)
    sl = torch.tensor(rng.normal(3.0, 2.0, (W, R, H)), dtype=torch.float32)
    sl[min(1, W - 1), 0, :] = -float("inf")
    sl[:, 2, 3] = -float("inf")
    out, lse = mla.mla_shard_merge(so.cuda(), sl.cuda())
    torch.cuda.synchronize()
    o_ref, l_ref = orc.lse_merge(so.double().numpy(), sl.double().numpy())
    got_o = out.float().cpu().numpy()
    check_out(got_o, o_ref, "bf16", "shard merge out", np.zeros_like(o_ref))
    assert max_err(lse.cpu().numpy(), l_ref) <= 1e-5
    assert np.all(got_o[2, 3] == 0.0) and lse[2, 3].item() == -float("inf")


@pytest.mark.parametrize("case", ["many_subpages", "many_shard_rows"])
def test_plan_paths_past_the_lds_staging(case):
    """The plan kernel keeps a request's sub-page ids (up to 4096) and its
    (shard, row) lengths (up to 1024) in LDS; larger requests take the path
    that reads the block table per cell. Both paths against the oracle, bit
    for bit, in one batch with a small request that stays on the LDS path."""
    rng = np.random.default_rng(21)
    if case == "many_subpages":        # 70000 tokens in 16-token sub-pages: 4375 > 4096
        W, B, S, Q = 1, 16, [70000, 300], [3, 2]
    else:                              # 64 shards x 17 rows = 1088 > 1024
        W, B, S, Q = 64, 16, [5000, 900], [17, 1]
    local = [-(-s // W) for s in S]
    nblk = [-(-l // B) for l in local]
    max_blocks = max(nblk)
    num_blocks = sum(nblk) + 7
    ids = rng.permutation(num_blocks)
    bt = np.full((2, max_blocks), -1, dtype=np.int32)
    bt[0, :nblk[0]] = ids[:nblk[0]]
    bt[1, :nblk[1]] = ids[nblk[0]:nblk[0] + nblk[1]]
    max_kv = max(local)
    p = _plan_raw(S, Q, W, bt, num_blocks, B, max_kv)
    q_start = np.concatenate([[0], np.cumsum(Q)]).astype(np.int64)
    ref = orc.plan(np.asarray(S), q_start, W, bt, B, max_kv)
    assert int(p["err_flag"].item()) == 0
    assert np.array_equal(p["row_lens"].cpu().numpy(), ref["row_lens"])
    assert np.array_equal(p["page_table"].cpu().numpy(), ref["page_table"])


@pytest.mark.parametrize("route", ["split1", "split3", "shards"])
def test_understated_max_qlen_gives_nan_not_garbage(route):
    """max_qlen sizes the grid; a request with more verify rows than it covers
    must not leave unwritten or silently wrong outputs: its uncovered (row,
    head) pairs come out NaN, every covered pair still matches the oracle."""
    spec = dict(N=3, H=16, qlens=[2, 9, 3], seq_lens=[50, 300, 120], block_size=16, W=3,
                kv_dtype="bf16", nseg=1)
    inp = wl.make_workload(spec, seed=3)
    dev = dict(wl.to_device(inp), max_qlen=4)      # 4 * 16 = 64 pairs per request covered
    if route == "shards":
        res = mla.mla_verify_forward_shards(dev)
    else:
        res = mla.mla_verify_forward(dev, nseg=int(route[-1]))
    torch.cuda.synchronize()
    out = res["out"].float().cpu().numpy().astype(np.float64)
    lse = res["lse"].cpu().numpy().astype(np.float64)
    out_ref, lse_ref = orc.verify_reference(inp)
    pair_of_row = lambda rho, i: (rho - int(inp["q_start"][i])) * inp["H"]
    covered = np.zeros((inp["R"], inp["H"]), dtype=bool)
    for i in range(inp["N"]):
        qs, Q = orc.request_rows(inp["q_start"], i)
        for t in range(Q):
            for h in range(inp["H"]):
                covered[qs + t, h] = t * inp["H"] + h < 64
    assert (~covered).sum() == 5 * 16                  # rows 4..8 of request 1
    assert np.all(np.isnan(out[~covered])) and np.all(np.isnan(lse[~covered]))
    check_out(out[covered], out_ref[covered], "bf16", f"covered pairs ({route})",
              weighted_abs_v(inp)[covered])
    assert max_err(lse[covered], lse_ref[covered]) <= TOL_LSE


def test_empty_page_table_is_safe():
    """max_kv_seq_len = 0: the plan flags every request (its shard-0 length
    exceeds the bound) and gives it length 0; the table has width 0 (a null or
    empty buffer). Both routes then read no table entry and return out 0,
    lse -inf for every row, with no NaN."""
    inp = wl.make_workload(small_spec(N=3, W=4, qlen=3, seq_range=(20, 90), block_size=16),
                           seed=2)
    dev = wl.to_device(inp)
    dev["max_kv_seq_len"] = 0
    for route in ("split", "shards"):
        if route == "split":
            res = mla.mla_verify_forward(dev, nseg=1)
        else:
            res = mla.mla_verify_forward_shards(dev)
        torch.cuda.synchronize()
        assert res["plan"]["pt_width"] == 0
        assert int(res["plan"]["err_flag"].item()) & mla.MLA_PLAN_ERR_BOUND
        assert int(res["plan"]["row_lens"].abs().sum().item()) == 0
        out = res["out"].float().cpu()
        lse = res["lse"].cpu()
        assert torch.all(out == 0), route
        assert torch.all(torch.isneginf(lse)), route
