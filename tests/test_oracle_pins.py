"""Pins of the fp64 oracle against things other than itself.

Each test checks an oracle function against a hand-worked example from the
pages (tests/golden/), a closed form, an invariant the pages state, brute
force, or a library routine. CPU only.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle as orc
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line)
    return rows


def _closed_form_count(w, r, W):
    """The pages' count: floor((w-1-r)/W) + 1 when w-1-r >= 0, else 0
    (vLLM #51705 digest, _build_dcp_verify_row_view snippet comment)."""
    d = w - 1 - r
    return d // W + 1 if d >= 0 else 0


# ----------------------------------------------------------------- plan ----

def test_subpage_size_golden():
    for line in _read_golden("subpage_sizes.txt"):
        b, p = line.split()
        if p == "error":
            with pytest.raises(ValueError):
                orc.subpage_size(int(b))
        else:
            assert orc.subpage_size(int(b)) == int(p), b


def test_subpage_size_divides_and_is_power_of_two():
    for b in range(1, 2049):
        p = orc.subpage_size(b)
        assert b % p == 0 and p & (p - 1) == 0 and p <= 128
        # maximality: doubling either breaks divisibility or the 128 cap
        assert b % (2 * p) != 0 or p == 128


def test_row_view_golden_example():
    lines = _read_golden("row_view_S10_Q4_W4.txt")
    want = np.array([[int(x) for x in l.split(":")[1].split()]
                     for l in lines if l[0].isdigit()])
    L = orc.row_view([10], [0, 4], 4)          # [W, R]
    assert np.array_equal(L.T, want)
    sub = np.array([[int(x) for x in l.split(":")[1].split()]
                    for l in lines if l.startswith("subtract_offset")])
    pre = [int(x) for x in [l for l in lines if l.startswith("prefix_only")][0].split(":")[1].split()]
    # the negative controls differ from the correct view on some row
    assert not np.array_equal(sub, want)
    assert any(list(want[t]) != pre for t in range(4))


@pytest.mark.parametrize("W", [1, 2, 3, 4, 7, 8])
def test_row_view_brute_force_matches_closed_form(W):
    rng = np.random.default_rng(W)
    S = rng.integers(1, 200, size=12)
    Q = np.minimum(rng.integers(1, 9, size=12), S)
    qs = np.concatenate([[0], np.cumsum(Q)])
    L = orc.row_view(S, qs, W)
    for i in range(len(S)):
        for t in range(Q[i]):
            w = orc.window_length(S[i], Q[i], t)
            for r in range(W):
                assert L[r, qs[i] + t] == _closed_form_count(w, r, W)


def test_row_view_invariants():
    """Sum over shards = window (T2); per-row causality (T1); one shard grows
    by one between consecutive rows; W=1 and Q=1 special cases."""
    rng = np.random.default_rng(7)
    for W in (1, 2, 3, 4, 8):
        S = rng.integers(1, 120, size=20)
        Q = np.minimum(rng.integers(1, 9, size=20), S)
        qs = np.concatenate([[0], np.cumsum(Q)])
        L = orc.row_view(S, qs, W)
        for i in range(20):
            for t in range(Q[i]):
                rho = qs[i] + t
                w = S[i] - Q[i] + 1 + t
                assert L[:, rho].sum() == w
                last = S[i] - Q[i] + t          # last visible global position
                for r in range(W):
                    j = L[r, rho]
                    if j > 0:
                        assert (j - 1) * W + r <= last
                    assert j * W + r > last     # the next local token is not visible
                if t > 0:
                    d = L[:, rho] - L[:, rho - 1]
                    assert set(d.tolist()) <= {0, 1} and d.sum() == 1
                    assert d[(S[i] - Q[i] + t) % W] == 1
            if W == 1:
                assert np.array_equal(L[0, qs[i]:qs[i + 1]],
                                      [S[i] - Q[i] + 1 + t for t in range(Q[i])])
        # Q = 1: the single row sees the whole sequence
        L1 = orc.row_view(S, np.arange(21), W)
        assert np.array_equal(L1.sum(axis=0), S)


def test_window_length_edges():
    assert orc.window_length(10, 4, 0) == 7
    assert orc.window_length(10, 4, 3) == 10       # last row sees everything
    assert orc.window_length(5, 1, 0) == 5         # plain decode
    assert orc.window_length(4, 4, 0) == 1         # all tokens are verify tokens


def test_qo_indptr():
    assert np.array_equal(orc.qo_indptr(5), [0, 1, 2, 3, 4, 5])


def _small_workload(seed=0, W=3, B=16, kv="bf16", N=4, H=2, seq=(20, 90), qlen=3,
                    interleave=1, **kw):
    spec = dict(N=N, H=H, qlen=qlen, seq_range=seq, block_size=B, W=W,
                kv_dtype=kv, nseg=1, interleave=interleave)
    return wl.make_workload(spec, seed, keep_logical=True, **kw)


def _logical_f64(inp, i):
    bits = inp["logical_kv_bits"][i]
    if inp["kv_dtype"] == "bf16":
        t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
        return t.to(torch.float64).numpy()
    fmt = torch.float8_e4m3fn if inp["kv_dtype"] == "fp8_e4m3" else torch.float8_e5m2
    t = torch.from_numpy(bits).view(fmt)
    return t.to(torch.float64).numpy() * inp["kv_scale"]


@pytest.mark.parametrize("W,B", [(1, 16), (2, 48), (3, 16), (4, 96), (8, 256)])
def test_page_table_reads_back_each_shards_local_sequence(W, B):
    """Viewing the cache as pages of P tokens (the pages' reinterpretation of
    the cache shape) and following a row's sub-page table must yield exactly
    the first L tokens of that shard's local sequence (global positions
    r, r+W, ...), taken from the generator's own logical KV."""
    inp = _small_workload(seed=W, W=W, B=B, seq=(5, 300))
    P = orc.subpage_size(B)
    plan = orc.plan(inp["seq_lens"], inp["q_start"], W, inp["block_table"], B,
                    inp["max_kv_seq_len"])
    pt, L = plan["page_table"], plan["row_lens"]
    assert plan["page_size"] == P
    assert pt.shape[2] == -(-inp["max_kv_seq_len"] // P)
    pages = inp["kv_bits"].reshape(W, -1, P, wl.HEAD_DIM)
    for i in range(inp["N"]):
        logical = inp["logical_kv_bits"][i]
        for rho in range(inp["q_start"][i], inp["q_start"][i + 1]):
            for r in range(W):
                n = L[r, rho]
                npg = -(-n // P)
                assert np.all(pt[r, rho, npg:] == -1)
                assert np.all(pt[r, rho, :npg] >= 0)
                got = pages[r, pt[r, rho, :npg]].reshape(-1, wl.HEAD_DIM)[:n]
                assert np.array_equal(got, logical[r::W][:n])
        # rows of one request share prefixes of the last row's table
        last = inp["q_start"][i + 1] - 1
        for rho in range(inp["q_start"][i], last):
            for r in range(W):
                k = -(-L[r, rho] // P)
                assert np.array_equal(pt[r, rho, :k], pt[r, last, :k])


def test_page_table_too_narrow_raises():
    with pytest.raises(ValueError):
        orc.subpage_table(np.array([[40]]), np.array([[0, 1, 2]]), [0, 1], 16, 16, 2)


# -------------------------------------------------------- number formats ---

def test_e4m3fn_table_matches_torch_cast_and_known_values():
    ours = orc.e4m3fn_table()
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    ok = ~np.isnan(ours)
    assert np.array_equal(ours[ok], lib[ok])
    assert ours[0x7E] == 448.0 and ours[0xFE] == -448.0
    assert ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6
    assert ours[0x38] == 1.0 and ours[0x00] == 0.0
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])
    assert np.sum(np.isnan(ours)) == 2 and not np.any(np.isinf(ours))


def test_e5m2_table_matches_torch_cast_and_known_values():
    ours = orc.e5m2_table()
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e5m2).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    ok = ~np.isnan(ours)
    assert np.array_equal(ours[ok], lib[ok])
    assert ours[0x7B] == 57344.0 and ours[0xFB] == -57344.0
    assert ours[0x01] == 2.0 ** -16 and ours[0x04] == 2.0 ** -14
    assert ours[0x3C] == 1.0 and ours[0x00] == 0.0
    assert ours[0x7C] == np.inf and ours[0xFC] == -np.inf
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFD])
    assert np.sum(np.isnan(ours)) == 6 and np.sum(np.isinf(ours)) == 2


def test_bf16_decode_matches_torch():
    bits = np.random.default_rng(0).integers(0, 65536, 4096, dtype=np.uint32).astype(np.uint16)
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ours = orc.decode_bf16(bits)
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    ok = ~np.isnan(ours)
    assert np.array_equal(ours[ok], lib[ok])


@pytest.mark.parametrize("kv,I", [("bf16", 1), ("fp8_e4m3", 1), ("fp8_e5m2", 1), ("bf16", 3)])
def test_gather_matches_generator_logical_kv(kv, I):
    inp = _small_workload(seed=3, W=4, B=16, kv=kv, interleave=I)
    for i in range(inp["N"]):
        got = orc.gather_request_kv(inp["kv_bits"], kv, inp["kv_scale"],
                                    inp["block_table"][i], inp["seq_lens"][i],
                                    inp["W"], inp["block_size"], I)
        assert np.array_equal(got, _logical_f64(inp, i))
        assert np.all(np.isfinite(got))


# ------------------------------------------------------------ attention ---

def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("S,Q", [(1, 1), (9, 1), (37, 1), (12, 4), (40, 7), (8, 8)])
def test_attention_zero_query_closed_form(S, Q):
    """q = 0: every score is 0, so lse = ln w exactly and out is the mean of V
    over the window; with V[p, 0] = p that mean is (w - 1) / 2."""
    H = 3
    K = _rand((S, 576), 1)
    K[:, 0] = np.arange(S)
    out, lse = orc.attention_rows(np.zeros((Q, H, 576)), K, S, Q, 0.3)
    for t in range(Q):
        w = S - Q + 1 + t
        assert np.allclose(lse[t], math.log(w), rtol=0, atol=1e-13)
        assert np.allclose(out[t, :, 0], (w - 1) / 2, rtol=0, atol=1e-12)
        assert np.allclose(out[t], K[:w, :512].mean(axis=0), rtol=0, atol=1e-12)


def test_attention_equal_keys_closed_form():
    """All keys equal k0: scores are all c = scale*<q,k0>, so lse = c + ln w
    and out = V row of k0."""
    S, Q, H = 30, 4, 2
    k0 = _rand((576,), 2)
    K = np.tile(k0, (S, 1))
    q = _rand((Q, H, 576), 3)
    out, lse = orc.attention_rows(q, K, S, Q, 0.05)
    for t in range(Q):
        c = 0.05 * (q[t] @ k0)
        assert np.allclose(lse[t], c + math.log(S - Q + 1 + t), atol=1e-12)
        assert np.allclose(out[t], np.tile(k0[:512], (H, 1)), atol=1e-12)


@pytest.mark.parametrize("S,Q,scale", [(17, 1, 1 / 24), (64, 1, 0.2), (50, 5, 1 / 24), (9, 9, 0.3)])
def test_attention_matches_torch_sdpa(S, Q, scale):
    """Library pin: torch's scaled_dot_product_attention in float64 with an
    explicit bottom-right causal mask gives out; an extra always-visible
    'sink' key with score 0 and a one-hot value recovers the natural-log LSE
    as ln(1/o_sink - 1)."""
    H = 4
    q = _rand((Q, H, 576), 5)
    K = _rand((S, 576), 6)
    out, lse = orc.attention_rows(q, K, S, Q, scale)
    qt = torch.from_numpy(q).permute(1, 0, 2)            # [H, Q, 576]
    kt = torch.from_numpy(np.vstack([K, np.zeros((1, 576))]))[None]   # sink key = 0
    v = np.zeros((S + 1, 513))
    v[:S, :512] = K[:, :512]
    v[S, 512] = 1.0
    vt = torch.from_numpy(v)[None]
    mask = torch.zeros(Q, S + 1, dtype=torch.bool)
    for t in range(Q):
        mask[t, :S - Q + 1 + t] = True
    mask[:, S] = True
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt.expand(H, -1, -1), vt.expand(H, -1, -1), attn_mask=mask,
        scale=scale).permute(1, 0, 2).numpy()             # [Q, H, 513]
    sink = o[..., 512]
    lib_lse = np.log(1.0 / sink - 1.0)
    lib_out = o[..., :512] / (1.0 - sink)[..., None]
    assert np.allclose(lse, lib_lse, atol=1e-10, rtol=0)
    assert np.allclose(out, lib_out, atol=1e-10, rtol=0)


def test_attention_values_argument():
    """values = K[:, :512] is the default; values = |V| matches torch's SDPA
    with |V| as the value tensor (the weights are the same softmax)."""
    S, Q, H, scale = 40, 3, 4, 0.1
    q = _rand((Q, H, 576), 7)
    K = _rand((S, 576), 8)
    a = orc.attention_rows(q, K, S, Q, scale)
    b = orc.attention_rows(q, K, S, Q, scale, values=K[:, :512])
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    c, _ = orc.attention_rows(q, K, S, Q, scale, values=np.abs(K[:, :512]))
    mask = torch.zeros(Q, S, dtype=torch.bool)
    for t in range(Q):
        mask[t, :S - Q + 1 + t] = True
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2), torch.from_numpy(K)[None].expand(H, -1, -1),
        torch.from_numpy(np.abs(K[:, :512]))[None].expand(H, -1, -1), attn_mask=mask,
        scale=scale).permute(1, 0, 2).numpy()
    assert np.allclose(c, ref, atol=1e-12, rtol=0)
    assert np.all(c >= np.abs(a[0]) - 1e-12)          # triangle inequality
    L = [S // 2, S // 3, 0]
    d, l = orc.shard_attention_rows(q, K, L, scale, values=np.abs(K[:, :512]))
    assert np.all(d[2] == 0) and np.all(np.isneginf(l[2]))
    e, _ = orc.attention_rows(q[:1], K, L[0], 1, scale, values=np.abs(K[:, :512]))
    assert np.allclose(d[0], e[0], atol=1e-12)


@pytest.mark.parametrize("n", [2, 3, 7, 64, 4000])
def test_bf16_weight_rounding_bound(n):
    """The bound the GPU parity tests use for the bf16 softmax weights fed to
    the matrix cores: rounding every weight p_j to bf16 (nearest even) moves
    sum_j p_j v_j / sum_j p_j by at most 2^-8 sum_j w_j |v_j|, w = p / sum p
    (each |bf16(p) - p| <= 2^-8 p). Checked on random logits and values, with
    the weights rounded by torch's own bf16 conversion."""
    rng = np.random.default_rng(n)
    worst = 0.0
    for trial in range(50):
        x = rng.normal(0.0, 1.5, n)
        p = np.exp2(x - x.max() + rng.uniform(0, 8))       # the lazy reference: p up to 2^8
        v = rng.normal(0.0, 1.0, (n, 64)) * rng.choice([1.0, 4.0], (n, 1))
        ph = torch.from_numpy(p).to(torch.bfloat16).double().numpy()
        err = np.abs((ph - p) @ v) / p.sum()
        bound = 2.0 ** -8 * ((p / p.sum()) @ np.abs(v))
        assert np.all(err <= bound * (1 + 1e-12))
        worst = max(worst, float(np.max(err / bound)))
    assert worst > 0.05        # the bound is not vacuous for short windows


@pytest.mark.parametrize("W,I", [(1, 1), (2, 1), (3, 1), (4, 1), (8, 1), (2, 2), (3, 4), (4, 3)])
def test_sharded_then_merged_equals_unsharded(W, I):
    """P5: per-shard rank-local attention over the row view, merged by
    natural-log LSE, reproduces the unsharded definition (also with runs of
    I > 1 positions per shard)."""
    rng = np.random.default_rng(W + 10 * I)
    for S, Q in [(1, 1), (5, 3), (29, 4), (70, 7)]:
        H = 2
        q = rng.standard_normal((Q, H, 576))
        K = rng.standard_normal((S, 576))
        out, lse = orc.attention_rows(q, K, S, Q, 0.1)
        L = orc.row_view([S], [0, Q], W, I)
        outs, lses = [], []
        for r in range(W):
            o, l = orc.shard_attention_rows(q, orc.shard_local_kv(K, W, r, I), L[r], 0.1)
            outs.append(o)
            lses.append(l)
            for t in range(Q):
                assert (L[r, t] == 0) == np.all(np.isneginf(l[t]))
        mo, ml = orc.lse_merge(np.stack(outs), np.stack(lses))
        assert np.allclose(mo, out, atol=1e-12, rtol=0)
        assert np.allclose(ml, lse, atol=1e-12, rtol=0)


@pytest.mark.parametrize("W,I", [(2, 2), (3, 2), (4, 3), (3, 5), (8, 4)])
def test_interleaved_row_view_invariants(W, I):
    """Runs of I consecutive positions dealt to the W shards in turn: every
    window is split without loss (sum over shards = w), each shard's part is
    a prefix of its local sequence (its first L positions are < w, the next
    one is not), local indices number each shard's positions 0, 1, 2, ... in
    increasing order, and I = 1 gives the round-robin closed form."""
    rng = np.random.default_rng(7 * W + I)
    for _ in range(10):
        S = int(rng.integers(1, 120))
        Q = int(rng.integers(1, min(S, 8) + 1))
        L = orc.row_view([S], [0, Q], W, I)
        pos = np.arange(S)
        owner = orc.shard_of(pos, W, I)
        loc = orc.local_index(pos, W, I)
        for r in range(W):
            mine = pos[owner == r]                  # increasing global positions
            assert np.array_equal(loc[owner == r], np.arange(len(mine)))
            for t in range(Q):
                w = S - Q + 1 + t
                n = int(L[r, t])
                assert np.all(mine[:n] < w) and (n == len(mine) or mine[n] >= w)
        for t in range(Q):
            assert L[:, t].sum() == S - Q + 1 + t
    # I >= every window: shard 0 holds all of it
    L = orc.row_view([7], [0, 3], W, 7)
    assert np.array_equal(L[0], [5, 6, 7]) and not np.any(L[1:])
    # I = 1 is the round-robin count
    L = orc.row_view([23], [0, 5], W, 1)
    for r in range(W):
        for t in range(5):
            w = 23 - 5 + 1 + t
            assert L[r, t] == ((w - 1 - r) // W + 1 if w - 1 - r >= 0 else 0)


def test_two_stage_decomposition_equals_row_view():
    """P8: the SGLang split (sharded committed prefix + dense verify window on
    shard 0, merged) equals the per-row view result."""
    rng = np.random.default_rng(11)
    for S, Q, W in [(20, 4, 4), (33, 7, 8), (7, 7, 2), (50, 1, 3)]:
        q = rng.standard_normal((Q, 3, 576))
        K = rng.standard_normal((S, 576))
        a = orc.attention_rows(q, K, S, Q, 0.07)
        b = orc.two_stage_verify(q, K, S, Q, W, 0.07)
        assert np.allclose(a[0], b[0], atol=1e-12) and np.allclose(a[1], b[1], atol=1e-12)


@pytest.mark.parametrize("W,I", [(1, 1), (4, 1), (3, 2), (8, 1)])
def test_two_stage_plan_splits_every_window(W, I):
    """The two-stage plan's stage-1 lengths are the committed prefix on each
    shard (they sum to S - Q, the same for every row of a request, and are a
    prefix of each shard's local sequence: each equals the one-stage length of
    a window of S - Q, computed by the closed form for I = 1), and stage 1 plus
    stage 2 is exactly the one-stage window w = S - Q + 1 + t of every row.
    The window table lists verify tokens q_start[i] .. q_start[i] + t."""
    rng = np.random.default_rng(3 + W)
    qlens = rng.integers(1, 8, size=6)
    seq = qlens + rng.integers(0, 300, size=6)
    seq[0] = qlens[0]                                   # empty committed prefix
    q_start = np.concatenate([[0], np.cumsum(qlens)])
    local = (seq // (I * W)) * I + np.minimum(seq % (I * W), I)
    B = 16
    nb = -(-local // B)
    bt = np.full((6, int(nb.max())), -1)
    perm = rng.permutation(int(nb.sum()) + 3)
    off = 0
    for i in range(6):
        bt[i, :nb[i]] = perm[off:off + nb[i]]
        off += int(nb[i])
    qmax = int(qlens.max()) + 1
    tp = orc.two_stage_plan(seq, q_start, W, bt, B, int(local.max()), qmax, I)
    one = orc.row_view(seq, q_start, W, I)
    L = tp["row_lens"]
    for i in range(6):
        qs, Q = orc.request_rows(q_start, i)
        for t in range(Q):
            rho = qs + t
            assert L[:W, rho].sum() == seq[i] - Q
            assert np.array_equal(L[:W, rho], L[:W, qs])
            assert L[W, rho] == t + 1
            assert L[:W, rho].sum() + L[W, rho] == one[:, rho].sum() == seq[i] - Q + 1 + t
            assert np.all(L[:W, rho] <= one[:, rho])
            if I == 1:
                assert all(L[r, rho] == _closed_form_count(seq[i] - Q, r, W) for r in range(W))
            assert list(tp["window_table"][rho]) == [qs + k if k <= t else -1
                                                     for k in range(qmax)]
    # stage-1 tables are the one-stage tables of the committed prefix
    ref = orc.subpage_table(L[:W], bt, q_start, B, B, tp["pt_width"])
    assert np.array_equal(tp["page_table"], ref)


# -------------------------------------------------------------- segments ---

@pytest.mark.parametrize("nseg,P", [(1, 16), (2, 16), (3, 4), (16, 4), (16, 1), (5, 128)])
def test_segments_merge_to_shard_result(nseg, P):
    """P6: the merged split-K partials equal rank-local attention whatever
    the number of segments and the tile size."""
    rng = np.random.default_rng(nseg * 131 + P)
    Q, H = 4, 3
    Lrows = [97, 98, 98, 100]
    q = rng.standard_normal((Q, H, 576))
    K = rng.standard_normal((100, 576))
    ref_o, ref_l = orc.shard_attention_rows(q, K, Lrows, 0.06)
    m2, e, O, act = orc.segment_partials(q, K, Lrows, nseg, P, 0.06)
    o, l = orc.segment_merge(m2, e, O, act[:, None, :])
    assert np.allclose(o, ref_o, atol=1e-12) and np.allclose(l, ref_l, atol=1e-12)
    # the tiles-per-segment partition: T = ceil(Lg / (nseg * P))
    T = -(-100 // (nseg * P))
    for t in range(Q):
        assert act[t].sum() == -(-Lrows[t] // (T * P))
        assert np.all(np.isneginf(m2[t][:, ~act[t]])) and np.all(O[t][:, ~act[t]] == 0)


def test_segments_have_inactive_tail():
    """Lg=100, P=4, 16 segments: T=2, span 8, so segments 13..15 are empty
    (like 132000-token rows over 8 shards with P=128 and 16 segments, where
    T=9 leaves the 16th segment empty)."""
    _, _, _, act = orc.segment_partials(np.zeros((1, 1, 576)), np.zeros((100, 576)),
                                        [100], 16, 4, 1.0)
    assert act[0].tolist() == [True] * 13 + [False] * 3
    assert -(-16500 // (16 * 128)) == 9 and 15 * 9 * 128 >= 16500


def test_single_segment_merge_is_normalisation():
    m2 = np.array([[1.5]])
    e = np.array([[3.0]])
    O = np.full((1, 1, 512), 6.0)
    o, l = orc.segment_merge(m2, e, O, np.array([[True]]))
    assert np.allclose(o, 2.0) and np.isclose(l[0], math.log(2) * (1.5 + math.log2(3.0)))


def test_segment_merge_all_inactive_is_empty_not_nan():
    o, l = orc.segment_merge(np.full((2, 3), -np.inf), np.zeros((2, 3)),
                             np.zeros((2, 3, 512)), np.zeros((2, 3), bool))
    assert np.all(o == 0) and np.all(np.isneginf(l))


# ---------------------------------------------------------------- merges ---

def test_lse_merge_identities():
    """P7: an empty (-inf) state is the identity; two halves of a window
    merge to the whole window; an all-empty merge is (0, -inf), never NaN."""
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 2, 576))
    K = rng.standard_normal((40, 576))
    whole = orc.shard_attention_rows(q, K, [40], 0.1)
    a = orc.shard_attention_rows(q, K[:17], [17], 0.1)
    b = orc.shard_attention_rows(q, K[17:], [23], 0.1)
    m = orc.lse_merge(np.stack([a[0], b[0]]), np.stack([a[1], b[1]]))
    assert np.allclose(m[0], whole[0], atol=1e-12) and np.allclose(m[1], whole[1], atol=1e-12)
    empty_o, empty_l = np.zeros_like(a[0]), np.full_like(a[1], -np.inf)
    m1 = orc.lse_merge(np.stack([a[0], empty_o]), np.stack([a[1], empty_l]))
    assert np.allclose(m1[0], a[0], atol=1e-15) and np.allclose(m1[1], a[1], atol=1e-15)
    m0 = orc.lse_merge(np.stack([empty_o, empty_o]), np.stack([empty_l, empty_l]))
    assert np.all(m0[0] == 0) and np.all(np.isneginf(m0[1]))


def test_base2_lse_in_natural_merge_is_wrong():
    """P7: feeding base-2 LSEs to the natural-log merge drifts by far more
    than the output tolerance (SGLang #34432 review item 4)."""
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 4, 576))
    K = rng.standard_normal((60, 576))
    whole = orc.shard_attention_rows(q, K, [60], 0.2)
    a = orc.shard_attention_rows(q, K[:10], [10], 0.2)
    b = orc.shard_attention_rows(q, K[10:], [50], 0.2)
    bad = orc.lse_merge(np.stack([a[0], b[0]]), np.stack([a[1] / math.log(2), b[1] / math.log(2)]))
    assert np.max(np.abs(bad[0] - whole[0])) > 1e-2


# ------------------------------------------------------ negative controls ---

def _wrong_row_lens(S, Q, W, kind):
    """Row lengths by the two wrong methods the pages reject."""
    full = orc.row_view([S], [0, 1], W)[:, 0]
    if kind == "subtract_offset":
        return np.stack([np.maximum(full - (Q - 1 - t), 0) for t in range(Q)], axis=1)
    # committed prefix only: positions [0, S-Q)
    committed = np.array([_closed_form_count(S - Q, r, W) for r in range(W)])
    return np.stack([committed] * Q, axis=1)


@pytest.mark.parametrize("kind", ["subtract_offset", "prefix_only"])
def test_negative_controls_fail_tolerance(kind):
    """P10: both wrong row views give outputs outside the bf16 tolerance."""
    inp = _small_workload(seed=5, W=4, B=16, N=6, H=4, seq=(30, 80), qlen=4)
    q = orc.decode_bf16(inp["q_bits"])
    worst = 0.0
    for i in range(inp["N"]):
        S = int(inp["seq_lens"][i])
        qs, Q = orc.request_rows(inp["q_start"], i)
        K = _logical_f64(inp, i)
        good, _ = orc.attention_rows(q[qs:qs + Q], K, S, Q, inp["sm_scale"])
        L = _wrong_row_lens(S, Q, 4, kind)
        outs, lses = [], []
        for r in range(4):
            o, l = orc.shard_attention_rows(q[qs:qs + Q], orc.shard_local_kv(K, 4, r), L[r], inp["sm_scale"])
            outs.append(o)
            lses.append(l)
        bad, _ = orc.lse_merge(np.stack(outs), np.stack(lses))
        worst = max(worst, float(np.max(np.abs(bad - good))))
    assert worst > 1e-2


def _bench_control(inp, kind):
    """Max-abs out / lse errors and the count of out elements over 1e-2 of a
    wrong row view over the whole workload, against the correct result."""
    q = orc.decode_bf16(inp["q_bits"])
    W = inp["W"]
    wo, wl_, over = 0.0, 0.0, 0
    for i in range(inp["N"]):
        S = int(inp["seq_lens"][i])
        qs, Q = orc.request_rows(inp["q_start"], i)
        K = orc.gather_request_kv(inp["kv_bits"], "bf16", 1.0, inp["block_table"][i], S, W,
                                  inp["block_size"])
        good, gl = orc.attention_rows(q[qs:qs + Q], K, S, Q, inp["sm_scale"])
        L = _wrong_row_lens(S, Q, W, kind)
        outs, lses = [], []
        for r in range(W):
            o, l = orc.shard_attention_rows(q[qs:qs + Q], orc.shard_local_kv(K, W, r), L[r],
                                            inp["sm_scale"])
            outs.append(o)
            lses.append(l)
        bad, bl = orc.lse_merge(np.stack(outs), np.stack(lses))
        d = np.abs(bad - good)
        wo = max(wo, float(d.max()))
        wl_ = max(wl_, float(np.abs(bl - gl).max()))
        over += int((d > 1e-2).sum())
    return wo, wl_, over


@pytest.mark.parametrize("name", ["tiny_decode_q4", "verify_dcp8"])
def test_negative_controls_on_benchmark_shapes(name):
    """P10 at the benchmark shapes: on the verify workload both wrong row views
    exceed the stated bounds on out (1e-2) and lse (1e-3); on the tiny
    decode shape with qlen 4 the committed-prefix-only view does, while
    subtract-offset coincides with the correct view there (one shard: the last
    row's length minus the offset is exactly each row's window)."""
    spec = dict(wl.CONFIGS["tiny_decode"], qlen=4) if name == "tiny_decode_q4" else name
    inp = wl.make_workload(spec, 0)
    for kind in ("subtract_offset", "prefix_only"):
        wo, wl_, over = _bench_control(inp, kind)
        n = inp["R"] * inp["H"] * 512
        print(f"{name} {kind}: max|dout|={wo:.4f} ({over}/{n} over 1e-2) max|dlse|={wl_:.4f}")
        if name == "tiny_decode_q4" and kind == "subtract_offset":
            assert wo == 0.0 and wl_ == 0.0
        else:
            assert wo > 1e-2 and wl_ > 1e-3 and over > 0


def test_verify_reference_matches_row_view_pipeline():
    """The full reference (logical KV read from the cache) equals plan ->
    per-shard segments -> segment merge -> LSE merge on the same cache."""
    inp = _small_workload(seed=9, W=3, B=16, N=3, H=2, seq=(20, 70), qlen=3)
    out, lse = orc.verify_reference(inp)
    plan = orc.plan(inp["seq_lens"], inp["q_start"], 3, inp["block_table"], 16,
                    inp["max_kv_seq_len"])
    q = orc.decode_bf16(inp["q_bits"])
    P = plan["page_size"]
    pages = orc.decode_bf16(inp["kv_bits"]).reshape(3, -1, P, 576)
    for i in range(inp["N"]):
        qs, Q = orc.request_rows(inp["q_start"], i)
        outs, lses = [], []
        for r in range(3):
            Lr = plan["row_lens"][r, qs:qs + Q]
            last = plan["page_table"][r, qs + Q - 1]
            local = pages[r, last[last >= 0]].reshape(-1, 576)
            m2, e, O, act = orc.segment_partials(q[qs:qs + Q], local, Lr, 3, P, inp["sm_scale"])
            o, l = orc.segment_merge(m2, e, O, act[:, None, :])
            outs.append(o)
            lses.append(l)
        mo, ml = orc.lse_merge(np.stack(outs), np.stack(lses))
        assert np.allclose(mo, out[qs:qs + Q], atol=1e-12)
        assert np.allclose(ml, lse[qs:qs + Q], atol=1e-12)
