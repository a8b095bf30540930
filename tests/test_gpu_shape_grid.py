"""Parity sweep over the shape grid of the pages' fp8 routing test (vLLM PR
#51011 digest, its fp8 routing test): KV dtype {bf16, e4m3fn, e5m2} x heads
{1, 2, 4, 5, 6, 8, 12, 16, 32, 128} x verify length {1, 2, 4, 5, 8, 15}.
There the grid checks which kernel a shape is routed to; here every shape
runs on the one kernel family through all three routes -- split-K partials
and the segment merge (two segments), the normalised per-shard route, and
the persistent schedule -- and out / lse are compared with the oracle at
the stated bounds (tests/helpers.py). Small sequences (3 shards, 16-token
blocks) keep each case to a few milliseconds of oracle work; the row counts
Q*H run from 1 to 1920, so row blocks are full, partial and many.
"""

import numpy as np
import pytest

import oracle as orc
import workloads as wl
from helpers import TOL_LSE, check_out, max_err, say, weighted_abs_v

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)
mla = pytest.importorskip("mla_paged_decode_verify_amd")

KV_DTYPES = ["bf16", "fp8_e4m3", "fp8_e5m2"]
HEADS = [1, 2, 4, 5, 6, 8, 12, 16, 32, 128]
QLENS = [1, 2, 4, 5, 8, 15]


def _spec(kv, H, Q):
    return dict(N=2, H=H, qlen=Q, seq_range=(Q + 3, 180), block_size=16, W=3, kv_dtype=kv,
                nseg=2)


def _host(t):
    return t.float().cpu().numpy().astype(np.float64)


def _check(inp, name, out, lse, out_ref, lse_ref, absv, handoff):
    assert np.all(np.isfinite(out)) and not np.any(np.isnan(lse)), name
    eo, _ = check_out(out, out_ref, inp["kv_dtype"], name, absv, handoff=handoff)
    el = max_err(lse, lse_ref)
    assert el <= TOL_LSE, (name, el)
    return eo, el


@pytest.mark.parametrize("H", HEADS)
@pytest.mark.parametrize("kv", KV_DTYPES)
def test_shape_grid_all_routes(kv, H):
    worst = [0.0, 0.0]
    for Q in QLENS:
        inp = wl.make_workload(_spec(kv, H, Q), seed=7)
        tag = f"{kv} H={H} Q={Q}"
        say(f"grid case {tag} S={inp['seq_lens'].tolist()}")
        out_ref, lse_ref = orc.verify_reference(inp)
        absv = weighted_abs_v(inp)
        dev = wl.to_device(inp)
        # split-K partials (two segments) and the segment merge
        res = mla.mla_verify_forward(dev, nseg=2)
        torch.cuda.synchronize()
        r = _check(inp, f"{tag} split", _host(res["out"]), res["lse"].cpu().numpy(), out_ref,
                   lse_ref, absv, False)
        worst = [max(worst[0], r[0]), max(worst[1], r[1])]
        # normalised route: per-shard bf16 sources, then the shard merge
        res = mla.mla_verify_forward_shards(dev, nseg=1)
        torch.cuda.synchronize()
        r = _check(inp, f"{tag} shards", _host(res["out"]), res["lse"].cpu().numpy(), out_ref,
                   lse_ref, absv, True)
        worst = [max(worst[0], r[0]), max(worst[1], r[1])]
        # persistent schedule on 8 workgroups (groups cut between them)
        res = mla.mla_verify_forward_shards(dev, persistent=True, ctas=8)
        torch.cuda.synchronize()
        r = _check(inp, f"{tag} persistent", _host(res["out"]), res["lse"].cpu().numpy(),
                   out_ref, lse_ref, absv, True)
        worst = [max(worst[0], r[0]), max(worst[1], r[1])]
    say(f"grid {kv} H={H}: max|dout|={worst[0]:.3e} max|dlse|={worst[1]:.3e}")
