"""The entry point that allocates nothing (mla_verify_attn_merge_static,
partials in the library's static scratch array) against the entry point it
varies (mla_verify_attn_merge, partials in a caller workspace): bit for bit on
two calls in a row, the second smaller, so stale contents of the shared
array from the first call cannot leak into the second; and against the
oracle."""

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


def _both(inp, nseg):
    dev = wl.to_device(inp)
    plan = mla.mla_verify_plan(dev["seq_lens"], dev["q_start"], dev["R"], dev["W"],
                               dev["block_table"], dev["num_blocks"], dev["block_size"],
                               dev["max_kv_seq_len"])
    R, H = inp["R"], inp["H"]
    kw = dict(page_size=plan["page_size"], max_qlen=dev["max_qlen"], nseg=nseg,
              sm_scale=dev["sm_scale"], kv_scale=dev["kv_scale"])
    ws = torch.full((mla.mla_verify_workspace_bytes(inp["W"], R, H, nseg),), 0xFF,
                    dtype=torch.uint8, device="cuda")
    out_w, lse_w = mla.mla_verify_attn_merge(dev["q"], dev["kv"], plan["row_lens"],
                                             plan["page_table"], dev["q_start"], workspace=ws,
                                             **kw)
    out_s = torch.full((R, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse_s = torch.full((R, H), float("nan"), dtype=torch.float32, device="cuda")
    mla.mla_verify_attn_merge_static(dev["q"], dev["kv"], plan["row_lens"], plan["page_table"],
                                     dev["q_start"], out=out_s, lse=lse_s, **kw)
    torch.cuda.synchronize()
    assert int(plan["err_flag"].item()) == 0
    return out_w.cpu(), lse_w.cpu(), out_s.cpu(), lse_s.cpu()


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
def test_static_entry_matches_workspace_entry_twice(kv_dtype):
    big = wl.make_workload(dict(N=6, H=16, qlen=4, seq_range=(300, 1500), block_size=64, W=4,
                                kv_dtype=kv_dtype, nseg=3), seed=21)
    small = wl.make_workload(dict(N=2, H=8, qlen=2, seq_range=(20, 200), block_size=16, W=2,
                                  kv_dtype=kv_dtype, nseg=2), seed=22)
    for name, inp in (("first, larger", big), ("second, smaller", small)):
        say(f"static entry, {kv_dtype}, {name} call: R={inp['R']} H={inp['H']} "
            f"W={inp['W']} nseg={inp['nseg']}")
        out_w, lse_w, out_s, lse_s = _both(inp, inp["nseg"])
        assert torch.equal(out_s, out_w) and torch.equal(lse_s, lse_w)
        out_ref, lse_ref = orc.verify_reference(inp)
        check_out(out_s.float().numpy(), out_ref, kv_dtype, "static entry out",
                  weighted_abs_v(inp))
        assert max_err(lse_s.numpy(), lse_ref) <= TOL_LSE
