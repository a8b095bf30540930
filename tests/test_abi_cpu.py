"""CPU checks of the C ABI: the library loads, exports what include/mla_verify.h
declares, and host-side validation rejects bad arguments before launching
anything (so these run without a GPU)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_verify.h")

mla = pytest.importorskip("mla_paged_decode_verify_amd")
from mla_paged_decode_verify_amd import _lib  # noqa: E402

FAKE = 4096  # a non-null pointer value that validation rejects before use


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_\w+)\s*\(", text)))


def test_header_declares_the_abi():
    names = _declared_functions()
    assert names == sorted(["mla_subpage_size", "mla_pt_width", "mla_verify_workspace_bytes",
                            "mla_verify_plan", "mla_verify_two_stage_plan", "mla_verify_attn",
                            "mla_lse_merge", "mla_verify_attn_shard", "mla_shard_merge",
                            "mla_verify_attn_merge", "mla_verify_attn_merge_static",
                            "mla_verify_attn_persistent",
                            "mla_verify_attn_persistent_workspace_bytes", "mla_last_error"])


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert set(_lib.EXPORTED) == set(_declared_functions())


def test_subpage_size_matches_golden_table():
    path = os.path.join(ROOT, "tests", "golden", "subpage_sizes.txt")
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        b, p = line.split()
        want = -1 if p == "error" else int(p)
        assert mla.mla_subpage_size(int(b)) == want, b


def test_pt_width_and_workspace():
    assert mla.mla_pt_width(16500, 128) == 129
    assert mla.mla_pt_width(0, 64) == 0
    assert mla.mla_pt_width(10, 0) == -1
    assert mla.mla_verify_workspace_bytes(8, 128, 16, 1) == 8 * 128 * 16 * 514 * 4
    assert mla.mla_verify_workspace_bytes(0, 1, 1, 1) == 0


def _plan(**over):
    a = dict(N=1, seq_lens=FAKE, q_start=FAKE, R=4, W=2, interleave=1, block_table=FAKE,
             max_blocks=4, num_blocks=8, block_size=64, page_size=64, max_kv_seq_len=100,
             pt_width=2, row_lens=FAKE, page_table=FAKE, qo_indptr=None, err_flag=None,
             stream=None)
    a.update(over)
    return _lib.lib.mla_verify_plan(*a.values())


@pytest.mark.parametrize("over,code,msg", [
    (dict(interleave=0), _lib.MLA_ERR_INVALID, "interleave"),
    (dict(interleave=1 << 29, W=4), _lib.MLA_ERR_INVALID, "interleave"),
    (dict(block_size=0, page_size=1), _lib.MLA_ERR_INVALID, "block_size"),
    (dict(page_size=32), _lib.MLA_ERR_INVALID, "page_size"),
    (dict(pt_width=1), _lib.MLA_ERR_INVALID, "pt_width"),
    (dict(N=0), _lib.MLA_ERR_INVALID, "N"),
    (dict(W=0), _lib.MLA_ERR_INVALID, "W"),
    (dict(max_blocks=0), _lib.MLA_ERR_INVALID, "max_blocks"),
    (dict(row_lens=None), _lib.MLA_ERR_INVALID, "null"),
])
def test_plan_rejects_bad_arguments(over, code, msg):
    assert _plan(**over) == code
    assert msg in mla.mla_last_error()


def _two_stage_plan(**over):
    a = dict(N=1, seq_lens=FAKE, q_start=FAKE, R=4, W=2, interleave=1, block_table=FAKE,
             max_blocks=4, num_blocks=8, block_size=64, page_size=64, max_kv_seq_len=100,
             pt_width=2, max_qlen=4, row_lens=FAKE, page_table=FAKE, window_table=FAKE,
             err_flag=None, stream=None)
    a.update(over)
    return _lib.lib.mla_verify_two_stage_plan(*a.values())


@pytest.mark.parametrize("over,msg", [
    (dict(interleave=0), "interleave"),
    (dict(page_size=32), "page_size"),
    (dict(pt_width=1), "pt_width"),
    (dict(N=0), "N"),
    (dict(max_qlen=0), "max_qlen"),
    (dict(window_table=None), "null"),
    (dict(row_lens=None), "null"),
])
def test_two_stage_plan_rejects_bad_arguments(over, msg):
    assert _two_stage_plan(**over) == _lib.MLA_ERR_INVALID
    err = mla.mla_last_error()
    assert msg in err and "mla_verify_two_stage_plan" in err


def _attn(**over):
    a = dict(q=FAKE, kv=FAKE, num_blocks=8, block_size=16, page_size=16, kv_dtype=0,
             kv_scale=1.0, sm_scale=0.04, row_lens=FAKE, page_table=FAKE, pt_width=4,
             q_start=FAKE, N=1, R=1, H=16, W=1, max_qlen=1, nseg=1, segm_out=FAKE,
             segm_max=FAKE, segm_expsum=FAKE, stream=None)
    a.update(over)
    return _lib.lib.mla_verify_attn(*a.values())


@pytest.mark.parametrize("over,code", [
    (dict(nseg=0), _lib.MLA_ERR_INVALID),
    (dict(H=0), _lib.MLA_ERR_INVALID),
    (dict(page_size=8), _lib.MLA_ERR_INVALID),
    (dict(kv_dtype=7), _lib.MLA_ERR_UNSUPPORTED),
    (dict(sm_scale=float("nan")), _lib.MLA_ERR_INVALID),
    (dict(kv_dtype=1, kv_scale=float("inf")), _lib.MLA_ERR_INVALID),
    (dict(sm_scale=0.0), _lib.MLA_ERR_INVALID),
    (dict(sm_scale=-0.04), _lib.MLA_ERR_INVALID),
    (dict(kv_dtype=1, kv_scale=-1.0), _lib.MLA_ERR_INVALID),
    (dict(kv_dtype=1, kv_scale=1e-40, sm_scale=1e-10), _lib.MLA_ERR_INVALID),
    (dict(q=None), _lib.MLA_ERR_INVALID),
    (dict(q=FAKE + 2), _lib.MLA_ERR_INVALID),
    (dict(max_qlen=0), _lib.MLA_ERR_INVALID),
])
def test_attn_rejects_bad_arguments(over, code):
    assert _attn(**over) == code
    assert mla.mla_last_error() != ""


def _merge(**over):
    a = dict(segm_out=FAKE, segm_max=FAKE, segm_expsum=FAKE, row_lens=FAKE, q_start=FAKE,
             N=1, page_size=16, R=1, H=1, W=1, nseg=1, shard_out=None, shard_lse=None,
             out=FAKE, lse=FAKE, stream=None)
    a.update(over)
    return _lib.lib.mla_lse_merge(*a.values())


@pytest.mark.parametrize("over", [dict(nseg=0), dict(page_size=48), dict(page_size=256),
                                  dict(out=None), dict(R=0), dict(shard_out=FAKE + 4)])
def test_merge_rejects_bad_arguments(over):
    assert _merge(**over) == _lib.MLA_ERR_INVALID


def test_python_binding_refuses_host_tensors():
    import torch
    with pytest.raises(TypeError):
        mla.mla_verify_plan(torch.zeros(1, dtype=torch.int32), torch.zeros(2, dtype=torch.int32),
                            1, 1, torch.zeros(1, 1, dtype=torch.int32), 1, 16, 16)


def _attn_shard(**over):
    a = dict(q=FAKE, kv=FAKE, num_blocks=8, block_size=16, page_size=16, kv_dtype=0,
             kv_scale=1.0, sm_scale=0.04, row_lens=FAKE, page_table=FAKE, pt_width=4,
             q_start=FAKE, N=1, R=1, H=16, W=1, max_qlen=1, nseg=1, shard_out=FAKE,
             shard_lse=FAKE, stream=None)
    a.update(over)
    return _lib.lib.mla_verify_attn_shard(*a.values())


@pytest.mark.parametrize("over,code", [
    (dict(H=0), _lib.MLA_ERR_INVALID),
    (dict(page_size=8), _lib.MLA_ERR_INVALID),
    (dict(kv_dtype=7), _lib.MLA_ERR_UNSUPPORTED),
    (dict(sm_scale=-0.04), _lib.MLA_ERR_INVALID),
    (dict(kv_dtype=1, kv_scale=0.0), _lib.MLA_ERR_INVALID),
    (dict(shard_out=None), _lib.MLA_ERR_INVALID),
    (dict(shard_lse=None), _lib.MLA_ERR_INVALID),
    (dict(shard_out=FAKE + 8), _lib.MLA_ERR_INVALID),
    (dict(max_qlen=0), _lib.MLA_ERR_INVALID),
    (dict(nseg=0), _lib.MLA_ERR_INVALID),
])
def test_attn_shard_rejects_bad_arguments(over, code):
    assert _attn_shard(**over) == code
    assert "mla_verify_attn_shard" in mla.mla_last_error()


def _shard_merge(**over):
    a = dict(shard_out=FAKE, shard_lse=FAKE, R=1, H=1, W=1, out=FAKE, lse=FAKE, stream=None)
    a.update(over)
    return _lib.lib.mla_shard_merge(*a.values())


@pytest.mark.parametrize("over,code", [
    (dict(R=0), _lib.MLA_ERR_INVALID),
    (dict(W=0), _lib.MLA_ERR_INVALID),
    (dict(W=1025), _lib.MLA_ERR_UNSUPPORTED),
    (dict(out=None), _lib.MLA_ERR_INVALID),
    (dict(shard_lse=None), _lib.MLA_ERR_INVALID),
    (dict(shard_out=FAKE + 2), _lib.MLA_ERR_INVALID),
])
def test_shard_merge_rejects_bad_arguments(over, code):
    assert _shard_merge(**over) == code
    assert "mla_shard_merge" in mla.mla_last_error()


def _attn_merge(fn, **over):
    a = dict(q=FAKE, kv=FAKE, num_blocks=8, block_size=16, page_size=16, kv_dtype=0,
             kv_scale=1.0, sm_scale=0.04, row_lens=FAKE, page_table=FAKE, pt_width=4,
             q_start=FAKE, N=1, R=1, H=16, W=1, max_qlen=1, nseg=1)
    if fn == "mla_verify_attn_merge":
        a.update(workspace=FAKE, workspace_bytes=1 << 20)
    a.update(out=FAKE, lse=FAKE, stream=None)
    a.update(over)
    return getattr(_lib.lib, fn)(*a.values())


@pytest.mark.parametrize("over,msg", [
    (dict(workspace_bytes=100), "workspace of 100 bytes"),
    (dict(workspace=None), "null workspace"),
    (dict(workspace=FAKE + 4), "aligned"),
    (dict(nseg=0), "nseg"),
    (dict(out=None), "null"),
])
def test_attn_merge_rejects_bad_arguments(over, msg):
    assert _attn_merge("mla_verify_attn_merge", **over) == _lib.MLA_ERR_INVALID
    assert msg in mla.mla_last_error()


def test_static_entry_rejects_sizes_beyond_its_scratch():
    """The no-allocation entry point refuses, before any device call, a size
    whose partials exceed the static array; one byte under the limit passes
    the size check (and then fails on the fake pointers' other checks)."""
    limit = _lib.MLA_STATIC_SCRATCH_BYTES
    per_cell = (512 + 2) * 4
    cells = limit // per_cell
    H = 16
    R = cells // H + 1                                   # W = nseg = 1: over the limit
    assert mla.mla_verify_workspace_bytes(1, R, H, 1) > limit
    assert _attn_merge("mla_verify_attn_merge_static", R=R, H=H) == _lib.MLA_ERR_INVALID
    err = mla.mla_last_error()
    assert "static scratch" in err and str(limit) in err
    R_ok = cells // H
    assert mla.mla_verify_workspace_bytes(1, R_ok, H, 1) <= limit
    assert _attn_merge("mla_verify_attn_merge_static", R=R_ok, H=H, out=None) == \
        _lib.MLA_ERR_INVALID
    assert "null" in mla.mla_last_error()


def _attn_persistent(**over):
    a = dict(q=FAKE, kv=FAKE, num_blocks=8, block_size=16, page_size=16, kv_dtype=0,
             kv_scale=1.0, sm_scale=0.04, row_lens=FAKE, page_table=FAKE, pt_width=4,
             q_start=FAKE, N=1, R=1, H=16, W=1, max_qlen=1, ctas=256, workspace=FAKE,
             workspace_bytes=1 << 30, shard_out=FAKE, shard_lse=FAKE, stream=None)
    a.update(over)
    return _lib.lib.mla_verify_attn_persistent(*a.values())


def test_persistent_workspace_bytes():
    """Counters (4 bytes per group, padded to 256) then two 135168-byte
    partial-state slots per workgroup."""
    ws = mla.mla_verify_attn_persistent_workspace_bytes
    assert ws(32, 8, 16, 4, 256) == 1024 + 2 * 256 * 135168     # 256 groups
    assert ws(3, 3, 12, 7, 8) == 256 + 2 * 8 * 135168            # 18 groups
    assert ws(0, 8, 16, 4, 256) == 0 and ws(1, 1, 1, 1, -1) == 0


@pytest.mark.parametrize("over,code,msg", [
    (dict(kv_dtype=7), _lib.MLA_ERR_UNSUPPORTED, "kv_dtype"),
    (dict(workspace=None), _lib.MLA_ERR_INVALID, "null"),
    (dict(workspace=FAKE + 16), _lib.MLA_ERR_INVALID, "256-byte"),
    (dict(workspace_bytes=1000), _lib.MLA_ERR_INVALID, "workspace of 1000 bytes"),
    (dict(ctas=-1), _lib.MLA_ERR_INVALID, "ctas"),
    (dict(N=2049), _lib.MLA_ERR_UNSUPPORTED, "groups"),
    (dict(pt_width=1 << 26), _lib.MLA_ERR_UNSUPPORTED, "tiles"),
    (dict(shard_out=FAKE + 8), _lib.MLA_ERR_INVALID, "aligned"),
    (dict(max_qlen=0), _lib.MLA_ERR_INVALID, "max_qlen"),
])
def test_persistent_rejects_bad_arguments(over, code, msg):
    """Every check runs before any device call (these are host pointers that
    are never dereferenced)."""
    assert _attn_persistent(**over) == code
    err = mla.mla_last_error()
    assert "mla_verify_attn_persistent" in err and msg in err

