"""MI355X (gfx950) paged MLA decode / causal multi-token verify over a
round-robin context-sharded KV cache.

Thin binding over the C ABI in include/mla_verify.h (libmla_verify.so): the
functions below only check and marshal torch tensors (device pointers, the
current HIP stream) and allocate outputs the caller did not pass. Every step
of the computation runs in the HIP kernels of the library.
"""

from __future__ import annotations

import torch

from . import _lib
from ._lib import (MLA_ERR_HIP, MLA_ERR_INVALID, MLA_ERR_UNSUPPORTED,  # noqa: F401
                   MLA_KV_BF16, MLA_KV_FP8_E4M3, MLA_KV_FP8_E5M2, MLA_OK,
                   MLA_PLAN_ERR_BLOCKS,
                   MLA_PLAN_ERR_BOUND, MLA_PLAN_ERR_QLEN, MLA_PLAN_ERR_ROWS)

HEAD_DIM = 576
V_DIM = 512
LIB_PATH = _lib.LIB_PATH


class MlaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status


def mla_last_error() -> str:
    return (_lib.lib.mla_last_error() or b"").decode()


def _check(status: int):
    if status != MLA_OK:
        raise MlaError(status, mla_last_error())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dev(t, dtype, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def mla_subpage_size(block_size: int) -> int:
    return int(_lib.lib.mla_subpage_size(int(block_size)))


def mla_pt_width(max_kv_seq_len: int, page_size: int) -> int:
    return int(_lib.lib.mla_pt_width(int(max_kv_seq_len), int(page_size)))


def mla_verify_workspace_bytes(W: int, R: int, H: int, nseg: int) -> int:
    return int(_lib.lib.mla_verify_workspace_bytes(int(W), int(R), int(H), int(nseg)))


def mla_verify_plan(seq_lens, q_start, R, W, block_table, num_blocks, block_size,
                    max_kv_seq_len, *, page_size=None, pt_width=None, interleave=1,
                    row_lens=None, page_table=None, qo_indptr=None, err_flag=None,
                    stream=None):
    """Row lengths [W, R], sub-page table [W, R, pt_width], qo_indptr [R+1] and
    the device error word (int32 view of the uint32 MLA_PLAN_ERR_* bits; sticky:
    bits are ORed in and never cleared, and a word allocated here starts at 0).
    seq_lens [N], q_start [N+1] and block_table [N, max_blocks] are int32
    device tensors; R = q_start[N] is passed by the caller (no device read)."""
    _dev(seq_lens, torch.int32, "seq_lens")
    _dev(q_start, torch.int32, "q_start")
    _dev(block_table, torch.int32, "block_table")
    N = seq_lens.shape[0]
    if q_start.shape != (N + 1,):
        raise ValueError("q_start must have N+1 entries")
    if block_table.dim() != 2 or block_table.shape[0] != N:
        raise ValueError("block_table must be [N, max_blocks]")
    if page_size is None:
        page_size = mla_subpage_size(block_size)
    if pt_width is None:
        pt_width = mla_pt_width(max_kv_seq_len, page_size)
    dev = seq_lens.device
    if row_lens is None:
        row_lens = torch.empty((W, R), dtype=torch.int32, device=dev)
    if page_table is None:
        page_table = torch.empty((W, R, max(pt_width, 0)), dtype=torch.int32, device=dev)
    if qo_indptr is None:
        qo_indptr = torch.empty((R + 1,), dtype=torch.int32, device=dev)
    if err_flag is None:
        err_flag = torch.zeros((1,), dtype=torch.int32, device=dev)  # sticky: starts clear
    for t, n in ((row_lens, "row_lens"), (page_table, "page_table"),
                 (qo_indptr, "qo_indptr"), (err_flag, "err_flag")):
        _dev(t, torch.int32, n)
    if tuple(row_lens.shape) != (W, R) or tuple(page_table.shape) != (W, R, pt_width) \
            or qo_indptr.numel() != R + 1:
        raise ValueError("row_lens / page_table shape mismatch")
    _check(_lib.lib.mla_verify_plan(
        N, _ptr(seq_lens), _ptr(q_start), int(R), int(W), interleave, _ptr(block_table),
        block_table.shape[1], int(num_blocks), block_size, page_size, max_kv_seq_len,
        pt_width, _ptr(row_lens), _ptr(page_table), _ptr(qo_indptr), _ptr(err_flag),
        _stream(stream)))
    return {"row_lens": row_lens, "page_table": page_table, "qo_indptr": qo_indptr,
            "err_flag": err_flag, "page_size": page_size, "pt_width": pt_width, "R": R}


def _kv_dtype(kv):
    if kv.dtype == torch.bfloat16:
        return MLA_KV_BF16
    if kv.dtype in (torch.uint8, torch.float8_e4m3fn):
        return MLA_KV_FP8_E4M3
    if kv.dtype == torch.float8_e5m2:
        return MLA_KV_FP8_E5M2
    raise TypeError(f"kv must be bfloat16, e4m3fn (uint8) or e5m2 codes, got {kv.dtype}")


def mla_verify_attn(q, kv, row_lens, page_table, q_start, *, page_size, max_qlen,
                    nseg, sm_scale, kv_scale=1.0, segm_out=None, segm_max=None,
                    segm_expsum=None, stream=None):
    """Split-K partials. q [R, H, 576] bf16; kv [W, num_blocks, block_size, 576]
    bf16, e4m3fn codes (uint8 or float8_e4m3fn) or e5m2 codes (float8_e5m2).
    Returns (segm_out, segm_max, segm_expsum)."""
    _dev(q, torch.bfloat16, "q")
    _dev(kv, None, "kv")
    kvd = _kv_dtype(kv)
    _dev(row_lens, torch.int32, "row_lens")
    _dev(page_table, torch.int32, "page_table")
    _dev(q_start, torch.int32, "q_start")
    R, H, D = q.shape
    W, num_blocks, block_size, D2 = kv.shape
    if D != HEAD_DIM or D2 != HEAD_DIM:
        raise ValueError("head dim must be 576")
    if tuple(row_lens.shape) != (W, R) or page_table.shape[:2] != (W, R):
        raise ValueError("plan tensors do not match q / kv")
    N = q_start.shape[0] - 1
    dev = q.device
    if segm_out is None:
        segm_out = torch.empty((W, R, H, nseg, V_DIM), dtype=torch.float32, device=dev)
    if segm_max is None:
        segm_max = torch.empty((W, R, H, nseg), dtype=torch.float32, device=dev)
    if segm_expsum is None:
        segm_expsum = torch.empty((W, R, H, nseg), dtype=torch.float32, device=dev)
    for t, n in ((segm_out, "segm_out"), (segm_max, "segm_max"), (segm_expsum, "segm_expsum")):
        _dev(t, torch.float32, n)
    if segm_out.numel() != W * R * H * nseg * V_DIM or segm_max.numel() != W * R * H * nseg \
            or segm_expsum.numel() != W * R * H * nseg:
        raise ValueError("partial buffers have the wrong size")
    _check(_lib.lib.mla_verify_attn(
        _ptr(q), _ptr(kv), num_blocks, block_size, page_size, kvd, float(kv_scale),
        float(sm_scale), _ptr(row_lens), _ptr(page_table), page_table.shape[2],
        _ptr(q_start), N, R, H, W, int(max_qlen), int(nseg), _ptr(segm_out),
        _ptr(segm_max), _ptr(segm_expsum), _stream(stream)))
    return segm_out, segm_max, segm_expsum


def mla_verify_attn_shard(q, kv, row_lens, page_table, q_start, *, page_size, max_qlen,
                          sm_scale, kv_scale=1.0, nseg=1, shard_out=None, shard_lse=None,
                          stream=None):
    """Attention with each (shard, segment) unit's result normalised: per
    source r * nseg + s, row and head the bf16 output and natural-log LSE, for
    mla_shard_merge over the W * nseg sources. Arguments as for
    mla_verify_attn. Returns (shard_out [W*nseg,R,H,512] bf16,
    shard_lse [W*nseg,R,H])."""
    _dev(q, torch.bfloat16, "q")
    _dev(kv, None, "kv")
    kvd = _kv_dtype(kv)
    _dev(row_lens, torch.int32, "row_lens")
    _dev(page_table, torch.int32, "page_table")
    _dev(q_start, torch.int32, "q_start")
    R, H, D = q.shape
    W, num_blocks, block_size, D2 = kv.shape
    if D != HEAD_DIM or D2 != HEAD_DIM:
        raise ValueError("head dim must be 576")
    if tuple(row_lens.shape) != (W, R) or page_table.shape[:2] != (W, R):
        raise ValueError("plan tensors do not match q / kv")
    N = q_start.shape[0] - 1
    S = W * int(nseg)
    dev = q.device
    if shard_out is None:
        shard_out = torch.empty((S, R, H, V_DIM), dtype=torch.bfloat16, device=dev)
    if shard_lse is None:
        shard_lse = torch.empty((S, R, H), dtype=torch.float32, device=dev)
    _dev(shard_out, torch.bfloat16, "shard_out")
    _dev(shard_lse, torch.float32, "shard_lse")
    if shard_out.numel() != S * R * H * V_DIM or shard_lse.numel() != S * R * H:
        raise ValueError("shard_out / shard_lse have the wrong size")
    _check(_lib.lib.mla_verify_attn_shard(
        _ptr(q), _ptr(kv), num_blocks, block_size, page_size, kvd, float(kv_scale),
        float(sm_scale), _ptr(row_lens), _ptr(page_table), page_table.shape[2],
        _ptr(q_start), N, R, H, W, int(max_qlen), int(nseg), _ptr(shard_out),
        _ptr(shard_lse), _stream(stream)))
    return shard_out, shard_lse


def mla_verify_attn_persistent_workspace_bytes(N: int, W: int, H: int, max_qlen: int,
                                               ctas: int = 0) -> int:
    return int(_lib.lib.mla_verify_attn_persistent_workspace_bytes(
        int(N), int(W), int(H), int(max_qlen), int(ctas)))


def mla_verify_attn_persistent(q, kv, row_lens, page_table, q_start, *, page_size, max_qlen,
                               sm_scale, kv_scale=1.0, ctas=0, workspace=None, shard_out=None,
                               shard_lse=None, stream=None):
    """mla_verify_attn_shard with one segment, on the balanced persistent
    schedule (ctas workgroups, 0 = one per compute unit). ``workspace``: a
    uint8 device tensor of mla_verify_attn_persistent_workspace_bytes bytes
    whose counters are zero (a new one is zero-filled here; every completed
    call leaves it zeroed for the next). Returns (shard_out [W,R,H,512] bf16,
    shard_lse [W,R,H])."""
    _dev(q, torch.bfloat16, "q")
    _dev(kv, None, "kv")
    kvd = _kv_dtype(kv)
    _dev(row_lens, torch.int32, "row_lens")
    _dev(page_table, torch.int32, "page_table")
    _dev(q_start, torch.int32, "q_start")
    R, H, D = q.shape
    W, num_blocks, block_size, D2 = kv.shape
    if D != HEAD_DIM or D2 != HEAD_DIM:
        raise ValueError("head dim must be 576")
    if tuple(row_lens.shape) != (W, R) or page_table.shape[:2] != (W, R):
        raise ValueError("plan tensors do not match q / kv")
    N = q_start.shape[0] - 1
    dev = q.device
    if workspace is None:
        nbytes = mla_verify_attn_persistent_workspace_bytes(N, W, H, max_qlen, ctas)
        if nbytes == 0:
            raise MlaError(_lib.MLA_ERR_INVALID, "persistent workspace size unavailable")
        workspace = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    _dev(workspace, torch.uint8, "workspace")
    if shard_out is None:
        shard_out = torch.empty((W, R, H, V_DIM), dtype=torch.bfloat16, device=dev)
    if shard_lse is None:
        shard_lse = torch.empty((W, R, H), dtype=torch.float32, device=dev)
    _dev(shard_out, torch.bfloat16, "shard_out")
    _dev(shard_lse, torch.float32, "shard_lse")
    if shard_out.numel() != W * R * H * V_DIM or shard_lse.numel() != W * R * H:
        raise ValueError("shard_out / shard_lse have the wrong size")
    _check(_lib.lib.mla_verify_attn_persistent(
        _ptr(q), _ptr(kv), num_blocks, block_size, page_size, kvd, float(kv_scale),
        float(sm_scale), _ptr(row_lens), _ptr(page_table), page_table.shape[2],
        _ptr(q_start), N, R, H, W, int(max_qlen), int(ctas), _ptr(workspace),
        workspace.numel(), _ptr(shard_out), _ptr(shard_lse), _stream(stream)))
    return shard_out, shard_lse


def _attn_merge_args(q, kv, row_lens, page_table, q_start, out, lse):
    _dev(q, torch.bfloat16, "q")
    _dev(kv, None, "kv")
    _dev(row_lens, torch.int32, "row_lens")
    _dev(page_table, torch.int32, "page_table")
    _dev(q_start, torch.int32, "q_start")
    R, H, D = q.shape
    W, num_blocks, block_size, D2 = kv.shape
    if D != HEAD_DIM or D2 != HEAD_DIM:
        raise ValueError("head dim must be 576")
    if tuple(row_lens.shape) != (W, R) or page_table.shape[:2] != (W, R):
        raise ValueError("plan tensors do not match q / kv")
    if out is None:
        out = torch.empty((R, H, V_DIM), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((R, H), dtype=torch.float32, device=q.device)
    _dev(out, torch.bfloat16, "out")
    _dev(lse, torch.float32, "lse")
    if out.numel() != R * H * V_DIM or lse.numel() != R * H:
        raise ValueError("out / lse have the wrong size")
    return R, H, W, num_blocks, block_size, out, lse


def mla_verify_attn_merge(q, kv, row_lens, page_table, q_start, *, page_size, max_qlen, nseg,
                          sm_scale, kv_scale=1.0, workspace=None, out=None, lse=None,
                          stream=None):
    """Attention + segment merge + shard merge in one call, the split-K
    partials in ``workspace`` (a device tensor of at least
    mla_verify_workspace_bytes(W, R, H, nseg) bytes; allocated here if not
    given). Returns (out [R,H,512] bf16, lse [R,H] fp32)."""
    R, H, W, num_blocks, block_size, out, lse = _attn_merge_args(q, kv, row_lens, page_table,
                                                                 q_start, out, lse)
    need = mla_verify_workspace_bytes(W, R, H, nseg)
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=q.device)
    _dev(workspace, None, "workspace")
    _check(_lib.lib.mla_verify_attn_merge(
        _ptr(q), _ptr(kv), num_blocks, block_size, page_size, _kv_dtype(kv), float(kv_scale),
        float(sm_scale), _ptr(row_lens), _ptr(page_table), page_table.shape[2], _ptr(q_start),
        q_start.shape[0] - 1, R, H, W, int(max_qlen), int(nseg), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse), _stream(stream)))
    return out, lse


def mla_verify_attn_merge_static(q, kv, row_lens, page_table, q_start, *, page_size, max_qlen,
                                 nseg, sm_scale, kv_scale=1.0, out, lse, stream=None):
    """mla_verify_attn_merge with the partials in the library's static
    scratch array (MLA_STATIC_SCRATCH_BYTES per GPU): the C call allocates
    nothing, so out and lse must be passed. Calls that overlap on one GPU
    race. Returns (out, lse)."""
    R, H, W, num_blocks, block_size, out, lse = _attn_merge_args(q, kv, row_lens, page_table,
                                                                 q_start, out, lse)
    _check(_lib.lib.mla_verify_attn_merge_static(
        _ptr(q), _ptr(kv), num_blocks, block_size, page_size, _kv_dtype(kv), float(kv_scale),
        float(sm_scale), _ptr(row_lens), _ptr(page_table), page_table.shape[2], _ptr(q_start),
        q_start.shape[0] - 1, R, H, W, int(max_qlen), int(nseg), _ptr(out), _ptr(lse),
        _stream(stream)))
    return out, lse


def mla_shard_merge(shard_out, shard_lse, *, out=None, lse=None, stream=None):
    """Shard LSE merge of per-shard bf16 outputs [W,R,H,512] and natural-log
    LSEs [W,R,H]. Returns (out [R,H,512] bf16, lse [R,H] fp32)."""
    _dev(shard_out, torch.bfloat16, "shard_out")
    _dev(shard_lse, torch.float32, "shard_lse")
    if shard_out.dim() != 4 or shard_out.shape[3] != V_DIM:
        raise ValueError("shard_out must be [W, R, H, 512]")
    W, R, H, _ = shard_out.shape
    if tuple(shard_lse.shape) != (W, R, H):
        raise ValueError("shard_lse must be [W, R, H]")
    dev = shard_out.device
    if out is None:
        out = torch.empty((R, H, V_DIM), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((R, H), dtype=torch.float32, device=dev)
    _dev(out, torch.bfloat16, "out")
    _dev(lse, torch.float32, "lse")
    if out.numel() != R * H * V_DIM or lse.numel() != R * H:
        raise ValueError("out / lse have the wrong size")
    _check(_lib.lib.mla_shard_merge(_ptr(shard_out), _ptr(shard_lse), R, H, W, _ptr(out),
                                    _ptr(lse), _stream(stream)))
    return out, lse


def mla_lse_merge(segm_out, segm_max, segm_expsum, row_lens, q_start, *, page_size,
                  H, nseg, out=None, lse=None, shard_out=None, shard_lse=None,
                  want_shards=False, stream=None):
    """Segment merge + shard LSE merge. Returns (out [R,H,512] bf16,
    lse [R,H] fp32, shard_out [W,R,H,512] bf16 or None, shard_lse or None)."""
    _dev(row_lens, torch.int32, "row_lens")
    _dev(q_start, torch.int32, "q_start")
    for t, n in ((segm_out, "segm_out"), (segm_max, "segm_max"), (segm_expsum, "segm_expsum")):
        _dev(t, torch.float32, n)
    W, R = row_lens.shape
    N = q_start.shape[0] - 1
    dev = row_lens.device
    if segm_out.numel() != W * R * H * nseg * V_DIM or segm_max.numel() != W * R * H * nseg:
        raise ValueError("partial buffers do not match W, R, H, nseg")
    if out is None:
        out = torch.empty((R, H, V_DIM), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((R, H), dtype=torch.float32, device=dev)
    if want_shards and shard_out is None:
        shard_out = torch.empty((W, R, H, V_DIM), dtype=torch.bfloat16, device=dev)
    if want_shards and shard_lse is None:
        shard_lse = torch.empty((W, R, H), dtype=torch.float32, device=dev)
    _dev(out, torch.bfloat16, "out")
    _dev(lse, torch.float32, "lse")
    if out.numel() != R * H * V_DIM or lse.numel() != R * H:
        raise ValueError("out / lse have the wrong size")
    if shard_out is not None:
        _dev(shard_out, torch.bfloat16, "shard_out")
        if shard_out.numel() != W * R * H * V_DIM:
            raise ValueError("shard_out has the wrong size")
    if shard_lse is not None:
        _dev(shard_lse, torch.float32, "shard_lse")
        if shard_lse.numel() != W * R * H:
            raise ValueError("shard_lse has the wrong size")
    _check(_lib.lib.mla_lse_merge(
        _ptr(segm_out), _ptr(segm_max), _ptr(segm_expsum), _ptr(row_lens), _ptr(q_start),
        N, page_size, R, H, W, nseg, _ptr(shard_out), _ptr(shard_lse), _ptr(out), _ptr(lse),
        _stream(stream)))
    return out, lse, shard_out, shard_lse


def mla_verify_forward(dev, *, nseg=1, plan=None, partials=None, out=None, lse=None,
                       want_shards=False, stream=None):
    """plan -> attention partials -> merge for a dict of device tensors
    (keys: q, kv, seq_lens, q_start, block_table, num_blocks, block_size, R, W,
    max_kv_seq_len, max_qlen, sm_scale, kv_scale). Returns a dict with the plan,
    the partials and (out, lse[, shard_out, shard_lse])."""
    if plan is None:
        plan = mla_verify_plan(dev["seq_lens"], dev["q_start"], dev["R"], dev["W"],
                               dev["block_table"], dev["num_blocks"], dev["block_size"],
                               dev["max_kv_seq_len"], interleave=dev.get("interleave", 1),
                               stream=stream)
    kw = {}
    if partials is not None:
        kw = dict(segm_out=partials[0], segm_max=partials[1], segm_expsum=partials[2])
    parts = mla_verify_attn(dev["q"], dev["kv"], plan["row_lens"], plan["page_table"],
                            dev["q_start"], page_size=plan["page_size"],
                            max_qlen=dev["max_qlen"], nseg=nseg, sm_scale=dev["sm_scale"],
                            kv_scale=dev["kv_scale"], stream=stream, **kw)
    o, l, so, sl = mla_lse_merge(*parts, plan["row_lens"], dev["q_start"],
                                 page_size=plan["page_size"], H=dev["q"].shape[1], nseg=nseg,
                                 out=out, lse=lse, want_shards=want_shards, stream=stream)
    return {"plan": plan, "partials": parts, "out": o, "lse": l, "shard_out": so,
            "shard_lse": sl}


def mla_verify_forward_shards(dev, *, nseg=1, plan=None, shards=None, out=None, lse=None,
                              persistent=False, ctas=0, workspace=None, stream=None):
    """plan -> attention with every (shard, segment) unit normalised (bf16
    output + LSE) -> one LSE merge over the W * nseg units, for the same dict
    as mla_verify_forward. ``shards`` may pass (shard_out, shard_lse) buffers.
    persistent: the attention runs on the balanced persistent schedule
    (mla_verify_attn_persistent; nseg must be 1), with ``ctas``
    workgroups and an optional zeroed ``workspace``.
    Returns a dict with the plan, shard_out, shard_lse, out and lse."""
    if plan is None:
        plan = mla_verify_plan(dev["seq_lens"], dev["q_start"], dev["R"], dev["W"],
                               dev["block_table"], dev["num_blocks"], dev["block_size"],
                               dev["max_kv_seq_len"], interleave=dev.get("interleave", 1),
                               stream=stream)
    kw = {}
    if shards is not None:
        kw = dict(shard_out=shards[0], shard_lse=shards[1])
    if persistent:
        if nseg != 1:
            raise ValueError("the persistent schedule takes nseg = 1")
        so, sl = mla_verify_attn_persistent(
            dev["q"], dev["kv"], plan["row_lens"], plan["page_table"], dev["q_start"],
            page_size=plan["page_size"], max_qlen=dev["max_qlen"], sm_scale=dev["sm_scale"],
            kv_scale=dev["kv_scale"], ctas=ctas, workspace=workspace, stream=stream, **kw)
    else:
        so, sl = mla_verify_attn_shard(dev["q"], dev["kv"], plan["row_lens"],
                                       plan["page_table"], dev["q_start"],
                                       page_size=plan["page_size"], max_qlen=dev["max_qlen"],
                                       sm_scale=dev["sm_scale"], kv_scale=dev["kv_scale"],
                                       nseg=nseg, stream=stream, **kw)
    o, l = mla_shard_merge(so, sl, out=out, lse=lse, stream=stream)
    return {"plan": plan, "shard_out": so, "shard_lse": sl, "out": o, "lse": l}


def mla_verify_two_stage_plan(seq_lens, q_start, R, W, block_table, num_blocks, block_size,
                              max_kv_seq_len, max_qlen, *, page_size=None, pt_width=None,
                              interleave=1, row_lens=None, page_table=None, window_table=None,
                              err_flag=None, stream=None):
    """Metadata of the two-stage verify (see mla_verify_two_stage): row lengths
    [W+1, R] (stage-1 committed prefix per shard in rows 0..W-1, stage-2 window
    t + 1 in row W), the stage-1 sub-page table [W, R, pt_width], the stage-2
    window token table [R, max_qlen] and the sticky device error word."""
    _dev(seq_lens, torch.int32, "seq_lens")
    _dev(q_start, torch.int32, "q_start")
    _dev(block_table, torch.int32, "block_table")
    N = seq_lens.shape[0]
    if q_start.shape != (N + 1,):
        raise ValueError("q_start must have N+1 entries")
    if block_table.dim() != 2 or block_table.shape[0] != N:
        raise ValueError("block_table must be [N, max_blocks]")
    if page_size is None:
        page_size = mla_subpage_size(block_size)
    if pt_width is None:
        pt_width = mla_pt_width(max_kv_seq_len, page_size)
    dev = seq_lens.device
    i32 = dict(dtype=torch.int32, device=dev)
    if row_lens is None:
        row_lens = torch.empty((W + 1, R), **i32)
    if page_table is None:
        page_table = torch.empty((W, R, max(pt_width, 0)), **i32)
    if window_table is None:
        window_table = torch.empty((R, max_qlen), **i32)
    if err_flag is None:
        err_flag = torch.zeros((1,), **i32)  # sticky: starts clear
    for t, n in ((row_lens, "row_lens"), (page_table, "page_table"),
                 (window_table, "window_table"), (err_flag, "err_flag")):
        _dev(t, torch.int32, n)
    if tuple(row_lens.shape) != (W + 1, R) or tuple(page_table.shape) != (W, R, pt_width) \
            or tuple(window_table.shape) != (R, max_qlen):
        raise ValueError("row_lens / page_table / window_table shape mismatch")
    _check(_lib.lib.mla_verify_two_stage_plan(
        N, _ptr(seq_lens), _ptr(q_start), int(R), int(W), interleave, _ptr(block_table),
        block_table.shape[1], int(num_blocks), block_size, page_size, max_kv_seq_len,
        pt_width, int(max_qlen), _ptr(row_lens), _ptr(page_table), _ptr(window_table),
        _ptr(err_flag), _stream(stream)))
    return {"row_lens": row_lens, "page_table": page_table, "window_table": window_table,
            "err_flag": err_flag, "page_size": page_size, "pt_width": pt_width, "R": R}


def mla_verify_two_stage(dev, k_window, *, plan=None, stream=None):
    """The SGLang decomposition of the same verify result, from native calls
    ([S34432] implementation items 2-3, the _forward_verify_dcp snippet):

      stage 1 -- every shard attends over its part of the request's committed
                 prefix [0, S_i - Q_i) (every verify row sees the same prefix);
      stage 2 -- one extra source attends over the dense causal window of the
                 request's Q_i verify tokens (row t sees verify tokens 0..t),
                 read from ``k_window`` [R, 576] bf16 (row rho = the entry of
                 verify token rho, request-major, as the snippet lays it out);
      merge   -- natural-log LSE merge over the W stage-1 shards and stage 2.

    mla_verify_two_stage_plan builds both stages' lengths and tables on the
    device; stage 2's pool is ``k_window`` viewed as R blocks of one token.
    ``dev`` is a dict as for mla_verify_forward. Returns (out, lse, err_flag):
    the plan's sticky error word (int32 device tensor, 0 when every request
    is valid)."""
    q, kv = dev["q"], dev["kv"]
    R, H, _ = q.shape
    W = dev["W"]
    _dev(k_window, torch.bfloat16, "k_window")
    if tuple(k_window.shape) != (R, HEAD_DIM):
        raise ValueError("k_window must be [R, 576]")
    qmax = int(dev["max_qlen"])
    if plan is None:
        plan = mla_verify_two_stage_plan(
            dev["seq_lens"], dev["q_start"], R, W, dev["block_table"], dev["num_blocks"],
            dev["block_size"], dev["max_kv_seq_len"], qmax,
            interleave=dev.get("interleave", 1), stream=stream)
    row_lens = plan["row_lens"]
    parts = (torch.empty((W + 1, R, H, 1, V_DIM), dtype=torch.float32, device=q.device),
             torch.empty((W + 1, R, H, 1), dtype=torch.float32, device=q.device),
             torch.empty((W + 1, R, H, 1), dtype=torch.float32, device=q.device))
    mla_verify_attn(q, kv, row_lens[:W], plan["page_table"], dev["q_start"],
                    page_size=plan["page_size"], max_qlen=qmax, nseg=1,
                    sm_scale=dev["sm_scale"], kv_scale=dev["kv_scale"],
                    segm_out=parts[0][:W], segm_max=parts[1][:W], segm_expsum=parts[2][:W],
                    stream=stream)
    mla_verify_attn(q, k_window.view(1, R, 1, HEAD_DIM), row_lens[W:],
                    plan["window_table"].view(1, R, qmax), dev["q_start"], page_size=1,
                    max_qlen=qmax, nseg=1, sm_scale=dev["sm_scale"],
                    segm_out=parts[0][W:], segm_max=parts[1][W:], segm_expsum=parts[2][W:],
                    stream=stream)
    out, lse, _, _ = mla_lse_merge(*parts, row_lens, dev["q_start"],
                                   page_size=plan["page_size"], H=H, nseg=1, stream=stream)
    return out, lse, plan["err_flag"]


__all__ = [
    "mla_subpage_size", "mla_pt_width", "mla_verify_workspace_bytes", "mla_verify_plan",
    "mla_verify_attn", "mla_lse_merge", "mla_verify_attn_shard", "mla_shard_merge",
    "mla_verify_attn_merge", "mla_verify_attn_merge_static",
    "mla_last_error", "mla_verify_forward", "mla_verify_forward_shards",
    "mla_verify_two_stage", "mla_verify_two_stage_plan", "MlaError", "HEAD_DIM", "V_DIM",
]
