"""fp64 CPU oracle: what the paged MLA verify path computes, written plainly.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): nothing on the product
path may import, call or link this module.

Sources (web pages, cited by title and section):

* [V51705] prhub digest of vLLM PR #51705, "ROCm AITER MLA supports causal
  multi-token speculative verify under DCP".
* [S34432] prhub report of SGLang PR #34432, "[AMD][DCP 1/N] add dcp support
  for aiter backend".
* [V51011] prhub digest of vLLM PR #51011, "fix silent wrong decode for fp8 KV
  in ROCm AITER MLA".

Notation: request i has global length S_i (tokens in the cache, the Q_i verify
tokens included) and Q_i verify rows; rows are request-major, row rho = qs_i+t
with qs = q_start. W shards hold the sequence round-robin with interleave 1.
Head dim D = 576 (512 latent + 64 rope); V is the 512-wide latent part.

Everything is float64 / Python int. Where the pages are silent or garbled the
reading taken is stated at the function; the full list of readings lives in
the repository's design notes.
"""

from __future__ import annotations

import math

import numpy as np

HEAD_DIM = 576  # q/k width: 512 latent (kv_lora_rank) + 64 rope
V_DIM = 512     # v is the latent part of the same cached entry
LN2 = math.log(2.0)
LOG2E = 1.0 / LN2

__all__ = [
    "HEAD_DIM", "V_DIM", "LN2", "LOG2E",
    "subpage_size", "window_length", "row_view", "qo_indptr", "subpage_table",
    "plan", "shard_of", "local_index", "decode_bf16", "e4m3fn_value", "e4m3fn_table", "decode_e4m3fn",
    "e5m2_value", "e5m2_table", "decode_e5m2",
    "gather_request_kv", "attention_rows", "shard_local_kv",
    "shard_attention_rows", "segment_partials", "segment_merge", "lse_merge",
    "two_stage_plan", "two_stage_verify", "verify_reference", "request_rows",
]


# --------------------------------------------------------------------------
# Plan: sub-page size, per-row causal window, rank-local row lengths, table
# --------------------------------------------------------------------------

def subpage_size(block_size: int) -> int:
    """Sub-page (tile) size for a physical KV block.

    [V51705] Implementation breakdown item 3 and the ``_segmented_mla_page_size``
    snippet: the largest power of two dividing the block size, capped at 128;
    a non-positive block size is an error.
    """
    block_size = int(block_size)
    if block_size <= 0:
        raise ValueError("block_size must be positive")
    p = 1
    rest = block_size
    while rest % 2 == 0 and p < 128:
        rest //= 2
        p *= 2
    return p


def window_length(seq_len: int, qlen: int, t: int) -> int:
    """Number of global positions verify row t may attend to.

    [V51705] Implementation breakdown item 2 and the ``_build_dcp_verify_row_view``
    docstring: row t sees the inclusive global range [0, S - Q + t], its own
    token included, so the window holds S - Q + 1 + t positions. (The same
    snippet's tensor expression is one larger; the docstring and the review
    thread agree on the inclusive bound, which is the reading taken.)
    """
    return int(seq_len) - int(qlen) + 1 + int(t)


def request_rows(q_start, i):
    """Rows (and qlen) of request i: rho in [q_start[i], q_start[i+1])."""
    return int(q_start[i]), int(q_start[i + 1]) - int(q_start[i])


def shard_of(p, W: int, interleave: int = 1):
    """Shard holding global position p under round-robin placement with the
    given interleave: consecutive runs of `interleave` positions are dealt to
    shards 0, 1, ..., W-1 in turn ([V51705] Implementation breakdown item 2
    and [S34432] key snippet for interleave 1, where local index j of shard r
    is global position j*W + r; interleave > 1 is this build's reading of the
    same layout -- the pages gate it off as unverified)."""
    return (np.asarray(p) // interleave) % W


def local_index(p, W: int, interleave: int = 1):
    """Index of global position p in its shard's local sequence: the run number
    times the interleave plus the offset inside the run (j*W + r for
    interleave 1). Increasing in p on every shard."""
    p = np.asarray(p)
    return (p // (interleave * W)) * interleave + p % interleave


def row_view(seq_lens, q_start, W: int, interleave: int = 1) -> np.ndarray:
    """Rank-local KV length of every verify row on every shard, by brute force.

    [V51705] Implementation breakdown item 2: a row's local length on shard r
    is the number of positions of its causal window that shard r holds (see
    shard_of). This function counts them one position at a time; it does not
    use a closed form. Returns int64 [W, R].
    """
    seq_lens = [int(s) for s in seq_lens]
    q_start = [int(x) for x in q_start]
    N = len(seq_lens)
    R = q_start[N]
    out = np.zeros((W, R), dtype=np.int64)
    for i in range(N):
        qs, Q = request_rows(q_start, i)
        for t in range(Q):
            w = window_length(seq_lens[i], Q, t)
            if w <= 0:
                continue
            owner = shard_of(np.arange(w, dtype=np.int64), W, interleave)
            out[:, qs + t] = np.bincount(owner, minlength=W)[:W]
    return out


def qo_indptr(R: int) -> np.ndarray:
    """One query per verify row, so the query index pointer is 0..R.

    [V51705] key snippet, ``AiterMLADCPVerifyMetadata.qo_indptr``.
    """
    return np.arange(R + 1, dtype=np.int64)


def subpage_table(row_lens, block_table, q_start, block_size: int,
                  page_size: int, pt_width: int) -> np.ndarray:
    """Per-row sub-page table [W, R, pt_width]; unused entries are -1.

    [V51705] Implementation breakdown item 3 and the sub-page snippet: the
    cache is viewed as pages of ``page_size`` tokens, so physical block b
    holds sub-pages b*n .. b*n+n-1 with n = block_size / page_size, sub-page
    b*n+k covering the block's tokens [k*page_size, (k+1)*page_size).
    Row rho on shard r needs the sub-pages that cover its local tokens
    [0, L). Local token j sits in physical block block_table[i][j // B] at
    offset j % B (one block table shared by all shards; a reading).
    """
    row_lens = np.asarray(row_lens)
    W, R = row_lens.shape
    n = block_size // page_size
    table = np.full((W, R, pt_width), -1, dtype=np.int64)
    N = len(q_start) - 1
    for i in range(N):
        qs, Q = request_rows(q_start, i)
        for rho in range(qs, qs + Q):
            for r in range(W):
                L = int(row_lens[r, rho])
                pages = -(-L // page_size)
                if pages > pt_width:
                    raise ValueError("page table too narrow for row length")
                for k in range(pages):
                    first = k * page_size            # first local token of page k
                    block = int(block_table[i][first // block_size])
                    table[r, rho, k] = block * n + (first % block_size) // page_size
    return table


def plan(seq_lens, q_start, W, block_table, block_size, max_kv_seq_len, interleave=1):
    """Everything the metadata builder produces, built once per forward.

    [V51705] key snippet, ``AiterMLADCPVerifyMetadata``: row lengths, the
    sub-page table, qo_indptr, the page size, and the kernel-visible KV bound.
    The table width is ceil(max_kv_seq_len / page_size).
    """
    P = subpage_size(block_size)
    L = row_view(seq_lens, q_start, W, interleave)
    width = -(-int(max_kv_seq_len) // P)
    pt = subpage_table(L, block_table, q_start, block_size, P, width)
    return {"page_size": P, "row_lens": L, "page_table": pt,
            "qo_indptr": qo_indptr(int(q_start[-1])), "pt_width": width}


# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------

def decode_bf16(bits) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (bf16 is the top half of an fp32)."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e4m3fn_value(byte: int) -> float:
    """Value of one OCP FP8 E4M3 ("fn": finite, no infinities) byte.

    [S34432] motivation / launch flags name the fp8_e4m3 KV cache; the format
    is taken from its published definition: 1 sign bit, 4 exponent bits with
    bias 7, 3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111
    is NaN; there is no infinity, so the largest finite value is 448.
    """
    byte = int(byte) & 0xFF
    sign = -1.0 if byte & 0x80 else 1.0
    exp = (byte >> 3) & 0xF
    man = byte & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


def e4m3fn_table() -> np.ndarray:
    return np.array([e4m3fn_value(b) for b in range(256)], dtype=np.float64)


_E4M3_TABLE = e4m3fn_table()


def decode_e4m3fn(codes) -> np.ndarray:
    return _E4M3_TABLE[np.asarray(codes).astype(np.int64)]


def e5m2_value(byte: int) -> float:
    """Value of one OCP FP8 E5M2 byte.

    [V51011] the new fp8 routing test lists fp8_e5m2 beside fp8_e4m3 as a KV
    cache dtype; the format is taken from its published definition: 1 sign
    bit, 5 exponent bits with bias 15, 2 mantissa bits; exponent 0 is
    subnormal (m/4 * 2^-14); exponent 31 is infinity (m = 0) or NaN, so the
    largest finite value is 1.75 * 2^15 = 57344.
    """
    byte = int(byte) & 0xFF
    sign = -1.0 if byte & 0x80 else 1.0
    exp = (byte >> 2) & 0x1F
    man = byte & 0x3
    if exp == 0x1F:
        return sign * float("inf") if man == 0 else float("nan")
    if exp == 0:
        return sign * (man / 4.0) * 2.0 ** (1 - 15)
    return sign * (1.0 + man / 4.0) * 2.0 ** (exp - 15)


def e5m2_table() -> np.ndarray:
    return np.array([e5m2_value(b) for b in range(256)], dtype=np.float64)


_E5M2_TABLE = e5m2_table()


def decode_e5m2(codes) -> np.ndarray:
    return _E5M2_TABLE[np.asarray(codes).astype(np.int64)]


# --------------------------------------------------------------------------
# Reading a request's logical KV back out of the sharded paged cache
# --------------------------------------------------------------------------

def gather_request_kv(cache, kv_dtype: str, kv_scale: float, block_table_row,
                      seq_len: int, W: int, block_size: int,
                      interleave: int = 1) -> np.ndarray:
    """Logical KV of one request, [S, 576] float64, read from the cache.

    ``cache`` holds raw bits, shaped [W, num_blocks, block_size, 576] (uint16
    bf16 bits or uint8 e4m3fn codes). Global position p is held by shard
    p mod W at local index j = p div W ([S34432] key snippet: j*W + r), i.e. in
    physical block block_table_row[j div B] at offset j mod B.
    fp8 entries are real = decode(code) * kv_scale ([S34432] key snippet: one
    per-tensor float scale, the same bytes serving K and V).
    """
    p = np.arange(int(seq_len), dtype=np.int64)
    shard = shard_of(p, W, interleave)
    local = local_index(p, W, interleave)
    blocks = np.asarray(block_table_row, dtype=np.int64)[local // block_size]
    raw = cache[shard, blocks, local % block_size, :]
    if kv_dtype == "bf16":
        return decode_bf16(raw)
    if kv_dtype == "fp8_e4m3":
        return decode_e4m3fn(raw) * float(kv_scale)
    if kv_dtype == "fp8_e5m2":
        return decode_e5m2(raw) * float(kv_scale)
    raise ValueError(kv_dtype)


# --------------------------------------------------------------------------
# Attention: the definition, per-shard pieces, segments, merges
# --------------------------------------------------------------------------

def attention_rows(q_rows, K, seq_len: int, qlen: int, sm_scale: float, values=None):
    """Causal multi-token verify attention for one request (the definition).

    q_rows [Q, H, 576], K [S, 576] (logical, dequantised). Row t attends to
    positions [0, S-Q+t] ([V51705] Implementation breakdown item 2). Scores
    are sm_scale * <q, k> over all 576 dims; V is K[:, :512] ([S34432] key
    snippet, the verify window's v is the latent part). Returns out
    [Q, H, 512] and the natural-log LSE [Q, H] of the scaled scores
    ([S34432] implementation item 1 and review item 4: LSE base e).
    Q = 1 is plain decode ([V51705] implementation item 4).
    ``values`` [S, n] replaces V (default K[:, :512]): the same softmax
    weights applied to other per-position values, e.g. |V| for an error bound.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = K[:, :V_DIM] if values is None else np.asarray(values, dtype=np.float64)
    Q, H, _ = q_rows.shape
    out = np.zeros((Q, H, V.shape[1]))
    lse = np.zeros((Q, H))
    for t in range(Q):
        w = window_length(seq_len, qlen, t)
        s = sm_scale * (q_rows[t] @ K[:w].T)          # [H, w]
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        z = p.sum(axis=1)
        out[t] = (p @ V[:w]) / z[:, None]
        lse[t] = m[:, 0] + np.log(z)
    return out, lse


def shard_local_kv(K, W: int, r: int, interleave: int = 1):
    """Shard r's local sequence: its global positions in increasing order
    (r, r+W, r+2W, ... for interleave 1)."""
    K = np.asarray(K)
    p = np.arange(K.shape[0])
    return K[shard_of(p, W, interleave) == r]


def shard_attention_rows(q_rows, K_local, L_rows, sm_scale: float, values=None):
    """Rank-local attention of each row over the first L local tokens.

    Each row's window restricted to one shard is a prefix of that shard's
    local sequence ([V51705] Implementation breakdown item 2: the local length
    is the count of window positions the shard holds). An empty prefix gives
    out 0 and lse -inf (a reading: nothing to attend to). ``values`` replaces
    V as in attention_rows.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    V = K_local[:, :V_DIM] if values is None else np.asarray(values, dtype=np.float64)
    Q, H, _ = q_rows.shape
    out = np.zeros((Q, H, V.shape[1]))
    lse = np.full((Q, H), -np.inf)
    for t in range(Q):
        L = int(L_rows[t])
        if L == 0:
            continue
        s = sm_scale * (q_rows[t] @ K_local[:L].T)
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        z = p.sum(axis=1)
        out[t] = (p @ V[:L]) / z[:, None]
        lse[t] = m[:, 0] + np.log(z)
    return out, lse


def segment_partials(q_rows, K_local, L_rows, nseg: int, page_size: int,
                     sm_scale: float, values=None):
    """Split-K partials of one (request, shard) group.

    [V51705] Implementation breakdown item 4 and the merge snippet: the
    sequence is cut into NUM_SEGMENTS segments of tiles_per_segment tiles of
    TILE_SIZE (= page size) tokens, tiles_per_segment =
    ceil(len / (NUM_SEGMENTS * TILE_SIZE)); each segment keeps a base-2
    running max, a sum of exp2 and an (unnormalised) output.
    Reading: the length is the group's longest row (its last row), so all rows
    of the group share segment boundaries; segment s covers local tokens
    [s*T*P, (s+1)*T*P) clipped to each row's own length. A segment with no
    tokens for a row is inactive: m2 = -inf, e = 0, O = 0.

    Returns m2 [Q, H, nseg] (max of scaled score * log2 e), e [Q, H, nseg]
    (sum of 2^(score2 - m2)), O [Q, H, nseg, 512], active [Q, nseg].
    ``values`` replaces V as in attention_rows (O then has its width).
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    V = K_local[:, :V_DIM] if values is None else np.asarray(values, dtype=np.float64)
    Q, H, _ = q_rows.shape
    Lg = int(max(L_rows)) if Q else 0
    span = -(-Lg // (nseg * page_size)) * page_size   # T * P tokens
    m2 = np.full((Q, H, nseg), -np.inf)
    e = np.zeros((Q, H, nseg))
    O = np.zeros((Q, H, nseg, V.shape[1]))
    active = np.zeros((Q, nseg), dtype=bool)
    for t in range(Q):
        L = int(L_rows[t])
        for s in range(nseg):
            lo = s * span
            hi = min((s + 1) * span, L)
            if lo >= hi:
                continue
            active[t, s] = True
            s2 = (sm_scale * (q_rows[t] @ K_local[lo:hi].T)) * LOG2E  # [H, n]
            mx = s2.max(axis=1)
            w = np.exp2(s2 - mx[:, None])
            m2[t, :, s] = mx
            e[t, :, s] = w.sum(axis=1)
            O[t, :, s] = w @ V[lo:hi]
    return m2, e, O, active


def segment_merge(m2, e, O, active):
    """Merge base-2 segment partials into (out, natural-log lse).

    [V51705] merge snippet: M = max over active segments of m2,
    E = sum e_s * 2^(m2_s - M), out = sum O_s * 2^(m2_s - M) / E, and the
    natural-log LSE is ln 2 * (M + log2 E) (the snippet's LOGE2 constant).
    Rows with no active segment give out 0 and lse -inf.
    Shapes: m2/e [..., nseg], O [..., nseg, 512], active broadcastable to m2.
    """
    m2 = np.asarray(m2, dtype=np.float64)
    act = np.broadcast_to(np.asarray(active, dtype=bool), m2.shape)
    masked = np.where(act, m2, -np.inf)
    M = masked.max(axis=-1)
    has = np.isfinite(M)
    Msafe = np.where(has, M, 0.0)
    scale = np.where(act, np.exp2(masked - Msafe[..., None]), 0.0)
    E = (np.asarray(e) * scale).sum(axis=-1)
    num = (np.asarray(O) * scale[..., None]).sum(axis=-2)
    out = np.where(has[..., None], num / np.where(has, E, 1.0)[..., None], 0.0)
    lse = np.where(has, LN2 * (Msafe + np.log2(np.where(has, E, 1.0))), -np.inf)
    return out, lse


def lse_merge(outs, lses):
    """Combine per-shard (out, natural-log lse) into the full result.

    [V51705] Motivation and implementation item 4 (rank-local partials are
    merged through the DCP attention merge using the natural-log LSE) and
    [S34432] review item 4 (the base must be e: exp/log, not exp2/log2).
    lse = ln sum_r exp(lse_r); out = sum_r exp(lse_r - lse) * out_r.
    Shards with lse_r = -inf contribute nothing; all -inf gives out 0, -inf.
    outs [W, ..., 512], lses [W, ...].
    """
    lses = np.asarray(lses, dtype=np.float64)
    outs = np.asarray(outs, dtype=np.float64)
    mx = lses.max(axis=0)
    has = np.isfinite(mx)
    mxs = np.where(has, mx, 0.0)
    wts = np.where(np.isfinite(lses), np.exp(lses - mxs), 0.0)
    tot = wts.sum(axis=0)
    lse = np.where(has, mxs + np.log(np.where(has, tot, 1.0)), -np.inf)
    frac = np.where(has, wts / np.where(has, tot, 1.0), 0.0)
    out = (frac[..., None] * outs).sum(axis=0)
    return out, lse


def two_stage_plan(seq_lens, q_start, W, block_table, block_size, max_kv_seq_len,
                   max_qlen, interleave=1):
    """Metadata of the two-stage verify, built per forward.

    [S34432] Implementation breakdown items 2-3 and the ``_forward_verify_dcp``
    snippet: stage 1 gives every verify row its request's committed prefix
    [0, S - Q) on each shard (a per-row local length and a per-row token table,
    read row by row); stage 2 gives row t the dense causal window of verify
    tokens 0..t, whose entries sit request-major in a separate window buffer
    (request i's verify token k at row q_start[i] + k).
    Stage-1 lengths are counted one position at a time, like ``row_view``.
    Returns row_lens [W+1, R] (stage 1 in rows 0..W-1, stage 2 in row W), the
    stage-1 sub-page table [W, R, width] and window_table [R, max_qlen]
    (-1 past each row's window).
    """
    seq_lens = [int(x) for x in seq_lens]
    q_start = [int(x) for x in q_start]
    N = len(seq_lens)
    R = q_start[N]
    P = subpage_size(block_size)
    L = np.zeros((W + 1, R), dtype=np.int64)
    win = np.full((R, int(max_qlen)), -1, dtype=np.int64)
    for i in range(N):
        qs, Q = request_rows(q_start, i)
        committed = seq_lens[i] - Q
        owner = shard_of(np.arange(committed, dtype=np.int64), W, interleave)
        counts = np.bincount(owner, minlength=W)[:W] if committed > 0 else np.zeros(W, np.int64)
        for t in range(Q):
            L[:W, qs + t] = counts
            L[W, qs + t] = t + 1
            for k in range(t + 1):
                win[qs + t, k] = qs + k
    width = -(-int(max_kv_seq_len) // P)
    pt = subpage_table(L[:W], block_table, q_start, block_size, P, width)
    return {"page_size": P, "row_lens": L, "page_table": pt, "window_table": win,
            "pt_width": width}


def two_stage_verify(q_rows, K, seq_len: int, qlen: int, W: int,
                     sm_scale: float):
    """The SGLang decomposition of the same result, used as a cross-check.

    [S34432] implementation item 3 and the ``_forward_verify_dcp`` snippet:
    stage 1, every shard attends over its part of the committed prefix
    [0, S-Q); stage 2, only shard 0 attends over the dense causal window of
    the Q verify tokens (row t sees verify tokens 0..t); the two stages are
    merged locally by LSE, then all shards are merged by LSE.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    Q, H, _ = q_rows.shape
    committed = seq_len - qlen
    outs = np.zeros((W, Q, H, V_DIM))
    lses = np.full((W, Q, H), -np.inf)
    for r in range(W):
        local = shard_local_kv(K[:committed], W, r)
        o1, l1 = shard_attention_rows(q_rows, local, [len(local)] * Q, sm_scale)
        if r == 0:
            window = K[committed:seq_len]
            o2, l2 = shard_attention_rows(q_rows, window,
                                          [t + 1 for t in range(Q)], sm_scale)
            o1, l1 = lse_merge(np.stack([o1, o2]), np.stack([l1, l2]))
        outs[r], lses[r] = o1, l1
    return lse_merge(outs, lses)


def verify_reference(inp, requests=None):
    """The full result (out [R, H, 512], lse [R, H]) from the definition.

    ``inp`` is a workload dict (see ``workloads.py``): raw q bits, the raw
    sharded cache and its block table. Each request's logical KV is read back
    from the cache and attention_rows is applied. ``requests`` restricts the
    work to a subset (rows of other requests are left NaN).
    """
    seq_lens = inp["seq_lens"]
    q_start = inp["q_start"]
    R = int(q_start[-1])
    H = int(inp["H"])
    q = decode_bf16(inp["q_bits"])
    out = np.full((R, H, V_DIM), np.nan)
    lse = np.full((R, H), np.nan)
    idx = range(len(seq_lens)) if requests is None else requests
    for i in idx:
        qs, Q = request_rows(q_start, i)
        K = gather_request_kv(inp["kv_bits"], inp["kv_dtype"], inp["kv_scale"],
                              inp["block_table"][i], int(seq_lens[i]),
                              int(inp["W"]), int(inp["block_size"]),
                              int(inp.get("interleave", 1)))
        o, l = attention_rows(q[qs:qs + Q], K, int(seq_lens[i]), Q,
                              float(inp["sm_scale"]))
        out[qs:qs + Q], lse[qs:qs + Q] = o, l
    return out, lse
