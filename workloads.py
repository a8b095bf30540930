"""Seeded synthetic inputs for the paged MLA verify path.

This module only draws random numbers and lays them out in the storage format
the path consumes; it holds none of the method's arithmetic. Both the HIP path
(through the tests, ``bench.py`` and ``smoke()``) and the CPU oracle read what
it produces.

Storage format (the input convention of the path):

* ``q``: bf16 [R, H, 576], rows request-major (row rho = q_start[i] + t).
* ``kv``: one pool per shard, [W, num_blocks, block_size, 576], bf16 bits or
  e4m3fn codes. Global position p of request i is written on shard p % W at
  local index j = p // W, i.e. block ``block_table[i][j // block_size]``,
  offset ``j % block_size`` (round-robin context sharding, interleave 1).
* ``block_table``: int32 [N, max_blocks], one table shared by all shards,
  -1 past each request's blocks. Physical block ids are a random permutation.
* Every slot that holds no token is a NaN canary (bf16 0x7FC0, e4m3fn 0x7F),
  so that a read outside any window shows up as a non-finite output.

The five named workloads follow the shapes of the pages' workloads (Kimi-K3
style MLA with 512 + 64 dims, DCP 4/8, fp8 e4m3 KV, 132k context, qlen
1 + 2*3). Draw order is fixed: seq_lens, qlens, block permutation, q, KV.
"""

from __future__ import annotations

import math

import numpy as np
import torch

HEAD_DIM = 576
BF16_NAN = 0x7FC0
E4M3_NAN = 0x7F
E5M2_NAN = 0x7F

CONFIGS = {
    # batch 2, 16 heads, qlen 1, seq_len {37, 64}, block 16, 1 shard
    "tiny_decode": dict(N=2, H=16, qlen=1, seq_lens=[37, 64], block_size=16,
                        W=1, kv_dtype="bf16", nseg=1),
    # batch 32, 16 heads, qlen 4, seq_len U[1024, 8192], block 64, 8 shards
    "verify_dcp8": dict(N=32, H=16, qlen=4, seq_range=(1024, 8192),
                        block_size=64, W=8, kv_dtype="bf16", nseg=1),
    # batch 64, 12 heads, qlen 7, seq_len U[4096, 32768], fp8 KV, 4 shards
    # (split-K segments: the count measured fastest for the unit-per-workgroup
    # kernel; the config leaves it open. "path": the route measured fastest)
    "fp8_verify_dcp4": dict(N=64, H=12, qlen=7, seq_range=(4096, 32768),
                            block_size=64, W=4, kv_dtype="fp8_e4m3", nseg=2,
                            path="persistent"),
    # batch 16, 16 heads, qlen 4, seq_len 132000, 8 shards, 16 segments
    # (nseg: the pages' split for the unit-per-workgroup kernel; "path": the
    # route measured fastest, the persistent kernel, whose balanced schedule
    # replaces the fixed split)
    "long_context_dcp8": dict(N=16, H=16, qlen=4, seq_lens=[132000] * 16,
                              block_size=128, W=8, kv_dtype="bf16", nseg=16,
                              path="persistent"),
    # 128 requests, 128 heads, qlen U{1..8}, seq_len log-U[256, 65536]
    # (split-K segments: the count measured fastest for the unit-per-workgroup
    # kernel; the config leaves it open. "path" as above)
    "ragged_mixed": dict(N=128, H=128, qlen_range=(1, 8),
                         seq_log_range=(256, 65536), block_size=256, W=1,
                         kv_dtype="bf16", nseg=4, path="persistent"),
}
CONFIG_ORDER = ["tiny_decode", "verify_dcp8", "fp8_verify_dcp4",
                "long_context_dcp8", "ragged_mixed"]


def _to_bf16_bits(x: torch.Tensor) -> np.ndarray:
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def make_workload(spec, seed: int = 0, *, q_mode: str = "normal",
                  kv_mode: str = "normal", spare_blocks: int = 2,
                  keep_logical: bool = False, sm_scale: float | None = None):
    """Draw one workload. ``spec`` is a CONFIGS name or a dict like them.

    q_mode: "normal" (N(0,1)) or "zero".
    kv_mode: "normal" (N(0,1)) or "position" (like normal, but latent column 0
      of global position p holds p, exact in bf16 for p <= 256).
    keep_logical: also return each request's logical KV bits [S, 576].
    """
    if isinstance(spec, str):
        name, spec = spec, CONFIGS[spec]
    else:
        name = spec.get("name", "custom")
    g = torch.Generator().manual_seed(seed)
    N, H, W, B = spec["N"], spec["H"], spec["W"], spec["block_size"]
    kv_dtype = spec["kv_dtype"]

    # 1. sequence lengths
    if "seq_lens" in spec:
        seq_lens = np.asarray(spec["seq_lens"], dtype=np.int64)
    elif "seq_range" in spec:
        lo, hi = spec["seq_range"]
        seq_lens = torch.randint(lo, hi + 1, (N,), generator=g).numpy().astype(np.int64)
    else:
        lo, hi = spec["seq_log_range"]
        u = torch.rand(N, generator=g, dtype=torch.float64).numpy()
        seq_lens = np.rint(np.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))).astype(np.int64)
    # 2. query lengths
    if "qlens" in spec:
        qlens = np.asarray(spec["qlens"], dtype=np.int64)
    elif "qlen_range" in spec:
        lo, hi = spec["qlen_range"]
        qlens = torch.randint(lo, hi + 1, (N,), generator=g).numpy().astype(np.int64)
    else:
        qlens = np.full(N, spec["qlen"], dtype=np.int64)
    q_start = np.zeros(N + 1, dtype=np.int64)
    q_start[1:] = np.cumsum(qlens)
    R = int(q_start[-1])

    # 3. paged storage: each request owns ceil(Lmax/B) blocks on every shard,
    # Lmax its longest shard-local sequence (shard 0's): ceil(S/W) for
    # interleave 1, c*I + min(S mod (I*W), I) with c = S div (I*W) in general
    I = int(spec.get("interleave", 1))
    local_max = (seq_lens // (I * W)) * I + np.minimum(seq_lens % (I * W), I)
    nblocks = -(-local_max // B)
    num_blocks = int(nblocks.sum()) + spare_blocks
    perm = torch.randperm(num_blocks, generator=g).numpy().astype(np.int64)
    max_blocks = int(spec.get("max_blocks", nblocks.max()))
    block_table = np.full((N, max_blocks), -1, dtype=np.int64)
    off = 0
    for i in range(N):
        block_table[i, :nblocks[i]] = perm[off:off + nblocks[i]]
        off += int(nblocks[i])

    # 4. queries
    if q_mode == "zero":
        q32 = torch.zeros(R, H, HEAD_DIM)
    else:
        q32 = torch.randn(R, H, HEAD_DIM, generator=g)
    q_bits = _to_bf16_bits(q32)
    del q32

    # 5. KV, drawn per request in order
    def draw(i):
        k = torch.randn(int(seq_lens[i]), HEAD_DIM, generator=g)
        if kv_mode == "position":
            k[:, 0] = torch.arange(int(seq_lens[i]), dtype=torch.float32)
        return k

    if kv_dtype == "bf16":
        cache = np.full((W, num_blocks, B, HEAD_DIM), BF16_NAN, dtype=np.uint16)
        kv_scale = 1.0
        per_req = (lambda i: _to_bf16_bits(draw(i)))
    elif kv_dtype == "fp8_e4m3":
        cache = np.full((W, num_blocks, B, HEAD_DIM), E4M3_NAN, dtype=np.uint8)
        ks = [draw(i) for i in range(N)]
        amax = max(float(k.abs().max()) for k in ks)
        kv_scale = amax / 448.0
        codes = [(k / kv_scale).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
                 .view(torch.uint8).numpy() for k in ks]
        del ks
        per_req = (lambda i: codes[i])
    elif kv_dtype == "fp8_e5m2":
        cache = np.full((W, num_blocks, B, HEAD_DIM), E5M2_NAN, dtype=np.uint8)
        ks = [draw(i) for i in range(N)]
        amax = max(float(k.abs().max()) for k in ks)
        kv_scale = amax / 57344.0
        codes = [(k / kv_scale).clamp(-57344.0, 57344.0).to(torch.float8_e5m2)
                 .view(torch.uint8).numpy() for k in ks]
        del ks
        per_req = (lambda i: codes[i])
    else:
        raise ValueError(kv_dtype)

    logical = [] if keep_logical else None
    for i in range(N):
        bits = per_req(i)
        S = int(seq_lens[i])
        p = np.arange(S)
        j = (p // (I * W)) * I + p % I                # local index on shard (p // I) % W
        cache[(p // I) % W, block_table[i][j // B], j % B, :] = bits
        if keep_logical:
            logical.append(bits.copy())
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    return {
        "name": name, "seed": seed, "N": N, "H": H, "W": W, "block_size": B,
        "interleave": I,
        "kv_dtype": kv_dtype, "kv_scale": float(kv_scale),
        "sm_scale": float(sm_scale), "nseg": int(spec.get("nseg", 1)),
        "path": spec.get("path", "shards"),
        "seq_lens": seq_lens, "qlens": qlens, "q_start": q_start, "R": R,
        "block_table": block_table, "num_blocks": num_blocks,
        "max_kv_seq_len": int(local_max.max()),
        "q_bits": q_bits, "kv_bits": cache, "logical_kv_bits": logical,
    }


def kv_bytes_per_token(kv_dtype: str) -> int:
    return HEAD_DIM * (2 if kv_dtype == "bf16" else 1)


def algorithmic_kv_bytes(inp) -> int:
    """Every cached token read once: sum_i S_i * 576 * bytes per element."""
    return int(np.sum(inp["seq_lens"])) * kv_bytes_per_token(inp["kv_dtype"])


def algorithmic_flops(inp) -> int:
    """Dense QK^T (2*576) and PV (2*512) flops over every row's causal window,
    summed over all heads: sum_i H * 2176 * sum_t (S_i - Q_i + 1 + t)."""
    S = inp["seq_lens"].astype(np.int64)
    Q = inp["qlens"].astype(np.int64)
    window_sum = Q * (S - Q) + Q * (Q + 1) // 2
    return int(window_sum.sum()) * int(inp["H"]) * (2 * 576 + 2 * 512)


def to_device(inp, device="cuda"):
    """Move a workload's inputs to the GPU in the layouts the library takes."""
    import torch as _t
    q = _t.from_numpy(inp["q_bits"].view(np.int16)).view(_t.bfloat16).to(device)
    if inp["kv_dtype"] == "bf16":
        kv = _t.from_numpy(inp["kv_bits"].view(np.int16)).view(_t.bfloat16).to(device)
    elif inp["kv_dtype"] == "fp8_e5m2":
        kv = _t.from_numpy(inp["kv_bits"]).view(_t.float8_e5m2).to(device)
    else:
        kv = _t.from_numpy(inp["kv_bits"]).to(device)
    i32 = lambda a: _t.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)
    return {
        "q": q, "kv": kv, "seq_lens": i32(inp["seq_lens"]), "q_start": i32(inp["q_start"]),
        "block_table": i32(inp["block_table"]), "num_blocks": int(inp["num_blocks"]),
        "block_size": int(inp["block_size"]), "R": int(inp["R"]), "W": int(inp["W"]),
        "interleave": int(inp.get("interleave", 1)),
        "max_kv_seq_len": int(inp["max_kv_seq_len"]), "max_qlen": int(np.max(inp["qlens"])),
        "sm_scale": float(inp["sm_scale"]), "kv_scale": float(inp["kv_scale"]),
    }
