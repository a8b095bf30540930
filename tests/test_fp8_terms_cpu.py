"""The two-term e4m3fn operand splits the fp8 kernels use, checked on the CPU
with torch's own e4m3fn rounding (round to nearest even, the same rounding
the device conversion applies to in-range values).

  * Q: x = q * 2^a with 2^a max|q| in [128, 256); hi = e4m3(x),
    lo = e4m3((x - hi) * 16): hi + lo / 16 == x exactly for every bf16 q
    whose magnitude is at least 2^-13 of the row's largest; smaller ones
    (whose residual falls under e4m3fn's subnormal spacing) err by at most
    2^-14 in x, i.e. 2^-21 of the row's largest.
  * P (weights in [0, 256] relative to the lazy reference): hi = e4m3(p),
    lo = e4m3((p - hi) * 16): |hi + lo / 16 - p| <= 2^-8 p + 2^-14.
These are the bounds the tolerance reading for fp8 caches rests on; the GPU
parity tests check the kernels' results themselves.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")


def e4m3(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .to(torch.float64).numpy()


def all_bf16_finite():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    return v[np.isfinite(v)]


def test_q_split_is_exact_for_bf16():
    q = all_bf16_finite()
    for amax_exp in (-20, -3, 0, 5, 40):           # rows whose largest |q| is 2^e .. 2^(e+1)
        amax = 2.0 ** amax_exp * 1.7
        a = 7 - amax_exp                           # 2^a * amax in [128, 256)
        x = q[np.abs(q) <= amax] * 2.0 ** a
        hi = e4m3(x)
        lo = e4m3((x - hi) * 16.0)
        big = np.abs(x) >= amax * 2.0 ** a * 2.0 ** -13
        assert np.array_equal((hi + lo / 16.0)[big], x[big]), amax_exp
        assert np.all(np.abs(hi + lo / 16.0 - x) <= 2.0 ** -14), amax_exp
        assert np.all(np.abs(x) < 256.0)


def test_p_split_bound():
    rng = np.random.default_rng(0)
    p = np.concatenate([rng.uniform(0, 256, 200000), np.exp2(rng.uniform(-30, 8, 200000)),
                        np.array([0.0, 1.0, 255.9, 2.0 ** -14, 2.0 ** -20])])
    p = p.astype(np.float32).astype(np.float64)    # the kernel's weights are fp32
    hi = e4m3(p)
    lo = e4m3((p - hi) * 16.0)
    err = np.abs(hi + lo / 16.0 - p)
    assert np.all(err <= 2.0 ** -8 * p + 2.0 ** -14)
    # and a single term would not do: its error reaches 2^-4 of the weight
    single = np.abs(hi - p)[p >= 1.0] / p[p >= 1.0]
    assert single.max() > 2.0 ** -5
