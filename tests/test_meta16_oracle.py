"""Pins of the oracle's fp16 scale / zero-point storage (no GPU).

The stored metadata must (a) be fp16 numbers, (b) be the specific fp16
neighbours the storage rule names: the zero-point the largest fp16 not above
the group minimum, the scale the smallest fp16 not below the scale computed
from that zero-point, and (c) keep the property the fp32 path has: every
value of the group lies on the covered range, codes stay in [0, 2^b - 1] and
the reconstruction error is at most half the stored scale.  The fp16
neighbours are checked against a brute-force search over every finite fp16
value (not against the oracle's own rounding code).
"""
import numpy as np
import pytest

from oracle import quant as Q
from oracle import cache as OC

F32 = np.float32
# every finite fp16 value, sorted (negative zero folded into zero)
_ALL = np.arange(1 << 16, dtype=np.uint16).view(np.float16)
FINITE = np.unique(_ALL[np.isfinite(_ALL)].astype(np.float64))


def brute_up(x):
    return FINITE[np.searchsorted(FINITE, np.asarray(x, np.float64), side="left")]


def brute_down(x):
    return FINITE[np.searchsorted(FINITE, np.asarray(x, np.float64), side="right") - 1]


def test_directed_fp16_rounding_matches_brute_force():
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.standard_normal(20000).astype(F32) * F32(3.0),
        (rng.standard_normal(4000) * 1e-6).astype(F32),          # fp16 subnormal range
        (rng.standard_normal(4000) * 3e4).astype(F32),
        FINITE[::97].astype(F32),                                  # exact fp16 values
        np.array([0.0, -0.0, 6.0e-8, -6.0e-8, 65504.0, -65504.0, 65519.0, -65519.0], F32),
    ]).astype(F32)
    x = x[np.abs(x) <= 65504.0]
    up, down = Q.f16_toward(x, up=True), Q.f16_toward(x, up=False)
    assert np.array_equal(up.astype(np.float64), brute_up(x))
    assert np.array_equal(down.astype(np.float64), brute_down(x))
    # exact fp16 values stay put
    ex = FINITE[::97].astype(F32)
    assert np.array_equal(Q.f16_toward(ex, True), ex) and np.array_equal(Q.f16_toward(ex, False), ex)


def test_directed_rounding_saturates_beyond_the_fp16_range():
    big = np.array([7.0e4, 1.0e9, -7.0e4, -1.0e9], F32)
    assert np.array_equal(Q.f16_toward(big, up=False), np.array([65504, 65504, -65504, -65504], F32))
    assert np.array_equal(Q.f16_toward(big, up=True), np.array([65504, 65504, -65504, -65504], F32))


def _groups(seed, n=400, G=32):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, G)).astype(F32)
    x[: n // 4] *= F32(60.0)                                # outlier-scale groups
    x[n // 4: n // 2] += F32(1000.0)                        # offset groups (zero far from 0)
    x[n // 2: n // 2 + 8] = F32(1.0001)                     # constant groups
    x[n // 2 + 8: n // 2 + 16] *= F32(1e-5)                 # tiny ranges (subnormal scales)
    return x


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_asym_fp16_metadata_rule_and_bound(bits):
    x = _groups(bits)
    qmax = F32(2 ** bits - 1)
    c, s, z = Q.asym_quantize(x, bits, axis=1, meta16=True)
    # fp16 numbers
    assert np.array_equal(s.astype(np.float16).astype(F32), s)
    assert np.array_equal(z.astype(np.float16).astype(F32), z)
    mn, mx = x.min(axis=1, keepdims=True), x.max(axis=1, keepdims=True)
    # the named neighbours, by brute force
    assert np.array_equal(z.astype(np.float64), brute_down(mn))
    s32 = (np.maximum((mx - z).astype(F32), F32(1e-8)) / qmax).astype(F32)
    assert np.array_equal(s.astype(np.float64), brute_up(s32))
    # codes in range and the bound: |x - x_hat| <= s/2 (plus fp32 rounding of the
    # reconstruction and of the range, a few ulps)
    assert c.min() >= 0 and c.max() <= qmax
    xh = Q.asym_dequantize(c, s, z)
    err = np.abs(x.astype(np.float64) - xh.astype(np.float64))
    slack = 4 * np.spacing(np.maximum(np.abs(x), np.abs(z)).astype(F32)).astype(np.float64)
    assert np.all(err <= s.astype(np.float64) / 2 + slack)


def test_sym_fp16_metadata_rule_and_bound():
    x = _groups(5)
    c, s = Q.sym_quantize(x, axis=1, meta16=True)
    assert np.array_equal(s.astype(np.float16).astype(F32), s)
    a = np.abs(x).max(axis=1, keepdims=True)
    assert np.array_equal(s.astype(np.float64), brute_up((np.maximum(a, F32(1e-8)) / F32(127)).astype(F32)))
    assert np.abs(c.astype(np.int32)).max() <= 127
    xh = Q.sym_dequantize(c, s)
    err = np.abs(x.astype(np.float64) - xh.astype(np.float64))
    assert np.all(err <= s.astype(np.float64) / 2 + 4 * np.spacing(np.abs(x)).astype(np.float64))


def test_fp32_metadata_unchanged_by_the_option():
    x = _groups(7)
    c0, s0, z0 = Q.asym_quantize(x, 4, axis=1)
    c1, s1, z1 = Q.asym_quantize(x, 4, axis=1, meta16=False)
    assert np.array_equal(c0, c1) and np.array_equal(s0, s1) and np.array_equal(z0, z1)
    assert np.array_equal(z0, x.min(axis=1, keepdims=True))


def test_cache_quantization_carries_the_option_per_side():
    rng = np.random.default_rng(3)
    K_ = rng.standard_normal((1, 2, 64, 128)).astype(F32)
    V_ = rng.standard_normal((1, 2, 64, 128)).astype(F32)
    k16 = OC.Spec(OC.INT_ASYM, 2, OC.PER_CHANNEL, 32, meta16=True)
    v16 = OC.Spec(OC.INT_ASYM, 2, OC.PER_TOKEN, 32, meta16=True)
    cfg = OC.Cfg(1, 4, 2, 128, k16, v16, R=32)
    st = OC.quantize_cache(cfg, K_, V_, 64)
    for side in ("k", "v"):
        for key in ("scale", "zero"):
            a = st[side][key]
            assert np.array_equal(a.astype(np.float16).astype(F32), a)
