"""The two ways the quantize kernels obtain rint of the correctly rounded fp32
quotient (x - z) / s without an IEEE division per element, checked against
correctly rounded division (numpy's float32 division: the float64 quotient
rounded to float32, which is correctly rounded because 53 >= 2 * 24 + 2).

1. Correction step (fp16-staged caches): y = RN(1 / s), q0 = RN(d y),
   r = d - s q0 (exact by FMA), q = RN(q0 + r y) equals RN(d / s).
2. Reciprocal and test (fp32-staged caches): q = RN(d rcp(s)) with rcp within
   one ulp; unless |q - rint(q)| >= 1/2 - (qmax + 1) 2^-20, rint(q) equals
   rint(RN(d / s)) after clamping to the code range.

Inputs: random quotients over the code ranges, quotients planted at
half-integers and their neighbours a few ulps away, and the values of real
groups (x at a group's exact midpoints, scale = RN(range / qmax)).
"""
from fractions import Fraction

import numpy as np

F32, F64 = np.float32, np.float64


def _rn32(fr: Fraction) -> float:
    """Round a positive Fraction to the nearest fp32 (ties to even; normal range)."""
    if fr == 0:
        return 0.0
    e = fr.numerator.bit_length() - fr.denominator.bit_length()
    while Fraction(2) ** e > fr:
        e -= 1
    while Fraction(2) ** (e + 1) <= fr:
        e += 1
    scaled = fr / Fraction(2) ** (e - 23)
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return float(Fraction(n) * Fraction(2) ** (e - 23))


def _correction_step(d, s):
    """q of rule 1, with every fp32 operation emulated in float64 and each
    float64 result either exact or rechecked exactly near an fp32 midpoint."""
    y = (F64(1) / s.astype(F64)).astype(F32)
    q0 = (d.astype(F64) * y.astype(F64)).astype(F32)                      # product exact in f64
    r = (d.astype(F64) - s.astype(F64) * q0.astype(F64)).astype(F32)      # exact difference in f64
    t = q0.astype(F64) + r.astype(F64) * y.astype(F64)
    q = t.astype(F32)
    # t may be rounded in float64: recheck exactly where it lies near an fp32 midpoint
    u = np.abs(np.nextafter(q, F32(np.inf)).astype(F64) - q.astype(F64))
    dist = np.minimum(np.abs(t - (q.astype(F64) + u / 2)), np.abs(t - (q.astype(F64) - u / 2)))
    for i in np.nonzero(dist <= 8 * np.abs(t) * 2.0 ** -52)[0]:
        exact = Fraction(float(q0[i])) + Fraction(float(r[i])) * Fraction(float(y[i]))
        q[i] = F32(_rn32(exact))
    return q


def _cases(rng, qmax, n):
    s = (rng.uniform(1, 2, n) * 2.0 ** rng.integers(-30, 16, n)).astype(F32)
    yield (s.astype(F64) * rng.uniform(0, qmax + 1, n)).astype(F32), s
    k = rng.integers(0, qmax + 1, n)
    base = ((k + 0.5) * s.astype(F64)).astype(F32)
    for step in (-3, -2, -1, 0, 1, 2, 3):
        d = base.copy()
        for _ in range(abs(step)):
            d = np.nextafter(d, F32(np.inf if step > 0 else -np.inf))
        yield d, s
    rng_v = (rng.uniform(1, 2, n) * 2.0 ** rng.integers(-12, 12, n)).astype(F32)
    sc = (rng_v.astype(F64) / qmax).astype(F32)
    j = rng.integers(0, 2 * qmax + 1, n)
    yield (rng_v.astype(F64) * j / (2 * qmax)).astype(F32), sc


def test_correction_step_is_correctly_rounded_division():
    rng = np.random.default_rng(11)
    for qmax in (3, 15, 255):
        for d, s in _cases(rng, qmax, 1 << 16):
            ref = (d.astype(F64) / s.astype(F64)).astype(F32)
            q = _correction_step(d, s)
            assert np.array_equal(q, ref), (qmax, int(np.count_nonzero(q != ref)))


def test_reciprocal_and_test_rule_gives_the_same_codes():
    rng = np.random.default_rng(12)
    for qmax in (3, 15, 255):
        m = F32((qmax + 1) * 2.0 ** -20)
        for case, (d, s) in enumerate(_cases(rng, qmax, 1 << 16)):
            ref = np.clip(np.rint((d.astype(F64) / s.astype(F64)).astype(F32)), 0, qmax)
            for ulp in (-1, 0, 1):                      # a reciprocal within one ulp either way
                rs = (F64(1) / s.astype(F64)).astype(F32)
                if ulp:
                    rs = np.nextafter(rs, F32(np.inf if ulp > 0 else -np.inf))
                q = (d.astype(F64) * rs.astype(F64)).astype(F32)
                r = np.rint(q)
                ok = np.abs((q - r).astype(F32)) < F32(0.5) - m
                got = np.where(ok, np.clip(r, 0, qmax), ref)     # rejected codes take the division
                assert np.array_equal(got, ref), (qmax, ulp)
                if case == 0:                            # random quotients: the test rarely rejects
                    assert ok.mean() > 0.99


def test_planted_mistake_fails():
    """Dropping the correction (q = RN(d y)) is not correctly rounded: the
    check above would catch a kernel that skipped it."""
    rng = np.random.default_rng(13)
    wrong = 0
    for d, s in _cases(rng, 15, 1 << 14):
        y = (F64(1) / s.astype(F64)).astype(F32)
        q0 = (d.astype(F64) * y.astype(F64)).astype(F32)
        wrong += int(np.count_nonzero(q0 != (d.astype(F64) / s.astype(F64)).astype(F32)))
    assert wrong > 0


def test_correction_step_over_the_fp8_scale_range():
    """The FP8 encoders take x / s through the same correction step, with
    per-head scales s in [2^-80, 2^80], quotients of either sign in
    [2^-17, 2^17] (below, every code is a signed zero; above, x is clamped to
    2^17 s first, where every code saturates)."""
    rng = np.random.default_rng(14)
    n = 1 << 16
    for lo, hi in ((-80, -40), (-40, 0), (0, 40), (40, 80)):
        s = (rng.uniform(1, 2, n) * 2.0 ** rng.integers(lo, hi, n)).astype(F32)
        q = rng.choice([-1.0, 1.0], n) * 2.0 ** rng.uniform(-17, 17, n)
        x = (s.astype(F64) * q).astype(F32)
        sign = np.sign(x)
        got = _correction_step(np.abs(x), s) * sign.astype(F32)
        ref = (x.astype(F64) / s.astype(F64)).astype(F32)
        assert np.array_equal(got, ref), (lo, hi)


def test_correction_step_loses_the_sign_of_zero_and_copysign_restores_it():
    """For x = -0 the correction step gives +0 (q0 = -0, r = -0 - s * -0 = +0,
    q = +0 * y + -0 = +0), while -0 / s = -0 and FP8 keeps the sign of zero
    (the E4M3 / E5M2 code of -0 is 0x80): the kernels take the sign from x."""
    s = F32(0.0105)
    y = F32(1) / s
    x = F32(-0.0)
    q0 = F32(x * y)
    r = F32(x - F32(s * q0))
    q = F32(q0 + F32(r * y))
    assert np.signbit(F32(x / s)) and not np.signbit(q)
    assert np.signbit(np.copysign(q, x))
    # copysign changes nothing for nonzero quotients: the correction never crosses zero
    rng = np.random.default_rng(15)
    xs = (rng.standard_normal(1 << 16) * 10.0 ** rng.uniform(-3, 3, 1 << 16)).astype(F32)
    ss = np.full(xs.shape, s, F32)
    q = _correction_step(np.abs(xs), ss) * np.sign(xs).astype(F32)
    assert np.array_equal(np.signbit(q), np.signbit(xs))


def test_scale_by_correction_step_with_reciprocal_of_qmax():
    """The fp16-staged append takes s = RN(range / qmax) as the correction
    step with y = RN(1 / qmax): correctly rounded for ranges in [1e-8, 2^17]
    (random ranges over the whole span, and ranges planted next to the
    quotient midpoints; the GPU probe checks every fp32 range there)."""
    rng = np.random.default_rng(16)
    n = 1 << 16
    for qmax in (3, 15, 127, 255):
        d = (2.0 ** rng.uniform(np.log2(1e-8), 17, n)).astype(F32)
        # ranges whose quotient sits next to a midpoint between two fp32 values
        qv = (2.0 ** rng.uniform(np.log2(1e-8 / qmax), np.log2(2.0 ** 17 / qmax), n)).astype(F32)
        half_ulp = (np.nextafter(qv, F32(np.inf)).astype(F64) - qv.astype(F64)) / 2
        mid = ((qv.astype(F64) + half_ulp) * qmax).astype(F32)
        for x in (d, mid, np.nextafter(mid, F32(np.inf)), np.nextafter(mid, F32(0))):
            x = x[(x >= F32(1e-8)) & (x <= F32(2.0 ** 17))]
            s = np.full(x.shape, F32(qmax))
            ref = (x.astype(F64) / F64(qmax)).astype(F32)
            assert np.array_equal(_correction_step(x, s), ref), qmax


def test_newton_reciprocal_depends_on_the_hardware_estimate():
    """One Newton step y0 + y0 (1 - s y0) from the correctly rounded 1/s gives
    it back, but from an estimate one ulp away it is not always correctly
    rounded (the all-ones significand is such a case): the kernels' use of the
    hardware reciprocal rests on the GPU probe, which checks every
    significand against the correctly rounded reciprocal."""
    from fractions import Fraction
    s = np.array([np.nextafter(F32(2.0), F32(0)) * F32(2.0) ** k for k in range(-30, 16)] +
                 [F32(1.5), F32(1.1), F32(3.0)], F32)
    ref = (F64(1) / s.astype(F64)).astype(F32)

    def step(y0):
        e = (F64(1) - s.astype(F64) * y0.astype(F64)).astype(F32)      # one rounding (exact product and sum)
        return np.array([F32(_rn32(Fraction(float(a)) + Fraction(float(b)) * Fraction(float(a))))
                         if (Fraction(float(a)) + Fraction(float(b)) * Fraction(float(a))) > 0 else F32(0)
                         for a, b in zip(y0, e)], F32)
    assert np.array_equal(step(ref), ref)
    low = np.nextafter(ref, F32(0))
    assert not np.array_equal(step(low)[:46], ref[:46])               # the all-ones significands fail from below
