"""CPU oracle: element quantizers (TEST INFRASTRUCTURE ONLY).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package.  It shares no code with the HIP library and never calls it.

Every routine works in IEEE fp32 with one rounding per operation, in the order
the pages' quantize-dequantize recipes state them (numpy never fuses a
multiply-add, and numpy's float32 division and rint are correctly rounded,
ties to even):

* asymmetric min-max, b bits ("KV Cache Quantization: Why Keys and Values Need
  Different Axes", section "Why does per-token key quantization destroy
  accuracy?", the quant_dequant listing): qmax = 2^b - 1,
  scale = max(max - min, 1e-8) / qmax, code = clamp(round((x - min)/scale),
  0, qmax), x_hat = code * scale + min;
* symmetric absmax INT8 ("FP8 KV Cache Quantization: Why Keys Break Before
  Values", section "Why does the K cache break before the V cache?", the
  qint8 listing): scale = absmax / 127, code = clamp(round(x/scale), -127,
  127), x_hat = code * scale;
* FP8 E4M3 (same page, section "Why do per-tensor scales waste bits on the K
  cache?": 3 mantissa bits, saturation at +-448): encoded here by an explicit
  nearest-point search over the 254 finite code points, ties to the even code.
* FP8 E5M2 (same section: 2 mantissa bits, saturation at +-57344; the section
  "How do you configure asymmetric KV cache quantization?" adds that it needs
  no scales): OCP E5M2, bias 15, the same nearest-point search over its
  246 finite code points, applied to the value itself (unit scale).
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
EPS = F32(1e-8)          # floor on (max - min) of the min-max listing; reused for absmax
E4M3_MAX = 448.0
E5M2_MAX = 57344.0


def stage(x: np.ndarray, through_fp16: bool) -> np.ndarray:
    """Cache staging of an input value: fp32, and rounded through fp16 (RNE)
    when the cache keeps a full-precision fp16 window of recent tokens."""
    x = np.asarray(x, dtype=F32)
    if through_fp16:
        return x.astype(np.float16).astype(F32)
    return x


# ----------------------------------------------------------------------------
# asymmetric min-max (scale + zero-point = group minimum)
# ----------------------------------------------------------------------------

F16_MAX = F32(65504.0)


def f16_toward(x, up: bool) -> np.ndarray:
    """The fp16 value next to fp32 ``x`` on the side of +inf (up) or -inf
    (down), returned as fp32, saturated at +-65504 (fp16 storage of a scale or
    zero-point that must not shrink the range it covers)."""
    x = np.asarray(x, dtype=F32)
    with np.errstate(over="ignore"):    # beyond +-65504: saturated below
        h = x.astype(np.float16)
        hf = h.astype(F32)
        wrong = (hf < x) if up else (hf > x)
        h = np.where(wrong, np.nextafter(h, np.float16(np.inf if up else -np.inf)), h)
    return np.clip(h.astype(F32), -F16_MAX, F16_MAX).astype(F32)


def asym_quantize(x: np.ndarray, bits: int, axis, meta16: bool = False):
    """Quantize fp32 ``x`` with one (scale, zero) per reduction over ``axis``.

    Returns (codes uint8, scale fp32, zero fp32) with scale/zero keeping the
    reduced dims (keepdims=True) so they broadcast against ``x``.

    meta16: the scale and zero-point are stored in fp16.  The zero-point is the
    group minimum rounded toward -inf and the scale is computed from it and
    rounded toward +inf, so the stored grid still covers [min, max] and the
    reconstruction error stays within half the stored scale; codes are then
    taken against the stored values.
    """
    x = np.asarray(x, dtype=F32)
    qmax = F32(2 ** bits - 1)
    mn = x.min(axis=axis, keepdims=True)
    mx = x.max(axis=axis, keepdims=True)
    z = f16_toward(mn, up=False) if meta16 else mn
    d = np.maximum((mx - z).astype(F32), EPS)
    s = (d / qmax).astype(F32)
    if meta16:
        s = f16_toward(s, up=True)
    t = ((x - z).astype(F32) / s).astype(F32)
    codes = np.clip(np.rint(t), F32(0), qmax).astype(np.uint8)
    # -0.0 vs 0.0 min is irrelevant for codes; keep the min as stored zero-point
    return codes, s, z.astype(F32)


def asym_dequantize(codes: np.ndarray, scale: np.ndarray, zero: np.ndarray) -> np.ndarray:
    """x_hat = fl(fl(code * scale) + zero): two roundings, no fused multiply-add."""
    prod = (codes.astype(F32) * scale).astype(F32)
    return (prod + zero).astype(F32)


# ----------------------------------------------------------------------------
# symmetric absmax INT8
# ----------------------------------------------------------------------------

def sym_quantize(x: np.ndarray, axis, meta16: bool = False):
    """Symmetric INT8 with scale = max(absmax, 1e-8) / 127 and codes in [-127, 127]
    (meta16: the scale stored in fp16, rounded toward +inf)."""
    x = np.asarray(x, dtype=F32)
    a = np.abs(x).max(axis=axis, keepdims=True)
    s = (np.maximum(a, EPS) / F32(127.0)).astype(F32)
    if meta16:
        s = f16_toward(s, up=True)
    t = (x / s).astype(F32)
    codes = np.clip(np.rint(t), F32(-127), F32(127)).astype(np.int8)
    return codes, s


def sym_dequantize(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    return (codes.astype(F32) * scale).astype(F32)


# ----------------------------------------------------------------------------
# FP8 E4M3 (OCP "FN" variant: bias 7, no infinities, S.1111.111 = NaN)
# ----------------------------------------------------------------------------

def e4m3_value_of_code(code) -> np.ndarray:
    """Closed-form value of E4M3 code bytes (float64; NaN for 0x7F / 0xFF)."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def _e4m3_grid():
    codes = np.arange(0x7F, dtype=np.int64)             # 0x00 .. 0x7E (0x7F is NaN)
    vals = e4m3_value_of_code(codes)
    assert np.all(np.diff(vals) > 0)
    return codes, vals


_GRID_CODES, _GRID_VALS = _e4m3_grid()


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """Encode fp32 values to E4M3 bytes: saturate to +-448, then round to the
    nearest representable magnitude with ties to the even code; the sign bit
    is kept (so -0.0 -> 0x80).  Inputs are assumed finite."""
    y = np.asarray(y, dtype=F32)
    a = np.minimum(np.abs(y).astype(np.float64), E4M3_MAX)
    hi = np.searchsorted(_GRID_VALS, a, side="left")        # first grid value >= a
    hi = np.clip(hi, 0, len(_GRID_VALS) - 1)
    lo = np.clip(hi - 1, 0, len(_GRID_VALS) - 1)
    d_hi = _GRID_VALS[hi] - a
    d_lo = a - _GRID_VALS[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & ((_GRID_CODES[lo] & 1) == 0))
    mag_code = np.where(pick_lo, _GRID_CODES[lo], _GRID_CODES[hi])
    mag_code = np.where(a == _GRID_VALS[hi], _GRID_CODES[hi], mag_code)
    sign = np.signbit(y).astype(np.int64) << 7
    return (mag_code | sign).astype(np.uint8)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """E4M3 bytes -> float32 (exact)."""
    return e4m3_value_of_code(codes).astype(F32)


def fp8_scale_from_absmax(absmax) -> np.ndarray:
    """Calibrated scale = absmax / 448 (fp32 division); 1.0 when absmax is 0
    (the unit-scale fallback of an uncalibrated cache)."""
    a = np.asarray(absmax, dtype=F32)
    s = (a / F32(E4M3_MAX)).astype(F32)
    return np.where(a == 0, F32(1.0), s).astype(F32)


def fp8_quantize(x: np.ndarray, scale) -> np.ndarray:
    """code = E4M3(fl(x / scale)) with saturation."""
    y = (np.asarray(x, dtype=F32) / np.asarray(scale, dtype=F32)).astype(F32)
    return e4m3_encode(y)


def fp8_dequantize(codes: np.ndarray, scale) -> np.ndarray:
    return (e4m3_decode(codes) * np.asarray(scale, dtype=F32)).astype(F32)


# ----------------------------------------------------------------------------
# FP8 E5M2 (OCP: bias 15, exponent field 31 = infinities and NaNs)
# ----------------------------------------------------------------------------

def e5m2_value_of_code(code) -> np.ndarray:
    """Closed-form value of E5M2 code bytes (float64; +-inf for 0x7C / 0xFC,
    NaN for 0x7D-0x7F / 0xFD-0xFF)."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 2) & 0x1F
    m = c & 0x3
    mag = np.where(e == 0, (m / 4.0) * 2.0 ** -14, (1.0 + m / 4.0) * np.exp2(e - 15.0))
    mag = np.where(e == 31, np.where(m == 0, np.inf, np.nan), mag)
    return sign * mag


def _e5m2_grid():
    codes = np.arange(0x7C, dtype=np.int64)             # 0x00 .. 0x7B (0x7C is +inf)
    vals = e5m2_value_of_code(codes)
    assert np.all(np.diff(vals) > 0)
    return codes, vals


_GRID5_CODES, _GRID5_VALS = _e5m2_grid()


def e5m2_encode(y: np.ndarray) -> np.ndarray:
    """Encode fp32 values to E5M2 bytes: saturate to +-57344, then round to
    the nearest representable magnitude with ties to the even code; the sign
    bit is kept (-0.0 -> 0x80).  Inputs are assumed finite."""
    y = np.asarray(y, dtype=F32)
    a = np.minimum(np.abs(y).astype(np.float64), E5M2_MAX)
    hi = np.searchsorted(_GRID5_VALS, a, side="left")
    hi = np.clip(hi, 0, len(_GRID5_VALS) - 1)
    lo = np.clip(hi - 1, 0, len(_GRID5_VALS) - 1)
    d_hi = _GRID5_VALS[hi] - a
    d_lo = a - _GRID5_VALS[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & ((_GRID5_CODES[lo] & 1) == 0))
    mag_code = np.where(pick_lo, _GRID5_CODES[lo], _GRID5_CODES[hi])
    mag_code = np.where(a == _GRID5_VALS[hi], _GRID5_CODES[hi], mag_code)
    sign = np.signbit(y).astype(np.int64) << 7
    return (mag_code | sign).astype(np.uint8)


def e5m2_decode(codes: np.ndarray) -> np.ndarray:
    """E5M2 bytes -> float32 (exact)."""
    return e5m2_value_of_code(codes).astype(F32)
