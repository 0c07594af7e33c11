"""CPU oracle: exact single-query softmax attention and RoPE in fp64
(TEST INFRASTRUCTURE ONLY).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package.  It shares no code with the HIP library.

* Attention ("FP8 KV Cache Quantization: Why Keys Break Before Values",
  section "Why does the K cache break before the V cache?"; "Why Keys Are More
  Sensitive Than Values in INT8 KV Cache Quantization", section "Computational
  Paths for Key and Value"): logits_j = q . k_j / sqrt(d), p = softmax(logits),
  out = sum_j p_j v_j.  Written as the plain definition, one query head at a time.
* GQA ("KV Cache Quantization: Why Keys and Values Need Different Axes",
  section "Why does this get worse with GQA and MLA?"): query head h reads kv
  head floor(h / (Hq / Hkv)).
* RoPE (same page, section "Where does RoPE break this?"): channel pairs
  (2i, 2i+1) rotate by position * theta_i; reading taken: theta_i =
  base^(-2i/D), [a, b] -> [a cos - b sin, a sin + b cos], positions from 0.
"""
from __future__ import annotations

import numpy as np


def rope(x: np.ndarray, positions: np.ndarray, base: float) -> np.ndarray:
    """Rotate the last axis of x [..., T, D] at integer positions [T] (fp64)."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    i = np.arange(D // 2, dtype=np.float64)
    theta = np.power(float(base), -2.0 * i / D)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def single_head(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float):
    """One query [D] against K, V [T, D]; returns (out [D], logits [T]) in fp64."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    logits = (K @ q) * sm_scale
    m = logits.max()
    e = np.exp(logits - m)
    p = e / e.sum()
    return p @ V, logits


def decode_attention(q: np.ndarray, K_hat: np.ndarray, V_hat: np.ndarray, sm_scale: float,
                     pre_rope_base: float | None = None, heads=None):
    """q [B, Hq, D]; K_hat, V_hat [B, Hkv, T, D] (pre-RoPE K when pre_rope_base is
    given: rotated here at positions 0..T-1).  Returns out [B, Hq, D] fp64 for
    the requested (b, hq) pairs (all when heads is None; others left NaN)."""
    B, Hq, D = q.shape
    Hkv, T = K_hat.shape[1], K_hat.shape[2]
    n_rep = Hq // Hkv
    out = np.full((B, Hq, D), np.nan)
    todo = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else list(heads)
    rotated = {}
    for b, h in todo:
        kv = h // n_rep
        key = (b, kv)
        if key not in rotated:
            Kb = np.asarray(K_hat[b, kv], dtype=np.float64)
            if pre_rope_base is not None:
                Kb = rope(Kb, np.arange(T), pre_rope_base)
            rotated[key] = Kb
        out[b, h], _ = single_head(q[b, h], rotated[key], V_hat[b, kv], sm_scale)
    return out


def rel_l2(a: np.ndarray, ref: np.ndarray) -> float:
    """||a - ref||_2 / ||ref||_2 in fp64 (the relative output error of "FP8 KV
    Cache Quantization: Why Keys Break Before Values", section "Why does the K
    cache break before the V cache?").  inf when either side holds a non-finite
    value, or when ref is zero and a is not; 0 when both are zero."""
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if not (np.isfinite(a).all() and np.isfinite(ref).all()):
        return float("inf")
    num = float(np.linalg.norm(a - ref))
    den = float(np.linalg.norm(ref))
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den


def max_rel_l2_per_head(out: np.ndarray, ref: np.ndarray, heads=None) -> float:
    """Largest per-(sequence, query head) relative L2 error of out [B, Hq, D]
    against ref, over every pair (heads=None) or the listed (b, hq) pairs.

    A pair whose output or reference holds a NaN or an infinity counts as an
    infinite error, so an output a kernel never wrote (left NaN) fails any
    tolerance wherever it sits.  The loop keeps the running maximum explicitly
    (Python's max() would skip a NaN that is not the first element)."""
    B, Hq = ref.shape[0], ref.shape[1]
    todo = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else list(heads)
    if not todo:
        raise ValueError("no (sequence, head) pairs to compare")
    worst = 0.0
    for b, h in todo:
        e = rel_l2(out[b, h], ref[b, h])
        if not (e <= worst):        # also true for e = nan or inf
            worst = e if e == e else float("inf")
    return worst
