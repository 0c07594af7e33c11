"""Seeded synthetic inputs for the five workloads (shapes, seeds, value
distributions only).

This module holds none of the quantization or attention arithmetic: it draws
Gaussian tensors, plants the outlier channels the pages describe, and rounds
to the storage dtype of the workload (bf16 by round-to-nearest-even on the
bit pattern).  Both the CPU oracle and the GPU path consume exactly the bytes
produced here.

Workload sources (page titles and sections):
  * "FP8 KV Cache Quantization: Why Keys Break Before Values", section
    "Why does the K cache break before the V cache?" (synthetic head d=128,
    4096 tokens, channels 7, 23, 88 scaled by 20).
  * "KV Cache Quantization: Why Keys and Values Need Different Axes",
    section "Why does per-token key quantization destroy accuracy?"
    (T=512, channels 3, 17, 44, 91 scaled by 60).
  * The three serving-shaped workloads (FP8 GQA batch 16 at 8K context,
    Llama-3.1-70B-shaped INT4 at 128K, KIVI-style INT2 at 32K) use the
    head counts and context lengths the pages discuss for Llama-3.x-70B/8B.

Large workloads are drawn chunk by chunk with a counter-style seed
``default_rng((seed, tensor_id, b, h))`` so any (sequence, kv-head) chunk can
be regenerated on its own for sampled parity checks.
"""
from __future__ import annotations

import numpy as np

# tensor ids for the per-chunk seeds
_TID_K, _TID_V, _TID_Q, _TID_KNEW, _TID_VNEW, _TID_OUTLIER = 1, 2, 3, 4, 5, 6
_TID_STEP_K, _TID_STEP_V, _TID_STEP_Q = 7, 8, 9

# ----------------------------------------------------------------------------
# dtype helpers (bit-pattern conversions of generated inputs)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# Workload table.  'k'/'v' give the cache spec of each side; 'schemes' lists
# the variants a workload compares.  Dtype names: f32, bf16.
# ----------------------------------------------------------------------------

WORKLOADS = {
    # single head, symmetric absmax INT8, four K/V scheme variants
    "c1_int8_sym_single_head": dict(
        B=1, Hq=1, Hkv=1, D=128, T=4096, dtype="f32", seed=0,
        outliers=[7, 23, 88], outlier_scale=20.0,
    ),
    # single head, 4-bit asymmetric min-max, K per-token vs per-channel
    "c2_int4_asym_single_head": dict(
        B=1, Hq=1, Hkv=1, D=128, T=512, dtype="f32", seed=0,
        outliers=[3, 17, 44, 91], outlier_scale=60.0,
    ),
    # FP8 E4M3 with calibrated per-head scales, GQA 32/8, 8K context
    "c3_fp8_e4m3_gqa_8k": dict(
        B=16, Hq=32, Hkv=8, D=128, T=8192, n_new=1, dtype="bf16", seed=3,
        n_outliers=4, outlier_scale=30.0,
    ),
    # the same inputs cached as FP8 E5M2 (no scales; the FP8 page's scale-free variant)
    "c3_fp8_e5m2_gqa_8k": dict(
        B=16, Hq=32, Hkv=8, D=128, T=8192, n_new=1, dtype="bf16", seed=3,
        n_outliers=4, outlier_scale=30.0,
    ),
    # Llama-3.1-70B shaped layer: INT4 K per-channel G128 + INT4 V per-token, R=128
    "c4_int4_llama70b_128k": dict(
        B=1, Hq=64, Hkv=8, D=128, T=131072, n_new=0, dtype="bf16", seed=4,
        n_outliers=6, outlier_scale=50.0,
    ),
    # KIVI-style INT2, pre-RoPE K, R=32, GQA 32/8, 32K context, decode + append
    "c5_int2_kivi_prerope_32k": dict(
        B=32, Hq=32, Hkv=8, D=128, T=32768, n_new=1, dtype="bf16", seed=5,
        outliers=[7, 23, 88], outlier_scale=20.0, rope_base=10000.0,
    ),
}


def single_head_inputs(name: str):
    """Inputs of the two single-head workloads, drawn in the pages' order.

    Returns float32 arrays K [T, D], V [T, D], q [D] and, for the T=512
    workload, the 8 extra queries q8 [8, D] used for the logit comparison.
    The first workload reproduces the printed INT8 table of the FP8 KV cache
    page when drawn with numpy's default_rng(0) in this order.
    """
    w = WORKLOADS[name]
    rng = np.random.default_rng(w["seed"])
    T, D = w["T"], w["D"]
    K = rng.standard_normal((T, D))
    V = rng.standard_normal((T, D))
    q = rng.standard_normal(D)
    extra = rng.standard_normal((8, D)) if name.startswith("c2") else None
    K[:, w["outliers"]] *= w["outlier_scale"]
    out = dict(K=K.astype(np.float32), V=V.astype(np.float32), q=q.astype(np.float32))
    if extra is not None:
        out["q8"] = extra.astype(np.float32)
    return out


def outlier_channels(name: str) -> np.ndarray:
    """[Hkv, n] outlier channel indices, fixed per kv head for the whole run."""
    w = WORKLOADS[name]
    if "outliers" in w:
        return np.tile(np.asarray(w["outliers"], dtype=np.int64), (w["Hkv"], 1))
    rng = np.random.default_rng((w["seed"], _TID_OUTLIER))
    return np.stack([rng.choice(w["D"], size=w["n_outliers"], replace=False)
                     for _ in range(w["Hkv"])]).astype(np.int64)


def _chunk(seed, tid, b, h, shape):
    return np.random.default_rng((seed, tid, b, h)).standard_normal(shape, dtype=np.float32)


def kv_chunk(name: str, b: int, h: int, which: str, t_begin: int = 0, n: int | None = None):
    """bf16 bits [n, D] of the prefill K or V chunk of (sequence b, kv head h).

    Keys carry the fixed outlier channels of head h.  The full chunk is drawn
    (so sub-ranges stay consistent) and then sliced.
    """
    w = WORKLOADS[name]
    T, D = w["T"], w["D"]
    x = _chunk(w["seed"], _TID_K if which == "k" else _TID_V, b, h, (T, D))
    if which == "k":
        x[:, outlier_channels(name)[h]] *= np.float32(w["outlier_scale"])
    n = T - t_begin if n is None else n
    return f32_to_bf16_bits(x[t_begin:t_begin + n])


def new_token_chunk(name: str, b: int, h: int, which: str):
    """bf16 bits [n_new, D] of the decode-time appended token(s) of (b, h)."""
    w = WORKLOADS[name]
    x = _chunk(w["seed"], _TID_KNEW if which == "k" else _TID_VNEW, b, h, (w["n_new"], w["D"]))
    if which == "k":
        x[:, outlier_channels(name)[h]] *= np.float32(w["outlier_scale"])
    return f32_to_bf16_bits(x)


def step_tokens(name: str, b: int, h: int, which: str, first: int, n: int) -> np.ndarray:
    """bf16 bits [n, D] of decode steps first .. first+n-1 of (b, h): the token
    appended at step i is drawn from its own seed (keys carry the head's fixed
    outlier channels), so any step can be regenerated alone."""
    w = WORKLOADS[name]
    rows = []
    for i in range(first, first + n):
        x = np.random.default_rng((w["seed"], _TID_STEP_K if which == "k" else _TID_STEP_V, b, h, i)) \
            .standard_normal((1, w["D"]), dtype=np.float32)
        if which == "k":
            x[:, outlier_channels(name)[h]] *= np.float32(w["outlier_scale"])
        rows.append(x)
    return f32_to_bf16_bits(np.concatenate(rows) if rows else np.zeros((0, w["D"]), np.float32))


def step_tokens_all(name: str, which: str, step: int) -> np.ndarray:
    """bf16 bits [B, Hkv, 1, D] of decode step ``step`` for every (b, h)."""
    w = WORKLOADS[name]
    out = np.empty((w["B"], w["Hkv"], 1, w["D"]), dtype=np.uint16)
    for b in range(w["B"]):
        for h in range(w["Hkv"]):
            out[b, h] = step_tokens(name, b, h, which, step, 1)
    return out


def step_query(name: str, step: int) -> np.ndarray:
    """bf16 bits [B, Hq, D] of the query of decode step ``step``."""
    w = WORKLOADS[name]
    x = np.random.default_rng((w["seed"], _TID_STEP_Q, step)).standard_normal((w["B"], w["Hq"], w["D"]),
                                                                            dtype=np.float32)
    return f32_to_bf16_bits(x)


def query(name: str) -> np.ndarray:
    """bf16 bits [B, Hq, D] of the decode query (already rotated when keys are pre-RoPE)."""
    w = WORKLOADS[name]
    x = np.random.default_rng((w["seed"], _TID_Q)).standard_normal((w["B"], w["Hq"], w["D"]),
                                                                   dtype=np.float32)
    return f32_to_bf16_bits(x)


def full_prefill(name: str, which: str, threads: int = 8) -> np.ndarray:
    """bf16 bits [B, Hkv, T, D] of the whole prefill K or V (large: 2 bytes/element).
    Chunks are independent streams, drawn on a few threads."""
    from concurrent.futures import ThreadPoolExecutor
    w = WORKLOADS[name]
    out = np.empty((w["B"], w["Hkv"], w["T"], w["D"]), dtype=np.uint16)

    def fill(bh):
        b, h = divmod(bh, w["Hkv"])
        out[b, h] = kv_chunk(name, b, h, which)

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(fill, range(w["B"] * w["Hkv"])))
    return out


def full_new_tokens(name: str, which: str) -> np.ndarray:
    w = WORKLOADS[name]
    out = np.empty((w["B"], w["Hkv"], w["n_new"], w["D"]), dtype=np.uint16)
    for b in range(w["B"]):
        for h in range(w["Hkv"]):
            out[b, h] = new_token_chunk(name, b, h, which)
    return out


def random_case(seed: int, B: int, Hkv: int, T: int, D: int, n_outliers: int = 3,
                outlier_scale: float = 20.0, dtype: str = "f32"):
    """Small random K, V [B, Hkv, T, D] with fixed outlier channels, for parity sweeps.

    Returns (K, V) as float32 arrays whose values are exactly representable in
    ``dtype`` (f32, bf16 or f16), plus the raw device-dtype payloads.
    """
    rng = np.random.default_rng((seed, 77))
    K = rng.standard_normal((B, Hkv, T, D), dtype=np.float32)
    V = rng.standard_normal((B, Hkv, T, D), dtype=np.float32)
    for h in range(Hkv):
        ch = rng.choice(D, size=min(n_outliers, D), replace=False)
        K[:, h][..., ch] *= np.float32(outlier_scale)
    return _as_dtype(K, dtype), _as_dtype(V, dtype)


def sink_case(seed: int, B: int, Hq: int, Hkv: int, T: int, D: int, sink_channel: int = 5,
              sink_value: float = 1300.0, q_sink: float = 0.1, outlier_scale: float = 5.0,
              dtype: str = "bf16"):
    """K, V [B, Hkv, T, D] and q [B, Hq, D] with a planted attention-sink key.

    Keys and values are N(0, 1) with three outlier channels (x outlier_scale)
    per kv head, as in ``random_case``; token 0 of every (sequence, kv head)
    is an attention sink whose key has ``sink_value`` in ``sink_channel``,
    beyond E4M3's +-448 at unit scale (the FP8 page's section "Why do
    per-tensor scales waste bits on the K cache?": sinks carry keys with
    outsized norms).  Every query has +``q_sink`` in that channel, so the sink
    takes most of the attention mass; the outlier channels avoid it.
    Returns ((K, K payload), (V, V payload), (q, q payload))."""
    rng = np.random.default_rng((seed, 79))
    K = rng.standard_normal((B, Hkv, T, D), dtype=np.float32)
    V = rng.standard_normal((B, Hkv, T, D), dtype=np.float32)
    for h in range(Hkv):
        ch = rng.choice([c for c in range(D) if c != sink_channel], size=3, replace=False)
        K[:, h][..., ch] *= np.float32(outlier_scale)
    K[:, :, 0, sink_channel] = np.float32(sink_value)
    q = rng.standard_normal((B, Hq, D), dtype=np.float32)
    q[:, :, sink_channel] = np.float32(q_sink)
    return _as_dtype(K, dtype), _as_dtype(V, dtype), _as_dtype(q, dtype)


def rope_study_case(seed: int, B: int, Hq: int, Hkv: int, T: int, D: int,
                    outliers=(3, 17, 44, 91), magnitude: float = 20.0, consistent: bool = True):
    """fp32 K, V [B, Hkv, T, D] and q [B, Hq, D] (N(0, 1)) with outlier key
    channels for the pre- vs post-RoPE study ("KV Cache Quantization: Why Keys
    and Values Need Different Axes", section "Where does RoPE break this?").

    consistent=True: each outlier channel is +-magnitude + N(0, 1) with a sign
    fixed per (kv head, channel): "the same channel is always huge".
    consistent=False: the outlier channels are N(0, 1) * magnitude, the
    random-sign scaling of the page's own listing."""
    rng = np.random.default_rng((seed, 80, int(consistent)))
    K = rng.standard_normal((B, Hkv, T, D), dtype=np.float32)
    V = rng.standard_normal((B, Hkv, T, D), dtype=np.float32)
    for h in range(Hkv):
        for c in outliers:
            if consistent:
                sgn = np.float32(1.0 if rng.random() < 0.5 else -1.0)
                K[:, h, :, c] = sgn * np.float32(magnitude) + K[:, h, :, c]
            else:
                K[:, h, :, c] *= np.float32(magnitude)
    q = rng.standard_normal((B, Hq, D), dtype=np.float32)
    return K, V, q


def edge_case_inputs(seed: int, B: int, Hkv: int, T: int, D: int, bits: int, big: bool = False):
    """fp32 K, V [B, Hkv, T, D] whose quantization groups hit the encoders'
    corner cases, planted over N(0, 1) background values.  Every planted value
    is an fp16 number (so staging through an fp16 window keeps it), except
    with big=True, which plants values beyond +-65504 (for caches without a
    window).  Keys (per-channel groups along tokens) get, per channel:
      0  the constant 3.0 (max - min = 0: the range floor decides the scale),
      1  -0.0 everywhere (a constant group whose minimum is negative zero),
      2  tiny values j * 2^-24 (fp16 subnormals; a scale far below fp16's
         normal range),
      3  exact half-way ties: 0 and 2^bits - 1 in every group of 32 tokens
         plus k + 1/2 elsewhere, so (x - min) / scale lands on k + 1/2,
      4  -0.0 and 0.0 mixed with 1, 2, 3,
      5  big=True: +-1e5 and 7e4 (beyond fp16), else large fp16 values +-6e4.
    Values (per-token groups along channels) get the same patterns along the
    channels of tokens 0..5 of every 32-token block."""
    rng = np.random.default_rng((seed, 81))
    K = rng.standard_normal((B, Hkv, T, D), dtype=np.float32)
    V = rng.standard_normal((B, Hkv, T, D), dtype=np.float32)
    qmax = float(2 ** bits - 1)

    def pattern(n, kind):
        j = np.arange(n)
        if kind == 0:
            return np.full(n, 3.0)
        if kind == 1:
            return np.full(n, -0.0)
        if kind == 2:
            return (j % 29 + 1) * 2.0 ** -24
        if kind == 3:
            v = (j % int(qmax)) + 0.5
            v[j % 32 == 0] = 0.0
            v[j % 32 == 1] = qmax
            return v
        if kind == 4:
            return np.array([-0.0, 0.0, 1.0, 2.0, 3.0, -0.0, 0.0])[j % 7]
        if big:
            return np.array([1e5, -1e5, 7e4, 2.0, -3.0])[j % 5]
        return np.array([6e4, -6e4, 0.5, 1.0])[j % 4]

    for kind in range(6):
        K[:, :, :, kind] = pattern(T, kind).astype(np.float32)
        for t0 in range(0, T, 32):
            if t0 + kind < T:
                V[:, :, t0 + kind, :] = pattern(D, kind).astype(np.float32)
    return K, V


def random_queries(seed: int, B: int, Hq: int, D: int, dtype: str = "f32"):
    rng = np.random.default_rng((seed, 78))
    return _as_dtype(rng.standard_normal((B, Hq, D), dtype=np.float32), dtype)


def _as_dtype(x: np.ndarray, dtype: str):
    """Return (float32 values, raw payload array in the device dtype)."""
    if dtype == "f32":
        x = np.ascontiguousarray(x, dtype=np.float32)
        return x, x
    if dtype == "bf16":
        bits = f32_to_bf16_bits(x)
        return bf16_bits_to_f32(bits), bits
    if dtype == "f16":
        h = x.astype(np.float16)
        return h.astype(np.float32), h
    raise ValueError(dtype)
