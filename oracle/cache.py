"""CPU oracle: whole-cache quantization and byte layout (TEST INFRASTRUCTURE ONLY).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package.  It shares no code with the HIP library.

What it computes, per (sequence, kv head) unless stated:

* The residual split.  "KV Cache Quantization: Why Keys and Values Need
  Different Axes", section "What should I actually turn on in production?",
  asks for a full-precision window of the most recent tokens, folded into the
  quantized cache in blocks; "FP8 KV Cache Quantization: Why Keys Break Before
  Values", section "Should you quantize keys pre-RoPE or post-RoPE?", explains
  why per-channel groups force block-wise appends.  Reading taken: with G_t the
  token-group size of a finite per-channel group (1 otherwise) and R the window,
  the first Tq(T) = G_t * floor(max(T - R, 0) / G_t) tokens are quantized and the
  rest stay in fp16.  Every token is staged through fp16 when such a window
  exists (R > 0 or G_t > 1).
* Grouping axes (same pages, "Why do per-tensor scales waste bits on the K
  cache?" and "Why does per-token key quantization destroy accuracy?"):
  per-tensor = one group per (sequence, kv head); per-channel = one group per
  channel over G consecutive tokens from position 0 (G = 0: all tokens);
  per-token = one group per token over Gc consecutive channels (Gc = 0: all).
* FP8 E4M3: one scale per kv head, absmax / 448 over the first call's tokens
  of all sequences (calibrated) or a caller-supplied / unit scale.
* FP8 E5M2: no scales (unit scale per kv head).

It also writes the documented byte layout of codes (K rows, V 32-token
blocks, fp16 ring) so tests can compare the library's cache bytes directly.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import quant as Q

NONE, INT_ASYM, INT_SYM, FP8_E4M3, FP8_E5M2 = 0, 1, 2, 3, 4
PER_TENSOR, PER_CHANNEL, PER_TOKEN = 0, 1, 2
VBLOCK = 32          # tokens per V code block
RING_ALIGN = 32      # ring slots are a multiple of this


@dataclass
class Spec:
    scheme: int
    bits: int = 8
    axis: int = PER_CHANNEL
    group: int = 0
    meta16: bool = False    # INT scale / zero-point stored in fp16 (quant.asym_quantize)


@dataclass
class Cfg:
    B: int
    Hq: int
    Hkv: int
    D: int
    k: Spec
    v: Spec
    R: int = 0
    pre_rope_k: bool = False
    rope_base: float = 10000.0
    extra: dict = field(default_factory=dict)

    @property
    def n_rep(self):
        return self.Hq // self.Hkv


def token_group(cfg: Cfg) -> int:
    """G_t: tokens per block that must be quantized together (1 = any token)."""
    g = 1
    for s in (cfg.k, cfg.v):
        if s.scheme in (INT_ASYM, INT_SYM) and s.axis == PER_CHANNEL and s.group > 0:
            g = s.group
    return g


def one_shot(cfg: Cfg) -> bool:
    """True when a group spans the whole token axis (per-tensor or per-channel G=0)."""
    for s in (cfg.k, cfg.v):
        if s.scheme in (INT_ASYM, INT_SYM) and (s.axis == PER_TENSOR or
                                                (s.axis == PER_CHANNEL and s.group == 0)):
            return True
    return False


def has_window(cfg: Cfg) -> bool:
    return cfg.R > 0 or token_group(cfg) > 1


def quantized_tokens(cfg: Cfg, T: int) -> int:
    if one_shot(cfg):
        return T
    g = token_group(cfg)
    return g * (max(T - cfg.R, 0) // g)


def ring_slots(cfg: Cfg) -> int:
    if not has_window(cfg):
        return 0
    n = cfg.R + token_group(cfg)
    return -(-n // RING_ALIGN) * RING_ALIGN


# ----------------------------------------------------------------------------
# quantization of one tensor's quantized part  x: [B, H, Tq, D] (staged fp32)
# ----------------------------------------------------------------------------

def quantize_part(x: np.ndarray, spec: Spec, fp8_scale=None):
    """Returns dict(codes, scale, zero, deq).  Shapes of scale/zero:
    per-tensor [B,H,1,1]; per-channel [B,H,ng,D]; per-token [B,H,Tq,D/Gc];
    FP8: scale [H].  codes [B,H,Tq,D] (uint8 / int8 / float16 / float32)."""
    B, H, T, D = x.shape
    if spec.scheme == NONE:
        if spec.bits == 16:
            c = x.astype(np.float16)
            return dict(codes=c, scale=None, zero=None, deq=c.astype(np.float32))
        return dict(codes=x.copy(), scale=None, zero=None, deq=x.copy())
    if spec.scheme == FP8_E4M3:
        s = np.asarray(fp8_scale, dtype=np.float32).reshape(1, H, 1, 1)
        codes = Q.fp8_quantize(x, s)
        return dict(codes=codes, scale=s.reshape(H), zero=None, deq=Q.fp8_dequantize(codes, s))
    if spec.scheme == FP8_E5M2:
        # no scales: the value itself is encoded (unit scale per kv head)
        codes = Q.e5m2_encode(x)
        return dict(codes=codes, scale=np.ones(H, dtype=np.float32), zero=None, deq=Q.e5m2_decode(codes))

    if spec.axis == PER_TENSOR:
        xg = x.reshape(B, H, 1, T * D)
        red = 3
    elif spec.axis == PER_CHANNEL:
        G = spec.group if spec.group > 0 else T
        assert T % G == 0
        xg = x.reshape(B, H, T // G, G, D)
        red = 3
    else:  # PER_TOKEN
        Gc = spec.group if spec.group > 0 else D
        xg = x.reshape(B, H, T, D // Gc, Gc)
        red = 4
    if spec.scheme == INT_ASYM:
        c, s, z = Q.asym_quantize(xg, spec.bits, axis=red, meta16=spec.meta16)
        deq = Q.asym_dequantize(c, s, z)
    else:
        c, s = Q.sym_quantize(xg, axis=red, meta16=spec.meta16)
        z = None
        deq = Q.sym_dequantize(c, s)
    s = np.squeeze(s, axis=red)
    z = None if z is None else np.squeeze(z, axis=red)
    if spec.axis == PER_TENSOR:
        s = s.reshape(B, H, 1, 1)
        z = None if z is None else z.reshape(B, H, 1, 1)
    return dict(codes=c.reshape(B, H, T, D), scale=s, zero=z, deq=deq.reshape(B, H, T, D))


def fp8_calibrate(x_first_call: np.ndarray) -> np.ndarray:
    """Per-kv-head scale = absmax over (sequence, token, channel) / 448."""
    a = np.abs(np.asarray(x_first_call, dtype=np.float32)).max(axis=(0, 2, 3))
    return Q.fp8_scale_from_absmax(a)


def quantize_cache(cfg: Cfg, K: np.ndarray, V: np.ndarray, T: int,
                   k_scale=None, v_scale=None, calibrate_tokens: int = 0):
    """Oracle state of a cache holding tokens [0, T) of K, V ([B, Hkv, >=T, D] fp32
    input values).

    ``calibrate_tokens`` > 0 computes FP8 scales from tokens [0, calibrate_tokens)
    (the first call's input); otherwise k_scale / v_scale (arrays [Hkv]) or the
    unit scale are used.  Returns a dict with Tq, per-tensor parts, fp16 window
    rows and the full dequantized K_hat, V_hat [B, Hkv, T, D] fp32 (pre-RoPE).
    """
    win = has_window(cfg)
    Ks = Q.stage(K[:, :, :T], win)
    Vs = Q.stage(V[:, :, :T], win)
    Tq = quantized_tokens(cfg, T)
    H = cfg.Hkv
    scales = {}
    for name, xs, spec, given in (("k", Ks, cfg.k, k_scale), ("v", Vs, cfg.v, v_scale)):
        if spec.scheme == FP8_E4M3:
            if calibrate_tokens > 0:
                scales[name] = fp8_calibrate(xs[:, :, :calibrate_tokens])
            elif given is not None:
                scales[name] = np.asarray(given, dtype=np.float32).reshape(H)
            else:
                scales[name] = np.ones(H, dtype=np.float32)
        else:
            scales[name] = None
    out = dict(Tq=Tq, T=T)
    for name, xs, spec in (("k", Ks, cfg.k), ("v", Vs, cfg.v)):
        part = quantize_part(xs[:, :, :Tq], spec, scales[name])
        full = np.concatenate([part["deq"], xs[:, :, Tq:]], axis=2)
        out[name] = part
        out[name + "_hat"] = full
        out[name + "_window"] = xs[:, :, Tq:].astype(np.float16)
    return out


# ----------------------------------------------------------------------------
# byte layout
# ----------------------------------------------------------------------------

def code_bits(spec: Spec) -> int:
    if spec.scheme == NONE:
        return spec.bits
    if spec.scheme in (FP8_E4M3, FP8_E5M2, INT_SYM):
        return 8
    return spec.bits


def _code_bytes_le(codes: np.ndarray, bits: int) -> np.ndarray:
    """Raw unsigned integer code fields for packing (uint8 / uint16 / uint32 views)."""
    if bits == 16:
        return codes.astype(np.float16).view(np.uint16)
    if bits == 32:
        return codes.astype(np.float32).view(np.uint32)
    return codes.view(np.uint8) if codes.dtype == np.int8 else codes.astype(np.uint8)


def pack_rows(codes: np.ndarray, bits: int) -> np.ndarray:
    """Token-row layout of K: each token's D codes packed along the channel axis,
    8/b codes per byte, channel c at bit b*(c mod 8/b), low bits first; 16/32-bit
    values stored little-endian.  codes [..., T, D] -> uint8 [..., T, D*b/8]."""
    u = _code_bytes_le(codes, bits)
    if bits >= 8:
        # row width given explicitly so that zero tokens give a [..., 0, D*b/8] array
        return np.ascontiguousarray(u).view(np.uint8).reshape(*u.shape[:-1], u.shape[-1] * (bits // 8))
    per = 8 // bits
    g = u.reshape(*u.shape[:-1], u.shape[-1] // per, per).astype(np.uint16)
    acc = np.zeros(g.shape[:-1], dtype=np.uint16)
    for r in range(per):
        acc |= g[..., r] << (bits * r)
    return acc.astype(np.uint8)


def pack_vblocks(codes: np.ndarray, bits: int) -> np.ndarray:
    """V layout: 32-token blocks.  Token t = 32*blk + 8*g + k, channel c = 16*i + n.
    Inside a block, lane l = 16*g + n owns a contiguous run of D/16 words; word i
    holds the 8 codes k = 0..7 of channel c for tokens 8g..8g+7, code k at bit
    offset k*b (little-endian).  A word is 8*b bits.  Tokens past the end of
    ``codes`` in the last block are zero.  codes [..., T, D] -> uint8
    [..., nblk, 32*D*b/8]."""
    u = _code_bytes_le(codes, bits)
    *lead, T, D = u.shape
    nblk = -(-T // VBLOCK)
    if nblk == 0:
        return np.zeros((*lead, 0, VBLOCK * D * bits // 8), dtype=np.uint8)
    pad = nblk * VBLOCK - T
    if pad:
        u = np.concatenate([u, np.zeros((*lead, pad, D), dtype=u.dtype)], axis=-2)
    # [..., blk, g, k, i, n] -> [..., blk, g, n, i, k]
    u = u.reshape(*lead, nblk, 4, 8, D // 16, 16)
    nl = len(lead)
    perm = list(range(nl)) + [nl, nl + 1, nl + 4, nl + 3, nl + 2]
    w = np.ascontiguousarray(u.transpose(perm))          # words of 8 codes
    if bits >= 8:
        b = w.view(np.uint8)
        return b.reshape(*lead, nblk, -1)
    per = 8 // bits
    wb = w.reshape(*w.shape[:-1], 8 // per, per).astype(np.uint16)
    acc = np.zeros(wb.shape[:-1], dtype=np.uint16)
    for r in range(per):
        acc |= wb[..., r] << (bits * r)
    return acc.astype(np.uint8).reshape(*lead, nblk, -1)


def unpack_vblocks(blocks: np.ndarray, bits: int, D: int, T: int) -> np.ndarray:
    """Inverse of pack_vblocks: uint8 [..., nblk, bytes] -> code fields [..., T, D]
    (uint8 for b <= 8, uint16 / uint32 raw bits for 16 / 32)."""
    *lead, nblk, nbytes = blocks.shape
    if bits == 16:
        w = np.ascontiguousarray(blocks).view(np.uint16)
    elif bits == 32:
        w = np.ascontiguousarray(blocks).view(np.uint32)
    elif bits == 8:
        w = blocks
    else:
        per = 8 // bits
        mask = (1 << bits) - 1
        w = np.stack([(blocks >> (bits * r)) & mask for r in range(per)], axis=-1)
    w = w.reshape(*lead, nblk, 4, 16, D // 16, 8)        # [blk, g, n, i, k]
    nl = len(lead)
    perm = list(range(nl)) + [nl, nl + 1, nl + 4, nl + 3, nl + 2]  # -> [blk, g, k, i, n]
    c = w.transpose(perm).reshape(*lead, nblk * VBLOCK, D)
    return c[..., :T, :]


def window_slots(cfg: Cfg, Tq: int, T: int) -> np.ndarray:
    """Ring slot of each window token t in [Tq, T): t mod ring_slots."""
    rs = ring_slots(cfg)
    return np.arange(Tq, T) % rs if rs else np.zeros(0, dtype=np.int64)


def cache_bytes_per_token(layers: int, kv_heads: int, head_dim: int, dtype_bytes: float) -> float:
    """bytes/token = 2 (K and V) * layers * kv_heads * head_dim * dtype_bytes
    ("KV Cache Quantization: Why Keys and Values Need Different Axes", section
    "Why is the KV cache the thing that actually runs out of memory?")."""
    return 2 * layers * kv_heads * head_dim * dtype_bytes


def dequantize_part(part: dict, spec: Spec) -> np.ndarray:
    """Rebuild x_hat [B, H, Tq, D] from a quantize_part result's codes and
    (scale, zero) alone, by the same element rules (used to time a decode step
    of the oracle from stored codes)."""
    codes = part["codes"]
    B, H, T, D = codes.shape
    if spec.scheme == NONE:
        return codes.astype(np.float32)
    if spec.scheme == FP8_E4M3:
        return Q.fp8_dequantize(codes, part["scale"].reshape(1, H, 1, 1))
    if spec.scheme == FP8_E5M2:
        return Q.e5m2_decode(codes)
    s, z = part["scale"], part["zero"]
    if spec.axis == PER_TENSOR:
        sb = s.reshape(B, H, 1, 1)
        zb = None if z is None else z.reshape(B, H, 1, 1)
        cg = codes
    elif spec.axis == PER_CHANNEL:
        G = spec.group if spec.group > 0 else T
        cg = codes.reshape(B, H, T // G, G, D)
        sb = s[:, :, :, None, :]
        zb = None if z is None else z[:, :, :, None, :]
    else:
        Gc = spec.group if spec.group > 0 else D
        cg = codes.reshape(B, H, T, D // Gc, Gc)
        sb = s[..., None]
        zb = None if z is None else z[..., None]
    if spec.scheme == INT_ASYM:
        out = Q.asym_dequantize(cg, sb, zb)
    else:
        out = Q.sym_dequantize(cg, sb)
    return out.reshape(B, H, T, D)
