"""Pre-RoPE vs post-RoPE per-channel key quantization on synthetic heads.

"KV Cache Quantization: Why Keys and Values Need Different Axes", section
"Where does RoPE break this?": RoPE rotates channel pairs by a
position-dependent angle, so a channel that is always large shares its
magnitude with its partner as a function of position; quantizing keys after
RoPE makes per-channel groups fight that rotation, quantizing before it (and
rotating after dequantization inside attention) keeps the clean structure.
The diagnostics are the ones the pages recommend for KV quantization: the
attention KL divergence against the unquantized keys and the agreement of
the top-k attended positions ("What should I actually turn on in
production?"), plus the relative error of the rotated keys.

Heads (``workloads.rope_study_case``): N(0, 1) keys with four outlier
channels of magnitude 20, either sign-consistent (+-20 + N(0, 1), "the same
channel is always huge") or random-sign (N(0, 1) * 20, the page's listing);
RoPE base 10000 at positions 0..T-1.  Keys INT{2,4,8} per-channel in groups
of G tokens; values INT8 per-token.  Pre-RoPE caches store raw keys
(pre_rope_k); post-RoPE caches store keys the caller rotated before the
append.  The pages print no numbers for this study (values unpinned); the
tests check the stated direction for sign-consistent outliers and report
both structures.
"""
import math

import numpy as np
import pytest

import workloads as W
from oracle import attention as OA
from oracle import cache as OC

B, HQ, HKV, T, D = 1, 8, 2, 4096, 128
BASE = 10000.0
TOPK = 32


def _rotate(K):
    pos = np.arange(K.shape[2])
    return np.stack([np.stack([OA.rope(K[b, h].astype(np.float64), pos, BASE) for h in range(K.shape[1])])
                     for b in range(K.shape[0])]).astype(np.float32)


def _probs(q, Krot):
    sm = 1.0 / math.sqrt(D)
    n_rep = HQ // HKV
    out = []
    for b in range(B):
        for h in range(HQ):
            _, lg = OA.single_head(q[b, h], Krot[b, h // n_rep], Krot[b, h // n_rep], sm)
            p = np.exp(lg - lg.max())
            out.append(p / p.sum())
    return np.array(out)


def _metrics(q, Krot, Krot_hat, P_ref):
    P = _probs(q, Krot_hat)
    kl = float(np.mean(np.sum(P_ref * (np.log(P_ref) - np.log(P)), axis=1)))
    top = float(np.mean([len(set(np.argsort(-P_ref[i])[:TOPK]) & set(np.argsort(-P[i])[:TOPK])) / TOPK
                         for i in range(P.shape[0])]))
    kerr = float(np.linalg.norm(Krot_hat - Krot) / np.linalg.norm(Krot))
    return dict(kl=kl, top=top, kerr=kerr)


def _cfg(bits, G, pre):
    return OC.Cfg(B, HQ, HKV, D, OC.Spec(OC.INT_ASYM, bits, OC.PER_CHANNEL, G),
                  OC.Spec(OC.INT_ASYM, 8, OC.PER_TOKEN, 0), 0, pre, BASE)


def _check(table):
    """Sign-consistent outliers: pre-RoPE beats post-RoPE in every metric at 2
    and 4 bits, by a wide margin in KL."""
    for bits in (2, 4):
        pre, post = table[("pre", bits)], table[("post", bits)]
        assert pre["kl"] * 2 < post["kl"], (bits, pre, post)
        assert pre["top"] > post["top"] and pre["kerr"] < post["kerr"], (bits, pre, post)


@pytest.mark.parametrize("G", [128])
def test_rope_study_oracle(G):
    Kf, Vf, qf = W.rope_study_case(41, B, HQ, HKV, T, D, consistent=True)
    Krot = _rotate(Kf)
    P_ref = _probs(qf, Krot)
    table = {}
    for bits in (2, 4, 8):
        st = OC.quantize_cache(_cfg(bits, G, True), Kf, Vf, T)
        table[("pre", bits)] = _metrics(qf, Krot, _rotate(st["k_hat"]), P_ref)
        st = OC.quantize_cache(_cfg(bits, G, False), Krot, Vf, T)
        table[("post", bits)] = _metrics(qf, Krot, st["k_hat"], P_ref)
    _check(table)


@pytest.mark.gpu
@pytest.mark.parametrize("G", [32, 128])
def test_rope_study_gpu(G):
    """Both structures, INT2/4/8 keys, pre- and post-RoPE caches through the C
    ABI: cache bytes bit-exact against the oracle, attention within 2e-3 of the
    oracle (both kernels), study metrics from the GPU's dequantized keys."""
    import quantized_decode_attention_05_amd as K
    from tests.kvq_harness import (ATTN_TOL, Case, GpuCache, attention_error, compare_dequant,
                                   compare_sections, say)
    for consistent in (True, False):
        Kf, Vf, qf = W.rope_study_case(41, B, HQ, HKV, T, D, consistent=consistent)
        Krot = _rotate(Kf)
        P_ref = _probs(qf, Krot)
        table = {}
        for bits in (2, 4, 8):
            for mode in ("pre", "post"):
                pre = mode == "pre"
                kin = Kf if pre else Krot
                case = Case(B=B, Hq=HQ, Hkv=HKV, D=D, dtype="f32", k=(K.INT_ASYM, bits, K.PER_CHANNEL, G),
                            v=(K.INT_ASYM, 8, K.PER_TOKEN, 0), R=0, pre_rope=pre, rope_base=BASE)
                gc = GpuCache(case, cap=T)
                gc.append(kin, Vf, 0)
                st = OC.quantize_cache(_cfg(bits, G, pre), kin, Vf, T)
                compare_sections(gc, st)
                compare_dequant(gc, st)
                for kern in (K.KERNEL_GENERIC, K.KERNEL_MFMA):
                    e = attention_error(gc.attention(qf, kernel=kern), qf, st, case)
                    assert e <= ATTN_TOL, (consistent, bits, mode, kern, e)
                kd, _ = gc.dequantize(T)
                table[(mode, bits)] = _metrics(qf, Krot, _rotate(kd) if pre else kd, P_ref)
                m = table[(mode, bits)]
                say(f"[rope study] {'consistent' if consistent else 'random-sign'} G{G} INT{bits} "
                    f"{mode:4s}-RoPE: attention KL {m['kl']:.4f}  top-{TOPK} agreement {m['top']:.3f}  "
                    f"rotated-key rel error {m['kerr']:.4f}")
        if consistent:
            _check(table)
