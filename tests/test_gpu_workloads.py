"""The five workloads at full size through the C ABI, against the CPU oracle.

Single-head workloads are compared whole.  The three large ones are run whole
on the GPU (prefill, then the decode-time append) and compared on sampled
(sequence, kv head) pairs that the oracle recomputes from the same seeded
chunks: codes, scales, window and dequantized values bit-exact, attention of
the pairs' query heads within 2e-3 relative L2.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import quantized_decode_attention_05_amd as K
import workloads as W
from oracle import attention as OA
from oracle import cache as OC
from tests.kvq_harness import (ATTN_TOL, Case, GpuCache, compare_dequant, compare_sections, say,
                               to_dev)

pytestmark = pytest.mark.gpu

A, S, F8, E5, NO = K.INT_ASYM, K.INT_SYM, K.FP8_E4M3, K.FP8_E5M2, K.NONE
CH, TOK, TEN = K.PER_CHANNEL, K.PER_TOKEN, K.PER_TENSOR
GOLD = os.path.join(os.path.dirname(__file__), "golden")

KERNELS = [K.KERNEL_GENERIC]


def _kernels_for(gc):
    ks = list(KERNELS)
    try:
        K.kvq_workspace_bytes(gc.cfg, max(gc.T, 1), K.KERNEL_MFMA)
        ks.append(K.KERNEL_MFMA)
    except K.KvqError:
        pass
    return ks


# ---------------------------------------------------------------------------
# single-head INT8 workload: the printed table through the library
# ---------------------------------------------------------------------------

C1_VARIANTS = {
    "K+V per-tensor INT8": ((S, 8, TEN, 0), (S, 8, TEN, 0)),
    "K per-channel, V per-token": ((S, 8, CH, 0), (S, 8, TOK, 0)),
    "V per-token only (K exact)": ((NO, 32, 0, 0), (S, 8, TOK, 0)),
    "K per-tensor only (V exact)": ((S, 8, TEN, 0), (NO, 32, 0, 0)),
}


@pytest.mark.parametrize("variant", list(C1_VARIANTS))
def test_c1_int8_single_head(variant):
    x = W.single_head_inputs("c1_int8_sym_single_head")
    kspec, vspec = C1_VARIANTS[variant]
    case = Case(B=1, Hq=1, Hkv=1, D=128, dtype="f32", k=kspec, v=vspec)
    Kf, Vf = x["K"][None, None], x["V"][None, None]
    gc = GpuCache(case, cap=4096)
    gc.append(Kf, Vf)
    st = OC.quantize_cache(case.oracle_cfg(), Kf, Vf, 4096)
    compare_sections(gc, st)
    compare_dequant(gc, st)
    sm = 1.0 / math.sqrt(128)
    ref_exact, lg_exact = OA.single_head(x["q"], x["K"], x["V"], sm)
    kd, vd = gc.dequantize()
    _, lg_q = OA.single_head(x["q"], kd[0, 0], vd[0, 0], sm)
    printed = json.load(open(os.path.join(GOLD, "int8_synthetic_head_table.json")))["rows"][variant]
    for kern in _kernels_for(gc):
        out = gc.attention(x["q"][None, None], kernel=kern)[0, 0]
        err_vs_oracle = OA.rel_l2(out, OA.single_head(x["q"], st["k_hat"][0, 0], st["v_hat"][0, 0], sm)[0])
        assert err_vs_oracle <= ATTN_TOL
        # the page's metric, measured on the library's output
        assert abs(OA.rel_l2(out, ref_exact) - printed[0]) < 5e-4, (variant, OA.rel_l2(out, ref_exact))
        say(f"[c1] {variant} kernel={kern} rel_err={OA.rel_l2(out, ref_exact):.4f} vs oracle {err_vs_oracle:.2e}")
    assert round(float(np.abs(lg_q - lg_exact).max()), 3) == pytest.approx(printed[1], abs=1e-12)


# ---------------------------------------------------------------------------
# single-head INT4 workload: per-token vs per-channel keys
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kaxis", [TOK, CH])
def test_c2_int4_single_head(kaxis):
    x = W.single_head_inputs("c2_int4_asym_single_head")
    case = Case(B=1, Hq=1, Hkv=1, D=128, dtype="f32", k=(A, 4, kaxis, 0), v=(A, 4, TOK, 0))
    Kf, Vf = x["K"][None, None], x["V"][None, None]
    gc = GpuCache(case, cap=512)
    gc.append(Kf, Vf)
    st = OC.quantize_cache(case.oracle_cfg(), Kf, Vf, 512)
    compare_sections(gc, st)
    compare_dequant(gc, st)
    sm = 1.0 / math.sqrt(128)
    for kern in _kernels_for(gc):
        out = gc.attention(x["q"][None, None], kernel=kern)[0, 0]
        ref = OA.single_head(x["q"], st["k_hat"][0, 0], st["v_hat"][0, 0], sm)[0]
        assert OA.rel_l2(out, ref) <= ATTN_TOL


# ---------------------------------------------------------------------------
# large workloads
# ---------------------------------------------------------------------------

LARGE = {
    "c3_fp8_e4m3_gqa_8k": dict(k=(F8, 8, 0, 0), v=(F8, 8, 0, 0), R=0),
    "c3_fp8_e5m2_gqa_8k": dict(k=(E5, 8, 0, 0), v=(E5, 8, 0, 0), R=0),
    "c4_int4_llama70b_128k": dict(k=(A, 4, CH, 128), v=(A, 4, TOK, 0), R=128),
    "c5_int2_kivi_prerope_32k": dict(k=(A, 2, CH, 32), v=(A, 2, TOK, 32), R=32, pre_rope=True),
    # the same caches with fp16 scales / zero-points
    "c4_int4_llama70b_128k+meta16": dict(k=(A, 4, CH, 128), v=(A, 4, TOK, 0), R=128, meta16=True,
                                         workload="c4_int4_llama70b_128k"),
    "c5_int2_kivi_prerope_32k+meta16": dict(k=(A, 2, CH, 32), v=(A, 2, TOK, 32), R=32, pre_rope=True,
                                            meta16=True, workload="c5_int2_kivi_prerope_32k"),
}


N_STEPS = 40          # decode steps of test_large_decode_steps_against_oracle


def _samples(w):
    """Every kv head of the first and the last sequence (all heads of a
    batch-1 workload): 16 pairs for the batch-16 and batch-32 caches, 8 for
    the batch-1 one."""
    B, H = w["B"], w["Hkv"]
    return sorted({(b, h) for b in (0, B - 1) for h in range(H)})


@pytest.fixture(scope="module", params=list(LARGE))
def large(request):
    label = request.param
    fmt = dict(LARGE[label])
    name = fmt.pop("workload", label)     # the workload whose inputs are used
    w = W.WORKLOADS[name]
    case = Case(B=w["B"], Hq=w["Hq"], Hkv=w["Hkv"], D=w["D"], dtype="bf16", **fmt)
    say(f"[{name}] generating inputs")
    Kp = W.full_prefill(name, "k")
    Vp = W.full_prefill(name, "v")
    n_new = w.get("n_new", 0)
    T = w["T"] + n_new
    gc = GpuCache(case, cap=T + (N_STEPS if n_new else 0))
    fp8 = fmt["k"][0] == F8
    say(f"[{name}] prefill append T={w['T']}")
    gc.append(Kp, Vp, K.CALIBRATE if fp8 else 0)
    if n_new:
        gc.append(W.full_new_tokens(name, "k"), W.full_new_tokens(name, "v"))
    torch.cuda.synchronize()
    scales = None
    if fp8:   # oracle calibration over all sequences of each head (prefill tokens only)
        amax_k = np.zeros(w["Hkv"], np.float32)
        amax_v = np.zeros(w["Hkv"], np.float32)
        for h in range(w["Hkv"]):
            amax_k[h] = np.abs(W.bf16_bits_to_f32(Kp[:, h])).max()
            amax_v[h] = np.abs(W.bf16_bits_to_f32(Vp[:, h])).max()
        from oracle import quant as OQ
        scales = (OQ.fp8_scale_from_absmax(amax_k), OQ.fp8_scale_from_absmax(amax_v))
    del Kp, Vp
    q = W.query(name)
    yield dict(name=name, w=w, case=case, gc=gc, T=T, scales=scales, q=q, oracle={})
    del gc
    torch.cuda.empty_cache()


def _oracle_pair(name, w, case, b, h, T, scales):
    n_new = w.get("n_new", 0)
    kb = W.kv_chunk(name, b, h, "k")
    vb = W.kv_chunk(name, b, h, "v")
    if n_new:
        kb = np.concatenate([kb, W.new_token_chunk(name, b, h, "k")])
        vb = np.concatenate([vb, W.new_token_chunk(name, b, h, "v")])
    Kf = W.bf16_bits_to_f32(kb)[None, None]
    Vf = W.bf16_bits_to_f32(vb)[None, None]
    sub = case.oracle_cfg(B=1, Hq=case.Hq // case.Hkv, Hkv=1)
    ks = vs = None
    if scales is not None:
        ks, vs = scales[0][h:h + 1], scales[1][h:h + 1]
    return OC.quantize_cache(sub, Kf, Vf, T, k_scale=ks, v_scale=vs)


def _oracle_cached(L, b, h):
    """The oracle state of one (sequence, kv head) of the fixture's cache,
    computed once per module and shared by the tests below."""
    key = (b, h)
    if key not in L["oracle"]:
        L["oracle"][key] = _oracle_pair(L["name"], L["w"], L["case"], b, h, L["T"], L["scales"])
    return L["oracle"][key]


def test_large_sections_bit_exact(large):
    L = large
    for (b, h) in _samples(L["w"]):
        say(f"[{L['name']}] sections of (b={b}, h={h})")
        st = _oracle_cached(L, b, h)
        compare_sections(L["gc"], st, bh_sel=(b, h))
        compare_dequant(L["gc"], st, bh_sel=(b, h))


def test_large_attention(large):
    L = large
    case, gc, T = L["case"], L["gc"], L["T"]
    n_rep = case.Hq // case.Hkv
    qf = W.bf16_bits_to_f32(L["q"])
    sm = 1.0 / math.sqrt(case.D)
    outs = {kern: gc.attention(L["q"], kernel=kern) for kern in _kernels_for(gc)}
    for (b, h) in _samples(L["w"]):
        st = _oracle_cached(L, b, h)
        qs = qf[b:b + 1, h * n_rep:(h + 1) * n_rep]
        ref = OA.decode_attention(qs, st["k_hat"], st["v_hat"], sm,
                                  pre_rope_base=case.rope_base if case.pre_rope else None)
        for kern, out in outs.items():
            got = out[b:b + 1, h * n_rep:(h + 1) * n_rep]
            err = OA.max_rel_l2_per_head(got, ref)
            say(f"[{L['name']}] (b={b}, h={h}) kernel={kern} max rel-L2 {err:.2e}")
            assert err <= ATTN_TOL
    if len(outs) > 1:
        # every head, not only the samples: the generic kernel is within ~1e-5 of
        # the oracle, so its distance to the MFMA kernel bounds the latter's error
        o1, o2 = outs[K.KERNEL_GENERIC], outs[K.KERNEL_MFMA]
        rel = np.linalg.norm(o1 - o2, axis=-1) / np.linalg.norm(o1, axis=-1)
        say(f"[{L['name']}] MFMA vs generic over all {rel.size} heads: max {rel.max():.2e} "
            f"mean {rel.mean():.2e} p99 {np.percentile(rel, 99):.2e}")
        assert rel.max() <= ATTN_TOL


def test_large_decode_steps_against_oracle(large):
    """kvq_decode_step, the call bench.py times, in its default launch
    configuration at the workload's full size: N_STEPS consecutive steps (the
    INT2 cache folds its fp16 window once among them; the FP8 caches encode the
    new token inside the attention launch), each with its own new tokens and
    query.  Afterwards the cache bytes of sampled (sequence, kv head) pairs
    match the oracle bit for bit, and the outputs of the first step, the first
    fold step and the last step are within tolerance of the oracle's attention
    over the cache as it stood at that step.  Runs after the tests above (it
    appends to the shared cache)."""
    L = large
    w, case, gc, name = L["w"], L["case"], L["gc"], L["name"]
    if not w.get("n_new"):
        pytest.skip("this workload appends nothing")
    B, Hq, Hkv, D = case.B, case.Hq, case.Hkv, case.D
    n_rep = Hq // Hkv
    T0 = gc.T
    sm = 1.0 / math.sqrt(D)
    ocfg = case.oracle_cfg()
    folds = [i for i in range(N_STEPS) if OC.quantized_tokens(ocfg, T0 + i + 1) > OC.quantized_tokens(ocfg, T0 + i)]
    if OC.token_group(ocfg) > 1:
        assert folds, "the steps should cross a fold"
    checks = sorted({0, N_STEPS - 1} | set(folds[:1]))
    ws = torch.zeros(K.kvq_workspace_bytes(gc.cfg, T0 + N_STEPS), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    outs = {}
    say(f"[{name}] {N_STEPS} decode steps from T={T0}, folds at steps {folds[:3]}")
    for i in range(N_STEPS):
        kn = to_dev(W.step_tokens_all(name, "k", i), "bf16")
        vn = to_dev(W.step_tokens_all(name, "v", i), "bf16")
        q = to_dev(W.step_query(name, i), "bf16")
        out.fill_(float("nan"))
        K.kvq_decode_step(gc.cfg, gc.arena, T0 + i, kn, vn, q, out, sm, ws)
        if i in checks:
            torch.cuda.synchronize()
            outs[i] = out.cpu().numpy()
            assert np.isfinite(outs[i]).all(), f"step {i}: outputs not written"
    torch.cuda.synchronize()
    gc.T = T0 + N_STEPS
    pairs = sorted({(0, 0), (0, Hkv - 1), (B - 1, 0), (B - 1, Hkv - 1)})
    sub = case.oracle_cfg(B=1, Hq=n_rep, Hkv=1)
    for (b, h) in pairs:
        kb = np.concatenate([W.kv_chunk(name, b, h, "k"), W.new_token_chunk(name, b, h, "k"),
                             W.step_tokens(name, b, h, "k", 0, N_STEPS)])
        vb = np.concatenate([W.kv_chunk(name, b, h, "v"), W.new_token_chunk(name, b, h, "v"),
                             W.step_tokens(name, b, h, "v", 0, N_STEPS)])
        Kf, Vf = W.bf16_bits_to_f32(kb)[None, None], W.bf16_bits_to_f32(vb)[None, None]
        ks = vs = None
        if L["scales"] is not None:
            ks, vs = L["scales"][0][h:h + 1], L["scales"][1][h:h + 1]
        st = OC.quantize_cache(sub, Kf, Vf, T0 + N_STEPS, k_scale=ks, v_scale=vs)
        compare_sections(gc, st, bh_sel=(b, h))
        compare_dequant(gc, st, bh_sel=(b, h))
        for i in checks:
            sti = OC.quantize_cache(sub, Kf, Vf, T0 + i + 1, k_scale=ks, v_scale=vs)
            qf = W.bf16_bits_to_f32(W.step_query(name, i))[b:b + 1, h * n_rep:(h + 1) * n_rep]
            ref = OA.decode_attention(qf, sti["k_hat"], sti["v_hat"], sm,
                                      pre_rope_base=case.rope_base if case.pre_rope else None)
            err = OA.max_rel_l2_per_head(outs[i][b:b + 1, h * n_rep:(h + 1) * n_rep], ref)
            say(f"[{name}] step {i} (T={T0 + i + 1}) (b={b}, h={h}) max rel-L2 {err:.2e}")
            assert err <= ATTN_TOL, (name, i, b, h, err)
