"""Seeded random configurations against the oracle: formats of the two sides
drawn independently (INT2/4/8 keys per channel with 32/64/128-token groups,
per-token keys, FP8 E4M3 / E5M2, symmetric INT8; values per token with
16..128-channel groups, FP8, symmetric INT8), fp16 windows of 0-2 key groups,
keys cached before RoPE, fp16 metadata, input dtypes, 1-33 query heads per kv
head, head sizes 64 and 128, lengths from 1 to ~1300 tokens appended in one
call or streamed across folds, and split counts from automatic to many.  Each
configuration runs through run_case: codes, scales, zero-points, window and
dequantized values bit-exact, attention within 2e-3 relative L2 on every
kernel that serves it (the MFMA kernel with head groups where the heads
need them)."""
import numpy as np
import pytest

import quantized_decode_attention_05_amd as K
from tests.kvq_harness import Case
from tests.test_gpu_parity import _schedule, run_case

pytestmark = pytest.mark.gpu

A, S, F8, E5 = K.INT_ASYM, K.INT_SYM, K.FP8_E4M3, K.FP8_E5M2
CH, TOK = K.PER_CHANNEL, K.PER_TOKEN
N_CASES = 40


def _draw(i):
    """Configuration i (deterministic): (case, T, schedule kind, splits)."""
    rng = np.random.default_rng((2027, i))
    while True:
        D = 128 if rng.random() < 0.85 else 64
        kk = rng.choice(["int_ch", "int_ch", "int_ch", "fp8", "e5m2", "int_tok", "sym8"])
        if kk == "int_ch":
            k = (A, int(rng.choice([2, 4, 8])), CH, int(rng.choice([32, 64, 128])))
        elif kk == "fp8":
            k = (F8, 8, 0, 0)
        elif kk == "e5m2":
            k = (E5, 8, 0, 0)
        elif kk == "int_tok":
            k = (A, int(rng.choice([2, 4, 8])), TOK, int(rng.choice([0, 32])))
        else:
            k = (S, 8, TOK, 0)
        vk = rng.choice(["int", "int", "int", "fp8", "e5m2", "sym8"])
        if vk == "int":
            gc = int(rng.choice([16, 32, 64, 0]))
            v = (A, int(rng.choice([2, 4, 8])), TOK, gc if gc <= D else 0)
        elif vk == "fp8":
            v = (F8, 8, 0, 0)
        elif vk == "e5m2":
            v = (E5, 8, 0, 0)
        else:
            v = (S, 8, TOK, 32)
        gt = k[3] if k[2] == CH else 32
        R = int(rng.choice([0, 0, 1, 2])) * gt
        pre_rope = bool(k[2] == CH or k[0] in (F8, E5)) and rng.random() < 0.35
        meta16 = rng.random() < 0.25
        Hkv = int(rng.choice([1, 2, 3]))
        n_rep = int(rng.choice([1, 2, 3, 4, 5, 8, 8, 12, 16, 20, 33]))
        B = int(rng.choice([1, 2, 3]))
        dtype = str(rng.choice(["f32", "f16", "bf16"]))
        T = int(rng.integers(1, 1300))
        sched = "oneshot" if rng.random() < 0.3 else "stream"
        splits = int(rng.choice([0, 0, 1, 2, 5, 13]))
        case = Case(B=B, Hq=Hkv * n_rep, Hkv=Hkv, D=D, dtype=dtype, k=k, v=v, R=R, pre_rope=pre_rope,
                    meta16=meta16)
        try:
            case.lib_cfg(T + 5)
        except K.KvqError:
            continue          # a combination the library refuses (checked by the ABI tests): draw again
        return case, T, sched, splits


@pytest.mark.parametrize("i", range(N_CASES), ids=[f"fuzz{i:02d}" for i in range(N_CASES)])
def test_random_configuration_matches_the_oracle(i):
    case, T, sched, splits = _draw(i)
    run_case(case, T, _schedule(sched, T), seed=500 + i, num_splits=splits)


N_PAGED = 16


def _draw_paged(i):
    """Paged configuration i: (case, page tokens, prefill lengths, chunk lengths, decode steps)."""
    rng = np.random.default_rng((2029, i))
    while True:
        kk = rng.choice(["int_ch", "int_ch", "fp8", "e5m2", "sym8"])
        if kk == "int_ch":
            k = (A, int(rng.choice([2, 4, 8])), CH, int(rng.choice([32, 64, 128])))
        elif kk == "fp8":
            k = (F8, 8, 0, 0)
        elif kk == "e5m2":
            k = (E5, 8, 0, 0)
        else:
            k = (S, 8, TOK, 0)
        vk = rng.choice(["int", "int", "fp8", "e5m2"])
        if vk == "int":
            v = (A, int(rng.choice([2, 4, 8])), TOK, int(rng.choice([16, 32, 64, 0])))
        elif vk == "fp8":
            v = (F8, 8, 0, 0)
        else:
            v = (E5, 8, 0, 0)
        gt = k[3] if k[2] == CH else 32
        P = gt * int(rng.choice([1, 2, 4])) if gt >= 32 else 32 * int(rng.choice([1, 2, 8]))
        R = int(rng.choice([0, 1, 2])) * gt
        pre_rope = bool(k[2] == CH or k[0] in (F8, E5)) and rng.random() < 0.35
        meta16 = rng.random() < 0.25
        Hkv = int(rng.choice([1, 2]))
        n_rep = int(rng.choice([1, 4, 8, 12, 20]))
        B = int(rng.choice([1, 2, 3, 4]))
        pre = [int(x) for x in rng.integers(0, 900, B)]
        chunk = [int(x) for x in rng.integers(0, 40, B)]
        # every sequence holds a token before its first decode step
        chunk = [c if p_ or c else 1 for p_, c in zip(pre, chunk)]
        steps = int(rng.integers(1, 40))
        case = Case(B=B, Hq=Hkv * n_rep, Hkv=Hkv, D=128, dtype="bf16", k=k, v=v, R=R, pre_rope=pre_rope,
                    meta16=meta16)
        try:
            K.make_config(batch=B, num_q_heads=case.Hq, num_kv_heads=Hkv, head_dim=128, max_tokens=1024, k=k, v=v,
                          in_dtype=K.BF16, out_dtype=K.F32, residual=R, pre_rope_k=pre_rope,
                          meta_dtype=K.F16 if meta16 else K.F32, page_tokens=P, num_pages=B * 40)
        except K.KvqError:
            continue
        return case, P, pre, chunk, steps


@pytest.mark.parametrize("i", range(N_PAGED), ids=[f"paged{i:02d}" for i in range(N_PAGED)])
def test_random_paged_configuration_matches_the_oracle(i):
    """A ragged prefill, a ragged chunk and decode steps through the paged
    entry points; each sequence's sections, dequantized values and attention
    (after the steps, on every kernel, at a drawn split count) against the
    oracle of that sequence alone."""
    import math
    import torch
    import workloads as W
    from oracle import attention as OA
    from tests.kvq_harness import ATTN_TOL, PagedCache, compare_paged_sequence
    from tests.test_gpu_paged import _fp8_scales, _kernels, _oracle_seq, _rows
    case, P, pre, chunk, steps = _draw_paged(i)
    seed = 700 + i
    Tmax = max(p + c for p, c in zip(pre, chunk)) + steps
    (Kf, Kp), (Vf, Vp) = W.random_case(seed, case.B, case.Hkv, Tmax, case.D, dtype="bf16")
    pc = PagedCache(case, P, cap=Tmax + 8, seed=seed)
    fp8 = case.k[0] == F8 or case.v[0] == F8
    n0 = max(max(pre), 1)
    pc.append(np.stack([_rows(Kp, b, 0, pre[b], n0) for b in range(case.B)]),
              np.stack([_rows(Vp, b, 0, pre[b], n0) for b in range(case.B)]), pre,
              K.INIT | (K.CALIBRATE if fp8 else 0))
    scales = _fp8_scales(case, Kf, Vf, pre)
    n1 = max(max(chunk), 1)
    pc.append(np.stack([_rows(Kp, b, pre[b], pre[b] + chunk[b], n1) for b in range(case.B)]),
              np.stack([_rows(Vp, b, pre[b], pre[b] + chunk[b], n1) for b in range(case.B)]), chunk)
    ws = torch.zeros(K.kvq_workspace_bytes(pc.cfg, Tmax + 8), dtype=torch.uint8, device="cuda")
    out = torch.empty((case.B, case.Hq, case.D), dtype=torch.float32, device="cuda")
    for s in range(steps):
        t = pc.lens.copy()
        kn = np.stack([Kp[b, :, t[b]:t[b] + 1] for b in range(case.B)])
        vn = np.stack([Vp[b, :, t[b]:t[b] + 1] for b in range(case.B)])
        pc.step(kn, vn, W.random_queries(seed + 100 + s, case.B, case.Hq, case.D, dtype="bf16")[1], ws, out)
    torch.cuda.synchronize()
    kd, vd = pc.dequantize()
    sm = 1.0 / math.sqrt(case.D)
    qf, qp = W.random_queries(seed + 7, case.B, case.Hq, case.D, dtype="bf16")
    splits = int(np.random.default_rng((2031, i)).choice([0, 1, 3, 9]))
    outs = {kern: pc.attention(qp, kernel=kern, num_splits=splits) for kern in _kernels(pc.cfg, int(pc.lens.max()))}
    for b in range(case.B):
        T = int(pc.lens[b])
        st = _oracle_seq(case, Kf, Vf, b, T, scales)
        compare_paged_sequence(pc, b, st, None if scales is None else {"k": scales[0], "v": scales[1]})
        assert np.array_equal(kd[b, :, :T], st["k_hat"][0]), f"seq {b}: dequantized K differs"
        assert np.array_equal(vd[b, :, :T], st["v_hat"][0]), f"seq {b}: dequantized V differs"
        ref = OA.decode_attention(qf[b:b + 1], st["k_hat"], st["v_hat"], sm,
                                  pre_rope_base=case.rope_base if case.pre_rope else None)
        for kern, o in outs.items():
            err = OA.max_rel_l2_per_head(o[b:b + 1], ref)
            assert err <= ATTN_TOL, (i, kern, splits, b, err)


N_STEP = 12


def _draw_step(i):
    """Decode-step configuration i: (case, prefill length, steps, splits)."""
    rng = np.random.default_rng((2033, i))
    while True:
        kk = rng.choice(["int_ch", "int_ch", "fp8", "e5m2"])
        if kk == "int_ch":
            k = (A, int(rng.choice([2, 4, 8])), CH, int(rng.choice([32, 64, 128])))
        elif kk == "fp8":
            k = (F8, 8, 0, 0)
        else:
            k = (E5, 8, 0, 0)
        vk = rng.choice(["int", "fp8", "e5m2"])
        v = (A, int(rng.choice([2, 4, 8])), TOK, int(rng.choice([16, 32, 0]))) if vk == "int" else \
            ((F8, 8, 0, 0) if vk == "fp8" else (E5, 8, 0, 0))
        gt = k[3] if k[2] == CH else 32
        R = int(rng.choice([0, 1, 2])) * gt
        pre_rope = rng.random() < 0.3
        Hkv = int(rng.choice([1, 2]))
        n_rep = int(rng.choice([1, 4, 8, 16, 24]))
        case = Case(B=int(rng.choice([1, 2, 3])), Hq=Hkv * n_rep, Hkv=Hkv, D=128, dtype="bf16", k=k, v=v, R=R,
                    pre_rope=pre_rope, meta16=rng.random() < 0.2)
        T0 = int(rng.integers(1, 700))
        steps = int(rng.integers(5, 45))
        splits = int(rng.choice([0, 1, 3, 7]))
        try:
            case.lib_cfg(T0 + steps)
        except K.KvqError:
            continue
        return case, T0, steps, splits


@pytest.mark.parametrize("i", range(N_STEP), ids=[f"step{i:02d}" for i in range(N_STEP)])
def test_random_decode_steps_equal_append_then_attention(i):
    """kvq_decode_step (the call bench.py times; the append runs inside the
    attention launch when the shape allows) against kvq_quantize_append
    followed by kvq_decode_attention on a second cache: the same cache bytes
    and the same outputs, bit for bit, at every step; the final output within
    tolerance of the oracle."""
    import math
    import torch
    import workloads as W
    from oracle import attention as OA
    from oracle import cache as OC
    from tests.kvq_harness import ATTN_TOL, GpuCache, to_dev
    case, T0, steps, splits = _draw_step(i)
    (Kf, Kp), (Vf, Vp) = W.random_case(900 + i, case.B, case.Hkv, T0 + steps, case.D, dtype="bf16")
    ga, gb = GpuCache(case, cap=T0 + steps), GpuCache(case, cap=T0 + steps)
    fp8 = case.k[0] == F8 or case.v[0] == F8
    flags = K.CALIBRATE if fp8 else 0
    ga.append(Kp[:, :, :T0], Vp[:, :, :T0], flags)
    gb.append(Kp[:, :, :T0], Vp[:, :, :T0], flags)
    sm = 1.0 / math.sqrt(case.D)
    wa = torch.zeros(K.kvq_workspace_bytes(ga.cfg, T0 + steps, 0, splits), dtype=torch.uint8, device="cuda")
    wb = torch.zeros(K.kvq_workspace_bytes(gb.cfg, T0 + steps, 0, splits), dtype=torch.uint8, device="cuda")
    oa = torch.empty((case.B, case.Hq, case.D), dtype=torch.float32, device="cuda")
    ob = torch.empty_like(oa)
    for s in range(steps):
        t = T0 + s
        kn, vn = to_dev(Kp[:, :, t:t + 1], "bf16"), to_dev(Vp[:, :, t:t + 1], "bf16")
        qf, qp = W.random_queries(3000 + 50 * i + s, case.B, case.Hq, case.D, dtype="bf16")
        q = to_dev(qp, "bf16")
        oa.fill_(float("nan"))
        ob.fill_(float("nan"))
        K.kvq_decode_step(ga.cfg, ga.arena, t, kn, vn, q, oa, sm, wa, 0, splits)
        K.kvq_quantize_append(gb.cfg, gb.arena, t, kn, vn)
        K.kvq_decode_attention(gb.cfg, gb.arena, t + 1, q, ob, sm, wb, 0, splits)
        torch.cuda.synchronize()
        assert torch.equal(ga.arena, gb.arena), (i, t, "cache bytes differ")
        assert torch.isfinite(oa).all() and torch.equal(oa, ob), (i, t, "outputs differ")
    T = T0 + steps
    st = OC.quantize_cache(case.oracle_cfg(), Kf, Vf, T, calibrate_tokens=T0 if fp8 else 0)
    ref = OA.decode_attention(qf, st["k_hat"], st["v_hat"], sm, pre_rope_base=case.rope_base if case.pre_rope else None)
    assert OA.max_rel_l2_per_head(oa.cpu().numpy(), ref) <= ATTN_TOL
