"""GPU parity on small shapes: quantize-append, dequantize and decode attention
through the C ABI against the CPU oracle (bit-exact codes, scales, window and
dequantized values; attention within 2e-3 max relative L2)."""
import zlib

import numpy as np
import pytest

import quantized_decode_attention_05_amd as K
import workloads as W
from oracle import cache as OC
from tests.kvq_harness import (ATTN_TOL, Case, GpuCache, attention_error, compare_dequant,
                               compare_sections, say)

pytestmark = pytest.mark.gpu

A, S, F8, E5, NO = K.INT_ASYM, K.INT_SYM, K.FP8_E4M3, K.FP8_E5M2, K.NONE
CH, TOK, TEN = K.PER_CHANNEL, K.PER_TOKEN, K.PER_TENSOR

# (name, case, T, append schedule, kernels)
FORMATS = [
    ("int4ch128_int4tok_R128", dict(k=(A, 4, CH, 128), v=(A, 4, TOK, 0), R=128)),
    ("int2ch32_int2tok32_R32", dict(k=(A, 2, CH, 32), v=(A, 2, TOK, 32), R=32)),
    ("int2ch32_int2tok32_R0", dict(k=(A, 2, CH, 32), v=(A, 2, TOK, 32), R=0)),
    ("int8ch64_int8tok16_R64", dict(k=(A, 8, CH, 64), v=(A, 8, TOK, 16), R=64)),
    ("int4tok_int4tok_R0", dict(k=(A, 4, TOK, 0), v=(A, 4, TOK, 0), R=0)),
    ("int4tok32_int2tok_R64", dict(k=(A, 4, TOK, 32), v=(A, 2, TOK, 64), R=64)),
    ("fp8_fp8", dict(k=(F8, 8, 0, 0), v=(F8, 8, 0, 0), R=0)),
    ("fp8_fp8_R32", dict(k=(F8, 8, 0, 0), v=(F8, 8, 0, 0), R=32)),
    ("e5m2_e5m2", dict(k=(E5, 8, 0, 0), v=(E5, 8, 0, 0), R=0)),
    ("e4m3_e5m2_R32", dict(k=(F8, 8, 0, 0), v=(E5, 8, 0, 0), R=32)),
    ("int4ch128_e5m2_R128", dict(k=(A, 4, CH, 128), v=(E5, 8, 0, 0), R=128)),
    ("sym8tok_sym8tok", dict(k=(S, 8, TOK, 0), v=(S, 8, TOK, 32), R=0)),
    ("none16_int4tok", dict(k=(NO, 16, 0, 0), v=(A, 4, TOK, 0), R=0)),
    ("int2ch32_none32", dict(k=(A, 2, CH, 32), v=(NO, 32, 0, 0), R=32)),
    ("prerope_int2ch32_int2tok32_R32", dict(k=(A, 2, CH, 32), v=(A, 2, TOK, 32), R=32, pre_rope=True)),
    ("prerope_int4ch128_R128", dict(k=(A, 4, CH, 128), v=(A, 4, TOK, 0), R=128, pre_rope=True,
                                    rope_base=500.0)),
    # FP8 keys cached before RoPE: both FP8 (wavefronts take every fourth step),
    # FP8 keys with INT values and a window, and E5M2
    ("prerope_fp8_fp8", dict(k=(F8, 8, 0, 0), v=(F8, 8, 0, 0), R=0, pre_rope=True)),
    ("prerope_fp8_int4tok32_R32", dict(k=(F8, 8, 0, 0), v=(A, 4, TOK, 32), R=32, pre_rope=True)),
    ("prerope_e5m2_e5m2_R32", dict(k=(E5, 8, 0, 0), v=(E5, 8, 0, 0), R=32, pre_rope=True)),
]
ONE_SHOT = [
    ("sym8ten_sym8ten", dict(k=(S, 8, TEN, 0), v=(S, 8, TEN, 0))),
    ("sym8chwhole_sym8tok", dict(k=(S, 8, CH, 0), v=(S, 8, TOK, 0))),
    ("int4chwhole_int4tok", dict(k=(A, 4, CH, 0), v=(A, 4, TOK, 0))),
    ("int4ten_none32", dict(k=(A, 4, TEN, 0), v=(NO, 32, 0, 0))),
]


def _schedule(kind, T):
    if kind == "oneshot":
        return [T]
    # prefill, a run of single-token appends across fold boundaries, then chunks
    first = max(1, T // 2)
    rest = T - first
    sched = [first]
    singles = min(rest, 37)
    sched += [1] * singles
    rest -= singles
    while rest > 0:
        n = min(rest, 19)
        sched.append(n)
        rest -= n
    return sched


def run_case(case: Case, T: int, schedule, seed=0, kernels=None, fp8_mode="calibrate",
             num_splits=0, inputs=None, queries=None):
    say(f"[case] {case} T={T} sched={schedule[:4]}... seed={seed}")
    if inputs is None:
        (Kf, Kp), (Vf, Vp) = W.random_case(seed, case.B, case.Hkv, T, case.D, dtype=case.dtype)
    else:
        (Kf, Kp), (Vf, Vp) = inputs
    qf, qp = W.random_queries(seed, case.B, case.Hq, case.D, dtype=case.dtype) if queries is None else queries
    gc = GpuCache(case, cap=T + 5)
    fp8 = case.k[0] == F8 or case.v[0] == F8
    ks = vs = None
    t = 0
    for i, n in enumerate(schedule):
        flags = 0
        if fp8 and i == 0 and fp8_mode == "calibrate":
            flags = K.CALIBRATE
        if fp8 and i == 0 and fp8_mode == "given":
            ks = np.linspace(0.05, 0.2, case.Hkv).astype(np.float32)
            vs = np.linspace(0.01, 0.02, case.Hkv).astype(np.float32)
            gc.append(Kp[:, :, t:t + n], Vp[:, :, t:t + n], 0, ks, vs)
        else:
            gc.append(Kp[:, :, t:t + n], Vp[:, :, t:t + n], flags)
        t += n
    ocfg = case.oracle_cfg()
    st = OC.quantize_cache(ocfg, Kf, Vf, T, k_scale=ks, v_scale=vs,
                           calibrate_tokens=schedule[0] if (fp8 and fp8_mode == "calibrate") else 0)
    compare_sections(gc, st)
    compare_dequant(gc, st)
    if kernels is None:
        kernels = [K.KERNEL_GENERIC]
        try:
            K.kvq_workspace_bytes(gc.cfg, T, K.KERNEL_MFMA)
            kernels.append(K.KERNEL_MFMA)
        except K.KvqError:
            pass
    errs = {}
    for kern in kernels:
        out = gc.attention(qp, kernel=kern, num_splits=num_splits)
        errs[kern] = attention_error(out, qf, st, case)
        assert errs[kern] <= ATTN_TOL, (kern, errs[kern])
    say(f"[ok] attention max rel-L2 {errs}")
    return gc, st, errs


@pytest.mark.parametrize("name,fmt", FORMATS, ids=[f[0] for f in FORMATS])
@pytest.mark.parametrize("sched", ["oneshot", "stream"])
def test_formats(name, fmt, sched):
    case = Case(B=2, Hq=8, Hkv=2, D=128, dtype="bf16", **fmt)
    T = 333
    run_case(case, T, _schedule(sched, T), seed=zlib.crc32(name.encode()) % 1000)


@pytest.mark.parametrize("name,fmt", ONE_SHOT, ids=[f[0] for f in ONE_SHOT])
def test_one_shot_formats(name, fmt):
    case = Case(B=2, Hq=4, Hkv=2, D=128, dtype="f32", **fmt)
    run_case(case, 300, [300], seed=3)


@pytest.mark.parametrize("D,n_rep,dtype", [(64, 1, "f32"), (64, 4, "f16"), (128, 1, "f16"),
                                           (128, 8, "bf16"), (128, 16, "bf16")])
def test_shapes_and_dtypes(D, n_rep, dtype):
    case = Case(B=2, Hq=2 * n_rep, Hkv=2, D=D, dtype=dtype, k=(A, 4, CH, 32), v=(A, 4, TOK, 32), R=32)
    run_case(case, 257, _schedule("stream", 257), seed=D + n_rep)


@pytest.mark.parametrize("T", [1, 5, 31, 32, 33, 64, 65])
def test_short_caches_all_in_window(T):
    """T below the window keeps every token in fp16 (Tq = 0 for T < R + G)."""
    case = Case(B=1, Hq=4, Hkv=1, D=128, dtype="bf16", k=(A, 2, CH, 32), v=(A, 2, TOK, 32), R=32)
    run_case(case, T, _schedule("stream", T) if T > 1 else [1], seed=T)


@pytest.mark.parametrize("mode", ["given", "unit"])
def test_fp8_scale_modes(mode):
    case = Case(B=2, Hq=4, Hkv=2, D=128, dtype="bf16", k=(F8, 8, 0, 0), v=(F8, 8, 0, 0))
    run_case(case, 200, [120, 1, 1, 78], seed=9, fp8_mode=mode)


def test_fp8_saturation_of_later_appends():
    """Tokens appended after calibration reuse the stored scale and saturate."""
    case = Case(B=1, Hq=4, Hkv=1, D=128, dtype="f32", k=(F8, 8, 0, 0), v=(F8, 8, 0, 0))
    (Kf, Kp), (Vf, Vp) = W.random_case(4, 1, 1, 40, 128, dtype="f32")
    Kf = Kf.copy(); Kf[:, :, 30:] *= 50.0          # far beyond the calibrated range
    gc = GpuCache(case, cap=64)
    gc.append(Kf[:, :, :30], Vf[:, :, :30], K.CALIBRATE)
    gc.append(Kf[:, :, 30:], Vf[:, :, 30:])
    st = OC.quantize_cache(case.oracle_cfg(), Kf, Vf, 40, calibrate_tokens=30)
    compare_sections(gc, st)
    codes = st["k"]["codes"][0, 0, 30:]
    assert np.any((codes & 0x7F) == 0x7E)           # saturated to +-448 * scale
    compare_dequant(gc, st)


def test_e4m3_decode_all_codes():
    """Write every finite E4M3 byte into the K code rows and dequantize."""
    case = Case(B=1, Hq=1, Hkv=1, D=128, dtype="f32", k=(F8, 8, 0, 0), v=(F8, 8, 0, 0))
    gc = GpuCache(case, cap=64)
    ks = np.array([1.0], np.float32)
    z = np.zeros((1, 1, 2, 128), np.float32)
    gc.append(z, z, 0, ks, ks)                     # scale 1.0 stored, T = 2
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    rows = codes.reshape(2, 127)
    buf = np.zeros((2, 128), np.uint8)
    buf[:, :127] = rows
    import torch
    gc.arena[gc.layout.k_codes: gc.layout.k_codes + 256] = torch.from_numpy(buf.reshape(-1)).cuda()
    kd, _ = gc.dequantize(2)
    from oracle import quant as OQ
    assert np.array_equal(kd[0, 0, :, :127], OQ.e4m3_decode(rows))


def test_e5m2_decode_all_codes_and_saturation():
    """Every finite E5M2 byte dequantizes to its closed-form value, and values
    beyond +-57344 saturate (no scale is stored but 1.0)."""
    import torch
    from oracle import quant as OQ
    case = Case(B=1, Hq=1, Hkv=1, D=128, dtype="f32", k=(E5, 8, 0, 0), v=(E5, 8, 0, 0))
    gc = GpuCache(case, cap=64)
    (Kf, _), (Vf, _) = W.random_case(6, 1, 1, 8, 128, dtype="f32")
    Kf = Kf.copy()
    Kf[0, 0, 2:4] *= 1e5                             # beyond the range
    gc.append(Kf[:, :, :4], Vf[:, :, :4], 0)
    st = OC.quantize_cache(case.oracle_cfg(), Kf, Vf, 4)
    compare_sections(gc, st)
    compare_dequant(gc, st)
    assert np.any((st["k"]["codes"][0, 0, 2:4] & 0x7F) == 0x7B)
    codes = np.array([c for c in range(256) if (c & 0x7F) < 0x7C], dtype=np.uint8)   # 248 finite
    rows = np.zeros((2, 128), np.uint8)
    rows.reshape(-1)[:codes.size] = codes
    gc.arena[gc.layout.k_codes: gc.layout.k_codes + 256] = torch.from_numpy(rows.reshape(-1)).cuda()
    kd, _ = gc.dequantize(2)
    assert np.array_equal(kd[0, 0], OQ.e5m2_decode(rows))


def test_attention_deterministic_and_split_invariant():
    case = Case(B=2, Hq=8, Hkv=2, D=128, dtype="bf16", k=(A, 4, CH, 128), v=(A, 4, TOK, 0), R=128)
    gc, st, _ = run_case(case, 1000, [1000], seed=11)
    (qf, qp) = W.random_queries(11, case.B, case.Hq, case.D, dtype="bf16")
    a = gc.attention(qp)
    b = gc.attention(qp)
    assert np.array_equal(a, b)
    for s in (1, 3, 16):
        for kern in (K.KERNEL_GENERIC, K.KERNEL_MFMA):
            o = gc.attention(qp, num_splits=s, kernel=kern)
            assert attention_error(o, qf, st, case) <= ATTN_TOL


def test_one_workspace_many_calls():
    """One workspace serves successive calls with different split counts: each
    call has to write every output (out is poisoned with NaN first), agree with
    the oracle, and give the same result for the same split count."""
    import math
    import torch
    case = Case(B=3, Hq=24, Hkv=3, D=128, dtype="bf16", k=(A, 4, CH, 128), v=(A, 4, TOK, 0), R=128)
    T = 2400
    gc, st, _ = run_case(case, T, [T], seed=23, kernels=[K.KERNEL_GENERIC])
    (qf, qp) = W.random_queries(23, case.B, case.Hq, case.D, dtype="bf16")
    from tests.kvq_harness import to_dev
    q = to_dev(qp, case.dtype)
    nbytes = max(K.kvq_workspace_bytes(gc.cfg, T, K.KERNEL_MFMA, s) for s in (1, 2, 3, 7, 16, 37))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty((case.B, case.Hq, case.D), dtype=torch.float32, device="cuda")
    first = None
    for s in (2, 1, 3, 7, 16, 37, 2, 2):
        out.fill_(float("nan"))
        K.kvq_decode_attention(gc.cfg, gc.arena, T, q, out, 1.0 / math.sqrt(case.D), ws, K.KERNEL_MFMA, s)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        assert np.isfinite(o).all(), f"splits={s}: outputs not written"
        assert attention_error(o, qf, st, case) <= ATTN_TOL, s
        if s == 2:
            if first is None:
                first = o
            else:
                assert np.array_equal(o, first), "same split count, different result"


@pytest.mark.parametrize("kern", [K.KERNEL_GENERIC, K.KERNEL_MFMA])
def test_output_dtypes_round_the_fp32_result(kern):
    """fp16 and bf16 outputs are the fp32 result rounded to nearest even (the
    merge converts once, at the end)."""
    import math
    import torch
    from tests.kvq_harness import to_dev
    case = Case(B=2, Hq=8, Hkv=2, D=128, dtype="bf16", k=(A, 2, CH, 32), v=(A, 2, TOK, 32), R=32,
                pre_rope=True)
    gc, st, _ = run_case(case, 700, [700], seed=29, kernels=[K.KERNEL_GENERIC])
    (qf, qp) = W.random_queries(29, case.B, case.Hq, case.D, dtype="bf16")
    q = to_dev(qp, case.dtype)
    sm = 1.0 / math.sqrt(case.D)
    ws = torch.zeros(K.kvq_workspace_bytes(gc.cfg, 700, kern), dtype=torch.uint8, device="cuda")
    ref = torch.full((case.B, case.Hq, case.D), float("nan"), dtype=torch.float32, device="cuda")
    K.kvq_decode_attention(gc.cfg, gc.arena, 700, q, ref, sm, ws, kern)
    for code, tdt in ((K.F16, torch.float16), (K.BF16, torch.bfloat16)):
        cfg = type(gc.cfg).from_buffer_copy(gc.cfg)
        cfg.out_dtype = code
        out = torch.full((case.B, case.Hq, case.D), float("nan"), dtype=tdt, device="cuda")
        K.kvq_decode_attention(cfg, gc.arena, 700, q, out, sm, ws, kern)
        torch.cuda.synchronize()
        assert torch.equal(out, ref.to(tdt)), (kern, tdt)


@pytest.mark.parametrize("name,fmt", [
    ("int2ch32_int2tok32_R32_prerope", dict(k=(A, 2, CH, 32), v=(A, 2, TOK, 32), R=32, pre_rope=True)),
    ("int4ch128_int4tok32_R128", dict(k=(A, 4, CH, 128), v=(A, 4, TOK, 32), R=128)),
    ("int2ch32_int4tok32_R0", dict(k=(A, 2, CH, 32), v=(A, 4, TOK, 32), R=0)),
])
def test_eight_heads_per_kv_head_four_value_groups(name, fmt):
    """8 query heads per kv head with 32-channel value groups: 32 (value
    group, head) PV rows, which the MFMA kernel covers with two A operands."""
    case = Case(B=2, Hq=16, Hkv=2, D=128, dtype="bf16", **fmt)
    gc, st, errs = run_case(case, 1100, _schedule("stream", 1100), seed=37)
    assert K.KERNEL_MFMA in errs, "the MFMA kernel should cover this shape"
    for s in (1, 3):
        out = gc.attention(W.random_queries(37, case.B, case.Hq, case.D, dtype="bf16")[1],
                           kernel=K.KERNEL_MFMA, num_splits=s)
        assert attention_error(out, W.random_queries(37, case.B, case.Hq, case.D, dtype="bf16")[0],
                               st, case) <= ATTN_TOL


@pytest.mark.parametrize("Hq,fmt", [
    (32, dict(k=(A, 4, CH, 128), v=(A, 4, TOK, 0), R=128)),
    (32, dict(k=(F8, 8, 0, 0), v=(F8, 8, 0, 0), R=0)),
    (24, dict(k=(A, 2, CH, 32), v=(A, 2, TOK, 0), R=32, pre_rope=True)),
])
def test_up_to_sixteen_heads_per_kv_head(Hq, fmt):
    """16 (and 12) query heads per kv head with one value group run on the
    MFMA kernel: the 16 query columns and PV rows are the heads."""
    case = Case(B=2, Hq=Hq, Hkv=2, D=128, dtype="bf16", **fmt)
    gc, st, errs = run_case(case, 900, _schedule("stream", 900), seed=43)
    assert K.KERNEL_MFMA in errs, "the MFMA kernel should cover this shape"


@pytest.mark.parametrize("name,fmt,fused", [
    ("int2ch32_int2tok32_R32_prerope", dict(k=(A, 2, CH, 32), v=(A, 2, TOK, 32), R=32, pre_rope=True), True),
    ("int4ch128_int4tok_R128", dict(k=(A, 4, CH, 128), v=(A, 4, TOK, 0), R=128), True),
    ("fp8_e4m3", dict(k=(F8, 8, 0, 0), v=(F8, 8, 0, 0), R=0), True),
    ("e4m3_k_e5m2_v", dict(k=(F8, 8, 0, 0), v=(E5, 8, 0, 0), R=0), True),
    ("fp8_e4m3_R32", dict(k=(F8, 8, 0, 0), v=(F8, 8, 0, 0), R=32), False),
    ("int4tok_int4tok_R0", dict(k=(A, 4, TOK, 0), v=(A, 4, TOK, 0), R=0), False),
    ("int2ch32_int2tok32_R32_prerope_meta16", dict(k=(A, 2, CH, 32), v=(A, 2, TOK, 32), R=32, pre_rope=True,
                                                   meta16=True), True),
])
@pytest.mark.parametrize("splits", [0, 1, 3, 7])
def test_decode_step_equals_append_then_attention(name, fmt, fused, splits):
    """kvq_decode_step (append inside the attention launch when no fold is due)
    leaves the same cache bytes and gives the same output, bit for bit, as
    kvq_quantize_append followed by kvq_decode_attention, over 40 steps that
    cross fold boundaries.  With 3 and 7 splits (chunks of 192 and 64 tokens)
    the new token lands in different splits and the window straddles the
    chunk boundary at 384, so only the work-group owning the new position may
    write it."""
    import math
    import torch
    from tests.kvq_harness import to_dev
    case = Case(B=2, Hq=8, Hkv=2, D=128, dtype="bf16", **fmt)
    T0, n = 360, 40
    (Kf, Kp), (Vf, Vp) = W.random_case(47, case.B, case.Hkv, T0 + n, case.D, dtype="bf16")
    ga, gb = GpuCache(case, cap=T0 + n), GpuCache(case, cap=T0 + n)
    flags = K.CALIBRATE if case.k[0] == F8 else 0
    ga.append(Kp[:, :, :T0], Vp[:, :, :T0], flags)
    gb.append(Kp[:, :, :T0], Vp[:, :, :T0], flags)
    sm = 1.0 / math.sqrt(case.D)
    wa = torch.zeros(K.kvq_workspace_bytes(ga.cfg, T0 + n, 0, splits), dtype=torch.uint8, device="cuda")
    wb = torch.zeros(K.kvq_workspace_bytes(gb.cfg, T0 + n, 0, splits), dtype=torch.uint8, device="cuda")
    oa = torch.empty((case.B, case.Hq, case.D), dtype=torch.float32, device="cuda")
    ob = torch.empty_like(oa)
    n_fused = 0
    for i in range(n):
        t = T0 + i
        kn, vn = to_dev(Kp[:, :, t:t + 1], case.dtype), to_dev(Vp[:, :, t:t + 1], case.dtype)
        q = to_dev(W.random_queries(1000 + i, case.B, case.Hq, case.D, dtype="bf16")[1], case.dtype)
        n_fused += K.kvq_decode_step_fused(ga.cfg, t, 0, splits)
        oa.fill_(float("nan"))
        ob.fill_(float("nan"))
        K.kvq_decode_step(ga.cfg, ga.arena, t, kn, vn, q, oa, sm, wa, 0, splits)
        K.kvq_quantize_append(gb.cfg, gb.arena, t, kn, vn)
        K.kvq_decode_attention(gb.cfg, gb.arena, t + 1, q, ob, sm, wb, 0, splits)
        torch.cuda.synchronize()
        assert torch.equal(ga.arena, gb.arena), (name, t, "cache bytes differ")
        assert torch.isfinite(oa).all() and torch.equal(oa, ob), (name, t, "outputs differ")
    assert (n_fused > 0) == fused, (name, n_fused)
    if fused and case.R:
        assert n_fused < n     # the steps that fold run the append separately


# fp16 scale / zero-point metadata: every metadata staging path of the MFMA
# kernel (value groups 1 / 2 / 4 / 8, two PV row halves, pre-RoPE keys, FP8 on
# one side) and the generic-only formats (symmetric, per-token keys,
# per-tensor), streamed across folds; (name, Hq for Hkv = 2, format, MFMA expected)
META16 = [
    ("int4ch128_int4tok_R128", 8, dict(k=(A, 4, CH, 128), v=(A, 4, TOK, 0), R=128), True),
    ("int4ch128_int4tok64_R128", 8, dict(k=(A, 4, CH, 128), v=(A, 4, TOK, 64), R=128), True),
    ("int2ch32_int2tok32_R32", 8, dict(k=(A, 2, CH, 32), v=(A, 2, TOK, 32), R=32), True),
    ("prerope_int2ch32_int2tok32_R32", 8, dict(k=(A, 2, CH, 32), v=(A, 2, TOK, 32), R=32, pre_rope=True), True),
    ("int8ch64_int8tok16_R64", 4, dict(k=(A, 8, CH, 64), v=(A, 8, TOK, 16), R=64), True),
    ("pv2_int4ch128_int4tok32_R128", 16, dict(k=(A, 4, CH, 128), v=(A, 4, TOK, 32), R=128), True),
    ("int4ch128_e4m3_R128", 8, dict(k=(A, 4, CH, 128), v=(F8, 8, 0, 0), R=128), True),
    ("fp8k_int4tok", 8, dict(k=(F8, 8, 0, 0), v=(A, 4, TOK, 0), R=0), True),
    ("int4ch128_e5m2_R128", 8, dict(k=(A, 4, CH, 128), v=(E5, 8, 0, 0), R=128), None),
    ("sym8tok_sym8tok", 8, dict(k=(S, 8, TOK, 0), v=(S, 8, TOK, 32), R=0), None),
    ("int4tok32_int2tok_R64", 8, dict(k=(A, 4, TOK, 32), v=(A, 2, TOK, 64), R=64), None),
]


@pytest.mark.parametrize("name,Hq,fmt,mfma", META16, ids=[m[0] for m in META16])
def test_fp16_metadata(name, Hq, fmt, mfma):
    """Codes, fp16 scales / zero-points and dequantized caches bit-exact against
    the oracle's fp16 rule; attention within tolerance on both kernels."""
    case = Case(B=2, Hq=Hq, Hkv=2, D=128, dtype="bf16", meta16=True, **fmt)
    T = 1100
    gc, st, errs = run_case(case, T, _schedule("stream", T), seed=zlib.crc32(name.encode()) % 1000)
    if mfma:
        assert K.KERNEL_MFMA in errs, "the MFMA kernel should cover this shape"
        for s in (1, 3):   # splits that start inside key groups
            out = gc.attention(W.random_queries(zlib.crc32(name.encode()) % 1000, case.B, case.Hq, case.D,
                                                dtype="bf16")[1], kernel=K.KERNEL_MFMA, num_splits=s)
            assert attention_error(out, W.random_queries(zlib.crc32(name.encode()) % 1000, case.B, case.Hq,
                                                         case.D, dtype="bf16")[0], st, case) <= ATTN_TOL


def test_fp16_metadata_one_shot_per_tensor():
    case = Case(B=2, Hq=4, Hkv=2, D=128, dtype="f32", meta16=True, k=(A, 4, TEN, 0), v=(S, 8, TEN, 0))
    run_case(case, 300, [300], seed=5)


@pytest.mark.parametrize("name,fmt", [
    ("e4m3_R0", dict(k=(F8, 8, 0, 0), v=(F8, 8, 0, 0), R=0)),
    ("e4m3_R32", dict(k=(F8, 8, 0, 0), v=(F8, 8, 0, 0), R=32)),
    ("e5m2_R0", dict(k=(E5, 8, 0, 0), v=(E5, 8, 0, 0), R=0)),
])
@pytest.mark.parametrize("T", [40, 161, 1100])
def test_fp8_step_interleave_over_split_counts(name, fmt, T):
    """FP8 caches hand the 32-token steps of a split to the four wavefronts in
    turn: splits with fewer steps than wavefronts, window steps starting at any
    offset, and one to many splits all stay within tolerance of the oracle."""
    case = Case(B=2, Hq=8, Hkv=2, D=128, dtype="bf16", **fmt)
    seed = zlib.crc32(f"{name}{T}".encode()) % 1000
    gc, st, errs = run_case(case, T, _schedule("stream", T), seed=seed)
    qf, qp = W.random_queries(seed, case.B, case.Hq, case.D, dtype="bf16")
    for s in (1, 2, 3, 5, 16, 64):
        out = gc.attention(qp, kernel=K.KERNEL_MFMA, num_splits=s)
        assert attention_error(out, qf, st, case) <= ATTN_TOL, (name, T, s)


# Quantizer corner cases (workloads.edge_case_inputs): constant groups (the
# 1e-8 range floor), a group of -0.0, fp16-subnormal ranges (fp16 metadata then
# stores subnormal scales), exact half-way ties, -0.0 mixed with positives,
# and values near or beyond the fp16 range.  Codes, scales, zero-points, window
# and dequantized values must match the oracle bit for bit; attention stays
# within tolerance on every kernel that serves the format.
# (name, format, code bits of the tie pattern, values beyond fp16, FP8 mode)
EDGE = [
    ("int2ch32_int2tok32_R32", dict(k=(A, 2, CH, 32), v=(A, 2, TOK, 32), R=32), 2, False),
    ("int2ch32_int2tok32_R32_meta16", dict(k=(A, 2, CH, 32), v=(A, 2, TOK, 32), R=32, meta16=True), 2, False),
    ("prerope_int2ch32_int2tok32_R32", dict(k=(A, 2, CH, 32), v=(A, 2, TOK, 32), R=32, pre_rope=True), 2, False),
    ("int4ch128_int4tok_R128", dict(k=(A, 4, CH, 128), v=(A, 4, TOK, 0), R=128), 4, False),
    ("int4ch128_int4tok_R128_meta16", dict(k=(A, 4, CH, 128), v=(A, 4, TOK, 0), R=128, meta16=True), 4, False),
    ("int8ch64_int8tok16_R64", dict(k=(A, 8, CH, 64), v=(A, 8, TOK, 16), R=64), 8, False),
    ("int8ch64_int8tok16_R64_meta16", dict(k=(A, 8, CH, 64), v=(A, 8, TOK, 16), R=64, meta16=True), 8, False),
    ("sym8tok_sym8tok32", dict(k=(S, 8, TOK, 0), v=(S, 8, TOK, 32), R=0), 8, True),
    ("int4tok_int2tok32_R0_big", dict(k=(A, 4, TOK, 0), v=(A, 2, TOK, 32), R=0), 4, True),
    ("int4tok_int2tok32_R0_big_meta16", dict(k=(A, 4, TOK, 0), v=(A, 2, TOK, 32), R=0, meta16=True), 4, True),
    ("sym8tok_sym8tok32_big_meta16", dict(k=(S, 8, TOK, 0), v=(S, 8, TOK, 32), R=0, meta16=True), 8, True),
    ("fp8_e4m3_calibrated", dict(k=(F8, 8, 0, 0), v=(F8, 8, 0, 0), R=0), 4, False),
    ("fp8_e5m2_big", dict(k=(E5, 8, 0, 0), v=(E5, 8, 0, 0), R=0), 4, True),
]


@pytest.mark.parametrize("name,fmt,bits,big", EDGE, ids=[e[0] for e in EDGE])
@pytest.mark.parametrize("sched", ["oneshot", "stream"])
def test_quantizer_edge_cases(name, fmt, bits, big, sched):
    case = Case(B=1, Hq=8, Hkv=2, D=128, dtype="f32", **fmt)
    T = 300
    Kf, Vf = W.edge_case_inputs(zlib.crc32(name.encode()) % 1000, case.B, case.Hkv, T, case.D, bits, big=big)
    # the query ignores key channels 4 and 5 (channel 5 holds values near or
    # beyond the fp16 range, and RoPE mixes it into its pair partner 4), so the
    # logits stay O(1) and the attention check measures the cache rather than
    # fp32 rounding of logits in the thousands
    qf, _ = W.random_queries(2, case.B, case.Hq, case.D)
    qf = qf.copy()
    qf[..., 4:6] = 0.0
    _, st, _ = run_case(case, T, _schedule(sched, T), seed=1, inputs=((Kf, Kf), (Vf, Vf)), queries=(qf, qf))
    # the planted groups reached the encoders: ties rounded to even somewhere,
    # a constant group stored the range floor
    if fmt["k"][0] == A and fmt["k"][2] == CH and st["Tq"] >= fmt["k"][3]:
        s_k = np.asarray(st["k"]["scale"])[0, 0, 0]
        assert s_k[0] == np.float32(np.float32(1e-8) / np.float32(2 ** bits - 1)) or fmt.get("meta16")
        codes = st["k"]["codes"][0, 0, :32, 3]
        assert set(codes.tolist()) <= set(range(2 ** bits)) and (codes % 2 == 0).sum() > (codes % 2 == 1).sum()


def _fp8_grid(e_bits, m_bits, vmax):
    """Positive finite values of an FP8 format (bias 2^(e_bits-1) - 1,
    subnormals below the first binade), up to vmax, from its definition."""
    bias = 2 ** (e_bits - 1) - 1
    vals = set()
    for e in range(0, 2 ** e_bits):
        for m in range(2 ** m_bits):
            v = (m / 2 ** m_bits) * 2.0 ** (1 - bias) if e == 0 else (1 + m / 2 ** m_bits) * 2.0 ** (e - bias)
            if v <= vmax:
                vals.add(v)
    return np.array(sorted(vals), np.float64)


@pytest.mark.parametrize("fmt8", ["e4m3", "e5m2"])
def test_fp8_codes_at_every_value_and_tie(fmt8):
    """With a unit scale the encoder sees every representable value, every
    midpoint between neighbours (ties go to the even code), the fp32 values
    either side of each midpoint, zeros of both signs, the saturation region
    past the largest value and the negatives of all of them: the codes must
    equal the oracle's bit for bit."""
    e_bits, m_bits, vmax = (4, 3, 448.0) if fmt8 == "e4m3" else (5, 2, 57344.0)
    g = _fp8_grid(e_bits, m_bits, vmax)
    mids = ((g[:-1] + g[1:]) / 2).astype(np.float32)
    vals = [g.astype(np.float32), mids, np.nextafter(mids, np.float32(np.inf)),
            np.nextafter(mids, np.float32(-np.inf)),
            np.array([0.0, vmax * 1.03, vmax * 1.0625, vmax * 4, 1e30], np.float32)]
    pos = np.concatenate(vals).astype(np.float32)
    x = np.concatenate([pos, -pos]).astype(np.float32)
    D, Hkv = 128, 2
    T = -(-x.size // (D * Hkv))
    flat = np.zeros(Hkv * T * D, np.float32)
    flat[:x.size] = x
    flat[x.size:] = -0.0
    Kf = flat.reshape(1, Hkv, T, D)
    Vf = Kf[:, ::-1].copy()          # the same values, the other head first
    spec = (F8, 8, 0, 0) if fmt8 == "e4m3" else (E5, 8, 0, 0)
    case = Case(B=1, Hq=2, Hkv=Hkv, D=D, dtype="f32", k=spec, v=spec, R=0)
    gc = GpuCache(case, cap=T)
    one = np.ones(Hkv, np.float32)
    if fmt8 == "e4m3":
        gc.append(Kf, Vf, 0, one, one)
        st = OC.quantize_cache(case.oracle_cfg(), Kf, Vf, T, k_scale=one, v_scale=one)
    else:
        gc.append(Kf, Vf, 0)
        st = OC.quantize_cache(case.oracle_cfg(), Kf, Vf, T)
    compare_sections(gc, st)
    codes = np.asarray(st["k"]["codes"]).ravel()
    assert (codes == 0x80).any() and (codes == 0x00).any()          # both zeros reached the encoder
