"""More query heads per kv head than one MFMA work-group's PV rows hold: the
heads of a kv head are split into groups (one work-group per group, each
streaming the kv head's cache), which covers every head count on the MFMA
kernel.  Each case is checked against the oracle like the other formats
(codes bit-exact, attention within 2e-3 max relative L2 on both kernels) and
the group sizes span the branches of the split: two PV row halves, groups of
the full row count, near-equal groups, a short last group, and one kv head
shared by every query head (multi-query attention)."""
import math

import pytest

import quantized_decode_attention_05_amd as K
import workloads as W
from tests.kvq_harness import ATTN_TOL, Case, GpuCache, attention_error
from tests.test_gpu_parity import _schedule, run_case

pytestmark = pytest.mark.gpu

A, F8 = K.INT_ASYM, K.FP8_E4M3
CH, TOK = K.PER_CHANNEL, K.PER_TOKEN

# (name, Hq, Hkv, format); the comment gives the heads per work-group
CASES = [
    # one value group: 16 rows per work-group -> 2 groups of 16
    ("int4ch128_int4tok_nrep32", 64, 2, dict(k=(A, 4, CH, 128), v=(A, 4, TOK, 0), R=128)),
    # FP8 values (one group): 20 heads -> 2 groups of 10
    ("fp8_nrep20", 40, 2, dict(k=(F8, 8, 0, 0), v=(F8, 8, 0, 0), R=0)),
    # four INT2 value groups, two PV row halves: 16 heads -> 2 groups of 8
    ("prerope_int2ch32_int2tok32_nrep16", 32, 2, dict(k=(A, 2, CH, 32), v=(A, 2, TOK, 32), R=32,
                                                       pre_rope=True)),
    # four INT4 value groups, 12 heads (not a multiple of 8) -> 3 groups of 4
    ("int4ch128_int4tok32_nrep12", 24, 2, dict(k=(A, 4, CH, 128), v=(A, 4, TOK, 32), R=128)),
    # four INT8 value groups: 6 heads -> 2 groups of 3
    ("int8ch64_int8tok32_nrep6", 12, 2, dict(k=(A, 8, CH, 64), v=(A, 8, TOK, 32), R=64)),
    # eight value groups: 5 heads -> groups of 2, 2 and 1
    ("int4ch128_int4tok16_nrep5", 10, 2, dict(k=(A, 4, CH, 128), v=(A, 4, TOK, 16), R=128)),
    # one kv head for 33 query heads, FP8 with a window -> 3 groups of 11
    ("mqa_fp8_R32_nrep33", 33, 1, dict(k=(F8, 8, 0, 0), v=(F8, 8, 0, 0), R=32)),
]


@pytest.mark.parametrize("name,Hq,Hkv,fmt", CASES, ids=[c[0] for c in CASES])
def test_head_groups_match_the_oracle(name, Hq, Hkv, fmt):
    case = Case(B=2, Hq=Hq, Hkv=Hkv, D=128, dtype="bf16", **fmt)
    T = 777
    gc, st, errs = run_case(case, T, _schedule("stream", T), seed=53)
    assert K.KERNEL_MFMA in errs, "the MFMA kernel should cover this shape"
    qf, qp = W.random_queries(53, case.B, case.Hq, case.D, dtype="bf16")
    for s in (1, 3, 13):
        out = gc.attention(qp, kernel=K.KERNEL_MFMA, num_splits=s)
        assert attention_error(out, qf, st, case) <= ATTN_TOL, (name, s)


def test_decode_step_with_head_groups_appends_before_the_launch():
    """With several head groups per kv head the decode step does not append
    inside the attention launch (the groups of one split would read the new
    token while one of them writes it): it appends first, and gives the same
    bytes and output as kvq_quantize_append then kvq_decode_attention."""
    import torch
    from tests.kvq_harness import to_dev
    case = Case(B=2, Hq=64, Hkv=2, D=128, dtype="bf16", k=(A, 4, CH, 128), v=(A, 4, TOK, 0), R=128)
    T0, n = 300, 12
    (Kf, Kp), (Vf, Vp) = W.random_case(59, case.B, case.Hkv, T0 + n, case.D, dtype="bf16")
    ga, gb = GpuCache(case, cap=T0 + n), GpuCache(case, cap=T0 + n)
    ga.append(Kp[:, :, :T0], Vp[:, :, :T0], 0)
    gb.append(Kp[:, :, :T0], Vp[:, :, :T0], 0)
    sm = 1.0 / math.sqrt(case.D)
    wa = torch.zeros(K.kvq_workspace_bytes(ga.cfg, T0 + n, 0, 0), dtype=torch.uint8, device="cuda")
    wb = torch.zeros(K.kvq_workspace_bytes(gb.cfg, T0 + n, 0, 0), dtype=torch.uint8, device="cuda")
    oa = torch.empty((case.B, case.Hq, case.D), dtype=torch.float32, device="cuda")
    ob = torch.empty_like(oa)
    for i in range(n):
        t = T0 + i
        assert K.kvq_decode_step_fused(ga.cfg, t, 0, 0) == 0
        kn, vn = to_dev(Kp[:, :, t:t + 1], case.dtype), to_dev(Vp[:, :, t:t + 1], case.dtype)
        q = to_dev(W.random_queries(2000 + i, case.B, case.Hq, case.D, dtype="bf16")[1], case.dtype)
        oa.fill_(float("nan"))
        ob.fill_(float("nan"))
        K.kvq_decode_step(ga.cfg, ga.arena, t, kn, vn, q, oa, sm, wa, 0, 0)
        K.kvq_quantize_append(gb.cfg, gb.arena, t, kn, vn)
        K.kvq_decode_attention(gb.cfg, gb.arena, t + 1, q, ob, sm, wb, 0, 0)
        torch.cuda.synchronize()
        assert torch.equal(ga.arena, gb.arena), (t, "cache bytes differ")
        assert torch.isfinite(oa).all() and torch.equal(oa, ob), (t, "outputs differ")
