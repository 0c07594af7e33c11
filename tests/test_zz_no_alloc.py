"""kvq_decode_attention_static (no workspace argument; the split partials live
in the library's own device array) against kvq_decode_attention on the same
caches: bit-identical outputs on two calls in a row, the second with a
smaller input, and a request larger than the array refused before any launch."""
import math

import numpy as np
import pytest
import torch

import quantized_decode_attention_05_amd as K
import workloads as W
from tests.kvq_harness import ATTN_TOL, Case, GpuCache, attention_error, say, to_dev
from oracle import cache as OC

pytestmark = pytest.mark.gpu

A, F8, CH, TOK = K.INT_ASYM, K.FP8_E4M3, K.PER_CHANNEL, K.PER_TOKEN


def _pair(case, T, seed, splits):
    """(static output, workspace output, oracle state, queries) of one cache."""
    (Kf, Kp), (Vf, Vp) = W.random_case(seed, case.B, case.Hkv, T, case.D, dtype=case.dtype)
    qf, qp = W.random_queries(seed, case.B, case.Hq, case.D, dtype=case.dtype)
    gc = GpuCache(case, cap=T)
    gc.append(Kp, Vp, K.CALIBRATE if case.k[0] == F8 else 0)
    q = to_dev(qp, case.dtype)
    sm = 1.0 / math.sqrt(case.D)
    o_ws = torch.full((case.B, case.Hq, case.D), float("nan"), dtype=torch.float32, device="cuda")
    o_st = torch.full_like(o_ws, float("nan"))
    ws = torch.zeros(K.kvq_workspace_bytes(gc.cfg, T, 0, splits), dtype=torch.uint8, device="cuda")
    K.kvq_decode_attention(gc.cfg, gc.arena, T, q, o_ws, sm, ws, 0, splits)
    K.kvq_decode_attention_static(gc.cfg, gc.arena, T, q, o_st, sm, 0, splits)
    torch.cuda.synchronize()
    st = OC.quantize_cache(case.oracle_cfg(), Kf, Vf, T, calibrate_tokens=T if case.k[0] == F8 else 0)
    return o_st.cpu().numpy(), o_ws.cpu().numpy(), st, qf


FORMATS = [
    ("int2_prerope", dict(k=(A, 2, CH, 32), v=(A, 2, TOK, 32), R=32, pre_rope=True)),
    ("int4_ch128", dict(k=(A, 4, CH, 128), v=(A, 4, TOK, 0), R=128)),
    ("fp8_e4m3", dict(k=(F8, 8, 0, 0), v=(F8, 8, 0, 0), R=0)),
]


@pytest.mark.parametrize("name,fmt", FORMATS, ids=[f[0] for f in FORMATS])
@pytest.mark.parametrize("splits", [0, 5])
def test_static_scratch_matches_workspace_entry_point(name, fmt, splits):
    big = Case(B=4, Hq=16, Hkv=4, D=128, dtype="bf16", **fmt)
    small = Case(B=2, Hq=8, Hkv=2, D=128, dtype="bf16", **fmt)
    for case, T, seed in ((big, 1500, 71), (small, 333, 72)):   # second call: smaller input
        say(f"[no-alloc] {name} B={case.B} T={T} splits={splits}")
        o_st, o_ws, st, qf = _pair(case, T, seed, splits)
        assert np.isfinite(o_st).all()
        assert np.array_equal(o_st, o_ws), "static-scratch output differs from the workspace entry point"
        assert attention_error(o_st, qf, st, case) <= ATTN_TOL


def test_static_scratch_refuses_requests_beyond_the_array():
    case = Case(B=64, Hq=64, Hkv=8, D=128, dtype="bf16", k=(A, 4, CH, 128), v=(A, 4, TOK, 0), R=128)
    cfg = case.lib_cfg(131072)
    need = K.kvq_workspace_bytes(cfg, 131072, 0, 64)
    assert need > K.STATIC_WORKSPACE_BYTES
    arena = torch.empty(256, dtype=torch.uint8, device="cuda")   # never touched: refused first
    q = torch.zeros((case.B, case.Hq, case.D), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((case.B, case.Hq, case.D), dtype=torch.float32, device="cuda")
    import ctypes as C
    o = K.AttnOptions()
    o.num_splits = 64
    st = K._lib.raw.kvq_decode_attention_static(C.byref(cfg), C.c_void_p(arena.data_ptr()), 131072,
                                                C.c_void_p(q.data_ptr()), C.c_void_p(out.data_ptr()),
                                                0.088, C.byref(o), None)
    assert st == -6
