"""C-ABI checks that need no GPU: symbols, validation, layout, byte accounting.

Every call here either fails validation (which runs on the host before any HIP
call) or is a host-only query, so nothing is launched.
"""
import ctypes as C
import json
import os
import re

import numpy as np
import pytest

import quantized_decode_attention_05_amd as K
from quantized_decode_attention_05_amd import _lib
from oracle import cache as OC

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "kvq.h")


def _cfg(**kw):
    base = dict(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, max_tokens=1024,
                k=(K.INT_ASYM, 4, K.PER_CHANNEL, 32), v=(K.INT_ASYM, 4, K.PER_TOKEN, 32),
                residual=32)
    base.update(kw)
    return K.make_config(**base)


def test_header_symbols_exported():
    text = open(HDR).read()
    declared = set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]*?\b(kvq_\w+)\s*\(", text, re.M))
    assert declared, "no declarations parsed"
    for name in declared:
        assert hasattr(_lib.raw, name), name
    assert set(K.EXPORTED) == declared


def test_struct_sizes_match_c_layout():
    assert C.sizeof(K.Config) == 88
    assert C.sizeof(K.Layout) == 136
    assert C.sizeof(K.TensorSpec) == 16
    assert C.sizeof(K.AttnOptions) == 32


def test_status_strings():
    for s in range(-7, 1):
        assert K.kvq_status_string(s) != "unknown status"
    assert K.kvq_status_string(-99) == "unknown status"


@pytest.mark.parametrize("bad", [
    dict(head_dim=96), dict(num_q_heads=7), dict(num_kv_heads=0), dict(num_q_heads=514, num_kv_heads=2),
    dict(k=(K.INT_ASYM, 3, K.PER_CHANNEL, 32)), dict(k=(K.INT_SYM, 4, K.PER_CHANNEL, 0)),
    dict(v=(K.INT_ASYM, 4, K.PER_TOKEN, 24)), dict(v=(K.INT_ASYM, 4, K.PER_TOKEN, 4)),
    dict(k=(K.NONE, 8, 0, 0)), dict(k=(K.FP8_E4M3, 4, 0, 0)), dict(k=(7, 8, 0, 0)),
    dict(residual=48),                                     # R % G != 0
    dict(residual=-1), dict(max_tokens=0), dict(in_dtype=5),
    dict(k=(K.INT_ASYM, 4, K.PER_CHANNEL, 0), residual=0),  # whole axis with a per-channel V group? no: with G V token
    dict(k=(K.INT_ASYM, 4, K.PER_TENSOR, 0), residual=32),
    dict(k=(K.INT_ASYM, 4, K.PER_CHANNEL, 32), v=(K.INT_ASYM, 4, K.PER_CHANNEL, 64)),
    dict(pre_rope_k=True, rope_base=0.0),
])
def test_invalid_configs(bad):
    cfg = _cfg(**bad)
    if bad == dict(k=(K.INT_ASYM, 4, K.PER_CHANNEL, 0), residual=0):
        # whole-axis K with a per-token V group is fine; make V per-channel grouped to be invalid
        cfg = _cfg(k=(K.INT_ASYM, 4, K.PER_CHANNEL, 0), v=(K.INT_ASYM, 4, K.PER_CHANNEL, 32), residual=0)
    assert K.kvq_validate_config(cfg) == -1
    n = C.c_size_t()
    assert _lib.raw.kvq_arena_bytes(C.byref(cfg), C.byref(n)) == -1


def _append(cfg, arena=0x100000, t0=0, n=4, k=0x200000, v=0x300000, ks=None, vs=None, flags=0):
    return _lib.raw.kvq_quantize_append(C.byref(cfg), arena, t0, n, k, v, ks, vs, flags, None)


def test_append_validation_paths():
    cfg = _cfg()
    assert _append(cfg, t0=1020, n=8) == -3                      # capacity
    assert _append(cfg, t0=-1) == -1
    assert _append(cfg, n=-2) == -1
    assert _append(cfg, n=0) == 0                                # no-op, no HIP call
    assert _append(cfg, arena=None) == -5
    assert _append(cfg, arena=0x100010) == -4                    # arena not 256-aligned
    assert _append(cfg, k=0x200004) == -4                        # input not 16-aligned
    assert _append(cfg, flags=K.CALIBRATE) == -1                 # calibrate without FP8
    assert _append(cfg, flags=8) == -1
    fp8 = _cfg(k=(K.FP8_E4M3, 8, 0, 0), v=(K.FP8_E4M3, 8, 0, 0), residual=0)
    assert _append(fp8, t0=8, flags=K.CALIBRATE) == -1           # calibrate only at t0 == 0
    assert _append(fp8, t0=8, ks=0x400000) == -1                 # scales only at t0 == 0
    assert _append(fp8, ks=0x400000, flags=K.CALIBRATE) == -1
    e5 = _cfg(k=(K.FP8_E5M2, 8, 0, 0), v=(K.FP8_E5M2, 8, 0, 0), residual=0)
    assert _append(e5, ks=0x400000) == -1                        # E5M2 takes no scale
    assert _append(e5, vs=0x400000) == -1
    mix = _cfg(k=(K.FP8_E4M3, 8, 0, 0), v=(K.FP8_E5M2, 8, 0, 0), residual=0)
    assert _append(mix, vs=0x400000) == -1
    assert _append(_cfg(k=(K.FP8_E5M2, 4, 0, 0)), t0=0) == -1    # FP8 is 8 bits
    whole = _cfg(k=(K.INT_ASYM, 4, K.PER_CHANNEL, 0), v=(K.INT_ASYM, 4, K.PER_TOKEN, 0), residual=0)
    assert _append(whole, t0=16) == -2                           # would rescale history
    tens = _cfg(k=(K.INT_SYM, 8, K.PER_TENSOR, 0), v=(K.NONE, 16, 0, 0), residual=0)
    assert _append(tens, t0=1) == -2


def test_attention_validation_paths():
    cfg = _cfg()
    raw = _lib.raw
    opt = K.AttnOptions()
    ws = K.kvq_workspace_bytes(cfg, 500)

    def call(T=500, arena=0x100000, q=0x200000, out=0x300000, sm=0.088, w=0x400000, wb=ws, o=opt):
        return raw.kvq_decode_attention(C.byref(cfg), arena, T, q, out, sm, w, wb, C.byref(o), None)

    assert call(T=0) == -3
    assert call(T=1025) == -3
    assert call(sm=0.0) == -1
    assert call(sm=float("nan")) == -1
    assert call(q=None) == -5
    assert call(out=0x300008) == -4
    assert call(w=0x400010) == -4
    assert call(wb=ws - 1) == -6
    bad = K.AttnOptions(); bad.kernel = 5
    assert call(o=bad) == -1
    bad = K.AttnOptions(); bad.reserved[2] = 1
    assert call(o=bad) == -1
    bad = K.AttnOptions(); bad.kernel = 2
    fp32none = _cfg(k=(K.NONE, 32, 0, 0), v=(K.NONE, 32, 0, 0), residual=0)
    assert raw.kvq_decode_attention(C.byref(fp32none), 0x100000, 10, 0x200000, 0x300000, 0.1,
                                    0x400000, 1 << 20, C.byref(bad), None) == -2


def test_dequantize_validation_paths():
    cfg = _cfg()
    raw = _lib.raw
    assert raw.kvq_dequantize(C.byref(cfg), 0x100000, 2000, 0x200000, None, None) == -3
    assert raw.kvq_dequantize(C.byref(cfg), 0x100000, 0, 0x200000, None, None) == 0
    assert raw.kvq_dequantize(C.byref(cfg), 0x100000, 10, None, None, None) == 0
    assert raw.kvq_dequantize(C.byref(cfg), None, 10, 0x200000, None, None) == -5
    assert raw.kvq_dequantize(C.byref(cfg), 0x100000, 10, 0x200008, None, None) == -4


def test_layout_sections_disjoint_and_sized():
    for cfg in [_cfg(), _cfg(k=(K.FP8_E4M3, 8, 0, 0), v=(K.FP8_E4M3, 8, 0, 0), residual=0),
                _cfg(pre_rope_k=True, k=(K.INT_ASYM, 2, K.PER_CHANNEL, 32), v=(K.INT_ASYM, 2, K.PER_TOKEN, 32)),
                _cfg(k=(K.INT_SYM, 8, K.PER_TENSOR, 0), v=(K.NONE, 32, 0, 0), residual=0)]:
        lay = K.kvq_arena_layout(cfg)
        B, H, D, Tc = cfg.batch, cfg.num_kv_heads, cfg.head_dim, lay.token_capacity
        assert Tc % 32 == 0 and Tc >= cfg.max_tokens
        bk = cfg.k.bits if cfg.k.scheme in (K.NONE, K.INT_ASYM) else 8
        bv = cfg.v.bits if cfg.v.scheme in (K.NONE, K.INT_ASYM) else 8
        assert lay.k_row_bytes == D * bk // 8 and lay.v_block_bytes == 32 * D * bv // 8
        secs = [(n, getattr(lay, n)) for n in ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale",
                                               "v_zero", "ring_k", "ring_v", "rope", "fp8_calib")]
        present = [(n, o) for n, o in secs if o != 2 ** 64 - 1]
        offs = [o for _, o in present]
        assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
        assert lay.total_bytes == K.kvq_arena_bytes(cfg)
        assert present[1][1] - present[0][1] >= B * H * Tc * lay.k_row_bytes


def test_fp16_cache_bytes_per_token_pin():
    """Scheme NONE at fp16 reproduces 2 * kv_heads * head_dim * 2 bytes per token per
    layer, i.e. 327,680 bytes/token for 80 Llama-3.1-70B layers."""
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "kv_bytes_facts.json")))
    T = 131072
    cfg = K.make_config(batch=1, num_q_heads=64, num_kv_heads=8, head_dim=128, max_tokens=T,
                        k=(K.NONE, 16, 0, 0), v=(K.NONE, 16, 0, 0))
    per_layer = K.kvq_arena_bytes(cfg)
    assert per_layer * 80 / T == g["fp16_bytes_per_token"]
    assert per_layer * 80 / 2 ** 30 == g["fp16_gib_at_128k"]
    fp8 = K.make_config(batch=1, num_q_heads=64, num_kv_heads=8, head_dim=128, max_tokens=T,
                        k=(K.FP8_E4M3, 8, 0, 0), v=(K.FP8_E4M3, 8, 0, 0))
    lay = K.kvq_arena_layout(fp8)
    code_bytes = lay.k_scale - lay.k_codes + (lay.v_scale - lay.v_codes)
    assert code_bytes * 80 / 2 ** 30 == g["fp8_gib_at_128k"]


@pytest.mark.parametrize("k,v,R", [
    ((K.INT_ASYM, 4, K.PER_CHANNEL, 128), (K.INT_ASYM, 4, K.PER_TOKEN, 0), 128),
    ((K.INT_ASYM, 2, K.PER_CHANNEL, 32), (K.INT_ASYM, 2, K.PER_TOKEN, 32), 32),
    ((K.INT_ASYM, 2, K.PER_CHANNEL, 32), (K.INT_ASYM, 2, K.PER_TOKEN, 32), 0),
    ((K.FP8_E4M3, 8, 0, 0), (K.FP8_E4M3, 8, 0, 0), 0),
    ((K.INT_ASYM, 4, K.PER_TOKEN, 0), (K.INT_ASYM, 4, K.PER_TOKEN, 0), 64),
    ((K.INT_SYM, 8, K.PER_CHANNEL, 0), (K.INT_SYM, 8, K.PER_TOKEN, 0), 0),
])
def test_quantized_tokens_matches_oracle(k, v, R):
    cfg = _cfg(k=k, v=v, residual=R, max_tokens=5000)
    ocfg = OC.Cfg(2, 8, 2, 128, OC.Spec(*k), OC.Spec(*v), R=R)
    assert K.kvq_arena_layout(cfg).ring_slots == OC.ring_slots(ocfg)
    for T in list(range(0, 300)) + [4095, 4096, 4097, 5000]:
        assert K.kvq_quantized_tokens(cfg, T) == OC.quantized_tokens(ocfg, T)
    with pytest.raises(K.KvqError):
        K.kvq_quantized_tokens(cfg, 5001)


@pytest.mark.parametrize("fmt", [dict(), dict(k=(K.FP8_E4M3, 8, 0, 0), v=(K.FP8_E4M3, 8, 0, 0), residual=0)])
def test_workspace_monotone_in_T(fmt):
    for B, H in [(1, 8), (2, 2), (32, 8)]:
        cfg = _cfg(batch=B, num_kv_heads=H, num_q_heads=4 * H, max_tokens=140000, **fmt)
        prev = 0
        for T in list(range(1, 2000, 13)) + [8193, 32769, 131072, 131136, 140000]:
            for kern in (1,):
                ws = K.kvq_workspace_bytes(cfg, T, kern)
                assert ws >= prev
                prev = ws


@pytest.mark.parametrize("Hq,Hkv,fmt", [
    (64, 2, dict()),                                                             # 32 per kv head
    (33, 1, dict(k=(K.FP8_E4M3, 8, 0, 0), v=(K.FP8_E4M3, 8, 0, 0), residual=0)),  # multi-query
    (512, 2, dict()),                                                            # the limit, 256
    (8, 2, dict(v=(K.INT_ASYM, 4, K.PER_TOKEN, 16))),                            # 4 x 8 value groups
])
def test_any_heads_per_kv_head_run_on_both_kernels(Hq, Hkv, fmt):
    """Host-only: query heads beyond one work-group's rows are split into head
    groups on both kernels, so every such config is accepted and sized, and a
    decode step with several groups appends before the launch."""
    cfg = _cfg(num_q_heads=Hq, num_kv_heads=Hkv, **fmt)
    for kern in (K.KERNEL_GENERIC, K.KERNEL_MFMA):
        ws = K.kvq_workspace_bytes(cfg, 1000, kern, 3)
        assert ws >= cfg.batch * Hq * 3 * 128 * 4      # one fp32 row per (sequence, head, split)
    # every case here has more than one MFMA head group: no step appends in the launch
    assert not any(K.kvq_decode_step_fused(cfg, t) for t in range(64, 140))


def test_decode_step_fusion_query_and_validation():
    """Host-only: which decode steps append inside the attention launch, and
    the step entry point's argument checks (no GPU needed)."""
    win = _cfg(batch=2, num_q_heads=8, num_kv_heads=2, max_tokens=1000, k=(K.INT_ASYM, 2, K.PER_CHANNEL, 32),
               v=(K.INT_ASYM, 2, K.PER_TOKEN, 32), residual=32)
    # window 32, key group 32: the step that completes a group of 32 beyond the window folds
    fused = [K.kvq_decode_step_fused(win, t) for t in range(64, 140)]
    for t, f in zip(range(64, 140), fused):
        folds = K.kvq_quantized_tokens(win, t + 1) != K.kvq_quantized_tokens(win, t)
        assert f == (not folds), t
    fp8 = _cfg(k=(K.FP8_E4M3, 8, 0, 0), v=(K.FP8_E5M2, 8, 0, 0), residual=0)
    assert all(K.kvq_decode_step_fused(fp8, t) for t in (1, 17, 500))
    fp8w = _cfg(k=(K.FP8_E4M3, 8, 0, 0), v=(K.FP8_E4M3, 8, 0, 0), residual=32)
    assert not K.kvq_decode_step_fused(fp8w, 100)             # every step folds one token
    assert not K.kvq_decode_step_fused(fp8, 100, kernel=K.KERNEL_GENERIC)
    tok = _cfg(k=(K.INT_ASYM, 4, K.PER_TOKEN, 0), v=(K.INT_ASYM, 4, K.PER_TOKEN, 0), residual=0)
    assert not K.kvq_decode_step_fused(tok, 100)              # quantizes the token (reductions)
    with pytest.raises(K.KvqError):
        K.kvq_decode_step_fused(win, 0)                       # a cache starts with quantize_append
    raw = _lib.raw
    ws = K.kvq_workspace_bytes(win, 101)
    o = K.AttnOptions()

    def step(t0=100, k=0x200000, v=0x300000, q=0x400000, out=0x500000, sm=0.088, w=0x600000, wb=ws):
        return raw.kvq_decode_step(C.byref(win), 0x100000, t0, k, v, q, out, sm, w, wb, C.byref(o), None)
    assert step(t0=0) == -1
    assert step(t0=1000) == -3
    assert step(k=0) == -5
    assert step(v=0x300004) == -4
    assert step(sm=0.0) == -1
    assert step(wb=16) == -6


def test_fp16_metadata_halves_the_int_metadata_sections():
    for k, v in [((K.INT_ASYM, 2, K.PER_CHANNEL, 32), (K.INT_ASYM, 2, K.PER_TOKEN, 32)),
                 ((K.INT_SYM, 8, K.PER_TOKEN, 0), (K.INT_SYM, 8, K.PER_TOKEN, 32))]:
        l32 = K.kvq_arena_layout(_cfg(k=k, v=v, residual=0))
        l16 = K.kvq_arena_layout(_cfg(k=k, v=v, residual=0, meta_dtype=K.F16))
        B, H = 2, 2
        for side, spec in (("k", k), ("v", v)):
            cols = getattr(l32, side + "_meta_cols")
            assert cols == getattr(l16, side + "_meta_cols")
            rows = (l32.token_capacity // spec[3]) if spec[2] == K.PER_CHANNEL else l32.token_capacity
            n = B * H * rows * cols
            def next_start(lay, off):
                """start of the section after the one at off (sections are in order)"""
                offs = [getattr(lay, f) for f in ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale",
                                                  "v_zero", "ring_k", "ring_v", "rope", "fp8_calib")]
                return min([o for o in offs if off < o < (1 << 63)] + [lay.total_bytes])
            # the scale section ends where the next one starts (256-byte aligned)
            s16, s32 = getattr(l16, side + "_scale"), getattr(l32, side + "_scale")
            assert next_start(l16, s16) - s16 == -(-2 * n // 256) * 256
            assert next_start(l32, s32) - s32 == -(-4 * n // 256) * 256
    # FP8 scales stay fp32 [H]; the option changes nothing for FP8 / NONE sides
    f8 = dict(k=(K.FP8_E4M3, 8, 0, 0), v=(K.FP8_E4M3, 8, 0, 0), residual=0)
    a, b = K.kvq_arena_layout(_cfg(**f8)), K.kvq_arena_layout(_cfg(**f8, meta_dtype=K.F16))
    assert a.total_bytes == b.total_bytes and a.v_codes == b.v_codes


def test_meta_dtype_validation():
    for bad in (2, -1, 7):
        with pytest.raises(K.KvqError):
            K.kvq_arena_bytes(_cfg(meta_dtype=bad))
    assert K.kvq_abi_version() == 5


def test_plain_c_caller(tmp_path):
    """include/kvq.h compiles as C11 and a C program links the library and
    calls its host-only entry points; its results match the Python binding."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime_api.h"):
        pytest.skip("gcc or the HIP headers are not available")
    pkg = os.path.dirname(_lib.__file__)
    exe = str(tmp_path / "host_queries")
    cmd = [gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           os.path.join(ROOT, "tests", "c_abi", "host_queries.c"), "-L", pkg, "-lkvq",
           f"-Wl,-rpath,{pkg}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    head, msg = r.stdout.split(" msg=", 1)
    got = dict(kv.split("=", 1) for kv in head.split())
    cfg = K.make_config(batch=32, num_q_heads=32, num_kv_heads=8, head_dim=128, max_tokens=32832,
                        k=(K.INT_ASYM, 2, K.PER_CHANNEL, 32), v=(K.INT_ASYM, 2, K.PER_TOKEN, 32),
                        residual=32, pre_rope_k=True)
    assert int(got["abi"]) == K.kvq_abi_version()
    assert int(got["arena"]) == K.kvq_arena_bytes(cfg)
    cfg.meta_dtype = K.F16
    assert int(got["arena16"]) == K.kvq_arena_bytes(cfg)
    assert int(got["tq"]) == 32736
    assert int(got["bad"]) == -1 and msg.strip() == K.kvq_status_string(-1)


# ---------------------------------------------------------------------------
# the Python binding's argument checks (CPU tensors: each rejection fires
# before the device check, and a fully correct CPU tensor is refused last)
# ---------------------------------------------------------------------------

def _tensors(cfg, T=16, n_new=4):
    import torch
    dt = {K.F32: torch.float32, K.F16: torch.float16, K.BF16: torch.bfloat16}[cfg.in_dtype]
    B, Hq, Hkv, D = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    return dict(arena=torch.zeros(K.kvq_arena_bytes(cfg), dtype=torch.uint8),
                k=torch.zeros(B, Hkv, n_new, D, dtype=dt), v=torch.zeros(B, Hkv, n_new, D, dtype=dt),
                q=torch.zeros(B, Hq, D, dtype=dt), out=torch.zeros(B, Hq, D, dtype=torch.float32),
                ws=torch.zeros(K.kvq_workspace_bytes(cfg, T), dtype=torch.uint8),
                ko=torch.zeros(B, Hkv, T, D, dtype=torch.float32))


def _rejects(fn, *args, match, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*args, **kw)


def test_binding_rejects_bad_append_arguments():
    import torch
    cfg = _cfg(in_dtype=K.BF16)
    t = _tensors(cfg)
    ap = K.kvq_quantize_append
    _rejects(ap, cfg, t["arena"][:-1], 0, t["k"], t["v"], match="arena holds")
    _rejects(ap, cfg, t["arena"], 0, t["k"].float(), t["v"], match="k_new has dtype")
    _rejects(ap, cfg, t["arena"], 0, t["k"][:, :1].contiguous(), t["v"][:, :1].contiguous(), match="k_new has shape")
    _rejects(ap, cfg, t["arena"], 0, t["k"].transpose(2, 3).contiguous().transpose(2, 3), t["v"],
             match="k_new must be contiguous")
    _rejects(ap, cfg, t["arena"], 0, t["k"], t["v"][:, :, :2].contiguous(), match="v_new has shape")
    _rejects(ap, cfg, t["arena"], 0, t["k"], t["v"], torch.ones(3), match="k_scale has shape")
    _rejects(ap, cfg, t["arena"], 0, t["k"], t["v"], match="arena must be a GPU tensor")
    _rejects(ap, cfg, t["arena"], 0, t["k"], None, match="v_new is required")


def test_binding_rejects_bad_attention_arguments():
    cfg = _cfg(in_dtype=K.BF16)
    t = _tensors(cfg)
    at = K.kvq_decode_attention
    sm = 0.088
    _rejects(at, cfg, t["arena"], 16, t["q"].float(), t["out"], sm, t["ws"], match="q has dtype")
    _rejects(at, cfg, t["arena"], 16, t["q"][:1], t["out"], sm, t["ws"], match="q has shape")
    _rejects(at, cfg, t["arena"], 16, t["q"], t["out"].half(), sm, t["ws"], match="out has dtype")
    _rejects(at, cfg, t["arena"], 16, t["q"], t["out"][:, :4].contiguous(), sm, t["ws"], match="out has shape")
    _rejects(at, cfg, t["arena"][:100], 16, t["q"], t["out"], sm, t["ws"], match="arena holds")
    _rejects(at, cfg, t["arena"], 16, t["q"], t["out"], sm, t["ws"], match="arena must be a GPU tensor")
    st = K.kvq_decode_step
    k1, v1 = t["k"][:, :, :1].contiguous(), t["v"][:, :, :1].contiguous()
    _rejects(st, cfg, t["arena"], 16, t["k"], t["v"], t["q"], t["out"], sm, t["ws"],
             match="a decode step appends 1")
    _rejects(st, cfg, t["arena"], 16, k1, v1, t["q"].permute(2, 1, 0).contiguous().permute(2, 1, 0), t["out"], sm, t["ws"],
             match="q must be contiguous")
    _rejects(st, cfg, t["arena"], 16, k1, v1, t["q"], t["out"], sm, t["ws"], match="arena must be a GPU tensor")


def test_binding_rejects_bad_dequantize_arguments():
    cfg = _cfg(in_dtype=K.BF16)
    t = _tensors(cfg, T=16)
    dq = K.kvq_dequantize
    _rejects(dq, cfg, t["arena"], 16, t["ko"][:, :, :8].contiguous(), match="k_out has shape")
    _rejects(dq, cfg, t["arena"], 16, t["ko"].double(), match="k_out has dtype")
    _rejects(dq, cfg, t["arena"], 16, None, t["ko"].half(), match="v_out has dtype")
    _rejects(dq, cfg, t["arena"], 16, t["ko"], match="arena must be a GPU tensor")


def test_static_scratch_entry_point_validation():
    """kvq_decode_attention_static refuses, before any HIP call, a request whose
    split partials exceed its device array, and bad pointers."""
    raw = _lib.raw
    cfg = _cfg()
    opt = K.AttnOptions()

    def call(c=cfg, T=500, arena=0x100000, q=0x200000, out=0x300000, o=opt):
        return raw.kvq_decode_attention_static(C.byref(c), arena, T, q, out, 0.088, C.byref(o), None)

    assert call(T=0) == -3
    assert call(q=None) == -5
    assert call(arena=0x100010) == -4
    big = _cfg(batch=64, num_q_heads=64, num_kv_heads=8, max_tokens=131072, k=(K.INT_ASYM, 4, K.PER_CHANNEL, 128),
               v=(K.INT_ASYM, 4, K.PER_TOKEN, 0), residual=128)
    o64 = K.AttnOptions()
    o64.num_splits = 64
    assert K.kvq_workspace_bytes(big, 131072, 0, 64) > K.STATIC_WORKSPACE_BYTES
    assert call(c=big, T=131072, o=o64) == -6
    # the serving-shaped workloads fit with their automatic split counts
    import workloads as W
    import bench
    for name in ("c3_fp8_e4m3_gqa_8k", "c4_int4_llama70b_128k", "c5_int2_kivi_prerope_32k"):
        w = W.WORKLOADS[name]
        kspec, vspec, R, pre, _ = bench.FORMATS[name]
        c = K.make_config(batch=w["B"], num_q_heads=w["Hq"], num_kv_heads=w["Hkv"], head_dim=128,
                          max_tokens=w["T"] + 64, k=kspec, v=vspec, residual=R, pre_rope_k=pre)
        assert K.kvq_workspace_bytes(c, w["T"] + 1) <= K.STATIC_WORKSPACE_BYTES, name


# ---------------------------------------------------------------------------
# paged caches: configuration rules, layout and host-side validation
# ---------------------------------------------------------------------------

def _pcfg(**kw):
    base = dict(page_tokens=64, num_pages=40)
    base.update(kw)
    return _cfg(**base)


@pytest.mark.parametrize("bad", [
    dict(page_tokens=48),                                   # not a multiple of 32
    dict(page_tokens=64, k=(K.INT_ASYM, 4, K.PER_CHANNEL, 128), residual=128),   # P % G != 0
    dict(num_pages=0),
    dict(page_tokens=0, num_pages=5),                        # pages without paging
    dict(page_tokens=-32),
    dict(k=(K.INT_ASYM, 4, K.PER_CHANNEL, 0), v=(K.INT_ASYM, 4, K.PER_TOKEN, 0), residual=0),  # whole axis
    dict(k=(K.INT_SYM, 8, K.PER_TENSOR, 0), v=(K.INT_ASYM, 4, K.PER_TOKEN, 0), residual=0),    # per tensor
    dict(k=(K.INT_ASYM, 4, K.PER_CHANNEL, 256), residual=256, page_tokens=256),  # key group over 128
])
def test_paged_invalid_configs(bad):
    assert K.kvq_validate_config(_pcfg(**bad)) == -1


def test_paged_layout_sizes():
    cfg = _pcfg()                   # INT4 K G32 + INT4 V G32, R 32, B 2, 2 kv heads, D 128
    lay = K.kvq_arena_layout(cfg)
    assert (lay.page_tokens, lay.pages) == (64, 40)
    rows = 40 * 2 * 64
    assert lay.k_scale - lay.k_codes >= rows * 64
    assert lay.k_zero - lay.k_scale >= rows // 32 * 128 * 4
    assert lay.v_codes - lay.k_zero >= rows // 32 * 128 * 4
    assert lay.v_scale - lay.v_codes >= rows // 32 * (32 * 128 * 4 // 8)
    assert lay.v_zero - lay.v_scale >= rows * 4 * 4          # 4 value groups of 32 channels per token
    c = K.kvq_arena_layout(_cfg())
    assert (c.page_tokens, c.pages) == (c.token_capacity, 2)


def test_paged_entry_point_validation():
    raw = _lib.raw
    pc, cc = _pcfg(), _cfg()
    bt, sl, arena, kn, q, out, ws = 0x500000, 0x600000, 0x100000, 0x200000, 0x300000, 0x380000, 0x400000
    opt = K.AttnOptions()
    wsb = K.kvq_workspace_bytes(pc, 640)

    def app(c=pc, bt_=bt, mb=10, sl_=sl, nl=None, n=4, flags=0, a=arena):
        return raw.kvq_paged_quantize_append(C.byref(c), a, bt_, mb, sl_, nl, n, kn, kn, None, None, flags, None)

    def att(c=pc, bt_=bt, mb=10, sl_=sl, T=640, w=wsb):
        return raw.kvq_paged_decode_attention(C.byref(c), arena, bt_, mb, sl_, T, q, out, 0.088, ws, w,
                                              C.byref(opt), None)

    assert app(c=cc) == -2                       # contiguous cache: the contiguous calls
    assert att(c=cc) == -2
    assert app(bt_=None) == -5 and att(sl_=None) == -5
    assert app(bt_=0x500002) == -4
    assert app(mb=0) == -1
    assert app(flags=K.CALIBRATE) == -1           # calibrate only when starting (and FP8)
    assert app(flags=16) == -1
    assert app(a=0x100010) == -4
    assert att(T=641) == -1                        # past max_blocks * P
    assert att(T=1025) == -3                       # past max_tokens
    assert att(w=wsb - 1) == -6
    # the contiguous entry points refuse a paged cache
    assert _append(pc) == -2
    assert raw.kvq_decode_attention(C.byref(pc), arena, 100, q, out, 0.088, ws, wsb, C.byref(opt), None) == -2
    assert raw.kvq_dequantize(C.byref(pc), arena, 100, 0x200000, None, None) == -2
    # paged workspace: a split's pages fit the attention kernel's table
    small = _pcfg(page_tokens=32, num_pages=4000, max_tokens=65536)
    for T in (1, 1000, 8192, 65536):
        b = K.kvq_workspace_bytes(small, T)
        assert b >= K.kvq_workspace_bytes(small, max(1, T // 2))
