"""Paged caches with ragged per-sequence lengths through the C ABI, against the
CPU oracle (each sequence quantized alone as the contiguous cache it is, the
pages gathered back into that order: oracle.paged) and against the contiguous
layout itself.

The bar: codes, scales, zero-points, window slots and dequantized values
bit-exact; attention within 2e-3 max relative L2 of the fp64 oracle; a paged
cache and a contiguous cache holding the same tokens give the same bytes and
the same attention output, bit for bit, at the same split count.
"""
import math
import zlib

import numpy as np
import pytest
import torch

import quantized_decode_attention_05_amd as K
import workloads as W
from oracle import attention as OA
from oracle import cache as OC
from oracle import paged as OP
from oracle import quant as OQ
from tests.kvq_harness import (ATTN_TOL, Case, GpuCache, PagedCache, compare_paged_sequence, payload_of, say,
                               to_dev)

pytestmark = pytest.mark.gpu

A, S, F8, E5, NO = K.INT_ASYM, K.INT_SYM, K.FP8_E4M3, K.FP8_E5M2, K.NONE
CH, TOK = K.PER_CHANNEL, K.PER_TOKEN

# (name, format, page tokens)
FORMATS = [
    ("int2_prerope_g32_r32", dict(k=(A, 2, CH, 32), v=(A, 2, TOK, 32), R=32, pre_rope=True), 64),
    ("int4_g128_r128", dict(k=(A, 4, CH, 128), v=(A, 4, TOK, 0), R=128), 128),
    ("int4_g64_meta16_r64", dict(k=(A, 4, CH, 64), v=(A, 4, TOK, 32), R=64, meta16=True), 128),
    ("int8_g64_int8tok16_r64", dict(k=(A, 8, CH, 64), v=(A, 8, TOK, 16), R=64), 64),
    ("fp8_e4m3", dict(k=(F8, 8, 0, 0), v=(F8, 8, 0, 0), R=0), 32),
    ("fp8_e5m2_r32", dict(k=(E5, 8, 0, 0), v=(E5, 8, 0, 0), R=32), 64),
    ("sym8tok", dict(k=(S, 8, TOK, 0), v=(S, 8, TOK, 32), R=0), 32),
    ("none16_int4tok", dict(k=(NO, 16, 0, 0), v=(A, 4, TOK, 0), R=0), 32),
]


def _kernels(cfg, T):
    ks = [K.KERNEL_GENERIC]
    try:
        K.kvq_workspace_bytes(cfg, T, K.KERNEL_MFMA)
        ks.append(K.KERNEL_MFMA)
    except K.KvqError:
        pass
    return ks


def _rows(x, b, lo, hi, n):
    """Rows [lo, hi) of sequence b padded to n rows (a ragged call's input)."""
    out = np.zeros((x.shape[1], n, x.shape[3]), dtype=x.dtype)
    out[:, :hi - lo] = x[b, :, lo:hi]
    return out


def _oracle_seq(case, Kf, Vf, b, T, scales):
    sub = case.oracle_cfg(B=1)
    ks = vs = None
    if scales is not None:
        ks, vs = scales
    return OC.quantize_cache(sub, Kf[b:b + 1], Vf[b:b + 1], T, k_scale=ks, v_scale=vs)


def _fp8_scales(case, Kf, Vf, lens):
    """Calibrated per-head scales over the first call's tokens of every sequence
    (ragged), staged as the cache stages them."""
    if case.k[0] != F8 and case.v[0] != F8:
        return None
    win = OC.has_window(case.oracle_cfg())
    out = []
    for x, spec in ((Kf, case.k), (Vf, case.v)):
        if spec[0] == F8:
            a = np.zeros(case.Hkv, np.float32)
            for b, n in enumerate(lens):
                if n:
                    a = np.maximum(a, np.abs(OQ.stage(x[b, :, :n], win)).max(axis=(1, 2)))
            out.append(OQ.fp8_scale_from_absmax(a))
        else:
            out.append(np.ones(case.Hkv, np.float32))
    return tuple(out)


@pytest.mark.parametrize("name,fmt,P", FORMATS, ids=[f[0] for f in FORMATS])
def test_paged_ragged_against_oracle(name, fmt, P):
    """Ragged prefill (one call, lengths 333 / 1100 / 65 / 0), a ragged chunk
    (19 / 0 / 40 / 7 tokens), then 37 decode steps crossing folds; every
    sequence compared with the oracle of that sequence alone."""
    case = Case(B=4, Hq=8, Hkv=2, D=128, dtype="bf16", **fmt)
    seed = zlib.crc32(name.encode()) % 1000
    pre, chunk, steps = [333, 1100, 65, 0], [19, 0, 40, 7], 37
    Tmax = max(p + c for p, c in zip(pre, chunk)) + steps
    (Kf, Kp), (Vf, Vp) = W.random_case(seed, case.B, case.Hkv, Tmax, case.D, dtype="bf16")
    pc = PagedCache(case, P, cap=Tmax + 8, seed=seed)
    fp8 = case.k[0] == F8 or case.v[0] == F8
    say(f"[paged] {name} P={P} pages={pc.pages} blocks/seq={pc.max_blocks}")
    flags = K.INIT | (K.CALIBRATE if fp8 else 0)
    n0 = max(pre)
    pc.append(np.stack([_rows(Kp, b, 0, pre[b], n0) for b in range(case.B)]),
              np.stack([_rows(Vp, b, 0, pre[b], n0) for b in range(case.B)]), pre, flags)
    scales = _fp8_scales(case, Kf, Vf, pre)
    n1 = max(chunk)
    pc.append(np.stack([_rows(Kp, b, pre[b], pre[b] + chunk[b], n1) for b in range(case.B)]),
              np.stack([_rows(Vp, b, pre[b], pre[b] + chunk[b], n1) for b in range(case.B)]), chunk)
    ws = torch.zeros(K.kvq_workspace_bytes(pc.cfg, Tmax + 8), dtype=torch.uint8, device="cuda")
    out = torch.empty((case.B, case.Hq, case.D), dtype=torch.float32, device="cuda")
    check = {0, 20, steps - 1}
    outs = {}
    for i in range(steps):
        t = pc.lens.copy()
        kn = np.stack([Kp[b, :, t[b]:t[b] + 1] for b in range(case.B)])
        vn = np.stack([Vp[b, :, t[b]:t[b] + 1] for b in range(case.B)])
        qf, qp = W.random_queries(seed + 100 + i, case.B, case.Hq, case.D, dtype="bf16")
        out.fill_(float("nan"))
        pc.step(kn, vn, qp, ws, out)
        if i in check:
            torch.cuda.synchronize()
            outs[i] = (out.cpu().numpy(), qf, pc.lens.copy())
    torch.cuda.synchronize()
    sm = 1.0 / math.sqrt(case.D)
    n_rep = case.Hq // case.Hkv
    kd, vd = pc.dequantize()
    for b in range(case.B):
        T = int(pc.lens[b])
        st = _oracle_seq(case, Kf, Vf, b, T, None if scales is None else (scales[0], scales[1]))
        compare_paged_sequence(pc, b, st, None if scales is None else {"k": scales[0], "v": scales[1]})
        assert np.array_equal(kd[b, :, :T], st["k_hat"][0]), f"seq {b}: dequantized K differs"
        assert np.array_equal(vd[b, :, :T], st["v_hat"][0]), f"seq {b}: dequantized V differs"
        for i, (o, qf, lens) in outs.items():
            sti = _oracle_seq(case, Kf, Vf, b, int(lens[b]), None if scales is None else scales)
            ref = OA.decode_attention(qf[b:b + 1], sti["k_hat"], sti["v_hat"], sm,
                                      pre_rope_base=case.rope_base if case.pre_rope else None)
            err = OA.max_rel_l2_per_head(o[b:b + 1], ref)
            assert err <= ATTN_TOL, (name, "step", i, "seq", b, err)
    # attention of the final cache on every kernel and a few split counts
    qf, qp = W.random_queries(seed + 7, case.B, case.Hq, case.D, dtype="bf16")
    for kern in _kernels(pc.cfg, int(pc.lens.max())):
        for splits in (0, 1, 3, 11):
            o = pc.attention(qp, kernel=kern, num_splits=splits)
            for b in range(case.B):
                st = _oracle_seq(case, Kf, Vf, b, int(pc.lens[b]), None if scales is None else scales)
                ref = OA.decode_attention(qf[b:b + 1], st["k_hat"], st["v_hat"], sm,
                                          pre_rope_base=case.rope_base if case.pre_rope else None)
                err = OA.max_rel_l2_per_head(o[b:b + 1], ref)
                assert err <= ATTN_TOL, (name, kern, splits, b, err)
    say(f"[paged] {name} lens={pc.lens.tolist()} ok")
    assert n_rep >= 1


@pytest.mark.parametrize("name,fmt,P", [f for f in FORMATS if f[0] in
                                        ("int2_prerope_g32_r32", "int4_g128_r128", "fp8_e4m3", "sym8tok")],
                         ids=["int2_prerope_g32_r32", "int4_g128_r128", "fp8_e4m3", "sym8tok"])
def test_paged_equals_contiguous(name, fmt, P):
    """The same tokens appended to a contiguous cache and to a paged one (equal
    lengths: a prefill, then decode steps through each layout's decode-step
    call): the gathered pages equal the contiguous sections byte for byte, the
    window rings match, and attention gives identical outputs at equal split
    counts on every kernel."""
    case = Case(B=2, Hq=8, Hkv=2, D=128, dtype="bf16", **fmt)
    seed = zlib.crc32(("eq" + name).encode()) % 1000
    T0, steps = 700, 40
    T = T0 + steps
    (Kf, Kp), (Vf, Vp) = W.random_case(seed, case.B, case.Hkv, T, case.D, dtype="bf16")
    gc = GpuCache(case, cap=T)
    pc = PagedCache(case, P, cap=T, seed=seed)
    fp8 = case.k[0] == F8
    gc.append(Kp[:, :, :T0], Vp[:, :, :T0], K.CALIBRATE if fp8 else 0)
    pc.append(Kp[:, :, :T0], Vp[:, :, :T0], [T0] * case.B, K.INIT | (K.CALIBRATE if fp8 else 0))
    sm = 1.0 / math.sqrt(case.D)
    wsg = torch.zeros(K.kvq_workspace_bytes(gc.cfg, T), dtype=torch.uint8, device="cuda")
    wsp = torch.zeros(K.kvq_workspace_bytes(pc.cfg, T), dtype=torch.uint8, device="cuda")
    og = torch.empty((case.B, case.Hq, case.D), dtype=torch.float32, device="cuda")
    op = torch.empty_like(og)
    for i in range(steps):
        t = T0 + i
        qf, qp = W.random_queries(seed + i, case.B, case.Hq, case.D, dtype="bf16")
        K.kvq_decode_step(gc.cfg, gc.arena, t, to_dev(Kp[:, :, t:t + 1], "bf16"), to_dev(Vp[:, :, t:t + 1], "bf16"),
                          to_dev(qp, "bf16"), og, sm, wsg)
        pc.step(Kp[:, :, t:t + 1], Vp[:, :, t:t + 1], qp, wsp, op)
        torch.cuda.synchronize()
        assert torch.equal(og, op), f"step {i}: paged and contiguous decode steps differ"
    gc.T = T
    lay = gc.layout
    H, D, Tc = case.Hkv, case.D, lay.token_capacity
    arena = gc.arena.cpu().numpy()

    def contiguous(off, per_tok_shape, dtype):
        n = int(np.prod(per_tok_shape)) * np.dtype(dtype).itemsize
        return arena[off: off + case.B * H * n].view(dtype).reshape((case.B, H) + tuple(per_tok_shape))

    def check(name_, ctg_shape, page_shape, dtype, count):
        ctg = contiguous(getattr(lay, name_), ctg_shape, dtype)
        sec = pc.section(name_, page_shape, dtype)
        for b in range(case.B):
            got = OP.gather_pages(sec, pc.block_table, b, P, T)[:, :count]
            assert np.array_equal(got, ctg[b][:, :count]), f"{name_} of sequence {b} differs"

    Tq = K.kvq_quantized_tokens(gc.cfg, T)
    check("k_codes", (Tc, lay.k_row_bytes), (P, lay.k_row_bytes), np.uint8, Tq)
    check("v_codes", (Tc // 32, lay.v_block_bytes), (P // 32, lay.v_block_bytes), np.uint8, Tq // 32)
    for side, spec in (("k", case.k), ("v", case.v)):
        if spec[0] not in (A, S):
            continue
        if spec[2] == CH:
            G = spec[3]
            shapes = ((Tc // G, D), (P // G, D), Tq // G)
        else:
            cols = D // (spec[3] or D)
            shapes = ((Tc, cols), (P, cols), Tq)
        check(side + "_scale", shapes[0], shapes[1], np.uint32, shapes[2])
        if spec[0] == A:
            check(side + "_zero", shapes[0], shapes[1], np.uint32, shapes[2])
    for sec in ("ring_k", "ring_v"):
        off_g, off_p = getattr(lay, sec), getattr(pc.layout, sec)
        if off_g >= (1 << 62):
            continue
        n = case.B * H * lay.ring_slots * D * 2
        assert torch.equal(gc.arena[off_g:off_g + n], pc.arena[off_p:off_p + n]), f"{sec} differs"
    qf, qp = W.random_queries(seed + 99, case.B, case.Hq, case.D, dtype="bf16")
    for kern in _kernels(gc.cfg, T):
        for splits in (1, 3):
            a = gc.attention(qp, kernel=kern, num_splits=splits)
            b_ = pc.attention(qp, kernel=kern, num_splits=splits)
            assert np.array_equal(a, b_), (name, kern, splits)


def test_paged_empty_and_out_of_capacity_sequences():
    """A sequence of length 0 attends to nothing (zero output); an append whose
    range does not fit the capacity is skipped and leaves its pages alone."""
    case = Case(B=3, Hq=8, Hkv=2, D=128, dtype="bf16", k=(A, 4, CH, 32), v=(A, 4, TOK, 32), R=32)
    P, cap = 64, 256
    (Kf, Kp), (Vf, Vp) = W.random_case(5, case.B, case.Hkv, 300, case.D, dtype="bf16")
    pc = PagedCache(case, P, cap=cap, seed=5)
    pc.append(Kp[:, :, :200], Vp[:, :, :200], [200, 0, 150], K.INIT)
    qf, qp = W.random_queries(5, case.B, case.Hq, case.D, dtype="bf16")
    for kern in _kernels(pc.cfg, 200):
        o = pc.attention(qp, kernel=kern)
        assert np.array_equal(o[1], np.zeros_like(o[1])), "an empty sequence must give a zero output"
    before = pc.arena.clone()
    # sequence 0 would end at 200 + 100 > cap = 256: skipped; the others append
    nl = torch.from_numpy(np.array([100, 30, 50], np.int32)).cuda()
    K.kvq_paged_quantize_append(pc.cfg, pc.arena, pc.bt, pc.seq_lens, to_dev(Kp[:, :, 200:300], "bf16"),
                                to_dev(Vp[:, :, 200:300], "bf16"), nl)
    torch.cuda.synchronize()
    lay = pc.layout
    sec_now = pc.section("k_codes", (P, lay.k_row_bytes), np.uint8)
    off = lay.k_codes
    n = pc.pages * case.Hkv * P * lay.k_row_bytes
    sec_before = before[off:off + n].cpu().numpy().reshape(pc.pages, case.Hkv, P, lay.k_row_bytes)
    for j in range(pc.max_blocks):
        pg = pc.block_table[0, j]
        assert np.array_equal(sec_now[pg], sec_before[pg]), "an append past the capacity wrote pages"
    ring = lay.ring_k
    m = case.Hkv * lay.ring_slots * case.D * 2
    assert torch.equal(pc.arena[ring:ring + m], before[ring:ring + m]), "an append past the capacity wrote the ring"


def test_paged_c5_shape_ragged_batch():
    """The KIVI-style INT2 pre-RoPE cache at its full shape (batch 32, 32/8
    heads, window 32) in 256-token pages with ragged lengths between 24577 and
    32768 tokens, prefilled in one call, then 40 decode steps: sampled
    (sequence, kv head) pairs bit-exact against the oracle, attention within
    tolerance."""
    name = "c5_int2_kivi_prerope_32k"
    w = W.WORKLOADS[name]
    B, Hq, Hkv, D, T0 = w["B"], w["Hq"], w["Hkv"], w["D"], w["T"]
    case = Case(B=B, Hq=Hq, Hkv=Hkv, D=D, dtype="bf16", k=(A, 2, CH, 32), v=(A, 2, TOK, 32), R=32, pre_rope=True)
    lens = np.array([T0 - (b * 1021) % 8192 for b in range(B)])
    steps, P = 40, 256
    say(f"[paged c5] generating inputs, lengths {lens.min()}..{lens.max()}")
    kp = torch.from_numpy(W.full_prefill(name, "k").view(np.int16)).view(torch.bfloat16).cuda()
    vp = torch.from_numpy(W.full_prefill(name, "v").view(np.int16)).view(torch.bfloat16).cuda()
    pc = PagedCache(case, P, cap=T0 + steps + 8, seed=55, spare_pages=17)
    nl = torch.from_numpy(lens.astype(np.int32)).cuda()
    K.kvq_paged_quantize_append(pc.cfg, pc.arena, pc.bt, pc.seq_lens, kp, vp, nl, flags=K.INIT)
    pc.lens += lens
    pc._sync_lens()
    del kp, vp
    torch.cuda.synchronize()
    ws = torch.zeros(K.kvq_workspace_bytes(pc.cfg, T0 + steps + 8), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    say(f"[paged c5] {steps} decode steps")
    for i in range(steps):
        kn = np.empty((B, Hkv, 1, D), np.uint16)
        vn = np.empty((B, Hkv, 1, D), np.uint16)
        for b in range(B):
            for h in range(Hkv):
                kn[b, h] = W.step_tokens(name, b, h, "k", i, 1)
                vn[b, h] = W.step_tokens(name, b, h, "v", i, 1)
        q = W.step_query(name, i)
        out.fill_(float("nan"))
        pc.step(kn, vn, q, ws, out)
    torch.cuda.synchronize()
    last = out.cpu().numpy()
    assert np.isfinite(last).all()
    sm = 1.0 / math.sqrt(D)
    n_rep = Hq // Hkv
    sub = case.oracle_cfg(B=1, Hq=n_rep, Hkv=1)
    q_last = W.bf16_bits_to_f32(W.step_query(name, steps - 1))
    for (b, h) in [(0, 0), (7, 3), (19, 5), (31, 7)]:
        T = int(pc.lens[b])
        L = int(lens[b])
        kb = np.concatenate([W.kv_chunk(name, b, h, "k")[:L], W.step_tokens(name, b, h, "k", 0, steps)])
        vb = np.concatenate([W.kv_chunk(name, b, h, "v")[:L], W.step_tokens(name, b, h, "v", 0, steps)])
        Kf, Vf = W.bf16_bits_to_f32(kb)[None, None], W.bf16_bits_to_f32(vb)[None, None]
        st = OC.quantize_cache(sub, Kf, Vf, T)
        # the pages of (b, h) gathered, against the oracle's sequence of one head
        lay = pc.layout
        kc = pc.section("k_codes", (P, lay.k_row_bytes), np.uint8)[:, h:h + 1]
        rows = OP.gather_pages(kc, pc.block_table, b, P, T)[:, :st["Tq"]]
        assert np.array_equal(rows, OC.pack_rows(st["k"]["codes"][0], 2)), f"(b={b}, h={h}): K rows differ"
        vcs = pc.section("v_codes", (P // 32, lay.v_block_bytes), np.uint8)[:, h:h + 1]
        vb_ = OP.gather_pages(vcs, pc.block_table, b, P, T)[:, :st["Tq"] // 32]
        assert np.array_equal(OC.unpack_vblocks(vb_, 2, D, st["Tq"]),
                              OC.unpack_vblocks(OC.pack_vblocks(st["v"]["codes"][0], 2), 2, D, st["Tq"])), \
            f"(b={b}, h={h}): V blocks differ"
        ks = pc.section("k_scale", (P // 32, D), np.float32)[:, h:h + 1]
        assert np.array_equal(OP.gather_pages(ks, pc.block_table, b, P, T)[:, :st["Tq"] // 32],
                              st["k"]["scale"][0]), f"(b={b}, h={h}): K scales differ"
        vz = pc.section("v_zero", (P, 4), np.float32)[:, h:h + 1]
        assert np.array_equal(OP.gather_pages(vz, pc.block_table, b, P, T)[:, :st["Tq"]],
                              st["v"]["zero"][0]), f"(b={b}, h={h}): V zero-points differ"
        ref = OA.decode_attention(q_last[b:b + 1, h * n_rep:(h + 1) * n_rep], st["k_hat"], st["v_hat"], sm,
                                  pre_rope_base=10000.0)
        err = OA.max_rel_l2_per_head(last[b:b + 1, h * n_rep:(h + 1) * n_rep], ref)
        say(f"[paged c5] (b={b}, h={h}) T={T} max rel-L2 {err:.2e}")
        assert err <= ATTN_TOL
