"""Parity harness: run the HIP library through the C ABI and compare it with
the CPU oracle on the same seeded inputs.

Comparisons (the bar):
  * integer / byte results bit-exact: K code rows, V code blocks (unpacked with
    the oracle's own unpacker), scales and zero-points, FP8 scales, fp16 window
    slots, and the dequantized fp32 values;
  * decode attention within a max (over sequence x query head) relative L2 of
    2e-3 against the oracle's fp64 attention on the oracle's dequantized cache.
"""
from __future__ import annotations

import math
import sys
from dataclasses import dataclass

import numpy as np
import torch

import quantized_decode_attention_05_amd as K
from oracle import attention as OA
from oracle import cache as OC

ATTN_TOL = 2e-3
_DT = {"f32": (K.F32, torch.float32), "f16": (K.F16, torch.float16), "bf16": (K.BF16, torch.bfloat16)}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@dataclass
class Case:
    B: int
    Hq: int
    Hkv: int
    D: int
    k: tuple
    v: tuple
    R: int = 0
    pre_rope: bool = False
    rope_base: float = 10000.0
    dtype: str = "f32"
    cap: int = 0
    meta16: bool = False     # INT scales / zero-points stored in fp16

    def lib_cfg(self, cap):
        return K.make_config(batch=self.B, num_q_heads=self.Hq, num_kv_heads=self.Hkv, head_dim=self.D,
                             max_tokens=cap, k=self.k, v=self.v, in_dtype=_DT[self.dtype][0],
                             out_dtype=K.F32, residual=self.R, pre_rope_k=self.pre_rope,
                             rope_base=self.rope_base, meta_dtype=K.F16 if self.meta16 else K.F32)

    def oracle_cfg(self, B=None, Hq=None, Hkv=None):
        return OC.Cfg(B or self.B, Hq or self.Hq, Hkv or self.Hkv, self.D, OC.Spec(*self.k, meta16=self.meta16),
                      OC.Spec(*self.v, meta16=self.meta16), self.R, self.pre_rope, self.rope_base)


def to_dev(payload: np.ndarray, dtype: str) -> torch.Tensor:
    """Upload a device-dtype payload (f32 values, f16 values or bf16 bits)."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(payload).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(payload)).cuda()


class GpuCache:
    """A cache arena on cuda:0 driven through the C ABI."""

    def __init__(self, case: Case, cap: int, fill: int = 0x5A):
        self.case = case
        self.cfg = case.lib_cfg(cap)
        self.layout = K.kvq_arena_layout(self.cfg)
        self.arena = torch.full((self.layout.total_bytes,), fill, dtype=torch.uint8, device="cuda")
        self.T = 0

    def append(self, k_payload, v_payload, flags=0, k_scale=None, v_scale=None):
        kd, vd = to_dev(k_payload, self.case.dtype), to_dev(v_payload, self.case.dtype)
        ks = None if k_scale is None else torch.as_tensor(k_scale, dtype=torch.float32).cuda()
        vs = None if v_scale is None else torch.as_tensor(v_scale, dtype=torch.float32).cuda()
        K.kvq_quantize_append(self.cfg, self.arena, self.T, kd, vd, ks, vs, flags)
        self.T += int(kd.shape[2])

    def attention(self, q_payload, sm_scale=None, kernel=0, num_splits=0, T=None):
        T = self.T if T is None else T
        c = self.case
        q = to_dev(q_payload, c.dtype)
        # poisoned, so an output the kernels never write cannot pass on a
        # stale buffer the allocator hands back
        out = torch.full((c.B, c.Hq, c.D), float("nan"), dtype=torch.float32, device="cuda")
        ws = torch.zeros(K.kvq_workspace_bytes(self.cfg, T, kernel, num_splits), dtype=torch.uint8,
                         device="cuda")
        sm = 1.0 / math.sqrt(c.D) if sm_scale is None else sm_scale
        K.kvq_decode_attention(self.cfg, self.arena, T, q, out, sm, ws, kernel, num_splits)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        assert np.isfinite(o).all(), f"attention output not finite (unwritten heads?) kernel={kernel} " \
                                     f"splits={num_splits} T={T}"
        return o

    def dequantize(self, T=None, bh_sel=None):
        T = self.T if T is None else T
        c = self.case
        ko = torch.full((c.B, c.Hkv, T, c.D), float("nan"), dtype=torch.float32, device="cuda")
        vo = torch.full_like(ko, float("nan"))
        K.kvq_dequantize(self.cfg, self.arena, T, ko, vo)
        torch.cuda.synchronize()
        if bh_sel is not None:
            b, h = bh_sel
            ko, vo = ko[b:b + 1, h:h + 1], vo[b:b + 1, h:h + 1]
        out = ko.cpu().numpy(), vo.cpu().numpy()
        del ko, vo
        return out

    def section(self, name, nbytes, offset=0):
        off = getattr(self.layout, name)
        return self.arena[off + offset: off + offset + nbytes].cpu().numpy()


# ---------------------------------------------------------------------------
# section comparisons
# ---------------------------------------------------------------------------

def _meta_shape(spec, B, H, D, Tc, Tq):
    scheme, bits, axis, group = spec
    if scheme in (OC.FP8_E4M3, OC.FP8_E5M2):
        return None
    if axis == OC.PER_TENSOR:
        return (B, H, 1, 1), (B, H, 1, 1)
    if axis == OC.PER_CHANNEL:
        rows = Tc // group if group else 1
        used = Tq // group if group else 1
        return (B, H, rows, D), (B, H, used, D)
    gc = group or D
    return (B, H, Tc, D // gc), (B, H, Tq, D // gc)


def compare_sections(gc: GpuCache, st: dict, bh_sel=None):
    """Bit-exact comparison of the arena with oracle state ``st``.  With bh_sel =
    (b, h) the oracle state covers that single (sequence, kv head) and only its
    slices are copied off the device."""
    c, lay = gc.case, gc.layout
    B, H, D, Tc = c.B, c.Hkv, c.D, lay.token_capacity
    Tq, T = st["Tq"], st["T"]
    arena = gc.arena

    def sl(off, per_bh, dtype):
        """[B', H', *per_bh] view of a [B][H][*per_bh] section (B' = H' = 1 with bh_sel)."""
        n = int(np.prod(per_bh)) * np.dtype(dtype).itemsize
        if bh_sel is None:
            raw = arena[off: off + n * B * H]
            return raw.cpu().numpy().view(dtype).reshape((B, H) + tuple(per_bh))
        b, h = bh_sel
        o = off + (b * H + h) * n
        return arena[o: o + n].cpu().numpy().view(dtype).reshape((1, 1) + tuple(per_bh))

    bits_k = OC.code_bits(OC.Spec(*c.k))
    rows = sl(lay.k_codes, (Tc, lay.k_row_bytes), np.uint8)[:, :, :Tq]
    exp_rows = OC.pack_rows(st["k"]["codes"], bits_k)
    assert np.array_equal(rows, exp_rows), "K code rows differ"

    bits_v = OC.code_bits(OC.Spec(*c.v))
    vb = sl(lay.v_codes, (Tc // 32, lay.v_block_bytes), np.uint8)
    got_v = OC.unpack_vblocks(vb, bits_v, D, Tq)
    exp_v = OC.unpack_vblocks(OC.pack_vblocks(st["v"]["codes"], bits_v), bits_v, D, Tq)
    assert np.array_equal(got_v, exp_v), "V code blocks differ"

    for side, spec in (("k", c.k), ("v", c.v)):
        part = st[side]
        if spec[0] in (OC.FP8_E4M3, OC.FP8_E5M2):
            off = getattr(lay, side + "_scale")
            s = arena[off: off + 4 * H].cpu().numpy().view(np.float32)
            if bh_sel is not None:
                s = s[bh_sel[1]:bh_sel[1] + 1]
            exp = np.asarray(part["scale"], np.float32)
            assert np.array_equal(s.view(np.uint32), exp.view(np.uint32)), \
                f"{side} fp8 scale differs: {s} vs {exp}"
            continue
        if spec[0] == OC.NONE:
            continue
        full, used = _meta_shape(spec, B, H, D, Tc, Tq)
        idx = (slice(None), slice(None)) + tuple(slice(0, u) for u in used[2:])
        # fp16 metadata: the oracle's stored values are fp16 numbers held in fp32
        mdt, bits_t = (np.float16, np.uint16) if c.meta16 else (np.float32, np.uint32)
        sc = sl(getattr(lay, side + "_scale"), full[2:], mdt)[idx]
        exp_s = part["scale"].reshape(sc.shape)
        if c.meta16:
            assert np.array_equal(exp_s.astype(np.float16).astype(np.float32), exp_s)
        assert np.array_equal(sc.view(bits_t), exp_s.astype(mdt).view(bits_t)), f"{side} scales differ"
        if spec[0] == OC.INT_ASYM:
            zz = sl(getattr(lay, side + "_zero"), full[2:], mdt)[idx]
            exp_z = part["zero"].reshape(zz.shape)
            assert np.array_equal(zz.astype(np.float32), exp_z), f"{side} zero-points differ"

    if T > Tq:
        Rs = lay.ring_slots
        slots = OC.window_slots(c.oracle_cfg(), Tq, T)
        rk = sl(lay.ring_k, (Rs, D), np.float16)[:, :, slots]
        assert np.array_equal(rk.view(np.uint16), st["k_window"].view(np.uint16)), "ring K differs"
        rvb = sl(lay.ring_v, (Rs // 32, 32 * D * 2), np.uint8)
        rv = OC.unpack_vblocks(rvb, 16, D, Rs)[:, :, slots]
        assert np.array_equal(rv.view(np.uint16), st["v_window"].view(np.uint16)), "ring V differs"


def compare_dequant(gc: GpuCache, st: dict, bh_sel=None):
    kd, vd = gc.dequantize(st["T"], bh_sel)
    assert np.array_equal(kd, st["k_hat"]), "dequantized K differs"
    assert np.array_equal(vd, st["v_hat"]), "dequantized V differs"


def attention_error(out_gpu: np.ndarray, q_f32: np.ndarray, st: dict, case: Case, heads=None,
                    sm_scale=None) -> float:
    sm = 1.0 / math.sqrt(case.D) if sm_scale is None else sm_scale
    ref = OA.decode_attention(q_f32, st["k_hat"], st["v_hat"], sm,
                              pre_rope_base=case.rope_base if case.pre_rope else None, heads=heads)
    return OA.max_rel_l2_per_head(out_gpu, ref, heads)


def payload_of(values_f32: np.ndarray, dtype: str) -> np.ndarray:
    """Device payload whose value is exactly values_f32 (which must be representable)."""
    if dtype == "f32":
        return np.ascontiguousarray(values_f32, dtype=np.float32)
    if dtype == "f16":
        return values_f32.astype(np.float16)
    u = np.ascontiguousarray(values_f32, dtype=np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0)
    return (u >> 16).astype(np.uint16)


# ---------------------------------------------------------------------------
# paged caches
# ---------------------------------------------------------------------------

class PagedCache:
    """A paged cache on cuda:0: a pool of pages, a block table with pages
    handed out in a shuffled order, and per-sequence lengths (ragged)."""

    def __init__(self, case: Case, P: int, cap: int, seed: int = 0, spare_pages: int = 3, fill: int = 0x5A):
        from oracle import paged as OP
        self.case, self.P, self.cap = case, P, cap
        self.max_blocks = OP.blocks_of(cap, P)
        self.pages = case.B * self.max_blocks + spare_pages
        self.cfg = K.make_config(batch=case.B, num_q_heads=case.Hq, num_kv_heads=case.Hkv, head_dim=case.D,
                                 max_tokens=cap, k=case.k, v=case.v, in_dtype=_DT[case.dtype][0],
                                 out_dtype=K.F32, residual=case.R, pre_rope_k=case.pre_rope,
                                 rope_base=case.rope_base, meta_dtype=K.F16 if case.meta16 else K.F32,
                                 page_tokens=P, num_pages=self.pages)
        self.layout = K.kvq_arena_layout(self.cfg)
        self.arena = torch.full((self.layout.total_bytes,), fill, dtype=torch.uint8, device="cuda")
        perm = np.random.default_rng((seed, 91)).permutation(self.pages)[:case.B * self.max_blocks]
        self.block_table = perm.reshape(case.B, self.max_blocks).astype(np.int32)
        self.bt = torch.from_numpy(self.block_table).cuda()
        self.lens = np.zeros(case.B, dtype=np.int64)
        self.seq_lens = torch.zeros(case.B, dtype=torch.int32, device="cuda")

    def _sync_lens(self):
        self.seq_lens.copy_(torch.from_numpy(self.lens.astype(np.int32)))

    def append(self, k_payload, v_payload, new_lens, flags=0, k_scale=None, v_scale=None):
        """k_payload, v_payload: [B, Hkv, n_max, D] device-dtype payloads; sequence
        b appends its first new_lens[b] rows."""
        kd, vd = to_dev(k_payload, self.case.dtype), to_dev(v_payload, self.case.dtype)
        nl = torch.from_numpy(np.asarray(new_lens, dtype=np.int32)).cuda()
        ks = None if k_scale is None else torch.as_tensor(k_scale, dtype=torch.float32).cuda()
        vs = None if v_scale is None else torch.as_tensor(v_scale, dtype=torch.float32).cuda()
        K.kvq_paged_quantize_append(self.cfg, self.arena, self.bt, self.seq_lens, kd, vd, nl, ks, vs, flags)
        self.lens += np.asarray(new_lens, dtype=np.int64)
        self._sync_lens()

    def step(self, k_payload, v_payload, q_payload, ws, out, sm=None, kernel=0, num_splits=0):
        """kvq_paged_decode_step: one token per sequence, attention over lens + 1."""
        c = self.case
        sm = 1.0 / math.sqrt(c.D) if sm is None else sm
        K.kvq_paged_decode_step(self.cfg, self.arena, self.bt, self.seq_lens, int(self.lens.max()) + 1,
                                to_dev(k_payload, c.dtype), to_dev(v_payload, c.dtype), to_dev(q_payload, c.dtype),
                                out, sm, ws, kernel, num_splits)
        self.lens += 1
        self._sync_lens()

    def attention(self, q_payload, kernel=0, num_splits=0, sm_scale=None):
        c = self.case
        maxT = int(self.lens.max())
        q = to_dev(q_payload, c.dtype)
        out = torch.full((c.B, c.Hq, c.D), float("nan"), dtype=torch.float32, device="cuda")
        ws = torch.zeros(K.kvq_workspace_bytes(self.cfg, maxT, kernel, num_splits), dtype=torch.uint8,
                         device="cuda")
        sm = 1.0 / math.sqrt(c.D) if sm_scale is None else sm_scale
        K.kvq_paged_decode_attention(self.cfg, self.arena, self.bt, self.seq_lens, maxT, q, out, sm, ws, kernel,
                                     num_splits)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        assert np.isfinite(o).all(), f"paged attention output not finite kernel={kernel} splits={num_splits}"
        return o

    def dequantize(self):
        c = self.case
        maxT = int(self.lens.max())
        ko = torch.full((c.B, c.Hkv, maxT, c.D), float("nan"), dtype=torch.float32, device="cuda")
        vo = torch.full_like(ko, float("nan"))
        K.kvq_paged_dequantize(self.cfg, self.arena, self.bt, self.seq_lens, maxT, ko, vo)
        torch.cuda.synchronize()
        return ko.cpu().numpy(), vo.cpu().numpy()

    def section(self, name, per_page_shape, dtype):
        """A token section as [pages][H][*per_page_shape] (host copy)."""
        off = getattr(self.layout, name)
        n = self.pages * self.case.Hkv * int(np.prod(per_page_shape)) * np.dtype(dtype).itemsize
        return self.arena[off: off + n].cpu().numpy().view(dtype).reshape(
            (self.pages, self.case.Hkv) + tuple(per_page_shape))


def compare_paged_sequence(pc: PagedCache, b: int, st: dict, fp8_scales=None):
    """Bit-exact comparison of sequence b of a paged cache with the oracle state
    st of that sequence alone (B = 1): the pages of each token section are
    gathered into the contiguous order (oracle.paged) and compared as
    compare_sections does; window slots from the sequence's ring."""
    from oracle import paged as OP
    c, lay, P = pc.case, pc.layout, pc.P
    H, D = c.Hkv, c.D
    Tq, T = st["Tq"], st["T"]
    bt = pc.block_table

    def gathered(name, per_page_shape, dtype, count):
        sec = pc.section(name, per_page_shape, dtype)
        return OP.gather_pages(sec, bt, b, P, T)[:, :count]

    bits_k = OC.code_bits(OC.Spec(*c.k))
    rows = gathered("k_codes", (P, lay.k_row_bytes), np.uint8, Tq)
    assert np.array_equal(rows, OC.pack_rows(st["k"]["codes"][0], bits_k)), f"seq {b}: K code rows differ"
    bits_v = OC.code_bits(OC.Spec(*c.v))
    vb = gathered("v_codes", (P // 32, lay.v_block_bytes), np.uint8, -(-Tq // 32))
    got_v = OC.unpack_vblocks(vb, bits_v, D, Tq)
    exp_v = OC.unpack_vblocks(OC.pack_vblocks(st["v"]["codes"][0], bits_v), bits_v, D, Tq)
    assert np.array_equal(got_v, exp_v), f"seq {b}: V code blocks differ"
    for side, spec in (("k", c.k), ("v", c.v)):
        part = st[side]
        if spec[0] in (OC.FP8_E4M3, OC.FP8_E5M2):
            off = getattr(lay, side + "_scale")
            s = pc.arena[off: off + 4 * H].cpu().numpy().view(np.float32)
            exp = np.asarray(part["scale"] if fp8_scales is None else fp8_scales[side], np.float32)
            assert np.array_equal(s.view(np.uint32), exp.view(np.uint32)), f"{side} fp8 scale differs"
            continue
        if spec[0] == OC.NONE:
            continue
        mdt, bits_t = (np.float16, np.uint16) if c.meta16 else (np.float32, np.uint32)
        if spec[2] == OC.PER_CHANNEL:
            G = spec[3]
            sc = gathered(side + "_scale", (P // G, D), mdt, Tq // G)
            zz = gathered(side + "_zero", (P // G, D), mdt, Tq // G) if spec[0] == OC.INT_ASYM else None
        else:
            cols = D // (spec[3] or D)
            sc = gathered(side + "_scale", (P, cols), mdt, Tq)
            zz = gathered(side + "_zero", (P, cols), mdt, Tq) if spec[0] == OC.INT_ASYM else None
        exp_s = part["scale"][0].reshape(sc.shape)
        assert np.array_equal(sc.view(bits_t), exp_s.astype(mdt).view(bits_t)), f"seq {b}: {side} scales differ"
        if zz is not None:
            assert np.array_equal(zz.astype(np.float32), part["zero"][0].reshape(zz.shape)), \
                f"seq {b}: {side} zero-points differ"
    if T > Tq:
        Rs = lay.ring_slots
        slots = OC.window_slots(c.oracle_cfg(), Tq, T)
        n = Rs * D * 2
        rk = pc.arena[lay.ring_k + b * H * n: lay.ring_k + (b + 1) * H * n].cpu().numpy().view(np.float16)
        rk = rk.reshape(H, Rs, D)[:, slots]
        assert np.array_equal(rk.view(np.uint16), st["k_window"][0].view(np.uint16)), f"seq {b}: ring K differs"
        rvb = pc.arena[lay.ring_v + b * H * n: lay.ring_v + (b + 1) * H * n].cpu().numpy()
        rv = OC.unpack_vblocks(rvb.reshape(H, Rs // 32, 32 * D * 2), 16, D, Rs)[:, slots]
        assert np.array_equal(rv.view(np.uint16), st["v_window"][0].view(np.uint16)), f"seq {b}: ring V differs"
