"""ctypes binding of libkvq.so (include/kvq.h): argument marshalling only.

Every computation runs in the library's HIP kernels.  Torch tensors are used
for device memory and streams: the wrappers pass ``data_ptr()`` and the
current HIP stream.  Importing this module fails loudly when the library has
not been built (``python quantized_decode_attention_05_amd/build.py``).
"""
from __future__ import annotations

import ctypes as C
import os

# torch ships its own HIP runtime (soname libamdhip64.so.7).  Loading it first
# makes libkvq.so bind to that same runtime instead of a second copy from
# /opt/rocm, which would fail to see the device once torch has opened it.
import torch  # noqa: F401  (device memory and streams)

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      f"`python quantized_decode_attention_05_amd/build.py`")
_lib = C.CDLL(LIB_PATH)

# ---- constants (mirror include/kvq.h) ------------------------------------------
KVQ_OK = 0
STATUS = {0: "KVQ_OK", -1: "KVQ_ERR_INVALID_ARG", -2: "KVQ_ERR_UNSUPPORTED", -3: "KVQ_ERR_CAPACITY",
          -4: "KVQ_ERR_ALIGN", -5: "KVQ_ERR_NULL", -6: "KVQ_ERR_WORKSPACE", -7: "KVQ_ERR_HIP"}
NONE, INT_ASYM, INT_SYM, FP8_E4M3, FP8_E5M2 = 0, 1, 2, 3, 4
PER_TENSOR, PER_CHANNEL, PER_TOKEN = 0, 1, 2
F32, F16, BF16 = 0, 1, 2
CALIBRATE = 1
INIT = 2            # paged appends: the call that starts the cache
KERNEL_AUTO, KERNEL_GENERIC, KERNEL_MFMA = 0, 1, 2


class TensorSpec(C.Structure):
    _fields_ = [("scheme", C.c_int32), ("bits", C.c_int32), ("axis", C.c_int32), ("group", C.c_int32)]


class Config(C.Structure):
    _fields_ = [("batch", C.c_int32), ("num_q_heads", C.c_int32), ("num_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("max_tokens", C.c_int64), ("in_dtype", C.c_int32),
                ("out_dtype", C.c_int32), ("k", TensorSpec), ("v", TensorSpec),
                ("residual", C.c_int32), ("pre_rope_k", C.c_int32), ("rope_base", C.c_float),
                ("meta_dtype", C.c_int32), ("page_tokens", C.c_int32), ("num_pages", C.c_int32)]


class Layout(C.Structure):
    _fields_ = [(n, C.c_size_t) for n in ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale",
                                          "v_zero", "ring_k", "ring_v", "rope", "fp8_calib",
                                          "total_bytes")] + \
               [("token_capacity", C.c_int64), ("k_row_bytes", C.c_int32), ("v_block_bytes", C.c_int32),
                ("ring_slots", C.c_int32), ("token_group", C.c_int32), ("k_meta_cols", C.c_int32),
                ("v_meta_cols", C.c_int32), ("page_tokens", C.c_int64), ("pages", C.c_int32),
                ("reserved", C.c_int32)]


class AttnOptions(C.Structure):
    _fields_ = [("kernel", C.c_int32), ("num_splits", C.c_int32), ("reserved", C.c_int32 * 6)]


_P = C.c_void_p
_CFG = C.POINTER(Config)
_sig = {
    "kvq_validate_config": (C.c_int, [_CFG]),
    "kvq_arena_layout": (C.c_int, [_CFG, C.POINTER(Layout)]),
    "kvq_arena_bytes": (C.c_int, [_CFG, C.POINTER(C.c_size_t)]),
    "kvq_quantized_tokens": (C.c_int64, [_CFG, C.c_int64]),
    "kvq_quantize_append": (C.c_int, [_CFG, _P, C.c_int64, C.c_int32, _P, _P, _P, _P, C.c_uint32, _P]),
    "kvq_workspace_bytes": (C.c_int, [_CFG, C.c_int64, C.POINTER(AttnOptions), C.POINTER(C.c_size_t)]),
    "kvq_decode_attention": (C.c_int, [_CFG, _P, C.c_int64, _P, _P, C.c_float, _P, C.c_size_t,
                                       C.POINTER(AttnOptions), _P]),
    "kvq_decode_attention_static": (C.c_int, [_CFG, _P, C.c_int64, _P, _P, C.c_float, C.POINTER(AttnOptions), _P]),
    "kvq_decode_step": (C.c_int, [_CFG, _P, C.c_int64, _P, _P, _P, _P, C.c_float, _P, C.c_size_t,
                                  C.POINTER(AttnOptions), _P]),
    "kvq_decode_step_fused": (C.c_int, [_CFG, C.c_int64, C.POINTER(AttnOptions)]),
    "kvq_dequantize": (C.c_int, [_CFG, _P, C.c_int64, _P, _P, _P]),
    "kvq_paged_quantize_append": (C.c_int, [_CFG, _P, _P, C.c_int32, _P, _P, C.c_int32, _P, _P, _P, _P,
                                            C.c_uint32, _P]),
    "kvq_paged_decode_attention": (C.c_int, [_CFG, _P, _P, C.c_int32, _P, C.c_int64, _P, _P, C.c_float, _P,
                                             C.c_size_t, C.POINTER(AttnOptions), _P]),
    "kvq_paged_decode_step": (C.c_int, [_CFG, _P, _P, C.c_int32, _P, C.c_int64, _P, _P, _P, _P, C.c_float, _P,
                                        C.c_size_t, C.POINTER(AttnOptions), _P]),
    "kvq_paged_dequantize": (C.c_int, [_CFG, _P, _P, C.c_int32, _P, C.c_int64, _P, _P, _P]),
    "kvq_status_string": (C.c_char_p, [C.c_int]),
    "kvq_abi_version": (C.c_int, []),
}
for _name, (_res, _args) in _sig.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_sig)


class KvqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} "
                         f"({_lib.kvq_status_string(status).decode()})")


def _check(st: int, where: str) -> int:
    if st != KVQ_OK:
        raise KvqError(st, where)
    return st


def make_config(*, batch, num_q_heads, num_kv_heads, head_dim, max_tokens, k, v,
                in_dtype=BF16, out_dtype=F32, residual=0, pre_rope_k=False,
                rope_base=10000.0, meta_dtype=F32, page_tokens=0, num_pages=0) -> Config:
    """k, v: (scheme, bits, axis, group) tuples; meta_dtype: F32 or F16 storage
    of the INT sides' scales and zero-points; page_tokens > 0: a paged cache
    of num_pages pages of page_tokens tokens."""
    return Config(batch, num_q_heads, num_kv_heads, head_dim, max_tokens, in_dtype, out_dtype,
                  TensorSpec(*k), TensorSpec(*v), residual, int(bool(pre_rope_k)), rope_base, meta_dtype,
                  page_tokens, num_pages)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


_TORCH_DTYPE = {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16}


def _need(t, name, *, dtype=None, shape=None, min_bytes=None):
    """Check a tensor argument before its pointer crosses the ABI: the C entry
    points take raw pointers and (for the arena) no size, so a wrong shape,
    dtype, layout or a too-small buffer here would become an out-of-bounds
    device access.  Checks run in this order (contiguity, dtype, shape, byte
    size) and raise ValueError naming the argument; each wrapper checks that
    its tensors live on the GPU (_on_gpu) after every argument passed these."""
    if t is None:
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if min_bytes is not None and t.numel() * t.element_size() < min_bytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, needs at least {min_bytes}")
    return t


def _on_gpu(**tensors):
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")


def _in_dtype(cfg):
    dt = _TORCH_DTYPE.get(cfg.in_dtype)
    if dt is None:
        raise ValueError(f"unknown in_dtype {cfg.in_dtype}")
    return dt


def _out_dtype(cfg):
    dt = _TORCH_DTYPE.get(cfg.out_dtype)
    if dt is None:
        raise ValueError(f"unknown out_dtype {cfg.out_dtype}")
    return dt


def _check_arena(cfg, arena):
    return _need(arena, "arena", min_bytes=kvq_arena_bytes(cfg))


def _check_new_tokens(cfg, k_new, v_new):
    _need(k_new, "k_new", dtype=_in_dtype(cfg))
    if k_new.dim() != 4 or tuple(k_new.shape[:2]) != (cfg.batch, cfg.num_kv_heads) or \
            k_new.shape[3] != cfg.head_dim:
        raise ValueError(f"k_new has shape {tuple(k_new.shape)}, expected "
                         f"({cfg.batch}, {cfg.num_kv_heads}, n_new, {cfg.head_dim})")
    _need(v_new, "v_new", dtype=_in_dtype(cfg), shape=k_new.shape)


def _check_query_out(cfg, q, out):
    _need(q, "q", dtype=_in_dtype(cfg), shape=(cfg.batch, cfg.num_q_heads, cfg.head_dim))
    _need(out, "out", dtype=_out_dtype(cfg), shape=(cfg.batch, cfg.num_q_heads, cfg.head_dim))


def _stream(stream, *tensors):
    if stream is not None:
        return C.c_void_p(stream)
    import torch
    for t in tensors:
        if t is not None and t.is_cuda:
            return C.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)
    return C.c_void_p(0)


def _opts(kernel=0, num_splits=0):
    o = AttnOptions()
    o.kernel, o.num_splits = kernel, num_splits
    return o


def kvq_abi_version() -> int:
    return _lib.kvq_abi_version()


def kvq_status_string(status: int) -> str:
    return _lib.kvq_status_string(status).decode()


def kvq_validate_config(cfg: Config) -> int:
    return _lib.kvq_validate_config(C.byref(cfg))


def kvq_arena_layout(cfg: Config) -> Layout:
    lay = Layout()
    _check(_lib.kvq_arena_layout(C.byref(cfg), C.byref(lay)), "kvq_arena_layout")
    return lay


def kvq_arena_bytes(cfg: Config) -> int:
    n = C.c_size_t()
    _check(_lib.kvq_arena_bytes(C.byref(cfg), C.byref(n)), "kvq_arena_bytes")
    return n.value


def kvq_quantized_tokens(cfg: Config, T: int) -> int:
    r = _lib.kvq_quantized_tokens(C.byref(cfg), T)
    if r < 0:
        raise KvqError(int(r), "kvq_quantized_tokens")
    return int(r)


def kvq_workspace_bytes(cfg: Config, T: int, kernel: int = 0, num_splits: int = 0) -> int:
    n = C.c_size_t()
    o = _opts(kernel, num_splits)
    _check(_lib.kvq_workspace_bytes(C.byref(cfg), T, C.byref(o), C.byref(n)), "kvq_workspace_bytes")
    return n.value


def kvq_quantize_append(cfg: Config, arena, t0: int, k_new, v_new, k_scale=None, v_scale=None,
                        flags: int = 0, stream=None) -> None:
    """k_new, v_new: device tensors [B, Hkv, n_new, D] in cfg.in_dtype;
    k_scale, v_scale: fp32 [Hkv] (FP8 E4M3 sides only) or None."""
    _check_arena(cfg, arena)
    _check_new_tokens(cfg, k_new, v_new)
    for nm, sc in (("k_scale", k_scale), ("v_scale", v_scale)):
        if sc is not None:
            _need(sc, nm, dtype=torch.float32, shape=(cfg.num_kv_heads,))
    _on_gpu(arena=arena, k_new=k_new, v_new=v_new, k_scale=k_scale, v_scale=v_scale)
    n_new = int(k_new.shape[2])
    st = _lib.kvq_quantize_append(C.byref(cfg), _ptr(arena), t0, n_new, _ptr(k_new), _ptr(v_new),
                                  _ptr(k_scale), _ptr(v_scale), flags,
                                  _stream(stream, arena, k_new))
    _check(st, "kvq_quantize_append")


def kvq_decode_attention(cfg: Config, arena, T: int, q, out, sm_scale: float, workspace,
                         kernel: int = 0, num_splits: int = 0, stream=None) -> None:
    """q: [B, Hq, D] in cfg.in_dtype; out: [B, Hq, D] in cfg.out_dtype."""
    o = _opts(kernel, num_splits)
    _check_arena(cfg, arena)
    _check_query_out(cfg, q, out)
    if workspace is not None:
        _need(workspace, "workspace")
    _on_gpu(arena=arena, q=q, out=out, workspace=workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib.kvq_decode_attention(C.byref(cfg), _ptr(arena), T, _ptr(q), _ptr(out), sm_scale,
                                   _ptr(workspace), ws_bytes, C.byref(o), _stream(stream, arena, q))
    _check(st, "kvq_decode_attention")


STATIC_WORKSPACE_BYTES = 16 << 20   # KVQ_STATIC_WORKSPACE_BYTES


def kvq_decode_attention_static(cfg: Config, arena, T: int, q, out, sm_scale: float, kernel: int = 0,
                                num_splits: int = 0, stream=None) -> None:
    """kvq_decode_attention with the split partials in the library's own
    device array (no workspace argument; calls on one GPU must not overlap)."""
    o = _opts(kernel, num_splits)
    _check_arena(cfg, arena)
    _check_query_out(cfg, q, out)
    _on_gpu(arena=arena, q=q, out=out)
    st = _lib.kvq_decode_attention_static(C.byref(cfg), _ptr(arena), T, _ptr(q), _ptr(out), sm_scale,
                                          C.byref(o), _stream(stream, arena, q))
    _check(st, "kvq_decode_attention_static")


def kvq_decode_step(cfg: Config, arena, t0: int, k_new, v_new, q, out, sm_scale: float, workspace,
                    kernel: int = 0, num_splits: int = 0, stream=None) -> None:
    """Append one token per sequence at t0 (k_new, v_new: [B, Hkv, 1, D]) and
    attend over t0 + 1 tokens (q: [B, Hq, D]; out: [B, Hq, D])."""
    o = _opts(kernel, num_splits)
    _check_arena(cfg, arena)
    _check_new_tokens(cfg, k_new, v_new)
    if k_new.shape[2] != 1:
        raise ValueError(f"k_new has {k_new.shape[2]} tokens per sequence, a decode step appends 1")
    _check_query_out(cfg, q, out)
    if workspace is not None:
        _need(workspace, "workspace")
    _on_gpu(arena=arena, k_new=k_new, v_new=v_new, q=q, out=out, workspace=workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib.kvq_decode_step(C.byref(cfg), _ptr(arena), t0, _ptr(k_new), _ptr(v_new), _ptr(q), _ptr(out),
                              sm_scale, _ptr(workspace), ws_bytes, C.byref(o), _stream(stream, arena, q))
    _check(st, "kvq_decode_step")


def kvq_decode_step_fused(cfg: Config, t0: int, kernel: int = 0, num_splits: int = 0) -> bool:
    """Whether kvq_decode_step at t0 appends inside the attention launch."""
    r = _lib.kvq_decode_step_fused(C.byref(cfg), t0, C.byref(_opts(kernel, num_splits)))
    if r < 0:
        raise KvqError(int(r), "kvq_decode_step_fused")
    return bool(r)


def kvq_dequantize(cfg: Config, arena, T: int, k_out=None, v_out=None, stream=None) -> None:
    """k_out, v_out: fp32 device tensors [B, Hkv, T, D] (either may be None)."""
    _check_arena(cfg, arena)
    for nm, t in (("k_out", k_out), ("v_out", v_out)):
        if t is not None:
            _need(t, nm, dtype=torch.float32, shape=(cfg.batch, cfg.num_kv_heads, T, cfg.head_dim))
    _on_gpu(arena=arena, k_out=k_out, v_out=v_out)
    st = _lib.kvq_dequantize(C.byref(cfg), _ptr(arena), T, _ptr(k_out), _ptr(v_out),
                             _stream(stream, arena))
    _check(st, "kvq_dequantize")


# raw entry points for tests that pass pointers directly
raw = _lib


# ---- paged caches ----------------------------------------------------------------

def _check_paged_tables(cfg, block_table, seq_lens, new_lens=None):
    _need(block_table, "block_table", dtype=torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != cfg.batch:
        raise ValueError(f"block_table has shape {tuple(block_table.shape)}, expected ({cfg.batch}, max_blocks)")
    _need(seq_lens, "seq_lens", dtype=torch.int32, shape=(cfg.batch,))
    if new_lens is not None:
        _need(new_lens, "new_lens", dtype=torch.int32, shape=(cfg.batch,))
    return int(block_table.shape[1])


def kvq_paged_quantize_append(cfg: Config, arena, block_table, seq_lens, k_new, v_new, new_lens=None,
                              k_scale=None, v_scale=None, flags: int = 0, stream=None) -> None:
    """Append to a paged cache: block_table int32 [B, max_blocks], seq_lens /
    new_lens int32 [B] (device), k_new / v_new [B, Hkv, n_max, D]."""
    _check_arena(cfg, arena)
    max_blocks = _check_paged_tables(cfg, block_table, seq_lens, new_lens)
    _check_new_tokens(cfg, k_new, v_new)
    for nm, sc in (("k_scale", k_scale), ("v_scale", v_scale)):
        if sc is not None:
            _need(sc, nm, dtype=torch.float32, shape=(cfg.num_kv_heads,))
    _on_gpu(arena=arena, block_table=block_table, seq_lens=seq_lens, new_lens=new_lens, k_new=k_new,
            v_new=v_new, k_scale=k_scale, v_scale=v_scale)
    st = _lib.kvq_paged_quantize_append(C.byref(cfg), _ptr(arena), _ptr(block_table), max_blocks, _ptr(seq_lens),
                                        _ptr(new_lens), int(k_new.shape[2]), _ptr(k_new), _ptr(v_new),
                                        _ptr(k_scale), _ptr(v_scale), flags, _stream(stream, arena, k_new))
    _check(st, "kvq_paged_quantize_append")


def kvq_paged_decode_attention(cfg: Config, arena, block_table, seq_lens, max_seq_len: int, q, out,
                               sm_scale: float, workspace, kernel: int = 0, num_splits: int = 0,
                               stream=None) -> None:
    o = _opts(kernel, num_splits)
    _check_arena(cfg, arena)
    max_blocks = _check_paged_tables(cfg, block_table, seq_lens)
    _check_query_out(cfg, q, out)
    if workspace is not None:
        _need(workspace, "workspace")
    _on_gpu(arena=arena, block_table=block_table, seq_lens=seq_lens, q=q, out=out, workspace=workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib.kvq_paged_decode_attention(C.byref(cfg), _ptr(arena), _ptr(block_table), max_blocks,
                                         _ptr(seq_lens), max_seq_len, _ptr(q), _ptr(out), sm_scale,
                                         _ptr(workspace), ws_bytes, C.byref(o), _stream(stream, arena, q))
    _check(st, "kvq_paged_decode_attention")


def kvq_paged_decode_step(cfg: Config, arena, block_table, seq_lens, max_seq_len: int, k_new, v_new, q, out,
                          sm_scale: float, workspace, kernel: int = 0, num_splits: int = 0,
                          stream=None) -> None:
    o = _opts(kernel, num_splits)
    _check_arena(cfg, arena)
    max_blocks = _check_paged_tables(cfg, block_table, seq_lens)
    _check_new_tokens(cfg, k_new, v_new)
    if k_new.shape[2] != 1:
        raise ValueError(f"k_new has {k_new.shape[2]} tokens per sequence, a decode step appends 1")
    _check_query_out(cfg, q, out)
    if workspace is not None:
        _need(workspace, "workspace")
    _on_gpu(arena=arena, block_table=block_table, seq_lens=seq_lens, k_new=k_new, v_new=v_new, q=q, out=out,
            workspace=workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib.kvq_paged_decode_step(C.byref(cfg), _ptr(arena), _ptr(block_table), max_blocks, _ptr(seq_lens),
                                    max_seq_len, _ptr(k_new), _ptr(v_new), _ptr(q), _ptr(out), sm_scale,
                                    _ptr(workspace), ws_bytes, C.byref(o), _stream(stream, arena, q))
    _check(st, "kvq_paged_decode_step")


def kvq_paged_dequantize(cfg: Config, arena, block_table, seq_lens, max_seq_len: int, k_out=None, v_out=None,
                         stream=None) -> None:
    _check_arena(cfg, arena)
    max_blocks = _check_paged_tables(cfg, block_table, seq_lens)
    for nm, t in (("k_out", k_out), ("v_out", v_out)):
        if t is not None:
            _need(t, nm, dtype=torch.float32, shape=(cfg.batch, cfg.num_kv_heads, max_seq_len, cfg.head_dim))
    _on_gpu(arena=arena, block_table=block_table, seq_lens=seq_lens, k_out=k_out, v_out=v_out)
    st = _lib.kvq_paged_dequantize(C.byref(cfg), _ptr(arena), _ptr(block_table), max_blocks, _ptr(seq_lens),
                                   max_seq_len, _ptr(k_out), _ptr(v_out), _stream(stream, arena))
    _check(st, "kvq_paged_dequantize")
