"""MI355X-native quantized KV cache and decode attention (HIP kernels behind a C ABI).

The binding in ``_lib`` mirrors include/kvq.h; torch is used only for device
memory and streams.
"""
from ._lib import (  # noqa: F401
    AttnOptions, Config, KvqError, Layout, TensorSpec, EXPORTED,
    NONE, INT_ASYM, INT_SYM, FP8_E4M3, FP8_E5M2, PER_TENSOR, PER_CHANNEL, PER_TOKEN, F32, F16, BF16,
    CALIBRATE, INIT, KERNEL_AUTO, KERNEL_GENERIC, KERNEL_MFMA,
    kvq_abi_version, kvq_arena_bytes, kvq_arena_layout, kvq_decode_attention, kvq_decode_attention_static, kvq_decode_step, kvq_decode_step_fused,
    kvq_dequantize, kvq_paged_decode_attention, kvq_paged_decode_step, kvq_paged_dequantize,
    kvq_paged_quantize_append,
    kvq_quantize_append, kvq_quantized_tokens, kvq_status_string, kvq_validate_config,
    kvq_workspace_bytes, make_config, STATIC_WORKSPACE_BYTES,
)
