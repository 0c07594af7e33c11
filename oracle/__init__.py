"""Plain, slow CPU oracle of KV-cache quantization and quantized decode attention.

TEST INFRASTRUCTURE ONLY: tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg are the only code allowed to import it.  It shares no code
with the HIP library (quantized_decode_attention_05_amd) and imports nothing
from it; both sides only share the seeded input generators in ``workloads``.

Modules:
  quant      element quantizers (asymmetric min-max, symmetric INT8, FP8 E4M3)
  cache      residual window, grouping axes, whole-cache quantization, byte layout
  attention  exact fp64 softmax attention, GQA mapping, RoPE
"""
from . import attention, cache, quant  # noqa: F401
