"""kvq: FP8 / 4-bit paged KV-cache quantization and decode attention for MI355X.

The compute path is the C-ABI HIP library ``libkvq.so`` (sources in ``csrc/``,
header ``include/kvq.h``); ``kvq`` is its thin ctypes binding.  Import
``quantized_decode_attention_calibrate_amd.kvq`` to load it.
"""
__all__ = ["kvq", "workloads"]
