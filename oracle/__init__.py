"""fp64 CPU oracle for the mixed-adapter LoRA linear layer.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import, call or link anything in this
directory.  It shares no code with the HIP library and never imports it.
Every function here cites the passage of the pages it follows (see
``oracle.py`` and ``lora_oracle.c``).  ``fp8.py`` (imported as
``oracle.fp8``) holds the E4M3 quantization and the FP8-base layer.
"""
from .oracle import (  # noqa: F401
    BF16, F32, adapter_param_count, affinity_cores, bf16_bits_from_f32, build_oracle, default_threads,
    f32_from_bf16_bits, lora_scale, oracle_rows, oracle_segmented, oracle_segments,
)
