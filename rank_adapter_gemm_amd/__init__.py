"""MI355X-native mixed-adapter LoRA linear layer.

    y = x W + s_a (x A_a) B_a      per token row, a = its adapter slot (-1 = none)

The layer runs in hand-written HIP kernels for gfx950 behind the C ABI of
include/lora.h (liblora.so, built in-tree by ``python -m
rank_adapter_gemm_amd.build``).  ``rank_adapter_gemm_amd.lora`` is the Python
binding (same names as the C functions); ``workloads`` draws seeded
synthetic batches.
"""
from . import lora  # noqa: F401
from .lora import AdapterPool, LoraError, Workspace  # noqa: F401
