"""Fused LoRA MLP / QKV projections for MI355X (gfx950).

The compute path lives in a HIP shared library behind a C ABI
(``include/lora_mi355x.h``); ``lora_fine_tuning_mlp_amd.binding`` is the thin
ctypes layer over it.  Importing this package does not load the library.
"""
__all__ = ["binding", "synthetic"]
