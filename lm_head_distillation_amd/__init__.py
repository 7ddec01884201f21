"""Fused-linear generalized-JSD distillation pass for AMD MI355X (gfx950).

The compute path is the HIP library libfljsd.so (C ABI: include/fljsd.h);
``lm_head_distillation_amd.fljsd`` is its Python binding.
"""
__all__ = ["fljsd"]
