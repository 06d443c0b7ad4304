"""MI355X-native forward pass of one DeepSeek-V3-style MoE block.

The compute lives in libmoe.so (HIP kernels for gfx950 behind a C ABI, see
include/moe.h). `mixture_experts_layer_14_amd.moe` is the thin ctypes binding;
`mixture_experts_layer_14_amd.inputs` draws seeded synthetic inputs.
Importing the package does not load the library; the binding does, and raises
if it is missing.
"""
__all__ = ["inputs", "moe"]
