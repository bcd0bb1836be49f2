"""qgemm for MI355X: C = A . dequant(Wq) through hand-written gfx950 HIP kernels.

The C library (include/qgemm.h) is reached through `weight_quantized_mixed_amd.qgemm`
(ctypes, same names as the C ABI); `weight_quantized_mixed_amd.device` wraps it for
torch device tensors.  Importing this package loads nothing.
"""
