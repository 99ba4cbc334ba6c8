"""MI355X-native MX quantization and block-scaled GEMM.

The compute path is the HIP library ``libmx.so`` (gfx950 kernels behind a C
ABI declared in ``include/mx.h``); ``fp4_quantization_block_amd.mx`` is its
ctypes binding.  Importing this package loads nothing: the library is loaded
on the first call and a missing library raises an error.
"""
__all__ = ["mx", "inputs"]
