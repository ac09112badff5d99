"""MI355X-native trellis-coded GEMV (QTIP / EXL3-style bitshift trellis + computed code + randomized Hadamard).

The compute lives in libtrellis_gemv.so (HIP kernels for gfx950, C ABI in
include/trellis_gemv.h); ``trellis_coded_gemv_amd.binding`` is the thin ctypes
layer over it, and ``trellis_coded_gemv_amd.inputs`` builds seeded synthetic
layers. Build the library with ``python -m trellis_coded_gemv_amd.build``.
"""
__all__ = ["binding", "inputs", "build"]
