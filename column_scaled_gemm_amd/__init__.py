"""FP8 (E4M3FN) activation quant + scaled GEMM for MI355X (gfx950).

The compute path is the C-ABI library ``libfp8sm.so`` (hand-written HIP
kernels); ``column_scaled_gemm_amd.fp8sm`` is its thin ctypes binding and
``column_scaled_gemm_amd.inputs`` the seeded synthetic inputs.  Importing the
package loads nothing native; the binding loads the library on first use and
raises if it is missing.
"""
