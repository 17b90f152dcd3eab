"""BitNet b1.58 BitLinear forward pass for AMD Instinct MI355X (gfx950).

The compute lives in ``libbitlinear.so`` (HIP kernels behind a C ABI,
declared in ``include/bitlinear.h``).  ``bit_gemm_bitlinear_amd.bitlinear``
is the thin ctypes binding over it; ``bit_gemm_bitlinear_amd.workloads``
draws the seeded synthetic inputs.  Importing this package loads nothing;
importing the binding loads the library and raises if it is missing.
"""

__all__ = ["bitlinear", "workloads"]
