"""MI355X-native persistent fused communication + GEMM kernels (mKernel's hot path).

The compute path lives in the HIP library built from ``csrc/`` (``libmk.so``),
whose C ABI is declared in ``include/mk.h``.  ``communication_gemm_persistent_amd.mk``
is the thin ctypes binding over it (argument marshalling only); importing this
package does not load the library.
"""
__version__ = "0.1.0"
