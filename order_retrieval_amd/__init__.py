"""MI355X-native ZETA causal top-k attention (Z-order selection + Adaptive Cauchy weighting).

The hot path lives in hand-written HIP kernels behind the C ABI declared in
``include/zeta.h``; :mod:`order_retrieval_amd.zeta` is the thin ctypes binding over it and
:mod:`order_retrieval_amd.inputs` holds the seeded synthetic workloads.  Nothing is imported
eagerly so that the input generator can be used without the native library.
"""

__all__ = ["inputs", "zeta"]
