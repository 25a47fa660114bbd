"""MI355X-native Prox two-stage sparse SwiGLU FFN decode step.

The compute path is the HIP library ``libprox.so`` (C ABI declared in
``include/prox.h``); ``free_sparse_swiglu_amd.prox`` is its thin ctypes
binding.  Importing this package does not load the library: the first call
into ``prox`` does, and it raises if the library is missing.
"""
__all__ = ["prox", "synth", "costmodel"]
