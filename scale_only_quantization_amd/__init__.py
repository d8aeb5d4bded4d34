"""Scale-only fake-quant training of a grouped MoE expert layer on AMD MI355X.

The HIP library (csrc/, built into libfq.so by ``build.py``) implements the
C ABI of include/fq.h; ``fqlib`` is its ctypes binding.  Import ``fqlib``
explicitly: it raises if the library has not been built.
"""
__all__ = ["fqlib", "build"]
