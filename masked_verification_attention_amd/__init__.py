"""MI355X-native verification step for self-speculative decoding.

The product is a C-ABI shared library of hand-written HIP kernels for gfx950
(``libspecverify.so``, declared in ``include/spec_verify.h``).  This package
holds its sources (``csrc/``), the build step (``build.py``), a thin ctypes
binding with the same entry-point names (``binding``), and the seeded
synthetic workloads (``workloads``).  The binding is loaded lazily, and every
call raises if the HIP library is missing: there is no CPU fallback.
"""

__all__ = ["binding", "workloads"]


def __getattr__(name):
    if name in __all__:
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
