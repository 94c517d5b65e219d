"""MI355X-native compressed-sparse-attention (CSA) decode path.

The compute lives in ``libcsa.so`` (hand-written HIP kernels for gfx950 behind
a C ABI declared in ``include/csa.h``).  ``binding`` marshals torch device
tensors into those calls; it is imported lazily so that the input generators
(``inputs``) can be used on a machine without the library.
"""
import importlib

__all__ = ["binding", "inputs"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
