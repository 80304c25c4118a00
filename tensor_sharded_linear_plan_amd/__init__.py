"""One rank's share of tensor-parallel linear layers on one MI355X.

The compute lives in ``libtsl.so`` (hand-written HIP kernels for gfx950
behind a C ABI declared in ``include/tsl.h``).  ``binding`` is a thin ctypes
layer over it with the same entry-point names; it raises ImportError when
the library has not been built -- there is no fallback.

``synth`` (seeded input generators), ``configs`` (workload sizes) and
``build`` (the compiler driver) do not need the library.
"""
import importlib

__all__ = ["binding", "synth", "configs"]


def __getattr__(name):
    if name in ("binding", "synth", "configs", "build"):
        return importlib.import_module("." + name, __name__)
    # entry points re-exported from the binding: loading it loads libtsl.so
    binding = importlib.import_module(".binding", __name__)
    if hasattr(binding, name):
        return getattr(binding, name)
    raise AttributeError(name)
