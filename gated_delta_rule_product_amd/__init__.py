"""Sparse Delta Memory (SDM) chunked write/read and decode step for AMD Instinct MI355X (gfx950).

The compute path is a C-ABI shared library of hand-written HIP kernels (``csrc/``, header ``include/sdm.h``);
``binding`` marshals torch tensors to it. ``synth`` draws seeded synthetic inputs.
"""
__all__ = ["binding", "synth", "build"]


def __getattr__(name):  # lazy: importing the package must not require the built library
    if name in ("binding", "synth", "build"):
        import importlib

        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
