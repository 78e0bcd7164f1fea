"""MI355X-native replayed SSM decode (Mamba-2 and Gated DeltaNet layers).

The compute path is the HIP library libreplayssm.so built from csrc/; the
Python side only marshals arguments (binding.py).  Submodules load lazily so
that the seeded input generators (synth.py) import without the GPU library.
"""
import importlib

__all__ = ["binding", "synth", "build"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
