"""MI355X-native Nystrom kernel attention (Laplacian, with SOFT's Gaussian
variant), forward pass.  The compute path is the C-ABI library liblapattn.so
(hand-written HIP for gfx950); :mod:`.api` is a thin PyTorch binding.

Submodules are imported lazily so that the input generator in
:mod:`.workloads` stays importable without loading the library.
"""
import importlib

__all__ = ["api", "workloads"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
