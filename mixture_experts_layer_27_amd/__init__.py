"""MI355X-native token-choice top-k MoE FFN layer (forward + backward).

The compute path is a C-ABI HIP library (``libmoe_mi355x.so``) built for gfx950;
``mixture_experts_layer_27_amd.binding`` is a thin ctypes layer over it.  The
binding is imported lazily so that the input generator and the config table can
be used without a built library.
"""
import importlib

__all__ = ["configs", "synth", "binding"]


def __getattr__(name):
    if name == "binding":
        return importlib.import_module(".binding", __name__)
    raise AttributeError(name)
