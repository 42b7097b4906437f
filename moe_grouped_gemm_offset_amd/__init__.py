"""MI355X-native grouped GEMMs for the MoE expert backward pass.

The product is the C-ABI library libgg_moe.so (declared in include/gg_moe.h);
the functions exported here are a thin ctypes binding with the same names.
Nothing is loaded at import time: the binding module loads the library on
first use and raises if it has not been built.
"""

_BINDING_NAMES = ("gg_wgrad", "gg_dglu", "gg_dsrelu", "gg_abi_version",
                  "gg_last_error", "gg_device_error", "load_library",
                  "GGError", "gg_wgrad_workspace_size", "gg_dglu_workspace_size",
                  "gg_dsrelu_workspace_size")


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
