"""One expert-parallel rank's share of a Mixture-of-Experts layer on MI355X.

Route -> dispatch -> grouped bf16 MFMA GEMMs (gate/up with SwiGLU, down) ->
combine, as hand-written HIP kernels for gfx950 behind a C ABI
(``include/moe_layer_03_amd.h``).  ``binding`` holds the ctypes wrappers;
``workloads`` the named workloads and the seeded input generator.

The library is loaded on first use of the binding; importing the package
touches neither HIP nor the GPU.
"""
from . import workloads  # noqa: F401

__all__ = ["workloads", "binding"]


def __getattr__(name):
    if name == "binding":
        import importlib
        return importlib.import_module(__name__ + ".binding")
    raise AttributeError(name)
