"""int4 routed-expert MoE layer for AMD MI355X (gfx950).

The layer is the per-token path of the Colibri engine pages (Route, Union,
then the int4 SwiGLU experts over the union, then the routing-weighted
combine), implemented as hand-written HIP kernels behind a C ABI
(``include/coli_moe.h``).  ``binding`` is the thin ctypes layer over that
library; it is imported lazily so that the input generator (``inputs``) and
the workload table (``configs``) load without the GPU library.
"""

__all__ = ["configs", "inputs", "binding"]


def __getattr__(name):
    if name == "binding":
        import importlib
        return importlib.import_module(__name__ + ".binding")
    raise AttributeError(name)
