"""FastMKA (route-fused memory-keyed attention) layer forward for MI355X (gfx950).

The compute path is a C-ABI shared library of hand-written HIP kernels
(``csrc/``, header ``include/mka.h``).  ``route_kv_memory_amd.mka`` is the thin
ctypes binding to it; ``route_kv_memory_amd.inputs`` holds the seeded synthetic
input generators and the workload shapes.  Importing the package loads nothing:
the binding is imported on first use of ``route_kv_memory_amd.mka``.
"""

__all__ = ["inputs", "mka"]


def __getattr__(name):
    if name in __all__:
        import importlib

        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
