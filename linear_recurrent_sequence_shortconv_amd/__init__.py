"""PRISM layer hot path on AMD MI355X (gfx950): HIP kernels behind a C ABI.

``forward`` and ``backward`` are thin bindings over ``libprism.so``; the
submodule ``workloads`` draws seeded synthetic inputs.  The binding is loaded
lazily so that ``workloads`` imports without touching the GPU runtime.
"""

__all__ = ["forward", "backward", "forward_workspace_bytes", "backward_workspace_bytes"]


def __getattr__(name):
    if name in __all__:
        from . import prism
        return getattr(prism, name)
    raise AttributeError(name)
