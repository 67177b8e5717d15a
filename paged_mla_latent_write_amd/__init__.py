"""Paged multi-head latent attention (MLA) over a block-table-indexed latent KV
cache, native to AMD MI355X (gfx950 / CDNA4).

The compute path is the C-ABI library ``libmla.so`` (hand-written HIP kernels);
``paged_mla_latent_write_amd.mla`` is a thin ctypes binding over it.  Importing
the binding raises if the library has not been built: there is no CPU fallback.
"""
import importlib

__all__ = ["mla", "workloads"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
