"""Paged-KV attention for MI355X (gfx950): HIP kernels behind a C ABI.

``binding`` exposes the library's calls (``decode``, ``mixed``,
``decode_partials``, ``merge_partials``, plan and metadata checks) on torch
tensors; it loads the built ``libpa_kv.so`` and raises if it is missing.
``accounting`` holds the algorithmic byte and flop counts.
"""
import importlib

from . import accounting  # noqa: F401

__all__ = ["accounting", "binding"]


def __getattr__(name):
    if name == "binding":
        return importlib.import_module(__name__ + ".binding")
    raise AttributeError(name)
