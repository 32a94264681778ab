"""POET-X orthogonal-equivalence linear layer for AMD MI355X (gfx950).

`poetx` is the ctypes binding of the C-ABI library libpoetx.so (built in-tree
by build_lib.build()); `PoetxLayer` wraps one layer's device buffers. Importing
the package fails if the library has not been built.
"""
from . import poetx  # noqa: F401  (loads libpoetx.so, raises if missing)
from .layer import PoetxLayer, build_many, param_grad_many  # noqa: F401

__all__ = ["poetx", "PoetxLayer", "build_many", "param_grad_many"]
