"""Routed expert layer for AMD Instinct MI355X (gfx950).

The computation runs in the HIP library libmoe.so (C ABI in include/moe.h);
`_lib` binds its entry points under the same names and `runtime` sequences
them into decode steps and prefill layers.
"""
from . import _lib  # noqa: F401  (raises ImportError if the HIP library is not built)
from ._lib import *  # noqa: F401,F403
