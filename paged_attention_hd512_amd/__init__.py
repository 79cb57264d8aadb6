"""Paged GQA attention at head_dim 512 for MI355X (gfx950): decode and prefill.

The compute lives in libpa.so (include/pa.h): a host planner and hand-written HIP kernels.
This package is its ctypes binding (``paged_attention_hd512_amd.pa``); PyTorch supplies
device memory and streams.  Importing the package does not load the library; the first
call does, and fails loudly if the library has not been built.
"""

from . import pa  # noqa: F401
from .pa import PagedDecode, PagedPrefill, PaError  # noqa: F401

__all__ = ["pa", "PagedDecode", "PagedPrefill", "PaError"]
