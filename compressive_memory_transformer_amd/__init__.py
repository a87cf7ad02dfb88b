"""Infini-attention segment forward for AMD MI355X (gfx950).

The compute path is the HIP library ``libinfini_attn.so`` built in-tree from
``csrc/`` (C ABI in ``include/infini_attn.h``); ``infini`` is its ctypes
binding and ``synthetic`` the seeded input generator.
"""

from .infini import InfiniAttention, InfiniError, LibraryNotBuilt, load_library  # noqa: F401

__all__ = ["InfiniAttention", "InfiniError", "LibraryNotBuilt", "load_library"]
