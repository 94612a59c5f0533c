"""LOCKS decode hot path for MI355X (gfx950): C ABI in liblocks.so, thin
ctypes binding in ``kv_cache_page_int4_amd.locks``."""

from . import locks  # noqa: F401
