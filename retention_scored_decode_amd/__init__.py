"""Retention-scored KV-cache eviction and renormalised decode attention for
MI355X (gfx950): a HIP library (libtrimkv.so) behind a C ABI, and this thin
ctypes binding.  See include/trimkv.h for the operations."""
from .trimkv import (  # noqa: F401
    BF16, F32, PAGE, Cache, TrimkvError, allocate, append, attn_mass, compact, decode_attn, lib,
    log_beta, score, select_global, strerror, validate_cache, workspace, workspace_size,
)
from . import trimkv  # noqa: F401
