"""MI355X-native DFlash drafter step and greedy block verification.

The compute lives in ``libdflash.so`` (hand-written HIP for gfx950, C ABI in
``include/dflash.h``); this package holds its ctypes binding and the device-memory
plumbing around it.
"""
from . import _lib  # noqa: F401
from .runtime import (Model, PagedKV, Workspace, draft_block, inject_ctx, kv_commit,  # noqa: F401
                      verify_accept)
