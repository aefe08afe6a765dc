"""ctypes binding of libdflash (argument marshalling only; every step runs in HIP).

The functions mirror include/dflash.h one to one.  Tensors are passed as raw device
pointers (``tensor.data_ptr()``) together with torch's current HIP stream.  There is no
fallback: if ``libdflash.so`` is not built, loading raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int32, c_size_t, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdflash.so")

DFLASH_F32, DFLASH_BF16 = 0, 1
LAYER_TENSORS = 6
W_G_IN, W_QKV, W_O, W_G_POST, W_GATE_UP, W_DOWN = range(6)
DEVERR_PAGE, DEVERR_TOKEN, DEVERR_TAU = 1, 2, 4

EXPORTS = ("dflash_model_create", "dflash_model_destroy", "dflash_status_str",
           "dflash_workspace_bytes", "dflash_inject_ctx", "dflash_draft_block",
           "dflash_verify_accept", "dflash_kv_commit", "dflash_timing_arm",
           "dflash_timing_read", "dflash_draft_block_sampled", "dflash_verify_sampled",
           "dflash_selector_workspace_bytes", "dflash_draft_block_select",
           "dflash_draft_block_noalloc", "dflash_probe_read")
NOALLOC_SCRATCH_BYTES = 64 << 20
KERNEL_LM_HEAD, KERNEL_GEMM_QKV, KERNEL_GEMM_O, KERNEL_GEMM_GATE_UP, KERNEL_GEMM_DOWN, \
    KERNEL_ATTENTION, KERNEL_INJECT_FUSE, KERNEL_INJECT_KV = range(8)


class ModelDesc(ctypes.Structure):
    _fields_ = [("dtype", c_int32), ("n_layers", c_int32), ("hidden", c_int32),
                ("n_q_heads", c_int32), ("n_kv_heads", c_int32), ("head_dim", c_int32),
                ("ffn", c_int32), ("vocab", c_int32), ("rms_eps", c_float),
                ("rope_base", c_float), ("mask_token_id", c_int32), ("n_taps", c_int32),
                ("tap_layers", POINTER(c_int32)), ("embed", c_void_p), ("lm_head", c_void_p),
                ("final_norm", c_void_p), ("w_c", c_void_p), ("g_c", c_void_p),
                ("layer_w", POINTER(c_void_p)), ("dconv", POINTER(c_void_p))]


class KV(ctypes.Structure):
    _fields_ = [("n_layers", c_int32), ("n_kv_heads", c_int32), ("head_dim", c_int32),
                ("page_size", c_int32), ("batch", c_int32), ("max_pages_per_seq", c_int32),
                ("num_pages", c_int32), ("k_pool", POINTER(c_void_p)),
                ("v_pool", POINTER(c_void_p)), ("block_table", c_void_p),
                ("seq_len", c_void_p), ("error_flags", c_void_p),
                ("capacity_tokens", c_int32), ("len_bound", c_int32)]


class Selector(ctypes.Structure):
    _fields_ = [("w_ab", c_void_p), ("w_h", c_void_p), ("rank", c_int32), ("top_k", c_int32)]


class DFlashError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_str(status)} ({status})")
        self.status = status


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                               "(python -m block_diffusion_drafter_03_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        L.dflash_model_create.argtypes = [POINTER(ModelDesc), POINTER(c_void_p)]
        L.dflash_model_create.restype = c_int32
        L.dflash_model_destroy.argtypes = [c_void_p]
        L.dflash_model_destroy.restype = None
        L.dflash_status_str.argtypes = [c_int32]
        L.dflash_status_str.restype = ctypes.c_char_p
        L.dflash_workspace_bytes.argtypes = [c_void_p, c_int32, c_int32, c_int32, c_int32]
        L.dflash_workspace_bytes.restype = c_size_t
        L.dflash_inject_ctx.argtypes = [c_void_p, POINTER(KV), c_void_p, c_int32, c_void_p,
                                        c_void_p, c_int32, c_int32, c_void_p, c_size_t, c_void_p]
        L.dflash_inject_ctx.restype = c_int32
        L.dflash_draft_block.argtypes = [c_void_p, POINTER(KV), c_void_p, c_int32, c_void_p,
                                         c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
        L.dflash_draft_block.restype = c_int32
        L.dflash_draft_block_noalloc.argtypes = [c_void_p, POINTER(KV), c_void_p, c_int32, c_void_p,
                                                 c_void_p, c_void_p, c_void_p]
        L.dflash_draft_block_noalloc.restype = c_int32
        L.dflash_verify_accept.argtypes = [c_void_p, POINTER(KV), c_void_p, c_void_p, c_int32,
                                           c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                           c_void_p, c_void_p, c_size_t, c_void_p]
        L.dflash_verify_accept.restype = c_int32
        L.dflash_draft_block_sampled.argtypes = [c_void_p, POINTER(KV), c_void_p, c_int32, c_float,
                                                 ctypes.c_uint64, c_int32, c_void_p, c_void_p,
                                                 c_void_p, c_size_t, c_void_p]
        L.dflash_draft_block_sampled.restype = c_int32
        L.dflash_verify_sampled.argtypes = [c_void_p, POINTER(KV), c_void_p, c_void_p, c_void_p,
                                            c_int32, c_float, ctypes.c_uint64, c_int32, c_void_p,
                                            c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                            c_void_p]
        L.dflash_verify_sampled.restype = c_int32
        L.dflash_selector_workspace_bytes.argtypes = [c_void_p, POINTER(Selector), c_int32, c_int32]
        L.dflash_selector_workspace_bytes.restype = c_size_t
        L.dflash_draft_block_select.argtypes = [c_void_p, POINTER(KV), c_void_p, c_int32,
                                                POINTER(Selector), c_void_p, c_void_p, c_void_p,
                                                c_void_p, c_size_t, c_void_p, c_size_t, c_void_p]
        L.dflash_draft_block_select.restype = c_int32
        L.dflash_kv_commit.argtypes = [POINTER(KV), POINTER(KV), c_void_p, c_int32, c_void_p]
        L.dflash_kv_commit.restype = c_int32
        L.dflash_timing_arm.argtypes = [c_int32, c_int32]
        L.dflash_timing_arm.restype = c_int32
        L.dflash_timing_read.argtypes = [POINTER(c_float), c_int32]
        L.dflash_timing_read.restype = c_int32
        L.dflash_probe_read.argtypes = [c_void_p, ctypes.c_size_t, c_int32, c_void_p, c_void_p]
        L.dflash_probe_read.restype = c_int32
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().dflash_status_str(int(status)).decode()


def _check(status: int, where: str):
    if status != 0:
        raise DFlashError(status, where)


def model_create(desc: ModelDesc) -> int:
    h = c_void_p()
    _check(lib().dflash_model_create(ctypes.byref(desc), ctypes.byref(h)), "dflash_model_create")
    return h.value


def model_destroy(handle: int):
    lib().dflash_model_destroy(c_void_p(handle))


def workspace_bytes(handle: int, batch: int, block: int, max_ctx: int, max_inject_rows: int) -> int:
    return int(lib().dflash_workspace_bytes(c_void_p(handle), batch, block, max_ctx, max_inject_rows))


def inject_ctx(handle, kv: KV, feats, n_rows, row_seq, row_pos, pos_relative, pos_limit, ws,
               ws_bytes, stream) -> int:
    return lib().dflash_inject_ctx(c_void_p(handle), ctypes.byref(kv), feats, n_rows, row_seq,
                                   row_pos, pos_relative, pos_limit, ws, ws_bytes, stream)


def draft_block(handle, kv: KV, anchor, block, draft_ids, logits_dbg, hidden_dbg, ws, ws_bytes,
                stream) -> int:
    return lib().dflash_draft_block(c_void_p(handle), ctypes.byref(kv), anchor, block, draft_ids,
                                    logits_dbg, hidden_dbg, ws, ws_bytes, stream)


def draft_block_noalloc(handle, kv: KV, anchor, block, draft_ids, logits_dbg, hidden_dbg,
                        stream) -> int:
    return lib().dflash_draft_block_noalloc(c_void_p(handle), ctypes.byref(kv), anchor, block,
                                            draft_ids, logits_dbg, hidden_dbg, stream)


def verify_accept(handle, kv: KV, anchor, draft_ids, block, feats_out, target_argmax, tau, bonus,
                  logits_dbg, hidden_dbg, ws, ws_bytes, stream) -> int:
    return lib().dflash_verify_accept(c_void_p(handle), ctypes.byref(kv), anchor, draft_ids, block,
                                      feats_out, target_argmax, tau, bonus, logits_dbg,
                                      hidden_dbg, ws, ws_bytes, stream)


def draft_block_sampled(handle, kv: KV, anchor, block, temperature, seed, counter, draft_ids,
                        draft_logits, ws, ws_bytes, stream) -> int:
    return lib().dflash_draft_block_sampled(c_void_p(handle), ctypes.byref(kv), anchor, block,
                                            temperature, seed, counter, draft_ids, draft_logits,
                                            ws, ws_bytes, stream)


def verify_sampled(handle, kv: KV, anchor, draft_ids, draft_logits, block, temperature, seed,
                   counter, feats_out, target_logits, tau, next_token, ws, ws_bytes, stream) -> int:
    return lib().dflash_verify_sampled(c_void_p(handle), ctypes.byref(kv), anchor, draft_ids,
                                       draft_logits, block, temperature, seed, counter, feats_out,
                                       target_logits, tau, next_token, ws, ws_bytes, stream)


def selector_workspace_bytes(handle, sel: Selector, batch: int, block: int) -> int:
    return int(lib().dflash_selector_workspace_bytes(c_void_p(handle), ctypes.byref(sel), batch, block))


def draft_block_select(handle, kv: KV, anchor, block, sel: Selector, draft_ids, draft_logits,
                       candidates, ws, ws_bytes, sel_ws, sel_ws_bytes, stream) -> int:
    return lib().dflash_draft_block_select(c_void_p(handle), ctypes.byref(kv), anchor, block,
                                           ctypes.byref(sel), draft_ids, draft_logits, candidates,
                                           ws, ws_bytes, sel_ws, sel_ws_bytes, stream)


def timing_arm(kernel: int, capacity: int):
    _check(lib().dflash_timing_arm(kernel, capacity), "dflash_timing_arm")


def timing_read(capacity: int) -> list:
    buf = (c_float * max(capacity, 1))()
    n = lib().dflash_timing_read(buf, capacity)
    if n < 0:
        raise DFlashError(n, "dflash_timing_read")
    return [float(buf[i]) for i in range(n)]


def probe_read(src, nbytes: int, nontemporal: bool, sink, stream):
    """Measurement utility: one read of nbytes at device pointer src (plain or non-temporal
    loads) into the 16 KiB device buffer sink."""
    _check(lib().dflash_probe_read(src, nbytes, 1 if nontemporal else 0, sink, stream), "dflash_probe_read")


def kv_commit(target_kv, draft_kv, tau, block, stream) -> int:
    t = ctypes.byref(target_kv) if target_kv is not None else None
    d = ctypes.byref(draft_kv) if draft_kv is not None else None
    return lib().dflash_kv_commit(t, d, tau, block, stream)
