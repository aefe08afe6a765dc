"""Device-memory plumbing around libdflash: packed weights, paged caches, workspaces,
and torch-tensor wrappers of the four entry points (same names as the C ABI).

PyTorch only allocates device memory and supplies the current HIP stream; every step of
the drafter / verifier runs in libdflash's kernels.
"""
from __future__ import annotations

import ctypes
from ctypes import POINTER, c_int32, c_void_p

import torch

from . import _lib

PAGE = 64


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dt_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return _lib.DFLASH_BF16
    if t == torch.float32:
        return _lib.DFLASH_F32
    raise ValueError(f"unsupported dtype {t}")


def rotary_interleave(w, n_heads, d):
    """Rows of each head reordered so rotate-half partners are adjacent: packed row 2i is
    row i and packed row 2i+1 is row i + d/2 (the layout DFLASH_W_QKV expects for q, k)."""
    D = w.shape[1]
    return w.view(n_heads, 2, d // 2, D).transpose(1, 2).reshape(n_heads * d, D)


def pack_qkv(wq, wk, wv, n_q_heads, n_kv_heads, d):
    return torch.cat([rotary_interleave(wq, n_q_heads, d), rotary_interleave(wk, n_kv_heads, d),
                      wv], 0).contiguous()


def pack_gate_up(wg, wu):
    """Packed row 2j = gate row j, packed row 2j+1 = up row j."""
    return torch.stack([wg, wu], 1).reshape(2 * wg.shape[0], wg.shape[1]).contiguous()


def frag_pack(w):
    """bf16 matrix [N, K] -> the MFMA B-fragment order libdflash reads for bfloat16 models:
    rows padded to a multiple of 16; one 1 KB block per (16-row tile t, 32-wide step s),
    blocks in (t, s) order, and inside a block lane g*16 + r holding row r, k = 8g .. 8g+7."""
    N, K = w.shape
    NT = (N + 15) // 16
    if NT * 16 != N:
        w = torch.cat([w, w.new_zeros(NT * 16 - N, K)], 0)
    return w.reshape(NT, 16, K // 32, 4, 8).permute(0, 2, 3, 1, 4).contiguous()


class Model:
    """A drafter (``draft=True``: needs W_c and g_c) or a target model; a DFlash 2 drafter
    also takes its two-tap convolutions (``dconv``: keys L{i}.dconv_{name}.{base,w_k}).

    ``weights`` uses the per-layer names L{i}.{g_in,wq,wk,wv,wo,g_post,wg,wu,wd}, plus g_f
    and (drafter) w_c, g_c; ``shared`` holds embed and lm_head.  Q/K/V and gate/up are
    packed into the interleaved row layouts the library consumes, and for bfloat16 models
    every matrix but the embedding into the B-fragment order (see include/dflash.h)."""

    def __init__(self, shape, weights: dict, shared: dict, n_taps: int, taps=None,
                 draft: bool = True, dconv: dict = None):
        self.shape = shape
        dtype = shared["embed"].dtype
        self.dtype = dtype
        self._keep = []
        mat = frag_pack if dtype == torch.bfloat16 else (lambda t: t.contiguous())
        lw = []
        for i in range(shape.n_layers):
            qkv = pack_qkv(weights[f"L{i}.wq"], weights[f"L{i}.wk"], weights[f"L{i}.wv"],
                           shape.n_q_heads, shape.n_kv_heads, shape.head_dim)
            gu = pack_gate_up(weights[f"L{i}.wg"], weights[f"L{i}.wu"])
            tensors = [weights[f"L{i}.g_in"].contiguous(), mat(qkv), mat(weights[f"L{i}.wo"]),
                       weights[f"L{i}.g_post"].contiguous(), mat(gu), mat(weights[f"L{i}.wd"])]
            self._keep += tensors
            lw += [t.data_ptr() for t in tensors]
        self._lw = (c_void_p * len(lw))(*lw)
        embed = shared["embed"].contiguous()
        lm_head = mat(shared["lm_head"])
        self._keep += [embed, lm_head, weights["g_f"]]
        d = _lib.ModelDesc()
        d.dtype = _dt_code(dtype)
        d.n_layers, d.hidden = shape.n_layers, shape.hidden
        d.n_q_heads, d.n_kv_heads, d.head_dim = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
        d.ffn, d.vocab = shape.ffn, shape.vocab
        d.rms_eps, d.rope_base = shape.rms_eps, shape.rope_base
        d.mask_token_id = shape.mask_token_id
        d.n_taps = n_taps
        if taps is not None and not draft:
            self._taps = (c_int32 * len(taps))(*taps)
            d.tap_layers = ctypes.cast(self._taps, POINTER(c_int32))
        d.embed = embed.data_ptr()
        d.lm_head = lm_head.data_ptr()
        d.final_norm = weights["g_f"].data_ptr()
        if draft:
            w_c = mat(weights["w_c"])
            self._keep += [w_c, weights["g_c"]]
            d.w_c = w_c.data_ptr()
            d.g_c = weights["g_c"].data_ptr()
        d.layer_w = ctypes.cast(self._lw, POINTER(c_void_p))
        if dconv is not None:
            # DFlash 2 convolutions: base [2, D] as is, W_k [D, D/8] as weight rows [D/8, D]
            cp = []
            for i in range(shape.n_layers):
                for name in ("pre_attn", "post_attn", "pre_ffn", "post_ffn"):
                    key = f"L{i}.dconv_{name}"
                    base = dconv[key + ".base"].to(dtype).contiguous()
                    w_k = mat(dconv[key + ".w_k"].t().to(dtype).contiguous())
                    self._keep += [base, w_k]
                    cp += [base.data_ptr(), w_k.data_ptr()]
            self._dc = (c_void_p * len(cp))(*cp)
            d.dconv = ctypes.cast(self._dc, POINTER(c_void_p))
        self.desc = d
        self.handle = _lib.model_create(d)
        self.n_taps = n_taps

    def workspace_bytes(self, batch, block, max_ctx, max_inject_rows=0) -> int:
        return _lib.workspace_bytes(self.handle, batch, block, max_ctx, max_inject_rows)

    def close(self):
        if self.handle:
            _lib.model_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class PagedKV:
    """Paged K/V pools of one model for `batch` sequences of up to `capacity` positions.

    K pool per layer [num_pages, Hkv, 64, d]; V pool [num_pages, Hkv, d, 64] (transposed
    pages).  ``page_order`` may permute the physical pages handed to the sequences.  Every
    page of the block table is mapped, so the struct's capacity_tokens is the capacity;
    its host-side len_bound follows ``set_seq_len`` and each commit."""

    def __init__(self, shape, batch, capacity, dtype, device, page_order=None, spare_pages=0):
        self.shape = shape
        self.batch = batch
        self.max_pages = (capacity + PAGE - 1) // PAGE
        self.capacity = self.max_pages * PAGE
        self.num_pages = batch * self.max_pages + spare_pages
        L, H, d = shape.n_layers, shape.n_kv_heads, shape.head_dim
        self.k = [torch.zeros(self.num_pages, H, PAGE, d, dtype=dtype, device=device) for _ in range(L)]
        self.v = [torch.zeros(self.num_pages, H, d, PAGE, dtype=dtype, device=device) for _ in range(L)]
        if page_order is None:
            page_order = torch.arange(batch * self.max_pages)
        self.block_table = page_order.to(torch.int32).reshape(batch, self.max_pages).to(device).contiguous()
        self.seq_len = torch.zeros(batch, dtype=torch.int32, device=device)
        self.err = torch.zeros(1, dtype=torch.int32, device=device)
        self._kp = (c_void_p * L)(*[t.data_ptr() for t in self.k])
        self._vp = (c_void_p * L)(*[t.data_ptr() for t in self.v])
        s = _lib.KV()
        s.n_layers, s.n_kv_heads, s.head_dim = L, H, d
        s.page_size, s.batch = PAGE, batch
        s.max_pages_per_seq, s.num_pages = self.max_pages, self.num_pages
        s.k_pool = ctypes.cast(self._kp, POINTER(c_void_p))
        s.v_pool = ctypes.cast(self._vp, POINTER(c_void_p))
        s.block_table = self.block_table.data_ptr()
        s.seq_len = self.seq_len.data_ptr()
        s.error_flags = self.err.data_ptr()
        s.capacity_tokens = self.capacity
        s.len_bound = 0
        self.struct = s

    def set_seq_len(self, lens):
        """Committed lengths: an int for every sequence, or one per sequence.  Sets the
        device seq_len and the host-side upper bound the library checks capacity with."""
        if isinstance(lens, int):
            lens = [lens] * self.batch
        lens = [int(x) for x in lens]
        self.seq_len.copy_(torch.tensor(lens, dtype=torch.int32))
        self.struct.len_bound = max(lens)

    def refresh_len_bound(self):
        """Tighten the host-side bound to the device lengths (synchronises the stream)."""
        self.struct.len_bound = int(self.seq_len.max().item())

    @property
    def len_bound(self) -> int:
        return int(self.struct.len_bound)

    # --- plumbing used to load a synthetic context and to read a cache back ---------------
    def _slots(self, b, start, n):
        pos = torch.arange(start, start + n, device=self.block_table.device)
        pages = self.block_table[b, (pos // PAGE).long()].long()
        return pages, (pos % PAGE).long()

    def write_dense(self, layer, b, K, V, start=0):
        """Store K, V [n, Hkv, d] (K already rotated) at positions start .. start+n-1."""
        pages, slots = self._slots(b, start, K.shape[0])
        self.k[layer][pages, :, slots, :] = K.to(self.k[layer].dtype)
        self.v[layer].permute(0, 3, 1, 2)[pages, slots] = V.to(self.v[layer].dtype)

    def read_dense(self, layer, b, n, start=0):
        pages, slots = self._slots(b, start, n)
        K = self.k[layer][pages, :, slots, :]
        V = self.v[layer].permute(0, 3, 1, 2)[pages, slots]
        return K, V

    # --- checkpoint / resume ----------------------------------------------------------
    def snapshot(self) -> dict:
        """The committed state as host tensors, independent of the page layout: seq_len and,
        per layer and sequence, the K/V rows of positions 0 .. seq_len-1 (positions past a
        sequence's length hold rejected draft rows and are not part of the state).
        Synchronises the stream."""
        lens = self.seq_len.cpu()
        out = {"seq_len": lens.clone()}
        for layer in range(len(self.k)):
            for b in range(self.batch):
                K, V = self.read_dense(layer, b, int(lens[b]))
                out[f"k.{layer}.{b}"] = K.cpu().contiguous()
                out[f"v.{layer}.{b}"] = V.cpu().contiguous()
        return out

    def restore(self, snap: dict):
        """Load a snapshot of a cache of the same shape and batch (any page layout and any
        capacity that holds the lengths)."""
        lens = [int(x) for x in snap["seq_len"]]
        if len(lens) != self.batch or max(lens, default=0) > self.capacity:
            raise ValueError("snapshot does not fit this cache")
        dev = self.block_table.device
        for layer in range(len(self.k)):
            for b in range(self.batch):
                self.write_dense(layer, b, snap[f"k.{layer}.{b}"].to(dev), snap[f"v.{layer}.{b}"].to(dev))
        self.set_seq_len(lens)


class Workspace:
    def __init__(self, nbytes, device):
        self.nbytes = int(nbytes)
        self.buf = torch.empty(max(self.nbytes, 256), dtype=torch.uint8, device=device)


# --- entry points (torch tensors in, status checked) --------------------------------------

def inject_ctx(model: Model, kv: PagedKV, feats, row_seq, row_pos, pos_relative, pos_limit,
               ws: Workspace):
    """pos_limit: every row_pos lies in [0, pos_limit) (absolute positions, or offsets from
    the sequence's length when pos_relative)."""
    st = _lib.inject_ctx(model.handle, kv.struct, _ptr(feats), int(feats.shape[0]), _ptr(row_seq),
                         _ptr(row_pos), int(pos_relative), int(pos_limit), _ptr(ws.buf), ws.nbytes,
                         _stream())
    _lib._check(st, "dflash_inject_ctx")


def draft_block(model: Model, kv: PagedKV, anchor, block, draft_ids, ws: Workspace,
                logits_dbg=None, hidden_dbg=None):
    st = _lib.draft_block(model.handle, kv.struct, _ptr(anchor), int(block), _ptr(draft_ids),
                          _ptr(logits_dbg), _ptr(hidden_dbg), _ptr(ws.buf), ws.nbytes, _stream())
    _lib._check(st, "dflash_draft_block")


def draft_block_noalloc(model: Model, kv: PagedKV, anchor, block, draft_ids, logits_dbg=None,
                        hidden_dbg=None):
    """draft_block with the library's own per-GPU scratch instead of a workspace."""
    st = _lib.draft_block_noalloc(model.handle, kv.struct, _ptr(anchor), int(block), _ptr(draft_ids),
                                  _ptr(logits_dbg), _ptr(hidden_dbg), _stream())
    _lib._check(st, "dflash_draft_block_noalloc")


def verify_accept(model: Model, kv: PagedKV, anchor, draft_ids, block, feats_out, target_argmax,
                  tau, bonus, ws: Workspace, logits_dbg=None, hidden_dbg=None):
    """anchor [batch] and draft_ids [batch, block-1] (contiguous int32) form the block."""
    st = _lib.verify_accept(model.handle, kv.struct, _ptr(anchor), _ptr(draft_ids), int(block),
                            _ptr(feats_out), _ptr(target_argmax), _ptr(tau), _ptr(bonus),
                            _ptr(logits_dbg), _ptr(hidden_dbg), _ptr(ws.buf), ws.nbytes,
                            _stream())
    _lib._check(st, "dflash_verify_accept")


def draft_block_sampled(model: Model, kv: PagedKV, anchor, block, temperature, seed, counter,
                        draft_ids, draft_logits, ws: Workspace):
    st = _lib.draft_block_sampled(model.handle, kv.struct, _ptr(anchor), int(block),
                                  float(temperature), int(seed), int(counter), _ptr(draft_ids),
                                  _ptr(draft_logits), _ptr(ws.buf), ws.nbytes, _stream())
    _lib._check(st, "dflash_draft_block_sampled")


def verify_sampled(model: Model, kv: PagedKV, anchor, draft_ids, draft_logits, block, temperature,
                   seed, counter, feats_out, target_logits, tau, next_token, ws: Workspace):
    st = _lib.verify_sampled(model.handle, kv.struct, _ptr(anchor), _ptr(draft_ids),
                             _ptr(draft_logits), int(block), float(temperature), int(seed),
                             int(counter), _ptr(feats_out), _ptr(target_logits), _ptr(tau),
                             _ptr(next_token), _ptr(ws.buf), ws.nbytes, _stream())
    _lib._check(st, "dflash_verify_sampled")


class Selector:
    """DFlash 2 path-selector weights for a drafter: w_a, w_b, w_h [hidden, rank] (the maps
    A, B, H of the pair score), packed as the library's [rank, hidden] weight rows in the
    drafter's dtype and layout."""

    def __init__(self, model: Model, w_a, w_b, w_h, top_k=16):
        mat = frag_pack if model.dtype == torch.bfloat16 else (lambda t: t.contiguous())
        self.rank = int(w_a.shape[1])
        self.top_k = int(top_k)
        self.w_ab = mat(torch.cat([w_a.t(), w_b.t()], 0).to(model.dtype).contiguous())
        self.w_h = mat(w_h.t().to(model.dtype).contiguous())
        s = _lib.Selector()
        s.w_ab, s.w_h = self.w_ab.data_ptr(), self.w_h.data_ptr()
        s.rank, s.top_k = self.rank, self.top_k
        self.struct = s

    def workspace_bytes(self, model: Model, batch, block) -> int:
        return _lib.selector_workspace_bytes(model.handle, self.struct, batch, block)


def draft_block_select(model: Model, kv: PagedKV, anchor, block, sel: Selector, draft_ids,
                       draft_logits, ws: Workspace, sel_ws: Workspace, candidates=None):
    st = _lib.draft_block_select(model.handle, kv.struct, _ptr(anchor), int(block), sel.struct,
                                 _ptr(draft_ids), _ptr(draft_logits), _ptr(candidates),
                                 _ptr(ws.buf), ws.nbytes, _ptr(sel_ws.buf), sel_ws.nbytes,
                                 _stream())
    _lib._check(st, "dflash_draft_block_select")


def kv_commit(target_kv, draft_kv, tau, block):
    st = _lib.kv_commit(target_kv.struct if target_kv is not None else None,
                        draft_kv.struct if draft_kv is not None else None, _ptr(tau), int(block),
                        _stream())
    _lib._check(st, "dflash_kv_commit")
