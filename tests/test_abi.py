"""C-ABI checks that need no GPU: the library loads, exports every function declared in
include/dflash.h, and host-side validation rejects bad arguments before any launch."""
import ctypes
import os
import re

import pytest

from block_diffusion_drafter_03_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dflash.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash_[a-z_]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert _declared() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    for name in _declared():
        assert hasattr(L, name), name


def test_status_strings():
    assert _lib.status_str(0) == "DFLASH_OK"
    for s in range(-1, -7, -1):
        assert _lib.status_str(s).startswith("DFLASH_E_")


def _desc(**kw):
    d = _lib.ModelDesc()
    d.dtype, d.n_layers, d.hidden = _lib.DFLASH_BF16, 1, 256
    d.n_q_heads, d.n_kv_heads, d.head_dim, d.ffn, d.vocab = 4, 2, 128, 256, 100
    d.rms_eps, d.rope_base, d.mask_token_id, d.n_taps = 1e-6, 10000.0, 99, 0
    fake = ctypes.c_void_p(0x1000)
    d.embed = d.lm_head = d.final_norm = fake.value
    arr = (ctypes.c_void_p * 6)(*([0x1000] * 6))
    d._arr = arr
    d.layer_w = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def _create(d):
    h = ctypes.c_void_p()
    st = _lib.lib().dflash_model_create(ctypes.byref(d), ctypes.byref(h))
    return st, h.value


def test_model_create_validates():
    st, h = _create(_desc())
    assert st == 0 and h
    _lib.model_destroy(h)
    assert _create(_desc(dtype=7))[0] == -3
    assert _create(_desc(head_dim=64))[0] == -2          # bf16 path needs head_dim 128
    assert _create(_desc(hidden=200))[0] == -2           # hidden % 128
    assert _create(_desc(n_kv_heads=3))[0] == -2         # GQA group must divide
    assert _create(_desc(mask_token_id=100))[0] == -1
    assert _create(_desc(embed=None))[0] == -1
    st, _ = _create(_desc(dtype=_lib.DFLASH_F32, head_dim=64, hidden=256, ffn=768))
    assert st == 0


def test_model_create_validates_convolutions():
    ptrs = (ctypes.c_void_p * 8)(*([0x7000] * 8))
    d = _desc()
    d.dconv = ctypes.cast(ptrs, ctypes.POINTER(ctypes.c_void_p))
    st, h = _create(d)
    assert st == 0
    _lib.model_destroy(h)
    ptrs[5] = None                       # a missing convolution tensor
    assert _create(d)[0] == -1
    ptrs[5] = 0x7000
    taps = (ctypes.c_int32 * 1)(0)       # a target (tapped layers) cannot hold convolutions
    d.n_taps, d.tap_layers = 1, ctypes.cast(taps, ctypes.POINTER(ctypes.c_int32))
    assert _create(d)[0] == -2


def test_workspace_bytes_and_entry_validation():
    st, h = _create(_desc())
    assert st == 0
    try:
        assert _lib.workspace_bytes(h, 1, 16, 4096, 0) > 0
        assert _lib.workspace_bytes(h, 1, 65, 4096, 0) == 0
        assert _lib.workspace_bytes(h, 0, 16, 4096, 0) == 0
        kv = _lib.KV()
        kv.n_layers, kv.n_kv_heads, kv.head_dim, kv.page_size = 1, 2, 128, 64
        kv.batch, kv.max_pages_per_seq, kv.num_pages = 1, 4, 4
        pools = (ctypes.c_void_p * 1)(0x2000)
        kv.k_pool = kv.v_pool = ctypes.cast(pools, ctypes.POINTER(ctypes.c_void_p))
        kv.block_table = kv.seq_len = 0x3000
        kv.capacity_tokens, kv.len_bound = 256, 0
        L = _lib.lib()
        one = ctypes.c_void_p(0x4000)
        # every rejection below happens on the host, before any kernel launch
        assert L.dflash_draft_block(h, ctypes.byref(kv), one, 0, one, None, None, one, 1 << 30, None) == -2
        assert L.dflash_draft_block(h, ctypes.byref(kv), one, 16, one, None, None, one, 16, None) == -5
        assert L.dflash_draft_block(h, ctypes.byref(kv), None, 16, one, None, None, one, 1 << 30, None) == -1
        kv.page_size = 32
        assert L.dflash_draft_block(h, ctypes.byref(kv), one, 16, one, None, None, one, 1 << 30, None) == -2
        kv.page_size = 64
        kv.head_dim = 64
        assert L.dflash_verify_accept(h, ctypes.byref(kv), one, one, 16, None, one, one, one, None,
                                      None, one, 1 << 30, None) == -2
        kv.head_dim = 128
        assert L.dflash_verify_accept(h, ctypes.byref(kv), one, None, 16, None, one, one, one, None,
                                      None, one, 1 << 30, None) == -1
        kv.head_dim = 128
        # drafter-only call on a model without W_c
        assert L.dflash_inject_ctx(h, ctypes.byref(kv), one, 4, one, one, 0, 1, one, 1 << 30, None) == -1
        assert L.dflash_kv_commit(None, None, one, 16, None) == -1
        assert L.dflash_kv_commit(ctypes.byref(kv), None, one, 0, None) == -2
        # sampling entry points: temperature, counter, required logits buffers, block >= 2
        ds = L.dflash_draft_block_sampled
        assert ds(h, ctypes.byref(kv), one, 16, 0.0, 1, 0, one, one, one, 1 << 30, None) == -1
        assert ds(h, ctypes.byref(kv), one, 16, 1.0, 1, -1, one, one, one, 1 << 30, None) == -1
        assert ds(h, ctypes.byref(kv), one, 16, 1.0, 1, 0, one, None, one, 1 << 30, None) == -1
        assert ds(h, ctypes.byref(kv), one, 1, 1.0, 1, 0, one, one, one, 1 << 30, None) == -2
        assert ds(h, ctypes.byref(kv), one, 16, 1.0, 1, 0, one, one, one, 16, None) == -5
        vs = L.dflash_verify_sampled
        assert vs(h, ctypes.byref(kv), one, one, one, 16, -1.0, 1, 0, None, one, one, one, one,
                  1 << 30, None) == -1
        assert vs(h, ctypes.byref(kv), one, one, None, 16, 1.0, 1, 0, None, one, one, one, one,
                  1 << 30, None) == -1
        assert vs(h, ctypes.byref(kv), one, one, one, 65, 1.0, 1, 0, None, one, one, one, one,
                  1 << 30, None) == -2
        # path selector: weights, rank (multiple of 16, <= 512), top_k (1 .. 16), logits buffer,
        # block >= 2, its own scratch
        sel = _lib.Selector()
        sel.w_ab, sel.w_h, sel.rank, sel.top_k = 0x5000, 0x6000, 256, 16
        assert _lib.selector_workspace_bytes(h, sel, 1, 16) > 0
        assert _lib.selector_workspace_bytes(h, sel, 1, 1) == 0
        dsel = L.dflash_draft_block_select

        def call(block=16, logits=one, sel_bytes=1 << 30):
            return dsel(h, ctypes.byref(kv), one, block, ctypes.byref(sel), one, logits, None, one,
                        1 << 30, one, sel_bytes, None)
        assert call(logits=None) == -1
        assert call(block=1) == -2
        assert call(sel_bytes=16) == -5
        for field, bad, code in (("rank", 100, -2), ("rank", 1024, -2), ("top_k", 0, -2),
                                 ("top_k", 17, -2), ("w_h", 0, -1)):
            keep = getattr(sel, field)
            setattr(sel, field, bad)
            assert call() == code, field
            assert _lib.selector_workspace_bytes(h, sel, 1, 16) == 0
            setattr(sel, field, keep)
    finally:
        _lib.model_destroy(h)


def _kv(capacity_tokens, len_bound, max_pages=4):
    kv = _lib.KV()
    kv.n_layers, kv.n_kv_heads, kv.head_dim, kv.page_size = 1, 2, 128, 64
    kv.batch, kv.max_pages_per_seq, kv.num_pages = 2, max_pages, 2 * max_pages
    pools = (ctypes.c_void_p * 1)(0x2000)
    kv._pools = pools
    kv.k_pool = kv.v_pool = ctypes.cast(pools, ctypes.POINTER(ctypes.c_void_p))
    kv.block_table = kv.seq_len = 0x3000
    kv.capacity_tokens, kv.len_bound = capacity_tokens, len_bound
    return kv


def test_capacity_is_refused_on_the_host_before_any_launch():
    """[DF] section 4.5: verification writes the block's K/V at n .. n+B-1 before acceptance
    is known.  A call whose rows could pass the mapped positions (capacity_tokens, with the
    host-side bound len_bound on every sequence length) returns DFLASH_E_CAPACITY (-4)
    without launching anything (no GPU here: a launch would fail differently)."""
    ptrs = (ctypes.c_void_p * 2)(0x1000, 0x1000)
    st, h = _create(_desc(w_c=ptrs[0], g_c=ptrs[1], n_taps=1))
    assert st == 0
    L = _lib.lib()
    one = ctypes.c_void_p(0x4000)
    big = 1 << 34
    try:
        kv = _kv(capacity_tokens=256, len_bound=250)
        # verify writes 16 rows at positions up to 250 + 15 >= 256
        assert L.dflash_verify_accept(h, ctypes.byref(kv), one, one, 16, None, one, one, one, None,
                                      None, one, big, None) == -4
        assert L.dflash_verify_sampled(h, ctypes.byref(kv), one, one, one, 16, 1.0, 1, 0, None, one,
                                       one, one, one, big, None) == -4
        # commit could advance a length past the mapped pages; the bound is left unchanged
        assert L.dflash_kv_commit(ctypes.byref(kv), None, one, 16, None) == -4
        assert L.dflash_kv_commit(None, ctypes.byref(kv), one, 16, None) == -4
        assert kv.len_bound == 250
        # injection: absolute rows up to pos_limit, relative rows up to len_bound + pos_limit
        assert L.dflash_inject_ctx(h, ctypes.byref(kv), one, 4, one, one, 0, 257, one, big, None) == -4
        assert L.dflash_inject_ctx(h, ctypes.byref(kv), one, 4, one, one, 1, 16, one, big, None) == -4
        assert L.dflash_inject_ctx(h, ctypes.byref(kv), one, 4, one, one, 1, 0, one, big, None) == -1
        # the drafter only reads its context, which must lie inside the mapped pages
        kv.len_bound = 257
        assert L.dflash_draft_block(h, ctypes.byref(kv), one, 16, one, None, None, one, big, None) == -4
        assert L.dflash_draft_block_sampled(h, ctypes.byref(kv), one, 16, 1.0, 1, 0, one, one, one,
                                            big, None) == -4
        # inconsistent host fields are argument errors
        for cap, bound in ((257, 0), (-1, 0), (256, -1)):
            kv = _kv(capacity_tokens=cap, len_bound=bound)
            assert L.dflash_verify_accept(h, ctypes.byref(kv), one, one, 16, None, one, one, one,
                                          None, None, one, big, None) == -1, (cap, bound)
    finally:
        _lib.model_destroy(h)


def test_noalloc_draft_block_refuses_steps_past_its_scratch():
    """dflash_draft_block_noalloc runs only steps whose scratch fits the library's array:
    a larger one is DFLASH_E_WORKSPACE (-5) on the host, before any launch or lookup."""
    st, h = _create(_desc())
    assert st == 0
    L = _lib.lib()
    one = ctypes.c_void_p(0x4000)
    try:
        kv = _kv(capacity_tokens=256, len_bound=0)
        kv.batch = 1024                       # 1024 x 64 rows of 256 floats: 64 MiB of h alone
        assert _lib.workspace_bytes(h, 1024, 64, 256, 0) > _lib.NOALLOC_SCRATCH_BYTES
        assert L.dflash_draft_block_noalloc(h, ctypes.byref(kv), one, 64, one, None, None, None) == -5
        assert L.dflash_draft_block_noalloc(h, ctypes.byref(kv), one, 65, one, None, None, None) == -2
        assert L.dflash_draft_block_noalloc(h, ctypes.byref(kv), None, 16, one, None, None, None) == -1
    finally:
        _lib.model_destroy(h)


def test_product_path_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError):
        _lib.lib()


def test_probe_read_validates_before_any_launch():
    # NULL source or sink, or a size that is not a multiple of 16: refused on the host
    L = _lib.lib()
    p = ctypes.c_void_p(16)    # never dereferenced: validation fails first
    assert L.dflash_probe_read(None, 1024, 0, p, None) == -1   # DFLASH_E_ARG
    assert L.dflash_probe_read(p, 1024, 1, None, None) == -1   # DFLASH_E_ARG
    assert L.dflash_probe_read(p, 1000, 0, p, None) == -1   # DFLASH_E_ARG
