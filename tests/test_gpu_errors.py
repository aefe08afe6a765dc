"""Device-side error reporting: every bad input the kernels can meet (an unmapped page, a
token id outside the vocabulary, an injection row outside its sequence's pages, tau outside
[1, block]) is clamped to a valid access, reported in the cache's error word, and leaves
the rest of the call's results as they would be without it."""
import pytest
import torch

import synth
from block_diffusion_drafter_03_amd import _lib
from block_diffusion_drafter_03_amd import runtime as rt

from harness import DEV, Setup, inject_all

pytestmark = pytest.mark.gpu


def _drafter(name="mid_bf16"):
    w = synth.workload(name)
    S = Setup(w)
    lens = synth.ctx_lengths(w)
    kv = S.kv(w.draft, max(lens) + w.block + 70)
    ws = S.workspace(S.draft, w.block, kv.capacity, inject_rows=sum(lens))
    feats = [synth.features(w, n, DEV, tag=f"feats.b{b}") for b, n in enumerate(lens)]
    inject_all(S, kv, feats, ws)
    torch.cuda.synchronize()
    assert kv.err.item() == 0
    return w, S, kv, ws, lens


def _draft(w, S, kv, ws, anchor):
    ids = torch.zeros(w.batch, w.block - 1, dtype=torch.int32, device=DEV)
    rt.draft_block(S.draft, kv, anchor, w.block, ids, ws)
    torch.cuda.synchronize()
    return ids.cpu()


def test_unmapped_context_page_is_flagged():
    w, S, kv, ws, lens = _drafter()
    anchor = synth.anchors(w, DEV)
    clean = _draft(w, S, kv, ws, anchor)
    assert lens[0] > 128
    kv.block_table[0, 1] = -1          # a page inside sequence 0's context
    ids = _draft(w, S, kv, ws, anchor)
    assert kv.err.item() & _lib.DEVERR_PAGE
    assert torch.equal(ids[1:], clean[1:])   # the other sequences are unaffected


def test_out_of_range_token_is_flagged():
    w, S, kv, ws, lens = _drafter()
    anchor = synth.anchors(w, DEV)
    clean = _draft(w, S, kv, ws, anchor)
    bad = anchor.clone()
    bad[1] = w.draft.vocab
    ids = _draft(w, S, kv, ws, bad)
    assert kv.err.item() & _lib.DEVERR_TOKEN
    assert torch.equal(ids[0], clean[0]) and torch.equal(ids[2], clean[2])


def test_injection_outside_the_pages_is_flagged_and_writes_nothing():
    w, S, kv, ws, lens = _drafter()
    before = [t.clone() for t in kv.k + kv.v]
    f = synth.features(w, 2, DEV, tag="feats.extra")
    row_seq = torch.tensor([0, w.batch], dtype=torch.int32, device=DEV)   # 2nd: no such sequence
    row_pos = torch.tensor([kv.capacity + 5, 0], dtype=torch.int32, device=DEV)
    rt.inject_ctx(S.draft, kv, f, row_seq, row_pos, 0, kv.capacity, ws)   # row 0 past pos_limit
    torch.cuda.synchronize()
    assert kv.err.item() & _lib.DEVERR_PAGE
    for a, b in zip(before, kv.k + kv.v):
        assert torch.equal(a, b)


def test_empty_injection_is_a_no_op():
    w, S, kv, ws, lens = _drafter()
    before = [t.clone() for t in kv.k + kv.v]
    f = synth.features(w, 0, DEV, tag="feats.none")
    empty = torch.zeros(0, dtype=torch.int32, device=DEV)
    rt.inject_ctx(S.draft, kv, f, empty, empty, 0, 1, ws)
    torch.cuda.synchronize()
    assert kv.err.item() == 0
    for a, b in zip(before, kv.k + kv.v):
        assert torch.equal(a, b)


def test_commit_clamps_and_flags_tau():
    w, S, kv, ws, lens = _drafter()
    tau = torch.tensor([0, w.block + 3, 2], dtype=torch.int32, device=DEV)
    rt.kv_commit(None, kv, tau, w.block)
    torch.cuda.synchronize()
    assert kv.err.item() & _lib.DEVERR_TAU
    assert kv.seq_len.cpu().tolist() == [lens[0] + 1, lens[1] + w.block, lens[2] + 2]


def test_selector_with_out_of_range_anchor_is_flagged():
    """The path selector gathers the anchor's embedding row for its first pair scores: an
    anchor outside the vocabulary is read as row 0 and flagged, like the embedding does,
    and the other sequences' picks are unaffected."""
    w, S, kv, ws, lens = _drafter()
    sw = synth.selector_weights(w, rank=64, device=DEV)
    sel = rt.Selector(S.draft, sw["w_a"].to(torch.bfloat16), sw["w_b"].to(torch.bfloat16),
                      sw["w_h"].to(torch.bfloat16), top_k=8)
    sws = rt.Workspace(sel.workspace_bytes(S.draft, w.batch, w.block), DEV)
    B, V = w.block, w.draft.vocab

    def run(anchor):
        ids = torch.zeros(w.batch, B - 1, dtype=torch.int32, device=DEV)
        zd = torch.zeros(w.batch, B - 1, V, device=DEV)
        rt.draft_block_select(S.draft, kv, anchor, B, sel, ids, zd, ws, sws)
        torch.cuda.synchronize()
        return ids.cpu()

    anchor = synth.anchors(w, DEV)
    clean = run(anchor)
    assert kv.err.item() == 0
    for bad_id in (V + 1000, -5):
        bad = anchor.clone()
        bad[1] = bad_id
        kv.err.zero_()
        ids = run(bad)
        assert kv.err.item() & _lib.DEVERR_TOKEN
        assert torch.equal(ids[0], clean[0]) and torch.equal(ids[2], clean[2])
