"""Exact ties of the LM-head argmax across workgroups: an LM head whose rows repeat with
period P gives every row's largest logit at n*, n* + P, n* + 2P, ... - bit-equal values in
different 16-column tiles, hence in different workgroups, whose 64-bit atomic maxima must
keep the lowest index ([DF] section 2.2, greedy decoding; ties to the lowest id as
everywhere in the oracle).  Checked at 16 block rows (the GEMV LM head, whose last
workgroup decodes the ids) and more (the tiled LM head), with and without the logits copy,
wherever the oracle's top-2 gap over the P distinct columns is clear."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from block_diffusion_drafter_03_amd import runtime as rt

from harness import DEV, NEAR_TIE, Setup, inject_all

pytestmark = pytest.mark.gpu

PERIOD = 100   # not a multiple of 16: the copies sit at different offsets of their tiles


@pytest.mark.parametrize("name", ["split_bf16", "mid_bf16", "narrow_bf16"])
def test_draft_ids_on_exact_ties_across_tiles(name):
    w = synth.workload(name)
    S = Setup(w)
    m = w.draft
    lm = S.shared["lm_head"]
    periodic = lm[torch.arange(m.vocab, device=lm.device) % PERIOD].contiguous()
    shared = {**S.shared, "lm_head": periodic}
    model = rt.Model(m, S.dw, shared, n_taps=w.n_taps, draft=True)
    np_shared = {**S.np_shared, "lm_head": synth.to_numpy(periodic)}
    lens = synth.ctx_lengths(w)
    B = w.block
    kv = S.kv(m, max(lens) + B + 70)
    ws = S.workspace(S.draft, B, kv.capacity, inject_rows=sum(lens))
    feats = [synth.features(w, n, DEV, tag=f"feats.b{b}") for b, n in enumerate(lens)]
    inject_all(S, kv, feats, ws)
    anchor = synth.anchors(w, DEV)
    ids = torch.zeros(w.batch, B - 1, dtype=torch.int32, device=DEV)
    logits = torch.zeros(w.batch, B - 1, m.vocab, device=DEV)
    rt.draft_block(model, kv, anchor, B, ids, ws, logits)       # logits copied
    ids2 = torch.zeros_like(ids)
    rt.draft_block(model, kv, anchor, B, ids2, ws)              # a decoding loop's call
    torch.cuda.synchronize()
    assert kv.err.item() == 0
    a_np = anchor.cpu().numpy()
    checked = 0
    for b, n in enumerate(lens):
        ctx = O.inject(synth.to_numpy(feats[b]), np.arange(n), S.np_dw, m, store=S.store)
        o_ids, o_z, _ = O.draft_block(S.np_dw, np_shared, m, ctx, int(a_np[b]), n, B, store=S.store)
        assert np.all(o_ids < PERIOD)   # the oracle's ties go to the lowest index
        clear = O.top2_gap(np.asarray(o_z[:, :PERIOD], dtype=np.float64)) >= NEAR_TIE
        for got, what in ((ids, "logits copied"), (ids2, "no copy")):
            g = got[b].cpu().numpy()
            bad = np.nonzero(clear & (g != o_ids))[0]
            assert bad.size == 0, f"{name} seq {b} {what}: ids {g[bad].tolist()} != {o_ids[bad].tolist()}"
            assert np.all(g < PERIOD), f"{name} seq {b} {what}: a tie not taken at the lowest index"
        checked += int(clear.sum())
    assert checked >= w.batch * (B - 1) // 2
    model.close()
