"""A draft block captured once in a HIP graph and replayed reproduces the eager block bit for
bit, on every replay, with eager work between the replays: the kernels keep no state across
calls except the split GEMMs' arrival counters, which the block's first kernel clears and
every split re-arms (no memset is recorded).  Batch 1 (M = 16: the K-split GEMVs and the LM
head's id decode) and the mid model at batch 3 (M = 48: row-resident K-split GEMMs and their
reduces, operand planes)."""
import pytest
import torch

import synth
from block_diffusion_drafter_03_amd import runtime as rt

from harness import DEV, Setup, inject_all

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["split_bf16", "mid_bf16"])
def test_captured_draft_block_replays_bit_for_bit(name):
    w = synth.workload(name)
    S = Setup(w)
    lens = synth.ctx_lengths(w)
    B, m = w.block, w.draft
    kv = S.kv(m, max(lens) + B + 70)
    ws = S.workspace(S.draft, B, kv.capacity, inject_rows=sum(lens))
    inject_all(S, kv, [synth.features(w, n, DEV, tag=f"feats.b{b}") for b, n in enumerate(lens)], ws)
    anchor = synth.anchors(w, DEV)
    ids = torch.zeros(w.batch, B - 1, dtype=torch.int32, device=DEV)
    logits = torch.zeros(w.batch, B - 1, m.vocab, device=DEV)
    rt.draft_block(S.draft, kv, anchor, B, ids, ws, logits)
    torch.cuda.synchronize()
    ids0, logits0 = ids.clone(), logits.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up on the capture stream
        rt.draft_block(S.draft, kv, anchor, B, ids, ws, logits)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rt.draft_block(S.draft, kv, anchor, B, ids, ws, logits)
    for rep in range(4):
        ids.zero_()
        logits.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ids, ids0), f"{name}: replay {rep} ids differ"
        assert torch.equal(logits, logits0), f"{name}: replay {rep} logits differ"
        # eager work on the same workspace between the replays
        rt.draft_block(S.draft, kv, anchor, B, ids, ws, logits)
        torch.cuda.synchronize()
        assert torch.equal(ids, ids0), f"{name}: eager run after replay {rep} differs"
