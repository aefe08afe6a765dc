"""Checkpoint / resume of the speculative loop: the committed state of both caches (K/V rows
of positions below seq_len, and seq_len) and the next anchors, written to a safetensors file
mid-run and restored into fresh caches whose pages are handed out in another order, continue
the token stream exactly as the uninterrupted run does (the lossless guarantee of DFlash
§4.5, "The Decoding Loop": the output is the target's greedy stream whatever happens between
cycles).  The restored caches hold zeros where the originals hold rejected draft rows past
seq_len, so the run also shows that no kernel reads a cache row at or past seq_len."""
import os

import numpy as np
import pytest
import torch
from safetensors.torch import load_file, save_file

import synth
from block_diffusion_drafter_03_amd import runtime as rt

from harness import DEV, Setup

pytestmark = pytest.mark.gpu


class Loop:
    """Prefill + draft / verify / inject / commit cycles of one workload at batch w.batch."""

    def __init__(self, S, n0, cap, seeds):
        w = S.w
        self.S, self.B, self.batch, self.k = S, w.block, w.batch, len(w.taps)
        self.tkv = S.kv(w.target, cap, seed=seeds[0])
        self.dkv = S.kv(w.draft, cap, seed=seeds[1])
        self.ws_t = S.workspace(S.target, max(self.B, n0), self.tkv.capacity)
        self.ws_d = S.workspace(S.draft, self.B, self.dkv.capacity, inject_rows=w.batch * max(self.B, n0))

    def verify(self, anchor, drafts, blk):
        S = self.S
        feats = torch.zeros(self.batch, blk, self.k * S.w.target.hidden, dtype=S.st, device=DEV)
        g = torch.zeros(self.batch, blk, dtype=torch.int32, device=DEV)
        tau = torch.zeros(self.batch, dtype=torch.int32, device=DEV)
        bonus = torch.zeros(self.batch, dtype=torch.int32, device=DEV)
        rt.verify_accept(S.target, self.tkv, anchor, drafts, blk, feats, g, tau, bonus, self.ws_t)
        return feats, g, tau, bonus

    def inject_rel(self, feats, blk):
        rs = torch.arange(self.batch, dtype=torch.int32, device=DEV).repeat_interleave(blk)
        rp = torch.arange(blk, dtype=torch.int32, device=DEV).repeat(self.batch)
        rt.inject_ctx(self.S.draft, self.dkv, feats.reshape(self.batch * blk, -1).contiguous(), rs, rp, 1,
                      blk, self.ws_d)

    def prefill(self, prompts):
        n0 = prompts.shape[1]
        ids = torch.tensor(prompts, dtype=torch.int32, device=DEV)
        feats, g, _, _ = self.verify(ids[:, 0].contiguous(), ids[:, 1:].contiguous(), n0)
        self.inject_rel(feats, n0)
        rt.kv_commit(self.tkv, self.dkv, torch.full((self.batch,), n0, dtype=torch.int32, device=DEV), n0)
        anchor = g[:, -1].contiguous()
        return anchor, [[int(a)] for a in anchor.cpu()]

    def cycles(self, anchor, emitted, n):
        drafts = torch.zeros(self.batch, self.B - 1, dtype=torch.int32, device=DEV)
        for _ in range(n):
            rt.draft_block(self.S.draft, self.dkv, anchor, self.B, drafts, self.ws_d)
            feats, g, tau, bonus = self.verify(anchor, drafts, self.B)
            self.inject_rel(feats, self.B)
            rt.kv_commit(self.tkv, self.dkv, tau, self.B)
            self.tkv.refresh_len_bound()
            self.dkv.refresh_len_bound()
            t, bo, d = tau.cpu().numpy(), bonus.cpu().numpy(), drafts.cpu().numpy()
            for b in range(self.batch):
                emitted[b] += [int(x) for x in d[b, : t[b] - 1]] + [int(bo[b])]
            anchor = bonus.clone()
        torch.cuda.synchronize()
        assert self.tkv.err.item() == 0 and self.dkv.err.item() == 0
        return anchor, emitted


@pytest.mark.parametrize("name", ["tiny_f32", "mid_bf16"])
def test_resume_from_checkpoint_continues_the_stream(name, tmp_path):
    w = synth.workload(name)
    S = Setup(w, target=True)
    n0, C = 40, 3
    prompts = np.stack([synth.prompt_tokens(w, n0, "cpu", tag=f"prompt{b}").numpy() for b in range(w.batch)])
    cap = n0 + 2 * C * w.block + 64

    # uninterrupted: prefill + 2C cycles
    run = Loop(S, n0, cap, seeds=(2, 3))
    anchor, emitted = run.prefill(prompts)
    anchor, ref = run.cycles(anchor, emitted, 2 * C)
    ref_state = (run.tkv.snapshot(), run.dkv.snapshot())
    ref_pages = run.tkv.block_table.cpu()
    del run
    torch.cuda.synchronize()

    # interrupted after C cycles: checkpoint to a file, drop every device object
    run = Loop(S, n0, cap, seeds=(2, 3))
    anchor, emitted = run.prefill(prompts)
    anchor, emitted = run.cycles(anchor, emitted, C)
    ck = {**{f"target.{k}": v for k, v in run.tkv.snapshot().items()},
          **{f"draft.{k}": v for k, v in run.dkv.snapshot().items()},
          "anchor": anchor.cpu()}
    path = os.path.join(tmp_path, "loop.safetensors")
    save_file(ck, path)
    del run, anchor, ck
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    # resume into caches with other page orders (and a larger capacity)
    ck = load_file(path)
    run = Loop(S, n0, cap + 64, seeds=(11, 12))
    run.tkv.restore({k[len("target."):]: v for k, v in ck.items() if k.startswith("target.")})
    run.dkv.restore({k[len("draft."):]: v for k, v in ck.items() if k.startswith("draft.")})
    assert not torch.equal(run.tkv.block_table.cpu()[:, :2], ref_pages[:, :2])
    anchor = ck["anchor"].to(DEV)
    anchor, got = run.cycles(anchor, emitted, C)

    assert got == ref, f"{name}: resumed stream differs"
    for model, snap_ref, kv in (("target", ref_state[0], run.tkv), ("draft", ref_state[1], run.dkv)):
        snap = kv.snapshot()
        assert torch.equal(snap["seq_len"], snap_ref["seq_len"]), f"{name} {model}: seq_len"
        for k, v in snap_ref.items():
            assert torch.equal(snap[k], v), f"{name} {model}: {k}"
