"""DFlash 2 two-tap dynamic convolution in the drafter on the GPU ([DF] section 7.1, Problem
2) against the oracle: every layer's output, the logits and the draft ids of a drafter with
convolutions, on the same seeded weights and context."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
import synth
from block_diffusion_drafter_03_amd import runtime as rt

from harness import DEV, NEAR_TIE, TOL, Setup, assert_close, assert_ids, assert_rows_close, inject_all

pytestmark = pytest.mark.gpu


def _draft(S, w):
    lens = synth.ctx_lengths(w)
    B, m = w.block, w.draft
    kv = S.kv(m, max(lens) + B + 70)
    ws = S.workspace(S.draft, B, kv.capacity, inject_rows=sum(lens))
    feats = [synth.features(w, n, DEV, tag=f"feats.b{b}") for b, n in enumerate(lens)]
    inject_all(S, kv, feats, ws)
    anchor = synth.anchors(w, DEV)
    ids = torch.zeros(w.batch, B - 1, dtype=torch.int32, device=DEV)
    logits = torch.zeros(w.batch, B - 1, m.vocab, device=DEV)
    hid = torch.zeros(m.n_layers + 1, w.batch, B, m.hidden, device=DEV)
    rt.draft_block(S.draft, kv, anchor, B, ids, ws, logits, hid)
    torch.cuda.synchronize()
    assert kv.err.item() == 0
    return lens, feats, anchor, ids, logits, hid


@pytest.mark.parametrize("name", ["tiny_f32", "mid_bf16"])
def test_convolved_drafter_matches_oracle(name):
    _check_against_oracle(synth.workload(name), name)


def test_convolution_fused_into_its_correction_gemv_matches_oracle():
    """One bf16 sequence of B = 16 rows (M = 16): every convolution runs as the epilogue of
    its correction GEMV instead of a separate launch (the batch-3 case above, M = 48, keeps
    the separate convolution kernel)."""
    w = dataclasses.replace(synth.workload("mid_bf16"), batch=1, ctx=(333,))
    assert w.batch * w.block <= 16
    _check_against_oracle(w, "mid_bf16 batch 1")


def test_convolution_fused_into_a_wider_correction_gemv_matches_oracle():
    """One sequence of a model with hidden 2560 (M = 16): 20 correction tiles of 128
    channels each, K = 2560 over 16 waves (5 steps a wave), every convolution the epilogue
    of its correction GEMV; the full-size 4K drafter with convolutions is checked in
    test_gpu_parity_full.py."""
    w = synth.workload("split_bf16")
    assert w.batch * w.block <= 16
    _check_against_oracle(w, "split_bf16 batch 1")


def _check_against_oracle(w, name):
    S = Setup(w, dconv=synth.dconv_weights(w, DEV))
    B, m, tol = w.block, w.draft, TOL[w.dtype]
    lens, feats, anchor, ids, logits, hid = _draft(S, w)
    checked = 0
    for b, n in enumerate(lens):
        ctx = O.inject(synth.to_numpy(feats[b]), np.arange(n), S.np_dw, m, store=S.store)
        o_ids, o_z, o_hid = O.draft_block(S.np_dw, S.np_shared, m, ctx, int(anchor[b]), n, B, store=S.store)
        for l in range(m.n_layers + 1):
            assert_close(hid[l, b].cpu().numpy(), o_hid[l], tol, f"{name} seq {b} hidden layer {l}")
        assert_rows_close(logits[b].cpu().numpy(), o_z, tol, f"{name} seq {b} logits")
        checked += assert_ids(ids[b].cpu().numpy(), o_ids, o_z, f"{name} seq {b} ids")
    assert checked >= (B - 1) * w.batch // 2


@pytest.mark.parametrize("name", ["tiny_f32", "mid_bf16"])
def test_identity_convolutions_give_the_plain_drafter(name):
    w = synth.workload(name)
    D = w.draft.hidden
    st = torch.float32 if w.dtype == "f32" else torch.bfloat16
    ident = {}
    for i in range(w.draft.n_layers):
        for nm in synth.DCONV_NAMES:
            ident[f"L{i}.dconv_{nm}.base"] = torch.stack([torch.ones(D), torch.zeros(D)]).to(st).to(DEV)
            ident[f"L{i}.dconv_{nm}.w_k"] = torch.zeros(D, D // 8, dtype=st, device=DEV)
    S1 = Setup(w, dconv=ident)
    *_, ids1, z1, h1 = _draft(S1, w)
    S0 = Setup(w)
    *_, ids0, z0, h0 = _draft(S0, w)
    # the convolution path materialises the normalised input instead of folding the norm
    # into the GEMM, so the two agree to rounding, not bit for bit
    tol = TOL[w.dtype]
    for b in range(w.batch):
        assert_rows_close(z1[b].cpu().numpy(), z0[b].cpu().numpy(), tol, f"{name} seq {b} logits")
        gaps = O.top2_gap(z0[b].cpu().numpy().astype(np.float64))
        sel = gaps >= NEAR_TIE
        assert np.array_equal(ids1[b].cpu().numpy()[sel], ids0[b].cpu().numpy()[sel])
    # and real convolution weights change the drafter
    S2 = Setup(w, dconv=synth.dconv_weights(w, DEV))
    *_, z2, _ = _draft(S2, w)
    assert float((z2 - z0).abs().max()) > 10 * tol * float(z0.abs().max())
