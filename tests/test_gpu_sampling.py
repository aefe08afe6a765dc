"""Sampling drafter and lossless rejection-sampling verification on the GPU against the
oracle (same counter-based draws on both sides).  A draw decided by floating point is
compared where the oracle's decision is not a near-tie: its top-2 sampling-key gap for a
sampled id, its |u - ratio| margin for an acceptance; elsewhere the kernel's decision must
follow the rule applied to its own logits."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from block_diffusion_drafter_03_amd import runtime as rt

from harness import DEV, NEAR_TIE, TOL, Setup, assert_rows_close, inject_all

pytestmark = pytest.mark.gpu

SEED = 0x5EED5EED1234
MARGIN = 2e-3      # |u - ratio| / max(ratio, 1) below which an acceptance is a near-tie


def _key_gap(keys):
    return float(O.top2_gap(np.asarray(keys, dtype=np.float64)))


@pytest.mark.parametrize("name,T", [("tiny_f32", 1.0), ("mid_bf16", 1.0), ("mid_bf16", 0.7)])
def test_sampled_draft_matches_oracle(name, T):
    w = synth.workload(name)
    S = Setup(w)
    lens = synth.ctx_lengths(w)
    B, tol, m = w.block, TOL[w.dtype], w.draft
    kv = S.kv(m, max(lens) + B + 70)
    ws = S.workspace(S.draft, B, kv.capacity, inject_rows=sum(lens))
    feats = [synth.features(w, n, DEV, tag=f"feats.b{b}") for b, n in enumerate(lens)]
    inject_all(S, kv, feats, ws)
    anchor = synth.anchors(w, DEV)
    ids = torch.zeros(w.batch, B - 1, dtype=torch.int32, device=DEV)
    zd = torch.zeros(w.batch, B - 1, m.vocab, device=DEV)
    counter = 17
    rt.draft_block_sampled(S.draft, kv, anchor, B, T, SEED, counter, ids, zd, ws)
    torch.cuda.synchronize()
    assert kv.err.item() == 0
    checked = 0
    for b, n in enumerate(lens):
        ctx = O.inject(synth.to_numpy(feats[b]), np.arange(n), S.np_dw, m, store=S.store)
        o_ids, o_z, o_keys = O.draft_block_sampled(S.np_dw, S.np_shared, m, ctx, int(anchor[b]), n, B,
                                                   T, SEED, counter, b, store=S.store)
        assert_rows_close(zd[b].cpu().numpy(), o_z, tol, f"{name} draft logits seq {b}")
        got = ids[b].cpu().numpy()
        for i in range(B - 1):
            if _key_gap(o_keys[i]) >= NEAR_TIE / T:
                assert got[i] == o_ids[i], f"{name} T={T} seq {b} position {i + 1}"
                checked += 1
    assert checked >= (B - 1) * w.batch // 2
    # a different counter draws different ids (the noise is not constant)
    ids2 = torch.zeros_like(ids)
    rt.draft_block_sampled(S.draft, kv, anchor, B, T, SEED, counter + 1, ids2, zd, ws)
    torch.cuda.synchronize()
    assert not torch.equal(ids, ids2)


def _target_cache(S, lens, B):
    w = S.w
    kv = S.kv(w.target, max(lens) + B + 70, seed=1)
    dense = synth.synthetic_ctx_kv(w, "target", lens, DEV)
    for l in range(w.target.n_layers):
        for b, n in enumerate(lens):
            kv.write_dense(l, b, dense[l][b][0], dense[l][b][1])
    kv.set_seq_len(lens)
    np_cache = [[(synth.to_numpy(dense[l][b][0]), synth.to_numpy(dense[l][b][1]))
                 for l in range(w.target.n_layers)] for b in range(len(lens))]
    return kv, np_cache


def _rule_on(drafts, zd, zt, T, seed, counter, b):
    """The acceptance rule applied (float64) to given logits: (a, ratios, uniforms)."""
    a, _, _, r, u, _ = O.accept_sampled(drafts, zd, zt, T, seed, counter, b)
    return a, r, u


@pytest.mark.parametrize("name,T", [("tiny_f32", 1.0), ("mid_bf16", 1.0), ("mid_bf16", 0.6)])
def test_sampled_verify_matches_oracle(name, T):
    """Both sides verify the same drafts against the same drafter distribution (the oracle's
    drafter logits, handed to the kernel as the proposal)."""
    w = synth.workload(name)
    S = Setup(w, target=True)
    lens = synth.ctx_lengths(w)
    B, tol, tm = w.block, TOL[w.dtype], w.target
    kv, np_cache = _target_cache(S, lens, B)
    rng = np.random.default_rng(7)
    anchors = synth.anchors(w, "cpu").numpy()
    # proposal: logits of a random "drafter" over the shared vocabulary, and drafts drawn
    # from it with the oracle's generator (purpose 0), so acceptances are a real mix
    zd_np = rng.normal(0, 1.5, (w.batch, B - 1, tm.vocab)).astype(np.float32)
    counter = 5
    drafts = np.stack([[int(O.argmax_lowest(O.sample_keys(zd_np[b, i - 1], T, SEED, counter, 0, b, i)))
                        for i in range(1, B)] for b in range(w.batch)])
    # half the sequences get the target's greedy continuation as their drafts instead
    for b in range(0, w.batch, 2):
        toks = [int(anchors[b])]
        for _ in range(B - 1):
            g, _, _, _, _ = O.verify(S.np_tw, S.np_shared, tm, np_cache[b], toks, lens[b], w.taps,
                                     store=S.store)
            toks.append(int(g[-1]))
        drafts[b] = toks[1:]
    k = len(w.taps)
    anchor_t = torch.tensor(anchors, dtype=torch.int32, device=DEV)
    drafts_t = torch.tensor(drafts, dtype=torch.int32, device=DEV)
    zd_t = torch.tensor(zd_np, device=DEV)
    fo = torch.zeros(w.batch, B, k * tm.hidden, dtype=S.st, device=DEV)
    zt = torch.zeros(w.batch, B, tm.vocab, device=DEV)
    tau = torch.zeros(w.batch, dtype=torch.int32, device=DEV)
    nxt = torch.zeros(w.batch, dtype=torch.int32, device=DEV)
    ws = S.workspace(S.target, B, kv.capacity)
    oz = []
    for b, n in enumerate(lens):
        block = [int(anchors[b])] + [int(x) for x in drafts[b]]
        oz.append(O.verify(S.np_tw, S.np_shared, tm, np_cache[b], block, n, w.taps, store=S.store)[1])
    compared, taus = 0, []
    for counter in range(6):          # several draws over the same logits
        rt.verify_sampled(S.target, kv, anchor_t, drafts_t, zd_t, B, T, SEED, counter, fo, zt, tau,
                          nxt, ws)
        torch.cuda.synchronize()
        assert kv.err.item() == 0
        for b, n in enumerate(lens):
            zt_b = zt[b].cpu().numpy()
            assert_rows_close(zt_b, oz[b], tol, f"{name} verify logits seq {b}")
            a, tau_o, tok, r, u, keys = O.accept_sampled(drafts[b], zd_np[b], oz[b], T, SEED, counter, b)
            margins = np.abs(u - r) / np.maximum(r, 1.0)
            decided = margins[: min(a + 1, B - 1)]     # the decisions that fix a
            t_g, n_g = int(tau[b]), int(nxt[b])
            taus.append(t_g)
            if np.all(decided >= MARGIN):
                assert t_g == tau_o, f"{name} T={T} seq {b} counter {counter}: tau {t_g} != {tau_o}"
                if _key_gap(keys) >= NEAR_TIE / T:
                    assert n_g == tok, f"{name} T={T} seq {b} counter {counter}: token {n_g} != {tok}"
                    compared += 1
            else:
                # a near-tie acceptance: the kernel's tau must be the rule on its own logits
                a_g, _, _ = _rule_on(drafts[b], zd_np[b], zt_b, T, SEED, counter, b)
                assert t_g == a_g + 1, f"{name} seq {b}: not the rule on its own logits"
            assert 1 <= t_g <= B
    assert compared >= 3 * w.batch
    # both branches of the rule were taken: a rejection somewhere, an acceptance somewhere
    assert min(taus) < B and max(taus) > 1


def test_sampled_cycles_keep_the_caches_in_step():
    """Sampling cycles (draft, verify, inject, commit) run end to end: every tau in range,
    no device error, both caches advance together, and the greedy-continuation drafts of a
    near-deterministic target (tiny temperature) are all accepted."""
    w = synth.workload("mid_bf16")
    S = Setup(w, target=True)
    T, D = w.target, w.draft
    B, n0 = w.block, 40
    prompts = [synth.prompt_tokens(w, n0, "cpu", tag=f"prompt{b}").numpy() for b in range(w.batch)]
    cap = n0 + 6 * B + 64
    tkv = S.kv(T, cap, seed=2)
    dkv = S.kv(D, cap, seed=3)
    k = len(w.taps)
    ws_t = S.workspace(S.target, max(B, n0), tkv.capacity)
    ws_d = S.workspace(S.draft, B, dkv.capacity, inject_rows=w.batch * max(B, n0))
    batch = w.batch
    # prefill with the greedy path (block of n0)
    ids = torch.tensor(np.stack(prompts), dtype=torch.int32, device=DEV)
    feats = torch.zeros(batch, n0, k * T.hidden, dtype=S.st, device=DEV)
    g = torch.zeros(batch, n0, dtype=torch.int32, device=DEV)
    tau = torch.zeros(batch, dtype=torch.int32, device=DEV)
    bonus = torch.zeros(batch, dtype=torch.int32, device=DEV)
    rt.verify_accept(S.target, tkv, ids[:, 0].contiguous(), ids[:, 1:].contiguous(), n0, feats, g, tau,
                     bonus, ws_t)
    rs = torch.arange(batch, dtype=torch.int32, device=DEV).repeat_interleave(n0)
    rp = torch.arange(n0, dtype=torch.int32, device=DEV).repeat(batch)
    rt.inject_ctx(S.draft, dkv, feats.reshape(batch * n0, -1).contiguous(), rs, rp, 1, n0, ws_d)
    rt.kv_commit(tkv, dkv, torch.full((batch,), n0, dtype=torch.int32, device=DEV), n0)
    anchor = g[:, -1].contiguous()
    drafts = torch.zeros(batch, B - 1, dtype=torch.int32, device=DEV)
    zd = torch.zeros(batch, B - 1, D.vocab, device=DEV)
    zt = torch.zeros(batch, B, T.vocab, device=DEV)
    fo = torch.zeros(batch, B, k * T.hidden, dtype=S.st, device=DEV)
    nxt = torch.zeros(batch, dtype=torch.int32, device=DEV)
    rs = torch.arange(batch, dtype=torch.int32, device=DEV).repeat_interleave(B)
    rp = torch.arange(B, dtype=torch.int32, device=DEV).repeat(batch)
    for c in range(4):
        rt.draft_block_sampled(S.draft, dkv, anchor, B, 1.0, SEED, c, drafts, zd, ws_d)
        rt.verify_sampled(S.target, tkv, anchor, drafts, zd, B, 1.0, SEED, c, fo, zt, tau, nxt, ws_t)
        rt.inject_ctx(S.draft, dkv, fo.reshape(batch * B, -1).contiguous(), rs, rp, 1, B, ws_d)
        rt.kv_commit(tkv, dkv, tau, B)
        tkv.refresh_len_bound()
        dkv.refresh_len_bound()
        t = tau.cpu().numpy()
        assert ((1 <= t) & (t <= B)).all()
        anchor = nxt.clone()
    torch.cuda.synchronize()
    assert tkv.err.item() == 0 and dkv.err.item() == 0
    assert torch.equal(tkv.seq_len, dkv.seq_len)
