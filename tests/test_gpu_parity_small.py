"""GPU vs oracle parity at sizes the oracle finishes in seconds: the tiny fp32 drafter, a
small bf16 GQA model whose shapes span several tiles and leave ragged tails (vocab 3000,
contexts 200 / 333 / 64, pages handed out in shuffled order), the same model at batch 24
(384 block rows, contexts in [1, 300]), a wide-vocabulary bf16 model (80 block rows x
40000 LM-head columns; contexts 130 / 0 / 257 / 1 / 64), a narrow one (hidden 256, 192 block
rows), a narrow one with a vocabulary of 120001 at batch 17 (272 x 120001 LM head) and a
batch-1 model (hidden 2560, FFN 8192) whose M = 16 GEMVs split K over workgroups."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from block_diffusion_drafter_03_amd import runtime as rt

from harness import (DEV, TOL, Setup, assert_accept, assert_close, assert_ids, assert_rows_close,
                     inject_all, read_cache)

pytestmark = pytest.mark.gpu

WORKLOADS = ["tiny_f32", "mid_bf16"]
# plus a wide-vocabulary model with empty and one-row contexts, the mid model at batch 24
# (384 block rows), a narrow model at batch 12 (192 rows, the LDS-staged GEMM) and the narrow
# model over 120001 vocabulary rows at batch 17 (the widest weight-direct LM-head tile) and
# at batch 5 (the four-wave row-resident LM head), and a batch-1 model whose QKV and down
# GEMVs take the K-split form on ragged shapes, for the draft / verify checks
WITH_WIDE = WORKLOADS + ["wide_bf16", "many_bf16", "narrow_bf16", "vast_bf16", "vast5_bf16", "split_bf16"]


def _feats(w, lens):
    return [synth.features(w, n, DEV, tag=f"feats.b{b}") for b, n in enumerate(lens)]


@pytest.mark.parametrize("name", WITH_WIDE)
def test_inject_and_draft_block(name):
    w = synth.workload(name)
    S = Setup(w)
    lens = synth.ctx_lengths(w)
    B, tol = w.block, TOL[w.dtype]
    kv = S.kv(w.draft, max(lens) + B + 70)
    ws = S.workspace(S.draft, B, kv.capacity, inject_rows=sum(lens))
    feats = _feats(w, lens)
    inject_all(S, kv, feats, ws)
    anchor = synth.anchors(w, DEV)
    m = w.draft
    ids = torch.zeros(w.batch, B - 1, dtype=torch.int32, device=DEV)
    logits = torch.zeros(w.batch, B - 1, m.vocab, device=DEV)
    hid = torch.zeros(m.n_layers + 1, w.batch, B, m.hidden, device=DEV)
    rt.draft_block(S.draft, kv, anchor, B, ids, ws, logits, hid)
    # without the logits and hidden-state copies (a decoding loop's call): the same ids
    ids2 = torch.zeros_like(ids)
    rt.draft_block(S.draft, kv, anchor, B, ids2, ws)
    torch.cuda.synchronize()
    assert kv.err.item() == 0
    assert torch.equal(ids2, ids), f"{name}: ids depend on the logits copy"
    a_np = anchor.cpu().numpy()
    for b, n in enumerate(lens):
        ctx = O.inject(synth.to_numpy(feats[b]), np.arange(n), S.np_dw, m, store=S.store)
        for l in range(m.n_layers):
            K, V = read_cache(kv, l, b, n)
            assert_close(K, ctx[l][0], tol, f"{name} ctx K layer {l} seq {b}")
            assert_close(V, ctx[l][1], tol, f"{name} ctx V layer {l} seq {b}")
        o_ids, o_z, o_hid = O.draft_block(S.np_dw, S.np_shared, m, ctx, int(a_np[b]), n, B, store=S.store)
        for l in range(m.n_layers + 1):
            assert_close(hid[l, b].cpu().numpy(), o_hid[l], tol, f"{name} hidden layer {l} seq {b}")
        assert_rows_close(logits[b].cpu().numpy(), o_z, tol, f"{name} logits seq {b}")
        assert_ids(ids[b].cpu().numpy(), o_ids, o_z, f"{name} draft ids seq {b}")


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


def _forced_block(S, np_cache, n, anchor, B, f, rng):
    """[anchor, g*_0 .. g*_{f-1}, random...]: the first f drafts equal the target's greedy
    continuation (computed by the oracle), so the target accepts exactly f of them unless
    a later random id happens to match."""
    w = S.w
    toks = [int(anchor)]
    for _ in range(f):
        g, _, _, _, _ = O.verify(S.np_tw, S.np_shared, w.target, np_cache, toks, n, w.taps, store=S.store)
        toks.append(int(g[-1]))
    while len(toks) < B:
        toks.append(int(rng.integers(0, w.target.vocab)))
    return toks


@pytest.mark.parametrize("name", WITH_WIDE)
def test_verify_accept(name):
    w = synth.workload(name)
    S = Setup(w, target=True)
    lens = synth.ctx_lengths(w)
    B, tol, m = w.block, TOL[w.dtype], w.target
    kv, np_cache = _target_cache(S, lens, B)
    rng = np.random.default_rng(5)
    anchors = synth.anchors(w, "cpu").numpy()
    blocks = []
    for b, n in enumerate(lens):
        f = [B - 1, 0, B // 2][b % 3]
        blocks.append(_forced_block(S, np_cache[b], n, anchors[b], B, f, rng))
    block_ids = torch.tensor(blocks, dtype=torch.int32, device=DEV)
    k = len(w.taps)
    feats = torch.zeros(w.batch, B, k * m.hidden, dtype=S.st, device=DEV)
    g = torch.zeros(w.batch, B, dtype=torch.int32, device=DEV)
    tau = torch.zeros(w.batch, dtype=torch.int32, device=DEV)
    bonus = torch.zeros(w.batch, dtype=torch.int32, device=DEV)
    logits = torch.zeros(w.batch, B, m.vocab, device=DEV)
    hid = torch.zeros(m.n_layers + 1, w.batch, B, m.hidden, device=DEV)
    ws = S.workspace(S.target, B, kv.capacity)
    rt.verify_accept(S.target, kv, block_ids[:, 0].contiguous(), block_ids[:, 1:].contiguous(), B,
                     feats, g, tau, bonus, ws, logits, hid)
    # the same verification without the logits and hidden-state copies (a decoding loop's
    # call): it rewrites the same block rows and must give the same decisions, bit for bit
    g2, tau2, bonus2 = torch.zeros_like(g), torch.zeros_like(tau), torch.zeros_like(bonus)
    feats2 = torch.zeros_like(feats)
    rt.verify_accept(S.target, kv, block_ids[:, 0].contiguous(), block_ids[:, 1:].contiguous(), B,
                     feats2, g2, tau2, bonus2, ws)
    torch.cuda.synchronize()
    assert kv.err.item() == 0
    assert torch.equal(feats2, feats)
    for x, y, what in ((g2, g, "argmax"), (tau2, tau, "tau"), (bonus2, bonus, "bonus")):
        assert torch.equal(x, y), f"{name}: {what} depends on the logits copy"
    for b, n in enumerate(lens):
        og, oz, of, onew, ohid = O.verify(S.np_tw, S.np_shared, m, np_cache[b], blocks[b], n, w.taps,
                                          store=S.store)
        for l in range(m.n_layers + 1):
            assert_close(hid[l, b].cpu().numpy(), ohid[l], tol, f"{name} verify hidden {l} seq {b}")
        assert_rows_close(logits[b].cpu().numpy(), oz, tol, f"{name} verify logits seq {b}")
        assert_close(synth.to_numpy(feats[b]), of, tol, f"{name} tapped feats seq {b}")
        assert_ids(g[b].cpu().numpy(), og, oz, f"{name} target argmax seq {b}")
        assert_accept(tau[b], bonus[b], g[b].cpu().numpy(), blocks[b][1:], og, oz, f"{name} accept seq {b}")
        assert 1 <= int(tau[b]) <= B

        # the block's K/V were written at n .. n+B-1
        for l in range(m.n_layers):
            K, V = read_cache(kv, l, b, n + B)
            assert_close(K[n:], onew[l][0], tol, f"{name} new K layer {l} seq {b}")
            assert_close(V[n:], onew[l][1], tol, f"{name} new V layer {l} seq {b}")
            Kc, Vc = np_cache[b][l]
            np.testing.assert_array_equal(K[:n], Kc)   # the old rows are untouched
    # forced prefixes: full acceptance for sequence 0 (f = B-1), when no near-tie decides
    og, oz, _, _, _ = O.verify(S.np_tw, S.np_shared, m, np_cache[0], blocks[0], lens[0], w.taps,
                               store=S.store)
    if np.all(O.top2_gap(oz) >= 1e-2):
        assert int(tau[0]) == B


@pytest.mark.parametrize("B", [16, 8])
def test_verify_accept_batch1_forced_prefixes(B):
    """Batch 1 of a bf16 model (the M <= 16 LM head whose last workgroup runs the greedy
    acceptance): blocks whose first f drafts are the target's greedy continuation, for f = 0,
    a middle run and B - 1, verified at the same position, against the oracle's argmax, tau
    and bonus."""
    w = synth.workload("split_bf16")
    S = Setup(w, target=True)
    lens = synth.ctx_lengths(w)
    m = w.target
    kv, np_cache = _target_cache(S, lens, B)
    rng = np.random.default_rng(11)
    anchor = int(synth.anchors(w, "cpu").numpy()[0])
    ws = S.workspace(S.target, B, kv.capacity)
    k = len(w.taps)
    for f in sorted({0, min(5, B - 1), B - 1}):
        block = _forced_block(S, np_cache[0], lens[0], anchor, B, f, rng)
        ids = torch.tensor([block], dtype=torch.int32, device=DEV)
        feats = torch.zeros(1, B, k * m.hidden, dtype=S.st, device=DEV)
        g = torch.zeros(1, B, dtype=torch.int32, device=DEV)
        tau = torch.zeros(1, dtype=torch.int32, device=DEV)
        bonus = torch.zeros(1, dtype=torch.int32, device=DEV)
        rt.verify_accept(S.target, kv, ids[:, 0].contiguous(), ids[:, 1:].contiguous(), B, feats, g, tau,
                         bonus, ws)
        torch.cuda.synchronize()
        assert kv.err.item() == 0
        og, oz, _, _, _ = O.verify(S.np_tw, S.np_shared, m, np_cache[0], block, lens[0], w.taps,
                                   store=S.store)
        assert_ids(g[0].cpu().numpy(), og, oz, f"B {B} f {f} target argmax")
        assert_accept(tau[0], bonus[0], g[0].cpu().numpy(), block[1:], og, oz, f"B {B} f {f} accept")
        if np.all(O.top2_gap(oz) >= 1e-2):
            assert int(tau[0]) >= f + 1, f"B {B} f {f}: tau {int(tau[0])}"


@pytest.mark.parametrize("name", WORKLOADS)
def test_block_of_one_is_single_token_decode(name):
    """B = 1: the drafter's one row attends to the context and itself; verify of one token
    is a plain decode step.  Both match the oracle."""
    w = synth.workload(name)
    S = Setup(w, target=True)
    lens = synth.ctx_lengths(w)
    tol = TOL[w.dtype]
    kv, np_cache = _target_cache(S, lens, 1)
    tok = torch.tensor([[7 + b] for b in range(w.batch)], dtype=torch.int32, device=DEV)
    m = w.target
    g = torch.zeros(w.batch, 1, dtype=torch.int32, device=DEV)
    tau = torch.zeros(w.batch, dtype=torch.int32, device=DEV)
    bonus = torch.zeros(w.batch, dtype=torch.int32, device=DEV)
    hid = torch.zeros(m.n_layers + 1, w.batch, 1, m.hidden, device=DEV)
    logits = torch.zeros(w.batch, 1, m.vocab, device=DEV)
    ws = S.workspace(S.target, 1, kv.capacity)
    rt.verify_accept(S.target, kv, tok[:, 0].contiguous(), None, 1, None, g, tau, bonus, ws, logits, hid)
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        og, oz, _, _, ohid = O.verify(S.np_tw, S.np_shared, m, np_cache[b], [7 + b], n, (), store=S.store)
        assert_close(hid[-1, b].cpu().numpy(), ohid[-1], tol, f"{name} B=1 verify seq {b}")
        assert int(tau[b]) == 1 and int(bonus[b]) == int(g[b, 0])
    # drafter with B = 1
    dkv = S.kv(w.draft, max(lens) + 70)
    dws = S.workspace(S.draft, 1, dkv.capacity, inject_rows=sum(lens))
    feats = _feats(w, lens)
    inject_all(S, dkv, feats, dws)
    anchor = synth.anchors(w, DEV)
    dh = torch.zeros(w.draft.n_layers + 1, w.batch, 1, w.draft.hidden, device=DEV)
    ids = torch.zeros(w.batch, 1, dtype=torch.int32, device=DEV)
    rt.draft_block(S.draft, dkv, anchor, 1, ids, dws, None, dh)
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        ctx = O.inject(synth.to_numpy(feats[b]), np.arange(n), S.np_dw, w.draft, store=S.store)
        _, _, ohid = O.draft_block(S.np_dw, S.np_shared, w.draft, ctx, int(anchor[b]), n, 1, store=S.store)
        assert_close(dh[-1, b].cpu().numpy(), ohid[-1], tol, f"{name} B=1 draft seq {b}")


@pytest.mark.parametrize("name", WORKLOADS)
def test_inject_chunking_is_bit_identical(name):
    w = synth.workload(name)
    S = Setup(w)
    lens = synth.ctx_lengths(w)
    feats = _feats(w, lens)
    caches = []
    for chunk in (None, 7, 64):
        kv = S.kv(w.draft, max(lens) + 70)
        ws = S.workspace(S.draft, w.block, kv.capacity, inject_rows=sum(lens))
        inject_all(S, kv, feats, ws, chunk=chunk)
        torch.cuda.synchronize()
        caches.append([read_cache(kv, l, b, n) for l in range(w.draft.n_layers)
                       for b, n in enumerate(lens)])
    # the per-row arithmetic is independent of the chunk, up to the GEMM path chosen for
    # the chunk's row count (skinny vs tiled): compare within tolerance, and exactly for
    # chunkings that use the same path
    for c in caches[1:]:
        for (K0, V0), (K1, V1) in zip(caches[0], c):
            assert_close(K1, K0, TOL[w.dtype], f"{name} chunked K")
            assert_close(V1, V0, TOL[w.dtype], f"{name} chunked V")


@pytest.mark.parametrize("name", WORKLOADS)
def test_draft_is_deterministic(name):
    w = synth.workload(name)
    S = Setup(w)
    lens = synth.ctx_lengths(w)
    kv = S.kv(w.draft, max(lens) + w.block + 70)
    ws = S.workspace(S.draft, w.block, kv.capacity, inject_rows=sum(lens))
    inject_all(S, kv, _feats(w, lens), ws)
    anchor = synth.anchors(w, DEV)
    outs = []
    for _ in range(2):
        ids = torch.zeros(w.batch, w.block - 1, dtype=torch.int32, device=DEV)
        logits = torch.zeros(w.batch, w.block - 1, w.draft.vocab, device=DEV)
        rt.draft_block(S.draft, kv, anchor, w.block, ids, ws, logits)
        outs.append((ids.clone(), logits.clone()))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("name", WORKLOADS)
def test_speculative_cycles_reproduce_greedy_decoding(name):
    """GPU cycles (draft, verify, inject, commit) emit the target's greedy stream computed
    by the oracle, up to the first position whose oracle top-2 gap is a near-tie."""
    w = synth.workload(name)
    S = Setup(w, target=True)
    B, T, D = w.block, w.target, w.draft
    n0, n_new = 40, 3 * B
    prompts = [synth.prompt_tokens(w, n0, "cpu", tag=f"prompt{b}").numpy() for b in range(w.batch)]
    cap = n0 + n_new + 2 * B + 64
    tkv = S.kv(T, cap, seed=2)
    dkv = S.kv(D, cap, seed=3)
    k = len(w.taps)
    ws_t = S.workspace(S.target, max(B, n0), tkv.capacity)
    ws_d = S.workspace(S.draft, B, dkv.capacity, inject_rows=w.batch * max(B, n0))
    batch = w.batch

    def verify(anchor, drafts, blk):
        feats = torch.zeros(batch, blk, k * T.hidden, dtype=S.st, device=DEV)
        g = torch.zeros(batch, blk, dtype=torch.int32, device=DEV)
        tau = torch.zeros(batch, dtype=torch.int32, device=DEV)
        bonus = torch.zeros(batch, dtype=torch.int32, device=DEV)
        rt.verify_accept(S.target, tkv, anchor, drafts, blk, feats, g, tau, bonus, ws_t)
        return feats, g, tau, bonus

    def inject_rel(feats, blk):
        rs = torch.arange(batch, dtype=torch.int32, device=DEV).repeat_interleave(blk)
        rp = torch.arange(blk, dtype=torch.int32, device=DEV).repeat(batch)
        rt.inject_ctx(S.draft, dkv, feats.reshape(batch * blk, -1).contiguous(), rs, rp, 1, blk, ws_d)

    # prefill: one causal pass over the prompt, inject its features, advance both caches
    ids = torch.tensor(np.stack(prompts), dtype=torch.int32, device=DEV)
    feats, g, _, _ = verify(ids[:, 0].contiguous(), ids[:, 1:].contiguous(), n0)
    inject_rel(feats, n0)
    rt.kv_commit(tkv, dkv, torch.full((batch,), n0, dtype=torch.int32, device=DEV), n0)
    anchor = g[:, -1].contiguous()
    emitted = [[int(a)] for a in anchor.cpu()]
    drafts = torch.zeros(batch, B - 1, dtype=torch.int32, device=DEV)
    while min(len(e) for e in emitted) < n_new:
        rt.draft_block(S.draft, dkv, anchor, B, drafts, ws_d)
        feats, g, tau, bonus = verify(anchor, drafts, B)
        inject_rel(feats, B)
        rt.kv_commit(tkv, dkv, tau, B)
        tkv.refresh_len_bound()
        dkv.refresh_len_bound()
        t, bo, d = tau.cpu().numpy(), bonus.cpu().numpy(), drafts.cpu().numpy()
        for b in range(batch):
            emitted[b] += [int(x) for x in d[b, : t[b] - 1]] + [int(bo[b])]
        anchor = bonus.clone()
    torch.cuda.synchronize()
    assert tkv.err.item() == 0 and dkv.err.item() == 0
    assert torch.equal(tkv.seq_len, dkv.seq_len)
    for b in range(batch):
        ref = O.greedy_decode(S.np_tw, S.np_shared, T, prompts[b], n_new, store=S.store)
        got = emitted[b][:n_new]
        if got != ref:
            # allowed only past a near-tie of the oracle's own logits
            i = next(i for i in range(n_new) if got[i] != ref[i])
            _, z, _, _, _ = O.target_forward(S.np_tw, S.np_shared, T, None,
                                             np.concatenate([prompts[b], ref[:i]]), 0, (), store=S.store)
            assert O.top2_gap(z[-1]) < 1e-2, f"{name} seq {b}: stream differs at {i}"
