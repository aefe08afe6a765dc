"""GPU vs oracle parity at the full workload sizes, through the C ABI, in the launch
configuration the bench uses.

 * Qwen3-8B-shaped drafter, batch 1, 4096 injected rows (512-row injection chunks):
   every cache row, every hidden state, every logit, every draft id; then blocks of 8 and
   10 on the same cache (the block size is a runtime argument).
 * batch 16, contexts in [2048, 8192], 64-token pages in shuffled order: the M = 256 tiled
   GEMM path and the ragged paged attention; injection of the 16 block rows of every
   sequence at its own position.
 * batch 1, 262144-row context: split-K attention over the whole context, plus two
   512-row injection chunks at positions up to 262143 (RoPE at large positions).
 * batch 8 with an 8-layer target over 8192-token caches: draft, verify (forced and random
   drafts), accept, inject of the verified rows, commit.

The oracle cannot afford to inject 80K-262K context rows (20-66 TFLOP on the host), so
for the long contexts both sides read the same synthetic context K/V (N(0, 1), taken as
already rotated) and injection is checked on sampled chunks instead.
"""
import gc

import numpy as np
import pytest
import torch

import oracle as O
import synth

from harness import (DEV, NEAR_TIE, TOL, Setup, assert_accept, assert_close, assert_ids,
                     assert_rows_close, check_selection, read_cache)
from block_diffusion_drafter_03_amd import runtime as rt

pytestmark = pytest.mark.gpu
TOLB = TOL["bf16"]


def _free():
    gc.collect()
    torch.cuda.empty_cache()


def _draft_outputs(S, kv, B, batch):
    m = S.w.draft
    ids = torch.zeros(batch, B - 1, dtype=torch.int32, device=DEV)
    logits = torch.zeros(batch, B - 1, m.vocab, device=DEV)
    hid = torch.zeros(m.n_layers + 1, batch, B, m.hidden, device=DEV)
    return ids, logits, hid


def _check_draft(S, b, ctx_np, n, anchor, ids, logits, hid, what, block=None):
    m = S.w.draft
    o_ids, o_z, o_hid = O.draft_block(S.np_dw, S.np_shared, m, ctx_np, int(anchor), n,
                                      block or S.w.block, store=S.store)
    for l in range(m.n_layers + 1):
        assert_close(hid[l, b].cpu().numpy(), o_hid[l], TOLB, f"{what} hidden layer {l}")
    assert_rows_close(logits[b].cpu().numpy(), o_z, TOLB, f"{what} logits")
    return assert_ids(ids[b].cpu().numpy(), o_ids, o_z, f"{what} draft ids")


def test_qwen3_8b_batch1_ctx4k():
    w = synth.workload("qwen3_8b_b1_ctx4k")
    S = Setup(w)
    n, B = w.ctx[0], w.block
    kv = S.kv(w.draft, n + B + 64)
    ws = S.workspace(S.draft, B, kv.capacity, inject_rows=512)
    feats = synth.features(w, n, DEV, tag="feats.b0")
    seq = torch.zeros(512, dtype=torch.int32, device=DEV)
    for a in range(0, n, 512):
        rt.inject_ctx(S.draft, kv, feats[a:a + 512].contiguous(), seq,
                      torch.arange(a, a + 512, dtype=torch.int32, device=DEV), 0, a + 512, ws)
    kv.set_seq_len(n)
    anchor = synth.anchors(w, DEV)
    ids, logits, hid = _draft_outputs(S, kv, B, 1)
    rt.draft_block(S.draft, kv, anchor, B, ids, ws, logits, hid)
    torch.cuda.synchronize()
    assert kv.err.item() == 0
    ctx = O.inject(synth.to_numpy(feats), np.arange(n), S.np_dw, w.draft, store=S.store)
    for l in range(w.draft.n_layers):
        K, V = read_cache(kv, l, 0, n)
        assert_close(K, ctx[l][0], TOLB, f"cfg 4k ctx K layer {l}")
        assert_close(V, ctx[l][1], TOLB, f"cfg 4k ctx V layer {l}")
    checked = _check_draft(S, 0, ctx, n, anchor[0], ids, logits, hid, "cfg 4k")
    assert checked >= 10    # the near-tie exclusion leaves most positions checked
    # the block size is a runtime argument: blocks of 8 and 10 on the same cache and
    # workspace (the schedule of a B = 16 design run at smaller B)
    for Bs in (8, 10):
        ids, logits, hid = _draft_outputs(S, kv, Bs, 1)
        rt.draft_block(S.draft, kv, anchor, Bs, ids, ws, logits, hid)
        torch.cuda.synchronize()
        assert kv.err.item() == 0
        checked = _check_draft(S, 0, ctx, n, anchor[0], ids, logits, hid, f"cfg 4k B={Bs}", block=Bs)
        assert checked >= Bs - 4
    # temperature sampling at T = 1 (the drafter's logits and its sampled ids)
    zd = torch.zeros(1, B - 1, w.draft.vocab, device=DEV)
    ids = torch.zeros(1, B - 1, dtype=torch.int32, device=DEV)
    rt.draft_block_sampled(S.draft, kv, anchor, B, 1.0, 99, 3, ids, zd, ws)
    torch.cuda.synchronize()
    assert kv.err.item() == 0
    o_ids, o_z, o_keys = O.draft_block_sampled(S.np_dw, S.np_shared, w.draft, ctx, int(anchor[0]), n, B,
                                               1.0, 99, 3, 0, store=S.store)
    assert_rows_close(zd[0].cpu().numpy(), o_z, TOLB, "cfg 4k sampled draft logits")
    gaps = O.top2_gap(o_keys.astype(np.float64))
    sel = gaps >= NEAR_TIE
    assert sel.sum() >= B - 4
    assert np.array_equal(ids[0].cpu().numpy()[sel], o_ids[sel]), "cfg 4k sampled draft ids"
    # DFlash 2 path selector at its full size: rank 256, top-16 candidates
    sw = synth.selector_weights(w, rank=256, device=DEV)
    w_a, w_b = ((sw[k].float() * 50.0).to(torch.bfloat16) for k in ("w_a", "w_b"))
    selr = rt.Selector(S.draft, w_a, w_b, sw["w_h"], top_k=16)
    sws = rt.Workspace(selr.workspace_bytes(S.draft, 1, B), DEV)
    ids = torch.zeros(1, B - 1, dtype=torch.int32, device=DEV)
    cand = torch.zeros(1, B - 1, 16, dtype=torch.int32, device=DEV)
    rt.draft_block_select(S.draft, kv, anchor, B, selr, ids, zd, ws, sws, candidates=cand)
    torch.cuda.synchronize()
    assert kv.err.item() == 0
    _, o_z, o_hid = O.draft_block(S.np_dw, S.np_shared, w.draft, ctx, int(anchor[0]), n, B, store=S.store)
    o_ids, o_cand, o_rows = O.select_path(o_z, o_hid[-1][1:], int(anchor[0]), S.np_shared["embed"],
                                          S.np_dw["g_f"], w.draft.rms_eps, synth.to_numpy(w_a),
                                          synth.to_numpy(w_b), synth.to_numpy(sw["w_h"]), top_k=16)
    assert_rows_close(zd[0].cpu().numpy(), o_z, TOLB, "cfg 4k selector draft logits")
    c, k = check_selection(ids[0].cpu().numpy(), cand[0].cpu().numpy(), o_ids, o_cand, o_rows, o_z, 16,
                           NEAR_TIE, "cfg 4k selector")
    assert c >= (B - 1) // 3 and k >= (B - 1) // 2, (c, k)
    # DFlash 2 two-tap convolutions around every sublayer of the full-size drafter
    dconv = synth.dconv_weights(w, DEV)
    conv = rt.Model(w.draft, S.dw, S.shared, n_taps=w.n_taps, draft=True, dconv=dconv)
    ids, logits, hid = _draft_outputs(S, kv, B, 1)
    rt.draft_block(conv, kv, anchor, B, ids, ws, logits, hid)
    torch.cuda.synchronize()
    assert kv.err.item() == 0
    np_conv = {**S.np_dw, **{k: synth.to_numpy(v) for k, v in dconv.items()}}
    o_ids, o_z, o_hid = O.draft_block(np_conv, S.np_shared, w.draft, ctx, int(anchor[0]), n, B, store=S.store)
    for l in range(w.draft.n_layers + 1):
        assert_close(hid[l, 0].cpu().numpy(), o_hid[l], TOLB, f"cfg 4k dconv hidden layer {l}")
    assert_rows_close(logits[0].cpu().numpy(), o_z, TOLB, "cfg 4k dconv logits")
    assert assert_ids(ids[0].cpu().numpy(), o_ids, o_z, "cfg 4k dconv draft ids") >= 10
    conv.close()


def test_qwen3_8b_batch16_paged_ragged():
    w = synth.workload("qwen3_8b_b16_paged")
    S = Setup(w)
    lens = synth.ctx_lengths(w)
    B, batch = w.block, w.batch
    kv = S.kv(w.draft, max(lens) + B + 64, seed=7)
    dense = synth.synthetic_ctx_kv(w, "draft", lens, DEV)
    for l in range(w.draft.n_layers):
        for b in range(batch):
            kv.write_dense(l, b, dense[l][b][0], dense[l][b][1])
    kv.set_seq_len(lens)
    ctx_np = [[(synth.to_numpy(dense[l][b][0]), synth.to_numpy(dense[l][b][1]))
               for l in range(w.draft.n_layers)] for b in range(batch)]
    del dense
    _free()
    ws = S.workspace(S.draft, B, kv.capacity, inject_rows=batch * B)
    anchor = synth.anchors(w, DEV)
    ids, logits, hid = _draft_outputs(S, kv, B, batch)
    rt.draft_block(S.draft, kv, anchor, B, ids, ws, logits, hid)
    torch.cuda.synchronize()
    assert kv.err.item() == 0
    checked = 0
    for b, n in enumerate(lens):
        checked += _check_draft(S, b, ctx_np[b], n, anchor[b], ids, logits, hid, f"cfg b16 seq {b}")
    assert checked >= 10 * batch
    # injection of every sequence's 16 block rows at its own (ragged) position, M = 256
    feats = synth.features(w, batch * B, DEV, tag="cycle.feats")
    rs = torch.arange(batch, dtype=torch.int32, device=DEV).repeat_interleave(B)
    rp = torch.arange(B, dtype=torch.int32, device=DEV).repeat(batch)
    rt.inject_ctx(S.draft, kv, feats, rs, rp, 1, B, ws)
    torch.cuda.synchronize()
    assert kv.err.item() == 0
    f_np = synth.to_numpy(feats)
    for b, n in enumerate(lens):
        inj = O.inject(f_np[b * B:(b + 1) * B], n + np.arange(B), S.np_dw, w.draft, store=S.store)
        for l in range(w.draft.n_layers):
            K, V = read_cache(kv, l, b, n + B)
            assert_close(K[n:], inj[l][0], TOLB, f"cfg b16 injected K seq {b} layer {l}")
            assert_close(V[n:], inj[l][1], TOLB, f"cfg b16 injected V seq {b} layer {l}")


def test_qwen3_8b_batch1_ctx256k():
    w = synth.workload("qwen3_8b_b1_ctx256k")
    S = Setup(w)
    n, B = w.ctx[0], w.block
    kv = S.kv(w.draft, n + B + 64, permute_pages=False)
    ctx_np = []
    for l in range(w.draft.n_layers):
        k = synth.normal((n, w.draft.n_kv_heads, w.draft.head_dim), 1.0, w.cid, f"draft.ctxK.L{l}.b0", DEV, w.dtype)
        v = synth.normal((n, w.draft.n_kv_heads, w.draft.head_dim), 1.0, w.cid, f"draft.ctxV.L{l}.b0", DEV, w.dtype)
        kv.write_dense(l, 0, k, v)
        ctx_np.append([synth.to_numpy(k), synth.to_numpy(v)])
        del k, v
    _free()
    kv.set_seq_len(n)
    # two 512-row injection chunks overwrite context rows, one at the far end of the context
    chunk = w.inject_chunk
    ws = S.workspace(S.draft, B, kv.capacity, inject_rows=chunk)
    seq = torch.zeros(chunk, dtype=torch.int32, device=DEV)
    for p0 in (4096, n - chunk):
        feats = synth.features(w, chunk, DEV, tag=f"chunk.{p0}")
        rt.inject_ctx(S.draft, kv, feats, seq, torch.arange(p0, p0 + chunk, dtype=torch.int32, device=DEV), 0,
                      p0 + chunk, ws)
        inj = O.inject(synth.to_numpy(feats), p0 + np.arange(chunk), S.np_dw, w.draft, store=S.store)
        torch.cuda.synchronize()
        for l in range(w.draft.n_layers):
            K, V = kv.read_dense(l, 0, chunk, start=p0)
            assert_close(synth.to_numpy(K), inj[l][0], TOLB, f"cfg 256k chunk@{p0} K layer {l}")
            assert_close(synth.to_numpy(V), inj[l][1], TOLB, f"cfg 256k chunk@{p0} V layer {l}")
            ctx_np[l][0][p0:p0 + chunk] = inj[l][0]     # the oracle's own rows from here on
            ctx_np[l][1][p0:p0 + chunk] = inj[l][1]
    anchor = synth.anchors(w, DEV)
    ids, logits, hid = _draft_outputs(S, kv, B, 1)
    rt.draft_block(S.draft, kv, anchor, B, ids, ws, logits, hid)
    torch.cuda.synchronize()
    assert kv.err.item() == 0
    checked = _check_draft(S, 0, [tuple(c) for c in ctx_np], n, anchor[0], ids, logits, hid, "cfg 256k")
    assert checked >= 10


def test_qwen3_8b_cycle_batch8_target8():
    w = synth.workload("qwen3_8b_cycle_b8")
    S = Setup(w, target=True)
    lens = synth.ctx_lengths(w)
    B, batch, T, D = w.block, w.batch, w.target, w.draft
    cap = max(lens) + 2 * B + 64
    tkv = S.kv(T, cap, seed=11)
    dkv = S.kv(D, cap, seed=12)
    tctx = synth.synthetic_ctx_kv(w, "target", lens, DEV)
    dctx = synth.synthetic_ctx_kv(w, "draft", lens, DEV)
    for kvc, dense, L in ((tkv, tctx, T.n_layers), (dkv, dctx, D.n_layers)):
        for l in range(L):
            for b in range(batch):
                kvc.write_dense(l, b, dense[l][b][0], dense[l][b][1])
        kvc.set_seq_len(lens)
    t_np = [[(synth.to_numpy(tctx[l][b][0]), synth.to_numpy(tctx[l][b][1])) for l in range(T.n_layers)]
            for b in range(batch)]
    d_np = [[(synth.to_numpy(dctx[l][b][0]), synth.to_numpy(dctx[l][b][1])) for l in range(D.n_layers)]
            for b in range(batch)]
    del tctx, dctx
    _free()
    ws_d = S.workspace(S.draft, B, dkv.capacity, inject_rows=batch * B)
    ws_t = S.workspace(S.target, B, tkv.capacity)
    anchor = synth.anchors(w, DEV)
    # draft (M = 128: tiled GEMMs) checked against the oracle
    ids, logits, hid = _draft_outputs(S, dkv, B, batch)
    rt.draft_block(S.draft, dkv, anchor, B, ids, ws_d, logits, hid)
    torch.cuda.synchronize()
    a_np = anchor.cpu().numpy()
    for b in (0, 5):
        _check_draft(S, b, d_np[b], lens[b], a_np[b], ids, logits, hid, f"cycle draft seq {b}")
    # verify input: sequence 0 drafts the target's own greedy continuation for 3 positions
    # (oracle pre-pass) and then a forced mismatch; the other sequences take seeded random
    # ids (mostly rejected at once)
    drafts = synth.uniform_ints((batch, B - 1), 0, T.vocab - 1, w.cid, "cycle.drafts").numpy().astype(np.int64)
    toks = [int(a_np[0])]
    for _ in range(4):
        g0, _, _, _, _ = O.verify(S.np_tw, S.np_shared, T, t_np[0], toks, lens[0], w.taps, store=S.store)
        toks.append(int(g0[-1]))
    drafts[0, :3] = toks[1:4]
    if drafts[0, 3] == toks[4]:
        drafts[0, 3] = (toks[4] + 1) % T.vocab
    d_dev = torch.tensor(drafts, dtype=torch.int32, device=DEV)
    k = len(w.taps)
    feats = torch.zeros(batch, B, k * T.hidden, dtype=torch.bfloat16, device=DEV)
    g = torch.zeros(batch, B, dtype=torch.int32, device=DEV)
    tau = torch.zeros(batch, dtype=torch.int32, device=DEV)
    bonus = torch.zeros(batch, dtype=torch.int32, device=DEV)
    vlog = torch.zeros(batch, B, T.vocab, device=DEV)
    vhid = torch.zeros(T.n_layers + 1, batch, B, T.hidden, device=DEV)
    rt.verify_accept(S.target, tkv, anchor, d_dev, B, feats, g, tau, bonus, ws_t, vlog, vhid)
    torch.cuda.synchronize()
    assert tkv.err.item() == 0
    tau_np, bonus_np, g_np = tau.cpu().numpy(), bonus.cpu().numpy(), g.cpu().numpy()
    oracle_rows = {}
    for b in (0, 3):
        block = [int(a_np[b])] + [int(x) for x in drafts[b]]
        og, oz, of, onew, ohid = O.verify(S.np_tw, S.np_shared, T, t_np[b], block, lens[b], w.taps,
                                          store=S.store)
        for l in range(T.n_layers + 1):
            assert_close(vhid[l, b].cpu().numpy(), ohid[l], TOLB, f"cycle verify hidden {l} seq {b}")
        assert_rows_close(vlog[b].cpu().numpy(), oz, TOLB, f"cycle verify logits seq {b}")
        assert_close(synth.to_numpy(feats[b]), of, TOLB, f"cycle tapped feats seq {b}")
        assert_ids(g_np[b], og, oz, f"cycle target argmax seq {b}")
        for l in (0, T.n_layers - 1):
            K, V = read_cache(tkv, l, b, lens[b] + B)
            assert_close(K[lens[b]:], onew[l][0], TOLB, f"cycle new target K seq {b} layer {l}")
            assert_close(V[lens[b]:], onew[l][1], TOLB, f"cycle new target V seq {b} layer {l}")
        if assert_accept(tau_np[b], bonus_np[b], g_np[b], drafts[b], og, oz, f"cycle accept seq {b}"):
            oracle_rows[b] = (O.accept(drafts[b], og)[1], of)
        if b == 0 and np.all(O.top2_gap(oz[:5]) >= 1e-2):
            assert int(tau_np[0]) == 4 and int(bonus_np[0]) == int(og[3])
    for b in range(batch):   # every sequence: the greedy rule on the kernel's own argmax
        a2 = 0
        while a2 < B - 1 and int(drafts[b, a2]) == int(g_np[b, a2]):
            a2 += 1
        assert (int(tau_np[b]), int(bonus_np[b])) == (a2 + 1, int(g_np[b, a2]))
    # inject all B verified rows at the old lengths, then commit tau
    rs = torch.arange(batch, dtype=torch.int32, device=DEV).repeat_interleave(B)
    rp = torch.arange(B, dtype=torch.int32, device=DEV).repeat(batch)
    rt.inject_ctx(S.draft, dkv, feats.reshape(batch * B, -1).contiguous(), rs, rp, 1, B, ws_d)
    rt.kv_commit(tkv, dkv, tau, B)
    torch.cuda.synchronize()
    assert dkv.err.item() == 0 and tkv.err.item() == 0
    assert tkv.seq_len.cpu().tolist() == [n + int(t) for n, t in zip(lens, tau_np)]
    assert dkv.seq_len.cpu().tolist() == tkv.seq_len.cpu().tolist()
    # the drafter's committed rows: the oracle injects its own tapped features
    for b, (t, of) in oracle_rows.items():
        n = lens[b]
        inj = O.inject(of[:t], n + np.arange(t), S.np_dw, D, store=S.store)
        K, V = read_cache(dkv, 0, b, n + t)
        assert_close(K[n:], inj[0][0], TOLB, f"cycle committed draft K seq {b}")
        assert_close(V[n:], inj[0][1], TOLB, f"cycle committed draft V seq {b}")
