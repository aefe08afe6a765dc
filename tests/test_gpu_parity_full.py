"""GPU vs oracle parity at the full workload sizes, through the C ABI, in the launch
configuration the bench uses.

 * Qwen3-8B-shaped drafter, batch 1, 4096 injected rows (512-row injection chunks):
   every cache row, every hidden state, every logit, every draft id; then blocks of 8 and
   10 on the same cache (the block size is a runtime argument).
 * batch 16, contexts in [2048, 8192], 64-token pages in shuffled order: the M = 256 tiled
   GEMM path and the ragged paged attention; injection of the 16 block rows of every
   sequence at its own position.
 * batch 1, 262144-row context: split-K attention over the whole context, plus nine
   512-row injection chunks (8 at seeded random places and the last one, positions up to
   262143: RoPE at large positions).
 * batch 8 with an 8-layer target over 8192-token caches: two full cycles of every
   sequence under the seeded p = 0.7 acceptance-forcing rule - draft, verify, accept,
   inject of the verified rows, commit - with both caches' committed rows checked.
 * the 4K, batch-16 and 262K draft blocks run twice with bitwise identical results.

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


def _repeat_is_bitwise(S, kv, anchor, B, batch, ws, first, what):
    """The same draft block run again: ids, logits and hidden states bit for bit (the
    argmax's 64-bit atomic maxima and the split-K merge run across many workgroups, so
    this checks that no result depends on their timing)."""
    again = _draft_outputs(S, kv, B, batch)
    rt.draft_block(S.draft, kv, anchor, B, again[0], ws, again[1], again[2])
    torch.cuda.synchronize()
    for x, y, name in zip(first, again, ("ids", "logits", "hidden")):
        assert torch.equal(x, y), f"{what}: repeated {name} differ"


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
    _repeat_is_bitwise(S, kv, anchor, B, 1, ws, (ids, logits, hid), "cfg 4k")
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


def _no_copy_matches(S, kv, anchor, B, batch, ws, ids, what):
    """Drafting without the logits and hidden-state copies (a decoding loop's call) gives
    the same ids, bit for bit."""
    ids2 = torch.zeros_like(ids)
    rt.draft_block(S.draft, kv, anchor, B, ids2, ws)
    torch.cuda.synchronize()
    assert kv.err.item() == 0
    assert torch.equal(ids2, ids), f"{what}: ids depend on the logits copy"


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
    _repeat_is_bitwise(S, kv, anchor, B, batch, ws, (ids, logits, hid), "cfg b16")
    _no_copy_matches(S, kv, anchor, B, batch, ws, ids, "cfg b16")
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
    # 512-row injection chunks overwrite context rows: 8 seeded random chunks (whole
    # chunks of the context) plus the last one, at the far end of the context
    chunk = w.inject_chunk
    ws = S.workspace(S.draft, B, kv.capacity, inject_rows=chunk)
    seq = torch.zeros(chunk, dtype=torch.int32, device=DEV)
    rng = np.random.Generator(np.random.PCG64(4096))
    starts = sorted(int(x) * chunk for x in rng.choice(n // chunk - 1, size=8, replace=False))
    for p0 in starts + [n - chunk]:
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
    _repeat_is_bitwise(S, kv, anchor, B, 1, ws, (ids, logits, hid), "cfg 256k")


P_FORCE = 0.7          # the forcing rule's probability for the full-size cycle test
FORCE_SEED = 4321
CYCLES = 2


def _greedy_continuation(S, T, cache, anchor, n, count):
    """The oracle target's greedy tokens g*_0 .. g*_{count-1} after `anchor` at position n
    (one causal pass per token over the growing block)."""
    toks = [int(anchor)]
    for _ in range(count):
        g, _, _, _, _ = O.verify(S.np_tw, S.np_shared, T, cache, toks, n, (), store=S.store)
        toks.append(int(g[-1]))
    return toks[1:]


def test_qwen3_8b_cycle_batch8_target8():
    """Full speculative cycles of the batch-8 workload, every sequence against the oracle:
    draft (hidden states, logits, ids), the seeded p = 0.7 forcing rule (drafts taken from
    the oracle's own greedy continuation of the target, a forced mismatch after the run of
    heads), verify (hidden states, logits, argmax, tapped features, the block's K/V in every
    target layer), acceptance (tau, bonus; tau = f + 1 under the rule), injection and commit
    (the committed rows of every layer of both caches), then the next cycle from the bonus
    token.  A sequence whose (tau, bonus) differs from the oracle's - allowed only where
    the oracle decides them by a near-tie - leaves the comparison from there on (the two
    sides then hold different lengths)."""
    w = synth.workload("qwen3_8b_cycle_b8")
    S = Setup(w, target=True)
    lens = synth.ctx_lengths(w)
    B, batch, T, D = w.block, w.batch, w.target, w.draft
    cap = max(lens) + (CYCLES + 1) * B + 64
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
    k = len(w.taps)
    anchor = synth.anchors(w, "cpu").numpy().astype(np.int64)
    n = list(lens)
    active = set(range(batch))
    rs = torch.arange(batch, dtype=torch.int32, device=DEV).repeat_interleave(B)
    rp = torch.arange(B, dtype=torch.int32, device=DEV).repeat(batch)
    compared_tau = 0
    for c in range(CYCLES):
        a_dev = torch.tensor(anchor, dtype=torch.int32, device=DEV)
        # ---- draft (M = 128: tiled GEMMs), every active sequence against the oracle ----
        ids, logits, hid = _draft_outputs(S, dkv, B, batch)
        rt.draft_block(S.draft, dkv, a_dev, B, ids, ws_d, logits, hid)
        torch.cuda.synchronize()
        assert dkv.err.item() == 0
        own = {}
        for b in sorted(active):
            o_ids, o_z, o_hid = O.draft_block(S.np_dw, S.np_shared, D, d_np[b], int(anchor[b]), n[b], B,
                                              store=S.store)
            for l in range(D.n_layers + 1):
                assert_close(hid[l, b].cpu().numpy(), o_hid[l], TOLB, f"cycle {c} draft hidden {l} seq {b}")
            assert_rows_close(logits[b].cpu().numpy(), o_z, TOLB, f"cycle {c} draft logits seq {b}")
            assert_ids(ids[b].cpu().numpy(), o_ids, o_z, f"cycle {c} draft ids seq {b}")
            own[b] = o_ids
        # ---- seeded forcing rule on the oracle's greedy continuation ----
        coins = synth.force_coins(FORCE_SEED, c, batch, B, P_FORCE)
        drafts = synth.uniform_ints((batch, B - 1), 0, T.vocab - 1, w.cid, f"cycle{c}.drafts").numpy()
        drafts = drafts.astype(np.int64)
        runs = {}
        for b in sorted(active):
            f = int(np.argmin(np.append(coins[b], False)))
            gstar = _greedy_continuation(S, T, t_np[b], anchor[b], n[b], f + 1)
            drafts[b], runs[b] = synth.forced_drafts(coins[b], gstar, own[b], T.vocab)
        d_dev = torch.tensor(drafts, dtype=torch.int32, device=DEV)
        # ---- verify + accept ----
        feats = torch.zeros(batch, B, k * T.hidden, dtype=torch.bfloat16, device=DEV)
        g = torch.zeros(batch, B, dtype=torch.int32, device=DEV)
        tau = torch.zeros(batch, dtype=torch.int32, device=DEV)
        bonus = torch.zeros(batch, dtype=torch.int32, device=DEV)
        vlog = torch.zeros(batch, B, T.vocab, device=DEV)
        vhid = torch.zeros(T.n_layers + 1, batch, B, T.hidden, device=DEV)
        rt.verify_accept(S.target, tkv, a_dev, d_dev, B, feats, g, tau, bonus, ws_t, vlog, vhid)
        torch.cuda.synchronize()
        assert tkv.err.item() == 0
        tau_np, bonus_np, g_np = tau.cpu().numpy(), bonus.cpu().numpy(), g.cpu().numpy()
        for b in range(batch):   # every sequence: the greedy rule on the kernel's own argmax
            a2 = 0
            while a2 < B - 1 and int(drafts[b, a2]) == int(g_np[b, a2]):
                a2 += 1
            assert (int(tau_np[b]), int(bonus_np[b])) == (a2 + 1, int(g_np[b, a2]))
        if c == 0:
            # the same verification without the logits and hidden-state copies (it rewrites
            # the same block rows): the same argmax, tau and bonus, bit for bit
            g2, tau2, bonus2 = torch.zeros_like(g), torch.zeros_like(tau), torch.zeros_like(bonus)
            rt.verify_accept(S.target, tkv, a_dev, d_dev, B, torch.zeros_like(feats), g2, tau2, bonus2, ws_t)
            torch.cuda.synchronize()
            assert tkv.err.item() == 0
            for x, y, what in ((g2, g, "argmax"), (tau2, tau, "tau"), (bonus2, bonus, "bonus")):
                assert torch.equal(x, y), f"cycle 0: {what} depends on the logits copy"
        oracle_commit = {}
        for b in sorted(active):
            block = [int(anchor[b])] + [int(x) for x in drafts[b]]
            og, oz, of, onew, ohid = O.verify(S.np_tw, S.np_shared, T, t_np[b], block, n[b], w.taps,
                                              store=S.store)
            what = f"cycle {c} verify seq {b}"
            for l in range(T.n_layers + 1):
                assert_close(vhid[l, b].cpu().numpy(), ohid[l], TOLB, f"{what} hidden {l}")
            assert_rows_close(vlog[b].cpu().numpy(), oz, TOLB, f"{what} logits")
            assert_close(synth.to_numpy(feats[b]), of, TOLB, f"{what} tapped feats")
            assert_ids(g_np[b], og, oz, f"{what} target argmax")
            for l in range(T.n_layers):
                K, V = read_cache(tkv, l, b, n[b] + B)
                assert_close(K[n[b]:], onew[l][0], TOLB, f"{what} block K layer {l}")
                assert_close(V[n[b]:], onew[l][1], TOLB, f"{what} block V layer {l}")
            assert_accept(tau_np[b], bonus_np[b], g_np[b], drafts[b], og, oz, what)
            a, t_o, bo = O.accept(drafts[b], og)
            if (int(tau_np[b]), int(bonus_np[b])) == (t_o, bo):   # both sides in the same state
                # the rule fixes tau = f + 1 (B after a full run of heads), unless one of the
                # rows deciding it is an oracle near-tie (the continuation came from shorter
                # passes, whose float32 rounding may order such a pair differently)
                expect = min(runs[b] + 1, B)
                if np.all(O.top2_gap(np.asarray(oz[:expect], dtype=np.float64)) >= NEAR_TIE):
                    assert t_o == expect, f"{what}: tau {t_o} under a run of {runs[b]} heads"
                compared_tau += 1
                oracle_commit[b] = (t_o, bo, onew, of)
            else:
                active.discard(b)    # differs at a near-tie (allowed above): states now differ
        # ---- inject all B verified rows at the old lengths, commit tau ----
        rt.inject_ctx(S.draft, dkv, feats.reshape(batch * B, -1).contiguous(), rs, rp, 1, B, ws_d)
        rt.kv_commit(tkv, dkv, tau, B)
        torch.cuda.synchronize()
        assert dkv.err.item() == 0 and tkv.err.item() == 0
        seq_t, seq_d = tkv.seq_len.cpu().tolist(), dkv.seq_len.cpu().tolist()
        assert seq_t == seq_d
        for b in range(batch):
            assert seq_t[b] == n[b] + int(tau_np[b])
        # ---- the committed rows of both caches, every layer, against the oracle's own ----
        for b, (t, bo, onew, of) in oracle_commit.items():
            t_np[b] = O.append_kv(t_np[b], onew, t)
            inj = O.inject(of[:t], n[b] + np.arange(t), S.np_dw, D, store=S.store)
            d_np[b] = O.append_kv(d_np[b], inj, t)
            for l in range(T.n_layers):
                K, V = read_cache(tkv, l, b, n[b] + t)
                assert_close(K, t_np[b][l][0], TOLB, f"cycle {c} committed target K seq {b} layer {l}")
                assert_close(V, t_np[b][l][1], TOLB, f"cycle {c} committed target V seq {b} layer {l}")
            for l in range(D.n_layers):
                K, V = read_cache(dkv, l, b, n[b] + t)
                assert_close(K[n[b]:], inj[l][0], TOLB, f"cycle {c} committed draft K seq {b} layer {l}")
                assert_close(V[n[b]:], inj[l][1], TOLB, f"cycle {c} committed draft V seq {b} layer {l}")
        n = [n[b] + int(tau_np[b]) for b in range(batch)]
        anchor = bonus_np.astype(np.int64)
    # near-ties take a sequence out rarely: most sequences are compared through every cycle
    assert compared_tau >= CYCLES * batch - 3, (compared_tau, sorted(active))
    print(f"cycle test: {compared_tau} accepts compared, {len(active)} sequences through every cycle")
