"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: brute-force loops,
closed forms, invariants of the method, textbook identities, or numbers printed on the
pages (fixtures under tests/golden/, with their citations).  A planted mistake in the
oracle (dropped term, wrong sign or index, transposed operand, wrong mask) makes at
least one of these fail.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle as O
import synth
from synth import ModelShape, Workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F64 = np.float64

TINY_SHAPE = ModelShape(n_layers=2, hidden=32, n_q_heads=4, n_kv_heads=2, head_dim=8, ffn=48,
                        vocab=64)
TINY_TGT = ModelShape(n_layers=3, hidden=32, n_q_heads=4, n_kv_heads=2, head_dim=8, ffn=40,
                      vocab=64)


def _wl(cid=900, draft=TINY_SHAPE, target=TINY_TGT, taps=(0, 1), block=4):
    return Workload(cid=cid, name=f"pin{cid}", dtype="f32", draft=draft, n_taps=len(taps),
                    block=block, batch=1, ctx=(5,), target=target, taps=taps)


def _np(d):
    return {k: synth.to_numpy(v).astype(F64) for k, v in d.items()}


def _models(cid=900, **kw):
    wl = _wl(cid, **kw)
    return wl, _np(synth.model_weights(wl, "draft")), _np(synth.model_weights(wl, "target")), \
        _np(synth.shared_weights(wl))


def _scale_mats(w, s):
    return {k: (v * s if v.ndim == 2 else v) for k, v in w.items()}


# ---------------------------------------------------------------------------------------
# attention


def _attn_bruteforce(q, k, v, visible):
    Tq, d = q.shape
    Tk = k.shape[0]
    out = np.zeros((Tq, v.shape[1]))
    for i in range(Tq):
        scores = []
        for j in range(Tk):
            if visible[i, j]:
                scores.append((j, sum(q[i, c] * k[j, c] for c in range(d)) / math.sqrt(d)))
        mx = max(s for _, s in scores)
        den = sum(math.exp(s - mx) for _, s in scores)
        for j, s in scores:
            wgt = math.exp(s - mx) / den
            for c in range(v.shape[1]):
                out[i, c] += wgt * v[j, c]
    return out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_attention_matches_bruteforce(seed):
    rng = np.random.default_rng(seed)
    Tq, Tk, d = 4, 7, 6
    q, k, v = rng.normal(size=(Tq, d)), rng.normal(size=(Tk, d)), rng.normal(size=(Tk, 5))
    visible = rng.random((Tq, Tk)) < 0.7
    visible[:, 0] = True
    np.testing.assert_allclose(O.attention(q, k, v, visible, F64),
                               _attn_bruteforce(q, k, v, visible), rtol=1e-12, atol=1e-12)


def test_softmax_rows_sum_to_one():
    rng = np.random.default_rng(3)
    q, k = rng.normal(size=(16, 32)) * 3, rng.normal(size=(300, 32)) * 3
    v = np.ones((300, 32))
    vis = rng.random((16, 300)) < 0.5
    vis[:, 0] = True
    np.testing.assert_allclose(O.attention(q, k, v, vis, F64), 1.0, rtol=0, atol=1e-13)
    np.testing.assert_allclose(O.attention(q, k, v, vis, np.float32), 1.0, rtol=0, atol=2e-6)


def test_lse_merge_identity():
    """attention over A u B = LSE-weighted merge of attention over A and over B."""
    rng = np.random.default_rng(4)
    q, k, v = rng.normal(size=(3, 8)), rng.normal(size=(20, 8)), rng.normal(size=(20, 8))
    full = O.attention(q, k, v, np.ones((3, 20), bool), F64)

    def part(sl):
        s = q @ k[sl].T / math.sqrt(8)
        m = s.max(-1, keepdims=True)
        p = np.exp(s - m)
        return m, p.sum(-1, keepdims=True), O.attention(q, k[sl], v[sl], np.ones((3, s.shape[1]), bool), F64)

    (m1, l1, o1), (m2, l2, o2) = part(slice(0, 9)), part(slice(9, 20))
    m = np.maximum(m1, m2)
    w1, w2 = l1 * np.exp(m1 - m), l2 * np.exp(m2 - m)
    np.testing.assert_allclose((o1 * w1 + o2 * w2) / (w1 + w2), full, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------------------
# RoPE


def test_rope_is_complex_rotation():
    rng = np.random.default_rng(5)
    d, base = 8, 500.0
    x = rng.normal(size=(6, 3, d))
    pos = np.array([0, 1, 7, 100, 4096, 262143])
    got = O.rope(x, pos, base, F64)
    z = x[..., : d // 2] + 1j * x[..., d // 2:]
    freq = base ** (-np.arange(d // 2) * 2.0 / d)
    rot = z * np.exp(1j * pos[:, None, None] * freq[None, None, :])
    np.testing.assert_allclose(got, np.concatenate([rot.real, rot.imag], -1), atol=1e-10)
    np.testing.assert_allclose(O.rope(x, np.zeros(6), base, F64), x, atol=0)


def test_rope_relative_position():
    rng = np.random.default_rng(6)
    q, k = rng.normal(size=(1, 1, 16)), rng.normal(size=(1, 1, 16))
    dots = [float(np.sum(O.rope(q, [p + s], 10000.0, F64) * O.rope(k, [p - 5 + s], 10000.0, F64)))
            for p, s in [(10, 0), (10, 1000), (10, 200000)]]
    np.testing.assert_allclose(dots, dots[0], rtol=1e-9)


# ---------------------------------------------------------------------------------------
# fusion / injection


def test_fusion_norm_follows_projection():
    """W_c = 2 * I: RMSNorm(W_c x) is scale-free, so H_t has unit RMS rows and equals
    RMSNorm(x); normalising before the projection would give 2 * RMSNorm(x)."""
    D = 16
    sh = ModelShape(1, D, 2, 2, 8, 8, 10)
    x = np.random.default_rng(7).normal(size=(5, D))
    w = {"w_c": 2.0 * np.eye(D), "g_c": np.ones(D)}
    Ht = O.fuse(x, w, sh, F64)
    np.testing.assert_allclose(np.sqrt(np.mean(Ht ** 2, -1)), 1.0, atol=1e-6)
    np.testing.assert_allclose(Ht, x / np.sqrt(np.mean(x ** 2, -1, keepdims=True) + 1e-6), rtol=1e-6)


def test_inject_rows_independent_of_chunking():
    wl, dw, _, _ = _models(901)
    sh = wl.draft
    feats = np.random.default_rng(8).normal(size=(11, wl.n_taps * sh.hidden))
    pos = np.arange(11) + 37
    whole = O.inject(feats, pos, dw, sh, F64)
    parts = [O.inject(feats[a:b], pos[a:b], dw, sh, F64) for a, b in [(0, 3), (3, 4), (4, 11)]]
    for i in range(sh.n_layers):
        np.testing.assert_allclose(np.concatenate([p[i][0] for p in parts]), whole[i][0], atol=1e-12)
        np.testing.assert_allclose(np.concatenate([p[i][1] for p in parts]), whole[i][1], atol=1e-12)


def test_inject_identity_projections():
    """With W_c = I, W_K = W_V = I (D = Hkv*d), context K = RoPE(RMSNorm(x)), V = RMSNorm(x)."""
    sh = ModelShape(1, 16, 2, 2, 8, 8, 10)
    x = np.random.default_rng(9).normal(size=(4, 16))
    I = np.eye(16)
    w = {"w_c": I, "g_c": np.ones(16), "L0.wk": I, "L0.wv": I}
    K, V = O.inject(x, np.array([3, 4, 5, 6]), w, sh, F64)[0]
    xn = x / np.sqrt(np.mean(x ** 2, -1, keepdims=True) + 1e-6)
    np.testing.assert_allclose(V.reshape(4, 16), xn, rtol=1e-12)
    np.testing.assert_allclose(K, O.rope(xn.reshape(4, 2, 8), [3, 4, 5, 6], 10000.0, F64), rtol=1e-12)


def test_structural_sizes():
    g = json.load(open(os.path.join(GOLDEN, "p1_accounting.json")))["fusion_weight"]
    sh = ModelShape(1, g["hidden"], 16, 4, 128, 64, 8)
    wl = Workload(cid=902, name="wc", dtype="bf16", draft=sh, n_taps=g["n_taps"], block=16, batch=1,
                  ctx=(1,))
    w_c = synth.model_weights(wl, "draft")["w_c"]
    mb = w_c.numel() * g["bytes_per_element"] / 1e6
    assert abs(mb - g["approx_mb"]) < 0.5, mb
    # K/V injected per token per draft layer: Hkv*d each (262144 rows, 5 layers, bf16)
    # gives the ~5.4 GB of context quoted for the long-context drafter workload.
    q = synth.QWEN3_8B_DRAFT
    feats = np.zeros((1, 5 * q.hidden), dtype=np.float32)
    per_tok = q.n_layers * 2 * q.n_kv_heads * q.head_dim * 2
    assert abs(262144 * per_tok / 1e9 - 5.37) < 0.01
    del feats


# ---------------------------------------------------------------------------------------
# decoder layer / drafter


def _layer_inputs(seed, T=3, n=5, sh=TINY_SHAPE):
    rng = np.random.default_rng(seed)
    h = rng.normal(size=(T, sh.hidden))
    ck = rng.normal(size=(n, sh.n_kv_heads, sh.head_dim))
    cv = rng.normal(size=(n, sh.n_kv_heads, sh.head_dim))
    return h, ck, cv


def test_block_of_one_is_single_token_decode():
    """B = 1: bidirectional and causal block attention coincide, and equal a textbook
    single-query decode over [context; own key]."""
    _, dw, _, _ = _models(903)
    sh = TINY_SHAPE
    h, ck, cv = _layer_inputs(10, T=1, n=6)
    pos = np.array([6])
    a, _, _ = O.decoder_layer(h, dw, 0, sh, pos, ck, cv, causal=False, dt=F64)
    b, _, _ = O.decoder_layer(h, dw, 0, sh, pos, ck, cv, causal=True, dt=F64)
    np.testing.assert_allclose(a, b, atol=0)
    # textbook decode, written out with explicit loops
    eps, d, G = sh.rms_eps, sh.head_dim, sh.group
    u = h[0] / math.sqrt(np.mean(h[0] ** 2) + eps)
    q = O.rope((dw["L0.wq"] @ u).reshape(1, sh.n_q_heads, d), pos, sh.rope_base, F64)[0]
    k = O.rope((dw["L0.wk"] @ u).reshape(1, sh.n_kv_heads, d), pos, sh.rope_base, F64)[0]
    v = (dw["L0.wv"] @ u).reshape(sh.n_kv_heads, d)
    o = np.zeros((sh.n_q_heads, d))
    for j in range(sh.n_q_heads):
        kv = j // G
        keys = [ck[t, kv] for t in range(6)] + [k[kv]]
        vals = [cv[t, kv] for t in range(6)] + [v[kv]]
        s = [float(q[j] @ kk) / math.sqrt(d) for kk in keys]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        o[j] = sum(ei * vv for ei, vv in zip(e, vals)) / sum(e)
    x = h[0] + dw["L0.wo"] @ o.reshape(-1)
    u2 = x / math.sqrt(np.mean(x ** 2) + eps)
    gt, up = dw["L0.wg"] @ u2, dw["L0.wu"] @ u2
    x = x + dw["L0.wd"] @ (gt / (1 + np.exp(-gt)) * up)
    np.testing.assert_allclose(a[0], x, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_uniform_attention_is_mean_of_visible_values(causal):
    """W_q = 0 makes every score 0: each head's output is the plain mean of the values it
    may see - all n context rows plus all block rows (drafter) or block rows <= j
    (target).  With W_o = I (Hq*d = D), W_down = 0, the layer adds exactly that mean."""
    sh = ModelShape(1, 16, 2, 2, 8, 8, 10)
    rng = np.random.default_rng(11)
    T, n = 4, 3
    h, ck, cv = rng.normal(size=(T, 16)), rng.normal(size=(n, 2, 8)), rng.normal(size=(n, 2, 8))
    w = {"L0.g_in": np.ones(16), "L0.wq": np.zeros((16, 16)), "L0.wk": rng.normal(size=(16, 16)),
         "L0.wv": rng.normal(size=(16, 16)), "L0.wo": np.eye(16), "L0.g_post": np.ones(16),
         "L0.wg": rng.normal(size=(8, 16)), "L0.wu": rng.normal(size=(8, 16)),
         "L0.wd": np.zeros((16, 8))}
    out, _, vb = O.decoder_layer(h, w, 0, sh, np.arange(T) + n, ck, cv, causal, F64)
    for j in range(T):
        seen = np.concatenate([cv, vb[: j + 1] if causal else vb])
        np.testing.assert_allclose(out[j] - h[j], seen.mean(0).reshape(-1), atol=1e-12)


def test_mask_rows_identical_without_position_signal():
    """All mask rows share token and (here) position: under bidirectional attention their
    outputs coincide; under a causal mask they would not."""
    _, dw, _, sh_emb = _models(904)
    sh = TINY_SHAPE
    rng = np.random.default_rng(12)
    e = rng.normal(size=sh.hidden)
    h = np.stack([rng.normal(size=sh.hidden)] + [e] * 3)
    _, ck, cv = _layer_inputs(13, T=4, n=5)
    pos = np.full(4, 9)
    bi, _, _ = O.decoder_layer(h, dw, 0, sh, pos, ck, cv, causal=False, dt=F64)
    ca, _, _ = O.decoder_layer(h, dw, 0, sh, pos, ck, cv, causal=True, dt=F64)
    np.testing.assert_allclose(bi[2], bi[1], atol=1e-12)
    np.testing.assert_allclose(bi[3], bi[1], atol=1e-12)
    assert np.max(np.abs(ca[3] - ca[1])) > 1e-6


def test_draft_invariant_to_context_row_order():
    wl, dw, _, shw = _models(905)
    sh = wl.draft
    rng = np.random.default_rng(14)
    n = 9
    ctx = [(rng.normal(size=(n, sh.n_kv_heads, sh.head_dim)), rng.normal(size=(n, sh.n_kv_heads, sh.head_dim)))
           for _ in range(sh.n_layers)]
    perm = rng.permutation(n)
    ids, z, _ = O.draft_block(dw, shw, sh, ctx, 5, n, 4, F64)
    ids2, z2, _ = O.draft_block(dw, shw, sh, [(k[perm], v[perm]) for k, v in ctx], 5, n, 4, F64)
    np.testing.assert_allclose(z, z2, rtol=1e-10, atol=1e-12)
    assert np.array_equal(ids, ids2)


def test_draft_without_layers_is_embedding_logits():
    """Zero residual updates (W_o = W_down = 0): logits = RMSNorm(E[mask]) W_lm^T, and the
    drafts are its argmax at every mask position."""
    wl, dw, _, shw = _models(906)
    sh = wl.draft
    for i in range(sh.n_layers):
        dw[f"L{i}.wo"] = np.zeros_like(dw[f"L{i}.wo"])
        dw[f"L{i}.wd"] = np.zeros_like(dw[f"L{i}.wd"])
    ctx = [(np.zeros((3, 2, 8)), np.zeros((3, 2, 8)))] * sh.n_layers
    ids, z, hid = O.draft_block(dw, shw, sh, ctx, 7, 3, 4, F64)
    e = shw["embed"][sh.mask_token_id]
    want = (e / np.sqrt(np.mean(e ** 2) + 1e-6)) @ shw["lm_head"].T
    np.testing.assert_allclose(z, np.tile(want, (3, 1)), rtol=1e-10)
    assert list(ids) == [int(np.argmax(want))] * 3
    assert hid.shape == (sh.n_layers + 1, 4, sh.hidden)


# ---------------------------------------------------------------------------------------
# verify / accept / cycle


def test_verify_with_cache_equals_full_causal_forward():
    """KV-cache decoding is the full causal forward: logits of block row j computed against
    the cache equal those of a from-scratch causal pass over prompt + block."""
    wl, _, tw, shw = _models(907)
    sh = wl.target
    rng = np.random.default_rng(15)
    prompt = rng.integers(0, sh.vocab, size=7)
    block = rng.integers(0, sh.vocab, size=4)
    _, _, _, kv, _ = O.target_forward(tw, shw, sh, None, prompt, 0, (), F64)
    cache = O.append_kv(O.empty_cache(sh, F64), kv, 7)
    g, z, _, _, _ = O.verify(tw, shw, sh, cache, block, 7, (), F64)
    g2, z2, _, _, _ = O.target_forward(tw, shw, sh, None, np.concatenate([prompt, block]), 0, (), F64)
    np.testing.assert_allclose(z, z2[7:], rtol=1e-9, atol=1e-11)
    assert np.array_equal(g, g2[7:])


def test_accept_bruteforce():
    B = 4
    rng = np.random.default_rng(16)
    for _ in range(300):
        g = rng.integers(0, 3, size=B)
        d = rng.integers(0, 3, size=B - 1)
        a, tau, bonus = O.accept(d, g)
        mism = [j - 1 for j in range(1, B) if d[j - 1] != g[j - 1]]
        want_a = min(mism) if mism else B - 1
        assert (a, tau, bonus) == (want_a, want_a + 1, int(g[want_a]))
        assert 1 <= tau <= B
    g = rng.integers(0, 50, size=16)
    assert O.accept(g[:15], g)[1] == 16          # drafts forced to the target's choice


def test_tap_rule_matches_printed_layers():
    g = json.load(open(os.path.join(GOLDEN, "p1_accounting.json")))["gemma_tap_layers"]
    # six taps of a 48-layer model (the last printed tap is its third-to-last layer)
    assert O.tap_layers(48, 6) == tuple(g["layers"])
    assert O.tap_layers(8, 5) == synth.workload(5).taps
    assert O.tap_layers(2, 2) == synth.TINY.taps
    assert O.tap_layers(6, 2) == synth.MID.taps


@pytest.mark.parametrize("mode", ["drafter", "random", "forced", "mixed"])
def test_speculative_decoding_is_lossless(mode):
    """Whatever the drafts, the committed stream equals plain greedy decoding of the target
    (verify, accept, commit/rollback and the bonus token together)."""
    wl, dw, tw, shw = _models(908)
    tw = _scale_mats(tw, 8.0)           # sharper target logits: longer greedy runs
    dsh, tsh = wl.draft, wl.target
    prompt = np.random.default_rng(17).integers(0, tsh.vocab, size=6)
    n_new = 18
    ref = O.greedy_decode(tw, shw, tsh, prompt, n_new, F64)
    rng = np.random.default_rng(18)
    stream = [None]

    def override(cycle, anchor, drafts):
        if mode == "drafter":
            return drafts
        if mode == "random":
            return rng.integers(0, tsh.vocab, size=len(drafts))
        # forced: the reference continuation after the anchor's position
        pos = len(stream[0])
        want = ref[pos: pos + len(drafts)]
        want = list(want) + [0] * (len(drafts) - len(want))
        if mode == "mixed" and cycle % 2:
            want[min(1, len(want) - 1)] = (want[min(1, len(want) - 1)] + 1) % tsh.vocab
        return want

    # track how many tokens were emitted before each cycle, for the forced override
    class Tracker(list):
        pass

    emitted = Tracker()

    def wrapped(cycle, anchor, drafts):
        stream[0] = emitted
        out = override(cycle, anchor, drafts)
        return out

    # run cycle by cycle to keep `emitted` current
    tcache, dctx, anchor = O.prefill(tw, shw, tsh, dw, dsh, prompt, wl.taps, F64)
    n = len(prompt)
    out = [anchor]
    taus = []
    cycle = 0
    while len(out) < n_new:
        emitted[:] = out
        drafts, _, _ = O.draft_block(dw, shw, dsh, dctx, anchor, n, wl.block, F64)
        drafts = np.asarray(wrapped(cycle, anchor, drafts), dtype=np.int64)
        g, _, feats, kv, _ = O.verify(tw, shw, tsh, tcache, np.concatenate([[anchor], drafts]), n, wl.taps, F64)
        a, tau, bonus = O.accept(drafts, g)
        tcache, dctx = O.commit(tcache, dctx, kv, feats, tau, n, dw, dsh, F64)
        out += [int(t) for t in drafts[:a]] + [bonus]
        taus.append(tau)
        n += tau
        anchor = bonus
        cycle += 1
    assert out[:n_new] == ref
    if mode == "forced":
        assert all(t == wl.block for t in taus[:-1])
    # the packaged driver agrees
    got, _ = O.spec_decode(tw, dw, shw, tsh, dsh, prompt, n_new, wl.block, wl.taps, dt=F64)
    assert got == ref


def test_commit_keeps_accepted_rows_only():
    wl, dw, tw, shw = _models(909)
    dsh, tsh = wl.draft, wl.target
    prompt = np.arange(5)
    tcache, dctx, anchor = O.prefill(tw, shw, tsh, dw, dsh, prompt, wl.taps, F64)
    block = np.array([anchor, 1, 2, 3])
    g, _, feats, kv, _ = O.verify(tw, shw, tsh, tcache, block, 5, wl.taps, F64)
    for tau in (1, 2, 4):
        tc, dc = O.commit(tcache, dctx, kv, feats, tau, 5, dw, dsh, F64)
        assert all(k.shape[0] == 5 + tau for k, _ in tc)
        assert all(k.shape[0] == 5 + tau for k, _ in dc)
        inj = O.inject(feats[:tau], 5 + np.arange(tau), dw, dsh, F64)
        np.testing.assert_allclose(dc[0][0][5:], inj[0][0], atol=1e-12)
        np.testing.assert_allclose(tc[1][1][5:], kv[1][1][:tau], atol=0)


# ---------------------------------------------------------------------------------------
# accounting pinned by the printed measurements


def _taus_for(cycles, accepted, block):
    t = np.ones(cycles, dtype=np.int64)
    left, i = accepted, 0
    while left:
        add = min(block - 1, left)
        t[i] += add
        left -= add
        i += 1
    return t


def test_accounting_matches_printed_tables():
    g = json.load(open(os.path.join(GOLDEN, "p1_accounting.json")))
    B = g["n_max_4"]["drafts_per_cycle"] + 1
    for row in g["n_max_4"]["turns"]:
        assert row["generated"] % (B - 1) == 0            # B-1 drafts every cycle
        cycles = row["generated"] // (B - 1)
        st = O.cycle_stats(_taus_for(cycles, row["accepted"], B), B)
        assert st["generated"] == row["generated"]
        assert round(100 * st["acceptance"], 2) == row["acceptance_pct"]
        assert abs(st["tokens"] - row["table3_tokens"]) <= 1   # tokens = cycles + accepted
        assert abs(row["table3_tokens"] / (row["table3_ms"] / 1000) - row["table3_tps"]) < 0.01


def test_accounting_matches_printed_log():
    g = json.load(open(os.path.join(GOLDEN, "p1_accounting.json")))["n_max_15_log"]
    B = g["drafts_per_cycle"] + 1
    assert g["generated"] % (B - 1) == 0
    cycles = g["generated"] // (B - 1)
    taus = _taus_for(cycles, g["accepted"], B)
    st = O.cycle_stats(taus, B)
    assert round(st["acceptance"], 5) == g["acceptance"]
    assert round(st["mean_len"], 2) == g["mean_len"]
    # the log's token count adds the first token emitted by the prompt pass
    assert st["tokens"] + 1 == g["eval_tokens"]
    # latency identity: L = (T_draft + T_verify) / tau over the run
    per_cycle = np.full(cycles, g["eval_ms"] / cycles)
    L = O.latency_per_token(per_cycle, np.zeros(cycles), np.append(taus, 1))
    assert round(L, 2) == g["ms_per_token"]


def test_splitmix64_published_vectors():
    out, _ = synth.splitmix64(0)
    assert out == 0xE220A8397B1DCDAF
    s, got = 1234567, []
    for _ in range(3):
        o, s = synth.splitmix64(s)
        got.append(o)
    assert got == [6457827717110365317, 3203168211198807973, 9817491932198370423]


@pytest.mark.parametrize("p", [0.3, 0.7, 1.0])
def test_forcing_rule_gives_expected_tau(p):
    B, batch, cycles = 16, 8, 250
    rng = np.random.default_rng(19)
    taus = []
    for c in range(cycles):
        coins = synth.force_coins(123, c, batch, B, p)
        for b in range(batch):
            g = rng.integers(0, 100, size=B)
            own = rng.integers(0, 100, size=B - 1)
            d, f = synth.forced_drafts(coins[b], g, own, 100)
            a, tau, _ = O.accept(d, g)
            assert tau == f + 1
            taus.append(tau)
    mu = O.expected_tau_forced(p, B)
    sd = np.std(taus) / np.sqrt(len(taus))
    assert abs(np.mean(taus) - mu) <= 4 * sd + 1e-12


def test_anchor_row_sits_where_the_target_verifies_it():
    """A drafter whose one layer is the target's layer 0, fed the target's own layer-0 K/V
    through injection (W_c = I on the embedding rows, so H_t = RMSNorm(E[x]) = the layer's
    normed input), computes for the anchor (B = 1) exactly the target's hidden state at
    that position - which holds only if both place the anchor at position n."""
    sh = ModelShape(n_layers=1, hidden=32, n_q_heads=4, n_kv_heads=2, head_dim=8, ffn=48, vocab=64)
    wl = Workload(cid=910, name="anchorpos", dtype="f32", draft=sh, n_taps=1, block=1, batch=1,
                  ctx=(6,), target=sh, taps=(0,))
    tw = _np(synth.model_weights(wl, "target"))
    shw = _np(synth.shared_weights(wl))
    dw = dict(tw)
    dw["w_c"], dw["g_c"] = np.eye(32), np.ones(32)
    prompt = np.array([3, 9, 27, 1, 40, 5])
    _, _, _, kv, _ = O.target_forward(tw, shw, sh, None, prompt, 0, (), F64)
    cache = O.append_kv(O.empty_cache(sh, F64), kv, 6)
    ctx = O.inject(shw["embed"][prompt], np.arange(6), dw, sh, F64)
    np.testing.assert_allclose(ctx[0][0], cache[0][0], atol=1e-12)
    _, _, hid_d = O.draft_block(dw, shw, sh, ctx, 11, 6, 1, F64)
    _, _, _, _, hid_t = O.verify(tw, shw, sh, cache, [11], 6, (), F64)
    np.testing.assert_allclose(hid_d[1, 0], hid_t[1, 0], rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------------------------------
# storage type of the cache and of handed-over features (bfloat16 models)


def test_bf16_storage_rounding_matches_library_and_hand_values():
    import torch
    g = np.random.default_rng(5)
    x = np.concatenate([g.standard_normal(20000) * s for s in (1e-30, 1e-3, 1.0, 1e3, 1e30)])
    # exact halfway cases between neighbouring bfloat16 values, both parities
    base = g.standard_normal(2000).astype(np.float32)
    u = (base.view(np.uint32) & 0xFFFF0000) | 0x8000
    ties = u.view(np.float32)
    x = np.concatenate([x.astype(np.float32), ties])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = O.to_storage(x, "bf16")
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties go to the even mantissa (1);
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    hand = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 3.0, 1 + 2.0 ** -7], np.float32)
    assert O.to_storage(hand, "bf16").tolist() == [1.0, 1 + 2.0 ** -6, -1.0, 3.0, 1 + 2.0 ** -7]
    assert O.to_storage(hand, None) is hand and O.to_storage(hand, "f32") is hand


def test_bf16_storage_applies_to_cache_rows_and_taps():
    wl, dw, tw, sh = _models(931)
    feats = np.random.default_rng(1).standard_normal((6, 2 * TINY_SHAPE.hidden))
    raw = O.inject(feats, np.arange(6), dw, TINY_SHAPE, F64)
    st = O.inject(feats, np.arange(6), dw, TINY_SHAPE, F64, store="bf16")
    for (K, V), (Ks, Vs) in zip(raw, st):
        assert np.array_equal(Ks, O.to_storage(K, "bf16")) and np.array_equal(Vs, O.to_storage(V, "bf16"))
    g, z, f, new_kv, hid = O.target_forward(tw, sh, TINY_TGT, None, [3, 5, 7], 0, (0, 2), F64, store="bf16")
    assert np.array_equal(f, O.to_storage(np.concatenate([hid[1], hid[3]], axis=-1), "bf16"))
    for k, v in new_kv:
        assert np.array_equal(k, O.to_storage(k, "bf16")) and np.array_equal(v, O.to_storage(v, "bf16"))
    # only the storage differs: the first layer's queries see the same keys up to rounding
    g0, z0, f0, _, hid0 = O.target_forward(tw, sh, TINY_TGT, None, [3, 5, 7], 0, (0, 2), F64)
    assert np.array_equal(hid[0], hid0[0])
    assert 0 < np.max(np.abs(hid[1] - hid0[1])) < 1e-2 * np.max(np.abs(hid0[1]))


def test_drafter_block_keys_are_not_stored_but_verified_rows_are():
    """Storage rounding applies where a cache is written, nothing else.  The drafter's own
    block K/V live only for its pass ([DF] section 4.3: the draft block's keys are not part
    of the injected context), so with an empty context a bf16-storage drafter computes
    exactly what an unrounded one does; the target's verification pass writes the block
    into its cache, so its block rows attend to rounded keys and return rounded K/V."""
    wl, dw, tw, sh = _models(933)
    ids_r, z_r, hid_r = O.draft_block(dw, sh, TINY_SHAPE, None, 5, 0, 4, F64, store="bf16")
    ids_p, z_p, hid_p = O.draft_block(dw, sh, TINY_SHAPE, None, 5, 0, 4, F64)
    assert np.array_equal(z_r, z_p) and np.array_equal(hid_r, hid_p)
    # a plain decoder layer call: the non-causal (drafter) pass returns unrounded rows
    h = np.asarray(sh["embed"], dtype=F64)[[5, 9, 9, 9]]
    _, kb, vb = O.decoder_layer(h, dw, 0, TINY_SHAPE, np.arange(4), None, None, False, F64, "bf16")
    assert not np.array_equal(kb, O.to_storage(kb, "bf16"))
    _, kb, vb = O.decoder_layer(h, dw, 0, TINY_SHAPE, np.arange(4), None, None, True, F64, "bf16")
    assert np.array_equal(kb, O.to_storage(kb, "bf16")) and np.array_equal(vb, O.to_storage(vb, "bf16"))
