"""CPU oracle for the DFlash drafter step and greedy block verification.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or execute
this module: only the tests, the smoke check and the bench's CPU-baseline leg use it.
It shares no code with the HIP library; it only reads the same seeded inputs.

Pages cited (by title, then section / equation / figure):
  [DF]   "DFlash - Block Diffusion for Flash Speculative Decoding" (paper notes page)
  [TRY]  "Trying "DFlash," a Diffusion-Model Approach to Parallel Draft-Token
         Generation, on Gemma" (llama.cpp experiment write-up)
  [LCPP] llama.cpp discussion "DFlash (Block Diffusion for Flash Speculative Decoding)"

Everything is computed one sequence at a time in a plain float dtype (float32 by
default; the pin tests also run it in float64), straight from the definitions, with
no blocking, fusion or reordering.  Readings taken where the pages are silent are
listed beside the function that takes them.

Storage type (reading): the models the pages measure are held in bfloat16, so the
buffers that carry values between passes - the K/V caches and the tapped features the
target hands to the drafter - hold bfloat16 values for such a model.  With
``store="bf16"`` K/V are rounded to bfloat16 (nearest, ties to even) where they are
written into a cache (the drafter's context by injection, the target's cache by the
verification pass, whose block rows then attend to their own keys as stored) and tapped
features are rounded where they are handed over.  The drafter's own block K/V live only
for its pass and are never stored, so they are not rounded.  All arithmetic stays in the
working float type.  ``store=None`` (float32 models) rounds nothing.

Conventions: a model's weights are a dict (keys as produced by ``synth.model_weights``),
matrices row-major [out, in]; ``shape`` is a ``synth.ModelShape``; a KV cache is a list
over layers of ``(K, V)`` with ``K, V`` of shape [n, H_kv, d] (K stored after RoPE).
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------------------
# Building blocks


def to_storage(x, store):
    """x as held in a buffer of storage type `store`: rounded to the nearest bfloat16
    (ties to even) for "bf16", unchanged for None / "f32".  Finite inputs only."""
    if store in (None, "f32"):
        return x
    assert store == "bf16", store
    x = np.asarray(x)
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(x.dtype)


def rmsnorm(x, g, eps, dt=np.float32):
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * g.  eps = 1e-6 everywhere
    (the pages give no value; the Qwen3-8B-shaped configuration states 1e-6)."""
    x = np.asarray(x, dtype=dt)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return (x / np.sqrt(ms + dt(eps))) * np.asarray(g, dtype=dt)


def silu(x):
    return x / (1.0 + np.exp(-x))


def rope_cos_sin(pos, d, base):
    """Rotary angles p * base^(-2i/d), i < d/2, evaluated in float64 (reading: at
    positions near 2.6e5 a float32 product p*theta errs by ~1e-2 rad)."""
    i = np.arange(d // 2, dtype=np.float64)
    theta = np.power(np.float64(base), -2.0 * i / d)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * theta[None, :]
    return np.cos(ang), np.sin(ang)


def rope(x, pos, base, dt=np.float32):
    """Rotate-half RoPE on x [T, H, d] at positions pos [T]: the pair (i, i + d/2) is
    rotated by angle p * theta_i (reading: the pages name no convention)."""
    x = np.asarray(x, dtype=dt)
    d = x.shape[-1]
    c, s = rope_cos_sin(pos, d, base)
    c = c.astype(dt)[:, None, :]
    s = s.astype(dt)[:, None, :]
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def attention(q, k, v, visible, dt=np.float32):
    """softmax(q k^T / sqrt(d) restricted to visible keys) v.
    q [Tq, d], k [Tk, d], v [Tk, d], visible bool [Tq, Tk]."""
    q = np.asarray(q, dtype=dt)
    k = np.asarray(k, dtype=dt)
    v = np.asarray(v, dtype=dt)
    s = (q @ k.T) / dt(np.sqrt(q.shape[-1]))
    s = np.where(visible, s, -np.inf)
    s = s - np.max(s, axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / np.sum(p, axis=-1, keepdims=True)
    return p @ v


def argmax_lowest(z):
    """Argmax along the last axis; ties go to the lowest index (reading: the pages do not
    say; numpy's first-occurrence rule)."""
    return np.argmax(z, axis=-1).astype(np.int64)


def top2_gap(z):
    """z_(1) - z_(2) along the last axis (used to exclude near-tie positions)."""
    part = np.partition(z, -2, axis=-1)
    return part[..., -1] - part[..., -2]


# ----------------------------------------------------------------------------------------
# Feature fusion and KV injection  [DF §4.2 fusion equation, §4.3 injection equations]


def tap_layers(n_layers, k):
    """0-indexed target layers whose outputs are tapped: k layers spread uniformly from
    the second layer to the third-to-last one ([DF §6.1]: "uniformly sampled between
    layer 2 and third-to-last"; the Gemma tap list printed in [TRY]'s appendix follows
    the same spacing).  When the range is empty (a 2-layer toy target) every layer
    is tapped in order."""
    lo, hi = 1, n_layers - 3
    if hi < lo or hi - lo + 1 < k:
        return tuple(range(min(k, n_layers)))
    return tuple(int(x) for x in np.round(np.linspace(lo, hi, k)))


def fuse(feats, w, shape, dt=np.float32):
    """H_t = RMSNorm(W_c [H^(l1); ...; H^(lk)]) for rows of concatenated tapped features
    [r, k*D] -> [r, D].  The norm follows the projection [DF §4.2] (the appendix of [TRY]
    mentions normalisation before injection without its order; [DF] is followed)."""
    x = np.asarray(feats, dtype=dt) @ np.asarray(w["w_c"], dtype=dt).T
    return rmsnorm(x, w["g_c"], shape.rms_eps, dt)


def inject(feats, positions, w, shape, dt=np.float32, store=None):
    """Context K/V for every draft layer from tapped features [DF §4.3]:
    K_i = RoPE(W_i^K H_t) at each row's absolute position, V_i = W_i^V H_t.
    Returns a list over draft layers of (K [r, Hkv, d], V [r, Hkv, d]) as stored.
    Reading: K is rotated at its own position and stored rotated."""
    Ht = fuse(feats, w, shape, dt)
    r = Ht.shape[0]
    out = []
    for i in range(shape.n_layers):
        K = (Ht @ np.asarray(w[f"L{i}.wk"], dtype=dt).T).reshape(r, shape.n_kv_heads, shape.head_dim)
        V = (Ht @ np.asarray(w[f"L{i}.wv"], dtype=dt).T).reshape(r, shape.n_kv_heads, shape.head_dim)
        out.append((to_storage(rope(K, positions, shape.rope_base, dt), store), to_storage(V, store)))
    return out


# ----------------------------------------------------------------------------------------
# Decoder layer shared by the drafter (bidirectional block) and the target (causal block)


# DFlash 2 two-tap dynamic convolution  [DF §7.1, "Problem 2: Suffix Decay"]: a depthwise
# convolution reaching one position back, Conv(x)_t = k_{t,0} * x_t + k_{t,1} * x_{t-1},
# inserted before and after each attention and feed-forward sublayer; each coefficient is a
# learned base kernel plus a content-dependent correction; the first position reads the last
# verified token and every later one its predecessor.  Readings (the page gives the formula,
# the placement and the parameter count, 16.5M for the 5-layer Qwen3.5-4B drafter):
#   * placement: inside each sublayer's branch - on the normalised input (after the
#     sublayer's RMSNorm, "before") and on the sublayer's output (before the residual add,
#     "after"): h <- h + Conv_post(Sub(Conv_pre(RMSNorm(h))));
#   * correction: linear in the convolution's own input x_t, one coefficient per tap per
#     group of 16 channels: k_{t,j}[c] = base_j[c] + (x_t W_k)[2 (c // 16) + j], W_k [D, D/8]
#     (columns interleave the taps of each group).  Per convolution 2D + D * D/8 parameters:
#     for D = 2560 and 4 convolutions in each of 5 layers, 20 x 824,320 = 16.49M - the page's
#     16.5M;
#   * the block's first row is the anchor, the last verified token; it reads itself
#     (x_{-1} = x_0), every later row its predecessor.


def dconv(x, base, w_k, dt=np.float32):
    """Two-tap dynamic convolution of the block rows x [T, D] (readings above).  base [2, D],
    w_k [D, D/8]."""
    x = np.asarray(x, dtype=dt)
    T, D = x.shape
    corr = x @ np.asarray(w_k, dtype=dt)                 # [T, 2 * D/16]
    grp = np.arange(D) // 16
    k0 = np.asarray(base[0], dtype=dt)[None, :] + corr[:, 2 * grp]
    k1 = np.asarray(base[1], dtype=dt)[None, :] + corr[:, 2 * grp + 1]
    prev = np.concatenate([x[:1], x[:-1]], axis=0)      # row 0 reads itself
    return k0 * x + k1 * prev


def _conv(w, i, which, x, dt):
    key = f"L{i}.dconv_{which}"
    if key + ".base" not in w:
        return x
    return dconv(x, w[key + ".base"], w[key + ".w_k"], dt)


def decoder_layer(h, w, i, shape, positions, ctx_k, ctx_v, causal, dt=np.float32, store=None):
    """One pre-norm decoder layer over the block rows h [T, D].

    The block's queries attend to the n context keys (all visible) followed by the
    block's own T keys: all of them for the drafter (non-causal, [TRY] appendix;
    masked-diffusion block), keys j' <= j for the target's verification pass
    ([TRY] Fig. 1, causal attention in the main model).  The context rows take no part
    in Q, O, the residual or the FFN ([DF §4.3]).  FFN: SwiGLU (the drafter is
    described as Qwen-style in [TRY]'s appendix).  The verification pass writes the
    block's K/V into the target's cache, so there they enter attention as stored
    (`store`); the drafter's block K/V are never stored ([DF §4.3]: the draft block's
    keys are not part of the injected context) and enter unrounded.  The returned k_blk,
    v_blk are the stored rows when causal.  A DFlash 2 drafter's weights may hold the two-tap convolutions
    (keys L{i}.dconv_{pre_attn,post_attn,pre_ffn,post_ffn}.{base,w_k}).  Returns (h_out,
    k_blk, v_blk)."""
    T = h.shape[0]
    Hq, Hkv, d = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    G = Hq // Hkv
    u = _conv(w, i, "pre_attn", rmsnorm(h, w[f"L{i}.g_in"], shape.rms_eps, dt), dt)
    q = (u @ np.asarray(w[f"L{i}.wq"], dtype=dt).T).reshape(T, Hq, d)
    kb = (u @ np.asarray(w[f"L{i}.wk"], dtype=dt).T).reshape(T, Hkv, d)
    vb = (u @ np.asarray(w[f"L{i}.wv"], dtype=dt).T).reshape(T, Hkv, d)
    q = rope(q, positions, shape.rope_base, dt)
    kb = rope(kb, positions, shape.rope_base, dt)
    if causal:   # written into the target's cache
        kb, vb = to_storage(kb, store), to_storage(vb, store)

    n = 0 if ctx_k is None else ctx_k.shape[0]
    visible = np.ones((T, n + T), dtype=bool)
    if causal:
        visible[:, n:] = np.tril(np.ones((T, T), dtype=bool))
    o = np.empty((T, Hq, d), dtype=dt)
    for kv in range(Hkv):
        if n:
            Kh = np.concatenate([np.asarray(ctx_k[:, kv, :], dtype=dt), kb[:, kv, :]], axis=0)
            Vh = np.concatenate([np.asarray(ctx_v[:, kv, :], dtype=dt), vb[:, kv, :]], axis=0)
        else:
            Kh, Vh = kb[:, kv, :], vb[:, kv, :]
        for j in range(kv * G, (kv + 1) * G):
            o[:, j, :] = attention(q[:, j, :], Kh, Vh, visible, dt)
    h = h + _conv(w, i, "post_attn", o.reshape(T, Hq * d) @ np.asarray(w[f"L{i}.wo"], dtype=dt).T, dt)
    u = _conv(w, i, "pre_ffn", rmsnorm(h, w[f"L{i}.g_post"], shape.rms_eps, dt), dt)
    a = silu(u @ np.asarray(w[f"L{i}.wg"], dtype=dt).T) * (u @ np.asarray(w[f"L{i}.wu"], dtype=dt).T)
    h = h + _conv(w, i, "post_ffn", a @ np.asarray(w[f"L{i}.wd"], dtype=dt).T, dt)
    return h, kb, vb


def lm_logits(h, w, shared, shape, dt=np.float32):
    """Final RMSNorm then the shared LM head [DF §5.2: embedding and LM head shared with
    the target]; logits stay in the working float type."""
    return rmsnorm(h, w["g_f"], shape.rms_eps, dt) @ np.asarray(shared["lm_head"], dtype=dt).T


# ----------------------------------------------------------------------------------------
# Drafter step  [DF §4.4 parallel drafting; §3.2 one forward pass for the whole block]


def draft_block(w, shared, shape, ctx, anchor, n, block, dt=np.float32, store=None):
    """One drafter forward pass over [anchor, MASK x (B-1)] at positions n .. n+B-1.

    ctx: list over draft layers of (K [n, Hkv, d], V [n, Hkv, d]) - the injected context.
    Each mask position is decoded independently by argmax of its logits ([DF §4.4],
    greedy).  Returns (draft_ids [B-1], logits [B-1, V], hiddens [L+1, B, D]).
    Readings: the anchor sits at position n, where the target later verifies it; no
    timestep input ([DF §4.4], single step); the mask token is the last vocab row."""
    tokens = np.array([anchor] + [shape.mask_token_id] * (block - 1), dtype=np.int64)
    positions = n + np.arange(block)
    h = np.asarray(shared["embed"], dtype=dt)[tokens]
    hiddens = [h]
    for i in range(shape.n_layers):
        ck, cv = ctx[i] if n else (None, None)
        if ck is not None:
            ck, cv = ck[:n], cv[:n]
        h, _, _ = decoder_layer(h, w, i, shape, positions, ck, cv, causal=False, dt=dt, store=store)
        hiddens.append(h)
    z = lm_logits(h[1:], w, shared, shape, dt)
    return argmax_lowest(z), z, np.stack(hiddens)


# ----------------------------------------------------------------------------------------
# Target verification, acceptance, commit  [DF §4.5 decoding cycle]


def target_forward(w, shared, shape, cache, tokens, n, taps, dt=np.float32, store=None):
    """Causal target pass over `tokens` at positions n .. n+T-1 with the first n cache rows
    visible.  Returns (g [T] greedy ids, logits [T, V], feats [T, k*D] = the tapped layer
    outputs concatenated in tap order, new_kv list of (K [T,Hkv,d], V [T,Hkv,d]),
    hiddens [L+1, T, D]).  A tap is the output of the whole decoder layer (after both
    residual adds, before the final norm) - reading; feats and new_kv are as stored."""
    tokens = np.asarray(tokens, dtype=np.int64)
    T = tokens.shape[0]
    positions = n + np.arange(T)
    h = np.asarray(shared["embed"], dtype=dt)[tokens]
    hiddens = [h]
    tapped = {}
    new_kv = []
    for i in range(shape.n_layers):
        if n and cache is not None:
            ck, cv = cache[i][0][:n], cache[i][1][:n]
        else:
            ck, cv = None, None
        h, kb, vb = decoder_layer(h, w, i, shape, positions, ck, cv, causal=True, dt=dt, store=store)
        new_kv.append((kb, vb))
        hiddens.append(h)
        if i in taps:
            tapped[i] = h
    feats = to_storage(np.concatenate([tapped[t] for t in taps], axis=-1), store) if taps else None
    z = lm_logits(h, w, shared, shape, dt)
    return argmax_lowest(z), z, feats, new_kv, np.stack(hiddens)


def verify(w, shared, shape, cache, block_ids, n, taps, dt=np.float32, store=None):
    """Verification of y = [x, d_1 .. d_{B-1}] in one causal target pass [DF §4.5 step 2]."""
    return target_forward(w, shared, shape, cache, block_ids, n, taps, dt, store)


def accept(draft_ids, g):
    """Greedy longest-prefix acceptance [DF §4.5 step 3]: accept d_j while d_j equals the
    target's greedy choice g_{j-1}; a = number accepted, tau = a + 1 (tau counts the bonus
    token, [DF §2.2]), bonus = g_a.  Returns (a, tau, bonus)."""
    a = 0
    for j in range(1, len(draft_ids) + 1):
        if int(draft_ids[j - 1]) != int(g[j - 1]):
            break
        a = j
    return a, a + 1, int(g[a])


def append_kv(cache, new_kv, count):
    """Cache after appending the first `count` rows of new_kv to every layer."""
    out = []
    for (K, V), (k, v) in zip(cache, new_kv):
        out.append((np.concatenate([K, k[:count]], axis=0), np.concatenate([V, v[:count]], axis=0)))
    return out


def commit(target_cache, draft_ctx, new_kv, feats, tau, n, draft_w, draft_shape, dt=np.float32,
           store=None):
    """Commit/rollback [DF §4.5]: the target keeps rows n .. n+tau-1 (anchor and accepted
    drafts) and drops the rest; the drafter's context receives the injected features of
    the same rows at their positions ([TRY]: the drafter's own KV cache is fed by
    injection from the main model's pass).  Returns (target_cache, draft_ctx)."""
    target_cache = append_kv(target_cache, new_kv, tau)
    inj = inject(feats[:tau], n + np.arange(tau), draft_w, draft_shape, dt, store)
    draft_ctx = append_kv(draft_ctx, inj, tau)
    return target_cache, draft_ctx


def empty_cache(shape, dt=np.float32):
    z = np.zeros((0, shape.n_kv_heads, shape.head_dim), dtype=dt)
    return [(z, z) for _ in range(shape.n_layers)]


def prefill(target_w, shared, tshape, draft_w, dshape, prompt, taps, dt=np.float32, store=None):
    """Causal target pass over the prompt from an empty cache; the drafter's context is
    injected from the prompt's tapped features; the first anchor is the greedy token at
    the last prompt row.  Returns (target_cache, draft_ctx, anchor)."""
    n = len(prompt)
    g, _, feats, new_kv, _ = target_forward(target_w, shared, tshape, None, prompt, 0, taps, dt, store)
    tcache = append_kv(empty_cache(tshape, dt), new_kv, n)
    dctx = inject(feats, np.arange(n), draft_w, dshape, dt, store)
    return tcache, dctx, int(g[-1])


def greedy_decode(target_w, shared, tshape, prompt, n_new, dt=np.float32, store=None):
    """Plain autoregressive greedy decoding with the target ([DF §1]); the reference that
    speculative decoding must reproduce exactly ([DF §4.5] lossless guarantee)."""
    prompt = list(int(t) for t in prompt)
    g, _, _, new_kv, _ = target_forward(target_w, shared, tshape, None, prompt, 0, (), dt, store)
    cache = append_kv(empty_cache(tshape, dt), new_kv, len(prompt))
    out = [int(g[-1])]
    n = len(prompt)
    while len(out) < n_new:
        g, _, _, new_kv, _ = target_forward(target_w, shared, tshape, cache, [out[-1]], n, (), dt, store)
        cache = append_kv(cache, new_kv, 1)
        n += 1
        out.append(int(g[0]))
    return out[:n_new]


def spec_decode(target_w, draft_w, shared, tshape, dshape, prompt, n_new, block, taps,
                draft_override=None, dt=np.float32, store=None):
    """Speculative decoding cycles [DF §4.5]: draft a block, verify it, accept the longest
    matching prefix plus the bonus token, commit, repeat.  `draft_override(cycle, anchor,
    drafts)` may replace the drafter's ids (random or forced drafts) - the emitted stream
    must not depend on it.  Returns (tokens [n_new], taus)."""
    tcache, dctx, anchor = prefill(target_w, shared, tshape, draft_w, dshape, prompt, taps, dt, store)
    n = len(prompt)
    out = [anchor]
    taus = []
    cycle = 0
    while len(out) < n_new:
        drafts, _, _ = draft_block(draft_w, shared, dshape, dctx, anchor, n, block, dt, store)
        if draft_override is not None:
            drafts = np.asarray(draft_override(cycle, anchor, drafts), dtype=np.int64)
        block_ids = np.concatenate([[anchor], drafts])
        g, _, feats, new_kv, _ = verify(target_w, shared, tshape, tcache, block_ids, n, taps, dt, store)
        a, tau, bonus = accept(drafts, g)
        tcache, dctx = commit(tcache, dctx, new_kv, feats, tau, n, draft_w, dshape, dt, store)
        out.extend(int(t) for t in drafts[:a])
        out.append(bonus)
        taus.append(tau)
        n += tau
        anchor = bonus
        cycle += 1
    return out[:n_new], taus


# ----------------------------------------------------------------------------------------
# Temperature sampling and lossless rejection-sampling verification  [DF §6.2: sampling at
# temperature 1 keeps the method lossless; the DFlash 2 notes (§7.2) name "lossless rejection
# sampling" as the verifier under sampling].  The pages give no further detail, so the
# readings are the standard speculative-sampling rule:
#   * the drafter samples each masked position i independently from q_i = softmax(z^d_i / T);
#   * the target's row j gives p_j = softmax(z^t_j / T) for the token at position j+1, so draft
#     d_i is checked against p_{i-1}: accepted when u_i < p_{i-1}(d_i) / q_i(d_i);
#   * at the first rejection i the cycle emits a token drawn from norm(max(0, p_{i-1} - q_i));
#     when all B-1 drafts pass it emits a token drawn from p_{B-1};
#   * tau = accepted + 1 as in the greedy rule; the emitted token is the next anchor.
# Random numbers come from a counter-based generator (splitmix64, Vigna's published mixing
# function over a Weyl sequence): stream number `index` of seed s is mix(s + (index + 1) *
# 0x9E3779B97F4A7C15), index = (((counter * 4 + purpose) * 4096 + b) * 128 + i) * 262144 + v.
# A uniform in (0, 1) takes the top 23 bits: u = ((r >> 41) + 0.5) / 2^23, exact in float32
# (24 significant bits) and strictly inside (0, 1), so -log(-log(u)) is always finite.
# Purposes: 0 = drafter Gumbel noise (b, position i, vocab id v), 1 = acceptance uniforms
# (b, position i, v = 0), 2 = Gumbel noise of the emitted token (b, target row, v).  Sampling
# from softmax(x) is argmax(x + G) with G = -log(-log(u)) (the Gumbel-max identity), keys
# formed in float32 as the kernels do: x = float32(z) / float32(T).

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)


def splitmix64_mix(z):
    """Vigna's splitmix64 output function on uint64 arrays."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def rng_index(counter, purpose, b, i, v):
    """64-bit stream index of draw (counter, purpose, b, i, v) - fields of 25, 2, 12, 7 and 18
    bits (v < 262144 covers every vocabulary here)."""
    with np.errstate(over="ignore"):
        c = np.uint64(counter) * np.uint64(4) + np.uint64(purpose)
        c = c * np.uint64(4096) + np.uint64(b)
        c = c * np.uint64(128) + np.uint64(i)
        return c * np.uint64(262144) + np.asarray(v, dtype=np.uint64)


def uniform01(seed, counter, purpose, b, i, v):
    """Counter-based uniforms in (0, 1), float32 (23 random bits), for an array of vocab ids v."""
    with np.errstate(over="ignore"):
        st = np.uint64(seed) + (rng_index(counter, purpose, b, i, v) + np.uint64(1)) * _GOLDEN
    r = splitmix64_mix(st)
    return ((r >> np.uint64(41)).astype(np.float32) + np.float32(0.5)) * np.float32(2.0 ** -23)


def gumbel(seed, counter, purpose, b, i, v):
    u = uniform01(seed, counter, purpose, b, i, v)
    return -np.log(-np.log(u))   # float32 throughout


def sample_keys(z, temperature, seed, counter, purpose, b, i):
    """float32 keys z / T + G of one logits row; their argmax (lowest index on ties) is a
    sample of softmax(z / T)."""
    z = np.asarray(z, dtype=np.float32)
    v = np.arange(z.shape[-1])
    return z / np.float32(temperature) + gumbel(seed, counter, purpose, b, i, v)


def log_softmax_t(z, temperature):
    """log softmax(z / T) in float64."""
    x = np.asarray(z, dtype=np.float64) / float(temperature)
    m = np.max(x, axis=-1, keepdims=True)
    return x - (m + np.log(np.sum(np.exp(x - m), axis=-1, keepdims=True)))


def draft_block_sampled(w, shared, shape, ctx, anchor, n, block, temperature, seed, counter, b=0,
                        dt=np.float32, store=None):
    """The drafter pass of draft_block, with each masked position i = 1 .. B-1 sampled from
    softmax(z_i / T) by the Gumbel-max identity (purpose 0, position i).  Returns
    (draft_ids [B-1], logits [B-1, V], keys [B-1, V])."""
    _, z, _ = draft_block(w, shared, shape, ctx, anchor, n, block, dt, store)
    keys = np.stack([sample_keys(z[i - 1], temperature, seed, counter, 0, b, i) for i in range(1, block)]) \
        if block > 1 else np.zeros((0, z.shape[-1]), np.float32)
    return argmax_lowest(keys), z, keys


def accept_sampled(draft_ids, draft_logits, target_logits, temperature, seed, counter, b=0):
    """Speculative-sampling acceptance of one block (readings above).  draft_ids [B-1],
    draft_logits [B-1, V] (rows for positions 1 .. B-1), target_logits [B, V].  Returns
    (a, tau, token, ratios [B-1], uniforms [B-1], keys of the emitted token's draw [V])."""
    B = target_logits.shape[0]
    lp = log_softmax_t(target_logits, temperature)
    lq = log_softmax_t(draft_logits, temperature) if B > 1 else np.zeros((0, lp.shape[-1]))
    ratios = np.zeros(B - 1)
    us = np.zeros(B - 1)
    a = 0
    rejected = False
    for i in range(1, B):
        d = int(draft_ids[i - 1])
        ratios[i - 1] = np.exp(lp[i - 1, d] - lq[i - 1, d])
        us[i - 1] = float(uniform01(seed, counter, 1, b, i, 0))
        if not rejected and us[i - 1] < ratios[i - 1]:
            a = i
        else:
            rejected = True
    v = np.arange(lp.shape[-1])
    g = gumbel(seed, counter, 2, b, a, v).astype(np.float64)
    if a < B - 1:   # residual norm(max(0, p_a - q_{a+1})): the normaliser does not move the argmax
        res = np.exp(lp[a]) - np.exp(lq[a])
        with np.errstate(divide="ignore"):
            keys = np.where(res > 0, np.log(np.maximum(res, 1e-300)), -np.inf) + g
    else:
        keys = lp[a] + g
    return a, a + 1, int(argmax_lowest(keys)), ratios, us, keys


def spec_decode_sampled(target_w, draft_w, shared, tshape, dshape, prompt, n_new, block, taps,
                        temperature, seed, dt=np.float32, store=None):
    """Sampling speculative decoding: drafter sampling, rejection verification, commit.
    The first token after the prompt is drawn from the target at the prompt's last row
    (purpose 2, row 0 of counter 0); cycle c uses counter c + 1.  Returns (tokens, taus)."""
    prompt = np.asarray(prompt, dtype=np.int64)
    _, z, feats, new_kv, _ = target_forward(target_w, shared, tshape, None, prompt, 0, taps, dt, store)
    n = len(prompt)
    tcache = append_kv(empty_cache(tshape, dt), new_kv, n)
    dctx = inject(feats, np.arange(n), draft_w, dshape, dt, store)
    lp = log_softmax_t(z[-1:], temperature)[0]
    anchor = int(argmax_lowest(lp + gumbel(seed, 0, 2, 0, 0, np.arange(lp.shape[-1])).astype(np.float64)))
    out = [anchor]
    taus = []
    counter = 1
    while len(out) < n_new:
        drafts, zd, _ = draft_block_sampled(draft_w, shared, dshape, dctx, anchor, n, block,
                                            temperature, seed, counter, 0, dt, store)
        block_ids = np.concatenate([[anchor], drafts])
        _, zt, feats, new_kv, _ = verify(target_w, shared, tshape, tcache, block_ids, n, taps, dt, store)
        a, tau, tok, _, _, _ = accept_sampled(drafts, zd, zt, temperature, seed, counter, 0)
        tcache, dctx = commit(tcache, dctx, new_kv, feats, tau, n, draft_w, dshape, dt, store)
        out.extend(int(t) for t in drafts[:a])
        out.append(tok)
        taus.append(tau)
        n += tau
        anchor = tok
        counter += 1
    return out[:n_new], taus


# ----------------------------------------------------------------------------------------
# Accounting  [DF §2.2 latency model; [TRY] acceptance tables and log lines]


def cycle_stats(taus, block):
    """Counters of a run of cycles: every cycle proposes B-1 drafts; accepted = sum(tau-1);
    tokens emitted = sum(tau) = cycles + accepted; acceptance = accepted / generated;
    mean accepted length = tokens / cycles."""
    taus = np.asarray(taus, dtype=np.int64)
    cycles = int(taus.size)
    accepted = int(np.sum(taus - 1))
    generated = cycles * (block - 1)
    tokens = cycles + accepted
    return {
        "cycles": cycles,
        "generated": generated,
        "accepted": accepted,
        "tokens": tokens,
        "acceptance": accepted / generated if generated else 0.0,
        "mean_len": tokens / cycles if cycles else 0.0,
    }


def latency_per_token(t_draft, t_verify, taus):
    """L = (T_draft + T_verify) / tau as a ratio of sums over cycles [DF §2.2]."""
    return (float(np.sum(t_draft)) + float(np.sum(t_verify))) / float(np.sum(taus))


def expected_tau_forced(p, block):
    """Mean tau when each draft position is independently forced to the target's choice
    with probability p and the first unforced position is made to differ:
    tau = 1 + (length of the leading run of forced positions)."""
    return 1.0 + sum(p ** k for k in range(1, block))


# ----------------------------------------------------------------------------------------
# DFlash 2 path selector  [DF §7.1, "Problem 1: Selection Headroom"]: the top-16 candidates
# of each masked position are kept and every adjacent pair (predecessor a, candidate b) is
# scored S_t(a, b) = U_t(b) + <A(a) * H(h_t), B(b)>, U_t(b) the drafter's own logit and
# A, B, H 256-dimensional projections; a greedy walk over the scores picks the drafts.
# The page names the pieces but not their inputs, so the readings are:
#   * A(a) = E[a] W_A and B(b) = E[b] W_B with E the shared token embedding, H(h) = h W_H
#     with h the drafter's final hidden state after the final RMSNorm (the LM head's
#     input); W_A, W_B, W_H are [D, 256] (for a 2560-wide 4B drafter, 3 x 2560 x 256 =
#     1.97M parameters - the page's 2.0M);
#   * U_t(b) is the raw logit z_t(b);
#   * the walk starts at the anchor (the last verified token): position 1's predecessor is
#     the anchor, position t's is the candidate chosen at t - 1;
#   * candidates are the top_k logits of a position, ties to the lower id; the walk's ties
#     go to the lower id as well.


def topk_lowest(z, k):
    """Ids of the k largest entries of each row of z, in descending value, ties to the lower
    id."""
    z = np.asarray(z)
    if z.ndim == 1:
        return topk_lowest(z[None], k)[0]
    ids = np.broadcast_to(np.arange(z.shape[-1]), z.shape)
    return np.lexsort((ids, -z), axis=-1)[:, :k]


def select_path(z, h_final, anchor, embed, g_f, eps, w_a, w_b, w_h, top_k=16, dt=np.float32):
    """Greedy path selection over a drafted block [DF §7.1].

    z: drafter logits of the masked positions [B-1, V]; h_final: the drafter's final hidden
    states of those positions before the final norm [B-1, D]; anchor: the block's first
    token.  Returns (draft_ids [B-1], candidates [B-1, top_k], scores [B-1, top_k] of the
    chosen predecessor's row at each position)."""
    z = np.asarray(z, dtype=dt)
    E = np.asarray(embed, dtype=dt)
    cand = topk_lowest(z, top_k)
    hh = rmsnorm(np.asarray(h_final, dtype=dt), g_f, eps, dt) @ np.asarray(w_h, dtype=dt)
    wa = np.asarray(w_a, dtype=dt)
    wb = np.asarray(w_b, dtype=dt)
    prev = int(anchor)
    out, rows = [], []
    for t in range(z.shape[0]):
        a_vec = E[prev] @ wa                               # A(a)
        b_vec = E[cand[t]] @ wb                            # B(b) for every candidate b
        s = z[t, cand[t]] + b_vec @ (a_vec * hh[t])        # S_t(a, b)
        best = max(range(top_k), key=lambda j: (s[j], -int(cand[t][j])))
        prev = int(cand[t][best])
        out.append(prev)
        rows.append(s)
    return np.array(out, dtype=np.int64), cand, np.array(rows)
