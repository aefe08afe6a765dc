"""Pins of the oracle's DFlash 2 two-tap dynamic convolution ([DF] section 7.1, Problem 2) to
facts other than its own formula: identity and pure-shift kernels, a hand-computed
content-dependent correction, the placement inside the sublayer branches, and the page's
parameter count for the reading of the correction's shape."""
import json
import os

import numpy as np

import oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "dflash2_conv_params.json")


def test_identity_and_shift_kernels():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 32))
    zero = np.zeros((32, 4))
    ident = np.stack([np.ones(32), np.zeros(32)])
    assert np.array_equal(O.dconv(x, ident, zero, np.float64), x)
    shift = np.stack([np.zeros(32), np.ones(32)])
    out = O.dconv(x, shift, zero, np.float64)
    assert np.array_equal(out[0], x[0])          # the anchor row reads itself
    assert np.array_equal(out[1:], x[:-1])       # later rows read their predecessor


def test_content_dependent_correction_by_hand():
    rng = np.random.default_rng(2)
    T, D = 4, 32                                  # two groups of 16 channels
    x = rng.standard_normal((T, D))
    base = rng.standard_normal((2, D))
    w_k = np.zeros((D, D // 8))
    w_k[5, 0] = 1.0                               # tap 0 of group 0 += x_t[5]
    w_k[20, 3] = 2.0                              # tap 1 of group 1 += 2 x_t[20]
    out = O.dconv(x, base, w_k, np.float64)
    for t in range(T):
        p = max(t - 1, 0)
        for c in range(D):
            k0 = base[0, c] + (x[t, 5] if c < 16 else 0.0)
            k1 = base[1, c] + (2.0 * x[t, 20] if c >= 16 else 0.0)
            assert abs(out[t, c] - (k0 * x[t, c] + k1 * x[p, c])) < 1e-12


def _layer_inputs(w, rng):
    m = w.draft
    dw = {k: synth.to_numpy(v).astype(np.float64) for k, v in synth.model_weights(w, "draft").items()}
    T, n = 4, 6
    h = rng.standard_normal((T, m.hidden))
    ck = rng.standard_normal((n, m.n_kv_heads, m.head_dim))
    cv = rng.standard_normal((n, m.n_kv_heads, m.head_dim))
    return m, dw, h, np.arange(n, n + T), ck, cv


def test_identity_convolutions_leave_the_layer_unchanged():
    w = synth.workload("tiny_f32")
    m, dw, h, pos, ck, cv = _layer_inputs(w, np.random.default_rng(3))
    plain, _, _ = O.decoder_layer(h, dw, 0, m, pos, ck, cv, causal=False, dt=np.float64)
    D = m.hidden
    for name in synth.DCONV_NAMES:
        dw[f"L0.dconv_{name}.base"] = np.stack([np.ones(D), np.zeros(D)])
        dw[f"L0.dconv_{name}.w_k"] = np.zeros((D, D // 8))
    conv, _, _ = O.decoder_layer(h, dw, 0, m, pos, ck, cv, causal=False, dt=np.float64)
    assert np.array_equal(conv, plain)


def test_post_convolutions_act_on_the_branch_before_the_residual_add():
    # zero post kernels silence both branches: the layer returns its input unchanged
    w = synth.workload("tiny_f32")
    m, dw, h, pos, ck, cv = _layer_inputs(w, np.random.default_rng(4))
    D = m.hidden
    for name in ("post_attn", "post_ffn"):
        dw[f"L0.dconv_{name}.base"] = np.zeros((2, D))
        dw[f"L0.dconv_{name}.w_k"] = np.zeros((D, D // 8))
    out, _, _ = O.decoder_layer(h, dw, 0, m, pos, ck, cv, causal=False, dt=np.float64)
    assert np.array_equal(out, h)
    # a zero pre-FFN kernel silences the FFN only: the output is the post-attention stream
    dw2 = {k: v for k, v in dw.items() if "dconv" not in k}
    dw2["L0.dconv_pre_ffn.base"] = np.zeros((2, D))
    dw2["L0.dconv_pre_ffn.w_k"] = np.zeros((D, D // 8))
    dw3 = {k: v for k, v in dw2.items()}
    dw3["L0.wd"] = np.zeros_like(dw3["L0.wd"])   # same layer with the FFN output forced to 0
    a, _, _ = O.decoder_layer(h, dw2, 0, m, pos, ck, cv, causal=False, dt=np.float64)
    b, _, _ = O.decoder_layer(h, {k: v for k, v in dw3.items() if "dconv" not in k}, 0, m, pos, ck, cv,
                              causal=False, dt=np.float64)
    assert np.allclose(a, b, rtol=0, atol=1e-12)


def test_parameter_count_matches_the_page():
    g = json.load(open(GOLDEN))
    shapes = synth.dconv_shapes(g["hidden_reading"])
    per_conv = sum(int(np.prod(s)) for s in shapes.values())
    total = per_conv * g["convolutions_per_layer"] * g["drafter_layers"]
    # equal to the printed figure at its printed precision (16.5M: three digits)
    assert float(f"{total:.{g['printed_digits']}g}") == g["params"], total
