"""Seeded tensor generators (no method arithmetic).

Distributions: matrices N(0, 0.02); RMSNorm gains 1; tapped features N(0, 1);
synthetic context / target K,V N(0, 1); token ids uniform; contexts of the
paged workload uniform integers in a range.  bf16 workloads draw in float32 and
round to bfloat16 with round-to-nearest-even (torch's conversion), so both sides
see exactly the bf16 values.
"""
from __future__ import annotations

import hashlib

import numpy as np
import torch

from .configs import ModelShape, Workload

WEIGHT_STD = 0.02
_M64 = (1 << 64) - 1


def seed_of(cid: int, name: str) -> int:
    h = hashlib.sha256(f"dflash/{cid}/{name}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _generator(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(seed)
    return g


def _storage(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def normal(shape, std: float, cid: int, name: str, device="cpu", dtype="f32") -> torch.Tensor:
    g = _generator(device, seed_of(cid, name))
    t = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(_storage(dtype))


def uniform_ints(shape, lo: int, hi_inclusive: int, cid: int, name: str, device="cpu") -> torch.Tensor:
    g = _generator(device, seed_of(cid, name))
    t = torch.randint(lo, hi_inclusive + 1, tuple(shape), generator=g, device=device,
                      dtype=torch.int64)
    return t.to(torch.int32)


def to_numpy(t: torch.Tensor) -> np.ndarray:
    """Host float32 (or int) copy of a tensor, for the oracle."""
    if t.dtype in (torch.int32, torch.int64):
        return t.detach().cpu().numpy()
    return t.detach().to(torch.float32).cpu().numpy()


def shared_weights(w: Workload, device="cpu") -> dict:
    """Token embedding E[V, D] and LM head W_lm[V, D], shared by drafter and target."""
    m = w.draft
    return {
        "embed": normal((m.vocab, m.hidden), WEIGHT_STD, w.cid, "embed", device, w.dtype),
        "lm_head": normal((m.vocab, m.hidden), WEIGHT_STD, w.cid, "lm_head", device, w.dtype),
    }


def model_weights(w: Workload, which: str, device="cpu") -> dict:
    """Per-layer weights of the drafter (``which="draft"``) or the target.

    Keys: ``L{i}.{g_in,wq,wk,wv,wo,g_post,wg,wu,wd}`` (matrices row-major [out, in]),
    ``g_f`` (final norm gain) and, for the drafter, ``w_c`` [D, k*D] and ``g_c`` [D].
    """
    m: ModelShape = w.draft if which == "draft" else w.target
    D, d = m.hidden, m.head_dim
    st = _storage(w.dtype)
    out = {}

    def mat(name, shape):
        out[name] = normal(shape, WEIGHT_STD, w.cid, f"{which}.{name}", device, w.dtype)

    def gain(name, n):
        out[name] = torch.ones(n, dtype=st, device=device)

    for i in range(m.n_layers):
        gain(f"L{i}.g_in", D)
        mat(f"L{i}.wq", (m.n_q_heads * d, D))
        mat(f"L{i}.wk", (m.n_kv_heads * d, D))
        mat(f"L{i}.wv", (m.n_kv_heads * d, D))
        mat(f"L{i}.wo", (D, m.n_q_heads * d))
        gain(f"L{i}.g_post", D)
        mat(f"L{i}.wg", (m.ffn, D))
        mat(f"L{i}.wu", (m.ffn, D))
        mat(f"L{i}.wd", (D, m.ffn))
    gain("g_f", D)
    if which == "draft":
        mat("w_c", (D, w.n_taps * D))
        gain("g_c", D)
    return out


def selector_weights(w: Workload, rank: int = 256, std: float = WEIGHT_STD, device="cpu") -> dict:
    """Path-selector maps of the drafter: w_a, w_b, w_h [hidden, rank], N(0, std^2)."""
    D = w.draft.hidden
    return {n: normal((D, rank), std, w.cid, f"selector.{n}", device, w.dtype)
            for n in ("w_a", "w_b", "w_h")}


DCONV_NAMES = ("pre_attn", "post_attn", "pre_ffn", "post_ffn")


def dconv_shapes(hidden: int) -> dict:
    """Shapes of one two-tap dynamic convolution: base [2, D] and the correction map
    W_k [D, D/8] (one coefficient per tap per group of 16 channels)."""
    return {"base": (2, hidden), "w_k": (hidden, hidden // 8)}


def dconv_weights(w: Workload, device="cpu", base1_std: float = 0.5, wk_scale: float = 0.3) -> dict:
    """Two-tap convolutions of every drafter layer (keys L{i}.dconv_{name}.{base,w_k}):
    base_0 = 1 + N(0, 0.1^2), base_1 = N(0, base1_std^2), W_k = N(0, (wk_scale^2 / D))."""
    m = w.draft
    D = m.hidden
    out = {}
    for i in range(m.n_layers):
        for name in DCONV_NAMES:
            key = f"L{i}.dconv_{name}"
            b0 = 1.0 + normal((1, D), 0.1, w.cid, key + ".b0", device)
            b1 = normal((1, D), base1_std, w.cid, key + ".b1", device)
            out[key + ".base"] = torch.cat([b0, b1], 0).to(_storage(w.dtype))
            out[key + ".w_k"] = normal(dconv_shapes(D)["w_k"], wk_scale / D ** 0.5, w.cid, key + ".w_k",
                                       device, w.dtype)
    return out


def features(w: Workload, rows: int, device="cpu", tag="feats") -> torch.Tensor:
    """Tapped target features [rows, k*D], N(0, 1)."""
    return normal((rows, w.n_taps * w.draft.hidden), 1.0, w.cid, tag, device, w.dtype)


def anchors(w: Workload, device="cpu", tag="anchor") -> torch.Tensor:
    return uniform_ints((w.batch,), 0, w.draft.vocab - 1, w.cid, tag, device)


def prompt_tokens(w: Workload, n: int, device="cpu", tag="prompt") -> torch.Tensor:
    return uniform_ints((n,), 0, w.draft.vocab - 2, w.cid, tag, device)


def ctx_lengths(w: Workload) -> list:
    if w.ctx is not None:
        return list(w.ctx)
    kind, lo, hi = w.ctx_rule
    assert kind == "uniform"
    rng = np.random.Generator(np.random.PCG64(seed_of(w.cid, "ctx_lengths")))
    return [int(x) for x in rng.integers(lo, hi + 1, size=w.batch)]


def synthetic_ctx_kv(w: Workload, which: str, lengths, device="cpu", std=1.0):
    """Dense per-layer context K/V of each sequence: list over layers of lists over
    sequences of (K [n_b, Hkv, d], V [n_b, Hkv, d]).  K is taken as already rotated."""
    m = w.draft if which == "draft" else w.target
    out = []
    for i in range(m.n_layers):
        per_seq = []
        for b, n in enumerate(lengths):
            k = normal((n, m.n_kv_heads, m.head_dim), std, w.cid, f"{which}.ctxK.L{i}.b{b}",
                       device, w.dtype)
            v = normal((n, m.n_kv_heads, m.head_dim), std, w.cid, f"{which}.ctxV.L{i}.b{b}",
                       device, w.dtype)
            per_seq.append((k, v))
        out.append(per_seq)
    return out


# ---------------------------------------------------------------------------------------
# splitmix64 (Vigna's published generator) drives the seeded acceptance-forcing coins.
def splitmix64(state: int) -> tuple:
    """One step: returns (output, new_state)."""
    state = (state + 0x9E3779B97F4A7C15) & _M64
    z = state
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31), state


def _uniform01(seed: int, cycle: int, b: int, j: int) -> float:
    key = ((seed & 0xFFFF) << 48) | ((cycle & 0xFFFFFF) << 24) | ((b & 0xFFF) << 12) | (j & 0xFFF)
    z, _ = splitmix64(key)
    return (z >> 11) * (1.0 / (1 << 53))


def force_coins(seed: int, cycle: int, batch: int, block: int, p: float) -> np.ndarray:
    """Coins c[b, j] = [u < p] for draft positions j = 1..B-1 (column j-1)."""
    c = np.zeros((batch, block - 1), dtype=bool)
    for b in range(batch):
        for j in range(1, block):
            c[b, j - 1] = _uniform01(seed, cycle, b, j) < p
    return c


def forced_drafts(coins_row, gstar, own_drafts, vocab):
    """Seeded acceptance forcing for one sequence's block: with f the length of the
    leading run of heads in coins_row (length B-1), d_j = g*_{j-1} for j <= f and, if
    f < B-1, d_{f+1} is the drafter's own id when it differs from g*_f, else
    (g*_f + 1) mod V; later positions keep the drafter's ids.  gstar holds the target's
    greedy continuation g*_0 .. g*_f (at least f+1 entries)."""
    coins_row = np.asarray(coins_row, dtype=bool)
    B1 = coins_row.shape[0]
    f = 0
    while f < B1 and coins_row[f]:
        f += 1
    d = np.array(own_drafts, dtype=np.int64).copy()
    for j in range(1, f + 1):
        d[j - 1] = int(gstar[j - 1])
    if f < B1:
        if int(d[f]) == int(gstar[f]):
            d[f] = (int(gstar[f]) + 1) % vocab
    return d, f
