"""Helpers shared by the GPU parity tests: build the HIP-side objects and the oracle's
inputs from the same seeded tensors, and compare results with the stated tolerances."""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
import synth
from block_diffusion_drafter_03_amd import runtime as rt

DEV = "cuda"
TOL = {"f32": 1e-4, "bf16": 2e-2}     # max |x - y| / max |y| per tensor (per row for logits)
NEAR_TIE = 1e-2                        # oracle top-2 logit gap below which ids are not compared


def maxrel(x, y):
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    assert x.shape == y.shape, f"shape {x.shape} != {y.shape}"
    if y.size == 0:   # e.g. the cache rows of an empty context
        return 0.0
    den = np.max(np.abs(y))
    return float(np.max(np.abs(x - y)) / den) if den > 0 else float(np.max(np.abs(x)))


def assert_close(x, y, tol, what):
    e = maxrel(x, y)
    assert e <= tol, f"{what}: max relative error {e:.3e} > {tol:.1e}"
    return e


def assert_rows_close(x, y, tol, what):
    worst = 0.0
    for i in range(y.shape[0]):
        worst = max(worst, assert_close(x[i], y[i], tol, f"{what} row {i}"))
    return worst


def assert_ids(gpu_ids, ora_ids, ora_logits, what):
    """Ids must match wherever the oracle's top-2 gap is >= NEAR_TIE."""
    gpu_ids = np.asarray(gpu_ids).reshape(-1)
    ora_ids = np.asarray(ora_ids).reshape(-1)
    gaps = O.top2_gap(np.asarray(ora_logits, dtype=np.float64).reshape(len(ora_ids), -1))
    checked = gaps >= NEAR_TIE
    bad = np.nonzero(checked & (gpu_ids != ora_ids))[0]
    assert bad.size == 0, f"{what}: ids differ at {bad.tolist()} (gaps {gaps[bad].tolist()})"
    return int(checked.sum())


def assert_accept(tau, bonus, gpu_g, drafts, og, oz, what):
    """(tau, bonus) must equal the oracle's acceptance where none of the rows that decide
    it (0 .. a) is a near-tie of the oracle's logits; otherwise they must be the greedy
    rule applied to the kernel's own argmax row (checked here with a plain loop)."""
    drafts = [int(x) for x in drafts]
    a, t, bo = O.accept(np.asarray(drafts), og)
    if np.all(O.top2_gap(np.asarray(oz[:a + 1], dtype=np.float64)) >= NEAR_TIE):
        assert (int(tau), int(bonus)) == (t, bo), f"{what}: ({tau}, {bonus}) != oracle ({t}, {bo})"
        return True
    gg = [int(x) for x in gpu_g]
    a2 = 0
    while a2 < len(drafts) and drafts[a2] == gg[a2]:
        a2 += 1
    assert (int(tau), int(bonus)) == (a2 + 1, gg[a2]), f"{what}: not the rule on its own argmax"
    return False


class Setup:
    """Drafter (+ target) of a workload on the GPU, with numpy float32 copies for the oracle."""

    def __init__(self, w: synth.Workload, target=False, device=DEV, dconv=None):
        """dconv: None, or the DFlash 2 convolution weights of the drafter (a dict as from
        synth.dconv_weights)."""
        self.w = w
        self.device = device
        self.dw = synth.model_weights(w, "draft", device)
        self.shared = synth.shared_weights(w, device)
        self.draft = rt.Model(w.draft, self.dw, self.shared, n_taps=w.n_taps, draft=True, dconv=dconv)
        if dconv is not None:
            self.dw = {**self.dw, **dconv}
        self.np_dw = {k: synth.to_numpy(v) for k, v in self.dw.items()}
        self.np_shared = {k: synth.to_numpy(v) for k, v in self.shared.items()}
        self.target = None
        if target:
            self.tw = synth.model_weights(w, "target", device)
            self.target = rt.Model(w.target, self.tw, self.shared, n_taps=len(w.taps), taps=w.taps,
                                   draft=False)
            self.np_tw = {k: synth.to_numpy(v) for k, v in self.tw.items()}

    @property
    def st(self):
        return torch.float32 if self.w.dtype == "f32" else torch.bfloat16

    @property
    def store(self):
        """Storage type of the cache and of handed-over features, as the oracle takes it."""
        return None if self.w.dtype == "f32" else "bf16"

    def kv(self, shape, capacity, permute_pages=True, seed=0, spare=0):
        g = torch.Generator().manual_seed(seed)
        b = self.w.batch
        maxp = (capacity + rt.PAGE - 1) // rt.PAGE
        order = torch.randperm(b * maxp, generator=g) if permute_pages else None
        return rt.PagedKV(shape, b, capacity, self.st, self.device, page_order=order, spare_pages=spare)

    def workspace(self, model, block, capacity, inject_rows=0):
        return rt.Workspace(model.workspace_bytes(self.w.batch, block, capacity, inject_rows),
                            self.device)


def inject_all(setup: Setup, kv, feats_per_seq, ws, chunk=None):
    """Inject each sequence's feature rows at positions 0..n-1 (absolute), optionally in
    chunks, and set seq_len to n."""
    rows_seq, rows_pos, feats = [], [], []
    for b, f in enumerate(feats_per_seq):
        n = f.shape[0]
        rows_seq.append(torch.full((n,), b, dtype=torch.int32))
        rows_pos.append(torch.arange(n, dtype=torch.int32))
        feats.append(f)
    rs = torch.cat(rows_seq).to(setup.device)
    rp = torch.cat(rows_pos).to(setup.device)
    F = torch.cat(feats).contiguous()
    R = F.shape[0]
    step = chunk or R
    for a in range(0, R, step):
        e = min(R, a + step)
        rt.inject_ctx(setup.draft, kv, F[a:e].contiguous(), rs[a:e].contiguous(),
                      rp[a:e].contiguous(), 0, max(f.shape[0] for f in feats_per_seq), ws)
    kv.set_seq_len([f.shape[0] for f in feats_per_seq])


def read_cache(kv, layer, b, n):
    K, V = kv.read_dense(layer, b, n)
    return synth.to_numpy(K), synth.to_numpy(V)


def check_selection(g_ids, g_cand, o_ids, o_cand, o_rows, z, top_k, tie, what):
    """Path-selector outputs of one sequence against the oracle's.  Candidate sets are
    compared where the oracle's top_k-th and next logits differ by >= tie; the walk's picks
    in order, a difference being allowed only where the oracle decides the pick by a
    near-tie of scores or where the candidate sets differ at a near-tie of the boundary
    (the walk stops being compared there: later picks depend on it).  Returns (candidate
    positions checked, picks checked)."""
    cand_checked = walk_checked = 0
    for t in range(len(o_ids)):
        srt = np.sort(z[t])[::-1]
        if srt[top_k - 1] - srt[top_k] >= tie:
            assert set(g_cand[t]) == set(o_cand[t]), f"{what} position {t + 1} candidates"
            cand_checked += 1
    for t in range(len(o_ids)):
        if g_ids[t] == o_ids[t]:
            walk_checked += 1
            continue
        srt = np.sort(z[t])[::-1]
        boundary_tie = set(g_cand[t]) != set(o_cand[t]) and srt[top_k - 1] - srt[top_k] < tie
        assert boundary_tie or float(O.top2_gap(o_rows[t])) < tie, f"{what} position {t + 1}"
        break
    return cand_checked, walk_checked
