#!/usr/bin/env python3
"""Benchmark of the DFlash drafter step on one MI355X.

One timed step is one speculative cycle of the Qwen3-8B-shaped drafter (5 layers, hidden
4096, 32/8 heads x 128, FFN 12288, vocab 151936, bf16) at batch 1 over a 4096-row injected
context with blocks of 16: draft_block, verify_accept by an 8-layer Qwen3-8B-shaped target
(FFN 14336) over a 4096-token cache, inject_ctx of the 16 verified feature rows, kv_commit.
All inputs are seeded synthetic tensors already resident in HBM.

Prints one JSON line: draft tokens/s of the draft block (b * (B-1) / T_draft_block) as
`value`, the cycle time as `ms_per_step`, per-call microseconds (means of the timed steps,
and medians with p10 / p90 over 50 more cycles), the roofline of the dominant kernel (the
weight-streaming GEMV of the gate/up projections with its SwiGLU epilogue) timed with HIP
events inside the timed region, the float32 tiny workload, the attention roofline at 64K
and 262K contexts, the M = 256 GEMMs against the bf16 MFMA peak, the batch-8 cycles under
the acceptance-forcing rule (tau, alpha, L), and the CPU oracle timed on the host on a
bounded sample (every call of the cycle).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs per draft block & draft tokens/s (B=16, ctx 4K–262K); % HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def stats(values):
    """median / p10 / p90 / mean of a list of timings (nearest rank)."""
    a = sorted(values)
    n = len(a)

    def q(f):
        return a[min(n - 1, max(0, int(round(f * (n - 1)))))]
    return {"median": round(q(0.5), 2), "p10": round(q(0.1), 2), "p90": round(q(0.9), 2),
            "mean": round(sum(a) / n, 2), "reps": n}


STATS_REPS = 50


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gemv_gate_up.qwen3_8b_b1_ctx4k.pmc_traffic.txt")


def measured_profile():
    """(HBM bytes per launch, rocprofv3 kernel-trace average duration in us) of the roofline
    kernel from the committed FETCH_SIZE/WRITE_SIZE summary, or (None, None) when the
    kernel's sources have changed since the counters were taken."""
    import hashlib
    try:
        fields = {}
        for line in open(TRAFFIC_SUMMARY):
            k, sep, v = line.partition(":")
            if sep:
                fields[k.strip()] = v.strip()
        h = hashlib.sha256()
        for src in fields["kernel_sources"].split():
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != fields["kernel_sources_sha256"]:
            return None, None
        trace = fields.get("kernel-trace average duration (same command without counters)", "")
        return int(fields["traffic_bytes_per_launch"]), (float(trace.split()[0]) if trace else None)
    except (OSError, KeyError, ValueError, IndexError):
        return None, None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=20)
    ap.add_argument("--no-workload-sweep", action="store_true",
                    help="skip the batch-16, 512-row injection and batch-8 cycle measurements")
    ap.add_argument("--no-context-sweep", action="store_true",
                    help="skip the draft block / attention timing at 4K, 64K and 262K contexts")
    ap.add_argument("--probe-copy", type=int, default=0, metavar="MB",
                    help="after the run, one elementwise pass reading and writing MB MiB, then "
                         "two reads of MB MiB with plain and non-temporal loads (calibrate the "
                         "HBM byte counters of profiler runs)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the drafter step is data-parallel over sequences, "
              "each GPU serving its own sequences with its own cache, and no collectives are run.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    from block_diffusion_drafter_03_amd import _lib
    from block_diffusion_drafter_03_amd import runtime as rt

    dev = "cuda"
    torch.cuda.set_device(0)
    w = synth.workload("qwen3_8b_b1_ctx4k")
    wt = synth.workload("qwen3_8b_cycle_b8")          # supplies the 8-layer target shape
    D, B, n = w.draft, w.block, w.ctx[0]
    T = wt.target
    taps = wt.taps
    K, W = args.steps, args.warmup
    log("generating weights on the GPU")
    dw = synth.model_weights(w, "draft", dev)
    shared = synth.shared_weights(w, dev)
    tw = synth.model_weights(wt, "target", dev)
    draft = rt.Model(D, dw, shared, n_taps=w.n_taps, draft=True)
    target = rt.Model(T, tw, shared, n_taps=len(taps), taps=taps, draft=False)
    cap = n + B * (K + W + 3 * 8 + 12 + 4 + STATS_REPS) + 64     # every cycle appends <= B rows
    dkv = rt.PagedKV(D, 1, cap, torch.bfloat16, dev)
    tkv = rt.PagedKV(T, 1, cap, torch.bfloat16, dev)
    chunk = 512
    ws_d = rt.Workspace(draft.workspace_bytes(1, B, dkv.capacity, chunk), dev)
    ws_t = rt.Workspace(target.workspace_bytes(1, B, tkv.capacity), dev)

    log("injecting the 4096-row drafter context (512-row chunks) and filling the target cache")
    feats0 = synth.features(w, n, dev, tag="feats.b0")
    seq0 = torch.zeros(chunk, dtype=torch.int32, device=dev)
    inj_ms = []
    for a in range(0, n, chunk):
        pos = torch.arange(a, a + chunk, dtype=torch.int32, device=dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        rt.inject_ctx(draft, dkv, feats0[a:a + chunk].contiguous(), seq0, pos, 0, a + chunk, ws_d)
        e1.record()
        inj_ms.append((e0, e1))
    dkv.set_seq_len(n)
    tctx = synth.synthetic_ctx_kv(wt, "target", [n], dev)
    for l in range(T.n_layers):
        tkv.write_dense(l, 0, tctx[l][0][0], tctx[l][0][1])
    del tctx
    tkv.set_seq_len(n)
    torch.cuda.synchronize()
    chunk_us = [a.elapsed_time(b) * 1e3 for a, b in inj_ms]

    anchor = synth.anchors(w, dev)
    bonus = torch.zeros(1, dtype=torch.int32, device=dev)
    drafts = torch.zeros(1, B - 1, dtype=torch.int32, device=dev)
    feats = torch.zeros(1, B, w.n_taps * D.hidden, dtype=torch.bfloat16, device=dev)
    g = torch.zeros(1, B, dtype=torch.int32, device=dev)
    tau = torch.zeros(1, dtype=torch.int32, device=dev)
    rseq = torch.zeros(B, dtype=torch.int32, device=dev)
    rpos = torch.arange(B, dtype=torch.int32, device=dev)
    feats2d = feats.view(B, -1)
    state = {"anchor": anchor, "bonus": bonus}

    def step(ev=None):
        a, bo = state["anchor"], state["bonus"]
        if ev: ev[0].record()
        rt.draft_block(draft, dkv, a, B, drafts, ws_d)
        if ev: ev[1].record()
        rt.verify_accept(target, tkv, a, drafts, B, feats, g, tau, bo, ws_t)
        if ev: ev[2].record()
        rt.inject_ctx(draft, dkv, feats2d, rseq, rpos, 1, B, ws_d)
        if ev: ev[3].record()
        rt.kv_commit(tkv, dkv, tau, B)
        if ev: ev[4].record()
        state["anchor"], state["bonus"] = bo, a          # the bonus is the next anchor

    log(f"warmup {W} steps")
    for _ in range(W):
        step()
    torch.cuda.synchronize()
    seq_before = int(tkv.seq_len.item())

    # dominant kernel over the cycle: gate/up projection GEMMs (5 drafter + 8 target launches)
    per_step = D.n_layers + T.n_layers
    _lib.timing_arm(_lib.KERNEL_GEMM_GATE_UP, per_step * K)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(K)]
    log(f"timing {K} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gu_ms = _lib.timing_read(per_step * K)
    seq_after = int(tkv.seq_len.item())
    assert int(tkv.err.item()) == 0 and int(dkv.err.item()) == 0

    ms_per_step = (t1 - t0) * 1e3 / K

    def mean_us(i, j):
        return sum(e[i].elapsed_time(e[j]) for e in evs) * 1e3 / K

    us_draft, us_verify, us_inject, us_commit = mean_us(0, 1), mean_us(1, 2), mean_us(2, 3), mean_us(3, 4)
    tau_mean = (seq_after - seq_before) / K
    draft_tok_s = 1 * (B - 1) / (us_draft * 1e-6)

    # roofline of the gate/up GEMM launches: algorithmic bytes = bf16 weights + gain, the
    # float32 hidden rows read and the float32 SwiGLU rows written
    def gu_bytes(m):
        return 2 * m.ffn * m.hidden * 2 + m.hidden * 2 + B * m.hidden * 4 + B * m.ffn * 4
    bytes_d, bytes_t = gu_bytes(D), gu_bytes(T)
    nbytes = [bytes_d if (i % per_step) < D.n_layers else bytes_t for i in range(len(gu_ms))]
    achieved = sum(nbytes) / (sum(gu_ms) * 1e-3) / 1e9
    avg_bytes = sum(nbytes) / len(nbytes)
    avg_us = sum(gu_ms) / len(gu_ms) * 1e3

    # per-class breakdown over a few extra (untimed) cycles
    classes = {"lm_head": _lib.KERNEL_LM_HEAD, "gemm_qkv": _lib.KERNEL_GEMM_QKV,
               "gemm_o": _lib.KERNEL_GEMM_O, "gemm_gate_up": _lib.KERNEL_GEMM_GATE_UP,
               "gemm_down": _lib.KERNEL_GEMM_DOWN, "attention": _lib.KERNEL_ATTENTION,
               "inject_fuse": _lib.KERNEL_INJECT_FUSE, "inject_kv": _lib.KERNEL_INJECT_KV}
    breakdown = {}
    for name, kid in classes.items():
        _lib.timing_arm(kid, 64)
        for _ in range(3):
            step()
        torch.cuda.synchronize()
        ms = _lib.timing_read(64)
        breakdown[name] = {"launches_per_cycle": len(ms) / 3,
                           "us_per_cycle": sum(ms) * 1e3 / 3}

    # per-call latency distribution: STATS_REPS more cycles, each call bracketed by events
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(STATS_REPS)]
    for i in range(STATS_REPS):
        step(evs[i])
    torch.cuda.synchronize()
    latency = {name: stats([e[j].elapsed_time(e[j + 1]) * 1e3 for e in evs])
               for j, name in enumerate(("draft_block", "verify_accept", "inject_16_rows", "kv_commit"))}
    assert int(tkv.err.item()) == 0 and int(dkv.err.item()) == 0

    # the block size is a runtime argument: draft blocks of 8, 10 and 16 on the same cache
    block_sweep = {}
    for Bs in (8, 10, 16):
        ids_s = torch.zeros(1, Bs - 1, dtype=torch.int32, device=dev)
        for _ in range(2):
            rt.draft_block(draft, dkv, state["anchor"], Bs, ids_s, ws_d)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            rt.draft_block(draft, dkv, state["anchor"], Bs, ids_s, ws_d)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / 10
        block_sweep[str(Bs)] = {"us_per_draft_block": round(us, 2),
                                "draft_tok_s": round((Bs - 1) / (us * 1e-6), 1)}

    # temperature sampling (T = 1) with rejection-sampling verification: 12 cycles
    sampling = sampled_cycles(draft, target, dkv, tkv, ws_d, ws_t, state["anchor"], B, w.n_taps,
                              D, T, dev)
    # DFlash 2 path selector (rank 256, top-16) on the same drafter and context
    selector = selector_timing(w, draft, dkv, ws_d, state["anchor"], B, D, dev)
    # DFlash 2 two-tap convolutions around every sublayer: the same drafter with them
    dconv = dconv_timing(w, dw, shared, dkv, state["anchor"], B, D, n, dev)
    hbm_bytes_draft = (D.n_layers * ((D.n_q_heads + 2 * D.n_kv_heads) * D.head_dim * D.hidden
                                     + D.hidden * D.n_q_heads * D.head_dim + 3 * D.ffn * D.hidden) * 2
                       + D.vocab * D.hidden * 2 + D.n_layers * n * D.n_kv_heads * D.head_dim * 2 * 2)

    traffic, prof_us = measured_profile()
    tiny = tiny_timing(dev)
    out = {
        "metric": METRIC,
        "value": round(draft_tok_s, 1),
        "unit": "draft tok/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "qwen3_8b_b1_ctx4k: Qwen3-8B-shaped drafter (5 layers, 4096, 32/8x128, "
                               "FFN 12288, V 151936), batch 1, 4096-row injected context, block 16; "
                               "verify by an 8-layer Qwen3-8B-shaped target (FFN 14336, 4096-token cache)",
                   "batch": 1, "block": B, "ctx": n},
        "us_per_draft_block": round(us_draft, 2),
        "us_per_verify": round(us_verify, 2),
        "us_per_inject_16_rows": round(us_inject, 2),
        "us_per_commit": round(us_commit, 2),
        "us_per_inject_512_rows": round(sum(chunk_us[1:]) / max(1, len(chunk_us) - 1), 2),
        "tau_mean": tau_mean,
        "L_us_per_token": round((us_draft + us_verify + us_inject + us_commit) / max(tau_mean, 1e-9), 2),
        "draft_block_hbm_gbs": round(hbm_bytes_draft / (us_draft * 1e-6) / 1e9, 1),
        "draft_block_hbm_frac": round(hbm_bytes_draft / (us_draft * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": {"kernel": "gemm_gemv_bf16 (gate/up projection + SwiGLU, M=16)", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "bytes_per_launch": int(avg_bytes), "avg_launch_us": round(avg_us, 2),
                     "launches": len(gu_ms),
                     # the rocprofv3 kernel-trace average of the committed profile (kernel only;
                     # the event pair above also holds the dispatch of the kernel, a few us)
                     "profile_avg_kernel_us": prof_us,
                     "frac_profile": (round(avg_bytes / (prof_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                                      if prof_us else None)},
        "latency_us": latency,
        "tiny_f32": tiny,
        "kernels": breakdown,
        "block_sweep": block_sweep,
        "sampling_t1": sampling,
        "path_selector": selector,
        "dconv": dconv,
    }
    if not args.no_context_sweep:
        out["context_sweep"] = context_sweep(draft, D, B, dev)
        out["roofline_attention"] = {
            ctx: {"bound": "hbm", "achieved": v["attention_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": v["attention_hbm_frac"], "bytes_per_launch": v["attention_bytes_per_layer"],
                  "median_us": v["attention_us_per_layer"]["median"]}
            for ctx, v in out["context_sweep"].items() if int(ctx) >= 65536}
    if not args.no_workload_sweep:
        out["workload_sweep"] = workload_sweep(draft, target, D, T, B, dev)
        out["roofline_gemm_m256"] = out["workload_sweep"]["qwen3_8b_b16_paged"]["gemms"]

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, wt, dw, tw, shared, feats0, anchor, tkv, args.cpu_reps,
                                           draft_tok_s)
    print(json.dumps(out), flush=True)
    if args.probe_copy > 0:
        src = torch.ones(args.probe_copy << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)      # reads and writes exactly probe_copy MiB each
        torch.cuda.synchronize()
        log(f"probe copy: {args.probe_copy} MiB read + {args.probe_copy} MiB written")
        # one read of the same bytes in each load form of the library (plain, then with the
        # non-temporal hint of its weight streams)
        import ctypes
        sink = torch.empty(16 << 10, dtype=torch.uint8, device=dev)
        for nt in (False, True):
            _lib.probe_read(ctypes.c_void_p(src.data_ptr()), src.numel() * 4, nt,
                            ctypes.c_void_p(sink.data_ptr()), rt._stream())
            torch.cuda.synchronize()
        log(f"probe reads: {args.probe_copy} MiB with plain loads, then with non-temporal loads")


def tiny_timing(dev, reps=STATS_REPS):
    """The float32 tiny workload (2 layers, hidden 256, 4 heads x 64, vocab 4096, block 4,
    128 injected context rows, batch 1): µs per draft block and per verify (2-layer target),
    launch-latency bound; median / p10 / p90 over `reps` calls each."""
    import torch
    import synth
    from block_diffusion_drafter_03_amd import runtime as rt

    w = synth.TINY
    m, t, B, n = w.draft, w.target, w.block, w.ctx[0]
    dw = synth.model_weights(w, "draft", dev)
    tw = synth.model_weights(w, "target", dev)
    sh = synth.shared_weights(w, dev)
    draft = rt.Model(m, dw, sh, n_taps=w.n_taps, draft=True)
    target = rt.Model(t, tw, sh, n_taps=len(w.taps), taps=w.taps, draft=False)
    dkv = rt.PagedKV(m, 1, n + B + 64, torch.float32, dev)
    tkv = rt.PagedKV(t, 1, n + B + 64, torch.float32, dev)
    ws = rt.Workspace(max(draft.workspace_bytes(1, B, dkv.capacity, n),
                          target.workspace_bytes(1, B, tkv.capacity)), dev)
    rt.inject_ctx(draft, dkv, synth.features(w, n, dev), torch.zeros(n, dtype=torch.int32, device=dev),
                  torch.arange(n, dtype=torch.int32, device=dev), 0, n, ws)
    dkv.set_seq_len(n)
    tctx = synth.synthetic_ctx_kv(w, "target", [n], dev)
    for l in range(t.n_layers):
        tkv.write_dense(l, 0, tctx[l][0][0], tctx[l][0][1])
    tkv.set_seq_len(n)
    anchor = synth.anchors(w, dev)
    ids = torch.zeros(1, B - 1, dtype=torch.int32, device=dev)
    g = torch.zeros(1, B, dtype=torch.int32, device=dev)
    tau = torch.zeros(1, dtype=torch.int32, device=dev)
    bonus = torch.zeros(1, dtype=torch.int32, device=dev)
    out = {}
    for name, call in (("draft_block", lambda: rt.draft_block(draft, dkv, anchor, B, ids, ws)),
                       ("verify_accept", lambda: rt.verify_accept(target, tkv, anchor, ids, B, None, g, tau,
                                                                  bonus, ws))):
        for _ in range(3):
            call()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for e0, e1 in evs:
            e0.record()
            call()
            e1.record()
        torch.cuda.synchronize()
        out["us_" + name] = stats([e0.elapsed_time(e1) * 1e3 for e0, e1 in evs])
    assert int(dkv.err.item()) == 0 and int(tkv.err.item()) == 0
    out["note"] = "launch-latency bound (about 11.5 MB of weights); no roofline fraction"
    draft.close()
    target.close()
    return out


def _filled_kv(rt, torch, shape, lens, cap, dev, seed):
    """Paged cache of len(lens) sequences with synthetic N(0, 1) K/V in every page."""
    kv = rt.PagedKV(shape, len(lens), cap, torch.bfloat16, dev)
    gen = torch.Generator(device=dev).manual_seed(seed)
    for t in kv.k + kv.v:
        t.normal_(generator=gen)
    kv.set_seq_len(lens)
    return kv


def _timed(torch, fn, reps):
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in evs:
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    return sum(e0.elapsed_time(e1) for e0, e1 in evs) * 1e3 / reps


def workload_sweep(draft, target, D, T, B, dev, reps=STATS_REPS, cycles=4):
    """The batched workloads, timed on the same models:
    * batch 16, contexts in [2048, 8192] in shuffled 64-token pages: draft block, and the
      gate/up GEMMs' useful bf16 rate against the dense MFMA peak (M = 256 rows);
    * one 512-row injection chunk (fusion + K/V of every draft layer), against MFMA peak;
    * batch 8, 8192-token caches, full cycles under the seeded acceptance-forcing rule
      for p in {0.3, 0.7, 1.0}: tau, T_draft = draft block, T_verify = verify + accept +
      inject + commit, L = (T_draft + T_verify) / tau per sequence."""
    import numpy as np
    import torch
    import synth
    from block_diffusion_drafter_03_amd import _lib
    from block_diffusion_drafter_03_amd import runtime as rt

    out = {}
    # ---- batch 16, ragged paged contexts ----
    w3 = synth.workload("qwen3_8b_b16_paged")
    lens = synth.ctx_lengths(w3)
    kv = _filled_kv(rt, torch, D, lens, max(lens) + B + 64, dev, 3)
    g = torch.Generator().manual_seed(7)
    perm = torch.randperm(kv.block_table.numel(), generator=g).to(torch.int32)
    kv.block_table.copy_(perm.reshape(kv.block_table.shape))
    ws = rt.Workspace(draft.workspace_bytes(w3.batch, B, kv.capacity, w3.batch * B), dev)
    anchor = synth.anchors(w3, dev)
    ids = torch.zeros(w3.batch, B - 1, dtype=torch.int32, device=dev)
    rt.draft_block(draft, kv, anchor, B, ids, ws)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in evs:
        e0.record()
        rt.draft_block(draft, kv, anchor, B, ids, ws)
        e1.record()
    torch.cuda.synchronize()
    blk = stats([e0.elapsed_time(e1) * 1e3 for e0, e1 in evs])
    us = blk["median"]
    M = w3.batch * B
    # every GEMM of the block at M = 256 rows: useful flops 2*M*N*K against the dense bf16
    # peak, and the MFMAs actually issued (float32 activations enter as compensated hi/lo
    # bf16 pairs: twice the useful flops)
    Nqkv = (D.n_q_heads + 2 * D.n_kv_heads) * D.head_dim
    shapes = {"qkv": (_lib.KERNEL_GEMM_QKV, Nqkv, D.hidden), "o": (_lib.KERNEL_GEMM_O, D.hidden, D.n_q_heads * D.head_dim),
              "gate_up": (_lib.KERNEL_GEMM_GATE_UP, 2 * D.ffn, D.hidden),
              "down": (_lib.KERNEL_GEMM_DOWN, D.hidden, D.ffn), "lm_head": (_lib.KERNEL_LM_HEAD, D.vocab, D.hidden)}
    gemms = {}
    for name, (kid, N_, K_) in shapes.items():
        launches = D.n_layers if name != "lm_head" else 1
        _lib.timing_arm(kid, reps * launches)
        for _ in range(reps):
            rt.draft_block(draft, kv, anchor, B, ids, ws)
        ms = _lib.timing_read(reps * launches)
        t_us = sorted(ms)[len(ms) // 2] * 1e3
        useful = 2.0 * M * N_ * K_ / (t_us * 1e-6) / 1e12
        gemms[name] = {"bound": "mfma", "M": M, "N": N_, "K": K_, "median_us": round(t_us, 2),
                       "achieved": round(useful, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                       "frac": round(useful / MFMA_BF16_PEAK_TFLOPS, 4),
                       "frac_issued": round(2 * useful / MFMA_BF16_PEAK_TFLOPS, 4)}
    assert int(kv.err.item()) == 0
    out["qwen3_8b_b16_paged"] = {
        "us_per_draft_block": blk, "draft_tok_s": round(w3.batch * (B - 1) / (us * 1e-6), 1),
        "gemms": gemms,
        "note": "frac: useful 2*M*N*K flops over the dense bf16 peak; frac_issued counts the "
                "compensated hi/lo MFMAs actually issued (twice the useful flops)"}
    log(f"batch 16: draft block {us:.1f} us; " + ", ".join(f"{k} {v['median_us']:.0f} us" for k, v in gemms.items()))
    # ---- one 512-row injection chunk ----
    rows = 512
    rs = torch.zeros(rows, dtype=torch.int32, device=dev)
    rp = torch.arange(rows, dtype=torch.int32, device=dev)
    feats = torch.randn(rows, 5 * D.hidden, device=dev).to(torch.bfloat16)
    kv1 = rt.PagedKV(D, 1, rows + 64, torch.bfloat16, dev)
    ws1 = rt.Workspace(draft.workspace_bytes(1, B, kv1.capacity, rows), dev)
    rt.inject_ctx(draft, kv1, feats, rs, rp, 0, rows, ws1)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in evs:
        e0.record()
        rt.inject_ctx(draft, kv1, feats, rs, rp, 0, rows, ws1)
        e1.record()
    torch.cuda.synchronize()
    inj = stats([e0.elapsed_time(e1) * 1e3 for e0, e1 in evs])
    us_inj = inj["median"]
    flops = 2.0 * rows * (5 * D.hidden * D.hidden + D.hidden * D.n_layers * 2 * D.n_kv_heads * D.head_dim)
    inj_tf = flops / (us_inj * 1e-6) / 1e12
    out["inject_512_rows"] = {"us": inj, "useful_tflops": round(inj_tf, 1),
                              "mfma_frac": round(inj_tf / MFMA_BF16_PEAK_TFLOPS, 4),
                              "note": "fusion GEMM over bf16 features (no compensation) + K/V GEMM"}
    log(f"inject 512 rows: {us_inj:.1f} us, {inj_tf:.0f} useful TFLOP/s")
    del kv, ws, kv1, ws1
    torch.cuda.empty_cache()
    # ---- batch 8 cycles with forced acceptance ----
    w5 = synth.workload("qwen3_8b_cycle_b8")
    lens5 = synth.ctx_lengths(w5)
    nb = w5.batch
    cap = max(lens5) + B * (3 * cycles + 2) + 64
    k = len(w5.taps)
    res = {}
    for pi, p_acc in enumerate(w5.accept_p):
        tkv = _filled_kv(rt, torch, T, lens5, cap, dev, 50 + pi)
        dkv = _filled_kv(rt, torch, D, lens5, cap, dev, 60 + pi)
        ws_d = rt.Workspace(draft.workspace_bytes(nb, B, dkv.capacity, nb * B), dev)
        ws_t = rt.Workspace(target.workspace_bytes(nb, B, tkv.capacity), dev)
        feats = torch.zeros(nb, B, k * T.hidden, dtype=torch.bfloat16, device=dev)
        gv = torch.zeros(nb, B, dtype=torch.int32, device=dev)
        tau = torch.zeros(nb, dtype=torch.int32, device=dev)
        bonus = torch.zeros(nb, dtype=torch.int32, device=dev)
        drafts = torch.zeros(nb, B - 1, dtype=torch.int32, device=dev)
        rs = torch.arange(nb, dtype=torch.int32, device=dev).repeat_interleave(B)
        rp = torch.arange(B, dtype=torch.int32, device=dev).repeat(nb)
        anchor = synth.anchors(w5, dev)
        t_draft, t_ver, taus = [], [], []
        for c in range(cycles):
            t_draft.append(_timed(torch, lambda: rt.draft_block(draft, dkv, anchor, B, drafts, ws_d), 1))
            # untimed pre-pass: the target's greedy continuation g*_0 .. g*_f of every sequence
            coins = synth.force_coins(1234 + pi, c, nb, B, p_acc)
            own = drafts.cpu().numpy()
            d = own.copy()
            fmax = int(max(np.argmin(np.append(cr, False)) for cr in coins))
            gstar = np.zeros((nb, B), dtype=np.int64)
            for j in range(fmax + 1):
                rt.verify_accept(target, tkv, anchor, torch.tensor(d, dtype=torch.int32, device=dev),
                                 B, feats, gv, tau, bonus, ws_t)
                gj = gv.cpu().numpy()
                gstar[:, j] = gj[:, j]
                if j < B - 1:
                    d[:, j] = gj[:, j]
            forced = np.stack([synth.forced_drafts(coins[b], gstar[b], own[b], T.vocab)[0] for b in range(nb)])
            drafts.copy_(torch.tensor(forced, dtype=torch.int32))
            torch.cuda.synchronize()

            def verify_cycle():
                rt.verify_accept(target, tkv, anchor, drafts, B, feats, gv, tau, bonus, ws_t)
                rt.inject_ctx(draft, dkv, feats.view(nb * B, -1), rs, rp, 1, B, ws_d)
                rt.kv_commit(tkv, dkv, tau, B)
            t_ver.append(_timed(torch, verify_cycle, 1))
            taus.append(tau.cpu().numpy().astype(float))
            anchor = bonus.clone()
        assert int(tkv.err.item()) == 0 and int(dkv.err.item()) == 0
        tau_mean = float(np.mean(taus))
        td, tv = float(np.mean(t_draft)), float(np.mean(t_ver))
        res[str(p_acc)] = {"tau_mean": round(tau_mean, 3),
                           "alpha": round((tau_mean - 1.0) / (B - 1), 4),
                           "expected_tau": round(1.0 + sum(p_acc ** j for j in range(1, B)), 3),
                           "us_draft": round(td, 2), "us_verify_inject_commit": round(tv, 2),
                           "L_us_per_token": round((td + tv) / tau_mean, 2)}
        log(f"batch 8, p={p_acc}: tau {tau_mean:.2f}, draft {td:.0f} us, verify+inject+commit {tv:.0f} us")
        del tkv, dkv, ws_d, ws_t
        torch.cuda.empty_cache()
    out["qwen3_8b_cycle_b8"] = res
    return out


def sampled_cycles(draft, target, dkv, tkv, ws_d, ws_t, anchor, B, n_taps, D, T, dev, cycles=12):
    """Cycles of sampled drafting (T = 1), rejection-sampling verification, injection and
    commit on the bench's caches: µs of the drafting and verifying calls and the mean tau
    (random synthetic weights, so the drafter and target barely agree)."""
    import torch
    from block_diffusion_drafter_03_amd import runtime as rt

    zd = torch.zeros(1, B - 1, D.vocab, device=dev)
    zt = torch.zeros(1, B, T.vocab, device=dev)
    drafts = torch.zeros(1, B - 1, dtype=torch.int32, device=dev)
    feats = torch.zeros(1, B, n_taps * D.hidden, dtype=torch.bfloat16, device=dev)
    tau = torch.zeros(1, dtype=torch.int32, device=dev)
    nxt = torch.zeros(1, dtype=torch.int32, device=dev)
    rseq = torch.zeros(B, dtype=torch.int32, device=dev)
    rpos = torch.arange(B, dtype=torch.int32, device=dev)
    a = anchor.clone()
    seq0 = int(tkv.seq_len.item())
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(cycles)]
    for c in range(cycles):
        ev = evs[c]
        ev[0].record()
        rt.draft_block_sampled(draft, dkv, a, B, 1.0, 2024, c, drafts, zd, ws_d)
        ev[1].record()
        rt.verify_sampled(target, tkv, a, drafts, zd, B, 1.0, 2024, c, feats, zt, tau, nxt, ws_t)
        ev[2].record()
        rt.inject_ctx(draft, dkv, feats.view(B, -1), rseq, rpos, 1, B, ws_d)
        rt.kv_commit(tkv, dkv, tau, B)
        a = nxt.clone()
    torch.cuda.synchronize()
    assert int(tkv.err.item()) == 0 and int(dkv.err.item()) == 0
    us_d = sum(e[0].elapsed_time(e[1]) for e in evs[2:]) * 1e3 / (cycles - 2)
    us_v = sum(e[1].elapsed_time(e[2]) for e in evs[2:]) * 1e3 / (cycles - 2)
    return {"us_per_sampled_draft_block": round(us_d, 2), "us_per_sampled_verify": round(us_v, 2),
            "tau_mean": round((int(tkv.seq_len.item()) - seq0) / cycles, 3),
            "note": "drafter and target weights are independent random draws"}


def selector_timing(w, draft, dkv, ws_d, anchor, B, D, dev, reps=10):
    """µs per draft block with the DFlash 2 path selector (rank 256, top-16; synthetic
    selector weights) against the plain greedy draft block on the same cache."""
    import torch
    import synth
    from block_diffusion_drafter_03_amd import runtime as rt

    sw = synth.selector_weights(w, rank=256, device=dev)
    sel = rt.Selector(draft, sw["w_a"], sw["w_b"], sw["w_h"], top_k=16)
    sws = rt.Workspace(sel.workspace_bytes(draft, 1, B), dev)
    ids = torch.zeros(1, B - 1, dtype=torch.int32, device=dev)
    zd = torch.zeros(1, B - 1, D.vocab, device=dev)
    out = {}
    for name, call in (("greedy", lambda: rt.draft_block(draft, dkv, anchor, B, ids, ws_d)),
                       ("selector", lambda: rt.draft_block_select(draft, dkv, anchor, B, sel, ids, zd,
                                                                  ws_d, sws))):
        for _ in range(3):
            call()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            call()
        e1.record()
        torch.cuda.synchronize()
        out["us_per_draft_block_" + name] = round(e0.elapsed_time(e1) * 1e3 / reps, 2)
    assert int(dkv.err.item()) == 0
    out["overhead_frac"] = round(out["us_per_draft_block_selector"] / out["us_per_draft_block_greedy"] - 1, 4)
    return out


def dconv_timing(w, dw, shared, dkv, anchor, B, D, n, dev, reps=10):
    """µs per draft block of the drafter with DFlash 2 convolutions (synthetic weights)
    against the plain drafter, on the same injected context."""
    import torch
    import synth
    from block_diffusion_drafter_03_amd import runtime as rt

    conv = rt.Model(D, dw, shared, n_taps=w.n_taps, draft=True, dconv=synth.dconv_weights(w, dev))
    plain = rt.Model(D, dw, shared, n_taps=w.n_taps, draft=True)
    ws = rt.Workspace(conv.workspace_bytes(1, B, dkv.capacity), dev)
    ids = torch.zeros(1, B - 1, dtype=torch.int32, device=dev)
    out = {}
    for name, model in (("plain", plain), ("dconv", conv)):
        for _ in range(3):
            rt.draft_block(model, dkv, anchor, B, ids, ws)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            rt.draft_block(model, dkv, anchor, B, ids, ws)
        e1.record()
        torch.cuda.synchronize()
        out["us_per_draft_block_" + name] = round(e0.elapsed_time(e1) * 1e3 / reps, 2)
    assert int(dkv.err.item()) == 0
    out["overhead_frac"] = round(out["us_per_draft_block_dconv"] / out["us_per_draft_block_plain"] - 1, 4)
    conv.close()
    plain.close()
    return out


def context_sweep(draft, shape, B, dev, contexts=(4096, 65536, 262144), reps=20):
    """Draft block at batch 1 over synthetic N(0,1) context K/V of each length: µs per draft
    block, and the attention launches (split-K kernel + merge) of every layer timed with
    the library's event hook, with their algorithmic HBM bytes (context K/V, block K/V,
    queries in, output out) per launch."""
    import torch
    from block_diffusion_drafter_03_amd import _lib
    from block_diffusion_drafter_03_amd import runtime as rt

    L, Hkv, d, Hq = shape.n_layers, shape.n_kv_heads, shape.head_dim, shape.n_q_heads
    out = {}
    for n in contexts:
        kv = rt.PagedKV(shape, 1, n + B + 64, torch.bfloat16, dev)
        gen = torch.Generator(device=dev).manual_seed(n)
        for t in kv.k + kv.v:
            t.normal_(generator=gen)
        kv.set_seq_len(n)
        ws = rt.Workspace(draft.workspace_bytes(1, B, kv.capacity), dev)
        anchor = torch.zeros(1, dtype=torch.int32, device=dev)
        ids = torch.zeros(1, B - 1, dtype=torch.int32, device=dev)
        for _ in range(2):
            rt.draft_block(draft, kv, anchor, B, ids, ws)
        torch.cuda.synchronize()
        _lib.timing_arm(_lib.KERNEL_ATTENTION, reps * L)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for e0, e1 in evs:
            e0.record()
            rt.draft_block(draft, kv, anchor, B, ids, ws)
            e1.record()
        torch.cuda.synchronize()
        attn_ms = _lib.timing_read(reps * L)
        assert int(kv.err.item()) == 0
        blk = stats([e0.elapsed_time(e1) * 1e3 for e0, e1 in evs])
        att = stats([x * 1e3 for x in attn_ms])
        blk_us, attn_us = blk["median"], att["median"]
        nbytes = (n + B) * Hkv * d * 2 * 2 + B * Hq * d * 4 * 2
        gbs = nbytes / (attn_us * 1e-6) / 1e9
        out[str(n)] = {"us_per_draft_block": blk,
                       "draft_tok_s": round((B - 1) / (blk_us * 1e-6), 1),
                       "attention_us_per_layer": att,
                       "attention_bytes_per_layer": int(nbytes),
                       "attention_gbs": round(gbs, 1),
                       "attention_hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
        log(f"context {n}: draft block {blk_us:.1f} us, attention {attn_us:.1f} us/layer ({gbs:.0f} GB/s)")
        del kv, ws
        torch.cuda.empty_cache()
    return out


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, wt, dw, tw, shared, feats0, anchor, tkv, reps, gpu_value):
    """The oracle on the host cores, on a bounded sample of the bench workload: the drafter's
    4096-row context injected once (timed), `reps` draft blocks, and a few of each other call
    of the cycle (16-row and 512-row injections, verification by the 8-layer target over its
    4096-token cache read back from the GPU, acceptance, commit)."""
    import numpy as np
    import synth
    import oracle as O
    from threadpoolctl import threadpool_info, threadpool_limits

    cores = len(os.sched_getaffinity(0))

    def med(fn, k):
        ts = []
        for _ in range(k):
            t0 = time.perf_counter()
            r = fn()
            ts.append(time.perf_counter() - t0)
        return sorted(ts)[len(ts) // 2] * 1e3, r

    with threadpool_limits(limits=cores):
        info = threadpool_info()
        used = max([i.get("num_threads", 1) for i in info] or [1])
        blas = sorted({f"{i.get('internal_api')} {i.get('version')}" for i in info if i.get("user_api") == "blas"})
        log(f"cpu baseline: copying weights to host ({cores} cores)")
        np_dw = {k: synth.to_numpy(v) for k, v in dw.items()}
        np_sh = {k: synth.to_numpy(v) for k, v in shared.items()}
        np_tw = {k: synth.to_numpy(v) for k, v in tw.items()}
        D, T, B, n = w.draft, wt.target, w.block, w.ctx[0]
        f_np = synth.to_numpy(feats0)
        calls = {}
        t0 = time.perf_counter()
        ctx = O.inject(f_np, np.arange(n), np_dw, D, store="bf16")
        calls["inject_ctx_4096_rows"] = round((time.perf_counter() - t0) * 1e3, 1)
        calls["inject_ctx_512_rows"] = round(med(lambda: O.inject(f_np[:512], np.arange(512), np_dw, D,
                                                                  store="bf16"), 3)[0], 1)
        calls["inject_ctx_16_rows"] = round(med(lambda: O.inject(f_np[:16], n + np.arange(16), np_dw, D,
                                                                 store="bf16"), 3)[0], 2)
        a = int(anchor[0])
        log(f"cpu baseline: timing {reps} oracle draft blocks")
        ts = []
        drafts = None
        for _ in range(reps):
            t0 = time.perf_counter()
            drafts, _, _ = O.draft_block(np_dw, np_sh, D, ctx, a, n, B, store="bf16")
            ts.append(time.perf_counter() - t0)
        t_draft = sorted(ts)[len(ts) // 2]
        calls["draft_block"] = round(t_draft * 1e3, 1)
        tcache = []
        for l in range(T.n_layers):
            K, V = tkv.read_dense(l, 0, n)
            tcache.append((synth.to_numpy(K), synth.to_numpy(V)))
        block = [a] + [int(x) for x in drafts]
        t_ver, (g, _, feats, new_kv, _) = med(lambda: O.verify(np_tw, np_sh, T, tcache, block, n, wt.taps,
                                                               store="bf16"), 3)
        calls["verify"] = round(t_ver, 1)
        t_acc, (_, tau, _) = med(lambda: O.accept(np.asarray(drafts), g), 1001)
        calls["accept"] = round(t_acc, 4)
        calls["kv_commit"] = round(med(lambda: O.commit(tcache, ctx, new_kv, feats, tau, n, np_dw, D,
                                                         store="bf16"), 3)[0], 2)
    return {"value": round((B - 1) / t_draft, 2), "unit": "draft tok/s", "cores": used, "kind": "oracle",
            "sample": f"{reps} oracle draft blocks (float32 NumPy, same weights and injected context), "
                      f"median {t_draft:.3f} s; other calls median of 3 (accept: 1001)",
            "calls_ms": calls, "cpu_model": _cpu_model(), "blas": blas, "blas_threads": used,
            "gpu_over_cpu": round(gpu_value / ((B - 1) / t_draft), 1)}


if __name__ == "__main__":
    main()
