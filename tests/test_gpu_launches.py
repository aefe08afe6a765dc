"""Each GEMM of a draft block is launched once: the LM head, whose kernel forms differ by row
count (the M <= 16 GEMV, the four- or eight-wave row-resident GEMM at 17 - 128 rows, the
weight-direct tiles beyond), must appear exactly once among the block's kernels (a second
launch would give the same ids and logits, so parity cannot see it)."""
import re

import pytest
import torch

import synth
from block_diffusion_drafter_03_amd import runtime as rt

from harness import DEV, Setup, inject_all

pytestmark = pytest.mark.gpu


def _kernel_names(fn):
    from torch.profiler import ProfilerActivity, profile
    with profile(activities=[ProfilerActivity.CUDA]) as prof:
        fn()
        torch.cuda.synchronize()
    return [e.name for e in prof.events() if e.device_type.name == "CUDA"]


@pytest.mark.parametrize("name", ["split_bf16", "vast5_bf16", "vast_bf16"])
def test_lm_head_launched_once_per_draft_block(name):
    w = synth.workload(name)
    S = Setup(w)
    lens = synth.ctx_lengths(w)
    B = w.block
    kv = S.kv(w.draft, max(lens) + B + 70)
    ws = S.workspace(S.draft, B, kv.capacity, inject_rows=sum(lens))
    inject_all(S, kv, [synth.features(w, n, DEV, tag=f"feats.b{b}") for b, n in enumerate(lens)], ws)
    anchor = synth.anchors(w, DEV)
    ids = torch.zeros(w.batch, B - 1, dtype=torch.int32, device=DEV)
    run = lambda: rt.draft_block(S.draft, kv, anchor, B, ids, ws)
    run()
    torch.cuda.synchronize()
    names = _kernel_names(run)
    if not any("dflash" in n for n in names):
        pytest.skip("the profiler records no device kernels on this build")
    # the LM head is the only argmax-epilogue GEMM of a draft block (epilogue kind 5, a
    # template argument of every GEMM kernel: "..., 5>" / "..., 5, ..." demangled, "Li5E"
    # mangled)
    kind5 = re.compile(r"[<,] ?5[,>]|Li5E")
    lm = [n for n in names if "dflash" in n and "gemm" in n and "reduce" not in n and kind5.search(n)]
    assert len(lm) == 1, f"{name}: LM head launched {len(lm)} times: {lm}"
