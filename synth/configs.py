"""Workload shapes: the five drafter/verify configurations plus small test-only ones.

Shapes follow the Qwen3-8B-sized drafter the DFlash notes page describes (5 draft
layers, 5 tapped target features, block 16: "DFlash - Block Diffusion for Flash
Speculative Decoding", §6.1 table) and a tiny fp32 model of the same structure.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class ModelShape:
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rms_eps: float = 1e-6
    rope_base: float = 10000.0

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def mask_token_id(self) -> int:
        # The mask token is the last vocabulary row (a descriptor field; any id works).
        return self.vocab - 1


@dataclass(frozen=True)
class Workload:
    cid: int                    # seed namespace
    name: str
    dtype: str                  # "f32" or "bf16": storage type of weights, caches and features
    draft: ModelShape
    n_taps: int                 # k: number of target layers whose outputs feed W_c
    block: int                  # B: anchor + (B-1) mask positions
    batch: int
    ctx: tuple | None           # per-sequence context lengths, or None when drawn (see ctx_rule)
    ctx_rule: tuple | None = None   # ("uniform", lo, hi): seeded integers in [lo, hi]
    target: ModelShape | None = None
    taps: tuple | None = None   # 0-indexed target decoder layers tapped (len == n_taps)
    page: int = 64
    inject_chunk: int | None = None
    accept_p: tuple = field(default_factory=tuple)
    note: str = ""


QWEN3_8B_DRAFT = ModelShape(n_layers=5, hidden=4096, n_q_heads=32, n_kv_heads=8,
                            head_dim=128, ffn=12288, vocab=151936)
QWEN3_8B_TARGET = ModelShape(n_layers=8, hidden=4096, n_q_heads=32, n_kv_heads=8,
                             head_dim=128, ffn=14336, vocab=151936)
_TINY_MODEL = ModelShape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=4, head_dim=64,
                         ffn=768, vocab=4096)

TINY = Workload(
    cid=1, name="tiny_f32", dtype="f32", draft=_TINY_MODEL, n_taps=2, block=4, batch=1,
    ctx=(128,), target=_TINY_MODEL, taps=(0, 1),
    note="2-layer fp32 drafter, D=256, 4x64 heads, F=768, V=4096, B=4, 128 context rows")

CFG2 = Workload(
    cid=2, name="qwen3_8b_b1_ctx4k", dtype="bf16", draft=QWEN3_8B_DRAFT, n_taps=5, block=16,
    batch=1, ctx=(4096,),
    note="Qwen3-8B-shaped drafter step, batch 1, 4096 injected context rows")

CFG3 = Workload(
    cid=3, name="qwen3_8b_b16_paged", dtype="bf16", draft=QWEN3_8B_DRAFT, n_taps=5, block=16,
    batch=16, ctx=None, ctx_rule=("uniform", 2048, 8192),
    note="batch 16, ragged contexts in [2048, 8192] in a 64-token paged cache")

CFG4 = Workload(
    cid=4, name="qwen3_8b_b1_ctx256k", dtype="bf16", draft=QWEN3_8B_DRAFT, n_taps=5, block=16,
    batch=1, ctx=(262144,), inject_chunk=512,
    note="batch 1, 262144-row context; injection timed per 512-row chunk")

CFG5 = Workload(
    cid=5, name="qwen3_8b_cycle_b8", dtype="bf16", draft=QWEN3_8B_DRAFT, n_taps=5, block=16,
    batch=8, ctx=(8192,) * 8, target=QWEN3_8B_TARGET, taps=(1, 2, 3, 4, 5),
    accept_p=(0.3, 0.7, 1.0),
    note="full cycle: draft, 8-layer target verify, accept, commit; forced acceptance rule")

# Test-only: small bf16 model whose sizes span several GEMM / attention tiles and leave
# ragged tails (vocab not a multiple of 16, contexts not a multiple of the page).
_MID_DRAFT = ModelShape(n_layers=2, hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128,
                        ffn=1536, vocab=3000)
_MID_TARGET = ModelShape(n_layers=6, hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128,
                         ffn=1792, vocab=3000)
MID = Workload(
    cid=101, name="mid_bf16", dtype="bf16", draft=_MID_DRAFT, n_taps=2, block=16, batch=3,
    ctx=(200, 333, 64), target=_MID_TARGET, taps=(1, 3),
    note="test-only bf16 model: ragged vocab / contexts, GQA 4, 6-layer target")

# Test-only: a wide vocabulary (LM-head GEMM of 80 block rows over 40000 columns: the
# wide-N MFMA GEMM path, with ragged row and column tails) and degenerate contexts (empty,
# one row, exactly one page, one page plus one row).
_WIDE_DRAFT = ModelShape(n_layers=1, hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128,
                         ffn=1536, vocab=40000)
_WIDE_TARGET = ModelShape(n_layers=2, hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128,
                          ffn=1536, vocab=40000)
WIDE = Workload(
    cid=102, name="wide_bf16", dtype="bf16", draft=_WIDE_DRAFT, n_taps=2, block=16, batch=5,
    ctx=(130, 0, 257, 1, 64), target=_WIDE_TARGET, taps=(0, 1),
    note="test-only bf16 model: vocab 40000, batch 5, contexts 130 / 0 / 257 / 1 / 64")

# Test-only: the mid model at batch 24 (384 block rows: more than one 256-row tile with a
# ragged last one, and LM-head / projection shapes that take the LDS-staged M > 16 GEMM),
# ragged contexts in [1, 300].
MANY = Workload(
    cid=103, name="many_bf16", dtype="bf16", draft=_MID_DRAFT, n_taps=2, block=16, batch=24,
    ctx=None, ctx_rule=("uniform", 1, 300), target=_MID_TARGET, taps=(1, 3),
    note="test-only bf16 model at batch 24: 384 block rows, contexts uniform in [1, 300]")

# Test-only: a narrow bf16 model (hidden 256) at batch 12: 192 block rows whose GEMMs are too
# short in K to split and too small in N for the weight-direct tiles, i.e. the LDS-staged
# M > 16 GEMM on compensated operand planes.
_NARROW_DRAFT = ModelShape(n_layers=2, hidden=256, n_q_heads=2, n_kv_heads=1, head_dim=128,
                           ffn=768, vocab=4000)
_NARROW_TARGET = ModelShape(n_layers=3, hidden=256, n_q_heads=2, n_kv_heads=1, head_dim=128,
                            ffn=768, vocab=4000)
NARROW = Workload(
    cid=104, name="narrow_bf16", dtype="bf16", draft=_NARROW_DRAFT, n_taps=2, block=16, batch=12,
    ctx=None, ctx_rule=("uniform", 1, 200), target=_NARROW_TARGET, taps=(0, 2),
    note="test-only bf16 model: hidden 256, batch 12 (192 block rows), contexts in [1, 200]")

# Test-only: the narrow model with a vocabulary of 120001 rows at batch 17: an LM head of 272
# block rows (five 64-row tiles, the last with 16 rows) over 235 column tiles of 512, more
# than four per CU, i.e. the widest weight-direct tile, with ragged row and column tails.
_VAST_DRAFT = ModelShape(n_layers=1, hidden=256, n_q_heads=2, n_kv_heads=1, head_dim=128,
                         ffn=768, vocab=120001)
_VAST_TARGET = ModelShape(n_layers=2, hidden=256, n_q_heads=2, n_kv_heads=1, head_dim=128,
                          ffn=768, vocab=120001)
VAST = Workload(
    cid=105, name="vast_bf16", dtype="bf16", draft=_VAST_DRAFT, n_taps=2, block=16, batch=17,
    ctx=None, ctx_rule=("uniform", 1, 150), target=_VAST_TARGET, taps=(0, 1),
    note="test-only bf16 model: hidden 256, vocab 120001, batch 17 (272 block rows)")

# Test-only: a batch-1 model whose M = 16 GEMVs take the K-split form on ragged shapes:
# QKV (K = 2560, 192 tiles: two-tile groups, two splits of five steps a wave, the last
# chunk clamped) and down (K = 8192 over 160 tiles: three-tile groups, the last holding
# one tile, four splits).
_SPLIT_DRAFT = ModelShape(n_layers=2, hidden=2560, n_q_heads=16, n_kv_heads=4, head_dim=128,
                          ffn=8192, vocab=5000)
_SPLIT_TARGET = ModelShape(n_layers=2, hidden=2560, n_q_heads=16, n_kv_heads=4, head_dim=128,
                           ffn=8192, vocab=5000)
SPLIT = Workload(
    cid=106, name="split_bf16", dtype="bf16", draft=_SPLIT_DRAFT, n_taps=2, block=16, batch=1,
    ctx=(300,), target=_SPLIT_TARGET, taps=(0, 1),
    note="test-only bf16 model: hidden 2560, FFN 8192, batch 1 (the K-split M = 16 GEMVs)")

# Test-only: the same model at batch 5: an LM head of 80 block rows over 120001 columns (the
# four-wave row-resident GEMM of vocabulary-wide N, one ragged 128-row tile), contexts as
# in the wide model (empty and one-row ones included).
VAST5 = Workload(
    cid=108, name="vast5_bf16", dtype="bf16", draft=_VAST_DRAFT, n_taps=2, block=16, batch=5,
    ctx=(130, 0, 257, 1, 64), target=_VAST_TARGET, taps=(0, 1),
    note="test-only bf16 model: hidden 256, vocab 120001, batch 5 (80 block rows)")

_ALL = (TINY, CFG2, CFG3, CFG4, CFG5, MID, WIDE, MANY, NARROW, VAST, SPLIT, VAST5)
WORKLOADS = {w.cid: w for w in _ALL}
WORKLOADS.update({w.name: w for w in _ALL})


def workload(key) -> Workload:
    return WORKLOADS[key]
