"""Seeded synthetic inputs shared by the HIP path's tests/bench and by the oracle.

This package holds shapes and random-number draws only: no step of the drafter,
the verifier or the acceptance rule is computed here.  Every tensor is drawn from
a ``torch.Generator`` seeded by a stable hash of ``(workload id, tensor name)``,
on whatever device the caller names, so the HIP path and the oracle always read
the very same values (the oracle receives host copies upcast to float32).
"""
from .configs import (ModelShape, Workload, WORKLOADS, workload, TINY, MID,
                      QWEN3_8B_DRAFT, QWEN3_8B_TARGET)
from .fixtures import (seed_of, normal, uniform_ints, model_weights, shared_weights, selector_weights,
                       dconv_shapes, dconv_weights, DCONV_NAMES,
                       features, anchors, ctx_lengths, synthetic_ctx_kv, to_numpy,
                       splitmix64, force_coins, forced_drafts, prompt_tokens)

__all__ = [
    "ModelShape", "Workload", "WORKLOADS", "workload", "TINY", "MID",
    "QWEN3_8B_DRAFT", "QWEN3_8B_TARGET",
    "seed_of", "normal", "uniform_ints", "model_weights", "shared_weights", "features",
    "anchors", "ctx_lengths", "synthetic_ctx_kv", "to_numpy", "splitmix64",
    "force_coins", "forced_drafts", "prompt_tokens",
]
