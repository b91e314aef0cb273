"""Seeded synthetic inputs for tree verification (shared by the oracle's tests and the GPU path).

This package only *draws* inputs: token trees as parent arrays, Q/K/V, KV-cache layouts
(contiguous or paged with a shuffled block table), target logits, draft tokens and
uniform draws, and a sampling drafter's logits and tokens.  It holds none of the method's arithmetic (no masks, no softmax, no
acceptance, no compaction); both the CPU oracle and the HIP library receive the same
arrays from here and compute independently.

The five workloads mirror the verification configurations of EAGLE/EAGLE-2 as
described in "SGLang EAGLE-2 Speculative Decoding" (Tech Radar, sec. 2, dynamic
tree-attention masking: trees of at most 64 nodes, depth 4-6, width 8) and the
Llama-2-7B / Llama-3-70B layer shapes.
"""
from .configs import CONFIGS, Config, config_by_name, scaled
from .generate import (Inputs, draft_tree_logits, generate, quantize_int4, round_to_bf16,
                       sampled_drafts, static_tree_26)

__all__ = [
    "CONFIGS", "Config", "config_by_name", "scaled",
    "Inputs", "draft_tree_logits", "generate", "quantize_int4", "round_to_bf16", "sampled_drafts",
    "static_tree_26",
]
