"""CPU oracle for tree verification — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct numpy implementation (float64 wherever floating point
is involved) of what one verification pass of a drafted token tree computes:

  tree.py       ancestor mask of a parent[] tree
  attention.py  tree-masked attention with an explicit mask, contiguous or paged KV
  accept.py     greedy longest-matching walk and rejection-sampling walk
  stochastic.py rejection-sampling walk for drafts sampled from a draft distribution
  compact.py    accepted-path KV compaction
  tree_build.py dynamic draft-tree construction (entropy-guided beam expansion)
  quant.py      INT4-quantised KV cache: unpacking and dequantisation

It shares no code with the HIP library and imports nothing from it.  Only the test
suite, the package's smoke check and the benchmark's CPU-baseline leg may import it;
the product path never calls it.

Sources ("the pages"):
  [EX]  "EAGLE — Draft head attached to an internal layer, 3x speedup" (troisinh.com,
        inference-frontier explainer), sections "Core idea" and "Why it works".
  [SN]  "EAGLE — guessing the next step in feature space instead of tokens"
        (estelledc.github.io study note), case 1 (vLLM) and case 3 (why it is lossless).
  [TR]  "Tech Radar: SGLang EAGLE-2 speculative decoding" (learn.tanhdev.com),
        sec. 2 (sequence diagram; dynamic tree-attention masking, mask equation M).

Every function is pinned by tests that do not re-type its formula (closed forms,
brute force, library special cases, invariants, and a chi-square test of the sampler).
The mapping from a given uniform draw to a token (sibling order, inverse-CDF order) is a
convention of this project, not of the pages: the pages pin the *distribution* only.
"""
from .tree import tree_mask, tree_mask_batch
from .attention import tree_attention, tree_attention_batch, gather_paged
from .accept import (greedy_walk, greedy_batch, target_probs, rejection_walk,
                     rejection_batch)
from .compact import kv_compact
from .stochastic import stochastic_walk, stochastic_batch
from .tree_build import TreeBuilder, build_batch, entropy
from .quant import bf16_nearest, dequant_int4, unpack_int4

__all__ = [
    "tree_mask", "tree_mask_batch", "tree_attention", "tree_attention_batch", "gather_paged",
    "greedy_walk", "greedy_batch", "target_probs", "rejection_walk", "rejection_batch",
    "kv_compact", "stochastic_walk", "stochastic_batch", "TreeBuilder", "build_batch", "entropy",
    "bf16_nearest", "dequant_int4", "unpack_int4",
]
