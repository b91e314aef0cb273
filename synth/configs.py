"""The five verification workloads, C1..C5, and helpers to shrink them for tests.

Each workload is one transformer layer's worth of tree verification for a batch of
sequences: tree attention of T node queries over a KV prefix of length L plus the
tree's own slots, then greedy and/or rejection acceptance over V-way logits, then
compaction of the accepted path's KV.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Tuple, Union


@dataclass(frozen=True)
class Config:
    name: str
    index: int                      # 1..5; the seed is 1000 + index
    B: int                          # sequences
    Hq: int                         # query heads
    Hkv: int                        # KV heads (Hq % Hkv == 0)
    d: int                          # head dim
    dtype: str                      # "f32" or "bf16" for Q/K/V/O
    L: Union[int, Tuple[int, int]]  # prefix length, fixed or inclusive range per sequence
    paged: bool
    block_size: int                 # paged KV block size (slots)
    T: int                          # tree nodes including the root
    tree: str                       # "spine3", "static26", "grow", "grow_spine6"
    max_depth: int
    max_children: int
    V: int                          # vocabulary
    accept: Tuple[str, ...]         # subset of ("greedy", "rejection")
    tau: float                      # rejection temperature
    compact: bool
    workload: str = ""              # human description

    def prefix_range(self) -> Tuple[int, int]:
        if isinstance(self.L, tuple):
            return self.L
        return (self.L, self.L)


CONFIGS = (
    Config("tiny_fp32", 1, B=1, Hq=4, Hkv=4, d=64, dtype="f32", L=128, paged=False,
           block_size=16, T=8, tree="spine3", max_depth=3, max_children=8, V=1000,
           accept=("greedy",), tau=0.7, compact=True,
           workload="tiny tree verify, fp32, MHA 4x64, L=128, 8-node tree depth 3, V=1000"),
    Config("llama2_7b_layer", 2, B=1, Hq=32, Hkv=32, d=128, dtype="bf16", L=2048, paged=False,
           block_size=16, T=26, tree="static26", max_depth=5, max_children=4, V=32000,
           accept=("greedy",), tau=0.7, compact=True,
           workload="Llama-2-7B-shaped layer, MHA 32x128, bf16, L=2048, static 26-node tree, V=32000"),
    Config("llama3_70b_layer", 3, B=1, Hq=64, Hkv=8, d=128, dtype="bf16", L=4096, paged=False,
           block_size=16, T=64, tree="grow", max_depth=6, max_children=8, V=128256,
           accept=("rejection",), tau=0.7, compact=True,
           workload="Llama-3-70B-shaped layer, GQA 64/8 d128, bf16, L=4096, 64-node tree, V=128256"),
    Config("batched_paged", 4, B=16, Hq=64, Hkv=8, d=128, dtype="bf16", L=(512, 8192), paged=True,
           block_size=16, T=64, tree="grow", max_depth=6, max_children=8, V=128256,
           accept=("rejection",), tau=0.7, compact=True,
           workload="batched paged verify, B=16, GQA 64/8 d128, bf16, L~U[512,8192], block 16"),
    Config("long_context", 5, B=4, Hq=64, Hkv=8, d=128, dtype="bf16", L=32768, paged=True,
           block_size=16, T=64, tree="grow_spine6", max_depth=6, max_children=8, V=128256,
           accept=("greedy", "rejection"), tau=0.7, compact=True,
           workload="long-context verify, B=4, GQA 64/8 d128, bf16, paged L=32768, depth-6 tree"),
)


def config_by_name(name: str) -> Config:
    for c in CONFIGS:
        if c.name == name or f"C{c.index}" == name:
            return c
    raise KeyError(name)


def scaled(cfg: Config, **overrides) -> Config:
    """A copy of `cfg` with some fields replaced (smaller L, V, B for tests)."""
    return dataclasses.replace(cfg, **overrides)
