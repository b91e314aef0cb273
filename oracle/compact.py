"""Accepted-path KV compaction (oracle; test infrastructure only).

[TR] sec. 2, sequence diagram: after verification the target keeps the KV of the
accepted branch and discards the wrong branches.  Reading: the tree's KV was written to
slots L .. L+T-1 in node order, so keeping the accepted path (0 = a_0 < a_1 < ... < a_k)
means moving slot L + a_m to slot L + m for m = 1..k, for K and V, every KV head and
every layer; the root stays at slot L and the new committed length is L + k + 1.
Slots at or beyond L + k + 1 keep whatever they held.

Sequential ascending m is safe in place: a_m >= m, so slot L + m is never the source of
a later move.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def _slot_ref(cache: np.ndarray, layer: Optional[int], b: int, slot: int, layout: str,
              block_table, block_size: int):
    base = cache if layer is None else cache[layer]
    if layout == "contiguous":
        return base, (b, slice(None), slot)
    blk = int(block_table[b][slot // block_size])
    if blk < 0 or blk >= base.shape[0]:
        raise ValueError("block table entry out of range")
    return base, (blk, slice(None), slot % block_size)


def kv_compact(k: np.ndarray, v: np.ndarray, prefix_len, path, accept_len, layout: str,
               block_table=None, block_size: int = 16, layered: bool = False):
    """Return (k', v', new_len) with the accepted path's KV moved next to the prefix.

    contiguous caches are [B][Hkv][cap][d], paged [n_blocks][Hkv][bs][d]; with
    layered=True each carries a leading layer axis.  Inputs are not modified.
    """
    k = np.array(k, copy=True)
    v = np.array(v, copy=True)
    B = len(prefix_len)
    layers = range(k.shape[0]) if layered else [None]
    new_len = np.zeros(B, dtype=np.int32)
    for b in range(B):
        L = int(prefix_len[b])
        kb = int(accept_len[b])
        for layer in layers:
            for cache in (k, v):
                for m in range(1, kb + 1):
                    src = L + int(path[b][m])
                    dst = L + m
                    sb, si = _slot_ref(cache, layer, b, src, layout, block_table, block_size)
                    db, di = _slot_ref(cache, layer, b, dst, layout, block_table, block_size)
                    db[di] = sb[si]
        new_len[b] = L + kb + 1
    return k, v, new_len
