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


def remap_plan(L: int, path, k: int, T: int, block_size: int):
    """Plan of a zero-copy compaction of one sequence ([TR] sec. 4: KV fragmentation and
    the radix cache; sec. 2: keep the accepted branch's KV).

    Destination slots L+1 .. L+k live in logical blocks X.  A block whose slots all lie
    past the root (X*bs > L) and whose moves share one offset a_m - m = D (a multiple of
    bs) needs no data movement: with D = 0 its content is already in place ("keep"); with
    D > 0 the block-table entry of X takes that of block X + D/bs ("remap").  Every other
    destination block is written by copying rows ("copy").  A remap whose source block is
    itself a live copy block would see its content overwritten, so it becomes a copy
    block too, repeated until no such remap is left.
    Returns {X: "keep" | "copy" | ("remap", source block)} for the blocks holding
    destination slots.
    """
    bs = block_size
    plan = {}
    for m in range(1, k + 1):
        plan.setdefault((L + m) // bs, []).append(m)
    out = {}
    for X, ms in plan.items():
        offsets = {int(path[m]) - m for m in ms}
        if X * bs <= L or len(offsets) != 1:
            out[X] = "copy"
            continue
        D = offsets.pop()
        if D == 0:
            out[X] = "keep"
        elif D % bs == 0:
            out[X] = ("remap", X + D // bs)
        else:
            out[X] = "copy"
    changed = True
    while changed:
        changed = False
        for X, p in sorted(out.items()):
            if isinstance(p, tuple) and out.get(p[1]) == "copy":
                out[X] = "copy"
                changed = True
    return out


def kv_compact_remap(k: np.ndarray, v: np.ndarray, prefix_len, path, accept_len, block_table,
                     block_size: int, T: int, layered: bool = False):
    """Zero-copy compaction of a paged cache: returns (k', v', table', new_len, freed,
    copied).

    table' is the block table after the remaps, with the entries of blocks at or beyond
    ceil(new_len / bs) that held tree slots set to -1; freed[b] lists, in ascending
    logical-block order, the physical blocks of the tree's blocks (those from block
    L // bs on) that table' no longer references among its live blocks; copied[b] counts
    the slots moved by copying.  The logical content of slots 0 .. new_len-1 equals
    kv_compact's.
    """
    k = np.array(k, copy=True)
    v = np.array(v, copy=True)
    table = np.array(block_table, copy=True)
    bs = block_size
    B = len(prefix_len)
    layers = range(k.shape[0]) if layered else [None]
    new_len = np.zeros(B, dtype=np.int32)
    freed, copied = [], np.zeros(B, dtype=np.int32)
    for b in range(B):
        L, kb = int(prefix_len[b]), int(accept_len[b])
        n_old = -(-(L + T) // bs)
        n_new = -(-(L + kb + 1) // bs)
        old = [int(x) for x in table[b]]
        plan = remap_plan(L, path[b], kb, T, bs)
        # copies read through the old table and write blocks whose entries do not change;
        # ascending m is safe in place (a_m >= m)
        for m in range(1, kb + 1):
            if plan[(L + m) // bs] != "copy":
                continue
            copied[b] += 1
            for layer in layers:
                for cache in (k, v):
                    base = cache if layer is None else cache[layer]
                    s, d = L + int(path[b][m]), L + m
                    base[old[d // bs], :, d % bs] = base[old[s // bs], :, s % bs]
        for X, p in plan.items():
            if isinstance(p, tuple):
                table[b][X] = old[p[1]]
        for X in range(n_new, n_old):
            table[b][X] = -1
        live = {int(table[b][X]) for X in range(L // bs, n_new)}
        fb = []
        for X in range(L // bs, n_old):
            if old[X] not in live and old[X] not in fb:
                fb.append(old[X])
        freed.append(fb)
        new_len[b] = L + kb + 1
    return k, v, table, new_len, freed, copied
