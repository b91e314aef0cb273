"""Ancestor mask of a drafted token tree (oracle; test infrastructure only).

[TR] sec. 2, mask equation M: the tree of at most 64 candidate nodes is encoded as a
non-causal mask with M[i][j] = 1 exactly when node j is node i itself or one of its
ancestors, and 0 otherwise.

Encoding (a reading; the pages give no data structure): the tree arrives as parent[T],
node 0 is the root (the last committed token, parent -1), and 0 <= parent[i] < i for
every other node, so the array is in topological order.  Row i of the mask is kept as a
Python int / uint64 whose bit j is M[i][j]; depth[i] counts edges from the root.
"""
from __future__ import annotations

import numpy as np

MAX_NODES = 64


class TreeError(ValueError):
    pass


def tree_mask(parent) -> tuple[np.ndarray, np.ndarray]:
    """Return (anc uint64[T], depth int32[T]) for one tree, walking each node to the root."""
    parent = [int(p) for p in parent]
    T = len(parent)
    if not 1 <= T <= MAX_NODES:
        raise TreeError(f"tree has {T} nodes; 1..{MAX_NODES} supported")
    if parent[0] != -1:
        raise TreeError("node 0 must be the root (parent -1)")
    for i in range(1, T):
        if not 0 <= parent[i] < i:
            raise TreeError(f"parent[{i}] = {parent[i]} is not an earlier node")
    anc = []
    depth = []
    for i in range(T):
        row = 0
        steps = 0
        u = i
        while u != -1:          # i itself, then each ancestor up to the root
            row |= 1 << u
            steps += 1
            u = parent[u]
        anc.append(row)
        depth.append(steps - 1)
    return np.array(anc, dtype=np.uint64), np.array(depth, dtype=np.int32)


def tree_mask_batch(parent: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """tree_mask over a batch parent[B][T]."""
    parent = np.asarray(parent)
    out = [tree_mask(p) for p in parent]
    return np.stack([a for a, _ in out]), np.stack([d for _, d in out])


def mask_matrix(anc_row_bits: np.ndarray) -> np.ndarray:
    """Expand per-node bit rows into the dense boolean T x T mask M[i][j]."""
    T = len(anc_row_bits)
    M = np.zeros((T, T), dtype=bool)
    for i in range(T):
        bits = int(anc_row_bits[i])
        for j in range(T):
            M[i, j] = (bits >> j) & 1 == 1
    return M
