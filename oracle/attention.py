"""Tree-masked attention with an explicit mask (oracle; test infrastructure only).

What is computed ([TR] sec. 2, sequence diagram and mask equation M; [EX] "Core idea";
[SN] case 1): the target model verifies every drafted node in ONE forward pass.  In
each attention layer, the query of tree node i attends to every position of the
sequence's committed KV prefix and to the tree nodes j with M[i][j] = 1 (its ancestors
and itself), never to other branches.

Readings where the pages are silent:
  * the tree's own keys/values sit in cache slots L .. L+T-1 in node order;
  * scores are scaled by 1/sqrt(head_dim) unless a scale is given; LSE uses the natural log;
  * query head h reads KV head h // (Hq / Hkv) (grouped-query attention).

This is the plain definition: for each (sequence, query head) one float64 matmul of
the node queries against all candidate keys, an explicit boolean [T][L+T] mask, a
max-shifted softmax, and a matmul with the values.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np


def gather_paged(pool: np.ndarray, table_row: np.ndarray, n_slots: int,
                 block_size: int) -> np.ndarray:
    """Logical slots 0..n_slots-1 of one sequence from a paged pool [n_blocks][Hkv][bs][d].

    Slot s lives in block table_row[s // bs] at offset s % bs.  Returns [Hkv][n_slots][d].
    """
    slots = np.arange(n_slots)
    blocks = np.asarray(table_row)[slots // block_size]
    if np.any(blocks < 0) or np.any(blocks >= pool.shape[0]):
        raise ValueError("block table entry out of range")
    rows = pool[blocks, :, slots % block_size, :]      # [n_slots][Hkv][d]
    return np.ascontiguousarray(np.transpose(rows, (1, 0, 2)))


def tree_attention(q: np.ndarray, k_seq: np.ndarray, v_seq: np.ndarray, prefix_len: int,
                   anc: np.ndarray, sm_scale: Optional[float] = None,
                   heads: Optional[list] = None) -> tuple[np.ndarray, np.ndarray]:
    """Attention of one sequence's tree nodes.

    q      [T][Hq][d]        node queries
    k_seq  [Hkv][>=L+T][d]   keys by logical slot; v_seq likewise
    anc    [T] uint64        bit j of anc[i] is M[i][j]
    heads  optional subset of query heads to compute (others are left NaN)
    Returns O [T][Hq][d] and LSE [T][Hq], float64.
    """
    q = np.asarray(q, dtype=np.float64)
    T, Hq, d = q.shape
    Hkv = k_seq.shape[0]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    L = int(prefix_len)
    n = L + T
    scale = 1.0 / math.sqrt(d) if sm_scale is None else float(sm_scale)

    mask = np.zeros((T, n), dtype=bool)
    mask[:, :L] = True                      # the whole committed prefix is visible
    for i in range(T):
        bits = int(anc[i])
        for j in range(T):
            if (bits >> j) & 1:
                mask[i, L + j] = True       # ancestor-or-self tree slot

    O = np.full((T, Hq, d), np.nan)
    LSE = np.full((T, Hq), np.nan)
    for h in (range(Hq) if heads is None else heads):
        g = h // G
        K = np.asarray(k_seq[g, :n], dtype=np.float64)
        V = np.asarray(v_seq[g, :n], dtype=np.float64)
        s = (q[:, h, :] @ K.T) * scale
        s = np.where(mask, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        z = e.sum(axis=1, keepdims=True)
        O[:, h, :] = (e / z) @ V
        LSE[:, h] = m[:, 0] + np.log(z[:, 0])
    return O, LSE


def tree_attention_batch(q: np.ndarray, k: np.ndarray, v: np.ndarray, prefix_len: np.ndarray,
                         anc: np.ndarray, layout: str = "contiguous",
                         block_table: Optional[np.ndarray] = None, block_size: int = 16,
                         sm_scale: Optional[float] = None, seqs: Optional[list] = None,
                         heads: Optional[list] = None) -> tuple[np.ndarray, np.ndarray]:
    """tree_attention for every sequence of a batch (or the subset `seqs`).

    contiguous: k, v are [B][Hkv][cap][d]; paged: [n_blocks][Hkv][bs][d] + block_table.
    """
    B, T, Hq, d = q.shape
    O = np.full((B, T, Hq, d), np.nan)
    LSE = np.full((B, T, Hq), np.nan)
    for b in (range(B) if seqs is None else seqs):
        n = int(prefix_len[b]) + T
        if layout == "contiguous":
            ks, vs = k[b], v[b]
        elif layout == "paged":
            ks = gather_paged(k, block_table[b], n, block_size)
            vs = gather_paged(v, block_table[b], n, block_size)
        else:
            raise ValueError(layout)
        O[b], LSE[b] = tree_attention(q[b], ks, vs, int(prefix_len[b]), anc[b], sm_scale, heads)
    return O, LSE
