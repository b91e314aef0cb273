"""Pins of the oracle's tree attention.

What fixes the result (Tech Radar sec. 2, mask equation M and sequence diagram; EAGLE
explainer "Core idea"): one pass in which every node sees the prefix plus its own
ancestors and itself.  Hence a chain-shaped tree is ordinary causal attention, and each
root-to-leaf path is exactly causal attention on that path alone.
"""
import math

import numpy as np
import pytest
import torch

from oracle import gather_paged, tree_attention, tree_attention_batch, tree_mask, tree_mask_batch
from synth import CONFIGS, generate, scaled


def sdpa(q, k, v, mask=None):
    """torch scaled_dot_product_attention on CPU in float64. q [Tq][d], k/v [Tk][d]."""
    tq = torch.from_numpy(np.asarray(q, np.float64))[None, None]
    tk = torch.from_numpy(np.asarray(k, np.float64))[None, None]
    tv = torch.from_numpy(np.asarray(v, np.float64))[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=m)[0, 0].numpy()


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("L,T,G", [(0, 1, 1), (5, 7, 2), (37, 16, 4), (128, 64, 1)])
def test_chain_tree_is_causal_attention(L, T, G):
    Hkv, d = 2, 32
    Hq = Hkv * G
    q = rand((T, Hq, d), 1)
    k = rand((Hkv, L + T, d), 2)
    v = rand((Hkv, L + T, d), 3)
    anc, _ = tree_mask(list(range(-1, T - 1)))
    O, LSE = tree_attention(q, k, v, L, anc)
    causal = np.tril(np.ones((T, L + T), dtype=bool), k=L)
    for h in range(Hq):
        g = h // G
        ref = sdpa(q[:, h], k[g], v[g], causal)
        assert np.abs(O[:, h] - ref).max() < 1e-12
        s = torch.from_numpy(q[:, h] @ k[g].T / math.sqrt(d))
        s = s.masked_fill(~torch.from_numpy(causal), -math.inf)
        assert np.abs(LSE[:, h] - torch.logsumexp(s, dim=1).numpy()).max() < 1e-12


@pytest.mark.parametrize("seed", range(6))
def test_each_root_to_leaf_path_is_independent_causal_attention(seed):
    rng = np.random.default_rng(100 + seed)
    T = int(rng.integers(2, 14))
    parent = [-1] + [int(rng.integers(i)) for i in range(1, T)]
    L, Hkv, G, d = int(rng.integers(0, 9)), 2, 2, 16
    Hq = Hkv * G
    q = rand((T, Hq, d), seed)
    k = rand((Hkv, L + T, d), seed + 1)
    v = rand((Hkv, L + T, d), seed + 2)
    anc, _ = tree_mask(parent)
    O, LSE = tree_attention(q, k, v, L, anc)
    leaves = [i for i in range(T) if i not in parent]
    for leaf in leaves:
        path = []
        u = leaf
        while u != -1:
            path.append(u)
            u = parent[u]
        path = path[::-1]                       # root .. leaf
        slots = list(range(L)) + [L + j for j in path]
        n = len(path)
        causal = np.tril(np.ones((n, L + n), dtype=bool), k=L)
        for h in range(Hq):
            g = h // G
            ref = sdpa(q[path, h], k[g][slots], v[g][slots], causal)
            assert np.abs(O[path, h] - ref).max() < 1e-12


def test_single_node_is_plain_decode_attention():
    L, Hq, d = 300, 4, 64
    q = rand((1, Hq, d), 5)
    k = rand((Hq, L + 1, d), 6)
    v = rand((Hq, L + 1, d), 7)
    anc, _ = tree_mask([-1])
    O, _ = tree_attention(q, k, v, L, anc)
    for h in range(Hq):
        assert np.abs(O[0, h] - sdpa(q[:, h], k[h], v[h])[0]).max() < 1e-12


def test_closed_forms_constant_values_and_zero_keys():
    rng = np.random.default_rng(9)
    T = 20
    parent = [-1] + [int(rng.integers(i)) for i in range(1, T)]
    anc, depth = tree_mask(parent)
    L, Hkv, G, d = 50, 2, 3, 16
    q = rand((T, Hkv * G, d), 10)
    k = rand((Hkv, L + T, d), 11)
    O, _ = tree_attention(q, k, np.ones((Hkv, L + T, d)), L, anc)
    assert np.abs(O - 1.0).max() < 1e-12             # convex combination of ones
    _, LSE = tree_attention(q, np.zeros((Hkv, L + T, d)), k, L, anc)
    expect = np.log(L + depth + 1.0)                   # all scores 0: ln(#visible keys)
    assert np.abs(LSE - expect[:, None]).max() < 1e-12


def test_prefix_permutation_invariance():
    rng = np.random.default_rng(12)
    T, L, Hkv, G, d = 9, 40, 2, 2, 16
    parent = [-1] + [int(rng.integers(i)) for i in range(1, T)]
    anc, _ = tree_mask(parent)
    q = rand((T, Hkv * G, d), 13)
    k = rand((Hkv, L + T, d), 14)
    v = rand((Hkv, L + T, d), 15)
    O, LSE = tree_attention(q, k, v, L, anc)
    perm = np.concatenate([rng.permutation(L), np.arange(L, L + T)])
    O2, LSE2 = tree_attention(q, k[:, perm], v[:, perm], L, anc)
    assert np.abs(O - O2).max() < 1e-12 and np.abs(LSE - LSE2).max() < 1e-12


def test_gqa_equals_mha_with_repeated_kv_heads():
    rng = np.random.default_rng(16)
    T, L, Hkv, G, d = 11, 30, 2, 4, 8
    parent = [-1] + [int(rng.integers(i)) for i in range(1, T)]
    anc, _ = tree_mask(parent)
    q = rand((T, Hkv * G, d), 17)
    k = rand((Hkv, L + T, d), 18)
    v = rand((Hkv, L + T, d), 19)
    O, LSE = tree_attention(q, k, v, L, anc)
    O2, LSE2 = tree_attention(q, np.repeat(k, G, axis=0), np.repeat(v, G, axis=0), L, anc)
    assert np.abs(O - O2).max() < 1e-14 and np.abs(LSE - LSE2).max() < 1e-14


def test_masked_slots_are_not_read():
    """NaN in every non-ancestor tree slot and beyond L+T leaves the outputs finite."""
    T, L, H, d = 6, 10, 1, 8
    parent = [-1, 0, 0, 1, 2, 2]
    anc, _ = tree_mask(parent)
    q = rand((T, H, d), 20)
    k = rand((H, L + T + 4, d), 21)
    v = rand((H, L + T + 4, d), 22)
    k[:, L + T:] = np.nan
    v[:, L + T:] = np.nan
    O, LSE = tree_attention(q, k, v, L, anc)
    assert np.isfinite(O).all() and np.isfinite(LSE).all()
    # node 3's output must not change when a non-ancestor tree slot changes
    k2 = k.copy()
    k2[:, L + 5] += 100.0                               # node 5 is not an ancestor of node 3
    O2, _ = tree_attention(q, k2, v, L, anc)
    assert np.array_equal(O[3], O2[3])


def test_paged_gather_equals_contiguous_layout():
    cfg = scaled(CONFIGS[3], B=3, L=(20, 70), V=32, T=9, Hq=4, Hkv=2, d=16)
    a = generate(cfg, layout="contiguous", with_logits=False)
    b = generate(cfg, layout="paged", with_logits=False)
    for s in range(cfg.B):
        n = int(a.prefix_len[s]) + cfg.T
        kp = gather_paged(b.k, b.block_table[s], n, cfg.block_size)
        assert np.array_equal(kp, a.k[s, :, :n])
    anc, _ = tree_mask_batch(a.parent)
    Oa, La = tree_attention_batch(a.q, a.k, a.v, a.prefix_len, anc)
    Ob, Lb = tree_attention_batch(b.q, b.k, b.v, b.prefix_len, anc, layout="paged",
                                  block_table=b.block_table, block_size=cfg.block_size)
    assert np.array_equal(Oa, Ob) and np.array_equal(La, Lb)
    assert np.isfinite(Oa).all()
