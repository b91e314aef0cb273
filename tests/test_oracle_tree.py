"""Pins of the oracle's ancestor mask (Tech Radar sec. 2, mask equation M)."""
import json
import os

import numpy as np
import pytest

from oracle import tree_mask, tree_mask_batch
from oracle.tree import TreeError, mask_matrix
from synth import CONFIGS, generate, scaled, static_tree_26


def closure_mask(parent):
    """Ancestor-or-self relation by Warshall's transitive closure of the child->parent edges."""
    T = len(parent)
    R = np.eye(T, dtype=bool)
    for i in range(1, T):
        R[i, parent[i]] = True
    for k in range(T):
        R = R | (R[:, [k]] & R[[k], :])
    return R


def test_golden_hand_written_masks(golden_dir):
    with open(os.path.join(golden_dir, "tree_masks.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        anc, depth = tree_mask(case["parent"])
        assert [int(a) for a in anc] == case["mask"], case["name"]
        assert depth.tolist() == case["depth"], case["name"]


@pytest.mark.parametrize("seed", range(20))
def test_matches_transitive_closure(seed):
    rng = np.random.default_rng(seed)
    T = int(rng.integers(1, 65))
    parent = [-1] + [int(rng.integers(i)) for i in range(1, T)]
    anc, depth = tree_mask(parent)
    M = mask_matrix(anc)
    assert np.array_equal(M, closure_mask(parent))
    # popcount(anc[i]) == depth[i] + 1, and a parent's set is a subset of its child's
    for i in range(T):
        assert bin(int(anc[i])).count("1") == depth[i] + 1
        if i:
            p = parent[i]
            assert int(anc[p]) & ~int(anc[i]) == 0
            assert depth[i] == depth[p] + 1


def test_chain_is_causal_and_star_is_diagonal_plus_root():
    T = 64
    anc, depth = tree_mask(list(range(-1, T - 1)))
    assert np.array_equal(mask_matrix(anc), np.tril(np.ones((T, T), dtype=bool)))
    assert depth.tolist() == list(range(T))
    assert int(anc[63]) == (1 << 64) - 1
    star = [-1] + [0] * (T - 1)
    anc, depth = tree_mask(star)
    expect = np.eye(T, dtype=bool)
    expect[:, 0] = True
    assert np.array_equal(mask_matrix(anc), expect)


@pytest.mark.parametrize("parent", [[], [0], [-1, 1], [-1, 0, 3, 1], [-1, -1], list(range(-1, 64))])
def test_rejects_invalid_trees(parent):
    with pytest.raises(TreeError):
        tree_mask(parent)


def test_workload_tree_shapes():
    # static 26-node tree: depth 5, <= 4 children, depth histogram 1/4/10/6/3/2
    anc, depth = tree_mask(static_tree_26())
    assert np.bincount(depth).tolist() == [1, 4, 10, 6, 3, 2]
    assert int((depth + 1).sum()) == 90
    assert np.bincount(static_tree_26()[1:]).max() <= 4
    for cfg in CONFIGS:
        inp = generate(scaled(cfg, L=32, V=64) if cfg.index != 4 else scaled(cfg, L=(32, 64), V=64, B=4),
                       with_kv=False, with_logits=False)
        _, depth = tree_mask_batch(inp.parent)
        assert inp.parent.shape == (inp.cfg.B, cfg.T)
        assert depth.max() <= cfg.max_depth
        for p in inp.parent:
            counts = np.bincount(p[1:], minlength=cfg.T)
            assert counts.max() <= cfg.max_children
        if cfg.tree in ("spine3", "grow_spine6"):
            assert (depth.max(axis=1) == cfg.max_depth).all()
