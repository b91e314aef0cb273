"""Pins of the draft-tree construction oracle (oracle/tree_build.py).

Each pin comes from outside the oracle's own code path: closed forms of the entropy, a
library entropy, brute-force top-k, a full enumeration of every path (no pruning), an
independent greedy-chain formulation for a beam of one, a hand-derived golden tree for
flat rows, and structural invariants of the emitted trees.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats

from oracle import tree_build as tbm
from oracle.accept import target_probs
from synth import draft_tree_logits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --- entropy and width ------------------------------------------------------------------

def test_entropy_of_uniform_is_log_v():
    for V in (2, 16, 1000):
        q = target_probs(np.zeros(V, np.float32), 1.0)
        assert tbm.entropy(q) == pytest.approx(math.log(V), rel=1e-14)


def test_entropy_two_point_closed_form():
    for a in (0.0, 0.5, 2.0, 7.0):
        q = target_probs(np.array([a, 0.0], np.float32), 1.0)
        p = 1.0 / (1.0 + math.exp(-a))
        assert tbm.entropy(q) == pytest.approx(-p * math.log(p) - (1 - p) * math.log(1 - p),
                                               rel=1e-12)


def test_entropy_matches_library_on_random_rows():
    rng = np.random.default_rng(5)
    for _ in range(20):
        row = (rng.uniform(0.5, 10) * rng.standard_normal(500)).astype(np.float32)
        q = target_probs(row, 0.9)
        ref = scipy.stats.entropy(scipy.special.softmax(row.astype(np.float64) / np.float64(np.float32(0.9))))
        assert tbm.entropy(q) == pytest.approx(ref, rel=1e-12)


def test_one_hot_row_has_width_one():
    row = np.zeros(4096, np.float32)
    row[17] = 100.0
    q = target_probs(row, 1.0)
    assert tbm.width(math.exp(tbm.entropy(q)), 8) == 1


@pytest.mark.parametrize("m", [1, 2, 3, 5, 8, 9, 20])
def test_m_equal_tokens_give_m_children(m):
    """m tied top logits and the rest far below (their exp underflows to exactly 0): the
    distribution is uniform over m tokens, perplexity m, width min(m, 8), and the children
    are the m tied tokens in token order."""
    rng = np.random.default_rng(m)
    V = 64
    row = np.full(V, -1e4, np.float32)
    top = np.sort(rng.choice(V, size=m, replace=False))
    row[top] = 3.0
    tb = tbm.TreeBuilder(beam=8, k_max=8, tau=1.0)
    toks, _ = tb.expand(row[None])
    k = min(m, 8)
    assert len(tb.cands) == k
    assert [c.token for c in tb.cands] == [int(t) for t in top[:k]]
    assert sorted(toks) == [int(t) for t in top[:k]]


def test_top_tokens_against_sorting():
    rng = np.random.default_rng(9)
    for _ in range(30):
        row = rng.integers(-3, 4, size=200).astype(np.float32)   # many ties
        k = int(rng.integers(1, 9))
        ref = [i for _, i in sorted((-float(v), i) for i, v in enumerate(row))][:k]
        assert tbm.top_tokens(row, k) == ref


# --- whole trees ---------------------------------------------------------------------------

def path_row(path, V, seed):
    """Logits keyed by the token path from the root (a drafter whose output depends on
    the whole path), with a per-path sharpness so widths vary."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, len(path)] + list(path)))
    return (rng.uniform(0.5, 4.0) * rng.standard_normal(V)).astype(np.float32)


def grow(builder, depths, V, seed):
    """Drive a TreeBuilder with path-keyed logits; returns the builder."""
    paths = {None: ()}
    for _ in range(depths):
        rows = np.stack([path_row(paths[None] if n is None else paths[n.id], V, seed)
                         for n in builder.frontier])
        builder.expand(rows)
        for c in builder.cands:
            if c.id not in paths:
                base = () if c.parent < 0 else paths[c.parent]
                paths[c.id] = base + (c.token,)
    return paths


def tree_paths(parent, tokens):
    out = []
    for i in range(1, len(parent)):
        p, j = [], i
        while j > 0:
            p.append(int(tokens[j]))
            j = parent[j]
        out.append(tuple(reversed(p)))
    return out


def brute_force(depths, V, seed, k_max, tau):
    """Every path of the unpruned expansion with its value, by direct recursion: library
    softmax and entropy, children = the k most probable tokens by sorting."""
    res = {}

    def rec(path, value, d):
        if d == depths:
            return
        row = path_row(path, V, seed)
        q = scipy.special.softmax(row.astype(np.float64) / np.float64(np.float32(tau)))
        ppl = math.exp(scipy.stats.entropy(q))
        k = int(min(k_max, max(1, math.floor(ppl + 0.5))))
        kids = [i for _, i in sorted((-float(row[i]), i) for i in range(V))][:k]
        for x in kids:
            res[path + (x,)] = value * float(q[x])
            rec(path + (x,), value * float(q[x]), d + 1)

    rec((), 1.0, 0)
    return res


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_unpruned_tree_equals_enumeration(seed):
    """A beam wide enough never prunes: the tree must be the n-1 best paths of the full
    expansion by product of draft probabilities, numbered by depth then value."""
    V, depths, k_max, n_nodes = 48, 3, 3, 20
    tb = tbm.TreeBuilder(beam=64, k_max=k_max, tau=1.0)
    grow(tb, depths, V, seed)
    parent, tokens = tb.finalize(n_nodes, root_token=7)
    ref = brute_force(depths, V, seed, k_max, 1.0)
    best = sorted(ref, key=lambda p: -ref[p])[:n_nodes - 1]
    got = tree_paths(parent, tokens)
    assert len(ref) > n_nodes                    # the cut is exercised
    assert set(got) == set(best)
    assert tokens[0] == 7 and parent[0] == -1
    for a, b in zip(got, got[1:]):               # depth, then value, order
        assert (len(a), -ref[a]) < (len(b), -ref[b])


@pytest.mark.parametrize("seed", [11, 12, 13])
def test_beam_of_one_is_a_greedy_chain_with_leaves(seed):
    """With one beam the frontier is the best child of the previous frontier node; the
    tree is that chain plus every expanded node's other children."""
    V, depths, k_max = 40, 4, 4
    tb = tbm.TreeBuilder(beam=1, k_max=k_max, tau=1.0)
    grow(tb, depths, V, seed)
    parent, tokens = tb.finalize(64, root_token=0)
    want, chain = set(), ()
    for _ in range(depths):
        row = path_row(chain, V, seed)
        q = scipy.special.softmax(row.astype(np.float64))
        k = int(min(k_max, max(1, math.floor(math.exp(scipy.stats.entropy(q)) + 0.5))))
        kids = [i for _, i in sorted((-float(row[i]), i) for i in range(V))][:k]
        want |= {chain + (x,) for x in kids}
        chain = chain + (kids[0],)
    assert set(tree_paths(parent, tokens)) == want


def test_flat_rows_golden():
    g = json.load(open(os.path.join(GOLDEN, "draft_tree_flat.json")))
    rows = [np.zeros((1, g["beam"], g["V"]), np.float32) for _ in range(g["depths"])]
    parent, tokens, sizes, fronts, _ = tbm.build_batch(rows, g["beam"], g["k_max"], 1.0,
                                                       g["n_nodes"], [g["root_token"]])
    assert parent[0].tolist() == g["parent"]
    assert tokens[0].tolist() == g["tokens"]
    assert sizes[0] == g["n_nodes"]
    for d in range(g["depths"]):
        assert fronts[d][0][0].tolist() == g["frontier_tokens"][d]
        assert fronts[d][1][0].tolist() == g["frontier_slots"][d]


def test_one_hot_rows_make_a_chain():
    """Near-deterministic rows ([TR] sec. 2: low entropy extends one branch to depth 6)."""
    depths, V = 6, 500
    rng = np.random.default_rng(3)
    spikes = rng.integers(0, V, size=(depths, 8))
    rows = []
    for d in range(depths):
        r = np.zeros((1, 8, V), np.float32)
        r[0, np.arange(8), spikes[d]] = 60.0
        rows.append(r)
    parent, tokens, sizes, fronts, _ = tbm.build_batch(rows, 8, 8, 1.0, 64, [1])
    assert sizes[0] == depths + 1
    assert parent[0, :depths + 1].tolist() == [-1] + list(range(depths))
    assert tokens[0, 1:depths + 1].tolist() == [int(spikes[d, 0]) for d in range(depths)]
    assert (parent[0, depths + 1:] == -1).all()


@pytest.mark.parametrize("B,V", [(3, 2000), (2, 128256)])
def test_structure_on_generated_inputs(B, V):
    dl = draft_tree_logits(B, V, depths=6, beam=8)
    parent, tokens, sizes, fronts, margins = tbm.build_batch(dl, 8, 8, 1.0, 64,
                                                             np.arange(B, dtype=np.int32))
    for b in range(B):
        n = int(sizes[b])
        assert 2 <= n <= 64
        assert parent[b, 0] == -1 and tokens[b, 0] == b
        depth = [0] * n
        for i in range(1, n):
            assert 0 <= parent[b, i] < i
            depth[i] = depth[parent[b, i]] + 1
            assert 0 <= tokens[b, i] < V
        assert depth == sorted(depth) and max(depth) <= 6
        kids = np.bincount(parent[b, 1:n], minlength=n)
        assert kids.max() <= 8
        for d in range(6):
            assert 1 <= fronts[d][2][b] <= 8
        assert all(m >= 0 for _, m in margins[b])
