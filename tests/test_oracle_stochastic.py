"""Pins of the oracle's acceptance with sampled drafts (draft distribution q).

Fixed by the pages: accepting a draft the target rates highly and otherwise rejecting
it and resampling from what is left leaves the emitted tokens distributed exactly as
the target's own samples (explainer "Why it works"; study note case 3).  Here the
children of a node are independent draws from q; the tests check the output
distribution by chi-square (with a negative control), the acceptance probability of a
single child against its closed form 1 - TV(p, q), the q = p case, and that a one-hot q
on single-child chains is exactly the point-mass rule of the pinned rejection oracle.
"""
import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle.stochastic as sto
from oracle import rejection_walk, stochastic_batch, stochastic_walk, target_probs

V = 8
TAU = np.float32(0.7)
PARENT = [-1, 0, 0, 0, 1, 1]


def _setup(seed):
    rng = np.random.default_rng(seed)
    logits = (2 * rng.standard_normal((6, V))).astype(np.float32)
    draft = (2 * rng.standard_normal((6, V))).astype(np.float32)
    p = [target_probs(logits[a], TAU) for a in range(6)]
    q = [target_probs(draft[a], TAU) for a in range(6)]
    return logits, draft, p, q


def _chi_square_run(n_trials, seed, update=sto._residual_update):
    """Children drawn i.i.d. from q at their parent; histogram of the emitted tokens."""
    logits, draft, p, q = _setup(seed)
    rng = np.random.default_rng(seed + 1)
    first = np.zeros(V, np.int64)
    second_given_1 = np.zeros(V, np.int64)
    for _ in range(n_trials):
        tokens = [0] + [int(rng.choice(V, p=q[PARENT[c]])) for c in range(1, 6)]
        u = rng.random(6)
        k, path, out = stochastic_walk(p.__getitem__, q.__getitem__, tokens, PARENT, u,
                                       update=update)
        first[out[0]] += 1
        if k >= 1 and path[1] == 1:
            second_given_1[out[1]] += 1
    pv0 = scipy.stats.chisquare(first, first.sum() * p[0]).pvalue
    pv1 = scipy.stats.chisquare(second_given_1, second_given_1.sum() * p[1]).pvalue
    return pv0, pv1


def test_sampled_drafts_preserve_target_distribution_chi_square():
    pv0, pv1 = _chi_square_run(100_000, 7)
    assert pv0 > 1e-3 and pv1 > 1e-3, (pv0, pv1)


def test_negative_control_without_residual_update():
    """Plant the classic mistake (testing every sibling against p itself): must fail."""
    keep = lambda W, s, Z, p, q: (W, s, Z)
    pv0, pv1 = _chi_square_run(100_000, 7, update=keep)
    assert min(pv0, pv1) < 1e-3


def test_single_child_acceptance_is_one_minus_total_variation():
    """P(accept the only child) = sum_x q(x) min(1, p(x)/q(x)) = 1 - TV(p, q)."""
    _, _, p, q = _setup(11)
    rng = np.random.default_rng(12)
    n = 100_000
    acc = 0
    for _ in range(n):
        x = int(rng.choice(V, p=q[0]))
        k, _, _ = stochastic_walk(p.__getitem__, q.__getitem__, [0, x], [-1, 0], rng.random(2))
        acc += k
    expect = float(np.minimum(p[0], q[0]).sum())
    assert abs(acc / n - expect) < 4 * np.sqrt(expect * (1 - expect) / n)


def test_draft_equal_to_target_accepts_the_first_child():
    _, _, p, _ = _setup(13)
    rng = np.random.default_rng(14)
    for _ in range(200):
        tokens = [0] + [int(rng.choice(V, p=p[PARENT[c]])) for c in range(1, 6)]
        k, path, _ = stochastic_walk(p.__getitem__, p.__getitem__, tokens, PARENT, rng.random(6))
        assert k >= 1 and path[1] == 1


@pytest.mark.parametrize("seed", range(20))
def test_one_hot_draft_on_chains_is_the_point_mass_rule(seed):
    """Single-child nodes whose q is a point mass at that child's token: the rule is the
    pinned deterministic-draft rejection walk, decision for decision."""
    rng = np.random.default_rng(100 + seed)
    T, Vb = 7, 12
    parent = [-1] + list(range(T - 1))                 # a chain
    logits = (2 * rng.standard_normal((T, Vb))).astype(np.float32)
    tokens = [0] + [int(rng.integers(Vb)) for _ in range(T - 1)]
    # plant: often make the drafted token likely
    for a in range(T - 1):
        if rng.random() < 0.7:
            logits[a, tokens[a + 1]] = logits[a].max() + 2.0
    draft = np.full((T, Vb), -1e30, np.float32)
    for a in range(T - 1):
        draft[a, tokens[a + 1]] = 0.0
    draft[T - 1, 0] = 0.0                              # the leaf has no children
    u = rng.random(T)
    p = [target_probs(logits[a], TAU) for a in range(T)]
    q = [target_probs(draft[a], TAU) for a in range(T)]
    assert all(abs(q[a][tokens[a + 1]] - 1.0) == 0.0 for a in range(T - 1))
    got = stochastic_walk(p.__getitem__, q.__getitem__, tokens, parent, u)
    ref = rejection_walk(p.__getitem__, tokens, parent, u)
    assert got == ref


def test_batch_wrapper_matches_per_tree_walks():
    rng = np.random.default_rng(3)
    B, T, Vb = 3, 9, 20
    parent = np.array([[-1] + [int(rng.integers(i)) for i in range(1, T)] for _ in range(B)], np.int32)
    logits = (2 * rng.standard_normal((B, T, Vb))).astype(np.float32)
    draft = (2 * rng.standard_normal((B, T, Vb))).astype(np.float32)
    tokens = rng.integers(0, Vb, (B, T)).astype(np.int32)
    u = rng.random((B, T))
    klen, paths, outs, margins = stochastic_batch(logits, draft, tokens, parent, 0.7, 0.9, u)
    for b in range(B):
        p = lambda a: target_probs(logits[b, a], 0.7)
        q = lambda a: target_probs(draft[b, a], 0.9)
        k, path, out = stochastic_walk(p, q, tokens[b], parent[b], u[b])
        assert klen[b] == k and list(paths[b][:k + 1]) == path and list(outs[b][:k + 1]) == out
        assert len(margins[b]) >= 1
