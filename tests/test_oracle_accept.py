"""Pins of the oracle's greedy and rejection acceptance.

Fixed by the pages: the accepted result is the longest verified prefix of a branch and
k accepted drafts emit k + 1 tokens (EAGLE explainer "Core idea"; study note case 1);
rejection sampling leaves the emitted tokens distributed exactly as the target's own
samples (explainer "Why it works"; study note case 3).  The tests below check those
facts by brute force, closed forms and a chi-square test with a negative control.
"""
import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle.accept as acc
from oracle import greedy_batch, greedy_walk, rejection_batch, rejection_walk, target_probs
from synth import CONFIGS, generate, scaled


def random_tree(rng, T):
    return [-1] + [int(rng.integers(i)) for i in range(1, T)]


def distinct_sibling_tokens(rng, parent, V):
    tok = [int(rng.integers(V))]
    used = {}
    for i in range(1, len(parent)):
        s = used.setdefault(parent[i], set())
        while True:
            x = int(rng.integers(V))
            if x not in s:
                break
        s.add(x)
        tok.append(x)
    return tok


def brute_force_greedy(logits, tokens, parent):
    """Longest root path whose every draft equals the target argmax at its parent."""
    T = len(parent)
    best = [0]
    for node in range(T):
        path = []
        u = node
        while u != -1:
            path.append(u)
            u = parent[u]
        path = path[::-1]
        ok = all(tokens[path[j]] == int(np.argmax(logits[path[j - 1]])) for j in range(1, len(path)))
        if ok and (len(path) > len(best) or (len(path) == len(best) and path < best)):
            best = path
    return best


@pytest.mark.parametrize("seed", range(40))
def test_greedy_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    T, V = int(rng.integers(1, 30)), int(rng.integers(2, 12))
    parent = random_tree(rng, T)
    tokens = distinct_sibling_tokens(rng, parent, max(V, T)) if V >= T else None
    if tokens is None:
        V = T
        tokens = distinct_sibling_tokens(rng, parent, V)
    logits = rng.standard_normal((T, V)).astype(np.float32)
    # make walks deep: often raise the logit of the lowest child's token
    for u in range(T):
        kids = [c for c in range(T) if parent[c] == u]
        if kids and rng.random() < 0.7:
            logits[u, tokens[kids[0]]] = 10.0
    k, path, out = greedy_walk(logits, tokens, parent)
    assert path == brute_force_greedy(logits, tokens, parent)
    assert k == len(path) - 1 and len(out) == k + 1
    # emitted tokens are sequential greedy decoding along the accepted path
    assert out == [int(np.argmax(logits[a])) for a in path]
    assert out[:k] == [tokens[c] for c in path[1:]]


def test_greedy_special_cases():
    V = 10
    parent = [-1, 0, 0, 1]
    logits = np.zeros((4, V), np.float32)
    logits[:, 7] = 1.0
    k, path, out = greedy_walk(logits, [0, 1, 2, 3], parent)     # no child drafts token 7
    assert (k, path, out) == (0, [0], [7])
    chain = list(range(-1, 63))
    tok = [int(t) for t in np.arange(64) % V]
    lg = np.zeros((64, V), np.float32)
    for i in range(63):
        lg[i, tok[i + 1]] = 1.0
    k, path, out = greedy_walk(lg, tok, chain)                   # every draft accepted
    assert k == 63 and path == list(range(64)) and len(out) == 64
    # ties: lowest token id wins, -0.0 == +0.0; duplicate siblings: lowest node index
    row = np.array([0.0, 3.0, 3.0, -0.0], np.float32)
    k, path, out = greedy_walk(np.stack([row, row, row]), [0, 2, 1], [-1, 0, 0])
    assert (k, path, out) == (1, [0, 2], [1, 1])
    neg = np.array([-0.0, 0.0, -1.0], np.float32)
    assert greedy_walk(neg[None], [0], [-1])[2] == [0]
    k, path, _ = greedy_walk(np.stack([row] * 4), [0, 1, 1, 1], [-1, 0, 0, 1])
    assert path[:2] == [0, 1]


def test_target_probs_contract():
    rng = np.random.default_rng(3)
    row = (2 * rng.standard_normal(5000)).astype(np.float32)
    p = target_probs(row, np.float32(0.7))
    ref = scipy.special.softmax(row.astype(np.float64) / np.float64(np.float32(0.7)))
    assert abs(p.sum() - 1.0) < 1e-14
    assert np.abs(p / ref - 1.0).max() < 1e-12


def _chi_square_run(n_trials, seed):
    """The pages' losslessness claim on a tiny tree: histogram of emitted tokens."""
    V, tau = 8, np.float32(0.7)
    parent = [-1, 0, 0, 0, 1, 1]
    rng = np.random.default_rng(seed)
    logits = (2 * rng.standard_normal((6, V))).astype(np.float32)
    top = int(np.argmax(logits[0]))
    tokens = [0, top, (top + 3) % V, (top + 5) % V, int(np.argmax(logits[1])), (int(np.argmax(logits[1])) + 2) % V]
    p = [target_probs(logits[a], tau) for a in range(6)]
    u = np.random.default_rng(seed + 1).random((n_trials, 6))
    first = np.zeros(V, np.int64)
    second_given_1 = np.zeros(V, np.int64)
    lens = np.zeros(3, np.int64)
    for trial in range(n_trials):
        k, path, out = rejection_walk(p.__getitem__, tokens, parent, u[trial])
        first[out[0]] += 1
        lens[k] += 1
        if k >= 1 and path[1] == 1:
            second_given_1[out[1]] += 1
    ref0 = scipy.special.softmax(logits[0].astype(np.float64) / np.float64(tau))
    ref1 = scipy.special.softmax(logits[1].astype(np.float64) / np.float64(tau))
    pv0 = scipy.stats.chisquare(first, first.sum() * ref0).pvalue
    pv1 = scipy.stats.chisquare(second_given_1, second_given_1.sum() * ref1).pvalue
    return pv0, pv1, lens


@pytest.mark.slow
def test_rejection_preserves_target_distribution_chi_square():
    pv0, pv1, lens = _chi_square_run(1_000_000, 2024)
    assert pv0 > 1e-3 and pv1 > 1e-3, (pv0, pv1)
    assert lens[1] > 0 and lens[2] > 0


def test_rejection_negative_control_without_renormalisation(monkeypatch):
    """Plant the classic mistake (test u < p, ignoring the shrinking residual): must fail."""
    monkeypatch.setattr(acc, "_accepts", lambda u, Z, p: u < p)
    pv0, pv1, _ = _chi_square_run(200_000, 2024)
    assert min(pv0, pv1) < 1e-3


def test_rejection_chain_expected_length_closed_form():
    """E[k] on a chain = sum_m prod_{j<=m} p_{j-1}(x_j)."""
    D, V, tau = 5, 6, np.float32(0.7)
    parent = list(range(-1, D))
    rng = np.random.default_rng(77)
    logits = (2 * rng.standard_normal((D + 1, V))).astype(np.float32)
    tokens = [0] + [int(rng.integers(V)) for _ in range(D)]
    for j in range(1, D + 1):
        logits[j - 1, tokens[j]] += 1.5
    p = [target_probs(logits[a], tau) for a in range(D + 1)]
    ref = [scipy.special.softmax(logits[a].astype(np.float64) / np.float64(tau)) for a in range(D + 1)]
    expect = sum(np.prod([ref[j - 1][tokens[j]] for j in range(1, m + 1)]) for m in range(1, D + 1))
    n = 200_000
    u = np.random.default_rng(78).random((n, D + 1))
    ks = np.array([rejection_walk(p.__getitem__, tokens, parent, u[t])[0] for t in range(n)])
    se = ks.std() / np.sqrt(n)
    assert abs(ks.mean() - expect) < 5 * se, (ks.mean(), expect, se)


def test_rejection_at_low_temperature_is_greedy():
    """tau = 0.05 with a top-2 gap >= 1: every accept probability is 1 - O(V e^-20)."""
    rng = np.random.default_rng(5)
    B, T, V = 8, 40, 500
    parents = np.array([random_tree(rng, T) for _ in range(B)], np.int32)
    tokens = np.array([distinct_sibling_tokens(rng, list(p), V) for p in parents], np.int32)
    logits = rng.standard_normal((B, T, V)).astype(np.float32)
    for b in range(B):
        for u in range(T):
            kids = [c for c in range(T) if parents[b, c] == u]
            x = tokens[b, kids[0]] if kids and rng.random() < 0.8 else int(rng.integers(V))
            logits[b, u, x] = logits[b, u].max() + 1.0 + rng.random()
    g = greedy_batch(logits, tokens, parents)
    r = rejection_batch(logits, tokens, parents, np.float32(0.05), rng.random((B, T)))
    for a, b_ in zip(g, r[:3]):
        assert np.array_equal(a, b_)
    assert g[0].max() >= 3


def test_rejection_planted_certain_path_is_always_accepted():
    D, V = 6, 50
    parent = [-1, 0, 1, 1, 2, 4, 5, 6]            # a depth-6 branch 0-1-2-4-5-6-7 plus a side node 3
    rng = np.random.default_rng(6)
    tokens = distinct_sibling_tokens(rng, parent, V)
    logits = rng.standard_normal((8, V)).astype(np.float32)
    for a, c in [(0, 1), (1, 2), (2, 4), (4, 5), (5, 6), (6, 7)]:
        logits[a, tokens[c]] = 1000.0              # p = 1 exactly in float64
    for trial in range(200):
        u = rng.random(8)
        k, path, out = rejection_walk(lambda a: target_probs(logits[a], 0.7), tokens, parent, u)
        assert path == [0, 1, 2, 4, 5, 6, 7] and k == D
        assert out[:D] == [tokens[c] for c in path[1:]]


def test_rejection_duplicate_sibling_is_skipped_and_bonus_avoids_rejected():
    V = 4
    logits = np.log(np.array([[0.1, 0.2, 0.3, 0.4]] * 3, np.float64)).astype(np.float32)
    tau = np.float32(1.0)
    p = [target_probs(logits[a], tau) for a in range(3)]
    margins = []
    # both children draft token 3; the first is rejected (u * 1 >= 0.4), the second is skipped
    k, path, out = rejection_walk(p.__getitem__, [0, 3, 3], [-1, 0, 0], [0.0, 0.9, 0.0], margins)
    assert k == 0 and out == [0] and len(margins) == 2
    # residual with token 3 removed: Z = 0.6; u0 = 0.99 -> t = 0.594 -> C = .1,.3,.6 -> token 2
    k, path, out = rejection_walk(p.__getitem__, [0, 3, 3], [-1, 0, 0], [0.99, 0.9, 0.0])
    assert out == [2]


def test_workload_acceptance_runs_and_is_deterministic():
    cfg = scaled(CONFIGS[2], V=4000, L=16)
    inp = generate(cfg, with_kv=False)
    r1 = rejection_batch(inp.logits, inp.tokens, inp.parent, inp.tau, inp.uniforms)
    r2 = rejection_batch(inp.logits, inp.tokens, inp.parent, inp.tau, inp.uniforms)
    for a, b in zip(r1[:3], r2[:3]):
        assert np.array_equal(a, b)
    k = int(r1[0][0])
    assert (r1[1][0][:k + 1] >= 0).all() and (r1[1][0][k + 1:] == -1).all()
    assert min(r1[3][0]) > 1e-12
    g = greedy_batch(inp.logits, inp.tokens, inp.parent)
    assert g[0][0] >= 1                           # planted drafts are the argmax at planted nodes
