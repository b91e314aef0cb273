"""Tree acceptance: greedy longest match and rejection sampling (oracle; test infrastructure only).

Both walk down the drafted tree from the root and stop at the first node none of whose
children is accepted ([EX] "Core idea": the target verifies all branches for the longest
accepted prefix; [SN] case 1: k accepted drafts advance the sequence by k + 1 tokens, the
last one produced by the target itself).

Greedy: at node a the target's choice is the lowest-index argmax of the float32 logit
row of a; the walk moves to the lowest-index child drafted with that token.

Rejection ([EX] "Why it works"; [SN] case 3): a draft the target rates highly is kept;
otherwise it is rejected with the leftover probability and the target resamples, so
the emitted tokens follow the target's own distribution exactly.  The drafts here are
deterministic (the draft head takes an argmax, [TR] sec. 2), so each child's draft
distribution is a point mass and the standard rule reduces to:
  start with Z = 1 and no rejected tokens;
  for each child c in ascending node index with draft token x not yet rejected:
      accept c  iff  u[c] * Z < p(x)
      else reject x:  Z -= p(x)   (x's mass leaves the residual)
  if no child is accepted (or a is a leaf) emit a token drawn from the residual
  (p without the rejected tokens, renormalised by Z) with the root uniform u[0].
Every step emits exactly p(.) in distribution (see the chi-square test of this module).

Arithmetic contract (shared with the device path so decisions agree):
  inv_tau = 1.0 / float64(tau);  s_y = float64(logit_y) * inv_tau;  M = max_y s_y;
  S = sum_y exp(s_y - M);  p(y) = exp(s_y - M) / S.
The residual draw is an inverse CDF in ascending token id: with t = u[0] * Z, the bonus
is the first y outside the rejected set whose running sum C_y = sum_{y' <= y, y' not
rejected} p(y') exceeds t; if rounding leaves none, the largest such y with p(y) > 0.
Each decision's margin (|u Z - p| for a test, distance of t to the bracketing partial
sums for the bonus) is reported so tests can tell a rounding tie from a real mismatch.
"""
from __future__ import annotations

import math
from typing import Callable, Optional

import numpy as np


def argmax_lowest(row: np.ndarray) -> int:
    """First index of the maximum of a float32 row (-0.0 and +0.0 compare equal)."""
    return int(np.argmax(row))


def children_of(parent, a: int) -> list:
    return [c for c in range(len(parent)) if int(parent[c]) == a]


def greedy_walk(logits: np.ndarray, tokens, parent) -> tuple[int, list, list]:
    """Greedy acceptance of one tree. Returns (k, path, emitted tokens)."""
    path = [0]
    out = []
    a = 0
    while True:
        y = argmax_lowest(logits[a])
        out.append(y)
        nxt = None
        for c in children_of(parent, a):
            if int(tokens[c]) == y:
                nxt = c
                break
        if nxt is None:
            break
        path.append(nxt)
        a = nxt
    return len(path) - 1, path, out


def target_probs(logit_row: np.ndarray, tau) -> np.ndarray:
    """p(y) of one node under the float64 arithmetic contract (module docstring)."""
    inv_tau = 1.0 / float(np.float32(tau))
    s = np.asarray(logit_row, dtype=np.float32).astype(np.float64) * inv_tau
    M = s.max()
    e = np.exp(s - M)
    S = math.fsum(e)
    return e / S


def _accepts(u: float, Z: float, p: float) -> bool:
    """Acceptance test of one child against the current residual mass Z."""
    return u * Z < p


def rejection_walk(prob: Callable[[int], np.ndarray], tokens, parent, u,
                   margins: Optional[list] = None) -> tuple[int, list, list]:
    """Rejection acceptance of one tree.

    prob(a) returns the target distribution of node a (float64, length V).
    u[c] (c >= 1) is the uniform of the test of node c; u[0] draws the bonus.
    Returns (k, path, emitted tokens); decision margins are appended to `margins`.
    """
    path = [0]
    out = []
    a = 0
    while True:
        p = prob(a)
        Z = 1.0
        rejected = []
        taken = None
        for c in children_of(parent, a):
            x = int(tokens[c])
            if x in rejected:
                continue
            if margins is not None:
                margins.append(abs(float(u[c]) * Z - float(p[x])))
            if _accepts(float(u[c]), Z, float(p[x])):
                taken = c
                break
            rejected.append(x)
            Z -= float(p[x])
        if taken is not None:
            out.append(int(tokens[taken]))
            path.append(taken)
            a = taken
            continue
        out.append(_residual_draw(p, rejected, float(u[0]) * Z, margins))
        return len(path) - 1, path, out


def _residual_draw(p: np.ndarray, rejected: list, t: float, margins: Optional[list]) -> int:
    skip = set(rejected)
    C = 0.0
    for y in range(len(p)):
        if y in skip:
            continue
        prev = C
        C += float(p[y])
        if C > t:
            if margins is not None:
                margins.append(min(t - prev, C - t))
            return y
    for y in range(len(p) - 1, -1, -1):     # rounding left t beyond the last partial sum
        if y not in skip and p[y] > 0.0:
            if margins is not None:
                margins.append(0.0)
            return y
    raise ValueError("residual distribution is empty")


def _pad(seq: list, T: int) -> np.ndarray:
    out = np.full(T, -1, dtype=np.int32)
    out[:len(seq)] = seq
    return out


def greedy_batch(logits: np.ndarray, tokens: np.ndarray, parent: np.ndarray):
    """Greedy acceptance of a batch: (accept_len[B], path[B][T], out_tokens[B][T]), -1 padded."""
    B, T = tokens.shape
    klen = np.zeros(B, dtype=np.int32)
    paths = np.full((B, T), -1, dtype=np.int32)
    outs = np.full((B, T), -1, dtype=np.int32)
    for b in range(B):
        k, path, out = greedy_walk(logits[b], tokens[b], parent[b])
        klen[b] = k
        paths[b] = _pad(path, T)
        outs[b] = _pad(out, T)
    return klen, paths, outs


def rejection_batch(logits: np.ndarray, tokens: np.ndarray, parent: np.ndarray, tau,
                    uniforms: np.ndarray):
    """Rejection acceptance of a batch.

    Returns (accept_len[B], path[B][T], out_tokens[B][T], margins) with margins a list
    (one list of floats per sequence).
    """
    B, T = tokens.shape
    klen = np.zeros(B, dtype=np.int32)
    paths = np.full((B, T), -1, dtype=np.int32)
    outs = np.full((B, T), -1, dtype=np.int32)
    all_margins = []
    for b in range(B):
        cache = {}

        def prob(a, b=b, cache=cache):
            if a not in cache:
                cache[a] = target_probs(logits[b, a], tau)
            return cache[a]

        m = []
        k, path, out = rejection_walk(prob, tokens[b], parent[b], uniforms[b], m)
        klen[b] = k
        paths[b] = _pad(path, T)
        outs[b] = _pad(out, T)
        all_margins.append(m)
    return klen, paths, outs, all_margins
