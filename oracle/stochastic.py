"""Tree acceptance with a stochastic draft distribution (oracle; test infrastructure only).

The pages' accept-or-resample rule ([EX] "Why it works"; [SN] case 3) for drafts that
were *sampled* from a draft distribution q rather than taken by argmax.  At node a the
target's distribution is p = p_a and the children were drawn independently from q = q_a
(duplicates allowed, each tested on its own):

    r <- p
    for each child c in ascending node index, drafted token x:
        accept c with probability min(1, r(x) / q(x))
        otherwise r <- max(0, r - q) / sum(max(0, r - q))
    no child accepted (or a leaf): emit a token drawn from r

Each step emits exactly p in distribution (the standard speculative-sampling argument,
step by step down the tree); the chi-square tests of this module check it.

Unnormalised form.  After j rejections r = W_j / Z_j with
    W_j(y) = max(0, p(y) - s_j q(y)),  Z_j = sum_y W_j(y),  s_1 = 0,  s_{j+1} = s_j + Z_j,
because subtracting q from W_j / Z_j and clearing negatives is the same as subtracting
Z_j q from W_j (where W_j = 0 the result stays 0 as s only grows).  So the residual is
one scalar s plus a full-vocabulary sum per rejection, which is how it is computed here
and on the device.

Arithmetic contract (float64; shared with the device path so decisions agree):
  p = target_probs(logits[a], tau), q = target_probs(draft_logits[a], draft_tau) (the
  contract of the greedy/rejection oracle: s_y = float64(logit_y) * (1 / float64(tau)),
  exp(s_y - max s) / sum);
  a child with token x is accepted iff  u[c] * q(x) * Z < W(x)  (u[c] < r(x) / q(x));
  the bonus is an inverse CDF of W over ascending token id with t = u[0] * Z: the first
  y whose running sum of W exceeds t; if rounding leaves none, the largest y with
  W(y) > 0.  Decision margins are reported as in the rejection oracle.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

from .accept import _pad, children_of, target_probs


def _residual_update(W: np.ndarray, s: float, Z: float, p: np.ndarray, q: np.ndarray):
    """One rejection: the shift grows by the residual mass (see the module docstring)."""
    s_new = s + Z
    W_new = np.maximum(0.0, p - s_new * q)
    return W_new, s_new, math.fsum(W_new)


def stochastic_walk(p_of, q_of, tokens, parent, u, margins: Optional[list] = None,
                    update=_residual_update) -> tuple[int, list, list]:
    """Acceptance of one tree with sampled drafts.

    p_of(a) / q_of(a): target and draft distributions of node a (float64, length V).
    u[c] (c >= 1) is the uniform of the test of node c; u[0] draws the bonus.
    Returns (k, path, emitted tokens); decision margins are appended to `margins`.
    """
    path = [0]
    out = []
    a = 0
    while True:
        p, q = p_of(a), q_of(a)
        s = 0.0
        W = np.maximum(0.0, p - s * q)
        Z = math.fsum(W)
        taken = None
        for c in children_of(parent, a):
            x = int(tokens[c])
            lhs = float(u[c]) * float(q[x]) * Z
            if margins is not None:
                margins.append(abs(lhs - float(W[x])))
            if lhs < float(W[x]):
                taken = c
                break
            W, s, Z = update(W, s, Z, p, q)
        if taken is not None:
            out.append(int(tokens[taken]))
            path.append(taken)
            a = taken
            continue
        out.append(_draw(W, float(u[0]) * Z, margins))
        return len(path) - 1, path, out


def _draw(W: np.ndarray, t: float, margins: Optional[list]) -> int:
    C = 0.0
    for y in range(len(W)):
        w = float(W[y])
        if w <= 0.0:
            continue
        prev = C
        C += w
        if C > t:
            if margins is not None:
                margins.append(min(t - prev, C - t))
            return y
    nz = np.flatnonzero(W > 0.0)
    if len(nz) == 0:
        raise ValueError("residual distribution is empty")
    if margins is not None:
        margins.append(0.0)
    return int(nz[-1])


def stochastic_batch(logits: np.ndarray, draft_logits: np.ndarray, tokens: np.ndarray,
                     parent: np.ndarray, tau, draft_tau, uniforms: np.ndarray):
    """Acceptance of a batch with sampled drafts.

    Returns (accept_len[B], path[B][T], out_tokens[B][T], margins) like rejection_batch.
    """
    B, T = tokens.shape
    klen = np.zeros(B, dtype=np.int32)
    paths = np.full((B, T), -1, dtype=np.int32)
    outs = np.full((B, T), -1, dtype=np.int32)
    all_margins = []
    for b in range(B):
        pc, qc = {}, {}

        def p_of(a, b=b, pc=pc):
            if a not in pc:
                pc[a] = target_probs(logits[b, a], tau)
            return pc[a]

        def q_of(a, b=b, qc=qc):
            if a not in qc:
                qc[a] = target_probs(draft_logits[b, a], draft_tau)
            return qc[a]

        m = []
        k, path, out = stochastic_walk(p_of, q_of, tokens[b], parent[b], uniforms[b], m)
        klen[b] = k
        paths[b] = _pad(path, T)
        outs[b] = _pad(out, T)
        all_margins.append(m)
    return klen, paths, outs, all_margins
