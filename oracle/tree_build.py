"""Dynamic draft-tree construction (oracle; test infrastructure only).

[TR] sec. 2 (sequence diagram and "Dynamic Tree-Attention Masking"): the drafter grows
the candidate tree in a loop of depth 4 to 6.  Each step judges the entropy of its
predicted distribution, H = -sum_i P(x_i) log P(x_i), and runs a beam search that prunes
weak branches.  A low-entropy (near-deterministic) context extends one branch as deep as
6; a high-entropy one widens to 8 children.  The tree handed to the verifier has at most
64 nodes, with its ancestor mask.  [SN] "pitfalls" item 4 places EAGLE-2's dynamic tree after
EAGLE-1's static one.

The pages leave the exact rules open; this oracle takes the plainest reading:
  * frontier node n has draft distribution q_n = softmax(draft_logits_n / tau) (the
    float64 contract of the acceptance oracle) and gets
        k_n = min(k_max, max(1, floor(exp(H(q_n)) + 1/2)))
    children.  exp(H) is the perplexity, the effective number of choices, so a
    near-deterministic node gets one child and a flat one gets k_max;
  * its children are its k_n most probable tokens (equal logits: lower token id first);
  * a node's value is the product of the draft probabilities along its path (root 1),
    the drafter's confidence that the whole path is right;
  * each depth keeps the W highest-valued new candidates as the next frontier (the beam)
    and prunes the rest, which stay as leaves;
  * after the last depth, the root and the N - 1 highest-valued candidates of all depths
    form the tree.  Since a child's value never exceeds its parent's, the chosen set
    holds every ancestor of its members.
  Ties between values go to the lower candidate id.  Ids run depth by depth, then by
  frontier slot, then by child rank, so a parent's id is below its children's.  Tree
  nodes are numbered by depth, then by value rank within the depth, so parent[i] < i and
  node 0 is the root.

The frontier at depth d holds at most W nodes; the caller's drafter produces one logit
row per frontier slot (row w follows frontier node w).  Rows of unused slots are ignored.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np

from .accept import target_probs


def entropy(q: np.ndarray) -> float:
    """H(q) = -sum q log q in nats, zero-probability terms dropped ([TR] sec. 2)."""
    nz = q[q > 0.0]
    return float(-np.sum(nz * np.log(nz)))


def width(ppl: float, k_max: int) -> int:
    """Children of a frontier node with perplexity ppl = exp(H)."""
    return int(min(k_max, max(1, math.floor(ppl + 0.5))))


def width_margin(ppl: float, k_max: int) -> float:
    """Distance of ppl + 1/2 from the nearest boundary that would change width()."""
    x = ppl + 0.5
    if x >= k_max + 1:
        return x - (k_max + 1)
    return min(x - math.floor(x), math.ceil(x) - x) if x != math.floor(x) else 0.0


def top_tokens(row: np.ndarray, k: int) -> list:
    """The k largest float32 logits of a row, equal logits ordered by lower token id."""
    order = np.lexsort((np.arange(len(row)), -row.astype(np.float64)))
    return [int(i) for i in order[:k]]


@dataclass
class Candidate:
    id: int
    depth: int
    parent: int            # candidate id of the parent, -1 for children of the root
    token: int
    value: float
    slot: int              # frontier slot of the parent at the previous depth (root: 0)


def _rank(cands: list) -> list:
    """Candidates by value, highest first; equal values by lower id."""
    return sorted(cands, key=lambda c: (-c.value, c.id))


def _gap_margins(ranked: list, upto: int) -> list:
    """Relative gaps between consecutive values of the first upto + 1 ranked candidates."""
    out = []
    for i in range(min(upto, len(ranked) - 1)):
        a, b = ranked[i].value, ranked[i + 1].value
        out.append((a - b) / a if a > 0 else 0.0)
    return out


class TreeBuilder:
    """Beam expansion of one sequence's draft tree, one depth per expand() call."""

    def __init__(self, beam: int, k_max: int, tau: float):
        self.beam, self.k_max, self.tau = beam, k_max, tau
        self.cands: list = []
        self.frontier: list = [None]        # None stands for the root
        self.margins: list = []

    def _value(self, slot) -> float:
        return 1.0 if slot is None else slot.value

    def expand(self, rows: np.ndarray):
        """Expand the current frontier; rows[w] is the draft logit row after slot w.

        Returns (tokens, parent_slots) of the new frontier, each of its length.
        """
        new = []
        for w, node in enumerate(self.frontier):
            q = target_probs(rows[w], self.tau)
            ppl = math.exp(entropy(q))
            self.margins.append(("width", width_margin(ppl, self.k_max) / ppl))
            k = width(ppl, self.k_max)
            for j, x in enumerate(top_tokens(rows[w], k)):
                c = Candidate(id=len(self.cands), depth=1 if node is None else node.depth + 1,
                              parent=-1 if node is None else node.id, token=x,
                              value=self._value(node) * float(q[x]), slot=w)
                self.cands.append(c)
                new.append(c)
        ranked = _rank(new)
        self.margins += [("beam", m) for m in _gap_margins(ranked, self.beam)]
        self.frontier = ranked[:self.beam]
        return [c.token for c in self.frontier], [c.slot for c in self.frontier]

    def finalize(self, n_nodes: int, root_token: int):
        """The tree: (parent[], tokens[]) of the root plus the n_nodes - 1 best candidates."""
        ranked = _rank(self.cands)
        self.margins += [("tree", m) for m in _gap_margins(ranked, n_nodes - 1)]
        chosen = ranked[:n_nodes - 1]
        rank = {c.id: r for r, c in enumerate(chosen)}
        order = sorted(chosen, key=lambda c: (c.depth, rank[c.id]))
        index = {c.id: i + 1 for i, c in enumerate(order)}
        parent = [-1] + [0 if c.parent < 0 else index[c.parent] for c in order]
        tokens = [int(root_token)] + [c.token for c in order]
        return parent, tokens


def build_batch(depth_logits: list, beam: int, k_max: int, tau, n_nodes: int, root_tokens):
    """Trees of a batch.

    depth_logits[d] is float32 [B][beam][V]: row w of sequence b is the drafter's logits
    after frontier slot w at depth d (depth 0: slot 0 is the root; other rows unused).
    Returns parent [B][n_nodes] and tokens [B][n_nodes] (-1 beyond the tree), the tree
    sizes [B], the frontier after each depth as (tokens [B][beam], parent slots
    [B][beam], counts [B]) (-1 padded), and every decision margin per sequence.
    """
    B = depth_logits[0].shape[0]
    parent = np.full((B, n_nodes), -1, np.int32)
    tokens = np.full((B, n_nodes), -1, np.int32)
    sizes = np.zeros(B, np.int32)
    frontiers = []
    for _ in depth_logits:
        frontiers.append((np.full((B, beam), -1, np.int32), np.full((B, beam), -1, np.int32),
                          np.zeros(B, np.int32)))
    margins = []
    for b in range(B):
        tb = TreeBuilder(beam, k_max, tau)
        for d, rows in enumerate(depth_logits):
            ft, fs = tb.expand(rows[b])
            frontiers[d][0][b, :len(ft)] = ft
            frontiers[d][1][b, :len(fs)] = fs
            frontiers[d][2][b] = len(ft)
        p, t = tb.finalize(n_nodes, root_tokens[b])
        parent[b, :len(p)] = p
        tokens[b, :len(t)] = t
        sizes[b] = len(p)
        margins.append(tb.margins)
    return parent, tokens, sizes, frontiers, margins
