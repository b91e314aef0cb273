"""Rejection acceptance: decisions taken from float32 statistics under their error bound,
and the float64 recomputation the walk falls back to.

ev_accept_rejection settles each node from float32 chunk sums when a bound on their error
cannot change the decision, and recomputes the node from float64 statistics otherwise.
These tests pin both paths to the float64 oracle bit for bit:
  * with the bound scaled to 1e300 every node the walk visits takes the float64 path;
  * uniforms placed a hair (1e-9) from a decision edge (a child test at u Z = p, a draw
    at a boundary of the cumulative mass) are inside the float32 bound, so those nodes
    take the float64 path, yet the oracle's margin (>= 1e-10) is far above a rounding tie.
"""
import contextlib

import numpy as np
import pytest

import oracle
import tree_attention_verification_ev_amd as ev
from synth import CONFIGS, generate, scaled
from synth.device import to_device

pytestmark = pytest.mark.gpu

C1, C2, C3, C4, C5 = CONFIGS


@contextlib.contextmanager
def bound_scale(s):
    old = ev.ev_accept_set_bound_scale(s)
    try:
        yield
    finally:
        ev.ev_accept_set_bound_scale(old)


def check(inp, min_margin=1e-12):
    dev = to_device(inp)
    got = [t.cpu().numpy() for t in
           ev.ev_accept_rejection(dev.logits, dev.tokens, dev.parent, dev.tau, dev.uniforms,
                                  check=True)]
    exp = oracle.rejection_batch(inp.logits, inp.tokens, inp.parent, inp.tau, inp.uniforms)
    margins = [m for ms in exp[3] for m in ms]
    assert min(margins) > min_margin
    for a, b in zip(got, exp[:3]):
        assert np.array_equal(a, b)
    return margins


FORCED = [
    ("C1", C1), ("C2", C2),
    ("C3_V5000", scaled(C3, V=5000, L=8)),
    ("C4_V3001", scaled(C4, V=3001, L=(8, 16))),
    ("C3_full", C3),
    ("C5_B2", scaled(C5, B=2, L=8)),
]


@pytest.mark.parametrize("mode", ["planted", "raw"])
@pytest.mark.parametrize("name,cfg", FORCED, ids=[n for n, _ in FORCED])
def test_float64_path_bit_exact(name, cfg, mode):
    """Every node the walk visits recomputed in float64 (bound scaled to 1e300)."""
    inp = generate(cfg, tokens=mode, with_kv=False)
    with bound_scale(1e300):
        check(inp)


def test_bound_scale_is_restored_and_validated():
    old = ev.ev_accept_set_bound_scale(2.0)
    assert ev.ev_accept_set_bound_scale(-1.0) == 2.0      # not > 0: unchanged
    assert ev.ev_accept_set_bound_scale(old) == 2.0


def _root_cumulative(inp, b):
    """The oracle's running sums at the root of sequence b (no token rejected)."""
    p = oracle.target_probs(inp.logits[b, 0], inp.tau)
    C = np.empty_like(p)
    acc = 0.0
    for y in range(len(p)):
        acc += float(p[y])
        C[y] = acc
    return p, C


@pytest.mark.parametrize("side", [+1, -1])
def test_draws_at_a_mass_boundary(side):
    """Root-only trees whose bonus threshold sits 1e-9 past (or before) the start of the
    heaviest token's interval: inside the float32 bound, outside a rounding tie."""
    cfg = scaled(C3, B=16, T=1, V=20000, L=8)
    inp = generate(cfg, tokens="raw", with_kv=False)
    for b in range(cfg.B):
        p, C = _root_cumulative(inp, b)
        # the heaviest token whose left neighbour also carries real mass, so that either
        # side of the edge is a token interval far wider than 1e-9
        both = (p[1:] > 1e-4) & (p[:-1] > 1e-4)
        y = 1 + int(np.argmax(np.where(both, p[1:], 0.0)))
        assert both[y - 1]
        inp.uniforms[b, 0] = C[y - 1] + side * 1e-9
    margins = check(inp, min_margin=1e-10)
    assert max(margins) < 1e-8                      # every draw was a near edge


@pytest.mark.parametrize("side", [+1, -1])
def test_child_tests_at_the_acceptance_edge(side):
    """Two-node chains whose child's uniform puts u Z within 1e-9 relative of p(x):
    accepted (side -1) or rejected (side +1) by a margin inside the float32 bound."""
    cfg = scaled(C3, B=16, T=2, tree="chain", V=20000, L=8)
    inp = generate(cfg, tokens="raw", with_kv=False)
    for b in range(cfg.B):
        p = oracle.target_probs(inp.logits[b, 0], inp.tau)
        x = int(np.argmax(p))
        inp.tokens[b, 1] = x
        inp.uniforms[b, 1] = float(p[x]) * (1.0 + side * 1e-9)
    margins = check(inp, min_margin=1e-13)
    assert min(margins) < 1e-8                      # the child tests were near edges
