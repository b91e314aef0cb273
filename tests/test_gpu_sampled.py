"""GPU parity of acceptance with sampled drafts (ev_accept_sampled) against the oracle.

Bar: accept_len, path and emitted tokens bit-exact on the same float32 logits, draft
logits and float64 uniforms, provided no decision of the oracle is a rounding tie
(every margin > 1e-12).  The GPU sampler's output distribution is also checked by
chi-square on many copies of a tiny tree whose drafts are drawn from q.
"""
import numpy as np
import pytest
import torch

import oracle
import tree_attention_verification_ev_amd as ev
from synth import CONFIGS, generate, sampled_drafts, scaled

pytestmark = pytest.mark.gpu

C1, C2, C3, C4, C5 = CONFIGS
DRAFT_TAU = 0.8


def max_children(parent):
    return max(int((p == a).sum()) for p in parent for a in range(parent.shape[1]))


def run_sampled(inp, draft, tokens, mc=None, ws=None):
    to = lambda x, dt: torch.from_numpy(np.ascontiguousarray(x)).to("cuda", dt)
    mc = max_children(inp.parent) if mc is None else mc
    out = ev.ev_accept_sampled(to(inp.logits, torch.float32), to(draft, torch.float32),
                               to(tokens, torch.int32), to(inp.parent, torch.int32), inp.tau,
                               DRAFT_TAU, to(inp.uniforms, torch.float64), mc, ws=ws, check=True)
    return [t.cpu().numpy() for t in out]


def oracle_sampled(inp, draft, tokens):
    return oracle.stochastic_batch(inp.logits, draft, tokens, inp.parent, inp.tau, DRAFT_TAU,
                                   inp.uniforms)


CASES = [
    ("C1", scaled(C1, V=1000)),
    ("C2_V4096", scaled(C2, V=4096, L=8)),
    ("C3_V4096", scaled(C3, V=4096, L=8)),
    ("C3_V5000_odd", scaled(C3, V=5001, L=8)),
    ("C4_B4", scaled(C4, B=4, V=3000, L=8)),
    ("C5_B2", scaled(C5, B=2, V=2048, L=8)),
    # 2048 rows of 3 chunks: the rounds after the first run over lists of undecided rows,
    # one chunk group (here the whole row) per work item
    ("C4_B32_V3000_list_rounds", scaled(C4, B=32, V=3000, L=8)),
]


@pytest.mark.parametrize("name,cfg", CASES, ids=[n for n, _ in CASES])
def test_sampled_bit_exact(name, cfg):
    inp = generate(cfg, with_kv=False)
    draft, tokens = sampled_drafts(inp, DRAFT_TAU)
    got = run_sampled(inp, draft, tokens)
    ref = oracle_sampled(inp, draft, tokens)
    assert min(min(m) for m in ref[3]) > 1e-12
    for a, b in zip(got, ref[:3]):
        assert np.array_equal(a, b)


# C3: every round over all rows (one chunk per wavefront); C4 with 3 sequences (two chunks
# per wavefront), 4 and 16 (four): later rounds over lists of the undecided rows, more
# work items than workgroups at 16
@pytest.mark.parametrize("cfg", [C3, scaled(C4, B=3), scaled(C4, B=4), C4],
                         ids=["C3_full", "C4_B3_fullV", "C4_B4_fullV", "C4_full"])
def test_sampled_full_vocabulary(cfg):
    inp = generate(cfg, with_kv=False)
    draft, tokens = sampled_drafts(inp, DRAFT_TAU)
    got = run_sampled(inp, draft, tokens)
    ref = oracle_sampled(inp, draft, tokens)
    assert min(min(m) for m in ref[3]) > 1e-12
    for a, b in zip(got, ref[:3]):
        assert np.array_equal(a, b)


def test_sampled_random_tokens_and_loose_width_bound():
    """Drafts unrelated to q (every child likely rejected, bonus from deep residuals) and a
    bound larger than needed (extra rounds find nothing left to decide)."""
    cfg = scaled(C3, B=3, V=1500, L=8)
    inp = generate(cfg, tokens="raw", with_kv=False)
    draft, _ = sampled_drafts(inp, DRAFT_TAU)
    got = run_sampled(inp, draft, inp.tokens, mc=cfg.T)
    ref = oracle_sampled(inp, draft, inp.tokens)
    assert min(min(m) for m in ref[3]) > 1e-12
    for a, b in zip(got, ref[:3]):
        assert np.array_equal(a, b)


def test_sampled_reports_too_many_children():
    cfg = scaled(C3, V=500, L=8)
    inp = generate(cfg, with_kv=False)
    draft, tokens = sampled_drafts(inp, DRAFT_TAU)
    with pytest.raises(ev.EvError) as e:
        run_sampled(inp, draft, tokens, mc=max_children(inp.parent) - 1)
    assert e.value.code == 105


def test_sampled_workspace_counters_return_to_zero():
    cfg = scaled(C3, B=2, V=3000, L=8)
    inp = generate(cfg, with_kv=False)
    draft, tokens = sampled_drafts(inp, DRAFT_TAU)
    ws = torch.zeros(ev.ev_accept_sampled_workspace(2, cfg.T, cfg.V), dtype=torch.uint8, device="cuda")
    ref = oracle_sampled(inp, draft, tokens)
    for _ in range(3):
        got = run_sampled(inp, draft, tokens, ws=ws)
        for a, b in zip(got, ref[:3]):
            assert np.array_equal(a, b)
        assert int(ws[:2 * 65536 * 4].count_nonzero()) == 0


def test_sampled_gpu_preserves_target_distribution_chi_square():
    """Drafts drawn from q on the host (Gumbel-max); the GPU's emitted tokens follow p."""
    import scipy.special
    import scipy.stats
    V, tau = 8, 0.7
    parent = np.array([-1, 0, 0, 0, 1, 1], np.int32)
    rng = np.random.default_rng(2024)
    logits = (2 * rng.standard_normal((6, V))).astype(np.float32)
    draft = (logits + rng.standard_normal((6, V))).astype(np.float32)
    inv_q = 1.0 / np.float64(np.float32(DRAFT_TAU))
    Bc, calls = 10000, 30
    lg = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(logits, (Bc, 6, V)))).cuda()
    dr = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(draft, (Bc, 6, V)))).cuda()
    pa = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(parent, (Bc, 6)))).cuda()
    first, second = np.zeros(V, np.int64), np.zeros(V, np.int64)
    for _ in range(calls):
        g = -np.log(-np.log(rng.random((Bc, 6, V))))
        tok = np.argmax(draft[parent[np.arange(6)].clip(0)][None] * inv_q + g, axis=-1).astype(np.int32)
        tok[:, 0] = 0
        u = torch.from_numpy(rng.random((Bc, 6))).cuda()
        acc, path, out = (t.cpu().numpy() for t in ev.ev_accept_sampled(
            lg, dr, torch.from_numpy(tok).cuda(), pa, tau, DRAFT_TAU, u, 3, check=True))
        first += np.bincount(out[:, 0], minlength=V)
        sel = (acc >= 1) & (path[:, 1] == 1)
        second += np.bincount(out[sel, 1], minlength=V)
    inv_tau = 1.0 / np.float64(np.float32(tau))
    ref0 = scipy.special.softmax(logits[0].astype(np.float64) * inv_tau)
    ref1 = scipy.special.softmax(logits[1].astype(np.float64) * inv_tau)
    pv0 = scipy.stats.chisquare(first, first.sum() * ref0).pvalue
    pv1 = scipy.stats.chisquare(second, second.sum() * ref1).pvalue
    assert pv0 > 1e-3 and pv1 > 1e-3, (pv0, pv1, first, second)


def test_sampled_root_only_trees():
    """T = 1: no child to test, every sequence emits one bonus token drawn from p (no rounds)."""
    cfg = scaled(C3, B=5, T=1, tree="grow", V=3000, L=8)
    inp = generate(cfg, with_kv=False)
    draft, tokens = sampled_drafts(inp, DRAFT_TAU)
    got = run_sampled(inp, draft, tokens, mc=0)
    ref = oracle_sampled(inp, draft, tokens)
    assert (got[0] == 0).all()
    for a, b in zip(got, ref[:3]):
        assert np.array_equal(a, b)


def test_sampled_list_rounds_reuse_workspace():
    """Calls that share one workspace, each on other trees and logits, with rounds over
    lists of undecided rows (2048 rows, four chunks per wavefront in the first round): the
    lists' counters start from zero in every call (the statistics launch clears them) and
    stale entries of an earlier call are never read."""
    cfg = scaled(C4, B=32, V=3000, L=8)
    ws = torch.zeros(ev.ev_accept_sampled_workspace(cfg.B, cfg.T, cfg.V), dtype=torch.uint8,
                     device="cuda")
    for seed in (11, 12, 13):
        inp = generate(cfg, with_kv=False, seed=seed)
        draft, tokens = sampled_drafts(inp, DRAFT_TAU)
        got = run_sampled(inp, draft, tokens, ws=ws)
        ref = oracle_sampled(inp, draft, tokens)
        assert min(min(m) for m in ref[3]) > 1e-12
        for a, b in zip(got, ref[:3]):
            assert np.array_equal(a, b), seed
        assert int(ws[:2 * 65536 * 4].count_nonzero()) == 0
