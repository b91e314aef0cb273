"""GPU parity: the HIP library against the float64 oracle on identical seeded inputs.

Bars: attention O within 1e-2 max-abs and LSE within 1e-3 (bf16 inputs, float32
softmax); float32 attention within 1e-5 / 1e-5; masks, acceptance (lengths, paths,
tokens) and compaction bit-exact.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import tree_attention_verification_ev_amd as ev
from synth import CONFIGS, generate, round_to_bf16, scaled
from synth.device import to_device

pytestmark = pytest.mark.gpu

C1, C2, C3, C4, C5 = CONFIGS
O_TOL_BF16, LSE_TOL_BF16 = 1e-2, 1e-3
O_TOL_F32, LSE_TOL_F32 = 1e-5, 1e-5


def bf16_bound(Oo, O_abs):
    """Elementwise error bound of a bf16 output, used above the 1e-2 bar where |O| is
    large (only reachable with a handful of visible keys, e.g. an empty prefix):
      - the output rounded to bf16: at most half an ulp, 2^-8 |O|;
      - the probabilities rounded to bf16 before the value product: each p by at most
        2^-9 relative, so at most 2^-9 sum_i p_i |v_i| / l = 2^-9 O_abs, where O_abs is
        the attention output over |V|;
      - fp16 split partials (pre-divided by their row's max): 2^-11 O_abs;
      - float32 products, sums and exponentials: below 1e-5 at these magnitudes."""
    return 2.0 ** -8 * np.abs(Oo) + (2.0 ** -9 + 2.0 ** -11) * O_abs + 1e-5


def o_error(O, Oo, sel, dtype, O_abs=None):
    """Largest error in units of the allowed tolerance (<= 1 passes) and the max-abs error.
    bf16: 1e-2, or the bf16_bound where that is larger and O_abs (the oracle's output over
    |V|) is given; f32: 1e-5."""
    mask = np.broadcast_to(sel[..., None], O.shape)
    err = np.abs(O - Oo)[mask]
    if dtype == "bf16":
        tol = O_TOL_BF16 if O_abs is None else np.maximum(O_TOL_BF16, bf16_bound(Oo[mask], O_abs[mask]))
    else:
        tol = O_TOL_F32
    return float((err / tol).max()), float(err.max())


def scale_of(cfg):
    return float(np.float32(1.0 / math.sqrt(cfg.d)))


def max_prefix(inp):
    """The batch's longest prefix: the bound the split plan is sized from."""
    return int(inp.prefix_len.max())


def gpu_attention(inp, dev):
    kv = ev.KvCache(dev.k, dev.v, dev.block_table)
    anc, depth = ev.ev_tree_mask_build(dev.parent, check=True)
    out, lse = ev.ev_tree_attention(dev.q, kv, dev.prefix_len, anc, scale_of(inp.cfg), check=True,
                                    max_prefix_len=max_prefix(inp))
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy(), anc, depth


def oracle_attention(inp, seqs=None, heads=None, abs_v=False):
    """The oracle on the batch; abs_v: over |V| (the magnitude term of the bf16 bound)."""
    anc, _ = oracle.tree_mask_batch(inp.parent)
    v = np.abs(inp.v) if abs_v else inp.v
    return oracle.tree_attention_batch(inp.q, inp.k, v, inp.prefix_len, anc, inp.layout,
                                       inp.block_table, inp.cfg.block_size, scale_of(inp.cfg),
                                       seqs=seqs, heads=heads)


def check_attention(inp, seqs=None, heads=None):
    dev = to_device(inp)
    O, LSE, _, _ = gpu_attention(inp, dev)
    Oo, Lo = oracle_attention(inp, seqs, heads)
    sel = np.isfinite(Lo)
    assert sel.any()
    # (the actual prefixes: a test may cut some after the cache is built)
    shortest = min(min(inp.cfg.prefix_range()), int(np.min(inp.prefix_len)))
    short = inp.cfg.dtype == "bf16" and shortest < 128
    O_abs = oracle_attention(inp, seqs, heads, abs_v=True)[0] if short else None
    o_ratio, o_err = o_error(O, Oo, sel, inp.cfg.dtype, O_abs)
    l_err = np.abs(LSE - Lo)[sel].max()
    tol_l = LSE_TOL_BF16 if inp.cfg.dtype == "bf16" else LSE_TOL_F32
    assert np.isfinite(O).all() and np.isfinite(LSE).all()
    assert o_ratio <= 1.0 and l_err <= tol_l, (o_err, l_err)
    if inp.cfg.L and shortest >= 128:
        assert o_err <= (O_TOL_BF16 if inp.cfg.dtype == "bf16" else O_TOL_F32)
    return o_err, l_err


# ---------------------------------------------------------------- mask
@pytest.mark.parametrize("seed", range(4))
def test_mask_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    B, T = 7, [1, 2, 17, 64][seed]
    parent = np.array([[-1] + [int(rng.integers(i)) for i in range(1, T)] for _ in range(B)], np.int32)
    anc, depth = ev.ev_tree_mask_build(torch.from_numpy(parent).cuda(), check=True)
    ao, do = oracle.tree_mask_batch(parent)
    assert np.array_equal(anc.cpu().numpy().view(np.uint64), ao)
    assert np.array_equal(depth.cpu().numpy(), do)


def test_mask_rejects_bad_parent():
    parent = torch.tensor([[-1, 0, 3, 1]], dtype=torch.int32, device="cuda")
    with pytest.raises(ev.EvError) as e:
        ev.ev_tree_mask_build(parent, check=True)
    assert e.value.code == 101


# ---------------------------------------------------------------- attention
ATTN_SMALL = [
    ("C1", C1),
    ("C2_L300", scaled(C2, L=300, V=64)),
    ("C3_L300", scaled(C3, L=300, V=64)),
    ("C3_L0", scaled(C3, L=0, V=64)),
    ("C3_L64_aligned", scaled(C3, L=64, V=64)),
    ("C4_small", scaled(C4, B=4, L=(40, 400), V=64)),
    ("C5_small", scaled(C5, B=2, L=700, V=64)),
    ("C3_varlen_contiguous", scaled(C3, B=3, L=(10, 900), V=64)),
    ("chain64_mha", scaled(C2, T=64, tree="chain", L=130, V=64, Hq=4, Hkv=4)),
    ("star64_gqa", scaled(C3, tree="star", L=77, V=64)),
    ("root_only", scaled(C3, T=1, tree="grow", L=200, V=64)),
    ("bf16_d64", scaled(C3, d=64, L=333, V=64)),
    # 16 x 8 x 2 = 256 work units: one split, the register-staged kernel's unsplit output
    ("bf16_d64_one_split", scaled(C4, d=64, L=(100, 900), V=64)),
    ("f32_d128", scaled(C1, d=128, L=190, Hq=8, Hkv=2, V=64)),
    # float32 blocks of 8 rows (eight wavefronts): d = 128, and paged d = 64
    ("f32_d128_8rows", scaled(C1, d=128, L=150, V=64)),
    ("f32_paged_8rows", scaled(C1, paged=True, L=(70, 200), B=3, V=64)),
    # float32 over a shuffled block table, 64 rows per KV head (two row blocks of 32)
    ("f32_paged_gqa", scaled(C4, dtype="f32", B=2, T=16, Hq=32, Hkv=8, L=(60, 300), V=64)),
    ("gqa4_T26", scaled(C2, Hq=32, Hkv=8, L=515, V=64)),
    # 64 rows per KV head: the two-wavefront DMA workgroup
    ("gqa8_T8", scaled(C3, T=8, L=257, V=64)),
    # 320 rows per KV head: the second eight-wavefront workgroup has six waves with no row
    ("gqa8_T40", scaled(C3, T=40, L=190, V=64)),
    # paged, 104 rows per KV head: the four-wavefront DMA workgroup over a block table
    ("paged_gqa4_T26", scaled(C4, B=2, T=26, Hq=32, Hkv=8, L=(100, 700), V=64)),
]


@pytest.mark.parametrize("name,cfg", ATTN_SMALL, ids=[n for n, _ in ATTN_SMALL])
def test_attention_small(name, cfg):
    check_attention(generate(cfg, with_logits=False))


@pytest.mark.parametrize("cfg", [C2, C3], ids=["C2_full", "C3_full"])
def test_attention_full_contiguous(cfg):
    check_attention(generate(cfg, with_logits=False))


def test_attention_full_batched_paged():
    check_attention(generate(C4, with_logits=False))


def test_attention_full_long_context_sampled_heads():
    inp = generate(C5, with_logits=False)
    check_attention(inp, heads=[0, 9, 18, 27, 36, 45, 54, 63])


@pytest.mark.parametrize("bs", [1, 2, 4, 8, 32, 64, 256])
def test_attention_paged_page_sizes(bs):
    """Pages of 1 and 2 tokens take the slot-by-slot tile fetch; pages of 4 or more the
    per-instruction one (each four-slot piece of a tile lies in one page), including
    pages longer than a 64-key tile.  GQA 64/8 with short splits: the 128-row key-split
    workgroups."""
    check_attention(generate(scaled(C4, B=2, L=(300, 1500), V=64, block_size=bs),
                             with_logits=False))


@pytest.mark.parametrize("bs", [4, 256])
def test_attention_paged_page_sizes_long_splits(bs):
    """As above with splits of more than 16 tiles: 256-row eight-wavefront workgroups,
    32 of them per split (8 splits, read off the workspace size)."""
    inp = generate(scaled(C4, B=2, L=(9000, 12000), V=64, block_size=bs), with_logits=False)
    dev = to_device(inp)
    kv = ev.KvCache(dev.k, dev.v, dev.block_table)
    rows = 2 * C4.T * C4.Hq                     # B = 2
    assert ev.ev_tree_attention_workspace(kv, 2, C4.T, C4.Hq, max_prefix(inp)) == rows * 8 * (2 * C4.d + 8)
    check_attention(inp)


@pytest.mark.parametrize("B,L,short", [(6, (2800, 4000), True), (3, (6000, 6100), False)])
def test_attention_mixed_prefix_lengths(B, L, short):
    """Sequences of different lengths, splits past the end of the shorter ones; `short`:
    two prefixes cut to 0 and 5 tokens after the cache is built (the tree then sits on the
    first slots, read the same way by the oracle)."""
    inp = generate(scaled(C4, B=B, L=L, V=64), with_logits=False)
    if short:
        inp.prefix_len[1], inp.prefix_len[2] = 0, 5
    check_attention(inp)


def check_attention_dev(inp, kv, dev, seqs=None, heads=None):
    """Attention on an already-built device cache (same logical contents as inp) against
    the oracle on inp."""
    anc, _ = ev.ev_tree_mask_build(dev.parent, check=True)
    out, lse = ev.ev_tree_attention(dev.q, kv, dev.prefix_len, anc, scale_of(inp.cfg), check=True,
                                    max_prefix_len=max_prefix(inp))
    O, LSE = out.float().cpu().numpy(), lse.cpu().numpy()
    Oo, Lo = oracle_attention(inp, seqs, heads)
    sel = np.isfinite(Lo)
    assert sel.any() and np.isfinite(O).all() and np.isfinite(LSE).all()
    o_ratio, o_err = o_error(O, Oo, sel, "bf16")
    l_err = np.abs(LSE - Lo)[sel].max()
    assert o_err <= O_TOL_BF16 and l_err <= LSE_TOL_BF16, (o_err, l_err)


def test_attention_serving_capacity_contiguous():
    """The Llama-3-70B-shaped layer over a cache sized for 32k tokens per sequence: the
    split plan follows the prefix (max_prefix_len), not the capacity, and the result is
    the tight cache's."""
    inp = generate(C3, with_logits=False)
    dev = to_device(inp)
    cap = 32848
    k = torch.full((1, C3.Hkv, cap, C3.d), float("nan"), dtype=torch.bfloat16, device="cuda")
    v = torch.full_like(k, float("nan"))
    k[:, :, :inp.cap] = dev.k
    v[:, :, :inp.cap] = dev.v
    kv_big, kv_tight = ev.KvCache(k, v), ev.KvCache(dev.k, dev.v)
    mpl = max_prefix(inp)
    assert (ev.ev_tree_attention_workspace(kv_big, 1, C3.T, C3.Hq, mpl)
            == ev.ev_tree_attention_workspace(kv_tight, 1, C3.T, C3.Hq, mpl))
    check_attention_dev(inp, kv_big, dev)


def test_attention_serving_capacity_paged():
    """The batched paged layer with a block table 2048 blocks wide (32k slots per sequence)
    and a pool with spare blocks: same result as the tight table, every head compared."""
    inp = generate(C4, with_logits=False)
    dev = to_device(inp)
    B, wide = C4.B, 2048
    table = torch.full((B, wide), -1, dtype=torch.int32, device="cuda")
    table[:, :inp.block_table.shape[1]] = dev.block_table
    check_attention_dev(inp, ev.KvCache(dev.k, dev.v, table), dev, seqs=[0, 5, 11])


@pytest.mark.parametrize("L", [300, 350, 410, 4000])
def test_attention_planned_beyond_the_prefix(L):
    """Splits planned for a 4096-token prefix over a shorter one: the contiguous kernel
    fetches each split's first two tiles before it knows the length, so with L = 300 or
    350 the sequence's partial last tile is such an early tile (its stale rows past the
    sequence must not reach the output) and later splits are empty."""
    inp = generate(scaled(C3, L=L, V=64), with_logits=False)
    dev = to_device(inp)
    cap = 4096 + C3.T + 16
    k = torch.full((1, C3.Hkv, cap, C3.d), float("nan"), dtype=torch.bfloat16, device="cuda")
    v = torch.full_like(k, float("nan"))
    k[:, :, :inp.cap] = dev.k
    v[:, :, :inp.cap] = dev.v
    kv = ev.KvCache(k, v)
    anc, _ = ev.ev_tree_mask_build(dev.parent, check=True)
    out, lse = ev.ev_tree_attention(dev.q, kv, dev.prefix_len, anc, scale_of(C3), check=True,
                                    max_prefix_len=4096)
    O, LSE = out.float().cpu().numpy(), lse.cpu().numpy()
    Oo, Lo = oracle_attention(inp)
    assert np.isfinite(O).all() and np.isfinite(LSE).all()
    assert np.abs(O - Oo).max() <= O_TOL_BF16 and np.abs(LSE - Lo).max() <= LSE_TOL_BF16


def test_attention_paged_planned_beyond_the_prefix():
    inp = generate(scaled(C4, B=3, L=(100, 700), V=64), with_logits=False)
    dev = to_device(inp)
    table = torch.full((3, 260), -1, dtype=torch.int32, device="cuda")
    table[:, :inp.block_table.shape[1]] = dev.block_table
    kv = ev.KvCache(dev.k, dev.v, table)
    anc, _ = ev.ev_tree_mask_build(dev.parent, check=True)
    out, lse = ev.ev_tree_attention(dev.q, kv, dev.prefix_len, anc, scale_of(C4), check=True,
                                    max_prefix_len=4000)
    Oo, Lo = oracle_attention(inp)
    O, LSE = out.float().cpu().numpy(), lse.cpu().numpy()
    ratio, _ = o_error(O, Oo, np.isfinite(Lo), "bf16")
    assert ratio <= 1.0 and np.abs(LSE - Lo).max() <= LSE_TOL_BF16


def test_paged_equals_contiguous_on_the_same_data():
    cfg = scaled(C4, B=3, L=(100, 900), V=64)
    a = generate(cfg, layout="contiguous", with_logits=False)
    b = generate(cfg, layout="paged", with_logits=False)
    Oa, La, _, _ = gpu_attention(a, to_device(a))
    Ob, Lb, _, _ = gpu_attention(b, to_device(b))
    assert np.abs(Oa - Ob).max() <= 2e-3 and np.abs(La - Lb).max() <= 1e-5


def test_attention_is_deterministic():
    """100 repeats are bitwise identical (no run-order or race dependence)."""
    inp = generate(scaled(C3, L=1000, V=64), with_logits=False)
    dev = to_device(inp)
    kv = ev.KvCache(dev.k, dev.v, dev.block_table)
    anc, _ = ev.ev_tree_mask_build(dev.parent, check=True)
    mpl = max_prefix(inp)
    O1, L1 = ev.ev_tree_attention(dev.q, kv, dev.prefix_len, anc, scale_of(inp.cfg), check=True,
                                  max_prefix_len=mpl)
    O2, L2 = torch.empty_like(O1), torch.empty_like(L1)
    ws = torch.zeros(max(1, ev.ev_tree_attention_workspace(kv, 1, inp.cfg.T, inp.cfg.Hq, mpl)),
                     dtype=torch.uint8, device="cuda")
    for _ in range(100):
        ev.ev_tree_attention(dev.q, kv, dev.prefix_len, anc, scale_of(inp.cfg), O2, L2, ws,
                             max_prefix_len=mpl)
        assert torch.equal(O1, O2) and torch.equal(L1, L2)


def test_attention_reports_prefix_beyond_cache():
    inp = generate(scaled(C3, L=100, V=64), with_logits=False)
    dev = to_device(inp)
    dev.prefix_len.fill_(inp.cap)                      # L + T > cap
    kv = ev.KvCache(dev.k, dev.v)
    anc, _ = ev.ev_tree_mask_build(dev.parent, check=True)
    with pytest.raises(ev.EvError) as e:
        ev.ev_tree_attention(dev.q, kv, dev.prefix_len, anc, check=True)
    assert e.value.code == 102


@pytest.mark.parametrize("paged", [False, True])
def test_attention_reports_prefix_beyond_bound(paged):
    """A prefix longer than the max_prefix_len the call was planned for is a device error
    (the splits do not cover it), even where the cache could hold it."""
    cfg = scaled(C4, B=3, L=(200, 900), V=64) if paged else scaled(C3, B=2, L=(300, 900), V=64)
    inp = generate(cfg, with_logits=False)
    dev = to_device(inp)
    kv = ev.KvCache(dev.k, dev.v, dev.block_table)
    anc, _ = ev.ev_tree_mask_build(dev.parent, check=True)
    with pytest.raises(ev.EvError) as e:
        ev.ev_tree_attention(dev.q, kv, dev.prefix_len, anc, check=True,
                             max_prefix_len=max_prefix(inp) - 1)
    assert e.value.code == 102


def test_attention_reports_bad_block_id():
    inp = generate(scaled(C4, B=2, L=(50, 90), V=64), with_logits=False)
    dev = to_device(inp)
    dev.block_table[1, 0] = inp.k.shape[0] + 5
    kv = ev.KvCache(dev.k, dev.v, dev.block_table)
    anc, _ = ev.ev_tree_mask_build(dev.parent, check=True)
    with pytest.raises(ev.EvError) as e:
        ev.ev_tree_attention(dev.q, kv, dev.prefix_len, anc, check=True)
    assert e.value.code == 102


# ---------------------------------------------------------------- acceptance
def run_greedy(inp, dev):
    out = ev.ev_accept_greedy(dev.logits, dev.tokens, dev.parent, check=True)
    return [t.cpu().numpy() for t in out]


def run_rejection(inp, dev):
    out = ev.ev_accept_rejection(dev.logits, dev.tokens, dev.parent, dev.tau, dev.uniforms, check=True)
    return [t.cpu().numpy() for t in out]


ACC_CASES = [
    ("C1", C1), ("C2", C2),
    ("C3_V5000", scaled(C3, V=5000, L=8)),
    ("C4_V3001", scaled(C4, V=3001, L=(8, 16))),
    ("C5_V128256_B2", scaled(C5, B=2, L=8)),
    ("V1", scaled(C3, V=1, T=1, L=8)),
    ("V7_chain", scaled(C3, V=70, T=64, tree="chain", L=8)),
]


@pytest.mark.parametrize("mode", ["planted", "raw"])
@pytest.mark.parametrize("name,cfg", ACC_CASES, ids=[n for n, _ in ACC_CASES])
def test_greedy_bit_exact(name, cfg, mode):
    inp = generate(cfg, tokens=mode, with_kv=False)
    g = run_greedy(inp, to_device(inp))
    o = oracle.greedy_batch(inp.logits, inp.tokens, inp.parent)
    for a, b in zip(g, o):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("mode", ["planted", "raw"])
@pytest.mark.parametrize("name,cfg", ACC_CASES, ids=[n for n, _ in ACC_CASES])
def test_rejection_bit_exact(name, cfg, mode):
    inp = generate(cfg, tokens=mode, with_kv=False)
    r = run_rejection(inp, to_device(inp))
    o = oracle.rejection_batch(inp.logits, inp.tokens, inp.parent, inp.tau, inp.uniforms)
    assert min(min(m) for m in o[3]) > 1e-12            # no decision is a rounding tie
    for a, b in zip(r, o[:3]):
        assert np.array_equal(a, b)


FULL_ACC = [C3, C4, scaled(C3, V=128255)]
FULL_ACC_IDS = ["C3_full", "C4_full", "C3_full_V128255_unaligned_rows"]


@pytest.mark.parametrize("cfg", FULL_ACC, ids=FULL_ACC_IDS)
def test_rejection_full_size(cfg):
    inp = generate(cfg, with_kv=False)
    r = run_rejection(inp, to_device(inp))
    o = oracle.rejection_batch(inp.logits, inp.tokens, inp.parent, inp.tau, inp.uniforms)
    assert min(min(m) for m in o[3]) > 1e-12
    for a, b in zip(r, o[:3]):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("cfg", FULL_ACC, ids=FULL_ACC_IDS)
def test_greedy_full_size(cfg):
    inp = generate(cfg, tokens="raw", with_kv=False)
    g = run_greedy(inp, to_device(inp))
    o = oracle.greedy_batch(inp.logits, inp.tokens, inp.parent)
    for a, b in zip(g, o):
        assert np.array_equal(a, b)


def test_rejection_many_seeds_bonus_paths():
    """Many sequences whose walks end in residual draws with rejected siblings."""
    cfg = scaled(C3, B=64, V=2000, L=8)
    inp = generate(cfg, tokens="raw", with_kv=False)
    r = run_rejection(inp, to_device(inp))
    o = oracle.rejection_batch(inp.logits, inp.tokens, inp.parent, inp.tau, inp.uniforms)
    for a, b in zip(r, o[:3]):
        assert np.array_equal(a, b)


def test_rejection_gpu_preserves_target_distribution_chi_square():
    """The GPU sampler itself emits the target's distribution (explainer "Why it works";
    study note case 3): 5e5 copies of a tiny tree with fresh uniforms.  The first emitted
    token must follow p_root, and the second, given node 1 was accepted, p_node1."""
    import scipy.special
    import scipy.stats
    V, tau = 8, 0.7
    parent = np.array([-1, 0, 0, 0, 1, 1], np.int32)
    rng = np.random.default_rng(2024)
    logits = (2 * rng.standard_normal((6, V))).astype(np.float32)
    top, t1 = int(np.argmax(logits[0])), int(np.argmax(logits[1]))
    tokens = np.array([0, top, (top + 3) % V, (top + 5) % V, t1, (t1 + 2) % V], np.int32)
    Bc, calls = 10000, 50
    lg = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(logits, (Bc, 6, V)))).cuda()
    tk = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(tokens, (Bc, 6)))).cuda()
    pa = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(parent, (Bc, 6)))).cuda()
    first, second, lens = np.zeros(V, np.int64), np.zeros(V, np.int64), np.zeros(3, np.int64)
    urng = np.random.default_rng(2025)
    for _ in range(calls):
        u = torch.from_numpy(urng.random((Bc, 6))).cuda()
        acc, path, out = (t.cpu().numpy() for t in
                          ev.ev_accept_rejection(lg, tk, pa, tau, u, check=True))
        first += np.bincount(out[:, 0], minlength=V)
        sel = (acc >= 1) & (path[:, 1] == 1)
        second += np.bincount(out[sel, 1], minlength=V)
        lens += np.bincount(acc, minlength=3)[:3]
    inv_tau = 1.0 / np.float64(np.float32(tau))
    ref0 = scipy.special.softmax(logits[0].astype(np.float64) * inv_tau)
    ref1 = scipy.special.softmax(logits[1].astype(np.float64) * inv_tau)
    pv0 = scipy.stats.chisquare(first, first.sum() * ref0).pvalue
    pv1 = scipy.stats.chisquare(second, second.sum() * ref1).pvalue
    assert pv0 > 1e-3 and pv1 > 1e-3, (pv0, pv1, first, second)
    assert lens[1] > 0 and lens[2] > 0


def test_accept_workspace_reuse_across_shapes():
    """One zeroed workspace serves consecutive calls of different shapes, and every call
    leaves the arrival counters at zero (the workspace contract of the acceptance calls)."""
    big = scaled(C3, B=4, V=20000, L=8)
    small = scaled(C3, B=2, V=3000, L=8)
    ws = torch.zeros(ev.ev_accept_workspace(4, big.T, big.V), dtype=torch.uint8, device="cuda")
    ws[ev.ev_accept_workspace(1, 1, 1):].fill_(0x5A)        # garbage beyond the counters
    counters = 2 * 65536 * 4
    for cfg, rej in ((big, True), (small, True), (big, False), (small, False), (big, True)):
        inp = generate(cfg, tokens="raw", with_kv=False)
        dev = to_device(inp)
        if rej:
            got = ev.ev_accept_rejection(dev.logits, dev.tokens, dev.parent, dev.tau, dev.uniforms,
                                         ws=ws, check=True)
            exp = oracle.rejection_batch(inp.logits, inp.tokens, inp.parent, inp.tau, inp.uniforms)
        else:
            got = ev.ev_accept_greedy(dev.logits, dev.tokens, dev.parent, ws=ws, check=True)
            exp = oracle.greedy_batch(inp.logits, inp.tokens, inp.parent)
        for a, b in zip(got, exp[:3]):
            assert np.array_equal(a.cpu().numpy(), b)
        assert int(ws[:counters].count_nonzero()) == 0


@pytest.mark.parametrize("V", [3001, 128256])
def test_greedy_rows_of_negative_infinity(V):
    """Rows whose logits are all -inf have argmax 0 (the lowest index of the maximum), on
    the GPU as in the oracle: never an id outside [0, V)."""
    cfg = scaled(C3, B=3, V=V, L=8)
    inp = generate(cfg, tokens="raw", with_kv=False)
    inp.logits[0, 0, :] = -np.inf                       # root row: bonus or first step
    inp.logits[1, :, :] = -np.inf                       # every row of a sequence
    kids = np.nonzero(inp.parent[1] == 0)[0]
    inp.tokens[1, kids[0]] = 0                          # a child drafting 0 is accepted
    g = run_greedy(inp, to_device(inp))
    o = oracle.greedy_batch(inp.logits, inp.tokens, inp.parent)
    for a, b in zip(g, o):
        assert np.array_equal(a, b)
    assert g[2].max() < V and g[2][0, 0] >= 0 and o[0][1] >= 1


def test_accept_reports_bad_token():
    inp = generate(scaled(C3, V=500, L=8), with_kv=False)
    dev = to_device(inp)
    dev.tokens[0, 5] = 500
    with pytest.raises(ev.EvError) as e:
        ev.ev_accept_greedy(dev.logits, dev.tokens, dev.parent, check=True)
    assert e.value.code == 103


# ---------------------------------------------------------------- compaction
def compaction_case(cfg, layout, n_layers, seed=0):
    inp = generate(cfg, layout=layout, with_logits=False)
    rng = np.random.default_rng(seed)
    B, T = cfg.B, cfg.T
    paths = np.full((B, T), -1, np.int32)
    acc = np.zeros(B, np.int32)
    for b in range(B):
        # a random root path of the drawn tree
        leaf = int(rng.integers(T))
        p = []
        u = leaf
        while u != -1:
            p.append(u)
            u = int(inp.parent[b, u])
        p = p[::-1]
        paths[b, :len(p)] = p
        acc[b] = len(p) - 1
    k = np.stack([inp.k + 1000.0 * layer for layer in range(n_layers)])
    v = np.stack([inp.v - 1000.0 * layer for layer in range(n_layers)])
    if cfg.dtype == "bf16":
        k, v = round_to_bf16(k), round_to_bf16(v)
    return inp, k, v, paths, acc


@pytest.mark.parametrize("layout", ["contiguous", "paged"])
@pytest.mark.parametrize("n_layers", [1, 3])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_compaction_bit_exact(layout, n_layers, dtype):
    cfg = scaled(C4, B=5, L=(10, 200), V=64, dtype=dtype)
    inp, k, v, paths, acc = compaction_case(cfg, layout, n_layers)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kd = torch.from_numpy(k).cuda().to(dt)
    vd = torch.from_numpy(v).cuda().to(dt)
    bt = None if layout == "contiguous" else torch.from_numpy(inp.block_table).cuda()
    kv = ev.KvCache(kd, vd, bt, layered=True)
    new_len = ev.ev_kv_compact(kv, torch.from_numpy(inp.prefix_len).cuda(), torch.from_numpy(paths).cuda(),
                               torch.from_numpy(acc).cuda(), check=True)
    ko, vo, nlo = oracle.kv_compact(k, v, inp.prefix_len, paths, acc, layout, inp.block_table,
                                    cfg.block_size, layered=True)
    assert np.array_equal(new_len.cpu().numpy(), nlo)
    assert np.array_equal(kd.float().cpu().numpy(), ko, equal_nan=True)
    assert np.array_equal(vd.float().cpu().numpy(), vo, equal_nan=True)


def test_compaction_maximal_overlap():
    cfg = scaled(C3, L=50, V=64, T=64, tree="chain")
    inp = generate(cfg, with_logits=False)
    paths = np.full((1, 64), -1, np.int32)
    paths[0, :63] = [0] + list(range(2, 64))               # a_m = m + 1
    acc = np.array([62], np.int32)
    kd = torch.from_numpy(inp.k).cuda().to(torch.bfloat16)
    vd = torch.from_numpy(inp.v).cuda().to(torch.bfloat16)
    ev.ev_kv_compact(ev.KvCache(kd, vd), torch.from_numpy(inp.prefix_len).cuda(),
                     torch.from_numpy(paths).cuda(), torch.from_numpy(acc).cuda(), check=True)
    ko, vo, _ = oracle.kv_compact(inp.k, inp.v, inp.prefix_len, paths, acc, "contiguous")
    assert np.array_equal(kd.float().cpu().numpy(), ko, equal_nan=True)
    assert np.array_equal(vd.float().cpu().numpy(), vo, equal_nan=True)


def test_compaction_reports_bad_path():
    cfg = scaled(C3, L=50, V=64)
    inp = generate(cfg, with_logits=False)
    dev = to_device(inp)
    paths = torch.tensor([[0, 5, 3] + [-1] * 61], dtype=torch.int32, device="cuda")
    before = dev.k.clone()
    with pytest.raises(ev.EvError) as e:
        ev.ev_kv_compact(ev.KvCache(dev.k, dev.v), dev.prefix_len, paths,
                         torch.tensor([2], dtype=torch.int32, device="cuda"), check=True)
    assert e.value.code == 104
    assert torch.equal(before.view(torch.int16), dev.k.view(torch.int16))


# ---------------------------------------------------------------- whole pass
@pytest.mark.parametrize("cfg", CONFIGS, ids=[f"C{c.index}" for c in CONFIGS])
def test_full_verification_pass(cfg):
    """mask -> attention -> acceptance -> compaction on the workload at full size,
    attention compared on a sample of sequences/heads, the rest exhaustively."""
    inp = generate(cfg)
    dev = to_device(inp)
    O, LSE, anc, _ = gpu_attention(inp, dev)
    seqs = list(range(min(cfg.B, 2)))
    heads = sorted({0, cfg.Hq // 2, cfg.Hq - 1})
    Oo, Lo = oracle_attention(inp, seqs=seqs, heads=heads)
    sel = np.isfinite(Lo)
    tol_o, tol_l = (O_TOL_BF16, LSE_TOL_BF16) if cfg.dtype == "bf16" else (O_TOL_F32, LSE_TOL_F32)
    assert np.abs(LSE - Lo)[sel].max() <= tol_l
    assert np.abs(O - Oo)[np.broadcast_to(sel[..., None], O.shape)].max() <= tol_o
    kmax = 0
    kv = ev.KvCache(dev.k, dev.v, dev.block_table)
    for mode in cfg.accept:
        if mode == "greedy":
            got = run_greedy(inp, dev)
            exp = oracle.greedy_batch(inp.logits, inp.tokens, inp.parent)
        else:
            got = run_rejection(inp, dev)
            exp = oracle.rejection_batch(inp.logits, inp.tokens, inp.parent, inp.tau, inp.uniforms)[:3]
        for a, b in zip(got, exp):
            assert np.array_equal(a, b), mode
        kmax = max(kmax, int(exp[0].max()))
    if cfg.B > 1:
        assert kmax >= 2                                    # planted trees walk deep
    acc, path = torch.from_numpy(exp[0]).cuda(), torch.from_numpy(exp[1]).cuda()
    new_len = ev.ev_kv_compact(kv, dev.prefix_len, path, acc, check=True)
    ko, vo, nlo = oracle.kv_compact(inp.k, inp.v, inp.prefix_len, exp[1], exp[0], inp.layout,
                                    inp.block_table, cfg.block_size)
    assert np.array_equal(new_len.cpu().numpy(), nlo)
    assert np.array_equal(dev.k.float().cpu().numpy(), ko, equal_nan=True)
    assert np.array_equal(dev.v.float().cpu().numpy(), vo, equal_nan=True)


# ---------------------------------------------------------------- graph capture
def test_graph_replays_match_eager():
    """The verification calls captured in a HIP graph give the eager results on every replay,
    with unrelated eager work and synchronisations between replays."""
    cfg = scaled(C3, L=700, V=6000)
    inp = generate(cfg)
    dev = to_device(inp)
    kv = ev.KvCache(dev.k, dev.v)
    B, T = cfg.B, cfg.T
    anc = torch.zeros((B, T), dtype=torch.int64, device="cuda")
    depth = torch.zeros((B, T), dtype=torch.int32, device="cuda")
    out = torch.empty_like(dev.q)
    lse = torch.zeros((B, T, cfg.Hq), dtype=torch.float32, device="cuda")
    acc = torch.zeros(B, dtype=torch.int32, device="cuda")
    path = torch.zeros((B, T), dtype=torch.int32, device="cuda")
    tok = torch.zeros((B, T), dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    mpl = max_prefix(inp)
    ws_a = torch.zeros(max(1, ev.ev_tree_attention_workspace(kv, B, T, cfg.Hq, mpl)),
                       dtype=torch.uint8, device="cuda")
    ws_r = torch.zeros(ev.ev_accept_workspace(B, T, cfg.V), dtype=torch.uint8, device="cuda")

    def step():
        ev.ev_tree_mask_build(dev.parent, anc, depth, status)
        ev.ev_tree_attention(dev.q, kv, dev.prefix_len, anc, scale_of(cfg), out, lse, ws_a, status,
                             max_prefix_len=mpl)
        ev.ev_accept_rejection(dev.logits, dev.tokens, dev.parent, dev.tau, dev.uniforms, acc, path,
                               tok, ws_r, status)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (anc, out, lse, acc, path, tok)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(4):
        for t in (anc, out, lse, acc, path, tok):
            t.zero_()
        junk = torch.randn(1 << 20, device="cuda").sum()      # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, (anc, out, lse, acc, path, tok)):
            assert torch.equal(a, b)
        assert int(status.item()) == 0 and torch.isfinite(junk)
