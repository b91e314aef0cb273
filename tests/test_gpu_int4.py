"""GPU parity of tree attention and compaction over an INT4-quantised KV cache against
the oracle (attention over the dequantised values bf16(scale * q); compaction and
zero-copy pruning bit-exact on the packed bytes and the scales).  Attention bars are those
of the bfloat16 path."""
import math

import numpy as np
import pytest
import torch

import oracle
import tree_attention_verification_ev_amd as ev
from synth import CONFIGS, generate, quantize_int4, scaled
from test_gpu_parity import LSE_TOL_BF16, O_TOL_BF16, o_error

pytestmark = pytest.mark.gpu
C1, C2, C3, C4, C5 = CONFIGS
c = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()


def int4_attention(inp, seqs=None, heads=None, one_split=None):
    cfg = inp.cfg
    kq, ks = quantize_int4(inp.k)
    vq, vs = quantize_int4(inp.v)
    bt = c(inp.block_table) if inp.block_table is not None else None
    kv = ev.KvCache(c(kq), c(vq), bt, k_scale=c(ks), v_scale=c(vs))
    scale = float(np.float32(1.0 / math.sqrt(cfg.d)))
    anc, _ = ev.ev_tree_mask_build(c(inp.parent), check=True)
    mpl = int(inp.prefix_len.max())
    if one_split is not None:     # the plan's split count shows in its workspace size
        assert (ev.ev_tree_attention_workspace(kv, cfg.B, cfg.T, cfg.Hq, mpl) == 0) == one_split
    out, lse = ev.ev_tree_attention(c(inp.q).to(torch.bfloat16), kv, c(inp.prefix_len), anc, scale,
                                    check=True, max_prefix_len=mpl)
    ao, _ = oracle.tree_mask_batch(inp.parent)
    Oo, Lo = oracle.tree_attention_batch(inp.q, oracle.dequant_int4(kq, ks), oracle.dequant_int4(vq, vs),
                                         inp.prefix_len, ao, inp.layout, inp.block_table,
                                         cfg.block_size, scale, seqs=seqs, heads=heads)
    O, L = out.float().cpu().numpy(), lse.cpu().numpy()
    sel = np.isfinite(Lo)
    O_abs = None
    if min(cfg.prefix_range()) < 128:      # |O| can exceed 1: the bf16 bound needs O over |V|
        O_abs, _ = oracle.tree_attention_batch(inp.q, oracle.dequant_int4(kq, ks),
                                               np.abs(oracle.dequant_int4(vq, vs)), inp.prefix_len,
                                               ao, inp.layout, inp.block_table, cfg.block_size,
                                               scale, seqs=seqs, heads=heads)
    ratio, err = o_error(O, Oo, sel, "bf16", O_abs)
    assert np.isfinite(O).all() and np.isfinite(L).all()
    assert ratio <= 1.0 and np.abs(L - Lo)[sel].max() <= LSE_TOL_BF16, (err, np.abs(L - Lo)[sel].max())


CASES = [
    ("C2_L300", scaled(C2, L=300, V=64)),
    ("C3_L300", scaled(C3, L=300, V=64)),
    ("C3_L0", scaled(C3, L=0, V=64)),
    ("C4_small_paged", scaled(C4, B=4, L=(40, 400), V=64)),
    ("C5_small_paged", scaled(C5, B=2, L=700, V=64)),
    ("d64", scaled(C3, d=64, L=333, V=64)),
    ("gqa4_T26", scaled(C2, Hq=32, Hkv=8, L=515, V=64)),
    ("C2_full_mha", scaled(C2, V=64)),
    ("C3_full", scaled(C3, V=64)),
]


@pytest.mark.parametrize("name,cfg", CASES, ids=[n for n, _ in CASES])
def test_int4_attention(name, cfg):
    int4_attention(generate(cfg, with_logits=False))


def test_int4_attention_full_batched_paged_one_split():
    """Full batched paged layer (B = 16): 256 work units, so one split and the unsplit
    output path (bf16 O and LSE written directly); three sequences compared, all heads."""
    int4_attention(generate(C4, with_logits=False), seqs=[0, 7, 15], one_split=True)


def test_int4_attention_full_long_context_sampled_heads():
    inp = generate(C5, with_logits=False)
    int4_attention(inp, heads=[0, 9, 18, 27, 36, 45, 54, 63], one_split=False)


@pytest.mark.parametrize("layout", ["contiguous", "paged"])
def test_int4_compaction_bit_exact(layout):
    cfg = scaled(C4, B=5, L=(10, 200), V=64)
    inp = generate(cfg, layout=layout, with_logits=False)
    kq, ks = quantize_int4(inp.k)
    vq, vs = quantize_int4(inp.v)
    rng = np.random.default_rng(5)
    T = cfg.T
    paths = np.full((cfg.B, T), -1, np.int32)
    acc = np.zeros(cfg.B, np.int32)
    for b in range(cfg.B):
        kb = int(rng.integers(0, 7))
        paths[b, :kb + 1] = [0] + sorted(rng.choice(np.arange(1, T), size=kb, replace=False).tolist())
        acc[b] = kb
    d = [c(kq), c(vq), c(ks), c(vs)]
    bt = c(inp.block_table) if layout == "paged" else None
    kv = ev.KvCache(d[0], d[1], bt, k_scale=d[2], v_scale=d[3])
    nl = ev.ev_kv_compact(kv, c(inp.prefix_len), c(paths), c(acc), check=True)
    want = [oracle.kv_compact(x, y, inp.prefix_len, paths, acc, layout, inp.block_table, cfg.block_size)
            for x, y in ((kq, vq), (ks, vs))]
    assert np.array_equal(nl.cpu().numpy(), want[0][2])
    assert np.array_equal(d[0].cpu().numpy(), want[0][0]) and np.array_equal(d[1].cpu().numpy(), want[0][1])
    assert np.array_equal(d[2].cpu().numpy(), want[1][0], equal_nan=True)
    assert np.array_equal(d[3].cpu().numpy(), want[1][1], equal_nan=True)


@pytest.mark.parametrize("bs", [1, 4])
def test_int4_remap_bit_exact(bs):
    from oracle.compact import kv_compact_remap
    from test_oracle_compact_remap import random_case
    rng = np.random.default_rng(20 + bs)
    L, table, k, v, paths, acc = random_case(rng, 3, 24, bs, layers=1, d=64, aligned=True)
    kq, ks = quantize_int4(k[0])
    vq, vs = quantize_int4(v[0])
    d = [c(kq), c(vq), c(ks), c(vs)]
    td = c(table)
    kv = ev.KvCache(d[0], d[1], td, k_scale=d[2], v_scale=d[3])
    ev.ev_kv_compact_remap(kv, c(L), c(paths), c(acc), check=True)
    for got, x, y in ((d[0:2], kq, vq), (d[2:4], ks, vs)):
        ko, vo, to, *_ = kv_compact_remap(x[None], y[None], L, paths, acc, table, bs, 24, layered=True)
        assert np.array_equal(got[0].cpu().numpy(), ko[0]) and np.array_equal(got[1].cpu().numpy(), vo[0])
    assert np.array_equal(td.cpu().numpy(), to)
