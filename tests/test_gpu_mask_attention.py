"""ev_tree_mask_attention: mask build and tree attention in one call.

The direct-to-LDS kernel (bf16, head_dim 128) builds the ancestor masks from parent[]
itself; other caches run the mask kernel first.  Either way the masks and depths must be
the oracle's bit for bit, and the attention outputs bit-identical to ev_tree_mask_build
followed by ev_tree_attention on the same inputs (the attention arithmetic is the same, so
the oracle parity of that path carries over); the full 70B-shaped layer and a paged batch
are also checked against the oracle directly.
"""
import numpy as np
import pytest
import torch

import oracle
import tree_attention_verification_ev_amd as ev
from synth import CONFIGS, generate, scaled
from synth.device import to_device

from test_gpu_parity import O_TOL_BF16, LSE_TOL_BF16, max_prefix, oracle_attention, scale_of

pytestmark = pytest.mark.gpu

C1, C2, C3, C4, C5 = CONFIGS

CASES = [
    ("C1_fp32", C1),                                       # float32: mask kernel first
    ("C2_L300", scaled(C2, L=300, V=64)),                  # MHA: two-wavefront key-split groups
    ("C3_L300", scaled(C3, L=300, V=64)),
    ("C3_L0", scaled(C3, L=0, V=64)),                      # every key a tree slot
    ("C3_L600_tree_over_two_splits", scaled(C3, L=600, V=64)),
    ("C3_L64_aligned", scaled(C3, L=64, V=64)),
    ("C4_small_paged", scaled(C4, B=4, L=(40, 400), V=64)),
    ("C5_small_paged", scaled(C5, B=2, L=700, V=64)),
    ("C3_varlen", scaled(C3, B=3, L=(10, 900), V=64)),
    ("chain64_mha", scaled(C2, T=64, tree="chain", L=130, V=64, Hq=4, Hkv=4)),
    ("star64", scaled(C3, tree="star", L=77, V=64)),
    ("root_only", scaled(C3, T=1, tree="grow", L=200, V=64)),
    ("gqa8_T8", scaled(C3, T=8, L=257, V=64)),
    ("gqa8_T40", scaled(C3, T=40, L=190, V=64)),
    ("paged_gqa4_T26", scaled(C4, B=2, T=26, Hq=32, Hkv=8, L=(100, 700), V=64)),
    ("bf16_d64", scaled(C3, d=64, L=333, V=64)),           # register-staged kernel: mask kernel first
    ("C3_full", C3),
    ("C4_full", C4),
]


def two_calls(inp, dev):
    kv = ev.KvCache(dev.k, dev.v, dev.block_table)
    anc, depth = ev.ev_tree_mask_build(dev.parent, check=True)
    out, lse = ev.ev_tree_attention(dev.q, kv, dev.prefix_len, anc, scale_of(inp.cfg), check=True,
                                    max_prefix_len=max_prefix(inp))
    return out, lse, anc, depth


def one_call(inp, dev):
    kv = ev.KvCache(dev.k, dev.v, dev.block_table)
    depth = torch.full(tuple(dev.parent.shape), -7, dtype=torch.int32, device="cuda")
    out, lse, anc, depth = ev.ev_tree_mask_attention(dev.q, kv, dev.prefix_len, dev.parent,
                                                     scale_of(inp.cfg), depth=depth, check=True,
                                                     max_prefix_len=max_prefix(inp))
    return out, lse, anc, depth


@pytest.mark.parametrize("name,cfg", CASES, ids=[n for n, _ in CASES])
def test_one_call_equals_two_calls(name, cfg):
    inp = generate(cfg, with_logits=False)
    dev = to_device(inp)
    o2, l2, a2, d2 = two_calls(inp, dev)
    o1, l1, a1, d1 = one_call(inp, dev)
    torch.cuda.synchronize()
    ao, do = oracle.tree_mask_batch(inp.parent)
    assert np.array_equal(a1.cpu().numpy().view(np.uint64), ao)
    assert np.array_equal(d1.cpu().numpy(), do)
    assert torch.equal(o1.view(torch.int16) if o1.dtype == torch.bfloat16 else o1,
                       o2.view(torch.int16) if o2.dtype == torch.bfloat16 else o2)
    assert torch.equal(l1, l2)


@pytest.mark.parametrize("name,cfg,heads", [("C3_full", C3, None),
                                            ("C4_full", C4, None),
                                            ("C5_full_sampled_heads", C5, [0, 9, 18, 27, 36, 45, 54, 63])],
                         ids=["C3_full", "C4_full", "C5_full_sampled_heads"])
def test_one_call_matches_oracle(name, cfg, heads):
    inp = generate(cfg, with_logits=False)
    dev = to_device(inp)
    out, lse, _, _ = one_call(inp, dev)
    torch.cuda.synchronize()
    O, LSE = out.float().cpu().numpy(), lse.cpu().numpy()
    Oo, Lo = oracle_attention(inp, heads=heads)
    sel = np.isfinite(Lo)
    assert sel.any() and np.isfinite(O).all()
    mask = np.broadcast_to(sel[..., None], O.shape)
    assert np.abs(O - Oo)[mask].max() <= O_TOL_BF16
    assert np.abs(LSE - Lo)[sel].max() <= LSE_TOL_BF16


@pytest.mark.parametrize("name,cfg", [("bf16_d128", scaled(C3, L=300, V=64)), ("f32", C1)],
                         ids=["bf16_d128", "f32"])
def test_one_call_reports_bad_parent(name, cfg):
    inp = generate(cfg, with_logits=False)
    inp.parent[0, 3] = 5                                   # not an earlier node
    dev = to_device(inp)
    with pytest.raises(ev.EvError) as e:
        one_call(inp, dev)
    assert e.value.code == 101
