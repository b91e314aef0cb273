"""The no-allocation attention entry point (fixed per-GPU scratch) against the ordinary
entry point with a caller workspace: two calls in a row, the second smaller, each
bit-identical to the ordinary call (same kernels and plan), and both within the
oracle's bars.  A call whose plan exceeds the scratch is refused before launching."""
import math

import numpy as np
import pytest
import torch

import oracle
import tree_attention_verification_ev_amd as ev
from synth import CONFIGS, generate, scaled
from synth.device import to_device

pytestmark = pytest.mark.gpu
C1, C2, C3, C4, C5 = CONFIGS


def both_calls(cfg):
    inp = generate(cfg, with_logits=False)
    dev = to_device(inp)
    kv = ev.KvCache(dev.k, dev.v, dev.block_table)
    anc, _ = ev.ev_tree_mask_build(dev.parent, check=True)
    mpl = int(inp.prefix_len.max())
    scale = float(np.float32(1.0 / math.sqrt(cfg.d)))
    need = ev.ev_tree_attention_workspace(kv, cfg.B, cfg.T, cfg.Hq, mpl)
    assert 0 < need <= ev.ev_tree_attention_noalloc_limit()    # the split path runs
    o1, l1 = ev.ev_tree_attention(dev.q, kv, dev.prefix_len, anc, scale, check=True,
                                  max_prefix_len=mpl)
    o2 = torch.full_like(o1, float("nan"))
    l2 = torch.full_like(l1, float("nan"))
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    ev.ev_tree_attention_noalloc(dev.q, kv, dev.prefix_len, anc, scale, o2, l2, st, check=True,
                                 max_prefix_len=mpl)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    Oo, Lo = oracle.tree_attention_batch(inp.q, inp.k, inp.v, inp.prefix_len,
                                         oracle.tree_mask_batch(inp.parent)[0], inp.layout,
                                         inp.block_table, cfg.block_size, scale,
                                         seqs=[0], heads=[0, cfg.Hq // 2, cfg.Hq - 1])
    sel = np.isfinite(Lo)
    O2 = o2.float().cpu().numpy()
    assert np.abs(O2 - Oo)[np.broadcast_to(sel[..., None], O2.shape)].max() <= 1e-2
    assert np.abs(l2.cpu().numpy() - Lo)[sel].max() <= 1e-3


def test_noalloc_matches_workspace_entry_two_calls():
    both_calls(C3)                                   # Llama-3-70B-shaped layer, 14 splits
    both_calls(scaled(C3, L=700, V=64))              # then a smaller call on the same scratch


def test_noalloc_refuses_plans_beyond_its_scratch():
    """One-token pages over a 32k-token prefix cap each split at 15 tiles (the block ids
    of a split must fit the kernel's LDS cache), so the batched layer's plan needs far
    more partial storage than the fixed scratch: refused on the host, nothing launched."""
    B, T, Hq, Hkv, d = 16, 64, 64, 8, 128
    bf = dict(dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((B, T, Hq, d), **bf)
    k = torch.zeros((64, Hkv, 1, d), **bf)
    table = torch.zeros((B, 32768 + T), dtype=torch.int32, device="cuda")
    kv = ev.KvCache(k, k, table)
    pl = torch.full((B,), 32768, dtype=torch.int32, device="cuda")
    anc = torch.ones((B, T), dtype=torch.int64, device="cuda")
    assert ev.ev_tree_attention_workspace(kv, B, T, Hq, 32768) > ev.ev_tree_attention_noalloc_limit()
    with pytest.raises(ev.EvError) as e:
        ev.ev_tree_attention_noalloc(q, kv, pl, anc, max_prefix_len=32768)
    assert e.value.code == 7
