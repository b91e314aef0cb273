"""GPU parity of zero-copy pruning (ev_kv_compact_remap) against the oracle: the block
table, both physical caches, new lengths, freed blocks and copy counts bit-exact."""
import numpy as np
import pytest
import torch

import tree_attention_verification_ev_amd as ev
from oracle.compact import kv_compact_remap
from test_oracle_compact_remap import random_case

pytestmark = pytest.mark.gpu


def run_case(L, table, k, v, paths, acc, bs, T, dtype):
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kd = torch.from_numpy(k).cuda().to(dt)
    vd = torch.from_numpy(v).cuda().to(dt)
    k0, v0 = kd.float().cpu().numpy(), vd.float().cpu().numpy()   # what both sides start from
    td = torch.from_numpy(np.ascontiguousarray(table)).cuda()
    kv = ev.KvCache(kd, vd, td, layered=True)
    c = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    new_len, freed, fcount, copied = ev.ev_kv_compact_remap(kv, c(L), c(paths), c(acc), check=True)
    ko, vo, to, nlo, fo, co = kv_compact_remap(k0, v0, L, paths, acc, table, bs, T, layered=True)
    assert np.array_equal(td.cpu().numpy(), to)
    assert np.array_equal(new_len.cpu().numpy(), nlo)
    assert np.array_equal(copied.cpu().numpy(), co)
    fc = fcount.cpu().numpy()
    fr = freed.cpu().numpy()
    for b in range(len(L)):
        assert fr[b, :fc[b]].tolist() == fo[b]
    assert np.array_equal(kd.float().cpu().numpy(), ko)
    assert np.array_equal(vd.float().cpu().numpy(), vo)
    return co


@pytest.mark.parametrize("bs", [1, 2, 4, 16])
@pytest.mark.parametrize("aligned", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_remap_matches_oracle(bs, aligned, dtype):
    rng = np.random.default_rng(100 * bs + 10 * aligned + (dtype == "f32"))
    for T in (24, 64):
        L, table, k, v, paths, acc = random_case(rng, 4, T, bs, layers=2, d=64, aligned=aligned)
        copied = run_case(L, table, k, v, paths, acc, bs, T, dtype)
        if bs == 1:
            assert copied.sum() == 0


@pytest.mark.parametrize("bs", [1, 16])
def test_remap_batched_paged_shape(bs):
    """B = 16, T = 64, L ~ U[512, 8192], 8 KV heads of d = 128, bf16, shuffled blocks."""
    rng = np.random.default_rng(7 + bs)
    B, T, Hkv, d = 16, 64, 8, 128
    L = rng.integers(512, 8193, size=B).astype(np.int32)
    max_blocks = (int(L.max()) + T + bs - 1) // bs
    n_blocks = int(sum((int(x) + T + bs - 1) // bs for x in L)) + 3
    perm = rng.permutation(n_blocks).astype(np.int32)
    table = np.full((B, max_blocks), -1, np.int32)
    at = 0
    for b in range(B):
        n = (int(L[b]) + T + bs - 1) // bs
        table[b, :n] = perm[at:at + n]
        at += n
    k = rng.standard_normal((1, n_blocks, Hkv, bs, d)).astype(np.float32)
    v = rng.standard_normal((1, n_blocks, Hkv, bs, d)).astype(np.float32)
    paths = np.full((B, T), -1, np.int32)
    acc = np.zeros(B, np.int32)
    for b in range(B):
        kb = int(rng.integers(0, 7))
        nodes = sorted(rng.choice(np.arange(1, T), size=kb, replace=False).tolist())
        paths[b, :kb + 1] = [0] + nodes
        acc[b] = kb
    run_case(L, table, k, v, paths, acc, bs, T, "bf16")


def test_remap_reports_bad_path_and_leaves_the_sequence():
    rng = np.random.default_rng(3)
    L, table, k, v, paths, acc = random_case(rng, 1, 24, 4, layers=1, d=64)
    paths[0, :3] = [0, 5, 3]
    acc[0] = 2
    td = torch.from_numpy(table).cuda()
    kd, vd = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    c = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    with pytest.raises(ev.EvError) as e:
        ev.ev_kv_compact_remap(ev.KvCache(kd, vd, td, layered=True), c(L), c(paths), c(acc),
                               check=True)
    assert e.value.code == 104
    assert np.array_equal(td.cpu().numpy(), table)
    assert np.array_equal(kd.cpu().numpy(), k)


def test_remap_with_nothing_accepted():
    """k = 0 everywhere: no slot moves; the tree's blocks past the root's are freed."""
    rng = np.random.default_rng(9)
    L, table, k, v, paths, acc = random_case(rng, 4, 24, 4, layers=1, d=64)
    paths[:, 1:] = -1
    acc[:] = 0
    copied = run_case(L, table, k, v, paths, acc, 4, 24, "bf16")
    assert copied.sum() == 0
