"""Pins of the zero-copy compaction oracle (oracle.compact.kv_compact_remap, remap_plan).

The logical content after a remap must equal the copy-based compaction (kv_compact,
pinned on its own), for every block size, shuffled block tables and layered caches;
with pages of one token nothing is copied; the freed list is exactly the tree's old
physical blocks that the new table no longer references; plans match hand-derived
cases, including remaps that fall back to copies."""
import json
import os

import numpy as np
import pytest

from oracle.compact import kv_compact, kv_compact_remap, remap_plan

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def random_case(rng, B, T, bs, layers, d=8, Hkv=2, aligned=False):
    L = rng.integers(0, 40, size=B).astype(np.int32)
    if aligned:                                  # L + 1 on a block boundary
        L = (L // bs) * bs + bs - 1
    max_blocks = (int(L.max()) + T + bs - 1) // bs + 1
    n_blocks = B * max_blocks + 5
    perm = rng.permutation(n_blocks).astype(np.int32)
    table = perm[:B * max_blocks].reshape(B, max_blocks)
    shape = (layers, n_blocks, Hkv, bs, d)
    k = rng.standard_normal(shape).astype(np.float32)
    v = rng.standard_normal(shape).astype(np.float32)
    paths = np.full((B, T), -1, np.int32)
    acc = np.zeros(B, np.int32)
    for b in range(B):
        kb = int(rng.integers(0, min(T - 1, 8) + 1))
        if aligned and rng.random() < 0.7:       # runs with a block-multiple offset
            D = bs * int(rng.integers(0, max(1, (T - 1 - kb) // bs) + 1))
            nodes = [m + D for m in range(1, kb + 1) if m + D < T]
            kb = len(nodes)
        else:
            nodes = sorted(rng.choice(np.arange(1, T), size=kb, replace=False).tolist())
        paths[b, :kb + 1] = [0] + nodes
        acc[b] = kb
    return L, table, k, v, paths, acc


def gather(cache, table, b, n, bs):
    """Logical slots 0..n-1 of sequence b, all layers and heads: [layers][n][Hkv][d]."""
    return np.stack([cache[:, table[b][s // bs], :, s % bs] for s in range(n)], axis=1)


@pytest.mark.parametrize("bs", [1, 2, 4, 16])
@pytest.mark.parametrize("aligned", [False, True])
def test_logical_content_equals_copy_compaction(bs, aligned):
    rng = np.random.default_rng(bs * 7 + aligned)
    for _ in range(15):
        B, T = 3, 24
        L, table, k, v, paths, acc = random_case(rng, B, T, bs, layers=2, aligned=aligned)
        k2, v2, table2, new_len, freed, copied = kv_compact_remap(k, v, L, paths, acc, table, bs, T,
                                                                  layered=True)
        k1, v1, nl1 = kv_compact(k, v, L, paths, acc, "paged", table, bs, layered=True)
        assert np.array_equal(new_len, nl1)
        for b in range(B):
            n = int(new_len[b])
            assert np.array_equal(gather(k2, table2, b, n, bs), gather(k1, table, b, n, bs))
            assert np.array_equal(gather(v2, table2, b, n, bs), gather(v1, table, b, n, bs))


def test_pages_of_one_token_copy_nothing():
    rng = np.random.default_rng(1)
    for _ in range(20):
        L, table, k, v, paths, acc = random_case(rng, 4, 32, 1, layers=1)
        *_, copied = kv_compact_remap(k, v, L, paths, acc, table, 1, 32, layered=True)
        assert int(copied.sum()) == 0


@pytest.mark.parametrize("bs", [1, 4, 16])
def test_freed_blocks_are_the_tree_blocks_no_longer_referenced(bs):
    rng = np.random.default_rng(40 + bs)
    for _ in range(15):
        T = 24
        L, table, k, v, paths, acc = random_case(rng, 3, T, bs, layers=1, aligned=True)
        _, _, table2, new_len, freed, _ = kv_compact_remap(k, v, L, paths, acc, table, bs, T,
                                                           layered=True)
        for b in range(3):
            lo, n_old, n_new = int(L[b]) // bs, -(-(int(L[b]) + T) // bs), -(-int(new_len[b]) // bs)
            old = set(int(x) for x in table[b][lo:n_old])
            live = set(int(x) for x in table2[b][lo:n_new])
            assert len(freed[b]) == len(set(freed[b]))
            assert set(freed[b]) == old - live
            assert live <= old                   # remaps only reuse the tree's own blocks
            assert (table2[b][n_new:n_old] == -1).all()
            assert np.array_equal(table2[b][:lo], table[b][:lo])


def test_plans_match_hand_derived_cases():
    g = json.load(open(os.path.join(GOLDEN, "compact_remap_plans.json")))
    for c in g["cases"]:
        k = len(c["path"]) - 1
        plan = remap_plan(c["L"], c["path"], k, c["T"], c["bs"])
        want = {int(X): (("remap", p[0]) if isinstance(p, list) else p) for X, p in c["plan"].items()}
        assert plan == want, c["name"]
