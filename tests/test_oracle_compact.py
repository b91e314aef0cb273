"""Pins of the oracle's accepted-path KV compaction (Tech Radar sec. 2 sequence diagram:
keep the accepted branch's KV, drop the wrong branches)."""
import numpy as np
import pytest

from oracle import kv_compact


def _cache(rng, B, H, cap, d):
    return rng.standard_normal((B, H, cap, d)).astype(np.float32)


def _gather_then_scatter(c, b, L, path, k):
    """Expected contents by a parallel-style reading: read every source first, then write."""
    out = c.copy()
    src = [c[b, :, L + path[m]].copy() for m in range(1, k + 1)]
    for m in range(1, k + 1):
        out[b, :, L + m] = src[m - 1]
    return out


@pytest.mark.parametrize("seed", range(10))
def test_compaction_moves_path_and_leaves_the_rest(seed):
    rng = np.random.default_rng(seed)
    B, H, d, T = 3, 2, 8, 20
    L = rng.integers(0, 30, size=B).astype(np.int32)
    cap = int(L.max()) + T + 5
    k, v = _cache(rng, B, H, cap, d), _cache(rng, B, H, cap, d)
    paths = np.full((B, T), -1, np.int32)
    acc = np.zeros(B, np.int32)
    for b in range(B):
        n = int(rng.integers(0, 8))
        nodes = np.sort(rng.choice(np.arange(1, T), size=n, replace=False))
        paths[b, :n + 1] = [0, *nodes]
        acc[b] = n
    k2, v2, new_len = kv_compact(k, v, L, paths, acc, "contiguous")
    assert new_len.tolist() == (L + acc + 1).tolist()
    for b in range(B):
        exp_k = _gather_then_scatter(k, b, int(L[b]), paths[b], int(acc[b]))
        exp_v = _gather_then_scatter(v, b, int(L[b]), paths[b], int(acc[b]))
        assert np.array_equal(k2[b], exp_k[b]) and np.array_equal(v2[b], exp_v[b])
        for m in range(1, int(acc[b]) + 1):      # slot L+m holds the old slot L+a_m, bitwise
            assert np.array_equal(k2[b, :, L[b] + m], k[b, :, L[b] + paths[b, m]])
        # slots outside [L+1, L+k] are untouched
        keep = [s for s in range(cap) if not (L[b] + 1 <= s <= L[b] + acc[b])]
        assert np.array_equal(k2[b][:, keep], k[b][:, keep])


def test_maximal_overlap_and_noops():
    rng = np.random.default_rng(1)
    H, d, T, L = 1, 4, 10, 5
    k = _cache(rng, 1, H, L + T, d)
    # a_m = m + 1 on m = 1..8: every destination except the first is an earlier source
    path = np.array([[0, 2, 3, 4, 5, 6, 7, 8, 9, -1]], np.int32)
    k2, _, _ = kv_compact(k, k, [L], path, [8], "contiguous")
    for m in range(1, 9):
        assert np.array_equal(k2[0, :, L + m], k[0, :, L + m + 1])
    chain = np.array([[0, 1, 2, 3, -1, -1, -1, -1, -1, -1]], np.int32)
    k3, _, n = kv_compact(k, k, [L], chain, [3], "contiguous")
    assert np.array_equal(k3, k) and n[0] == L + 4
    k4, _, n = kv_compact(k, k, [L], np.full((1, T), -1, np.int32), [0], "contiguous")
    assert np.array_equal(k4, k) and n[0] == L + 1


def test_paged_and_layered_agree_with_contiguous():
    rng = np.random.default_rng(2)
    B, H, d, T, bs, nl = 2, 2, 4, 12, 4, 3
    L = np.array([7, 13], np.int32)
    n = L + T
    nb = (n + bs - 1) // bs
    n_blocks = int(nb.sum()) + 3
    perm = rng.permutation(n_blocks)
    table = np.full((B, nb.max()), -1, np.int32)
    table[0, :nb[0]] = perm[:nb[0]]
    table[1, :nb[1]] = perm[nb[0]:nb[0] + nb[1]]
    pool = rng.standard_normal((nl, n_blocks, H, bs, d)).astype(np.float32)
    cont = np.zeros((nl, B, H, int(n.max()), d), np.float32)
    for layer in range(nl):
        for b in range(B):
            for s in range(n[b]):
                cont[layer, b, :, s] = pool[layer, table[b, s // bs], :, s % bs]
    path = np.array([[0, 2, 5, 11] + [-1] * 8, [0, 1, 3, 4] + [-1] * 8], np.int32)
    acc = np.array([3, 3], np.int32)
    pk, _, nlen = kv_compact(pool, pool, L, path, acc, "paged", table, bs, layered=True)
    ck, _, nlen2 = kv_compact(cont, cont, L, path, acc, "contiguous", layered=True)
    assert np.array_equal(nlen, nlen2)
    for layer in range(nl):
        for b in range(B):
            for s in range(n[b]):
                assert np.array_equal(pk[layer, table[b, s // bs], :, s % bs], ck[layer, b, :, s])
