"""Host model of the draft-tree finalize selection (no GPU): the place of a candidate in
the whole order "larger value first, then lower id" is its rank within its own depth plus,
for every other depth, the number of that depth's candidates before it (a binary search in
the depth's rank-ordered list).  Checked against a full sort on random candidate sets with
many ties, across depth counts and fill levels."""
import random


def before(v, i, v2, i2):
    return v > v2 or (v == v2 and i < i2)


def places_by_search(depths):
    """depths: list of lists of values (slot order).  Returns {id: place} for every
    candidate, ids = depth * 64 + slot, computed the way the kernel does."""
    lists = []
    for e, vals in enumerate(depths):
        ids = [e * 64 + s for s in range(len(vals))]
        # rank within the depth: larger value first, then lower slot
        order = sorted(ids, key=lambda i: (-vals[i - e * 64], i))
        lists.append(order)
    val = {e * 64 + s: v for e, vals in enumerate(depths) for s, v in enumerate(vals)}
    out = {}
    for e, order in enumerate(lists):
        for r, cid in enumerate(order):
            place = r
            for e2, order2 in enumerate(lists):
                if e2 == e:
                    continue
                lo, hi = 0, len(order2)
                while lo < hi:
                    mid = (lo + hi) // 2
                    if before(val[order2[mid]], order2[mid], val[cid], cid):
                        lo = mid + 1
                    else:
                        hi = mid
                place += lo
            out[cid] = place
    return out


def places_by_sort(depths):
    allc = [(v, e * 64 + s) for e, vals in enumerate(depths) for s, v in enumerate(vals)]
    allc.sort(key=lambda t: (-t[0], t[1]))
    return {cid: p for p, (_, cid) in enumerate(allc)}


def test_selection_matches_full_sort():
    rng = random.Random(20261203)
    for trial in range(300):
        n_exp = rng.randint(1, 16)
        levels = rng.choice([3, 10, 1000])          # few distinct values: many ties
        depths = [[rng.randint(0, levels) / levels for _ in range(rng.randint(0, 64))]
                  for _ in range(n_exp)]
        assert places_by_search(depths) == places_by_sort(depths), trial
