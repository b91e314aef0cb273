"""The seeded input generators: determinism, shapes, value ranges, poisoning."""
import numpy as np

from synth import CONFIGS, generate, round_to_bf16, scaled


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, 1.0 + 2 ** -9, -2.5, 0.0], np.float32)
    r = round_to_bf16(x)
    assert r.tolist() == [1.0, 1.0, 1.0 + 2 ** -7, 1.0, -2.5, 0.0]
    y = np.random.default_rng(0).standard_normal(10000).astype(np.float32)
    ry = round_to_bf16(y)
    assert (ry.view(np.uint32) & 0xFFFF == 0).all()
    assert np.abs(ry - y).max() <= np.abs(y).max() * 2 ** -8


def test_same_seed_same_bytes_and_streams_are_independent():
    cfg = scaled(CONFIGS[3], B=3, L=(40, 90), V=300)
    a = generate(cfg)
    b = generate(cfg)
    for name in ("parent", "tokens", "prefix_len", "q", "k", "v", "block_table", "logits", "uniforms"):
        assert np.array_equal(getattr(a, name), getattr(b, name), equal_nan=True), name
    raw = generate(cfg, tokens="raw")
    assert np.array_equal(raw.uniforms, a.uniforms) and np.array_equal(raw.tokens, a.tokens)
    assert np.array_equal(raw.q, a.q)
    differs = ~np.all(raw.logits == a.logits, axis=2)
    assert np.array_equal(differs, a.planted)


def test_shapes_poison_and_distributions():
    for cfg in CONFIGS:
        small = scaled(cfg, B=min(cfg.B, 3), V=500,
                       L=(64, 200) if isinstance(cfg.L, tuple) else min(cfg.L, 300))
        inp = generate(small)
        B, T = small.B, small.T
        assert inp.q.shape == (B, T, small.Hq, small.d)
        assert inp.logits.shape == (B, T, small.V) and inp.logits.dtype == np.float32
        assert inp.uniforms.shape == (B, T) and ((inp.uniforms >= 0) & (inp.uniforms < 1)).all()
        if small.dtype == "bf16":
            assert (inp.q.view(np.uint32) & 0xFFFF == 0).all()
        for b in range(B):
            L = int(inp.prefix_len[b])
            if inp.layout == "contiguous":
                used = inp.k[b, :, :L + T]
                assert np.isfinite(used).all() and np.isnan(inp.k[b, :, L + T:]).all()
            else:
                bs = small.block_size
                nb = (L + T + bs - 1) // bs
                ids = inp.block_table[b, :nb]
                assert (ids >= 0).all() and (inp.block_table[b, nb:] == -1).all()
                tail = inp.k[ids[-1], :, (L + T) - (nb - 1) * bs:]
                assert np.isnan(tail).all()
                assert np.isfinite(inp.k[ids[:-1]]).all()
        if inp.layout == "paged":
            used = set(inp.block_table[inp.block_table >= 0].tolist())
            assert len(used) == (inp.block_table >= 0).sum()       # no block shared
            spare = [i for i in range(inp.k.shape[0]) if i not in used]
            assert spare and np.isnan(inp.k[spare]).all()
        # siblings draft distinct tokens
        for b in range(B):
            for u in range(T):
                kids = np.nonzero(inp.parent[b] == u)[0]
                assert len(set(inp.tokens[b, kids].tolist())) == len(kids)
    big = generate(scaled(CONFIGS[2], L=16), with_kv=False, tokens="raw")
    assert abs(big.logits.std() - 2.0) < 0.01 and abs(big.logits.mean()) < 0.01


def test_planted_token_is_the_row_argmax():
    inp = generate(scaled(CONFIGS[2], L=16, V=20000), with_kv=False)
    for u in np.nonzero(inp.planted[0])[0]:
        kids = np.nonzero(inp.parent[0] == u)[0]
        assert int(np.argmax(inp.logits[0, u])) == int(inp.tokens[0, kids.min()])
    assert 0.6 < inp.planted[0].sum() / max(1, len(set(inp.parent[0, 1:].tolist()))) <= 1.0
