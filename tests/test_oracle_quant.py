"""Pins of the INT4 cache oracle (oracle/quant.py): nibble order and sign by hand,
bfloat16 rounding against torch's own conversion, exact round trips where the product is
a bfloat16, the quantiser's error bound, and attention over an INT4 cache equal to
attention over the equivalent float cache."""
import math

import numpy as np
import torch

import oracle
from oracle.quant import bf16_nearest, dequant_int4, unpack_int4
from synth import quantize_int4


def test_unpack_by_hand():
    packed = np.array([[0x7F, 0x80, 0x01, 0xF8]], np.uint8)
    assert unpack_int4(packed).tolist() == [[-1, 7, 0, -8, 1, 0, -8, -1]]


def test_bf16_nearest_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0]   # ties either way
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(bf16_nearest(x), ref)


def test_power_of_two_scales_round_trip_exactly():
    rng = np.random.default_rng(1)
    q = rng.integers(-8, 8, size=(5, 7, 64)).astype(np.int16)
    s = (2.0 ** rng.integers(-6, 3, size=(5, 7))).astype(np.float32)
    u = (q & 0xF).astype(np.uint8)
    packed = u[..., 0::2] | (u[..., 1::2] << 4)
    assert np.array_equal(dequant_int4(packed, s), s[..., None].astype(np.float64) * q)


def test_quantiser_error_bound():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((50, 128)).astype(np.float32)
    packed, s = quantize_int4(x)
    xd = dequant_int4(packed, s)
    # rounding to the 4-bit grid (half a step) plus the bfloat16 rounding of the product
    bound = s[:, None] / 2 + np.abs(xd) * 2.0 ** -8 + 1e-12
    assert (np.abs(xd - x) <= bound).all()
    assert (np.abs(unpack_int4(packed)) <= 8).all()


def test_attention_over_int4_equals_attention_over_its_values():
    """An INT4 cache with power-of-two scales holds exactly scale * q: attention over it is
    attention over that float cache."""
    rng = np.random.default_rng(3)
    B, Hkv, Hq, T, L, d = 2, 2, 4, 5, 9, 64
    cap = L + T
    q = rng.standard_normal((B, T, Hq, d))
    qi = rng.integers(-8, 8, size=(2, B, Hkv, cap, d)).astype(np.int16)
    s = (2.0 ** rng.integers(-3, 1, size=(2, B, Hkv, cap))).astype(np.float32)
    u = (qi & 0xF).astype(np.uint8)
    packed = u[..., 0::2] | (u[..., 1::2] << 4)
    kf = s[0][..., None].astype(np.float64) * qi[0]
    vf = s[1][..., None].astype(np.float64) * qi[1]
    parent = np.array([-1, 0, 0, 1, 2])
    anc, _ = oracle.tree_mask_batch(np.stack([parent, parent]))
    L_arr = np.array([L, L - 3], np.int32)
    o1, l1 = oracle.tree_attention_batch(q, kf, vf, L_arr, anc, "contiguous", None, 16, 1 / math.sqrt(d))
    o2, l2 = oracle.tree_attention_batch(q, dequant_int4(packed[0], s[0]), dequant_int4(packed[1], s[1]),
                                         L_arr, anc, "contiguous", None, 16, 1 / math.sqrt(d))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
