"""The C-ABI library loads, exports every entry point its header declares, and rejects
host-visible argument errors before launching anything (no GPU needed)."""
import ctypes
import os
import re

import pytest

import tree_attention_verification_ev_amd as ev

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ev.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ev_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ev.LIB_PATH):
        pytest.fail("libev.so is not built (run __graft_entry__.build())")
    return ev.lib()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(ev.EXPORTED)
    for name in names:
        assert hasattr(lib, name), name


def test_exports_calibration_kernels(lib):
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "ev_peaks.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(ev_[a-z0-9_]+)\s*\(", text)))
    assert set(names) == set(ev.EXPORTED_PEAKS)
    for name in names:
        assert hasattr(lib, name), name
    P = 0x1000
    assert lib.ev_peak_mfma_bf16(0, 10, P, None) == 2
    assert lib.ev_peak_mfma_bf16(4, 0, P, None) == 2
    assert lib.ev_peak_mfma_bf16(4, 10, None, None) == 1
    assert lib.ev_peak_copy(None, P, 16, None) == 1
    assert lib.ev_peak_copy(P + 8, P, 16, None) == 5
    assert lib.ev_peak_copy(P, P, 24, None) == 5
    assert lib.ev_peak_copy(P, P, 0, None) == 0
    assert lib.ev_peak_read(None, 16, P, 4, None) == 1
    assert lib.ev_peak_read(P, 20, P, 4, None) == 5
    assert lib.ev_peak_read(P, 16, P, 0, None) == 2


def test_status_strings(lib):
    for code in ev.STATUS_NAMES:
        assert ev.ev_status_string(code) not in ("", "unknown status")
    assert ev.ev_status_string(12345) == "unknown status"


def _kv(**kw):
    d = ev.EvKvDesc()
    d.dtype, d.n_kv_heads, d.head_dim, d.paged = ev.EV_BF16, 8, 128, 0
    d.k = d.v = 0x1000
    d.n_layers, d.layer_stride, d.cap = 1, 0, 4176
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_workspace_queries(lib):
    d = _kv()
    ws = lib.ev_tree_attention_workspace(ctypes.byref(d), 1, 64, 64, 4096)
    assert ws % 256 == 0
    assert lib.ev_tree_attention_workspace(ctypes.byref(d), 1, 65, 64, 4096) == 0
    assert lib.ev_tree_attention_workspace(ctypes.byref(_kv(head_dim=96)), 1, 64, 64, 4096) == 0
    assert lib.ev_tree_attention_workspace(ctypes.byref(d), 1, 64, 64, -1) == 0
    # the split plan follows the longest prefix, not the capacity: a cache eight times as
    # large as the prefix needs the same workspace
    big = _kv(cap=8 * 4176)
    assert lib.ev_tree_attention_workspace(ctypes.byref(big), 1, 64, 64, 4096) == ws
    # a bound beyond the cache is clamped to what the cache holds (4176 slots)
    assert (lib.ev_tree_attention_workspace(ctypes.byref(d), 1, 64, 64, 10**12)
            == lib.ev_tree_attention_workspace(ctypes.byref(d), 1, 64, 64, 4176 - 64))
    counters = 2 * 65536 * 4                       # fixed row and sequence counter areas
    stats = 64 * 126 * 16                          # (max, sum) per 1024-logit chunk per row
    assert lib.ev_accept_workspace(1, 64, 128256) == counters + stats + 64 * 8
    assert lib.ev_accept_workspace(1, 64, 128256) % 256 == 0
    assert lib.ev_accept_workspace(0, 64, 10) == 0
    # sampled drafts: counters, (max, sum) of both rows and the residual mass per chunk,
    # the row states (48 bytes), the node words, the per-round list counters (65, padded to
    # 256 bytes) and two lists of undecided rows (64 bytes per row each)
    rows, chunks = 64, 126
    assert lib.ev_accept_sampled_workspace(1, 64, 128256) == (
        counters + 2 * rows * chunks * 16 + rows * chunks * 8 + rows * 48 + rows * 8 + 512
        + 2 * rows * 64)


def test_host_errors_return_before_launch(lib):
    P = 0x1000
    d = _kv()
    assert lib.ev_tree_mask_build(P, 1, 0, P, P, None, None) == 2
    assert lib.ev_tree_mask_build(P, 1, 65, P, P, None, None) == 2
    assert lib.ev_tree_mask_build(None, 1, 8, P, P, None, None) == 1
    assert lib.ev_tree_mask_build(None, 0, 8, None, None, None, None) == 0   # empty batch
    att = lambda desc, T=64, Hq=64, scale=0.088, ws=None, nbytes=0, q=P, mpl=4096: \
        lib.ev_tree_attention(q, ctypes.byref(desc), P, P, 1, T, Hq, mpl, scale, P, P, ws, nbytes,
                              None, None)
    assert att(d, Hq=60) == 2                       # Hq not a multiple of Hkv
    assert att(d, mpl=-5) == 2                      # negative prefix bound
    assert att(_kv(head_dim=96)) == 2
    assert att(_kv(dtype=7)) == 3
    assert att(d, scale=0.0) == 5
    assert att(d, scale=float("nan")) == 5
    assert att(d, q=None) == 1
    assert att(d, q=P + 8) == 5                     # rows read in 16-byte pieces
    assert att(_kv(k=P + 2)) == 5
    assert att(d) == 4                              # split workspace missing
    assert att(_kv(paged=1, block_table=None)) == 1
    assert att(_kv(paged=1, block_table=P, block_size=12, max_blocks_per_seq=4, n_blocks=9)) == 2
    assert lib.ev_accept_greedy(P, P, P, 1, 8, 0, P, P, P, P, 10, None, None) == 2
    assert lib.ev_accept_greedy(P, P, P, 1, 8, 100, P, P, P, P, 10, None, None) == 4
    assert lib.ev_accept_rejection(P, P, P, 1, 8, 100, 0.0, P, P, P, P, P, 10**6, None, None) == 5
    assert lib.ev_accept_rejection(P, P, P, 1, 8, 100, float("inf"), P, P, P, P, P, 10**6, None, None) == 5
    assert lib.ev_accept_rejection(P, P, P, 1, 8, 100, 0.7, None, P, P, P, P, 10**6, None, None) == 1
    samp = lambda tau=0.7, dtau=0.9, mc=3, ws=P, nbytes=10**8, logits=P, draft=P, T=8, V=100: \
        lib.ev_accept_sampled(logits, draft, P, P, 1, T, V, tau, dtau, P, mc, P, P, P, ws, nbytes,
                              None, None)
    assert samp(tau=0.0) == 5
    assert samp(dtau=float("nan")) == 5
    assert samp(mc=-1) == 2
    assert samp(mc=9) == 2                          # more than T
    assert samp(T=65) == 2
    assert samp(V=0) == 2
    assert samp(draft=None) == 1
    assert samp(nbytes=100) == 4
    assert lib.ev_accept_sampled_workspace(1, 64, 128256) >= 2 * 65536 * 4 + 64 * 126 * 40
    exp = lambda B=1, W=8, V=1000, depth=0, tau=1.0, k=8, ws=P, nbytes=10**8, logits=P: \
        lib.ev_draft_tree_expand(logits, B, W, V, depth, tau, k, P, P, P, ws, nbytes, None, None)
    assert exp(tau=0.0) == 5
    assert exp(tau=float("inf")) == 5
    assert exp(W=0) == 2 and exp(W=9) == 2
    assert exp(k=0) == 2 and exp(k=9) == 2
    assert exp(depth=-1) == 2 and exp(depth=16) == 2
    assert exp(V=0) == 2
    assert exp(logits=None) == 1
    assert exp(nbytes=100) == 4
    assert exp(B=0, logits=None) == 0               # empty batch
    fin = lambda B=1, W=8, V=1000, n=64, nbytes=10**8: lib.ev_draft_tree_finalize(
        P, B, W, V, n, P, P, P, P, nbytes, None)
    assert fin(n=0) == 2 and fin(n=65) == 2
    assert fin(W=9) == 2
    assert fin(nbytes=100) == 4
    assert lib.ev_draft_tree_workspace(1, 9, 100) == 0
    assert lib.ev_draft_tree_workspace(16, 8, 128256) % 256 == 0
    rm = lambda desc, ws=P, nbytes=10**6, pl=P: lib.ev_kv_compact_remap(
        ctypes.byref(desc), pl, P, P, 1, 8, P, P, P, P, ws, nbytes, None, None)
    paged = dict(paged=1, block_table=P, block_size=16, max_blocks_per_seq=8, n_blocks=64)
    assert rm(_kv()) == 5                            # contiguous: nothing to remap
    assert rm(_kv(**paged), pl=None) == 1
    assert rm(_kv(**paged), nbytes=8) == 4
    assert rm(_kv(**dict(paged, block_size=12))) == 2
    assert lib.ev_kv_compact_remap_workspace(0) == 0
    assert lib.ev_kv_compact(ctypes.byref(_kv(n_layers=0)), P, P, P, 1, 8, P, None, None) == 2
    assert lib.ev_kv_compact(ctypes.byref(_kv(n_layers=2, layer_stride=0)), P, P, P, 1, 8, P, None, None) == 2
    assert lib.ev_kv_compact(ctypes.byref(d), None, P, P, 1, 8, P, None, None) == 1


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        ev.ev_tree_mask_build(torch.zeros((1, 4), dtype=torch.int32))
