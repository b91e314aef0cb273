"""The calibration kernels of include/ev_peaks.h do what their timings assume: the copy moves
every byte, the read touches every byte (its per-workgroup XORs fold to the XOR of the
data), and the matrix-core loop runs to completion with finite results."""
import numpy as np
import pytest
import torch

import tree_attention_verification_ev_amd as ev

pytestmark = pytest.mark.gpu


def test_peak_copy_moves_every_byte():
    g = torch.Generator().manual_seed(7)
    src = torch.randint(0, 256, ((3 << 20) + 48,), dtype=torch.uint8, generator=g).cuda()
    dst = torch.zeros_like(src)
    ev.ev_peak_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


def test_peak_read_folds_every_byte():
    rng = np.random.default_rng(11)
    data = rng.integers(0, 2**32, size=(1 << 20) + 36, dtype=np.uint32)
    src = torch.from_numpy(data.view(np.int32)).cuda()
    sink = torch.zeros(97, dtype=torch.int32, device="cuda")
    ev.ev_peak_read(src, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(data)


def test_peak_mfma_finishes_with_finite_results():
    sink = torch.full((64,), float("nan"), dtype=torch.float32, device="cuda")
    ev.ev_peak_mfma_bf16(64, 50, sink)
    torch.cuda.synchronize()
    assert torch.isfinite(sink).all()
