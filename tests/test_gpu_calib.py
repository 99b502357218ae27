"""The measurement helpers behind the bench's attainable peaks, checked against
closed forms: the read kernel must read every word once (XOR of its sink = XOR
of the buffer) and the MFMA kernel must run iters x 8 products per wave (sum of
its sink = the sum of the products' entries, which depends only on the column
sums of the two operands)."""
import numpy as np
import pytest
import torch

import int4_weight_only_moe_amd as moe

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("blocks,workgroups", [(32, 64), (1, 64), (37, 5)])
def test_hbm_read_reads_every_word_once(blocks, workgroups):
    g = moe.moe_calib_read_granule()
    rng = np.random.default_rng(blocks * 100 + workgroups)
    host = rng.integers(-2**31, 2**31, blocks * g // 4, dtype=np.int64).astype(np.int32)
    buf = torch.from_numpy(host).cuda()
    sink = torch.full((workgroups * 256,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    moe.moe_calib_hbm_read(buf, sink)
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.view(np.uint32))
    assert got == want


def operand(lane, i, s):
    """Host copy of the kernel's operand hash: fp16 with magnitude in [0.5, 1)."""
    m = 0xFFFFFFFF
    h = ((lane * 0x9E3779B1) & m) ^ (((i + 8 * s) * 0x85EBCA77) & m)
    h ^= h >> 15
    h = (h * 0x2C1B3C6D) & m
    h ^= h >> 12
    bits = ((h >> 16) & 0x8000) | 0x3800 | (h & 0x3FF)
    return float(np.array([bits], dtype=np.uint16).view(np.float16)[0])


def product_sum(sa, sb):
    """Sum of all 256 entries of one 16x16x32 product: lanes 16g..16g+15 hold
    element e of the same K index in both operands, so it is the sum over
    (g, e) of the operands' column sums multiplied."""
    total = 0.0
    for g in range(4):
        for e in range(8):
            ca = sum(operand(16 * g + r, e, sa) for r in range(16))
            cb = sum(operand(16 * g + r, e, sb) for r in range(16))
            total += ca * cb
    return total


@pytest.mark.parametrize("iters,workgroups", [(16, 3), (0, 2), (1, 1)])
def test_mfma_runs_every_product(iters, workgroups):
    sink = torch.full((workgroups * 256,), 7.0, dtype=torch.float32, device="cuda")
    moe.moe_calib_mfma_f16(iters, sink)
    s = sink.cpu().numpy().astype(np.float64).reshape(workgroups * 4, 64).sum(axis=1)  # per wave
    # accumulator 2j + i multiplies A operand i by B operand 2 + j
    per_iter = sum(product_sum(i, 2 + j) for i in range(2) for j in range(4))
    scale = iters * sum(abs(operand(l, e, q)) for l in range(64) for e in range(8) for q in range(6))
    np.testing.assert_allclose(s, iters * per_iter, rtol=0, atol=1e-5 * max(scale, 1.0))
    if iters:
        assert abs(per_iter) > 1e-3 * scale / iters  # the check is not vacuous
