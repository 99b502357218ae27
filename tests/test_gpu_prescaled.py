"""The pre-scaled tiled GEMM (128-row tiles; INT4 weights enter the matrix
core as fp16(q * s * 2^-sigma), the activation rows as fp16 copies scaled by a
power of two): the per-row exponent shifts the repack stores after the INT4
tiles, and every element against the oracle where fp16 alone would overflow
or lose precision (huge and tiny group scales, activation rows far outside
fp16's range, all-zero rows)."""
import numpy as np
import pytest
import torch

import int4_weight_only_moe_amd as moe
import oracle
import workloads as wl
from gpu_common import (DeviceLayer, assert_output_close, assert_route_matches, route_host, run_layer, to_dev)

pytestmark = pytest.mark.gpu

SHAPE = wl.LayerShape(E=8, H=256, I=256, k=2)
M = 300  # 75 assignments per expert: the pre-scaled kernel's regime


def expected_sigma(scales_f16: np.ndarray) -> np.ndarray:
    """clamp(floor(log2(max_g |s|)) - 11, -15, 4) per weight row, 0 for a row of zero scales."""
    m = np.abs(scales_f16.astype(np.float64)).max(axis=-1)
    _, ex = np.frexp(m)  # m = f * 2^ex, f in [0.5, 1): floor(log2 m) = ex - 1
    sig = np.clip(ex - 1 - 11, -15, 4)
    return np.where(m == 0, 0, sig).astype(np.int8)


def layer_with_scales(factor13: float, factor2: float, seed: int = 41, shape=SHAPE):
    w13, s13, w2, s2 = wl.layer_weights(shape, seed)
    s13 = (s13.astype(np.float64) * factor13).astype(np.float16)
    s2 = (s2.astype(np.float64) * factor2).astype(np.float16)
    return (w13, s13, w2, s2), DeviceLayer(shape, w13, s13, w2, s2)


def experts_of(host):
    w13, s13, w2, s2 = host
    return oracle.DequantCache(lambda e: (w13[e], s13[e], w2[e], s2[e]))


def test_sigma_trailer_matches_the_scales():
    rng = np.random.default_rng(5)
    E, N, K = 3, 64, 256
    q = torch.from_numpy(rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)).cuda()
    # per-row magnitudes from fp16 subnormals to the top of the range, one all-zero row
    mag = np.exp2(rng.uniform(-23, 15.9, (E, N, 1)))
    s = (rng.uniform(0.5, 1.0, (E, N, K // 32)) * mag).astype(np.float16)
    s[1, 7] = 0
    s[2, 3, 0] = -s[2, 3, 0]  # the sign does not count
    packed = moe.repack(q, torch.from_numpy(s.view(np.int16)).cuda().view(torch.float16), moe.KIND_W2)
    torch.cuda.synchronize()
    body = E * N * K * 9 // 16
    assert packed.numel() == body + E * N
    got = packed[body:].cpu().numpy().view(np.int8).reshape(E, N)
    np.testing.assert_array_equal(got, expected_sigma(s))
    assert got.min() == -15 and got.max() == 4


@pytest.mark.parametrize("factor13,factor2", [(2.0 ** 19, 2.0 ** 18), (2.0 ** -12, 2.0 ** -11), (2.0 ** 19, 2.0 ** -12)])
def test_prescaled_extreme_scales(factor13, factor2):
    """Group scales up to ~1e4 (q * s beyond fp16's range without the row shift)
    and fp16-subnormal scales (rows shifted up by 2^15)."""
    host, layer = layer_with_scales(factor13, factor2)
    t = wl.tokens(SHAPE, M, 42)
    for block_m in (16, 64):
        rb, out = run_layer(layer, t.logits, t.x_bits, block_m)
        ids, w = assert_route_matches(route_host(rb), t.logits, SHAPE.E, SHAPE.k, block_m)
        ref = oracle.moe_forward(wl.f32_from_bf16_bits(t.x_bits).astype(np.float64), ids, w, experts_of(host))
        assert np.all(np.isfinite(out))
        rel, mx = assert_output_close(out, ref, f"scales x{factor13:g}/x{factor2:g} B={block_m}")
        print(f"prescaled scales x{factor13:g}/x{factor2:g} B={block_m}: rel-L2 {rel:.2e}", flush=True)


# the fp16 row copies: hidden 256, 7168 and 8192 hold a row in registers (2,
# 14 and 16 vectors per lane), 8448 takes the two-pass loop
@pytest.mark.parametrize("H", [256, 7168, 8192, 8448])
def test_prescaled_activation_rows_outside_fp16(H):
    """Rows scaled by 1e6 (beyond 65504) and 1e-6, and all-zero rows: each row
    keeps its own power-of-two scale; zero rows give exactly zero."""
    shape = wl.LayerShape(E=SHAPE.E, H=H, I=SHAPE.I, k=SHAPE.k)
    host, layer = layer_with_scales(1.0, 1.0, shape=shape)
    t = wl.tokens(shape, M, 43)
    x = wl.f32_from_bf16_bits(t.x_bits)
    x[0::3] *= 1e6
    x[1::3] *= 1e-6
    x[5] = 0.0
    x[77] = 0.0
    x_bits = wl.bf16_bits_from_f32(x)
    print(f"prescaled activation rows H={H}", flush=True)
    rb, out = run_layer(layer, t.logits, x_bits, 64)
    ids, w = assert_route_matches(route_host(rb), t.logits, shape.E, shape.k, 64)
    ref = oracle.moe_forward(wl.f32_from_bf16_bits(x_bits).astype(np.float64), ids, w, experts_of(host))
    assert np.all(out[5] == 0) and np.all(out[77] == 0)
    # each magnitude class against the oracle on its own rows
    for rows, what in ((np.arange(0, M, 3), "x1e6"), (np.arange(1, M, 3), "x1e-6"), (np.arange(2, M, 3), "x1")):
        rows = rows[(rows != 5) & (rows != 77)]
        assert_output_close(out[rows], ref[rows], what)
