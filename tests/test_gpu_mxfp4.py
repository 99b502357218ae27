"""MXFP4 expert weights (moe_mxfp4_*) on the GPU against the oracle: the
repack round trip bit-exact, every element of the forward and the layer call
at sizes the oracle finishes in seconds (narrow, wide and tiled grouped
kernels; decode, routed and grouped layer paths), a wide spread of group
scales, a closed form and sampled rows at the 384-expert sizes."""
import numpy as np
import pytest
import torch

import int4_weight_only_moe_amd as moe
import oracle
import workloads as wl
from gpu_common import (DeviceLayer, assert_output_close, assert_route_matches, covering_rows, device_layer,
                        k26_mxfp4_layer, oracle_experts, oracle_rows_parallel, route_host, run_layer, to_dev, x_device)

pytestmark = pytest.mark.gpu

SHAPES = [
    # (shape, weight seed): the first two have 16 pairs per FC1 row block (wide
    # kernel, routed FC1), the third has ragged pair counts
    (wl.TINY, 0),
    (wl.LayerShape(E=128, H=1024, I=256, k=8), 7),
    (wl.LayerShape(E=64, H=1024, I=384, k=6), 3),
]


def _x(t):
    return wl.f32_from_bf16_bits(t.x_bits).astype(np.float64)


def test_mxfp4_repack_round_trip():
    rng = np.random.default_rng(5)
    for kind, (E, N, K) in ((moe.KIND_W13, (3, 256, 384)), (moe.KIND_W2, (2, 384, 256))):
        q = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
        s = rng.integers(0, 256, (E, N, K // 32), dtype=np.uint8)
        packed = moe.repack_mxfp4(to_dev(q), to_dev(s), kind)
        assert packed.numel() == E * N * K * 17 // 32
        q2 = torch.empty((E, N, K // 2), dtype=torch.uint8, device="cuda")
        s2 = torch.empty((E, N, K // 32), dtype=torch.uint8, device="cuda")
        moe.moe_mxfp4_unpack(packed, E, N, K, kind, q2, s2)
        torch.cuda.synchronize()
        assert np.array_equal(q2.cpu().numpy(), q) and np.array_equal(s2.cpu().numpy(), s)


@pytest.mark.parametrize("case", range(len(SHAPES)))
@pytest.mark.parametrize("M,block_m", [(1, 16), (5, 16), (33, 32), (33, 64), (300, 32), (300, 64), (33, 128),
                                       (300, 128)])
def test_mxfp4_forward_matches_oracle(case, M, block_m):
    shape, seed = SHAPES[case]
    print(f"mxfp4 forward {shape} M={M} block_m={block_m}", flush=True)
    layer = device_layer(shape, seed, fmt="mxfp4")
    t = wl.tokens(shape, M, 100 + M)
    rb, out = run_layer(layer, t.logits, t.x_bits, block_m)
    ids, w = assert_route_matches(route_host(rb), t.logits, shape.E, shape.k, block_m)
    ref = oracle.moe_forward(_x(t), ids, w, oracle_experts(shape, seed, fmt="mxfp4"))
    assert np.all(np.isfinite(out))
    assert_output_close(out, ref, f"mxfp4 {shape} M={M} B={block_m}")


@pytest.mark.parametrize("case", range(len(SHAPES)))
@pytest.mark.parametrize("M", [1, 2, 3, 5, 9, 16, 17, 40])
def test_mxfp4_layer_matches_oracle(case, M):
    shape, seed = SHAPES[case]
    print(f"mxfp4 layer {shape} M={M}", flush=True)
    layer = device_layer(shape, seed, fmt="mxfp4")
    block_m = moe.moe_w4a16_preferred_block_m(M, shape.E, shape.H, shape.I, shape.k)
    t = wl.tokens(shape, M, 200 + M)
    rb = moe.alloc_route_buffers(M, shape.E, shape.k, block_m)
    out = moe.layer(to_dev(t.logits), x_device(t.x_bits), rb, shape.I, layer.w13, layer.w2, fmt="mxfp4")
    torch.cuda.synchronize()
    ids, w = assert_route_matches(route_host(rb), t.logits, shape.E, shape.k, block_m)
    ref = oracle.moe_forward(_x(t), ids, w, oracle_experts(shape, seed, fmt="mxfp4"))
    assert_output_close(out.float().cpu().numpy(), ref, f"mxfp4 layer {shape} M={M}")


def test_mxfp4_wide_scale_spread():
    """Group scales from 2^-20 to 2^10 (each group its own): the scale of every
    group reaches its 32 products."""
    shape = wl.LayerShape(E=8, H=512, I=256, k=2)
    rng = np.random.default_rng(9)
    w13 = rng.integers(0, 256, (shape.E, 2 * shape.I, shape.H // 2), dtype=np.uint8)
    w2 = rng.integers(0, 256, (shape.E, shape.H, shape.I // 2), dtype=np.uint8)
    s13 = (127 + rng.integers(-20, -9, (shape.E, 2 * shape.I, shape.H // 32))).astype(np.uint8)
    s2 = (127 + rng.integers(0, 11, (shape.E, shape.H, shape.I // 32))).astype(np.uint8)
    layer = DeviceLayer(shape, w13, s13, w2, s2, fmt="mxfp4")
    experts = oracle.DequantCache(lambda e: (w13[e], s13[e], w2[e], s2[e]), fmt="mxfp4")
    for M, block_m in ((3, 16), (40, 32), (200, 64), (200, 128)):
        t = wl.tokens(shape, M, 300 + M)
        rb, out = run_layer(layer, t.logits, t.x_bits, block_m)
        ids, w = assert_route_matches(route_host(rb), t.logits, shape.E, shape.k, block_m)
        assert_output_close(out, oracle.moe_forward(_x(t), ids, w, experts), f"spread M={M}")


def test_mxfp4_k26_closed_form():
    """FP4 code 2 (1.0) with scale 2^-7 everywhere and x = 1: every output is
    exactly 50176 (FC1: 7168 / 128 = 56, act = bf16(silu(56) * 56) = 3136; FC2:
    2048 / 128 * 3136), through the decode path and the grouped path."""
    s = wl.K26
    q13 = torch.full((s.E, 2 * s.I, s.H // 2), 0x22, dtype=torch.uint8, device="cuda")
    q2 = torch.full((s.E, s.H, s.I // 2), 0x22, dtype=torch.uint8, device="cuda")
    sc13 = torch.full((s.E, 2 * s.I, s.H // 32), 120, dtype=torch.uint8, device="cuda")
    sc2 = torch.full((s.E, s.H, s.I // 32), 120, dtype=torch.uint8, device="cuda")
    w13 = moe.repack_mxfp4(q13, sc13, moe.KIND_W13)
    w2 = moe.repack_mxfp4(q2, sc2, moe.KIND_W2)
    del q13, q2, sc13, sc2
    rng = np.random.default_rng(12)
    for M in (1, 4, 40):
        logits = rng.standard_normal((M, s.E)).astype(np.float32)
        x = x_device(wl.bf16_bits_from_f32(np.ones((M, s.H), np.float32)))
        block_m = moe.moe_w4a16_preferred_block_m(M, s.E, s.H, s.I, s.k)
        rb = moe.alloc_route_buffers(M, s.E, s.k, block_m)
        out = moe.layer(to_dev(logits), x, rb, s.I, w13, w2, fmt="mxfp4").float().cpu().numpy()
        assert np.all(np.abs(out - 50176.0) <= 50176.0 * 2 ** -8), f"M={M}: {out.min()} .. {out.max()}"
    del w13, w2


K26_SAMPLES = {"k26_m1": [0], "k26_m4": [0, 3], "k26_m9": [0, 8], "k26_m90": [0, 89], "k26_m1024": [0, 1023],
               "k26_m4096": [0, 4095]}
COVER = ("k26_m1024", "k26_m4096")  # every routed expert in a checked row


@pytest.mark.parametrize("name", list(K26_SAMPLES))
def test_mxfp4_k26_sampled(name):
    w = wl.WORKLOADS[name]
    s = w.shape
    print(f"mxfp4 {name}: building/using the 384-expert MXFP4 layer", flush=True)
    layer = k26_mxfp4_layer()
    t = wl.workload_tokens(w)
    block_m = moe.moe_w4a16_preferred_block_m(w.M, s.E, s.H, s.I, s.k)
    rb = moe.alloc_route_buffers(w.M, s.E, s.k, block_m)
    out = moe.layer(to_dev(t.logits), x_device(t.x_bits), rb, s.I, layer.w13, layer.w2, fmt="mxfp4")
    out = out.float().cpu().numpy()
    ids, wts = assert_route_matches(route_host(rb), t.logits, s.E, s.k, block_m)
    assert np.all(np.isfinite(out))
    rows = K26_SAMPLES[name]
    if name in COVER:
        rows = covering_rows(ids, rows)
    ref = oracle_rows_parallel(s, 2026, _x(t), ids, wts, rows, fmt="mxfp4")
    rel, mx = assert_output_close(out[rows], ref[rows], f"mxfp4 {name}")
    print(f"mxfp4 {name}: {len(rows)} rows, experts covered {np.unique(ids[rows]).size}/{np.unique(ids).size}, "
          f"rel-L2 {rel:.2e} max abs {mx:.3f}", flush=True)


@pytest.mark.parametrize("M", [2, 5])
def test_mxfp4_layer_graph_replays(M):
    """The MXFP4 layer call captured in a HIP graph: every replay equals the
    eager call (decode path at M = 2, routed FC1 + per-token FC2 at M = 5)."""
    shape, seed = SHAPES[1]
    layer = device_layer(shape, seed, fmt="mxfp4")
    t = wl.tokens(shape, M, 400 + M)
    lg, x = to_dev(t.logits), x_device(t.x_bits)
    rb = moe.alloc_route_buffers(M, shape.E, shape.k, 16)
    ws = torch.empty(moe.moe_w4a16_workspace_bytes(M, shape.E, shape.H, shape.I, shape.k), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((M, shape.H), dtype=torch.bfloat16, device="cuda")
    moe.layer(lg, x, rb, shape.I, layer.w13, layer.w2, workspace=ws, out=out, fmt="mxfp4")
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.layer(lg, x, rb, shape.I, layer.w13, layer.w2, workspace=ws, out=out, fmt="mxfp4")
    y = torch.randn(512, 512, device="cuda")
    for _ in range(4):
        out.fill_(0)
        rb.topk_ids.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
        (y @ y).sum().item()
