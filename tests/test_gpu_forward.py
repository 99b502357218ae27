"""The full layer (moe_route_align + moe_w4a16_forward) on the GPU against the
oracle: every element at sizes the oracle finishes in seconds (several tiles,
ragged tails), sampled token rows at the 384-expert sizes, closed forms, and
edge cases."""
import math

import numpy as np
import pytest
import torch

import int4_weight_only_moe_amd as moe
import oracle
import workloads as wl
from gpu_common import (DeviceLayer, assert_output_close, assert_route_matches, covering_rows, device_layer,
                        k26_layer, oracle_experts, oracle_rows_parallel, route_host, run_layer,
                        tile_rows_of_hot_experts, to_dev, x_device)

pytestmark = pytest.mark.gpu

MID_SHAPES = [
    # (shape, M, weight seed, token seed): several tiles in N and K, ragged M
    (wl.TINY, 16, 0, 0),
    (wl.LayerShape(E=16, H=512, I=256, k=4), 37, 1, 2),
    (wl.LayerShape(E=64, H=1024, I=384, k=6), 100, 3, 4),
    (wl.LayerShape(E=32, H=384, I=640, k=1), 70, 5, 6),
    (wl.LayerShape(E=4, H=256, I=128, k=4), 200, 7, 8),   # every expert gets every token: many blocks
    (wl.LayerShape(E=1024, H=256, I=128, k=16), 50, 9, 10),  # the largest E and top-k the ABI takes
]


@pytest.mark.parametrize("case", range(len(MID_SHAPES)))
@pytest.mark.parametrize("block_m", [16, 32, 64, 128])
def test_full_parity_mid_shapes(case, block_m):
    shape, M, wseed, tseed = MID_SHAPES[case]
    print(f"forward {shape} M={M} block_m={block_m}", flush=True)
    layer = device_layer(shape, wseed)
    t = wl.tokens(shape, M, tseed)
    rb, out = run_layer(layer, t.logits, t.x_bits, block_m)
    ids, w = assert_route_matches(route_host(rb), t.logits, shape.E, shape.k, block_m)
    x = wl.f32_from_bf16_bits(t.x_bits).astype(np.float64)
    ref = oracle.moe_forward(x, ids, w, oracle_experts(shape, wseed))
    assert np.all(np.isfinite(out))
    assert_output_close(out, ref, f"{shape} M={M} B={block_m}")


def const_layer(shape, byte=0x99, scale_bits=0x2000):
    E, H, I = shape.E, shape.H, shape.I
    q13 = torch.full((E, 2 * I, H // 2), byte, dtype=torch.uint8, device="cuda")
    s13 = torch.full((E, 2 * I, H // 32), scale_bits, dtype=torch.int16, device="cuda").view(torch.float16)
    q2 = torch.full((E, H, I // 2), byte, dtype=torch.uint8, device="cuda")
    s2 = torch.full((E, H, I // 32), scale_bits, dtype=torch.int16, device="cuda").view(torch.float16)
    layer = DeviceLayer.__new__(DeviceLayer)
    layer.shape = shape
    layer.fmt = "int4"
    layer.w13 = moe.repack(q13, s13, moe.KIND_W13)
    layer.w2 = moe.repack(q2, s2, moe.KIND_W2)
    torch.cuda.synchronize()
    return layer


@pytest.mark.parametrize("case", [1, 3])
def test_block_kernels_with_oversized_route_buffers(case):
    """Route buffers allocated for a batch 400 times larger (cap far above
    this batch's capacity) through the block kernels (wide and narrow): their
    grid is sized from the batch, so the result is unchanged."""
    shape, M, wseed, tseed = MID_SHAPES[case]
    layer = device_layer(shape, wseed)
    t = wl.tokens(shape, M, tseed)
    for block_m in (16, 32, 64, 128):
        big = moe.alloc_route_buffers(400 * M, shape.E, shape.k, block_m)
        assert big.cap >= 5 * moe.moe_route_align_capacity(M, shape.E, shape.k, block_m)
        rb = moe.RouteBuffers(M, shape.E, shape.k, block_m, big.cap, big.topk_ids[:M], big.topk_weights[:M],
                              big.sorted_token_ids, big.block_expert_ids, big.expert_offsets,
                              big.num_tokens_post_pad)
        moe.route_align(to_dev(t.logits), rb)
        out = moe.forward(x_device(t.x_bits), rb, shape.I, layer.w13, layer.w2).float().cpu().numpy()
        torch.cuda.synchronize()
        ids, w = assert_route_matches(route_host(rb), t.logits, shape.E, shape.k, block_m)
        ref = oracle.moe_forward(wl.f32_from_bf16_bits(t.x_bits).astype(np.float64), ids, w,
                                 oracle_experts(shape, wseed))
        assert_output_close(out, ref, f"{shape} M={M} oversized cap B={block_m}")


@pytest.mark.parametrize("case", [1, 3, 5])
def test_block_m_128_half_map(case):
    """block_m = 128 outside the tiled kernel: the block kernels take at most
    64 rows, so the forward runs each block as its two 64-row halves through
    a map of the halves' experts left where the tile table would be (after
    the tile count's 256 bytes): the expert for a half that holds a row, -1
    for an all-padding half (skipped, its weights not read) and for halves
    past the padded total. Checked against the routing outputs, and the
    output against the oracle."""
    shape, M, wseed, tseed = MID_SHAPES[case]
    assert M * shape.k / shape.E < 16  # the block kernels, not the tiled one
    layer = device_layer(shape, wseed)
    t = wl.tokens(shape, M, tseed)
    rb = moe.alloc_route_buffers(M, shape.E, shape.k, 128)
    moe.route_align(to_dev(t.logits), rb)
    ws = torch.full((moe.moe_w4a16_workspace_bytes(M, shape.E, shape.H, shape.I, shape.k),), 0x5A, dtype=torch.uint8,
                    device="cuda")
    out = moe.forward(x_device(t.x_bits), rb, shape.I, layer.w13, layer.w2, workspace=ws)
    torch.cuda.synchronize()
    h = route_host(rb)
    MK = M * shape.k
    cap = moe.moe_route_align_capacity(M, shape.E, shape.k, 128)
    npp = h["num_tokens_post_pad"]
    srt, blk = h["sorted_token_ids"], h["block_expert_ids"]
    want = [int(blk[i // 2]) if i * 64 < npp and srt[i * 64] < MK else -1 for i in range(cap // 64)]
    assert any(v == -1 for v in want[: npp // 64])  # some all-padding halves inside the list

    def a256(v):
        return (v + 255) // 256 * 256
    off = a256(M * shape.H * 4) + a256(MK * shape.I * 2) + 256
    got = ws.cpu().numpy()[off:off + 4 * len(want)].view(np.int32)
    assert got.tolist() == want
    ids, w = assert_route_matches(h, t.logits, shape.E, shape.k, 128)
    ref = oracle.moe_forward(wl.f32_from_bf16_bits(t.x_bits).astype(np.float64), ids, w,
                             oracle_experts(shape, wseed))
    assert_output_close(out.float().cpu().numpy(), ref, f"{shape} M={M} B=128 halves")


@pytest.mark.parametrize("shape,M,expect", [
    (wl.TINY, 16, 3.515625),   # act = bf16(silu(2) * 2) = 3.515625, y = act * I/128 = act
    (wl.K26, 3, 50176.0),      # gate = up = 56, act = 3136, y = 16 * 3136, all exact
])
def test_closed_form_constant_weights(shape, M, expect):
    """q = +1, s = 2^-7, x = 1: out = (I/128) * bf16(silu(H/128) * H/128), exactly."""
    layer = const_layer(shape)
    rng = np.random.default_rng(11)
    logits = rng.standard_normal((M, shape.E)).astype(np.float32)
    x_bits = wl.bf16_bits_from_f32(np.ones((M, shape.H), np.float32))
    for block_m in (16, 64):
        _, out = run_layer(layer, logits, x_bits, block_m)
        assert np.all(out == expect), (block_m, np.unique(out)[:8])
    h = shape.H / 128
    act = h / (1 + math.exp(-h)) * h
    assert abs(act * shape.I / 128 - expect) <= 2 ** -7 * expect  # the bf16 rounding of act


def test_zero_input_gives_zero_output():
    shape = wl.LayerShape(E=16, H=512, I=256, k=4)
    layer = device_layer(shape, 1)
    rng = np.random.default_rng(2)
    logits = rng.standard_normal((40, shape.E)).astype(np.float32)
    x_bits = np.zeros((40, shape.H), np.uint16)
    _, out = run_layer(layer, logits, x_bits, 16)
    assert np.all(out == 0.0)


def test_empty_batch_is_a_no_op():
    shape = wl.TINY
    layer = device_layer(shape, 0)
    rb = moe.alloc_route_buffers(0, shape.E, shape.k, 16)
    out = torch.full((0, shape.H), 1.0, dtype=torch.bfloat16, device="cuda")
    x = torch.empty((0, shape.H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    moe.moe_w4a16_forward(x, shape.E, shape.I, shape.k, 16, rb.topk_weights, rb.sorted_token_ids,
                          rb.block_expert_ids, rb.expert_offsets, rb.num_tokens_post_pad, layer.w13, layer.w2,
                          ws, out, cap=rb.cap)
    torch.cuda.synchronize()


def test_empty_batch_layer_is_a_no_op():
    shape = wl.TINY
    layer = device_layer(shape, 0)
    rb = moe.alloc_route_buffers(0, shape.E, shape.k, 16)
    out = torch.full((0, shape.H), 1.0, dtype=torch.bfloat16, device="cuda")
    x = torch.empty((0, shape.H), dtype=torch.bfloat16, device="cuda")
    logits = torch.empty((0, shape.E), dtype=torch.float32, device="cuda")
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    moe.moe_w4a16_layer(logits, x, shape.I, shape.k, 16, rb.topk_ids, rb.topk_weights, rb.sorted_token_ids,
                        rb.block_expert_ids, rb.expert_offsets, rb.num_tokens_post_pad, layer.w13, layer.w2,
                        ws, out, cap=rb.cap)
    torch.cuda.synchronize()


def test_output_guard_bands_and_reuse():
    """Output rows outside [0, M) untouched; a second, smaller call reuses the workspace."""
    shape = wl.LayerShape(E=16, H=512, I=256, k=4)
    layer = device_layer(shape, 1)
    big = moe.moe_w4a16_workspace_bytes(60, shape.E, shape.H, shape.I, shape.k)
    ws = torch.full((big,), 0xAB, dtype=torch.uint8, device="cuda")
    experts = oracle_experts(shape, 1)
    for M in (60, 23):
        t = wl.tokens(shape, M, 100 + M)
        rb = moe.alloc_route_buffers(M, shape.E, shape.k, 16)
        moe.route_align(to_dev(t.logits), rb)
        G = 3
        guarded = torch.full((M + 2 * G, shape.H), -7.0, dtype=torch.bfloat16, device="cuda")
        moe.forward(x_device(t.x_bits), rb, shape.I, layer.w13, layer.w2, workspace=ws, out=guarded[G:G + M])
        torch.cuda.synchronize()
        g = guarded.float().cpu().numpy()
        assert np.all(g[:G] == -7.0) and np.all(g[-G:] == -7.0)
        ids, w = assert_route_matches(route_host(rb), t.logits, shape.E, shape.k, 16)
        x = wl.f32_from_bf16_bits(t.x_bits).astype(np.float64)
        assert_output_close(g[G:G + M], oracle.moe_forward(x, ids, w, experts), f"M={M}")


# ---------------------------------------------------------------- 384-expert layer
# Token rows compared with the oracle at the 384-expert sizes: a few fixed
# rows, and for the workloads named in COVER a greedy set of rows that
# together hold every expert the batch routes to (for the skewed batch also
# a row in every tile of each expert holding more than one 128-row tile).
K26_SAMPLES = {
    "k26_m1": [0],
    "k26_m9": [0, 4, 8],
    "k26_m90": [0, 57, 89],
    "k26_m256": [0, 255],
    "k26_m512": [0, 300, 511],
    "k26_m1024": [0, 700, 1023],
    "k26_m1024_skew": [0, 1023],
    "k26_m2048": [0, 2047],
    "k26_m4096": [1, 4095],
    "k26_m8192": [0, 5000, 8191],
}
COVER = ("k26_m90", "k26_m1024", "k26_m1024_skew", "k26_m4096")


@pytest.mark.parametrize("name", list(K26_SAMPLES))
def test_k26_sampled_parity(name):
    w = wl.WORKLOADS[name]
    s = w.shape
    print(f"forward {name}: building/using the 384-expert layer", flush=True)
    layer = k26_layer()
    t = wl.workload_tokens(w)
    block_m = moe.moe_w4a16_preferred_block_m(w.M, s.E, s.H, s.I, s.k)
    rb, out = run_layer(layer, t.logits, t.x_bits, block_m)
    print(f"forward {name}: block_m={block_m}, checking routing", flush=True)
    ids, wts = assert_route_matches(route_host(rb), t.logits, s.E, s.k, block_m)
    assert np.all(np.isfinite(out))
    rows = list(K26_SAMPLES[name])
    if name in COVER:
        rows = covering_rows(ids, rows + (tile_rows_of_hot_experts(ids, 128) if name.endswith("skew") else []))
    touched = np.unique(ids)
    covered = np.unique(ids[rows])
    x = wl.f32_from_bf16_bits(t.x_bits).astype(np.float64)
    ref = oracle_rows_parallel(s, 2026, x, ids, wts, rows)
    rel, mx = assert_output_close(out[rows], ref[rows], name)
    print(f"forward {name}: {len(rows)} rows, experts covered {covered.size}/{touched.size}, "
          f"rel-L2 {rel:.2e} max abs {mx:.3f}", flush=True)
    if name in COVER:
        assert covered.size == touched.size


@pytest.mark.parametrize("block_m", [16, 32, 64, 128])
def test_k26_m90_every_block_m(block_m):
    w = wl.WORKLOADS["k26_m90"]
    s = w.shape
    layer = k26_layer()
    t = wl.workload_tokens(w)
    rb, out = run_layer(layer, t.logits, t.x_bits, block_m)
    ids, wts = assert_route_matches(route_host(rb), t.logits, s.E, s.k, block_m)
    x = wl.f32_from_bf16_bits(t.x_bits).astype(np.float64)
    rows = [13]
    ref = oracle.moe_forward(x, ids, wts, oracle_experts(s, 2026, keep=0), tokens_subset=rows)
    assert_output_close(out[rows], ref[rows], f"k26_m90 B={block_m}")


@pytest.mark.parametrize("name", ["k26_m1024", "k26_m1024_skew"])
def test_k26_block_m_128_tiled(name):
    """The 384-expert layer with 128-row blocks on the tiled path (each block
    one tile; the skewed batch's hot experts several): every element of a
    set of token rows that together touch every routed expert."""
    w = wl.WORKLOADS[name]
    s = w.shape
    layer = k26_layer()
    t = wl.workload_tokens(w)
    rb, out = run_layer(layer, t.logits, t.x_bits, 128)
    ids, wts = assert_route_matches(route_host(rb), t.logits, s.E, s.k, 128)
    assert np.all(np.isfinite(out))
    rows = covering_rows(ids, [0] + (tile_rows_of_hot_experts(ids, 128) if name.endswith("skew") else []))
    covered, touched = np.unique(ids[rows]), np.unique(ids)
    x = wl.f32_from_bf16_bits(t.x_bits).astype(np.float64)
    ref = oracle_rows_parallel(s, 2026, x, ids, wts, rows)
    assert_output_close(out[rows], ref[rows], f"{name} B=128")
    print(f"forward {name} B=128: {len(rows)} rows, experts covered {covered.size}/{touched.size}", flush=True)
    assert covered.size == touched.size
