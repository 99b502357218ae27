"""moe_w4a16_layer: the one-call layer. M = 1 runs the two-kernel decode
path (routing inside FC1, output-stationary FC2); while few experts are
touched (M <= 16, M*k <= 256; every small shape here, M = 3..7 on the
384-expert layer) routing and grouping run inside the FC1 kernel; otherwise
the decode path where it fits, else the four-kernel path. Integers must
equal moe_route_align's, the output must meet the oracle bar, and the decode
path's output must be identical on every call."""
import numpy as np
import pytest
import torch

import int4_weight_only_moe_amd as moe
import oracle
import workloads as wl
from gpu_common import (assert_output_close, assert_route_matches, covering_rows, device_layer, k26_layer,
                        oracle_experts, oracle_rows_parallel, route_host, to_dev, x_device)

pytestmark = pytest.mark.gpu

SHAPES = {
    "tiny": (wl.TINY, 0),
    "mid": (wl.LayerShape(E=64, H=1024, I=384, k=6), 3),
    "k16": (wl.LayerShape(E=32, H=256, I=128, k=16), 4),   # M*k up to 64
    "k1": (wl.LayerShape(E=32, H=384, I=640, k=1), 5),
    "e1024": (wl.LayerShape(E=1024, H=256, I=128, k=8), 6),  # 16 logits per lane in the top-k
    # M = 5..16 take the routed FC1 on every shape (M*k <= 256). "wide": the
    # straight-line chunk loop (H = 1024), per-token FC2 at M = 5, grouped FC2
    # and several items per workgroup at 16; "wide_e1024": 16 logits per lane,
    # k = 16 (grouped FC2), several items per workgroup from M = 9
    "wide": (wl.LayerShape(E=128, H=1024, I=256, k=8), 7),
    "wide_e1024": (wl.LayerShape(E=1024, H=256, I=256, k=16), 8),
    # E not a multiple of 32 or 64: a partial last word in the routing bitmap,
    # masked lanes in the top-k
    "odd_e": (wl.LayerShape(E=100, H=512, I=256, k=5), 9),
}


def run_layer_call(layer, logits, x_bits, block_m, reps=1):
    s = layer.shape
    M = logits.shape[0]
    rb = moe.alloc_route_buffers(M, s.E, s.k, block_m)
    lg, x = to_dev(logits), x_device(x_bits)
    outs = []
    for _ in range(reps):
        outs.append(moe.layer(lg, x, rb, s.I, layer.w13, layer.w2).float().cpu().numpy())
    torch.cuda.synchronize()
    return rb, outs


@pytest.mark.parametrize("shape_name", list(SHAPES))
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 9, 16, 17])
@pytest.mark.parametrize("block_m", [16, 32, 64, 128])
def test_layer_matches_oracle(shape_name, M, block_m):
    shape, seed = SHAPES[shape_name]
    if M * shape.k > 64 and M <= 4:
        pytest.skip("not a decode-path size")
    print(f"layer {shape_name} M={M} block_m={block_m}", flush=True)
    layer = device_layer(shape, seed)
    t = wl.tokens(shape, M, 1000 + M)
    rb, outs = run_layer_call(layer, t.logits, t.x_bits, block_m, reps=3)
    ids, w = assert_route_matches(route_host(rb), t.logits, shape.E, shape.k, block_m)
    ref = oracle.moe_forward(wl.f32_from_bf16_bits(t.x_bits).astype(np.float64), ids, w,
                             oracle_experts(shape, seed))
    assert_output_close(outs[0], ref, f"{shape_name} M={M}")
    if M == 1:
        for o in outs[1:]:
            assert np.array_equal(o, outs[0]), "decode path must be deterministic"


def test_layer_k26_decode_sizes():
    layer = k26_layer()
    s = layer.shape
    for M in (1, 2, 4):
        t = wl.tokens(s, M, 4242 + M)
        rb, outs = run_layer_call(layer, t.logits, t.x_bits, 16, reps=2)
        ids, w = assert_route_matches(route_host(rb), t.logits, s.E, s.k, 16)
        assert np.array_equal(outs[0], outs[1])
        rows = [0, M - 1]
        ref = oracle.moe_forward(wl.f32_from_bf16_bits(t.x_bits).astype(np.float64), ids, w,
                                 oracle_experts(s, 2026, keep=0), tokens_subset=rows)
        rel, mx = assert_output_close(outs[0][rows], ref[rows], f"k26 M={M}")
        print(f"layer k26 M={M}: rel-L2 {rel:.2e} max abs {mx:.3f}", flush=True)


@pytest.mark.parametrize("fmt", ["int4", "mxfp4"])
def test_layer_decode_four_tokens_wide_fc1(fmt):
    """Four tokens, 384 experts, top-8, I = 3840: the routed FC1 would need
    about 31 distinct experts x 15 groups of 16 pairs = 470 workgroups, more
    than 1.75 rounds of 256 CUs, while the k activation rows of FC2 still fit
    64 KB of LDS, so the layer call takes the four-token decode kernels (the
    only shapes that reach them), in both weight formats."""
    shape, seed = wl.LayerShape(E=384, H=128, I=3840, k=8), 12
    print(f"layer decode M=4 {fmt} {shape}", flush=True)
    layer = device_layer(shape, seed, fmt=fmt)
    t = wl.tokens(shape, 4, 77)
    rb = moe.alloc_route_buffers(4, shape.E, shape.k, 16)
    lg, x = to_dev(t.logits), x_device(t.x_bits)
    outs = [moe.layer(lg, x, rb, shape.I, layer.w13, layer.w2, fmt=fmt).float().cpu().numpy() for _ in range(2)]
    torch.cuda.synchronize()
    assert np.array_equal(outs[0], outs[1]), "decode path must be deterministic"
    ids, w = assert_route_matches(route_host(rb), t.logits, shape.E, shape.k, 16)
    ref = oracle.moe_forward(wl.f32_from_bf16_bits(t.x_bits).astype(np.float64), ids, w,
                             oracle_experts(shape, seed, fmt=fmt))
    assert_output_close(outs[0], ref, f"decode M=4 {fmt}")


@pytest.mark.parametrize("M", [3, 5, 6, 7, 9, 16, 17, 90])
def test_layer_k26_grouped_sizes(M):
    """The layer call past the decode sizes, as the benchmark times it: the
    routed FC1 at M = 3..7 (several items per workgroup from M = 5), the
    grouped FC1 from 9; FC2 per token up to 16 tokens, the grouped FC2 and
    its finalize above."""
    layer = k26_layer()
    s = layer.shape
    block_m = moe.moe_w4a16_preferred_block_m(M, s.E, s.H, s.I, s.k)
    t = wl.tokens(s, M, 5150 + M)
    rb, outs = run_layer_call(layer, t.logits, t.x_bits, block_m)
    ids, w = assert_route_matches(route_host(rb), t.logits, s.E, s.k, block_m)
    assert np.all(np.isfinite(outs[0]))
    # rows that together hold every expert the batch routes to
    rows = covering_rows(ids, [0, M // 2, M - 1])
    ref = oracle_rows_parallel(s, 2026, wl.f32_from_bf16_bits(t.x_bits).astype(np.float64), ids, w, rows)
    rel, mx = assert_output_close(outs[0][rows], ref[rows], f"k26 layer M={M}")
    print(f"layer k26 M={M} B={block_m}: {len(rows)} rows, experts covered "
          f"{np.unique(ids[rows]).size}/{np.unique(ids).size}, rel-L2 {rel:.2e} max abs {mx:.3f}", flush=True)


def test_layer_k26_m1_closed_form():
    """Constant weights (q = +1, s = 2^-7) and x = 1: exactly 50176 through the decode path."""
    from test_gpu_forward import const_layer
    layer = const_layer(wl.K26)
    rng = np.random.default_rng(12)
    logits = rng.standard_normal((1, 384)).astype(np.float32)
    x_bits = wl.bf16_bits_from_f32(np.ones((1, 7168), np.float32))
    _, outs = run_layer_call(layer, logits, x_bits, 16)
    assert np.all(outs[0] == 50176.0)


@pytest.mark.parametrize("shape_name,M", [("mid", 2), ("wide", 5)])
def test_layer_graph_replays(shape_name, M):
    shape, seed = SHAPES[shape_name]
    layer = device_layer(shape, seed)
    t = wl.tokens(shape, M, 5)
    lg, x = to_dev(t.logits), x_device(t.x_bits)
    rb = moe.alloc_route_buffers(M, shape.E, shape.k, 16)
    ws = torch.empty(moe.moe_w4a16_workspace_bytes(M, shape.E, shape.H, shape.I, shape.k), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((M, shape.H), dtype=torch.bfloat16, device="cuda")
    moe.layer(lg, x, rb, shape.I, layer.w13, layer.w2, workspace=ws, out=out)
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.layer(lg, x, rb, shape.I, layer.w13, layer.w2, workspace=ws, out=out)
    y = torch.randn(512, 512, device="cuda")
    for _ in range(4):
        out.fill_(0)
        rb.topk_ids.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
        (y @ y).sum().item()


def test_layer_decode_ties_and_shared_experts():
    """Equal logits at the top-k boundary and tokens sharing experts, through the decode path."""
    shape = wl.LayerShape(E=64, H=256, I=128, k=8)
    layer = device_layer(shape, 21)
    base = np.full((3, 64), -1.0, np.float32)
    base[:, [3, 9, 17, 40, 41, 50, 60, 63, 5, 7]] = 2.0          # 10 equal maxima: lowest 8 indices win
    base[1, 12] = 3.0
    base[2] = np.linspace(1, 0, 64, dtype=np.float32)               # shares experts 0..7 with nobody
    base[2, 3] = 5.0                                                # shares expert 3 with tokens 0 and 1
    x_bits = wl.bf16_bits_from_f32(np.random.default_rng(3).standard_normal((3, 256)).astype(np.float32))
    for M in (1, 2, 3):
        rb, outs = run_layer_call(layer, base[:M], x_bits[:M], 16, reps=2)
        ids, w = assert_route_matches(route_host(rb), base[:M], shape.E, shape.k, 16)
        ref = oracle.moe_forward(wl.f32_from_bf16_bits(x_bits[:M]).astype(np.float64), ids, w,
                                 oracle_experts(shape, 21))
        assert_output_close(outs[0], ref, f"ties M={M}")
        assert np.array_equal(outs[0], outs[1])


def test_layer_routed_sizes_with_tiled_grouped_gemm():
    """Sixteen tokens on 8 experts with top-8: few experts are touched, so the
    routed FC1 would be preferred, but every expert holds 16 assignments, so
    the grouped GEMM is the tiled one. The routed FC1 writes no tile table, so
    the layer call must take routing + tiled FC1 + tiled FC2 here."""
    shape, M = wl.LayerShape(E=8, H=256, I=256, k=8), 16
    assert M * shape.k / shape.E >= 16          # the tiled grouped GEMM's threshold
    assert M <= 16 and M * shape.k <= 256       # the routed FC1's size limits
    assert M * shape.k > 1.2 * shape.E          # not the per-token FC2: the grouped FC2 follows
    layer = device_layer(shape, 31)
    t = wl.tokens(shape, M, 32)
    for block_m in (16, 32, 64, 128):
        rb, outs = run_layer_call(layer, t.logits, t.x_bits, block_m)
        ids, w = assert_route_matches(route_host(rb), t.logits, shape.E, shape.k, block_m)
        ref = oracle.moe_forward(wl.f32_from_bf16_bits(t.x_bits).astype(np.float64), ids, w,
                                 oracle_experts(shape, 31))
        assert_output_close(outs[0], ref, f"routed-size tiled B={block_m}")
