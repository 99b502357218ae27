"""A layer call captured in a HIP graph: every replay, with eager work and
synchronisations between replays, matches the eager result and the oracle."""
import numpy as np
import pytest
import torch

import int4_weight_only_moe_amd as moe
import oracle
import workloads as wl
from gpu_common import assert_output_close, device_layer, oracle_experts, to_dev, x_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("block_m", [16, 32])
def test_graph_replays_match_eager(block_m):
    shape = wl.LayerShape(E=16, H=512, I=256, k=4)
    layer = device_layer(shape, 1)
    M = 29
    t = wl.tokens(shape, M, 77)
    logits, x = to_dev(t.logits), x_device(t.x_bits)
    rb = moe.alloc_route_buffers(M, shape.E, shape.k, block_m)
    ws = torch.empty(moe.moe_w4a16_workspace_bytes(M, shape.E, shape.H, shape.I, shape.k), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((M, shape.H), dtype=torch.bfloat16, device="cuda")

    def call():
        moe.route_align(logits, rb)
        moe.forward(x, rb, shape.I, layer.w13, layer.w2, workspace=ws, out=out)

    call()
    torch.cuda.synchronize()
    eager = out.float().cpu().numpy()
    ids = rb.topk_ids.cpu().numpy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    xx = torch.randn(1024, 1024, device="cuda")
    ref = oracle.moe_forward(wl.f32_from_bf16_bits(t.x_bits).astype(np.float64), *oracle.route(t.logits, shape.k),
                             oracle_experts(shape, 1))
    for rep in range(4):
        out.fill_(-1.0)
        rb.sorted_token_ids.fill_(-5)
        g.replay()
        torch.cuda.synchronize()
        got = out.float().cpu().numpy()
        assert np.array_equal(rb.topk_ids.cpu().numpy(), ids)
        d = np.abs(got - eager).max()
        assert d <= 2 ** -7 * np.abs(eager).max(), f"replay {rep}: {d}"
        assert_output_close(got, ref, f"replay {rep}")
        (xx @ xx).sum().item()  # eager work between replays
