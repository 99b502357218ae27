"""moe_w4a16_layer_noalloc (the library's static scratch as the workspace)
against moe_w4a16_layer with a caller workspace: two calls in a row on each
path (the second with a smaller batch, so the scratch holds the first call's
contents), integers identical, outputs within the oracle bar of each other
and of the oracle; a batch too large for the scratch is refused before any
launch."""
import numpy as np
import pytest
import torch

import int4_weight_only_moe_amd as moe
import oracle
import workloads as wl
from gpu_common import assert_output_close, device_layer, oracle_experts, route_host, to_dev, x_device

pytestmark = pytest.mark.gpu

CASES = [
    # (shape, weight seed, batch sizes in call order): grouped block kernels,
    # per-token FC2, the decode path, the routed FC1, the tiled kernels
    (wl.LayerShape(E=64, H=1024, I=384, k=6), 3, (64, 16)),
    (wl.LayerShape(E=64, H=1024, I=384, k=6), 3, (5, 1)),
    (wl.LayerShape(E=8, H=256, I=256, k=2), 11, (300, 70)),
]


def _call(layer, logits, x_bits, block_m, noalloc):
    s = layer.shape
    M = logits.shape[0]
    rb = moe.alloc_route_buffers(M, s.E, s.k, block_m)
    out = torch.full((M, s.H), -3.0, dtype=torch.bfloat16, device="cuda")
    lg, x = to_dev(logits), x_device(x_bits)
    if noalloc:
        moe.moe_w4a16_layer_noalloc(lg, x, s.I, s.k, block_m, rb.topk_ids, rb.topk_weights, rb.sorted_token_ids,
                                    rb.block_expert_ids, rb.expert_offsets, rb.num_tokens_post_pad, layer.w13,
                                    layer.w2, out, cap=rb.cap)
    else:
        moe.layer(lg, x, rb, s.I, layer.w13, layer.w2, out=out)
    torch.cuda.synchronize()
    return route_host(rb), out.float().cpu().numpy()


@pytest.mark.parametrize("case", range(len(CASES)))
def test_noalloc_matches_layer(case):
    shape, seed, sizes = CASES[case]
    layer = device_layer(shape, seed)
    experts = oracle_experts(shape, seed)
    for M in sizes:
        print(f"noalloc {shape} M={M}", flush=True)
        t = wl.tokens(shape, M, 900 + M)
        block_m = moe.moe_w4a16_preferred_block_m(M, shape.E, shape.H, shape.I, shape.k)
        r_ref, o_ref = _call(layer, t.logits, t.x_bits, block_m, noalloc=False)
        r_na, o_na = _call(layer, t.logits, t.x_bits, block_m, noalloc=True)
        for key in ("topk_ids", "expert_offsets", "sorted_token_ids", "block_expert_ids"):
            np.testing.assert_array_equal(r_na[key], r_ref[key], err_msg=key)
        assert r_na["num_tokens_post_pad"] == r_ref["num_tokens_post_pad"]
        np.testing.assert_array_equal(r_na["topk_weights"], r_ref["topk_weights"])
        assert np.all(np.isfinite(o_na))
        assert_output_close(o_na, o_ref.astype(np.float64), f"noalloc vs layer M={M}")
        if M == 1:  # the decode path is deterministic: identical bits
            assert np.array_equal(o_na, o_ref)
        ids, w = oracle.route(t.logits, shape.k)
        ref = oracle.moe_forward(wl.f32_from_bf16_bits(t.x_bits).astype(np.float64), ids, w, experts)
        assert_output_close(o_na, ref, f"noalloc vs oracle M={M}")


def test_noalloc_refuses_a_batch_beyond_the_scratch():
    shape = wl.LayerShape(E=8, H=256, I=128, k=2)
    M = 40000
    assert moe.moe_w4a16_workspace_bytes(M, shape.E, shape.H, shape.I, shape.k) > moe.NOALLOC_SCRATCH_BYTES
    layer = device_layer(shape, 0)
    rb = moe.alloc_route_buffers(M, shape.E, shape.k, 64)
    lg = torch.zeros((M, shape.E), dtype=torch.float32, device="cuda")
    x = torch.zeros((M, shape.H), dtype=torch.bfloat16, device="cuda")
    out = torch.full((M, shape.H), 5.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_w4a16_layer_noalloc(lg, x, shape.I, shape.k, 64, rb.topk_ids, rb.topk_weights, rb.sorted_token_ids,
                                    rb.block_expert_ids, rb.expert_offsets, rb.num_tokens_post_pad, layer.w13,
                                    layer.w2, out, cap=rb.cap)
    assert ei.value.status == moe.MOE_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((out == 5.0).all())  # nothing was launched
