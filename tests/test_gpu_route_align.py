"""moe_route_align on the GPU against the oracle: integers bit-exact, weights
to 2e-6, on every workload, every block_m, every launch shape (fused for
M <= 16; above, the top-k kernel and a one-workgroup grouping kernel, or from
4096 assignments a grid of grouping workgroups), constructed ties and load
extremes."""
import numpy as np
import pytest
import torch

import int4_weight_only_moe_amd as moe
import workloads as wl
from gpu_common import assert_route_matches, route_host, to_dev

pytestmark = pytest.mark.gpu


def run_route(logits: np.ndarray, k: int, block_m: int):
    M, E = logits.shape
    rb = moe.alloc_route_buffers(M, E, k, block_m)
    moe.route_align(to_dev(logits), rb)
    return rb, route_host(rb)


@pytest.mark.parametrize("name", list(wl.WORKLOADS))
@pytest.mark.parametrize("block_m", [16, 32, 64, 128])
def test_workloads(name, block_m):
    w = wl.WORKLOADS[name]
    t = wl.workload_tokens(w)
    print(f"route_align {name} M={w.M} block_m={block_m}", flush=True)
    _, got = run_route(t.logits, w.shape.k, block_m)
    assert_route_matches(got, t.logits, w.shape.E, w.shape.k, block_m)


@pytest.mark.parametrize("E,k,M", [(5, 5, 3), (64, 4, 17), (65, 16, 40), (130, 3, 16), (300, 8, 200),
                                   (1000, 12, 33), (1024, 16, 1), (1024, 1, 700), (8, 2, 2000),
                                   # the grid grouping kernel (from 4096 assignments): a last segment of
                                   # two assignments, E = 1024, an odd E, segments longer than 2048
                                   # (more than 256 * 2048 assignments)
                                   (8, 2, 2049), (1024, 16, 700), (100, 5, 1000), (64, 8, 70000)])
def test_shapes_cover_every_lane_width(E, k, M):
    rng = np.random.default_rng(E * 7 + M)
    logits = rng.standard_normal((M, E)).astype(np.float32)
    for block_m in (16, 64, 128):
        print(f"route_align E={E} k={k} M={M} block_m={block_m}", flush=True)
        _, got = run_route(logits, k, block_m)
        assert_route_matches(got, logits, E, k, block_m)


def test_ties_and_signed_zero():
    E, k = 384, 8
    rows = [np.zeros(E, np.float32),                                      # all equal
            np.where(np.arange(E) % 3 == 0, 1.0, -1.0).astype(np.float32),  # many ties at the boundary
            np.full(E, -5.0, np.float32)]
    r = np.full(E, -1.0, np.float32)
    r[[7, 100, 383]] = 0.0
    r[[3, 250]] = -0.0
    rows.append(r)                                                      # -0.0 ties with +0.0
    r2 = np.full(E, -2.0, np.float32)
    r2[::37] = 0.5
    rows.append(r2)
    logits = np.stack(rows * 5)
    for M in (len(rows), logits.shape[0]):  # fused and two-kernel paths
        _, got = run_route(logits[:M], k, 16)
        assert_route_matches(got, logits[:M], E, k, 16)


def test_single_hot_expert_and_block_boundaries():
    E, k = 64, 2
    rng = np.random.default_rng(5)
    for M in (16, 17, 32, 33, 100):   # counts exactly B, B+1, 2B, 2B+1 for the hot expert
        logits = rng.standard_normal((M, E)).astype(np.float32)
        logits[:, 9] += 100.0          # expert 9 is every token's first choice
        for block_m in (16, 32):
            _, got = run_route(logits, k, block_m)
            assert_route_matches(got, logits, E, k, block_m)


def test_deterministic_integers():
    w = wl.WORKLOADS["k26_m1024_skew"]
    t = wl.workload_tokens(w)
    rb = moe.alloc_route_buffers(w.M, w.shape.E, w.shape.k, 32)
    lg = to_dev(t.logits)
    moe.route_align(lg, rb)
    first = route_host(rb)
    for _ in range(100):
        rb.sorted_token_ids.fill_(-7)
        moe.route_align(lg, rb)
        again = route_host(rb)
        for key in ("topk_ids", "expert_offsets", "sorted_token_ids", "block_expert_ids"):
            np.testing.assert_array_equal(again[key], first[key])
        np.testing.assert_array_equal(again["topk_weights"], first["topk_weights"])


@pytest.mark.parametrize("name", ["k26_m90", "k26_m2048"])  # one-workgroup and grid grouping
def test_guard_bands_untouched(name):
    w = wl.WORKLOADS[name]
    t = wl.workload_tokens(w)
    E, k, B, M = w.shape.E, w.shape.k, 16, w.M
    cap = moe.moe_route_align_capacity(M, E, k, B)
    G = 64
    canary = -123456789

    def guarded(n):
        return torch.full((n + 2 * G,), canary, dtype=torch.int32, device="cuda")

    ids, srt, blk, off, npp = guarded(M * k), guarded(cap), guarded(cap // B), guarded(E + 1), guarded(1)
    wts = torch.full((M * k + 2 * G,), -3.5, dtype=torch.float32, device="cuda")
    moe.moe_route_align(to_dev(t.logits), k, B, ids[G:G + M * k], wts[G:G + M * k], srt[G:G + cap],
                        blk[G:G + cap // B], off[G:G + E + 1], npp[G:G + 1], cap=cap)
    torch.cuda.synchronize()
    for buf in (ids, srt, blk, off, npp):
        h = buf.cpu().numpy()
        assert np.all(h[:G] == canary) and np.all(h[-G:] == canary)
    hw = wts.cpu().numpy()
    assert np.all(hw[:G] == -3.5) and np.all(hw[-G:] == -3.5)


def test_empty_batch_is_a_no_op():
    rb = moe.alloc_route_buffers(0, 8, 2, 16)
    rb.num_tokens_post_pad.fill_(77)
    moe.route_align(torch.empty((0, 8), dtype=torch.float32, device="cuda"), rb)
    torch.cuda.synchronize()
    assert int(rb.num_tokens_post_pad.item()) == 77
