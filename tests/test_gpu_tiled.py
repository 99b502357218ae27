"""The tiled grouped GEMM, which the forward takes once experts average at
least 16 assignments (and every pair group and K-chunk count divides
evenly): the pre-scaled kernel (tiles of up to 128 rows of whole blocks,
cut per expert). Every element against the oracle on shapes
whose experts hold from one small tile up to several full tiles, with
partial tiles of every sub-tile count, all block sizes, and skewed routing
(a per-expert logit bias) that piles hundreds of rows onto a few experts."""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_common import assert_output_close, assert_route_matches, device_layer, oracle_experts, route_host, run_layer

pytestmark = pytest.mark.gpu

SMALL = wl.LayerShape(E=8, H=256, I=256, k=2)
WIDER = wl.LayerShape(E=32, H=512, I=512, k=4)

TILED = [
    # (shape, M, bias sigma, weight seed, token seed)
    (SMALL, 64, 0.0, 11, 12),    # 16 assignments per expert: tiles of 1-2 sub-tiles
    (SMALL, 128, 0.0, 11, 17),   # 32 per expert: tiles of 2-3 sub-tiles
    (SMALL, 300, 0.0, 11, 13),   # ~75 per expert: one tile each, 4 to 6 sub-tiles
    (SMALL, 700, 2.0, 11, 14),   # skewed: several full tiles on the hot experts
    (WIDER, 320, 1.0, 15, 16),   # 40 per expert, mildly skewed
]


@pytest.mark.parametrize("case", range(len(TILED)))
@pytest.mark.parametrize("block_m", [16, 32, 64, 128])
def test_tiled_full_parity(case, block_m):
    shape, M, sigma, wseed, tseed = TILED[case]
    assert M * shape.k / shape.E >= 16
    print(f"tiled {shape} M={M} sigma={sigma} block_m={block_m}", flush=True)
    layer = device_layer(shape, wseed)
    t = wl.tokens(shape, M, tseed, sigma)
    rb, out = run_layer(layer, t.logits, t.x_bits, block_m)
    ids, w = assert_route_matches(route_host(rb), t.logits, shape.E, shape.k, block_m)
    counts = np.bincount(ids.reshape(-1), minlength=shape.E)
    print(f"tiled: rows per expert {sorted(counts.tolist(), reverse=True)[:6]}", flush=True)
    x = wl.f32_from_bf16_bits(t.x_bits).astype(np.float64)
    ref = oracle.moe_forward(x, ids, w, oracle_experts(shape, wseed))
    assert np.all(np.isfinite(out))
    assert_output_close(out, ref, f"tiled {shape} M={M} B={block_m}")


@pytest.mark.parametrize("block_m", [16, 32, 64, 128])
def test_tiled_at_the_size_limits(block_m):
    """1024 experts (the largest E) with top-16 (the largest k) at 16
    assignments per expert: the pre-scaled kernel with 1024 experts' tiles;
    every element of 12 token rows (173 of the experts) against the oracle."""
    shape = wl.LayerShape(E=1024, H=256, I=256, k=16)
    M = 1024
    assert M * shape.k / shape.E >= 16
    layer = device_layer(shape, 21)
    t = wl.tokens(shape, M, 22, 0.0)
    rb, out = run_layer(layer, t.logits, t.x_bits, block_m)
    ids, w = assert_route_matches(route_host(rb), t.logits, shape.E, shape.k, block_m)
    rows = list(range(0, M, M // 12))[:12]
    x = wl.f32_from_bf16_bits(t.x_bits).astype(np.float64)
    ref = oracle.moe_forward(x, ids, w, oracle_experts(shape, 21), tokens_subset=rows)
    assert np.all(np.isfinite(out))
    print(f"size limits B={block_m}: experts covered {np.unique(ids[rows]).size}/{np.unique(ids).size}", flush=True)
    assert_output_close(out[rows], ref[rows], f"E=1024 k=16 M={M} B={block_m}")


def test_tiled_skew_has_multi_tile_experts():
    """The skewed case really exercises experts of several 128-row tiles, and
    tiles whose last sub-tile is partial."""
    shape, M, sigma, _, tseed = TILED[3]
    t = wl.tokens(shape, M, tseed, sigma)
    ids, _ = oracle.route(t.logits, shape.k)
    counts = np.bincount(ids.reshape(-1), minlength=shape.E)
    assert counts.max() > 2 * 128
    assert any(c > 128 and c % 16 for c in counts)


def test_tiled_with_oversized_route_buffers():
    """Route buffers allocated for a much larger batch (cap far above the
    capacity of this one): the tiled grid and its tile table depend only on
    the batch, so the result is unchanged."""
    import int4_weight_only_moe_amd as moe
    import torch
    from gpu_common import to_dev, x_device
    shape, M, sigma, wseed, tseed = TILED[2]
    layer = device_layer(shape, wseed)
    t = wl.tokens(shape, M, tseed, sigma)
    for block_m in (16, 64):
        big = moe.alloc_route_buffers(40 * M, shape.E, shape.k, block_m)
        assert big.cap >= 20 * moe.moe_route_align_capacity(M, shape.E, shape.k, block_m)
        rb = moe.RouteBuffers(M, shape.E, shape.k, block_m, big.cap, big.topk_ids[:M], big.topk_weights[:M],
                              big.sorted_token_ids, big.block_expert_ids, big.expert_offsets,
                              big.num_tokens_post_pad)
        moe.route_align(to_dev(t.logits), rb)
        out = moe.forward(x_device(t.x_bits), rb, shape.I, layer.w13, layer.w2).float().cpu().numpy()
        torch.cuda.synchronize()
        ids, w = assert_route_matches(route_host(rb), t.logits, shape.E, shape.k, block_m)
        ref = oracle.moe_forward(wl.f32_from_bf16_bits(t.x_bits).astype(np.float64), ids, w,
                                 oracle_experts(shape, wseed))
        assert_output_close(out, ref, f"oversized cap B={block_m}")


def expected_tiles(block_expert, sorted_ids, npp, block_m, tile_rows, MK):
    """The tile list the plan must write: each expert's run of r blocks cut
    into n = ceil(r / bpt) tiles, tile j starting at block floor(j r / n) of
    the run; a tile's sub-tile count covers its real rows; the reuse flag
    marks experts of several tiles."""
    nblk, bpt = npp // block_m, tile_rows // block_m
    out = []
    b = 0
    while b < nblk:
        e, end = block_expert[b], b
        while end < nblk and block_expert[end] == e:
            end += 1
        r = end - b
        n = -(-r // bpt)
        for j in range(n):
            h, nb = b + j * r // n, (j + 1) * r // n - j * r // n
            assert 1 <= nb <= bpt
            nsub = nb * block_m // 16
            while nsub > 1 and sorted_ids[h * block_m + (nsub - 1) * 16] >= MK:
                nsub -= 1
            out.append((h * block_m, nsub | (16 if n > 1 else 0) | (int(e) << 8)))
        b = end
    return out


@pytest.mark.parametrize("case", [2, 3, 4])
@pytest.mark.parametrize("block_m", [16, 32, 64, 128])
def test_tile_plan_cuts_each_expert_into_equal_tiles(case, block_m):
    """White-box check of the tile table the forward leaves in its workspace
    (layout: fp32 accumulator, bf16 activations, tile count, tile table): one
    tile per expert of up to 128 rows, whatever the
    expert's offset in the padded list, longer experts in tiles of equal
    size, and every block in exactly one tile."""
    import int4_weight_only_moe_amd as moe
    import torch
    from gpu_common import to_dev, x_device
    shape, M, sigma, wseed, tseed = TILED[case]
    layer = device_layer(shape, wseed)
    t = wl.tokens(shape, M, tseed, sigma)
    rb = moe.alloc_route_buffers(M, shape.E, shape.k, block_m)
    moe.route_align(to_dev(t.logits), rb)
    ws = torch.zeros(moe.moe_w4a16_workspace_bytes(M, shape.E, shape.H, shape.I, shape.k), dtype=torch.uint8,
                     device="cuda")
    moe.forward(x_device(t.x_bits), rb, shape.I, layer.w13, layer.w2, workspace=ws)
    torch.cuda.synchronize()
    h = route_host(rb)

    def a256(v):
        return (v + 255) // 256 * 256
    ntiles_off = a256(M * shape.H * 4) + a256(M * shape.k * shape.I * 2)
    raw = ws.cpu().numpy()
    ntiles = int(raw[ntiles_off:ntiles_off + 4].view(np.int32)[0])
    table = raw[ntiles_off + 256:].view(np.int32)[:2 * ntiles].reshape(ntiles, 2)
    tile_rows = 128  # a multiple of every block size
    want = expected_tiles(h["block_expert_ids"], h["sorted_token_ids"], int(h["num_tokens_post_pad"]), block_m,
                          tile_rows, M * shape.k)
    assert [tuple(map(int, r)) for r in table] == want
    counts = np.bincount(h["topk_ids"].reshape(-1), minlength=shape.E)
    small = int(np.sum((counts > 0) & (counts <= tile_rows)))
    assert sum(1 for _, meta in want if not meta & 16) == small  # every such expert is one tile


def logits_with_counts(E: int, counts, seed: int) -> np.ndarray:
    """Top-2 logits that give expert e exactly counts[e] assignments (no count
    above half the total): the sorted multiset of experts, entry i paired with
    entry i + total / 2 (always a different expert), large logits for the pair,
    small noise elsewhere; tokens in random order."""
    rng = np.random.default_rng(seed)
    pool = np.repeat(np.arange(E), counts)
    half = pool.size // 2
    assert pool.size == 2 * half and max(counts) <= half
    pairs = np.stack([pool[:half], pool[half:]], axis=1)
    assert np.all(pairs[:, 0] != pairs[:, 1])
    pairs = pairs[rng.permutation(half)]
    logits = rng.uniform(-1.0, 0.0, (half, E)).astype(np.float32)
    top = (10.0 + rng.uniform(0.0, 1.0, (half, 2))).astype(np.float32)
    logits[np.arange(half)[:, None], pairs] = top
    return logits


# per-expert row counts at the tile-size edges: 128 (one tile), 129 (two),
# 256 and 257 (two and three), 16 (one full sub-tile), 1, 81, 0
EDGE_COUNTS = [129, 128, 257, 256, 16, 1, 81, 0]


@pytest.mark.parametrize("block_m", [16, 32, 64, 128])
def test_tile_edges_full_parity(block_m):
    """Experts of exactly one and just over one, two and three tiles: the
    tile table and every output element against the oracle."""
    import int4_weight_only_moe_amd as moe
    import torch
    from gpu_common import to_dev, x_device
    shape = SMALL
    logits = logits_with_counts(shape.E, EDGE_COUNTS, 31)
    M = logits.shape[0]
    x_bits = wl.tokens(shape, M, 32).x_bits
    layer = device_layer(shape, 11)
    rb = moe.alloc_route_buffers(M, shape.E, shape.k, block_m)
    moe.route_align(to_dev(logits), rb)
    ws = torch.zeros(moe.moe_w4a16_workspace_bytes(M, shape.E, shape.H, shape.I, shape.k), dtype=torch.uint8,
                     device="cuda")
    out = moe.forward(x_device(x_bits), rb, shape.I, layer.w13, layer.w2, workspace=ws).float().cpu().numpy()
    torch.cuda.synchronize()
    h = route_host(rb)
    ids, w = assert_route_matches(h, logits, shape.E, shape.k, block_m)
    np.testing.assert_array_equal(np.bincount(ids.reshape(-1), minlength=shape.E), EDGE_COUNTS)

    def a256(v):
        return (v + 255) // 256 * 256
    ntiles_off = a256(M * shape.H * 4) + a256(M * shape.k * shape.I * 2)
    raw = ws.cpu().numpy()
    ntiles = int(raw[ntiles_off:ntiles_off + 4].view(np.int32)[0])
    table = [tuple(map(int, r)) for r in raw[ntiles_off + 256:].view(np.int32)[:2 * ntiles].reshape(ntiles, 2)]
    assert table == expected_tiles(h["block_expert_ids"], h["sorted_token_ids"], int(h["num_tokens_post_pad"]),
                                   block_m, 128, M * shape.k)
    tiles_per_expert = np.bincount([meta >> 8 for _, meta in table], minlength=shape.E)
    np.testing.assert_array_equal(tiles_per_expert, [2, 1, 3, 2, 1, 1, 1, 0])
    ref = oracle.moe_forward(wl.f32_from_bf16_bits(x_bits).astype(np.float64), ids, w, oracle_experts(shape, 11))
    assert np.all(np.isfinite(out))
    assert_output_close(out, ref, f"tile edges B={block_m}")
