"""Helpers shared by the GPU tests: device copies of the seeded inputs, the
HIP path through the binding, and oracle references on the CPU."""
from __future__ import annotations

import functools
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import int4_weight_only_moe_amd as moe
import oracle
import workloads as wl

DEV = "cuda"


def to_dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(DEV)


def x_device(x_bits: np.ndarray) -> torch.Tensor:
    return to_dev(x_bits.view(np.int16)).view(torch.bfloat16)


class DeviceLayer:
    """Repacked weights of one layer on the device (fmt "int4" or "mxfp4")."""

    def __init__(self, shape: wl.LayerShape, w13, s13, w2, s2, fmt: str = "int4"):
        self.shape = shape
        self.fmt = fmt
        q13, q2 = to_dev(w13), to_dev(w2)
        if fmt == "mxfp4":
            sc13, sc2 = to_dev(s13), to_dev(s2)
            self.w13 = moe.repack_mxfp4(q13, sc13, moe.KIND_W13)
            self.w2 = moe.repack_mxfp4(q2, sc2, moe.KIND_W2)
        else:
            sc13 = to_dev(s13.view(np.uint16)).view(torch.float16)
            sc2 = to_dev(s2.view(np.uint16)).view(torch.float16)
            self.w13 = moe.repack(q13, sc13, moe.KIND_W13)
            self.w2 = moe.repack(q2, sc2, moe.KIND_W2)
        torch.cuda.synchronize()
        del q13, q2, sc13, sc2


def device_layer(shape: wl.LayerShape, seed: int, fmt: str = "int4") -> DeviceLayer:
    return DeviceLayer(shape, *wl.layer_weights(shape, seed, fmt=fmt), fmt=fmt)


def oracle_experts(shape: wl.LayerShape, seed: int, keep: int = 64, fmt: str = "int4"):
    def get(e):
        ew = wl.expert_weights(shape, seed, e, fmt)
        return ew.w13, ew.s13, ew.w2, ew.s2
    return oracle.DequantCache(get, max_items=keep, fmt=fmt)


def run_layer(layer: DeviceLayer, logits: np.ndarray, x_bits: np.ndarray, block_m: int):
    """route_align + forward on the device; returns (route buffers, out bf16 as float32 numpy)."""
    s = layer.shape
    M = logits.shape[0]
    rb = moe.alloc_route_buffers(M, s.E, s.k, block_m)
    moe.route_align(to_dev(logits), rb)
    out = moe.forward(x_device(x_bits), rb, s.I, layer.w13, layer.w2, fmt=layer.fmt)
    torch.cuda.synchronize()
    return rb, out.float().cpu().numpy()


def route_host(rb: moe.RouteBuffers) -> dict:
    torch.cuda.synchronize()
    npp = int(rb.num_tokens_post_pad.item())
    return {
        "topk_ids": rb.topk_ids.cpu().numpy(),
        "topk_weights": rb.topk_weights.cpu().numpy(),
        "expert_offsets": rb.expert_offsets.cpu().numpy(),
        "num_tokens_post_pad": npp,
        "sorted_token_ids": rb.sorted_token_ids.cpu().numpy()[:npp],
        "block_expert_ids": rb.block_expert_ids.cpu().numpy()[: npp // rb.block_m],
    }


def assert_route_matches(got: dict, logits: np.ndarray, E: int, k: int, block_m: int):
    ids, w = oracle.route(logits, k)
    al = oracle.align(ids, E, block_m)
    np.testing.assert_array_equal(got["topk_ids"], ids)
    np.testing.assert_allclose(got["topk_weights"], w, rtol=0, atol=2e-6)
    assert got["num_tokens_post_pad"] == al["num_tokens_post_pad"]
    np.testing.assert_array_equal(got["expert_offsets"], al["expert_offsets"])
    np.testing.assert_array_equal(got["sorted_token_ids"], al["sorted_token_ids"])
    np.testing.assert_array_equal(got["block_expert_ids"], al["block_expert_ids"])
    return ids, w


def output_errors(got: np.ndarray, ref: np.ndarray):
    """(rel-L2, max abs error, max-abs bound) of the bf16 output against the oracle.

    The bound is 3e-2 * max(1, rms(ref)): the absolute 3e-2 taken relative to the
    output's scale (the bf16 rounding of an output of rms ~23 alone is ~0.06).
    """
    d = got.astype(np.float64) - ref
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-30))
    mx = float(np.abs(d).max()) if d.size else 0.0
    bound = 3e-2 * max(1.0, float(np.sqrt(np.mean(ref ** 2))) if ref.size else 1.0)
    return rel, mx, bound


def assert_output_close(got: np.ndarray, ref: np.ndarray, what: str = ""):
    rel, mx, bound = output_errors(got, ref)
    print(f"parity {what}: rel-L2 {rel:.3e} (<= 5e-3), max abs {mx:.3e} (<= {bound:.3e})", flush=True)
    assert rel <= 5e-3, f"{what}: rel-L2 {rel:.3e} > 5e-3"
    assert mx <= bound, f"{what}: max abs {mx:.3e} > {bound:.3e}"
    return rel, mx


@functools.lru_cache(maxsize=None)
def k26_layer() -> DeviceLayer:
    """The 384-expert layer (9.5 GB of weights), generated and repacked once per session."""
    return device_layer(wl.K26, 2026)


@functools.lru_cache(maxsize=None)
def k26_mxfp4_layer() -> DeviceLayer:
    """The 384-expert layer with MXFP4 weights (9.0 GB), generated and repacked once per session."""
    return device_layer(wl.K26, 2026, fmt="mxfp4")


def covering_rows(ids: np.ndarray, must=()) -> list:
    """Token rows that together hold every expert the batch routes to, chosen
    greedily (each pick the row with the most experts not yet held), plus the
    rows in ``must``; ascending."""
    E = int(ids.max()) + 1
    inc = np.zeros((ids.shape[0], E), bool)
    inc[np.arange(ids.shape[0])[:, None], ids] = True
    rows = set(int(r) for r in must)
    left = inc.any(axis=0)
    for r in rows:
        left &= ~inc[r]
    while left.any():
        r = int(np.argmax(inc[:, left].sum(axis=1)))
        rows.add(r)
        left &= ~inc[r]
    return sorted(rows)


def tile_rows_of_hot_experts(ids: np.ndarray, tile_rows: int, stride: int = 64) -> list:
    """Tokens in every tile of each expert holding more than one tile: the
    expert's assignments in ascending f, one every `stride` entries. The
    tiled kernel cuts such an expert into tiles of equal whole-block size,
    at least two 32-row blocks each, so a stride of 64 lands in every tile."""
    k = ids.shape[1]
    flat = ids.reshape(-1)
    rows = []
    for e in np.unique(flat):
        fs = np.nonzero(flat == e)[0]
        if fs.size > tile_rows:
            rows += [int(fs[i] // k) for i in range(0, fs.size, stride)]
    return rows


def oracle_rows_parallel(shape: wl.LayerShape, seed: int, x: np.ndarray, ids: np.ndarray, w: np.ndarray,
                         rows: list, fmt: str = "int4") -> np.ndarray:
    """The oracle's output for the given token rows, its per-expert work run
    on the host's cores (each worker generates and dequantises one expert)."""
    from threadpoolctl import threadpool_limits

    def experts(e):
        ew = wl.expert_weights(shape, seed, e, fmt)
        dq = oracle.DEQUANT[fmt]
        return dq(ew.w13, ew.s13), dq(ew.w2, ew.s2)

    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with threadpool_limits(limits=1), ThreadPoolExecutor(workers) as pool:
        y = oracle.expert_outputs(x, ids, experts, rows, map_fn=pool.map)
    return oracle.combine(w, y, x.shape[0], x.shape[1], rows)
