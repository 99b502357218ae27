"""Pins of the CPU oracle against things other than itself.

Each test fixes a part of the oracle with hand-worked values (tests/golden),
brute force on tiny inputs, closed forms, an independent formulation, or an
invariance, chosen so that a plausible slip (swapped nibbles, a wrong scale
group, gate/up swapped, a wrong tie rule, a transposed operand, a dropped
routing weight) fails at least one of them.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as wl


def load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------- O1, O2
def test_unpack_hand_packed(golden_dir):
    g = load(golden_dir, "nibbles.json")
    for case in g["cases"]:
        q = oracle.unpack_int4(np.array([case["bytes"]], np.uint8))[0]
        assert q.tolist() == case["q"], case["why"]


def test_dequant_hand_packed(golden_dir):
    g = load(golden_dir, "nibbles.json")
    for case in g["dequant"]:
        qb = np.zeros((1, 16), np.uint8)  # one group of 32 channels
        qb[0, : len(case["bytes"])] = case["bytes"]
        s = np.array([[case["scale_f16_bits"]]], np.uint16).view(np.float16)
        assert float(s[0, 0]) == case["scale"]
        W = oracle.dequantize(qb, s)[0]
        assert W[: len(case["W"])].tolist() == case["W"]


def test_dequant_group_boundary(golden_dir):
    gb = load(golden_dir, "nibbles.json")["group_boundary"]
    qb = np.full((1, gb["K"] // 2), gb["byte"], np.uint8)
    s = np.array([gb["scale_f16_bits"]], np.uint16).view(np.float16)
    W = oracle.dequantize(qb, s)[0]
    assert W[0] == gb["W_first"]
    assert W[31] == gb["W_last_of_group0"]
    assert W[32] == gb["W_first_of_group1"]
    assert np.all(W[:32] == W[0]) and np.all(W[32:] == W[32])


def test_dequant_matches_bytewise_brute_force():
    rng = np.random.default_rng(7)
    qb = rng.integers(0, 256, (3, 48), dtype=np.uint8)
    s = rng.uniform(0.005, 0.02, (3, 3)).astype(np.float16)
    W = oracle.dequantize(qb, s)
    for n in range(3):
        for c in range(96):
            byte = int(qb[n, c // 2])
            nib = (byte & 15) if c % 2 == 0 else (byte >> 4)
            assert W[n, c] == (nib - 8) * float(s[n, c // 32])


# ----------------------------------------------------------------- O3
def test_route_hand_rows(golden_dir):
    for case in load(golden_dir, "routing.json")["cases"]:
        L = np.array([case["logits"]], np.float32)
        ids, w = oracle.route(L, case["k"])
        assert ids[0].tolist() == case["ids"], case["why"]
        np.testing.assert_allclose(w[0], case["w"], rtol=0, atol=case["tol"])


def _brute_topk(row, k):
    """All C(E, k) subsets: keep the max exact sum, ties to the smallest index list."""
    best, best_key = None, None
    for sub in itertools.combinations(range(len(row)), k):
        key = (sum(Fraction(float(row[e])) for e in sub), tuple(-e for e in sub))
        if best_key is None or key > best_key:
            best, best_key = sub, key
    return sorted(best, key=lambda e: (-float(row[e]), e))


def _softmax_topk_renorm(row, ids):
    z = np.asarray(row, np.float64)
    p = np.exp(z - z.max())
    p /= p.sum()
    kept = p[list(ids)]
    return kept / kept.sum()


@pytest.mark.parametrize("k", [1, 2, 3])
def test_route_brute_force_tiny(k):
    t = wl.workload_tokens(wl.WORKLOADS["tiny"])
    L = t.logits
    # add rows with ties at the k-th boundary
    L = np.concatenate([L, np.array([[1, 1, 1, 1, 0, 0, 0, 0], [0.5, 2, 0.5, 0.5, 2, -1, 0.5, 3]], np.float32)])
    ids, w = oracle.route(L, k)
    for t_ in range(L.shape[0]):
        want = _brute_topk(L[t_], k)
        assert ids[t_].tolist() == want
        np.testing.assert_allclose(w[t_], _softmax_topk_renorm(L[t_], want), rtol=1e-12, atol=0)
        assert abs(w[t_].sum() - 1.0) < 1e-12


# ----------------------------------------------------------------- O4
def test_align_hand(golden_dir):
    for case in load(golden_dir, "align.json")["cases"]:
        a = oracle.align(np.array(case["topk_ids"]), case["E"], case["block_m"])
        for key in ("counts", "expert_offsets", "sorted_token_ids", "block_expert_ids"):
            assert a[key].tolist() == case[key], (key, case["why"])
        assert a["num_tokens_post_pad"] == case["num_tokens_post_pad"]


@pytest.mark.parametrize("E,k,M,B", [(8, 2, 16, 16), (8, 2, 16, 4), (384, 8, 90, 32), (5, 5, 7, 2), (64, 4, 300, 64)])
def test_align_invariants_and_argsort(E, k, M, B):
    rng = np.random.default_rng(E * 1000 + M)
    L = rng.standard_normal((M, E)).astype(np.float32)
    ids, _ = oracle.route(L, k)
    a = oracle.align(ids, E, B)
    flat = ids.reshape(-1)
    counts, off, npp = a["counts"], a["expert_offsets"], a["num_tokens_post_pad"]
    s, blk = a["sorted_token_ids"], a["block_expert_ids"]
    assert counts.sum() == M * k
    assert np.all(off % B == 0) and off[0] == 0 and off[-1] == npp
    real = s[s < M * k]
    assert sorted(real.tolist()) == list(range(M * k))
    assert (s == M * k).sum() == npp - M * k
    assert np.all(np.diff(blk) >= 0) and len(blk) == npp // B
    # brute force: a stable argsort of the flat expert ids, regrouped with padding
    order = np.argsort(flat, kind="stable")
    pos = 0
    for e in range(E):
        lst = order[pos: pos + counts[e]]
        pos += counts[e]
        seg = s[off[e]: off[e + 1]]
        assert seg[: counts[e]].tolist() == lst.tolist()
        assert np.all(seg[counts[e]:] == M * k)
        assert np.all(blk[off[e] // B: off[e + 1] // B] == e)
    # capacity bound used to size the buffers
    assert npp <= M * k + min(E, M * k) * (B - 1)


# ----------------------------------------------------------------- O5 - O7
def _const_expert(shape, byte=0x99, scale_bits=0x2000):
    H, I = shape.H, shape.I
    w13 = np.full((2 * I, H // 2), byte, np.uint8)
    s13 = np.full((2 * I, H // 32), scale_bits, np.uint16).view(np.float16)
    w2 = np.full((H, I // 2), byte, np.uint8)
    s2 = np.full((H, I // 32), scale_bits, np.uint16).view(np.float16)
    return w13, s13, w2, s2


@pytest.mark.parametrize("shape,expect", [(wl.TINY, 2.0 / (1 + math.exp(-2.0)) * 2.0), (wl.K26, 50176.0)])
def test_closed_form_constant_weights(shape, expect):
    """q = +1, s = 2^-7, x = 1: gate = up = H/128, y = (I/128) silu(H/128) (H/128), sum w = 1."""
    cache = oracle.DequantCache(lambda e: _const_expert(shape), max_items=1)
    const = cache(0)
    M = 2
    x = np.ones((M, shape.H))
    rng = np.random.default_rng(3)
    L = rng.standard_normal((M, shape.E)).astype(np.float32)
    out, ids, w = oracle.layer(x, L, shape.k, lambda e: const)
    I, H = shape.I, shape.H
    closed = (I / 128) * (H / 128) / (1 + math.exp(-H / 128)) * (H / 128)
    assert closed == pytest.approx(expect, rel=1e-15)
    np.testing.assert_allclose(out, closed, rtol=1e-13, atol=0)


def _tiny_expert_fn(seed=0):
    shape = wl.TINY
    return oracle.DequantCache(lambda e: tuple(vars(wl.expert_weights(shape, seed, e)).values()))


def test_dense_masked_formulation_tiny():
    """out = G @ [MLP_e(x)]_e with a dense [M, E] gate matrix (no sort, no pad)."""
    shape = wl.TINY
    t = wl.workload_tokens(wl.WORKLOADS["tiny"])
    x = wl.f32_from_bf16_bits(t.x_bits).astype(np.float64)
    experts = _tiny_expert_fn()
    out, _, _ = oracle.layer(x, t.logits, shape.k, experts)
    # independent gate matrix: full softmax, zero all but the k largest (stable), renormalise
    z = t.logits.astype(np.float64)
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    keep = np.argsort(-t.logits, axis=1, kind="stable")[:, : shape.k]
    G = np.zeros_like(p)
    np.put_along_axis(G, keep, np.take_along_axis(p, keep, 1), 1)
    G /= G.sum(axis=1, keepdims=True)
    # every expert on every token, through torch (independent of the oracle's MLP code)
    Y = np.zeros((shape.E, x.shape[0], shape.H))
    for e in range(shape.E):
        W13, W2 = experts(e)
        h = torch.from_numpy(x) @ torch.from_numpy(W13).T
        a = torch.nn.functional.silu(h[:, : shape.I]) * h[:, shape.I:]
        Y[e] = (a @ torch.from_numpy(W2).T).numpy()
    dense = np.einsum("te,teh->th", G, Y.transpose(1, 0, 2))
    np.testing.assert_allclose(out, dense, rtol=1e-12, atol=1e-12)


def test_k1_single_expert_is_textbook_swiglu():
    """k = 1, one expert: the layer is y = W2 (silu(Wg x) * (Wu x)) with weight 1."""
    shape = wl.LayerShape(E=1, H=256, I=128, k=1)
    ew = wl.expert_weights(shape, 11, 0)
    x = wl.f32_from_bf16_bits(wl.bf16_bits_from_f32(np.random.default_rng(1).standard_normal((5, 256)).astype(np.float32))).astype(np.float64)
    L = np.zeros((5, 1), np.float32)
    cache = oracle.DequantCache(lambda e: (ew.w13, ew.s13, ew.w2, ew.s2))
    out, ids, w = oracle.layer(x, L, 1, cache)
    assert np.all(ids == 0) and np.all(w == 1.0)
    # textbook SwiGLU with torch, weights dequantised bytewise right here
    def deq(qb, s):
        qb = torch.from_numpy(qb.astype(np.int64))
        q = torch.stack([(qb & 15) - 8, (qb >> 4) - 8], dim=-1).reshape(qb.shape[0], -1).double()
        return q * torch.from_numpy(s.astype(np.float64)).repeat_interleave(32, dim=1)
    W13, W2 = deq(ew.w13, ew.s13), deq(ew.w2, ew.s2)
    Wg, Wu = W13[:128], W13[128:]
    xt = torch.from_numpy(x)
    y = torch.nn.functional.linear(torch.nn.functional.silu(torch.nn.functional.linear(xt, Wg)) * torch.nn.functional.linear(xt, Wu), W2)
    np.testing.assert_allclose(out, y.numpy(), rtol=1e-12, atol=1e-12)


def test_identical_experts_ignore_logits():
    shape = wl.TINY
    ew = wl.expert_weights(shape, 5, 0)
    cache = oracle.DequantCache(lambda e: (ew.w13, ew.s13, ew.w2, ew.s2), max_items=1)
    W = cache(0)
    t = wl.workload_tokens(wl.WORKLOADS["tiny"])
    x = wl.f32_from_bf16_bits(t.x_bits).astype(np.float64)
    out1, _, _ = oracle.layer(x, t.logits, 2, lambda e: W)
    out2, _, _ = oracle.layer(x, -3.0 * t.logits, 2, lambda e: W)
    single = np.stack([oracle.expert_mlp(x[i], *W) for i in range(x.shape[0])])
    np.testing.assert_allclose(out1, single, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out2, single, rtol=1e-12, atol=1e-12)


def test_expert_permutation_invariance():
    shape = wl.TINY
    experts = _tiny_expert_fn()
    t = wl.workload_tokens(wl.WORKLOADS["tiny"])
    x = wl.f32_from_bf16_bits(t.x_bits).astype(np.float64)
    out, ids, w = oracle.layer(x, t.logits, 2, experts)
    pi = np.random.default_rng(9).permutation(shape.E)  # new index of old expert e is pi[e]
    inv = np.argsort(pi)
    Lp = np.empty_like(t.logits)
    Lp[:, pi] = t.logits
    out_p, ids_p, w_p = oracle.layer(x, Lp, 2, lambda e: experts(int(inv[e])))
    assert np.array_equal(ids_p, pi[ids])
    assert np.array_equal(w_p, w)
    assert np.array_equal(out_p, out)


def test_zero_tokens_and_empty_batch():
    shape = wl.TINY
    experts = _tiny_expert_fn()
    L = np.random.default_rng(2).standard_normal((4, shape.E)).astype(np.float32)
    out, _, _ = oracle.layer(np.zeros((4, shape.H)), L, 2, experts)
    assert np.all(out == 0.0)
    out0, ids0, w0 = oracle.layer(np.zeros((0, shape.H)), np.zeros((0, shape.E), np.float32), 2, experts)
    assert out0.shape == (0, shape.H) and ids0.shape == (0, 2)


def test_w2_scale_doubling_doubles_output():
    shape = wl.TINY
    t = wl.workload_tokens(wl.WORKLOADS["tiny"])
    x = wl.f32_from_bf16_bits(t.x_bits).astype(np.float64)

    def get(e, mul):
        ew = wl.expert_weights(shape, 0, e)
        return ew.w13, ew.s13, ew.w2, (ew.s2.astype(np.float32) * mul).astype(np.float16)

    out1, _, _ = oracle.layer(x, t.logits, 2, oracle.DequantCache(lambda e: get(e, 1)))
    out2, _, _ = oracle.layer(x, t.logits, 2, oracle.DequantCache(lambda e: get(e, 2)))
    assert np.array_equal(out2, 2 * out1)


def test_gate_up_order_matters():
    """Swapping the gate and up halves changes the result (guards the W13 row reading)."""
    shape = wl.TINY
    ew = wl.expert_weights(shape, 0, 0)
    W13, W2 = oracle.dequantize(ew.w13, ew.s13), oracle.dequantize(ew.w2, ew.s2)
    x = np.linspace(-1, 1, shape.H)
    a = oracle.expert_mlp(x, W13, W2)
    b = oracle.expert_mlp(x, np.concatenate([W13[shape.I:], W13[: shape.I]]), W2)
    assert not np.allclose(a, b)
    h = W13 @ x
    np.testing.assert_allclose(a, W2 @ (h[: shape.I] / (1 + np.exp(-h[: shape.I])) * h[shape.I:]), rtol=1e-14)


def test_workload_recipe_pins(golden_dir):
    """The seeded inputs follow the written recipe, and the oracle's routing and
    grouping of them match values derived independently from that recipe."""
    g = load(golden_dir, "recipe.json")
    t = wl.workload_tokens(wl.WORKLOADS["tiny"])
    ids, w = oracle.route(t.logits, wl.TINY.k)
    T = g["tiny"]
    assert ids[:4].tolist() == T["ids_rows_0_3"]
    assert np.bincount(ids.reshape(-1), minlength=wl.TINY.E).tolist() == T["counts"]
    assert np.allclose(w[0], T["w_row0"], atol=1e-8)
    assert [format(int(v), "04x") for v in t.x_bits[0, :4]] == T["x_bits_row0"]
    assert oracle.align(ids, wl.TINY.E, 16)["num_tokens_post_pad"] == T["npp_b16"]
    for name, p in g["k26"].items():
        tt = wl.workload_tokens(wl.WORKLOADS[name])
        ids, _ = oracle.route(tt.logits, wl.K26.k)
        counts = np.bincount(ids.reshape(-1), minlength=wl.K26.E)
        assert int((counts > 0).sum()) == p["D"], name
        assert int(counts.max()) == p["max"], name
        assert oracle.align(ids, wl.K26.E, 32)["num_tokens_post_pad"] == p["npp_b32"], name
        if "ids_row0" in p:
            assert ids[0].tolist() == p["ids_row0"], name
