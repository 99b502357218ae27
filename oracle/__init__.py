"""Plain CPU oracle of the weight-only INT4 (group 32) MoE layer.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this package. The
product path (the HIP library and its Python binding) never reaches it and
fails loudly when its native library is missing.

What the layer computes comes from "The Throughput Lever: Quantifying the MoE
GEMM and Mapping the Road to B300":
  * section "Phase 3: The INT4 Marlin MoE Throughput Lever": the MoE layer is
    a grouped GEMM over the experts, run on a dense token batch;
  * section "Building the Benchmark": expert weights are INT4 with group size
    32 (GPTQ-style: one scale per 32 consecutive input channels);
  * section "The Result: Two Regimes": each token is routed to 8 of 384
    experts (top-8 routing) and the layer streams the weights of the experts
    that are touched.
The benchmark workload fixes the routing as softmax over the experts, top-k,
and renormalisation of the k kept weights, and the expert MLP as FC1
(gate/up) -> SiLU(gate) * up -> FC2, with the k expert outputs summed with
the routing weights. Where the pages leave a step open, the plainest reading
is taken; each reading is named in the function that uses it.

Everything floating-point here is float64. The dequantised weight q*s is exact
in float64 (a 4-bit integer times an 11-bit fp16 significand).

MXFP4 expert weights (``dequantize_mxfp4``) are the same layer with FP4
e2m1 weights and E8M0 scales.

Pins (what checks this oracle against something other than itself) live in
``tests/test_oracle_*.py``: hand-packed nibbles, brute-force routing,
argsort-based alignment, closed forms, a dense masked formulation, a textbook
SwiGLU MLP for k = 1, and invariances. No function here is "parity unpinned".
"""
from __future__ import annotations

from typing import Callable, Dict, Tuple

import numpy as np

GROUP = 32


# --------------------------------------------------------------------------
# O1, O2: INT4 unpack and group-32 dequantisation
# --------------------------------------------------------------------------
def unpack_int4(qweight: np.ndarray) -> np.ndarray:
    """Signed 4-bit values q in [-8, 7] from the canonical packed bytes.

    Reading of "Building the Benchmark" (GPTQ-format INT4): byte i of a row
    holds input channel 2i in its low nibble and 2i+1 in its high nibble,
    and a nibble u stands for q = u - 8 (zero point 8, symmetric range).
    Input uint8 [..., K/2]; output int16 [..., K].
    """
    qb = np.asarray(qweight, dtype=np.uint8)
    lo = (qb & 0x0F).astype(np.int16) - 8
    hi = (qb >> 4).astype(np.int16) - 8
    q = np.empty(qb.shape[:-1] + (2 * qb.shape[-1],), dtype=np.int16)
    q[..., 0::2] = lo
    q[..., 1::2] = hi
    return q


def dequantize(qweight: np.ndarray, scales_f16: np.ndarray, out: np.ndarray | None = None) -> np.ndarray:
    """W[n, c] = q[n, c] * s[n, c // 32] in float64 (group size 32 along K).

    "Building the Benchmark": INT4 weights with group size 32. Reading: one
    fp16 scale per (row, group of 32 channels), symmetric, no zero point
    beyond the offset of 8 in the nibble code (q = u - 8, as in unpack_int4).
    ``out`` (float64 [..., K]) may be passed to reuse memory; the values are
    written in place: the nibbles, minus 8, times the group's scale.
    """
    qb = np.asarray(qweight, dtype=np.uint8)
    s = np.asarray(scales_f16, dtype=np.float16).astype(np.float64)
    K = 2 * qb.shape[-1]
    if K != s.shape[-1] * GROUP:
        raise ValueError(f"K={K} does not match {s.shape[-1]} groups of {GROUP}")
    W = np.empty(qb.shape[:-1] + (K,), dtype=np.float64) if out is None else out
    pairs = W.reshape(qb.shape + (2,))
    np.bitwise_and(qb, 0x0F, out=pairs[..., 0], casting="unsafe")  # channel 2i: low nibble
    np.right_shift(qb, 4, out=pairs[..., 1], casting="unsafe")      # channel 2i+1: high nibble
    W -= 8.0
    groups = W.reshape(qb.shape[:-1] + (K // GROUP, GROUP))
    groups *= s[..., None]
    return W


# --------------------------------------------------------------------------
# O3: top-k routing
# --------------------------------------------------------------------------
def route(logits: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """Top-k experts per token and their renormalised softmax weights.

    "The Result: Two Regimes": each token activates 8 of the 384 experts via
    top-8 routing. The workload defines the weights as softmax over all
    experts, keep the k largest, renormalise them to sum 1.

    Readings:
      * selection is made on the float32 logits (softmax is monotone, so the
        set is the same in exact arithmetic);
      * ties go to the lower expert index, and -0.0 ties with +0.0;
      * slot j holds the (j+1)-th largest logit;
      * the full-softmax denominator cancels in the renormalisation, so
        w_j = exp(L_j - L_max) / sum_i exp(L_i - L_max) over the k kept
        logits, computed in float64.
    Returns topk_ids int32 [M, k] and topk_weights float64 [M, k].
    """
    L = np.asarray(logits, dtype=np.float32)
    M, E = L.shape
    if not 1 <= k <= E:
        raise ValueError("k must be in [1, E]")
    ids = np.empty((M, k), dtype=np.int32)
    w = np.empty((M, k), dtype=np.float64)
    for t in range(M):
        row = [float(v) + 0.0 for v in L[t]]  # -0.0 + 0.0 == +0.0
        order = sorted(range(E), key=lambda e: (-row[e], e))
        chosen = order[:k]
        ids[t] = chosen
        top = np.array([row[e] for e in chosen], dtype=np.float64)
        ex = np.exp(top - top[0])
        w[t] = ex / ex.sum()
    return ids, w


# --------------------------------------------------------------------------
# O4: per-expert token grouping (histogram, padded offsets, stable order)
# --------------------------------------------------------------------------
def align(topk_ids: np.ndarray, E: int, block_m: int):
    """Group the M*k assignments by expert, each group padded to block_m.

    The grouped GEMM of "Phase 3: The INT4 Marlin MoE Throughput Lever" runs
    each expert over the tokens routed to it; the workload asks for a
    per-expert histogram, a prefix sum, a permutation and padding of each
    expert's list to the tile size.

    Readings: assignment f = t*k + j; an expert's list is in ascending f
    (a stable counting sort); padding entries hold the sentinel M*k; experts
    with no token get no block.
    Returns dict with counts [E], expert_offsets [E+1], num_tokens_post_pad,
    sorted_token_ids [NPP], block_expert_ids [NPP/block_m].
    """
    ids = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    n_assign = ids.size
    counts = np.zeros(E, dtype=np.int64)
    for e in ids:
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        padded = -(-counts[e] // block_m) * block_m
        offsets[e + 1] = offsets[e] + padded
    npp = int(offsets[E])
    sorted_ids = np.full(npp, n_assign, dtype=np.int64)
    fill = offsets[:E].copy()
    for f in range(n_assign):
        e = ids[f]
        sorted_ids[fill[e]] = f
        fill[e] += 1
    blocks = np.empty(npp // block_m, dtype=np.int64)
    for e in range(E):
        blocks[offsets[e] // block_m: offsets[e + 1] // block_m] = e
    return {
        "counts": counts.astype(np.int32),
        "expert_offsets": offsets.astype(np.int32),
        "num_tokens_post_pad": npp,
        "sorted_token_ids": sorted_ids.astype(np.int32),
        "block_expert_ids": blocks.astype(np.int32),
    }


# --------------------------------------------------------------------------
# O5 - O7: expert MLPs and the weighted combine
# --------------------------------------------------------------------------
def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    return z / (1.0 + np.exp(-z))


def expert_mlp(x: np.ndarray, W13: np.ndarray, W2: np.ndarray) -> np.ndarray:
    """One expert on one token: FC1 (gate rows then up rows), SiLU(gate)*up, FC2.

    Reading: W13 has 2I rows, [0, I) the gate projection and [I, 2I) the up
    projection.
    """
    I = W13.shape[0] // 2
    h = W13 @ x
    act = silu(h[:I]) * h[I:]
    return W2 @ act


# --------------------------------------------------------------------------
# O1', O2': MXFP4 expert weights (FP4 e2m1 codes, E8M0 scale per 32)
# --------------------------------------------------------------------------
# "From 1,060 to 4,016 tok/s on one B300, and why it wasn't the kernels"
# (opening section) serves a MoE whose experts are MXFP4. The pages do not
# define the format; the reading taken is the OCP Microscaling (MX) v1.0
# MXFP4: blocks of 32 elements along K sharing one E8M0 scale, elements in
# FP4 E2M1. The codes are packed like the INT4 ones (channel 2i in the low
# nibble of byte i).
def decode_fp4_e2m1(codes: np.ndarray) -> np.ndarray:
    """Value of 4-bit E2M1 codes: bit 3 sign, bits 2..1 exponent (bias 1),
    bit 0 mantissa; exponent 0 is subnormal (mantissa * 0.5), otherwise
    2^(exponent - 1) * (1 + mantissa / 2). float64, same shape."""
    c = np.asarray(codes, dtype=np.int64)
    sign = (c >> 3) & 1
    exp = (c >> 1) & 3
    man = c & 1
    mag = np.where(exp == 0, 0.5 * man, np.ldexp(1.0 + 0.5 * man, exp - 1))
    return np.where(sign == 1, -mag, mag)


def decode_e8m0(scales: np.ndarray) -> np.ndarray:
    """E8M0 scale bytes s -> 2^(s - 127) in float64; s = 255 is NaN."""
    s = np.asarray(scales, dtype=np.int64)
    return np.where(s == 255, np.nan, np.ldexp(1.0, s - 127))


def dequantize_mxfp4(qweight: np.ndarray, scales_e8m0: np.ndarray, out: np.ndarray | None = None) -> np.ndarray:
    """W[n, c] = e2m1(code[n, c]) * 2^(s[n, c // 32] - 127) in float64 (exact:
    a 2-bit significand times a power of two)."""
    qb = np.asarray(qweight, dtype=np.uint8)
    s = decode_e8m0(scales_e8m0)
    K = 2 * qb.shape[-1]
    if K != s.shape[-1] * GROUP:
        raise ValueError(f"K={K} does not match {s.shape[-1]} groups of {GROUP}")
    W = np.empty(qb.shape[:-1] + (K,), dtype=np.float64) if out is None else out
    pairs = W.reshape(qb.shape + (2,))
    pairs[..., 0] = decode_fp4_e2m1(qb & 0x0F)  # channel 2i: low nibble
    pairs[..., 1] = decode_fp4_e2m1(qb >> 4)    # channel 2i+1: high nibble
    groups = W.reshape(qb.shape[:-1] + (K // GROUP, GROUP))
    groups *= s[..., None]
    return W


ExpertFn = Callable[[int], Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]]
DEQUANT = {"int4": dequantize, "mxfp4": dequantize_mxfp4}


class DequantCache:
    """Dequantised experts on demand, for weight format ``fmt`` ("int4":
    ``dequantize``, "mxfp4": ``dequantize_mxfp4``).

    Keeps up to ``max_items`` experts; with ``max_items == 0`` it keeps none
    and rewrites one pair of scratch buffers on every call (the caller uses
    an expert's matrices before asking for the next one).
    """

    def __init__(self, get_expert: ExpertFn, max_items: int = 64, fmt: str = "int4"):
        self.get_expert = get_expert
        self.max_items = max_items
        self.dequant = DEQUANT[fmt]
        self.items: Dict[int, Tuple[np.ndarray, np.ndarray]] = {}
        self.scratch = None

    def __call__(self, e: int):
        if e in self.items:
            return self.items[e]
        w13, s13, w2, s2 = self.get_expert(e)
        dq = self.dequant
        if self.max_items == 0:
            if self.scratch is None or self.scratch[0].shape != (w13.shape[0], 2 * w13.shape[1]):
                self.scratch = (np.empty((w13.shape[0], 2 * w13.shape[1])),
                                np.empty((w2.shape[0], 2 * w2.shape[1])))
            return dq(w13, s13, self.scratch[0]), dq(w2, s2, self.scratch[1])
        if len(self.items) >= self.max_items:
            self.items.pop(next(iter(self.items)))
        self.items[e] = (dq(w13, s13), dq(w2, s2))
        return self.items[e]


def expert_outputs(x: np.ndarray, topk_ids: np.ndarray,
                   experts: Callable[[int], Tuple[np.ndarray, np.ndarray]],
                   tokens_subset=None, map_fn=map) -> Dict[Tuple[int, int], np.ndarray]:
    """y[(t, j)] = MLP_{ids[t, j]}(x_t) for every slot j of the given tokens.

    Each expert is asked for once (``experts(e)`` may dequantise it) and
    applied to every (token, slot) routed to it. ``map_fn`` runs the
    per-expert work (the built-in map: one expert after another in ascending
    order; a pool's map runs them concurrently, which needs an ``experts``
    that is safe to call from several threads).
    """
    x = np.asarray(x, dtype=np.float64)
    rows = range(x.shape[0]) if tokens_subset is None else tokens_subset
    by_expert: Dict[int, list] = {}
    for t in rows:
        for j in range(topk_ids.shape[1]):
            by_expert.setdefault(int(topk_ids[t, j]), []).append((t, j))

    def one_expert(e):
        W13, W2 = experts(e)
        return [((t, j), expert_mlp(x[t], W13, W2)) for t, j in by_expert[e]]

    y = {}
    for part in map_fn(one_expert, sorted(by_expert)):
        y.update(part)
    return y


def combine(topk_weights: np.ndarray, y: Dict[Tuple[int, int], np.ndarray], M: int, H: int,
            tokens_subset=None) -> np.ndarray:
    """out[t] = sum_j w[t, j] * y[(t, j)], accumulated in slot order (float64).

    "The Result: Two Regimes": a token's output is the routing-weighted sum of
    its k experts' outputs. Token rows not computed are NaN.
    """
    out = np.full((M, H), np.nan)
    rows = range(M) if tokens_subset is None else tokens_subset
    for t in rows:
        acc = np.zeros(H, dtype=np.float64)
        for j in range(topk_weights.shape[1]):
            acc += topk_weights[t, j] * y[(t, j)]
        out[t] = acc
    return out


def moe_forward(x: np.ndarray, topk_ids: np.ndarray, topk_weights: np.ndarray,
                experts: Callable[[int], Tuple[np.ndarray, np.ndarray]],
                tokens_subset=None) -> np.ndarray:
    """out[t] = sum_j w[t, j] * MLP_{ids[t, j]}(x_t), summed in slot order.

    x: float [M, H] (the bf16 activations widened exactly); experts(e) returns
    the dequantised (W13 [2I, H], W2 [H, I]) of expert e. ``tokens_subset``
    limits the work to some token rows (the others are returned as NaN).
    Returns float64 [M, H].
    """
    x = np.asarray(x, dtype=np.float64)
    M, H = x.shape
    y = expert_outputs(x, topk_ids, experts, tokens_subset)
    return combine(topk_weights, y, M, H, tokens_subset)


def layer(x: np.ndarray, logits: np.ndarray, k: int, experts, tokens_subset=None):
    """Routing followed by the expert MLPs and the combine."""
    ids, w = route(logits, k)
    return moe_forward(x, ids, w, experts, tokens_subset), ids, w
