"""Seeded synthetic inputs for the INT4 (group 32) weight-only MoE layer.

This module only draws random numbers. It holds none of the layer's arithmetic
(no unpacking, dequantisation, routing, GEMM or combine), so that the CPU oracle
and the HIP path can both take their inputs from it without sharing any of the
method. Everything is numpy ``default_rng`` based and deterministic.

Shapes follow "The Throughput Lever: Quantifying the MoE GEMM and Mapping the
Road to B300", section "Building the Benchmark" (384 experts, hidden 7168,
intermediate 2048, INT4 with group size 32, randomly generated GPTQ-format
weights) and section "The Result: Two Regimes" (top-8 routing, M = 1 ... 1024
tokens per layer call). The token count M = streams x q_len comes from the
section "What It Means for the Engine" of the same page.

Canonical weight format (the input of the repack call):
  qweight  uint8  [N, K/2]   byte i of a row holds K index 2i in its low nibble
                             and 2i+1 in its high nibble; nibble u encodes the
                             signed value q = u - 8 (offset binary)
  scales   fp16   [N, K/32]  one scale per 32 consecutive K values
For W13, N = 2*I (rows [0, I) are the gate projection, [I, 2I) the up
projection) and K = H. For W2, N = H and K = I.

Recipe (all draws in the order listed):
  per expert e of a layer with weight seed S: rng = default_rng([S, e]);
    w13 = integers(0, 256, (2I, H/2), uint8)
    s13 = uniform(0.005, 0.02, (2I, H/32)).astype(float16)
    w2  = integers(0, 256, (H, I/2), uint8)
    s2  = uniform(0.005, 0.02, (H, I/32)).astype(float16)
  tokens with seed T: rng = default_rng(T);
    if a per-expert bias sigma is given: bias = normal(0, sigma, E).astype(float32)
    logits = standard_normal((M, E), float32) (+ bias[None, :] in float32)
    x = bf16 round-to-nearest-even of standard_normal((M, H), float32)
Uniform random bytes make both nibbles uniform on [0, 15], so q is uniform on
[-8, 7]. One generator per expert lets a caller draw only the experts it needs.
"""
from __future__ import annotations

import hashlib
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

GROUP = 32
SCALE_LO, SCALE_HI = 0.005, 0.02


@dataclass(frozen=True)
class LayerShape:
    E: int  # experts
    H: int  # hidden size (FC1 K, FC2 N)
    I: int  # intermediate size (FC1 N = 2I, FC2 K)
    k: int  # experts per token (top-k)


@dataclass(frozen=True)
class Workload:
    name: str
    shape: LayerShape
    M: int
    weight_seed: int
    token_seed: int
    bias_sigma: float = 0.0
    note: str = field(default="", compare=False)


TINY = LayerShape(E=8, H=256, I=128, k=2)
K26 = LayerShape(E=384, H=7168, I=2048, k=8)

# The workloads: a tiny layer the oracle runs in milliseconds, and the
# 384-expert layer at the token counts the pages measure (1 = one stream
# decoding, 4 = four streams decoding, 9 = one stream verifying a tree of
# budget 8, 90 = ten such
# streams, 256 / 512 / 1024 = multi-stream batches), plus M=1024 with a
# per-expert routing bias that skews the expert load.
WORKLOADS = {
    "tiny": Workload("tiny", TINY, 16, 0, 0, note="8 experts, H=256, I=128, top-2, M=16"),
    "k26_m1": Workload("k26_m1", K26, 1, 2026, 1, note="decode, one stream"),
    "k26_m4": Workload("k26_m4", K26, 4, 2026, 4, note="decode, four streams"),
    "k26_m9": Workload("k26_m9", K26, 9, 2026, 9, note="tree verify, 1 stream x q_len 9"),
    "k26_m90": Workload("k26_m90", K26, 90, 2026, 90, note="tree verify, 10 streams x q_len 9"),
    "k26_m256": Workload("k26_m256", K26, 256, 2026, 256, note="all experts touched on average"),
    "k26_m512": Workload("k26_m512", K26, 512, 2026, 512, note="plateau sample point"),
    "k26_m768": Workload("k26_m768", K26, 768, 2026, 768, note="multi-stream chunk (16 assignments per expert)"),
    "k26_m1024": Workload("k26_m1024", K26, 1024, 2026, 1024, note="dense multi-stream chunk"),
    "k26_m1536": Workload("k26_m1536", K26, 1536, 2026, 1536, note="multi-stream chunk (32 assignments per expert)"),
    "k26_m1024_skew": Workload("k26_m1024_skew", K26, 1024, 2026, 2048, bias_sigma=2.0,
                               note="router logits + per-expert bias N(0, 2)"),
    # prefill chunks: past M ~ 4200 tokens the layer's arithmetic intensity
    # crosses the MI355X ridge (the grouped GEMM turns from streaming weights
    # into matrix work)
    "k26_m2048": Workload("k26_m2048", K26, 2048, 2026, 2048, note="prefill chunk"),
    "k26_m4096": Workload("k26_m4096", K26, 4096, 2026, 4096, note="prefill chunk"),
    "k26_m8192": Workload("k26_m8192", K26, 8192, 2026, 8192, note="prefill chunk"),
}


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return the uint16 bits."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def f32_from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_from_f16_bits(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


@dataclass
class ExpertWeights:
    w13: np.ndarray  # uint8 [2I, H/2]
    s13: np.ndarray  # float16 (INT4) or uint8 E8M0 (MXFP4) [2I, H/32]
    w2: np.ndarray   # uint8 [H, I/2]
    s2: np.ndarray   # float16 or uint8 [H, I/32]


# MXFP4 scales: 2^-6, 2^-5 or 2^-4 with equal probability (E8M0 bytes 121..123),
# so that e2m1 codes (magnitudes up to 6) give weights of the INT4 draws' size.
MXFP4_SCALE_EXP = (-6, -3)


def expert_weights(shape: LayerShape, seed: int, e: int, fmt: str = "int4") -> ExpertWeights:
    """Draw the canonical weights and scales of expert ``e``: INT4 codes and
    fp16 scales, or (fmt "mxfp4", a stream of its own) FP4 e2m1 codes and
    E8M0 scales."""
    H, I = shape.H, shape.I
    if fmt == "mxfp4":
        rng = np.random.default_rng([seed, e, 4])
        lo, hi = MXFP4_SCALE_EXP
        w13 = rng.integers(0, 256, (2 * I, H // 2), dtype=np.uint8)
        s13 = (127 + rng.integers(lo, hi, (2 * I, H // GROUP))).astype(np.uint8)
        w2 = rng.integers(0, 256, (H, I // 2), dtype=np.uint8)
        s2 = (127 + rng.integers(lo, hi, (H, I // GROUP))).astype(np.uint8)
        return ExpertWeights(w13, s13, w2, s2)
    rng = np.random.default_rng([seed, e])
    w13 = rng.integers(0, 256, (2 * I, H // 2), dtype=np.uint8)
    s13 = rng.uniform(SCALE_LO, SCALE_HI, (2 * I, H // GROUP)).astype(np.float16)
    w2 = rng.integers(0, 256, (H, I // 2), dtype=np.uint8)
    s2 = rng.uniform(SCALE_LO, SCALE_HI, (H, I // GROUP)).astype(np.float16)
    return ExpertWeights(w13, s13, w2, s2)


def layer_weights(shape: LayerShape, seed: int, threads: int | None = None, fmt: str = "int4"):
    """Draw all experts of a layer as stacked arrays (w13, s13, w2, s2).

    Experts are drawn in parallel threads (numpy releases the GIL while
    filling arrays); the result does not depend on the thread count.
    """
    E, H, I = shape.E, shape.H, shape.I
    sdt = np.uint8 if fmt == "mxfp4" else np.float16
    w13 = np.empty((E, 2 * I, H // 2), np.uint8)
    s13 = np.empty((E, 2 * I, H // GROUP), sdt)
    w2 = np.empty((E, H, I // 2), np.uint8)
    s2 = np.empty((E, H, I // GROUP), sdt)

    def fill(e):
        ew = expert_weights(shape, seed, e, fmt)
        w13[e], s13[e], w2[e], s2[e] = ew.w13, ew.s13, ew.w2, ew.s2

    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(fill, range(E)))
    return w13, s13, w2, s2


@dataclass
class Tokens:
    logits: np.ndarray  # float32 [M, E]
    x_bits: np.ndarray  # uint16 [M, H], bfloat16 bit patterns


def tokens(shape: LayerShape, M: int, seed: int, bias_sigma: float = 0.0) -> Tokens:
    rng = np.random.default_rng(seed)
    bias = None
    if bias_sigma:
        bias = rng.normal(0.0, bias_sigma, shape.E).astype(np.float32)
    logits = rng.standard_normal((M, shape.E), dtype=np.float32)
    if bias is not None:
        logits = (logits + bias[None, :]).astype(np.float32)
    x = rng.standard_normal((M, shape.H), dtype=np.float32)
    return Tokens(logits=logits, x_bits=bf16_bits_from_f32(x))


def workload_tokens(w: Workload) -> Tokens:
    return tokens(w.shape, w.M, w.token_seed, w.bias_sigma)


def sha16(*arrays: np.ndarray) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()[:16]
