"""MI355X-native weight-only INT4 (group 32) MoE layer.

The layer of "The Throughput Lever: Quantifying the MoE GEMM and Mapping the
Road to B300" (section "Phase 3: The INT4 Marlin MoE Throughput Lever"):
top-k routing, per-expert grouping padded to the tile size, FC1 gate/up with
SiLU*mul and FC2 with the routing-weighted sum, as HIP kernels for gfx950
behind the C ABI of include/moe_w4a16.h. This package is the Python binding
(ctypes; PyTorch only provides device memory and streams) plus two helpers
that allocate the buffers a layer call needs.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from ._binding import (  # noqa: F401
    GROUP, KIND_W13, KIND_W2, MOE_ERR_CAPACITY, MOE_ERR_HIP, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED,
    MOE_ERR_SCRATCH, MOE_ERR_WORKSPACE, MOE_OK, NOALLOC_SCRATCH_BYTES, MoeError, lib, library_path, moe_route_align, moe_route_align_capacity,
    moe_w4a16_abi_version, moe_w4a16_fc1, moe_w4a16_fc2, moe_w4a16_forward, moe_w4a16_layer, moe_w4a16_layer_noalloc, moe_w4a16_packed_bytes,
    moe_w4a16_preferred_block_m, moe_w4a16_repack, moe_w4a16_unpack, moe_w4a16_workspace_bytes,
    moe_mxfp4_fc1, moe_mxfp4_fc2, moe_mxfp4_forward, moe_mxfp4_layer, moe_mxfp4_packed_bytes, moe_mxfp4_repack,
    moe_mxfp4_unpack, status_string, moe_calib_read_granule, moe_calib_hbm_read, moe_calib_mfma_f16,
)

FORMATS = ("int4", "mxfp4")  # weight formats: INT4 g32 + fp16 scales, MXFP4 (e2m1 + E8M0 per 32)


@dataclass
class RouteBuffers:
    """Outputs of moe_route_align for a batch of M tokens."""
    M: int
    E: int
    top_k: int
    block_m: int
    cap: int
    topk_ids: torch.Tensor
    topk_weights: torch.Tensor
    sorted_token_ids: torch.Tensor
    block_expert_ids: torch.Tensor
    expert_offsets: torch.Tensor
    num_tokens_post_pad: torch.Tensor


def alloc_route_buffers(M: int, E: int, top_k: int, block_m: int, device="cuda") -> RouteBuffers:
    cap = moe_route_align_capacity(M, E, top_k, block_m)
    if cap < 0:
        raise ValueError("unsupported routing sizes")
    i32 = dict(dtype=torch.int32, device=device)
    return RouteBuffers(
        M, E, top_k, block_m, cap,
        torch.empty((M, top_k), **i32), torch.empty((M, top_k), dtype=torch.float32, device=device),
        torch.empty(max(cap, 1), **i32), torch.empty(max(cap // block_m, 1), **i32),
        torch.empty(E + 1, **i32), torch.empty(1, **i32))


def route_align(logits: torch.Tensor, rb: RouteBuffers, stream=None) -> RouteBuffers:
    moe_route_align(logits, rb.top_k, rb.block_m, rb.topk_ids, rb.topk_weights, rb.sorted_token_ids,
                    rb.block_expert_ids, rb.expert_offsets, rb.num_tokens_post_pad, cap=rb.cap, stream=stream)
    return rb


def repack(qweight: torch.Tensor, scales_f16: torch.Tensor, kind: int, stream=None) -> torch.Tensor:
    """Repack canonical [E, N, K/2] nibbles + [E, N, K/32] fp16 scales into a new device blob."""
    E, N, K2 = qweight.shape
    nbytes = moe_w4a16_packed_bytes(E, N, 2 * K2)
    if nbytes < 0:
        raise ValueError("unsupported weight shape")
    packed = torch.empty(nbytes, dtype=torch.uint8, device=qweight.device)
    moe_w4a16_repack(qweight, scales_f16, kind, packed, stream=stream)
    return packed


def repack_mxfp4(qweight: torch.Tensor, scales_e8m0: torch.Tensor, kind: int, stream=None) -> torch.Tensor:
    """Repack canonical [E, N, K/2] FP4 codes + [E, N, K/32] E8M0 scales into a new device blob."""
    E, N, K2 = qweight.shape
    nbytes = moe_mxfp4_packed_bytes(E, N, 2 * K2)
    if nbytes < 0:
        raise ValueError("unsupported weight shape")
    packed = torch.empty(nbytes, dtype=torch.uint8, device=qweight.device)
    moe_mxfp4_repack(qweight, scales_e8m0, kind, packed, stream=stream)
    return packed


def _check_fmt(fmt: str) -> None:
    if fmt not in FORMATS:
        raise ValueError(f"fmt must be one of {FORMATS}")


def forward(x: torch.Tensor, rb: RouteBuffers, I: int, w13_packed: torch.Tensor, w2_packed: torch.Tensor,
            workspace: torch.Tensor | None = None, out: torch.Tensor | None = None, stream=None,
            fmt: str = "int4") -> torch.Tensor:
    _check_fmt(fmt)
    M, H = x.shape
    if workspace is None:
        workspace = torch.empty(max(moe_w4a16_workspace_bytes(M, rb.E, H, I, rb.top_k), 16),
                                dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty((M, H), dtype=torch.bfloat16, device=x.device)
    fwd = moe_mxfp4_forward if fmt == "mxfp4" else moe_w4a16_forward
    fwd(x, rb.E, I, rb.top_k, rb.block_m, rb.topk_weights, rb.sorted_token_ids, rb.block_expert_ids,
        rb.expert_offsets, rb.num_tokens_post_pad, w13_packed, w2_packed, workspace, out, cap=rb.cap, stream=stream)
    return out


def layer(logits: torch.Tensor, x: torch.Tensor, rb: RouteBuffers, I: int, w13_packed: torch.Tensor,
          w2_packed: torch.Tensor, workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
          stream=None, stage_events=None, fmt: str = "int4") -> torch.Tensor:
    """Routing + expert MLPs in one call. Two kernels while few experts are
    touched (routing inside FC1, FC2 per token: M = 1 on the decode path,
    up to 16 tokens on the routed FC1), else three up to 16 tokens (routing,
    grouped FC1, FC2 per token), and routing + grouped FC1 + grouped FC2 +
    finalize above. fmt: "int4" (moe_w4a16_repack weights) or "mxfp4"
    (moe_mxfp4_repack weights)."""
    _check_fmt(fmt)
    M, H = x.shape
    if workspace is None:
        workspace = torch.empty(max(moe_w4a16_workspace_bytes(M, rb.E, H, I, rb.top_k), 16),
                                dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty((M, H), dtype=torch.bfloat16, device=x.device)
    call = moe_mxfp4_layer if fmt == "mxfp4" else moe_w4a16_layer
    call(logits, x, I, rb.top_k, rb.block_m, rb.topk_ids, rb.topk_weights, rb.sorted_token_ids,
         rb.block_expert_ids, rb.expert_offsets, rb.num_tokens_post_pad, w13_packed, w2_packed,
         workspace, out, cap=rb.cap, stream=stream, stage_events=stage_events)
    return out
