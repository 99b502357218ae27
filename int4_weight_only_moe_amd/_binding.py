"""ctypes binding of libmoe_w4a16.so (the C ABI declared in include/moe_w4a16.h).

Argument marshalling only: every function here checks the tensors it is
given (device, dtype, contiguity, shape), turns them into raw pointers and
calls the entry point of the same name on the caller's current HIP stream.
All the work runs in the library's kernels. There is no fallback: if the
library is not built, or a call returns an error status, an exception is
raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libmoe_w4a16.so")
_lib = None

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_CAPACITY = -3
MOE_ERR_WORKSPACE = -4
MOE_ERR_HIP = -5
MOE_ERR_SCRATCH = -6

KIND_W13 = 0
KIND_W2 = 1
GROUP = 32

_i32, _i64, _vp, _cp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_char_p

# name -> (restype, argtypes), in the order of the header
_SIGNATURES = {
    "moe_w4a16_abi_version": (_i32, []),
    "moe_w4a16_status_string": (_cp, [ctypes.c_int]),
    "moe_route_align_capacity": (_i64, [_i32, _i32, _i32, _i32]),
    "moe_route_align": (ctypes.c_int, [_vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp]),
    "moe_w4a16_packed_bytes": (_i64, [_i32, _i32, _i32, _i32]),
    "moe_w4a16_repack": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp]),
    "moe_w4a16_unpack": (ctypes.c_int, [_vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp]),
    "moe_w4a16_workspace_bytes": (_i64, [_i32, _i32, _i32, _i32, _i32]),
    "moe_w4a16_preferred_block_m": (_i32, [_i32, _i32, _i32, _i32, _i32]),
    "moe_w4a16_forward": (ctypes.c_int, [_vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp,
                                         _i64, _vp, _vp, _vp, _i64, _vp, _vp]),
    "moe_w4a16_fc1": (ctypes.c_int, [_vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _i64, _vp, _vp,
                                     _i64, _vp]),
    "moe_w4a16_fc2": (ctypes.c_int, [_i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _i64, _vp, _vp,
                                     _i64, _vp, _vp]),
    "moe_w4a16_layer": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                       _i64, _vp, _vp, _vp, _i64, _vp, _vp, _vp]),
    "moe_mxfp4_packed_bytes": (_i64, [_i32, _i32, _i32]),
    "moe_mxfp4_repack": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp]),
    "moe_mxfp4_unpack": (ctypes.c_int, [_vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp]),
}
_SIGNATURES["moe_calib_read_granule"] = (_i64, [])
_SIGNATURES["moe_calib_hbm_read"] = (ctypes.c_int, [_vp, _i64, _i32, _vp, _vp])
_SIGNATURES["moe_calib_mfma_f16"] = (ctypes.c_int, [_i64, _i32, _vp, _vp])
_SIGNATURES["moe_w4a16_layer_noalloc"] = (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp,
                                                          _vp, _vp, _vp, _i64, _vp, _vp, _vp, _vp])
# the MXFP4 stages take the same arguments as the INT4 ones
for _stage in ("fc1", "fc2", "forward", "layer"):
    _SIGNATURES["moe_mxfp4_" + _stage] = _SIGNATURES["moe_w4a16_" + _stage]


class MoeError(RuntimeError):
    def __init__(self, name: str, status: int):
        super().__init__(f"{name} failed with status {status}: {status_string(status)}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """Load the HIP library (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing: build it with `python -m int4_weight_only_moe_amd.build` "
                "(the MoE path has no CPU fallback)")
        handle = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().moe_w4a16_status_string(status).decode()


def _check(name: str, status: int) -> None:
    if status != MOE_OK:
        raise MoeError(name, status)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t: torch.Tensor | None, dtype: torch.dtype, what: str) -> int:
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{what} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t.data_ptr()


# ------------------------------------------------------------------ host helpers
def moe_w4a16_abi_version() -> int:
    return lib().moe_w4a16_abi_version()


def moe_route_align_capacity(M: int, E: int, top_k: int, block_m: int) -> int:
    return lib().moe_route_align_capacity(M, E, top_k, block_m)


def moe_w4a16_packed_bytes(E: int, N: int, K: int, group: int = GROUP) -> int:
    return lib().moe_w4a16_packed_bytes(E, N, K, group)


def moe_mxfp4_packed_bytes(E: int, N: int, K: int) -> int:
    return lib().moe_mxfp4_packed_bytes(E, N, K)


def moe_w4a16_workspace_bytes(M: int, E: int, H: int, I: int, top_k: int) -> int:
    return lib().moe_w4a16_workspace_bytes(M, E, H, I, top_k)


def moe_w4a16_preferred_block_m(M: int, E: int, H: int, I: int, top_k: int) -> int:
    return lib().moe_w4a16_preferred_block_m(M, E, H, I, top_k)


# ------------------------------------------------------------------ device calls
def moe_route_align(logits: torch.Tensor, top_k: int, block_m: int, topk_ids: torch.Tensor,
                    topk_weights: torch.Tensor, sorted_token_ids: torch.Tensor,
                    block_expert_ids: torch.Tensor, expert_offsets: torch.Tensor,
                    num_tokens_post_pad: torch.Tensor, cap: int | None = None, stream=None) -> None:
    M, E = logits.shape
    if cap is None:
        cap = sorted_token_ids.numel()
    st = lib().moe_route_align(
        _ptr(logits, torch.float32, "logits"), M, E, top_k, block_m,
        _ptr(topk_ids, torch.int32, "topk_ids"), _ptr(topk_weights, torch.float32, "topk_weights"),
        _ptr(sorted_token_ids, torch.int32, "sorted_token_ids"),
        _ptr(block_expert_ids, torch.int32, "block_expert_ids"),
        _ptr(expert_offsets, torch.int32, "expert_offsets"),
        _ptr(num_tokens_post_pad, torch.int32, "num_tokens_post_pad"), cap, _stream(stream))
    _check("moe_route_align", st)


def moe_w4a16_repack(qweight: torch.Tensor, scales_f16: torch.Tensor, kind: int, packed: torch.Tensor,
                     stream=None) -> None:
    E, N, K2 = qweight.shape
    st = lib().moe_w4a16_repack(
        _ptr(qweight, torch.uint8, "qweight"), _ptr(scales_f16, torch.float16, "scales"),
        E, N, 2 * K2, GROUP, kind, _ptr(packed, torch.uint8, "packed"), _stream(stream))
    _check("moe_w4a16_repack", st)


def moe_w4a16_unpack(packed: torch.Tensor, E: int, N: int, K: int, kind: int, qweight: torch.Tensor,
                     scales_f16: torch.Tensor, stream=None) -> None:
    st = lib().moe_w4a16_unpack(
        _ptr(packed, torch.uint8, "packed"), E, N, K, GROUP, kind,
        _ptr(qweight, torch.uint8, "qweight"), _ptr(scales_f16, torch.float16, "scales"), _stream(stream))
    _check("moe_w4a16_unpack", st)


def moe_mxfp4_repack(qweight: torch.Tensor, scales_e8m0: torch.Tensor, kind: int, packed: torch.Tensor,
                     stream=None) -> None:
    E, N, K2 = qweight.shape
    st = lib().moe_mxfp4_repack(
        _ptr(qweight, torch.uint8, "qweight"), _ptr(scales_e8m0, torch.uint8, "scales_e8m0"),
        E, N, 2 * K2, kind, _ptr(packed, torch.uint8, "packed"), _stream(stream))
    _check("moe_mxfp4_repack", st)


def moe_mxfp4_unpack(packed: torch.Tensor, E: int, N: int, K: int, kind: int, qweight: torch.Tensor,
                     scales_e8m0: torch.Tensor, stream=None) -> None:
    st = lib().moe_mxfp4_unpack(
        _ptr(packed, torch.uint8, "packed"), E, N, K, kind,
        _ptr(qweight, torch.uint8, "qweight"), _ptr(scales_e8m0, torch.uint8, "scales_e8m0"), _stream(stream))
    _check("moe_mxfp4_unpack", st)


def moe_w4a16_forward(x: torch.Tensor, E: int, I: int, top_k: int, block_m: int,
                      topk_weights: torch.Tensor, sorted_token_ids: torch.Tensor,
                      block_expert_ids: torch.Tensor, expert_offsets: torch.Tensor,
                      num_tokens_post_pad: torch.Tensor, w13_packed: torch.Tensor, w2_packed: torch.Tensor,
                      workspace: torch.Tensor, out: torch.Tensor, cap: int | None = None, stream=None,
                      _prefix: str = "moe_w4a16") -> None:
    M, H = x.shape
    if cap is None:
        cap = sorted_token_ids.numel()
    st = getattr(lib(), _prefix + "_forward")(
        _ptr(x, torch.bfloat16, "x"), M, E, H, I, top_k, block_m,
        _ptr(topk_weights, torch.float32, "topk_weights"),
        _ptr(sorted_token_ids, torch.int32, "sorted_token_ids"),
        _ptr(block_expert_ids, torch.int32, "block_expert_ids"),
        _ptr(expert_offsets, torch.int32, "expert_offsets"),
        _ptr(num_tokens_post_pad, torch.int32, "num_tokens_post_pad"), cap,
        _ptr(w13_packed, torch.uint8, "w13_packed"), _ptr(w2_packed, torch.uint8, "w2_packed"),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
        _ptr(out, torch.bfloat16, "out"), _stream(stream))
    _check(_prefix + "_forward", st)


def moe_w4a16_fc1(x: torch.Tensor, E: int, I: int, top_k: int, block_m: int, sorted_token_ids: torch.Tensor,
                  block_expert_ids: torch.Tensor, num_tokens_post_pad: torch.Tensor, w13_packed: torch.Tensor,
                  workspace: torch.Tensor, cap: int | None = None, stream=None, _prefix: str = "moe_w4a16") -> None:
    M, H = x.shape
    if cap is None:
        cap = sorted_token_ids.numel()
    st = getattr(lib(), _prefix + "_fc1")(
        _ptr(x, torch.bfloat16, "x"), M, E, H, I, top_k, block_m,
        _ptr(sorted_token_ids, torch.int32, "sorted_token_ids"),
        _ptr(block_expert_ids, torch.int32, "block_expert_ids"),
        _ptr(num_tokens_post_pad, torch.int32, "num_tokens_post_pad"), cap,
        _ptr(w13_packed, torch.uint8, "w13_packed"), _ptr(workspace, torch.uint8, "workspace"),
        workspace.numel(), _stream(stream))
    _check(_prefix + "_fc1", st)


def moe_w4a16_fc2(M: int, E: int, H: int, I: int, top_k: int, block_m: int, topk_weights: torch.Tensor,
                  sorted_token_ids: torch.Tensor, block_expert_ids: torch.Tensor,
                  num_tokens_post_pad: torch.Tensor, w2_packed: torch.Tensor, workspace: torch.Tensor,
                  out: torch.Tensor, cap: int | None = None, stream=None, _prefix: str = "moe_w4a16") -> None:
    if cap is None:
        cap = sorted_token_ids.numel()
    st = getattr(lib(), _prefix + "_fc2")(
        M, E, H, I, top_k, block_m, _ptr(topk_weights, torch.float32, "topk_weights"),
        _ptr(sorted_token_ids, torch.int32, "sorted_token_ids"),
        _ptr(block_expert_ids, torch.int32, "block_expert_ids"),
        _ptr(num_tokens_post_pad, torch.int32, "num_tokens_post_pad"), cap,
        _ptr(w2_packed, torch.uint8, "w2_packed"), _ptr(workspace, torch.uint8, "workspace"),
        workspace.numel(), _ptr(out, torch.bfloat16, "out"), _stream(stream))
    _check(_prefix + "_fc2", st)


def moe_w4a16_layer(logits: torch.Tensor, x: torch.Tensor, I: int, top_k: int, block_m: int,
                    topk_ids: torch.Tensor, topk_weights: torch.Tensor, sorted_token_ids: torch.Tensor,
                    block_expert_ids: torch.Tensor, expert_offsets: torch.Tensor,
                    num_tokens_post_pad: torch.Tensor, w13_packed: torch.Tensor, w2_packed: torch.Tensor,
                    workspace: torch.Tensor, out: torch.Tensor, cap: int | None = None, stream=None,
                    stage_events=None, _prefix: str = "moe_w4a16") -> None:
    """stage_events: None or a pair of raw hipEvent_t handles (ints)."""
    M, E = logits.shape
    H = x.shape[1]
    if x.shape[0] != M:
        raise ValueError("logits and x must have the same number of rows")
    if cap is None:
        cap = sorted_token_ids.numel()
    ev = None
    if stage_events is not None:
        ev = (ctypes.c_void_p * 2)(int(stage_events[0]), int(stage_events[1]))
    st = getattr(lib(), _prefix + "_layer")(
        _ptr(logits, torch.float32, "logits"), _ptr(x, torch.bfloat16, "x"), M, E, H, I, top_k, block_m,
        _ptr(topk_ids, torch.int32, "topk_ids"), _ptr(topk_weights, torch.float32, "topk_weights"),
        _ptr(sorted_token_ids, torch.int32, "sorted_token_ids"),
        _ptr(block_expert_ids, torch.int32, "block_expert_ids"),
        _ptr(expert_offsets, torch.int32, "expert_offsets"),
        _ptr(num_tokens_post_pad, torch.int32, "num_tokens_post_pad"), cap,
        _ptr(w13_packed, torch.uint8, "w13_packed"), _ptr(w2_packed, torch.uint8, "w2_packed"),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _ptr(out, torch.bfloat16, "out"),
        _stream(stream), ev)
    _check(_prefix + "_layer", st)


def moe_w4a16_layer_noalloc(logits: torch.Tensor, x: torch.Tensor, I: int, top_k: int, block_m: int,
                            topk_ids: torch.Tensor, topk_weights: torch.Tensor, sorted_token_ids: torch.Tensor,
                            block_expert_ids: torch.Tensor, expert_offsets: torch.Tensor,
                            num_tokens_post_pad: torch.Tensor, w13_packed: torch.Tensor, w2_packed: torch.Tensor,
                            out: torch.Tensor, cap: int | None = None, stream=None) -> None:
    """moe_w4a16_layer with the library's static scratch as the workspace."""
    M, E = logits.shape
    H = x.shape[1]
    if x.shape[0] != M:
        raise ValueError("logits and x must have the same number of rows")
    if cap is None:
        cap = sorted_token_ids.numel()
    st = lib().moe_w4a16_layer_noalloc(
        _ptr(logits, torch.float32, "logits"), _ptr(x, torch.bfloat16, "x"), M, E, H, I, top_k, block_m,
        _ptr(topk_ids, torch.int32, "topk_ids"), _ptr(topk_weights, torch.float32, "topk_weights"),
        _ptr(sorted_token_ids, torch.int32, "sorted_token_ids"),
        _ptr(block_expert_ids, torch.int32, "block_expert_ids"),
        _ptr(expert_offsets, torch.int32, "expert_offsets"),
        _ptr(num_tokens_post_pad, torch.int32, "num_tokens_post_pad"), cap,
        _ptr(w13_packed, torch.uint8, "w13_packed"), _ptr(w2_packed, torch.uint8, "w2_packed"),
        _ptr(out, torch.bfloat16, "out"), _stream(stream))
    _check("moe_w4a16_layer_noalloc", st)


NOALLOC_SCRATCH_BYTES = 48 << 20  # MOE_W4A16_NOALLOC_SCRATCH_BYTES in the header


def moe_mxfp4_forward(*args, **kw) -> None:
    """moe_w4a16_forward with moe_mxfp4_repack weights."""
    moe_w4a16_forward(*args, _prefix="moe_mxfp4", **kw)


def moe_mxfp4_fc1(*args, **kw) -> None:
    """moe_w4a16_fc1 with moe_mxfp4_repack weights."""
    moe_w4a16_fc1(*args, _prefix="moe_mxfp4", **kw)


def moe_mxfp4_fc2(*args, **kw) -> None:
    """moe_w4a16_fc2 with moe_mxfp4_repack weights."""
    moe_w4a16_fc2(*args, _prefix="moe_mxfp4", **kw)


def moe_mxfp4_layer(*args, **kw) -> None:
    """moe_w4a16_layer with moe_mxfp4_repack weights."""
    moe_w4a16_layer(*args, _prefix="moe_mxfp4", **kw)


# ------------------------------------------------------------------ measurement helpers
def moe_calib_read_granule() -> int:
    return lib().moe_calib_read_granule()


def moe_calib_hbm_read(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Read every byte of `buf` once (attainable HBM read rate); sink: int32
    [workgroups * 256], its XOR = the XOR of buf's 32-bit words."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    nbytes = buf.numel() * buf.element_size()
    st = lib().moe_calib_hbm_read(buf.data_ptr(), nbytes, sink.numel() // 256,
                                  _ptr(sink, torch.int32, "sink"), _stream(stream))
    _check("moe_calib_hbm_read", st)


def moe_calib_mfma_f16(iters: int, sink: torch.Tensor, stream=None) -> None:
    """iters * 8 fp16 MFMAs per wave, 4 waves per workgroup, sink.numel() // 256
    workgroups (attainable matrix-core rate); sink: float32 [workgroups * 256]."""
    st = lib().moe_calib_mfma_f16(iters, sink.numel() // 256, _ptr(sink, torch.float32, "sink"), _stream(stream))
    _check("moe_calib_mfma_f16", st)
