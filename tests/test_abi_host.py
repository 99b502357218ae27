"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function include/moe_w4a16.h declares,
and reject invalid arguments with the documented status before any HIP call
(so these calls never touch a device). Sizes returned by the helpers are
checked against their closed forms.
"""
import ctypes
import os
import re

import pytest

import int4_weight_only_moe_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_w4a16.h")
FAKE = 0x10000  # an aligned non-null address; validation fails before any use


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = ctypes.CDLL(moe.library_path())
    names = declared_functions()
    assert len(names) >= 12
    for name in names:
        assert hasattr(lib, name), name
    assert moe.moe_w4a16_abi_version() == 3


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert moe.status_string(code) and moe.status_string(code) != "unknown status"
    assert moe.status_string(42) == "unknown status"


@pytest.mark.parametrize("M,E,k,B", [(1, 384, 8, 16), (1024, 384, 8, 32), (1024, 384, 8, 64), (16, 8, 2, 16),
                                     (0, 8, 2, 16), (3, 4, 4, 64), (90, 384, 8, 128), (3, 4, 4, 128)])
def test_capacity_formula(M, E, k, B):
    raw = M * k + min(E, M * k) * (B - 1)
    assert moe.moe_route_align_capacity(M, E, k, B) == -(-raw // B) * B


def test_capacity_rejects():
    assert moe.moe_route_align_capacity(1, 384, 8, 8) == -1
    assert moe.moe_route_align_capacity(1, 384, 8, 256) == -1
    assert moe.moe_route_align_capacity(1, 384, 8, 48) == -1
    assert moe.moe_route_align_capacity(1, 2000, 8, 16) == -1
    assert moe.moe_route_align_capacity(1, 4, 5, 16) == -1
    assert moe.moe_route_align_capacity(-1, 4, 2, 16) == -1


def test_packed_bytes():
    # nibbles + fp16 scales (9/16 byte per weight), then one int8 exponent shift per weight row
    assert moe.moe_w4a16_packed_bytes(384, 4096, 7168) == 384 * 4096 * 7168 * 9 // 16 + 384 * 4096
    assert moe.moe_w4a16_packed_bytes(384, 7168, 2048) == 384 * 7168 * 2048 * 9 // 16 + 384 * 7168
    total = moe.moe_w4a16_packed_bytes(384, 4096, 7168) + moe.moe_w4a16_packed_bytes(384, 7168, 2048)
    assert total == 9_512_681_472 + 384 * (4096 + 7168)  # the 384-expert layer
    assert moe.moe_w4a16_packed_bytes(1, 48, 128) == -1     # N not a multiple of 32
    assert moe.moe_w4a16_packed_bytes(1, 32, 96) == -1      # K not a multiple of 128
    assert moe.moe_w4a16_packed_bytes(1, 32, 128, 64) == -1  # only group 32


def test_mxfp4_packed_bytes():
    # FP4 codes (half a byte) + one E8M0 byte per 32 weights = 17/32 byte per weight
    assert moe.moe_mxfp4_packed_bytes(384, 4096, 7168) == 384 * 4096 * 7168 * 17 // 32
    total = moe.moe_mxfp4_packed_bytes(384, 4096, 7168) + moe.moe_mxfp4_packed_bytes(384, 7168, 2048)
    assert total == 8_984_199_168
    assert moe.moe_mxfp4_packed_bytes(1, 48, 128) == -1
    assert moe.moe_mxfp4_packed_bytes(1, 32, 96) == -1
    assert moe.moe_mxfp4_packed_bytes(0, 32, 128) == -1


def test_workspace_bytes():
    def a256(v):
        return (v + 255) // 256 * 256
    M, E, H, I, k = 512, 384, 7168, 2048, 8
    # fp32 accumulator, bf16 activations, tile count, tile table (2*M*k + 16 entries of 8 bytes)
    want = a256(M * H * 4) + a256(M * k * I * 2) + 256 + a256((2 * M * k + 16) * 8)
    assert moe.moe_w4a16_workspace_bytes(M, E, H, I, k) == want
    # from 16 assignments per expert on (M*k >= 16*E): also the fp16 copies of the
    # A rows (x, then the activations, in one region) and their row exponents
    M = 768
    want = (a256(M * H * 4) + a256(M * k * I * 2) + 256 + a256((2 * M * k + 16) * 8)
            + a256(max(M * H, M * k * I) * 2) + a256(M * k * 4))
    assert moe.moe_w4a16_workspace_bytes(M, E, H, I, k) == want
    assert moe.moe_w4a16_workspace_bytes(1, E, 7000, I, k) == -1


def test_preferred_block_m():
    assert moe.moe_w4a16_preferred_block_m(1, 384, 7168, 2048, 8) == 16
    assert moe.moe_w4a16_preferred_block_m(4, 384, 7168, 2048, 8) == 16
    assert moe.moe_w4a16_preferred_block_m(9, 384, 7168, 2048, 8) == 32
    assert moe.moe_w4a16_preferred_block_m(90, 384, 7168, 2048, 8) == 32
    # 16 per expert and up: the pre-scaled tiled kernel, 128-row tiles of 32-row blocks
    assert moe.moe_w4a16_preferred_block_m(768, 384, 7168, 2048, 8) == 32
    assert moe.moe_w4a16_preferred_block_m(1024, 384, 7168, 2048, 8) == 32
    assert moe.moe_w4a16_preferred_block_m(4096, 384, 7168, 2048, 8) == 32
    # H/32 not whole pair groups: no pre-scaled kernel; the wide block kernel,
    # 64-row blocks above 24 assignments per expert
    assert moe.moe_w4a16_preferred_block_m(1024, 384, 7040, 2048, 8) == 32
    assert moe.moe_w4a16_preferred_block_m(1200, 384, 7040, 2048, 8) == 64


def _route(lib, M=4, E=384, k=8, B=16, cap=None, ptr=FAKE, logits=FAKE):
    if cap is None:
        cap = moe.moe_route_align_capacity(max(M, 0), E, k, B) if M >= 0 else 0
    return lib.moe_route_align(logits, M, E, k, B, ptr, ptr, ptr, ptr, ptr, ptr, cap, None)


def test_route_align_validation():
    lib = moe.lib()
    assert _route(lib, M=0, ptr=None, logits=None) == moe.MOE_OK  # empty batch: no launch
    assert _route(lib, M=-1) == moe.MOE_ERR_INVALID_ARG
    assert _route(lib, E=1025) == moe.MOE_ERR_UNSUPPORTED
    assert _route(lib, k=17, E=64) == moe.MOE_ERR_UNSUPPORTED
    assert _route(lib, k=9, E=8) == moe.MOE_ERR_UNSUPPORTED
    assert _route(lib, B=8, cap=1024) == moe.MOE_ERR_UNSUPPORTED
    assert _route(lib, B=256, cap=4096) == moe.MOE_ERR_UNSUPPORTED
    cap128 = moe.moe_route_align_capacity(4, 384, 8, 128)
    assert _route(lib, B=128, cap=cap128 - 128) == moe.MOE_ERR_CAPACITY  # 128 passes the block_m check
    assert _route(lib, logits=None) == moe.MOE_ERR_INVALID_ARG
    assert _route(lib, logits=FAKE + 2) == moe.MOE_ERR_INVALID_ARG
    cap = moe.moe_route_align_capacity(4, 384, 8, 16)
    assert _route(lib, cap=cap - 16) == moe.MOE_ERR_CAPACITY
    assert _route(lib, cap=cap + 1) == moe.MOE_ERR_CAPACITY  # not a multiple of block_m


def test_repack_validation():
    lib = moe.lib()
    assert lib.moe_w4a16_repack(FAKE, FAKE, 2, 64, 128, 32, 2, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_w4a16_repack(FAKE, FAKE, 2, 48, 128, 32, 1, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_w4a16_repack(FAKE, FAKE, 2, 64, 96, 32, 1, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_w4a16_repack(FAKE, FAKE, 2, 64, 128, 16, 1, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_w4a16_repack(None, FAKE, 2, 64, 128, 32, 1, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_w4a16_repack(FAKE + 8, FAKE, 2, 64, 128, 32, 1, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_w4a16_unpack(FAKE, 2, 64, 128, 32, 0, None, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    # MXFP4: same rules (no group argument)
    assert lib.moe_mxfp4_repack(FAKE, FAKE, 2, 64, 128, 2, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_mxfp4_repack(FAKE, FAKE, 2, 48, 128, 1, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_mxfp4_repack(FAKE, FAKE, 2, 64, 96, 1, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_mxfp4_repack(FAKE, None, 2, 64, 128, 1, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_mxfp4_repack(FAKE, FAKE + 4, 2, 64, 128, 1, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_mxfp4_unpack(FAKE, 2, 64, 128, 0, None, FAKE, None) == moe.MOE_ERR_INVALID_ARG


def _fwd(lib, M=4, E=384, H=7168, I=2048, k=8, B=16, cap=None, ws=None, x=FAKE, out=FAKE):
    if cap is None:
        cap = moe.moe_route_align_capacity(max(M, 0), E, k, B)
    if ws is None:
        ws = moe.moe_w4a16_workspace_bytes(max(M, 0), E, H, I, k)
    p = FAKE
    return lib.moe_w4a16_forward(x, M, E, H, I, k, B, p, p, p, p, p, cap, p, p, p, ws, out, None)


def test_forward_validation():
    lib = moe.lib()
    assert lib.moe_w4a16_forward(None, 0, 384, 7168, 2048, 8, 16, None, None, None, None, None, 0, None, None,
                                 None, 0, None, None) == moe.MOE_OK
    assert _fwd(lib, H=7000) == moe.MOE_ERR_UNSUPPORTED
    assert _fwd(lib, I=2000) == moe.MOE_ERR_UNSUPPORTED
    assert _fwd(lib, B=256) == moe.MOE_ERR_UNSUPPORTED
    assert _fwd(lib, B=48) == moe.MOE_ERR_UNSUPPORTED
    cap128 = moe.moe_route_align_capacity(4, 384, 8, 128)
    assert _fwd(lib, B=128, cap=cap128 - 128) == moe.MOE_ERR_CAPACITY  # 128 passes the block_m check
    assert _fwd(lib, k=0) == moe.MOE_ERR_INVALID_ARG
    cap = moe.moe_route_align_capacity(4, 384, 8, 16)
    assert _fwd(lib, cap=cap - 16) == moe.MOE_ERR_CAPACITY
    ws = moe.moe_w4a16_workspace_bytes(4, 384, 7168, 2048, 8)
    assert _fwd(lib, ws=ws - 1) == moe.MOE_ERR_WORKSPACE
    assert _fwd(lib, x=None) == moe.MOE_ERR_INVALID_ARG
    assert _fwd(lib, out=FAKE + 4) == moe.MOE_ERR_INVALID_ARG
    assert _fwd(lib, M=1 << 20) == moe.MOE_ERR_UNSUPPORTED  # M*k*max(H, I) >= 2^31


def test_fc_stage_validation():
    lib = moe.lib()
    cap = moe.moe_route_align_capacity(4, 384, 8, 16)
    ws = moe.moe_w4a16_workspace_bytes(4, 384, 7168, 2048, 8)
    p = FAKE
    assert lib.moe_w4a16_fc1(p, 4, 384, 7168, 2048, 8, 16, p, p, p, cap, p, p, ws - 16, None) == moe.MOE_ERR_WORKSPACE
    assert lib.moe_w4a16_fc2(4, 384, 7168, 2048, 8, 16, p, p, p, p, cap, p, p, ws, None, None) == moe.MOE_ERR_INVALID_ARG


def test_layer_validation():
    lib = moe.lib()
    p = FAKE
    cap = moe.moe_route_align_capacity(4, 384, 8, 16)
    ws = moe.moe_w4a16_workspace_bytes(4, 384, 7168, 2048, 8)

    def call(M=4, E=384, H=7168, I=2048, k=8, B=16, cap=cap, ws=ws, logits=p, x=p, ev=None):
        return lib.moe_w4a16_layer(logits, x, M, E, H, I, k, B, p, p, p, p, p, p, cap, p, p, p, ws, p, None, ev)

    assert lib.moe_w4a16_layer(None, None, 0, 384, 7168, 2048, 8, 16, None, None, None, None, None, None, 0,
                               None, None, None, 0, None, None, None) == moe.MOE_OK
    assert call(H=7000) == moe.MOE_ERR_UNSUPPORTED
    assert call(cap=cap - 16) == moe.MOE_ERR_CAPACITY
    assert call(ws=ws - 1) == moe.MOE_ERR_WORKSPACE
    assert call(logits=None) == moe.MOE_ERR_INVALID_ARG
    assert call(x=p + 2) == moe.MOE_ERR_INVALID_ARG
    assert call(E=1025) == moe.MOE_ERR_UNSUPPORTED


@pytest.mark.parametrize("prefix", ["moe_w4a16", "moe_mxfp4"])
def test_both_formats_validate_alike(prefix):
    """The MXFP4 stages share the INT4 stages' argument checks."""
    lib = moe.lib()
    p = FAKE
    cap = moe.moe_route_align_capacity(4, 384, 8, 16)
    ws = moe.moe_w4a16_workspace_bytes(4, 384, 7168, 2048, 8)
    fwd, layer = getattr(lib, prefix + "_forward"), getattr(lib, prefix + "_layer")
    fc1, fc2 = getattr(lib, prefix + "_fc1"), getattr(lib, prefix + "_fc2")
    assert fwd(None, 0, 384, 7168, 2048, 8, 16, None, None, None, None, None, 0, None, None, None, 0, None,
               None) == moe.MOE_OK
    assert fwd(p, 4, 384, 7000, 2048, 8, 16, p, p, p, p, p, cap, p, p, p, ws, p, None) == moe.MOE_ERR_UNSUPPORTED
    assert fwd(p, 4, 384, 7168, 2048, 8, 16, p, p, p, p, p, cap - 16, p, p, p, ws, p, None) == moe.MOE_ERR_CAPACITY
    assert fwd(p, 4, 384, 7168, 2048, 8, 16, p, p, p, p, p, cap, p, p, p, ws - 1, p, None) == moe.MOE_ERR_WORKSPACE
    assert layer(None, p, 4, 384, 7168, 2048, 8, 16, p, p, p, p, p, p, cap, p, p, p, ws, p, None,
                 None) == moe.MOE_ERR_INVALID_ARG
    assert layer(p, p, 4, 1025, 7168, 2048, 8, 16, p, p, p, p, p, p, cap, p, p, p, ws, p, None,
                 None) == moe.MOE_ERR_UNSUPPORTED
    assert fc1(p, 4, 384, 7168, 2048, 8, 16, p, p, p, cap, p, p, ws - 16, None) == moe.MOE_ERR_WORKSPACE
    assert fc2(4, 384, 7168, 2048, 8, 16, p, p, p, p, cap, p, p, ws, None, None) == moe.MOE_ERR_INVALID_ARG


def test_calib_validation():
    lib = moe.lib()
    g = moe.moe_calib_read_granule()
    assert g == 256 * 8 * 16
    sink = FAKE
    assert lib.moe_calib_hbm_read(None, g, 1, sink, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_calib_hbm_read(FAKE, g, 1, None, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_calib_hbm_read(FAKE, 0, 1, sink, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_calib_hbm_read(FAKE, g + 16, 1, sink, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_calib_hbm_read(FAKE, g, 0, sink, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_calib_hbm_read(FAKE, g, (1 << 20) + 1, sink, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_calib_hbm_read(FAKE + 8, g, 1, sink, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_calib_hbm_read(FAKE, g, 1, sink + 2, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_calib_mfma_f16(1, 1, None, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_calib_mfma_f16(-1, 1, sink, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_calib_mfma_f16(1, 0, sink, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_calib_mfma_f16(1, 1, sink + 2, None) == moe.MOE_ERR_INVALID_ARG
