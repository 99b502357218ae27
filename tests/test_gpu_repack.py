"""moe_w4a16_repack / moe_w4a16_unpack on the GPU: exact round trip, and
spot checks of the documented device layout computed by hand."""
import numpy as np
import pytest
import torch

import int4_weight_only_moe_amd as moe
from gpu_common import to_dev

pytestmark = pytest.mark.gpu


def canonical(E, N, K, seed):
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    s = rng.uniform(0.005, 0.02, (E, N, K // 32)).astype(np.float16)
    return q, s


@pytest.mark.parametrize("E,N,K", [(8, 256, 256), (8, 256, 128), (3, 96, 384), (2, 4096, 7168), (2, 7168, 2048)])
@pytest.mark.parametrize("kind", [0, 1])
def test_round_trip(E, N, K, kind):
    q, s = canonical(E, N, K, E + N + K + kind)
    qd, sd = to_dev(q), to_dev(s.view(np.uint16)).view(torch.float16)
    packed = moe.repack(qd, sd, kind)
    assert packed.numel() == moe.moe_w4a16_packed_bytes(E, N, K)
    q2 = torch.full_like(qd, 0x5A)
    s2 = torch.zeros_like(sd)
    moe.moe_w4a16_unpack(packed, E, N, K, kind, q2, s2)
    torch.cuda.synchronize()
    assert torch.equal(q2, qd)
    assert torch.equal(s2.view(torch.int16), sd.view(torch.int16))


def test_layout_by_hand():
    """Device byte positions of a few values, from the layout description.

    Pair p covers W13 gate rows 16p..16p+15 (tile 0) and up rows I+16p.. (tile 1);
    a tile is 16 rows x 128 channels: 1024 B of nibbles + 128 B of scales; lane L
    holds row L%16, channels 32j + 8(L/16) + i in dword j, code i at bit
    4*(i//2) + 16*(i%2).
    """
    E, N, K = 2, 64, 256   # W13 with I = 32: two pairs, two K-chunks per pair
    q, s = canonical(E, N, K, 99)
    packed = moe.repack(to_dev(q), to_dev(s.view(np.uint16)).view(torch.float16), 0).cpu().numpy()
    per_expert = (N // 32) * (K // 128) * 2 * 1152
    nkc = K // 128

    def nibble(e, n, c):
        b = q[e, n, c // 2]
        return (b >> 4) if c % 2 else (b & 15)

    for (e, n, c) in [(0, 0, 0), (0, 5, 17), (1, 31, 255), (1, 40, 130), (0, 63, 77), (1, 16, 200)]:
        I = N // 2
        h = 0 if n < I else 1
        p = (n % I) // 16
        r = (n % I) % 16
        kc, cc = divmod(c, 128)
        j, rem = divmod(cc, 32)
        sb, i = divmod(rem, 8)
        L = 16 * sb + r
        tile = (p * nkc + kc) * 2 + h
        off = e * per_expert + tile * 1152 + 16 * L + 4 * j
        dword = int.from_bytes(packed[off:off + 4].tobytes(), "little")
        bit = 4 * (i // 2) + 16 * (i % 2)
        assert (dword >> bit) & 15 == nibble(e, n, c), (e, n, c)
        soff = e * per_expert + tile * 1152 + 1024 + 8 * r + 2 * j
        assert packed[soff:soff + 2].view(np.float16)[0] == s[e, n, kc * 4 + j]


def test_w2_layout_rows():
    E, N, K = 1, 64, 128   # W2: pair p = rows 32p..32p+31 as two tiles of 16
    q, s = canonical(E, N, K, 5)
    packed = moe.repack(to_dev(q), to_dev(s.view(np.uint16)).view(torch.float16), 1).cpu().numpy()
    for n in (0, 15, 16, 31, 32, 47, 63):
        p, h, r = n // 32, (n % 32) // 16, n % 16
        tile = p * 2 + h
        off = tile * 1152 + 16 * r  # L = r (sb = 0), j = 0: channels 0..7
        dword = int.from_bytes(packed[off:off + 4].tobytes(), "little")
        assert dword & 15 == q[0, n, 0] & 15
        assert (dword >> 16) & 15 == q[0, n, 0] >> 4
