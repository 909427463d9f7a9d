"""w4a16_repack writes the documented packed layout, bit for bit.

The layout (one 1024-byte nibble unit and one 64-entry scale unit per
(expert, 64-channel n-block, 32-wide group); lane l's dword c holds column
16c + (l & 15), k = 32g + 8(l >> 4) + 0..7, element 2j in bits [4j, 4j+4) and
element 2j+1 in bits [16+4j, 20+4j), code = int4 + 8; gate/up interleaved per
32 channels) is decoded here independently and compared with the input."""
import numpy as np
import pytest
import torch

import synthetic
from _gpu import say, to_dev

import w4a16_grouped_gemm_amd as w

pytestmark = pytest.mark.gpu


def decode_packed(buf: np.ndarray, E: int, N: int, K: int, gate_up_I: int):
    G, NB = K // 32, N // 64
    nq = E * N * K // 2
    nq_al = (nq + 255) // 256 * 256
    nib = buf[:nq].view(np.uint32).reshape(E, NB, G, 64, 4)      # [e, nb, g, lane, c]
    sc = buf[nq_al:nq_al + E * N * G * 2].view(np.uint16).reshape(E, NB, G, 16, 4)  # [e, nb, g, col, c]
    q = np.zeros((E, N, K), np.int8)
    s = np.zeros((E, N, G), np.uint16)
    lane = np.arange(64)
    for c in range(4):
        j = lane & 15
        for nb in range(NB):
            if gate_up_I:
                ch = 32 * nb + 16 * (c & 1) + j
                row = ch if c < 2 else gate_up_I + ch
            else:
                row = nb * 64 + 16 * c + j
            for g in range(G):
                word = nib[:, nb, g, :, c]  # [E, 64]
                for jj in range(4):
                    for half, k_off in ((0, 2 * jj), (1, 2 * jj + 1)):
                        code = (word >> (16 * half + 4 * jj)) & 0xF
                        k = 32 * g + 8 * (lane >> 4) + k_off
                        q[:, row, k] = (code.astype(np.int16) - 8).astype(np.int8)
                s[:, row[:16], g] = sc[:, nb, g, :, c]
    return q, s


@pytest.mark.parametrize("E,H,I", [(3, 128, 64), (2, 256, 96), (1, 192, 32)])
def test_repack_layout(E, H, I):
    say(f"repack E={E} H={H} I={I}")
    rng = np.random.default_rng(E * 1000 + H + I)
    qi13 = rng.integers(-8, 8, size=(E, 2 * I, H))
    qi2 = rng.integers(-8, 8, size=(E, H, I))
    s13 = rng.integers(0, 65536, size=(E, 2 * I, H // 32)).astype(np.uint16)
    s2 = rng.integers(0, 65536, size=(E, H, I // 32)).astype(np.uint16)
    shape = w.make_shape(E, H, I)
    n13, n2 = w.w4a16_packed_bytes(shape)
    p13 = torch.zeros(n13, dtype=torch.uint8, device="cuda")
    p2 = torch.zeros(n2, dtype=torch.uint8, device="cuda")
    w.w4a16_repack(shape, to_dev(synthetic.pack_int4(qi13)), to_dev(s13), to_dev(synthetic.pack_int4(qi2)), to_dev(s2),
                   p13, p2)
    torch.cuda.synchronize()
    q, s = decode_packed(p13.cpu().numpy(), E, 2 * I, H, I)
    np.testing.assert_array_equal(q, qi13)
    np.testing.assert_array_equal(s, s13)
    q, s = decode_packed(p2.cpu().numpy(), E, H, I, 0)
    np.testing.assert_array_equal(q, qi2)
    np.testing.assert_array_equal(s, s2)
