"""w4a16_repack writes the documented packed layout, bit for bit.

The layout (one 1024-byte nibble unit and one 64-entry scale unit per
(expert, 64-channel n-block, 32-wide group); lane l's dword c holds column
16c + (l & 15), k = 32g + 8(l >> 4) + 0..7, element 2j in bits [4j, 4j+4) and
element 2j+1 in bits [16+4j, 20+4j), code = int4 + 8; gate/up interleaved per
32 channels) is decoded here independently and compared with the input.

The fp16 copy of the scales is checked against its definition: per packed
channel, E = unbiased exponent of the largest |s| (0 for an all-zero channel,
-126 when the largest is a bf16 subnormal) and each entry = fp16(s * 2^-E),
computed here with numpy's own conversions."""
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
    ns_al = (E * N * G * 2 + 255) // 256 * 256
    nib = buf[:nq].view(np.uint32).reshape(E, NB, G, 64, 4)      # [e, nb, g, lane, c]
    sc = buf[nq_al:nq_al + E * N * G * 2].view(np.uint16).reshape(E, NB, G, 16, 4)  # [e, nb, g, col, c]
    sc16 = buf[nq_al + ns_al:nq_al + ns_al + E * N * G * 2].view(np.float16).reshape(E, NB, G, 16, 4)
    off = nq_al + 2 * ns_al
    cexp = buf[off:off + E * N * 4].view(np.int32).reshape(E, NB, 4, 16)  # [e, nb, c, col]
    q = np.zeros((E, N, K), np.int8)
    s = np.zeros((E, N, G), np.uint16)
    s16 = np.zeros((E, N, G), np.float16)
    ex = np.zeros((E, N), np.int32)
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
                s16[:, row[:16], g] = sc16[:, nb, g, :, c]
            ex[:, row[:16]] = cexp[:, nb, c, :]
    return q, s, s16, ex


def expected_f16(s_bits: np.ndarray):
    """Channel exponents (the largest |s|'s exponent minus 4) and normalised fp16
    scales (largest in [16, 32)) of bf16 scale bits [E, N, G]."""
    mx = (s_bits & 0x7FFF).max(axis=-1).astype(np.int32)
    ef = mx >> 7
    ex = (np.where(mx == 0, 0, np.where(ef == 0, -126, ef - 127)) - 4).astype(np.int32)
    v = np.ldexp((s_bits.astype(np.uint32) << 16).view(np.float32), -ex[..., None]).astype(np.float32)
    return ex, v.astype(np.float16)


def random_bf16_scales(rng, shape):
    """Finite bf16 bit patterns over the whole exponent range (0 included)."""
    sign = rng.integers(0, 2, size=shape) << 15
    expo = rng.integers(0, 255, size=shape) << 7
    mant = rng.integers(0, 128, size=shape)
    return (sign | expo | mant).astype(np.uint16)


@pytest.mark.parametrize("E,H,I", [(3, 128, 64), (2, 256, 96), (1, 192, 32)])
def test_repack_layout(E, H, I):
    say(f"repack E={E} H={H} I={I}")
    rng = np.random.default_rng(E * 1000 + H + I)
    qi13 = rng.integers(-8, 8, size=(E, 2 * I, H))
    qi2 = rng.integers(-8, 8, size=(E, H, I))
    s13 = random_bf16_scales(rng, (E, 2 * I, H // 32))
    s2 = random_bf16_scales(rng, (E, H, I // 32))
    s2[0, :3] = 0  # all-zero channels
    # channels with realistic scales next to the random full-range ones
    s13[:, :8] = synthetic.to_bf16_bits(rng.uniform(0.005, 0.02, size=(E, 8, H // 32)).astype(np.float32))
    s2[:, 3:9] = synthetic.to_bf16_bits(rng.uniform(1e-4, 30.0, size=(E, 6, I // 32)).astype(np.float32))
    shape = w.make_shape(E, H, I)
    n13, n2 = w.w4a16_packed_bytes(shape)
    p13 = torch.zeros(n13, dtype=torch.uint8, device="cuda")
    p2 = torch.zeros(n2, dtype=torch.uint8, device="cuda")
    w.w4a16_repack(shape, to_dev(synthetic.pack_int4(qi13)), to_dev(s13), to_dev(synthetic.pack_int4(qi2)), to_dev(s2),
                   p13, p2)
    torch.cuda.synchronize()
    for buf, N, K, gI, qi, si in ((p13, 2 * I, H, I, qi13, s13), (p2, H, I, 0, qi2, s2)):
        q, s, s16, ex = decode_packed(buf.cpu().numpy(), E, N, K, gI)
        np.testing.assert_array_equal(q, qi)
        np.testing.assert_array_equal(s, si)
        ex_ref, s16_ref = expected_f16(si)
        np.testing.assert_array_equal(ex, ex_ref)
        np.testing.assert_array_equal(s16.view(np.uint16), s16_ref.view(np.uint16))
