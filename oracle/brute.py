"""Second, independent fp64 writing of the oracle, for tiny inputs only.

Test infrastructure: it exists to cross-check ``w4a16_moe_oracle.c``. It
decodes nibbles with explicit bit operations, dequantizes whole weight tensors
in numpy fp64, and uses library matmuls per slot. h is rounded to bf16
directly from fp64, round-to-nearest-even on the integer bit pattern
(round_bf16_f64), not through an fp32 cast.
"""
from __future__ import annotations

import numpy as np


def unpack_int4(q: np.ndarray, K: int) -> np.ndarray:
    """uint8 [..., K/2] -> int8 [..., K]; element 2b is the low nibble of byte b."""
    q = np.asarray(q, np.uint8)
    lo = (q & 0x0F).astype(np.int16)
    hi = (q >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(q.shape[:-1] + (K,), np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def round_bf16_f64(a) -> np.ndarray:
    """Nearest bf16 value of fp64 inputs, ties to even, for the normal bf16 range.

    bf16 keeps 7 of the 52 fp64 fraction bits; round the dropped 45 bits to
    nearest-even on the integer bit pattern (a carry moves into the exponent).
    """
    a = np.ascontiguousarray(a, np.float64)
    bits = a.view(np.uint64)
    lsb = (bits >> np.uint64(45)) & np.uint64(1)
    rounded = (bits + (np.uint64((1 << 44) - 1) + lsb)) & ~np.uint64((1 << 45) - 1)
    return rounded.view(np.float64)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def dequant_f64(q: np.ndarray, s: np.ndarray, K: int) -> np.ndarray:
    qi = unpack_int4(q, K).astype(np.float64)
    sc = np.repeat(bf16_bits_to_f64(s), 32, axis=-1)
    return qi * sc


def layer(x_bits, topk_ids, topk_weights, w13_q, w13_s, w2_q, w2_s, E, I, round_h=True):
    x = bf16_bits_to_f64(x_bits)
    T, H = x.shape
    w13 = dequant_f64(np.asarray(w13_q).reshape(E, 2 * I, H // 2), np.asarray(w13_s).reshape(E, 2 * I, H // 32), H)
    w2 = dequant_f64(np.asarray(w2_q).reshape(E, H, I // 2), np.asarray(w2_s).reshape(E, H, I // 32), I)
    out = np.zeros((T, H), np.float64)
    ids = np.asarray(topk_ids)
    wts = np.asarray(topk_weights, np.float64)
    for t in range(T):
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            if e < 0 or e >= E:
                continue
            g = w13[e] @ x[t]
            a = g[:I] / (1.0 + np.exp(-g[:I])) * g[I:]
            if round_h:
                a = round_bf16_f64(a)
            out[t] += wts[t, j] * (w2[e] @ a)
    return out
