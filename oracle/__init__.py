"""CPU oracle for the W4A16 fused MoE layer — test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The GPU library never imports, links or
calls it, and it shares no code with the GPU library.

``w4a16_moe_oracle.c`` holds the reference itself (alignment as a stable
counting sort; exact fp32 dequant of INT4 times its BF16 group scale; per-token,
per-expert fp64 matmuls; SiLU-and-mul with h rounded to bf16; fp64 weighted
combine). ``brute.py`` is a second, independent numpy fp64 writing used only to
cross-check the C code on tiny inputs. Page citations are in the C file's header.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "w4a16_moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (plain -O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32 = ctypes.c_int
        lib.oracle_moe_align.argtypes = [P, i32, i32, i32, i32, P, i32, P, P, P]
        lib.oracle_moe_align.restype = i32
        lib.oracle_dequant.argtypes = [P, P, i32, i32, P]
        lib.oracle_dequant.restype = None
        lib.oracle_moe_layer.argtypes = [P, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, i32, i32, P]
        lib.oracle_moe_layer.restype = None
        lib.oracle_round_bf16.argtypes = [ctypes.c_double]
        lib.oracle_round_bf16.restype = ctypes.c_double
        lib.oracle_route_topk.argtypes = [P, P, i32, i32, i32, P, P]
        lib.oracle_route_topk.restype = i32
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = i32
        lib.oracle_set_num_threads.argtypes = [i32]
        lib.oracle_set_num_threads.restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def align_capacity(T: int, topk: int, E: int, block_m: int) -> int:
    """Over-allocated length of sorted_token_ids: every expert may waste block_m-1 slots."""
    return T * topk + E * (block_m - 1)


def moe_align(topk_ids, E: int, block_m: int, capacity: int | None = None):
    """Stable counting-sort alignment.

    Returns (sorted_token_ids [capacity], expert_ids [ceil(capacity/block_m)],
    num_tokens_post_padded (int), expert_counts [E]).
    """
    ids = _c(topk_ids, np.int32)
    T, topk = ids.shape
    cap = align_capacity(T, topk, E, block_m) if capacity is None else int(capacity)
    sorted_ids = np.empty(cap, np.int32)
    nblk = (cap + block_m - 1) // block_m
    expert_ids = np.empty(nblk, np.int32)
    ntpp = np.zeros(1, np.int32)
    counts = np.zeros(E, np.int32)
    rc = _load().oracle_moe_align(_ptr(ids), T, topk, E, block_m, _ptr(sorted_ids), cap,
                                  _ptr(expert_ids), _ptr(ntpp), _ptr(counts))
    if rc != 0:
        raise ValueError("capacity too small for the alignment")
    return sorted_ids, expert_ids, int(ntpp[0]), counts


def route_topk(logits, topk: int, bias=None):
    """Router: (ids int32 [T, topk], weights fp64 [T, topk]) from fp32 logits [T, Eg]
    and an optional fp32 bias [Eg]; see oracle_route_topk for the definition."""
    lg = _c(logits, np.float32)
    T, Eg = lg.shape
    b = None if bias is None else _c(bias, np.float32)
    ids = np.empty((T, topk), np.int32)
    w = np.empty((T, topk), np.float64)
    rc = _load().oracle_route_topk(_ptr(lg), None if b is None else _ptr(b), T, Eg, topk, _ptr(ids), _ptr(w))
    if rc != 0:
        raise ValueError("topk must be in [1, number of experts]")
    return ids, w


def dequant(q, s, N: int, K: int) -> np.ndarray:
    """[N, K/2] packed nibbles and [N, K/32] bf16 bits -> fp32 [N, K] (exact)."""
    q = _c(q, np.uint8).reshape(N, K // 2)
    s = _c(s, np.uint16).reshape(N, K // 32)
    w = np.empty((N, K), np.float32)
    _load().oracle_dequant(_ptr(q), _ptr(s), N, K, _ptr(w))
    return w


def expert_rows(a_bits, row_expert, w_q, w_s, N: int, K: int) -> np.ndarray:
    """fp64 [R, N]: each activation row times its expert's weights, transposed.

    Row r of a (bf16 bits [R, K]) against the exactly dequantised weights
    (int4 times bf16 group scale) of expert row_expert[r] ([E, N, K/2] nibbles,
    [E, N, K/32] scales); rows whose expert is negative give 0. This is one
    projection of one local slot in the layer definition (g = x . W13^T before
    SiLU-and-mul, y = h . W2^T before the weighted combine), for checking a
    GEMM stage on the very rows it was given. The matmul is numpy's, in fp64.
    """
    a = _c(a_bits, np.uint16)
    R = a.shape[0]
    assert a.shape == (R, K)
    af = (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ex = np.asarray(row_expert, np.int64).reshape(R)
    E = _c(w_q, np.uint8).size // (N * (K // 2))
    q = _c(w_q, np.uint8).reshape(E, N, K // 2)
    sc = _c(w_s, np.uint16).reshape(E, N, K // 32)
    out = np.zeros((R, N), np.float64)
    for e in np.unique(ex[ex >= 0]):
        rows = np.nonzero(ex == e)[0]
        out[rows] = af[rows] @ dequant(q[e], sc[e], N, K).astype(np.float64).T
    return out


def round_bf16(v: float) -> float:
    """The oracle's own double -> bf16 round-to-nearest-even."""
    return _load().oracle_round_bf16(float(v))


def num_threads() -> int:
    return _load().oracle_num_threads()


def set_num_threads(n: int) -> None:
    """Threads the following layer calls use (the baseline's one-core timing)."""
    _load().oracle_set_num_threads(int(n))


def moe_layer(x_bits, topk_ids, topk_weights, w13_q, w13_s, w2_q, w2_s, E: int, I: int,
              tokens=None, round_h: bool = True) -> np.ndarray:
    """fp64 layer output for ``tokens`` (default: all), shape [len(tokens), H].

    x_bits: uint16 bf16 bits [T, H]; topk_ids int32 [T, k]; topk_weights fp32 [T, k];
    w13_q uint8 [E, 2I, H/2]; w13_s uint16 [E, 2I, H/32]; w2_q uint8 [E, H, I/2];
    w2_s uint16 [E, H, I/32].
    """
    x = _c(x_bits, np.uint16)
    T, H = x.shape
    ids = _c(topk_ids, np.int32)
    wts = _c(topk_weights, np.float32)
    topk = ids.shape[1]
    assert ids.shape == (T, topk) and wts.shape == (T, topk)
    q13 = _c(w13_q, np.uint8); s13 = _c(w13_s, np.uint16)
    q2 = _c(w2_q, np.uint8); s2 = _c(w2_s, np.uint16)
    assert q13.size == E * 2 * I * (H // 2) and s13.size == E * 2 * I * (H // 32)
    assert q2.size == E * H * (I // 2) and s2.size == E * H * (I // 32)
    tok = np.arange(T, dtype=np.int32) if tokens is None else _c(tokens, np.int32)
    out = np.zeros((len(tok), H), np.float64)
    if len(tok):
        _load().oracle_moe_layer(_ptr(x), T, H, I, E, topk, _ptr(ids), _ptr(wts), _ptr(q13), _ptr(s13),
                                 _ptr(q2), _ptr(s2), _ptr(tok), len(tok), 1 if round_h else 0, _ptr(out))
    return out


def grouped_contiguous(x_bits, m_indices, w13_q, w13_s, w2_q, w2_s, E: int, I: int, rows=None,
                       round_h: bool = True) -> np.ndarray:
    """Contiguous grouped layout (Chord page, section "그룹 SM90 커널 기법": contiguous
    prefill, each expert's rows padded to a 128-row boundary): row r belongs to expert
    m_indices[r]; a value outside [0, E) marks padding. Output row r (fp64) is the
    layer's per-slot result for that row alone, with no routing weight:
    down_e(bf16(silu(gate_e x_r) * up_e x_r)); padding rows are zero. That is the
    layer definition with one slot of weight 1 per row."""
    ids = np.asarray(m_indices, np.int32).reshape(-1, 1)
    ones = np.ones(ids.shape, np.float32)
    return moe_layer(x_bits, ids, ones, w13_q, w13_s, w2_q, w2_s, E, I, tokens=rows, round_h=round_h)


def masked_row_ids(masked_m, max_m: int) -> np.ndarray:
    """Masked grouped layout (same page and section: a fixed budget of max_m rows per
    expert): the expert of each of the E * max_m rows, -1 past masked_m[e]
    (masked_m clamped to [0, max_m])."""
    m = np.clip(np.asarray(masked_m, np.int64), 0, max_m)
    E = len(m)
    i = np.arange(max_m)[None, :]
    return np.where(i < m[:, None], np.arange(E)[:, None], -1).astype(np.int32).reshape(-1)


def grouped_masked(x_bits, masked_m, w13_q, w13_s, w2_q, w2_s, I: int, rows=None) -> np.ndarray:
    """x_bits uint16 [E, max_m, H]; output [E * max_m, H] (fp64), or the listed flat rows."""
    x = np.asarray(x_bits)
    E, max_m, H = x.shape
    return grouped_contiguous(x.reshape(E * max_m, H), masked_row_ids(masked_m, max_m), w13_q, w13_s, w2_q, w2_s,
                              E, I, rows=rows)
