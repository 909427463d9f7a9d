"""Seeded synthetic inputs for the W4A16 fused MoE layer.

This module only draws random numbers and builds the router's top-k choice
(the harness side of the layer); it holds none of the layer's arithmetic. Both
the CPU oracle tests and the GPU tests/benchmark take their inputs from here.

The pages measure on Kimi K2.x serving traffic (Chord page, section
"엔드투엔드 서빙 영향": Kimi-K2.6 with ShareGPT). No such data is available, so
these seeded draws stand in for it with Kimi-K2 layer shapes (hidden 7168,
384 experts, top-8, MoE intermediate 2048):

* activations  x ~ N(0, 1) in fp32, rounded to bf16 (round-to-nearest-even, by torch)
* int4 codes   uniform over the 16 two's-complement values [-8, 7] (a random byte
               holds two independent uniform nibbles)
* scales       U[0.005, 0.02] in fp32, rounded to bf16
* routing      fp32 N(0, 1) logits over the global experts; top-k by a stable
               descending sort (ties to the lower id); weights are the softmax
               over the k chosen logits; ids outside the local slice stay in
               topk_ids and are "not resident" for the layer.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 array -> uint16 bf16 bit patterns (torch's round-to-nearest-even)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def pack_int4(q: np.ndarray) -> np.ndarray:
    """int [..., K] in [-8, 7] -> uint8 [..., K/2], element 2b in the low nibble of byte b."""
    q = np.asarray(q).astype(np.int16)
    lo = (q[..., 0::2] & 0xF).astype(np.uint8)
    hi = (q[..., 1::2] & 0xF).astype(np.uint8)
    return (lo | (hi << 4)).astype(np.uint8)


def route_topk(logits: np.ndarray, topk: int):
    """Stable descending top-k; weights = softmax over the chosen logits."""
    order = np.argsort(-logits, axis=1, kind="stable")[:, :topk].astype(np.int32)
    chosen = np.take_along_axis(logits, order, axis=1).astype(np.float64)
    z = np.exp(chosen - chosen.max(axis=1, keepdims=True))
    w = (z / z.sum(axis=1, keepdims=True)).astype(np.float32)
    return order, w


@dataclass
class MoECase:
    name: str
    T: int
    H: int
    I: int
    E: int            # experts resident in this call (the local slice)
    topk: int
    block_m: int
    x: np.ndarray            # uint16 bf16 bits [T, H]
    topk_ids: np.ndarray     # int32 [T, topk] (global ids; >= E means not resident)
    topk_weights: np.ndarray  # fp32 [T, topk]
    w13_q: np.ndarray        # uint8 [E, 2I, H/2]
    w13_s: np.ndarray        # uint16 [E, 2I, H/32]
    w2_q: np.ndarray         # uint8 [E, H, I/2]
    w2_s: np.ndarray         # uint16 [E, H, I/32]
    meta: dict = field(default_factory=dict)

    def local_slots(self) -> int:
        return int(((self.topk_ids >= 0) & (self.topk_ids < self.E)).sum())


def make_weights(E: int, H: int, I: int, seed: int, s_lo=0.005, s_hi=0.02):
    rng = np.random.default_rng(seed)
    w13_q = np.empty((E, 2 * I, H // 2), np.uint8)
    w13_s = np.empty((E, 2 * I, H // 32), np.uint16)
    w2_q = np.empty((E, H, I // 2), np.uint8)
    w2_s = np.empty((E, H, I // 32), np.uint16)
    for e in range(E):
        w13_q[e] = rng.integers(0, 256, size=(2 * I, H // 2), dtype=np.uint8)
        w13_s[e] = to_bf16_bits(rng.uniform(s_lo, s_hi, size=(2 * I, H // 32)).astype(np.float32))
        w2_q[e] = rng.integers(0, 256, size=(H, I // 2), dtype=np.uint8)
        w2_s[e] = to_bf16_bits(rng.uniform(s_lo, s_hi, size=(H, I // 32)).astype(np.float32))
    return w13_q, w13_s, w2_q, w2_s


def make_x(T: int, H: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))


def router_logits(T: int, E_global: int, seed: int, ties: bool = False) -> np.ndarray:
    """fp32 N(0, 1) router logits [T, E_global]; ties=True rounds them to multiples
    of 1/2 so that equal scores are common (the tie-break is then exercised)."""
    lg = np.random.default_rng(seed).standard_normal((T, E_global), dtype=np.float32)
    return (np.round(lg * 2) / 2).astype(np.float32) if ties else lg


def random_case(name, T, H, I, E, topk, block_m, seed, E_global=None, logit_bias=None, weights=True) -> MoECase:
    """Generic case: N(0,1) logits over E_global experts (default E), local slice [0, E).

    weights=False skips x and the weights (routing-only cases for the alignment)."""
    Eg = E if E_global is None else E_global
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, Eg), dtype=np.float32)
    if logit_bias is not None:
        logits = (logits + logit_bias[None, :]).astype(np.float32)
    ids, w = route_topk(logits, topk)
    if not weights:
        return MoECase(name, T, H, I, E, topk, block_m, None, ids, w, None, None, None, None,
                       meta={"E_global": Eg, "seed": seed})
    x = make_x(T, H, seed + 100)
    w13_q, w13_s, w2_q, w2_s = make_weights(E, H, I, seed + 200)
    return MoECase(name, T, H, I, E, topk, block_m, x, ids, w, w13_q, w13_s, w2_q, w2_s,
                   meta={"E_global": Eg, "seed": seed})


# ---------------------------------------------------------------------------
# The five workloads (tiny parity gate, decode slice, intermediate slice,
# contiguous prefill, skewed prefill).
# ---------------------------------------------------------------------------

KIMI_H, KIMI_I, KIMI_E, KIMI_TOPK = 7168, 2048, 384, 8

WORKLOADS = ("tiny", "decode_ep48", "islice_tp8", "prefill_contig48", "prefill_skew48", "prefill_skew48_identity")


def contiguous_case(seed=4, T=768, E=48, H=KIMI_H, I=KIMI_I, topk=KIMI_TOPK, block_m=128, weights=True) -> MoECase:
    """Every expert gets exactly T*topk/E slots; each token has topk distinct experts.

    Tokens are taken in groups of E/topk; each group splits a seeded permutation
    of the E experts into E/topk rows of topk. Weights ~ Dirichlet(1,...,1).
    """
    assert E % topk == 0 and T % (E // topk) == 0
    rng = np.random.default_rng(seed)
    per = E // topk
    ids = np.empty((T, topk), np.int32)
    for g0 in range(0, T, per):
        perm = rng.permutation(E).astype(np.int32)
        ids[g0:g0 + per] = perm.reshape(per, topk)
    w = rng.dirichlet(np.ones(topk), size=T).astype(np.float32)
    if not weights:
        return MoECase("prefill_contig48", T, H, I, E, topk, block_m, None, ids, w, None, None, None, None,
                       meta={"E_global": E, "seed": seed, "rows_per_expert": T * topk // E})
    x = make_x(T, H, seed + 100)
    w13_q, w13_s, w2_q, w2_s = make_weights(E, H, I, seed + 200)
    return MoECase("prefill_contig48", T, H, I, E, topk, block_m, x, ids, w, w13_q, w13_s, w2_q, w2_s,
                   meta={"E_global": E, "seed": seed, "rows_per_expert": T * topk // E})


def zipf_bias(E_global=KIMI_E, s=1.1, identity=False, perm_seed=0) -> np.ndarray:
    """Expert popularity bias -s*ln(rank); ranks a seeded permutation of 1..E (or identity)."""
    ranks = np.arange(1, E_global + 1) if identity else np.random.default_rng(perm_seed).permutation(np.arange(1, E_global + 1))
    return (-s * np.log(ranks)).astype(np.float32)


def workload(name: str, block_m: int | None = None, weights: bool = True) -> MoECase:
    """Build one of the named workloads. block_m None -> the workload's default.

    weights=False builds the routing only (x and weights are None)."""
    kw = dict(weights=weights)
    if name == "tiny":
        c = random_case("tiny", T=16, H=256, I=128, E=8, topk=2, block_m=16, seed=1, **kw)
    elif name == "decode_ep48":
        c = random_case("decode_ep48", T=128, H=KIMI_H, I=KIMI_I, E=48, topk=KIMI_TOPK, block_m=16, seed=2,
                        E_global=KIMI_E, **kw)
    elif name == "islice_tp8":
        c = random_case("islice_tp8", T=512, H=KIMI_H, I=256, E=KIMI_E, topk=KIMI_TOPK, block_m=32, seed=3, **kw)
    elif name == "prefill_contig48":
        c = contiguous_case(**kw)
    elif name == "prefill_skew48":
        c = random_case("prefill_skew48", T=16384, H=KIMI_H, I=KIMI_I, E=48, topk=KIMI_TOPK, block_m=128, seed=5,
                        E_global=KIMI_E, logit_bias=zipf_bias(), **kw)
    elif name == "prefill_skew48_identity":
        c = random_case("prefill_skew48_identity", T=16384, H=KIMI_H, I=KIMI_I, E=48, topk=KIMI_TOPK, block_m=128,
                        seed=5, E_global=KIMI_E, logit_bias=zipf_bias(identity=True), **kw)
    else:
        raise KeyError(name)
    if block_m is not None:
        c.block_m = block_m
    return c
