"""Pins for the oracle's dequant, bf16 rounding and layer.

Each test fixes a value from something other than the oracle itself: an
independent inverse (packing), powers-of-two scales, closed forms with
permutation / constant / zero weights, library bf16 rounding, invariants of the
layer (linearity in W2 scales and combine weights, expert- and
intermediate-slice additivity, relabelling, token permutation), and an
independent numpy fp64 brute force on small inputs.
"""
import numpy as np
import pytest
import torch

import synthetic
from oracle import brute


def _bf16_of_f32(v):
    """torch's fp32 -> bf16 rounding (library reference for fp32-representable inputs)."""
    return torch.tensor(np.asarray(v, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def _bf16(v):
    """Direct fp64 -> bf16 rounding (bit-level, independent of the oracle's frexp/nearbyint)."""
    return brute.round_bf16_f64(np.asarray(v, np.float64))


def test_nibble_decode_exhaustive(oracle_lib):
    # all 16 codes at even and odd positions, scale 1.0 (bf16 0x3F80)
    vals = np.arange(-8, 8)
    q = np.concatenate([vals, vals[::-1]])[None, :]  # [1, 32]
    w = oracle_lib.dequant(synthetic.pack_int4(q), np.full((1, 1), 0x3F80, np.uint16), 1, 32)
    assert w[0].tolist() == q[0].astype(np.float32).tolist()
    # every byte value decodes to (low nibble, high nibble) as signed ints
    b = np.arange(256, dtype=np.uint8).reshape(4, 64)
    w = oracle_lib.dequant(b, np.full((4, 4), 0x3F80, np.uint16), 4, 128)
    for byte in range(256):
        r, c = divmod(byte, 64)
        lo, hi = byte & 15, byte >> 4
        assert w[r, 2 * c] == (lo if lo < 8 else lo - 16)
        assert w[r, 2 * c + 1] == (hi if hi < 8 else hi - 16)


def test_group_scale_index(oracle_lib):
    # q = 1 everywhere, scale of group g in row r = 2^(g - r): w[r, k] = 2^(k//32 - r)
    N, K = 3, 128
    q = synthetic.pack_int4(np.ones((N, K), np.int8))
    s = np.array([[2.0 ** (g - r) for g in range(K // 32)] for r in range(N)], np.float32)
    w = oracle_lib.dequant(q, synthetic.to_bf16_bits(s), N, K)
    for r in range(N):
        for k in range(K):
            assert w[r, k] == 2.0 ** (k // 32 - r)


def test_dequant_is_exact_product(oracle_lib):
    rng = np.random.default_rng(0)
    N, K = 64, 256
    qi = rng.integers(-8, 8, size=(N, K))
    s = synthetic.to_bf16_bits(rng.uniform(0.005, 0.02, size=(N, K // 32)).astype(np.float32))
    w = oracle_lib.dequant(synthetic.pack_int4(qi), s, N, K)
    exact = qi.astype(np.float64) * np.repeat(synthetic.bf16_bits_to_f32(s).astype(np.float64), 32, axis=1)
    assert np.array_equal(w.astype(np.float64), exact)


def test_round_bf16(oracle_lib):
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-30, 30, 2000),
                        [0.0, -0.0, 1.0, -3.5, 1e-40, -1e-41]]).astype(np.float32)
    ref = _bf16_of_f32(v)
    got = np.array([oracle_lib.round_bf16(float(a)) for a in v])
    assert np.array_equal(got, ref)
    # ties go to even: 1 + 2^-8 is halfway between 1 and 1 + 2^-7
    assert oracle_lib.round_bf16(1.0 + 2.0 ** -8) == 1.0
    assert oracle_lib.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    # rounding is done once from the double (no detour through fp32)
    assert oracle_lib.round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7
    # the bit-level direct rounding agrees on random doubles, including near-ties
    d = rng.standard_normal(3000) * 10.0 ** rng.integers(-20, 20, 3000)
    ties = (1.0 + (2 * rng.integers(0, 128, 500) + 1) * 2.0 ** -8) * (1 + rng.choice([-1, 0, 1], 500) * 2.0 ** -40)
    d = np.concatenate([d, ties, -ties])
    assert np.array_equal(np.array([oracle_lib.round_bf16(float(a)) for a in d]), _bf16(d))


def _perm_case(T=5, H=128, I=64, E=2, topk=2, seed=0):
    """Weights that pick single inputs: gate row c reads x[pi_e(c)] with scale 2^(group-1),
    up row c reads 2*x[sig_e(c)], W2 sends h[c] to output column tau_e(c)."""
    rng = np.random.default_rng(seed)
    q13 = np.zeros((E, 2 * I, H), np.int8)
    s13 = np.zeros((E, 2 * I, H // 32), np.float32)
    q2 = np.zeros((E, H, I), np.int8)
    s2 = np.ones((E, H, I // 32), np.float32)
    pis, sigs, taus = [], [], []
    for e in range(E):
        pi, sig = rng.permutation(H)[:I], rng.permutation(H)[:I]
        tau = rng.permutation(H)[:I]
        for c in range(I):
            q13[e, c, pi[c]] = 1
            q13[e, I + c, sig[c]] = 2
            q2[e, tau[c], c] = 1
        for g in range(H // 32):
            s13[e, :, g] = 2.0 ** ((g % 3) - 1)
        pis.append(pi); sigs.append(sig); taus.append(tau)
    x = synthetic.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    ids = np.stack([rng.permutation(E)[:topk] for _ in range(T)]).astype(np.int32)
    wts = rng.uniform(0.1, 1.0, size=(T, topk)).astype(np.float32)
    arrays = (x, ids, wts, synthetic.pack_int4(q13), synthetic.to_bf16_bits(s13),
              synthetic.pack_int4(q2), synthetic.to_bf16_bits(s2))
    return arrays, (pis, sigs, taus)


def test_closed_form_permutation_weights(oracle_lib):
    T, H, I, E, topk = 5, 128, 64, 2, 2
    arrays, (pis, sigs, taus) = _perm_case(T, H, I, E, topk)
    x, ids, wts = arrays[:3]
    out = oracle_lib.moe_layer(*arrays, E=E, I=I)
    xf = synthetic.bf16_bits_to_f32(x).astype(np.float64)
    expect = np.zeros((T, H))
    for t in range(T):
        for j in range(topk):
            e = ids[t, j]
            for c in range(I):
                gate = xf[t, pis[e][c]] * 2.0 ** ((pis[e][c] // 32) % 3 - 1)
                up = 2.0 * xf[t, sigs[e][c]] * 2.0 ** ((sigs[e][c] // 32) % 3 - 1)
                hval = _bf16(gate / (1.0 + np.exp(-gate)) * up)[0]
                expect[t, taus[e][c]] += float(wts[t, j]) * float(hval)
    np.testing.assert_allclose(out, expect, rtol=1e-12, atol=1e-12)
    # swapping gate and up changes the answer (the closed form pins the order)
    swapped = list(arrays)
    q13 = brute.unpack_int4(arrays[3], H).reshape(E, 2 * I, H)
    q13 = np.concatenate([q13[:, I:], q13[:, :I]], axis=1)
    swapped[3] = synthetic.pack_int4(q13)
    s13 = arrays[4].reshape(E, 2 * I, H // 32)
    swapped[4] = np.concatenate([s13[:, I:], s13[:, :I]], axis=1)
    assert not np.allclose(oracle_lib.moe_layer(*swapped, E=E, I=I), expect, rtol=1e-3)


def test_closed_form_constant_weights(oracle_lib):
    # q = 1, all scales c: gate = up = c * sum(x); h = bf16(silu(g) * g); y[n] = c * sum_c h = c*I*h
    T, H, I, E = 3, 64, 32, 1
    c = 0.015625  # 2^-6, exact
    x = synthetic.to_bf16_bits(np.random.default_rng(2).standard_normal((T, H)).astype(np.float32))
    ids = np.zeros((T, 1), np.int32)
    wts = np.array([[1.0], [0.5], [0.25]], np.float32)
    q13 = synthetic.pack_int4(np.ones((E, 2 * I, H), np.int8))
    q2 = synthetic.pack_int4(np.ones((E, H, I), np.int8))
    s13 = synthetic.to_bf16_bits(np.full((E, 2 * I, H // 32), c, np.float32))
    s2 = synthetic.to_bf16_bits(np.full((E, H, I // 32), c, np.float32))
    out = oracle_lib.moe_layer(x, ids, wts, q13, s13, q2, s2, E=E, I=I)
    xs = synthetic.bf16_bits_to_f32(x).astype(np.float64).sum(axis=1)
    for t in range(T):
        g = c * xs[t]
        h = float(_bf16(g / (1 + np.exp(-g)) * g)[0])
        np.testing.assert_allclose(out[t], wts[t, 0] * c * I * h, rtol=1e-13)


def test_zero_weights_and_no_resident_slot(oracle_lib):
    case = synthetic.random_case("z", T=6, H=64, I=32, E=4, topk=2, block_m=16, seed=3)
    zq = np.zeros_like(case.w13_q)
    out = oracle_lib.moe_layer(case.x, case.topk_ids, case.topk_weights, zq, case.w13_s, case.w2_q, case.w2_s,
                               E=4, I=32)
    assert np.all(out == 0)
    ids = case.topk_ids.copy()
    ids[2] = [7, -1]  # token 2 has no resident expert
    out = oracle_lib.moe_layer(case.x, ids, case.topk_weights, case.w13_q, case.w13_s, case.w2_q, case.w2_s,
                               E=4, I=32)
    assert np.all(out[2] == 0) and np.any(out[1] != 0)


def _small(seed=5, T=12, H=128, I=64, E=6, topk=3):
    return synthetic.random_case("s", T=T, H=H, I=I, E=E, topk=topk, block_m=16, seed=seed)


def _run(o, c, **kw):
    return o.moe_layer(c.x, c.topk_ids, c.topk_weights, c.w13_q, c.w13_s, c.w2_q, c.w2_s, E=c.E, I=c.I, **kw)


def test_matches_numpy_brute_force(oracle_lib):
    for c in (synthetic.workload("tiny"), _small()):
        ref = brute.layer(c.x, c.topk_ids, c.topk_weights, c.w13_q, c.w13_s, c.w2_q, c.w2_s, c.E, c.I, round_h=False)
        got = _run(oracle_lib, c, round_h=False)
        np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-10)
        ref = brute.layer(c.x, c.topk_ids, c.topk_weights, c.w13_q, c.w13_s, c.w2_q, c.w2_s, c.E, c.I)
        got = _run(oracle_lib, c)
        np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-10)


def test_scale_doubling_and_weight_linearity(oracle_lib):
    c = _small()
    base = _run(oracle_lib, c)
    s2 = synthetic.to_bf16_bits(2 * synthetic.bf16_bits_to_f32(c.w2_s))
    d = oracle_lib.moe_layer(c.x, c.topk_ids, c.topk_weights, c.w13_q, c.w13_s, c.w2_q, s2, E=c.E, I=c.I)
    assert np.array_equal(d, 2 * base)
    d = oracle_lib.moe_layer(c.x, c.topk_ids, 2 * c.topk_weights, c.w13_q, c.w13_s, c.w2_q, c.w2_s, E=c.E, I=c.I)
    assert np.array_equal(d, 2 * base)


def test_expert_slice_additivity(oracle_lib):
    # the full layer equals the sum of the layers on disjoint expert slices
    c = _small(seed=6, E=8)
    full = _run(oracle_lib, c)
    parts = np.zeros_like(full)
    for lo, hi in ((0, 3), (3, 8)):
        ids = np.where((c.topk_ids >= lo) & (c.topk_ids < hi), c.topk_ids - lo, -1).astype(np.int32)
        parts += oracle_lib.moe_layer(c.x, ids, c.topk_weights, c.w13_q[lo:hi], c.w13_s[lo:hi], c.w2_q[lo:hi],
                                      c.w2_s[lo:hi], E=hi - lo, I=c.I)
    np.testing.assert_allclose(parts, full, rtol=1e-12, atol=1e-12)


def test_intermediate_slice_additivity(oracle_lib):
    # the full layer equals the sum over intermediate slices (h is elementwise in the intermediate index)
    c = _small(seed=7, I=96)
    full = _run(oracle_lib, c)
    I, H = c.I, c.H
    parts = np.zeros_like(full)
    for lo, hi in ((0, 32), (32, 96)):
        w13_q = np.concatenate([c.w13_q[:, lo:hi], c.w13_q[:, I + lo:I + hi]], axis=1)
        w13_s = np.concatenate([c.w13_s[:, lo:hi], c.w13_s[:, I + lo:I + hi]], axis=1)
        w2_q = np.ascontiguousarray(c.w2_q[:, :, lo // 2:hi // 2])
        w2_s = np.ascontiguousarray(c.w2_s[:, :, lo // 32:hi // 32])
        parts += oracle_lib.moe_layer(c.x, c.topk_ids, c.topk_weights, w13_q, w13_s, w2_q, w2_s, E=c.E, I=hi - lo)
    np.testing.assert_allclose(parts, full, rtol=1e-12, atol=1e-12)


def test_relabel_and_token_permutation(oracle_lib):
    c = _small(seed=8)
    full = _run(oracle_lib, c)
    rng = np.random.default_rng(9)
    perm = rng.permutation(c.E)           # new expert e' holds old expert perm[e']
    inv = np.argsort(perm)
    ids = inv[c.topk_ids].astype(np.int32)
    out = oracle_lib.moe_layer(c.x, ids, c.topk_weights, c.w13_q[perm], c.w13_s[perm], c.w2_q[perm], c.w2_s[perm],
                               E=c.E, I=c.I)
    assert np.array_equal(out, full)
    tp = rng.permutation(c.T)
    out = oracle_lib.moe_layer(c.x[tp], c.topk_ids[tp], c.topk_weights[tp], c.w13_q, c.w13_s, c.w2_q, c.w2_s,
                               E=c.E, I=c.I)
    assert np.array_equal(out, full[tp])
    # a token subset gives exactly those rows
    sub = np.array([3, 0, 11], np.int32)
    assert np.array_equal(_run(oracle_lib, c, tokens=sub), full[sub])


def test_one_hot_routing_is_single_expert_ffn(oracle_lib):
    c = _small(seed=10, topk=1)
    c.topk_weights[:] = 1.0
    out = _run(oracle_lib, c)
    xf = synthetic.bf16_bits_to_f32(c.x).astype(np.float64)
    for t in range(c.T):
        e = c.topk_ids[t, 0]
        w13 = brute.dequant_f64(c.w13_q[e], c.w13_s[e], c.H)
        w2 = brute.dequant_f64(c.w2_q[e], c.w2_s[e], c.I)
        g = w13 @ xf[t]
        h = _bf16(g[:c.I] / (1 + np.exp(-g[:c.I])) * g[c.I:])
        np.testing.assert_allclose(out[t], w2 @ h, rtol=1e-9, atol=1e-9)


def test_expert_rows_brute_force_and_one_hot(oracle_lib):
    """expert_rows against pure-Python loops with their own nibble decode, and
    one-hot rows that pick out one dequantised weight column exactly."""
    import oracle

    rng = np.random.default_rng(11)
    E, N, K, R = 3, 5, 64, 7
    qv = rng.integers(-8, 8, size=(E, N, K))
    codes = (qv & 0xF).astype(np.uint8)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    s_bits = synthetic.to_bf16_bits(rng.uniform(0.005, 0.02, size=(E, N, K // 32)).astype(np.float32))
    x_bits = synthetic.to_bf16_bits(rng.standard_normal((R, K)).astype(np.float32))
    ex = np.array([0, 2, -1, 1, 2, 0, 1])
    got = oracle.expert_rows(x_bits, ex, packed, s_bits, N, K)

    def f(bits):
        return float(np.array([int(bits) << 16], np.uint32).view(np.float32)[0])

    for r in range(R):
        for n in range(N):
            ref = 0.0
            if ex[r] >= 0:
                for k in range(K):
                    byte = int(packed[ex[r], n, k // 2])
                    nib = (byte >> 4) if k % 2 else (byte & 0xF)
                    qi = nib - 16 if nib >= 8 else nib
                    ref += f(x_bits[r, k]) * qi * f(s_bits[ex[r], n, k // 32])
            assert abs(got[r, n] - ref) <= 1e-12 * max(1.0, abs(ref)), (r, n)
    # one-hot rows: the weight q * s of column k, exactly
    one = np.zeros((K, K), np.float32)
    one[np.arange(K), np.arange(K)] = 1.0
    cols = oracle.expert_rows(synthetic.to_bf16_bits(one), np.full(K, 1), packed, s_bits, N, K)
    want = qv[1].T * np.repeat(brute.bf16_bits_to_f64(s_bits[1]), 32, axis=1).T
    assert np.array_equal(cols, want)


def test_expert_rows_recompose_layer(oracle_lib):
    """The layer rebuilt from expert_rows (gate_up rows, bf16 SiLU-and-mul, down
    rows, weighted sum in slot order) equals the layer oracle."""
    import oracle

    c = _small()
    T, k = c.topk_ids.shape
    ids = c.topk_ids.reshape(-1)
    local = (ids >= 0) & (ids < c.E)
    ex = np.where(local, ids, -1)
    xr = np.repeat(c.x, k, axis=0)
    g = oracle.expert_rows(xr, ex, c.w13_q, c.w13_s, 2 * c.I, c.H)
    a = g[:, :c.I] / (1.0 + np.exp(-g[:, :c.I])) * g[:, c.I:]
    h = synthetic.to_bf16_bits(_bf16(a).astype(np.float32))
    y = oracle.expert_rows(h, ex, c.w2_q, c.w2_s, c.H, c.I)
    out = np.zeros((T, c.H))
    for j in range(k):
        out += np.where(local.reshape(T, k)[:, j:j + 1], c.topk_weights[:, j:j + 1] * y.reshape(T, k, -1)[:, j], 0.0)
    np.testing.assert_allclose(out, _run(oracle_lib, c), rtol=1e-9, atol=1e-9)
