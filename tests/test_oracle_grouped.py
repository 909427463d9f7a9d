"""Pins for the oracle's grouped layouts (oracle.grouped_contiguous / grouped_masked).
They tie the layout bookkeeping to the routed layer (oracle.moe_layer): permuting a
routed batch into the contiguous layout and summing its weighted rows back per token
gives the routed layer's output; masked rows equal the same rows computed in the
contiguous layout; padding and masked-off rows are exactly zero; row order inside an
expert is free."""
import numpy as np
import pytest

import oracle
import synthetic

H, I, E = 128, 64, 4


@pytest.fixture(scope="module")
def weights():
    return synthetic.make_weights(E, H, I, seed=31)


def contiguous_from_routing(ids, E, pad=128):
    """Slots grouped by expert in slot order, each expert padded to a multiple of `pad`:
    returns (m_indices, slot of each row or -1)."""
    T, k = ids.shape
    m, slot = [], []
    for e in range(E):
        s = [i for i in range(T * k) if ids.flat[i] == e]
        n = -(-len(s) // pad) * pad
        m += [e] * len(s) + [-1] * (n - len(s))
        slot += s + [-1] * (n - len(s))
    return np.array(m, np.int32), np.array(slot, np.int64)


def test_contiguous_recombines_to_the_routed_layer(weights):
    q13, s13, q2, s2 = weights
    T, k = 12, 2
    rng = np.random.default_rng(5)
    ids = np.stack([rng.choice(E + 2, size=k, replace=False) for _ in range(T)]).astype(np.int32)  # some non-local
    w = rng.uniform(0.1, 1.0, size=(T, k)).astype(np.float32)
    x = synthetic.make_x(T, H, seed=6)
    m, slot = contiguous_from_routing(ids, E)
    xc = np.zeros((len(m), H), np.uint16)
    live = slot >= 0
    xc[live] = x[slot[live] // k]
    yc = oracle.grouped_contiguous(xc, m, q13, s13, q2, s2, E, I)
    assert np.all(yc[~live] == 0.0)
    back = np.zeros((T, H))
    for j in range(k):  # the routed layer's order: sum over j of w * y
        for t in range(T):
            r = np.nonzero(slot == t * k + j)[0]
            if len(r):
                back[t] += np.float64(w[t, j]) * yc[r[0]]
    ref = oracle.moe_layer(x, ids, w, q13, s13, q2, s2, E, I)
    np.testing.assert_allclose(back, ref, rtol=1e-12, atol=1e-12)


def test_masked_rows_match_contiguous_and_padding_is_zero(weights):
    q13, s13, q2, s2 = weights
    max_m = 16
    masked = np.array([3, 0, 16, 20], np.int32)  # 20 clamps to the budget
    x = synthetic.make_x(E * max_m, H, seed=8).reshape(E, max_m, H)
    y = oracle.grouped_masked(x, masked, q13, s13, q2, s2, I)
    ids = oracle.masked_row_ids(masked, max_m)
    assert ids.tolist()[:max_m] == [0, 0, 0] + [-1] * 13
    assert np.all(ids[16:32] == -1) and np.all(ids[32:48] == 2) and np.all(ids[48:64] == 3)
    assert np.all(y[ids < 0] == 0.0)
    live = np.nonzero(ids >= 0)[0]
    yc = oracle.grouped_contiguous(x.reshape(-1, H)[live], ids[live], q13, s13, q2, s2, E, I)
    np.testing.assert_array_equal(y[live], yc)


def test_row_order_within_an_expert_is_free(weights):
    q13, s13, q2, s2 = weights
    x = synthetic.make_x(128, H, seed=9)
    m = np.full(128, 2, np.int32)
    m[100:] = -1
    y = oracle.grouped_contiguous(x, m, q13, s13, q2, s2, E, I)
    perm = np.random.default_rng(1).permutation(100)
    xp = x.copy()
    xp[:100] = x[perm]
    yp = oracle.grouped_contiguous(xp, m, q13, s13, q2, s2, E, I)
    np.testing.assert_array_equal(yp[:100], y[perm])
