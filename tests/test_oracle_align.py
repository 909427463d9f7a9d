"""Pins for the oracle's alignment (stable counting sort into block_m-padded expert segments).

The pages name the buffers (sorted_token_ids, expert_ids, num_tokens_post_padded,
expert_counts) but print no example; these tests pin the oracle to a hand-worked
example, to an independent brute force (numpy stable argsort) and to the
invariants any correct alignment must satisfy.
"""
import numpy as np
import pytest


def test_hand_worked_example(oracle_lib):
    # T=3 tokens, top-2, E=4 experts, block_m=2.
    # Flat slots: 0->e1, 1->e0, 2->e1, 3->e3, 4->e0, 5->e1.
    # counts [2,3,0,1]; padded [2,4,0,2]; offsets [0,2,6,6,8]; total 8.
    # capacity = 6 + 4*(2-1) = 10; sentinel = T*k = 6.
    ids = np.array([[1, 0], [1, 3], [0, 1]], np.int32)
    s, eid, ntpp, cnt = oracle_lib.moe_align(ids, E=4, block_m=2)
    assert s.tolist() == [1, 4, 0, 2, 5, 6, 3, 6, 6, 6]
    assert eid.tolist() == [0, 1, 1, 3, -1]
    assert ntpp == 8
    assert cnt.tolist() == [2, 3, 0, 1]


def _brute(ids, E, bm):
    flat = ids.reshape(-1)
    n = flat.size
    local = (flat >= 0) & (flat < E)
    order = np.argsort(np.where(local, flat, E), kind="stable")
    counts = np.bincount(flat[local], minlength=E)
    padded = (counts + bm - 1) // bm * bm
    cap = n + E * (bm - 1)
    out = np.full(cap, n, np.int32)
    pos = 0
    k = 0
    for e in range(E):
        out[pos:pos + counts[e]] = order[k:k + counts[e]]
        k += counts[e]
        pos += padded[e]
    eids = np.full((cap + bm - 1) // bm, -1, np.int32)
    eids[: pos // bm] = np.repeat(np.arange(E), padded // bm)
    return out, eids, pos, counts


@pytest.mark.parametrize("T,topk,E,Eg,bm,seed", [
    (1, 1, 1, 1, 16, 0), (7, 2, 8, 8, 16, 1), (64, 8, 48, 384, 16, 2), (100, 4, 16, 16, 32, 3),
    (33, 6, 20, 64, 64, 4), (256, 8, 384, 384, 128, 5), (5, 3, 4, 4, 128, 6), (300, 8, 48, 384, 128, 7),
])
def test_matches_brute_force(oracle_lib, T, topk, E, Eg, bm, seed):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.permutation(Eg)[:topk] for _ in range(T)]).astype(np.int32)
    if seed % 2:
        ids[rng.random(ids.shape) < 0.1] = -1  # non-resident marker of another kind
    s, eid, ntpp, cnt = oracle_lib.moe_align(ids, E=E, block_m=bm)
    bs, beid, bntpp, bcnt = _brute(ids, E, bm)
    assert ntpp == bntpp
    np.testing.assert_array_equal(cnt, bcnt)
    np.testing.assert_array_equal(s, bs)
    np.testing.assert_array_equal(eid, beid)


@pytest.mark.parametrize("seed", range(6))
def test_invariants(oracle_lib, seed):
    rng = np.random.default_rng(100 + seed)
    T = int(rng.integers(1, 400))
    topk = int(rng.integers(1, 9))
    Eg = int(rng.integers(topk, 200))
    E = int(rng.integers(1, Eg + 1))
    bm = int(rng.choice([16, 32, 64, 128]))
    ids = np.stack([rng.permutation(Eg)[:topk] for _ in range(T)]).astype(np.int32)
    s, eid, ntpp, cnt = oracle_lib.moe_align(ids, E=E, block_m=bm)
    flat = ids.reshape(-1)
    n = flat.size
    local = (flat < E)
    # sum of expert counts = number of resident slots (T*topk when all are resident)
    assert cnt.sum() == local.sum()
    # padded total = sum over experts of ceil(count/bm)*bm, a multiple of bm
    assert ntpp == int(((cnt + bm - 1) // bm * bm).sum()) and ntpp % bm == 0
    assert len(s) == n + E * (bm - 1)
    # every resident slot appears exactly once; everything else is the sentinel n
    real = s[s < n]
    assert sorted(real.tolist()) == np.nonzero(local)[0].tolist()
    assert np.all(s[ntpp:] == n)
    # each real entry sits in a block labelled with its own expert, ascending within the expert
    for p in np.nonzero(s < n)[0]:
        assert p < ntpp and eid[p // bm] == flat[s[p]]
    for e in range(E):
        seg = s[(eid.repeat(bm)[: len(s)] == e)]
        seg = seg[seg < n]
        assert np.all(np.diff(seg) > 0)
    assert np.all(eid[ntpp // bm:] == -1)


def test_edge_cases(oracle_lib):
    # no tokens
    s, eid, ntpp, cnt = oracle_lib.moe_align(np.zeros((0, 4), np.int32), E=8, block_m=16)
    assert ntpp == 0 and np.all(s == 0) and np.all(eid == -1) and cnt.sum() == 0
    # nothing resident
    ids = np.full((5, 2), 9, np.int32)
    s, eid, ntpp, cnt = oracle_lib.moe_align(ids, E=8, block_m=16)
    assert ntpp == 0 and np.all(s == 10) and np.all(eid == -1)
    # one expert gets everything
    ids = np.zeros((40, 1), np.int32)
    s, eid, ntpp, cnt = oracle_lib.moe_align(ids, E=3, block_m=16)
    assert ntpp == 48 and s[:40].tolist() == list(range(40)) and np.all(s[40:] == 40)
    assert eid.tolist()[:3] == [0, 0, 0] and np.all(eid[3:] == -1)
    # capacity check refuses a too-small buffer
    with pytest.raises(ValueError):
        oracle_lib.moe_align(ids, E=3, block_m=16, capacity=40)
