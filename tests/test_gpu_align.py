"""GPU moe_align vs the oracle: bit-exact on every output, deterministic."""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from _gpu import say, to_dev

import w4a16_grouped_gemm_amd as w

pytestmark = pytest.mark.gpu


def run_align(ids: np.ndarray, E: int, bm: int, extra_capacity: int = 0):
    T, topk = ids.shape
    cap = w.moe_align_capacity(T, topk, E, bm) + extra_capacity
    nblk = (cap + bm - 1) // bm
    d_ids = to_dev(ids.astype(np.int32)) if ids.size else torch.empty((T, topk), dtype=torch.int32, device="cuda")
    s = torch.full((max(cap, 1),), -7, dtype=torch.int32, device="cuda")[:cap]
    eids = torch.full((max(nblk, 1),), -7, dtype=torch.int32, device="cuda")[:nblk]
    ntpp = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((E,), -7, dtype=torch.int32, device="cuda")
    wsb = w.moe_align_workspace_bytes(T, topk, E, bm)
    ws = torch.full((max(wsb, 1),), 0x55, dtype=torch.uint8, device="cuda") if wsb else None
    w.moe_align(d_ids, E, bm, s, eids, ntpp, cnt, ws)
    torch.cuda.synchronize()
    return s.cpu().numpy(), eids.cpu().numpy(), int(ntpp.item()), cnt.cpu().numpy()


def check(ids, E, bm, extra=0, what=""):
    say(f"align {what}: T={ids.shape[0]} topk={ids.shape[1] if ids.ndim == 2 else 0} E={E} bm={bm}")
    gs, ge, gn, gc = run_align(ids, E, bm, extra)
    T, topk = ids.shape
    os_, oe, on, oc = oracle.moe_align(ids, E, bm, capacity=w.moe_align_capacity(T, topk, E, bm) + extra)
    assert gn == on
    np.testing.assert_array_equal(gc, oc)
    np.testing.assert_array_equal(gs, os_)
    np.testing.assert_array_equal(ge, oe)


@pytest.mark.parametrize("name", synthetic.WORKLOADS)
def test_align_workloads(name):
    c = synthetic.workload(name, weights=False)
    for bm in sorted({c.block_m, 16, 128}):
        check(c.topk_ids, c.E, bm, what=name)


@pytest.mark.parametrize("n_ids", [4096, 8191, 8192, 8193, 16384, 16385, 24577])
def test_align_path_boundaries(n_ids):
    rng = np.random.default_rng(n_ids)
    ids = rng.integers(-3, 70, size=(n_ids, 1)).astype(np.int32)
    check(ids, 64, 32, what=f"boundary {n_ids}")


@pytest.mark.parametrize("n_ids,E,bm", [(1, 1, 16), (2, 48, 16), (8, 48, 128), (63, 512, 16), (64, 7, 32),
                                         (64, 512, 64), (65, 48, 16)])
def test_align_one_wave_path(n_ids, E, bm):
    """Up to 64 ids one wave aligns them (the path the fused router uses for up to 8 tokens of top-8)."""
    rng = np.random.default_rng(n_ids * 1000 + E)
    ids = rng.integers(-2, E + 3, size=(n_ids, 1)).astype(np.int32)
    ids[: n_ids // 2] = rng.integers(0, max(1, E // 4), size=(n_ids // 2, 1))  # repeated experts
    check(ids, E, bm, what=f"one-wave n={n_ids}")


@pytest.mark.parametrize("seed", range(12))
def test_align_fuzz(seed):
    rng = np.random.default_rng(1000 + seed)
    T = int(rng.integers(1, 20000 if seed % 3 == 0 else 600))
    topk = int(rng.integers(1, 9))
    E = int(rng.choice([1, 2, 7, 48, 128, 384, 512]))
    bm = int(rng.choice([16, 32, 64, 128]))
    ids = rng.integers(-2, E + 40, size=(T, topk)).astype(np.int32)
    if seed % 4 == 1:
        ids[:] = rng.integers(0, max(1, E // 8), size=ids.shape)  # heavy skew
    ids[rng.random(ids.shape) < 0.01] = np.iinfo(np.int32).max
    check(ids, E, bm, extra=int(rng.integers(0, 300)), what=f"fuzz {seed}")


def test_align_empty_and_nothing_resident():
    check(np.zeros((0, 8), np.int32), 48, 16, what="T=0")
    check(np.full((37, 4), 99, np.int32), 48, 64, what="none resident")
    check(np.zeros((1, 1), np.int32), 1, 128, what="single slot")


def test_align_deterministic():
    c = synthetic.workload("prefill_skew48", weights=False)
    first = run_align(c.topk_ids, c.E, 128)
    for _ in range(20):
        again = run_align(c.topk_ids, c.E, 128)
        for a, b in zip(first, again):
            assert np.array_equal(a, b)
