"""GPU moe_route_align vs the oracle: top-k ids bit-exact against
oracle.route_topk, weights within fp32 rounding of the fp64 softmax, and every
alignment output bit-exact against oracle.moe_align over the oracle's ids."""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from _gpu import say, to_dev

import w4a16_grouped_gemm_amd as w

pytestmark = pytest.mark.gpu

# fp32 expf, an fp32 sum of <= 32 terms and one division against the fp64
# softmax: a few ulp, with the fp32 rounding of (logit - max) as the largest
# part for logits a few units apart.
W_RTOL = 5e-6


def run(logits: np.ndarray, topk: int, E: int, bm: int, bias=None):
    T, Eg = logits.shape
    cap = w.moe_align_capacity(T, topk, E, bm)
    nblk = (cap + bm - 1) // bm
    d_lg = to_dev(logits) if T else torch.empty((0, Eg), dtype=torch.float32, device="cuda")
    d_b = None if bias is None else to_dev(bias)
    ids = torch.full((T, topk), -7, dtype=torch.int32, device="cuda")
    wts = torch.full((T, topk), -7.0, dtype=torch.float32, device="cuda")
    s = torch.full((max(cap, 1),), -7, dtype=torch.int32, device="cuda")[:cap]
    eids = torch.full((max(nblk, 1),), -7, dtype=torch.int32, device="cuda")[:nblk]
    ntpp = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((E,), -7, dtype=torch.int32, device="cuda")
    wsb = w.moe_align_workspace_bytes(T, topk, E, bm)
    ws = torch.full((max(wsb, 1),), 0x55, dtype=torch.uint8, device="cuda") if wsb else None
    w.moe_route_align(d_lg, topk, E, bm, ids, wts, s, eids, ntpp, bias=d_b, expert_counts=cnt, workspace=ws)
    torch.cuda.synchronize()
    return (ids.cpu().numpy(), wts.cpu().numpy(), s.cpu().numpy(), eids.cpu().numpy(), int(ntpp.item()),
            cnt.cpu().numpy())


def check(logits, topk, E, bm, bias=None, what=""):
    T, Eg = logits.shape
    say(f"route_align {what}: T={T} Eg={Eg} topk={topk} E={E} bm={bm} bias={bias is not None}")
    gi, gw, gs, ge, gn, gc = run(logits, topk, E, bm, bias)
    oi, ow = oracle.route_topk(logits, topk, bias=bias)
    np.testing.assert_array_equal(gi, oi)
    np.testing.assert_allclose(gw.astype(np.float64), ow, rtol=W_RTOL, atol=0)
    os_, oe, on, oc = oracle.moe_align(oi, E, bm)
    assert gn == on
    np.testing.assert_array_equal(gc, oc)
    np.testing.assert_array_equal(gs, os_)
    np.testing.assert_array_equal(ge, oe)
    return gi, gw, gs, ge


CASES = [
    # (name, T, Eg, topk, E, bm, seed, bias, ties)
    ("one token", 1, 384, 8, 48, 16, 1, False, False),
    ("one token, bias", 1, 384, 8, 48, 16, 2, True, False),
    ("16 tokens fused, all local", 16, 384, 8, 384, 16, 3, True, False),
    ("17 tokens, two launches, ties", 17, 256, 8, 256, 32, 4, False, True),
    ("decode 128 x 384, bias", 128, 384, 8, 48, 16, 5, True, False),
    ("n = 12000 ids, multi-chunk alignment", 1500, 384, 8, 48, 64, 6, True, True),
    ("topk 32", 7, 64, 32, 64, 128, 7, False, True),
    ("1024 routed experts", 40, 1024, 4, 512, 16, 8, True, False),
    ("ragged expert count", 33, 100, 3, 50, 16, 9, False, True),
    ("tiny expert count", 5, 2, 2, 1, 16, 10, False, False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_route_align(case):
    name, T, Eg, topk, E, bm, seed, with_bias, ties = case
    lg = synthetic.router_logits(T, Eg, seed, ties=ties)
    bias = synthetic.zipf_bias(Eg, perm_seed=seed) if with_bias else None
    check(lg, topk, E, bm, bias, what=name)


def test_exact_ties_and_signed_zeros():
    Eg = 96
    lg = np.zeros((6, Eg), np.float32)
    lg[1] = -0.0                       # every score -0: ids 0..k-1
    lg[2, ::2] = -0.0                  # -0 and +0 compare equal
    lg[3, 70] = 1.0                    # one clear winner, then the zero ties
    lg[4] = np.float32(-1e30)          # large equal negatives
    lg[5, [5, 64, 65]] = 2.0           # a tie across lanes and slots
    gi, gw, _, _ = check(lg, 5, 32, 16, what="ties")
    assert gi[0].tolist() == [0, 1, 2, 3, 4]
    assert gi[5].tolist()[:3] == [5, 64, 65]


def test_empty():
    say("route_align empty")
    gi, gw, gs, ge, gn, gc = run(np.zeros((0, 384), np.float32), 8, 48, 16)
    assert gn == 0 and np.all(gc == 0)
    assert np.all(gs == 0) and np.all(ge == -1)  # sentinel T*topk = 0


@pytest.mark.parametrize("name", ["decode_ep48", "prefill_skew48"])
def test_workload_sizes_deterministic(name):
    """The router on a workload's size (skewed prefill: 16384 tokens, Zipf bias) twice: equal to the
    oracle and bitwise equal across calls."""
    c = synthetic.workload(name, weights=False)
    Eg = c.meta["E_global"]
    lg = synthetic.router_logits(c.T, Eg, 100 + c.meta["seed"])
    bias = synthetic.zipf_bias(Eg) if name == "prefill_skew48" else None
    first = check(lg, c.topk, c.E, c.block_m, bias, what=name)
    second = run(lg, c.topk, c.E, c.block_m, bias)
    for a, b in zip(first, second[:4]):
        assert a.tobytes() == b.tobytes()
