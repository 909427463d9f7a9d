"""GPU filtered alignment (moe_align_filtered) and the one-call routed layer
(w4a16_moe_routed_forward, per-expert tile sizes on skewed routing) vs the oracle:
a filtered alignment is bit-exact against the oracle's alignment of the same ids
with the dropped experts marked not resident; the routed layer is within the
layer tolerance, and equals w4a16_moe_forward bit for bit when it runs one
alignment."""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from _gpu import DeviceCase, parity, say, to_dev

import w4a16_grouped_gemm_amd as w

pytestmark = pytest.mark.gpu


def filtered_ids(ids, E, lo, hi):
    """The oracle side of a count filter: experts with a resident count outside [lo, hi] become -1."""
    local = (ids >= 0) & (ids < E)
    cnt = np.bincount(ids[local], minlength=E)
    drop = (cnt < lo) | (cnt > hi)
    out = ids.copy()
    out[local & drop[np.clip(ids, 0, E - 1)]] = -1
    return out


@pytest.mark.parametrize("T,topk,E,bm,lo,hi,seed", [
    (300, 4, 16, 16, 1, 31, 1),          # single block, light set
    (300, 4, 16, 128, 32, 2**31 - 1, 1),  # single block, heavy set
    (5000, 8, 48, 16, 1, 31, 2),         # several chunks, light set
    (5000, 8, 48, 128, 32, 2**31 - 1, 2),  # several chunks, heavy set
    (64, 8, 8, 32, 5, 9, 3),             # a band
])
def test_align_filtered(T, topk, E, bm, lo, hi, seed):
    rng = np.random.default_rng(seed)
    p = rng.zipf(1.3, size=E * 4).astype(np.float64)[:E + 4]
    ids = np.stack([rng.choice(E + 4, size=topk, replace=False, p=p / p.sum()) for _ in range(T)]).astype(np.int32)
    say(f"align filtered T={T} topk={topk} E={E} bm={bm} range=[{lo},{hi}]")
    cap = w.moe_align_capacity(T, topk, E, bm)
    nblk = (cap + bm - 1) // bm
    s = torch.full((cap,), -7, dtype=torch.int32, device="cuda")
    eids = torch.full((nblk,), -7, dtype=torch.int32, device="cuda")
    ntpp = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((E,), -7, dtype=torch.int32, device="cuda")
    wsb = w.moe_align_workspace_bytes(T, topk, E, bm)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda") if wsb else None
    w.moe_align_filtered(to_dev(ids), E, bm, lo, hi, s, eids, ntpp, cnt, ws)
    torch.cuda.synchronize()
    os_, oe, on, oc = oracle.moe_align(filtered_ids(ids, E, lo, hi), E, bm, capacity=cap)
    assert int(ntpp.item()) == on
    np.testing.assert_array_equal(cnt.cpu().numpy(), oc)
    np.testing.assert_array_equal(s.cpu().numpy(), os_)
    np.testing.assert_array_equal(eids.cpu().numpy(), oe)


@pytest.mark.parametrize("T,topk,E,split,hbm,lbm,seed", [
    (300, 4, 16, 32, 128, 16, 1),        # one block per set
    (5000, 8, 48, 32, 128, 16, 2),       # several chunks: the joined scatter
    (5000, 8, 48, 2, 64, 32, 3),         # light set = experts with exactly one slot
    (3000, 4, 16, 100000, 128, 16, 4),   # every resident expert light, heavy set empty
    (0, 4, 16, 32, 128, 16, 5),          # no tokens
])
def test_align_split(T, topk, E, split, hbm, lbm, seed):
    """Both sets of the one-pass split equal the oracle's alignments of the count-filtered ids."""
    rng = np.random.default_rng(seed)
    p = rng.zipf(1.3, size=E * 4).astype(np.float64)[:E + 4]
    ids = (np.stack([rng.choice(E + 4, size=topk, replace=False, p=p / p.sum()) for _ in range(T)])
           if T else np.zeros((0, topk))).astype(np.int32)
    say(f"align split T={T} topk={topk} E={E} split={split} block_m {hbm}/{lbm}")
    hcap = w.moe_align_capacity(T, topk, E, hbm) + 5          # not a multiple of anything
    per = -(-(split - 1) // lbm) * lbm
    lcap = min(w.moe_align_capacity(T, topk, E, lbm), E * per)
    s = torch.full((hcap + lcap,), -7, dtype=torch.int32, device="cuda")
    he = torch.full((-(-hcap // hbm),), -7, dtype=torch.int32, device="cuda")
    le = torch.full((-(-lcap // lbm),), -7, dtype=torch.int32, device="cuda")
    hn = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    ln = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    wsb = w.moe_align_workspace_bytes(T, topk, E, hbm)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda") if wsb else None
    dev_ids = to_dev(ids) if T else torch.zeros((0, topk), dtype=torch.int32, device="cuda")
    w.moe_align_split(dev_ids, E, split, hbm, hcap, he, hn, lbm, le, ln, s, ws)
    torch.cuda.synchronize()
    got = s.cpu().numpy()
    for what, lo, hi, bm, cap, sl, e_, n_ in [("heavy", split, 2**31 - 1, hbm, hcap, slice(0, hcap), he, hn),
                                             ("light", 1, split - 1, lbm, lcap, slice(hcap, hcap + lcap), le, ln)]:
        os_, oe, on, _ = oracle.moe_align(filtered_ids(ids, E, lo, hi), E, bm, capacity=cap)
        assert int(n_.item()) == on, what
        np.testing.assert_array_equal(got[sl], os_, err_msg=what)
        np.testing.assert_array_equal(e_.cpu().numpy(), oe, err_msg=what)


def routed(d, Eg, x=None):
    c = d.case
    ws = torch.empty(w.w4a16_moe_routed_workspace_bytes(d.shape, c.T, c.topk, Eg), dtype=torch.uint8, device="cuda")
    out = torch.full((c.T, c.H), -1, dtype=torch.int16, device="cuda")
    w.w4a16_moe_routed_forward(d.shape, d.x if x is None else x, d.ids, d.wts, Eg, d.w13p, d.w2p, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("T,topk,E,Eg,s", [
    (512, 2, 8, 16, 1.5),     # 1024 routed ids: one alignment block per set
    (4096, 4, 16, 64, 1.1),   # 16384 routed ids: several chunks, one joined scatter for both sets
])
def test_routed_small_skewed(T, topk, E, Eg, s):
    """An expert slice with block_m 128 by the tokens-per-expert rule and a split: Zipf
    popularity leaves some local experts heavy and some light."""
    c = synthetic.random_case("routed_small", T=T, H=256, I=128, E=E, topk=topk, block_m=128, seed=33, E_global=Eg,
                              logit_bias=synthetic.zipf_bias(Eg, s=s))
    ids = c.topk_ids
    cnt = np.bincount(ids[ids < c.E], minlength=c.E)
    d = DeviceCase(c)
    assert w.w4a16_moe_routed_split(d.shape, c.T, c.topk, Eg) == 17
    assert (cnt >= 17).any() and ((cnt > 0) & (cnt < 17)).any(), cnt
    say(f"routed small T={T}: counts {cnt.tolist()}")
    out = routed(d, Eg)
    ref = oracle.moe_layer(c.x, c.topk_ids, c.topk_weights, c.w13_q, c.w13_s, c.w2_q, c.w2_s, c.E, c.I)
    parity(out, ref, f"routed small skewed T={T}")
    assert np.array_equal(out, routed(d, Eg)), "run-to-run difference"


@pytest.mark.parametrize("kind", ["split", "aligned_in_gate_up"])
def test_routed_graph_replays(kind):
    """The call captured in a HIP graph (through torch) and replayed with eager work in between:
    every replay equals the eager result. split: the heavy/light prefill call; aligned_in_gate_up:
    a decode-sized call whose alignment runs inside the gate_up launch."""
    if kind == "split":
        Eg = 16
        c = synthetic.random_case("routed_graph", T=512, H=256, I=128, E=8, topk=2, block_m=128, seed=34, E_global=Eg,
                                  logit_bias=synthetic.zipf_bias(Eg, s=1.5))
    else:
        Eg = 384
        c = synthetic.random_case("routed_graph_dec", T=128, H=2048, I=256, E=48, topk=8, block_m=16, seed=35,
                                  E_global=Eg)
    d = DeviceCase(c)
    assert (w.w4a16_moe_routed_split(d.shape, c.T, c.topk, Eg) > 0) == (kind == "split")
    eager = routed(d, Eg)
    ws = torch.empty(w.w4a16_moe_routed_workspace_bytes(d.shape, c.T, c.topk, Eg), dtype=torch.uint8, device="cuda")
    out = torch.zeros((c.T, c.H), dtype=torch.int16, device="cuda")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        w.w4a16_moe_routed_forward(d.shape, d.x, d.ids, d.wts, Eg, d.w13p, d.w2p, out, ws)  # warm-up on s
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        w.w4a16_moe_routed_forward(d.shape, d.x, d.ids, d.wts, Eg, d.w13p, d.w2p, out, ws)
    for i in range(4):
        out.fill_(-1)
        junk = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        say(f"routed graph replay {kind} {i}")
        assert np.array_equal(out.cpu().numpy().view(np.uint16), eager), f"replay {i} differs"
        del junk


@pytest.mark.parametrize("T,topk,E,Eg,I,seed", [
    (128, 8, 48, 384, 256, 41),   # the decode shape: 1024 routed ids, the largest call aligned in gate_up
    (1, 8, 48, 384, 256, 42),     # one token
    (16, 4, 64, 64, 256, 43),     # every routed expert local, 64 of them
    (40, 6, 5, 40, 128, 44),      # few local experts, most ids elsewhere
])
def test_routed_alignment_inside_gate_up(T, topk, E, Eg, I, seed):
    """Decode-sized calls at block_m 16 align their ids inside the gate_up launch (every
    workgroup sorts them in LDS, workgroup 0 also writes the buffers the down GEMM reads): the
    layer must equal, bit for bit, moe_align + w4a16_moe_forward at block_m 16, and the oracle."""
    c = synthetic.random_case("fused_align", T=T, H=2048, I=I, E=E, topk=topk, block_m=16, seed=seed, E_global=Eg)
    d = DeviceCase(c)
    assert w.w4a16_choose_block_m(c.T, c.topk, c.E, Eg) == 16
    assert w.w4a16_moe_routed_split(d.shape, c.T, c.topk, Eg) == 0
    say(f"routed with in-launch alignment T={T} topk={topk} E={E}/{Eg}")
    out = routed(d, Eg)
    assert np.array_equal(out, d.forward(16)), "differs from a separate alignment"
    ref = oracle.moe_layer(c.x, c.topk_ids, c.topk_weights, c.w13_q, c.w13_s, c.w2_q, c.w2_s, c.E, c.I)
    parity(out, ref, f"routed in-launch alignment T={T}")
    assert np.array_equal(out, routed(d, Eg)), "run-to-run difference"


def test_routed_single_alignment_equals_forward():
    c = synthetic.workload("tiny")
    d = DeviceCase(c)
    Eg = c.meta["E_global"]
    assert w.w4a16_moe_routed_split(d.shape, c.T, c.topk, Eg) == 0
    bm = w.w4a16_choose_block_m(c.T, c.topk, c.E, Eg)
    say(f"routed tiny: block_m {bm}")
    assert np.array_equal(routed(d, Eg), d.forward(bm))


def test_routed_full_size_skewed_sampled():
    c = synthetic.workload("prefill_skew48")
    d = DeviceCase(c)
    Eg = c.meta["E_global"]
    say(f"routed full-size prefill_skew48: T={c.T} split={w.w4a16_moe_routed_split(d.shape, c.T, c.topk, Eg)}")
    out = routed(d, Eg)
    local = ((c.topk_ids >= 0) & (c.topk_ids < c.E))
    cnt = np.bincount(c.topk_ids[local], minlength=c.E)
    # tokens routed to the heaviest expert, to light experts only, and to none
    heavy_e, light_e = int(np.argmax(cnt)), [e for e in range(c.E) if 0 < cnt[e] < 32]
    rng = np.random.default_rng(7)
    pick = set(np.nonzero((c.topk_ids == heavy_e).any(axis=1))[0][:4].tolist())
    for e in light_e[:6]:
        pick |= set(np.nonzero((c.topk_ids == e).any(axis=1))[0][:1].tolist())
    none = np.nonzero(local.sum(axis=1) == 0)[0]
    pick |= set(none[:2].tolist()) | set(rng.choice(c.T, size=4, replace=False).tolist())
    tokens = np.array(sorted(pick), np.int32)
    ref = oracle.moe_layer(c.x, c.topk_ids, c.topk_weights, c.w13_q, c.w13_s, c.w2_q, c.w2_s, c.E, c.I,
                           tokens=tokens)
    parity(out[tokens], ref, f"routed prefill_skew48 ({len(tokens)} sampled tokens)")
    assert np.all(out[none] == 0)


def test_routed_full_size_skewed_identity_sampled():
    """The heavily skewed prefill (Zipf ranks in expert order: all 48 local experts
    heavy, 127,817 resident slots, about 1,000 row blocks of 128, several rounds of
    tiles per workgroup). Sampled: the tokens of the last slots of the busiest
    experts (their last, partly filled row blocks), tokens from the last row blocks
    of the whole call (the last tiles the persistent grid runs), the first slot of
    an expert, tokens without a resident slot and random others."""
    c = synthetic.workload("prefill_skew48_identity")
    d = DeviceCase(c)
    Eg = c.meta["E_global"]
    local = (c.topk_ids >= 0) & (c.topk_ids < c.E)
    cnt = np.bincount(c.topk_ids[local], minlength=c.E)
    say(f"routed full-size prefill_skew48_identity: T={c.T} slots={int(cnt.sum())} "
        f"split={w.w4a16_moe_routed_split(d.shape, c.T, c.topk, Eg)} counts {cnt.min()}..{cnt.max()}")
    out = routed(d, Eg)
    flat = c.topk_ids.reshape(-1)
    pick = set()
    for e in np.argsort(-cnt, kind="stable")[:3]:      # busiest experts: their last slots
        sl = np.nonzero(flat == e)[0]
        pick |= set((sl[-3:] // c.topk).tolist())
    last_e = int(np.nonzero(cnt)[0][-1])                # the last expert's last row block
    sl = np.nonzero(flat == last_e)[0]
    nb = (len(sl) - 1) // 128
    pick |= set((sl[nb * 128:][[0, -1]] // c.topk).tolist())
    pick |= {int(np.nonzero(flat == 0)[0][0] // c.topk)}   # the first slot of the first expert
    none = np.nonzero(local.sum(axis=1) == 0)[0]
    rng = np.random.default_rng(8)
    pick |= set(none[:2].tolist()) | set(rng.choice(c.T, size=6, replace=False).tolist())
    tokens = np.array(sorted(pick), np.int32)
    ref = oracle.moe_layer(c.x, c.topk_ids, c.topk_weights, c.w13_q, c.w13_s, c.w2_q, c.w2_s, c.E, c.I,
                           tokens=tokens)
    parity(out[tokens], ref, f"routed prefill_skew48_identity ({len(tokens)} sampled tokens)")
    assert np.all(out[none] == 0)
    assert np.array_equal(out, routed(d, Eg)), "run-to-run difference"
