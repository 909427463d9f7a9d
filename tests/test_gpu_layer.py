"""GPU W4A16 MoE layer vs the CPU oracle: |gpu - oracle| <= 2e-2 * max(1, |oracle|)
per element, on small cases in full and on the full-size workloads on sampled
tokens (the oracle computes sampled rows one by one)."""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from _gpu import DeviceCase, bf16_to_f64, check_own_rows, parity, run_stages, say, to_dev

import w4a16_grouped_gemm_amd as w

pytestmark = pytest.mark.gpu


def oracle_rows(c, tokens=None, ids=None, wts=None):
    ids = c.topk_ids if ids is None else ids
    wts = c.topk_weights if wts is None else wts
    return oracle.moe_layer(c.x, ids, wts, c.w13_q, c.w13_s, c.w2_q, c.w2_s, E=c.E, I=c.I, tokens=tokens)


@pytest.mark.parametrize("block_m", [16, 32, 64, 128])
def test_tiny_all_block_sizes(block_m):
    c = synthetic.workload("tiny")
    say(f"layer tiny bm={block_m}")
    d = DeviceCase(c)
    parity(d.forward(block_m), oracle_rows(c), f"tiny bm{block_m}")


SMALL = [
    # name, T, H, I, E, topk, E_global, block_m
    ("several tiles", 64, 512, 256, 16, 4, 16, 16),
    ("ep slice, ragged", 77, 1024, 320, 12, 6, 24, 32),
    ("k tail (G=18)", 40, 576, 96, 5, 3, 5, 16),
    ("single token", 1, 256, 128, 8, 8, 8, 16),
    ("bm64 skew", 150, 512, 160, 6, 2, 6, 64),
    ("bm128", 300, 384, 128, 4, 2, 4, 128),
    ("bm128 mixed paths", 200, 320, 128, 4, 2, 4, 128),   # gate_up tiled, down streamed (H % 256 != 0)
    ("bm128 streamed", 200, 512, 96, 4, 2, 4, 128),       # neither GEMM fits the tiled kernel
    ("many experts", 96, 256, 64, 200, 8, 256, 16),
    # the declared maxima: 512 resident experts, top-32 routing
    ("max experts, max topk", 40, 256, 64, 512, 32, 512, 16),
    ("max topk bm128", 48, 384, 128, 40, 32, 40, 128),
    # short reductions: the down projection's waves run through several n-blocks
    ("short K bm16", 64, 1024, 256, 8, 2, 8, 16),
    ("short K bm32", 64, 1024, 256, 8, 2, 8, 32),
    ("short K bm64", 200, 1024, 256, 4, 2, 4, 64),
    # long reductions at block_m 16: two waves split each n-block's K (gate_up K = 2048; down K = 2048)
    ("split K gate_up", 40, 2048, 128, 8, 2, 16, 16),
    ("split K down", 40, 256, 2048, 8, 2, 16, 16),
    ("split K both, ragged", 9, 2304, 2304, 6, 3, 6, 16),
]


@pytest.mark.parametrize("name,T,H,I,E,topk,Eg,bm", SMALL, ids=[s[0] for s in SMALL])
def test_small_cases(name, T, H, I, E, topk, Eg, bm):
    say(f"layer {name}: T={T} H={H} I={I} E={E} topk={topk} Eg={Eg} bm={bm}")
    c = synthetic.random_case(name, T=T, H=H, I=I, E=E, topk=topk, block_m=bm, seed=T + H + I, E_global=Eg)
    d = DeviceCase(c)
    parity(d.forward(bm), oracle_rows(c), name)


def _random_shapes(n=24, seed=2024):
    """Seeded random layer shapes over every block_m and kernel family: H a
    multiple of 64 and I of 32 (the supported shapes; some multiples of 256 for
    the tiled and LDS-ring kernels, some not), ragged token counts, expert
    slices of a larger routed set."""
    rng = np.random.default_rng(seed)
    out = []
    for k in range(n):
        bm = int(rng.choice([16, 32, 64, 128]))
        H = int(64 * rng.integers(1, 17))     # 64 .. 1024
        I = int(32 * rng.integers(1, 17))     # 32 .. 512
        if k % 3 == 0:                        # shapes the 256-wide kernels take
            H, I = 256 * int(rng.integers(1, 5)), 128 * int(rng.integers(1, 5))
        E = int(rng.integers(1, 65))
        topk = int(rng.integers(1, min(8, E) + 1))
        Eg = E + int(rng.integers(0, E + 1))
        T = int(rng.integers(1, 201))
        out.append((f"r{k}", T, H, I, E, topk, Eg, bm))
    return out


RANDOM = _random_shapes()


@pytest.mark.parametrize("name,T,H,I,E,topk,Eg,bm", RANDOM, ids=[r[0] for r in RANDOM])
def test_random_shapes(name, T, H, I, E, topk, Eg, bm):
    say(f"layer random {name}: T={T} H={H} I={I} E={E} topk={topk} Eg={Eg} bm={bm}")
    c = synthetic.random_case(name, T=T, H=H, I=I, E=E, topk=topk, block_m=bm, seed=1000 + T + H + I + E,
                              E_global=Eg)
    d = DeviceCase(c)
    out = d.forward(bm)
    parity(out, oracle_rows(c), f"random {name}")
    assert np.array_equal(out, d.forward(bm)), "run-to-run difference"


def test_wide_dynamic_range_block_m_128():
    """Operands outside the fp16 range: activation rows of N(0,1) * 2^(r - 20)
    for r in -24..8 (down to 2^-44, far below fp16's smallest subnormal), gate_up
    scales near 2^13 (q * s beyond 65504), SiLU-and-mul outputs beyond 65504 in
    the largest rows, one gate channel whose scales span 2^20 and one row with an
    element 2^40 below its largest (both round on the fp16 subnormal grid after
    normalisation). Output rows then span 2^-60..2^8.

    Both block sizes meet the usual bound against the oracle. The bound's floor
    of 1 hides errors in the tiny rows, so the fp16-operand path (block_m 128)
    is also held to the bf16 streaming path (block_m 16, no fp16 anywhere) with
    the floor taken per row: |y128 - y16| <= 2e-2 * max(rowmax / 32, |y16|) (a
    normalisation slip would be off by O(rowmax))."""
    c = synthetic.random_case("range", T=200, H=384, I=128, E=4, topk=2, block_m=128, seed=21)
    x = synthetic.bf16_bits_to_f32(c.x).astype(np.float64)
    r = (np.arange(c.T) % 9) * 4 - 24
    x = x * np.exp2(r - 20.0)[:, None]
    x[33, 5] = np.exp2(-20.0 - 40.0 + float(r[33]))  # 2^40 below its row
    c.x = synthetic.to_bf16_bits(x.astype(np.float32))
    s13 = synthetic.bf16_bits_to_f32(c.w13_s).astype(np.float64) * 2.0 ** 20
    G = c.H // 32
    s13[:, 3, :] = 2.0 ** (13 - np.linspace(0, 20, G))
    c.w13_s = synthetic.to_bf16_bits(s13.astype(np.float32))
    c.w2_s = synthetic.to_bf16_bits(synthetic.bf16_bits_to_f32(c.w2_s) * np.float32(2.0 ** -10))
    say("layer wide dynamic range bm128")
    d = DeviceCase(c)
    ref = oracle_rows(c)
    y128, y16 = d.forward(128), d.forward(16)
    parity(y128, ref, "wide range bm128")
    parity(y16, ref, "wide range bm16")
    a, b = bf16_to_f64(y128), bf16_to_f64(y16)
    floor = np.abs(b).max(axis=1, keepdims=True) / 32
    assert floor.max() > 1.0 and floor[floor > 0].min() < 1e-15
    err, tol = np.abs(a - b), 2e-2 * np.maximum(floor, np.abs(b))
    say(f"  wide range bm128 vs bm16, per-row floor: max err/tol {(err / np.maximum(tol, 1e-300)).max():.4f}")
    assert np.all(err <= tol), f"{(err > tol).sum()} elements differ beyond the per-row bound"


def test_tokens_without_resident_expert_are_zero():
    c = synthetic.random_case("holes", T=50, H=256, I=64, E=6, topk=3, block_m=16, seed=7, E_global=30)
    ids = c.topk_ids.copy()
    ids[::4] = 29  # these tokens have no resident expert
    ids[1, 0] = -1
    d = DeviceCase(c)
    out = d.forward(16, ids=to_dev(ids))
    assert np.all(out[::4] == 0)
    parity(out, oracle_rows(c, ids=ids), "holes")


@pytest.mark.parametrize("bm", [32, 128])
def test_stages_equal_forward_and_deterministic(bm):
    c = synthetic.random_case("stages", T=90, H=512, I=128, E=10, topk=4, block_m=bm, seed=11, E_global=20)
    d = DeviceCase(c)
    ref = d.forward(bm)
    again = d.forward(bm)
    assert np.array_equal(ref, again)
    buf = d.align(bm)
    cap = buf["sorted_token_ids"].numel()
    h = torch.zeros((cap, c.I), dtype=torch.int16, device="cuda")
    y = torch.zeros((c.T * c.topk, c.H), dtype=torch.float32, device="cuda")
    out = torch.full((c.T, c.H), -1, dtype=torch.int16, device="cuda")
    nws = w.w4a16_moe_stage_workspace_bytes(d.shape, c.T, c.topk, bm)
    assert (nws > 0) == (bm == 128)
    ws = torch.zeros(nws, dtype=torch.uint8, device="cuda") if nws else None
    srt, eid, ntpp = buf["sorted_token_ids"], buf["expert_ids"], buf["num_tokens_post_padded"]
    w.w4a16_moe_prepare_x(d.shape, d.x, d.ids, bm, ws)
    w.w4a16_moe_gate_up(d.shape, d.x, c.T, c.topk, srt, eid, ntpp, bm, d.w13p, h, ws)
    w.w4a16_moe_prepare_h(d.shape, c.T, c.topk, h, srt, ntpp, bm, ws)
    w.w4a16_moe_down(d.shape, c.T, c.topk, h, srt, eid, ntpp, bm, d.w2p, y, ws)
    w.w4a16_moe_combine(d.shape, d.ids, d.wts, y, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint16), ref)


def test_zero_tokens():
    c = synthetic.random_case("empty", T=4, H=256, I=64, E=4, topk=2, block_m=16, seed=3)
    d = DeviceCase(c)
    ids = torch.empty((0, 2), dtype=torch.int32, device="cuda")
    wts = torch.empty((0, 2), dtype=torch.float32, device="cuda")
    x = torch.empty((0, 256), dtype=torch.int16, device="cuda")
    assert d.forward(16, ids=ids, wts=wts, x=x).shape == (0, 256)


# 48 experts x 128 rows (contiguous routing) with more 128 x 256 tiles than
# resident workgroups, so every workgroup runs several tiles. Each GEMM stage
# is checked on the very rows it was given (the exact projections of those
# rows), so a wrong tile shows at once with a bound far tighter than the
# layer's, whatever the bf16 rounding of h does elsewhere: with I = 128 the
# layer output itself can exceed the layer bound on a few elements of a row
# whose h has one element rounded the other way on the two sides.
TILED_STAGES = [
    ("gate_up many tiles", 128, 2048),   # gate_up: 768 tiles of 2 stages; down streamed (H < 256)
    ("down many tiles", 7168, 128),      # down: 1344 tiles of 2 stages; gate_up 48 tiles of 112
]


@pytest.mark.parametrize("name,H,I", TILED_STAGES, ids=[s[0] for s in TILED_STAGES])
def test_tiled_stages_on_own_rows(name, H, I):
    c = synthetic.contiguous_case(seed=7, H=H, I=I)
    bm, T, k = c.block_m, c.T, c.topk
    say(f"layer {name}: T={T} H={H} I={I} E={c.E} bm={bm}")
    d = DeviceCase(c)
    buf = d.align(bm)
    srt, eid, ntpp = buf["sorted_token_ids"], buf["expert_ids"], buf["num_tokens_post_padded"]
    h = torch.zeros((srt.numel(), I), dtype=torch.int16, device="cuda")
    y = torch.zeros((T * k, H), dtype=torch.float32, device="cuda")
    out = torch.full((T, H), -1, dtype=torch.int16, device="cuda")
    ws = torch.empty(w.w4a16_moe_stage_workspace_bytes(d.shape, T, k, bm), dtype=torch.uint8, device="cuda")
    w.w4a16_moe_prepare_x(d.shape, d.x, d.ids, bm, ws)
    w.w4a16_moe_gate_up(d.shape, d.x, T, k, srt, eid, ntpp, bm, d.w13p, h, ws)
    w.w4a16_moe_prepare_h(d.shape, T, k, h, srt, ntpp, bm, ws)
    w.w4a16_moe_down(d.shape, T, k, h, srt, eid, ntpp, bm, d.w2p, y, ws)
    w.w4a16_moe_combine(d.shape, d.ids, d.wts, y, out)
    torch.cuda.synchronize()
    n = int(ntpp.item())
    rows = np.arange(n)
    slot = srt.cpu().numpy()[:n]
    real = slot < T * k
    rows, slot = rows[real], slot[real]
    ex = eid.cpu().numpy()[rows // bm]
    # gate_up: h = bf16(silu(g) * u) with g, u the exact fp64 projections of the row's token
    g = oracle.expert_rows(c.x[slot // k], ex, c.w13_q, c.w13_s, 2 * I, H)
    h_exact = g[:, :I] / (1.0 + np.exp(-g[:, :I])) * g[:, I:]
    h_gpu = bf16_to_f64(h.cpu().numpy()[rows])
    err = np.abs(h_gpu - h_exact)
    tol = 2.0**-6 * np.abs(h_exact) + 1e-4
    say(f"  gate_up rows: max err/tol {float((err / tol).max()):.4f}")
    assert np.all(err <= tol), f"{name}: gate_up rows off, e.g. {np.argwhere(err > tol)[:5].tolist()}"
    # down: y = h . W2^T of the GPU's own h rows, in fp32 against fp64
    y_ref = oracle.expert_rows(h.cpu().numpy()[rows].view(np.uint16), ex, c.w2_q, c.w2_s, H, I)
    y_gpu = y.cpu().numpy()[slot].astype(np.float64)
    err = np.abs(y_gpu - y_ref)
    tol = 1e-4 * (np.abs(y_ref) + np.abs(y_ref).max(axis=1, keepdims=True))
    say(f"  down rows: max err/tol {float((err / tol).max()):.4f}")
    assert np.all(err <= tol), f"{name}: down rows off, e.g. {np.argwhere(err > tol)[:5].tolist()}"
    # the one-call layer gives the same bits, run after run
    one = d.forward(bm)
    assert np.array_equal(out.cpu().numpy().view(np.uint16), one)
    assert np.array_equal(one, d.forward(bm)), "run-to-run difference"


FULL = ["decode_ep48", "islice_tp8", "prefill_contig48", "prefill_skew48"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    say(f"layer full-size {name}: building inputs")
    c = synthetic.workload(name)
    d = DeviceCase(c)
    say(f"layer full-size {name}: T={c.T} E={c.E} bm={c.block_m} slots={c.local_slots()}")
    out = d.forward(c.block_m)
    # sample tokens: the busiest, some with several resident slots, some with none, random others
    rng = np.random.default_rng(0)
    local = ((c.topk_ids >= 0) & (c.topk_ids < c.E)).sum(axis=1)
    order = np.argsort(-local, kind="stable")
    pick = set(order[:4].tolist()) | set(rng.choice(c.T, size=8, replace=False).tolist())
    none = np.nonzero(local == 0)[0]
    pick |= set(none[:2].tolist())
    tokens = np.array(sorted(pick), np.int32)
    ref = oracle_rows(c, tokens=tokens)
    parity(out[tokens], ref, f"{name} ({len(tokens)} sampled tokens)")
    assert np.all(out[none] == 0)
    d2 = d.forward(c.block_m)
    assert np.array_equal(out, d2), "run-to-run difference"


@pytest.mark.parametrize("name", FULL)
def test_full_size_every_row(name):
    """Every row of the full-size workload, not a sample: both GEMMs on every real aligned row
    against the exact fp64 projections of that row's own inputs (check_own_rows), then the combine
    of every token from the GPU's own fp32 y rows against their fp64 weighted sum (one bf16
    rounding apart at most), the staged sequence equal to the one-call forward bit for bit, and the
    layer output of every token against the oracle at the stated tolerance."""
    c = synthetic.workload(name)
    d = DeviceCase(c)
    bm = c.block_m
    buf = d.align(bm)
    srt, eid, ntpp = buf["sorted_token_ids"], buf["expert_ids"], buf["num_tokens_post_padded"]
    say(f"layer full-size every row {name}: T={c.T} slots={c.local_slots()} bm={bm} "
        f"row blocks {int(ntpp.item()) // bm}")
    h, y = run_stages(d, bm, srt, eid, ntpp, c.T, c.topk)
    rows, slot, ex, h_bits, flips, row_flip, y_own = check_own_rows(c, c.x, h, y, srt, eid, ntpp, bm, c.topk,
                                                                   f"{name} full size", detail=True)
    out = torch.full((c.T, c.H), -1, dtype=torch.int16, device="cuda")
    w.w4a16_moe_combine(d.shape, d.ids, d.wts, y, out)
    torch.cuda.synchronize()
    out_bits = out.cpu().numpy().view(np.uint16)
    assert np.array_equal(out_bits, d.forward(bm)), "staged sequence differs from forward"
    # combine: the weighted sum over resident slots of the GPU's own y rows, exact in fp64;
    # the GPU sums in fp32 in j order (each of the <= topk additions rounds by at most 2^-24 of
    # the sum of |w y| so far) and rounds the result to bf16 once (half an ulp, one ulp allowed)
    yh = y.cpu().numpy().reshape(c.T, c.topk, c.H)
    res = (c.topk_ids >= 0) & (c.topk_ids < c.E)
    o64 = np.zeros((c.T, c.H))
    mag = np.zeros((c.T, c.H))
    for j in range(c.topk):
        m = res[:, j]
        term = c.topk_weights[m, j].astype(np.float32).astype(np.float64)[:, None] * yh[m, j].astype(np.float64)
        o64[m] += term
        mag[m] += np.abs(term)
    o = bf16_to_f64(out_bits)
    ulp = np.zeros_like(o64)
    nz = o64 != 0
    ulp[nz] = 2.0 ** (np.floor(np.log2(np.abs(o64[nz]))) - 7)
    tol = ulp + c.topk * 2.0**-24 * mag
    err = np.abs(o - o64)
    say(f"  {name} combine of every token: max err/tol {float((err / np.maximum(tol, 1e-300)).max()):.3f}")
    assert np.all(err <= tol), f"{name}: combine off, e.g. {np.argwhere(err > tol)[:5].tolist()}"
    # The layer of every token: against the layer recomputed exactly (fp64) from the GPU's own h
    # rows, at the stated tolerance everywhere; against the oracle (h rounded from fp64 g, u), at
    # the stated tolerance everywhere except in tokens where some h element of a resident slot
    # rounded to the other bf16 neighbour (the GPU's g, u are fp32 sums), which shifts the whole
    # output row by ulp(h_i) * w2[:, i] * weight. Such elements are counted and reported.
    o_own = np.zeros((c.T, c.H))
    tok_flip = np.zeros(c.T, bool)
    wts64 = c.topk_weights.astype(np.float32).astype(np.float64)
    for r, sl in enumerate(slot):
        t, j = divmod(int(sl), c.topk)
        o_own[t] += wts64[t, j] * y_own[r]
        tok_flip[t] |= bool(row_flip[r])
    parity(out_bits, o_own, f"{name} (every token, on the GPU's own h)")
    say(f"  {name}: oracle over all {c.T} tokens")
    ref = oracle_rows(c)
    g = bf16_to_f64(out_bits)
    tol = 2e-2 * np.maximum(1.0, np.abs(ref))
    over = np.abs(g - ref) > tol
    n_over, t_over = int(over.sum()), np.unique(np.nonzero(over)[0])
    shift = float((np.abs(o_own - ref)[over] / tol[over]).max()) if n_over else 0.0
    say(f"  {name} (every token) against the oracle: {n_over}/{over.size} elements beyond the stated bound "
        f"(max err/tol {float((np.abs(g - ref) / tol).max()):.3f}), in tokens {t_over.tolist()[:10]}; there the "
        f"exact layer on the GPU's own h is already {shift:.3f} x tol from the oracle; tokens with an h element "
        f"on the other bf16 neighbour: {int(tok_flip.sum())}/{c.T}")
    assert np.all(np.isfinite(g))
    assert np.all(tok_flip[t_over]), "an element beyond the bound in a token without an h rounding flip"


def test_split_k_several_units_per_workgroup():
    """block_m 16 at the Kimi-K2 shapes (both reductions split between two waves per
    n-block) with far more live units than the persistent grid's workgroups: 400
    tokens routed top-8 over 48 local experts give about 240 row blocks, so each
    workgroup runs two (gate_up) or four (down) units one after the other, and the
    LDS that held one unit's partial-sum exchange is the next unit's A ring. Every
    real row of both GEMMs is checked on its own inputs, the layer on sampled
    tokens, and two runs are compared bit for bit."""
    c = synthetic.random_case("split_units", T=400, H=7168, I=2048, E=48, topk=8, block_m=16, seed=41)
    d = DeviceCase(c)
    bm = 16
    buf = d.align(bm)
    srt, eid, ntpp = buf["sorted_token_ids"], buf["expert_ids"], buf["num_tokens_post_padded"]
    n = int(ntpp.item())
    say(f"layer split-K, several units per workgroup: {n // bm} row blocks, "
        f"{n // bm * 32} gate_up units, {n // bm * 56} down units")
    assert n // bm * 32 > 4096  # more units than 256 CUs x 4 workgroups x 4
    h, y = run_stages(d, bm, srt, eid, ntpp, c.T, c.topk)
    check_own_rows(c, c.x, h, y, srt, eid, ntpp, bm, c.topk, "split-K units")
    out = d.forward(bm)
    rng = np.random.default_rng(5)
    tokens = np.array(sorted(set(rng.choice(c.T, size=10, replace=False).tolist()) | {0, c.T - 1}), np.int32)
    parity(out[tokens], oracle_rows(c, tokens=tokens), f"split-K units ({len(tokens)} sampled tokens)")
    assert np.array_equal(out, d.forward(bm)), "run-to-run difference"
    h2, y2 = run_stages(d, bm, srt, eid, ntpp, c.T, c.topk)
    assert torch.equal(h, h2) and torch.equal(y, y2), "stage run-to-run difference"
