"""GPU grouped-layout entry points (w4a16_moe_contiguous_forward,
w4a16_moe_masked_forward) vs the oracle's grouped layouts, element by element
within the layer tolerance; padding and masked-off rows exactly zero; every row
written; deterministic."""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from _gpu import DeviceCase, check_own_rows, parity, run_stages, say, to_dev

import w4a16_grouped_gemm_amd as w

pytestmark = pytest.mark.gpu


def contiguous_layout(counts, pad=128, junk=None):
    """m_indices for experts with the given live row counts, each padded to `pad` rows;
    padding rows get -1, or the id `junk` (an id outside the local experts)."""
    m = []
    for e, n in enumerate(counts):
        tot = -(-n // pad) * pad
        m += [e] * n + [(-1 if junk is None else junk)] * (tot - n)
    return np.array(m, np.int32)


def run_contiguous(d, x_bits, m):
    M = len(m)
    x = to_dev(x_bits)
    mi = to_dev(m)
    ws = torch.empty(max(1, w.w4a16_moe_contiguous_workspace_bytes(d.shape, M)), dtype=torch.uint8, device="cuda")
    out = torch.full((M, d.case.H), -1, dtype=torch.int16, device="cuda")  # poison: every row must be written
    w.w4a16_moe_contiguous_forward(d.shape, x, mi, d.w13p, d.w2p, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16)


def run_masked(d, x_bits, masked, bm):
    E, max_m, H = x_bits.shape
    x = to_dev(x_bits)
    mm = to_dev(np.asarray(masked, np.int32))
    ws = torch.empty(max(1, w.w4a16_moe_masked_workspace_bytes(d.shape, max_m, bm)), dtype=torch.uint8,
                     device="cuda")
    out = torch.full((E, max_m, H), -1, dtype=torch.int16, device="cuda")
    w.w4a16_moe_masked_forward(d.shape, x, mm, bm, d.w13p, d.w2p, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16).reshape(E * max_m, H)


@pytest.fixture(scope="module")
def small():
    # weights only: x comes from each test
    c = synthetic.random_case("grouped_small", T=1, H=256, I=128, E=8, topk=1, block_m=128, seed=21)
    return DeviceCase(c)


@pytest.mark.parametrize("junk", [None, 11])
def test_contiguous_small(small, junk):
    c = small.case
    m = contiguous_layout([3, 130, 0, 128, 1, 0, 0, 255], junk=junk)
    say(f"grouped contiguous small: M={len(m)} junk={junk}")
    x = synthetic.make_x(len(m), c.H, seed=22)
    out = run_contiguous(small, x, m)
    ref = oracle.grouped_contiguous(x, m, c.w13_q, c.w13_s, c.w2_q, c.w2_s, c.E, c.I)
    parity(out, ref, "contiguous small", row_floor=True)
    assert np.all(out[(m < 0) | (m >= c.E)] == 0)
    assert np.array_equal(out, run_contiguous(small, x, m)), "run-to-run difference"


def test_contiguous_row_breaking_the_block_rule_is_zero(small):
    c = small.case
    m = contiguous_layout([100, 128])
    m[110] = 1  # a live row of expert 1 inside expert 0's padded block
    say("grouped contiguous: block-rule violation")
    x = synthetic.make_x(len(m), c.H, seed=23)
    out = run_contiguous(small, x, m)
    assert np.all(out[110] == 0)
    m_ref = m.copy()
    m_ref[110] = -1
    ref = oracle.grouped_contiguous(x, m_ref, c.w13_q, c.w13_s, c.w2_q, c.w2_s, c.E, c.I)
    parity(out, ref, "contiguous, rule-breaking row as padding", row_floor=True)


def test_contiguous_empty(small):
    say("grouped contiguous: M = 0")
    out = run_contiguous(small, np.zeros((0, small.case.H), np.uint16), np.zeros(0, np.int32))
    assert out.shape == (0, small.case.H)


@pytest.mark.parametrize("max_m,bm", [(32, 32), (32, 16), (128, 128), (64, 64)])
def test_masked_small(small, max_m, bm):
    c = small.case
    masked = np.array([0, 1, 5, 16, 17, max_m, max_m - 1, max_m + 9], np.int32)
    say(f"grouped masked small: max_m={max_m} bm={bm}")
    x = synthetic.make_x(c.E * max_m, c.H, seed=24 + max_m).reshape(c.E, max_m, c.H)
    out = run_masked(small, x, masked, bm)
    ref = oracle.grouped_masked(x, masked, c.w13_q, c.w13_s, c.w2_q, c.w2_s, c.I)
    parity(out, ref, f"masked max_m={max_m} bm={bm}", row_floor=True)
    ids = oracle.masked_row_ids(masked, max_m)
    assert np.all(out[ids < 0] == 0)


@pytest.fixture(scope="module")
def kimi48():
    say("grouped full-size: building the 48-expert Kimi-K2 slice (H 7168, I 2048)")
    c = synthetic.workload("prefill_contig48")
    return DeviceCase(c)


def test_contiguous_full_size_sampled(kimi48):
    """Contiguous prefill at 128 rows per expert over the 48-expert slice (M = 6144)."""
    c = kimi48.case
    slots = np.argsort(c.topk_ids.reshape(-1), kind="stable")  # slots grouped by expert, slot order inside
    m = c.topk_ids.reshape(-1)[slots].astype(np.int32)
    counts = np.bincount(m, minlength=c.E)
    assert np.all(counts % 128 == 0), "the workload holds 128 rows per expert"
    x = c.x[slots // c.topk]
    say(f"grouped contiguous full: M={len(m)}")
    out = run_contiguous(kimi48, x, m)
    rng = np.random.default_rng(3)
    rows = np.array(sorted(set(rng.choice(len(m), size=14, replace=False).tolist()) | {0, len(m) - 1}), np.int32)
    ref = oracle.grouped_contiguous(x, m, c.w13_q, c.w13_s, c.w2_q, c.w2_s, c.E, c.I, rows=rows)
    parity(out[rows], ref, f"contiguous full ({len(rows)} sampled rows)", row_floor=True)
    assert np.array_equal(out, run_contiguous(kimi48, x, m)), "run-to-run difference"


def test_masked_full_size_sampled(kimi48):
    """Masked decode, 32-row budget per expert over the same 48 experts."""
    c = kimi48.case
    max_m = 32
    rng = np.random.default_rng(4)
    masked = rng.integers(0, max_m + 1, size=c.E).astype(np.int32)
    masked[:3] = [0, max_m, 1]
    bm = w.w4a16_moe_masked_block_m(max_m, 32)
    x = synthetic.make_x(c.E * max_m, c.H, seed=25).reshape(c.E, max_m, c.H)
    say(f"grouped masked full: E={c.E} max_m={max_m} bm={bm}")
    out = run_masked(kimi48, x, masked, bm)
    ids = oracle.masked_row_ids(masked, max_m)
    live = np.nonzero(ids >= 0)[0]
    rows = np.array(sorted(set(rng.choice(live, size=14, replace=False).tolist()) | {int(live[0]), int(live[-1])}),
                    np.int32)
    ref = oracle.grouped_masked(x, masked, c.w13_q, c.w13_s, c.w2_q, c.w2_s, c.I, rows=rows)
    parity(out[rows], ref, f"masked full ({len(rows)} sampled rows)", row_floor=True)
    assert np.all(out[ids < 0] == 0)


def grouped_alignment(row_expert, E, bm):
    """The alignment a grouped layout stands for (readings of the contiguous and masked
    layouts): live row p is slot p of a one-slot-per-row batch, a block's expert is
    its first row's, and the padded total is the row count (the layout is padded
    already). A row whose expert differs from its block's is not live."""
    row_expert = np.asarray(row_expert, np.int32)
    M = len(row_expert)
    cap = w.moe_align_capacity(M, 1, E, bm)
    first = row_expert[(np.arange(M) // bm) * bm]
    live = (row_expert >= 0) & (row_expert < E) & (row_expert == first)
    srt = np.full(cap, M, np.int32)
    srt[np.nonzero(live)[0]] = np.nonzero(live)[0]
    eid = np.full(-(-cap // bm), -1, np.int32)
    b0 = row_expert[0:M:bm]
    eid[:len(b0)] = np.where((b0 >= 0) & (b0 < E), b0, -1)
    ids = np.where(live, row_expert, -1).astype(np.int32).reshape(M, 1)
    return to_dev(srt), to_dev(eid), to_dev(np.array([M], np.int32)), to_dev(ids), live


def own_rows_grouped(d, x_bits, row_expert, out, bm, what):
    """The grouped output against the layer's stages run on the same rows: every live
    row equals bf16_RNE of the fp32 down output of the stage path bit for bit (the
    bf16 epilogue rounds the same fp32 accumulators once), and those stages hold
    the tight own-rows bounds (h within bf16 rounding of the exact fp64 projections,
    y within 1e-4 of the exact projection of the GPU's own h). Rows that are not
    live are exactly zero."""
    c = d.case
    M = len(row_expert)
    srt, eid, ntpp, ids, live = grouped_alignment(row_expert, c.E, bm)
    x = to_dev(x_bits)
    h, y = run_stages(d, bm, srt, eid, ntpp, M, 1, row_ids=ids, x=x)
    rows, slot, ex, h_bits, flips = check_own_rows(c, x_bits, h, y, srt, eid, ntpp, bm, 1, what)
    assert np.array_equal(np.sort(slot), np.nonzero(live)[0])
    yb = synthetic.to_bf16_bits(y.cpu().numpy()[slot])
    diff = int((out[slot] != yb).sum())
    say(f"  {what}: {len(slot)} live rows, bf16 output vs bf16(y) of the stages: {diff} elements differ")
    assert diff == 0, f"{what}: the bf16 epilogue differs from bf16(y)"
    assert np.all(out[~live] == 0)
    return flips


@pytest.mark.parametrize("junk", [None, 11])
def test_contiguous_small_own_rows(small, junk):
    c = small.case
    m = contiguous_layout([3, 130, 0, 128, 1, 0, 0, 255], junk=junk)
    x = synthetic.make_x(len(m), c.H, seed=22)
    say(f"grouped contiguous small, own rows: M={len(m)} junk={junk}")
    own_rows_grouped(small, x, m, run_contiguous(small, x, m), 128, "contiguous small")


@pytest.mark.parametrize("max_m,bm", [(32, 32), (32, 16), (128, 128), (64, 64)])
def test_masked_small_own_rows(small, max_m, bm):
    c = small.case
    masked = np.array([0, 1, 5, 16, 17, max_m, max_m - 1, max_m + 9], np.int32)
    x = synthetic.make_x(c.E * max_m, c.H, seed=24 + max_m).reshape(c.E, max_m, c.H)
    say(f"grouped masked small, own rows: max_m={max_m} bm={bm}")
    out = run_masked(small, x, masked, bm)
    own_rows_grouped(small, x.reshape(c.E * max_m, c.H), oracle.masked_row_ids(masked, max_m), out, bm,
                     f"masked small max_m={max_m} bm={bm}")


def test_contiguous_full_size_own_rows(kimi48):
    """Every live row of the 48 x 128-row contiguous prefill (the tiled block_m 128
    GEMMs and their bf16 output epilogue) under the own-rows bounds."""
    c = kimi48.case
    slots = np.argsort(c.topk_ids.reshape(-1), kind="stable")
    m = c.topk_ids.reshape(-1)[slots].astype(np.int32)
    x = c.x[slots // c.topk]
    say(f"grouped contiguous full, own rows: M={len(m)}")
    flips = own_rows_grouped(kimi48, x, m, run_contiguous(kimi48, x, m), 128, "contiguous full")
    assert flips > 0  # the tolerance discussion rests on these existing at this size


def test_masked_full_size_own_rows(kimi48):
    """Every live row of the masked decode layout (32-row budget over the 48 experts,
    the block_m 32 streaming GEMMs and their bf16 output epilogue)."""
    c = kimi48.case
    max_m = 32
    rng = np.random.default_rng(4)
    masked = rng.integers(0, max_m + 1, size=c.E).astype(np.int32)
    masked[:3] = [0, max_m, 1]
    bm = w.w4a16_moe_masked_block_m(max_m, 32)
    x = synthetic.make_x(c.E * max_m, c.H, seed=25).reshape(c.E, max_m, c.H)
    say(f"grouped masked full, own rows: E={c.E} max_m={max_m} bm={bm}")
    out = run_masked(kimi48, x, masked, bm)
    own_rows_grouped(kimi48, x.reshape(c.E * max_m, c.H), oracle.masked_row_ids(masked, max_m), out, bm,
                     "masked full")
