"""Helpers for the GPU tests: upload a synthetic case, run the library through
the C ABI, and compare with the CPU oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import w4a16_grouped_gemm_amd as w

TOL = 2e-2  # |gpu - oracle| <= TOL * max(1, |oracle|), per element


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits).view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


class DeviceCase:
    """A MoECase resident on the GPU, weights repacked once."""

    def __init__(self, case):
        self.case = case
        self.shape = w.make_shape(case.E, case.H, case.I)
        n13, n2 = w.w4a16_packed_bytes(self.shape)
        self.w13p = torch.empty(n13, dtype=torch.uint8, device="cuda")
        self.w2p = torch.empty(n2, dtype=torch.uint8, device="cuda")
        q13, s13, q2, s2 = (to_dev(case.w13_q), to_dev(case.w13_s), to_dev(case.w2_q), to_dev(case.w2_s))
        w.w4a16_repack(self.shape, q13, s13, q2, s2, self.w13p, self.w2p)
        torch.cuda.synchronize()
        del q13, s13, q2, s2
        self.x = to_dev(case.x)
        self.ids = to_dev(case.topk_ids.astype(np.int32))
        self.wts = to_dev(case.topk_weights.astype(np.float32))

    def align(self, block_m, ids=None):
        ids = self.ids if ids is None else ids
        T, topk = ids.shape
        buf = w.align_buffers(T, topk, self.case.E, block_m)
        w.moe_align(ids, self.case.E, block_m, buf["sorted_token_ids"], buf["expert_ids"],
                    buf["num_tokens_post_padded"], buf["expert_counts"], buf["workspace"])
        return buf

    def forward(self, block_m, ids=None, wts=None, x=None):
        ids = self.ids if ids is None else ids
        wts = self.wts if wts is None else wts
        x = self.x if x is None else x
        T, topk = ids.shape
        buf = self.align(block_m, ids)
        ws = torch.empty(max(1, w.w4a16_moe_workspace_bytes(self.shape, T, topk, block_m)), dtype=torch.uint8,
                         device="cuda")
        out = torch.full((T, self.case.H), -1, dtype=torch.int16, device="cuda")  # poison: every row must be written
        w.w4a16_moe_forward(self.shape, x, ids, wts, buf["sorted_token_ids"], buf["expert_ids"],
                            buf["num_tokens_post_padded"], block_m, self.w13p, self.w2p, out, ws)
        torch.cuda.synchronize()
        return out.cpu().numpy().view(np.uint16)


def parity(gpu_bits: np.ndarray, ref: np.ndarray, what: str, row_floor: bool = False):
    """Assert the per-element bound; return the max of |err| / tol.

    row_floor: for rows that are one unweighted slot (the grouped layouts), the floor of
    the bound is also the row's largest |ref| / 32: a bf16 rounding of h that falls the
    other way on the two sides (fp32 against fp64 sums of g and u) shifts every output
    of the row by ulp(h_i) * |w2[c, i]|, an error that scales with the row, not with the
    element. In the routed layer the routing weights (< 1, over top-k slots) scale the
    same shift down, and the floor of 1 suffices."""
    g = bf16_to_f64(gpu_bits)
    tol = TOL * np.maximum(1.0, np.abs(ref))
    if row_floor and ref.size:
        tol = np.maximum(tol, TOL * np.abs(ref).max(axis=-1, keepdims=True) / 32)
    err = np.abs(g - ref)
    ratio = float((err / tol).max()) if err.size else 0.0
    nfail = int((err > tol).sum())
    bad = np.argwhere(err > tol)[:5].tolist()
    say(f"  parity {what}: max err/tol {ratio:.4f}, fails {nfail}/{err.size}")
    assert nfail == 0 and np.all(np.isfinite(g)), f"{what}: {nfail} elements out of tolerance, e.g. {bad}"
    return ratio


def run_stages(d, bm, srt, eid, ntpp, T, topk, row_ids=None, x=None):
    """The layer's GEMM stages one by one on the given alignment buffers: returns
    the GPU's h [capacity, I] (int16 bits) and y [T*topk, H] fp32 as torch tensors.
    row_ids: the per-token routed ids the prepare stage reads (default d.ids)."""
    c = d.case
    x = d.x if x is None else x
    row_ids = d.ids if row_ids is None else row_ids
    cap = srt.numel()
    h = torch.zeros((cap, c.I), dtype=torch.int16, device="cuda")
    y = torch.zeros((T * topk, c.H), dtype=torch.float32, device="cuda")
    nws = w.w4a16_moe_stage_workspace_bytes(d.shape, T, topk, bm)
    ws = torch.zeros(nws, dtype=torch.uint8, device="cuda") if nws else None
    w.w4a16_moe_prepare_x(d.shape, x, row_ids, bm, ws)
    w.w4a16_moe_gate_up(d.shape, x, T, topk, srt, eid, ntpp, bm, d.w13p, h, ws)
    w.w4a16_moe_prepare_h(d.shape, T, topk, h, srt, ntpp, bm, ws)
    w.w4a16_moe_down(d.shape, T, topk, h, srt, eid, ntpp, bm, d.w2p, y, ws)
    torch.cuda.synchronize()
    return h, y


def check_own_rows(c, x_bits, h, y, srt, eid, ntpp, bm, topk, what, detail=False):
    """Each GEMM stage on the very rows it was given, for every real aligned row:
    h = bf16(silu(g) * u) against g, u the exact fp64 projections of the row's
    activation (within bf16 rounding plus the fp32 sum's error), and y against
    the exact fp64 projection of the GPU's own h row. Returns (rows, slots, experts,
    h rows as bf16 bits, number of h elements whose bf16 rounding differs from
    the exact value's); with detail, also per row whether any of its h elements
    did, and the fp64 down projection of the GPU's own h rows)."""
    import oracle

    I, H = c.I, c.H
    n = int(ntpp.item())
    s = srt.cpu().numpy()[:n]
    rows = np.nonzero(s < x_bits.shape[0] * topk)[0]
    slot = s[rows]
    ex = eid.cpu().numpy()[rows // bm]
    g = oracle.expert_rows(x_bits[slot // topk], ex, c.w13_q, c.w13_s, 2 * I, H)
    h_exact = g[:, :I] / (1.0 + np.exp(-g[:, :I])) * g[:, I:]
    h_bits = h.cpu().numpy()[rows].view(np.uint16)
    h_gpu = bf16_to_f64(h_bits)
    err = np.abs(h_gpu - h_exact)
    tol = 2.0**-6 * np.abs(h_exact) + 1e-4
    say(f"  {what} gate_up rows ({len(rows)}): max err/tol {float((err / tol).max()):.4f}")
    assert np.all(err <= tol), f"{what}: gate_up rows off, e.g. {np.argwhere(err > tol)[:5].tolist()}"
    import synthetic

    flip = h_bits != synthetic.to_bf16_bits(h_exact.astype(np.float32))
    flips = int(flip.sum())
    y_ref = oracle.expert_rows(h_bits, ex, c.w2_q, c.w2_s, H, I)
    y_gpu = y.cpu().numpy()[slot].astype(np.float64)
    err = np.abs(y_gpu - y_ref)
    tol = 1e-4 * (np.abs(y_ref) + np.abs(y_ref).max(axis=1, keepdims=True))
    say(f"  {what} down rows: max err/tol {float((err / tol).max()):.4f}; "
        f"h elements rounded to the other bf16 neighbour than the exact value: {flips}/{h_bits.size}")
    assert np.all(err <= tol), f"{what}: down rows off, e.g. {np.argwhere(err > tol)[:5].tolist()}"
    if detail:
        return rows, slot, ex, h_bits, flips, flip.any(axis=1), y_ref
    return rows, slot, ex, h_bits, flips
