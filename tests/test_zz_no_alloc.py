"""w4a16_moe_routed_forward_noalloc (the routed layer with its workspace in the
library's static per-GPU array, for callers that cannot allocate) against
w4a16_moe_routed_forward with a caller workspace: the same bits, on two calls in
a row, the second with a smaller input; and the host-side refusal of calls that
need more scratch than the array holds."""
import ctypes

import numpy as np
import pytest
import torch

import synthetic
from _gpu import DeviceCase, say, to_dev

import w4a16_grouped_gemm_amd as w


def test_noalloc_limit_refused_on_host():
    """A call whose routed workspace exceeds the static array is refused before any
    device work (no GPU needed), with the dedicated status."""
    lib = w.load()
    shape = w.make_shape(48, 7168, 2048)
    T = 4096
    assert w.w4a16_moe_routed_workspace_bytes(shape, T, 8, 384) > w.NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(256)
    st = lib.w4a16_moe_routed_forward_noalloc(ctypes.byref(shape), fake, T, 8, 384, fake, fake, fake, fake, fake,
                                              None)
    assert st == 6 and "static array" in w.w4a16_status_string(st)
    # invalid arguments keep the routed entry point's codes
    assert lib.w4a16_moe_routed_forward_noalloc(ctypes.byref(shape), fake, 4, 8, 8, fake, fake, fake, fake, fake,
                                                None) == 1  # fewer global than local experts


def _routed(d, x, ids, wts, Eg):
    T = ids.shape[0]
    ws = torch.empty(w.w4a16_moe_routed_workspace_bytes(d.shape, T, ids.shape[1], Eg), dtype=torch.uint8,
                     device="cuda")
    out = torch.full((T, d.case.H), -1, dtype=torch.int16, device="cuda")
    w.w4a16_moe_routed_forward(d.shape, x, ids, wts, Eg, d.w13p, d.w2p, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _noalloc(d, x, ids, wts, Eg):
    out = torch.full((ids.shape[0], d.case.H), -1, dtype=torch.int16, device="cuda")
    w.w4a16_moe_routed_forward_noalloc(d.shape, x, ids, wts, Eg, d.w13p, d.w2p, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["decode_ep48", "skewed_split"])
def test_noalloc_equals_routed_two_calls(name):
    if name == "decode_ep48":
        c = synthetic.workload("decode_ep48")  # 128 tokens, top-8 over 384, 48 experts resident
    else:  # block_m 128 by the rule, heavy/light split over a Zipf-skewed expert slice
        c = synthetic.random_case("noalloc_split", T=512, H=256, I=128, E=8, topk=2, block_m=128, seed=35,
                                  E_global=16, logit_bias=synthetic.zipf_bias(16, s=1.5))
    Eg = c.meta["E_global"]
    d = DeviceCase(c)
    # the second call is smaller: the first half of the tokens
    for T in (c.T, c.T // 2):
        need = w.w4a16_moe_routed_workspace_bytes(d.shape, T, c.topk, Eg)
        say(f"noalloc {name}: T={T} needs {need / 2**20:.1f} MiB of {w.NOALLOC_SCRATCH_BYTES >> 20} MiB, "
            f"split={w.w4a16_moe_routed_split(d.shape, T, c.topk, Eg)}")
        assert need <= w.NOALLOC_SCRATCH_BYTES
        x, ids, wts = d.x[:T], d.ids[:T], d.wts[:T]
        got = _noalloc(d, x, ids, wts, Eg)
        ref = _routed(d, x, ids, wts, Eg)
        assert np.array_equal(got, ref), f"{name} T={T}: no-alloc output differs from the routed entry point"
        assert not np.any(got == -1), "every row must be written"
