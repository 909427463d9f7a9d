"""The C-ABI library builds, loads, exports every declared symbol, and rejects
bad arguments on the host (no GPU needed: validation runs before any launch)."""
import ctypes
import os
import re
import subprocess

import pytest

import w4a16_grouped_gemm_amd as w

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16_moe.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(w.LIB_PATH):
        from w4a16_grouped_gemm_amd import build
        build.build()
    return w.load()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", src, flags=re.M)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 12, names
    out = subprocess.run(["nm", "-D", "--defined-only", w.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert n in w._lib.SIGNATURES, f"binding lacks {n}"


def test_status_strings(lib):
    for code in range(7):
        assert w.w4a16_status_string(code) not in ("", "unknown status")
    assert w.w4a16_status_string(99) == "unknown status"


def test_sizes_and_heuristic(lib):
    assert w.moe_align_capacity(3, 2, 4, 16) == 6 + 4 * 15
    assert w.moe_align_capacity(0, 8, 48, 128) == 48 * 127
    assert w.moe_align_capacity(3, 2, 4, 48) == 0  # unsupported block_m
    assert w.moe_align_workspace_bytes(128, 8, 48, 16) == 0  # single-launch path
    assert w.moe_align_workspace_bytes(16384, 8, 48, 128) > 0
    s = w.make_shape(48, 7168, 2048)
    q13, q2 = w.w4a16_packed_bytes(s)
    # nibbles, bf16 scales, fp16 scales, int32 channel exponents (all sizes here are 256-byte multiples)
    assert q13 == 48 * 4096 * 7168 // 2 + 2 * 48 * 4096 * 224 * 2 + 48 * 4096 * 4
    assert q2 == 48 * 7168 * 2048 // 2 + 2 * 48 * 7168 * 64 * 2 + 48 * 7168 * 4
    cap = w.moe_align_capacity(128, 8, 48, 16)
    assert w.w4a16_moe_workspace_bytes(s, 128, 8, 16) >= cap * 2048 * 2 + 128 * 8 * 7168 * 4
    # block_m 128: plus fp16 copies of the x rows or of the aligned h rows, with a row exponent each
    cap = w.moe_align_capacity(768, 8, 48, 128)
    stage = w.w4a16_moe_stage_workspace_bytes(s, 768, 8, 128)
    assert stage >= max(768 * 7168 * 2 + 768 * 4, cap * 2048 * 2 + cap * 4)
    assert w.w4a16_moe_workspace_bytes(s, 768, 8, 128) >= cap * 2048 * 2 + 768 * 8 * 7168 * 4 + stage
    # tokens per expert drives the row-block size
    assert w.w4a16_choose_block_m(128, 8, 48, 384) == 16
    assert w.w4a16_choose_block_m(512, 8, 384, 384) == 32
    assert w.w4a16_choose_block_m(768, 8, 48, 48) == 128
    assert w.w4a16_choose_block_m(16384, 8, 48, 384) == 128
    assert w.w4a16_choose_block_m(1, 8, 48, 384) == 16
    assert w.w4a16_choose_block_m(1024, 8, 48, 384) == 32   # tok_e 21: 32 rows (64 measured 37% slower)
    assert w.w4a16_choose_block_m(1920, 8, 48, 384) == 32   # tok_e 40
    assert w.w4a16_choose_block_m(1944, 8, 48, 384) == 128  # tok_e 40.5
    assert w.w4a16_choose_block_m(8, 8, 48, 8) == 0  # local > global


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def _fwd(lib, shape, T=4, topk=2, cap=None, bm=16, ws_bytes=1 << 40, x=FAKE, ws=FAKE):
    cap = w.moe_align_capacity(T, topk, shape.num_experts, bm) if cap is None else cap
    return lib.w4a16_moe_forward(ctypes.byref(shape), x, T, topk, FAKE, FAKE, FAKE, cap, FAKE, FAKE, bm, FAKE, FAKE,
                                 FAKE, ws, ws_bytes, None)


def test_validation_status_codes(lib):
    good = w.make_shape(8, 256, 128)
    a, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert lib.w4a16_packed_bytes(ctypes.byref(w.make_shape(8, 256, 128, 64)), ctypes.byref(a), ctypes.byref(b)) == 2
    assert lib.w4a16_packed_bytes(None, ctypes.byref(a), ctypes.byref(b)) == 1
    assert lib.w4a16_packed_bytes(ctypes.byref(good), None, None) == 1
    for bad, code in [(w.make_shape(0, 256, 128), 1), (w.make_shape(8, 96, 128), 2), (w.make_shape(8, 256, 48), 2),
                      (w.make_shape(513, 256, 128), 2), (w.make_shape(8, -64, 128), 1)]:
        assert _fwd(lib, bad) == code, (bad.num_experts, bad.hidden, bad.intermediate)
    assert _fwd(lib, good, bm=48) == 2                      # unsupported block_m
    assert _fwd(lib, good, topk=33) == 2                     # topk above the maximum
    assert _fwd(lib, good, T=-1) == 1
    assert _fwd(lib, good, x=None) == 1                      # null activation
    assert _fwd(lib, good, cap=w.moe_align_capacity(4, 2, 8, 16) - 1) == 3
    assert _fwd(lib, good, ws_bytes=100) == 4
    assert _fwd(lib, good, ws=None) == 4
    odd_ptr = ctypes.c_void_p(0x1008)                        # 8-byte aligned only
    assert _fwd(lib, good, x=odd_ptr) == 1
    assert _fwd(lib, good, ws=odd_ptr) == 1
    assert lib.w4a16_moe_combine(ctypes.byref(good), 4, 2, FAKE, FAKE, FAKE, odd_ptr, None) == 1
    # alignment
    assert lib.moe_align(FAKE, 4, 2, 8, 16, FAKE, 10, FAKE, FAKE, None, None, 0, None) == 3
    assert lib.moe_align(FAKE, 4, 2, 8, 24, FAKE, 1000, FAKE, FAKE, None, None, 0, None) == 2
    assert lib.moe_align(None, 4, 2, 8, 16, FAKE, 1000, FAKE, FAKE, None, None, 0, None) == 1
    cap = w.moe_align_capacity(16384, 8, 48, 128)
    assert lib.moe_align(FAKE, 16384, 8, 48, 128, FAKE, cap, FAKE, FAKE, None, None, 0, None) == 4
    # router + alignment: (logits, bias, T, Eg, topk, E, block_m, ids, weights, sorted, cap, expert_ids, ntpp,
    # counts, workspace, workspace_bytes, stream)
    def ra(T=4, Eg=64, topk=2, E=8, bm=16, logits=FAKE, cap=1000, ws=None, wsb=0):
        return lib.moe_route_align(logits, None, T, Eg, topk, E, bm, FAKE, FAKE, FAKE, cap, FAKE, FAKE, None, ws,
                                   wsb, None)
    assert ra(Eg=4) == 1                                     # fewer routed experts than local ones
    assert ra(Eg=64, topk=33) == 2                            # topk above the maximum of 32
    assert ra(Eg=8, topk=9, E=4) == 1                         # topk > routed experts
    assert ra(Eg=1025) == 2                                   # routed experts above the maximum
    assert ra(logits=None) == 1
    assert ra(bm=8) == 2
    assert ra(cap=w.moe_align_capacity(4, 2, 8, 16) - 1) == 3
    cap = w.moe_align_capacity(16384, 8, 48, 128)
    assert ra(T=16384, Eg=384, topk=8, E=48, bm=128, cap=cap) == 4
    assert ra(T=16384, Eg=384, topk=8, E=48, bm=128, cap=cap, ws=FAKE, wsb=16) == 4
    # grouped layouts
    assert lib.w4a16_moe_contiguous_forward(ctypes.byref(good), FAKE, 100, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                                            None) == 1      # M not a multiple of 128
    assert lib.w4a16_moe_contiguous_forward(ctypes.byref(good), FAKE, 128, None, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                                            None) == 1      # null m_indices
    need = w.w4a16_moe_contiguous_workspace_bytes(good, 256)
    assert need > 0 and w.w4a16_moe_contiguous_workspace_bytes(good, 100) == 0
    assert lib.w4a16_moe_contiguous_forward(ctypes.byref(good), FAKE, 256, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1,
                                            None) == 4
    assert lib.w4a16_moe_masked_forward(ctypes.byref(good), FAKE, 40, FAKE, 16, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                                        None) == 1          # max_m not a multiple of block_m
    assert lib.w4a16_moe_masked_forward(ctypes.byref(good), FAKE, 48, FAKE, 24, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                                        None) == 2          # unsupported block_m
    need = w.w4a16_moe_masked_workspace_bytes(good, 32, 32)
    assert need > 0 and w.w4a16_moe_masked_workspace_bytes(good, 40, 16) == 0
    assert lib.w4a16_moe_masked_forward(ctypes.byref(good), FAKE, 32, FAKE, 32, FAKE, FAKE, FAKE, FAKE, need - 1,
                                        None) == 4
    # masked block_m: the tokens-per-expert rule on expected_m, halved until it divides max_m
    assert w.w4a16_moe_masked_block_m(32, 32) == 32
    assert w.w4a16_moe_masked_block_m(256, 32) == 32
    assert w.w4a16_moe_masked_block_m(64, 200) == 64       # 128 halved to divide max_m
    assert w.w4a16_moe_masked_block_m(256, 200) == 128
    assert w.w4a16_moe_masked_block_m(48, 4) == 16
    assert w.w4a16_moe_masked_block_m(40, 4) == 0          # not a multiple of 16
    # filtered alignment and the one-call routed layer
    assert lib.moe_align_filtered(FAKE, 4, 2, 8, 16, -1, 5, FAKE, 1000, FAKE, FAKE, None, None, 0, None) == 1
    assert lib.moe_align_filtered(FAKE, 4, 2, 8, 16, 6, 5, FAKE, 1000, FAKE, FAKE, None, None, 0, None) == 1
    assert lib.moe_align_filtered(FAKE, 4, 2, 8, 16, 1, 5, FAKE, 10, FAKE, FAKE, None, None, 0, None) == 3
    # split alignment: T=4, topk=2, E=8; heavy needs 8 + 8*127 = 1024, light min(8 + 8*15, 8*32) = 128
    def sp(split=32, hbm=128, hcap=1024, lbm=16, lcap=128, leids=FAKE):
        return lib.moe_align_split(FAKE, 4, 2, 8, split, hbm, hcap, FAKE, FAKE, lbm, lcap, leids, FAKE, FAKE, None, 0,
                                   None)
    assert sp(split=1) == 1
    assert sp(hbm=48) == 2 and sp(lbm=48) == 2              # unsupported block_m
    assert sp(leids=None) == 1
    assert sp(hcap=1023) == 3
    assert sp(lcap=127) == 3
    assert sp(hcap=2**31 - 100, lcap=200) == 3             # joined array beyond int32
    kimi = w.make_shape(48, 7168, 2048)
    assert w.w4a16_moe_routed_split(kimi, 16384, 8, 384) == 17     # prefill: heavy experts from 17 slots
    assert w.w4a16_moe_routed_split(kimi, 128, 8, 384) == 0        # decode: one alignment
    assert w.w4a16_moe_routed_split(kimi, 128, 8, 40) == -1        # fewer global than local experts
    need = w.w4a16_moe_routed_workspace_bytes(kimi, 16384, 8, 384)
    assert need > w.w4a16_moe_workspace_bytes(kimi, 16384, 8, 128)
    def rf(T=16384, Eg=384, x=FAKE, ws=FAKE, wsb=need):
        return lib.w4a16_moe_routed_forward(ctypes.byref(kimi), x, T, 8, Eg, FAKE, FAKE, FAKE, FAKE, FAKE, ws, wsb,
                                            None)
    assert rf(wsb=need - 1) == 4
    assert rf(x=None) == 1
    assert rf(Eg=40) == 1
    assert rf(ws=ctypes.c_void_p(0x1004)) == 1
    # repack and stages
    assert lib.w4a16_repack(ctypes.byref(good), FAKE, None, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert lib.w4a16_moe_combine(ctypes.byref(good), 4, 0, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert lib.w4a16_moe_gate_up(ctypes.byref(good), FAKE, 4, 2, FAKE, 3, FAKE, FAKE, 16, FAKE, FAKE, None, 0,
                                 None) == 3
    assert lib.w4a16_moe_gate_up(ctypes.byref(good), None, 4, 2, FAKE, 1000, FAKE, FAKE, 16, FAKE, FAKE, None, 0,
                                 None) == 1
    assert lib.w4a16_moe_down(ctypes.byref(good), 4, 2, None, FAKE, 1000, FAKE, FAKE, 16, FAKE, FAKE, None, 0,
                              None) == 1
    assert lib.w4a16_moe_prepare_x(ctypes.byref(good), FAKE, 4, 2, None, 16, None, 0, None) == 1
    assert lib.w4a16_moe_prepare_h(ctypes.byref(good), 4, 2, FAKE, FAKE, 3, FAKE, 16, None, 0, None) == 3
    # block_m 16 needs no stage scratch: the prepare stages are no-ops
    assert w.w4a16_moe_stage_workspace_bytes(good, 4, 2, 16) == 0
    assert lib.w4a16_moe_prepare_x(ctypes.byref(good), FAKE, 4, 2, FAKE, 16, None, 0, None) == 0
    # block_m 128 needs it
    need = w.w4a16_moe_stage_workspace_bytes(good, 4, 2, 128)
    assert need > 0
    cap = w.moe_align_capacity(4, 2, 8, 128)
    assert lib.w4a16_moe_prepare_x(ctypes.byref(good), FAKE, 4, 2, FAKE, 128, None, 0, None) == 4
    assert lib.w4a16_moe_prepare_h(ctypes.byref(good), 4, 2, FAKE, FAKE, cap, FAKE, 128, FAKE, need - 1, None) == 4
    assert lib.w4a16_moe_gate_up(ctypes.byref(good), FAKE, 4, 2, FAKE, cap, FAKE, FAKE, 128, FAKE, FAKE, None, 0,
                                 None) == 4
    assert lib.w4a16_moe_down(ctypes.byref(good), 4, 2, FAKE, FAKE, cap, FAKE, FAKE, 128, FAKE, FAKE, FAKE, need - 1,
                              None) == 4
    # shapes the tiled GEMMs do not take need none either (H = 320: down N % 256 != 0 but gate_up is tiled)
    odd = w.make_shape(8, 320, 96)
    assert w.w4a16_moe_stage_workspace_bytes(odd, 4, 2, 128) == 0


def test_binding_raises(lib):
    with pytest.raises(w.W4A16Error) as ei:
        w.w4a16_packed_bytes(w.make_shape(8, 256, 128, 128))
    assert ei.value.status == 2
