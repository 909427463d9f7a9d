"""W4A16 fused MoE layer for MI355X (gfx950): Python binding of the C ABI.

Every function here has the name of an entry point in include/w4a16_moe.h and
does argument marshalling only: torch tensors supply device memory and the
current HIP stream; all computation runs in the library's HIP kernels. A
non-OK status raises W4A16Error.
"""
from __future__ import annotations

import ctypes

from ._lib import LIB_PATH, Shape, load

__all__ = [
    "W4A16Error", "Shape", "LIB_PATH", "load", "make_shape", "w4a16_status_string", "w4a16_packed_bytes",
    "w4a16_repack", "moe_align_capacity", "moe_align_workspace_bytes", "w4a16_choose_block_m", "moe_align",
    "moe_route_align", "moe_align_filtered", "moe_align_split", "w4a16_moe_routed_workspace_bytes", "w4a16_moe_routed_split",
    "w4a16_moe_routed_forward", "w4a16_moe_routed_forward_noalloc", "NOALLOC_SCRATCH_BYTES",
    "w4a16_moe_contiguous_workspace_bytes", "w4a16_moe_contiguous_forward",
    "w4a16_moe_masked_block_m", "w4a16_moe_masked_workspace_bytes", "w4a16_moe_masked_forward",
    "w4a16_moe_stage_workspace_bytes", "w4a16_moe_prepare_x", "w4a16_moe_prepare_h",
    "w4a16_moe_workspace_bytes", "w4a16_moe_forward", "w4a16_moe_gate_up", "w4a16_moe_down",
    "w4a16_moe_combine", "align_buffers",
]

OK = 0


class W4A16Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {w4a16_status_string(status)} (status {status})")


def make_shape(num_experts: int, hidden: int, intermediate: int, group_size: int = 32) -> Shape:
    return Shape(num_experts, hidden, intermediate, group_size)


def _p(t):
    """Device pointer of a tensor (None -> NULL)."""
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status: int, where: str):
    if status != OK:
        raise W4A16Error(status, where)


def w4a16_status_string(status: int) -> str:
    return load().w4a16_status_string(status).decode()


def w4a16_packed_bytes(shape: Shape) -> tuple[int, int]:
    a, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(load().w4a16_packed_bytes(ctypes.byref(shape), ctypes.byref(a), ctypes.byref(b)), "w4a16_packed_bytes")
    return a.value, b.value


def w4a16_repack(shape: Shape, w13_q, w13_s, w2_q, w2_s, w13_packed, w2_packed, stream=None):
    _check(load().w4a16_repack(ctypes.byref(shape), _p(w13_q), _p(w13_s), _p(w2_q), _p(w2_s), _p(w13_packed),
                               _p(w2_packed), _stream(stream)), "w4a16_repack")


def moe_align_capacity(T: int, topk: int, num_experts: int, block_m: int) -> int:
    return load().moe_align_capacity(T, topk, num_experts, block_m)


def moe_align_workspace_bytes(T: int, topk: int, num_experts: int, block_m: int) -> int:
    return load().moe_align_workspace_bytes(T, topk, num_experts, block_m)


def w4a16_choose_block_m(T: int, topk: int, num_experts_local: int, num_experts_global: int) -> int:
    return load().w4a16_choose_block_m(T, topk, num_experts_local, num_experts_global)


def moe_align(topk_ids, num_experts: int, block_m: int, sorted_token_ids, expert_ids, num_tokens_post_padded,
              expert_counts=None, workspace=None, stream=None):
    T, topk = topk_ids.shape
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().moe_align(_p(topk_ids), T, topk, num_experts, block_m, _p(sorted_token_ids),
                            sorted_token_ids.numel(), _p(expert_ids), _p(num_tokens_post_padded),
                            _p(expert_counts), _p(workspace), nbytes, _stream(stream)), "moe_align")


def moe_route_align(logits, topk: int, num_experts: int, block_m: int, topk_ids, topk_weights, sorted_token_ids,
                    expert_ids, num_tokens_post_padded, bias=None, expert_counts=None, workspace=None, stream=None):
    T, Eg = logits.shape
    _check(load().moe_route_align(_p(logits), _p(bias), T, Eg, topk, num_experts, block_m, _p(topk_ids),
                                  _p(topk_weights), _p(sorted_token_ids), sorted_token_ids.numel(), _p(expert_ids),
                                  _p(num_tokens_post_padded), _p(expert_counts), _p(workspace), _nbytes(workspace),
                                  _stream(stream)), "moe_route_align")


def w4a16_moe_contiguous_workspace_bytes(shape: Shape, M: int) -> int:
    return load().w4a16_moe_contiguous_workspace_bytes(ctypes.byref(shape), M)


def w4a16_moe_contiguous_forward(shape: Shape, x, m_indices, w13_packed, w2_packed, out, workspace, stream=None):
    M = x.shape[0]
    _check(load().w4a16_moe_contiguous_forward(ctypes.byref(shape), _p(x), M, _p(m_indices), _p(w13_packed),
                                               _p(w2_packed), _p(out), _p(workspace), _nbytes(workspace),
                                               _stream(stream)), "w4a16_moe_contiguous_forward")


def w4a16_moe_masked_block_m(max_m: int, expected_m: int) -> int:
    return load().w4a16_moe_masked_block_m(max_m, expected_m)


def w4a16_moe_masked_workspace_bytes(shape: Shape, max_m: int, block_m: int) -> int:
    return load().w4a16_moe_masked_workspace_bytes(ctypes.byref(shape), max_m, block_m)


def w4a16_moe_masked_forward(shape: Shape, x, masked_m, block_m: int, w13_packed, w2_packed, out, workspace,
                             stream=None):
    max_m = x.shape[1]
    _check(load().w4a16_moe_masked_forward(ctypes.byref(shape), _p(x), max_m, _p(masked_m), block_m,
                                           _p(w13_packed), _p(w2_packed), _p(out), _p(workspace),
                                           _nbytes(workspace), _stream(stream)), "w4a16_moe_masked_forward")


def moe_align_filtered(topk_ids, num_experts: int, block_m: int, min_count: int, max_count: int, sorted_token_ids,
                       expert_ids, num_tokens_post_padded, expert_counts=None, workspace=None, stream=None):
    T, topk = topk_ids.shape
    _check(load().moe_align_filtered(_p(topk_ids), T, topk, num_experts, block_m, min_count, max_count,
                                     _p(sorted_token_ids), sorted_token_ids.numel(), _p(expert_ids),
                                     _p(num_tokens_post_padded), _p(expert_counts), _p(workspace), _nbytes(workspace),
                                     _stream(stream)), "moe_align_filtered")


def moe_align_split(topk_ids, num_experts: int, split_count: int, heavy_block_m: int, heavy_capacity: int,
                    heavy_expert_ids, heavy_num_tokens_post_padded, light_block_m: int, light_expert_ids,
                    light_num_tokens_post_padded, sorted_token_ids, workspace=None, stream=None):
    """Heavy and light alignments in one pass; sorted_token_ids holds the heavy set's
    heavy_capacity ids, then the light set's (the rest of the tensor)."""
    T, topk = topk_ids.shape
    light_capacity = sorted_token_ids.numel() - heavy_capacity
    _check(load().moe_align_split(_p(topk_ids), T, topk, num_experts, split_count, heavy_block_m, heavy_capacity,
                                  _p(heavy_expert_ids), _p(heavy_num_tokens_post_padded), light_block_m,
                                  light_capacity, _p(light_expert_ids), _p(light_num_tokens_post_padded),
                                  _p(sorted_token_ids), _p(workspace), _nbytes(workspace), _stream(stream)),
           "moe_align_split")


def w4a16_moe_routed_workspace_bytes(shape: Shape, T: int, topk: int, num_experts_global: int) -> int:
    return load().w4a16_moe_routed_workspace_bytes(ctypes.byref(shape), T, topk, num_experts_global)


def w4a16_moe_routed_split(shape: Shape, T: int, topk: int, num_experts_global: int) -> int:
    return load().w4a16_moe_routed_split(ctypes.byref(shape), T, topk, num_experts_global)


def w4a16_moe_routed_forward(shape: Shape, x, topk_ids, topk_weights, num_experts_global: int, w13_packed, w2_packed,
                             out, workspace, stream=None):
    T, topk = topk_ids.shape
    _check(load().w4a16_moe_routed_forward(ctypes.byref(shape), _p(x), T, topk, num_experts_global, _p(topk_ids),
                                           _p(topk_weights), _p(w13_packed), _p(w2_packed), _p(out), _p(workspace),
                                           _nbytes(workspace), _stream(stream)), "w4a16_moe_routed_forward")


# W4A16_NOALLOC_SCRATCH_BYTES of include/w4a16_moe.h
NOALLOC_SCRATCH_BYTES = 64 << 20


def w4a16_moe_routed_forward_noalloc(shape: Shape, x, topk_ids, topk_weights, num_experts_global: int, w13_packed,
                                     w2_packed, out, stream=None):
    T, topk = topk_ids.shape
    _check(load().w4a16_moe_routed_forward_noalloc(ctypes.byref(shape), _p(x), T, topk, num_experts_global,
                                                   _p(topk_ids), _p(topk_weights), _p(w13_packed), _p(w2_packed),
                                                   _p(out), _stream(stream)), "w4a16_moe_routed_forward_noalloc")


def w4a16_moe_workspace_bytes(shape: Shape, T: int, topk: int, block_m: int) -> int:
    return load().w4a16_moe_workspace_bytes(ctypes.byref(shape), T, topk, block_m)


def w4a16_moe_forward(shape: Shape, x, topk_ids, topk_weights, sorted_token_ids, expert_ids, num_tokens_post_padded,
                      block_m: int, w13_packed, w2_packed, out, workspace, stream=None):
    T, topk = topk_ids.shape
    nbytes = workspace.numel() * workspace.element_size()
    _check(load().w4a16_moe_forward(ctypes.byref(shape), _p(x), T, topk, _p(topk_ids), _p(topk_weights),
                                    _p(sorted_token_ids), sorted_token_ids.numel(), _p(expert_ids),
                                    _p(num_tokens_post_padded), block_m, _p(w13_packed), _p(w2_packed), _p(out),
                                    _p(workspace), nbytes, _stream(stream)), "w4a16_moe_forward")


def w4a16_moe_stage_workspace_bytes(shape: Shape, T: int, topk: int, block_m: int) -> int:
    return load().w4a16_moe_stage_workspace_bytes(ctypes.byref(shape), T, topk, block_m)


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def w4a16_moe_prepare_x(shape: Shape, x, topk_ids, block_m: int, workspace=None, stream=None):
    T, topk = topk_ids.shape
    _check(load().w4a16_moe_prepare_x(ctypes.byref(shape), _p(x), T, topk, _p(topk_ids), block_m, _p(workspace),
                                      _nbytes(workspace), _stream(stream)), "w4a16_moe_prepare_x")


def w4a16_moe_gate_up(shape: Shape, x, T: int, topk: int, sorted_token_ids, expert_ids, num_tokens_post_padded,
                      block_m: int, w13_packed, h, workspace=None, stream=None):
    _check(load().w4a16_moe_gate_up(ctypes.byref(shape), _p(x), T, topk, _p(sorted_token_ids),
                                    sorted_token_ids.numel(), _p(expert_ids), _p(num_tokens_post_padded), block_m,
                                    _p(w13_packed), _p(h), _p(workspace), _nbytes(workspace), _stream(stream)),
           "w4a16_moe_gate_up")


def w4a16_moe_prepare_h(shape: Shape, T: int, topk: int, h, sorted_token_ids, num_tokens_post_padded, block_m: int,
                        workspace=None, stream=None):
    _check(load().w4a16_moe_prepare_h(ctypes.byref(shape), T, topk, _p(h), _p(sorted_token_ids),
                                      sorted_token_ids.numel(), _p(num_tokens_post_padded), block_m, _p(workspace),
                                      _nbytes(workspace), _stream(stream)), "w4a16_moe_prepare_h")


def w4a16_moe_down(shape: Shape, T: int, topk: int, h, sorted_token_ids, expert_ids, num_tokens_post_padded,
                   block_m: int, w2_packed, y, workspace=None, stream=None):
    _check(load().w4a16_moe_down(ctypes.byref(shape), T, topk, _p(h), _p(sorted_token_ids), sorted_token_ids.numel(),
                                 _p(expert_ids), _p(num_tokens_post_padded), block_m, _p(w2_packed), _p(y),
                                 _p(workspace), _nbytes(workspace), _stream(stream)), "w4a16_moe_down")


def w4a16_moe_combine(shape: Shape, topk_ids, topk_weights, y, out, stream=None):
    T, topk = topk_ids.shape
    _check(load().w4a16_moe_combine(ctypes.byref(shape), T, topk, _p(topk_ids), _p(topk_weights), _p(y), _p(out),
                                    _stream(stream)), "w4a16_moe_combine")


def align_buffers(T: int, topk: int, num_experts: int, block_m: int, device="cuda"):
    """Allocate (torch) the alignment outputs and workspace for one call."""
    import torch

    cap = moe_align_capacity(T, topk, num_experts, block_m)
    if cap == 0 and T * topk + num_experts * (block_m - 1) != 0:
        raise W4A16Error(2, "moe_align_capacity")
    nblk = (cap + block_m - 1) // block_m
    ws = moe_align_workspace_bytes(T, topk, num_experts, block_m)
    return dict(
        sorted_token_ids=torch.empty(max(cap, 1), dtype=torch.int32, device=device)[:cap],
        expert_ids=torch.empty(max(nblk, 1), dtype=torch.int32, device=device)[:nblk],
        num_tokens_post_padded=torch.empty(1, dtype=torch.int32, device=device),
        expert_counts=torch.empty(num_experts, dtype=torch.int32, device=device),
        workspace=torch.empty(max(ws, 1), dtype=torch.uint8, device=device) if ws else None,
    )
