// Grouped activation layouts: the two expert-grouped layouts of Chord's
// grouped kernel family (Chord page "vLLM 및 Novita AI, Kimi K2.x용 더 빠른 INT4
// MoE 커널 출시: Chord", sections "핵심 기여" and "그룹 SM90 커널 기법"):
//  * contiguous prefill: the rows are already grouped by expert, every
//    expert's group padded to a multiple of 128 rows; a per-row expert index
//    (-1 or any id outside the local experts for padding rows) says which;
//  * masked decode: a fixed budget of max_m rows per expert, [E, max_m, H],
//    of which the first masked_m[e] rows of expert e are live.
// Neither needs an alignment pass over routed ids: this kernel writes the
// alignment buffers the GEMM stages read (row position p maps to row p; one
// expert per block_m-row block, -1 for blocks without a live first row) plus
// a per-row expert id, and zeroes the output rows that are not live (the down
// GEMM writes the live ones). One thread per position, grid-strided; every
// output is written on every call.
// block_m is a power of two and, for the masked layout, divides max_m.
#include "internal.h"

#include <algorithm>

namespace w4a16 {
namespace {

__global__ __launch_bounds__(256) void grouped_index_kernel(GroupedLayout kind, const int32_t* __restrict__ m_indices,
                                                            const int32_t* __restrict__ masked_m, int32_t M,
                                                            int32_t max_m, int32_t E, int32_t bm,
                                                            int32_t* __restrict__ row_ids,
                                                            int32_t* __restrict__ sorted, int32_t capacity,
                                                            int32_t* __restrict__ expert_ids, int32_t nblk,
                                                            int32_t* __restrict__ ntpp) {
  const int t0 = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  const int step = (int)(gridDim.x * blockDim.x);
  // expert of position p, or -1 when p holds no live row
  const auto expert_of = [&](int p) -> int {
    if (p >= M) return -1;
    if (kind == kContiguous) {
      const int e = m_indices[p];
      return (unsigned)e < (unsigned)E ? e : -1;
    }
    const int e = p / max_m;
    const int live = min(max(masked_m[e], 0), max_m);
    return p - e * max_m < live ? e : -1;
  };
  for (int p = t0; p < capacity; p += step) {
    // a row is computed with its block's expert: a row whose expert differs
    // from the block's (a contiguous layout that breaks the 128-row padding
    // rule) is treated as padding and its output row is zero
    int e = expert_of(p);
    if (e >= 0 && kind == kContiguous && expert_of(p & -bm) != e) e = -1;
    sorted[p] = e >= 0 ? p : M;  // sentinel M: not a live row
    if (p < M) row_ids[p] = e;
  }
  for (int b = t0; b < nblk; b += step) expert_ids[b] = expert_of(b * bm);
  if (t0 == 0) *ntpp = M;
}

// Zeroes the rows of out [M, H] bf16 whose row_ids entry is negative, 16 bytes
// per thread and step (H is a multiple of 8).
__global__ __launch_bounds__(256) void zero_dead_rows_kernel(const int32_t* __restrict__ row_ids, int32_t M, int32_t H,
                                                             uint16_t* __restrict__ out) {
  const int64_t chunks_per_row = H / 8;
  const int64_t total = (int64_t)M * chunks_per_row;
  const uint4 zero = {0u, 0u, 0u, 0u};
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total; c += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = c / chunks_per_row;
    if (row_ids[row] < 0) reinterpret_cast<uint4*>(out)[c] = zero;
  }
}

}  // namespace

hipError_t launch_grouped_index(GroupedLayout kind, const int32_t* m_indices, const int32_t* masked_m, int32_t M,
                                int32_t max_m, int32_t E, int32_t block_m, int32_t* row_ids, int32_t* sorted, int32_t capacity, int32_t* expert_ids, int32_t* ntpp,
                                uint16_t* out, int32_t H, hipStream_t stream) {
  const int nblk = (capacity + block_m - 1) / block_m;
  const int grid = (int)std::min<int64_t>(2048, std::max<int64_t>(1, ((int64_t)capacity + 255) / 256));
  hipLaunchKernelGGL(grouped_index_kernel, dim3(grid), dim3(256), 0, stream, kind, m_indices, masked_m, M, max_m, E,
                     block_m, row_ids, sorted, capacity, expert_ids, nblk, ntpp);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !out || M == 0) return err;
  const int zgrid = (int)std::min<int64_t>(4096, ((int64_t)M * (H / 8) + 255) / 256);
  hipLaunchKernelGGL(zero_dead_rows_kernel, dim3(zgrid), dim3(256), 0, stream, row_ids, M, H, out);
  return hipGetLastError();
}

}  // namespace w4a16
