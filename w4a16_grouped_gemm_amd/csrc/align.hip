// Token-to-expert alignment on gfx950.
//
// Groups the T*topk routed slots by expert into block_m-padded segments, in
// ascending slot order inside each expert (a stable counting sort), and labels
// each block_m-row block with its expert. These are the buffers vLLM's
// moe_align_block_size hands to the indexed W4A16 kernel (Chord page "vLLM 및
// Novita AI, Kimi K2.x용 더 빠른 INT4 MoE 커널 출시: Chord", section "런타임
// 고려사항") and that the FlashInfer Kimi-K3 fused router also emits (page
// "[flashinfer] FlashInfer, B200 GPU에서 Kimi-K3 MoE 라우터 성능 최적화", section
// "코드 분석"). Like that router, every counter is zeroed at kernel entry
// (section "커널 내부 로직 변경 (추정)"), so no workspace needs clearing.
//
// Design:
//  * histogram: LDS atomics on per-expert counters (counts are order-free, so
//    the result is deterministic);
//  * offsets: one wave scans the padded counts with lane shuffles;
//  * ranking: a 1024-thread block walks its ids in rounds of 1024; inside a
//    wave, lanes holding the same expert are found with one ballot per bit of
//    the expert id, and a lane's rank is the mbcnt of its peers below it; the
//    per-wave counts are prefix-summed across the 16 waves per expert in LDS.
//    Positions therefore depend only on the input, never on timing.
//  * small inputs (<= kSmallMax ids) run all phases in one block and one launch;
//    larger ones split the ids over blocks: histogram kernel, one-block scan
//    kernel, then a ranking/scatter kernel whose blocks start from the scanned
//    per-block bases.
#include "internal.h"

namespace w4a16 {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kSmallMax = 4096;  // ids handled by the single-launch path
constexpr int kChunk = 4096;     // ids per block in the multi-block path


// Number of set bits of `mask` in lanes below this one.
__device__ __forceinline__ int rank_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ int padded(int c, int bm) { return (c + bm - 1) / bm * bm; }

// Histogram of resident ids in [lo, hi) into LDS `hist` (zeroed by the caller).
__device__ void count_ids(const int32_t* __restrict__ ids, int lo, int hi, int E, int* hist) {
  for (int i = lo + (int)threadIdx.x; i < hi; i += kThreads) {
    const int e = ids[i];
    if ((unsigned)e < (unsigned)E) atomicAdd(&hist[e], 1);
  }
}

// Wave 0 writes off[0..E] = exclusive prefix of padded counts; off[E] = total.
__device__ void scan_offsets(const int* counts, int E, int bm, int* off) {
  if (threadIdx.x < 64) {
    const int lane = (int)threadIdx.x;
    const int per = (E + 63) / 64;
    const int start = lane * per;
    int local = 0;
    for (int k = 0; k < per; ++k) {
      const int e = start + k;
      if (e < E) local += padded(counts[e], bm);
    }
    int incl = local;
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d, 64);
      if (lane >= d) incl += v;
    }
    int run = incl - local;
    for (int k = 0; k < per; ++k) {
      const int e = start + k;
      if (e < E) {
        off[e] = run;
        run += padded(counts[e], bm);
      }
    }
    if (lane == 63) off[E] = incl;
  }
}

// Largest e in [0, E) with off[e] <= p (requires p < off[E]).
__device__ __forceinline__ int find_expert(const int* off, int E, int p) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off[mid] <= p) lo = mid; else hi = mid;
  }
  return lo;
}

// expert_ids for blocks [b0, nblk) with stride `step`; -1 past the used blocks.
__device__ void fill_expert_ids(const int* off, int E, int bm, int ntpp, int32_t* expert_ids, int nblk,
                                int b0, int step) {
  for (int b = b0; b < nblk; b += step) {
    const int p = b * bm;
    expert_ids[b] = (p < ntpp) ? find_expert(off, E, p) : -1;
  }
}

// Sentinel for every padding position in [p0, capacity) with stride `step`:
// positions past ntpp, and the tail of each expert's padded segment.
__device__ void fill_padding(const int* off, const int* counts, int E, int ntpp, int32_t* sorted, int capacity,
                             int sentinel, int p0, int step) {
  for (int p = p0; p < capacity; p += step) {
    if (p >= ntpp) {
      sorted[p] = sentinel;
    } else {
      const int e = find_expert(off, E, p);
      if (p - off[e] >= counts[e]) sorted[p] = sentinel;
    }
  }
}

// Stable scatter of the resident ids in [lo, hi): the id at flat index i goes
// to cursor[e] + (resident ids of e in [lo, i)). cursor is advanced in place.
// wtab is LDS scratch of kWaves * E ints.
__device__ void scatter_ids(const int32_t* __restrict__ ids, int lo, int hi, int E, int nbits, int* cursor,
                            int* wtab, int32_t* __restrict__ sorted) {
  const int wave = (int)threadIdx.x >> 6;
  for (int base = lo; base < hi; base += kThreads) {
    const int i = base + (int)threadIdx.x;
    const int e = (i < hi) ? ids[i] : -1;
    const bool local = (unsigned)e < (unsigned)E;
    for (int k = (int)threadIdx.x; k < kWaves * E; k += kThreads) wtab[k] = 0;
    // lanes of this wave holding the same expert: intersect one ballot per id bit
    uint64_t peers = __ballot(local);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(local && bit);
      peers &= bit ? m : ~m;
    }
    const int rank = rank_below(peers);
    __syncthreads();  // wtab cleared
    if (local && rank == 0) wtab[wave * E + e] = __popcll(peers);
    __syncthreads();  // per-wave counts visible
    for (int x = (int)threadIdx.x; x < E; x += kThreads) {
      int run = cursor[x];
      for (int w = 0; w < kWaves; ++w) {
        const int c = wtab[w * E + x];
        wtab[w * E + x] = run;
        run += c;
      }
      cursor[x] = run;
    }
    __syncthreads();  // per-wave bases visible
    if (local) sorted[wtab[wave * E + e] + rank] = i;
    __syncthreads();  // bases consumed before the next round clears wtab
  }
}

__device__ __forceinline__ int id_bits(int E) { return E > 1 ? 32 - __clz(E - 1) : 0; }

// ---- single-launch path -----------------------------------------------------
// LDS: counts[E], off[E+1], cursor[E], wtab[kWaves*E]
__global__ __launch_bounds__(kThreads) void align_small_kernel(const int32_t* __restrict__ ids, int n, int E, int bm,
                                                               int32_t* __restrict__ sorted, int capacity,
                                                               int32_t* __restrict__ expert_ids, int nblk,
                                                               int32_t* __restrict__ ntpp_out,
                                                               int32_t* __restrict__ counts_out) {
  extern __shared__ int smem[];
  int* counts = smem;
  int* off = counts + E;
  int* cursor = off + E + 1;
  int* wtab = cursor + E;
  for (int e = (int)threadIdx.x; e < E; e += kThreads) counts[e] = 0;
  __syncthreads();
  count_ids(ids, 0, n, E, counts);
  __syncthreads();
  scan_offsets(counts, E, bm, off);
  __syncthreads();
  const int ntpp = off[E];
  if (threadIdx.x == 0) *ntpp_out = ntpp;
  for (int e = (int)threadIdx.x; e < E; e += kThreads) {
    cursor[e] = off[e];
    if (counts_out) counts_out[e] = counts[e];
  }
  fill_expert_ids(off, E, bm, ntpp, expert_ids, nblk, (int)threadIdx.x, kThreads);
  fill_padding(off, counts, E, ntpp, sorted, capacity, n, (int)threadIdx.x, kThreads);
  __syncthreads();
  scatter_ids(ids, 0, n, E, id_bits(E), cursor, wtab, sorted);
}

// ---- multi-block path -------------------------------------------------------
// Workspace: hist[nchunks * E] (per-chunk counts, then per-chunk bases),
// off[E + 1], counts[E].

__global__ __launch_bounds__(kThreads) void align_hist_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                              int* __restrict__ hist) {
  extern __shared__ int smem[];
  for (int e = (int)threadIdx.x; e < E; e += kThreads) smem[e] = 0;
  __syncthreads();
  const int lo = (int)blockIdx.x * kChunk;
  count_ids(ids, lo, min(n, lo + kChunk), E, smem);
  __syncthreads();
  for (int e = (int)threadIdx.x; e < E; e += kThreads) hist[(size_t)blockIdx.x * E + e] = smem[e];
}

__global__ __launch_bounds__(kThreads) void align_scan_kernel(int* __restrict__ hist, int nchunks, int E, int bm,
                                                              int* __restrict__ off_out, int* __restrict__ counts_ws,
                                                              int32_t* __restrict__ expert_ids, int nblk,
                                                              int32_t* __restrict__ ntpp_out,
                                                              int32_t* __restrict__ counts_out) {
  extern __shared__ int smem[];
  int* counts = smem;
  int* off = counts + E;
  for (int e = (int)threadIdx.x; e < E; e += kThreads) {
    int run = 0;
    for (int b = 0; b < nchunks; ++b) {
      const int c = hist[(size_t)b * E + e];
      hist[(size_t)b * E + e] = run;  // exclusive prefix over chunks (relative to off[e])
      run += c;
    }
    counts[e] = run;
  }
  __syncthreads();
  scan_offsets(counts, E, bm, off);
  __syncthreads();
  const int ntpp = off[E];
  if (threadIdx.x == 0) *ntpp_out = ntpp;
  for (int e = (int)threadIdx.x; e <= E; e += kThreads) off_out[e] = off[e];
  for (int e = (int)threadIdx.x; e < E; e += kThreads) {
    counts_ws[e] = counts[e];
    if (counts_out) counts_out[e] = counts[e];
  }
  fill_expert_ids(off, E, bm, ntpp, expert_ids, nblk, (int)threadIdx.x, kThreads);
}

// LDS: off[E+1], counts[E], cursor[E], wtab[kWaves*E]
__global__ __launch_bounds__(kThreads) void align_scatter_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                                 const int* __restrict__ hist,
                                                                 const int* __restrict__ off_ws,
                                                                 const int* __restrict__ counts_ws,
                                                                 int32_t* __restrict__ sorted, int capacity) {
  extern __shared__ int smem[];
  int* off = smem;
  int* counts = off + E + 1;
  int* cursor = counts + E;
  int* wtab = cursor + E;
  for (int e = (int)threadIdx.x; e <= E; e += kThreads) off[e] = off_ws[e];
  for (int e = (int)threadIdx.x; e < E; e += kThreads) counts[e] = counts_ws[e];
  __syncthreads();
  for (int e = (int)threadIdx.x; e < E; e += kThreads) cursor[e] = off[e] + hist[(size_t)blockIdx.x * E + e];
  fill_padding(off, counts, E, off[E], sorted, capacity, n, (int)(blockIdx.x * kThreads + threadIdx.x),
               (int)(gridDim.x * kThreads));
  __syncthreads();
  const int lo = (int)blockIdx.x * kChunk;
  scatter_ids(ids, lo, min(n, lo + kChunk), E, id_bits(E), cursor, wtab, sorted);
}

// T == 0 or nothing to rank: every output is a sentinel.
__global__ void align_empty_kernel(int32_t* sorted, int capacity, int sentinel, int32_t* expert_ids, int nblk,
                                   int32_t* ntpp_out, int32_t* counts_out, int E) {
  const int tid = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  const int step = (int)(gridDim.x * blockDim.x);
  for (int p = tid; p < capacity; p += step) sorted[p] = sentinel;
  for (int b = tid; b < nblk; b += step) expert_ids[b] = -1;
  for (int e = tid; e < E; e += step) if (counts_out) counts_out[e] = 0;
  if (tid == 0) *ntpp_out = 0;
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace

size_t align_workspace_bytes(int64_t n, int32_t E) {
  if (n <= kSmallMax) return 0;
  const int64_t nchunks = (n + kChunk - 1) / kChunk;
  return round_up(sizeof(int) * (size_t)(nchunks * E + 2 * E + 1), 256);
}

hipError_t launch_align(const int32_t* ids, int32_t n, int32_t E, int32_t bm, int32_t* sorted, int32_t capacity,
                        int32_t* expert_ids, int32_t* ntpp, int32_t* counts, void* workspace, hipStream_t stream) {
  const int nblk = (capacity + bm - 1) / bm;
  if (n == 0) {
    const int grid = (int)std::min<int64_t>(1024, std::max<int64_t>(1, ((int64_t)capacity + 255) / 256));
    hipLaunchKernelGGL(align_empty_kernel, dim3(grid), dim3(256), 0, stream, sorted, capacity, n, expert_ids, nblk,
                       ntpp, counts, E);
    return hipGetLastError();
  }
  if (n <= kSmallMax) {
    const size_t lds = sizeof(int) * (size_t)(3 * E + 1 + kWaves * E);
    hipLaunchKernelGGL(align_small_kernel, dim3(1), dim3(kThreads), lds, stream, ids, n, E, bm, sorted, capacity,
                       expert_ids, nblk, ntpp, counts);
    return hipGetLastError();
  }
  const int nchunks = (n + kChunk - 1) / kChunk;
  int* hist = static_cast<int*>(workspace);
  int* off = hist + (size_t)nchunks * E;
  int* counts_ws = off + E + 1;
  hipLaunchKernelGGL(align_hist_kernel, dim3(nchunks), dim3(kThreads), sizeof(int) * (size_t)E, stream, ids, n, E,
                     hist);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(align_scan_kernel, dim3(1), dim3(kThreads), sizeof(int) * (size_t)(2 * E + 1), stream, hist,
                     nchunks, E, bm, off, counts_ws, expert_ids, nblk, ntpp, counts);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const size_t lds = sizeof(int) * (size_t)(3 * E + 1 + kWaves * E);
  hipLaunchKernelGGL(align_scatter_kernel, dim3(nchunks), dim3(kThreads), lds, stream, ids, n, E, hist, off,
                     counts_ws, sorted, capacity);
  return hipGetLastError();
}

}  // namespace w4a16
