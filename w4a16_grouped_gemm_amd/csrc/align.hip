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
// Design (the work is tiny; the kernels are written against latency):
//  * every thread loads its ids once, up front, into registers;
//  * histogram: LDS atomics on per-expert counters (order-free, so deterministic);
//  * offsets: one wave scans the padded counts with DPP (row shifts and row
//    broadcasts, no LDS round trips);
//  * ranking: each wave owns a contiguous segment of ids and ranks it 64 at a
//    time against its own per-expert counters in LDS (lanes of one expert are
//    found with one ballot per bit of the expert id; a lane's rank is the
//    mbcnt of its peers below it); one 16-lane DPP row scan per expert across
//    the 16 waves gives the bases. Positions depend only on the input, never
//    on timing;
//  * each expert's thread labels its blocks and writes its padding sentinels
//    (no search); the unused tail is a plain fill: no per-position search over
//    the over-allocated buffer;
//  * barriers order LDS traffic only; they never wait for global stores.
// Small inputs run in one block and one launch. Larger ones use two launches:
// per-chunk histograms, then one block per chunk that recomputes the (small)
// expert prefix itself from all chunk histograms and scatters its chunk.
// A heavy/light split by per-expert count (two block sizes for skewed
// routing) shares the histogram launch and one scatter launch: each block
// scans both count bands and scatters into the two sets' joined sorted array.
#include "internal.h"
#include "w4a16_moe.h"

#include <algorithm>

namespace w4a16 {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kPerThread = 8;                        // ids per thread held in registers
constexpr int kSmallMax = kThreads * kPerThread;     // single-launch paths up to here (8192)
constexpr int kChunk = kThreads;                     // ids per block of the two-launch path
// The scatter's per-wave counters are stored expert-major, wtab[e * kWtabStride +
// wave]: the 16 waves' counters of one expert are consecutive (the per-expert
// scan reads them as one conflict-free row), and the stride of 17 puts the
// experts a wave's lanes touch in one ranking step on different LDS banks
// (a wave-major table with a row stride of E = 384 put the scan's 16 lanes on
// one bank).
constexpr int kWtabStride = kWaves + 1;

// Number of set bits of `mask` in lanes below this one.
__device__ __forceinline__ int rank_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Workgroup barrier for LDS traffic only: this wave's LDS accesses complete,
// then s_barrier. Outstanding global stores are not waited for: no thread of
// these kernels reads what another thread of its block stored to global memory.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// v + the value DPP moves in (0 where the row mask or the row bound leaves none).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_add(int v) {
  return v + __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xf, false);
}

// Inclusive prefix sum inside each row of 16 lanes (row_shr 1, 2, 4, 8); all
// 16 lanes of a row must be active.
__device__ __forceinline__ int row_incl_scan(int v) {
  v = dpp_add<0x111, 0xf>(v);
  v = dpp_add<0x112, 0xf>(v);
  v = dpp_add<0x114, 0xf>(v);
  return dpp_add<0x118, 0xf>(v);
}

// Inclusive prefix sum over the wave: row scans, then row 0's total into row 1
// and row 2's into row 3 (row_bcast:15), then rows 0-1's total into rows 2-3
// (row_bcast:31). All 64 lanes must be active.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v = row_incl_scan(v);
  v = dpp_add<0x142, 0xa>(v);
  return dpp_add<0x143, 0xc>(v);
}

__device__ __forceinline__ int padded(int c, int bm) { return (c + bm - 1) & -bm; }  // bm: a power of two

__device__ __forceinline__ int id_bits(int E) { return E > 1 ? 32 - __clz(E - 1) : 0; }

// Steps per wave for the ids [lo, hi) of one block: each of the 16 waves owns
// a contiguous segment of 64 * steps ids and walks it 64 per step.
__device__ __forceinline__ int block_steps(int lo, int hi) { return max(1, (hi - lo + kThreads - 1) / kThreads); }

__device__ __forceinline__ int id_index(int lo, int steps, int r) {
  return lo + ((int)threadIdx.x >> 6) * 64 * steps + 64 * r + ((int)threadIdx.x & 63);
}

// This lane's ids, one per step; -1 past `hi` and for unused steps.
__device__ __forceinline__ void load_ids(const int32_t* __restrict__ ids, int lo, int hi, int steps,
                                         int (&v)[kPerThread]) {
#pragma unroll
  for (int r = 0; r < kPerThread; ++r) {
    const int i = id_index(lo, steps, r);
    v[r] = (r < steps && i < hi) ? ids[i] : -1;
  }
}

__device__ __forceinline__ void count_ids(const int (&v)[kPerThread], int E, int* hist) {
#pragma unroll
  for (int r = 0; r < kPerThread; ++r)
    if ((unsigned)v[r] < (unsigned)E) atomicAdd(&hist[v[r]], 1);
}

// Wave 0 writes off[0..E] = exclusive prefix of padded counts (off[E] = the
// padded total), cursor[e] = off[e] (+ the old cursor[e] when add_cursor), and,
// where the pointers are not null, the counts and the padded total to global
// memory. An expert whose count lies outside `keep` is dropped: its count
// becomes 0 (in LDS too, which the scatter reads) and its ids are skipped.
// Lane l owns experts [l * per, (l + 1) * per), held in registers; one DPP
// wave scan. E <= 64 * kMaxExpertsPerLane.
constexpr int kMaxExpertsPerLane = 8;

// Experts kept by an alignment: those with lo <= count <= hi.
struct CountRange {
  int lo, hi;
};
constexpr CountRange kAllCounts = {0, 0x7fffffff};
static_assert(64 * kMaxExpertsPerLane >= W4A16_MAX_EXPERTS, "one scan wave must hold every expert");

__device__ void scan_offsets(int* counts, int E, int bm, int* off, int* cursor, bool add_cursor,
                             int32_t* __restrict__ counts_out, int32_t* __restrict__ ntpp_out, CountRange keep) {
  if (threadIdx.x < 64) {
    const int lane = (int)threadIdx.x;
    const int per = (E + 63) / 64;
    const int start = lane * per;
    int c[kMaxExpertsPerLane];
    int local = 0;
#pragma unroll
    for (int k = 0; k < kMaxExpertsPerLane; ++k) {
      c[k] = (k < per && start + k < E) ? counts[start + k] : 0;
      if (c[k] < keep.lo || c[k] > keep.hi) c[k] = 0;  // an expert outside the range is not resident
      local += padded(c[k], bm);
    }
    const int incl = wave_incl_scan(local);
    int run = incl - local;
#pragma unroll
    for (int k = 0; k < kMaxExpertsPerLane; ++k) {
      const int e = start + k;
      if (k < per && e < E) {
        counts[e] = c[k];
        off[e] = run;
        cursor[e] = (add_cursor ? cursor[e] : 0) + run;
        if (counts_out) counts_out[e] = c[k];
        run += padded(c[k], bm);
      }
    }
    if (lane == 63) {
      off[E] = incl;
      if (ntpp_out) *ntpp_out = incl;
    }
  }
}

// Block labels and padding sentinels from the experts' side: the 16-lane group
// of expert e (experts g0, g0 + gstep, ...) writes expert_ids for e's blocks and
// the sentinel into e's padding slots (only an expert's last block holds
// padding, at most block_m - 1 slots), 16 at a time. An expert knows its own
// blocks, so no block has to search for its expert (a per-block 16-way search
// over the offsets cost 5.3 of 16.5 us for 4096 ids over 384 experts).
__device__ void label_experts(const int* off, const int* counts, int E, int bm, int32_t* sorted, int32_t* expert_ids,
                              int nblk, int capacity, int sentinel, int g0, int gstep) {
  const int sub = (int)threadIdx.x & 15;
  for (int e = g0; e < E; e += gstep) {
    const int c = counts[e];
    if (c == 0) continue;
    const int end = off[e] + padded(c, bm);
    for (int b = off[e] / bm + sub; b < min(end / bm, nblk); b += 16) expert_ids[b] = e;
    for (int p = off[e] + c + sub; p < min(end, capacity); p += 16) sorted[p] = sentinel;
  }
}

// Expert groups of a launch, interleaved over its blocks so that every block
// (compute unit) takes a share of the label stores: group (thread / 16) of
// block b is global group (thread / 16) * gridDim + b.
__device__ __forceinline__ int expert_group0() { return ((int)threadIdx.x >> 4) * (int)gridDim.x + (int)blockIdx.x; }
__device__ __forceinline__ int expert_gstep() { return (kThreads / 16) * (int)gridDim.x; }

// Unused tail: sorted[ntpp, capacity) = sentinel, expert_ids[ntpp / bm, nblk) = -1.
__device__ void fill_tail(int ntpp, int bm, int32_t* sorted, int capacity, int32_t* expert_ids, int nblk,
                          int sentinel, int t0, int step) {
  for (int p = ntpp + t0; p < capacity; p += step) sorted[p] = sentinel;
  for (int b = ntpp / bm + t0; b < nblk; b += step) expert_ids[b] = -1;
}

// Stable scatter of the block's ids (held in v, see id_index): the id at flat
// index i goes to cursor[e] + (resident ids of e before i in this block).
// Each wave ranks its own contiguous segment step by step against its own
// counters wcnt[e * kWtabStride + wave] in LDS (lanes of one expert in a step
// are found with one ballot per id bit; the rank is the mbcnt of the peers
// below), so the steps need no workgroup barrier. The 16 per-wave counts of an
// expert are then turned into per-wave bases by one 16-lane row scan. wcnt is
// LDS scratch of kWtabStride * E ints, zeroed by the caller before its last barrier.
__device__ void scatter_ids(const int (&v)[kPerThread], int steps, int E, int nbits, const int* counts,
                            const int* cursor, int* wcnt, int32_t* __restrict__ sorted, int capacity, int lo) {
  const int wave = (int)threadIdx.x >> 6;
  int* row = wcnt + wave;  // this wave's counter of expert e: row[e * kWtabStride]
  int rank[kPerThread];
#pragma unroll
  for (int r = 0; r < kPerThread; ++r) {
    rank[r] = 0;
    if (r < steps) {  // uniform
      const int e = v[r];
      const bool local = (unsigned)e < (unsigned)E && counts[e] > 0;  // resident and kept
      uint64_t peers = __ballot(local);
      for (int b = 0; b < nbits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t m = __ballot(local && bit);
        peers &= bit ? m : ~m;
      }
      const int below = rank_below(peers);
      const int prev = local ? row[e * kWtabStride] : 0;  // every lane reads before the leader writes
      rank[r] = prev + below;
      if (local && below == 0) row[e * kWtabStride] = prev + __popcll(peers);
    }
  }
  lds_barrier();  // all waves' counts final
  // pair (expert x, wave w) at thread index 16 x + w: one 16-lane row holds one
  // expert's consecutive counters; kWaves * E is a multiple of 16, so every row
  // is fully active
  for (int idx = (int)threadIdx.x; idx < kWaves * E; idx += kThreads) {
    const int x = idx >> 4, w = idx & 15;
    const int c = wcnt[x * kWtabStride + w];
    wcnt[x * kWtabStride + w] = cursor[x] + row_incl_scan(c) - c;  // only this lane ever touches this entry
  }
  lds_barrier();  // per-wave bases visible
#pragma unroll
  for (int r = 0; r < kPerThread; ++r)
    if (r < steps && (unsigned)v[r] < (unsigned)E && counts[v[r]] > 0) {
      const int pos = row[v[r] * kWtabStride] + rank[r];  // < capacity: the capacity covers every padded count
      if ((unsigned)pos < (unsigned)capacity) sorted[pos] = id_index(lo, steps, r);
    }
}

// ---- single-launch path -----------------------------------------------------
// The whole alignment of n <= kSmallMax ids held in v (see id_index, lo = 0) by
// one block. LDS: counts[E], off[E+1], cursor[E], wtab[kWtabStride*E]
__device__ void align_block(const int (&v)[kPerThread], int n, int E, int bm, int* smem, int32_t* __restrict__ sorted,
                            int capacity, int32_t* __restrict__ expert_ids, int nblk, int32_t* __restrict__ ntpp_out,
                            int32_t* __restrict__ counts_out, CountRange keep) {
  int* counts = smem;
  int* off = counts + E;
  int* cursor = off + E + 1;
  int* wtab = cursor + E;
  const int steps = block_steps(0, n);
  for (int e = (int)threadIdx.x; e < E; e += kThreads) counts[e] = 0;
  for (int k = (int)threadIdx.x; k < kWtabStride * E; k += kThreads) wtab[k] = 0;
  lds_barrier();
  count_ids(v, E, counts);
  lds_barrier();
  scan_offsets(counts, E, bm, off, cursor, false, counts_out, ntpp_out, keep);
  lds_barrier();
  const int ntpp = off[E];
  label_experts(off, counts, E, bm, sorted, expert_ids, nblk, capacity, n, expert_group0(), expert_gstep());
  fill_tail(ntpp, bm, sorted, capacity, expert_ids, nblk, n, (int)threadIdx.x, kThreads);
  lds_barrier();
  scatter_ids(v, steps, E, id_bits(E), counts, cursor, wtab, sorted, capacity, 0);
}

// The alignment of n <= 64 ids by wave 0 alone (lane i holds id i in v0, -1
// past n). The caller has already zeroed counts[E] in LDS and filled the whole
// of sorted with the sentinel n and expert_ids with -1, and has passed a
// __syncthreads() since (it orders those stores before the ones here). The
// wave ranks, counts, scans (its LDS accesses run in order: no barrier), then
// writes the resident ids and labels its used blocks; padding and tail are
// already right. LDS: counts[E], off[E+1], cursor[E].
constexpr int kWaveMax = 64;

__device__ void prefill_outputs(int E, int32_t* __restrict__ sorted, int capacity, int32_t* __restrict__ expert_ids,
                                int nblk, int sentinel, int* counts) {
  for (int e = (int)threadIdx.x; e < E; e += kThreads) counts[e] = 0;
  for (int p = (int)threadIdx.x; p < capacity; p += kThreads) sorted[p] = sentinel;
  for (int b = (int)threadIdx.x; b < nblk; b += kThreads) expert_ids[b] = -1;
}

__device__ void align_wave(int v0, int E, int bm, int* smem, int32_t* __restrict__ sorted, int capacity,
                           int32_t* __restrict__ expert_ids, int nblk, int32_t* __restrict__ ntpp_out,
                           int32_t* __restrict__ counts_out, CountRange keep) {
  if (threadIdx.x >= 64) return;
  int* counts = smem;
  int* off = counts + E;
  int* cursor = off + E + 1;
  const int lane = (int)threadIdx.x;
  const int e = v0;
  const bool local = (unsigned)e < (unsigned)E;
  uint64_t peers = __ballot(local);
  const int nbits = id_bits(E);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t m = __ballot(local && bit);
    peers &= bit ? m : ~m;
  }
  const int rank = rank_below(peers);  // resident ids of e in lanes below: the stable order
  if (local && rank == 0) counts[e] = __popcll(peers);
  scan_offsets(counts, E, bm, off, cursor, false, counts_out, ntpp_out, keep);
  if (local && counts[e] > 0) {  // kept by the count range
    const int base = off[e];
    const int pos = base + rank;
    if ((unsigned)pos < (unsigned)capacity) sorted[pos] = lane;
    if (rank == 0)  // the expert's leader labels its blocks
      for (int b = base / bm; b < min((base + padded(counts[e], bm)) / bm, nblk); ++b) expert_ids[b] = e;
  }
}

__global__ __launch_bounds__(kThreads) void align_small_kernel(const int32_t* __restrict__ ids, int n, int E, int bm,
                                                               int32_t* __restrict__ sorted, int capacity,
                                                               int32_t* __restrict__ expert_ids, int nblk,
                                                               int32_t* __restrict__ ntpp_out,
                                                               int32_t* __restrict__ counts_out, CountRange keep) {
  extern __shared__ int smem[];
  if (n <= kWaveMax) {  // uniform
    const int v0 = threadIdx.x < (unsigned)n ? ids[threadIdx.x] : -1;
    prefill_outputs(E, sorted, capacity, expert_ids, nblk, n, smem);
    __syncthreads();  // also waits for the prefill stores
    align_wave(v0, E, bm, smem, sorted, capacity, expert_ids, nblk, ntpp_out, counts_out, keep);
    return;
  }
  int v[kPerThread];
  load_ids(ids, 0, n, block_steps(0, n), v);
  align_block(v, n, E, bm, smem, sorted, capacity, expert_ids, nblk, ntpp_out, counts_out, keep);
}

// ---- one launch, several blocks ----------------------------------------------
// n ids in (kThreads, kSmallMax]: block b scatters the ids [b kSpread, (b+1)
// kSpread) (one per thread of its first kSpread) and labels its share of the
// experts; every block
// counts all n ids itself (they are few and L2-resident after the first block
// reads them), along with the ids of each expert before its own chunk, so no
// block waits for another and there is no separate histogram launch. The
// alignment's stores, mostly scattered 4-byte writes, then leave through
// several compute units' memory pipelines instead of one (one block took
// 13.6 us for 4096 ids over 384 experts, most of it in its stores; chunks of
// 256 rather than 1024 ids: 7.0 -> 6.6 us there, 5.8 -> 5.4 us for 6144 ids
// over 48 experts).
// LDS: counts[E], off[E+1], cursor[E], wtab[kWtabStride*E]
constexpr int kSpread = kThreads / 4;

__global__ __launch_bounds__(kThreads) void align_spread_kernel(const int32_t* __restrict__ ids, int n, int E, int bm,
                                                                int32_t* __restrict__ sorted, int capacity,
                                                                int32_t* __restrict__ expert_ids, int nblk,
                                                                int32_t* __restrict__ ntpp_out,
                                                                int32_t* __restrict__ counts_out, CountRange keep) {
  extern __shared__ int smem[];
  int* counts = smem;
  int* off = counts + E;
  int* cursor = off + E + 1;
  int* wtab = cursor + E;
  const int lo = (int)blockIdx.x * kSpread;
  const int hi = min(n, lo + kSpread);
  int v[kPerThread];
  load_ids(ids, lo, hi, 1, v);
  for (int e = (int)threadIdx.x; e < E; e += kThreads) counts[e] = cursor[e] = 0;
  for (int k = (int)threadIdx.x; k < kWtabStride * E; k += kThreads) wtab[k] = 0;
  lds_barrier();
  // every id, and the ids before this chunk (into cursor: this chunk's base
  // inside each expert); all loads are issued before the first count
  const int steps = block_steps(0, n);
  int va[kPerThread];
  load_ids(ids, 0, n, steps, va);
#pragma unroll
  for (int r = 0; r < kPerThread; ++r)
    if ((unsigned)va[r] < (unsigned)E) {
      atomicAdd(&counts[va[r]], 1);
      if (id_index(0, steps, r) < lo) atomicAdd(&cursor[va[r]], 1);
    }
  lds_barrier();
  const bool first = blockIdx.x == 0;
  scan_offsets(counts, E, bm, off, cursor, true, first ? counts_out : nullptr, first ? ntpp_out : nullptr, keep);
  lds_barrier();
  const int gt = (int)(blockIdx.x * kThreads + threadIdx.x), gstep = (int)(gridDim.x * kThreads);
  label_experts(off, counts, E, bm, sorted, expert_ids, nblk, capacity, n, expert_group0(), expert_gstep());
  fill_tail(off[E], bm, sorted, capacity, expert_ids, nblk, n, gt, gstep);
  lds_barrier();
  scatter_ids(v, 1, E, id_bits(E), counts, cursor, wtab, sorted, capacity, lo);
}

// ---- multi-block path -------------------------------------------------------
// Workspace: hist[nchunks * E], the per-chunk resident counts.
__global__ __launch_bounds__(kThreads) void align_hist_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                              int* __restrict__ hist) {
  extern __shared__ int smem[];
  int v[kPerThread];
  const int lo = (int)blockIdx.x * kChunk;
  load_ids(ids, lo, min(n, lo + kChunk), block_steps(lo, min(n, lo + kChunk)), v);
  for (int e = (int)threadIdx.x; e < E; e += kThreads) smem[e] = 0;
  lds_barrier();
  count_ids(v, E, smem);
  lds_barrier();
  for (int e = (int)threadIdx.x; e < E; e += kThreads) hist[(size_t)blockIdx.x * E + e] = smem[e];
}

// Expert totals and this block's base inside each expert from the per-chunk
// histograms: a wave per expert, its lanes reading the chunks' counts in
// parallel (L2 hits), then wave-wide sums; written to total/before and, when
// given, their copies total2/before2.
__device__ void chunk_sums(const int* __restrict__ hist, int nchunks, int E, int* total, int* before,
                           int* total2 = nullptr, int* before2 = nullptr) {
  const int wave = (int)threadIdx.x >> 6, lane = (int)threadIdx.x & 63;
  for (int e = wave; e < E; e += kWaves) {  // uniform per wave: every lane takes part in the sums
    int t = 0, b = 0;
    for (int k = lane; k < nchunks; k += 64) {
      const int c = hist[(size_t)k * E + e];
      t += c;
      b += k < (int)blockIdx.x ? c : 0;
    }
    t = __builtin_amdgcn_readlane(wave_incl_scan(t), 63);
    b = __builtin_amdgcn_readlane(wave_incl_scan(b), 63);
    if (lane == 0) {
      total[e] = t;
      before[e] = b;
      if (total2) {
        total2[e] = t;
        before2[e] = b;
      }
    }
  }
}

// One block per chunk. Every block reads all chunk histograms (nchunks * E
// entries) to get the expert totals, the offsets and its own chunk's base;
// block 0 also writes the counts, the padded total and the block labels; all
// blocks share the sentinel fill of the tail.
// LDS: counts[E], off[E+1], cursor[E], wtab[kWtabStride*E]
__global__ __launch_bounds__(kThreads) void align_scatter_kernel(const int32_t* __restrict__ ids, int n, int E, int bm,
                                                                 const int* __restrict__ hist, int nchunks,
                                                                 int32_t* __restrict__ sorted, int capacity,
                                                                 int32_t* __restrict__ expert_ids, int nblk,
                                                                 int32_t* __restrict__ ntpp_out,
                                                                 int32_t* __restrict__ counts_out, CountRange keep) {
  extern __shared__ int smem[];
  int* counts = smem;
  int* off = counts + E;
  int* cursor = off + E + 1;
  int* wtab = cursor + E;
  int v[kPerThread];
  const int lo = (int)blockIdx.x * kChunk;
  const int steps = block_steps(lo, min(n, lo + kChunk));
  load_ids(ids, lo, min(n, lo + kChunk), steps, v);
  for (int k = (int)threadIdx.x; k < kWtabStride * E; k += kThreads) wtab[k] = 0;
  chunk_sums(hist, nchunks, E, counts, cursor);  // cursor: this chunk's base inside each expert, before off[e]
  lds_barrier();
  scan_offsets(counts, E, bm, off, cursor, true, blockIdx.x == 0 ? counts_out : nullptr,
               blockIdx.x == 0 ? ntpp_out : nullptr, keep);
  lds_barrier();
  const int ntpp = off[E];
  const int gt = (int)(blockIdx.x * kThreads + threadIdx.x), gstep = (int)(gridDim.x * kThreads);
  label_experts(off, counts, E, bm, sorted, expert_ids, nblk, capacity, n, expert_group0(), expert_gstep());
  fill_tail(ntpp, bm, sorted, capacity, expert_ids, nblk, n, gt, gstep);
  lds_barrier();
  scatter_ids(v, steps, E, id_bits(E), counts, cursor, wtab, sorted, capacity, lo);
}

// Two alignments of the same ids in one pass: experts with at least `split`
// resident ids form set 0 (block_m bm0), those with 1 .. split - 1 set 1
// (block_m bm1); each set's outputs are exactly the one-set alignment with
// that count range. Set 1's sorted array directly follows set 0's (sorted +
// cap0), so one stable scatter into the joined array serves both: an expert of
// set 1 starts its cursor at cap0 + its offset in set 1.
// LDS: cnt0[E], off0[E+1], cur0[E], wtab[kWtabStride*E], cnt1[E], off1[E+1],
// cur1[E], kept[E]
__global__ __launch_bounds__(kThreads) void align_scatter2_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                                  int split, const int* __restrict__ hist, int nchunks,
                                                                  int32_t* __restrict__ sorted, int bm0, int cap0,
                                                                  int32_t* __restrict__ eids0, int nblk0,
                                                                  int32_t* __restrict__ ntpp0, int bm1, int cap1,
                                                                  int32_t* __restrict__ eids1, int nblk1,
                                                                  int32_t* __restrict__ ntpp1) {
  extern __shared__ int smem[];
  int* cnt0 = smem;
  int* off0 = cnt0 + E;
  int* cur0 = off0 + E + 1;
  int* wtab = cur0 + E;
  int* cnt1 = wtab + kWtabStride * E;
  int* off1 = cnt1 + E;
  int* cur1 = off1 + E + 1;
  int* kept = cur1 + E;
  int v[kPerThread];
  const int lo = (int)blockIdx.x * kChunk;
  const int steps = block_steps(lo, min(n, lo + kChunk));
  load_ids(ids, lo, min(n, lo + kChunk), steps, v);
  for (int k = (int)threadIdx.x; k < kWtabStride * E; k += kThreads) wtab[k] = 0;
  chunk_sums(hist, nchunks, E, cnt0, cur0, cnt1, cur1);
  lds_barrier();
  const bool first = blockIdx.x == 0;
  // both scans run on wave 0, one after the other (its LDS accesses stay in order)
  scan_offsets(cnt0, E, bm0, off0, cur0, true, nullptr, first ? ntpp0 : nullptr, CountRange{split, 0x7fffffff});
  scan_offsets(cnt1, E, bm1, off1, cur1, true, nullptr, first ? ntpp1 : nullptr, CountRange{1, split - 1});
  lds_barrier();
  const int gt = (int)(blockIdx.x * kThreads + threadIdx.x), gstep = (int)(gridDim.x * kThreads);
  label_experts(off0, cnt0, E, bm0, sorted, eids0, nblk0, cap0, n, expert_group0(), expert_gstep());
  label_experts(off1, cnt1, E, bm1, sorted + cap0, eids1, nblk1, cap1, n, expert_group0(), expert_gstep());
  fill_tail(off0[E], bm0, sorted, cap0, eids0, nblk0, n, gt, gstep);
  fill_tail(off1[E], bm1, sorted + cap0, cap1, eids1, nblk1, n, gt, gstep);
  // joined view: kept[e] = the expert's count in whichever set holds it (the
  // ranges are disjoint), cur1[e] = its cursor in the joined array
  for (int e = (int)threadIdx.x; e < E; e += kThreads) {
    kept[e] = cnt0[e] + cnt1[e];
    cur1[e] = cnt0[e] > 0 ? cur0[e] : cap0 + cur1[e];
  }
  lds_barrier();
  scatter_ids(v, steps, E, id_bits(E), kept, cur1, wtab, sorted, cap0 + cap1, lo);
}

// T == 0: every output is a sentinel.
__global__ void align_empty_kernel(int32_t* sorted, int capacity, int sentinel, int32_t* expert_ids, int nblk,
                                   int32_t* ntpp_out, int32_t* counts_out, int E) {
  const int tid = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  const int step = (int)(gridDim.x * blockDim.x);
  for (int p = tid; p < capacity; p += step) sorted[p] = sentinel;
  for (int b = tid; b < nblk; b += step) expert_ids[b] = -1;
  for (int e = tid; e < E; e += step) if (counts_out) counts_out[e] = 0;
  if (tid == 0) *ntpp_out = 0;
}

// ---- router ------------------------------------------------------------------
// Top-k routing of one token by one wave, the step the FlashInfer Kimi-K3 fused
// router runs before its alignment (page "[flashinfer] FlashInfer, B200 GPU에서
// Kimi-K3 MoE 라우터 성능 최적화", sections "코드 분석" and "커널 내부 로직 변경
// (추정)"). The page shows the router's interface (logits, bias -> top-k
// weights, ids and the alignment buffers) but not its arithmetic; the
// definition here: score = logit + bias in fp32, the topk highest scores in
// descending order with an equal score going to the lower expert id, weights =
// softmax over the chosen raw logits (the bias steers the choice only).
//
// Lane l holds experts l, l + 64, l + 128, ... (coalesced row reads), each
// score as an order-preserving integer key. Each of the topk rounds is one
// wave-wide integer max over DPP (quad swaps, row mirrors, row broadcasts: no
// LDS round trips), then one ballot per expert slot finds the lowest expert
// holding that key; keys compare exactly as the fp32 scores do, so ties
// resolve exactly as the definition says.

constexpr int kRouteWaves = 4;  // tokens per block of the stand-alone router

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_mov(float v, float old) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old), __builtin_bit_cast(int, v),
                                                               CTRL, ROW_MASK, 0xf, false));
}

// Wave-wide max / sum, returned to every lane. Steps: quad_perm [1,0,3,2] and
// [2,3,0,1] (quads), row_half_mirror (8 lanes), row_mirror (16 lanes), then
// row_bcast:15 into rows 1 and 3 and row_bcast:31 into rows 2 and 3: lane 63
// ends with the whole wave. Rows a step does not write keep `old` (the
// operation's identity).
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_mov<0xb1, 0xf>(v, v));
  v = fmaxf(v, dpp_mov<0x4e, 0xf>(v, v));
  v = fmaxf(v, dpp_mov<0x141, 0xf>(v, v));
  v = fmaxf(v, dpp_mov<0x140, 0xf>(v, v));
  v = fmaxf(v, dpp_mov<0x142, 0xa>(v, v));
  v = fmaxf(v, dpp_mov<0x143, 0xc>(v, v));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_mov<0xb1, 0xf>(v, 0.f);
  v += dpp_mov<0x4e, 0xf>(v, 0.f);
  v += dpp_mov<0x141, 0xf>(v, 0.f);
  v += dpp_mov<0x140, 0xf>(v, 0.f);
  v += dpp_mov<0x142, 0xa>(v, 0.f);
  v += dpp_mov<0x143, 0xc>(v, 0.f);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Order-preserving map of a non-NaN float to a uint32 key >= 0x007fffff
// (-inf); -0 and +0 share one key, as they compare equal. Key 0 marks an
// expert already chosen (or absent).
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  if (u == 0x80000000u) return 0x80000000u;  // -0 -> key of +0
  return (u >> 31) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xb1, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4e, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xa, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Routes token t (the calling wave, all 64 lanes active). Lane j < topk writes
// topk_ids[t, j] and topk_weights[t, j] and returns the id; other lanes return -1.
// SLOTS * 64 >= Eg; requires 1 <= topk <= min(Eg, 64).
template <int SLOTS>
__device__ int route_token(const float* __restrict__ logits, const float* __restrict__ bias, int t, int Eg, int topk,
                           int32_t* __restrict__ topk_ids, float* __restrict__ topk_weights) {
  const int lane = (int)threadIdx.x & 63;
  const float* row = logits + (size_t)t * Eg;
  float raw[SLOTS], b[SLOTS];
  uint32_t key[SLOTS];
  // unconditional (clamped) loads, so all of them are in flight at once
#pragma unroll
  for (int j = 0; j < SLOTS; ++j) raw[j] = row[min(lane + 64 * j, Eg - 1)];
  if (bias) {
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) b[j] = bias[min(lane + 64 * j, Eg - 1)];
  } else {
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) b[j] = 0.f;  // x + 0 orders like x
  }
#pragma unroll
  for (int j = 0; j < SLOTS; ++j) key[j] = lane + 64 * j < Eg ? order_key(raw[j] + b[j]) : 0u;
  int my_id = -1;
  float my_logit = -INFINITY;
  for (int r = 0; r < topk; ++r) {
    uint32_t best = key[0];
#pragma unroll
    for (int j = 1; j < SLOTS; ++j) best = max(best, key[j]);
    const uint32_t m = wave_max_u32(best);  // > 0: an open expert remains (topk <= Eg)
    // lowest expert id holding key m: the first slot with a hit, then its lowest lane
    int wj = 0, wl = 0;
#pragma unroll
    for (int j = SLOTS - 1; j >= 0; --j) {
      const uint64_t hit = __ballot(key[j] == m);
      if (hit) {
        wj = j;
        wl = (int)__builtin_ctzll(hit);
      }
    }
    float sel = raw[0];
#pragma unroll
    for (int j = 1; j < SLOTS; ++j) sel = j == wj ? raw[j] : sel;
    const float lg = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sel), wl));
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) key[j] = (j == wj && lane == wl) ? 0u : key[j];
    if (lane == r) {
      my_id = wl + 64 * wj;
      my_logit = lg;
    }
  }
  const float mx = wave_max(my_logit);  // lanes >= topk hold -inf
  const float ex = lane < topk ? expf(my_logit - mx) : 0.f;
  const float sum = wave_sum(ex);
  if (lane < topk) {
    topk_ids[(size_t)t * topk + lane] = my_id;
    topk_weights[(size_t)t * topk + lane] = ex / sum;
  }
  return my_id;
}

// Stand-alone router: one wave per token.
template <int SLOTS>
__global__ __launch_bounds__(64 * kRouteWaves) void route_kernel(const float* __restrict__ logits,
                                                                 const float* __restrict__ bias, int T, int Eg,
                                                                 int topk, int32_t* __restrict__ topk_ids,
                                                                 float* __restrict__ topk_weights) {
  const int t = (int)blockIdx.x * kRouteWaves + ((int)threadIdx.x >> 6);
  if (t < T) route_token<SLOTS>(logits, bias, t, Eg, topk, topk_ids, topk_weights);
}

// Router and alignment in one launch for T <= kWaves tokens: wave w routes
// token w and leaves its ids in LDS, then the block aligns them (every counter
// is set inside the kernel, nothing is read from a previous call).
// LDS: ids[kWaves * 32] (32 = the largest topk), then the alignment's tables.
constexpr int kFusedIds = kWaves * 32;
static_assert(32 >= W4A16_MAX_TOPK, "fused ids buffer");

template <int SLOTS>
__global__ __launch_bounds__(kThreads) void route_align_small_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int T, int Eg, int topk, int E, int bm,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_weights, int32_t* __restrict__ sorted, int capacity,
    int32_t* __restrict__ expert_ids, int nblk, int32_t* __restrict__ ntpp_out, int32_t* __restrict__ counts_out) {
  extern __shared__ int smem[];
  int* ids = smem;
  const int wave = (int)threadIdx.x >> 6, lane = (int)threadIdx.x & 63;
  const int n = T * topk;
  // up to 64 ids: the output prefill runs while the waves route
  if (n <= kWaveMax) prefill_outputs(E, sorted, capacity, expert_ids, nblk, n, smem + kFusedIds);
  if (wave < T) {
    const int id = route_token<SLOTS>(logits, bias, wave, Eg, topk, topk_ids, topk_weights);
    if (lane < topk) ids[wave * topk + lane] = id;
  }
  if (n <= kWaveMax) {  // uniform
    __syncthreads();  // ids in LDS, and the prefill stores done
    const int v0 = threadIdx.x < (unsigned)n ? ids[threadIdx.x] : -1;
    align_wave(v0, E, bm, smem + kFusedIds, sorted, capacity, expert_ids, nblk, ntpp_out, counts_out, kAllCounts);
    return;
  }
  lds_barrier();
  int v[kPerThread];
#pragma unroll
  for (int r = 0; r < kPerThread; ++r) {
    const int i = id_index(0, 1, r);  // n <= kThreads: one step
    v[r] = (r == 0 && i < n) ? ids[i] : -1;
  }
  align_block(v, n, E, bm, smem + kFusedIds, sorted, capacity, expert_ids, nblk, ntpp_out, counts_out, kAllCounts);
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

size_t scatter_lds(int E) { return sizeof(int) * (size_t)(3 * E + 1 + kWtabStride * E); }
// align_scatter2_kernel: the one-set layout, then cnt1[E], off1[E+1], cur1[E], kept[E]
size_t scatter2_lds(int E) { return scatter_lds(E) + sizeof(int) * (size_t)(4 * E + 1); }

}  // namespace

size_t align_workspace_bytes(int64_t n, int32_t E) {
  if (n <= kSmallMax) return 0;
  const int64_t nchunks = (n + kChunk - 1) / kChunk;
  return round_up(sizeof(int) * (size_t)(nchunks * E), 256);
}

hipError_t launch_align(const int32_t* ids, int32_t n, int32_t E, int32_t bm, int32_t* sorted, int32_t capacity,
                        int32_t* expert_ids, int32_t* ntpp, int32_t* counts, void* workspace, hipStream_t stream,
                        int32_t min_count, int32_t max_count) {
  const int nblk = (capacity + bm - 1) / bm;
  const CountRange keep = {min_count, max_count};
  if (n == 0) {
    const int grid = (int)std::min<int64_t>(1024, std::max<int64_t>(1, ((int64_t)capacity + 255) / 256));
    hipLaunchKernelGGL(align_empty_kernel, dim3(grid), dim3(256), 0, stream, sorted, capacity, n, expert_ids, nblk,
                       ntpp, counts, E);
    return hipGetLastError();
  }
  if (n <= kThreads) {  // one block: the whole alignment (one wave up to 64 ids)
    hipLaunchKernelGGL(align_small_kernel, dim3(1), dim3(kThreads), scatter_lds(E), stream, ids, n, E, bm, sorted,
                       capacity, expert_ids, nblk, ntpp, counts, keep);
    return hipGetLastError();
  }
  if (n <= kSmallMax) {
    hipLaunchKernelGGL(align_spread_kernel, dim3((n + kSpread - 1) / kSpread), dim3(kThreads), scatter_lds(E), stream,
                       ids, n, E, bm, sorted, capacity, expert_ids, nblk, ntpp, counts, keep);
    return hipGetLastError();
  }
  const int nchunks = (n + kChunk - 1) / kChunk;
  int* hist = static_cast<int*>(workspace);
  hipLaunchKernelGGL(align_hist_kernel, dim3(nchunks), dim3(kThreads), sizeof(int) * (size_t)E, stream, ids, n, E,
                     hist);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(align_scatter_kernel, dim3(nchunks), dim3(kThreads), scatter_lds(E), stream, ids, n, E, bm, hist,
                     nchunks, sorted, capacity, expert_ids, nblk, ntpp, counts, keep);
  return hipGetLastError();
}

hipError_t launch_align_split(const int32_t* ids, int32_t n, int32_t E, int32_t split, int32_t* sorted, int32_t bm0,
                              int32_t cap0, int32_t* eids0, int32_t* ntpp0, int32_t bm1, int32_t cap1,
                              int32_t* eids1, int32_t* ntpp1, void* workspace, hipStream_t stream) {
  if (n <= kSmallMax) {  // one block per set already: the two one-set alignments
    const hipError_t err = launch_align(ids, n, E, bm0, sorted, cap0, eids0, ntpp0, nullptr, workspace, stream,
                                        split, 0x7fffffff);
    if (err != hipSuccess) return err;
    return launch_align(ids, n, E, bm1, sorted + cap0, cap1, eids1, ntpp1, nullptr, workspace, stream, 1, split - 1);
  }
  const int nchunks = (n + kChunk - 1) / kChunk;
  int* hist = static_cast<int*>(workspace);
  hipLaunchKernelGGL(align_hist_kernel, dim3(nchunks), dim3(kThreads), sizeof(int) * (size_t)E, stream, ids, n, E,
                     hist);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(align_scatter2_kernel, dim3(nchunks), dim3(kThreads), scatter2_lds(E), stream, ids, n, E, split,
                     hist, nchunks, sorted, bm0, cap0, eids0, (cap0 + bm0 - 1) / bm0, ntpp0, bm1, cap1, eids1,
                     (cap1 + bm1 - 1) / bm1, ntpp1);
  return hipGetLastError();
}

namespace {
template <int SLOTS>
hipError_t launch_route_align_slots(const float* logits, const float* bias, int32_t T, int32_t Eg, int32_t topk,
                                    int32_t E, int32_t bm, int32_t* topk_ids, float* topk_weights, int32_t* sorted,
                                    int32_t capacity, int32_t* expert_ids, int32_t* ntpp, int32_t* counts,
                                    void* workspace, hipStream_t stream) {
  if (T <= kWaves) {
    const int nblk = (capacity + bm - 1) / bm;
    hipLaunchKernelGGL(route_align_small_kernel<SLOTS>, dim3(1), dim3(kThreads),
                       sizeof(int) * kFusedIds + scatter_lds(E), stream, logits, bias, T, Eg, topk, E, bm, topk_ids,
                       topk_weights, sorted, capacity, expert_ids, nblk, ntpp, counts);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(route_kernel<SLOTS>, dim3((T + kRouteWaves - 1) / kRouteWaves), dim3(64 * kRouteWaves), 0,
                     stream, logits, bias, T, Eg, topk, topk_ids, topk_weights);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_align(topk_ids, T * topk, E, bm, sorted, capacity, expert_ids, ntpp, counts, workspace, stream);
}
}  // namespace

hipError_t launch_route_align(const float* logits, const float* bias, int32_t T, int32_t Eg, int32_t topk, int32_t E,
                              int32_t bm, int32_t* topk_ids, float* topk_weights, int32_t* sorted, int32_t capacity,
                              int32_t* expert_ids, int32_t* ntpp, int32_t* counts, void* workspace,
                              hipStream_t stream) {
  if (T == 0) return launch_align(topk_ids, 0, E, bm, sorted, capacity, expert_ids, ntpp, counts, workspace, stream);
  if (Eg <= 128)
    return launch_route_align_slots<2>(logits, bias, T, Eg, topk, E, bm, topk_ids, topk_weights, sorted, capacity,
                                       expert_ids, ntpp, counts, workspace, stream);
  if (Eg <= 256)
    return launch_route_align_slots<4>(logits, bias, T, Eg, topk, E, bm, topk_ids, topk_weights, sorted, capacity,
                                       expert_ids, ntpp, counts, workspace, stream);
  if (Eg <= 512)
    return launch_route_align_slots<8>(logits, bias, T, Eg, topk, E, bm, topk_ids, topk_weights, sorted, capacity,
                                       expert_ids, ntpp, counts, workspace, stream);
  return launch_route_align_slots<16>(logits, bias, T, Eg, topk, E, bm, topk_ids, topk_weights, sorted, capacity,
                                      expert_ids, ntpp, counts, workspace, stream);
}

}  // namespace w4a16
