// Weight-streaming W4A16 expert GEMM for few tokens per expert (block_m 16 to 64).
//
// With a few routed tokens per expert the layer is a weight stream: every
// byte of each active expert's packed weights is read once, and the kernel's
// job is to keep enough of them in flight to run HBM at full rate (decode is
// HBM-bound; Chord page "vLLM 및 Novita AI, Kimi K2.x용 더 빠른 INT4 MoE 커널
// 출시: Chord", "핵심 기여" and the latency-tuned buffered-K depth of "그룹 SM90
// 커널 기법"). The arithmetic: exact integer operands q + 136 on
// v_mfma_f32_16x16x32_bf16, a -136 * sum(x) correction in the C input, one
// fp32 FMA per output per 32-wide group for the BF16 scale (the tiled kernel
// instead folds the scale into exact fp16 operands).
//
// Work unit: (row block of block_m rows, 4 KN consecutive 64-channel n-blocks)
// for one 256-thread workgroup; wave w streams n-blocks w KN .. w KN + KN - 1 of
// the unit, whose packed weights are one contiguous region (n-block-major, then
// group), so its pipeline runs through KN x K/32 groups without a restart and
// flushes its accumulators at every n-block boundary. KN > 1 only for short
// reductions (K/32 groups too few to fill the pipeline, e.g. the down
// projection of an intermediate-sliced layer). Only the weight nibbles are held
// in registers: a ring of DEPTH batches of U groups, so DEPTH - 1 batches
// (DEPTH - 1 KiB x U per wave) are in flight while one is computed. The row
// block's A fragments (gathered activation rows, shared by the four waves) and
// each wave's group scales go global -> LDS by global_load_lds (no registers in
// flight) into rings of the same depth. Copies and loads of a batch are issued
// together, so the in-order vmcnt covers them all: a wave waits for its own
// batch, then a fence-free barrier publishes every wave's A copies and proves
// the slot refilled next has been consumed.
#include "internal.h"

#include <algorithm>

namespace w4a16 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int kThreads = 256;
constexpr int kUnitNBlocks = 4;  // n-blocks per workgroup unit (one per wave)
// Weights are read exactly once: non-temporal loads keep them from displacing
// reused data in L2 / Infinity Cache and raised a streaming read from 5.8 to
// 6.4 TB/s in a probe. (Cache-policy operand of global_load_lds: 2 = nt.)
constexpr int kNonTemporal = 2;
constexpr uint32_t kCodeMask = 0x000F000Fu;
constexpr uint32_t kBf16_128 = 0x43004300u;
constexpr uint32_t kBf16_Minus136 = 0xC308C308u;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// (a & mask) | magic, one v_and_or_b32. Plain C, not inline asm: the result
// feeds an MFMA operand directly, and an MFMA that reads a VGPR needs two wait
// states after the VALU write of it, which the compiler counts only for
// instructions it can see (inline asm written there left one).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t magic) {
  return (a & mask) | magic;
}

__device__ __forceinline__ bf16x8 codes_to_bf16(uint32_t w, uint32_t magic) {
  u32x4 r;
  r.x = and_or(w, kCodeMask, magic);
  r.y = and_or(w >> 4, kCodeMask, magic);
  r.z = and_or(w >> 8, kCodeMask, magic);
  r.w = and_or(w >> 12, kCodeMask, magic);
  return as_bf16x8(r);
}

__device__ __forceinline__ floatx4 mfma16(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Stores n-block nb of a unit (row block mb) and clears the accumulators.
// Element i of a 16x16 tile is row 4 (lane >> 4) + i, column lane & 15; ids
// yields those rows' sorted_token_ids entries.
template <int MODE, int RB, typename Ids>
__device__ __forceinline__ void store_nblock(const GemmParams& p, floatx4 (&acc)[RB][4], const Ids& ids, int mb,
                                             int nb, int lane) {
  constexpr int BM = 16 * RB;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int prow = mb * BM + rb * 16 + 4 * (lane >> 4) + i;
      const int id = ids(rb, i);
      if ((unsigned)id >= (unsigned)p.n_slots) continue;
      if (MODE == kGateUp) {
        __bf16* h = static_cast<__bf16*>(p.out) + (int64_t)prow * p.out_ld + nb * 32 + (lane & 15);
        h[0] = (__bf16)silu_mul(acc[rb][0][i], acc[rb][2][i]);
        h[16] = (__bf16)silu_mul(acc[rb][1][i], acc[rb][3][i]);
      } else if (p.out_bf16) {
        __bf16* o = static_cast<__bf16*>(p.out) + (int64_t)id * p.out_ld + nb * kNBlock + (lane & 15);
#pragma unroll
        for (int c = 0; c < 4; ++c) o[16 * c] = (__bf16)acc[rb][c][i];
      } else {
        float* y = static_cast<float*>(p.out) + (int64_t)id * p.out_ld + nb * kNBlock + (lane & 15);
#pragma unroll
        for (int c = 0; c < 4; ++c) y[16 * c] = acc[rb][c][i];
      }
    }
  }
  const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[rb][c] = zero4;
}

// KS: waves per n-block (1, 2 or 4). KS > 1 splits each n-block's reduction
// between KS waves of the workgroup (wave part p reduces groups
// [p G/KS, (p+1) G/KS)); a unit then covers 4/KS n-blocks, so a call has KS
// times the units, and the partial sums meet in LDS at the end of the unit,
// added in part order (deterministic).
template <int RB, int U, int DEPTH, int KS = 1>
struct Cfg {
  static constexpr int kABlocks = KS * RB * U;            // 1 KiB A fragments per batch (both halves)
  static constexpr int kACopiesPerWave = kABlocks / 4;    // spread over the 4 waves
  static constexpr int kSCopies = U / 2;                  // 256-byte scale copies per wave per batch
  static constexpr int kOpsPerBatch = kACopiesPerWave + kSCopies + U;
  static constexpr int kABatchBytes = kABlocks * 1024;
  static constexpr int kSBatchBytes = U * kScaleUnitElems * 2;
  static constexpr int kIdsBytes = 16 * RB * 4;  // the row block's sorted_token_ids
  static constexpr int kLdsBytes = DEPTH * kABatchBytes + 4 * DEPTH * kSBatchBytes + kIdsBytes;
  static_assert(kABlocks % 4 == 0 && U % 2 == 0, "batch shape");
  static_assert(kOpsPerBatch * (DEPTH - 2) < 64, "vmcnt range");
};

// Issue batch b (groups b U .. b U + U - 1) into ring slot `slot`: this wave's
// A fragment copies, its scale copies, then its nibble loads (in that order,
// so a wait for the nibbles also covers the copies).
// a_slot < 0: the A fragments of this batch are already resident (short K,
// see the kernel); otherwise they are copied into A slot a_slot.
template <int RB, int U, int DEPTH, int KS>
__device__ __forceinline__ void issue_batch(u32x4 (&nib)[U], int slot, int a_slot, int b, int G, int wave,
                                            const uint8_t* const* a_src,
                                            const uint8_t* ws, const uint8_t* wq, uint8_t* a_ring, uint8_t* s_ring) {
  using C = Cfg<RB, U, DEPTH, KS>;
  int g0 = b * U;
  asm volatile("" : "+s"(g0));  // keep the look-ahead where it is written
  const int ga = g0 % G;        // the A rows cycle through K once per n-block
  if (a_slot >= 0) {
#pragma unroll
    for (int t = 0; t < C::kACopiesPerWave; ++t) {
      const int j = wave + 4 * t;
      __builtin_amdgcn_global_load_lds(a_src[t] + (int64_t)ga * (kGroup * 2),
                                       LDS_PTR(a_ring + a_slot * C::kABatchBytes + j * 1024), 16, 0, 0);
    }
  }
#pragma unroll
  for (int t = 0; t < C::kSCopies; ++t)
    __builtin_amdgcn_global_load_lds(ws + (int64_t)(g0 + 2 * t) * (kScaleUnitElems * 2),
                                     LDS_PTR(s_ring + slot * C::kSBatchBytes + t * 256), 4, 0, kNonTemporal);
#pragma unroll
  for (int uu = 0; uu < U; ++uu)
    nib[uu] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wq + (int64_t)(g0 + uu) * kNibUnitBytes));
}

// ---- alignment inside the gate_up launch (decode-sized calls) ---------------
// For a few routed ids (n <= kFuseMaxIds over E <= kFuseMaxExperts local
// experts, block_m 16) the alignment is cheaper to redo in every workgroup of
// the gate_up launch than to run as a launch of its own ahead of it: each
// workgroup sorts the ids in LDS exactly as moe_align does (stable counting
// sort, blocks of 16 rows padded with the sentinel n, experts in order),
// keeps its own units' row ids and experts, and workgroup 0 also writes
// sorted_token_ids, expert_ids and num_tokens_post_padded for the down GEMM.
constexpr int kFuseMaxIds = 1024;
constexpr int kFuseMaxExperts = 64;
constexpr int kFuseMaxUnitsPerWg = 4;
constexpr int kFuseVWaves = kFuseMaxIds / 64;  // 64-id slices of the ids, in order
constexpr int kUnitTab = 17;                   // per unit: expert, then its 16 row ids

struct FusedAlign {
  const int32_t* ids;  // topk_ids, n of them
  int n;
  int32_t* sorted;  // outputs as moe_align writes them (capacity p.capacity)
  int32_t* expert_ids;
  int32_t* ntpp;
};

// Bytes of LDS the in-launch alignment uses before the weight stream starts
// (inside the A ring): per-slice counts, offsets, the sorted rows and the
// block experts.
__host__ __device__ constexpr size_t fused_align_scratch_bytes(int capacity) {
  return 4 * ((size_t)kFuseVWaves * kFuseMaxExperts + kFuseMaxExperts + 1 + (size_t)capacity + (capacity + 15) / 16);
}

// Returns num_tokens_post_padded; fills tab[k] (k < units of this workgroup)
// with the expert and the 16 row ids of unit u_begin + k. All 256 threads.
__device__ int fused_align(const FusedAlign& fa, int E, int capacity, int NG, int* scratch, int* tab) {
  const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nblk = (capacity + 15) / 16;
  int* wcnt = scratch;                              // [slice][expert]
  int* off = wcnt + kFuseVWaves * kFuseMaxExperts;  // [expert], then the padded total
  int* srt = off + kFuseMaxExperts + 1;             // [capacity]
  int* ex = srt + capacity;                         // [nblk]
  for (int i = tid; i < kFuseVWaves * kFuseMaxExperts; i += kThreads) wcnt[i] = 0;
  for (int i = tid; i < capacity; i += kThreads) srt[i] = fa.n;
  for (int i = tid; i < nblk; i += kThreads) ex[i] = -1;
  constexpr int kRounds = kFuseMaxIds / kThreads;
  int v[kRounds], rank[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int j = r * kThreads + tid;
    v[r] = j < fa.n ? fa.ids[j] : -1;
  }
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  // slice r * 4 + wave holds ids [64 (r * 4 + wave), +64): ranks by ballot over the expert bits
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int e = v[r];
    const bool local = (unsigned)e < (unsigned)E;
    uint64_t peers = __ballot(local);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(local && bit);
      peers &= bit ? m : ~m;
    }
    rank[r] = __builtin_amdgcn_mbcnt_hi((uint32_t)(peers >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)peers, 0));
    if (local && rank[r] == 0) wcnt[(r * 4 + wave) * kFuseMaxExperts + e] = __popcll(peers);
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  if (wave == 0) {
    // lane e: the expert's count before each slice, its padded size, its offset
    int before = 0;
    for (int q = 0; q < kFuseVWaves; ++q) {
      const int c = wcnt[q * kFuseMaxExperts + lane];
      wcnt[q * kFuseMaxExperts + lane] = before;
      before += c;
    }
    const int pc = lane < E ? (before + 15) & ~15 : 0;
    int incl = pc;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int t = __shfl_up(incl, d);
      if (lane >= d) incl += t;
    }
    const int o = incl - pc;
    off[lane] = o;
    if (lane == 63) off[kFuseMaxExperts] = incl;
    for (int b = o / 16; b < (o + pc) / 16 && b < nblk; ++b) ex[b] = lane;
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int e = v[r];
    if ((unsigned)e < (unsigned)E) {
      const int pos = off[e] + wcnt[(r * 4 + wave) * kFuseMaxExperts + e] + rank[r];
      if (pos < capacity) srt[pos] = r * kThreads + tid;
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  const int ntpp = min(off[kFuseMaxExperts], capacity);
  if (blockIdx.x == 0) {
    for (int i = tid; i < capacity; i += kThreads) fa.sorted[i] = srt[i];
    for (int i = tid; i < nblk; i += kThreads) fa.expert_ids[i] = ex[i];
    if (tid == 0) *fa.ntpp = ntpp;
  }
  const int units = ntpp / 16 * NG;
  const int per_wg = (units + (int)gridDim.x - 1) / (int)gridDim.x;
  const int u_begin = (int)blockIdx.x * per_wg;
  const int nu = min(min(units - u_begin, per_wg), kFuseMaxUnitsPerWg);
  for (int i = tid; i < nu * kUnitTab; i += kThreads) {
    const int k = i / kUnitTab, j = i - k * kUnitTab;
    const int mb = (u_begin + k) / NG;
    tab[i] = j == 0 ? ex[mb] : srt[mb * 16 + j - 1];
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  return ntpp;
}

// MULTI: KN > 1 (n-block boundaries inside the batch loop); otherwise KN == 1
// and the single n-block is stored after the loop, which keeps the common
// long-K kernel's register count where it was. With MULTI and K / 32 <= U x DEPTH
// groups the row block's A fragments for the whole of K fit the A ring: they
// are copied during the first n-block only and stay resident for the others.
// ALIGN: the alignment runs inside this launch (fused_align; RB 1, no MULTI):
// expert and row ids come from the workgroup's unit table in LDS.
template <int MODE, int RB, int U, int DEPTH, bool MULTI, int KS, bool ALIGN = false>
__global__ __launch_bounds__(kThreads) void moe_gemm_stream_lds_kernel(GemmParams p, int KN, FusedAlign fa) {
  static_assert(KS == 1 || ((KS == 2 || KS == 4) && !MULTI), "a split reduction runs one n-block per wave");
  static_assert(!ALIGN || (RB == 1 && !MULTI), "the in-launch alignment serves 16-row units");
  using C = Cfg<RB, U, DEPTH, KS>;
  constexpr int BM = 16 * RB;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = (int)threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  __builtin_assume(wave >= 0 && wave < kThreads / 64);  // lets copy indices fold per unrolled step
  uint8_t* a_ring = lds;
  uint8_t* s_ring = lds + DEPTH * C::kABatchBytes + wave * DEPTH * C::kSBatchBytes;
  int* row_ids = reinterpret_cast<int*>(lds + DEPTH * C::kABatchBytes + 4 * DEPTH * C::kSBatchBytes);
  int* unit_tab = row_ids + C::kIdsBytes / 4;  // ALIGN only

  const int NB = p.N / kNBlock;
  const int NG = NB / (kUnitNBlocks / KS * KN);  // units per row block
  const int ntpp = ALIGN ? fused_align(fa, p.E, p.capacity, NG, reinterpret_cast<int*>(lds), unit_tab)
                         : min(*p.ntpp, p.capacity);
  const int n_mblocks = ntpp / BM;
  const int G = p.K / kGroup;
  const int Gw = G / KS;                    // groups of one n-block this wave reduces
  const int kh = KS > 1 ? wave % KS : 0;    // which part of K
  const int nbatch = KN * Gw / U;           // batches per wave per unit
  const int kbatch = Gw / U;                // batches per n-block
  const bool a_resident = MULTI && kbatch <= DEPTH;
  const int units = n_mblocks * NG;
  const int per_wg = (units + (int)gridDim.x - 1) / (int)gridDim.x;
  const int u_begin = (int)blockIdx.x * per_wg;
  const int u_end = min(units, u_begin + per_wg);
  uint32_t magic = kBf16_128;
  asm volatile("v_mov_b32 %0, %1" : "=v"(magic) : "s"(magic));
  const bf16x8 minus136 = as_bf16x8(u32x4{kBf16_Minus136, kBf16_Minus136, kBf16_Minus136, kBf16_Minus136});
  const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};

  for (int unit = u_begin; unit < u_end; ++unit) {
    const int mb = unit / NG;
    const int ng = unit - mb * NG;
    const int* tab = unit_tab + (unit - u_begin) * kUnitTab;  // ALIGN only
    const int e = ALIGN ? tab[0] : p.expert_ids[mb];
    if ((unsigned)e >= (unsigned)p.E) continue;  // uniform across the workgroup
    const int nb0 = (ng * (kUnitNBlocks / KS) + wave / KS) * KN;  // this wave's first n-block

    // A copy sources: this wave copies fragment blocks j = wave + 4 t of each
    // batch, block j = (part of K j / (RB U), row block, group); the part
    // offsets the source by Gw groups. Padding rows read the row block's first
    // row; their results are never stored.
    const uint8_t* a_src[C::kACopiesPerWave];
#pragma unroll
    for (int t = 0; t < C::kACopiesPerWave; ++t) {
      const int j = wave + 4 * t;
      const int khj = KS > 1 ? j / (RB * U) : 0, jj = KS > 1 ? j % (RB * U) : j;
      const int rb = jj / U, uu = jj % U;
      const int prow = mb * BM + rb * 16 + (lane & 15);
      const int id = ALIGN ? tab[1 + rb * 16 + (lane & 15)] : p.sorted[prow];
      const bool real = (unsigned)id < (unsigned)p.n_slots;
      int64_t src;
      if (MODE == kGateUp) {
        const int id0 = ALIGN ? tab[1] : p.sorted[mb * BM];
        src = (real ? id : id0) / p.topk;
      } else {
        src = real ? prow : mb * BM;
      }
      a_src[t] = reinterpret_cast<const uint8_t*>(p.a + src * p.K) + 16 * (lane >> 4) + uu * (kGroup * 2) +
                 (int64_t)khj * Gw * (kGroup * 2);
    }
    const int64_t unit0 = ((int64_t)e * NB + nb0) * G + (int64_t)kh * Gw;
    const uint8_t* wq = p.wq + unit0 * kNibUnitBytes + 16 * lane;
    const uint8_t* ws = reinterpret_cast<const uint8_t*>(p.ws + unit0 * kScaleUnitElems) + 4 * lane;

    floatx4 acc[RB][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[rb][c] = zero4;

    u32x4 nib[DEPTH][U];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    ring_barrier();  // the previous unit's reads of every slot are done
    if (MULTI) {
      // Stores inside the weight stream read the row ids from LDS: a global
      // load there would make the wave wait for every batch in flight.
      if (threadIdx.x < BM) row_ids[threadIdx.x] = p.sorted[mb * BM + threadIdx.x];
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // visible after the next barrier
    }
    const auto lds_ids = [&](int rb, int i) { return row_ids[rb * 16 + 4 * (lane >> 4) + i]; };
    const auto mem_ids = [&](int rb, int i) {
      return ALIGN ? tab[1 + rb * 16 + 4 * (lane >> 4) + i] : p.sorted[mb * BM + rb * 16 + 4 * (lane >> 4) + i];
    };
#pragma unroll
    for (int s = 0; s < DEPTH - 1; ++s)
      if (s < nbatch)
        issue_batch<RB, U, DEPTH, KS>(nib[s], s, a_resident ? (s < kbatch ? s : -1) : s, s, G, wave, a_src, ws,
                                      wq, a_ring, s_ring);

    for (int b0 = 0; b0 < nbatch; b0 += DEPTH) {
#pragma unroll
      for (int k = 0; k < DEPTH; ++k) {
        const int b = b0 + k;
        if (b < nbatch) {
          // own copies and loads of batch b landed (later ones may be pending;
          // with resident A, later batches may hold fewer ops, so count without
          // A copies: that waits for at least as much as needed) ...
          if (b + DEPTH - 2 < nbatch) {
            if (MULTI) wait_vmcnt<(C::kOpsPerBatch - C::kACopiesPerWave) * (DEPTH - 2)>();
            else wait_vmcnt<C::kOpsPerBatch * (DEPTH - 2)>();
          } else {
            wait_vmcnt<0>();
          }
          // ... and everyone's; everyone also finished computing batch b - 1
          ring_barrier();
          if (b + DEPTH - 1 < nbatch) {
            const int bn = b + DEPTH - 1, sn = (k + DEPTH - 1) % DEPTH;
            issue_batch<RB, U, DEPTH, KS>(nib[sn], sn, a_resident ? (bn < kbatch ? bn : -1) : sn, bn, G, wave, a_src,
                                          ws, wq, a_ring, s_ring);
          }
          const uint8_t* abase = a_ring + (a_resident ? b % kbatch : k) * C::kABatchBytes + kh * (RB * U * 1024);
          const uint8_t* sbase = s_ring + k * C::kSBatchBytes;
#pragma unroll
          for (int uu = 0; uu < U; ++uu) {
            const u32x2 sc = *reinterpret_cast<const u32x2*>(sbase + uu * 128 + 8 * (lane & 15));
            const float scale[4] = {__uint_as_float(sc.x << 16), __uint_as_float(sc.x & 0xFFFF0000u),
                                    __uint_as_float(sc.y << 16), __uint_as_float(sc.y & 0xFFFF0000u)};
            bf16x8 w[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) w[c] = codes_to_bf16(nib[k][uu][c], magic);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
              const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(abase + (rb * U + uu) * 1024 + 16 * lane));
              const floatx4 corr = mfma16(a, minus136, zero4);
#pragma unroll
              for (int c = 0; c < 4; ++c) acc[rb][c] += scale[c] * mfma16(a, w[c], corr);
            }
          }
          // the last batch of an n-block: store it (uniform branch)
          if (MULTI && ((b + 1) * U) % G == 0) store_nblock<MODE, RB>(p, acc, lds_ids, mb, nb0 + ((b + 1) * U) / G - 1, lane);
        }
      }
    }
    if (KS > 1) {
      // the parts' waves hand their partial sums to part 0's wave through LDS
      // (the rings are free once every wave passed this barrier with its own
      // ring reads complete); part 0 adds them in part order
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      ring_barrier();
      constexpr int kPart = RB * 16 * 64;  // floats of one wave's accumulators
      float* xch = reinterpret_cast<float*>(lds) + (wave / KS) * (KS - 1) * kPart;
      if (kh > 0) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) xch[(kh - 1) * kPart + ((rb * 4 + c) * 4 + i) * 64 + lane] = acc[rb][c][i];
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      ring_barrier();
      if (kh == 0) {
#pragma unroll
        for (int q = 0; q < KS - 1; ++q)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[rb][c][i] += xch[q * kPart + ((rb * 4 + c) * 4 + i) * 64 + lane];
        store_nblock<MODE, RB>(p, acc, mem_ids, mb, nb0, lane);
      }
    } else if (!MULTI) {
      store_nblock<MODE, RB>(p, acc, mem_ids, mb, nb0, lane);
    }
  }
}

// n-blocks per wave: enough for about kMinGroupsPerWave groups of pipeline per
// unit when K is short, a divisor of the n-blocks per wave lane so units tile N.
constexpr int kMinGroupsPerWave = 64;
int n_blocks_per_wave(const GemmParams& p) {
  const int G = p.K / kGroup;
  const int NG = p.N / (kNBlock * kUnitNBlocks);
  int kn = 1;
  for (int k = 1; k <= NG && (k - 1) * G < kMinGroupsPerWave; ++k)
    if (NG % k == 0) kn = k;
  return kn;
}

template <int MODE, int RB, int U, int DEPTH, bool MULTI, int KS>
hipError_t launch_kn(const GemmParams& p, int kn, hipStream_t stream) {
  using C = Cfg<RB, U, DEPTH, KS>;
  constexpr int BM = 16 * RB;
  const int64_t units_max = (int64_t)(p.capacity / BM) * (p.N / (kNBlock * (kUnitNBlocks / KS) * kn));
  if (units_max == 0) return hipSuccess;
  static int blocks_per_cu = [] {
    (void)hipFuncSetAttribute(
        reinterpret_cast<const void*>(moe_gemm_stream_lds_kernel<MODE, RB, U, DEPTH, MULTI, KS>),
        hipFuncAttributeMaxDynamicSharedMemorySize, C::kLdsBytes);
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, moe_gemm_stream_lds_kernel<MODE, RB, U, DEPTH, MULTI, KS>,
                                                     kThreads, C::kLdsBytes) != hipSuccess ||
        n < 1)
      n = 1;
    return n;
  }();
  // Up to 4x the resident workgroups: when the live units outnumber the
  // resident slots, queued workgroups start as others finish, instead of a
  // resident workgroup restarting its pipeline for a second unit (measured
  // faster for the decode down projection).
  const int64_t grid = std::min<int64_t>(units_max, (int64_t)device_cu_count() * blocks_per_cu * 4);
  hipLaunchKernelGGL((moe_gemm_stream_lds_kernel<MODE, RB, U, DEPTH, MULTI, KS>), dim3((int)grid), dim3(kThreads),
                     C::kLdsBytes, stream, p, kn, FusedAlign{});
  return hipGetLastError();
}

// Reductions of at least kSplitMinGroups groups at block_m 16 split each
// n-block between two waves: the decode weight stream has too few units to
// give every resident workgroup one (e.g. 40 active experts x 16 units against
// 1024 resident slots), and twice the units keep more of it in flight.
constexpr int kSplitMinGroups = 64;

template <int MODE, int RB, int U, int DEPTH>
hipError_t launch(const GemmParams& p, hipStream_t stream) {
  const int kn = n_blocks_per_wave(p);
  if (kn > 1) return launch_kn<MODE, RB, U, DEPTH, true, 1>(p, kn, stream);
  if (RB == 1 && p.K / kGroup >= kSplitMinGroups && (p.K / kGroup) % (2 * U) == 0 &&
      (p.N / kNBlock) % (kUnitNBlocks / 2) == 0)
    return launch_kn<MODE, RB, U, DEPTH, false, 2>(p, 1, stream);
  return launch_kn<MODE, RB, U, DEPTH, false, 1>(p, 1, stream);
}

template <int MODE>
hipError_t launch_mode(int32_t block_m, const GemmParams& p, hipStream_t stream) {
  switch (block_m) {
    // gate_up's reduction (K = hidden) is long enough to use a 4-deep ring
    // (3 batches in flight; 3 waves per SIMD); the down projection's shorter
    // one runs better at 3 deep and 4 waves per SIMD
    case 16: return MODE == kGateUp ? launch<MODE, 1, 4, 4>(p, stream) : launch<MODE, 1, 4, 3>(p, stream);
    case 32: return launch<MODE, 2, 4, 4>(p, stream);
    case 64: return launch<MODE, 4, 4, 3>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gate_up_fused_align(const GemmParams& p, const int32_t* ids, int32_t n, int32_t* sorted,
                                      int32_t* expert_ids, int32_t* ntpp, hipStream_t stream) {
  constexpr int RB = 1, U = 4, DEPTH = 4, KS = 2;
  using C = Cfg<RB, U, DEPTH, KS>;
  const int G = p.K / kGroup;
  const int NB = p.N / kNBlock;
  // the block_m 16 split configuration launch() picks for a long gate_up reduction
  if (n < 1 || n > kFuseMaxIds || p.E > kFuseMaxExperts || !stream_lds_supported(16, p) ||
      n_blocks_per_wave(p) != 1 || G < kSplitMinGroups || G % (2 * U) != 0 || NB % (kUnitNBlocks / KS) != 0)
    return hipErrorNotSupported;
  if (fused_align_scratch_bytes(p.capacity) > (size_t)DEPTH * C::kABatchBytes) return hipErrorNotSupported;
  const int NG = NB / (kUnitNBlocks / KS);
  const int64_t units_max = (int64_t)(p.capacity / 16) * NG;
  if (units_max == 0) return hipErrorNotSupported;
  constexpr int kLds = C::kLdsBytes + kFuseMaxUnitsPerWg * kUnitTab * 4;
  static int blocks_per_cu = [] {
    (void)hipFuncSetAttribute(
        reinterpret_cast<const void*>(moe_gemm_stream_lds_kernel<kGateUp, RB, U, DEPTH, false, KS, true>),
        hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, moe_gemm_stream_lds_kernel<kGateUp, RB, U, DEPTH, false, KS, true>,
                                                     kThreads, kLds) != hipSuccess ||
        b < 1)
      b = 1;
    return b;
  }();
  const int64_t grid = std::min<int64_t>(units_max, (int64_t)device_cu_count() * blocks_per_cu * 4);
  if ((units_max + grid - 1) / grid > kFuseMaxUnitsPerWg) return hipErrorNotSupported;
  const FusedAlign fa{ids, n, sorted, expert_ids, ntpp};
  hipLaunchKernelGGL((moe_gemm_stream_lds_kernel<kGateUp, RB, U, DEPTH, false, KS, true>), dim3((int)grid),
                     dim3(kThreads), kLds, stream, p, 1, fa);
  return hipGetLastError();
}

bool stream_lds_supported(int32_t block_m, const GemmParams& p) {
  return (block_m == 16 || block_m == 32 || block_m == 64) && p.N % (kNBlock * kUnitNBlocks) == 0 &&
         (p.K / kGroup) % 4 == 0;
}

hipError_t launch_moe_gemm_stream_lds(GemmMode mode, int32_t block_m, const GemmParams& p, hipStream_t stream) {
  return mode == kGateUp ? launch_mode<kGateUp>(block_m, p, stream) : launch_mode<kDown>(block_m, p, stream);
}

}  // namespace w4a16
