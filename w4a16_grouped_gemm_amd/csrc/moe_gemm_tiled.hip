// Tiled W4A16 expert GEMM for many tokens per expert (block_m = 128).
//
// Once experts carry enough rows, the MFMA work rather than weight streaming
// sets the time (the pages' observation that tokens per expert, not total
// tokens, decides which schedule wins: Chord page "vLLM 및 Novita AI, Kimi
// K2.x용 더 빠른 INT4 MoE 커널 출시: Chord", section "핵심 기여"; and the
// small- vs large-batch pipelines of the Humming announcement, "Humming:
// vLLM과 Ant Group, 양자화 추론을 위한 범용 커널 라이브러리 오픈소스 공개",
// section "워크로드별 튜닝 및 JIT 컴파일").
//
// Arithmetic: fp16 operands on v_mfma_f32_16x16x32_f16, fp32 accumulation.
// Both operands are exact images of the bf16/int4 inputs:
//   * weights: q * s' where s' = s * 2^-E_n is the group scale normalised by a
//     power of two per output channel (the channel's largest scale lands in
//     [16, 32)). q has at most 3 significant bits and s' at most 8, so q * s'
//     is an exact fp16 value; it is formed with one exact packed-fp16 fma
//     from the code (q + 8), rotated to bits 6-9 of a half and OR-ed into the
//     mantissa of fp16 16.0 (see dequant_half).
//   * activations: rows converted by rows_to_f16 with a power-of-two row factor
//     (largest element mapped into [2^14, 2^15)).
// Every product is exact, the sum is fp32 (as the scalar definition), and the
// epilogue restores 2^(row exponent + E_n) with one ldexp per output. No
// per-group rescale is needed: the group scale lives in the B operand.
// The one approximation is fp16's subnormal floor: an activation more than 2^31
// below its row's largest (a bf16 value, 8 significant bits, is exact in fp16
// down to 2^-17), or a scale more than 2^17 below its channel's
// largest, is rounded to the fp16 subnormal grid (absolute error at most 2^-39
// of the row's largest element, resp. 2^-25 of the channel's largest scale),
// far below the rounding of the fp32 sum itself. SiLU's exponential tail puts
// such tiny elements in h routinely; they cannot move a result that the fp32
// sum resolves.
//
// Tile: a 512-thread workgroup (8 waves) computes 128 rows x 512 channels
// (eight 64-channel n-blocks) over the whole reduction; a half tile (256
// channels) uses four of the waves. Wave w owns all 128 rows and the four
// 16-channel column blocks of n-block w (for gate_up: gate channels in blocks
// 0, 1 and the matching up channels in 2, 3), so each weight is dequantised by
// exactly one wave and feeds 8 row blocks of MFMAs, and each A fragment read
// from LDS feeds 4 MFMAs. The K loop moves in stages of two groups:
//   A  128 rows x 64 k of fp16 (16 KiB), gathered through sorted_token_ids and
//      shared by the waves of the tile,
//   B  per wave, its own n-block's 2 groups of packed nibbles (2 KiB) and fp16
//      scales (256 B),
// copied global -> LDS by global_load_lds_dwordx4 / _dword (no VGPRs in flight)
// into a ring of kStages stages. LDS A is fragment-major (row block, group,
// lane, 16 bytes): every MFMA operand is one conflict-free ds_read_b128. The
// in-order vmcnt tracks the copies. A wave's weights are its own copies, so it
// reads and dequantises the next stage's first group as soon as its own copies
// of that stage landed, under the current stage's second group of MFMAs; the A
// fragments need every wave's copies, published by one workgroup barrier per
// stage, which also proves the slot refilled next has been consumed.
//
#include "internal.h"

#include <algorithm>

namespace w4a16 {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kStages = 3;            // LDS ring depth
constexpr int kTileM = 128;
constexpr int kRowBlocks = kTileM / 16;
constexpr int kTileNBlocks = kWaves;  // full tile: 8 x 64 = 512 channels, one n-block per wave
constexpr int kHalfNBlocks = kTileNBlocks / 2;
constexpr int kStageGroups = 2;       // 64 k per stage
constexpr int kABytes = kTileM * kStageGroups * kGroup * 2;                  // 16 KiB
constexpr int kBWaveBytes = kStageGroups * kNibUnitBytes;                    // 2 KiB
constexpr int kSWaveBytes = kStageGroups * kScaleUnitElems * 2;              // 256 B
constexpr int kBOffset = kABytes;
constexpr int kSOffset = kABytes + kWaves * kBWaveBytes;
constexpr int kStageBytes = kSOffset + kWaves * kSWaveBytes;                 // 34 KiB
// row blocks a wave copies when nw waves work on the tile
constexpr int a_blocks_per_wave(int nw) { return kRowBlocks / nw; }
// copies per wave and stage: its A row blocks x groups, its nibbles (one per
// group) and its scales (both groups in one)
constexpr int copies_per_wave_stage(int nw) { return a_blocks_per_wave(nw) * kStageGroups + kStageGroups + 1; }
// A fragments read ahead of the MFMAs that use them
constexpr int kAhead = 4;
// Weights and scales are read once per tile: they are copied with the
// non-temporal policy (nt) so they do not evict the A tile shared through L2.
constexpr bool kWeightsNonTemporal = true;

constexpr uint32_t kCodeMid = 0x03C003C0u;  // bits 6-9 of each half
constexpr uint32_t kF16_16 = 0x4C004C00u;    // fp16 16.0 in both halves

// (a & mask) | magic as one v_and_or_b32 (in C the compiler folds the rotate
// before it into other instructions). Its result only ever feeds the fma of
// dequant_half, a VALU: an MFMA never reads a register this asm writes, so the
// two wait states an MFMA needs after a VALU write of its operand, which the
// compiler counts only for instructions it can see, are not at stake here.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t magic) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(mask), "v"(magic));
  return r;
}

// Four of the eight codes of one column block -> fp16 (code - 8) * s, exactly:
// half 0 gives elements 0-3 (codes at bits 0-3 and 4-7 of each 16-bit half of
// w), half 1 elements 4-7 (bits 8-11 and 12-15). A rotation brings a code to
// bits 6-9 of its half, where OR-ed into fp16 16.0 (mantissa unit 1/64) it
// makes 16 + code; one fma then gives (16 + code) * s - 24 * s. That is exact:
// s is an 8-bit significand times a power of two, so 24 * s = 8 * (3 * s)
// needs at most 10 significant bits and the result (code - 8) * s at most 11,
// and the fma rounds an exact value once. (An offset of 1024 + code would need
// 1032 * s, 16 bits: only codes at bits 5 or 6 of a half give an offset whose
// multiple of s fits fp16.) c2 holds -24 * s.
__device__ __forceinline__ u32x2 dequant_half(uint32_t w, int half, f16x2 s2, f16x2 c2, uint32_t magic) {
  const uint32_t r0 = __builtin_amdgcn_alignbit(w, w, half ? 2 : 26);   // rotate right
  const uint32_t r1 = __builtin_amdgcn_alignbit(w, w, half ? 6 : 30);
  f16x2 t0 = __builtin_bit_cast(f16x2, and_or(r0, kCodeMid, magic));
  f16x2 t1 = __builtin_bit_cast(f16x2, and_or(r1, kCodeMid, magic));
  t0 = __builtin_elementwise_fma(t0, s2, c2);
  t1 = __builtin_elementwise_fma(t1, s2, c2);
  return u32x2{__builtin_bit_cast(uint32_t, t0), __builtin_bit_cast(uint32_t, t1)};
}

__device__ __forceinline__ f16x8 join_halves(u32x2 lo, u32x2 hi) {
  return __builtin_bit_cast(f16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
}

__device__ __forceinline__ floatx4 mfma16(f16x8 a, f16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}


__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Lane quads (lanes 4m .. 4m + 3) transpose a 4 x 4 block: before, lane j
// holds a[i] = M[i][j]; after, lane j holds a[i] = M[j][i]. Two rounds of DPP
// quad permutations: swap with lane j ^ 1 the elements whose index differs
// from j in bit 0, then with lane j ^ 2 those that differ in bit 1.
template <int CTRL>
__device__ __forceinline__ float quad_dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ void quad_transpose(float (&a)[4], int lane) {
  constexpr int kSwap1 = 0xB1;  // quad_perm [1, 0, 3, 2]
  constexpr int kSwap2 = 0x4E;  // quad_perm [2, 3, 0, 1]
  const bool odd = lane & 1, hi = lane & 2;
  {
    const float t0 = quad_dpp<kSwap1>(a[1]), t1 = quad_dpp<kSwap1>(a[0]);
    const float t2 = quad_dpp<kSwap1>(a[3]), t3 = quad_dpp<kSwap1>(a[2]);
    a[0] = odd ? t0 : a[0];
    a[1] = odd ? a[1] : t1;
    a[2] = odd ? t2 : a[2];
    a[3] = odd ? a[3] : t3;
  }
  {
    const float t0 = quad_dpp<kSwap2>(a[2]), t1 = quad_dpp<kSwap2>(a[3]);
    const float t2 = quad_dpp<kSwap2>(a[0]), t3 = quad_dpp<kSwap2>(a[1]);
    a[0] = hi ? t0 : a[0];
    a[1] = hi ? t1 : a[1];
    a[2] = hi ? a[2] : t2;
    a[3] = hi ? a[3] : t3;
  }
}

__device__ __forceinline__ f16x2 splat(uint32_t bits16) {
  const _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)bits16);
  return f16x2{h, h};
}

// Wait until at most N of this wave's vector-memory operations are pending.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Global -> LDS copy of BYTES per lane (16 or 4) into LDS at `lds` + 4/16 * lane,
// issued from an asm block: the compiler counts a global_load_lds builtin as
// a possible LDS access on the LDS counter, and then makes every later LDS
// read wait for all of them (lgkmcnt(0)) instead of for its own. The copy
// has no register result (it writes LDS); its address is read at issue. The
// waits for the copies are explicit (wait_vmcnt), and the "memory" clobber
// keeps LDS reads on their side of it. M0 holds the LDS base; setting it needs
// one wait state before the copy. M0 is a register the compiler reserves (it
// warns about the clobber); no code in this file keeps a value in it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int BYTES, bool NT>
__device__ __forceinline__ void copy_to_lds(const void* src, const void* lds) {
  const uint32_t base = (uint32_t)(uintptr_t)LDS_PTR(lds);
  if (BYTES == 16 && NT)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src), "s"(base)
                 : "memory", "m0");
  else if (BYTES == 16)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(base)
                 : "memory", "m0");
  else if (NT)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off nt" ::"v"(src), "s"(base)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(base)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Workgroup barrier without a memory fence. __syncthreads() would make every
// wave drain all of its in-flight copies first (vmcnt(0)); here each wave has
// already waited for exactly the copies that must have landed, and the
// "memory" clobbers keep the compiler from moving LDS reads across the barrier.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait until this wave's copies of a stage landed while the copies of
// `later` stages issued after it may still be in flight (0 <= later < kStages - 1).
template <int NW>
__device__ __forceinline__ void wait_stage(int later) {
  static_assert(kStages <= 4, "wait_stage covers up to two later stages");
  if (kStages > 3 && later >= 2) wait_vmcnt<2 * copies_per_wave_stage(NW)>();
  else if (later >= 1) wait_vmcnt<copies_per_wave_stage(NW)>();
  else wait_vmcnt<0>();
}

struct TileCtx {
  const uint8_t* a_src[a_blocks_per_wave(kWaves / 2)];  // this lane's A copy sources (row start + 16-byte k offset)
  const uint8_t* wq;  // this wave's n-block: nibble units from group 0, + 16 lane
  const uint8_t* ws;  // this wave's n-block: fp16 scale units from group 0, + 4 lane
};

// Issue this wave's copies of stage `s` (groups 2s, 2s+1) into ring slot `slot`:
// its own nibbles and scales, then its share (nab row blocks) of the A tile.
__device__ __forceinline__ void issue_stage(const TileCtx& c, uint8_t* ring, int slot, int s, int wave, int nab) {
  uint8_t* base = ring + slot * kStageBytes;
  const int g0 = s * kStageGroups;
#pragma unroll
  for (int j = 0; j < kStageGroups; ++j)
    copy_to_lds<16, kWeightsNonTemporal>(c.wq + (int64_t)(g0 + j) * kNibUnitBytes,
                          base + kBOffset + wave * kBWaveBytes + j * kNibUnitBytes);
  // the two groups' scale units are adjacent: 64 lanes x 4 bytes cover both
  copy_to_lds<4, kWeightsNonTemporal>(c.ws + (int64_t)g0 * (kScaleUnitElems * 2), base + kSOffset + wave * kSWaveBytes);
#pragma unroll
  for (int t = 0; t < nab; ++t)
#pragma unroll
    for (int j = 0; j < kStageGroups; ++j) {
      const int rb = nab * wave + t;
      copy_to_lds<16, false>(c.a_src[t] + (int64_t)(g0 + j) * (kGroup * 2), base + (rb * kStageGroups + j) * 1024);
    }
}

// The K loop and epilogue of one tile (NW waves, NW n-blocks from nb0) for the
// wave owning n-block nb0 + wave.
template <int MODE, int NW>
__device__ __forceinline__ void tile_body(const GemmParams& p, const TileCtx& c, uint8_t* ring, int nstages,
                                          int mb, int nb0, int e, int wave, int lane) {
  const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
  uint32_t magic = kF16_16;
  asm volatile("v_mov_b32 %0, %1" : "=v"(magic) : "s"(magic));
  floatx4 acc[kRowBlocks][4];
#pragma unroll
  for (int rb = 0; rb < kRowBlocks; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = zero4;

  // this wave's own weights of a stage: group j's 16 bytes of nibbles and the
  // four scales of its column (entry 4 * (lane & 15) + cb of the unit)
  const auto nib_of = [&](int slot, int j) {
    return *reinterpret_cast<const u32x4*>(ring + slot * kStageBytes + kBOffset + wave * kBWaveBytes +
                                           j * kNibUnitBytes + 16 * lane);
  };
  const auto sc_of = [&](int slot, int j) {
    return *reinterpret_cast<const u32x2*>(ring + slot * kStageBytes + kSOffset + wave * kSWaveBytes +
                                           j * (kScaleUnitElems * 2) + 8 * (lane & 15));
  };
  // -24 * s for the four column blocks' scales of a group (two per word)
  // (the words are copied out first: a bit cast of a vector element lvalue
  // compiles to a read of the vector's first element)
  const auto neg24 = [](const u32x2& sc) {
    const f16x2 m24 = {(_Float16)-24.0f, (_Float16)-24.0f};
    const uint32_t lo = sc.x, hi = sc.y;
    return u32x2{__builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, lo) * m24),
                 __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, hi) * m24)};
  };
  // half h of column block cb's dequantised fragment
  const auto deqh = [&](const u32x4& nib, const u32x2& sc, const u32x2& cs, int cb, int h) {
    const uint32_t sbits = (cb & 2) ? sc.y : sc.x, cbits = (cb & 2) ? cs.y : cs.x;
    const f16x2 s2 = splat((cb & 1) ? sbits >> 16 : sbits & 0xFFFFu);
    const f16x2 c2 = splat((cb & 1) ? cbits >> 16 : cbits & 0xFFFFu);
    return dequant_half(nib[cb], h, s2, c2, magic);
  };

  // the previous tile's reads of every slot are done before it is refilled
  ring_barrier();
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s)
    if (s < nstages) issue_stage(c, ring, s, s, wave, a_blocks_per_wave(NW));

  // stage 0's first group, dequantised before the loop, and its second
  // group's nibbles and scales (own copies only)
  wait_stage<NW>(min(nstages, kStages - 1) - 1);
  f16x8 w[4];
  u32x4 nib1 = nib_of(0, 1);
  u32x2 sc1 = sc_of(0, 1);
  {
    const u32x4 nb = nib_of(0, 0);
    const u32x2 sc = sc_of(0, 0);
    const u32x2 cs = neg24(sc);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) w[cb] = join_halves(deqh(nb, sc, cs, cb, 0), deqh(nb, sc, cs, cb, 1));
  }

  for (int s = 0; s < nstages; ++s) {
    const int slot = s % kStages;
    // every wave waited for its own copies of stage s before this barrier;
    // everyone also finished reading stage s - 1, whose slot is refilled here
    ring_barrier();
    // Waves w and w + 4 share a SIMD and its MFMA pipe, and issue ties go to
    // the older wave: left alone, waves 0-3 reached each stage's barrier about
    // 850 cycles (a quarter of a stage) before waves 4-7 (per-wave cycle
    // counters, prefill_contig48). The younger wave leads the first group and
    // the older one the second, which keeps the pair in step.
    if (NW == kWaves) {
      if (wave >= kWaves / 2) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    }
    if (s + kStages - 1 < nstages) issue_stage(c, ring, (s + kStages - 1) % kStages, s + kStages - 1, wave, a_blocks_per_wave(NW));

    // Software pipeline inside the stage: while a group's MFMAs run, the wave
    // reads the A fragments kAhead row blocks ahead and dequantises the next
    // group's weights (for the second group: the next stage's first group);
    // each row block's MFMAs sit in their own scheduling region so the
    // compiler keeps that interleave.
    const uint8_t* abase = ring + slot * kStageBytes;
    const auto lds_a = [&](int rb, int j) {
      return __builtin_bit_cast(f16x8,
                                *reinterpret_cast<const u32x4*>(abase + (rb * kStageGroups + j) * 1024 + 16 * lane));
    };
    f16x8 a[kRowBlocks];
#pragma unroll
    for (int rb = 0; rb < kAhead; ++rb) a[rb] = lds_a(rb, 0);
    {
      // the eight half fragments of the next group, one under each row block's
      // MFMAs (1.5 VALU per MFMA spread evenly)
      const u32x4 nb = nib1;
      const u32x2 sc = sc1;
      const u32x2 cs = neg24(sc);
      u32x2 hv[kRowBlocks];
#pragma unroll
      for (int rb = 0; rb < kRowBlocks; ++rb) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = mfma16(a[rb], w[cb], acc[rb][cb]);
        if (rb + kAhead < kRowBlocks) a[rb + kAhead] = lds_a(rb + kAhead, 0);
        else a[rb + kAhead - kRowBlocks] = lds_a(rb + kAhead - kRowBlocks, 1);
        hv[rb] = deqh(nb, sc, cs, rb >> 1, rb & 1);
      }
      // keep the dequantisation here, under these MFMAs: without a use in this
      // block the compiler sinks it past the wait below, into the next group
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        f16x8 v = join_halves(hv[2 * cb], hv[2 * cb + 1]);
        asm volatile("" : "+v"(v));
        w[cb] = v;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (NW == kWaves) {
      if (wave >= kWaves / 2) __builtin_amdgcn_s_setprio(0);
      else __builtin_amdgcn_s_setprio(1);
    }
    // own copies of stage s + 1 landed (stage s + 2 may still be in flight);
    // after the last stage the reads below see a stale slot whose values are unused
    wait_stage<NW>(min(nstages, s + kStages) - (s + 2));
    {
      // the next stage's weights: the first group is dequantised under this
      // group's MFMAs, the second is read now for the next stage's first group
      const int nslot = (s + 1) % kStages;
      const u32x4 nb = nib_of(nslot, 0);
      const u32x2 sc = sc_of(nslot, 0);
      nib1 = nib_of(nslot, 1);
      sc1 = sc_of(nslot, 1);
      // these nibbles were just read: the first row block's MFMAs cover the
      // read, and its two halves go under the last row block
      u32x2 cs, hv[kRowBlocks];
#pragma unroll
      for (int rb = 0; rb < kRowBlocks; ++rb) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = mfma16(a[rb], w[cb], acc[rb][cb]);
        if (rb + kAhead < kRowBlocks) a[rb + kAhead] = lds_a(rb + kAhead, 1);
        if (rb == 1) cs = neg24(sc);
        if (rb >= 1) hv[rb - 1] = deqh(nb, sc, cs, (rb - 1) >> 1, (rb - 1) & 1);
        if (rb == kRowBlocks - 1) hv[rb] = deqh(nb, sc, cs, rb >> 1, rb & 1);
      }
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) w[cb] = join_halves(hv[2 * cb], hv[2 * cb + 1]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  __builtin_amdgcn_s_setprio(0);
  // Epilogue: rows 16 rb + 4 (lane >> 4) + i of the tile; packed channels
  // 64 nb + 16 cb + (lane & 15).
  const int nb = nb0 + wave;
  const int pc0 = nb * kNBlock + (lane & 15);
  const int32_t* cexp = p.col_exp + (int64_t)e * p.N;
  int ce[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) ce[cb] = cexp[pc0 + 16 * cb];
  const int q = lane & 3;
  if (MODE == kDown && !p.out_bf16) {
    // fp32 rows of y: a 4 x 4 transpose inside each lane quad turns a lane's
    // four rows of one channel into one row of four consecutive channels, so
    // each lane stores 16 bytes per row block and column block (a quarter of
    // the store instructions of one float per row)
    float* ybase = static_cast<float*>(p.out) + nb * kNBlock + 4 * ((lane & 15) >> 2);
#pragma unroll
    for (int rb = 0; rb < kRowBlocks; ++rb) {
      int ids[4], re[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int prow = mb * kTileM + 16 * rb + 4 * (lane >> 4) + i;
        ids[i] = p.sorted[prow];
        re[i] = p.row_exp[prow];  // padding rows: any value, never stored
      }
      const int id = q == 0 ? ids[0] : q == 1 ? ids[1] : q == 2 ? ids[2] : ids[3];
      float* y = ybase + (int64_t)id * p.out_ld;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __builtin_amdgcn_ldexpf(acc[rb][cb][i], re[i] + ce[cb]);
        quad_transpose(v, lane);
        if ((unsigned)id < (unsigned)p.n_slots)
          *reinterpret_cast<floatx4*>(y + 16 * cb) = floatx4{v[0], v[1], v[2], v[3]};
      }
    }
    return;
  }
  if (MODE == kGateUp) {
    // h rows: the same quad transpose, four consecutive bf16 channels of one
    // row per lane in one 8-byte store
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    __bf16* hbase = static_cast<__bf16*>(p.out) + nb * 32 + 4 * ((lane & 15) >> 2);
#pragma unroll
    for (int rb = 0; rb < kRowBlocks; ++rb) {
      bool real[4];
      int re[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int prow = mb * kTileM + 16 * rb + 4 * (lane >> 4) + i;
        const int id = p.sorted[prow];
        real[i] = (unsigned)id < (unsigned)p.n_slots;
        re[i] = real[i] ? p.row_exp[id / p.topk] : 0;  // padding rows: never stored
      }
      const bool mine = q == 0 ? real[0] : q == 1 ? real[1] : q == 2 ? real[2] : real[3];
      const int prow = mb * kTileM + 16 * rb + 4 * (lane >> 4) + q;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        float hv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          hv[i] = silu_mul(__builtin_amdgcn_ldexpf(acc[rb][cb][i], re[i] + ce[cb]),
                           __builtin_amdgcn_ldexpf(acc[rb][cb + 2][i], re[i] + ce[cb + 2]));
        quad_transpose(hv, lane);
        if (mine)
          *reinterpret_cast<bf16x4*>(hbase + (int64_t)prow * p.out_ld + 16 * cb) =
              bf16x4{(__bf16)hv[0], (__bf16)hv[1], (__bf16)hv[2], (__bf16)hv[3]};
      }
    }
    return;
  }
  // down with bf16 output rows (the expert-grouped layouts)
#pragma unroll
  for (int rb = 0; rb < kRowBlocks; ++rb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int prow = mb * kTileM + 16 * rb + 4 * (lane >> 4) + i;
      const int id = p.sorted[prow];
      if ((unsigned)id >= (unsigned)p.n_slots) continue;
      const int re = p.row_exp[prow];
      __bf16* o = static_cast<__bf16*>(p.out) + (int64_t)id * p.out_ld + pc0;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) o[16 * cb] = (__bf16)__builtin_amdgcn_ldexpf(acc[rb][cb][i], re + ce[cb]);
    }
  }
}

// Sets up a wave's copy sources for the tile (row block mb, NW n-blocks from
// nb0) and runs it: the wave copies A row blocks a_blocks_per_wave(NW) * wave + t;
// padding rows read the block's first row (their results are discarded).
template <int MODE, int NW>
__device__ __forceinline__ void run_tile(const GemmParams& p, uint8_t* ring, int nstages, int mb, int nb0, int e,
                                         int wave, int lane) {
  const int G = p.K / kGroup;
  TileCtx c;
#pragma unroll
  for (int t = 0; t < a_blocks_per_wave(NW); ++t) {
    const int prow = mb * kTileM + 16 * (a_blocks_per_wave(NW) * wave + t) + (lane & 15);
    const int id = p.sorted[prow];
    const bool real = (unsigned)id < (unsigned)p.n_slots;
    int64_t src;
    if (MODE == kGateUp) {
      const int id0 = p.sorted[mb * kTileM];
      src = (real ? id : id0) / p.topk;
    } else {
      src = real ? prow : mb * kTileM;
    }
    c.a_src[t] = reinterpret_cast<const uint8_t*>(p.a16 + src * p.K) + 16 * (lane >> 4);
  }
  const int64_t unit = ((int64_t)e * (p.N / kNBlock) + nb0 + wave) * G;
  c.wq = p.wq + unit * kNibUnitBytes + 16 * lane;
  c.ws = reinterpret_cast<const uint8_t*>(p.ws16 + unit * kScaleUnitElems) + 4 * lane;
  tile_body<MODE, NW>(p, c, ring, nstages, mb, nb0, e, wave, lane);
}

// Persistent workgroups of 8 waves. Work items are full tiles (128 rows x 512
// channels, 8 waves) and half tiles (128 x 256, 4 waves; the other 4 take the
// same barriers and nothing else). A row block's channels are its full tiles
// plus, when N / 64 is an odd multiple of 4, one half tile at the end.
//
// Tile order is XCD-aware: workgroup b runs on XCD b % 8, and the items an XCD
// runs are those of the row blocks mb = xcd (mod 8), so a row block's A tile
// is shared through that XCD's L2. An XCD's full tiles run in rounds of one
// per workgroup; when the last round would leave at least half of the XCD's
// workgroups idle, its tiles run as twice as many half tiles instead, one per
// workgroup (a workgroup with half a tile runs it faster than a full one, and
// every CU keeps a share of the round).
template <int MODE>
__global__ __launch_bounds__(kThreads) void moe_gemm_tiled_kernel(GemmParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t ring[];
  const int lane = (int)threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int ntpp = min(*p.ntpp, p.capacity);
  const int n_mblocks = ntpp / kTileM;
  const int NB = p.N / kNBlock;
  const int F = NB / kTileNBlocks;                      // full tiles per row block
  const int Ht = (NB % kTileNBlocks) ? 1 : 0;           // trailing half tile per row block
  const int nstages = p.K / kGroup / kStageGroups;

  const int xcd = (int)blockIdx.x & 7;
  const int per_xcd = (int)gridDim.x >> 3;  // grid is a multiple of 8
  const int nmb = (n_mblocks + 7 - xcd) / 8;  // row blocks of this XCD: xcd + 8 j
  const int nfull = nmb * F;
  const int rounds = nfull / per_xcd, rem = nfull - rounds * per_xcd;
  const bool split = rem > 0 && 2 * rem <= per_xcd;
  const int n_full_items = split ? rounds * per_xcd : nfull;
  const int n_split_halves = split ? 2 * rem : 0;
  const int n_items = n_full_items + n_split_halves + nmb * Ht;
  for (int i = (int)blockIdx.x >> 3; i < n_items; i += per_xcd) {
    int j, nb0;
    bool half;
    if (i < n_full_items) {
      j = i / F;
      nb0 = (i - j * F) * kTileNBlocks;
      half = false;
    } else if (i < n_full_items + n_split_halves) {
      const int h = i - n_full_items, q = n_full_items + h / 2;
      j = q / F;
      nb0 = (q - j * F) * kTileNBlocks + (h & 1) * kHalfNBlocks;
      half = true;
    } else {
      j = i - n_full_items - n_split_halves;
      nb0 = F * kTileNBlocks;
      half = true;
    }
    const int mb = xcd + 8 * j;
    const int e = p.expert_ids[mb];
    if ((unsigned)e >= (unsigned)p.E) continue;  // uniform across the workgroup
    if (!half) {
      run_tile<MODE, kWaves>(p, ring, nstages, mb, nb0, e, wave, lane);
    } else if (wave < kWaves / 2) {
      run_tile<MODE, kWaves / 2>(p, ring, nstages, mb, nb0, e, wave, lane);
    } else {
      // the barriers of the half tile: one before its prologue, one per stage
      for (int s = 0; s <= nstages; ++s) ring_barrier();
    }
  }
}

// Rows of a bf16 matrix -> fp16 with a power-of-two factor per row: the row's
// largest magnitude is mapped into [2^14, 2^15), which keeps every element
// exact unless it is more than 2^31 below that largest one (then it rounds on
// the fp16 subnormal grid, an error below 2^-39 of the row's largest element).
// dst[r] = src[r] * 2^-row_exp[r]. One wave per row, four rows per workgroup,
// no workgroup barrier: the wave reads its row once into registers, takes the
// largest magnitude with a wave-wide reduction and writes the converted row.
// Rows that no GEMM reads are skipped: by token (a resident topk id) or by
// aligned row (real slot).
constexpr int kRowWaves = 4;
// REGS: 16-byte chunks per lane held in registers (rows up to 512 REGS
// elements; longer rows re-read the rest). Rows of up to 2048 elements take
// the 4-register build, whose smaller VGPR budget keeps twice as many waves
// (rows) in flight.

template <bool BY_TOKEN, int REGS>
__global__ __launch_bounds__(64 * kRowWaves) void rows_to_f16_kernel(
    const uint16_t* __restrict__ src, int32_t K, int32_t nrows, const int32_t* __restrict__ topk_ids, int32_t topk,
    int32_t E, const int32_t* __restrict__ sorted, const int32_t* __restrict__ ntpp, int32_t n_slots,
    uint16_t* __restrict__ dst, int32_t* __restrict__ row_exp) {
  const int lane = (int)threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int chunks = K / 8;
  const int live = BY_TOKEN ? nrows : min(*ntpp, nrows);
  for (int r = (int)blockIdx.x * kRowWaves + wave; r < live; r += (int)gridDim.x * kRowWaves) {
    bool need;
    if (BY_TOKEN) {
      // topk <= 64: lane j looks at the token's j-th routed id
      const int id = lane < topk ? topk_ids[(int64_t)r * topk + lane] : -1;
      need = __builtin_amdgcn_ballot_w64((unsigned)id < (unsigned)E) != 0;
    } else {
      need = (unsigned)sorted[r] < (unsigned)n_slots;
    }
    if (!need) continue;  // uniform across the wave
    const u32x4* row = reinterpret_cast<const u32x4*>(src + (int64_t)r * K);
    u32x4 v[REGS];
    // largest |x| as a bf16 bit pattern (sign cleared: integer order = magnitude order)
    uint32_t mx = 0;
#pragma unroll
    for (int i = 0; i < REGS; ++i) {
      const int ch = lane + 64 * i;
      v[i] = ch < chunks ? __builtin_nontemporal_load(row + ch) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < REGS; ++i)
#pragma unroll
      for (int d = 0; d < 4; ++d) mx = max(mx, max(v[i][d] & 0x7FFFu, (v[i][d] >> 16) & 0x7FFFu));
    for (int ch = lane + 64 * REGS; ch < chunks; ch += 64) {
      const u32x4 w = row[ch];
#pragma unroll
      for (int d = 0; d < 4; ++d) mx = max(mx, max(w[d] & 0x7FFFu, (w[d] >> 16) & 0x7FFFu));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off));
    // unbiased exponent of the largest element (subnormals count as -126)
    const int ef = (int)(mx >> 7);
    const int ex = mx == 0 ? 14 : (ef == 0 ? -126 : ef - 127);
    const int e = ex - 14;
    if (lane == 0) row_exp[r] = e;
    u32x4* out = reinterpret_cast<u32x4*>(dst + (int64_t)r * K);
    const auto convert = [&](u32x4 w) {
      u32x4 o;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float lo = __builtin_amdgcn_ldexpf(__uint_as_float(w[d] << 16), -e);
        const float hi = __builtin_amdgcn_ldexpf(__uint_as_float(w[d] & 0xFFFF0000u), -e);
        const f16x2 h = {(_Float16)lo, (_Float16)hi};
        o[d] = __builtin_bit_cast(uint32_t, h);
      }
      return o;
    };
#pragma unroll
    for (int i = 0; i < REGS; ++i) {
      const int ch = lane + 64 * i;
      if (ch < chunks) out[ch] = convert(v[i]);
    }
    for (int ch = lane + 64 * REGS; ch < chunks; ch += 64) out[ch] = convert(row[ch]);
  }
}

template <int MODE>
hipError_t launch_tiled_mode(const GemmParams& p, hipStream_t stream) {
  const int64_t mblocks_max = p.capacity / kTileM;
  const int NB = p.N / kNBlock;
  const int64_t tiles_max = mblocks_max * (NB / kTileNBlocks + (NB % kTileNBlocks ? 1 : 0));
  if (tiles_max == 0) return hipSuccess;
  static int blocks_per_cu = [] {
    // the LDS ring exceeds the default 64 KiB dynamic limit
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(moe_gemm_tiled_kernel<MODE>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, kStages * kStageBytes);
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, moe_gemm_tiled_kernel<MODE>, kThreads,
                                                     kStages * kStageBytes) != hipSuccess ||
        n < 1)
      n = 1;
    return n;
  }();
  // persistent grid, a multiple of 8 (one share per XCD)
  int64_t grid = (int64_t)device_cu_count() * blocks_per_cu;
  grid = std::min<int64_t>(grid, ((tiles_max + 7) / 8) * 8);
  grid = std::max<int64_t>(8, grid / 8 * 8);
  hipLaunchKernelGGL((moe_gemm_tiled_kernel<MODE>), dim3((int)grid), dim3(kThreads), kStages * kStageBytes, stream,
                     p);
  return hipGetLastError();
}

}  // namespace

bool tiled_gemm_supported(int32_t block_m, int32_t N, int32_t K) {
  return block_m == kTileM && (K / kGroup) % kStageGroups == 0 && N % (kNBlock * kHalfNBlocks) == 0;
}

size_t tiled_scratch_bytes(int64_t rows, int32_t K) {
  const size_t a = (size_t)rows * K * 2;
  return (a + 255) / 256 * 256 + (size_t)rows * 4;
}

namespace {
int32_t* row_exp_of(void* scratch, int64_t rows, int32_t K) {
  return reinterpret_cast<int32_t*>(static_cast<uint8_t*>(scratch) + ((size_t)rows * K * 2 + 255) / 256 * 256);
}
int rows_grid(int64_t rows) {
  return (int)std::max<int64_t>(1, std::min<int64_t>((rows + kRowWaves - 1) / kRowWaves, (int64_t)device_cu_count() * 16));
}
}  // namespace

hipError_t launch_rows_to_f16_tokens(const uint16_t* x, int32_t T, int32_t K, const int32_t* topk_ids, int32_t topk,
                                     int32_t E, void* scratch, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const auto kern = K <= 2048 ? rows_to_f16_kernel<true, 4> : rows_to_f16_kernel<true, 16>;
  hipLaunchKernelGGL(kern, dim3(rows_grid(T)), dim3(64 * kRowWaves), 0, stream, x, K, T, topk_ids, topk, E,
                     nullptr, nullptr, 0, static_cast<uint16_t*>(scratch), row_exp_of(scratch, T, K));
  return hipGetLastError();
}

hipError_t launch_rows_to_f16_aligned(const uint16_t* h, int32_t capacity, int32_t K, const int32_t* sorted,
                                      const int32_t* ntpp, int32_t n_slots, void* scratch, hipStream_t stream) {
  if (capacity == 0) return hipSuccess;
  const auto kern = K <= 2048 ? rows_to_f16_kernel<false, 4> : rows_to_f16_kernel<false, 16>;
  hipLaunchKernelGGL(kern, dim3(rows_grid(capacity)), dim3(64 * kRowWaves), 0, stream, h, K, capacity,
                     nullptr, 0, 0, sorted, ntpp, n_slots, static_cast<uint16_t*>(scratch),
                     row_exp_of(scratch, capacity, K));
  return hipGetLastError();
}

hipError_t launch_moe_gemm_tiled(GemmMode mode, const GemmParams& p, void* scratch, hipStream_t stream) {
  // scratch holds the fp16 A rows and row exponents written by the matching
  // launch_rows_to_f16_*: T token rows (gate_up) or capacity aligned rows (down)
  const int64_t rows = mode == kGateUp ? (int64_t)p.n_slots / p.topk : p.capacity;
  GemmParams q = p;
  q.a16 = static_cast<const uint16_t*>(scratch);
  q.row_exp = row_exp_of(scratch, rows, p.K);
  return mode == kGateUp ? launch_tiled_mode<kGateUp>(q, stream) : launch_tiled_mode<kDown>(q, stream);
}

}  // namespace w4a16
