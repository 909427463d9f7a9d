// Tiled W4A16 expert GEMM for many tokens per expert (block_m = 128).
//
// Once experts carry enough rows, the MFMA work rather than weight streaming
// sets the time (the pages' observation that tokens per expert, not total
// tokens, decides which schedule wins: Chord page "vLLM 및 Novita AI, Kimi
// K2.x용 더 빠른 INT4 MoE 커널 출시: Chord", section "핵심 기여"; and the
// small- vs large-batch pipelines of the Humming announcement, "Humming:
// vLLM과 Ant Group, 양자화 추론을 위한 범용 커널 라이브러리 오픈소스 공개",
// section "워크로드별 튜닝 및 JIT 컴파일"). The arithmetic is the same as the
// streaming kernel's: exact integer operands (q + 136) on
// v_mfma_f32_16x16x32_bf16 with a -136 * sum(x) correction in the C input,
// then one fp32 FMA per output per 32-wide group for the BF16 group scale.
//
// Tile: a 512-thread workgroup (8 waves, 2 x 4) computes 128 rows x 256
// channels (four 64-channel n-blocks) over the whole reduction; each wave owns
// 64 rows x one n-block. The K loop moves in stages of two groups (64 k):
//   A  128 rows x 64 k of bf16 (16 KiB), gathered through sorted_token_ids,
//   B  4 n-blocks x 2 groups of packed nibbles (8 KiB) and their scales (1 KiB),
// all copied global -> LDS by global_load_lds_dwordx4 / _dword (no VGPRs in
// flight), into a ring of kStages stages. LDS A is laid out fragment-major
// (row block, group, lane, 16 bytes), so every MFMA operand is one
// conflict-free ds_read_b128 per lane. The hardware's in-order vmcnt tracks
// the copies: a wave waits until its copies of the stage it is about to use
// have landed, then a workgroup barrier makes all waves' copies visible; the
// same barrier proves that the slot refilled next has been consumed.
//
// Tile order is XCD-aware: workgroup b runs on XCD b % 8, and the tiles an
// XCD runs are the n-tiles of the row blocks mb = xcd (mod 8), so the row
// block's A tile (gathered activations) is shared through that XCD's L2.
#include "internal.h"

#include <algorithm>

namespace w4a16 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int kThreads = 512;
constexpr int kWaves = 8;
constexpr int kStages = 3;           // LDS ring depth
constexpr int kTileM = 128;
constexpr int kTileNBlocks = 4;      // 4 x 64 = 256 channels
constexpr int kStageGroups = 2;      // 64 k per stage
constexpr int kABytes = kTileM * kStageGroups * kGroup * 2;                  // 16 KiB
constexpr int kBBytes = kTileNBlocks * kStageGroups * kNibUnitBytes;         // 8 KiB
constexpr int kSBytes = kTileNBlocks * kStageGroups * kScaleUnitElems * 2;   // 1 KiB
constexpr int kStageBytes = kABytes + kBBytes + kSBytes;
constexpr int kCopiesPerWaveStage = 4;  // 2 A blocks + 1 nibble unit + 1 scale unit
// Weights and scales are read once per tile: copied with the non-temporal
// policy (operand 2 = nt) so they do not evict the A tile shared through L2.
constexpr int kNonTemporal = 2;

constexpr uint32_t kCodeMask = 0x000F000Fu;
constexpr uint32_t kBf16_128 = 0x43004300u;
constexpr uint32_t kBf16_Minus136 = 0xC308C308u;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t magic) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(mask), "v"(magic));
  return r;
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

// Wait until at most N of this wave's vector-memory operations are pending.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier without a memory fence. __syncthreads() would make every
// wave drain all of its in-flight copies first (vmcnt(0)); here each wave has
// already waited for exactly the copies that must have landed, and the
// "memory" clobbers keep the compiler from moving LDS reads across the barrier.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

struct TileCtx {
  const uint8_t* a_src;  // this lane's A copy source (row start + 16-byte k offset)
  const uint8_t* wq;     // nibble units of this wave's copy n-block, group 0
  const uint8_t* ws;     // scale units of this wave's copy n-block, group 0
  int copy_rb;           // row block this wave copies
  int copy_nb, copy_j;   // nibble / scale unit this wave copies: n-block, group in stage
};

// Issue this wave's copies of stage `s` (groups 2s, 2s+1) into ring slot `slot`.
__device__ __forceinline__ void issue_stage(const TileCtx& c, uint8_t* ring, int slot, int s, int lane) {
  uint8_t* base = ring + slot * kStageBytes;
  const int g0 = s * kStageGroups;
#pragma unroll
  for (int j = 0; j < kStageGroups; ++j) {
    const uint8_t* src = c.a_src + (int64_t)(g0 + j) * (kGroup * 2);
    __builtin_amdgcn_global_load_lds(src, LDS_PTR(base + (c.copy_rb * kStageGroups + j) * 1024), 16, 0, 0);
  }
  {
    const uint8_t* src = c.wq + (int64_t)(g0 + c.copy_j) * kNibUnitBytes + 16 * lane;
    __builtin_amdgcn_global_load_lds(src, LDS_PTR(base + kABytes + (c.copy_nb * kStageGroups + c.copy_j) * 1024), 16,
                                     0, kNonTemporal);
  }
  // 128 bytes of scales: a dword copy lands at LDS base + 4 * lane, so only
  // lanes 0..31 take part (one instruction per wave either way, which keeps
  // every wave's count of pending copies the same)
  if (lane < 32) {
    const uint8_t* src = c.ws + (int64_t)(g0 + c.copy_j) * (kScaleUnitElems * 2) + 4 * lane;
    __builtin_amdgcn_global_load_lds(
        src, LDS_PTR(base + kABytes + kBBytes + (c.copy_nb * kStageGroups + c.copy_j) * 128), 4, 0, kNonTemporal);
  }
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void moe_gemm_tiled_kernel(GemmParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t ring[];
  const int lane = (int)threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int wm = wave >> 2;  // 64-row half of the tile
  const int wn = wave & 3;   // n-block of the tile
  const int ntpp = min(*p.ntpp, p.capacity);
  const int n_mblocks = ntpp / kTileM;
  const int NB = p.N / kNBlock;
  const int NT = NB / kTileNBlocks;  // n-tiles per row block
  const int G = p.K / kGroup;
  const int nstages = G / kStageGroups;
  uint32_t magic = kBf16_128;
  asm volatile("v_mov_b32 %0, %1" : "=v"(magic) : "s"(magic));
  const bf16x8 minus136 = as_bf16x8(u32x4{kBf16_Minus136, kBf16_Minus136, kBf16_Minus136, kBf16_Minus136});
  const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};

  // XCD-aware order: local tile index q of XCD x covers row block x + 8 (q / NT).
  const int xcd = (int)blockIdx.x & 7;
  const int per_xcd = (int)gridDim.x >> 3;  // grid is a multiple of 8
  const int q_total = ((n_mblocks + 7 - xcd) / 8) * NT;
  for (int q = (int)blockIdx.x >> 3; q < q_total; q += per_xcd) {
    const int mb = xcd + 8 * (q / NT);
    const int nt = q - (q / NT) * NT;
    const int e = p.expert_ids[mb];
    if ((unsigned)e >= (unsigned)p.E) continue;  // uniform across the workgroup

    // this wave copies A row block `wave` (rows 16 wave .. 16 wave + 15)
    TileCtx c;
    c.copy_rb = wave;
    c.copy_nb = wave >> 1;
    c.copy_j = wave & 1;
    {
      const int prow = mb * kTileM + 16 * wave + (lane & 15);
      const int id = p.sorted[prow];
      const bool real = (unsigned)id < (unsigned)p.n_slots;
      int64_t src;
      if (MODE == kGateUp) {
        const int id0 = p.sorted[mb * kTileM];
        src = (real ? id : id0) / p.topk;
      } else {
        src = real ? prow : mb * kTileM;
      }
      c.a_src = reinterpret_cast<const uint8_t*>(p.a + src * p.K) + 16 * (lane >> 4);
    }
    const int64_t unit_copy = ((int64_t)e * NB + nt * kTileNBlocks + c.copy_nb) * G;
    c.wq = p.wq + unit_copy * kNibUnitBytes;
    c.ws = reinterpret_cast<const uint8_t*>(p.ws + unit_copy * kScaleUnitElems);

    floatx4 acc[4][4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = zero4;

    // the previous tile's reads of every slot are done before it is refilled
    ring_barrier();
#pragma unroll
    for (int s = 0; s < kStages - 1; ++s)
      if (s < nstages) issue_stage(c, ring, s, s, lane);

    for (int s = 0; s < nstages; ++s) {
      // own copies of stage s landed (later stages may still be in flight) ...
      if (s + kStages - 2 < nstages) wait_vmcnt<(kStages - 2) * kCopiesPerWaveStage>();
      else wait_vmcnt<0>();
      // ... and everyone's; everyone also finished reading stage s - 1
      ring_barrier();
      if (s + kStages - 1 < nstages) issue_stage(c, ring, (s + kStages - 1) % kStages, s + kStages - 1, lane);

      const uint8_t* base = ring + (s % kStages) * kStageBytes;
#pragma unroll
      for (int j = 0; j < kStageGroups; ++j) {
        const u32x4 nib = *reinterpret_cast<const u32x4*>(base + kABytes + (wn * kStageGroups + j) * 1024 + 16 * lane);
        const u32x2 sc = *reinterpret_cast<const u32x2*>(base + kABytes + kBBytes + (wn * kStageGroups + j) * 128 +
                                                         8 * (lane & 15));
        const float scale[4] = {__uint_as_float(sc.x << 16), __uint_as_float(sc.x & 0xFFFF0000u),
                                __uint_as_float(sc.y << 16), __uint_as_float(sc.y & 0xFFFF0000u)};
        bf16x8 w[4];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) w[cb] = codes_to_bf16(nib[cb], magic);
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const bf16x8 a = as_bf16x8(
              *reinterpret_cast<const u32x4*>(base + ((4 * wm + rb) * kStageGroups + j) * 1024 + 16 * lane));
          const floatx4 corr = mfma16(a, minus136, zero4);
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) acc[rb][cb] += scale[cb] * mfma16(a, w[cb], corr);
        }
      }
    }

    // Epilogue: wave rows 64 wm + 16 rb + 4 (lane >> 4) + i, n-block nt * 4 + wn.
    const int nb = nt * kTileNBlocks + wn;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int prow = mb * kTileM + 64 * wm + 16 * rb + 4 * (lane >> 4) + i;
        const int id = p.sorted[prow];
        if ((unsigned)id >= (unsigned)p.n_slots) continue;
        if (MODE == kGateUp) {
          __bf16* h = static_cast<__bf16*>(p.out) + (int64_t)prow * p.out_ld + nb * 32 + (lane & 15);
          h[0] = (__bf16)silu_mul(acc[rb][0][i], acc[rb][2][i]);
          h[16] = (__bf16)silu_mul(acc[rb][1][i], acc[rb][3][i]);
        } else {
          float* y = static_cast<float*>(p.out) + (int64_t)id * p.out_ld + nb * kNBlock + (lane & 15);
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) y[16 * cb] = acc[rb][cb][i];
        }
      }
    }
  }
}

template <int MODE>
hipError_t launch_tiled_mode(const GemmParams& p, hipStream_t stream) {
  const int64_t mblocks_max = p.capacity / kTileM;
  const int64_t tiles_max = mblocks_max * (p.N / (kNBlock * kTileNBlocks));
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

bool tiled_gemm_supported(int32_t block_m, const GemmParams& p) {
  return block_m == kTileM && (p.K / kGroup) % kStageGroups == 0 && p.N % (kNBlock * kTileNBlocks) == 0;
}

hipError_t launch_moe_gemm_tiled(GemmMode mode, const GemmParams& p, hipStream_t stream) {
  return mode == kGateUp ? launch_tiled_mode<kGateUp>(p, stream) : launch_tiled_mode<kDown>(p, stream);
}

}  // namespace w4a16
