// Expert-grouped W4A16 GEMMs and the top-k combine on gfx950.
//
// The computation is the indexed W4A16 MoE operator of the Chord page ("vLLM 및
// Novita AI, Kimi K2.x용 더 빠른 INT4 MoE 커널 출시: Chord", TL;DR and "핵심
// 기여"): rows are gathered through the alignment buffers, multiplied by the
// expert's INT4 weights times their BF16 group-32 scales with fp32
// accumulation, gate_up is followed by SiLU-and-mul, then the down projection,
// then the top-k weighted sum (moe_fused_mul_sum on the Humming PR page,
// "[vllm] vLLM에 고성능 JIT 양자화 커널 'Humming' 도입하기", "왜 이게 좋은가" 3).
//
// Exact weights on bf16 MFMA. A weight is q * s with q in [-8, 7] and s a
// bf16 scale; q * s needs up to 11 significant bits, more than bf16 holds, so
// the scale cannot be folded into the bf16 operand. Instead the MFMA sees the
// exact integer (as the bf16 value q + 136, built by OR-ing the stored code
// into the mantissa of 128.0), its C input carries -136 * sum(x) of the same
// 32-wide group (one extra MFMA against a constant -136 operand, shared by the
// four column blocks of a row block), so each v_mfma_f32_16x16x32_bf16 yields
// the exact group partial sum(x * q) in fp32; the fp32 group scale is then
// applied with one FMA per output per group.
//
// Work decomposition. A work unit is (block_m-row block mb, 64-channel n-block
// nb), computed by one wave over the whole reduction: the unit's packed weights
// are one contiguous stream (K/32 KiB of nibbles plus K/16 scales bytes per
// 64 channels). Waves are persistent: a grid sized to the resident wave count
// strides over units, and the number of live row blocks is read from
// num_tokens_post_padded on the device, so the over-allocated alignment buffer
// costs nothing (Chord page, "런타임 고려사항").
#include "internal.h"

#include <algorithm>
#include <atomic>

namespace w4a16 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr uint32_t kCodeMask = 0x000F000Fu;
constexpr uint32_t kBf16_128 = 0x43004300u;    // two bf16 128.0
constexpr uint32_t kBf16_Minus136 = 0xC308C308u;  // two bf16 -136.0

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Eight stored codes (q + 8) -> eight exact bf16 values q + 136, k-order.
__device__ __forceinline__ bf16x8 codes_to_bf16(uint32_t w) {
  u32x4 r;
  r.x = (w & kCodeMask) | kBf16_128;
  r.y = ((w >> 4) & kCodeMask) | kBf16_128;
  r.z = ((w >> 8) & kCodeMask) | kBf16_128;
  r.w = ((w >> 12) & kCodeMask) | kBf16_128;
  return as_bf16x8(r);
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

__device__ __forceinline__ floatx4 mfma16(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// RB row blocks of 16 (block_m = 16 RB); U groups of 32 loaded per batch.
template <int MODE, int RB, int U>
__global__ __launch_bounds__(256) void moe_gemm_stream_kernel(GemmParams p) {
  constexpr int BM = 16 * RB;
  const int lane = (int)threadIdx.x & 63;
  const int wave = (int)blockIdx.x * 4 + ((int)threadIdx.x >> 6);
  const int nwaves = (int)gridDim.x * 4;
  const int ntpp = min(*p.ntpp, p.capacity);
  const int n_mblocks = ntpp / BM;
  const int NB = p.N / kNBlock;
  const int G = p.K / kGroup;
  const int units = n_mblocks * NB;
  const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
  const bf16x8 minus136 = as_bf16x8(u32x4{kBf16_Minus136, kBf16_Minus136, kBf16_Minus136, kBf16_Minus136});

  for (int u = wave; u < units; u += nwaves) {
    const int mb = u / NB;
    const int nb = u - mb * NB;
    const int e = p.expert_ids[mb];
    if ((unsigned)e >= (unsigned)p.E) continue;

    const u32x4* arow[RB];
    bool real[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int prow = mb * BM + rb * 16 + (lane & 15);
      const int id = p.sorted[prow];
      real[rb] = (unsigned)id < (unsigned)p.n_slots;
      const int64_t src = (MODE == kGateUp) ? (real[rb] ? id / p.topk : 0) : prow;
      arow[rb] = reinterpret_cast<const u32x4*>(p.a + src * p.K + 8 * (lane >> 4));
    }
    const int64_t unit0 = ((int64_t)e * NB + nb) * G;
    const u32x4* wq = reinterpret_cast<const u32x4*>(p.wq + unit0 * kNibUnitBytes) + lane;
    const u32x2* ws = reinterpret_cast<const u32x2*>(p.ws + unit0 * kScaleUnitElems) + (lane & 15);

    floatx4 acc[RB][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[rb][c] = zero4;

    for (int g0 = 0; g0 < G; g0 += U) {
      u32x4 nib[U];
      u32x2 sc[U];
      u32x4 av[RB][U];
#pragma unroll
      for (int uu = 0; uu < U; ++uu) {
        const int g = g0 + uu;
        const bool ok = g < G;
        nib[uu] = ok ? wq[(int64_t)g * 64] : u32x4{0u, 0u, 0u, 0u};
        sc[uu] = ok ? ws[(int64_t)g * 16] : u32x2{0u, 0u};
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) av[rb][uu] = (ok && real[rb]) ? arow[rb][g * 4] : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int uu = 0; uu < U; ++uu) {
        const float s[4] = {bf16_lo(sc[uu].x), bf16_hi(sc[uu].x), bf16_lo(sc[uu].y), bf16_hi(sc[uu].y)};
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const bf16x8 a = as_bf16x8(av[rb][uu]);
          const floatx4 corr = mfma16(a, minus136, zero4);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const floatx4 part = mfma16(a, codes_to_bf16(nib[uu][c]), corr);
            acc[rb][c] += s[c] * part;
          }
        }
      }
    }

    // Epilogue. Output element i of a 16x16 tile sits at row 4 (lane >> 4) + i,
    // column lane & 15.
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int prow = mb * BM + rb * 16 + 4 * (lane >> 4) + i;
        const int id = p.sorted[prow];
        if ((unsigned)id >= (unsigned)p.n_slots) continue;
        if (MODE == kGateUp) {
          __bf16* h = static_cast<__bf16*>(p.out) + (int64_t)prow * p.out_ld + nb * 32 + (lane & 15);
          h[0] = (__bf16)silu_mul(acc[rb][0][i], acc[rb][2][i]);
          h[16] = (__bf16)silu_mul(acc[rb][1][i], acc[rb][3][i]);
        } else {
          float* y = static_cast<float*>(p.out) + (int64_t)id * p.out_ld + nb * kNBlock + (lane & 15);
#pragma unroll
          for (int c = 0; c < 4; ++c) y[16 * c] = acc[rb][c][i];
        }
      }
    }
  }
}

// out[t, n] = bf16(sum_j resident(t, j) * w[t, j] * y[t*topk + j, n]), fp32 in j order.
__global__ __launch_bounds__(256) void combine_kernel(const int32_t* __restrict__ ids, const float* __restrict__ w,
                                                      const float* __restrict__ y, uint16_t* __restrict__ out, int topk,
                                                      int H, int E) {
  const int chunks = (H / 4 + 255) / 256;
  const int t = (int)blockIdx.x / chunks;
  const int n0 = (((int)blockIdx.x - t * chunks) * 256 + (int)threadIdx.x) * 4;
  if (n0 >= H) return;
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < topk; ++j) {
    const int slot = t * topk + j;
    const int e = ids[slot];
    if ((unsigned)e >= (unsigned)E) continue;
    const float wt = w[slot];
    const floatx4 v = *reinterpret_cast<const floatx4*>(y + (int64_t)slot * H + n0);
    acc += wt * v;
  }
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 r;
  r[0] = (__bf16)acc[0];
  r[1] = (__bf16)acc[1];
  r[2] = (__bf16)acc[2];
  r[3] = (__bf16)acc[3];
  *reinterpret_cast<bf16x4*>(out + (int64_t)t * H + n0) = r;
}

std::atomic<int> g_cu_count[64];

template <int MODE, int RB, int U>
hipError_t launch_stream(const GemmParams& p, hipStream_t stream) {
  constexpr int BM = 16 * RB;
  const int64_t units_max = (int64_t)(p.capacity / BM) * (p.N / kNBlock);
  if (units_max == 0) return hipSuccess;
  static int blocks_per_cu = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, moe_gemm_stream_kernel<MODE, RB, U>, 256, 0) != hipSuccess ||
        n < 1)
      n = 1;
    return n;
  }();
  const int64_t resident_waves = (int64_t)device_cu_count() * blocks_per_cu * 4;
  const int64_t waves = std::min(units_max, resident_waves);
  const int grid = (int)((waves + 3) / 4);
  hipLaunchKernelGGL((moe_gemm_stream_kernel<MODE, RB, U>), dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_mode(int block_m, const GemmParams& p, hipStream_t stream) {
  switch (block_m) {
    case 16: return launch_stream<MODE, 1, 8>(p, stream);
    case 32: return launch_stream<MODE, 2, 4>(p, stream);
    case 64: return launch_stream<MODE, 4, 2>(p, stream);
    case 128: return launch_stream<MODE, 8, 1>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = g_cu_count[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
    g_cu_count[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

hipError_t launch_moe_gemm(GemmMode mode, int32_t block_m, const GemmParams& p, hipStream_t stream) {
  return mode == kGateUp ? launch_mode<kGateUp>(block_m, p, stream) : launch_mode<kDown>(block_m, p, stream);
}

hipError_t launch_combine(const int32_t* ids, const float* w, const float* y, uint16_t* out, int32_t T, int32_t topk,
                          int32_t H, int32_t E, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int chunks = (H / 4 + 255) / 256;
  hipLaunchKernelGGL(combine_kernel, dim3(T * chunks), dim3(256), 0, stream, ids, w, y, out, topk, H, E);
  return hipGetLastError();
}

}  // namespace w4a16
