// One-time weight repack: canonical group-32 INT4 nibbles and BF16 scales ->
// the MFMA-ready layout described in internal.h (the load-time "validate,
// pad, repack into the kernel's layout" step of the Humming announcement,
// "Humming: vLLM과 Ant Group, 양자화 추론을 위한 범용 커널 라이브러리 오픈소스 공개",
// section "워크로드별 튜닝 및 JIT 컴파일"; transposed scales and kernel-specific
// packing as in the Chord page, section "그룹 SM90 커널 기법").
//
// Canonical input per expert: q [N, K/2] bytes (element k in the low nibble of
// byte k/2 when k is even; two's complement), s [N, K/32] bf16.
// Each thread writes one packed dword (8 codes) or one packed scale; reads are
// 4-byte gathers from the canonical rows. This runs once at load, so it is
// written for clarity rather than bandwidth.
#include "internal.h"

namespace w4a16 {
namespace {

// Canonical row holding packed column `col` of n-block `nb` (column block c, lane column j).
__device__ __forceinline__ int source_row(int nb, int c, int j, int interleave_I) {
  if (interleave_I > 0) {
    const int ch = 32 * nb + 16 * (c & 1) + j;
    return (c < 2) ? ch : interleave_I + ch;
  }
  return nb * kNBlock + 16 * c + j;
}

__global__ void repack_nibbles_kernel(const uint8_t* __restrict__ q, uint32_t* __restrict__ out, int N, int K,
                                      int interleave_I, int64_t total_dwords) {
  const int G = K / kGroup;
  const int NB = N / kNBlock;
  for (int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; d < total_dwords;
       d += (int64_t)gridDim.x * blockDim.x) {
    const int64_t unit = d >> 8;          // 256 dwords per 1024-byte unit
    const int within = (int)(d & 255);
    const int lane = within >> 2, c = within & 3;
    const int g = (int)(unit % G);
    const int64_t t = unit / G;
    const int nb = (int)(t % NB);
    const int64_t e = t / NB;
    const int row = source_row(nb, c, lane & 15, interleave_I);
    const int k0 = kGroup * g + 8 * (lane >> 4);
    const uint32_t v = *reinterpret_cast<const uint32_t*>(q + ((e * N + row) * (int64_t)(K / 2)) + k0 / 2);
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t byte = (v >> (8 * j)) & 0xFFu;
      const uint32_t even = (byte & 0xFu) ^ 0x8u;  // int4 value + 8
      const uint32_t odd = (byte >> 4) ^ 0x8u;
      w |= (even << (4 * j)) | (odd << (16 + 4 * j));
    }
    out[d] = w;
  }
}

__global__ void repack_scales_kernel(const uint16_t* __restrict__ s, uint16_t* __restrict__ out, int N, int K,
                                     int interleave_I, int64_t total) {
  const int G = K / kGroup;
  const int NB = N / kNBlock;
  for (int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; d < total; d += (int64_t)gridDim.x * blockDim.x) {
    const int64_t unit = d / kScaleUnitElems;
    const int w = (int)(d % kScaleUnitElems);
    const int j = w >> 2, c = w & 3;
    const int g = (int)(unit % G);
    const int64_t t = unit / G;
    const int nb = (int)(t % NB);
    const int64_t e = t / NB;
    const int row = source_row(nb, c, j, interleave_I);
    out[d] = s[(e * N + row) * (int64_t)G + g];
  }
}

// Normalised fp16 scales and channel exponents: one thread per (expert, packed
// channel). E_n is the unbiased exponent of the channel's largest |s| minus 4
// (a zero channel counts as exponent 0, bf16 subnormals as 2^-126), and every
// group scale is stored as fp16(s * 2^-E_n), a value in (-32, 32): the largest
// lands in [16, 32), so -24 * s, which the tiled GEMM also uses (at most 10
// significant bits, magnitude below 768), stays exact wherever s is.
__global__ void repack_f16_scales_kernel(const uint16_t* __restrict__ s, uint16_t* __restrict__ out,
                                         int32_t* __restrict__ col_exp, int N, int K, int interleave_I,
                                         int64_t total) {
  const int G = K / kGroup;
  const int NB = N / kNBlock;
  for (int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; d < total; d += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = d / N;
    const int pc = (int)(d % N);
    const int nb = pc / kNBlock, c = (pc % kNBlock) / 16, j = pc % 16;
    const uint16_t* src = s + (e * N + source_row(nb, c, j, interleave_I)) * (int64_t)G;
    uint32_t mx = 0;
    for (int g = 0; g < G; ++g) mx = max(mx, (uint32_t)(src[g] & 0x7FFFu));
    const int ef = (int)(mx >> 7);
    const int ex = (mx == 0 ? 0 : (ef == 0 ? -126 : ef - 127)) - 4;
    col_exp[d] = ex;
    for (int g = 0; g < G; ++g) {
      const float v = __builtin_amdgcn_ldexpf(__uint_as_float((uint32_t)src[g] << 16), -ex);
      out[((e * NB + nb) * G + g) * kScaleUnitElems + 4 * j + c] = __builtin_bit_cast(uint16_t, (_Float16)v);
    }
  }
}

}  // namespace

hipError_t launch_repack(const uint8_t* q, const uint16_t* s, int32_t E, int32_t N, int32_t K, int32_t interleave_I,
                         uint8_t* packed, hipStream_t stream) {
  const PackedRegions r = packed_regions(E, N, K);
  uint8_t* out_q = packed + r.nib;
  uint16_t* out_s = reinterpret_cast<uint16_t*>(packed + r.s_bf16);
  const int64_t dwords = (int64_t)E * N * K / 8;
  const int64_t scales = (int64_t)E * N * (K / kGroup);
  const int grid_q = (int)std::min<int64_t>(65536, (dwords + 255) / 256);
  const int grid_s = (int)std::min<int64_t>(65536, (scales + 255) / 256);
  hipLaunchKernelGGL(repack_nibbles_kernel, dim3(grid_q), dim3(256), 0, stream, q,
                     reinterpret_cast<uint32_t*>(out_q), N, K, interleave_I, dwords);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(repack_scales_kernel, dim3(grid_s), dim3(256), 0, stream, s, out_s, N, K, interleave_I, scales);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t cols = (int64_t)E * N;
  const int grid_c = (int)std::min<int64_t>(65536, (cols + 255) / 256);
  hipLaunchKernelGGL(repack_f16_scales_kernel, dim3(grid_c), dim3(256), 0, stream, s,
                     reinterpret_cast<uint16_t*>(packed + r.s_f16), reinterpret_cast<int32_t*>(packed + r.cexp), N, K,
                     interleave_I, cols);
  return hipGetLastError();
}

}  // namespace w4a16
