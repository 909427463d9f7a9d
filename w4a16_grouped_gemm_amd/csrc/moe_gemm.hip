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
// are one contiguous stream (K/32 KiB of nibbles plus K/16 scale bytes per
// 64 channels). Waves are persistent: the grid is sized to the resident wave
// count, the number of live row blocks is read from num_tokens_post_padded on
// the device (so the over-allocated alignment buffer costs nothing; Chord page,
// "런타임 고려사항"), and the live units are split evenly over the waves.
//
// Latency hiding. Each wave keeps two batches of U groups in registers and
// issues the loads of one while it computes the other; sched_barrier pins
// that order against the scheduler, and the batch offset is made opaque so the
// look-ahead load is not re-materialized next to its use.
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
constexpr uint32_t kBf16_128 = 0x43004300u;       // two bf16 128.0
constexpr uint32_t kBf16_Minus136 = 0xC308C308u;  // two bf16 -136.0

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// (a & mask) | magic, one v_and_or_b32 (VOP3 takes at most one scalar operand:
// the mask comes from an SGPR, the magic from a VGPR). Plain C, not inline
// asm: the result feeds an MFMA operand directly, and an MFMA that reads a
// VGPR needs two wait states after the VALU write of it, which the compiler
// counts only for instructions it can see (inline asm written there left one).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t magic) {
  return (a & mask) | magic;
}

// Eight stored codes (q + 8) -> eight exact bf16 values q + 136, in k order.
__device__ __forceinline__ bf16x8 codes_to_bf16(uint32_t w, uint32_t magic) {
  u32x4 r;
  r.x = and_or(w, kCodeMask, magic);
  r.y = and_or(w >> 4, kCodeMask, magic);
  r.z = and_or(w >> 8, kCodeMask, magic);
  r.w = and_or(w >> 12, kCodeMask, magic);
  return as_bf16x8(r);
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

__device__ __forceinline__ floatx4 mfma16(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Registers of U consecutive 32-wide groups for one wave: its 16-byte nibble
// chunk and 8-byte scale chunk per group, and its A fragment per row block.
template <int RB, int U>
struct Batch {
  u32x4 nib[U];
  u32x2 sc[U];
  u32x4 a[RB][U];
};

// Per-wave stream pointers: wave-uniform bases (SGPRs) plus fixed per-lane offsets.
template <int RB>
struct Streams {
  const uint8_t* wq;  // nibble units of this (expert, n-block), uniform
  const uint8_t* ws;  // scale units, uniform
  uint32_t q_lane;    // 16 * lane
  uint32_t s_lane;    // 8 * (lane & 15)
  const uint8_t* a[RB];  // this lane's A row (+ its 8-element k offset)
};

// Loads groups [g0, g0 + U). g0 is made opaque to the optimizer so that a
// prefetch issued one batch early is not re-materialized at its use.
template <int RB, int U>
__device__ __forceinline__ void load_batch(Batch<RB, U>& b, const Streams<RB>& st, int g0) {
  asm volatile("" : "+s"(g0));
  const uint8_t* q = st.wq + (int64_t)g0 * kNibUnitBytes + st.q_lane;
  const uint8_t* sc = st.ws + (int64_t)g0 * (kScaleUnitElems * 2) + st.s_lane;
#pragma unroll
  for (int uu = 0; uu < U; ++uu) {
    // weights are read once: non-temporal loads keep them out of the way of reused data
    b.nib[uu] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(q + uu * kNibUnitBytes));
    b.sc[uu] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(sc + uu * (kScaleUnitElems * 2)));
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      b.a[rb][uu] = *reinterpret_cast<const u32x4*>(st.a[rb] + (int64_t)(g0 + uu) * (kGroup * 2));
  }
}

// acc[rb][c] += s_c * (sum over the group of a * q): one correction MFMA per
// row block, four code MFMAs, four FMAs per output.
template <int RB, int U>
__device__ __forceinline__ void compute_batch(const Batch<RB, U>& b, floatx4 (&acc)[RB][4], uint32_t magic,
                                              bf16x8 minus136) {
  const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int uu = 0; uu < U; ++uu) {
    const float s[4] = {bf16_lo(b.sc[uu].x), bf16_hi(b.sc[uu].x), bf16_lo(b.sc[uu].y), bf16_hi(b.sc[uu].y)};
    bf16x8 w[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) w[c] = codes_to_bf16(b.nib[uu][c], magic);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const bf16x8 a = as_bf16x8(b.a[rb][uu]);
      const floatx4 corr = mfma16(a, minus136, zero4);
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[rb][c] += s[c] * mfma16(a, w[c], corr);
    }
  }
}

// RB row blocks of 16 (block_m = 16 RB); batches of U groups; NS batches in
// registers: while one is computed the loads of the next NS - 1 are in flight.
template <int MODE, int RB, int U, int NS>
__global__ __launch_bounds__(256) void moe_gemm_stream_kernel(GemmParams p) {
  constexpr int BM = 16 * RB;
  const int lane = (int)threadIdx.x & 63;
  const int wave = (int)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int nwaves = (int)gridDim.x * 4;
  const int ntpp = min(*p.ntpp, p.capacity);
  const int n_mblocks = ntpp / BM;
  const int NB = p.N / kNBlock;
  const int G = p.K / kGroup;
  const int nbatch = G / U;  // pipelined full batches; groups [nbatch * U, G) are the tail
  const int units = n_mblocks * NB;
  uint32_t magic = kBf16_128;
  asm volatile("v_mov_b32 %0, %1" : "=v"(magic) : "s"(magic));
  const bf16x8 minus136 = as_bf16x8(u32x4{kBf16_Minus136, kBf16_Minus136, kBf16_Minus136, kBf16_Minus136});

  // Balanced static split: every active wave takes the same number of
  // consecutive units (consecutive n-blocks of one row block share A rows).
  const int per_wave = (units + nwaves - 1) / nwaves;
  const int u_begin = wave * per_wave;
  const int u_end = min(units, u_begin + per_wave);
  for (int u = u_begin; u < u_end; ++u) {
    const int mb = u / NB;
    const int nb = u - mb * NB;
    const int e = p.expert_ids[mb];
    if ((unsigned)e >= (unsigned)p.E) continue;

    // A rows. A padding row reads the block's first row (always a real one, so
    // all padding lanes share one address); its results land only in that
    // row of the tile, which is never stored.
    Streams<RB> st;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int prow = mb * BM + rb * 16 + (lane & 15);
      const int id = p.sorted[prow];
      const bool real = (unsigned)id < (unsigned)p.n_slots;
      int64_t src;
      if (MODE == kGateUp) {
        const int id0 = p.sorted[mb * BM];
        src = (real ? id : id0) / p.topk;
      } else {
        src = real ? prow : mb * BM;
      }
      st.a[rb] = reinterpret_cast<const uint8_t*>(p.a + src * p.K + 8 * (lane >> 4));
    }
    const int64_t unit0 = ((int64_t)e * NB + nb) * G;
    st.wq = p.wq + unit0 * kNibUnitBytes;
    st.ws = reinterpret_cast<const uint8_t*>(p.ws + unit0 * kScaleUnitElems);
    st.q_lane = 16u * (uint32_t)lane;
    st.s_lane = 8u * (uint32_t)(lane & 15);

    floatx4 acc[RB][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[rb][c] = floatx4{0.f, 0.f, 0.f, 0.f};

    if (nbatch > 0) {
      Batch<RB, U> b[NS];
#pragma unroll
      for (int j = 0; j < NS - 1; ++j) load_batch(b[j], st, min(j, nbatch - 1) * U);
      for (int i = 0; i < nbatch; i += NS) {
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          // look-ahead NS - 1 batches; past the end it re-reads the last batch
          load_batch(b[(j + NS - 1) % NS], st, min(i + j + NS - 1, nbatch - 1) * U);
          __builtin_amdgcn_sched_barrier(0);  // keep the look-ahead loads ahead of the math
          if (i + j < nbatch) compute_batch(b[j], acc, magic, minus136);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    for (int g = nbatch * U; g < G; ++g) {
      Batch<RB, 1> t;
      load_batch(t, st, g);
      compute_batch(t, acc, magic, minus136);
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
  }
}

// out[t, n] = bf16(sum_j resident(t, j) * w[t, j] * y[t*topk + j, n]), fp32 in j order.
// One 256-thread block per (token, `cols` columns); each thread owns 8
// consecutive columns at a time (two 16-byte reads per resident slot, one
// 16-byte store). Tokens with no resident slot only write zeros.
__global__ __launch_bounds__(256) void combine_kernel(const int32_t* __restrict__ ids, const float* __restrict__ w,
                                                      const float* __restrict__ y, uint16_t* __restrict__ out, int topk,
                                                      int H, int E, int cols) {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  const int chunks = (H + cols - 1) / cols;
  const int t = (int)blockIdx.x / chunks;
  const int c0 = ((int)blockIdx.x - t * chunks) * cols;
  const int c1 = min(H, c0 + cols);
  // the token's resident slots as a bit mask (topk <= 32): lane j of every
  // wave reads routed id j once, so a row without a resident slot is stores only
  const int lane = (int)threadIdx.x & 63;
  const int my_id = lane < topk ? ids[(int64_t)t * topk + lane] : -1;
  const uint64_t resident = __ballot((unsigned)my_id < (unsigned)E);
  for (int n0 = c0 + 8 * (int)threadIdx.x; n0 < c1; n0 += 8 * 256) {
    floatx4 lo = {0.f, 0.f, 0.f, 0.f}, hi = {0.f, 0.f, 0.f, 0.f};
    for (uint64_t m = resident; m; m &= m - 1) {  // resident slots in j order
      const int slot = t * topk + __builtin_ctzll(m);
      const float wt = w[slot];
      const floatx4* src = reinterpret_cast<const floatx4*>(y + (int64_t)slot * H + n0);
      lo += wt * src[0];
      hi += wt * src[1];
    }
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r[i] = (__bf16)lo[i];
      r[4 + i] = (__bf16)hi[i];
    }
    *reinterpret_cast<bf16x8*>(out + (int64_t)t * H + n0) = r;
  }
}

std::atomic<int> g_cu_count[64];

template <int MODE, int RB, int U, int NS>
hipError_t launch_stream(const GemmParams& p, hipStream_t stream) {
  constexpr int BM = 16 * RB;
  const int64_t units_max = (int64_t)(p.capacity / BM) * (p.N / kNBlock);
  if (units_max == 0) return hipSuccess;
  static int blocks_per_cu = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, moe_gemm_stream_kernel<MODE, RB, U, NS>, 256, 0) != hipSuccess ||
        n < 1)
      n = 1;
    return n;
  }();
  const int64_t resident_waves = (int64_t)device_cu_count() * blocks_per_cu * 4;
  const int64_t waves = std::min(units_max, resident_waves);
  const int grid = (int)((waves + 3) / 4);
  hipLaunchKernelGGL((moe_gemm_stream_kernel<MODE, RB, U, NS>), dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_mode(int block_m, const GemmParams& p, hipStream_t stream) {
  switch (block_m) {
    case 16: return launch_stream<MODE, 1, 4, 2>(p, stream);
    case 32: return launch_stream<MODE, 2, 2, 2>(p, stream);
    case 64: return launch_stream<MODE, 4, 1, 2>(p, stream);
    case 128: return launch_stream<MODE, 8, 1, 2>(p, stream);
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

hipError_t launch_moe_gemm(GemmMode mode, int32_t block_m, const GemmParams& p, void* scratch, hipStream_t stream) {
  if (tiled_gemm_supported(block_m, p.N, p.K)) return launch_moe_gemm_tiled(mode, p, scratch, stream);
  if (stream_lds_supported(block_m, p)) return launch_moe_gemm_stream_lds(mode, block_m, p, stream);
  return mode == kGateUp ? launch_mode<kGateUp>(block_m, p, stream) : launch_mode<kDown>(block_m, p, stream);
}

hipError_t launch_combine(const int32_t* ids, const float* w, const float* y, uint16_t* out, int32_t T, int32_t topk,
                          int32_t H, int32_t E, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  // few tokens: split rows over blocks for parallelism; many tokens: a block per row
  const int cols = T >= 256 ? H : 8 * 256;
  const int64_t blocks = (int64_t)T * ((H + cols - 1) / cols);
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, ids, w, y, out, topk, H, E, cols);
  return hipGetLastError();
}

}  // namespace w4a16
