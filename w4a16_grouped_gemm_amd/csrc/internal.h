// Internal declarations of the gfx950 W4A16 MoE library: kernel launchers
// called by the C ABI in api.hip, and the packed-weight layout they share.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w4a16 {

// ---------------------------------------------------------------------------
// Packed weight layout (written once by the repack kernels, read by the GEMMs)
//
// A projection W of one expert has N output channels and a reduction length
// K = 32 * G. Channels are taken in n-blocks of 64, each split into four
// 16-wide column blocks c = 0..3, which is the B-operand width of
// v_mfma_f32_16x16x32_bf16. For gate_up (N = 2I) an n-block nb holds gate
// channels 32nb..32nb+31 in c = 0, 1 and the matching up channels
// I+32nb..I+32nb+31 in c = 2, 3, so one wave sees both halves of SiLU-and-mul.
//
// Nibbles: one 1024-byte unit per (expert e, n-block nb, group g), units ordered
// e-major, then nb, then g (one n-block streams all of K contiguously). In a
// unit, lane l (0..63) owns bytes [16 l, 16 l + 16): dword c holds the eight
// codes of column 16c + (l & 15), k = 32g + 8(l >> 4) + 0..7, with element
// 2j in bits [4j, 4j+4) and element 2j+1 in bits [16+4j, 20+4j), j = 0..3.
// A code is the weight's int4 value plus 8 (0..15), so OR-ing it into the
// mantissa of bf16 128.0 (0x4300) yields the exact bf16 value q + 136.
//
// Scales: one 64-entry unit of bf16 per (e, nb, g), same unit order; entry
// 4 * (l & 15) + c is the scale of column 16c + (l & 15), so a lane reads its
// four scales as one 8-byte load.
//
// Normalised scales (read by the fp16-operand tiled GEMM): the same units in
// fp16, holding s * 2^-E_n, where E_n (int32 per expert and packed channel
// 64 nb + 16 c + j, stored after them) is the unbiased exponent of the
// channel's largest |s|. The normalised scales are exact copies of the bf16
// ones down to 2^-17 of the channel's largest (smaller ones round to the fp16
// subnormal grid).
//
// A projection's packed buffer is four 256-byte aligned regions: nibbles,
// bf16 scales, fp16 scales, channel exponents (see packed_regions).
// ---------------------------------------------------------------------------
constexpr int kGroup = 32;
constexpr int kNBlock = 64;
constexpr int kNibUnitBytes = 1024;
constexpr int kScaleUnitElems = 64;

struct PackedRegions {
  size_t nib, s_bf16, s_f16, cexp, total;  // byte offsets of the regions, total size
};
inline size_t round_up256(size_t v) { return (v + 255) / 256 * 256; }
inline PackedRegions packed_regions(size_t E, size_t N, size_t K) {
  PackedRegions r;
  r.nib = 0;
  r.s_bf16 = round_up256(E * N * K / 2);
  r.s_f16 = r.s_bf16 + round_up256(E * N * (K / kGroup) * 2);
  r.cexp = r.s_f16 + round_up256(E * N * (K / kGroup) * 2);
  r.total = r.cexp + round_up256(E * N * 4);
  return r;
}

struct GemmParams {
  const uint16_t* a;       // gate_up: x [T, H]; down: h [capacity, I]
  const uint8_t* wq;       // packed nibbles of this projection, all experts
  const uint16_t* ws;      // packed bf16 scales of this projection, all experts
  const uint16_t* ws16;    // packed normalised fp16 scales (tiled path)
  const int32_t* col_exp;  // channel exponents E_n [E, N] (tiled path)
  const int32_t* row_exp;  // A row exponents (tiled path, set by its launcher)
  const uint16_t* a16;     // fp16 copy of the A rows (tiled path, set by its launcher)
  const int32_t* sorted;   // sorted_token_ids [capacity]
  const int32_t* expert_ids;
  const int32_t* ntpp;     // num_tokens_post_padded (device)
  void* out;               // gate_up: h bf16 [capacity, I]; down: y fp32 [n_slots, H] (bf16 with out_bf16)
  int32_t K;               // reduction length (H or I)
  int32_t N;               // output channels (2I or H)
  int32_t E;
  int32_t topk;
  int32_t n_slots;         // T * topk: ids >= this are padding
  int32_t capacity;
  int32_t out_ld;          // leading dimension of out (I or H)
  int32_t out_bf16;        // down only: write each slot's row rounded to bf16 instead of fp32
};

enum GemmMode { kGateUp = 0, kDown = 1 };

// Launchers: return hipSuccess or the launch error. All run on `stream`.
// Alignment of n routed ids over experts [0, E). Experts whose resident count
// lies outside [min_count, max_count] are treated as not resident.
hipError_t launch_align(const int32_t* ids, int32_t n, int32_t E, int32_t block_m, int32_t* sorted,
                        int32_t capacity, int32_t* expert_ids, int32_t* ntpp, int32_t* counts,
                        void* workspace, hipStream_t stream, int32_t min_count = 0,
                        int32_t max_count = 0x7fffffff);
// Two count-range alignments of the same ids: [split, max] at block_m bm0 into
// sorted[0, cap0), and [1, split - 1] at bm1 into sorted[cap0, cap0 + cap1);
// each equals launch_align with that range. Same workspace as launch_align.
hipError_t launch_align_split(const int32_t* ids, int32_t n, int32_t E, int32_t split, int32_t* sorted, int32_t bm0,
                              int32_t cap0, int32_t* eids0, int32_t* ntpp0, int32_t bm1, int32_t cap1,
                              int32_t* eids1, int32_t* ntpp1, void* workspace, hipStream_t stream);
size_t align_workspace_bytes(int64_t n, int32_t E);

// Top-k routing of fp32 logits [T, Eg] (+ optional bias [Eg]) into topk_ids /
// topk_weights, then the alignment of those ids over the local experts [0, E).
// Eg <= 1024, topk <= min(Eg, 32). Same workspace as launch_align.
hipError_t launch_route_align(const float* logits, const float* bias, int32_t T, int32_t Eg, int32_t topk, int32_t E,
                              int32_t block_m, int32_t* topk_ids, float* topk_weights, int32_t* sorted,
                              int32_t capacity, int32_t* expert_ids, int32_t* ntpp, int32_t* counts, void* workspace,
                              hipStream_t stream);

// Alignment buffers for the expert-grouped activation layouts (no routed ids):
// kContiguous takes a per-row expert index m_indices [M]; kMasked takes
// masked_m [E] live rows of each expert's max_m-row budget (M = E * max_m).
// Writes sorted [capacity] (p for a live row p, else the sentinel M),
// expert_ids [ceil(capacity / block_m)] (the expert of the block's first row,
// -1 when that row is not live), *ntpp = M and row_ids [M] (the row's expert,
// or -1 for a row that is not live).
// Then, when out is not null, zeroes the rows of out [M, H] (bf16) that are not
// live (the GEMMs write only live rows).
enum GroupedLayout { kContiguous = 0, kMasked = 1 };
hipError_t launch_grouped_index(GroupedLayout kind, const int32_t* m_indices, const int32_t* masked_m, int32_t M,
                                int32_t max_m, int32_t E, int32_t block_m, int32_t* row_ids, int32_t* sorted,
                                int32_t capacity, int32_t* expert_ids, int32_t* ntpp, uint16_t* out, int32_t H,
                                hipStream_t stream);

// Writes all four regions of one projection's packed buffer.
hipError_t launch_repack(const uint8_t* q, const uint16_t* s, int32_t E, int32_t N, int32_t K,
                         int32_t interleave_I, uint8_t* packed, hipStream_t stream);

// `scratch` (device, >= gemm_scratch_bytes) is used by the tiled path only.
hipError_t launch_moe_gemm(GemmMode mode, int32_t block_m, const GemmParams& p, void* scratch, hipStream_t stream);

// Tiled (LDS-staged, 128 x 256 tile, fp16 operands) variant for block_m == 128;
// used by launch_moe_gemm when the shape fits it. Its A operand is an fp16 copy
// of the activation rows with a power-of-two exponent per row, written into
// `scratch` (tiled_scratch_bytes(rows, K)) beforehand: by
// launch_rows_to_f16_tokens for gate_up (rows = T, token rows with a resident
// slot) and launch_rows_to_f16_aligned for down (rows = capacity, real aligned rows).
bool tiled_gemm_supported(int32_t block_m, int32_t N, int32_t K);
size_t tiled_scratch_bytes(int64_t rows, int32_t K);
hipError_t launch_rows_to_f16_tokens(const uint16_t* x, int32_t T, int32_t K, const int32_t* topk_ids, int32_t topk,
                                     int32_t E, void* scratch, hipStream_t stream);
hipError_t launch_rows_to_f16_aligned(const uint16_t* h, int32_t capacity, int32_t K, const int32_t* sorted,
                                      const int32_t* ntpp, int32_t n_slots, void* scratch, hipStream_t stream);
hipError_t launch_moe_gemm_tiled(GemmMode mode, const GemmParams& p, void* scratch, hipStream_t stream);

// Weight-streaming variant for block_m 16..64 with LDS rings for A and scales;
// used when N is a multiple of 256 and K / 32 a multiple of 4.
bool stream_lds_supported(int32_t block_m, const GemmParams& p);
hipError_t launch_moe_gemm_stream_lds(GemmMode mode, int32_t block_m, const GemmParams& p, hipStream_t stream);

// The block_m 16 gate_up GEMM with the alignment of its n routed ids done
// inside the same launch (n <= 1024 over E <= 64 experts; p.sorted,
// p.expert_ids, p.ntpp are ignored): sorted, expert_ids and ntpp (capacity
// p.capacity) are written as launch_align writes them, for the down GEMM.
// hipErrorNotSupported, with nothing launched, when the shape is outside that.
hipError_t launch_gate_up_fused_align(const GemmParams& p, const int32_t* ids, int32_t n, int32_t* sorted,
                                      int32_t* expert_ids, int32_t* ntpp, hipStream_t stream);

hipError_t launch_combine(const int32_t* ids, const float* w, const float* y, uint16_t* out, int32_t T,
                          int32_t topk, int32_t H, int32_t E, hipStream_t stream);

// Compute units of the current device (cached per device).
int device_cu_count();

}  // namespace w4a16
