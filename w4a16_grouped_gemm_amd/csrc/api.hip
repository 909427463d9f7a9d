// C ABI of the W4A16 MoE library: argument validation on the host, workspace
// carving, and launch order on the caller's stream. Declarations, argument
// meaning and error behaviour are documented in include/w4a16_moe.h.
#include "w4a16_moe.h"

#include <limits.h>

#include <algorithm>

#include "internal.h"

using namespace w4a16;

namespace {

constexpr size_t kAlign = 256;
size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Capacity the light set of a split alignment needs: every light expert holds
// at most split - 1 ids, so at most that many rounded up to block_m once padded.
size_t split_light_capacity(int32_t T, int32_t topk, int32_t E, int32_t split, int32_t bm) {
  const size_t per = ((size_t)(split - 1) + bm - 1) / bm * bm;
  return std::min<size_t>((size_t)T * topk + (size_t)E * (bm - 1), (size_t)E * per);
}

bool block_m_ok(int32_t bm) { return bm == 16 || bm == 32 || bm == 64 || bm == 128; }

int check_shape(const w4a16_moe_shape* s) {
  if (!s) return W4A16_ERR_INVALID_ARG;
  if (s->num_experts < 1 || s->hidden < 1 || s->intermediate < 1) return W4A16_ERR_INVALID_ARG;
  if (s->group_size != W4A16_GROUP_SIZE) return W4A16_ERR_UNSUPPORTED;
  if (s->num_experts > W4A16_MAX_EXPERTS) return W4A16_ERR_UNSUPPORTED;
  if (s->hidden % 64 != 0 || s->intermediate % 32 != 0) return W4A16_ERR_UNSUPPORTED;
  // per-expert weight offsets and row products are computed in 64-bit; keep every
  // index that stays 32-bit (rows, channels, groups) far from overflow
  if (s->hidden > (1 << 20) || s->intermediate > (1 << 20)) return W4A16_ERR_UNSUPPORTED;
  return W4A16_OK;
}

// T, topk and the derived sizes must fit the kernels' 32-bit slot indices.
int check_tokens(int32_t T, int32_t topk, int32_t E, int32_t block_m) {
  if (T < 0 || topk < 1 || E < 1) return W4A16_ERR_INVALID_ARG;
  if (topk > W4A16_MAX_TOPK || E > W4A16_MAX_EXPERTS) return W4A16_ERR_UNSUPPORTED;
  if (!block_m_ok(block_m)) return W4A16_ERR_UNSUPPORTED;
  const int64_t cap = (int64_t)T * topk + (int64_t)E * (block_m - 1);
  if (cap > INT_MAX / 2) return W4A16_ERR_UNSUPPORTED;
  return W4A16_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP; }

// The kernels move activations, weights and outputs 16 bytes at a time.
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
template <typename... Ps>
bool all_aligned16(const Ps*... ps) {
  return (aligned16(ps) && ...);
}

GemmParams gemm_params(const w4a16_moe_shape* s, int32_t T, int32_t topk, const int32_t* sorted, int32_t capacity,
                       const int32_t* expert_ids, const int32_t* ntpp, const void* packed, int32_t N, int32_t K) {
  GemmParams p{};
  const PackedRegions r = packed_regions((size_t)s->num_experts, (size_t)N, (size_t)K);
  const uint8_t* base = static_cast<const uint8_t*>(packed);
  p.wq = base + r.nib;
  p.ws = reinterpret_cast<const uint16_t*>(base + r.s_bf16);
  p.ws16 = reinterpret_cast<const uint16_t*>(base + r.s_f16);
  p.col_exp = reinterpret_cast<const int32_t*>(base + r.cexp);
  p.N = N;
  p.K = K;
  p.sorted = sorted;
  p.expert_ids = expert_ids;
  p.ntpp = ntpp;
  p.E = s->num_experts;
  p.topk = topk;
  p.n_slots = T * topk;
  p.capacity = capacity;
  return p;
}

}  // namespace

extern "C" {

const char* w4a16_status_string(int status) {
  switch (status) {
    case W4A16_OK: return "ok";
    case W4A16_ERR_INVALID_ARG: return "invalid argument";
    case W4A16_ERR_UNSUPPORTED: return "unsupported configuration";
    case W4A16_ERR_CAPACITY: return "sorted_token_ids capacity too small";
    case W4A16_ERR_WORKSPACE: return "workspace too small";
    case W4A16_ERR_HIP: return "HIP runtime error";
    case W4A16_ERR_NOALLOC_LIMIT: return "call needs more scratch than the no-alloc entry point's static array";
    default: return "unknown status";
  }
}

int w4a16_packed_bytes(const w4a16_moe_shape* shape, size_t* w13_bytes, size_t* w2_bytes) {
  const int st = check_shape(shape);
  if (st != W4A16_OK) return st;
  if (!w13_bytes || !w2_bytes) return W4A16_ERR_INVALID_ARG;
  const size_t E = (size_t)shape->num_experts, H = (size_t)shape->hidden, I = (size_t)shape->intermediate;
  *w13_bytes = packed_regions(E, 2 * I, H).total;
  *w2_bytes = packed_regions(E, H, I).total;
  return W4A16_OK;
}

int w4a16_repack(const w4a16_moe_shape* shape, const uint8_t* w13_q, const uint16_t* w13_s, const uint8_t* w2_q,
                 const uint16_t* w2_s, void* w13_packed, void* w2_packed, void* stream) {
  const int st = check_shape(shape);
  if (st != W4A16_OK) return st;
  if (!w13_q || !w13_s || !w2_q || !w2_s || !w13_packed || !w2_packed) return W4A16_ERR_INVALID_ARG;
  const int32_t E = shape->num_experts, H = shape->hidden, I = shape->intermediate;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_repack(w13_q, w13_s, E, 2 * I, H, I, static_cast<uint8_t*>(w13_packed), s);
  if (e != hipSuccess) return W4A16_ERR_HIP;
  e = launch_repack(w2_q, w2_s, E, H, I, 0, static_cast<uint8_t*>(w2_packed), s);
  return hip_status(e);
}

size_t moe_align_capacity(int32_t T, int32_t topk, int32_t num_experts, int32_t block_m) {
  if (check_tokens(T, topk, num_experts, block_m) != W4A16_OK) return 0;
  return (size_t)T * topk + (size_t)num_experts * (block_m - 1);
}

size_t moe_align_workspace_bytes(int32_t T, int32_t topk, int32_t num_experts, int32_t block_m) {
  if (check_tokens(T, topk, num_experts, block_m) != W4A16_OK) return 0;
  return align_workspace_bytes((int64_t)T * topk, num_experts);
}

int32_t w4a16_choose_block_m(int32_t T, int32_t topk, int32_t num_experts_local, int32_t num_experts_global) {
  if (T < 0 || topk < 1 || num_experts_local < 1 || num_experts_global < num_experts_local) return 0;
  // Expected routed tokens per expert. Row blocks must hold the typical
  // busiest expert in one block while tokens are few (decode: weight streaming,
  // each extra block re-reads the expert's weights), and grow to 128 rows once
  // experts carry enough tokens to make the MFMA tile the limit. Measured on
  // the 48-expert Kimi-K2 slice (layer at every block_m, T = 1 .. 8192): 16 is
  // best up to tok_e 10.7, 32 at 21 (64 is 37% slower there: its 64-row
  // streaming kernel holds 2 waves per SIMD), 64 and 128 within 7% at 43, 128
  // from 85 on. With the 16/32 switch at 6 the rule stays within 8% of the best
  // block_m at every measured point with resident slots, and the intermediate-sliced layer (384
  // experts, tok_e 10.7) keeps 32, measured 3% faster than 16 there.
  const double tok_e = (double)T * topk / num_experts_global;
  if (tok_e <= 6.0) return 16;
  if (tok_e <= 40.0) return 32;
  return 128;
}

int moe_align(const int32_t* topk_ids, int32_t T, int32_t topk, int32_t num_experts, int32_t block_m,
              int32_t* sorted_token_ids, int32_t capacity, int32_t* expert_ids, int32_t* num_tokens_post_padded,
              int32_t* expert_counts, void* workspace, size_t workspace_bytes, void* stream) {
  return moe_align_filtered(topk_ids, T, topk, num_experts, block_m, 0, INT32_MAX, sorted_token_ids, capacity,
                            expert_ids, num_tokens_post_padded, expert_counts, workspace, workspace_bytes, stream);
}

int moe_align_filtered(const int32_t* topk_ids, int32_t T, int32_t topk, int32_t num_experts, int32_t block_m,
                       int32_t min_count, int32_t max_count, int32_t* sorted_token_ids, int32_t capacity,
                       int32_t* expert_ids, int32_t* num_tokens_post_padded, int32_t* expert_counts, void* workspace,
                       size_t workspace_bytes, void* stream) {
  const int st = check_tokens(T, topk, num_experts, block_m);
  if (st != W4A16_OK) return st;
  if (min_count < 0 || max_count < min_count) return W4A16_ERR_INVALID_ARG;
  if ((T > 0 && !topk_ids) || !sorted_token_ids || !expert_ids || !num_tokens_post_padded)
    return W4A16_ERR_INVALID_ARG;
  if (capacity < 0 || (size_t)capacity < moe_align_capacity(T, topk, num_experts, block_m)) return W4A16_ERR_CAPACITY;
  const size_t ws = align_workspace_bytes((int64_t)T * topk, num_experts);
  if (ws > 0 && (!workspace || workspace_bytes < ws)) return W4A16_ERR_WORKSPACE;
  return hip_status(launch_align(topk_ids, T * topk, num_experts, block_m, sorted_token_ids, capacity, expert_ids,
                                 num_tokens_post_padded, expert_counts, workspace, static_cast<hipStream_t>(stream),
                                 min_count, max_count));
}

int moe_align_split(const int32_t* topk_ids, int32_t T, int32_t topk, int32_t num_experts, int32_t split_count,
                    int32_t heavy_block_m, int32_t heavy_capacity, int32_t* heavy_expert_ids,
                    int32_t* heavy_num_tokens_post_padded, int32_t light_block_m, int32_t light_capacity,
                    int32_t* light_expert_ids, int32_t* light_num_tokens_post_padded, int32_t* sorted_token_ids,
                    void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_tokens(T, topk, num_experts, heavy_block_m);
  if (st != W4A16_OK) return st;
  if ((st = check_tokens(T, topk, num_experts, light_block_m)) != W4A16_OK) return st;
  if (split_count < 2) return W4A16_ERR_INVALID_ARG;
  if ((T > 0 && !topk_ids) || !sorted_token_ids || !heavy_expert_ids || !heavy_num_tokens_post_padded ||
      !light_expert_ids || !light_num_tokens_post_padded)
    return W4A16_ERR_INVALID_ARG;
  if (heavy_capacity < 0 || (size_t)heavy_capacity < moe_align_capacity(T, topk, num_experts, heavy_block_m))
    return W4A16_ERR_CAPACITY;
  if (light_capacity < 0 || (size_t)light_capacity < split_light_capacity(T, topk, num_experts, split_count,
                                                                          light_block_m))
    return W4A16_ERR_CAPACITY;
  if ((int64_t)heavy_capacity + light_capacity > INT32_MAX) return W4A16_ERR_CAPACITY;
  const size_t ws = align_workspace_bytes((int64_t)T * topk, num_experts);
  if (ws > 0 && (!workspace || workspace_bytes < ws)) return W4A16_ERR_WORKSPACE;
  return hip_status(launch_align_split(topk_ids, T * topk, num_experts, split_count, sorted_token_ids, heavy_block_m,
                                       heavy_capacity, heavy_expert_ids, heavy_num_tokens_post_padded, light_block_m,
                                       light_capacity, light_expert_ids, light_num_tokens_post_padded, workspace,
                                       static_cast<hipStream_t>(stream)));
}

int moe_route_align(const float* logits, const float* bias, int32_t T, int32_t num_routed_experts, int32_t topk,
                    int32_t num_experts, int32_t block_m, int32_t* topk_ids, float* topk_weights,
                    int32_t* sorted_token_ids, int32_t capacity, int32_t* expert_ids, int32_t* num_tokens_post_padded,
                    int32_t* expert_counts, void* workspace, size_t workspace_bytes, void* stream) {
  const int st = check_tokens(T, topk, num_experts, block_m);
  if (st != W4A16_OK) return st;
  if (num_routed_experts < num_experts || topk > num_routed_experts) return W4A16_ERR_INVALID_ARG;
  if (num_routed_experts > W4A16_MAX_ROUTED_EXPERTS) return W4A16_ERR_UNSUPPORTED;
  if ((T > 0 && (!logits || !topk_ids || !topk_weights)) || !sorted_token_ids || !expert_ids ||
      !num_tokens_post_padded)
    return W4A16_ERR_INVALID_ARG;
  if (capacity < 0 || (size_t)capacity < moe_align_capacity(T, topk, num_experts, block_m)) return W4A16_ERR_CAPACITY;
  const size_t ws = align_workspace_bytes((int64_t)T * topk, num_experts);
  if (ws > 0 && (!workspace || workspace_bytes < ws)) return W4A16_ERR_WORKSPACE;
  return hip_status(launch_route_align(logits, bias, T, num_routed_experts, topk, num_experts, block_m, topk_ids,
                                       topk_weights, sorted_token_ids, capacity, expert_ids, num_tokens_post_padded,
                                       expert_counts, workspace, static_cast<hipStream_t>(stream)));
}

size_t w4a16_moe_stage_workspace_bytes(const w4a16_moe_shape* shape, int32_t T, int32_t topk, int32_t block_m) {
  if (check_shape(shape) != W4A16_OK) return 0;
  if (check_tokens(T, topk, shape->num_experts, block_m) != W4A16_OK) return 0;
  const int32_t H = shape->hidden, I = shape->intermediate;
  // the tiled path's fp16 A rows: x rows for gate_up, aligned h rows for down
  // (the two GEMMs run one after the other and share the region)
  const size_t cap = moe_align_capacity(T, topk, shape->num_experts, block_m);
  size_t need = 0;
  if (tiled_gemm_supported(block_m, 2 * I, H)) need = std::max(need, tiled_scratch_bytes(T, H));
  if (tiled_gemm_supported(block_m, H, I)) need = std::max(need, tiled_scratch_bytes((int64_t)cap, I));
  return round_up(need);
}

size_t w4a16_moe_workspace_bytes(const w4a16_moe_shape* shape, int32_t T, int32_t topk, int32_t block_m) {
  if (check_shape(shape) != W4A16_OK) return 0;
  if (check_tokens(T, topk, shape->num_experts, block_m) != W4A16_OK) return 0;
  const size_t cap = moe_align_capacity(T, topk, shape->num_experts, block_m);
  return round_up(cap * (size_t)shape->intermediate * 2) + round_up((size_t)T * topk * shape->hidden * 4) +
         w4a16_moe_stage_workspace_bytes(shape, T, topk, block_m);
}

namespace {
int check_stage_workspace(const w4a16_moe_shape* shape, int32_t T, int32_t topk, int32_t block_m, const void* ws,
                          size_t ws_bytes) {
  const size_t need = w4a16_moe_stage_workspace_bytes(shape, T, topk, block_m);
  return (need > 0 && (!ws || ws_bytes < need)) ? W4A16_ERR_WORKSPACE : W4A16_OK;
}
}  // namespace

int w4a16_moe_prepare_x(const w4a16_moe_shape* shape, const uint16_t* x, int32_t T, int32_t topk,
                        const int32_t* topk_ids, int32_t block_m, void* workspace, size_t workspace_bytes,
                        void* stream) {
  int st = check_shape(shape);
  if (st != W4A16_OK) return st;
  st = check_tokens(T, topk, shape->num_experts, block_m);
  if (st != W4A16_OK) return st;
  if (T > 0 && (!x || !topk_ids)) return W4A16_ERR_INVALID_ARG;
  if (!all_aligned16(x, workspace)) return W4A16_ERR_INVALID_ARG;
  st = check_stage_workspace(shape, T, topk, block_m, workspace, workspace_bytes);
  if (st != W4A16_OK) return st;
  if (!tiled_gemm_supported(block_m, 2 * shape->intermediate, shape->hidden)) return W4A16_OK;  // nothing to prepare
  return hip_status(launch_rows_to_f16_tokens(x, T, shape->hidden, topk_ids, topk, shape->num_experts, workspace,
                                              static_cast<hipStream_t>(stream)));
}

int w4a16_moe_gate_up(const w4a16_moe_shape* shape, const uint16_t* x, int32_t T, int32_t topk,
                      const int32_t* sorted_token_ids, int32_t capacity, const int32_t* expert_ids,
                      const int32_t* num_tokens_post_padded, int32_t block_m, const void* w13_packed, uint16_t* h,
                      void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_shape(shape);
  if (st != W4A16_OK) return st;
  st = check_tokens(T, topk, shape->num_experts, block_m);
  if (st != W4A16_OK) return st;
  if ((T > 0 && !x) || !sorted_token_ids || !expert_ids || !num_tokens_post_padded || !w13_packed || !h)
    return W4A16_ERR_INVALID_ARG;
  if (!all_aligned16(x, w13_packed, h, workspace)) return W4A16_ERR_INVALID_ARG;
  if (capacity < 0 || (size_t)capacity < moe_align_capacity(T, topk, shape->num_experts, block_m))
    return W4A16_ERR_CAPACITY;
  st = check_stage_workspace(shape, T, topk, block_m, workspace, workspace_bytes);
  if (st != W4A16_OK) return st;
  const int32_t H = shape->hidden, I = shape->intermediate;
  GemmParams p = gemm_params(shape, T, topk, sorted_token_ids, capacity, expert_ids, num_tokens_post_padded,
                             w13_packed, 2 * I, H);
  p.a = x;
  p.out = h;
  p.out_ld = I;
  return hip_status(launch_moe_gemm(kGateUp, block_m, p, workspace, static_cast<hipStream_t>(stream)));
}

int w4a16_moe_prepare_h(const w4a16_moe_shape* shape, int32_t T, int32_t topk, const uint16_t* h,
                        const int32_t* sorted_token_ids, int32_t capacity, const int32_t* num_tokens_post_padded,
                        int32_t block_m, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_shape(shape);
  if (st != W4A16_OK) return st;
  st = check_tokens(T, topk, shape->num_experts, block_m);
  if (st != W4A16_OK) return st;
  if (!h || !sorted_token_ids || !num_tokens_post_padded) return W4A16_ERR_INVALID_ARG;
  if (!all_aligned16(h, workspace)) return W4A16_ERR_INVALID_ARG;
  if (capacity < 0 || (size_t)capacity < moe_align_capacity(T, topk, shape->num_experts, block_m))
    return W4A16_ERR_CAPACITY;
  st = check_stage_workspace(shape, T, topk, block_m, workspace, workspace_bytes);
  if (st != W4A16_OK) return st;
  if (!tiled_gemm_supported(block_m, shape->hidden, shape->intermediate)) return W4A16_OK;  // nothing to prepare
  // rows past moe_align_capacity are never live (num_tokens_post_padded <= it)
  const int32_t cap_min = (int32_t)moe_align_capacity(T, topk, shape->num_experts, block_m);
  return hip_status(launch_rows_to_f16_aligned(h, cap_min, shape->intermediate, sorted_token_ids,
                                               num_tokens_post_padded, T * topk, workspace,
                                               static_cast<hipStream_t>(stream)));
}

int w4a16_moe_down(const w4a16_moe_shape* shape, int32_t T, int32_t topk, const uint16_t* h,
                   const int32_t* sorted_token_ids, int32_t capacity, const int32_t* expert_ids,
                   const int32_t* num_tokens_post_padded, int32_t block_m, const void* w2_packed, float* y,
                   void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_shape(shape);
  if (st != W4A16_OK) return st;
  st = check_tokens(T, topk, shape->num_experts, block_m);
  if (st != W4A16_OK) return st;
  if (!h || !sorted_token_ids || !expert_ids || !num_tokens_post_padded || !w2_packed || (T > 0 && !y))
    return W4A16_ERR_INVALID_ARG;
  if (!all_aligned16(h, w2_packed, y, workspace)) return W4A16_ERR_INVALID_ARG;
  if (capacity < 0 || (size_t)capacity < moe_align_capacity(T, topk, shape->num_experts, block_m))
    return W4A16_ERR_CAPACITY;
  st = check_stage_workspace(shape, T, topk, block_m, workspace, workspace_bytes);
  if (st != W4A16_OK) return st;
  // the tiled path's prepared rows cover moe_align_capacity rows; rows past it
  // are never live, so the GEMM is given that capacity
  const size_t cap_min = moe_align_capacity(T, topk, shape->num_experts, block_m);
  const int32_t H = shape->hidden, I = shape->intermediate;
  GemmParams p = gemm_params(shape, T, topk, sorted_token_ids, (int32_t)cap_min, expert_ids, num_tokens_post_padded,
                             w2_packed, H, I);
  p.a = h;
  p.out = y;
  p.out_ld = H;
  return hip_status(launch_moe_gemm(kDown, block_m, p, workspace, static_cast<hipStream_t>(stream)));
}

int w4a16_moe_combine(const w4a16_moe_shape* shape, int32_t T, int32_t topk, const int32_t* topk_ids,
                      const float* topk_weights, const float* y, uint16_t* out, void* stream) {
  const int st = check_shape(shape);
  if (st != W4A16_OK) return st;
  if (T < 0 || topk < 1) return W4A16_ERR_INVALID_ARG;
  if (topk > W4A16_MAX_TOPK) return W4A16_ERR_UNSUPPORTED;
  if ((int64_t)T * topk > INT_MAX / 2) return W4A16_ERR_UNSUPPORTED;
  if (T > 0 && (!topk_ids || !topk_weights || !y || !out)) return W4A16_ERR_INVALID_ARG;
  if (!all_aligned16(y, out)) return W4A16_ERR_INVALID_ARG;
  return hip_status(launch_combine(topk_ids, topk_weights, y, out, T, topk, shape->hidden, shape->num_experts,
                                   static_cast<hipStream_t>(stream)));
}

int w4a16_moe_forward(const w4a16_moe_shape* shape, const uint16_t* x, int32_t T, int32_t topk,
                      const int32_t* topk_ids, const float* topk_weights, const int32_t* sorted_token_ids,
                      int32_t capacity, const int32_t* expert_ids, const int32_t* num_tokens_post_padded,
                      int32_t block_m, const void* w13_packed, const void* w2_packed, uint16_t* out, void* workspace,
                      size_t workspace_bytes, void* stream) {
  int st = check_shape(shape);
  if (st != W4A16_OK) return st;
  st = check_tokens(T, topk, shape->num_experts, block_m);
  if (st != W4A16_OK) return st;
  if ((T > 0 && (!x || !topk_ids || !topk_weights || !out)) || !sorted_token_ids || !expert_ids ||
      !num_tokens_post_padded || !w13_packed || !w2_packed)
    return W4A16_ERR_INVALID_ARG;
  if (!all_aligned16(x, out, w13_packed, w2_packed, workspace)) return W4A16_ERR_INVALID_ARG;
  if (capacity < 0 || (size_t)capacity < moe_align_capacity(T, topk, shape->num_experts, block_m))
    return W4A16_ERR_CAPACITY;
  const size_t need = w4a16_moe_workspace_bytes(shape, T, topk, block_m);
  if (!workspace || workspace_bytes < need) return W4A16_ERR_WORKSPACE;
  if (T == 0) return W4A16_OK;
  // workspace: h [cap_min, I] bf16, then y [T*topk, H] fp32, then the stages' scratch
  const size_t cap_min = moe_align_capacity(T, topk, shape->num_experts, block_m);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint16_t* h = reinterpret_cast<uint16_t*>(ws);
  const size_t h_bytes = round_up(cap_min * shape->intermediate * 2);
  float* y = reinterpret_cast<float*>(ws + h_bytes);
  const size_t y_bytes = round_up((size_t)T * topk * shape->hidden * 4);
  void* scratch = ws + h_bytes + y_bytes;
  const size_t scratch_bytes = workspace_bytes - h_bytes - y_bytes;
  // Rows past cap_min are never live: num_tokens_post_padded <= cap_min.
  st = w4a16_moe_prepare_x(shape, x, T, topk, topk_ids, block_m, scratch, scratch_bytes, stream);
  if (st != W4A16_OK) return st;
  st = w4a16_moe_gate_up(shape, x, T, topk, sorted_token_ids, (int32_t)cap_min, expert_ids, num_tokens_post_padded,
                         block_m, w13_packed, h, scratch, scratch_bytes, stream);
  if (st != W4A16_OK) return st;
  st = w4a16_moe_prepare_h(shape, T, topk, h, sorted_token_ids, (int32_t)cap_min, num_tokens_post_padded, block_m,
                           scratch, scratch_bytes, stream);
  if (st != W4A16_OK) return st;
  st = w4a16_moe_down(shape, T, topk, h, sorted_token_ids, (int32_t)cap_min, expert_ids, num_tokens_post_padded,
                      block_m, w2_packed, y, scratch, scratch_bytes, stream);
  if (st != W4A16_OK) return st;
  return w4a16_moe_combine(shape, T, topk, topk_ids, topk_weights, y, out, stream);
}

}  // extern "C"

namespace {
// Workspace of the grouped-layout entry points: row_ids [M] |
// sorted [capacity] | expert_ids [nblk] | ntpp | h [capacity, I] bf16 | the
// GEMM stages' scratch. The down GEMM writes the output rows directly (bf16),
// so there is no fp32 row buffer and no combine pass.
struct GroupedWorkspace {
  size_t row_ids, sorted, expert_ids, ntpp, h, scratch, scratch_bytes, total;
  int32_t capacity;
};

GroupedWorkspace grouped_workspace(const w4a16_moe_shape* s, int32_t M, int32_t bm) {
  GroupedWorkspace g{};
  g.capacity = (int32_t)moe_align_capacity(M, 1, s->num_experts, bm);
  const size_t nblk = ((size_t)g.capacity + bm - 1) / bm;
  g.row_ids = 0;
  g.sorted = g.row_ids + round_up((size_t)M * 4);
  g.expert_ids = g.sorted + round_up((size_t)g.capacity * 4);
  g.ntpp = g.expert_ids + round_up(nblk * 4);
  g.h = g.ntpp + kAlign;
  g.scratch = g.h + round_up((size_t)g.capacity * s->intermediate * 2);
  g.scratch_bytes = w4a16_moe_stage_workspace_bytes(s, M, 1, bm);
  g.total = g.scratch + g.scratch_bytes;
  return g;
}

constexpr int32_t kContiguousBlockM = 128;

int grouped_forward(GroupedLayout kind, const w4a16_moe_shape* shape, const uint16_t* x, int32_t M, int32_t max_m,
                    const int32_t* m_indices, const int32_t* masked_m, int32_t block_m, const void* w13_packed,
                    const void* w2_packed, uint16_t* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!all_aligned16(x, out, w13_packed, w2_packed, workspace)) return W4A16_ERR_INVALID_ARG;
  const GroupedWorkspace g = grouped_workspace(shape, M, block_m);
  if (!workspace || workspace_bytes < g.total) return W4A16_ERR_WORKSPACE;
  if (M == 0) return W4A16_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int32_t* row_ids = reinterpret_cast<int32_t*>(ws + g.row_ids);
  int32_t* sorted = reinterpret_cast<int32_t*>(ws + g.sorted);
  int32_t* expert_ids = reinterpret_cast<int32_t*>(ws + g.expert_ids);
  int32_t* ntpp = reinterpret_cast<int32_t*>(ws + g.ntpp);
  uint16_t* h = reinterpret_cast<uint16_t*>(ws + g.h);
  void* scratch = ws + g.scratch;
  const int32_t H = shape->hidden, I = shape->intermediate;
  // index buffers, and zeros in the output rows that are not live
  int rc = hip_status(launch_grouped_index(kind, m_indices, masked_m, M, max_m, shape->num_experts, block_m, row_ids,
                                           sorted, g.capacity, expert_ids, ntpp, out, H, st));
  if (rc != W4A16_OK) return rc;
  // every row is one slot (topk 1): the layer's stages up to down
  rc = w4a16_moe_prepare_x(shape, x, M, 1, row_ids, block_m, scratch, g.scratch_bytes, stream);
  if (rc != W4A16_OK) return rc;
  rc = w4a16_moe_gate_up(shape, x, M, 1, sorted, g.capacity, expert_ids, ntpp, block_m, w13_packed, h, scratch,
                         g.scratch_bytes, stream);
  if (rc != W4A16_OK) return rc;
  rc = w4a16_moe_prepare_h(shape, M, 1, h, sorted, g.capacity, ntpp, block_m, scratch, g.scratch_bytes, stream);
  if (rc != W4A16_OK) return rc;
  // down writes each live row's result straight into out, rounded once to bf16
  GemmParams p = gemm_params(shape, M, 1, sorted, g.capacity, expert_ids, ntpp, w2_packed, H, I);
  p.a = h;
  p.out = out;
  p.out_ld = H;
  p.out_bf16 = 1;
  return hip_status(launch_moe_gemm(kDown, block_m, p, scratch, st));
}
}  // namespace

extern "C" {

size_t w4a16_moe_contiguous_workspace_bytes(const w4a16_moe_shape* shape, int32_t M) {
  if (check_shape(shape) != W4A16_OK || M < 0 || M % kContiguousBlockM != 0) return 0;
  if (check_tokens(M, 1, shape->num_experts, kContiguousBlockM) != W4A16_OK) return 0;
  return grouped_workspace(shape, M, kContiguousBlockM).total;
}

int w4a16_moe_contiguous_forward(const w4a16_moe_shape* shape, const uint16_t* x, int32_t M,
                                 const int32_t* m_indices, const void* w13_packed, const void* w2_packed,
                                 uint16_t* out, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_shape(shape);
  if (st != W4A16_OK) return st;
  if (M < 0 || M % kContiguousBlockM != 0) return W4A16_ERR_INVALID_ARG;
  st = check_tokens(M, 1, shape->num_experts, kContiguousBlockM);
  if (st != W4A16_OK) return st;
  if ((M > 0 && (!x || !m_indices || !out)) || !w13_packed || !w2_packed) return W4A16_ERR_INVALID_ARG;
  return grouped_forward(kContiguous, shape, x, M, 0, m_indices, nullptr, kContiguousBlockM, w13_packed, w2_packed,
                         out, workspace, workspace_bytes, stream);
}

int32_t w4a16_moe_masked_block_m(int32_t max_m, int32_t expected_m) {
  if (max_m < 16 || max_m % 16 != 0 || expected_m < 0) return 0;
  int32_t bm = w4a16_choose_block_m(expected_m, 1, 1, 1);  // tokens per expert = expected_m
  while (max_m % bm != 0) bm /= 2;
  return bm;
}

size_t w4a16_moe_masked_workspace_bytes(const w4a16_moe_shape* shape, int32_t max_m, int32_t block_m) {
  if (check_shape(shape) != W4A16_OK || !block_m_ok(block_m) || max_m < 0 || max_m % block_m != 0) return 0;
  const int64_t M = (int64_t)shape->num_experts * max_m;
  if (M > INT_MAX || check_tokens((int32_t)M, 1, shape->num_experts, block_m) != W4A16_OK) return 0;
  return grouped_workspace(shape, (int32_t)M, block_m).total;
}

int w4a16_moe_masked_forward(const w4a16_moe_shape* shape, const uint16_t* x, int32_t max_m,
                             const int32_t* masked_m, int32_t block_m, const void* w13_packed, const void* w2_packed,
                             uint16_t* out, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_shape(shape);
  if (st != W4A16_OK) return st;
  if (!block_m_ok(block_m)) return W4A16_ERR_UNSUPPORTED;
  if (max_m < 0 || max_m % block_m != 0) return W4A16_ERR_INVALID_ARG;
  const int64_t M = (int64_t)shape->num_experts * max_m;
  if (M > INT_MAX) return W4A16_ERR_UNSUPPORTED;
  st = check_tokens((int32_t)M, 1, shape->num_experts, block_m);
  if (st != W4A16_OK) return st;
  if ((M > 0 && (!x || !masked_m || !out)) || !w13_packed || !w2_packed) return W4A16_ERR_INVALID_ARG;
  return grouped_forward(kMasked, shape, x, (int32_t)M, max_m, nullptr, masked_m, block_m, w13_packed, w2_packed,
                         out, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {
// The routed layer in one call. Prefill-sized calls on an expert slice
// (block_m 128 by the tokens-per-expert rule, tiled GEMMs available, fewer
// local than routed experts, so the local counts can be very uneven) split the
// experts by their resident count: experts with at least kHeavyRows slots run
// in 128-row tiles on the MFMA-bound tiled GEMMs, the lighter ones in 16-row
// blocks on the weight-streaming GEMMs, so a light expert no longer pays for a
// mostly empty 128-row tile. Other calls use one alignment at the rule's
// block_m. (Running the light set on a second stream, next to the heavy
// tiles, was measured: both kernels slowed down by about what they overlapped,
// so the sets run one after the other on the caller's stream.)
// The threshold is one more than the light block size: every light expert
// then fits one 16-row block and streams its weights once. Experts with 17 to
// 31 slots cost about as much either way by a per-expert model (two weight
// streams against one mostly padded 128-row tile row), and on the tiled side
// they mostly fill resident slots that the heavy launch leaves idle (the
// skewed 48-expert prefill: heavy set 25 -> 30 row blocks, still one round of
// tiles; light set 24 -> 14 row blocks; layer 543 -> 521 us, against 538 us
// at a threshold of 24 and 543 us at 32).
constexpr int32_t kLightBlockM = 16;
constexpr int32_t kHeavyRows = kLightBlockM + 1;
constexpr int32_t kHeavyBlockM = 128;

struct AlignSet {
  size_t sorted, expert_ids, ntpp, h;
  int32_t block_m, capacity;
  int32_t gemm_rows;  // rows the set's GEMMs cover: the live rows fit in them (ntpp <= gemm_rows <= capacity)
};

struct RoutedWorkspace {
  bool split;
  AlignSet set[2];  // [0]: the only set, or the heavy set; [1]: the light set
  size_t hist, y, scratch, scratch_bytes, total;
};

RoutedWorkspace routed_workspace(const w4a16_moe_shape* s, int32_t T, int32_t topk, int32_t num_experts_global) {
  RoutedWorkspace r{};
  const int32_t E = s->num_experts, H = s->hidden, I = s->intermediate;
  const int32_t bm = w4a16_choose_block_m(T, topk, E, num_experts_global);
  r.split = bm == kHeavyBlockM && tiled_gemm_supported(kHeavyBlockM, 2 * I, H) && num_experts_global > E;
  const int nsets = r.split ? 2 : 1;
  r.set[0].block_m = r.split ? kHeavyBlockM : bm;
  r.set[1].block_m = kLightBlockM;
  size_t off = 0;
  r.hist = off;
  off += round_up(align_workspace_bytes((int64_t)T * topk, E));
  r.set[0].capacity = (int32_t)moe_align_capacity(T, topk, E, r.set[0].block_m);
  // the tiled stages place their prepared rows and row exponents by this row
  // count, so it stays the one the stage workspace is sized for
  r.set[0].gemm_rows = r.set[0].capacity;
  if (r.split) {
    // one joined scatter fills both sets: the light set's sorted array follows
    // the heavy set's, whose capacity is rounded up to 64 ids so the light
    // array keeps the 256-byte alignment of the other buffers
    r.set[0].capacity = (r.set[0].capacity + 63) / 64 * 64;
    r.set[1].capacity = (int32_t)split_light_capacity(T, topk, E, kHeavyRows, kLightBlockM);
    r.set[1].gemm_rows = r.set[1].capacity;
  }
  r.set[0].sorted = off;
  off += (size_t)r.set[0].capacity * 4;
  if (r.split) {
    r.set[1].sorted = off;
    off += (size_t)r.set[1].capacity * 4;
  }
  off = round_up(off);
  for (int k = 0; k < nsets; ++k) {
    AlignSet& a = r.set[k];
    a.expert_ids = off;
    off += round_up(((size_t)a.capacity + a.block_m - 1) / a.block_m * 4);
    a.ntpp = off;
    off += kAlign;
    a.h = off;
    off += round_up((size_t)a.capacity * I * 2);
  }
  r.y = off;
  off += round_up((size_t)T * topk * H * 4);
  r.scratch = off;
  r.scratch_bytes = w4a16_moe_stage_workspace_bytes(s, T, topk, r.set[0].block_m);
  r.total = off + r.scratch_bytes;
  return r;
}
}  // namespace

extern "C" {

size_t w4a16_moe_routed_workspace_bytes(const w4a16_moe_shape* shape, int32_t T, int32_t topk,
                                        int32_t num_experts_global) {
  if (check_shape(shape) != W4A16_OK || num_experts_global < shape->num_experts) return 0;
  if (check_tokens(T, topk, shape->num_experts, kHeavyBlockM) != W4A16_OK) return 0;
  return routed_workspace(shape, T, topk, num_experts_global).total;
}

int32_t w4a16_moe_routed_split(const w4a16_moe_shape* shape, int32_t T, int32_t topk, int32_t num_experts_global) {
  if (check_shape(shape) != W4A16_OK || num_experts_global < shape->num_experts) return -1;
  if (check_tokens(T, topk, shape->num_experts, kHeavyBlockM) != W4A16_OK) return -1;
  return routed_workspace(shape, T, topk, num_experts_global).split ? kHeavyRows : 0;
}

int w4a16_moe_routed_forward(const w4a16_moe_shape* shape, const uint16_t* x, int32_t T, int32_t topk,
                             int32_t num_experts_global, const int32_t* topk_ids, const float* topk_weights,
                             const void* w13_packed, const void* w2_packed, uint16_t* out, void* workspace,
                             size_t workspace_bytes, void* stream) {
  int st = check_shape(shape);
  if (st != W4A16_OK) return st;
  if (num_experts_global < shape->num_experts) return W4A16_ERR_INVALID_ARG;
  st = check_tokens(T, topk, shape->num_experts, kHeavyBlockM);  // the largest capacity any set uses
  if (st != W4A16_OK) return st;
  if ((T > 0 && (!x || !topk_ids || !topk_weights || !out)) || !w13_packed || !w2_packed)
    return W4A16_ERR_INVALID_ARG;
  if (!all_aligned16(x, out, w13_packed, w2_packed, workspace)) return W4A16_ERR_INVALID_ARG;
  const RoutedWorkspace r = routed_workspace(shape, T, topk, num_experts_global);
  if (!workspace || workspace_bytes < r.total) return W4A16_ERR_WORKSPACE;
  if (T == 0) return W4A16_OK;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const int32_t E = shape->num_experts;
  const int nsets = r.split ? 2 : 1;
  int32_t* sorted[2];
  int32_t* eids[2];
  int32_t* ntpp[2];
  uint16_t* h[2];
  for (int k = 0; k < nsets; ++k) {
    sorted[k] = reinterpret_cast<int32_t*>(ws + r.set[k].sorted);
    eids[k] = reinterpret_cast<int32_t*>(ws + r.set[k].expert_ids);
    ntpp[k] = reinterpret_cast<int32_t*>(ws + r.set[k].ntpp);
    h[k] = reinterpret_cast<uint16_t*>(ws + r.set[k].h);
  }
  float* y = reinterpret_cast<float*>(ws + r.y);
  void* scratch = ws + r.scratch;
  void* hist = ws + r.hist;
  const int32_t H = shape->hidden, I = shape->intermediate;
  // the light set's capacity is below moe_align_capacity, so its GEMMs are launched here directly
  const auto gemm_params_of = [&](GemmMode mode, int k) {
    const bool up = mode == kGateUp;
    GemmParams p = gemm_params(shape, T, topk, sorted[k], r.set[k].gemm_rows, eids[k], ntpp[k],
                               up ? w13_packed : w2_packed, up ? 2 * I : H, up ? H : I);
    p.a = up ? x : h[k];
    p.out = up ? static_cast<void*>(h[k]) : static_cast<void*>(y);
    p.out_ld = up ? I : H;
    return p;
  };
  const auto gemm = [&](GemmMode mode, int k) {
    return hip_status(launch_moe_gemm(mode, r.set[k].block_m, gemm_params_of(mode, k), scratch, hs));
  };
  // Decode-sized calls at block_m 16: the alignment runs inside the gate_up
  // launch (one launch less on the path); otherwise it is a launch of its own.
  bool aligned_in_gate_up = false;
  if (!r.split && r.set[0].block_m == 16) {
    const hipError_t e = launch_gate_up_fused_align(gemm_params_of(kGateUp, 0), topk_ids, T * topk, sorted[0],
                                                    eids[0], ntpp[0], hs);
    if (e == hipSuccess) aligned_in_gate_up = true;
    else if (e != hipErrorNotSupported) return hip_status(e);
  }
  if (!aligned_in_gate_up) {
    if (r.split)  // both sets in one pass over the ids
      st = hip_status(launch_align_split(topk_ids, T * topk, E, kHeavyRows, sorted[0], r.set[0].block_m,
                                         r.set[0].capacity, eids[0], ntpp[0], r.set[1].block_m, r.set[1].capacity,
                                         eids[1], ntpp[1], hist, hs));
    else
      st = hip_status(launch_align(topk_ids, T * topk, E, r.set[0].block_m, sorted[0], r.set[0].capacity, eids[0],
                                   ntpp[0], nullptr, hist, hs));
    if (st != W4A16_OK) return st;
  }
  st = w4a16_moe_prepare_x(shape, x, T, topk, topk_ids, r.set[0].block_m, scratch, r.scratch_bytes, stream);
  if (st != W4A16_OK) return st;
  for (int k = aligned_in_gate_up ? 1 : 0; k < nsets; ++k)
    if ((st = gemm(kGateUp, k)) != W4A16_OK) return st;
  st = w4a16_moe_prepare_h(shape, T, topk, h[0], sorted[0], r.set[0].gemm_rows, ntpp[0], r.set[0].block_m, scratch,
                           r.scratch_bytes, stream);
  if (st != W4A16_OK) return st;
  for (int k = 0; k < nsets; ++k)
    if ((st = gemm(kDown, k)) != W4A16_OK) return st;
  return w4a16_moe_combine(shape, T, topk, topk_ids, topk_weights, y, out, stream);
}

}  // extern "C"
