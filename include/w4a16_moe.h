/*
 * w4a16_moe.h — C ABI of the MI355X (gfx950) W4A16 fused mixture-of-experts layer.
 *
 * The layer: BF16 activations routed top-k to experts whose weights are
 * symmetric INT4 with one BF16 scale per group of 32 along the reduction
 * dimension ("W4A16 그룹 스케일 형식", group-32 key: Chord page "vLLM 및 Novita AI,
 * Kimi K2.x용 더 빠른 INT4 MoE 커널 출시: Chord", sections "vLLM과의 통합" and
 * "런타임 고려사항"). The entry points, all on the caller's HIP stream:
 *
 *   moe_align           topk_ids -> sorted_token_ids, expert_ids, num_tokens_post_padded
 *   moe_align_filtered / moe_align_split
 *                       the same restricted to a band of per-expert counts; both
 *                       bands of a heavy/light split in one pass
 *   moe_route_align     router logits -> top-k ids and weights, then moe_align
 *   w4a16_moe_forward   gate_up GEMM + SiLU-and-mul, down GEMM, top-k weighted combine
 *   w4a16_moe_routed_forward  alignment + the layer in one call, per-expert tile sizes
 *   w4a16_moe_routed_forward_noalloc  the same with its workspace in a static device array
 *   w4a16_moe_contiguous_forward / w4a16_moe_masked_forward
 *                       the layer on expert-grouped activation layouts
 *   w4a16_repack        once at weight load: canonical int4 + scales -> kernel layout
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Ownership: the caller allocates and owns every buffer. Pointers named "device"
 *   are device memory of the current HIP device; the library never allocates,
 *   frees or synchronizes, and launches only on the given stream (`stream` is a
 *   hipStream_t; NULL is the null stream). Calls are stateless apart from a
 *   per-device cache of the compute-unit count, and are safe to capture in a
 *   HIP graph (no host synchronization, no memset nodes).
 * Errors: every function validates its arguments on the host before touching
 *   the device and returns a w4a16_status. No fallback path exists: an
 *   unsupported configuration is an error, never a silent switch (Chord page,
 *   "vLLM과의 통합": unsupported quantization schemes raise instead of falling
 *   back). W4A16_ERR_HIP means a HIP launch reported an error.
 * Numerics: fp32 accumulation only; there is no f16-accumulation or
 *   batch-invariant option (Chord page, "런타임 고려사항"; Humming PR page
 *   "[vllm] vLLM에 고성능 JIT 양자화 커널 'Humming' 도입하기", section "코드 분석" 2).
 * Routing ids outside [0, num_experts) mean "expert not resident in this call"
 *   (one GPU's expert slice) and are skipped, not errors; weights are used as given.
 * Dtypes: bf16 values travel as their uint16_t bit patterns.
 * Alignment: activation, weight, output and workspace buffers are moved 16
 *   bytes at a time and must be 16-byte aligned (W4A16_ERR_INVALID_ARG
 *   otherwise); torch and hipMalloc allocations are.
 */
#ifndef W4A16_MOE_H
#define W4A16_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  W4A16_OK = 0,
  W4A16_ERR_INVALID_ARG = 1, /* null pointer, negative size, inconsistent sizes */
  W4A16_ERR_UNSUPPORTED = 2, /* a valid request outside what the kernels implement */
  W4A16_ERR_CAPACITY = 3,    /* sorted_token_ids buffer shorter than moe_align_capacity */
  W4A16_ERR_WORKSPACE = 4,   /* workspace smaller than the matching *_workspace_bytes */
  W4A16_ERR_HIP = 5,         /* a HIP runtime call failed */
  W4A16_ERR_NOALLOC_LIMIT = 6 /* the call needs more scratch than w4a16_moe_routed_forward_noalloc holds */
} w4a16_status;

/* Layer shape. group_size must be 32; hidden must be a multiple of 64 and
 * intermediate a multiple of 32; 1 <= num_experts <= W4A16_MAX_EXPERTS. */
typedef struct {
  int32_t num_experts;  /* E: experts resident in this call */
  int32_t hidden;       /* H */
  int32_t intermediate; /* I: the gate_up projection has 2*I outputs */
  int32_t group_size;   /* 32 */
} w4a16_moe_shape;

#define W4A16_GROUP_SIZE 32
#define W4A16_MAX_EXPERTS 512
#define W4A16_MAX_TOPK 32
#define W4A16_MAX_ROUTED_EXPERTS 1024

/* Human-readable name of a status code (static string; never NULL). */
const char* w4a16_status_string(int status);

/* ------------------------------------------------------------------------ */
/* Load time: weight repack                                                  */
/* ------------------------------------------------------------------------ */

/* Bytes of the two packed weight buffers written by w4a16_repack: the canonical
 * nibbles and bf16 scales rearranged, plus a second copy of the scales in fp16
 * normalised by a power of two per output channel and the channel exponents
 * (read by the many-tokens-per-expert GEMM), about 1.13x the canonical size. */
int w4a16_packed_bytes(const w4a16_moe_shape* shape, size_t* w13_bytes, size_t* w2_bytes);

/* Rearrange canonical weights into the kernels' layout, once, before inference
 * (the preprocessing step "validate, pad, repack into the target kernel's
 * layout" of the Humming announcement, "Humming: vLLM과 Ant Group, 양자화 추론을
 * 위한 범용 커널 라이브러리 오픈소스 공개", section "워크로드별 튜닝 및 JIT 컴파일";
 * scales stored transposed for contiguous loads, Chord page "그룹 SM90 커널 기법").
 *
 * Canonical input (device):
 *   w13_q  uint8  [E, 2I, H/2]  row r of W13: rows [0, I) gate, rows [I, 2I) up;
 *                               element k in the low nibble of byte k/2 when k is
 *                               even, high nibble otherwise; two's complement int4
 *   w13_s  uint16 [E, 2I, H/32] bf16 scale of (row, group of 32 along H)
 *   w2_q   uint8  [E, H, I/2]   down projection, same nibble convention
 *   w2_s   uint16 [E, H, I/32]
 * Output (device): w13_packed, w2_packed of the sizes from w4a16_packed_bytes.
 * The packed layout is private to the library and may change between versions. */
int w4a16_repack(const w4a16_moe_shape* shape, const uint8_t* w13_q, const uint16_t* w13_s,
                 const uint8_t* w2_q, const uint16_t* w2_s, void* w13_packed, void* w2_packed,
                 void* stream);

/* ------------------------------------------------------------------------ */
/* Token-to-expert alignment                                                 */
/* ------------------------------------------------------------------------ */

/* Length the caller must allocate for sorted_token_ids: T*topk + E*(block_m-1)
 * (each expert can waste at most block_m-1 padding slots). expert_ids then has
 * ceil(capacity / block_m) entries. Returns 0 for invalid arguments. */
size_t moe_align_capacity(int32_t T, int32_t topk, int32_t num_experts, int32_t block_m);

/* Device scratch bytes moe_align needs (0 for small inputs). */
size_t moe_align_workspace_bytes(int32_t T, int32_t topk, int32_t num_experts, int32_t block_m);

/* block_m for a call, from the expected routed tokens per expert (tok_e =
 * T*topk/E_global): a tile sized by tokens-per-expert, not by total tokens
 * (Chord page, "핵심 기여" and "인덱스 커널 기법": tok_e heuristic): 16 up to
 * tok_e 6, 32 up to 40, else 128 (thresholds from a measured sweep of the
 * layer at every block_m over T = 1 .. 8192 on a 48-expert Kimi-K2 slice).
 * Returns 16, 32 or 128 (64 stays available to callers that pass it); 0 for
 * invalid arguments. */
int32_t w4a16_choose_block_m(int32_t T, int32_t topk, int32_t num_experts_local, int32_t num_experts_global);

/* Group the T*topk routed slots by expert, each expert padded to a multiple of
 * block_m, into the over-allocated buffers the GEMMs read (vLLM's
 * moe_align_block_size buffers, Chord page "런타임 고려사항"; the same output
 * set as the FlashInfer Kimi-K3 fused router, page "[flashinfer] FlashInfer,
 * B200 GPU에서 Kimi-K3 MoE 라우터 성능 최적화", section "코드 분석").
 *
 *   topk_ids               device int32 [T, topk]; ids outside [0, E) are skipped
 *   block_m                16, 32, 64 or 128
 *   sorted_token_ids       device int32 [capacity]: flat slot ids t*topk+j grouped
 *                          by expert in ascending slot order; padding and the
 *                          unused tail hold the sentinel T*topk
 *   capacity               >= moe_align_capacity(T, topk, E, block_m)
 *   expert_ids             device int32 [ceil(capacity/block_m)]: expert of each
 *                          block_m-row block, -1 past the used blocks
 *   num_tokens_post_padded device int32 [1]: sum over experts of ceil(count/block_m)*block_m
 *   expert_counts          device int32 [E] or NULL: resident slots per expert
 *   workspace              device, >= moe_align_workspace_bytes(...) bytes (may be
 *                          NULL when that is 0); fully rewritten on every call
 * The result is deterministic and unique (a stable counting sort). */
int moe_align(const int32_t* topk_ids, int32_t T, int32_t topk, int32_t num_experts, int32_t block_m,
              int32_t* sorted_token_ids, int32_t capacity, int32_t* expert_ids,
              int32_t* num_tokens_post_padded, int32_t* expert_counts, void* workspace,
              size_t workspace_bytes, void* stream);

/* moe_align restricted to the experts whose resident slot count c satisfies
 * min_count <= c <= max_count; the other experts are treated exactly like
 * ids outside [0, E) (not resident: no slots, no blocks, count 0). Two calls
 * with complementary ranges split one routing into a light and a heavy set
 * with their own block_m (per-expert tile sizes for skewed routing: Chord
 * page, "인덱스 커널 기법", where the tokens-per-expert count picks the block
 * size). W4A16_ERR_INVALID_ARG for min_count < 0 or max_count < min_count;
 * otherwise as moe_align. */
int moe_align_filtered(const int32_t* topk_ids, int32_t T, int32_t topk, int32_t num_experts, int32_t block_m,
                       int32_t min_count, int32_t max_count, int32_t* sorted_token_ids, int32_t capacity,
                       int32_t* expert_ids, int32_t* num_tokens_post_padded, int32_t* expert_counts,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Both halves of that split in one pass over the ids (per-expert tile sizes
 * chosen by each expert's token count: Chord page, "인덱스 커널 기법"): the
 * heavy set (experts with c >= split_count) at heavy_block_m and the light set
 * (1 <= c < split_count) at light_block_m. The two sets share one sorted array:
 * sorted_token_ids[0, heavy_capacity) is the heavy set's and
 * sorted_token_ids[heavy_capacity, heavy_capacity + light_capacity) the light
 * set's. Each set's sorted ids, expert ids and padded total are bit for bit
 * those of moe_align_filtered with the matching range (expert counts are not
 * written).
 *   split_count      >= 2
 *   heavy_capacity   >= moe_align_capacity(T, topk, E, heavy_block_m)
 *   light_capacity   >= min(moe_align_capacity(T, topk, E, light_block_m),
 *                           E * ceil((split_count - 1) / light_block_m) * light_block_m)
 *   *_expert_ids     device int32 [ceil(*_capacity / *_block_m)]
 *   workspace        as moe_align
 * heavy_capacity + light_capacity must fit int32 (else W4A16_ERR_CAPACITY).
 * W4A16_ERR_INVALID_ARG for split_count < 2 or a missing output; otherwise as
 * moe_align. */
int moe_align_split(const int32_t* topk_ids, int32_t T, int32_t topk, int32_t num_experts, int32_t split_count,
                    int32_t heavy_block_m, int32_t heavy_capacity, int32_t* heavy_expert_ids,
                    int32_t* heavy_num_tokens_post_padded, int32_t light_block_m, int32_t light_capacity,
                    int32_t* light_expert_ids, int32_t* light_num_tokens_post_padded, int32_t* sorted_token_ids,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Router and alignment in one call: the step in front of the layer, with the
 * outputs of the FlashInfer Kimi-K3 fused router (page "[flashinfer]
 * FlashInfer, B200 GPU에서 Kimi-K3 MoE 라우터 성능 최적화", section "코드 분석":
 * logits and bias in; top-k weights and ids, sorted_token_ids, expert_ids,
 * num_tokens_post_padded and the expert counts out). That page gives the
 * interface, not the arithmetic; the routing computed here is:
 *   score[t, e]   = logits[t, e] + bias[e]            (fp32 add; bias may be NULL)
 *   topk_ids[t]   = the topk experts with the highest scores, in descending
 *                   score order; an equal score goes to the lower expert id
 *   topk_weights  = softmax over the chosen raw logits (the bias steers the
 *                   choice only; weights are fp32, not renormalized further)
 * and the alignment is exactly moe_align's over the ids just written. As on
 * the page (section "커널 내부 로직 변경 (추정)"), every counter is set inside
 * the call, so nothing carries over from a previous call.
 *
 *   logits                 device fp32 [T, num_routed_experts], finite (NaN
 *                          logits give unspecified ids, never an out-of-bounds access)
 *   bias                   device fp32 [num_routed_experts], finite, or NULL
 *   num_routed_experts     experts the router chooses among, <= W4A16_MAX_ROUTED_EXPERTS;
 *                          the local slice is ids [0, num_experts) of them
 *   topk                   1 <= topk <= min(num_routed_experts, W4A16_MAX_TOPK)
 *   num_experts            local experts, <= num_routed_experts
 *   topk_ids               device int32 [T, topk], written (global ids)
 *   topk_weights           device fp32 [T, topk], written
 *   sorted_token_ids ...   as for moe_align (same capacity rule, same workspace:
 *   workspace              >= moe_align_workspace_bytes(T, topk, num_experts, block_m))
 * Returns W4A16_ERR_INVALID_ARG for num_routed_experts < num_experts or
 * topk > num_routed_experts, W4A16_ERR_UNSUPPORTED past the limits, and the
 * moe_align codes otherwise. T <= 16 runs as one launch; larger T as a router
 * launch followed by the alignment launches. Deterministic. */
int moe_route_align(const float* logits, const float* bias, int32_t T, int32_t num_routed_experts, int32_t topk,
                    int32_t num_experts, int32_t block_m, int32_t* topk_ids, float* topk_weights,
                    int32_t* sorted_token_ids, int32_t capacity, int32_t* expert_ids,
                    int32_t* num_tokens_post_padded, int32_t* expert_counts, void* workspace,
                    size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* The layer                                                                 */
/* ------------------------------------------------------------------------ */

/* Device scratch bytes of w4a16_moe_forward: the bf16 SiLU-and-mul output
 * h [capacity, I], the fp32 per-slot down outputs y [T*topk, H], and the
 * scratch of the two GEMM stages (w4a16_moe_stage_workspace_bytes). */
size_t w4a16_moe_workspace_bytes(const w4a16_moe_shape* shape, int32_t T, int32_t topk, int32_t block_m);

/* Device scratch bytes of the GEMM stages (one region shared by all of them,
 * since they run one after the other): with block_m = 128 the GEMMs read fp16
 * copies of their activation rows with a power-of-two factor per row, written
 * by w4a16_moe_prepare_x (T rows of x) and w4a16_moe_prepare_h
 * (moe_align_capacity rows of h); 0 for the other block_m values. */
size_t w4a16_moe_stage_workspace_bytes(const w4a16_moe_shape* shape, int32_t T, int32_t topk, int32_t block_m);

/* out[t, :] = bf16( sum_j [0 <= topk_ids[t,j] < E] * topk_weights[t,j] *
 *                    W2[e] . bf16(silu(W13_gate[e] . x[t]) * (W13_up[e] . x[t])) )
 * with e = topk_ids[t, j] and W = int4 * group scale, exactly (Chord page, TL;DR
 * and "핵심 기여": the indexed W4A16 MoE operator; the top-k weight multiply and
 * sum fused as moe_fused_mul_sum, Humming PR page, "왜 이게 좋은가" item 3).
 *
 *   x                  device bf16 [T, H]
 *   topk_ids           device int32 [T, topk] (as given to moe_align)
 *   topk_weights       device fp32 [T, topk]
 *   sorted_token_ids, capacity, expert_ids, num_tokens_post_padded, block_m:
 *                      moe_align's outputs for the same topk_ids and block_m; the
 *                      padded count is read on the device (no host sync)
 *   w13_packed, w2_packed  w4a16_repack's outputs for this shape
 *   out                device bf16 [T, H]; every row is written (0 for tokens
 *                      with no resident expert)
 *   workspace          device, >= w4a16_moe_workspace_bytes(shape, T, topk, block_m)
 * The shard profile is taken from the shapes alone; there is no shard argument
 * (Chord page, "런타임 고려사항"). */
int w4a16_moe_forward(const w4a16_moe_shape* shape, const uint16_t* x, int32_t T, int32_t topk,
                      const int32_t* topk_ids, const float* topk_weights,
                      const int32_t* sorted_token_ids, int32_t capacity, const int32_t* expert_ids,
                      const int32_t* num_tokens_post_padded, int32_t block_m, const void* w13_packed,
                      const void* w2_packed, uint16_t* out, void* workspace, size_t workspace_bytes,
                      void* stream);

/* The stages of w4a16_moe_forward, callable one by one with the same
 * arguments and conventions; forward == prepare_x, gate_up, prepare_h, down,
 * combine. prepare_x, gate_up, prepare_h and down share a scratch region of
 * w4a16_moe_stage_workspace_bytes (may be NULL when that is 0); each call may
 * overwrite it, and the GEMMs read what the preceding prepare call left there.
 *
 * prepare_x / prepare_h: with block_m = 128 the GEMMs run on exact fp16
 *   operands (the weight side is the normalised fp16 scales of the packed
 *   buffer). These stages write the activation side: every x row of a token
 *   with a resident slot (prepare_x) and every real row of h (prepare_h) as
 *   fp16(row * 2^-e) with e chosen per row so that its largest magnitude lands
 *   in [2^14, 2^15), plus e. Exact except for elements more than 2^31 below
 *   their row's largest (fp16 holds a bf16 value exactly down to 2^-17), which
 *   round to the fp16 subnormal grid: an absolute error of at most 2^-39 of the
 *   row's largest element. No-ops for
 *   the other block_m values.
 * gate_up: h[p, c] = bf16(silu(g[p, c]) * g[p, I + c]) for every real row p of
 *   the aligned order (sorted_token_ids[p] < T*topk), g = x[sorted[p]/topk] . W13^T.
 *   h: device bf16 [capacity, I]; padding rows are left untouched.
 * down: y[sorted[p], n] = h[p, :] . W2[e, n, :] for every real row p, in fp32.
 *   y: device fp32 [T*topk, H]; rows of non-resident slots are left untouched.
 * combine: out[t, n] = bf16(sum_j resident(t, j) * topk_weights[t, j] * y[t*topk+j, n]),
 *   summed in fp32 in j order.
 * Stage boundaries follow the layer definition of w4a16_moe_forward (the
 * gate_up GEMM with its fused SiLU-and-mul, the down GEMM, the weighted top-k
 * sum); the prepare stages are this implementation's operand conversion for
 * the many-tokens-per-expert GEMM. */
int w4a16_moe_prepare_x(const w4a16_moe_shape* shape, const uint16_t* x, int32_t T, int32_t topk,
                        const int32_t* topk_ids, int32_t block_m, void* workspace, size_t workspace_bytes,
                        void* stream);
int w4a16_moe_gate_up(const w4a16_moe_shape* shape, const uint16_t* x, int32_t T, int32_t topk,
                      const int32_t* sorted_token_ids, int32_t capacity, const int32_t* expert_ids,
                      const int32_t* num_tokens_post_padded, int32_t block_m, const void* w13_packed,
                      uint16_t* h, void* workspace, size_t workspace_bytes, void* stream);
int w4a16_moe_prepare_h(const w4a16_moe_shape* shape, int32_t T, int32_t topk, const uint16_t* h,
                        const int32_t* sorted_token_ids, int32_t capacity, const int32_t* num_tokens_post_padded,
                        int32_t block_m, void* workspace, size_t workspace_bytes, void* stream);
int w4a16_moe_down(const w4a16_moe_shape* shape, int32_t T, int32_t topk, const uint16_t* h,
                   const int32_t* sorted_token_ids, int32_t capacity, const int32_t* expert_ids,
                   const int32_t* num_tokens_post_padded, int32_t block_m, const void* w2_packed,
                   float* y, void* workspace, size_t workspace_bytes, void* stream);
int w4a16_moe_combine(const w4a16_moe_shape* shape, int32_t T, int32_t topk, const int32_t* topk_ids,
                      const float* topk_weights, const float* y, uint16_t* out, void* stream);

/* The routed layer in one call, alignment included: topk_ids and weights in,
 * out written. The block size comes from the tokens-per-expert rule
 * (w4a16_choose_block_m with num_experts_global). When that rule picks 128
 * (prefill) the experts are split on the device by their resident count:
 * experts with at least w4a16_moe_routed_split(...) slots run in 128-row
 * tiles, lighter ones in 16-row blocks on the weight-streaming GEMMs, so a
 * skewed routing does not pay a mostly empty 128-row tile for every lightly
 * used expert (adaptive per-expert tiles; Chord page, "인덱스 커널 기법": the
 * tile follows the tokens per expert, not the total token count). The result
 * equals w4a16_moe_forward's up to the fp32 summation inside each GEMM.
 *
 *   x, topk_ids, topk_weights, out   as for w4a16_moe_forward
 *   num_experts_global               experts the router chose among (>= num_experts)
 *   workspace   device, >= w4a16_moe_routed_workspace_bytes(shape, T, topk, num_experts_global)
 * Same error codes as w4a16_moe_forward. */
size_t w4a16_moe_routed_workspace_bytes(const w4a16_moe_shape* shape, int32_t T, int32_t topk,
                                        int32_t num_experts_global);
/* The heavy-expert threshold the call uses (slots per expert), 0 when it runs
 * one alignment, -1 for invalid arguments. */
int32_t w4a16_moe_routed_split(const w4a16_moe_shape* shape, int32_t T, int32_t topk, int32_t num_experts_global);
int w4a16_moe_routed_forward(const w4a16_moe_shape* shape, const uint16_t* x, int32_t T, int32_t topk,
                             int32_t num_experts_global, const int32_t* topk_ids, const float* topk_weights,
                             const void* w13_packed, const void* w2_packed, uint16_t* out, void* workspace,
                             size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture
 * that must not allocate, tight serving loops, harnesses that forbid hipMalloc):
 * w4a16_moe_routed_forward with its workspace in a static device array of
 * W4A16_NOALLOC_SCRATCH_BYTES inside the library instead of a caller buffer.
 * The caller still passes inputs and outputs, as for w4a16_moe_routed_forward.
 *
 * Ownership: each GPU the library runs on holds its own copy of the array from
 * the first call on that GPU until the process ends; the call allocates and
 * frees nothing. Every call on one GPU shares that GPU's array, which keeps the
 * last call's contents: calls that overlap on one GPU (several streams, or
 * several host threads with work in flight at once) race on it and must be
 * serialised by the caller. Nothing needs the array cleared between calls.
 * Errors: those of w4a16_moe_routed_forward, plus W4A16_ERR_NOALLOC_LIMIT when
 * w4a16_moe_routed_workspace_bytes(shape, T, topk, num_experts_global) exceeds
 * W4A16_NOALLOC_SCRATCH_BYTES (e.g. decode-sized calls of the Kimi-K2 expert
 * slice fit: 128 tokens x top-8 over 48 of 384 experts need about 37 MiB), and
 * W4A16_ERR_HIP when the array's address cannot be obtained. Bits of the
 * output equal those of w4a16_moe_routed_forward on the same inputs. */
#define W4A16_NOALLOC_SCRATCH_BYTES (64u << 20)
int w4a16_moe_routed_forward_noalloc(const w4a16_moe_shape* shape, const uint16_t* x, int32_t T, int32_t topk,
                                     int32_t num_experts_global, const int32_t* topk_ids, const float* topk_weights,
                                     const void* w13_packed, const void* w2_packed, uint16_t* out, void* stream);

/* ------------------------------------------------------------------------ */
/* Expert-grouped activation layouts                                         */
/* ------------------------------------------------------------------------ */

/* The layer on the contiguous grouped layout of Chord's grouped kernels (Chord
 * page, sections "핵심 기여" and "그룹 SM90 커널 기법": contiguous prefill, every
 * expert's rows padded to a 128-row boundary). No routed ids and no alignment
 * pass: the rows are already grouped.
 *
 *   x          device bf16 [M, H]; M a multiple of 128 (else W4A16_ERR_INVALID_ARG)
 *   m_indices  device int32 [M]: the expert of each row; a value outside
 *              [0, num_experts) marks a padding row. An expert's rows start at a
 *              multiple of 128 and its padding rows follow its live rows, so a
 *              128-row block holds one expert; a live row whose expert differs
 *              from that of its block's first row is treated as padding.
 *   out        device bf16 [M, H], every row written: out[r] = the row's down
 *              output (fp32 accumulation, rounded once to bf16, no routing
 *              weight), zeros for padding rows
 *   workspace  device, >= w4a16_moe_contiguous_workspace_bytes(shape, M)
 * Runs an index stage (which also zeroes the padding rows of out), then the
 * layer's stages with block_m 128 and one slot per row; the down GEMM writes
 * the live rows of out directly. Same error codes as w4a16_moe_forward. */
size_t w4a16_moe_contiguous_workspace_bytes(const w4a16_moe_shape* shape, int32_t M);
int w4a16_moe_contiguous_forward(const w4a16_moe_shape* shape, const uint16_t* x, int32_t M,
                                 const int32_t* m_indices, const void* w13_packed, const void* w2_packed,
                                 uint16_t* out, void* workspace, size_t workspace_bytes, void* stream);

/* block_m for the masked layout: the tokens-per-expert rule of
 * w4a16_choose_block_m applied to expected_m (the rows an expert is expected
 * to hold; Chord page, "그룹 SM90 커널 기법": the block size follows the
 * expected token count), halved until it divides max_m. 0 when max_m is not a
 * positive multiple of 16 or expected_m < 0. */
int32_t w4a16_moe_masked_block_m(int32_t max_m, int32_t expected_m);

/* The layer on the masked grouped layout (Chord page, "그룹 SM90 커널 기법":
 * masked decode reserves a fixed row budget per expert): a graph-friendly
 * decode form whose buffers have a fixed size whatever the routing.
 *
 *   x          device bf16 [E, max_m, H]
 *   max_m      rows per expert, a multiple of block_m (else W4A16_ERR_INVALID_ARG)
 *   masked_m   device int32 [E]: live rows of each expert (rows 0 .. masked_m[e]-1;
 *              values are clamped to [0, max_m])
 *   block_m    16, 32, 64 or 128 (see w4a16_moe_masked_block_m)
 *   out        device bf16 [E, max_m, H], every row written: the row's down
 *              output for live rows, zeros for the others
 *   workspace  device, >= w4a16_moe_masked_workspace_bytes(shape, max_m, block_m)
 * Blocks of block_m rows past an expert's live rows are skipped by the GEMMs;
 * the down GEMM writes the live rows of out directly. Same error codes as
 * w4a16_moe_forward. */
size_t w4a16_moe_masked_workspace_bytes(const w4a16_moe_shape* shape, int32_t max_m, int32_t block_m);
int w4a16_moe_masked_forward(const w4a16_moe_shape* shape, const uint16_t* x, int32_t max_m,
                             const int32_t* masked_m, int32_t block_m, const void* w13_packed, const void* w2_packed,
                             uint16_t* out, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_MOE_H */
