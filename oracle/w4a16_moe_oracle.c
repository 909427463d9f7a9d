/*
 * CPU oracle for the W4A16 fused mixture-of-experts layer.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, plain reference that the
 * GPU library is checked against. Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may build, load or call it. It shares no code,
 * header, table or helper with the GPU library, and the library never calls it.
 *
 * What it computes, and where each step comes from:
 *
 *  - moe_align: the alignment buffers named on the FlashInfer Kimi-K3 fused
 *    router page ("[flashinfer] FlashInfer, B200 GPU에서 Kimi-K3 MoE 라우터 성능
 *    최적화", section "코드 분석", the arg_plan of the new 1-token kernel:
 *    sorted_token_ids, expert_ids, num_tokens_post_padded, expert_counts), padded
 *    to block_m (same page, benchmark table with block_m 8 and 16), and consumed
 *    from an over-allocated buffer (Chord page, "vLLM 및 Novita AI, Kimi K2.x용 더
 *    빠른 INT4 MoE 커널 출시: Chord", section "런타임 고려사항"). The pages give no
 *    ordering rule; this oracle takes the plainest one, a stable counting sort:
 *    slots of one expert appear in ascending flat slot index t*topk+j. Padding
 *    slots hold the sentinel T*topk, unused block entries hold -1, experts with
 *    no slot get no block, and ids outside [0, E) are not resident and skipped.
 *
 *  - dequant: group-32 INT4 weights with BF16 group scales, "W4A16 group-scale
 *    format" (Chord page, section "vLLM과의 통합"; group-32 key in
 *    "런타임 고려사항"). Symmetric: a weight is its signed 4-bit integer times its
 *    group's scale (no zero point), two's complement nibbles, element k of a row
 *    in the low nibble of byte k/2 when k is even. The product q*s is formed in
 *    fp32, where it is exact.
 *
 *  - layer: per token and per resident expert slot, g = x . W13^T (rows [0, I)
 *    gate, rows [I, 2I) up), h = bf16_rne(silu(gate) * up), y = h . W2^T, and
 *    the combine out[t] = sum_j w[t, j] * y_j (Humming PR page, "[vllm] vLLM에
 *    고성능 JIT 양자화 커널 'Humming' 도입하기", section "왜 이게 좋은가" item 3:
 *    the top-k weight multiply fused with the sum). All sums are in fp64; h is
 *    rounded to bf16 because it is the BF16 activation of the down projection
 *    (W4A16 = INT4 weights, BF16 activations, Chord page TL;DR). The per-slot
 *    outputs y stay unrounded.
 *
 *  - route_topk: the router in front of the alignment, fused with it on the
 *    FlashInfer Kimi-K3 page (same section: the kernel takes logits and a bias
 *    and writes topk_weights and topk_ids next to the alignment buffers; its
 *    1-token cell ranks the winners of every token). The page does not define
 *    the scoring; this oracle takes the plain reading: the score of expert e is
 *    the fp32 sum logit + bias[e] (no bias: the logit), the top k scores are
 *    taken in a stable descending order (equal scores: lower id first), and the
 *    weights are the softmax over the k chosen raw logits (the bias steers the
 *    choice only). The weights are computed in fp64.
 *
 * Parity pins for every function here live in tests/test_oracle_*.py: brute
 * force on tiny inputs, closed forms (permutation / constant / zero weights,
 * one-hot routing), invariants (scale doubling, expert-slice and
 * intermediate-slice additivity, relabelling, token permutation) and a
 * hand-worked alignment example.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* bf16 bit pattern -> float: a bf16 is the top half of an fp32. */
static float bf16_bits_to_float(uint16_t b) {
  uint32_t u = ((uint32_t)b) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* Round a double to the nearest bf16 value (ties to even), returned as a
 * double. bf16 has 8 significant bits, exponent range of fp32, subnormals
 * down to 2^-133. Rounding is done once, directly from the double. */
double oracle_round_bf16(double d) {
  if (d == 0.0 || isnan(d) || isinf(d)) return d;
  int e;
  (void)frexp(d, &e);           /* d = m * 2^e, 0.5 <= |m| < 1 */
  int q = e - 8;                /* ulp exponent for 8 significant bits */
  if (q < -133) q = -133;       /* bf16 subnormal spacing */
  double scaled = ldexp(d, -q); /* exact: power-of-two scaling */
  double r = nearbyint(scaled); /* default rounding mode: nearest, ties even */
  double out = ldexp(r, q);
  /* largest finite bf16 is (2 - 2^-7) * 2^127 */
  if (fabs(out) > ldexp(255.0, 120)) out = copysign(INFINITY, d);
  return out;
}

/* Decode one signed 4-bit code (two's complement). */
static int decode_nibble(unsigned n) { return (n & 8u) ? (int)n - 16 : (int)n; }

/* Signed integer weight at (row r, column k) of a [N, K/2] packed matrix. */
static int weight_int(const uint8_t* q, int K, long r, int k) {
  uint8_t byte = q[r * (long)(K / 2) + k / 2];
  unsigned n = (k % 2 == 0) ? (byte & 0x0Fu) : (byte >> 4);
  return decode_nibble(n);
}

/* Dequantize a [N, K] matrix: w[r, k] = float(q[r, k]) * float(s[r, k / 32]),
 * exact in fp32. q is [N, K/2] bytes, s is [N, K/32] bf16 bits. */
void oracle_dequant(const uint8_t* q, const uint16_t* s, int N, int K, float* w) {
  for (long r = 0; r < N; ++r)
    for (int k = 0; k < K; ++k)
      w[r * K + k] = (float)weight_int(q, K, r, k) * bf16_bits_to_float(s[r * (long)(K / 32) + k / 32]);
}

/* Stable counting-sort alignment. Returns 0 on success, -1 if the output
 * buffers are too small. expert_ids has ceil(capacity / block_m) entries. */
int oracle_moe_align(const int32_t* topk_ids, int T, int topk, int E, int block_m,
                     int32_t* sorted_token_ids, int capacity, int32_t* expert_ids,
                     int32_t* num_tokens_post_padded, int32_t* expert_counts) {
  long n = (long)T * topk;
  long* count = (long*)calloc((size_t)E + 1, sizeof(long));
  long* offset = (long*)calloc((size_t)E + 1, sizeof(long));
  long* cursor = (long*)calloc((size_t)E + 1, sizeof(long));
  if (!count || !offset || !cursor) { free(count); free(offset); free(cursor); return -1; }

  for (long i = 0; i < n; ++i) {
    int e = topk_ids[i];
    if (e >= 0 && e < E) count[e] += 1;
  }
  offset[0] = 0;
  for (int e = 0; e < E; ++e) {
    long padded = ((count[e] + block_m - 1) / block_m) * block_m;
    offset[e + 1] = offset[e] + padded;
  }
  long total = offset[E];
  if (total > capacity) { free(count); free(offset); free(cursor); return -1; }

  for (long p = 0; p < capacity; ++p) sorted_token_ids[p] = (int32_t)n; /* sentinel */
  for (long i = 0; i < n; ++i) {
    int e = topk_ids[i];
    if (e >= 0 && e < E) {
      sorted_token_ids[offset[e] + cursor[e]] = (int32_t)i;
      cursor[e] += 1;
    }
  }
  long nblocks = ((long)capacity + block_m - 1) / block_m;
  for (long b = 0; b < nblocks; ++b) expert_ids[b] = -1;
  for (int e = 0; e < E; ++e)
    for (long b = offset[e] / block_m; b < offset[e + 1] / block_m; ++b) expert_ids[b] = e;
  *num_tokens_post_padded = (int32_t)total;
  if (expert_counts)
    for (int e = 0; e < E; ++e) expert_counts[e] = (int32_t)count[e];
  free(count); free(offset); free(cursor);
  return 0;
}

/*
 * The layer for a chosen list of tokens (all of them, or a sample).
 *
 * x             bf16 bits [T, H]
 * topk_ids      int32 [T, topk]      ids outside [0, E) are not resident
 * topk_weights  fp32 [T, topk]       used as given (no renormalization)
 * w13_q, w13_s  [E, 2I, H/2] bytes, [E, 2I, H/32] bf16 bits
 * w2_q,  w2_s   [E, H, I/2] bytes,   [E, H, I/32] bf16 bits
 * tokens        int32 [n_tokens]     which rows of the output to compute
 * round_h       1: h rounded to bf16 (the layer); 0: h kept in fp64 (diagnostic)
 * out           fp64 [n_tokens, H]
 *
 * Tokens are independent, so they are spread over OpenMP threads.
 */
void oracle_moe_layer(const uint16_t* x, int T, int H, int I, int E, int topk,
                      const int32_t* topk_ids, const float* topk_weights,
                      const uint8_t* w13_q, const uint16_t* w13_s,
                      const uint8_t* w2_q, const uint16_t* w2_s,
                      const int32_t* tokens, int n_tokens, int round_h, double* out) {
  (void)T;
  const long w13_rows = 2L * I;
  const long w13_q_expert = w13_rows * (H / 2), w13_s_expert = w13_rows * (H / 32);
  const long w2_q_expert = (long)H * (I / 2), w2_s_expert = (long)H * (I / 32);

#pragma omp parallel for schedule(dynamic, 1)
  for (int ti = 0; ti < n_tokens; ++ti) {
    const long t = tokens[ti];
    double* acc = out + (long)ti * H;
    double* g = (double*)malloc(sizeof(double) * (size_t)w13_rows);
    double* h = (double*)malloc(sizeof(double) * (size_t)I);
    double* xt = (double*)malloc(sizeof(double) * (size_t)H);
    for (int n = 0; n < H; ++n) acc[n] = 0.0;
    for (int k = 0; k < H; ++k) xt[k] = (double)bf16_bits_to_float(x[t * H + k]);

    for (int j = 0; j < topk; ++j) {
      int e = topk_ids[t * topk + j];
      if (e < 0 || e >= E) continue;
      const uint8_t* q13 = w13_q + e * w13_q_expert;
      const uint16_t* s13 = w13_s + e * w13_s_expert;
      const uint8_t* q2 = w2_q + e * w2_q_expert;
      const uint16_t* s2 = w2_s + e * w2_s_expert;

      /* gate_up projection: g[c] = sum_k x[k] * w13[c, k] */
      for (long c = 0; c < w13_rows; ++c) {
        double sum = 0.0;
        for (int k = 0; k < H; ++k) {
          float w = (float)weight_int(q13, H, c, k) * bf16_bits_to_float(s13[c * (H / 32) + k / 32]);
          sum += xt[k] * (double)w;
        }
        g[c] = sum;
      }
      /* SiLU-and-mul: gate is rows [0, I), up is rows [I, 2I) */
      for (int c = 0; c < I; ++c) {
        double gate = g[c], up = g[I + c];
        double a = gate / (1.0 + exp(-gate)) * up;
        h[c] = round_h ? oracle_round_bf16(a) : a;
      }
      /* down projection and weighted combine */
      double wt = (double)topk_weights[t * topk + j];
      for (long n = 0; n < H; ++n) {
        double y = 0.0;
        for (int c = 0; c < I; ++c) {
          float w = (float)weight_int(q2, I, n, c) * bf16_bits_to_float(s2[n * (I / 32) + c / 32]);
          y += h[c] * (double)w;
        }
        acc[n] += wt * y;
      }
    }
    free(g); free(h); free(xt);
  }
}

/* Router: ids [T, topk] and weights [T, topk] (fp64) from logits [T, Eg]
 * (fp32) and an optional bias [Eg] (fp32, NULL = none). Selection on the fp32
 * score logit + bias, largest first, equal scores by lower id; weights =
 * softmax over the chosen raw logits, in fp64. Returns 0, or -1 if topk is
 * not in [1, Eg]. */
int oracle_route_topk(const float* logits, const float* bias, int T, int Eg, int topk, int32_t* ids,
                      double* weights) {
  if (topk < 1 || topk > Eg) return -1;
  char* taken = (char*)malloc((size_t)Eg);
  for (int t = 0; t < T; ++t) {
    const float* lg = logits + (size_t)t * Eg;
    memset(taken, 0, (size_t)Eg);
    for (int j = 0; j < topk; ++j) {
      int best = -1;
      float best_score = 0.0f;
      for (int e = 0; e < Eg; ++e) {
        if (taken[e]) continue;
        const float score = bias ? lg[e] + bias[e] : lg[e];
        if (best < 0 || score > best_score) {  /* strict: an equal score keeps the lower id */
          best = e;
          best_score = score;
        }
      }
      taken[best] = 1;
      ids[(size_t)t * topk + j] = best;
    }
    double mx = -INFINITY;
    for (int j = 0; j < topk; ++j) {
      const double v = lg[ids[(size_t)t * topk + j]];
      if (v > mx) mx = v;
    }
    double sum = 0.0;
    for (int j = 0; j < topk; ++j) sum += exp((double)lg[ids[(size_t)t * topk + j]] - mx);
    for (int j = 0; j < topk; ++j)
      weights[(size_t)t * topk + j] = exp((double)lg[ids[(size_t)t * topk + j]] - mx) / sum;
  }
  free(taken);
  return 0;
}

/* Number of OpenMP threads the layer would use (for reporting). */
int oracle_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads the next layer calls use (n >= 1; for timing the baseline on one core). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  extern void omp_set_num_threads(int);
  omp_set_num_threads(n < 1 ? 1 : n);
#else
  (void)n;
#endif
}
