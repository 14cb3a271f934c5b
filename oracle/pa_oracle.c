/*
 * pa_oracle.c -- fp64 CPU oracle for single-token paged decode attention over
 * an fp8-e4m3fn KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code, header or table with the HIP path.
 *
 * What it computes (the plain definition, evaluated in double precision):
 *
 *   For every sequence s, query head h and output dim d, with G = Hq / Hkv,
 *   kv head k = floor(h / G) and n = seq_lens[s] cached tokens:
 *     token t lives in physical block  p_t = block_tables[s][t / 16]
 *                        at slot       j   = t % 16
 *     K_t[e] = fp8(k_cache[p_t][k][e / 16][j][e % 16]) * k_scale
 *     V_t[e] = fp8(v_cache[p_t][k][e][j])              * v_scale
 *     z_t    = scale * sum_e q[s][h][e] * K_t[e]
 *     out[s][h][d] = sum_t exp(z_t - max z) V_t[d] / sum_t exp(z_t - max z)
 *
 * Sources (cited by page title and section):
 *  - vLLM pull request lishuoshuo-amd/vllm #3 (ROCM_ATTN asm decode),
 *    Overview and Details > Layout:
 *    paged fp8 cache with 16-token blocks; K cache laid out as
 *    [blocks, kv_heads, head_size/16, 16, 16], V cache as
 *    [blocks, kv_heads, head_size, 16]; pages addressed by a dense stride.
 *  - API page "vllm.v1.attention.backends.rocm_aiter_unified_attn",
 *    RocmAiterUnifiedAttentionImpl.forward: query [num_tokens, num_heads,
 *    head_size], seqused_k (tokens per sequence), block_table, softmax_scale,
 *    k_descale / v_descale (per-tensor scales multiplied on read).
 *
 * Readings where the pages leave a step open:
 *  - query head h reads kv head floor(h / G) (consecutive heads share);
 *  - fp8 is the OCP e4m3fn format: bias 7, 3 mantissa bits, subnormals
 *    m * 2^-9, largest finite 448, no infinities, S.1111.111 is NaN;
 *  - scales multiply the decoded value;
 *  - seq_lens[s] == 0 gives an all-zero output row;
 *  - tokens at or beyond seq_lens[s] and table entries past
 *    ceil(seq_lens[s] / 16) are never read;
 *  - seq_lens[s] > 16 * max_blocks_per_seq is a caller error (return -3).
 *
 * The split-KV variant (pa_oracle_decode_partitioned) evaluates the same
 * quantity as a log-sum-exp merge of per-partition partial results; it exists
 * to pin that merge formula against the unsplit definition.
 *
 * Per-slot scales (pa_oracle_decode_slot_scales): the same quantity with K_t
 * and V_t dequantised by k_scales[p_t][k][j] and v_scales[p_t][k][j], one fp32
 * scale per (block, kv head, slot) instead of one per tensor (pull request
 * #3, Details > Scale tables: the asm kernel reads [blocks, kv_heads,
 * block_size] tables).
 *
 * Several query tokens per sequence (pa_oracle_attend_multi): sequence s owns
 * query rows cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1, its q_len newest tokens,
 * already in the cache (API page, RocmAiterUnifiedAttentionImpl.forward:
 * cu_seqlens_q / query_start_loc, seqused_k, causal=True; the cache update
 * runs before it).  Reading of the causal mask: query i (0-based) of a sequence
 * with n = seq_lens[s] tokens sits at position n - q_len + i and sees tokens
 * 0 .. n - q_len + i.  q_len > n is a caller error (return -5).
 *
 * Attention options of the unified backend (pa_oracle_attend_ext; API page,
 * RocmAiterUnifiedAttentionImpl.__init__ / forward: sliding_window as
 * window_size, logits_soft_cap as softcap, alibi_slopes, sinks), on top of the
 * several-queries form above.  Readings, for the query at position p of head h:
 *   - window w > 0: it sees tokens max(0, p - w + 1) .. p (w tokens ending at
 *     its own position); w = 0: no window;
 *   - softcap c > 0: the scaled logit z = scale * q.K becomes c * tanh(z / c);
 *   - ALiBi slope a_h: the logit gains a_h * (t - p) (after the softcap); a
 *     per-query constant would not change the result;
 *   - sink s_h: one more softmax term exp(s_h) with no value, so
 *     out = sum_t exp(z_t - M) V_t / (sum_t exp(z_t - M) + exp(s_h - M)),
 *     M = max(max_t z_t, s_h); a query that sees no token gets zeros.
 *
 * Token-row cache layouts (pa_oracle_decode_strided): the same quantity with
 * each token's 128 dims stored contiguously, as the flash-style caches of the
 * API page's unified backend keep them (the forward docstring's
 * [num_blocks, 2, block_size, num_kv_heads, head_size]; _split_kv_cache's
 * views of the packed (blocks, heads, tokens, 2 * head_size) and of the
 * shuffled (2, blocks, tokens, heads, head_size) caches).  With byte strides
 * for block, token and kv head (dims contiguous):
 *   K_t[e] = fp8(k_cache[p_t * block_stride + j * token_stride + k * head_stride + e]) * k_scale
 *   V_t[e] = fp8(v_cache[p_t * block_stride + j * token_stride + k * head_stride + e]) * v_scale
 *
 * Cache write (pa_oracle_cache_write): the step that fills the cache the
 * decode reads (API page, do_kv_cache_update: new tokens' key and value, the
 * two caches, slot_mapping and the per-tensor k/v scales go to the cache
 * writer; pull request #3, Details > Layout, for the page layout).  For every
 * token t with slot_mapping[t] >= 0, block = slot / 16, slot in block = slot % 16:
 *   k_cache[block][kvh][d / 16][slot % 16][d % 16] = fp8(key[t][kvh][d] / k_scale)
 *   v_cache[block][kvh][d][slot % 16]             = fp8(value[t][kvh][d] / v_scale)
 * Readings: the division is done in fp32 (the precision the kernel decides the
 * code in), fp8() rounds to nearest even and saturates to +-448 (infinities
 * too), NaN stays NaN with its sign, and a negative slot means "not cached".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define PA_HEAD_DIM 128
#define PA_BLOCK 16

/* Value of one OCP fp8 e4m3fn byte, from the format's definition. */
double pa_oracle_fp8_e4m3fn(uint8_t b) {
  const int sign = (b >> 7) & 1;
  const int e = (b >> 3) & 0xF;
  const int m = b & 0x7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)m / 8.0, -6); /* subnormal: 0.m * 2^(1 - 7) */
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -mag : mag;
}

/* fp8 e4m3fn code of an fp32 value: nearest, ties to even; magnitudes above
 * 448 (including infinity) saturate to 448; NaN gives S.1111.111. */
uint8_t pa_oracle_fp8_e4m3fn_encode(float y) {
  const uint8_t sign = signbit(y) ? 0x80u : 0u;
  if (isnan(y)) return sign | 0x7Fu;
  const double a = fabs((double)y);
  if (a > 448.0) return sign | 0x7Eu;
  if (a < ldexp(1.0, -6)) {
    /* subnormal range: multiples of 2^-9; q = 8 is the smallest normal, code 0x08 */
    const double q = nearbyint(ldexp(a, 9));
    return sign | (uint8_t)q;
  }
  int e;
  (void)frexp(a, &e);
  e -= 1;                                   /* a = 1.f * 2^e, -6 <= e <= 8 */
  double m = nearbyint((ldexp(a, -e) - 1.0) * 8.0);
  if (m == 8.0) {
    m = 0.0;
    e += 1;
  }
  if (e + 7 > 15 || (e + 7 == 15 && m == 7.0)) return sign | 0x7Eu;
  return sign | (uint8_t)(((e + 7) << 3) | (int)m);
}

/* Value of one bfloat16 (upper half of an IEEE binary32). */
double pa_oracle_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Correctly rounded (nearest, ties to even) bfloat16 of a double. */
uint16_t pa_oracle_bf16_rne(double x) {
  uint16_t sign = signbit(x) ? 0x8000u : 0u;
  double a = fabs(x);
  if (isnan(x)) return 0x7FC0u;
  if (a == 0.0) return sign;
  /* bf16: 8 significant bits, normal exponents -126..127, subnormal step 2^-133 */
  int e;
  (void)frexp(a, &e); /* a = f * 2^e, 0.5 <= f < 1; leading bit weight 2^(e-1) */
  int step_exp = (e - 1) - 7;
  if (step_exp < -133) step_exp = -133;
  double q = nearbyint(ldexp(a, -step_exp)); /* default rounding mode: ties even */
  double r = ldexp(q, step_exp);
  if (r > ldexp(2.0 - ldexp(1.0, -7), 127))
    return sign | 0x7F80u; /* rounds past the largest finite bf16: infinity */
  float f = (float)r;      /* exact: r has at most 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return sign | (uint16_t)(u >> 16);
}

/* Dequantisation scales: one per tensor, or (when the tables are not NULL) one
 * per (block, kv head, slot) from tables [num_blocks][num_kv_heads][16].
 * token_rows != 0 selects the token-row layout with the three byte strides
 * instead of the page layout. */
typedef struct {
  double k_scale, v_scale;
  const float* k_slot;
  const float* v_slot;
  int token_rows;
  int64_t block_stride, token_stride, head_stride;
} scales_t;

/* Gather + dequantise token t of sequence s for kv head k (one row of K and V). */
static void load_token(const uint8_t* k_cache, const uint8_t* v_cache,
                       const int32_t* bt_row, int num_kv_heads, int k, int t,
                       const scales_t* sc, double* K, double* V) {
  const int64_t p = bt_row[t / PA_BLOCK];
  const int j = t % PA_BLOCK;
  double k_scale = sc->k_scale, v_scale = sc->v_scale;
  if (sc->k_slot) {
    k_scale = sc->k_slot[(p * num_kv_heads + k) * PA_BLOCK + j];
    v_scale = sc->v_slot[(p * num_kv_heads + k) * PA_BLOCK + j];
  }
  if (sc->token_rows) {
    const int64_t row = p * sc->block_stride + j * sc->token_stride + k * sc->head_stride;
    for (int e = 0; e < PA_HEAD_DIM; ++e) {
      K[e] = pa_oracle_fp8_e4m3fn(k_cache[row + e]) * k_scale;
      V[e] = pa_oracle_fp8_e4m3fn(v_cache[row + e]) * v_scale;
    }
    return;
  }
  const uint8_t* kpage = k_cache + (p * num_kv_heads + k) * (int64_t)(PA_HEAD_DIM * PA_BLOCK);
  const uint8_t* vpage = v_cache + (p * num_kv_heads + k) * (int64_t)(PA_HEAD_DIM * PA_BLOCK);
  for (int e = 0; e < PA_HEAD_DIM; ++e) {
    /* K page is [head_size/16][16 slots][16 dims]; V page is [head_size][16 slots] */
    K[e] = pa_oracle_fp8_e4m3fn(kpage[(e / 16) * (PA_BLOCK * 16) + j * 16 + (e % 16)]) * k_scale;
    V[e] = pa_oracle_fp8_e4m3fn(vpage[e * PA_BLOCK + j]) * v_scale;
  }
}

static int check_args(int S, int Hq, int Hkv, int W, const int32_t* seq_lens) {
  if (S < 0 || Hq <= 0 || Hkv <= 0 || W < 0) return -1;
  if (Hq % Hkv != 0) return -2;
  for (int s = 0; s < S; ++s)
    if (seq_lens[s] < 0 || seq_lens[s] > PA_BLOCK * W) return -3;
  return 0;
}

/* One output row: query row q_row (bf16 bits) of kv head k against the first
 * n tokens of the sequence whose block-table row is bt_row. */
static void attend_row(const uint16_t* q_row, const uint8_t* k_cache, const uint8_t* v_cache,
                       const int32_t* bt_row, int Hkv, int k, int n, float scale,
                       const scales_t* sc, double* o) {
  double q[PA_HEAD_DIM], K[PA_HEAD_DIM], V[PA_HEAD_DIM];
  for (int e = 0; e < PA_HEAD_DIM; ++e) q[e] = pa_oracle_bf16(q_row[e]);
  for (int d = 0; d < PA_HEAD_DIM; ++d) o[d] = 0.0;
  if (n <= 0) return;
  double* z = (double*)malloc(sizeof(double) * (size_t)n);
  /* logits */
  double zmax = -INFINITY;
  for (int t = 0; t < n; ++t) {
    load_token(k_cache, v_cache, bt_row, Hkv, k, t, sc, K, V);
    double dot = 0.0;
    for (int e = 0; e < PA_HEAD_DIM; ++e) dot += q[e] * K[e];
    z[t] = (double)scale * dot;
    if (z[t] > zmax) zmax = z[t];
  }
  /* softmax-weighted sum of V */
  double den = 0.0;
  for (int t = 0; t < n; ++t) {
    load_token(k_cache, v_cache, bt_row, Hkv, k, t, sc, K, V);
    const double w = exp(z[t] - zmax);
    den += w;
    for (int d = 0; d < PA_HEAD_DIM; ++d) o[d] += w * V[d];
  }
  for (int d = 0; d < PA_HEAD_DIM; ++d) o[d] /= den;
  free(z);
}

/* attend_row with the unified backend's options (window, softcap, ALiBi
 * slope, sink) for the query at position p = n - 1. */
typedef struct {
  int window;
  double softcap;
  double slope;
  int has_sink;
  double sink;
} row_options_t;

static void attend_row_ext(const uint16_t* q_row, const uint8_t* k_cache, const uint8_t* v_cache,
                           const int32_t* bt_row, int Hkv, int k, int n, float scale,
                           const scales_t* sc, const row_options_t* op, double* o) {
  double q[PA_HEAD_DIM], K[PA_HEAD_DIM], V[PA_HEAD_DIM];
  for (int e = 0; e < PA_HEAD_DIM; ++e) q[e] = pa_oracle_bf16(q_row[e]);
  for (int d = 0; d < PA_HEAD_DIM; ++d) o[d] = 0.0;
  const int p = n - 1;
  const int lo = (op->window > 0 && p - op->window + 1 > 0) ? p - op->window + 1 : 0;
  if (n <= 0) return;
  double* z = (double*)malloc(sizeof(double) * (size_t)n);
  /* logits of the visible tokens lo .. p */
  double zmax = op->has_sink ? op->sink : -INFINITY;
  for (int t = lo; t < n; ++t) {
    load_token(k_cache, v_cache, bt_row, Hkv, k, t, sc, K, V);
    double dot = 0.0;
    for (int e = 0; e < PA_HEAD_DIM; ++e) dot += q[e] * K[e];
    double zt = (double)scale * dot;
    if (op->softcap > 0.0) zt = op->softcap * tanh(zt / op->softcap);
    zt += op->slope * (double)(t - p);
    z[t] = zt;
    if (zt > zmax) zmax = zt;
  }
  /* softmax-weighted sum of V, the sink only in the denominator */
  double den = op->has_sink ? exp(op->sink - zmax) : 0.0;
  for (int t = lo; t < n; ++t) {
    load_token(k_cache, v_cache, bt_row, Hkv, k, t, sc, K, V);
    const double w = exp(z[t] - zmax);
    den += w;
    for (int d = 0; d < PA_HEAD_DIM; ++d) o[d] += w * V[d];
  }
  for (int d = 0; d < PA_HEAD_DIM; ++d) o[d] /= den;
  free(z);
}

static int decode_impl(const uint16_t* q_bits, const uint8_t* k_cache, const uint8_t* v_cache,
                       const int32_t* block_tables, const int32_t* seq_lens, int S, int Hq,
                       int Hkv, int W, float scale, const scales_t* sc, double* out,
                       int num_threads) {
  int rc = check_args(S, Hq, Hkv, W, seq_lens);
  if (rc) return rc;
  const int G = Hq / Hkv;
  (void)num_threads;
#pragma omp parallel for collapse(2) schedule(dynamic, 1) num_threads(num_threads > 0 ? num_threads : 1)
  for (int s = 0; s < S; ++s)
    for (int h = 0; h < Hq; ++h)
      attend_row(q_bits + ((int64_t)s * Hq + h) * PA_HEAD_DIM, k_cache, v_cache,
                 block_tables + (int64_t)s * W, Hkv, h / G, seq_lens[s], scale, sc,
                 out + ((int64_t)s * Hq + h) * PA_HEAD_DIM);
  return 0;
}

/*
 * out: [S][Hq][128] doubles.  q_bits: bf16 bit patterns [S][Hq][128].
 * Returns 0, or a negative code for bad arguments (nothing is written then).
 */
int pa_oracle_decode(const uint16_t* q_bits, const uint8_t* k_cache,
                     const uint8_t* v_cache, const int32_t* block_tables,
                     const int32_t* seq_lens, int S, int Hq, int Hkv, int W,
                     float scale, float k_scale, float v_scale, double* out,
                     int num_threads) {
  const scales_t sc = {k_scale, v_scale, NULL, NULL};
  return decode_impl(q_bits, k_cache, v_cache, block_tables, seq_lens, S, Hq, Hkv, W, scale, &sc,
                     out, num_threads);
}

/* pa_oracle_decode over a token-row cache layout (byte strides; dims contiguous). */
int pa_oracle_decode_strided(const uint16_t* q_bits, const uint8_t* k_cache,
                             const uint8_t* v_cache, int64_t block_stride, int64_t token_stride,
                             int64_t head_stride, const int32_t* block_tables,
                             const int32_t* seq_lens, int S, int Hq, int Hkv, int W, float scale,
                             float k_scale, float v_scale, double* out, int num_threads) {
  if (block_stride <= 0 || token_stride <= 0 || head_stride <= 0) return -4;
  const scales_t sc = {k_scale, v_scale, NULL, NULL, 1, block_stride, token_stride, head_stride};
  return decode_impl(q_bits, k_cache, v_cache, block_tables, seq_lens, S, Hq, Hkv, W, scale, &sc,
                     out, num_threads);
}

/* pa_oracle_decode with per-slot scale tables [num_blocks][Hkv][16] (fp32). */
int pa_oracle_decode_slot_scales(const uint16_t* q_bits, const uint8_t* k_cache,
                                 const uint8_t* v_cache, const int32_t* block_tables,
                                 const int32_t* seq_lens, int S, int Hq, int Hkv, int W,
                                 float scale, const float* k_scales, const float* v_scales,
                                 double* out, int num_threads) {
  const scales_t sc = {1.0, 1.0, k_scales, v_scales};
  return decode_impl(q_bits, k_cache, v_cache, block_tables, seq_lens, S, Hq, Hkv, W, scale, &sc,
                     out, num_threads);
}

/*
 * Same quantity, computed as independent partitions followed by a log-sum-exp
 * merge.  The partitions cut the block-table row, as a launch plan made from
 * shapes alone must (it cannot see seq_lens): partition p covers tokens
 * p * tokens_per_part .. (p + 1) * tokens_per_part - 1 of the 16 * W a row can
 * address, so a context shorter than the row leaves the trailing partitions
 * without a token.
 *   partition p with tokens: m_p = max z,  l_p = sum exp(z - m_p),
 *                            a_p[d] = sum exp(z - m_p) V[d];
 *   partition p without tokens: m_p = -inf, l_p = 0, a_p = 0 (empty);
 *   merge:  M = max over the non-empty partitions of m_p,  w_p = exp(m_p - M),
 *           out = sum_p w_p a_p / sum_p w_p l_p, over the non-empty partitions
 *           only (an empty one would need exp(-inf - M), and -inf - (-inf) where
 *           every partition is empty; a context of no tokens gives zeros).
 * empty_parts (may be NULL) receives the number of empty partitions formed
 * over all (sequence, head) rows.
 */
int pa_oracle_decode_partitioned(const uint16_t* q_bits, const uint8_t* k_cache,
                                 const uint8_t* v_cache, const int32_t* block_tables,
                                 const int32_t* seq_lens, int S, int Hq, int Hkv, int W,
                                 float scale, float k_scale, float v_scale,
                                 int tokens_per_part, double* out, int64_t* empty_parts) {
  int rc = check_args(S, Hq, Hkv, W, seq_lens);
  if (rc) return rc;
  if (tokens_per_part <= 0) return -4;
  const int G = Hq / Hkv;
  const scales_t sc = {k_scale, v_scale, NULL, NULL};
  const int nparts = (PA_BLOCK * W + tokens_per_part - 1) / tokens_per_part;
  int64_t empty = 0;
  for (int s = 0; s < S; ++s) {
    for (int h = 0; h < Hq; ++h) {
      const int n = seq_lens[s];
      const int k = h / G;
      double* o = out + ((int64_t)s * Hq + h) * PA_HEAD_DIM;
      double q[PA_HEAD_DIM], K[PA_HEAD_DIM], V[PA_HEAD_DIM];
      for (int e = 0; e < PA_HEAD_DIM; ++e)
        q[e] = pa_oracle_bf16(q_bits[((int64_t)s * Hq + h) * PA_HEAD_DIM + e]);
      for (int d = 0; d < PA_HEAD_DIM; ++d) o[d] = 0.0;
      double* m = (double*)malloc(sizeof(double) * (size_t)(nparts > 0 ? nparts : 1));
      double* l = (double*)malloc(sizeof(double) * (size_t)(nparts > 0 ? nparts : 1));
      double* a = (double*)calloc((size_t)(nparts > 0 ? nparts : 1) * PA_HEAD_DIM, sizeof(double));
      const int32_t* bt_row = block_tables + (int64_t)s * W;
      for (int p = 0; p < nparts; ++p) {
        const int t0 = p * tokens_per_part;
        const int t1 = (t0 + tokens_per_part < n) ? t0 + tokens_per_part : n;
        m[p] = -INFINITY;
        l[p] = 0.0;
        if (t0 >= t1) {
          ++empty;
          continue;
        }
        double zmax = -INFINITY;
        for (int t = t0; t < t1; ++t) {
          load_token(k_cache, v_cache, bt_row, Hkv, k, t, &sc, K, V);
          double dot = 0.0;
          for (int e = 0; e < PA_HEAD_DIM; ++e) dot += q[e] * K[e];
          double zt = (double)scale * dot;
          if (zt > zmax) zmax = zt;
        }
        m[p] = zmax;
        for (int t = t0; t < t1; ++t) {
          load_token(k_cache, v_cache, bt_row, Hkv, k, t, &sc, K, V);
          double dot = 0.0;
          for (int e = 0; e < PA_HEAD_DIM; ++e) dot += q[e] * K[e];
          const double w = exp((double)scale * dot - zmax);
          l[p] += w;
          for (int d = 0; d < PA_HEAD_DIM; ++d) a[(int64_t)p * PA_HEAD_DIM + d] += w * V[d];
        }
      }
      double M = -INFINITY;
      for (int p = 0; p < nparts; ++p)
        if (l[p] > 0.0 && m[p] > M) M = m[p];
      double den = 0.0;
      for (int p = 0; p < nparts; ++p) {
        if (l[p] == 0.0) continue; /* empty partition: skipped */
        const double w = exp(m[p] - M);
        den += w * l[p];
        for (int d = 0; d < PA_HEAD_DIM; ++d) o[d] += w * a[(int64_t)p * PA_HEAD_DIM + d];
      }
      if (den > 0.0)
        for (int d = 0; d < PA_HEAD_DIM; ++d) o[d] /= den;
      free(m);
      free(l);
      free(a);
    }
  }
  if (empty_parts) *empty_parts = empty;
  return 0;
}

/*
 * key, value: bf16 bit patterns, token t / kv head k / dim d at
 * [t * key_stride + k * 128 + d] (value_stride likewise).  Returns 0, or -3 if a
 * slot points past the caches (nothing is written for that call then).
 */
int pa_oracle_cache_write(const uint16_t* key, const uint16_t* value, int64_t key_stride,
                          int64_t value_stride, uint8_t* k_cache, uint8_t* v_cache,
                          const int64_t* slot_mapping, int T, int Hkv, int64_t num_blocks,
                          float k_scale, float v_scale) {
  for (int t = 0; t < T; ++t)
    if (slot_mapping[t] >= num_blocks * PA_BLOCK) return -3;
  for (int t = 0; t < T; ++t) {
    const int64_t slot = slot_mapping[t];
    if (slot < 0) continue;
    const int64_t block = slot / PA_BLOCK;
    const int j = (int)(slot % PA_BLOCK);
    for (int k = 0; k < Hkv; ++k) {
      uint8_t* kpage = k_cache + (block * Hkv + k) * (int64_t)(PA_HEAD_DIM * PA_BLOCK);
      uint8_t* vpage = v_cache + (block * Hkv + k) * (int64_t)(PA_HEAD_DIM * PA_BLOCK);
      for (int d = 0; d < PA_HEAD_DIM; ++d) {
        const float xk = (float)pa_oracle_bf16(key[t * key_stride + k * PA_HEAD_DIM + d]);
        const float xv = (float)pa_oracle_bf16(value[t * value_stride + k * PA_HEAD_DIM + d]);
        kpage[(d / 16) * (PA_BLOCK * 16) + j * 16 + (d % 16)] = pa_oracle_fp8_e4m3fn_encode(xk / k_scale);
        vpage[d * PA_BLOCK + j] = pa_oracle_fp8_e4m3fn_encode(xv / v_scale);
      }
    }
  }
  return 0;
}

/*
 * q_bits: bf16 [T][Hq][128] with T = cu_seqlens_q[S]; out: [T][Hq][128] doubles.
 */
int pa_oracle_attend_multi(const uint16_t* q_bits, const int32_t* cu_seqlens_q,
                           const uint8_t* k_cache, const uint8_t* v_cache,
                           const int32_t* block_tables, const int32_t* seq_lens, int S, int Hq,
                           int Hkv, int W, float scale, float k_scale, float v_scale, double* out,
                           int num_threads) {
  int rc = check_args(S, Hq, Hkv, W, seq_lens);
  if (rc) return rc;
  if (cu_seqlens_q[0] != 0) return -5;
  for (int s = 0; s < S; ++s) {
    const int q_len = cu_seqlens_q[s + 1] - cu_seqlens_q[s];
    if (q_len < 0 || q_len > seq_lens[s]) return -5;
  }
  const int G = Hq / Hkv;
  const scales_t sc = {k_scale, v_scale, NULL, NULL};
  (void)num_threads;
#pragma omp parallel for schedule(dynamic, 1) num_threads(num_threads > 0 ? num_threads : 1)
  for (int s = 0; s < S; ++s) {
    const int q0 = cu_seqlens_q[s];
    const int q_len = cu_seqlens_q[s + 1] - q0;
    for (int i = 0; i < q_len; ++i) {
      const int visible = seq_lens[s] - q_len + i + 1;
      for (int h = 0; h < Hq; ++h)
        attend_row(q_bits + ((int64_t)(q0 + i) * Hq + h) * PA_HEAD_DIM, k_cache, v_cache,
                   block_tables + (int64_t)s * W, Hkv, h / G, visible, scale, &sc,
                   out + ((int64_t)(q0 + i) * Hq + h) * PA_HEAD_DIM);
    }
  }
  return 0;
}

/*
 * pa_oracle_attend_multi with the unified backend's options: sliding_window
 * (0 = none), softcap (0 = none), alibi_slopes [Hq] or NULL, sinks [Hq] or NULL.
 */
int pa_oracle_attend_ext(const uint16_t* q_bits, const int32_t* cu_seqlens_q,
                         const uint8_t* k_cache, const uint8_t* v_cache,
                         const int32_t* block_tables, const int32_t* seq_lens, int S, int Hq,
                         int Hkv, int W, float scale, float k_scale, float v_scale,
                         int sliding_window, float softcap, const float* alibi_slopes,
                         const float* sinks, double* out, int num_threads) {
  int rc = check_args(S, Hq, Hkv, W, seq_lens);
  if (rc) return rc;
  if (cu_seqlens_q[0] != 0 || sliding_window < 0 || !(softcap >= 0.0f)) return -5;
  for (int s = 0; s < S; ++s) {
    const int q_len = cu_seqlens_q[s + 1] - cu_seqlens_q[s];
    if (q_len < 0 || q_len > seq_lens[s]) return -5;
  }
  const int G = Hq / Hkv;
  const scales_t sc = {k_scale, v_scale, NULL, NULL};
  (void)num_threads;
#pragma omp parallel for schedule(dynamic, 1) num_threads(num_threads > 0 ? num_threads : 1)
  for (int s = 0; s < S; ++s) {
    const int q0 = cu_seqlens_q[s];
    const int q_len = cu_seqlens_q[s + 1] - q0;
    for (int i = 0; i < q_len; ++i) {
      const int visible = seq_lens[s] - q_len + i + 1;
      for (int h = 0; h < Hq; ++h) {
        row_options_t op;
        op.window = sliding_window;
        op.softcap = softcap;
        op.slope = alibi_slopes ? (double)alibi_slopes[h] : 0.0;
        op.has_sink = sinks != NULL;
        op.sink = sinks ? (double)sinks[h] : 0.0;
        attend_row_ext(q_bits + ((int64_t)(q0 + i) * Hq + h) * PA_HEAD_DIM, k_cache, v_cache,
                       block_tables + (int64_t)s * W, Hkv, h / G, visible, scale, &sc, &op,
                       out + ((int64_t)(q0 + i) * Hq + h) * PA_HEAD_DIM);
      }
    }
  }
  return 0;
}
