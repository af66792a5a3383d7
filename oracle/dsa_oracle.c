/*
 * CPU oracle for the selected-index NoPE MLA paged decode.
 *
 * TEST INFRASTRUCTURE ONLY: used by tests/, the smoke check and the
 * benchmark's CPU baseline, never by the product path. Independent of the HIP
 * library (no shared code, headers, tables or generated constants).
 *
 * Written from the definition of the operation in double precision, one row
 * and one head at a time. Page citations use:
 *   [attend]   page "spark_model/layers/glm5next_dsa/attend.rs"
 *   [decode_k] page "metrale_model_arch/glm5next_dsa/layer/decode_k.rs"
 *   [build]    page "spark_model/layers/glm5next_dsa/build.rs"
 */
#include "dsa_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* OCP 8-bit floating point, E4M3FN variant. value = (-1)^s * 2^(e-7) * (1 + m/8)
 * for e > 0, (-1)^s * 2^-6 * (m/8) for e == 0; e == 15 with m == 7 is NaN. */
double dsa_oracle_fp8_e4m3fn(uint8_t code) {
  int sign = (code >> 7) & 1;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double mag;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    mag = ldexp((double)m / 8.0, -6);
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -mag : mag;
}

/* bfloat16 is the top 16 bits of an IEEE binary32. */
double dsa_oracle_bf16(uint16_t bits) {
  uint32_t w = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

static int cmp_i32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/* [attend] module doc, "Why this is not the masked kernel": the gather equals
 * dense attention under a pure set-membership mask, so the row's selection is
 * a set. Holes (-1, and by extension every negative id) and ids past the
 * row's valid length select nothing; repeats count once. Computed the plain
 * way: keep the valid ids, sort them, drop repeats. */
int32_t dsa_oracle_select_row(const int32_t* sel, int32_t width,
                              int32_t seq_len, int32_t* out_ids) {
  int32_t n = 0, u = 0;
  for (int32_t j = 0; j < width; ++j) {
    int32_t t = sel[j];
    if (t >= 0 && t < seq_len) out_ids[n++] = t;
  }
  qsort(out_ids, (size_t)n, sizeof(int32_t), cmp_i32);
  for (int32_t i = 0; i < n; ++i)
    if (i == 0 || out_ids[i] != out_ids[i - 1]) out_ids[u++] = out_ids[i];
  return u;
}

/* [decode_k] slot of a position: physical page from the block table at
 * position / block_size, then position mod block_size inside the page; a
 * page is cache_stride_bytes long and a token is kv_lora_rank FP8 bytes
 * ([decode_k] DsaDecodePaging construction; [attend] single latent KV head). */
uint64_t dsa_oracle_token_offset(const int32_t* bt_row, int32_t t,
                                 int32_t block_size,
                                 uint64_t cache_stride_bytes,
                                 int32_t kv_lora_rank) {
  int64_t page = bt_row[t / block_size];
  int64_t slot_in_page = t % block_size;
  return (uint64_t)page * cache_stride_bytes +
         (uint64_t)slot_in_page * (uint64_t)kv_lora_rank;
}

int32_t dsa_oracle_max_threads(void) {
#ifdef _OPENMP
  return (int32_t)omp_get_max_threads();
#else
  return 1;
#endif
}

/* One (row, head): scores against the dequantised token rows (all Dqk
 * bytes), softmax, weighted sum of the first Dv bytes of the same rows read
 * as V ([attend] DsaDecodeInputs: K and V are the same latent buffer,
 * dequantised with k_scale and v_scale; the output stays in the latent space,
 * which [build] o_absorb consumes). NoPE tokens have Dqk == Dv. */
static void decode_one_head(int32_t Dqk, int32_t Dv, int32_t n, const uint64_t* offs,
                            double sm_scale, double k_scale, double v_scale,
                            const uint16_t* q_head, const uint8_t* k_cache,
                            const uint8_t* v_cache, double* s, double* o) {
  for (int32_t d = 0; d < Dv; ++d) o[d] = 0.0;
  if (n == 0) return; /* nothing selected: the output row is zero */

  double m = -INFINITY;
  for (int32_t i = 0; i < n; ++i) {
    const uint8_t* krow = k_cache + offs[i];
    double dot = 0.0;
    for (int32_t d = 0; d < Dqk; ++d)
      dot += dsa_oracle_bf16(q_head[d]) *
             (k_scale * dsa_oracle_fp8_e4m3fn(krow[d]));
    s[i] = sm_scale * dot;
    if (s[i] > m) m = s[i];
  }
  double l = 0.0;
  for (int32_t i = 0; i < n; ++i) {
    s[i] = exp(s[i] - m); /* p_i, reusing the score buffer */
    l += s[i];
  }
  for (int32_t i = 0; i < n; ++i) {
    const uint8_t* vrow = v_cache + offs[i];
    for (int32_t d = 0; d < Dv; ++d)
      o[d] += s[i] * (v_scale * dsa_oracle_fp8_e4m3fn(vrow[d]));
  }
  for (int32_t d = 0; d < Dv; ++d) o[d] /= l;
}

int dsa_oracle_decode(int32_t rows, int32_t heads, int32_t kv_lora_rank,
                      int32_t width, int32_t block_size, int32_t bt_stride,
                      uint64_t cache_stride_bytes, double sm_scale,
                      double k_scale, double v_scale,
                      const uint16_t* q, const uint8_t* k_cache,
                      const uint8_t* v_cache, const int32_t* block_tables,
                      const int32_t* seq_lens, const int32_t* sel,
                      double* out, int32_t num_threads) {
  return dsa_oracle_decode_qkv(rows, heads, kv_lora_rank, kv_lora_rank, width,
                               block_size, bt_stride, cache_stride_bytes,
                               sm_scale, k_scale, v_scale, q, k_cache, v_cache,
                               block_tables, seq_lens, sel, out, num_threads);
}

int dsa_oracle_decode_qkv(int32_t rows, int32_t heads, int32_t qk_dim,
                          int32_t v_dim, int32_t width, int32_t block_size,
                          int32_t bt_stride, uint64_t cache_stride_bytes,
                          double sm_scale, double k_scale, double v_scale,
                          const uint16_t* q, const uint8_t* k_cache,
                          const uint8_t* v_cache, const int32_t* block_tables,
                          const int32_t* seq_lens, const int32_t* sel,
                          double* out, int32_t num_threads) {
  if (rows < 0 || heads <= 0 || qk_dim <= 0 || v_dim <= 0 || v_dim > qk_dim ||
      width < 0 || block_size <= 0 || bt_stride < 0)
    return -1;
  if (rows == 0) return 0;
  const int32_t D = qk_dim; /* bytes per cached token, and q's width */

  /* Per row: the selected set and each member's byte offset. */
  int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)rows * (size_t)(width ? width : 1));
  uint64_t* offs = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)rows * (size_t)(width ? width : 1));
  int32_t* count = (int32_t*)malloc(sizeof(int32_t) * (size_t)rows);
  if (!ids || !offs || !count) {
    free(ids); free(offs); free(count);
    return -1;
  }
  for (int32_t r = 0; r < rows; ++r) {
    int32_t* rid = ids + (size_t)r * width;
    uint64_t* roff = offs + (size_t)r * width;
    const int32_t* bt_row = block_tables + (size_t)r * (size_t)bt_stride; /* stride 0: shared table */
    count[r] = dsa_oracle_select_row(sel + (size_t)r * width, width, seq_lens[r], rid);
    for (int32_t i = 0; i < count[r]; ++i)
      roff[i] = dsa_oracle_token_offset(bt_row, rid[i], block_size,
                                        cache_stride_bytes, D);
  }

  const int64_t pairs = (int64_t)rows * heads;
  int fail = 0;
#ifdef _OPENMP
  int nt = num_threads > 0 ? num_threads : omp_get_max_threads();
#pragma omp parallel num_threads(nt)
#endif
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(width ? width : 1));
    if (!s) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      fail = 1;
    }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
    for (int64_t pr = 0; pr < pairs; ++pr) {
      if (!s) continue;
      int32_t r = (int32_t)(pr / heads), h = (int32_t)(pr % heads);
      decode_one_head(D, v_dim, count[r], offs + (size_t)r * width, sm_scale,
                      k_scale, v_scale,
                      q + ((size_t)r * heads + h) * (size_t)D, k_cache,
                      v_cache, s, out + ((size_t)r * heads + h) * (size_t)v_dim);
    }
    free(s);
  }
  free(ids); free(offs); free(count);
  return fail ? -1 : 0;
}

/* Nearest finite E4M3FN code by exhaustive search over the 127 non-negative
 * finite codes (their values increase with the code), ties to the even
 * mantissa field; beyond 448, 448 (saturating). */
uint8_t dsa_oracle_fp8_e4m3fn_encode(double x) {
  const int neg = signbit(x) ? 1 : 0;
  const double a = fabs(x);
  int best = 0;
  double best_err = INFINITY;
  if (a >= 448.0) {
    best = 0x7E;
  } else {
    for (int c = 0; c <= 0x7E; ++c) {
      const double err = fabs(dsa_oracle_fp8_e4m3fn((uint8_t)c) - a);
      if (err < best_err || (err == best_err && (c & 1) == 0)) {
        best_err = err;
        best = c;
      }
    }
  }
  return (uint8_t)(best | (neg << 7));
}

/* [decode_k] latent_write: RMSNorm of the kv_a row times the layernorm
 * weight, scaled by 1/kv_scale, quantised to FP8 into the token's slot of the
 * paged pool. Plain double arithmetic in index order. */
int dsa_oracle_latent_write(int32_t rows, int32_t kv_lora_rank,
                            const uint16_t* kv_a, const uint16_t* weight,
                            const int64_t* slots, int32_t block_size,
                            uint64_t cache_stride_bytes, double eps,
                            double inv_kv_scale, uint8_t* pool,
                            uint64_t pool_bytes, double* values) {
  const int32_t D = kv_lora_rank;
  if (rows < 0 || D <= 0 || block_size <= 0 || !(eps >= 0.0)) return -1;
  if (rows > 0 && (!kv_a || !weight || !slots || !pool)) return -1;
  if (cache_stride_bytes == 0) cache_stride_bytes = (uint64_t)block_size * (uint64_t)D;
  for (int32_t i = 0; i < rows; ++i) {
    const uint16_t* x = kv_a + (size_t)i * D;
    double* yv = values ? values + (size_t)i * D : NULL;
    const int64_t slot = slots[i];
    if (slot < 0) {
      if (yv) for (int32_t d = 0; d < D; ++d) yv[d] = 0.0;
      continue;
    }
    const uint64_t off = (uint64_t)(slot / block_size) * cache_stride_bytes +
                         (uint64_t)(slot % block_size) * (uint64_t)D;
    if (off + (uint64_t)D > pool_bytes) return -1;
    double ss = 0.0;
    for (int32_t d = 0; d < D; ++d) {
      const double v = dsa_oracle_bf16(x[d]);
      ss += v * v;
    }
    const double inv_rms = 1.0 / sqrt(ss / (double)D + eps);
    for (int32_t d = 0; d < D; ++d) {
      const double y = dsa_oracle_bf16(x[d]) * inv_rms * dsa_oracle_bf16(weight[d]) * inv_kv_scale;
      if (yv) yv[d] = y;
      pool[off + (uint64_t)d] = dsa_oracle_fp8_e4m3fn_encode(y);
    }
  }
  return 0;
}
