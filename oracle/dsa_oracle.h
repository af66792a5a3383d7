/*
 * CPU oracle for the selected-index NoPE MLA paged decode.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link or
 * call this library: only the tests, the smoke check and the benchmark's CPU
 * baseline use it. It shares no code, header, table or constant with the HIP
 * library under sparse_attention_decode_row_amd/csrc.
 *
 * Everything is computed in double precision from the definition of the
 * operation, one row and one head at a time, with no blocking or fusion.
 *
 * Sources (the web pages the method is described on):
 *   [attend]   page "spark_model/layers/glm5next_dsa/attend.rs"
 *   [decode_k] page "metrale_model_arch/glm5next_dsa/layer/decode_k.rs"
 *   [build]    page "spark_model/layers/glm5next_dsa/build.rs"
 *
 * Parity status: every function here is pinned by CPU tests against
 * something other than itself (torch's float8 casts in both directions,
 * Python set semantics, a dense masked-attention brute force over a logically
 * contiguous cache, closed forms of the RMS normalisation, hand-placed
 * slots). None is "parity unpinned".
 */
#ifndef DSA_ORACLE_H
#define DSA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Value of one OCP FP8 E4M3FN code: 1 sign bit, 4 exponent bits with bias 7,
 * 3 mantissa bits; exponent field 0 is subnormal (m/8 * 2^-6); the two codes
 * with all exponent and mantissa bits set are NaN; there is no infinity.
 * The cache is "FP8" per [attend] DsaDecodeInputs; the E4M3 variant is the
 * one the decode is specified over. */
double dsa_oracle_fp8_e4m3fn(uint8_t code);

/* Value of one bfloat16 bit pattern (the upper half of an IEEE binary32). */
double dsa_oracle_bf16(uint16_t bits);

/* Selection of one row as a set ([attend] module doc, "Why this is not the
 * masked kernel": membership only, duplicates collapse, -1 is a hole).
 * Writes the sorted distinct ids t of sel[0..width) with 0 <= t < seq_len to
 * out_ids (capacity width) and returns their count. Any negative id is a
 * hole; ids at or beyond seq_len are dropped. */
int32_t dsa_oracle_select_row(const int32_t* sel, int32_t width,
                              int32_t seq_len, int32_t* out_ids);

/* Byte offset of logical token t of a row inside the paged pool:
 * page = bt_row[t / block_size], offset = page * cache_stride_bytes
 * + (t mod block_size) * kv_lora_rank. One FP8 byte per latent element and a
 * single KV head ([decode_k] slot computation and DsaDecodePaging stride;
 * [attend] DsaDecodePaging::validate). */
uint64_t dsa_oracle_token_offset(const int32_t* bt_row, int32_t t,
                                 int32_t block_size,
                                 uint64_t cache_stride_bytes,
                                 int32_t kv_lora_rank);

/* The whole decode.
 *   q            [rows, heads, D] bf16 bits (absorbed queries, latent space)
 *   k_cache      FP8 E4M3FN pool, v_cache the same layout (may alias)
 *   block_tables [rows, bt_stride] int32; bt_stride 0 = every row uses row 0
 *   seq_lens     [rows] int32
 *   sel          [rows, width] int32
 *   out          [rows, heads, D] double
 * For each row and head, over the row's selected set S:
 *   s_t = sm_scale * sum_d q[d] * (k_scale * dec(K_t[d]))
 *   p_t = exp(s_t - max s), out = sum_t p_t * (v_scale * dec(V_t[d])) / sum p
 * and out = 0 when S is empty. num_threads <= 0 uses the OpenMP default.
 * Returns 0, or -1 on a bad argument. */
int dsa_oracle_decode(int32_t rows, int32_t heads, int32_t kv_lora_rank,
                      int32_t width, int32_t block_size, int32_t bt_stride,
                      uint64_t cache_stride_bytes, double sm_scale,
                      double k_scale, double v_scale,
                      const uint16_t* q, const uint8_t* k_cache,
                      const uint8_t* v_cache, const int32_t* block_tables,
                      const int32_t* seq_lens, const int32_t* sel,
                      double* out, int32_t num_threads);

/* The decode for cache tokens that carry a tail after the latent: a token is
 * qk_dim FP8 bytes, its first v_dim of them the latent. The scores run over
 * all qk_dim bytes of token t's own row, the values and the output over its
 * first v_dim ([attend] module doc, "NoPE, and why no common/ kernel would
 * do", and decode_attention's scale comment: a DeepSeek-V4 token is the
 * 512-wide latent plus a 64-wide rope tail, 576 in all; the tail arrives
 * already rotated, and belongs to the token whose row holds it).
 *   q    [rows, heads, qk_dim] bf16 bits
 *   out  [rows, heads, v_dim] double
 * Token t of a row sits at page * cache_stride_bytes + (t mod block_size) *
 * qk_dim. Otherwise as dsa_oracle_decode, which is this function with
 * qk_dim == v_dim == kv_lora_rank. Returns 0, or -1 on a bad argument
 * (including v_dim > qk_dim). */
int dsa_oracle_decode_qkv(int32_t rows, int32_t heads, int32_t qk_dim,
                          int32_t v_dim, int32_t width, int32_t block_size,
                          int32_t bt_stride, uint64_t cache_stride_bytes,
                          double sm_scale, double k_scale, double v_scale,
                          const uint16_t* q, const uint8_t* k_cache,
                          const uint8_t* v_cache, const int32_t* block_tables,
                          const int32_t* seq_lens, const int32_t* sel,
                          double* out, int32_t num_threads);

/* Number of threads an OpenMP parallel region of the decode would use. */
int32_t dsa_oracle_max_threads(void);

/* FP8 E4M3FN code of x, rounded to the nearest finite code (ties to the code
 * with an even mantissa field) and saturated to +-448 beyond the largest
 * finite value (never NaN). The sign of a zero result is the sign of x. This
 * is how latent rows are quantised into the cache (value / kv_scale, stored
 * as FP8; [decode_k] latent_write launch). x must not be NaN. */
uint8_t dsa_oracle_fp8_e4m3fn_encode(double x);

/* The cache writer ([decode_k] latent_write launch: one kv_a row, the
 * kv_a_layernorm weight, the pool, the token's slot, rms_eps, 1/kv_scale).
 * For each row i with slots[i] >= 0 (a negative slot writes nothing):
 *   y_d = x_d / sqrt(mean_d(x_d^2) + eps) * w_d * inv_kv_scale
 * with x = kv_a[i] and w both bf16 bits, computed in double; the FP8 codes
 * of y (dsa_oracle_fp8_e4m3fn_encode) go to the pool bytes
 *   (slot / block_size) * cache_stride_bytes + (slot mod block_size) * D
 * (the decode's addressing of a token row). values, if not NULL, receives y
 * as [rows, D] doubles (rows with a negative slot: 0). Returns 0, or -1 on a
 * bad argument or a row that would fall outside pool_bytes. */
int dsa_oracle_latent_write(int32_t rows, int32_t kv_lora_rank,
                            const uint16_t* kv_a, const uint16_t* weight,
                            const int64_t* slots, int32_t block_size,
                            uint64_t cache_stride_bytes, double eps,
                            double inv_kv_scale, uint8_t* pool,
                            uint64_t pool_bytes, double* values);

#ifdef __cplusplus
}
#endif

#endif
