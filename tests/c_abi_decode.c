/* The decode driven from plain C through the library's C ABI alone (no
 * Python, no torch): device memory from the HIP runtime's C API, the plan,
 * workspace, launch and selection read-back from include/dsa_decode.h, and
 * the result checked against the CPU oracle (test infrastructure, linked
 * here because this program is a test).
 *
 * The inputs are drawn from a fixed linear congruential generator: rows of
 * different lengths over a shuffled page table, selections mixing valid
 * ids, repeats, -1 holes and ids past the row's length, FP8 E4M3FN latents
 * with every finite code possible. Exit status 0 when every (row, head)
 * output is within the decode's bar (normwise relative error <= 1e-2) and
 * the attended sets equal the oracle's; 1 otherwise; 2 on a setup error. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "dsa_decode.h"
#include "dsa_oracle.h"

/* rows, heads, latent width, page size, selection width, longest row,
 * block-table entries per row, pages in the pool */
enum { R = 5, H = 40, D = 256, B = 16, W = 300, MAXLEN = 900, STRIDE = MAXLEN / B + 1,
       PAGES = R * STRIDE };

static uint32_t rng_state = 20250901u;
static uint32_t next_u32(void) {
  rng_state = rng_state * 1664525u + 1013904223u;
  return rng_state >> 8;
}

/* bf16 bits of x, round to nearest even (x finite) */
static uint16_t to_bf16(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

#define CHECK_HIP(call)                                                   \
  do {                                                                    \
    hipError_t e_ = (call);                                               \
    if (e_ != hipSuccess) {                                               \
      fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));          \
      return 2;                                                           \
    }                                                                     \
  } while (0)

int main(void) {
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count < 1) {
    fprintf(stderr, "no HIP device\n");
    return 2;
  }
  static uint16_t q[R * H * D];
  static uint8_t pool[(size_t)PAGES * B * D];
  static int32_t bt[R * STRIDE], seq_lens[R], sel[R * W];
  static uint16_t out[R * H * D];
  static double want[R * H * D];

  for (int i = 0; i < R * H * D; ++i)
    q[i] = to_bf16(((float)(next_u32() % 4001u) - 2000.f) / 1000.f);
  for (size_t i = 0; i < sizeof(pool); ++i) {
    uint8_t c = (uint8_t)next_u32();
    if ((c & 0x7fu) == 0x7fu) c ^= 1u; /* no NaN codes */
    pool[i] = c;
  }
  int perm[PAGES];
  for (int i = 0; i < PAGES; ++i) perm[i] = i;
  for (int i = PAGES - 1; i > 0; --i) {
    const int j = (int)(next_u32() % (uint32_t)(i + 1));
    const int t = perm[i];
    perm[i] = perm[j];
    perm[j] = t;
  }
  for (int r = 0; r < R; ++r) {
    for (int e = 0; e < STRIDE; ++e) bt[r * STRIDE + e] = perm[r * STRIDE + e];
    seq_lens[r] = 1 + (int)(next_u32() % MAXLEN);
    for (int j = 0; j < W; ++j) {
      const uint32_t kind = next_u32() % 10u;
      int32_t t;
      if (kind == 0) t = -1;                                         /* hole */
      else if (kind == 1 && j > 0) t = sel[r * W + (int)(next_u32() % (uint32_t)j)]; /* repeat */
      else if (kind == 2) t = seq_lens[r] + (int32_t)(next_u32() % 5u); /* past the end */
      else t = (int32_t)(next_u32() % (uint32_t)seq_lens[r]);
      sel[r * W + j] = t;
    }
  }
  const float k_scale = 0.03f, v_scale = 0.05f, sm_scale = 1.0f / 16.0f;

  void *d_q, *d_pool, *d_bt, *d_sl, *d_sel, *d_out, *d_ws, *d_ids, *d_counts;
  CHECK_HIP(hipMalloc(&d_q, sizeof(q)));
  CHECK_HIP(hipMalloc(&d_pool, sizeof(pool)));
  CHECK_HIP(hipMalloc(&d_bt, sizeof(bt)));
  CHECK_HIP(hipMalloc(&d_sl, sizeof(seq_lens)));
  CHECK_HIP(hipMalloc(&d_sel, sizeof(sel)));
  CHECK_HIP(hipMalloc(&d_out, sizeof(out)));
  CHECK_HIP(hipMalloc(&d_ids, sizeof(int32_t) * R * W));
  CHECK_HIP(hipMalloc(&d_counts, sizeof(int32_t) * R));
  CHECK_HIP(hipMemcpy(d_q, q, sizeof(q), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_pool, pool, sizeof(pool), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_bt, bt, sizeof(bt), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_sl, seq_lens, sizeof(seq_lens), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_sel, sel, sizeof(sel), hipMemcpyHostToDevice));

  dsa_decode_params p;
  memset(&p, 0, sizeof(p));
  p.num_rows = R;
  p.num_q_heads = H;
  p.num_kv_heads = 1;
  p.kv_lora_rank = D;
  p.block_size = B;
  p.index_kpool = 4;
  p.sel_width = W;
  p.block_table_stride = STRIDE;
  p.max_seq_len = MAXLEN;
  p.sm_scale = sm_scale;
  p.flags = DSA_DECODE_FLAG_EXPORT_SELECTION;
  dsa_decode_plan_t plan = NULL;
  if (dsa_decode_plan(&p, 0, &plan) != DSA_DECODE_OK) {
    fprintf(stderr, "plan: %s\n", dsa_decode_last_error());
    return 2;
  }
  const size_t ws_bytes = dsa_decode_workspace_bytes(plan);
  CHECK_HIP(hipMalloc(&d_ws, ws_bytes));
  if (dsa_decode_workspace_init(plan, d_ws, ws_bytes, NULL) != DSA_DECODE_OK ||
      dsa_decode_launch(plan, d_q, d_pool, d_pool, (const int32_t*)d_bt,
                        (const int32_t*)d_sl, (const int32_t*)d_sel, k_scale, v_scale,
                        d_out, d_ws, ws_bytes, NULL) != DSA_DECODE_OK ||
      dsa_decode_read_selection(plan, d_ws, ws_bytes, (int32_t*)d_ids,
                                (int32_t*)d_counts, NULL, NULL) != DSA_DECODE_OK) {
    fprintf(stderr, "launch: %s\n", dsa_decode_last_error());
    return 2;
  }
  CHECK_HIP(hipDeviceSynchronize());
  CHECK_HIP(hipMemcpy(out, d_out, sizeof(out), hipMemcpyDeviceToHost));
  static int32_t ids[R * W], counts[R], want_ids[W];
  CHECK_HIP(hipMemcpy(ids, d_ids, sizeof(ids), hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(counts, d_counts, sizeof(counts), hipMemcpyDeviceToHost));

  /* the oracle takes the page stride literally (the library reads 0 as B * D) */
  if (dsa_oracle_decode(R, H, D, W, B, STRIDE, (uint64_t)B * D, sm_scale, k_scale, v_scale, q, pool, pool,
                        bt, seq_lens, sel, want, 0) != 0) {
    fprintf(stderr, "oracle refused the inputs\n");
    return 2;
  }
  int sets_ok = 1;
  for (int r = 0; r < R; ++r) {
    const int32_t n = dsa_oracle_select_row(sel + r * W, W, seq_lens[r], want_ids);
    if (n != counts[r] || memcmp(want_ids, ids + r * W, sizeof(int32_t) * (size_t)n) != 0) {
      fprintf(stderr, "row %d: attended set differs (%d vs %d ids)\n", r, counts[r], n);
      sets_ok = 0;
    }
  }
  double worst = 0.0;
  for (int rh = 0; rh < R * H; ++rh) {
    double num = 0.0, den = 0.0;
    for (int d = 0; d < D; ++d) {
      const uint32_t u = (uint32_t)out[rh * D + d] << 16;
      float g;
      memcpy(&g, &u, 4);
      num = fmax(num, fabs((double)g - want[rh * D + d]));
      den = fmax(den, fabs(want[rh * D + d]));
    }
    const double err = den > 0.0 ? num / den : num;
    if (err > worst) worst = err;
  }
  printf("c_abi_decode: rows %d heads %d D %d W %d, max normwise rel err %.3e, sets %s\n", R, H,
         D, W, worst, sets_ok ? "equal" : "DIFFER");
  dsa_decode_plan_destroy(plan);
  hipFree(d_q);
  hipFree(d_pool);
  hipFree(d_bt);
  hipFree(d_sl);
  hipFree(d_sel);
  hipFree(d_out);
  hipFree(d_ws);
  hipFree(d_ids);
  hipFree(d_counts);
  return (worst <= 1e-2 && sets_ok) ? 0 : 1;
}
