// gfx950 dense masked-attention reference of the selected-index decode: a
// plain fp32 kernel kept apart from the decode kernel (no shared device
// code), used to cross-check the decode on every row of large workloads.
//
// What it computes is the dense form the page "spark_model/layers/
// glm5next_dsa/attend.rs" (module doc, "Why this is not the masked kernel")
// states the selected-index decode equals: attention of each query row over
// every cached position t < seq_len, with a mask that keeps exactly the
// positions listed in the row's selection (holes, repeats and ids outside
// [0, seq_len) select nothing). K and V are the dequantised FP8 latent rows
// (one latent head, V = the same row scaled by v_scale), the output stays
// in the latent space, [heads, kv_lora_rank] per row ("spark_model/layers/
// glm5next_dsa/build.rs"). A row with an empty mask gives zeros.
//
// How: one workgroup per (row, head). It marks the row's mask in an LDS
// bitmap over [0, seq_len), walks the positions in ascending order keeping
// the marked ones, scores each kept token with one wave (fp32 dot product
// over the dequantised row), takes max and sum in fp32 and accumulates the
// output one latent column per thread. Nothing here is tuned.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <sstream>

#include "plan.hpp"

namespace dsa {
namespace {

constexpr int kRefThreads = 256;
constexpr int kRefWaves = kRefThreads / 64;
// Dynamic LDS one workgroup may use (gfx950 has 160 KiB per workgroup; the
// rest holds the static reduction scratch).
constexpr size_t kRefLdsLimit = 159 * 1024;

// OCP E4M3FN: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0
// is subnormal (m * 2^-9); 0x7f / 0xff are NaN; no infinities.
__device__ float ref_fp8_value(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  float v;
  if (e == 15u && m == 7u) v = __builtin_nanf("");
  else if (e == 0u) v = ldexpf((float)m, -9);
  else v = ldexpf((float)(8u + m), (int)e - 10);
  return (b & 0x80u) ? -v : v;
}

__device__ float ref_bf16_value(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ float ref_wave_sum(float x) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ float ref_wave_max(float x) {
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

struct RefArgs {
  const uint16_t* q;
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const int32_t* sel;
  float* out;
  uint64_t cache_stride;
  int rows, H, D, width, max_seq_len, bt_stride, block_size;
  int words;  // bitmap words: ceil(max_seq_len / 32)
  float k_scale, v_scale, sm_scale;
};

// Byte offset of position t's latent row.
__device__ uint64_t ref_row_offset(const RefArgs& a, int r, int t) {
  const int32_t page = a.block_tables[(size_t)r * a.bt_stride + t / a.block_size];
  return (uint64_t)(uint32_t)page * a.cache_stride + (uint64_t)(t % a.block_size) * (uint64_t)a.D;
}

__global__ __launch_bounds__(kRefThreads)
void dsa_decode_masked_reference_kernel(RefArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t ref_lds[];
  uint32_t* mask = ref_lds;                                // [words]
  int32_t* kept = (int32_t*)(ref_lds + a.words);           // [width] ascending kept positions
  float* score = (float*)(kept + a.width);                 // [width]
  __shared__ float red[kRefWaves];
  __shared__ int cnt_sh[kRefWaves];

  const int r = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int L = a.seq_lens[r];
  L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
  const int nwords = (L + 31) / 32;

  // ---- the mask over [0, L)
  for (int w = tid; w < nwords; w += kRefThreads) mask[w] = 0u;
  __syncthreads();
  for (int j = tid; j < a.width; j += kRefThreads) {
    const int t = a.sel[(size_t)r * a.width + j];
    if (t >= 0 && t < L) atomicOr(&mask[t >> 5], 1u << (t & 31));
  }
  __syncthreads();

  // ---- every position in ascending order; the marked ones are kept
  int n = 0;
  for (int w0 = 0; w0 < nwords; w0 += kRefThreads) {
    const int w = w0 + tid;
    const uint32_t bits = w < nwords ? mask[w] : 0u;
    const int c = __popc(bits);
    int incl = c;
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    if (lane == 63) cnt_sh[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
    for (int k = 0; k < kRefWaves; ++k) {
      before += k < wave ? cnt_sh[k] : 0;
      total += cnt_sh[k];
    }
    int pos = n + before + incl - c;
    for (int b = 0; b < 32; ++b)
      if (bits & (1u << b)) kept[pos++] = w * 32 + b;
    n += total;
    __syncthreads();
  }

  float* orow = a.out + ((size_t)r * a.H + h) * a.D;
  if (n == 0) {
    for (int d = tid; d < a.D; d += kRefThreads) orow[d] = 0.f;
    return;
  }

  // ---- scores: one wave per kept token, fp32 over the dequantised row
  const uint16_t* qrow = a.q + ((size_t)r * a.H + h) * a.D;
  for (int i = wave; i < n; i += kRefWaves) {
    const uint8_t* krow = a.k_cache + ref_row_offset(a, r, kept[i]);
    float acc = 0.f;
    for (int d = lane; d < a.D; d += 64) acc += ref_bf16_value(qrow[d]) * ref_fp8_value(krow[d]);
    acc = ref_wave_sum(acc);
    if (lane == 0) score[i] = acc * a.k_scale * a.sm_scale;
  }
  __syncthreads();

  // ---- softmax over the kept tokens: max, then weights and their sum
  float m = -INFINITY;
  for (int i = tid; i < n; i += kRefThreads) m = fmaxf(m, score[i]);
  m = ref_wave_max(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  m = red[0];
  for (int k = 1; k < kRefWaves; ++k) m = fmaxf(m, red[k]);
  __syncthreads();
  float l = 0.f;
  for (int i = tid; i < n; i += kRefThreads) {
    const float p = expf(score[i] - m);
    score[i] = p;
    l += p;
  }
  l = ref_wave_sum(l);
  if (lane == 0) red[wave] = l;
  __syncthreads();
  l = 0.f;
  for (int k = 0; k < kRefWaves; ++k) l += red[k];

  // ---- output: one latent column per thread, tokens in ascending order
  for (int d = tid; d < a.D; d += kRefThreads) {
    float o = 0.f;
    for (int i = 0; i < n; ++i)
      o += score[i] * ref_fp8_value(a.v_cache[ref_row_offset(a, r, kept[i]) + d]);
    orow[d] = o * a.v_scale / l;
  }
}

}  // namespace
}  // namespace dsa

extern "C" {

int dsa_decode_masked_reference(const dsa_decode_params* params, const void* q,
                         const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* seq_lens,
                         const int32_t* sel_indices, float k_scale, float v_scale,
                         float* out, void* stream) {
  using namespace dsa;
  dsa_decode_params p{};
  int st = validate_params(params, &p);
  if (st != DSA_DECODE_OK) return st;
  if (p.qk_rope_dim != 0)
    return fail(DSA_DECODE_ERR_UNSUPPORTED,
                "dsa_decode_masked_reference: tokens with a rope tail are not supported");
  if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !sel_indices || !out)
    return fail(DSA_DECODE_ERR_INVALID, "dsa_decode_masked_reference: NULL buffer");
  if (!std::isfinite(k_scale) || !std::isfinite(v_scale))
    return fail(DSA_DECODE_ERR_INVALID, "dsa_decode_masked_reference: k_scale and v_scale must be finite");
  const size_t words = ((size_t)p.max_seq_len + 31) / 32;
  const size_t lds = 4 * words + 8 * (size_t)p.sel_width;
  if (lds > kRefLdsLimit) {
    std::ostringstream m;
    m << "dsa_decode_masked_reference: max_seq_len " << p.max_seq_len << " and sel_width "
      << p.sel_width << " need " << lds << " bytes of LDS per workgroup (limit "
      << kRefLdsLimit << ")";
    return fail(DSA_DECODE_ERR_INVALID, m.str());
  }
  int dev = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(DSA_DECODE_ERR_DEVICE, "dsa_decode_masked_reference: no HIP device");
  }
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
    std::ostringstream m;
    m << "dsa_decode_masked_reference: device " << dev << " is " << prop.gcnArchName
      << "; this library is built for gfx950 only";
    return fail(DSA_DECODE_ERR_DEVICE, m.str());
  }
  RefArgs a;
  a.q = (const uint16_t*)q;
  a.k_cache = (const uint8_t*)k_cache;
  a.v_cache = (const uint8_t*)v_cache;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.sel = sel_indices;
  a.out = out;
  a.cache_stride = p.cache_stride_bytes;
  a.rows = p.num_rows;
  a.H = p.num_q_heads;
  a.D = p.kv_lora_rank;
  a.width = p.sel_width;
  a.max_seq_len = p.max_seq_len;
  a.bt_stride = p.block_table_stride;
  a.block_size = p.block_size;
  a.words = (int)words;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.sm_scale = p.sm_scale;
  const size_t grid = (size_t)p.num_rows * (size_t)p.num_q_heads;
  if (grid > 0x7fffffff)
    return fail(DSA_DECODE_ERR_INVALID, "dsa_decode_masked_reference: rows x heads too large");
  if (lds > 64 * 1024 &&
      hipFuncSetAttribute((const void*)dsa_decode_masked_reference_kernel,
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess) {
    (void)hipGetLastError();
    return fail(DSA_DECODE_ERR_LAUNCH, "dsa_decode_masked_reference: cannot raise the LDS limit");
  }
  hipLaunchKernelGGL(dsa_decode_masked_reference_kernel, dim3((unsigned)grid), dim3(kRefThreads),
                     lds, (hipStream_t)stream, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(DSA_DECODE_ERR_LAUNCH,
                std::string("dsa_decode_masked_reference: launch: ") + hipGetErrorString(e));
  set_error("");
  return DSA_DECODE_OK;
}

}  // extern "C"
