// gfx950 kernel of the cache writer: RMSNorm of a kv_a row times the
// layernorm weight, scaled by 1/kv_scale, rounded to FP8 E4M3FN into the
// token's slot of the paged pool.
//
// What is computed is defined on the page "metrale_model_arch/glm5next_dsa/
// layer/decode_k.rs" (the latent_write launch and the slot of a position).
// How: one wave per row, D/64 elements per lane (one 16-byte load of the row
// and of the weight at D = 512), the sum of squares reduced across the wave
// with DPP and cross-row swaps, the conversion on the hardware's FP8
// converter after clamping to the largest finite value, one store per lane.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <sstream>

#include "plan.hpp"

namespace dsa {
namespace {

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRowsPerBlock = 4;  // one wave each
constexpr float kFp8Max = 448.0f;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Sum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_sum(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  x += __shfl_xor(x, 8);
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// E (1, 2, 4 or 8) consecutive bf16 values at p, as floats.
template <int E>
__device__ __forceinline__ void load_bf16(const uint16_t* p, float (&v)[E]) {
  if constexpr (E == 8) {
    const u32x4 w = *(const u32x4*)p;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_to_f32(w[i] & 0xffffu);
      v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
  } else if constexpr (E == 4) {
    const u32x2 w = *(const u32x2*)p;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      v[2 * i] = bf16_to_f32(w[i] & 0xffffu);
      v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
  } else if constexpr (E == 2) {
    const uint32_t w = *(const uint32_t*)p;
    v[0] = bf16_to_f32(w & 0xffffu);
    v[1] = bf16_to_f32(w >> 16);
  } else {
    v[0] = bf16_to_f32(*p);
  }
}

// Four floats -> four FP8 E4M3FN codes (nearest, ties to even), byte i = x_i;
// the inputs are already within +-448.
__device__ __forceinline__ uint32_t pack_fp8x4(float x0, float x1, float x2, float x3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
}

template <int D>
__global__ __launch_bounds__(kRowsPerBlock * 64)
void dsa_latent_write_kernel(const uint16_t* kv_a, const uint16_t* weight,
                             const int64_t* slots, int rows, int block_size,
                             uint64_t stride, float eps, float inv_kv_scale,
                             uint8_t* pool) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerBlock + (int)(threadIdx.x >> 6);
  if (row >= rows) return;
  const int64_t slot = slots[row];
  if (slot < 0) return;  // no slot: nothing is written

  float x[E], w[E];
  load_bf16<E>(kv_a + (size_t)row * D + lane * E, x);
  load_bf16<E>(weight + lane * E, w);
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < E; ++i) ss = fmaf(x[i], x[i], ss);
  ss = wave_sum(ss);
  const float inv_rms = 1.0f / sqrtf(ss * (1.0f / D) + eps);

  float y[E < 4 ? 4 : E];
#pragma unroll
  for (int i = 0; i < (E < 4 ? 4 : E); ++i) y[i] = 0.f;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const float v = x[i] * inv_rms * w[i] * inv_kv_scale;
    y[i] = fminf(fmaxf(v, -kFp8Max), kFp8Max);  // saturate (never NaN)
  }
  const int64_t page = slot / block_size;
  const int64_t in_page = slot - page * block_size;
  uint8_t* dst = pool + (uint64_t)page * stride + (uint64_t)in_page * D + lane * E;
  if constexpr (E == 8) {
    const u32x2 c = {pack_fp8x4(y[0], y[1], y[2], y[3]), pack_fp8x4(y[4], y[5], y[6], y[7])};
    *(u32x2*)dst = c;
  } else if constexpr (E == 4) {
    *(uint32_t*)dst = pack_fp8x4(y[0], y[1], y[2], y[3]);
  } else if constexpr (E == 2) {
    *(uint16_t*)dst = (uint16_t)(pack_fp8x4(y[0], y[1], 0.f, 0.f) & 0xffffu);
  } else {
    *dst = (uint8_t)(pack_fp8x4(y[0], 0.f, 0.f, 0.f) & 0xffu);
  }
}

template <int D>
hipError_t launch_writer(const void* kv_a, const void* weight, const int64_t* slots, int rows,
                         int block_size, uint64_t stride, float eps, float inv, void* pool,
                         hipStream_t st) {
  const dim3 grid((rows + kRowsPerBlock - 1) / kRowsPerBlock), block(kRowsPerBlock * 64);
  hipLaunchKernelGGL((dsa_latent_write_kernel<D>), grid, block, 0, st, (const uint16_t*)kv_a,
                     (const uint16_t*)weight, slots, rows, block_size, stride, eps, inv,
                     (uint8_t*)pool);
  return hipGetLastError();
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace
}  // namespace dsa

extern "C" int dsa_decode_latent_write(const void* kv_a, const void* weight,
                                       const int64_t* slots, int32_t num_rows,
                                       int32_t kv_lora_rank, int32_t block_size,
                                       uint64_t cache_stride_bytes, float rms_eps,
                                       float inv_kv_scale, void* k_pool, void* stream) {
  using namespace dsa;
  const char* who = "dsa_decode_latent_write";
  std::ostringstream m;
  if (num_rows < 0) {
    m << who << ": num_rows must be >= 0, got " << num_rows;
    return fail(DSA_DECODE_ERR_INVALID, m.str());
  }
  if (kv_lora_rank != 64 && kv_lora_rank != 128 && kv_lora_rank != 256 && kv_lora_rank != 512) {
    m << who << ": kv_lora_rank " << kv_lora_rank << " is not compiled in (supported: 64, 128, 256, 512)";
    return fail(DSA_DECODE_ERR_UNSUPPORTED, m.str());
  }
  if (block_size <= 0) {
    m << who << ": block_size must be > 0, got " << block_size;
    return fail(DSA_DECODE_ERR_INVALID, m.str());
  }
  const uint64_t row_pitch = (uint64_t)block_size * (uint64_t)kv_lora_rank;
  const uint64_t stride = cache_stride_bytes ? cache_stride_bytes : row_pitch;
  if (stride < row_pitch || stride % 16 != 0) {
    m << who << ": cache_stride_bytes " << cache_stride_bytes << " must be 0 or >= block_size * "
      << "kv_lora_rank (" << row_pitch << ") and a multiple of 16";
    return fail(DSA_DECODE_ERR_INVALID, m.str());
  }
  if (!std::isfinite(rms_eps) || rms_eps < 0.f || !std::isfinite(inv_kv_scale) ||
      !(inv_kv_scale > 0.f)) {
    m << who << ": rms_eps must be finite and >= 0 and inv_kv_scale finite and > 0 (got "
      << rms_eps << ", " << inv_kv_scale << ")";
    return fail(DSA_DECODE_ERR_INVALID, m.str());
  }
  if (num_rows == 0) return DSA_DECODE_OK;
  if (!kv_a || !weight || !slots || !k_pool)
    return fail(DSA_DECODE_ERR_INVALID, std::string(who) + ": NULL device pointer");
  if (!aligned16(kv_a) || !aligned16(weight) || !aligned16(k_pool))
    return fail(DSA_DECODE_ERR_INVALID,
                std::string(who) + ": kv_a, weight and k_pool must be 16-byte aligned");
  const hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  switch (kv_lora_rank) {
    case 64: e = launch_writer<64>(kv_a, weight, slots, num_rows, block_size, stride, rms_eps, inv_kv_scale, k_pool, st); break;
    case 128: e = launch_writer<128>(kv_a, weight, slots, num_rows, block_size, stride, rms_eps, inv_kv_scale, k_pool, st); break;
    case 256: e = launch_writer<256>(kv_a, weight, slots, num_rows, block_size, stride, rms_eps, inv_kv_scale, k_pool, st); break;
    default: e = launch_writer<512>(kv_a, weight, slots, num_rows, block_size, stride, rms_eps, inv_kv_scale, k_pool, st); break;
  }
  if (e != hipSuccess)
    return fail(DSA_DECODE_ERR_LAUNCH, std::string(who) + ": " + hipGetErrorString(e));
  return DSA_DECODE_OK;
}
