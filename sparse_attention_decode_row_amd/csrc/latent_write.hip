// gfx950 kernel of the cache writer: RMSNorm of a kv_a row times the
// layernorm weight, scaled by 1/kv_scale, rounded to FP8 E4M3FN into the
// token's slot of the paged pool.
//
// What is computed is defined on the page "metrale_model_arch/glm5next_dsa/
// layer/decode_k.rs" (the latent_write launch and the slot of a position).
// How: one wave per two rows, D/64 elements per lane (one 16-byte load per
// row and one of the weight at D = 512); both rows' loads are issued before
// either reduction, so each wave keeps 2 KiB in flight. The sum of squares is
// reduced across the wave with DPP and cross-row swaps, the conversion runs on
// the hardware's FP8 converter after clamping to the largest finite value,
// one store per lane and row. kv_a rows are read once and pool rows written
// once here, so both go through the nontemporal (streaming) cache policy.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <sstream>

#include "plan.hpp"

namespace dsa {
namespace {

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWavesPerBlock = 4;
constexpr int kRowsPerWave = 2;
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

// E (1, 2, 4 or 8) consecutive bf16 values at p, as raw 16-bit fields packed
// in 32-bit words; NT: streaming load.
template <int E, bool NT>
__device__ __forceinline__ void load_raw(const uint16_t* p, uint32_t (&r)[(E + 1) / 2]) {
  if constexpr (E == 8) {
    const u32x4* q = (const u32x4*)p;
    const u32x4 w = NT ? __builtin_nontemporal_load(q) : *q;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = w[i];
  } else if constexpr (E == 4) {
    const u32x2* q = (const u32x2*)p;
    const u32x2 w = NT ? __builtin_nontemporal_load(q) : *q;
    r[0] = w[0];
    r[1] = w[1];
  } else if constexpr (E == 2) {
    const uint32_t* q = (const uint32_t*)p;
    r[0] = NT ? __builtin_nontemporal_load(q) : *q;
  } else {
    r[0] = NT ? __builtin_nontemporal_load(p) : *p;
  }
}

template <int E>
__device__ __forceinline__ float raw_elem(const uint32_t (&r)[(E + 1) / 2], int i) {
  return bf16_to_f32((i & 1) ? (r[i >> 1] >> 16) : (r[i >> 1] & 0xffffu));
}

// Four floats -> four FP8 E4M3FN codes (nearest, ties to even), byte i = x_i;
// the inputs are already within +-448.
__device__ __forceinline__ uint32_t pack_fp8x4(float x0, float x1, float x2, float x3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
}

template <int D>
__global__ __launch_bounds__(kWavesPerBlock * 64)
void dsa_latent_write_kernel(const uint16_t* kv_a, const uint16_t* weight,
                             const int64_t* slots, int rows, int block_size,
                             uint64_t stride, float eps, float inv_kv_scale,
                             uint8_t* pool) {
  constexpr int E = D / 64;
  constexpr int W = (E + 1) / 2;
  const int lane = threadIdx.x & 63;
  const int row0 = (blockIdx.x * kWavesPerBlock + (int)(threadIdx.x >> 6)) * kRowsPerWave;
  int64_t slot[kRowsPerWave];
#pragma unroll
  for (int j = 0; j < kRowsPerWave; ++j) slot[j] = row0 + j < rows ? slots[row0 + j] : -1;
  // a negative slot (or a row past the end) writes nothing; the row itself is
  // loaded whenever it exists, so that its load does not wait for the slot's
  uint32_t raw[kRowsPerWave][W];
#pragma unroll
  for (int j = 0; j < kRowsPerWave; ++j) {
    if (row0 + j < rows) {
      load_raw<E, true>(kv_a + (size_t)(row0 + j) * D + lane * E, raw[j]);
    } else {
#pragma unroll
      for (int i = 0; i < W; ++i) raw[j][i] = 0u;
    }
  }
  uint32_t wraw[W];
  load_raw<E, false>(weight + lane * E, wraw);

  float ss[kRowsPerWave];
#pragma unroll
  for (int j = 0; j < kRowsPerWave; ++j) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const float x = raw_elem<E>(raw[j], i);
      acc = fmaf(x, x, acc);
    }
    ss[j] = acc;
  }
#pragma unroll
  for (int j = 0; j < kRowsPerWave; ++j) ss[j] = wave_sum(ss[j]);

#pragma unroll
  for (int j = 0; j < kRowsPerWave; ++j) {
    if (slot[j] < 0) continue;
    const float inv_rms = 1.0f / sqrtf(ss[j] * (1.0f / D) + eps);
    float y[E < 4 ? 4 : E];
#pragma unroll
    for (int i = 0; i < (E < 4 ? 4 : E); ++i) y[i] = 0.f;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const float v = raw_elem<E>(raw[j], i) * inv_rms * raw_elem<E>(wraw, i) * inv_kv_scale;
      y[i] = fminf(fmaxf(v, -kFp8Max), kFp8Max);  // saturate (never NaN)
    }
    const int64_t page = slot[j] / block_size;
    const int64_t in_page = slot[j] - page * block_size;
    uint8_t* dst = pool + (uint64_t)page * stride + (uint64_t)in_page * D + lane * E;
    if constexpr (E == 8) {
      const u32x2 c = {pack_fp8x4(y[0], y[1], y[2], y[3]), pack_fp8x4(y[4], y[5], y[6], y[7])};
      __builtin_nontemporal_store(c, (u32x2*)dst);
    } else if constexpr (E == 4) {
      __builtin_nontemporal_store(pack_fp8x4(y[0], y[1], y[2], y[3]), (uint32_t*)dst);
    } else if constexpr (E == 2) {
      __builtin_nontemporal_store((uint16_t)(pack_fp8x4(y[0], y[1], 0.f, 0.f) & 0xffffu),
                                  (uint16_t*)dst);
    } else {
      __builtin_nontemporal_store((uint8_t)(pack_fp8x4(y[0], 0.f, 0.f, 0.f) & 0xffu), dst);
    }
  }
}

template <int D>
hipError_t launch_writer(const void* kv_a, const void* weight, const int64_t* slots, int rows,
                         int block_size, uint64_t stride, float eps, float inv, void* pool,
                         hipStream_t st) {
  constexpr int kRowsPerBlock = kWavesPerBlock * kRowsPerWave;
  const dim3 grid((rows + kRowsPerBlock - 1) / kRowsPerBlock), block(kWavesPerBlock * 64);
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
