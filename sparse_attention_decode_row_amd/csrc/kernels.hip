// gfx950 kernels and the launcher of the selected-index NoPE MLA paged decode.
//
// What is computed is defined on the pages (cited by title):
//   [attend]   "spark_model/layers/glm5next_dsa/attend.rs"
//   [decode_k] "metrale_model_arch/glm5next_dsa/layer/decode_k.rs"
//   [build]    "spark_model/layers/glm5next_dsa/build.rs"
// How it is computed here is this library's own design for CDNA4 (wave64,
// MFMA, 160 KiB LDS, LDS DMA, transposing LDS reads):
//
//   dsa_select_kernel   one workgroup per row: the selection row becomes a
//                       set through an LDS bitmap over [0, seq_len) (holes,
//                       repeats and out-of-range ids vanish; [attend] module
//                       doc, "Why this is not the masked kernel"), read back
//                       in ascending order, and every id is translated to the
//                       byte offset of its FP8 latent row through the block
//                       table ([decode_k] slot of a position).
//   dsa_attend_kernel   one workgroup per (row, 64-head block, chunk of the
//                       sorted set); 128-token tiles of latent rows are DMA'd
//                       straight into LDS, double buffered. Each wave owns 16
//                       heads. Both contractions run on the FP8 matrix cores
//                       (16x16x128, fp32 accumulation) with the cached latent
//                       bytes as they are, so nothing is converted per token:
//                         S^T = K Q^T : Q (bf16) enters as an exact sum of two
//                                       FP8 terms under a per-head power-of-two
//                                       scale (8 significant bits = 4 + 4);
//                         O^T = V^T P^T: the softmax weights enter as a sum of
//                                       two FP8 terms (relative error <= 2^-9,
//                                       below bf16's 2^-8); the V operand comes
//                                       from ds_read_tr8_b64, which hands each
//                                       lane 8 tokens of one latent column.
//                       Online softmax in the exp2 domain. One chunk per row:
//                       the BF16 output is written directly; several: fp32
//                       partials plus (max, sum) per head.
//   dsa_combine_kernel  merges the chunk partials of a row
//                       (log-sum-exp weights) and writes BF16.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <sstream>
#include <type_traits>

#include "plan.hpp"

namespace dsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
#define DSA_LDS __attribute__((address_space(3)))

constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kWave * kWaves;
constexpr float kLog2e = 1.4426950408889634f;

// ------------------------------------------------------------------ helpers

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier that does not wait for outstanding global/DMA loads
// (a plain __syncthreads would drain the prefetch pipeline). LDS reads and
// writes issued before it are complete once every wave arrives.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// D = 16x16 fp32 += A (16x128 FP8 E4M3) * B (128x16 FP8 E4M3). Lane l holds
// A row l%16 and B column l%16, k = 32*(l/16) + [0, 32) as 32 bytes.
__device__ __forceinline__ f32x4 mfma_fp8(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Four floats -> four FP8 E4M3 codes (round to nearest even), byte i = x_i.
__device__ __forceinline__ int pack_fp8x4(float x0, float x1, float x2, float x3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
}

// x = hi + lo with hi, lo FP8: hi is x rounded to 4 significant bits and lo
// the exactly computed remainder rounded to 4 more. For |x| < 448 the
// remainder is a multiple of x's last bf16 bit and at most 8 of them, so a
// bf16 x (8 significant bits) is represented exactly while lo stays in the
// FP8 normal/subnormal range; otherwise the error is at most half of lo's
// last place (relative 2^-9).
__device__ __forceinline__ void split_fp8x4(float x0, float x1, float x2, float x3,
                                            int& hi, int& lo) {
  hi = pack_fp8x4(x0, x1, x2, x3);
  const f32x2 h01 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
  const f32x2 h23 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
  lo = pack_fp8x4(x0 - h01[0], x1 - h01[1], x2 - h23[0], x3 - h23[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// LDS layout of one staged tile: token-major rows of D bytes; the 16-byte
// chunks of a row are XOR-permuted by the token index so that the 16 tokens
// one MFMA operand read touches, and the 8 rows of one transposing read,
// land in distinct bank groups.
template <int D>
__device__ __forceinline__ int tile_swizzle(int tok) {
  constexpr int kChunks = D / 16;
  constexpr int kMask = (kChunks < 16 ? kChunks : 16) - 1;
  return ((tok & 15) ^ ((tok & 16) >> 1)) & kMask;
}
template <int D>
__device__ __forceinline__ int tile_offset(int tok, int chunk) {
  return tok * D + ((chunk ^ tile_swizzle<D>(tok)) << 4);
}

// ---------------------------------------------------- selection normalisation

constexpr int kSelThreads = 256;
constexpr int kWindowWords = 8192;   // 262144 positions per pass over the row
constexpr int kSelIdsLds = 4096;     // sorted ids kept in LDS when W fits

__device__ __forceinline__ int block_exclusive_scan(int v, int* sh, int* total) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  int x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) sh[w] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int k = 0; k < kSelThreads / kWave; ++k) {
    int s = sh[k];
    all += s;
    if (k < w) before += s;
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

struct SelectArgs {
  const int32_t* sel;
  const int32_t* seq_lens;
  const int32_t* block_tables;
  int32_t* ids;
  uint64_t* offsets;
  int32_t* counts;
  uint64_t cache_stride;
  int width;
  int max_seq_len;
  int bt_stride;
  int block_size;
  int D;
};

__global__ __launch_bounds__(kSelThreads) void dsa_select_kernel(SelectArgs a) {
  __shared__ uint32_t bitmap[kWindowWords];
  __shared__ int32_t ids_lds[kSelIdsLds];
  __shared__ int scan_sh[kSelThreads / kWave];
  const int r = blockIdx.x, tid = threadIdx.x;
  int L = a.seq_lens[r];
  L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
  const int32_t* srow = a.sel + (size_t)r * a.width;
  const int32_t* bt = a.block_tables + (size_t)r * a.bt_stride;
  int32_t* idrow = a.ids + (size_t)r * a.width;
  uint64_t* offrow = a.offsets + (size_t)r * a.width;
  const bool ids_in_lds = a.width <= kSelIdsLds;

  // Phase 1: membership bitmap per window of positions, read back in order.
  int total = 0;
  for (int base = 0; base < L; base += kWindowWords * 32) {
    const int span = min(kWindowWords * 32, L - base);
    const int nwords = (span + 31) >> 5;
    for (int i = tid; i < nwords; i += kSelThreads) bitmap[i] = 0u;
    __syncthreads();
    // a hole (any negative id) or an id outside [0, L) sets nothing
    for (int j = tid; j < a.width; j += kSelThreads) {
      const int t = srow[j];
      if (t >= base && t - base < span)
        atomicOr(&bitmap[(t - base) >> 5], 1u << ((t - base) & 31));
    }
    __syncthreads();
    const int per = (nwords + kSelThreads - 1) / kSelThreads;
    const int w0 = min(tid * per, nwords), w1 = min(w0 + per, nwords);
    int cnt = 0;
    for (int w = w0; w < w1; ++w) cnt += __popc(bitmap[w]);
    int blk_total;
    int pos = total + block_exclusive_scan(cnt, scan_sh, &blk_total);
    for (int w = w0; w < w1; ++w) {
      uint32_t bits = bitmap[w];
      while (bits) {
        const int b = __ffs(bits) - 1;
        bits &= bits - 1;
        const int t = base + (w << 5) + b;
        if (ids_in_lds) ids_lds[pos] = t;
        else idrow[pos] = t;
        ++pos;
      }
    }
    total += blk_total;
    __syncthreads();
  }

  // Phase 2: ids in order -> byte offsets, four independent table lookups
  // in flight per thread.
  for (int i0 = tid; i0 < total; i0 += 4 * kSelThreads) {
    int t[4];
    uint32_t page[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * kSelThreads;
      t[u] = i < total ? (ids_in_lds ? ids_lds[i] : idrow[i]) : 0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      page[u] = i0 + u * kSelThreads < total ? (uint32_t)bt[t[u] / a.block_size] : 0u;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * kSelThreads;
      if (i < total) {
        if (ids_in_lds) idrow[i] = t[u];
        offrow[i] = (uint64_t)page[u] * a.cache_stride +
                    (uint64_t)(t[u] % a.block_size) * (uint64_t)a.D;
      }
    }
  }
  if (tid == 0) a.counts[r] = total;
}

// ------------------------------------------------------------ gather-attend

struct AttendArgs {
  const uint16_t* q;
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const int32_t* counts;
  const uint64_t* offsets;
  uint16_t* out;
  float* part_o;
  float* part_ml;
  int H;
  int width;
  int chunks;
  int chunk_tokens;
  int head_blocks;
  float scale_log2;  // sm_scale * k_scale * log2(e)
  float v_scale;
};

// Value of the lane 16 (resp. 32) apart, and max-reductions over those lane
// pairs, through the cross-row lane swaps (no LDS traffic).
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ int partner_xor32(int x, int lane) {
  const auto r = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
  return (int)((lane & 32) ? r[0] : r[1]);
}

// O^T (16 latent columns x 16 heads) += V^T P^T over 128 tokens, with P given
// as FP8 codes under per-block E8M0 exponents (scale_b) and V unscaled.
__device__ __forceinline__ f32x4 mfma_fp8_pscaled(i32x8 v, i32x8 p, int pscale, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(v, p, c, 0, 0, 0, 127, 0, pscale);
}

// How far (log2 domain) a score may exceed the per-head reference before the
// chunk is recomputed against the exact maximum: weights up to 2^96 keep the
// E8M0 block exponents in range and the fp32 sums (at most 2^96 * 448 * 2048
// per element) finite.
constexpr float kSlack = 96.0f;

// kTS: waves that share one 16-head group and split each tile's tokens
// (1 when the block has 64 heads, 2 for 32, 4 for 16 or fewer).
// kSplitV: V is read from its own buffer (staged next to K).
template <int D, int kTS, bool kSplitV>
__global__ __launch_bounds__(kThreads, 1) void dsa_attend_kernel(AttendArgs a) {
  constexpr int kTile = kSplitV ? 64 : 128;         // tokens per stage
  constexpr int kStages = 2;
  constexpr int kKSteps = (D + 127) / 128;         // QK MFMA steps over the latent width
  constexpr int kDBlocks = D / 16;                 // PV output column blocks
  constexpr int kChunks = D / 16;                  // 16-byte chunks per latent row
  constexpr int kChunkMask = (kChunks < 16 ? kChunks : 16) - 1;
  constexpr int kJ0 = kDBlocks < 16 ? kDBlocks : 16;
  constexpr int kJ1 = kDBlocks / kJ0;              // 2 when D = 512
  constexpr int kTileBytes = kTile * D;
  constexpr int kStageBytes = kTileBytes * (kSplitV ? 2 : 1);
  constexpr int kLanesPerTok = D / 16;
  constexpr int kTokPerInstr = kWave / kLanesPerTok;
  constexpr int kInstrPerWave = kTileBytes / (kWave * 16) / kWaves;
  constexpr int kGroups = kWaves / kTS;            // 16-head groups per workgroup
  constexpr int kNB = kTile / 16 / kTS;            // 16-token blocks per wave per tile (<= 8)
  constexpr int kSlotFloats = kDBlocks * 4 * kWave + 2 * kWave;
  static_assert(kInstrPerWave >= 1, "tile too small for the DMA split");
  static_assert(kNB >= 1 && kNB <= 8, "one PV operand covers 8 blocks of 16 tokens");
  static_assert(kTS == 1 || 2 * kSlotFloats * 4 <= kStages * kStageBytes,
                "merge scratch must fit in the tile buffers");
  static_assert(16 * 7 * D + 256 * ((kKSteps - 1) >> 1) < 65536,
                "K operand offsets must fit the LDS instruction offset field");

  __shared__ __attribute__((aligned(16))) uint8_t smem[kStages * kStageBytes];
  __shared__ uint64_t offs_lds[kMaxChunkTokens];

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int g = lane >> 4, li = lane & 15;

  int wg = blockIdx.x;
  const int c = wg % a.chunks;
  wg /= a.chunks;
  const int hb = wg % a.head_blocks;
  const int r = wg / a.head_blocks;

  const int hg = wave % kGroups, tp = wave / kGroups;
  const int head = hb * kHeadsPerBlock + hg * 16 + li;
  const bool head_ok = head < a.H;

  const int n_row = a.counts[r];
  const int cstart = c * a.chunk_tokens;
  const int n = max(0, min(a.chunk_tokens, n_row - cstart));
  const int ntiles = (n + kTile - 1) / kTile;

  // Byte offsets of this chunk's rows, padded to whole tiles with the last
  // real row (the padding is loaded but weighted by exactly zero).
  const uint64_t* orow = a.offsets + (size_t)r * a.width + cstart;
  for (int i = tid; i < ntiles * kTile; i += kThreads) offs_lds[i] = orow[min(i, n - 1)];

  // ---- query slice of this lane: head li, latent columns 128*ks + 32*g + [0, 32)
  // as two FP8 terms under a per-head power-of-two scale that puts the head's
  // largest |q| in [128, 256).
  i32x8 qhi[kKSteps], qlo[kKSteps];
  float score_scale;
  {
    u32x4 raw[kKSteps][4];
    float amax = 0.f;
    const uint16_t* qrow = a.q + ((size_t)r * a.H + (head_ok ? head : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      const int d0 = 128 * ks + 32 * g;
      const bool ok = head_ok && d0 < D;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        raw[ks][v] = ok ? *(const u32x4*)(qrow + d0 + 8 * v) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(raw[ks][v][e])), fabsf(bf16_hi(raw[ks][v][e]))));
      }
    }
    amax = max_xor32(max_xor16(amax));
    int e = amax > 0.f ? (int)((__float_as_uint(amax) >> 23) & 0xff) - 127 : 0;
    int sh = 7 - e;
    sh = sh < -120 ? -120 : (sh > 120 ? 120 : sh);
    const float qs = __uint_as_float((uint32_t)(127 + sh) << 23);       // 2^sh
    const float qs_inv = __uint_as_float((uint32_t)(127 - sh) << 23);   // 2^-sh
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks)
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const unsigned w0 = raw[ks][v][2 * h2], w1 = raw[ks][v][2 * h2 + 1];
          int hi, lo;
          split_fp8x4(bf16_lo(w0) * qs, bf16_hi(w0) * qs, bf16_lo(w1) * qs, bf16_hi(w1) * qs,
                      hi, lo);
          qhi[ks][2 * v + h2] = hi;
          qlo[ks][2 * v + h2] = lo;
        }
    score_scale = a.scale_log2 * qs_inv;
  }
  __syncthreads();

  auto issue_tile = [&](int tile, int stage) {
    uint8_t* sbase = smem + stage * kStageBytes;
#pragma unroll
    for (int k = 0; k < kInstrPerWave; ++k) {
      const int gi = wave * kInstrPerWave + k;
      const int tt = gi * kTokPerInstr + lane / kLanesPerTok;
      const int ci = lane % kLanesPerTok;
      const uint64_t off = offs_lds[tile * kTile + tt] +
                           (uint64_t)((ci ^ tile_swizzle<D>(tt)) << 4);
      __builtin_amdgcn_global_load_lds(a.k_cache + off,
                                       (DSA_LDS void*)(sbase + gi * (kWave * 16)),
                                       16, 0, 0);
      if constexpr (kSplitV)
        __builtin_amdgcn_global_load_lds(
            a.v_cache + off, (DSA_LDS void*)(sbase + kTileBytes + gi * (kWave * 16)),
            16, 0, 0);
    }
  };

  // K operand addresses. Token 16*b + li, chunk 8*ks + 2*g + h sits at chunk
  // position (chunk ^ swizzle); with swizzle = li ^ 8*(b & 1) that position is
  // 16*(ks >> 1) + (((2*g + h) ^ li) ^ 8*((ks ^ b) & 1)), so four per-lane
  // offsets plus compile-time immediates cover every read.
  int kofs[2][2];
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      kofs[p][h] = li * D + 16 * ((((2 * g + h) ^ li) ^ (8 * p)) & kChunkMask);

  // V operand rows: read q (0..3) of a PV operand covers operand bytes
  // 8q..8q+7, i.e. block slots 2q and 2q+1; lanes 2k and 2k+1 of a 16-lane
  // group supply row k (halves 0 and 1).
  int vrow[4], vswz[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int rrow = li >> 1;
    const int slot = 2 * q + (rrow >> 2);
    const int b = slot < kNB ? tp + kTS * slot : tp;   // slots past this wave's blocks weigh zero
    const int tok = 16 * b + 4 * g + (rrow & 3);
    vrow[q] = tok * D + 8 * (li & 1);
    vswz[q] = tile_swizzle<D>(tok) << 4;
  }

  // The accumulators are touched only by the matrix cores inside the tile
  // loop: softmax weights are taken against a fixed per-head reference (the
  // first tile's max). Each 16-token x 2-lane-group block of weights carries
  // its own E8M0 exponent, so a later score may exceed the reference by up
  // to 2^kSlack without leaving the FP8 range or fp32 accumulation. Should a
  // score ever exceed it by more (only with pathological inputs), the chunk
  // is recomputed with the reference set to the exact maximum seen.
  DSA_LDS uint8_t* lds = (DSA_LDS uint8_t*)smem;
  __shared__ int redo_flag;
  f32x4 O[kDBlocks];
  float l_part = 0.f;       // this lane's share of sum_t 2^(s_t - m_ref)
  float m_ref = -INFINITY;  // reference of this head's scores (log2 domain)
  float m_seen = -INFINITY; // exact max of this head's scores so far

  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int jd = 0; jd < kDBlocks; ++jd) O[jd] = f32x4{0.f, 0.f, 0.f, 0.f};
    l_part = 0.f;
    if (pass == 1) m_ref = m_seen;
    bool overflow = false;
    if (tid == 0) redo_flag = 0;

    if (ntiles > 0) issue_tile(0, 0);
    for (int it = 0; it < ntiles; ++it) {
      wait_vmcnt<0>();
      barrier_lds();  // tile `it` is in LDS for every wave; tile it-1 is consumed
      if (it + 1 < ntiles) issue_tile(it + 1, (it + 1) % kStages);

      const int stage_off = (it % kStages) * kStageBytes;
      const DSA_LDS uint8_t* kt = lds + stage_off;
      const DSA_LDS uint8_t* vt = kSplitV ? kt + kTileBytes : kt;

      // ---- S^T = K Q^T, K operands prefetched two MFMA steps ahead
      constexpr int kSteps = kNB * kKSteps;
      auto load_k = [&](int s) -> i32x8 {
        const int k = s / kKSteps, ks = s % kKSteps;
        const int b = tp + kTS * k;
        i32x8 kop = {0, 0, 0, 0, 0, 0, 0, 0};
        if (128 * ks + 32 * g < D) {
          const int p = (ks ^ b) & 1;
          const DSA_LDS uint8_t* base = kt + 16 * b * D + 256 * (ks >> 1);
          const u32x4 lo = *(const DSA_LDS u32x4*)(base + kofs[p][0]);
          const u32x4 hi = *(const DSA_LDS u32x4*)(base + kofs[p][1]);
          kop = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                      (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
        return kop;
      };
      f32x4 S[kNB];
      i32x8 kbuf[3];
      kbuf[0] = load_k(0);
      if (kSteps > 1) kbuf[1] = load_k(1);
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        const int k = s / kKSteps, ks = s % kKSteps;
        if (s + 2 < kSteps) kbuf[(s + 2) % 3] = load_k(s + 2);
        __builtin_amdgcn_sched_barrier(0);
        if (ks == 0) S[k] = f32x4{0.f, 0.f, 0.f, 0.f};
        S[k] = mfma_fp8(kbuf[s % 3], qhi[ks], S[k]);
        S[k] = mfma_fp8(kbuf[s % 3], qlo[ks], S[k]);
        __builtin_amdgcn_sched_barrier(0);
      }

      // ---- weights; lane holds head li, tokens 16*b + 4*g + i. Slots 0-3 and
      // 4-7 of the lane, each joined with the lane 16 apart, are the blocks
      // that share one FP8 exponent.
      const int nvalid = n - it * kTile;
      if (__builtin_expect(nvalid < kTile, 0)) {
#pragma unroll
        for (int k = 0; k < kNB; ++k)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (16 * (tp + kTS * k) + 4 * g + i >= nvalid) S[k][i] = -INFINITY;
      }
      float mlo = -INFINITY, mhi = -INFINITY;
#pragma unroll
      for (int k = 0; k < kNB; ++k) {
        const float m4 = fmaxf(fmaxf(S[k][0], S[k][1]), fmaxf(S[k][2], S[k][3]));
        if (k < 4) mlo = fmaxf(mlo, m4);
        else mhi = fmaxf(mhi, m4);
      }
      mlo = max_xor16(mlo) * score_scale;   // score_scale > 0
      mhi = max_xor16(mhi) * score_scale;
      const float tmax = max_xor32(fmaxf(mlo, mhi));
      m_seen = fmaxf(m_seen, tmax);
      if (m_ref == -INFINITY) m_ref = tmax;   // first tile of pass 0
      overflow |= tmax > m_ref + kSlack;
      const float mbase = m_ref == -INFINITY ? 0.f : m_ref;
      // block exponents: the block's largest weight maps to [128, 256)
      int elo = mlo == -INFINITY ? 0 : (int)floorf(mlo - mbase);
      int ehi = mhi == -INFINITY ? 0 : (int)floorf(mhi - mbase);
      elo = elo < -100 ? -100 : (elo > 100 ? 100 : elo);
      ehi = ehi < -100 ? -100 : (ehi > 100 ? 100 : ehi);
      const float blo = mbase + (float)(elo - 7), bhi = mbase + (float)(ehi - 7);
      i32x8 phi = {0, 0, 0, 0, 0, 0, 0, 0}, plo = {0, 0, 0, 0, 0, 0, 0, 0};
      float slo = 0.f, shi = 0.f;
#pragma unroll
      for (int k = 0; k < kNB; ++k) {
        const float bsub = k < 4 ? blo : bhi;
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = fast_exp2(fmaf(S[k][i], score_scale, -bsub));
        if (k < 4) slo += (p[0] + p[1]) + (p[2] + p[3]);
        else shi += (p[0] + p[1]) + (p[2] + p[3]);
        int hi, lo;
        split_fp8x4(p[0], p[1], p[2], p[3], hi, lo);
        phi[k] = hi;
        plo[k] = lo;
      }
      l_part += slo * __uint_as_float((uint32_t)(127 + elo - 7) << 23) +
                shi * __uint_as_float((uint32_t)(127 + ehi - 7) << 23);
      // E8M0 scale operand: lane group 0 scales bytes 0-15 of groups {0,1},
      // group 1 bytes 0-15 of {2,3}, group 2 bytes 16-31 of {0,1}, group 3
      // bytes 16-31 of {2,3}.
      const int epack = (elo + 120) | ((ehi + 120) << 8);
      const int eother = partner_xor32(epack, lane);
      const int psc = g == 0 ? (epack & 0xff)
                    : g == 1 ? (eother & 0xff)
                    : g == 2 ? (eother >> 8) : (epack >> 8);

      // ---- O^T += V^T P^T over the tile (one 128-token operand per MFMA),
      // V operands of the next column group prefetched.
      auto load_v = [&](int j0, i32x8 (&vop)[kJ1]) {
        int vaddr[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) vaddr[q] = ((j0 << 4) ^ vswz[q]) + vrow[q];
#pragma unroll
        for (int j1 = 0; j1 < kJ1; ++j1)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (DSA_LDS i32x2*)(vt + vaddr[q] + 256 * j1));
            vop[j1][2 * q] = x.x;
            vop[j1][2 * q + 1] = x.y;
          }
      };
      i32x8 vbuf[2][kJ1];
      load_v(0, vbuf[0]);
#pragma unroll
      for (int j0 = 0; j0 < kJ0; ++j0) {
        if (j0 + 1 < kJ0) load_v(j0 + 1, vbuf[(j0 + 1) % 2]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j1 = 0; j1 < kJ1; ++j1) {
          const int jd = 16 * j1 + j0;
          O[jd] = mfma_fp8_pscaled(vbuf[j0 % 2][j1], phi, psc, O[jd]);
          O[jd] = mfma_fp8_pscaled(vbuf[j0 % 2][j1], plo, psc, O[jd]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // Recompute the chunk only if some wave saw a score beyond the slack.
    if (pass == 0) {
      if (__any(overflow) && lane == 0) redo_flag = 1;
      __syncthreads();
      const bool redo = redo_flag != 0;
      __syncthreads();
      if (!redo) break;
    }
  }

  // Sum of this head's weights over the four lane groups.
  float l_run = sum_xor32(sum_xor16(l_part));
  float m_run = ntiles > 0 ? m_ref : -INFINITY;

  // Waves that split the tokens of one head group merge (max, sum, O).
  if constexpr (kTS > 1) {
    __syncthreads();  // tiles fully consumed; no DMA outstanding
    float* scratch = (float*)smem;
#pragma unroll
    for (int step = kTS / 2; step >= 1; step /= 2) {
      if (tp >= step && tp < 2 * step) {
        float* slot = scratch + (hg * step + (tp - step)) * kSlotFloats;
#pragma unroll
        for (int jd = 0; jd < kDBlocks; ++jd)
#pragma unroll
          for (int i = 0; i < 4; ++i) slot[(jd * 4 + i) * kWave + lane] = O[jd][i];
        slot[kDBlocks * 4 * kWave + lane] = m_run;
        slot[kDBlocks * 4 * kWave + kWave + lane] = l_run;
      }
      __syncthreads();
      if (tp < step) {
        const float* slot = scratch + (hg * step + tp) * kSlotFloats;
        const float mb = slot[kDBlocks * 4 * kWave + lane];
        const float lb = slot[kDBlocks * 4 * kWave + kWave + lane];
        const float mn = fmaxf(m_run, mb);
        const float mu = mn == -INFINITY ? 0.f : mn;
        const float fa = fast_exp2(m_run - mu), fb = fast_exp2(mb - mu);
#pragma unroll
        for (int jd = 0; jd < kDBlocks; ++jd)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            O[jd][i] = O[jd][i] * fa + slot[(jd * 4 + i) * kWave + lane] * fb;
        l_run = l_run * fa + lb * fb;
        m_run = mn;
      }
      __syncthreads();
    }
  }

  if (tp != 0 || !head_ok) return;
  // Lane holds O^T rows d = 16*jd + 4*g + i for head li.
  if (a.chunks == 1) {
    const float inv = l_run > 0.f ? a.v_scale / l_run : 0.f;
    uint16_t* orow_out = a.out + ((size_t)r * a.H + head) * D;
#pragma unroll
    for (int jd = 0; jd < kDBlocks; ++jd) {
      bf16x4 v = {(__bf16)(O[jd][0] * inv), (__bf16)(O[jd][1] * inv),
                  (__bf16)(O[jd][2] * inv), (__bf16)(O[jd][3] * inv)};
      *(bf16x4*)(orow_out + 16 * jd + 4 * g) = v;
    }
  } else {
    const size_t ph = ((size_t)r * a.chunks + c) * a.H + head;
    float* po = a.part_o + ph * D;
#pragma unroll
    for (int jd = 0; jd < kDBlocks; ++jd) *(f32x4*)(po + 16 * jd + 4 * g) = O[jd];
    if (g == 0) {
      a.part_ml[ph * 2 + 0] = m_run;
      a.part_ml[ph * 2 + 1] = l_run;
    }
  }
}

// ------------------------------------------------------------------ combine

struct CombineArgs {
  const float* part_o;
  const float* part_ml;
  uint16_t* out;
  int H;
  int chunks;
  int head_groups;  // blocks of kCombineHeads per row
  float v_scale;
};

template <int D>
__global__ __launch_bounds__(256) void dsa_combine_kernel(CombineArgs a) {
  constexpr int kTPH = D / 8;        // threads per head, 8 columns each
  constexpr int kHPB = 256 / kTPH;   // heads per workgroup
  const int r = blockIdx.x / a.head_groups;
  const int head = (blockIdx.x % a.head_groups) * kHPB + threadIdx.x / kTPH;
  if (head >= a.H) return;
  const int d0 = (threadIdx.x % kTPH) * 8;
  float M = -INFINITY;
  for (int c = 0; c < a.chunks; ++c)
    M = fmaxf(M, a.part_ml[(((size_t)r * a.chunks + c) * a.H + head) * 2]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  if (M != -INFINITY) {
    for (int c = 0; c < a.chunks; ++c) {
      const size_t ph = ((size_t)r * a.chunks + c) * a.H + head;
      const float mc = a.part_ml[ph * 2];
      if (mc == -INFINITY) continue;  // empty chunk: nothing was written
      const float w = fast_exp2(mc - M);
      L += w * a.part_ml[ph * 2 + 1];
      const f32x4 x0 = *(const f32x4*)(a.part_o + ph * D + d0);
      const f32x4 x1 = *(const f32x4*)(a.part_o + ph * D + d0 + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i] += w * x0[i];
        acc[4 + i] += w * x1[i];
      }
    }
  }
  const float inv = L > 0.f ? a.v_scale / L : 0.f;
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (__bf16)(acc[i] * inv);
  *(bf16x8*)(a.out + ((size_t)r * a.H + head) * D + d0) = v;
}

// ------------------------------------------------------------------ launch

template <int D, int kTS>
hipError_t launch_attend_ts(bool split_v, dim3 grid, hipStream_t st, const AttendArgs& args) {
  if (split_v)
    hipLaunchKernelGGL((dsa_attend_kernel<D, kTS, true>), grid, dim3(kThreads), 0, st, args);
  else
    hipLaunchKernelGGL((dsa_attend_kernel<D, kTS, false>), grid, dim3(kThreads), 0, st, args);
  return hipGetLastError();
}

template <int D>
hipError_t launch_attend_d(int ts, bool split_v, dim3 grid, hipStream_t st,
                           const AttendArgs& args) {
  switch (ts) {
    case 1: return launch_attend_ts<D, 1>(split_v, grid, st, args);
    case 2: return launch_attend_ts<D, 2>(split_v, grid, st, args);
    default: return launch_attend_ts<D, 4>(split_v, grid, st, args);
  }
}

template <int D>
hipError_t launch_combine_d(int R, hipStream_t st, CombineArgs args) {
  constexpr int kHPB = 256 / (D / 8);
  args.head_groups = (args.H + kHPB - 1) / kHPB;
  hipLaunchKernelGGL((dsa_combine_kernel<D>), dim3(R * args.head_groups), dim3(256), 0, st, args);
  return hipGetLastError();
}

// Token-split factor of a head block: how many waves share one 16-head group.
int token_split(int heads_in_block) {
  const int groups = (heads_in_block + 15) / 16;
  if (groups >= 3) return 1;
  if (groups == 2) return 2;
  return 4;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

}  // namespace
}  // namespace dsa

extern "C" {

void dsa_decode_plan_destroy(dsa_decode_plan_t plan) {
  if (!plan) return;
  for (void* e : plan->events)
    if (e) (void)hipEventDestroy((hipEvent_t)e);
  delete plan;
}

int dsa_decode_launch(dsa_decode_plan_t plan, const void* q, const void* k_cache,
                      const void* v_cache, const int32_t* block_tables,
                      const int32_t* seq_lens, const int32_t* sel_indices,
                      float k_scale, float v_scale, void* out, void* workspace,
                      size_t workspace_bytes, void* stream) {
  using namespace dsa;
  if (!plan) return fail(DSA_DECODE_ERR_INVALID, "dsa_decode_launch: plan is NULL");
  if (plan->device < 0)
    return fail(DSA_DECODE_ERR_INVALID,
                "dsa_decode_launch: host-only plan (device -1) cannot launch");
  if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !sel_indices || !out)
    return fail(DSA_DECODE_ERR_INVALID, "dsa_decode_launch: NULL device pointer");
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return fail(DSA_DECODE_ERR_INVALID,
                "dsa_decode_launch: q, out, k_cache and v_cache must be 16-byte aligned");
  if (!std::isfinite(k_scale) || !std::isfinite(v_scale))
    return fail(DSA_DECODE_ERR_INVALID, "dsa_decode_launch: k_scale and v_scale must be finite");
  if (!workspace || !aligned(workspace, kWsAlign) || workspace_bytes < plan->ws.total) {
    std::ostringstream m;
    m << "dsa_decode_launch: workspace " << workspace << " of " << workspace_bytes
      << " bytes; need " << plan->ws.total << " bytes, 256-byte aligned";
    return fail(DSA_DECODE_ERR_WORKSPACE, m.str());
  }
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur != plan->device) {
    std::ostringstream m;
    m << "dsa_decode_launch: current HIP device is " << cur << ", plan was made for "
      << plan->device;
    return fail(DSA_DECODE_ERR_DEVICE, m.str());
  }

  const dsa_decode_params& p = plan->p;
  hipStream_t st = (hipStream_t)stream;
  uint8_t* ws = (uint8_t*)workspace;
  int32_t* ids = (int32_t*)(ws + plan->ws.ids);
  uint64_t* offs = (uint64_t*)(ws + plan->ws.offsets);
  int32_t* counts = (int32_t*)(ws + plan->ws.counts);

  hipEvent_t* ev = nullptr;
  if (plan->timing_count < plan->timing_capacity)
    ev = (hipEvent_t*)&plan->events[4 * plan->timing_count++];
  if (ev) (void)hipEventRecord(ev[0], st);

  SelectArgs sa;
  sa.sel = sel_indices;
  sa.seq_lens = seq_lens;
  sa.block_tables = block_tables;
  sa.ids = ids;
  sa.offsets = offs;
  sa.counts = counts;
  sa.cache_stride = p.cache_stride_bytes;
  sa.width = p.sel_width;
  sa.max_seq_len = p.max_seq_len;
  sa.bt_stride = p.block_table_stride;
  sa.block_size = p.block_size;
  sa.D = p.kv_lora_rank;
  hipLaunchKernelGGL(dsa_select_kernel, dim3(p.num_rows), dim3(kSelThreads), 0, st, sa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(DSA_DECODE_ERR_LAUNCH,
                std::string("dsa_decode_launch: selection kernel: ") + hipGetErrorString(e));
  if (ev) (void)hipEventRecord(ev[1], st);

  AttendArgs aa;
  aa.q = (const uint16_t*)q;
  aa.k_cache = (const uint8_t*)k_cache;
  aa.v_cache = (const uint8_t*)v_cache;
  aa.counts = counts;
  aa.offsets = offs;
  aa.out = (uint16_t*)out;
  aa.part_o = plan->chunks > 1 ? (float*)(ws + plan->ws.part_o) : nullptr;
  aa.part_ml = plan->chunks > 1 ? (float*)(ws + plan->ws.part_ml) : nullptr;
  aa.H = p.num_q_heads;
  aa.width = p.sel_width;
  aa.chunks = plan->chunks;
  aa.chunk_tokens = plan->chunk_tokens;
  aa.head_blocks = plan->head_blocks;
  aa.scale_log2 = p.sm_scale * k_scale * kLog2e;
  aa.v_scale = v_scale;
  const int ts = token_split(p.num_q_heads < kHeadsPerBlock ? p.num_q_heads : kHeadsPerBlock);
  const bool split_v = k_cache != v_cache;
  const dim3 grid(p.num_rows * plan->head_blocks * plan->chunks);
  switch (p.kv_lora_rank) {
    case 64: e = launch_attend_d<64>(ts, split_v, grid, st, aa); break;
    case 128: e = launch_attend_d<128>(ts, split_v, grid, st, aa); break;
    case 256: e = launch_attend_d<256>(ts, split_v, grid, st, aa); break;
    default: e = launch_attend_d<512>(ts, split_v, grid, st, aa); break;
  }
  if (e != hipSuccess)
    return fail(DSA_DECODE_ERR_LAUNCH,
                std::string("dsa_decode_launch: attend kernel: ") + hipGetErrorString(e));
  if (ev) (void)hipEventRecord(ev[2], st);

  if (plan->chunks > 1) {
    CombineArgs ca;
    ca.part_o = aa.part_o;
    ca.part_ml = aa.part_ml;
    ca.out = (uint16_t*)out;
    ca.H = p.num_q_heads;
    ca.chunks = plan->chunks;
    ca.head_groups = 0;
    ca.v_scale = v_scale;
    switch (p.kv_lora_rank) {
      case 64: e = launch_combine_d<64>(p.num_rows, st, ca); break;
      case 128: e = launch_combine_d<128>(p.num_rows, st, ca); break;
      case 256: e = launch_combine_d<256>(p.num_rows, st, ca); break;
      default: e = launch_combine_d<512>(p.num_rows, st, ca); break;
    }
    if (e != hipSuccess)
      return fail(DSA_DECODE_ERR_LAUNCH,
                  std::string("dsa_decode_launch: combine kernel: ") + hipGetErrorString(e));
  }
  if (ev) (void)hipEventRecord(ev[3], st);
  return DSA_DECODE_OK;
}

int dsa_decode_read_selection(dsa_decode_plan_t plan, const void* workspace,
                              size_t workspace_bytes, int32_t* ids, int32_t* counts,
                              uint64_t* offsets, void* stream) {
  using namespace dsa;
  if (!plan || !workspace)
    return fail(DSA_DECODE_ERR_INVALID, "dsa_decode_read_selection: NULL plan or workspace");
  if (plan->device < 0)
    return fail(DSA_DECODE_ERR_INVALID, "dsa_decode_read_selection: host-only plan");
  if (workspace_bytes < plan->ws.total)
    return fail(DSA_DECODE_ERR_WORKSPACE, "dsa_decode_read_selection: workspace too small");
  const uint8_t* ws = (const uint8_t*)workspace;
  const size_t RW = (size_t)plan->p.num_rows * plan->p.sel_width;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (ids && e == hipSuccess)
    e = hipMemcpyAsync(ids, ws + plan->ws.ids, RW * sizeof(int32_t), hipMemcpyDeviceToDevice, st);
  if (counts && e == hipSuccess)
    e = hipMemcpyAsync(counts, ws + plan->ws.counts, plan->p.num_rows * sizeof(int32_t),
                       hipMemcpyDeviceToDevice, st);
  if (offsets && e == hipSuccess)
    e = hipMemcpyAsync(offsets, ws + plan->ws.offsets, RW * sizeof(uint64_t),
                       hipMemcpyDeviceToDevice, st);
  if (e != hipSuccess)
    return fail(DSA_DECODE_ERR_LAUNCH,
                std::string("dsa_decode_read_selection: ") + hipGetErrorString(e));
  return DSA_DECODE_OK;
}

int dsa_decode_timing_begin(dsa_decode_plan_t plan, int32_t max_launches) {
  using namespace dsa;
  if (!plan || plan->device < 0 || max_launches <= 0 || max_launches > 1000000)
    return fail(DSA_DECODE_ERR_INVALID, "dsa_decode_timing_begin: bad plan or count");
  for (void* e : plan->events)
    if (e) (void)hipEventDestroy((hipEvent_t)e);
  plan->events.assign((size_t)4 * max_launches, nullptr);
  for (auto& e : plan->events) {
    hipEvent_t h;
    if (hipEventCreate(&h) != hipSuccess)
      return fail(DSA_DECODE_ERR_DEVICE, "dsa_decode_timing_begin: hipEventCreate failed");
    e = (void*)h;
  }
  plan->timing_capacity = max_launches;
  plan->timing_count = 0;
  return DSA_DECODE_OK;
}

int dsa_decode_timing_end(dsa_decode_plan_t plan, float* kernel_ms, int32_t* launches) {
  using namespace dsa;
  if (!plan || !kernel_ms || !launches)
    return fail(DSA_DECODE_ERR_INVALID, "dsa_decode_timing_end: NULL argument");
  kernel_ms[0] = kernel_ms[1] = kernel_ms[2] = 0.f;
  *launches = plan->timing_count;
  int status = DSA_DECODE_OK;
  for (int i = 0; i < plan->timing_count; ++i) {
    hipEvent_t* ev = (hipEvent_t*)&plan->events[4 * i];
    if (hipEventSynchronize(ev[3]) != hipSuccess) {
      status = fail(DSA_DECODE_ERR_DEVICE, "dsa_decode_timing_end: hipEventSynchronize failed");
      break;
    }
    for (int k = 0; k < 3; ++k) {
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, ev[k], ev[k + 1]) == hipSuccess) kernel_ms[k] += ms;
    }
  }
  for (void* e : plan->events)
    if (e) (void)hipEventDestroy((hipEvent_t)e);
  plan->events.clear();
  plan->timing_capacity = 0;
  plan->timing_count = 0;
  return status;
}

}  // extern "C"
