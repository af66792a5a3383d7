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
//                       sorted set). 64-token tiles of latent rows are DMA'd
//                       straight into LDS, three deep. Each wave owns 16
//                       heads: S^T = K Q^T and O^T = V^T P^T run on bf16
//                       MFMA (16x16x32) with the FP8 rows converted to bf16
//                       on the LDS->register path; the V operand comes from
//                       ds_read_tr8_b64, which hands each lane 8 tokens of
//                       one latent column. Online softmax in the exp2 domain.
//                       One chunk: the BF16 output is written directly;
//                       several: fp32 partials plus (max, sum) per head.
//   dsa_combine_kernel  merges the chunk partials of a row
//                       (log-sum-exp weights) and writes BF16.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <sstream>

#include "plan.hpp"

namespace dsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
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

// 8 FP8 E4M3FN codes (two dwords, little-endian byte order) -> 8 bf16.
// The conversion is exact: every finite E4M3FN value is a bf16 value.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(unsigned lo, unsigned hi) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  bf16x8 r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  return r;
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// LDS layout of one staged tile: token-major rows of D bytes; the 16-byte
// chunks of a row are XOR-permuted by the token index so that the 16 tokens
// an MFMA reads at one logical column land in distinct bank groups.
template <int D>
__device__ __forceinline__ int tile_swizzle(int tok) {
  constexpr int kChunks = D / 16;
  constexpr int kMask = (kChunks < 16 ? kChunks : 16) - 1;
  return tok & kMask;
}
template <int D>
__device__ __forceinline__ int tile_offset(int tok, int chunk) {
  return tok * D + ((chunk ^ tile_swizzle<D>(tok)) << 4);
}

// ---------------------------------------------------- selection normalisation

constexpr int kSelThreads = 256;
constexpr int kWindowWords = 8192;  // 262144 positions per pass over the row

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
  __shared__ int scan_sh[kSelThreads / kWave];
  const int r = blockIdx.x, tid = threadIdx.x;
  int L = a.seq_lens[r];
  L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
  const int32_t* srow = a.sel + (size_t)r * a.width;
  const int32_t* bt = a.block_tables + (size_t)r * a.bt_stride;
  int32_t* idrow = a.ids + (size_t)r * a.width;
  uint64_t* offrow = a.offsets + (size_t)r * a.width;
  int total = 0;
  for (int base = 0; base < L; base += kWindowWords * 32) {
    const int span = min(kWindowWords * 32, L - base);
    const int nwords = (span + 31) >> 5;
    for (int i = tid; i < nwords; i += kSelThreads) bitmap[i] = 0u;
    __syncthreads();
    // membership: a hole (any negative id) or an id outside [0, L) sets nothing
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
        idrow[pos] = t;
        const uint32_t page = (uint32_t)bt[t / a.block_size];
        offrow[pos] = (uint64_t)page * a.cache_stride +
                      (uint64_t)(t % a.block_size) * (uint64_t)a.D;
        ++pos;
      }
    }
    total += blk_total;
    __syncthreads();
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

// kTS: waves that share one 16-head group and split each tile's tokens
// (1 when the block has 64 heads, 2 for 32, 4 for 16 or fewer).
template <int D, int kTS, bool kSplitV, int kStages>
__global__ __launch_bounds__(kThreads, 1) void dsa_attend_kernel(AttendArgs a) {
  constexpr int kSteps = D / 32;          // QK MFMA steps over the latent width
  constexpr int kReads = D / 64;          // 16-byte LDS reads per lane per token
  constexpr int kDBlocks = D / 16;        // PV output column blocks
  constexpr int kTileBytes = kTileTokens * D;
  constexpr int kStageBytes = kTileBytes * (kSplitV ? 2 : 1);
  constexpr int kLanesPerTok = D / 16;
  constexpr int kTokPerInstr = kWave / kLanesPerTok;
  constexpr int kInstrPerWave = kTileBytes / (kWave * 16) / kWaves;
  constexpr int kLoadsPerTile = kInstrPerWave * (kSplitV ? 2 : 1);
  constexpr int kGroups = kWaves / kTS;   // 16-head groups per workgroup
  constexpr int kNB = 4 / kTS;            // 16-token blocks per wave per tile
  constexpr int kSlotFloats = kDBlocks * 4 * kWave + 2 * kWave;
  static_assert(kInstrPerWave >= 1, "tile too small for the DMA split");
  static_assert(kStages >= 2 && kStages <= 4, "pipeline depth");
  static_assert(kTS == 1 || 2 * kSlotFloats * 4 <= kStages * kStageBytes,
                "merge scratch must fit in the tile buffers");

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
  const int ntiles = (n + kTileTokens - 1) / kTileTokens;

  // Byte offsets of this chunk's rows, padded to whole tiles with the last
  // real row (the padding is loaded but weighted by exactly zero).
  const uint64_t* orow = a.offsets + (size_t)r * a.width + cstart;
  for (int i = tid; i < ntiles * kTileTokens; i += kThreads)
    offs_lds[i] = orow[min(i, n - 1)];

  // This lane's query slice, the B operand of S^T = K Q^T: step j = 2*rr + hh
  // covers latent columns 64*rr + 16*g + 8*hh + [0, 8).
  bf16x8 qv[kSteps];
  {
    const uint16_t* qrow = a.q + ((size_t)r * a.H + (head_ok ? head : 0)) * D;
#pragma unroll
    for (int rr = 0; rr < kReads; ++rr)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (head_ok) v = *(const u32x4*)(qrow + 64 * rr + 16 * g + 8 * hh);
        qv[2 * rr + hh] = __builtin_bit_cast(bf16x8, v);
      }
  }
  __syncthreads();

  auto issue_tile = [&](int tile, int stage) {
    uint8_t* sbase = smem + stage * kStageBytes;
#pragma unroll
    for (int k = 0; k < kInstrPerWave; ++k) {
      const int gi = wave * kInstrPerWave + k;
      const int tt = gi * kTokPerInstr + lane / kLanesPerTok;
      const int ci = lane % kLanesPerTok;
      const uint64_t off = offs_lds[tile * kTileTokens + tt] +
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

  f32x4 O[kDBlocks];
#pragma unroll
  for (int jd = 0; jd < kDBlocks; ++jd) O[jd] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // running max of this head's scores (log2 domain)
  float l_part = 0.f;       // this lane's share of the running sum

  for (int s = 0; s < kStages - 1 && s < ntiles; ++s) issue_tile(s, s);

  for (int it = 0; it < ntiles; ++it) {
    // Tiles issued after this one: min(kStages - 2, ntiles - 1 - it).
    const int ahead = min(kStages - 2, ntiles - 1 - it);
    if (ahead >= 2) wait_vmcnt<2 * kLoadsPerTile>();
    else if (ahead == 1) wait_vmcnt<kLoadsPerTile>();
    else wait_vmcnt<0>();
    barrier_lds();  // every wave's rows of tile `it` are in LDS; tile it-1 is consumed
    if (it + kStages - 1 < ntiles) issue_tile(it + kStages - 1, (it + kStages - 1) % kStages);

    const uint8_t* kt = smem + (it % kStages) * kStageBytes;
    const uint8_t* vt = kSplitV ? kt + kTileBytes : kt;

    // ---- S^T = K Q^T for this wave's 16-token blocks
    f32x4 S[kNB];
#pragma unroll
    for (int k = 0; k < kNB; ++k) {
      const int tok = 16 * (tp + kTS * k) + li;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int rr = 0; rr < kReads; ++rr) {
        const u32x4 kv = *(const u32x4*)(kt + tile_offset<D>(tok, 4 * rr + g));
        acc = mfma16(fp8x8_to_bf16x8(kv.x, kv.y), qv[2 * rr], acc);
        acc = mfma16(fp8x8_to_bf16x8(kv.z, kv.w), qv[2 * rr + 1], acc);
      }
      S[k] = acc;
    }

    // ---- online softmax; lane holds head li, tokens 16*b + 4*g + i
    const int tbase = it * kTileTokens;
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < kNB; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = tbase + 16 * (tp + kTS * k) + 4 * g + i;
        const float s = tok < n ? S[k][i] * a.scale_log2 : -INFINITY;
        S[k][i] = s;
        mx = fmaxf(mx, s);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int k = 0; k < kNB; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = fast_exp2(S[k][i] - m_use);
        S[k][i] = p;
        psum += p;
      }
    l_part = l_part * alpha + psum;
#pragma unroll
    for (int jd = 0; jd < kDBlocks; ++jd) O[jd] *= alpha;

    // ---- O^T += V^T P^T, 32 tokens (two 16-token blocks) per MFMA
#pragma unroll
    for (int pp = 0; pp < (kNB + 1) / 2; ++pp) {
      const int k0 = 2 * pp, k1 = 2 * pp + 1;
      const bool has1 = k1 < kNB;
      const int b0 = tp + kTS * k0;
      const int b1 = has1 ? tp + kTS * k1 : b0;
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pb[e] = (__bf16)S[k0][e];
        pb[4 + e] = has1 ? (__bf16)S[k1 < kNB ? k1 : k0][e] : (__bf16)0.f;
      }
      // transposing read: lanes 2k, 2k+1 of a 16-lane group address the two
      // 8-byte halves of row k; lane li receives column li of all 8 rows.
      const int krow = li >> 1;
      const int vtok = (krow < 4 ? 16 * b0 : 16 * b1) + 4 * g + (krow & 3);
      const int half = (li & 1) * 8;
#pragma unroll
      for (int jd = 0; jd < kDBlocks; ++jd) {
        const i32x2 raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (DSA_LDS i32x2*)(vt + tile_offset<D>(vtok, jd) + half));
        O[jd] = mfma16(fp8x8_to_bf16x8((unsigned)raw.x, (unsigned)raw.y), pb, O[jd]);
      }
    }
  }

  // Sum of this head's weights over the four lane groups.
  l_part += __shfl_xor(l_part, 16);
  l_part += __shfl_xor(l_part, 32);
  float l_run = l_part;

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
    hipLaunchKernelGGL((dsa_attend_kernel<D, kTS, true, 2>), grid, dim3(kThreads), 0, st, args);
  else
    hipLaunchKernelGGL((dsa_attend_kernel<D, kTS, false, 3>), grid, dim3(kThreads), 0, st, args);
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
