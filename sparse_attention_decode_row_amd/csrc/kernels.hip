// gfx950 kernel and launcher of the selected-index NoPE MLA paged decode.
//
// What is computed is defined on the pages (cited by title):
//   [attend]   "spark_model/layers/glm5next_dsa/attend.rs"
//   [decode_k] "metrale_model_arch/glm5next_dsa/layer/decode_k.rs"
//   [build]    "spark_model/layers/glm5next_dsa/build.rs"
// How it is computed is this library's own design for CDNA4 (wave64, FP8
// matrix cores, 160 KiB LDS, LDS DMA, transposing LDS reads). One kernel does
// the whole decode. A workgroup owns one (row, block of up to 32 heads, chunk
// of the row's selected set) and runs eight waves: per 16-head group two
// scoring waves, and four PV waves shared by the groups.
//
//   1. selection   the row's ids become a set through an LDS bitmap over
//                  [0, seq_len): holes, repeats and out-of-range ids vanish
//                  ([attend] module doc, "Why this is not the masked kernel").
//                  The workgroup keeps the ascending ids whose rank falls in
//                  its chunk and translates each through the block table to
//                  the index of its FP8 latent row ([decode_k], slot of a
//                  position).
//   2. gather      64-token tiles of latent rows are DMA'd straight from HBM
//                  into LDS (four buffers: one tile scored, one accumulated,
//                  two in flight).
//   3. attend      both contractions run on the FP8 matrix cores (16x16x128,
//                  fp32 accumulation) over the cached bytes as they are:
//                    S^T = K Q^T   the two scoring waves of a head group each
//                                  score half of the tile's tokens. Q (bf16)
//                                  enters as an exact sum of two FP8 terms
//                                  under a per-head power-of-two scale;
//                    O^T = V^T P^T each PV wave accumulates a quarter of the
//                                  latent columns, for every head group, over
//                                  all of the tile's tokens, one tile behind
//                                  the scoring. The softmax weights enter as
//                                  two FP8 terms (relative error <= 2^-9,
//                                  below bf16's 2^-8) under an E8M0 exponent
//                                  per 16-token block and head, exchanged
//                                  through LDS; V comes from
//                                  ds_read_b64_tr_b8, which hands each lane 8
//                                  tokens of one latent column.
//                  Weights are taken against a fixed per-head reference (the
//                  first tile's max); the block exponents absorb later
//                  growth, so the accumulators are never rescaled.
//   4. merge       one chunk: BF16 output directly. Several: fp32 partials
//                  plus (reference, weight sum) per head, and the last chunk
//                  of the row to finish merges them with log-sum-exp weights
//                  ([attend], the split softmax and its combine).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <sstream>

#include "plan.hpp"

namespace dsa {
namespace {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
#define DSA_LDS __attribute__((address_space(3)))

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// How far (log2 domain) a score may exceed the per-head reference before the
// chunk is recomputed against the exact maximum: weights up to 2^96 keep the
// E8M0 block exponents in range and the fp32 sums (at most 2^96 * 448 * 2048
// per element) finite.
constexpr float kSlack = 96.0f;

// ------------------------------------------------------------------ helpers

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// One 16-byte-per-lane DMA from global memory into LDS: lane l's 16 bytes
// land at l_base + 16*l. Issued as inline assembly on purpose: the
// compiler's wait-count pass cannot tell when such a transfer completes, and
// with the builtin in a loop it falls back to waiting for every outstanding
// LDS read at each use, which defeats operand prefetching. Completion is
// ordered explicitly here: wait_vmcnt<0>() and a barrier before the tile is
// read. M0 needs one wait state after it is written.
__device__ __forceinline__ void dma16(const void* g, DSA_LDS void* l_base) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)l_base);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(m0v) : "memory", "m0");
}

// Same with 4 bytes per lane: lane l's word lands at l_base + 4*l.
__device__ __forceinline__ void dma4(const void* g, DSA_LDS void* l_base) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)l_base);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(g), "s"(m0v) : "memory", "m0");
}

// Workgroup barrier that does not wait for outstanding global/DMA loads
// (a plain __syncthreads would drain the prefetch pipeline). LDS reads and
// writes issued before it are complete once every wave arrives.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// D = 16x16 fp32 += A (16x128 FP8 E4M3) * B (128x16 FP8 E4M3). Lane l holds
// A row l%16 and B column l%16 as 32 bytes of the k dimension
// (k = 32*(l/16) + byte).
__device__ __forceinline__ f32x4 mfma_fp8(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Same with the B operand under per-lane E8M0 exponents (2^(byte - 127)).
// Lane group 0 (lanes 0-15) scales bytes 0-15 of lane groups 0 and 1, group 1
// bytes 0-15 of groups 2 and 3, group 2 bytes 16-31 of groups 0 and 1, group
// 3 bytes 16-31 of groups 2 and 3 (each lane for its own column).
__device__ __forceinline__ f32x4 mfma_fp8_bscaled(i32x8 a, i32x8 b, int bscale, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, bscale);
}

// Four floats -> four FP8 E4M3 codes (round to nearest even), byte i = x_i.
// (The first conversion writes the low half of a register whose other half
// the second one overwrites, so that register's prior content is irrelevant:
// an empty asm hands it over without a copy of 0.)
__device__ __forceinline__ int pack_fp8x4(float x0, float x1, float x2, float x3) {
  int any;
  asm volatile("" : "=v"(any));
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, any, false);
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
__device__ __forceinline__ float pow2i(int e) {  // 2^e for e in [-126, 127]
  return __uint_as_float((uint32_t)(127 + e) << 23);
}

__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// Device-coherent (agent-scope) scalar store: written through to the level
// shared by all XCDs, so the split partials leave no dirty L2 lines for the
// release fence to write back.
__device__ __forceinline__ void store_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 16-byte device-coherent store (written through to the level all XCDs
// share). Inline assembly: the compiler does not track its completion, so
// the caller waits with wait_vmcnt<0>() before publishing the data; nor does
// it see the store-data hazard (a store of more than 8 bytes reads its data
// registers after issue), so the wait states that let the next instruction
// overwrite them are inside the statement.
__device__ __forceinline__ void store_dev16(float* p, f32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" :: "v"(p), "v"(v) : "memory");
}

// Device-scope (coherent) loads of what other workgroups published with
// device-scope stores: they read past any stale copy in this CU's or this
// XCD's caches, so the reader needs no cache invalidation.
__device__ __forceinline__ float load_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x4 load_dev16(const float* p) {
  uint64_t* q = (uint64_t*)const_cast<float*>(p);
  const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return f32x4{__uint_as_float((uint32_t)lo), __uint_as_float((uint32_t)(lo >> 32)),
               __uint_as_float((uint32_t)hi), __uint_as_float((uint32_t)(hi >> 32))};
}

// Maximum of two values that are never NaN, as one median-of-three against
// +inf: the compiler's maximum first quiets each operand (one more
// instruction apiece). The +inf is passed in a register the compiler cannot
// see through, so that the median is not turned back into that maximum.
__device__ __forceinline__ float opaque_inf() {
  float x = INFINITY;
  asm volatile("" : "+v"(x));
  return x;
}
__device__ __forceinline__ float max2(float a, float b, float pinf) {
  return __builtin_amdgcn_fmed3f(a, b, pinf);
}

// Max / sum over lane pairs 16 (resp. 32) apart through the cross-row lane
// swaps (no LDS traffic).
__device__ __forceinline__ float max_xor16(float x, float pinf = INFINITY) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return max2(__uint_as_float(r[0]), __uint_as_float(r[1]), pinf);
}
__device__ __forceinline__ float max_xor32(float x, float pinf = INFINITY) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return max2(__uint_as_float(r[0]), __uint_as_float(r[1]), pinf);
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
// The value held by the lane 32 apart.
__device__ __forceinline__ int partner_xor32(int x, int lane) {
  const auto r = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
  return (int)((lane & 32) ? r[0] : r[1]);
}

// LDS layout of one staged tile: slot-major rows of D bytes; the 16-byte
// chunks of a row are XOR-permuted by the slot index so that the 16 rows one
// MFMA operand read touches, and the 8 rows of one transposing read, land in
// distinct bank groups.
template <int D>
__device__ __forceinline__ int tile_swizzle(int slot) {
  constexpr int kChunks = D / 16;
  constexpr int kMask = (kChunks < 16 ? kChunks : 16) - 1;
  return ((slot & 15) ^ ((slot & 16) >> 1)) & kMask;
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts
// (within rows of 16 lanes) and row broadcasts (across rows); lanes a shift
// leaves without a source, and rows a broadcast does not target, add 0.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return x;
}

struct DecodeArgs {
  const uint16_t* q;
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const int32_t* sel;
  uint16_t* out;
  int32_t* ws_status;    // 0 healthy; 1 once a split merge gave up waiting (outputs NaN until re-init)
  int32_t* ws_ids;       // [R, W] distinct ids, ascending (export only)
  uint64_t* ws_offsets;  // [R, W] their latent-row byte offsets (export only)
  int32_t* ws_counts;    // [R] (export only)
  int32_t* ws_arrivals;  // [2][R * head_blocks] chunks arrived / partials published; reset by the merger
  float* part_o;         // [R, head_blocks, C, heads_per_block, D] (per-wave register order)
  float* part_ml;        // [R, head_blocks, C, heads_per_block, 2]
  uint32_t stride_rows;  // cache_stride_bytes / D
  int rows;
  int H;
  int width;
  int max_seq_len;
  int bt_stride;
  int bt_entries;    // block-table entries a row needs: ceil(max_seq_len / block_size)
  int block_size;
  int bs_shift;      // log2(block_size) when it is a power of two, else -1
  int chunks;
  int chunk_tokens;
  int chunk_lead;    // extra tokens of chunk 0 (ranks shift by this for c > 0)
  int head_blocks;
  int heads_per_block;  // 16 * kGroups
  int rows_hb;       // R * head_blocks (stride between the two counter arrays)
  int group_units;   // (row, chunk) units co-scheduled on one XCD (1: none)
  float scale_log2;  // sm_scale * k_scale * log2(e), > 0
  float v_scale;
  int export_sel;    // write the selection (ids, offsets, counts) for the read-back hook
  int merge_in_kernel;  // split rows: 1 the last chunk merges, 0 every chunk publishes for the combine kernel
};

// Longest a merging workgroup waits for the other chunks' partials, in ticks
// of the 100 MHz real-time counter (0.1 s): they have all arrived when the
// wait starts, so it ends within microseconds unless a counter is broken.
constexpr uint64_t kMergeWaitTicks = 10000000;

// Waves of a workgroup: per 16-head group kParts scoring waves, each taking
// a 64 / kParts-token share of a 64-token tile (QK^T and the softmax
// weights), and as many PV waves, which split the latent columns between
// them and accumulate every head group. Scoring wave w and PV wave
// w + kWaves/2 share a SIMD, so the vector work of one runs under the
// matrix work of the other.
constexpr int kTile = 64;     // tokens per staged tile
constexpr int kBuffers = 4;   // tile buffers: two in use, two in flight
// Scoring waves per 16-head group: four (16 tokens of a tile each) with one
// group per workgroup, two (32 tokens each) with two, one (the whole tile)
// with four, so that a workgroup always has eight waves, two per SIMD.
__host__ __device__ constexpr int parts_of(int groups) { return 4 / groups; }
__host__ __device__ constexpr int waves_of(int groups) { return 2 * parts_of(groups) * groups; }

// kGroups: 16-head groups per workgroup (1, 2 or 4).
// kSplitV: V is read from its own buffer (two K and two V tile buffers;
// the next tile's K and this tile's V load while the current ones are
// consumed). Otherwise K and V are the same bytes, in four tile buffers:
// tile i is scored while tile i-1 is accumulated and tiles i+1, i+2 load.
// kRope: 0, or the width of a rope tail each cached token carries after its
// D latent bytes ([attend] module doc, "NoPE, and why no common/ kernel would
// do": the DeepSeek-V4 token, 512 + 64). The tail is scored with the
// latent (one more MFMA per 16-token block, hi and lo query terms side by
// side in its 128-deep k dimension) and staged in its own region of each
// tile buffer; the values and the output are the latent alone.
template <int D, int kGroups, bool kSplitV, int kRope = 0>
__global__ __launch_bounds__(waves_of(kGroups) * kWave, 1)
void dsa_decode_kernel(DecodeArgs a) {
  constexpr int kParts = parts_of(kGroups);
  constexpr int kBPW = 4 / kParts;                  // 16-token blocks per scoring wave
  // Weight blocks (16 tokens of a head under one exponent) per scoring lane:
  // with two or four products a block pairs two products' halves (a lane and
  // the lane 16 apart), so four products make two such sets.
  constexpr int kWB = kBPW == 4 ? 2 : 1;
  constexpr int kQKWaves = kParts * kGroups;
  constexpr int kPVWaves = kQKWaves;
  constexpr int kWaves = kQKWaves + kPVWaves;
  constexpr int kThreads = kWave * kWaves;
  static_assert(kRope == 0 || (kRope == 64 && D == 512 && !kSplitV), "rope tail: 512 + 64, one K/V buffer");
  constexpr int kRowBytes = D + kRope;              // bytes of a cached token
  constexpr int kTileBytes = kTile * D;             // a tile buffer: the tile's latent rows
  constexpr int kBufBytes = kTileBytes;
  // Rope tails: only the scoring waves read them, in the step that scores
  // the tile, so three tail slots after the tile buffers serve the tile
  // being scored and the two in flight (the slot tile i + 2 loads into held
  // tile i - 1, scored in the step before).
  constexpr int kTailBytes = kTile * kRope;         // one tile's tails
  constexpr int kTailSlots = kRope ? 3 : 0;
  constexpr int kTailOff = kBuffers * kBufBytes;
  constexpr int kSmemBytes = kBuffers * kBufBytes + kTailSlots * kTailBytes;
  constexpr int kMaxChunk = kMaxChunkTokens;        // rows one workgroup takes (its row table is in LDS)
  constexpr int kTailInstr = kTailBytes / (16 * kWave);  // tail DMAs per tile (one per wave)
  constexpr int kKSteps = (D + 127) / 128;          // QK MFMA steps over the latent width
  constexpr int kDBlocks = D / 16;                  // 16-column blocks of the output
  constexpr int kCB = kDBlocks / kPVWaves;          // column blocks per PV wave (all groups)
  constexpr int kChunkMask = (kDBlocks < 16 ? kDBlocks : 16) - 1;
  // Gather: a latent row is D/16 lanes of 16 bytes. Every wave moves part of
  // each tile (as many waves as there are DMA instructions per tile).
  constexpr int kLanesPerTok = D / 16;
  constexpr int kTokPerInstr = kWave / kLanesPerTok;
  constexpr int kInstrPerTile = kTile / kTokPerInstr;
  constexpr int kDmaWaves = kInstrPerTile < kWaves ? kInstrPerTile : kWaves;
  constexpr int kTPW = kTile / kDmaWaves;           // tokens each DMA wave moves per tile
  constexpr int kInstr = kTPW / kTokPerInstr;       // DMA instructions per DMA wave per tile
  constexpr int kNd = kSplitV ? 2 * kInstr : kInstr;  // DMA instructions per wave per step
  // Selection: before the first tile the tile buffers hold the membership
  // bitmap of a window of positions (a quarter), each word's rank (a
  // quarter) and the row's block-table entries (the upper half).
  constexpr int kWinWords = kSmemBytes / 16;
  constexpr int kBtCap = kSmemBytes / 8;
  static_assert(kCB >= 1 && kCB * kPVWaves == kDBlocks, "PV column split");
  static_assert(kInstr >= 1 && kInstr * kTokPerInstr == kTPW, "DMA split");
  static_assert(kBtCap % kWave == 0 && kWinWords % 4 == 0, "selection areas");
  static_assert(16 * D + 256 * ((kKSteps - 1) >> 1) < 65536,
                "K operand offsets must fit the LDS instruction offset field");

  __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];
  __shared__ __attribute__((aligned(16))) uint32_t rows_lds[kMaxChunk];
  // softmax weights of a tile as PV B operands: [tile parity][group][operand half][lane] x 16 bytes
  __shared__ __attribute__((aligned(16))) i32x4 xch_p[2][kGroups][2][kWave];
  __shared__ int xch_e[2][kGroups][4][16];  // their E8M0 exponent bytes, per 16-token block and head
  __shared__ float xch_f[kWaves][kWave];         // per-head scalars between waves
  __shared__ float xch_m[kGroups][kWave];        // per-head reference, for the PV waves
  __shared__ int scan_sh[kWaves];
  __shared__ int flag_sh;

  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform: role branches are scalar
  const int g = lane >> 4, li = lane & 15;
  const bool is_qk = wave < kQKWaves;
  // Scoring role: head group hg, tile half `part` (tokens 32*part .. +31).
  const int hg = wave % kGroups, part = (wave % kQKWaves) / kGroups;
  // PV role: every head group, column blocks jbase .. jbase + kCB - 1.
  const int pw = wave - kQKWaves, jbase = (wave % kPVWaves) * kCB;

  // Workgroup -> (row, chunk, head block). The head blocks of one (row,
  // chunk) read the same latent rows, so they get ids 8 apart: the same XCD
  // (ids are dealt to the 8 XCDs round-robin) and its L2 serves the second
  // read. Ids come in rounds of 8 (one per XCD) per head block. When a row
  // is split into chunks, or the rows of a sequence are co-scheduled, the
  // group_units (row, chunk) units of the sequence take group_units
  // consecutive rounds on one XCD, for the same reason (they share the
  // query and ids, or most of the latent rows).
  const int bid = blockIdx.x;
  const int hb = (bid >> 3) % a.head_blocks;
  int rc = (bid / (8 * a.head_blocks)) * 8 + (bid & 7);
  if (a.group_units > 1) {
    const int round = rc >> 3, xcd = rc & 7;
    const int blk = round / a.group_units, i = round - blk * a.group_units;
    rc = (blk * 8 + xcd) * a.group_units + i;
  }
  if (rc >= a.rows * a.chunks) return;  // grid padding
  const int r = rc / a.chunks, c = rc % a.chunks;

  DSA_LDS uint8_t* lds = (DSA_LDS uint8_t*)smem;

  // ------------------------------------------------------------ 1. selection
  // Membership bitmap over one window of positions at a time. The workgroup
  // keeps the ids of ascending rank cstart .. cend - 1. Chunk 0 takes
  // chunk_lead extra ranks: it finishes last and merges, by which time the
  // other chunks' partials are out.
  const int cstart = c * a.chunk_tokens + (c > 0 ? a.chunk_lead : 0);
  const int cend = (c + 1) * a.chunk_tokens + a.chunk_lead;
  const int32_t* srow = a.sel + (size_t)r * a.width;
  // The length and the first 2048 ids of the row (kPre per thread) are
  // loaded first, from addresses clamped into their buffers (no branches),
  // then the row's block-table entries go straight into LDS, then this
  // wave's share of the query.
  constexpr int kPre = (2048 + kThreads - 1) / kThreads;
  int L = a.seq_lens[r];
  int tpre[kPre];  // ids tid + u*kThreads (u < kPre); the rest of a wider row is loaded per window
#pragma unroll
  for (int u = 0; u < kPre; ++u) tpre[u] = srow[min(tid + u * kThreads, a.width - 1)];
#pragma unroll
  for (int u = 0; u < kPre; ++u)
    if (tid + u * kThreads >= a.width) tpre[u] = -1;
  const int32_t* bt = a.block_tables + (size_t)r * a.bt_stride;
  const int nbt = min(a.bt_entries, kBtCap);
  for (int i = wave; i * kWave < nbt; i += kWaves)
    dma4(bt + min(i * kWave + lane, nbt - 1), (DSA_LDS void*)(lds + kSmemBytes / 2 + i * 4 * kWave));
  L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);

  // The query as FP8 terms is prepared by all waves: wave w converts head
  // group w % kGroups, k-steps ks = 4*i + w / kGroups, and the terms are
  // exchanged through tile buffers 2 and 3 (4 KiB per group and k-step). A
  // single k-step is loaded by every wave.
  constexpr int kQWaysPerGroup = kWaves / kGroups;  // 4, or 8 with one group
  const int qsub = wave / kGroups;
  const int q_head = hb * a.heads_per_block + hg * 16 + li;
  const bool q_ok = q_head < a.H;
  constexpr bool kShareQ = kKSteps >= 2;
  constexpr int kKOwn = kShareQ ? (kKSteps + kQWaysPerGroup - 1) / kQWaysPerGroup : kKSteps;
  // With a rope tail the exchange holds one more k-step slot (ks = kKSteps)
  // for the tail's terms, which the first wave of each group converts
  // (lanes of groups 0 and 1 hold its 64 values).
  constexpr int kKX = kKSteps + (kRope ? 1 : 0);   // k-step slots in the exchange
  constexpr int kQxOff = 2 * kBufBytes;
  static_assert(!kShareQ || kGroups * kKX * 4096 <= 2 * kBufBytes, "query exchange area");
  static_assert(kRope == 0 || kRope == 64, "the tail is half a k-step");
  const bool q_tail = kRope && qsub == 0;  // this wave also converts its group's tail
  auto own_ks = [&](int i) { return kShareQ ? kQWaysPerGroup * i + qsub : i; };
  u32x4 qraw[kKOwn][4];
  u32x4 qtraw[4];
  static_assert(kKOwn <= 2, "at most two k-steps of the query per wave (four 16-byte loads each)");
  auto load_q = [&]() {
    const uint16_t* qrow = a.q + ((size_t)r * a.H + (q_ok ? q_head : 0)) * kRowBytes;
#pragma unroll
    for (int i = 0; i < kKOwn; ++i) {
      const int ks = min(own_ks(i), kKSteps - 1);
      const int d0 = min(128 * ks + 32 * g, D - 32);
#pragma unroll
      for (int v = 0; v < 4; ++v) qraw[i][v] = *(const u32x4*)(qrow + d0 + 8 * v);
    }
    if (q_tail)
#pragma unroll
      for (int v = 0; v < 4; ++v) qtraw[v] = *(const u32x4*)(qrow + D + 32 * (g & 1) + 8 * v);
  };
  load_q();

  // the block-table DMA has landed once at most the query loads issued after
  // it are outstanding (the window loop's barriers then publish it)
  if (q_tail) wait_vmcnt<4 * kKOwn + 4>();
  else wait_vmcnt<4 * kKOwn>();

  uint32_t* bitmap = (uint32_t*)smem;
  const DSA_LDS u32x4* bitmap4 = (const DSA_LDS u32x4*)smem;
  const DSA_LDS uint32_t* bitmap_l = (const DSA_LDS uint32_t*)smem;
  u32x4* wrank4 = (u32x4*)(smem + kSmemBytes / 4);
  const DSA_LDS uint32_t* wrank_l = (const DSA_LDS uint32_t*)(smem + kSmemBytes / 4);
  if (tid == 0) flag_sh = 0;
  // A workspace whose status word is set makes every output NaN (read now,
  // used at the stores).
  const bool sticky_bad = __hip_atomic_load(a.ws_status, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT) != 0;
  // Head block 0 exports the row's ids and byte offsets, straight from the
  // placement below, when the read-back hook is wanted.
  const bool exporter = hb == 0 && a.export_sel;
  const DSA_LDS int32_t* btl = (const DSA_LDS int32_t*)(lds + kSmemBytes / 2);
  const bool bt_fast = nbt == a.bt_entries && a.bs_shift >= 0 && !exporter;
  int total = 0;
  for (int base = 0; base < L; base += kWinWords * 32) {
    const int span = min(kWinWords * 32, L - base);
    const int nw4 = (((span + 31) >> 5) + 3) & ~3;                  // words in use
    const int per = ((nw4 / 4 + kThreads - 1) / kThreads) * 4;      // words per thread
    for (int i = tid; i < nw4 / 4; i += kThreads) ((u32x4*)bitmap)[i] = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
    // a hole (any negative id) or an id outside [0, L) sets nothing
#pragma unroll
    for (int u = 0; u < kPre; ++u)
      if (tpre[u] >= base && tpre[u] - base < span)
        atomicOr(&bitmap[(tpre[u] - base) >> 5], 1u << ((tpre[u] - base) & 31));
    for (int j = tid + kPre * kThreads; j < a.width; j += kThreads) {
      const int t = srow[j];
      if (t >= base && t - base < span)
        atomicOr(&bitmap[(t - base) >> 5], 1u << ((t - base) & 31));
    }
    __syncthreads();
    // rank of each word: this thread's words are w0 .. w1 - 1; wave scan of
    // their counts, then the waves before it
    const int w0 = tid * per, w1 = min(w0 + per, nw4);
    int cnt = 0;
    for (int w = w0; w < w1; w += 4) {
      const u32x4 x = bitmap4[w >> 2];
      cnt += __popc(x.x) + __popc(x.y) + __popc(x.z) + __popc(x.w);
    }
    const int incl = wave_inclusive_scan(cnt);
    if (lane == kWave - 1) scan_sh[wave] = incl;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) {
      const int sw = scan_sh[k];
      all += sw;
      before += k < wave ? sw : 0;
    }
    int run = before + incl - cnt;
    for (int w = w0; w < w1; w += 4) {
      const u32x4 x = bitmap4[w >> 2];
      u32x4 rk;
      rk.x = (unsigned)run;
      run += __popc(x.x);
      rk.y = (unsigned)run;
      run += __popc(x.y);
      rk.z = (unsigned)run;
      run += __popc(x.z);
      rk.w = (unsigned)run;
      run += __popc(x.w);
      wrank4[w >> 2] = rk;
    }
    __syncthreads();
    // Each id finds its own rank: its word's rank plus the set bits below it
    // in the word, and goes straight through the block table (the entries
    // in LDS; global memory for a page beyond them) to the index of its
    // latent row (page * rows per page + slot in page). Repeats of an id
    // write the same entries with the same values.
    auto place = [&](int t) {
      if (t >= base && t - base < span) {
        const int o = t - base, w = o >> 5;
        const int rank = total + (int)wrank_l[w] + __popc(bitmap_l[w] & ((1u << (o & 31)) - 1u));
        if (rank >= cstart && rank < cend) {
          const int pi = a.bs_shift >= 0 ? t >> a.bs_shift : t / a.block_size;
          const int slot = t - pi * a.block_size;
          const uint32_t page = (uint32_t)(pi < nbt ? btl[pi] : bt[pi]);
          const uint32_t lrow = page * a.stride_rows + (uint32_t)slot;
          rows_lds[rank - cstart] = lrow;
          if (exporter) {
            a.ws_ids[(size_t)r * a.width + rank] = t;
            a.ws_offsets[(size_t)r * a.width + rank] = (uint64_t)lrow * (uint64_t)kRowBytes;
          }
        }
      }
    };
    if (bt_fast) {
      // The whole block-table row is in LDS, the block size a power of two
      // and nothing is exported: the preloaded ids branch-free, every lane
      // reading (a lane outside the window reads word 0 and entry 0 and
      // stores nothing).
#pragma unroll
      for (int u = 0; u < kPre; ++u) {
        const int t = tpre[u];
        const unsigned o = (unsigned)t - (unsigned)base;
        const bool in = o < (unsigned)span;
        const int w = in ? (int)(o >> 5) : 0;
        const int rank = total + (int)wrank_l[w] + __popc(bitmap_l[w] & ((1u << (o & 31)) - 1u));
        const int pi = in ? t >> a.bs_shift : 0;
        const uint32_t lrow = (uint32_t)btl[pi] * a.stride_rows + (uint32_t)(t & (a.block_size - 1));
        if (in && rank >= cstart && rank < cend) rows_lds[rank - cstart] = lrow;
      }
    } else {
#pragma unroll
      for (int u = 0; u < kPre; ++u) place(tpre[u]);
    }
    for (int j = tid + kPre * kThreads; j < a.width; j += kThreads) place(srow[j]);
    total += all;
    __syncthreads();  // the id table is complete; the bitmap is reused by the next window
  }
  const int n = max(0, min(cend - cstart, total - cstart));
  const int ntiles = (n + kTile - 1) / kTile;
  if (exporter && c == 0 && tid == 0) a.ws_counts[r] = total;

  // pad the row table to whole tiles with the last real row (loaded,
  // weighted by zero)
  if (n > 0)
    for (int p = n + tid; p < ntiles * kTile; p += kThreads) rows_lds[p] = rows_lds[n - 1];

  // ---- the query as two FP8 terms under a per-head power-of-two scale that
  // puts the head's largest |q| in [128, 256). Each wave's share of the
  // maximum goes out with the row table (the barrier below publishes both).
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < kKOwn; ++i) {
    const int ks = own_ks(i);
    if (!q_ok || ks >= kKSteps || 128 * ks + 32 * g >= D)
#pragma unroll
      for (int v = 0; v < 4; ++v) qraw[i][v] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(qraw[i][v][e])), fabsf(bf16_hi(qraw[i][v][e]))));
  }
  if (q_tail) {
    // lanes of groups 0 and 1 hold the tail's 64 values; the rest none
    if (!q_ok || g >= 2)
#pragma unroll
      for (int v = 0; v < 4; ++v) qtraw[v] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(qtraw[v][e])), fabsf(bf16_hi(qtraw[v][e]))));
  }
  amax = max_xor32(max_xor16(amax));
  if constexpr (kShareQ) xch_f[wave][lane] = amax;

  __syncthreads();  // the row table is complete (padded to whole tiles), the query maxima visible

  // -------------------------------------------------------------- 2. gather
  // Wave w (< kDmaWaves) moves tokens [w*kTPW, (w+1)*kTPW) of a tile. Its
  // instruction k writes kTokPerInstr consecutive LDS slots; DMA lane l
  // carries chunk l % kLanesPerTok of token w*kTPW + (l / kLanesPerTok)*kInstr
  // + k, so a lane's kInstr row indices are contiguous in the row table.
  const DSA_LDS uint32_t* rows_l = (const DSA_LDS uint32_t*)rows_lds;
  const bool dma_wave = wave < kDmaWaves;
  const int pw_s = dma_wave ? wave : 0;
  auto tile_rows = [&](int tile, uint32_t (&row)[kInstr]) {
    const DSA_LDS uint32_t* rr =
        rows_l + tile * kTile + pw_s * kTPW + (lane / kLanesPerTok) * kInstr;
#pragma unroll
    for (int k = 0; k < kInstr; ++k) row[k] = rr[k];
  };
  // Lane l carries chunk ci of token slot0 + j. slot0 is a multiple of
  // kTokPerInstr (a power of two) and j < kTokPerInstr, so the token's
  // swizzle is the uniform swizzle of slot0 XOR j: one per-lane constant.
  const uint32_t dma_c0 =
      (uint32_t)(((lane % kLanesPerTok) ^ ((lane / kLanesPerTok) & kChunkMask)) << 4);
  auto dma_one = [&](int k, uint32_t row, int dst_off, const uint8_t* src,
                     uint32_t c0) {
    const int slot0 = pw_s * kTPW + k * kTokPerInstr;
    const uint32_t chunk = c0 ^ ((uint32_t)tile_swizzle<D>(slot0) << 4);  // < D
    const uint64_t off = (uint64_t)row * (uint64_t)kRowBytes + (uint64_t)chunk;
    dma16(src + off, (DSA_LDS void*)(lds + dst_off + slot0 * D));
  };
  auto issue_tile = [&](int tile, int dst_off, const uint8_t* src) {
    uint32_t row[kInstr];
    tile_rows(tile, row);
#pragma unroll
    for (int k = 0; k < kInstr; ++k) dma_one(k, row[k], dst_off, src, dma_c0);
  };
  // Token index (within the tile) held by LDS slot s.
  auto token_of_slot = [&](int s) {
    const int w = s / kTPW, sw = s % kTPW;
    return w * kTPW + (sw % kTokPerInstr) * kInstr + sw / kTokPerInstr;
  };
  // LDS byte offsets of the buffers holding tile i's K and V.
  auto k_off = [&](int i) { return kSplitV ? (i & 1) * kBufBytes : (i & 3) * kBufBytes; };
  auto v_off = [&](int i) { return kSplitV ? (2 + (i & 1)) * kBufBytes : (i & 3) * kBufBytes; };
  // Rope tail of a tile: wave w < kTailInstr moves LDS slots 16w .. 16w + 15,
  // lane l the 16 bytes at position l % 4 of slot 16w + l / 4, which hold the
  // token the latent region holds at that slot. The tail's 16-byte chunks are
  // XOR-permuted by bits 2-3 of the slot, so the 16 slots one MFMA operand
  // read touches land in distinct bank groups.
  auto tail_off = [&](int tile) { return kTailOff + (tile % 3) * kTailBytes; };
  auto tail_dma = [&](int tile) {
    if (kRope && wave < kTailInstr && tile < ntiles) {
      const int slot = 16 * wave + (lane >> 2);
      const uint32_t row = rows_l[tile * kTile + token_of_slot(slot)];
      const uint32_t chunk = (uint32_t)((lane & 3) ^ ((slot >> 2) & 3)) << 4;
      dma16(a.k_cache + (uint64_t)row * kRowBytes + D + chunk,
            (DSA_LDS void*)(lds + tail_off(tile) + wave * 16 * kWave));
    }
  };
  // Tile it has landed for this wave once only the DMAs of the next tile
  // (issued in the previous step) may still be outstanding.
  // (At step 0 only tile 0 is out, so step 0 waits for every load.)
  auto wait_tile = [&](int it) {
    if (kSplitV || it + 1 >= ntiles || it == 0) wait_vmcnt<0>();
    else if (kRope && wave < kTailInstr) wait_vmcnt<kInstr + 1>();
    else wait_vmcnt<kInstr>();
  };
  // Tile 0 goes out now, and tile 1 (K and V the same bytes) at the start of
  // step 0, once tile 0 has landed: every workgroup issues its first loads
  // (ids, block-table rows, query rows) and its first tile together, and tile
  // 0 lands sooner when that launch-wide burst does not also carry every
  // workgroup's second tile (8 MiB fewer on the long-context shape). A
  // separate V buffer is filled in the loop after every wave has read its
  // query terms out of it.
  auto issue_first = [&]() {
    if (dma_wave) {
      if (ntiles > 0) issue_tile(0, k_off(0), a.k_cache);
      tail_dma(0);
    }
  };
  auto issue_second = [&]() {  // step 0, after its barrier
    if (!kSplitV && dma_wave) {
      if (ntiles > 1) issue_tile(1, k_off(1), a.k_cache);
      tail_dma(1);
    }
  };

  // Tile 0 loads while the query terms are prepared (issued after
  // the query registers were first read, so that no wait for the query
  // loads can also wait for these).
  issue_first();
  float score_scale;
  i32x8 qhi[kKSteps], qlo[kKSteps];
  {
    if constexpr (kShareQ)
#pragma unroll
      for (int p = 0; p < kQWaysPerGroup; ++p) amax = fmaxf(amax, xch_f[hg + kGroups * p][lane]);
    const int e = amax > 0.f ? (int)((__float_as_uint(amax) >> 23) & 0xff) - 127 : 0;
    int sh = 7 - e;
    sh = sh < -120 ? -120 : (sh > 120 ? 120 : sh);
    const float qs = pow2i(sh);
    // exchange area: [group][ks][hi|lo][half][lane]
    u32x4* qx = (u32x4*)(smem + kQxOff);
    // 32 bf16 values (16 words) -> hi and lo FP8 terms, 8 words each
    auto split_q = [&](const u32x4 (&raw)[4], u32x4 (&h)[2], u32x4 (&l)[2]) {
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const unsigned w0 = raw[v][2 * h2], w1 = raw[v][2 * h2 + 1];
          int hi, lo;
          split_fp8x4(bf16_lo(w0) * qs, bf16_hi(w0) * qs, bf16_lo(w1) * qs, bf16_hi(w1) * qs,
                      hi, lo);
          h[v >> 1][2 * (v & 1) + h2] = (unsigned)hi;
          l[v >> 1][2 * (v & 1) + h2] = (unsigned)lo;
        }
    };
    if (q_tail) {
      u32x4 h[2], l[2];
      split_q(qtraw, h, l);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        qx[(((hg * kKX + kKSteps) * 2 + 0) * 2 + half) * kWave + lane] = h[half];
        qx[(((hg * kKX + kKSteps) * 2 + 1) * 2 + half) * kWave + lane] = l[half];
      }
    }
#pragma unroll
    for (int i = 0; i < kKOwn; ++i) {
      const int ks = own_ks(i);
      if (ks >= kKSteps) continue;
      u32x4 h[2], l[2];
      split_q(qraw[i], h, l);
      if constexpr (kShareQ) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          qx[(((hg * kKX + ks) * 2 + 0) * 2 + half) * kWave + lane] = h[half];
          qx[(((hg * kKX + ks) * 2 + 1) * 2 + half) * kWave + lane] = l[half];
        }
      } else {
        qhi[ks] = i32x8{(int)h[0].x, (int)h[0].y, (int)h[0].z, (int)h[0].w,
                        (int)h[1].x, (int)h[1].y, (int)h[1].z, (int)h[1].w};
        qlo[ks] = i32x8{(int)l[0].x, (int)l[0].y, (int)l[0].z, (int)l[0].w,
                        (int)l[1].x, (int)l[1].y, (int)l[1].z, (int)l[1].w};
      }
    }
    score_scale = a.scale_log2 * pow2i(-sh);
  }
  __syncthreads();  // the groups' FP8 terms visible

  // The tail's B operand: k 0..63 its hi terms, k 64..127 its lo terms, so
  // one MFMA per block adds K_tail . (hi + lo). Lane group G takes the
  // words that lane group G % 2 converted, hi for G < 2 and lo otherwise.
  i32x8 qtail = {0, 0, 0, 0, 0, 0, 0, 0};
  // Read by the scoring waves before the first barrier of the loop (after
  // it the gather overwrites the area). With four head groups they are read
  // at the start of the scoring branch: held from here instead, across the
  // branch, they crowded the PV branch's registers (71 registers spilled,
  // reloaded inside the loop with a wait for every gather in flight).
  // Otherwise they are read here (the same reads written out below: wrapped
  // in this lambda the compiler builds their addresses differently).
  auto load_qterms = [&]() {
    if constexpr (kShareQ) {
      const u32x4* qx = (const u32x4*)(smem + kQxOff);
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        const u32x4 h0 = qx[(((hg * kKX + ks) * 2 + 0) * 2 + 0) * kWave + lane];
        const u32x4 h1 = qx[(((hg * kKX + ks) * 2 + 0) * 2 + 1) * kWave + lane];
        const u32x4 l0 = qx[(((hg * kKX + ks) * 2 + 1) * 2 + 0) * kWave + lane];
        const u32x4 l1 = qx[(((hg * kKX + ks) * 2 + 1) * 2 + 1) * kWave + lane];
        qhi[ks] = i32x8{(int)h0.x, (int)h0.y, (int)h0.z, (int)h0.w, (int)h1.x, (int)h1.y, (int)h1.z, (int)h1.w};
        qlo[ks] = i32x8{(int)l0.x, (int)l0.y, (int)l0.z, (int)l0.w, (int)l1.x, (int)l1.y, (int)l1.z, (int)l1.w};
      }
      // (64-head blocks carry no rope tail)
    }
  };
  if constexpr (kShareQ && kGroups != 4) {
    if (is_qk) {
      const u32x4* qx = (const u32x4*)(smem + kQxOff);
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        const u32x4 h0 = qx[(((hg * kKX + ks) * 2 + 0) * 2 + 0) * kWave + lane];
        const u32x4 h1 = qx[(((hg * kKX + ks) * 2 + 0) * 2 + 1) * kWave + lane];
        const u32x4 l0 = qx[(((hg * kKX + ks) * 2 + 1) * 2 + 0) * kWave + lane];
        const u32x4 l1 = qx[(((hg * kKX + ks) * 2 + 1) * 2 + 1) * kWave + lane];
        qhi[ks] = i32x8{(int)h0.x, (int)h0.y, (int)h0.z, (int)h0.w, (int)h1.x, (int)h1.y, (int)h1.z, (int)h1.w};
        qlo[ks] = i32x8{(int)l0.x, (int)l0.y, (int)l0.z, (int)l0.w, (int)l1.x, (int)l1.y, (int)l1.z, (int)l1.w};
      }
      if constexpr (kRope > 0) {
        const int src = (g & 1) * 16 + li;
        const u32x4 t0 = qx[(((hg * kKX + kKSteps) * 2 + (g >> 1)) * 2 + 0) * kWave + src];
        const u32x4 t1 = qx[(((hg * kKX + kKSteps) * 2 + (g >> 1)) * 2 + 1) * kWave + src];
        qtail = i32x8{(int)t0.x, (int)t0.y, (int)t0.z, (int)t0.w, (int)t1.x, (int)t1.y, (int)t1.z, (int)t1.w};
      }
    }
  }

  // K operand addresses of a scoring wave. It scores blocks b = kBPW*part +
  // k (k < kBPW) of 16 slots. Slot 16*b + li, chunk 8*ks + 2*g + h sits at
  // chunk position (chunk ^ swizzle); with swizzle = li ^ 8*(b & 1) that
  // position is 16*(ks >> 1) + (((2*g + h) ^ li) ^ 8*((ks ^ b) & 1)), so four
  // per-lane offsets (b's parity folded in when a wave has one block) plus
  // compile-time immediates cover every read.
  int kofs[2][2];
  const int bpar = kBPW == 1 ? (part & 1) : 0;
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      kofs[p][h] = 16 * kBPW * D * part + li * D +
                   16 * ((((2 * g + h) ^ li) ^ (8 * (p ^ bpar))) & kChunkMask);

  // PV operands. The matrix core scales B (the weights) in four blocks of
  // 32 k-positions: bytes 0-15 (then 16-31) of lane groups {0, 1} (then
  // {2, 3}); lane group G supplies block G's exponent. Each block carries 16
  // tokens of the tile, their hi terms and their lo terms, so those 16
  // tokens of a head share one exponent. In lane group G, bytes 16*h ..
  // 16*h + 7 hold the hi terms of 8 slots and bytes 16*h + 8 .. +15 their lo
  // terms:
  // - two blocks per scoring wave (four: each pair as the two of one part,
  //   pair h in operand half h): slots 32*h + 16*(G & 1) + 8*(G >> 1) ..
  //   +7. Block 2*h + (G >> 1) thus holds the 8 slots that scoring lane
  //   group g of wave part h holds in each of its two products, for
  //   g = 2*(G >> 1) and g + 1: a lane and the lane 16 apart. Slot 32*h +
  //   16*k + 8*(G >> 1) + 4*(g & 1) + i comes from lane group g of product
  //   k, byte 4*(g & 1) + i.
  // - one block per scoring wave: slots 32*h + 8*G .. +7, so block 2*h +
  //   (G >> 1) is the 16 slots of scoring wave part 2*h + (G >> 1). Slot
  //   16*part + 4*g + i comes from its lane group g, in PV lane group
  //   2*(part & 1) + (g >> 1), byte 4*(g & 1) + i.
  // A (V): lane group G needs the latent column of those 8 slots twice per
  // half. A transposing read hands lane li the 8 bytes of its column from 8
  // rows; lanes 2k and 2k+1 of the 16-lane group supply row k (column halves
  // 0 and 1). (The slots that lane groups 0 and 1, and 2 and 3, read
  // together sit at distinct chunk positions under the swizzle.)
  int vrow[2], vswz[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int slot = kBPW >= 2 ? 32 * h + 16 * (g & 1) + 8 * (g >> 1) + (li >> 1)
                               : 32 * h + 8 * g + (li >> 1);
    vrow[h] = slot * D + 8 * (li & 1);
    vswz[h] = tile_swizzle<D>(slot) << 4;
  }

  // The gather of step it: tile it + 2 (or, with a separate V buffer, K of
  // it + 1 and V of it), this wave's kNd instructions, spread by each role
  // over its matrix steps so that the vector memory queue never stalls a
  // wave for long. (The lane constant is laundered per step: the address
  // arithmetic is then redone each time instead of being held in registers.)
  auto dma_rows = [&](int it, uint32_t (&drow)[kNd]) {
    if (kSplitV ? it + 1 < ntiles : it + 2 < ntiles) {
      uint32_t rk[kInstr];
      tile_rows(kSplitV ? it + 1 : it + 2, rk);
#pragma unroll
      for (int k = 0; k < kInstr; ++k) drow[k] = rk[k];
    }
    if (kSplitV && it < ntiles) {
      uint32_t rv[kInstr];
      tile_rows(it, rv);
#pragma unroll
      for (int k = 0; k < kInstr; ++k) drow[kNd - kInstr + k] = rv[k];
    }
  };
  auto dma_step = [&](int it, int d, const uint32_t (&drow)[kNd], uint32_t c0) {
    if (!dma_wave) return;
    if (d < kInstr) {
      if (kSplitV ? it + 1 < ntiles : it + 2 < ntiles)
        dma_one(d, drow[d], k_off(kSplitV ? it + 1 : it + 2), a.k_cache, c0);
    } else {
      if (kSplitV && it < ntiles) dma_one(d - kInstr, drow[d], v_off(it), a.v_cache, c0);
    }
  };

  // -------------------------------------------------------------- 3. attend
  // Step i scores tile i (scoring waves) and accumulates tile i - 1 (PV
  // waves), between one barrier and the next. The accumulators are touched
  // only by the matrix cores: weights are taken against a fixed per-head
  // reference (the first tile's max), and each block of 16 weights of a
  // head carries its own E8M0 exponent, so a later score may exceed the
  // reference by up to 2^kSlack without leaving the FP8 range or fp32
  // accumulation. Should a score ever exceed it by more (only with
  // pathological inputs), the chunk is recomputed with the reference set to
  // the exact maximum seen.
  f32x4 O[kGroups][kCB];
  float l_part = 0.f;        // this scoring wave's share of sum_t 2^(s_t - m_ref), per head
  float m_ref = -INFINITY;   // reference of this head's scores (log2 domain)
  float mb7 = -7.f;          // (m_ref, or 0 while it is -inf) - 7
  float m_seen = -INFINITY;  // exact max of the lane pair's scores so far (unscaled MFMA units)
  // After the first pass: recompute the chunk only if some scoring wave saw
  // a score beyond the slack (every wave takes part; two barriers).
  auto redo_needed = [&](bool overflow) {
    if (__any(overflow) && lane == 0) flag_sh = 1;
    xch_f[wave][lane] = max_xor32(m_seen) * score_scale;  // score_scale > 0 (m_seen: lane pair's)
    __syncthreads();
    const bool redo = flag_sh != 0;
    if (redo && is_qk) {
      float m = -INFINITY;
#pragma unroll
      for (int p = 0; p < kParts; ++p) m = fmaxf(m, xch_f[hg + kGroups * p][lane]);
      m_ref = m;
      mb7 = (m_ref == -INFINITY ? 0.f : m_ref) - 7.f;
    }
    __syncthreads();
    return redo;
  };

  // Both roles run the same sequence of barriers: one at the top of each
  // step, in the first step of the first pass one more for the reference,
  // and two after the first pass. Step i scores tile i and accumulates tile
  // i - 1. Each role keeps its own registers (the query terms, the
  // accumulators) inside its own branch.
  if (is_qk) {
    if constexpr (kGroups == 4) load_qterms();
    const float pinf = opaque_inf();
    for (int pass = 0; pass < 2; ++pass) {
      l_part = 0.f;
      bool overflow = false;
      if (pass == 1) issue_first();
        for (int it = 0; it <= ntiles; ++it) {
          // this wave's share of tile it has landed (the next tile's may
          // still be in flight); after the barrier tile it's K is in LDS and
          // every read of the weights of it - 2 is done
          wait_tile(it);
          barrier_lds();
          if (it == 0) issue_second();
          const bool score = it < ntiles;
          uint32_t drow[kNd];
          uint32_t c0 = dma_c0;
          asm volatile("" : "+v"(c0));
          if (dma_wave) dma_rows(it, drow);
          if (!kSplitV) tail_dma(it + 2);

          // ---- S^T = K Q^T over this wave's blocks, K operands
          // prefetched kKPre MFMA steps ahead
          f32x4 S[kBPW];
          float mh[kWB];  // max of this lane's weight block(s)
#pragma unroll
          for (int w = 0; w < kWB; ++w) mh[w] = -INFINITY;
          if (score) {
            const DSA_LDS uint8_t* kt = lds + k_off(it);
            constexpr int kSteps = kBPW * kKSteps;
            auto load_k = [&](int s) -> i32x8 {
              const int k = s / kKSteps, ks = s % kKSteps;
              i32x8 kop = {0, 0, 0, 0, 0, 0, 0, 0};
              if (128 * ks + 32 * g < D) {
                const int p = (ks ^ k) & 1;
                const DSA_LDS uint8_t* base = kt + 16 * k * D + 256 * (ks >> 1);
                const u32x4 lo = *(const DSA_LDS u32x4*)(base + kofs[p][0]);
                const u32x4 hi = *(const DSA_LDS u32x4*)(base + kofs[p][1]);
                kop = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                            (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
              }
              return kop;
            };
            // Rope tail of block k: slot 16*(kBPW*part + k) + li, bytes
            // 32*(g & 1) .. + 31 (chunks XOR-permuted by slot bits 2-3).
            auto load_tail = [&](int k) -> i32x8 {
              const DSA_LDS uint8_t* tb = lds + tail_off(it) + (16 * (kBPW * part + k) + li) * kRope;
              const int sw = (li >> 2) & 3, c = 2 * (g & 1);
              const u32x4 lo = *(const DSA_LDS u32x4*)(tb + 16 * (c ^ sw));
              const u32x4 hi = *(const DSA_LDS u32x4*)(tb + 16 * ((c + 1) ^ sw));
              return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                           (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            };
            constexpr int kKPre = 3;
            i32x8 kbuf[kKPre + 1];
            i32x8 ktail = {0, 0, 0, 0, 0, 0, 0, 0};
            // The scoring wave's matrix work goes first on its SIMD; the PV
            // wave's then runs under this wave's softmax.
            __builtin_amdgcn_s_setprio(2);
#pragma unroll
            for (int s = 0; s < kKPre && s < kSteps; ++s) kbuf[s] = load_k(s);
#pragma unroll
            for (int s = 0; s < kSteps; ++s) {
              const int k = s / kKSteps, ks = s % kKSteps;
              if (s + kKPre < kSteps) kbuf[(s + kKPre) % (kKPre + 1)] = load_k(s + kKPre);
              if (kRope && ks == 0) ktail = load_tail(k);
#pragma unroll
              for (int d = s * kNd / kSteps; d < (s + 1) * kNd / kSteps; ++d) dma_step(it, d, drow, c0);
              __builtin_amdgcn_sched_barrier(0);
              if (ks == 0) S[k] = f32x4{0.f, 0.f, 0.f, 0.f};
              S[k] = mfma_fp8(kbuf[s % (kKPre + 1)], qhi[ks], S[k]);
              S[k] = mfma_fp8(kbuf[s % (kKPre + 1)], qlo[ks], S[k]);
              if (kRope && ks == kKSteps - 1) S[k] = mfma_fp8(ktail, qtail, S[k]);
              __builtin_amdgcn_sched_barrier(0);
            }
            __builtin_amdgcn_s_setprio(0);
            // Vector instructions read (or mask) the scores next. The matrix
            // core's result of this product shape is readable 11 wait states
            // after issue, and nothing interlocks; the compiler's own hazard
            // padding has been seen to fall short here (3 wait states), so
            // the padding is explicit.
            asm volatile("s_nop 7\n\ts_nop 2" ::: "memory");
            // The lane holds head li at slots 16*(kBPW*part + k) + 4*g + i.
            const int nvalid = n - it * kTile;
            if (__builtin_expect(nvalid < kTile, 0)) {
#pragma unroll
              for (int k = 0; k < kBPW; ++k)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  if (token_of_slot(16 * (kBPW * part + k) + 4 * g + i) >= nvalid) S[k][i] = -INFINITY;
            }
            if constexpr (kWB == 1) {
              // A weight block's 16 tokens: with two products per wave, this
              // lane's 8 (4 in each) and those of the lane 16 apart (one lane
              // swap); with one, the 4 of each lane group (two swaps). The
              // maximum stays in MFMA units; the log2-domain value is taken
              // with one fma where it is used.
              float a = max2(max2(S[0][0], S[0][1], pinf), max2(S[0][2], S[0][3], pinf), pinf);
              if constexpr (kBPW == 2)
                a = max2(a, max2(max2(S[1][0], S[1][1], pinf), max2(S[1][2], S[1][3], pinf), pinf), pinf);
              mh[0] = max_xor16(a, pinf);
              if constexpr (kBPW == 1) mh[0] = max_xor32(mh[0], pinf);
              m_seen = max2(m_seen, mh[0], pinf);
            } else {
              // Four products: two weight blocks, each pairing products 2w and
              // 2w + 1 as two products do.
#pragma unroll
              for (int w = 0; w < kWB; ++w) {
                const int k0 = 2 * w;
                const float a = max2(max2(max2(S[k0][0], S[k0][1], pinf), max2(S[k0][2], S[k0][3], pinf), pinf),
                                     max2(max2(S[k0 + 1][0], S[k0 + 1][1], pinf),
                                          max2(S[k0 + 1][2], S[k0 + 1][3], pinf), pinf), pinf);
                mh[w] = max_xor16(a, pinf);
                m_seen = max2(m_seen, mh[w], pinf);
              }
            }
          }
          if (pass == 0 && it == 0) {
            // first tile: the reference is the tile's max over the group's
            // scoring waves
            if (score)  // score_scale > 0
              xch_f[wave][lane] = max_xor32(kWB == 2 ? max2(mh[0], mh[kWB - 1], pinf) : mh[0], pinf) * score_scale;
            barrier_lds();
            if (ntiles > 0) {
              float m = -INFINITY;
#pragma unroll
              for (int p = 0; p < kParts; ++p) m = fmaxf(m, xch_f[hg + kGroups * p][lane]);
              m_ref = m;
              mb7 = (m_ref == -INFINITY ? 0.f : m_ref) - 7.f;
            }
          }
          if (score) {
            if constexpr (kWB == 1) {
              // ---- weights, per 16-token block: the block's largest weight of
              // the head maps to [128, 256) (a block with no valid token:
              // exponent -100, weights 0)
              const float x = fmaf(mh[0], score_scale, -(mb7 + 7.f));  // log2 domain, against the reference
              overflow |= x >= kSlack;
              const float ef = floorf(__builtin_amdgcn_fmed3f(x, -100.f, 100.f));
              const float bsub = mb7 + ef;
              const int eb = (int)ef + 120;  // E8M0 byte of 2^(e - 7)
              float psum = 0.f;
#pragma unroll
              for (int k = 0; k < kBPW; ++k) {
                float p[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) p[i] = fast_exp2(fmaf(S[k][i], score_scale, -bsub));
                psum += (p[0] + p[1]) + (p[2] + p[3]);
                int phi, plo;
                split_fp8x4(p[0], p[1], p[2], p[3], phi, plo);
                // head li, word (g & 1) (hi) and 2 + (g & 1) (lo) of PV lane
                // group 2*(g >> 1) + k, operand half part (two products), or
                // of lane group 2*(part & 1) + (g >> 1), half part >> 1 (one)
                int* dst = kBPW == 2 ? (int*)&xch_p[it & 1][hg][part][(2 * (g >> 1) + k) * 16 + li]
                                     : (int*)&xch_p[it & 1][hg][part >> 1][(2 * (part & 1) + (g >> 1)) * 16 + li];
                dst[g & 1] = phi;
                dst[2 + (g & 1)] = plo;
              }
              l_part += psum * __uint_as_float((uint32_t)eb << 23);
              // scale of weight block 2*part + (g >> 1), or part (the lanes
              // that share the block write the same byte)
              xch_e[it & 1][hg][kBPW == 2 ? 2 * part + (g >> 1) : part][li] = eb;
            } else {
              // Four products: weight blocks 2w + (g >> 1) from products 2w
              // and 2w + 1, in operand half w, laid out as two products lay
              // out their part's half.
#pragma unroll
              for (int w = 0; w < kWB; ++w) {
                const float x = fmaf(mh[w], score_scale, -(mb7 + 7.f));
                overflow |= x >= kSlack;
                const float ef = floorf(__builtin_amdgcn_fmed3f(x, -100.f, 100.f));
                const float bsub = mb7 + ef;
                const int eb = (int)ef + 120;
                float psum = 0.f;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                  float p[4];
#pragma unroll
                  for (int i = 0; i < 4; ++i) p[i] = fast_exp2(fmaf(S[2 * w + kk][i], score_scale, -bsub));
                  psum += (p[0] + p[1]) + (p[2] + p[3]);
                  int phi, plo;
                  split_fp8x4(p[0], p[1], p[2], p[3], phi, plo);
                  int* dst = (int*)&xch_p[it & 1][hg][w][(2 * (g >> 1) + kk) * 16 + li];
                  dst[g & 1] = phi;
                  dst[2 + (g & 1)] = plo;
                }
                l_part += psum * __uint_as_float((uint32_t)eb << 23);
                xch_e[it & 1][hg][2 * w + (g >> 1)][li] = eb;
              }
            }
          }
        }
      if (pass == 0 && !redo_needed(overflow)) break;
    }
  } else {
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
      for (int x = 0; x < kGroups; ++x)
#pragma unroll
        for (int j = 0; j < kCB; ++j) O[x][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (pass == 1) issue_first();
        for (int it = 0; it <= ntiles; ++it) {
          // Tile it has landed: wait for every DMA of this wave but the next
          // tile's, then the barrier (tile it - 1's V and weights visible,
          // every read of tile it - 2's buffer done).
          wait_tile(it);
          barrier_lds();
          if (it == 0) issue_second();
          if (pass == 0 && it == 0) barrier_lds();  // the scoring waves' reference exchange

          uint32_t drow[kNd];
          uint32_t c0 = dma_c0;
          asm volatile("" : "+v"(c0));
          if (dma_wave) dma_rows(it, drow);
          // (with 16-head blocks PV waves also move a quarter of the tail)
          if (!kSplitV) tail_dma(it + 2);
          if (it == 0) {
#pragma unroll
            for (int d = 0; d < kNd; ++d) dma_step(it, d, drow, c0);
            continue;
          }
          // ---- O^T += V^T P^T for tile it - 1 over this wave's column
          // blocks: one MFMA per head group and block (64 tokens, hi and lo
          // terms), V operands prefetched kVPre blocks ahead.
          const int pt = it - 1;
          // With four head groups the accumulators leave no room to hold the
          // lane's LDS addresses through the loop: they are recomputed each
          // step from a laundered lane id.
          int ln = lane, jb = jbase << 4;
          if constexpr (kGroups == 4) asm volatile("" : "+v"(ln), "+v"(jb));
          i32x8 pB[kGroups];
          int psc[kGroups];
#pragma unroll
          for (int x = 0; x < kGroups; ++x) {
            const int pl = kGroups == 4 ? ln : lane;
            const i32x4 h0 = xch_p[pt & 1][x][0][pl], h1 = xch_p[pt & 1][x][1][pl];
            pB[x] = i32x8{h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
            psc[x] = kGroups == 4 ? xch_e[pt & 1][x][ln >> 4][ln & 15] : xch_e[pt & 1][x][g][li];
          }
          const DSA_LDS uint8_t* vt = lds + v_off(pt);
          int vr[2] = {vrow[0], vrow[1]}, vs[2] = {vswz[0], vswz[1]};
          if constexpr (kGroups == 4) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int slot = 32 * h + 16 * ((ln >> 4) & 1) + 8 * (ln >> 5) + ((ln & 15) >> 1);
              vr[h] = slot * D + 8 * (ln & 1);
              vs[h] = tile_swizzle<D>(slot) << 4;
            }
          }
          auto load_v = [&](int j0) -> i32x8 {
            i32x8 vop;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int addr = kGroups == 4 ? ((jb + (j0 << 4)) ^ vs[u]) + vr[u]
                                            : (((jbase + j0) << 4) ^ vswz[u]) + vrow[u];
              const i32x2 v2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((DSA_LDS i32x2*)(vt + addr));
              vop[4 * u] = v2.x;      // against the hi terms
              vop[4 * u + 1] = v2.y;
              vop[4 * u + 2] = v2.x;  // against the lo terms
              vop[4 * u + 3] = v2.y;
            }
            return vop;
          };
          constexpr int kVPre = kGroups == 4 ? 1 : 2;
          i32x8 vbuf[kVPre + 1];
#pragma unroll
          for (int j = 0; j < kVPre && j < kCB; ++j) vbuf[j] = load_v(j);
#pragma unroll
          for (int j0 = 0; j0 < kCB; ++j0) {
            if (j0 + kVPre < kCB) vbuf[(j0 + kVPre) % (kVPre + 1)] = load_v(j0 + kVPre);
#pragma unroll
            for (int d = j0 * kNd / kCB; d < (j0 + 1) * kNd / kCB; ++d) dma_step(it, d, drow, c0);
            __builtin_amdgcn_sched_barrier(0);
            const i32x8& vop = vbuf[j0 % (kVPre + 1)];
#pragma unroll
            for (int x = 0; x < kGroups; ++x)
              O[x][j0] = mfma_fp8_bscaled(vop, pB[x], psc[x], O[x][j0]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
          if (pass == 0 && !redo_needed(false)) break;
    }
  }

  // Weight sums and references of the heads, for the PV waves.
  if (is_qk) {
    xch_f[wave][lane] = sum_xor32(sum_xor16(l_part));
    if (part == 0) xch_m[hg][lane] = ntiles > 0 ? m_ref : -INFINITY;
  }
  __syncthreads();
  float l_run[kGroups], m_run[kGroups];
#pragma unroll
  for (int x = 0; x < kGroups; ++x) {
    l_run[x] = 0.f;
#pragma unroll
    for (int p = 0; p < kParts; ++p) l_run[x] += xch_f[x + kGroups * p][lane];
    m_run[x] = xch_m[x][lane];
  }

  // --------------------------------------------------------------- 4. merge
  // A PV lane holds O^T rows d = 16*(jbase + j) + 4*g + i for head li of
  // group x.
  auto store_out = [&](int x, const f32x4* o, float lsum) {
    const int hx = hb * a.heads_per_block + x * 16 + li;
    if (hx >= a.H) return;
    const float inv = sticky_bad ? __builtin_nanf("") : (lsum > 0.f ? a.v_scale / lsum : 0.f);
    uint16_t* orow = a.out + ((size_t)r * a.H + hx) * D;
#pragma unroll
    for (int j = 0; j < kCB; ++j) {
      const bf16x4 v = {(__bf16)(o[j][0] * inv), (__bf16)(o[j][1] * inv),
                        (__bf16)(o[j][2] * inv), (__bf16)(o[j][3] * inv)};
      *(bf16x4*)(orow + 16 * (jbase + j) + 4 * g) = v;
    }
  };
  if (a.chunks == 1) {
    // The block's output rows are contiguous in `out`: they are staged in
    // the (now idle) tile buffers as bf16, rows 2*D + 16 bytes apart so that
    // the 16 rows one staging store touches fall in distinct banks, and then
    // written as whole 16-byte pieces, consecutive lanes on consecutive bytes,
    // with streaming stores (nothing here reads them again, so they need not
    // wait in L2 for the end-of-kernel write-back).
    constexpr int kStageRow = 2 * D + 16;
    static_assert(kGroups * 16 * kStageRow <= kSmemBytes, "output staging");
    if (!is_qk)
#pragma unroll
      for (int x = 0; x < kGroups; ++x) {
        const float inv = sticky_bad ? __builtin_nanf("") : (l_run[x] > 0.f ? a.v_scale / l_run[x] : 0.f);
#pragma unroll
        for (int j = 0; j < kCB; ++j) {
          const bf16x4 v = {(__bf16)(O[x][j][0] * inv), (__bf16)(O[x][j][1] * inv),
                            (__bf16)(O[x][j][2] * inv), (__bf16)(O[x][j][3] * inv)};
          *(bf16x4*)(smem + (x * 16 + li) * kStageRow + 2 * (16 * (jbase + j) + 4 * g)) = v;
        }
      }
    __syncthreads();
    const int h0 = hb * a.heads_per_block;
    const int rows = min(a.heads_per_block, a.H - h0);
    uint8_t* ob = (uint8_t*)(a.out + ((size_t)r * a.H + h0) * D);
    constexpr int kPieces = 2 * D / 16;  // 16-byte pieces per row
    for (int i = tid; i < rows * kPieces; i += kThreads) {
      const int row = i / kPieces, pc = i - row * kPieces;
      __builtin_nontemporal_store(*(const u32x4*)(smem + row * kStageRow + 16 * pc),
                                  (u32x4*)(ob + (size_t)row * (2 * D) + 16 * pc));
    }
    return;
  }
  // Split chunks. Each workgroup counts itself in; the last one to arrive
  // merges. The others publish their partials (each PV wave's accumulators
  // as they sit in its registers, 1 KiB per store, then (reference, sum) of
  // the block's heads) with device-scope stores, wait for those stores to
  // complete, and only then count themselves published: the stores are
  // visible at device scope without a cache write-back. The merger waits for
  // that count and reads the partials with device-scope loads, so no cache
  // is written back or invalidated on either side. Only workgroups that have
  // already arrived are waited for, so the wait always ends; a bounded spin
  // turns a broken count into NaN output instead of a hang.
  constexpr int kPartFloats = kGroups * kCB * kWave * 4;  // per PV wave
  const size_t wg_slot = (size_t)(r * a.head_blocks + hb) * a.chunks;
  const int rh = r * a.head_blocks + hb;
  int32_t* arrived = a.ws_arrivals + rh;
  int32_t* published = a.ws_arrivals + (size_t)a.rows_hb + rh;
  auto part_o_of = [&](int cc, int src) {
    return a.part_o + ((wg_slot + cc) * kPVWaves + src) * kPartFloats;
  };
  auto part_ml_of = [&](int cc, int x) {
    return a.part_ml + ((wg_slot + cc) * a.heads_per_block + x * 16 + li) * 2;
  };
  if (!a.merge_in_kernel) {
    // Every chunk publishes; the combine kernel, launched next on the same
    // stream, merges them (the kernel boundary orders the stores). The
    // partial is stored normalised by the chunk's own weight sum, as fp16:
    // a weighted mean of FP8 codes, so |o / l| <= 448, with a relative
    // error of at most 2^-11 per element.
    if (!is_qk) {
      _Float16* po = (_Float16*)part_o_of(c, pw);
#pragma unroll
      for (int x = 0; x < kGroups; ++x) {
        const float il = l_run[x] > 0.f ? 1.f / l_run[x] : 0.f;
#pragma unroll
        for (int j = 0; j < kCB; ++j) {
          const f16x4 h = {(_Float16)(O[x][j][0] * il), (_Float16)(O[x][j][1] * il),
                           (_Float16)(O[x][j][2] * il), (_Float16)(O[x][j][3] * il)};
          *(f16x4*)(po + ((x * kCB + j) * kWave + lane) * 4) = h;
        }
      }
      if (pw == 0 && g == 0)
#pragma unroll
        for (int x = 0; x < kGroups; ++x) {
          float* pml = part_ml_of(c, x);
          pml[0] = m_run[x];
          pml[1] = l_run[x];
        }
    }
    return;
  }
  // (the planner refuses the in-kernel merge for blocks of four head groups)
  if constexpr (kGroups <= 2) {
  if (tid == 0) flag_sh = atomicAdd(arrived, 1) == a.chunks - 1 ? 2 : 0;
  __syncthreads();
  if (flag_sh != 2) {
    if (!is_qk) {
      float* po = part_o_of(c, pw);
#pragma unroll
      for (int x = 0; x < kGroups; ++x)
#pragma unroll
        for (int j = 0; j < kCB; ++j) store_dev16(po + ((x * kCB + j) * kWave + lane) * 4, O[x][j]);
      if (pw == 0 && g == 0)
#pragma unroll
        for (int x = 0; x < kGroups; ++x) {
          float* pml = part_ml_of(c, x);
          store_dev(pml, m_run[x]);
          store_dev(pml + 1, l_run[x]);
        }
    }
    wait_vmcnt<0>();  // this wave's stores are complete before the barrier
    __syncthreads();
    if (tid == 0) atomicAdd(published, 1);
    return;
  }
  // The merger: the PV waves stage their own chunk's accumulators in LDS
  // (same layout as a published partial) while thread 0 waits for the
  // others; then every wave merges an equal share of the block's output.
  f32x4* own = (f32x4*)smem;  // [PV wave][group][column block][lane]
  static_assert(kPVWaves * kGroups * kCB * kWave * 16 <= kSmemBytes, "merge staging area");
  if (!is_qk)
#pragma unroll
    for (int x = 0; x < kGroups; ++x)
#pragma unroll
      for (int j = 0; j < kCB; ++j) own[((pw * kGroups + x) * kCB + j) * kWave + lane] = O[x][j];
  if (tid == 0) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    bool ok = true;
    while (__hip_atomic_load(published, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
           a.chunks - 1) {
      if (__builtin_amdgcn_s_memrealtime() - t0 > kMergeWaitTicks) {
        ok = false;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    flag_sh = ok ? 2 : 3;
    // Every chunk has arrived: the arrival count restarts at 0. The
    // published count drops by the chunks-1 publishes this launch owes, so
    // it is back at 0 once they are all in, even if some come after a
    // timed-out wait. A timeout also marks the workspace, so that every
    // later launch on it is poisoned until it is zeroed again.
    __hip_atomic_store(arrived, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_add(published, -(a.chunks - 1), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    if (!ok) __hip_atomic_store(a.ws_status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  const float poison = flag_sh == 2 && !sticky_bad ? 0.f : __builtin_nanf("");
  // Wave w merges units (group x, column block j) half*kU .. half*kU + kU - 1
  // of PV wave src = w % kPVWaves's register order (unit = x * kCB + j); a
  // PV wave's single unit is merged by the first half of the waves alone.
  constexpr int kHalves = kGroups * kCB >= 2 ? 2 : 1;
  constexpr int kU = kGroups * kCB / kHalves;
  static_assert(kU >= 1 && kHalves * kU == kGroups * kCB && 2 * kPVWaves == kWaves, "merge split");
  const int src = wave % kPVWaves, half = wave / kPVWaves;
  if (half >= kHalves) return;  // (no barrier follows)
  auto unit_x = [&](int u) { return (half * kU + u) / kCB; };
  auto unit_j = [&](int u) { return (half * kU + u) % kCB; };
  // Online log-sum-exp merge over batches of kB chunks in fixed order
  // (deterministic whichever chunk merges): every load of a batch (each
  // chunk's reference, sum and partial) is issued before any is used, so a
  // batch costs one memory latency; a new batch maximum rescales what has
  // been accumulated. A wave's units all belong to one head group, xw.
  static_assert(kGroups == 1 || kU == kCB, "one head group per merging wave");
  const int xw = unit_x(0);
  constexpr int kB = 4;
  float Mw = -INFINITY, Lw = 0.f;
  f32x4 acc[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float m_own = kGroups == 1 ? m_run[0] : (xw == 0 ? m_run[0] : m_run[kGroups - 1]);
  const float l_own = kGroups == 1 ? l_run[0] : (xw == 0 ? l_run[0] : l_run[kGroups - 1]);
  for (int c0 = 0; c0 < a.chunks; c0 += kB) {
    f32x4 pv[kB][kU];
    float mv[kB], lv[kB];
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      const int cc = c0 + b;
      if (cc >= a.chunks) {
        mv[b] = -INFINITY;
        lv[b] = 0.f;
#pragma unroll
        for (int u = 0; u < kU; ++u) pv[b][u] = f32x4{0.f, 0.f, 0.f, 0.f};
      } else if (cc == c) {
        mv[b] = m_own;
        lv[b] = l_own;
#pragma unroll
        for (int u = 0; u < kU; ++u)
          pv[b][u] = own[((src * kGroups + xw) * kCB + unit_j(u)) * kWave + lane];
      } else {
        const float* pml = part_ml_of(cc, xw);
        mv[b] = load_dev(pml);
        lv[b] = load_dev(pml + 1);
        const float* po = part_o_of(cc, src);
#pragma unroll
        for (int u = 0; u < kU; ++u)
          pv[b][u] = load_dev16(po + ((xw * kCB + unit_j(u)) * kWave + lane) * 4);
      }
    }
    // the batch's maximum; what is accumulated so far is rescaled to it (an
    // empty chunk has m = -inf and weighs 0)
    float mb = Mw;
#pragma unroll
    for (int b = 0; b < kB; ++b) mb = fmaxf(mb, mv[b]);
    const float sc = Mw == -INFINITY ? 0.f : fast_exp2(Mw - mb);
    Lw *= sc;
#pragma unroll
    for (int u = 0; u < kU; ++u) acc[u] *= sc;
    Mw = mb;
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      const float w = mv[b] == -INFINITY ? 0.f : fast_exp2(mv[b] - mb);
      if (w != 0.f) {
        Lw += lv[b] * w;
#pragma unroll
        for (int u = 0; u < kU; ++u) acc[u] += pv[b][u] * w;
      }
    }
  }
  // Lane li of a unit holds head li of group xw, latent columns
  // 16 * (src * kCB + j) + 4 * g .. + 3.
  const int hx = hb * a.heads_per_block + xw * 16 + li;
  if (hx < a.H) {
    const float inv = Lw > 0.f ? a.v_scale / Lw : 0.f;
    uint16_t* orow = a.out + ((size_t)r * a.H + hx) * D;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const f32x4 o = acc[u] + poison;
      const bf16x4 v = {(__bf16)(o[0] * inv), (__bf16)(o[1] * inv), (__bf16)(o[2] * inv),
                        (__bf16)(o[3] * inv)};
      *(bf16x4*)(orow + 16 * (src * kCB + unit_j(u)) + 4 * g) = v;
    }
  }
  }  // kGroups <= 2
}

// Scratch of the entry point that allocates nothing (dsa_decode_launch_static):
// the decode's workspace (status word, arrival counters, split partials) for
// callers that cannot allocate device memory. Every GPU the library runs on
// holds its own copy until the process ends; calls on one GPU share it.
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

// Merge of split rows ([attend], the split softmax and its combine), one
// thread per 4 output columns of one head. Every chunk c of (row r, head
// block hb) left its accumulators normalised by its weight sum, a_c = o_c /
// l_c (fp16, in its PV waves' register order), its reference m_c (log2
// domain) and l_c; with M = max_c m_c and w_c = 2^(m_c - M) l_c the output is
//   out = v_scale * sum_c w_c a_c / sum_c w_c
// (0 when every chunk is empty), the chunks taken in order. Thread t of a
// (row, head block) reads element group t of each chunk's partial: in the
// register order that is PV wave src, head group x, column block j, lane
// (head li, column quarter g), the layout the decode kernel stores.
// The chunks are read kBatch at a time, every load of a batch issued before
// any is used (one memory round trip per batch); a later batch with a larger
// reference rescales the sums so far (with at most kBatch chunks, M is the
// batch's maximum and nothing is rescaled). The status word was written, if
// at all, by an earlier kernel on the stream, so a plain load sees it.
template <int D, int kGroups>
__global__ __launch_bounds__(256)
void dsa_combine_kernel(DecodeArgs a) {
  constexpr int kPVWaves = parts_of(kGroups) * kGroups;
  constexpr int kCB = D / 16 / kPVWaves;
  constexpr int kUnits = kPVWaves * kGroups * kCB * kWave;  // float4s per chunk partial
  constexpr int kBlocksPerUnit = kUnits / 256;
  constexpr int kBatch = 4;
  static_assert(kUnits % 256 == 0, "whole blocks per (row, head block)");
  const int rh = blockIdx.x / kBlocksPerUnit;  // r * head_blocks + hb
  const int t = (blockIdx.x % kBlocksPerUnit) * 256 + threadIdx.x;
  if (rh >= a.rows * a.head_blocks) return;
  const bool bad = *a.ws_status != 0;
  const int r = rh / a.head_blocks, hb = rh % a.head_blocks;
  const int lane = t % kWave, li = lane & 15, g = lane >> 4;
  const int j = (t / kWave) % kCB, x = (t / (kWave * kCB)) % kGroups;
  const int src = t / (kWave * kCB * kGroups);
  const int hx = hb * a.heads_per_block + x * 16 + li;  // (past H: computed, not stored)
  const size_t slot0 = (size_t)rh * a.chunks;
  // (m_c, l_c) of this head: float pairs, heads_per_block pairs per chunk
  const float2* ml = (const float2*)a.part_ml + slot0 * a.heads_per_block + x * 16 + li;
  const size_t ml_stride = (size_t)a.heads_per_block;
  // Each chunk keeps an fp32-sized slot of kUnits * 4 floats, one
  // kPartFloats region per PV wave; the fp16 partial fills the first half
  // of its wave's region, 4 halves per (group, block, lane) unit u.
  constexpr int kPartFloats = kGroups * kCB * kWave * 4;
  const int u = t % (kGroups * kCB * kWave);
  const _Float16* p0 = (const _Float16*)(a.part_o + slot0 * kUnits * 4 + src * kPartFloats) + u * 4;
  constexpr size_t kChunkHalves = (size_t)kUnits * 4 * 2;
  float M = -INFINITY, L = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < a.chunks; c0 += kBatch) {
    float2 mlv[kBatch];
    f16x4 h[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int c = min(c0 + k, a.chunks - 1);  // past the last chunk: a repeat, weighted 0
      mlv[k] = ml[c * ml_stride];
      h[k] = *(const f16x4*)(p0 + c * kChunkHalves);
    }
    float mb = M;
#pragma unroll
    for (int k = 0; k < kBatch; ++k)
      if (c0 + k < a.chunks) mb = fmaxf(mb, mlv[k].x);
    if (mb != M) {  // M < mb: rescale what the earlier batches added (nothing when M is -inf)
      const float sc = M == -INFINITY ? 0.f : fast_exp2(M - mb);
      L *= sc;
      o *= sc;
      M = mb;
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const bool use = c0 + k < a.chunks && mlv[k].x != -INFINITY;  // an empty chunk adds nothing
      const float w = use ? fast_exp2(mlv[k].x - M) * mlv[k].y : 0.f;
      const f32x4 hv = use ? f32x4{(float)h[k][0], (float)h[k][1], (float)h[k][2], (float)h[k][3]}
                           : f32x4{0.f, 0.f, 0.f, 0.f};
      L += w;
      o += hv * w;
    }
  }
  const float inv = bad ? __builtin_nanf("") : (L > 0.f ? a.v_scale / L : 0.f);
  const bf16x4 v = {(__bf16)(o[0] * inv), (__bf16)(o[1] * inv), (__bf16)(o[2] * inv),
                    (__bf16)(o[3] * inv)};
  constexpr int kJPerBlock = 256 / kWave;  // column blocks a 256-thread block covers
  if constexpr (kCB % kJPerBlock == 0) {
    // The block's results are 16 heads x 64 consecutive columns (its 4 column
    // blocks of one source wave): staged in LDS, then written as whole
    // 16-byte pieces, 128 bytes of a head row per 8 lanes.
    constexpr int kBlkCols = kJPerBlock * 16;
    constexpr int kStage = 2 * kBlkCols + 16;
    __shared__ __attribute__((aligned(16))) uint8_t stage[16 * kStage];
    const int jj = (t / kWave) % kJPerBlock;
    *(bf16x4*)(stage + li * kStage + 2 * (16 * jj + 4 * g)) = v;
    __syncthreads();
    constexpr int kPieces = 2 * kBlkCols / 16;  // 8 per head row
    if (threadIdx.x < 16 * kPieces) {
      const int row = threadIdx.x / kPieces, pc = threadIdx.x % kPieces;
      const int head = hb * a.heads_per_block + x * 16 + row;
      const int col0 = 16 * (src * kCB + j - jj);  // the block's first column
      if (head < a.H)
        __builtin_nontemporal_store(*(const u32x4*)(stage + row * kStage + 16 * pc),  // (streaming)
                                    (u32x4*)((uint8_t*)(a.out + ((size_t)r * a.H + head) * D + col0) + 16 * pc));
    }
  } else {
    if (hx < a.H) *(bf16x4*)(a.out + ((size_t)r * a.H + hx) * D + 16 * (src * kCB + j) + 4 * g) = v;
  }
}

// Zero a word range (workspace set-up; a kernel rather than a memset so that
// it can sit in a captured graph).
__global__ void dsa_zero_kernel(int32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

// ------------------------------------------------------------------ launch

template <int D, int kGroups>
hipError_t launch_g(bool split_v, bool rope, bool combine, dim3 grid, hipStream_t st,
                    const DecodeArgs& args) {
  const dim3 block(waves_of(kGroups) * kWave);
  if (rope) {
    if constexpr (D == 512 && kGroups <= 2)  // (the planner keeps rope tails to 32-head blocks)
      hipLaunchKernelGGL((dsa_decode_kernel<D, kGroups, false, 64>), grid, block, 0, st, args);
  } else if (split_v) {
    hipLaunchKernelGGL((dsa_decode_kernel<D, kGroups, true>), grid, block, 0, st, args);
  } else {
    hipLaunchKernelGGL((dsa_decode_kernel<D, kGroups, false>), grid, block, 0, st, args);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !combine) return e;
  constexpr int kUnits = D * kGroups * 4;  // float4s of one (row, head block)'s partial
  const dim3 cgrid((unsigned)((size_t)args.rows * args.head_blocks * (kUnits / 256)));
  hipLaunchKernelGGL((dsa_combine_kernel<D, kGroups>), cgrid, dim3(256), 0, st, args);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(int groups, bool split_v, bool rope, bool combine, dim3 grid,
                    hipStream_t st, const DecodeArgs& args) {
  if (groups == 1) return launch_g<D, 1>(split_v, rope, combine, grid, st, args);
  if (groups == 2) return launch_g<D, 2>(split_v, rope, combine, grid, st, args);
  if constexpr (D == 512) return launch_g<D, 4>(split_v, rope, combine, grid, st, args);
  return hipErrorInvalidValue;  // (64-head blocks are planned for kv_lora_rank 512 only)
}


bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int check_workspace(dsa_decode_plan_t plan, const void* workspace, size_t workspace_bytes,
                    const char* who) {
  if (!workspace || !aligned(workspace, kWsAlign) || workspace_bytes < plan->ws.total) {
    std::ostringstream m;
    m << who << ": workspace " << workspace << " of " << workspace_bytes << " bytes; need "
      << plan->ws.total << " bytes, 256-byte aligned";
    return fail(DSA_DECODE_ERR_WORKSPACE, m.str());
  }
  return DSA_DECODE_OK;
}

int check_device(dsa_decode_plan_t plan, const char* who) {
  if (plan->device < 0) {
    std::ostringstream m;
    m << who << ": host-only plan (device -1) cannot launch";
    return fail(DSA_DECODE_ERR_INVALID, m.str());
  }
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur != plan->device) {
    std::ostringstream m;
    m << who << ": current HIP device is " << cur << ", plan was made for " << plan->device;
    return fail(DSA_DECODE_ERR_DEVICE, m.str());
  }
  return DSA_DECODE_OK;
}

int check_launch(dsa_decode_plan_t plan, const void* q, const void* k_cache,
                 const void* v_cache, const int32_t* block_tables, const int32_t* seq_lens,
                 const int32_t* sel_indices, float k_scale, float v_scale, const void* out,
                 const char* who) {
  if (!plan) return fail(DSA_DECODE_ERR_INVALID, std::string(who) + ": plan is NULL");
  int st = check_device(plan, who);
  if (st != DSA_DECODE_OK) return st;
  if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !sel_indices || !out)
    return fail(DSA_DECODE_ERR_INVALID, std::string(who) + ": NULL device pointer");
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return fail(DSA_DECODE_ERR_INVALID,
                std::string(who) + ": q, out, k_cache and v_cache must be 16-byte aligned");
  if (!std::isfinite(k_scale) || !(k_scale > 0.f) || !std::isfinite(v_scale)) {
    std::ostringstream m;
    m << who << ": k_scale must be finite and > 0 and v_scale finite (got " << k_scale
      << ", " << v_scale << ")";
    return fail(DSA_DECODE_ERR_INVALID, m.str());
  }
  // A rope-tail token is one buffer: the values are its latent bytes.
  if (plan->p.qk_rope_dim != 0 && k_cache != v_cache)
    return fail(DSA_DECODE_ERR_INVALID,
                std::string(who) + ": with a rope tail the values are the latent part of "
                "the same tokens; v_cache must equal k_cache");
  return DSA_DECODE_OK;
}

int enqueue_decode(dsa_decode_plan_t plan, const void* q, const void* k_cache,
                   const void* v_cache, const int32_t* block_tables, const int32_t* seq_lens,
                   const int32_t* sel_indices, float k_scale, float v_scale, void* out,
                   void* workspace, hipStream_t stream_h, const char* who);

// Device address of this device's copy of `scratch`, looked up once per
// device (with that device current) and kept. In host code the array's name
// is only a stand-in for the symbol, never a device address.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int static_scratch(int device, void** out, const char* who) {
  if (device < 0 || device >= kMaxDevices) {
    std::ostringstream m;
    m << who << ": device " << device << " is beyond the " << kMaxDevices
      << " devices the static scratch table covers";
    return fail(DSA_DECODE_ERR_DEVICE, m.str());
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return fail(DSA_DECODE_ERR_DEVICE, std::string(who) + ": hipGetSymbolAddress(scratch): " +
                                             hipGetErrorString(e));
    }
    g_scratch_ptr[device] = ptr;
  }
  *out = g_scratch_ptr[device];
  return DSA_DECODE_OK;
}

}  // namespace
}  // namespace dsa

extern "C" {

void dsa_decode_plan_destroy(dsa_decode_plan_t plan) {
  if (!plan) return;
  for (void* e : plan->events)
    if (e) (void)hipEventDestroy((hipEvent_t)e);
  delete plan;
}

int dsa_decode_workspace_init(dsa_decode_plan_t plan, void* workspace, size_t workspace_bytes,
                              void* stream) {
  using namespace dsa;
  if (!plan) return fail(DSA_DECODE_ERR_INVALID, "dsa_decode_workspace_init: plan is NULL");
  int st = check_device(plan, "dsa_decode_workspace_init");
  if (st != DSA_DECODE_OK) return st;
  st = check_workspace(plan, workspace, workspace_bytes, "dsa_decode_workspace_init");
  if (st != DSA_DECODE_OK) return st;
  const size_t words = plan->ws.total / sizeof(int32_t);
  const int blocks = (int)std::min<size_t>((words + 255) / 256, 1024);
  hipLaunchKernelGGL(dsa_zero_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                     (int32_t*)workspace, words);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(DSA_DECODE_ERR_LAUNCH,
                std::string("dsa_decode_workspace_init: ") + hipGetErrorString(e));
  return DSA_DECODE_OK;
}

int dsa_decode_launch(dsa_decode_plan_t plan, const void* q, const void* k_cache,
                      const void* v_cache, const int32_t* block_tables,
                      const int32_t* seq_lens, const int32_t* sel_indices,
                      float k_scale, float v_scale, void* out, void* workspace,
                      size_t workspace_bytes, void* stream) {
  using namespace dsa;
  int st = check_launch(plan, q, k_cache, v_cache, block_tables, seq_lens, sel_indices,
                        k_scale, v_scale, out, "dsa_decode_launch");
  if (st != DSA_DECODE_OK) return st;
  st = check_workspace(plan, workspace, workspace_bytes, "dsa_decode_launch");
  if (st != DSA_DECODE_OK) return st;
  return enqueue_decode(plan, q, k_cache, v_cache, block_tables, seq_lens, sel_indices,
                        k_scale, v_scale, out, workspace, (hipStream_t)stream,
                        "dsa_decode_launch");
}

int dsa_decode_launch_static(dsa_decode_plan_t plan, const void* q, const void* k_cache,
                             const void* v_cache, const int32_t* block_tables,
                             const int32_t* seq_lens, const int32_t* sel_indices,
                             float k_scale, float v_scale, void* out, void* stream) {
  using namespace dsa;
  const char* who = "dsa_decode_launch_static";
  int st = check_launch(plan, q, k_cache, v_cache, block_tables, seq_lens, sel_indices,
                        k_scale, v_scale, out, who);
  if (st != DSA_DECODE_OK) return st;
  if (plan->p.flags & DSA_DECODE_FLAG_EXPORT_SELECTION)
    return fail(DSA_DECODE_ERR_INVALID,
                std::string(who) + ": the selection export is read back from a caller "
                "workspace; make the plan without DSA_DECODE_FLAG_EXPORT_SELECTION");
  if (plan->ws.total > kStaticScratchBytes) {
    std::ostringstream m;
    m << who << ": the plan needs " << plan->ws.total
      << " bytes of scratch, more than the library's static " << kStaticScratchBytes
      << " bytes; use dsa_decode_launch with a workspace";
    return fail(DSA_DECODE_ERR_WORKSPACE, m.str());
  }
  void* ws = nullptr;
  st = static_scratch(plan->device, &ws, who);
  if (st != DSA_DECODE_OK) return st;
  // The scratch keeps whatever the last call on this device left in it. The
  // status word and the arrival counters must start at zero: cleared by a
  // fill kernel (not a memset, so the call can be captured in a graph).
  const hipStream_t s = (hipStream_t)stream;
  const size_t words = (plan->ws.arrivals + sizeof(int32_t) * 2 * (size_t)plan->p.num_rows *
                        (size_t)plan->head_blocks) / sizeof(int32_t);
  hipLaunchKernelGGL(dsa_zero_kernel, dim3((unsigned)std::min<size_t>((words + 255) / 256, 1024)),
                     dim3(256), 0, s, (int32_t*)ws, words);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(DSA_DECODE_ERR_LAUNCH, std::string(who) + ": " + hipGetErrorString(e));
  return enqueue_decode(plan, q, k_cache, v_cache, block_tables, seq_lens, sel_indices,
                        k_scale, v_scale, out, ws, s, who);
}

}  // extern "C"

namespace dsa {
namespace {

int enqueue_decode(dsa_decode_plan_t plan, const void* q, const void* k_cache,
                   const void* v_cache, const int32_t* block_tables, const int32_t* seq_lens,
                   const int32_t* sel_indices, float k_scale, float v_scale, void* out,
                   void* workspace, hipStream_t stream_h, const char* who) {
  const dsa_decode_params& p = plan->p;
  uint8_t* ws = (uint8_t*)workspace;

  hipEvent_t* ev = nullptr;
  if (plan->timing_count < plan->timing_capacity)
    ev = (hipEvent_t*)&plan->events[2 * plan->timing_count++];
  if (ev) (void)hipEventRecord(ev[0], stream_h);

  DecodeArgs da;
  da.q = (const uint16_t*)q;
  da.k_cache = (const uint8_t*)k_cache;
  da.v_cache = (const uint8_t*)v_cache;
  da.block_tables = block_tables;
  da.seq_lens = seq_lens;
  da.sel = sel_indices;
  da.out = (uint16_t*)out;
  da.export_sel = (p.flags & DSA_DECODE_FLAG_EXPORT_SELECTION) != 0;
  da.ws_status = (int32_t*)(ws + plan->ws.status);
  da.ws_ids = da.export_sel ? (int32_t*)(ws + plan->ws.ids) : nullptr;
  da.ws_offsets = da.export_sel ? (uint64_t*)(ws + plan->ws.offsets) : nullptr;
  da.ws_counts = da.export_sel ? (int32_t*)(ws + plan->ws.counts) : nullptr;
  da.ws_arrivals = (int32_t*)(ws + plan->ws.arrivals);
  da.part_o = plan->chunks > 1 ? (float*)(ws + plan->ws.part_o) : nullptr;
  da.part_ml = plan->chunks > 1 ? (float*)(ws + plan->ws.part_ml) : nullptr;
  da.stride_rows = (uint32_t)(p.cache_stride_bytes / token_bytes(p));
  da.rows = p.num_rows;
  da.H = p.num_q_heads;
  da.width = p.sel_width;
  da.max_seq_len = p.max_seq_len;
  da.bt_stride = p.block_table_stride;
  da.bt_entries = (int)(((int64_t)p.max_seq_len + p.block_size - 1) / p.block_size);
  da.block_size = p.block_size;
  da.bs_shift = (p.block_size & (p.block_size - 1)) == 0 ? __builtin_ctz((unsigned)p.block_size) : -1;
  da.chunks = plan->chunks;
  da.chunk_tokens = plan->chunk_tokens;
  da.chunk_lead = plan->chunk_lead;
  da.head_blocks = plan->head_blocks;
  da.heads_per_block = plan->heads_per_block;
  da.rows_hb = p.num_rows * plan->head_blocks;
  da.group_units = plan->group_units;
  da.scale_log2 = p.sm_scale * k_scale * kLog2e;
  da.v_scale = v_scale;
  da.merge_in_kernel = plan->merge_in_kernel ? 1 : 0;
  const int groups = plan->heads_per_block / 16;
  const bool split_v = k_cache != v_cache;
  const bool rope = p.qk_rope_dim != 0;
  const bool combine = plan->chunks > 1 && !plan->merge_in_kernel;
  const dim3 grid(plan->workgroups);
  hipError_t e;
  switch (p.kv_lora_rank) {
    case 64: e = launch_d<64>(groups, split_v, rope, combine, grid, stream_h, da); break;
    case 128: e = launch_d<128>(groups, split_v, rope, combine, grid, stream_h, da); break;
    case 256: e = launch_d<256>(groups, split_v, rope, combine, grid, stream_h, da); break;
    default: e = launch_d<512>(groups, split_v, rope, combine, grid, stream_h, da); break;
  }
  if (e != hipSuccess)
    return fail(DSA_DECODE_ERR_LAUNCH,
                std::string(who) + ": decode kernel: " + hipGetErrorString(e));
  if (ev) (void)hipEventRecord(ev[1], stream_h);
  return DSA_DECODE_OK;
}

}  // namespace
}  // namespace dsa

extern "C" {

int dsa_decode_read_selection(dsa_decode_plan_t plan, const void* workspace,
                              size_t workspace_bytes, int32_t* ids, int32_t* counts,
                              uint64_t* offsets, void* stream) {
  using namespace dsa;
  if (!plan || !workspace)
    return fail(DSA_DECODE_ERR_INVALID, "dsa_decode_read_selection: NULL plan or workspace");
  int st = check_device(plan, "dsa_decode_read_selection");
  if (st != DSA_DECODE_OK) return st;
  if (workspace_bytes < plan->ws.total)
    return fail(DSA_DECODE_ERR_WORKSPACE, "dsa_decode_read_selection: workspace too small");
  if (!(plan->p.flags & DSA_DECODE_FLAG_EXPORT_SELECTION))
    return fail(DSA_DECODE_ERR_INVALID,
                "dsa_decode_read_selection: the plan was made without "
                "DSA_DECODE_FLAG_EXPORT_SELECTION, so launches do not export the selection");
  const uint8_t* ws = (const uint8_t*)workspace;
  const size_t RW = (size_t)plan->p.num_rows * plan->p.sel_width;
  const hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (ids && e == hipSuccess)
    e = hipMemcpyAsync(ids, ws + plan->ws.ids, RW * sizeof(int32_t), hipMemcpyDeviceToDevice, s);
  if (counts && e == hipSuccess)
    e = hipMemcpyAsync(counts, ws + plan->ws.counts, plan->p.num_rows * sizeof(int32_t),
                       hipMemcpyDeviceToDevice, s);
  if (offsets && e == hipSuccess)
    e = hipMemcpyAsync(offsets, ws + plan->ws.offsets, RW * sizeof(uint64_t),
                       hipMemcpyDeviceToDevice, s);
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
  plan->events.assign((size_t)2 * max_launches, nullptr);
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
  *kernel_ms = 0.f;
  *launches = plan->timing_count;
  int status = DSA_DECODE_OK;
  for (int i = 0; i < plan->timing_count; ++i) {
    hipEvent_t* ev = (hipEvent_t*)&plan->events[2 * i];
    if (hipEventSynchronize(ev[1]) != hipSuccess) {
      status = fail(DSA_DECODE_ERR_DEVICE, "dsa_decode_timing_end: hipEventSynchronize failed");
      break;
    }
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, ev[0], ev[1]) == hipSuccess) *kernel_ms += ms;
  }
  for (void* e : plan->events)
    if (e) (void)hipEventDestroy((hipEvent_t)e);
  plan->events.clear();
  plan->timing_capacity = 0;
  plan->timing_count = 0;
  return status;
}

}  // extern "C"
