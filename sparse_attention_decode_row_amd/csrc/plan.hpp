// Internal plan shared by the host planner (plan.cpp) and the launcher
// (kernels.hip). Not part of the public ABI (include/dsa_decode.h).
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "dsa_decode.h"

namespace dsa {

// Granularity of a chunk (the selected tokens one workgroup takes).
constexpr int kTileTokens = 64;  // chunk sizes are multiples of this
// Largest chunk one workgroup handles (its latent-row table lives in LDS:
// 2048 x 4 B = 8 KiB).
constexpr int kMaxChunkTokens = 2048;
// A plan's largest chunk: a workgroup holds its latent-row table in LDS
// (with or without a rope tail).
inline int max_chunk_tokens(const dsa_decode_params& p) {
  (void)p;
  return kMaxChunkTokens;
}
// Bytes of one cached token.
inline uint64_t token_bytes(const dsa_decode_params& p) {
  return (uint64_t)p.kv_lora_rank + (uint64_t)p.qk_rope_dim;
}

// Heads one workgroup covers: 2 groups of 16 heads (four waves per group),
// or a single group.
constexpr int kHeadsPerBlock = 32;
constexpr int kHeadsPerSmallBlock = 16;
constexpr int kHeadsPerLargeBlock = 64;  // four 16-head groups (kv_lora_rank 512, no rope tail)
// Workspace sub-buffer alignment.
constexpr size_t kWsAlign = 256;

struct WorkspaceLayout {
  size_t status = 0;    // int32: 0 healthy, 1 after a split merge gave up waiting (sticky)
  size_t arrivals = 0;  // int32 [2, R, head_blocks] arrived / published counts (zero between launches)
  size_t ids = 0;       // int32 [R, W]  (DSA_DECODE_FLAG_EXPORT_SELECTION only)
  size_t offsets = 0;   // uint64 [R, W] (DSA_DECODE_FLAG_EXPORT_SELECTION only)
  size_t counts = 0;    // int32 [R]     (DSA_DECODE_FLAG_EXPORT_SELECTION only)
  size_t part_o = 0;    // float [R, head_blocks, C, heads_per_block, D] (C > 1 only)
  size_t part_ml = 0;   // float [R, head_blocks, C, heads_per_block, 2] (C > 1 only)
  size_t total = 0;
};

}  // namespace dsa

struct dsa_decode_plan_s {
  dsa_decode_params p{};          // validated; cache_stride_bytes filled in
  int device = -1;
  int num_cus = 256;
  int chunk_tokens = 0;           // multiple of kTileTokens, <= kMaxChunkTokens
  int chunks = 1;                 // per row per head block
  int chunk_lead = 0;             // extra tokens of chunk 0 (multiple of kTileTokens)
  bool merge_in_kernel = false;   // split rows merged by their last chunk, not by a combine kernel
  int head_blocks = 1;
  int heads_per_block = dsa::kHeadsPerBlock;
  int layout = DSA_DECODE_LAYOUT_HEADS32;
  int workgroups = 0;             // launched grid (rows x chunks padded to 8, x head blocks)
  int group_units = 1;            // (row, chunk) units co-scheduled on one XCD: rows_per_sequence x chunks, or 1
  dsa::WorkspaceLayout ws;
  // benchmark timing (dsa_decode_timing_begin / _end)
  std::vector<void*> events;      // hipEvent_t, 2 per recorded launch
  int timing_capacity = 0;
  int timing_count = 0;
};

namespace dsa {

// Thread-local error text.
void set_error(const std::string& msg);
int fail(int status, const std::string& msg);

// Pure host validation of params (no GPU needed). Returns a status and sets
// the error text on failure; fills *norm with the normalised params.
int validate_params(const dsa_decode_params* p, dsa_decode_params* norm);

// Split decomposition and workspace layout for validated params.
void plan_layout(dsa_decode_plan_s* plan);

}  // namespace dsa
