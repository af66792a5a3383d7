// Host-side validation and planning of the selected-index NoPE MLA decode.
//
// The geometry rules come from the launcher page "spark_model/layers/
// glm5next_dsa/attend.rs" (DsaDecodePaging::validate and decode_attention's
// guards) and the block-table capacity check of "metrale_model_arch/
// glm5next_dsa/layer/decode_k.rs". Every rule is an error with the
// offending values in the message; nothing falls back to another path.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <sstream>

#include "plan.hpp"

namespace dsa {

namespace {
thread_local std::string g_error;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool supported_rank(int32_t d) { return d == 64 || d == 128 || d == 256 || d == 512; }
}  // namespace

void set_error(const std::string& msg) { g_error = msg; }

int fail(int status, const std::string& msg) {
  g_error = msg;
  return status;
}

int validate_params(const dsa_decode_params* p, dsa_decode_params* norm) {
  if (!p) return fail(DSA_DECODE_ERR_INVALID, "dsa_decode_plan: params is NULL");
  std::ostringstream m;
  // A launch with no rows or no heads is refused as degenerate.
  if (p->num_rows <= 0 || p->num_q_heads <= 0) {
    m << "dsa_decode_plan: degenerate launch (" << p->num_rows << " rows, "
      << p->num_q_heads << " heads)";
    return fail(DSA_DECODE_ERR_INVALID, m.str());
  }
  if (p->block_size <= 0) {
    m << "dsa_decode_plan: block_size must be > 0, got " << p->block_size;
    return fail(DSA_DECODE_ERR_INVALID, m.str());
  }
  if (p->index_kpool <= 0) {
    m << "dsa_decode_plan: index_kpool must be > 0, got " << p->index_kpool;
    return fail(DSA_DECODE_ERR_INVALID, m.str());
  }
  // The selector builds pools over absolute positions; a page size that is
  // not a whole number of pools would split a pool across two pages.
  if (p->block_size % p->index_kpool != 0) {
    m << "dsa_decode_plan: block_size " << p->block_size
      << " is not a multiple of index_kpool " << p->index_kpool
      << " (a selector pool would straddle a page boundary)";
    return fail(DSA_DECODE_ERR_INVALID, m.str());
  }
  // MLA keeps one latent KV head.
  if (p->num_kv_heads != 1) {
    m << "dsa_decode_plan: MLA has a single latent KV head, got num_kv_heads "
      << p->num_kv_heads;
    return fail(DSA_DECODE_ERR_INVALID, m.str());
  }
  // The kernels are compiled for a fixed set of latent widths; any other
  // width would mis-tile silently, so it is refused.
  if (!supported_rank(p->kv_lora_rank)) {
    m << "dsa_decode_plan: kv_lora_rank " << p->kv_lora_rank
      << " is not compiled in (supported: 64, 128, 256, 512)";
    return fail(DSA_DECODE_ERR_UNSUPPORTED, m.str());
  }
  // The rope-tail token is compiled for one shape only: 512 + 64.
  if (p->qk_rope_dim != 0 && p->qk_rope_dim != 64) {
    m << "dsa_decode_plan: qk_rope_dim " << p->qk_rope_dim
      << " is not compiled in (supported: 0, 64)";
    return fail(DSA_DECODE_ERR_UNSUPPORTED, m.str());
  }
  if (p->qk_rope_dim == 64 && p->kv_lora_rank != 512) {
    m << "dsa_decode_plan: a 64-wide rope tail is compiled for kv_lora_rank 512 only, got "
      << p->kv_lora_rank;
    return fail(DSA_DECODE_ERR_UNSUPPORTED, m.str());
  }
  if (p->sel_width <= 0) {
    m << "dsa_decode_plan: sel_width must be > 0, got " << p->sel_width;
    return fail(DSA_DECODE_ERR_INVALID, m.str());
  }
  if (p->max_seq_len <= 0) {
    m << "dsa_decode_plan: max_seq_len must be > 0, got " << p->max_seq_len;
    return fail(DSA_DECODE_ERR_INVALID, m.str());
  }
  if (p->block_table_stride < 0) {
    m << "dsa_decode_plan: block_table_stride must be >= 0, got "
      << p->block_table_stride;
    return fail(DSA_DECODE_ERR_INVALID, m.str());
  }
  const uint64_t tok = token_bytes(*p);  // kv_lora_rank (+ qk_rope_dim)
  const uint64_t row_bytes = (uint64_t)p->block_size * tok;
  const uint64_t stride = p->cache_stride_bytes ? p->cache_stride_bytes : row_bytes;
  if (stride < row_bytes) {
    m << "dsa_decode_plan: cache_stride_bytes " << stride
      << " is smaller than one page (block_size * token bytes = " << row_bytes << ")";
    return fail(DSA_DECODE_ERR_INVALID, m.str());
  }
  // Token rows are addressed by index (byte offset / token bytes), so a
  // page must start on a row boundary.
  if (stride % tok != 0) {
    m << "dsa_decode_plan: cache_stride_bytes " << stride
      << " is not a multiple of the token's " << tok << " bytes";
    return fail(DSA_DECODE_ERR_INVALID, m.str());
  }
  if (stride / tok > UINT32_MAX) {
    m << "dsa_decode_plan: cache_stride_bytes " << stride
      << " spans more than 2^32 latent rows";
    return fail(DSA_DECODE_ERR_INVALID, m.str());
  }
  // A per-row table must cover every position the row may attend: its entry
  // count is a number of pages, max_seq_len a number of tokens.
  if (p->block_table_stride > 0 &&
      (int64_t)p->max_seq_len > (int64_t)p->block_table_stride * p->block_size) {
    m << "dsa_decode_plan: max_seq_len " << p->max_seq_len
      << " tokens needs " << (p->max_seq_len + p->block_size - 1) / p->block_size
      << " block-table entries per row but block_table_stride is "
      << p->block_table_stride << " (block_size " << p->block_size << ")";
    return fail(DSA_DECODE_ERR_INVALID, m.str());
  }
  if (!std::isfinite(p->sm_scale)) {
    m << "dsa_decode_plan: sm_scale must be finite, got " << p->sm_scale;
    return fail(DSA_DECODE_ERR_INVALID, m.str());
  }
  if (p->chunk_tokens < 0 ||
      (p->chunk_tokens > 0 && (p->chunk_tokens % kTileTokens != 0 ||
                               p->chunk_tokens > max_chunk_tokens(*p)))) {
    m << "dsa_decode_plan: chunk_tokens " << p->chunk_tokens
      << " must be 0 or a multiple of " << kTileTokens << " up to "
      << max_chunk_tokens(*p);
    return fail(DSA_DECODE_ERR_INVALID, m.str());
  }
  if (p->rows_per_sequence < 0 ||
      (p->rows_per_sequence > 1 && p->num_rows % p->rows_per_sequence != 0)) {
    m << "dsa_decode_plan: rows_per_sequence " << p->rows_per_sequence
      << " must be 0, 1, or a k > 1 that divides num_rows " << p->num_rows;
    return fail(DSA_DECODE_ERR_INVALID, m.str());
  }
  for (int i = 0; i < 2; ++i)
    if (p->reserved[i] != 0)
      return fail(DSA_DECODE_ERR_INVALID, "dsa_decode_plan: reserved fields must be zero");
  if ((p->flags & ~(DSA_DECODE_FLAG_EXPORT_SELECTION | DSA_DECODE_FLAG_MERGE_IN_KERNEL)) != 0) {
    m << "dsa_decode_plan: unknown flags 0x" << std::hex << p->flags;
    return fail(DSA_DECODE_ERR_INVALID, m.str());
  }
  if (p->layout < DSA_DECODE_LAYOUT_AUTO || p->layout > DSA_DECODE_LAYOUT_HEADS64) {
    m << "dsa_decode_plan: layout " << p->layout
      << " is not 0 (auto), 1 (32-head blocks), 2 (16-head blocks) or 3 (64-head blocks)";
    return fail(DSA_DECODE_ERR_INVALID, m.str());
  }
  // 64-head blocks are compiled for the 512-wide latent alone; their LDS
  // leaves no room for rope tails, and the in-kernel merge takes at most two
  // head groups per workgroup.
  if (p->layout == DSA_DECODE_LAYOUT_HEADS64 &&
      (p->kv_lora_rank != 512 || p->qk_rope_dim != 0 ||
       (p->flags & DSA_DECODE_FLAG_MERGE_IN_KERNEL))) {
    m << "dsa_decode_plan: 64-head blocks (layout 3) need kv_lora_rank 512, no rope tail and "
         "no DSA_DECODE_FLAG_MERGE_IN_KERNEL (got kv_lora_rank " << p->kv_lora_rank
      << ", qk_rope_dim " << p->qk_rope_dim << ", flags 0x" << std::hex << p->flags << ")";
    return fail(DSA_DECODE_ERR_UNSUPPORTED, m.str());
  }
  // Offsets into the selection, q and out are formed in 64-bit arithmetic
  // on the device; the per-row element counts must fit 32 bits.
  if ((int64_t)p->num_q_heads * p->kv_lora_rank > INT32_MAX) {
    m << "dsa_decode_plan: num_q_heads * kv_lora_rank overflows int32";
    return fail(DSA_DECODE_ERR_INVALID, m.str());
  }
  *norm = *p;
  norm->cache_stride_bytes = stride;
  return DSA_DECODE_OK;
}

void plan_layout(dsa_decode_plan_s* plan) {
  const dsa_decode_params& p = plan->p;
  const int64_t R = p.num_rows, H = p.num_q_heads, D = p.kv_lora_rank,
                W = p.sel_width;
  // Blocks of 32 heads (two 16-head groups, eight waves) unless the heads
  // fit one group, or 64-head blocks where they still give every CU a
  // workgroup without splitting rows (many rows: one step over four head
  // groups costs less than two steps over two) and are compiled (512-wide
  // latent, no rope tail, no in-kernel merge). Every workgroup holds a CU's
  // LDS, so the grid aims at one workgroup per CU.
  int layout = p.layout;
  const int64_t wg_target = plan->num_cus;
  if (layout == DSA_DECODE_LAYOUT_AUTO) {
    const bool h64_ok = D == 512 && p.qk_rope_dim == 0 &&
                        !(p.flags & DSA_DECODE_FLAG_MERGE_IN_KERNEL);
    if (H <= kHeadsPerSmallBlock)
      layout = DSA_DECODE_LAYOUT_HEADS16;
    else if (h64_ok && H > kHeadsPerBlock &&
             R * ((H + kHeadsPerLargeBlock - 1) / kHeadsPerLargeBlock) >= wg_target)
      layout = DSA_DECODE_LAYOUT_HEADS64;
    else
      layout = DSA_DECODE_LAYOUT_HEADS32;
  }
  plan->layout = layout;
  plan->heads_per_block = layout == DSA_DECODE_LAYOUT_HEADS16   ? kHeadsPerSmallBlock
                           : layout == DSA_DECODE_LAYOUT_HEADS64 ? kHeadsPerLargeBlock
                                                                 : kHeadsPerBlock;
  plan->head_blocks = (int)((H + plan->heads_per_block - 1) / plan->heads_per_block);
  // A row can attend at most min(W, max_seq_len) distinct tokens.
  const int64_t wmax = std::min<int64_t>(W, p.max_seq_len);
  int64_t ct;
  if (p.chunk_tokens > 0) {
    ct = p.chunk_tokens;
  } else {
    // Spread the largest possible per-row work over the compute units:
    // tokens one workgroup should take so that rows x head blocks x chunks
    // is about one workgroup per CU.
    const int64_t units = R * plan->head_blocks;
    int64_t per_wg = (wmax * units + wg_target - 1) / wg_target;
    ct = (per_wg + kTileTokens - 1) / kTileTokens * kTileTokens;
    ct = std::max<int64_t>(ct, kTileTokens);
    ct = std::min<int64_t>(ct, max_chunk_tokens(p));
  }
  const int64_t wmax_tiles = (wmax + kTileTokens - 1) / kTileTokens * kTileTokens;
  ct = std::min<int64_t>(ct, std::max<int64_t>(wmax_tiles, kTileTokens));
  plan->chunk_tokens = (int)ct;
  plan->chunks = (int)((wmax + ct - 1) / ct);
  if (plan->chunks < 1) plan->chunks = 1;
  // With several chunks, either a combine kernel merges every chunk's
  // partials, or (DSA_DECODE_FLAG_MERGE_IN_KERNEL) the last chunk of a row to
  // finish merges the others'. In the second case chunk 0 gets one more
  // 128-token tile (and the last chunk one fewer), which makes it that last
  // one, so the others publish their partials while it still computes. The
  // rank ranges still cover [0, chunks * ct).
  plan->chunk_lead = 0;
  plan->merge_in_kernel = (p.flags & DSA_DECODE_FLAG_MERGE_IN_KERNEL) != 0;
  if (plan->chunks > 1 && p.chunk_tokens == 0 && plan->merge_in_kernel) {
    const int64_t lead = std::min<int64_t>(2 * kTileTokens, max_chunk_tokens(p) - ct);
    if (lead > 0 && ct > lead) {
      plan->chunk_lead = (int)lead;
      // The lead can leave the last chunk without any rank: count the chunks
      // again. If chunk 0 then holds every rank, one chunk of that size it is.
      const int64_t c2 = std::max<int64_t>(1, (wmax - lead + ct - 1) / ct);
      if (c2 == 1) {
        plan->chunks = 1;
        plan->chunk_lead = 0;
        plan->chunk_tokens = (int)((wmax + kTileTokens - 1) / kTileTokens * kTileTokens);
      } else {
        plan->chunks = (int)c2;
      }
    }
  }

  WorkspaceLayout& L = plan->ws;
  size_t off = 0;
  L.status = off;
  off = align_up(off + sizeof(int32_t), kWsAlign);
  L.arrivals = off;
  off = align_up(off + sizeof(int32_t) * 2 * R * plan->head_blocks, kWsAlign);
  if (p.flags & DSA_DECODE_FLAG_EXPORT_SELECTION) {
    L.ids = off;
    off = align_up(off + sizeof(int32_t) * R * W, kWsAlign);
    L.offsets = off;
    off = align_up(off + sizeof(uint64_t) * R * W, kWsAlign);
    L.counts = off;
    off = align_up(off + sizeof(int32_t) * R, kWsAlign);
  }
  if (plan->chunks > 1) {
    // Partials are kept per workgroup for a full block of heads_per_block
    // heads (a block that holds fewer heads still stores whole head groups).
    const int64_t slots = R * plan->head_blocks * plan->chunks * plan->heads_per_block;
    L.part_o = off;
    off = align_up(off + sizeof(float) * slots * D, kWsAlign);
    L.part_ml = off;
    off = align_up(off + sizeof(float) * slots * 2, kWsAlign);
  }
  L.total = off;
  // Workgroup ids: the head blocks of one (row, chunk) are 8 apart, so the
  // (row, chunk) count is padded to a multiple of 8 (padding ids exit).
  // Grouped units: the rows_per_sequence x chunks units of one sequence (a
  // sequence is one row unless rows are co-scheduled) take consecutive
  // rounds of 8 ids on one XCD, 8 sequences per block of rounds, so the unit
  // count is padded to whole blocks. The units of a group read the same
  // query rows and ids (the chunks of a row) or largely the same latent rows
  // (the rows of a sequence), which that XCD's L2 then serves once.
  const int64_t k = p.rows_per_sequence > 1 ? p.rows_per_sequence : 1;
  plan->group_units = (k > 1 || plan->chunks > 1) ? (int)(k * plan->chunks) : 1;
  if (plan->group_units > 1) {
    const int64_t seqs = R / k;
    plan->workgroups = (int)((seqs + 7) / 8 * 8 * plan->group_units * plan->head_blocks);
  } else {
    plan->workgroups = (int)((R * plan->chunks + 7) / 8 * 8 * plan->head_blocks);
  }
}

}  // namespace dsa

extern "C" {

const char* dsa_decode_last_error(void) { return dsa::g_error.c_str(); }

int dsa_decode_version(void) { return DSA_DECODE_VERSION; }

int dsa_decode_plan(const dsa_decode_params* params, int device,
                    dsa_decode_plan_t* out) {
  if (!out) return dsa::fail(DSA_DECODE_ERR_INVALID, "dsa_decode_plan: out is NULL");
  *out = nullptr;
  dsa_decode_params norm{};
  int st = dsa::validate_params(params, &norm);
  if (st != DSA_DECODE_OK) return st;

  int num_cus = 256;
  if (device >= 0) {
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || device >= count) {
      (void)hipGetLastError();
      std::ostringstream m;
      m << "dsa_decode_plan: HIP device " << device << " not found ("
        << count << " visible)";
      return dsa::fail(DSA_DECODE_ERR_DEVICE, m.str());
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) {
      (void)hipGetLastError();
      return dsa::fail(DSA_DECODE_ERR_DEVICE,
                       "dsa_decode_plan: hipGetDeviceProperties failed");
    }
    // The kernels are gfx950 code objects; any other device is an error,
    // never a fallback to some other implementation.
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
      std::ostringstream m;
      m << "dsa_decode_plan: device " << device << " is " << prop.gcnArchName
        << "; this library is built for gfx950 only";
      return dsa::fail(DSA_DECODE_ERR_DEVICE, m.str());
    }
    num_cus = prop.multiProcessorCount;
  } else if (device != -1) {
    return dsa::fail(DSA_DECODE_ERR_INVALID,
                     "dsa_decode_plan: device must be >= 0, or -1 for a host-only plan");
  }

  dsa_decode_plan_s* plan = new (std::nothrow) dsa_decode_plan_s();
  if (!plan) return dsa::fail(DSA_DECODE_ERR_INVALID, "dsa_decode_plan: out of host memory");
  plan->p = norm;
  plan->device = device;
  plan->num_cus = num_cus;
  dsa::plan_layout(plan);
  *out = plan;
  dsa::set_error("");
  return DSA_DECODE_OK;
}

size_t dsa_decode_workspace_bytes(dsa_decode_plan_t plan) {
  return plan ? plan->ws.total : 0;
}

int dsa_decode_plan_get_info(dsa_decode_plan_t plan, dsa_decode_plan_info* info) {
  if (!plan || !info)
    return dsa::fail(DSA_DECODE_ERR_INVALID, "dsa_decode_plan_get_info: NULL argument");
  info->device = plan->device;
  info->chunk_tokens = plan->chunk_tokens;
  info->chunks_per_row = plan->chunks;
  info->head_blocks = plan->head_blocks;
  info->workgroups = plan->workgroups;
  info->merges_chunks = plan->chunks > 1 ? (plan->merge_in_kernel ? 2 : 1) : 0;
  info->num_cus = plan->num_cus;
  info->chunk_lead = plan->chunk_lead;
  info->layout = plan->layout;
  info->heads_per_block = plan->heads_per_block;
  info->rows_per_sequence = plan->p.rows_per_sequence > 1 ? plan->p.rows_per_sequence : 1;
  info->workspace_bytes = plan->ws.total;
  info->flags = plan->p.flags;
  info->qk_rope_dim = plan->p.qk_rope_dim;
  info->status_offset = plan->ws.status;
  info->counters_offset = plan->ws.arrivals;
  return DSA_DECODE_OK;
}

}  // extern "C"
