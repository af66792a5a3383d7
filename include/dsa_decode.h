/*
 * dsa_decode.h — C ABI of the MI355X (gfx950) selected-index NoPE MLA paged
 * decode.
 *
 * What it computes, per query row r and local head h (pages cited by title):
 *   [attend]   page "spark_model/layers/glm5next_dsa/attend.rs"
 *   [decode_k] page "metrale_model_arch/glm5next_dsa/layer/decode_k.rs"
 *   [build]    page "spark_model/layers/glm5next_dsa/build.rs"
 *
 *   S_r   = the SET of ids t in sel_indices[r, :] with 0 <= t < seq_lens[r]
 *           ([attend] module doc, "Why this is not the masked kernel": the
 *           gather is exactly dense attention under a set-membership mask;
 *           -1 is a hole and repeats collapse). Negative ids are holes; ids
 *           at or past seq_lens[r] are dropped.
 *   row_t = the kv_lora_rank FP8 E4M3FN bytes of token t, found through the
 *           block table ([decode_k] slot computation: page =
 *           block_tables[r*stride + t/block_size], byte offset =
 *           page*cache_stride_bytes + (t % block_size)*kv_lora_rank).
 *   s_t   = sm_scale * k_scale * sum_d q[r,h,d] * fp8(row_t[d])
 *   out[r,h,:] = v_scale * sum_t softmax(s)_t * fp8(vrow_t[:])   (0 if S_r is empty)
 *           where vrow_t is read from v_cache at row_t's offset ([attend]
 *           DsaDecodeInputs: K and V are one latent buffer in absorbed NoPE
 *           MLA; both pointers are taken). The output stays in the latent
 *           space ([build] o_absorb consumes [heads, kv_lora_rank]).
 *
 * Every function returns DSA_DECODE_OK (0) or a negative status; the reason,
 * with the offending values, is then available from dsa_decode_last_error()
 * (thread-local). Nothing falls back to another code path: an unsupported
 * shape or device is an error ([attend] Glm5NextDsaDecodeKernel::resolve).
 */
#ifndef DSA_DECODE_H
#define DSA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_DECODE_OK 0
#define DSA_DECODE_ERR_INVALID (-1)     /* bad geometry, pointer or size */
#define DSA_DECODE_ERR_UNSUPPORTED (-2) /* kv_lora_rank not compiled in */
#define DSA_DECODE_ERR_DEVICE (-3)      /* no device, or it is not gfx950 */
#define DSA_DECODE_ERR_WORKSPACE (-4)   /* workspace null, misaligned or small */
#define DSA_DECODE_ERR_LAUNCH (-5)      /* the HIP runtime refused a launch */

/* Geometry of one decode. All counts are elements unless named _bytes. */
typedef struct dsa_decode_params {
  /* Query rows. One row per decoded sequence; q, out, seq_lens and the
   * selection all have this many rows ([attend] decode_attention refuses a
   * selection whose row count differs from the sequence count). */
  int32_t num_rows;
  /* Local query heads (this tensor-parallel rank's heads). > 0. */
  int32_t num_q_heads;
  /* Latent KV heads. Must be 1: MLA keeps a single latent head
   * ([attend] DsaDecodePaging::validate). */
  int32_t num_kv_heads;
  /* D, the latent width and the FP8 bytes per cached token. Supported:
   * 64, 128, 256, 512. Anything else is DSA_DECODE_ERR_UNSUPPORTED, never
   * a silent mis-tiling ([attend] decode_attention's kv_lora_rank guard). */
  int32_t kv_lora_rank;
  /* Tokens per cache page. > 0. */
  int32_t block_size;
  /* The selector's pool width. > 0, and block_size % index_kpool == 0 so a
   * pool never straddles two pages ([attend] DsaDecodePaging::validate). */
  int32_t index_kpool;
  /* W: ids per selection row. > 0. */
  int32_t sel_width;
  /* Entries between consecutive rows of block_tables; 0 = every row reads
   * row 0's table ([decode_k] the attend's block-table row stride). */
  int32_t block_table_stride;
  /* Bytes between consecutive pages of the cache; 0 selects
   * block_size * kv_lora_rank. Must be >= block_size * kv_lora_rank and a
   * multiple of kv_lora_rank (latent rows are addressed by index). */
  uint64_t cache_stride_bytes;
  /* Upper bound on every seq_lens[r]; > 0. When block_table_stride > 0 it
   * must not exceed block_table_stride * block_size (a table row must cover
   * every position it can be asked for: [decode_k] block-table capacity
   * check). Ids are clamped to it, so a larger seq_lens[r] cannot make the
   * library read past a table row. */
  int32_t max_seq_len;
  /* Softmax scale applied to q . k (explicit; [attend] passes
   * kv_lora_rank^-0.5, the GLM-5.3 configurations use qk_head_dim^-0.5). */
  float sm_scale;
  /* 0: the planner picks how many selected tokens one workgroup handles.
   * Otherwise a positive multiple of 64 that forces that split (used to test
   * that the result does not depend on the split). */
  int32_t chunk_tokens;
  /* Heads per workgroup: DSA_DECODE_LAYOUT_AUTO (0) lets the planner choose
   * (16 when num_q_heads <= 16; 64 when num_rows * ceil(num_q_heads / 64)
   * workgroups already give every compute unit one and 64-head blocks are
   * allowed, see below; else 32); DSA_DECODE_LAYOUT_HEADS32 (1):
   * blocks of up to 32 heads, eight waves per workgroup (two scoring waves
   * of 32 tokens per 16-head group); DSA_DECODE_LAYOUT_HEADS16 (2): blocks
   * of up to 16 heads, also eight waves (four scoring waves of 16 tokens);
   * DSA_DECODE_LAYOUT_HEADS64 (3): blocks of up to 64 heads, eight waves
   * (one scoring wave of the whole tile per 16-head group), for
   * kv_lora_rank 512 without a rope tail or DSA_DECODE_FLAG_MERGE_IN_KERNEL
   * (otherwise DSA_DECODE_ERR_UNSUPPORTED).
   * The head blocks of a row read the same latent rows through the same L2.
   * The result does not depend on it. */
  int32_t layout;
  /* 0 or 1: rows are scheduled independently. k > 1: rows s*k .. s*k + k - 1
   * are the k consecutive query rows of one sequence in a k-token decode
   * step ([decode_k]: k rows per sequence at positions pos .. pos + k - 1,
   * each with its own selection and seq_len, all reading the sequence's
   * block-table row), so their selections overlap. The planner puts the
   * workgroups of those k rows on one XCD in the same dispatch round, so
   * the latent rows their selections share are fetched from HBM about once
   * and served to the others by that XCD's L2. num_rows must be a multiple
   * of k. The result does not depend on it. */
  int32_t rows_per_sequence;
  /* Bit set of DSA_DECODE_FLAG_* (0: none). */
  int32_t flags;
  /* Width of a rope tail carried by every cached token after its latent.
   * 0: NoPE, the latent is the whole token ([attend] module doc, "NoPE, and
   * why no common/ kernel would do"). 64: the DeepSeek-V4-style token that
   * the same passage and decode_attention's scale comment describe: each
   * token is kv_lora_rank (must be 512) latent bytes followed by 64 bytes of
   * an already rotated rope tail, 576 FP8 E4M3FN bytes in all; q carries
   * 576 values per head, the scores run over all 576 (token t's own tail
   * against q's tail, never the next token's bytes), the values and the
   * output are the first 512. Nothing is rotated here. Any other value is
   * DSA_DECODE_ERR_UNSUPPORTED. */
  int32_t qk_rope_dim;
  int32_t reserved[2]; /* must be zero */
} dsa_decode_params;

#define DSA_DECODE_LAYOUT_AUTO 0
#define DSA_DECODE_LAYOUT_HEADS32 1
#define DSA_DECODE_LAYOUT_HEADS16 2
#define DSA_DECODE_LAYOUT_HEADS64 3

/* flags: every launch also writes the normalised selection (ids, counts and
 * byte offsets) into the workspace, for dsa_decode_read_selection. Off by
 * default: the decode itself never needs it, and it costs 12 bytes of
 * workspace and of HBM writes per selection slot. */
#define DSA_DECODE_FLAG_EXPORT_SELECTION 1
/* flags: split rows (chunks_per_row > 1) are merged inside the decode kernel
 * by the last chunk of each (row, head block) to finish, which waits for the
 * others' partials, instead of by a separate combine kernel over every CU
 * (the default). The result is the same either way. */
#define DSA_DECODE_FLAG_MERGE_IN_KERNEL 2

/* Opaque plan: validated geometry plus the launch decomposition. Host
 * memory owned by the library; free it with dsa_decode_plan_destroy. */
typedef struct dsa_decode_plan_s* dsa_decode_plan_t;

/* Read-only description of a plan. */
typedef struct dsa_decode_plan_info {
  int32_t device;          /* HIP device id, or -1 for a host-only plan */
  int32_t chunk_tokens;    /* selected tokens per workgroup */
  int32_t chunks_per_row;  /* workgroups per row per head block */
  int32_t head_blocks;     /* groups of up to heads_per_block heads */
  int32_t workgroups;      /* launched: rows * chunks_per_row rounded up to
                            * a multiple of 8 (of 8 * rows_per_sequence when
                            * rows are co-scheduled), times head_blocks */
  int32_t merges_chunks;   /* 0: rows are not split; 1: split rows are merged
                            * by a separate combine kernel (a second launch on
                            * the same stream); 2: by the last chunk of a row
                            * to finish, inside the decode kernel
                            * (DSA_DECODE_FLAG_MERGE_IN_KERNEL) */
  int32_t num_cus;         /* compute units the plan was sized for */
  int32_t chunk_lead;      /* extra selected tokens of chunk 0 when split rows
                            * are merged in the kernel (it then finishes last
                            * and merges); the last chunk has that many fewer */
  uint64_t workspace_bytes;
  int32_t layout;          /* DSA_DECODE_LAYOUT_HEADS32, _HEADS16 or _HEADS64 (resolved) */
  int32_t heads_per_block; /* 32 or 16 */
  int32_t rows_per_sequence; /* rows co-scheduled on one XCD (1: none) */
  int32_t flags;           /* params.flags */
  int32_t qk_rope_dim;     /* params.qk_rope_dim */
  /* Byte offsets inside the workspace, for diagnostics and tests:
   *   status_offset    int32, 0 while healthy; set to 1 by a launch whose
   *                    split merge gave up waiting (see dsa_decode_launch)
   *   counters_offset  int32 [2][num_rows * head_blocks]: chunks arrived,
   *                    then partials published, per (row, head block);
   *                    zero between launches */
  uint64_t status_offset;
  uint64_t counters_offset;
} dsa_decode_plan_info;

/* Validate params and build a plan.
 *   params  host pointer, read only, not retained.
 *   device  HIP device the plan launches on; the device must be gfx950.
 *           Pass -1 for a host-only plan (validation and sizing without a
 *           GPU); such a plan cannot be launched.
 *   out     receives the plan on success, NULL on failure.
 * Errors: DSA_DECODE_ERR_INVALID for any geometry rule above,
 * DSA_DECODE_ERR_UNSUPPORTED for kv_lora_rank, DSA_DECODE_ERR_DEVICE when
 * the device is missing or not gfx950. */
int dsa_decode_plan(const dsa_decode_params* params, int device,
                    dsa_decode_plan_t* out);

/* Free a plan (NULL is ignored). */
void dsa_decode_plan_destroy(dsa_decode_plan_t plan);

/* Device scratch bytes dsa_decode_launch needs (a status word, per-row
 * arrival counters, split partials when chunks_per_row > 1, and with
 * DSA_DECODE_FLAG_EXPORT_SELECTION the selection ids, token byte offsets and
 * per-row counts). The caller allocates it; 0 for a NULL plan. */
size_t dsa_decode_workspace_bytes(dsa_decode_plan_t plan);

/* Zero a workspace for `plan` on `stream` (a fill kernel, no memset, so it
 * may be captured in a graph). Required once after the workspace is
 * allocated, and again before it is used with a different plan: the arrival
 * counters a launch relies on must start at zero. Every completed launch
 * leaves them at zero again, so back-to-back launches (and graph replays)
 * need no further initialisation. Zeroing the buffer any other way (e.g. a
 * zero-filled allocation) is equivalent.
 * Errors: DSA_DECODE_ERR_INVALID (NULL or host-only plan),
 * DSA_DECODE_ERR_DEVICE, DSA_DECODE_ERR_WORKSPACE, DSA_DECODE_ERR_LAUNCH. */
int dsa_decode_workspace_init(dsa_decode_plan_t plan, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Fill *info. DSA_DECODE_ERR_INVALID for a NULL argument. */
int dsa_decode_plan_get_info(dsa_decode_plan_t plan, dsa_decode_plan_info* info);

/* Enqueue the decode on `stream` (a hipStream_t; NULL = the default stream).
 * Asynchronous: nothing is synchronised, nothing is allocated, and nothing is
 * retained after return ([attend] decode_attention enqueues without
 * synchronising; DsaDecodeInputs are caller-owned).
 * Device pointers, all caller-owned:
 *   q            bf16  [num_rows, num_q_heads, kv_lora_rank], 16-byte aligned
 *   k_cache      FP8 E4M3FN pool; token rows as described above; 16-byte aligned
 *   v_cache      same layout as k_cache (may equal it); 16-byte aligned
 *   block_tables int32 [num_rows or 1, block_table_stride or as needed]
 *   seq_lens     int32 [num_rows]
 *   sel_indices  int32 [num_rows, sel_width]
 *   out          bf16  [num_rows, num_q_heads, kv_lora_rank], 16-byte aligned
 *   workspace    >= dsa_decode_workspace_bytes(plan) bytes, 256-byte aligned,
 *                zeroed once by dsa_decode_workspace_init for this plan;
 *                overwritten; must not be shared by launches in flight.
 * k_scale, v_scale: per-tensor dequantisation scales (finite).
 * Split rows (chunks_per_row > 1): the last chunk of a (row, head block) to
 * finish waits for the others' partials, which every other chunk publishes
 * after it has arrived, so the wait ends within microseconds. Should it not
 * end within about 0.1 s (a broken counter), that (row, head block) is
 * written as NaN and the workspace's status word is set: from then on every
 * output of every launch on this workspace is NaN, until
 * dsa_decode_workspace_init zeroes it again. The counters themselves return
 * to zero once the late chunks publish.
 * Device-side preconditions (not checked by the kernels): every page id a
 * selected token maps to lies inside the pool; the pool holds fewer than
 * 2^32 latent rows (page * cache_stride_bytes / kv_lora_rank + block_size
 * < 2^32, i.e. under 2 TiB at kv_lora_rank 512); with block_table_stride 0
 * the shared table has an entry for every position < max_seq_len.
 * Errors: DSA_DECODE_ERR_INVALID (NULL/misaligned pointer, host-only plan,
 * non-finite scale), DSA_DECODE_ERR_WORKSPACE, DSA_DECODE_ERR_LAUNCH. */
int dsa_decode_launch(dsa_decode_plan_t plan, const void* q,
                      const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* seq_lens,
                      const int32_t* sel_indices, float k_scale, float v_scale,
                      void* out, void* workspace, size_t workspace_bytes,
                      void* stream);

/* dsa_decode_launch without a caller workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. It allocates nothing (no hipMalloc, no
 * allocating library call): the workspace is a static device array of the
 * library, 32 MiB, one copy on every GPU the library runs on, held until the
 * process ends (its address is looked up once per device). Before the decode
 * it clears the status word and the arrival counters with a fill kernel on
 * `stream` (the array keeps whatever the last call on the GPU left in it);
 * the split partials need no clearing. Arguments, results and asynchrony as
 * for dsa_decode_launch. Calls that overlap on one GPU (other streams, other
 * threads, graphs replayed concurrently) share the array and race: serialise
 * them. Errors as for dsa_decode_launch, plus DSA_DECODE_ERR_WORKSPACE when
 * the plan's workspace (dsa_decode_workspace_bytes) exceeds 32 MiB, and
 * DSA_DECODE_ERR_INVALID for a plan with DSA_DECODE_FLAG_EXPORT_SELECTION
 * (the export is read back from a caller workspace). */
int dsa_decode_launch_static(dsa_decode_plan_t plan, const void* q,
                             const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, const int32_t* seq_lens,
                             const int32_t* sel_indices, float k_scale,
                             float v_scale, void* out, void* stream);

/* Copy the normalised selection the last launch on `workspace` computed
 * (what the attention consumed) into caller device memory, on `stream`.
 * Only for plans made with DSA_DECODE_FLAG_EXPORT_SELECTION (otherwise
 * DSA_DECODE_ERR_INVALID):
 *   ids      int32  [num_rows, sel_width]: row r's distinct valid ids in
 *            ascending order in its first counts[r] entries; the rest is
 *            unspecified
 *   counts   int32  [num_rows]
 *   offsets  uint64 [num_rows, sel_width]: byte offset of each id's latent
 *            row in the pool, same order as ids
 * Any of the three may be NULL. Asynchronous. */
int dsa_decode_read_selection(dsa_decode_plan_t plan, const void* workspace,
                              size_t workspace_bytes, int32_t* ids,
                              int32_t* counts, uint64_t* offsets, void* stream);

/* Kernel timing for benchmarks. dsa_decode_timing_begin makes the next
 * max_launches launches of this plan record HIP events around the decode
 * kernel on the launch stream (events are created here, not in the launch).
 * dsa_decode_timing_end waits for the recorded events and returns in
 * *kernel_ms the milliseconds spent in the decode kernel, summed over the
 * recorded launches, and their number in *launches; it then stops
 * recording. */
int dsa_decode_timing_begin(dsa_decode_plan_t plan, int32_t max_launches);
int dsa_decode_timing_end(dsa_decode_plan_t plan, float* kernel_ms,
                          int32_t* launches);

/* The cache writer ([decode_k] latent_write launch, which passes one kv_a
 * row, the kv_a_layernorm weight, the pool, the token's slot, rms_eps and
 * 1/kv_scale). For each row i < num_rows with slots[i] >= 0:
 *   y_d = x_d / sqrt(mean_d(x_d^2) + rms_eps) * w_d * inv_kv_scale
 * computed in fp32, rounded to FP8 E4M3FN (nearest, ties to even, saturating
 * at +-448, never NaN) and stored at byte
 *   (slot / block_size) * cache_stride_bytes + (slot mod block_size) * D
 * of k_pool (the decode's addressing of a token row; the slot of a position
 * is physical page * block_size + position mod block_size). A negative slot
 * writes nothing. Device pointers, caller-owned:
 *   kv_a     bf16  [num_rows, kv_lora_rank], 16-byte aligned
 *   weight   bf16  [kv_lora_rank], 16-byte aligned
 *   slots    int64 [num_rows]
 *   k_pool   FP8 E4M3FN pool, 16-byte aligned
 * cache_stride_bytes 0 means block_size * kv_lora_rank; otherwise at least
 * that and a multiple of 16. rms_eps >= 0 and inv_kv_scale > 0, finite.
 * Enqueued on `stream` (NULL = default); nothing is allocated or retained.
 * num_rows == 0 is a no-op. Device-side precondition (not checked): every
 * slot's row lies inside the pool. Errors: DSA_DECODE_ERR_INVALID,
 * DSA_DECODE_ERR_UNSUPPORTED (kv_lora_rank), DSA_DECODE_ERR_LAUNCH. */
int dsa_decode_latent_write(const void* kv_a, const void* weight,
                            const int64_t* slots, int32_t num_rows,
                            int32_t kv_lora_rank, int32_t block_size,
                            uint64_t cache_stride_bytes, float rms_eps,
                            float inv_kv_scale, void* k_pool, void* stream);

/* Dense masked-attention reference of the decode, for cross-checking it on
 * the GPU at full size ([attend] module doc, "Why this is not the masked
 * kernel": the selected-index decode equals attention over every position
 * t < seq_lens[r] with a mask keeping exactly the selected positions).
 * Plain fp32, one workgroup per (row, head), untuned and separate from the
 * decode kernel. For each row r and head h:
 *   S = { t in [0, L) : t appears in sel_indices[r, :] },
 *       L = min(max(seq_lens[r], 0), max_seq_len)
 *   s_t = sm_scale * k_scale * sum_d q[r,h,d] * fp8(k row of t)[d]
 *   out[r,h,d] = v_scale * sum_t exp(s_t - max s) * fp8(v row of t)[d]
 *                / sum_t exp(s_t - max s),      t in S ascending
 * and out[r,h,:] = 0 when S is empty. Geometry, buffers and addressing are
 * those of dsa_decode_launch (params as for dsa_decode_plan; q bf16
 * [R, H, D], pools FP8 E4M3FN, block_tables, seq_lens, sel_indices int32),
 * except that out is float32 [R, H, D]. Runs on the current HIP device,
 * which must be gfx950, enqueued on `stream` (NULL = default); allocates
 * and retains nothing. Errors: DSA_DECODE_ERR_INVALID (params, a NULL
 * buffer, non-finite scales, or 4 * ceil(max_seq_len / 32) + 8 * sel_width
 * bytes of LDS above 159 KiB), DSA_DECODE_ERR_UNSUPPORTED, _DEVICE, _LAUNCH.
 * Device-side preconditions as for dsa_decode_launch. */
int dsa_decode_masked_reference(const dsa_decode_params* params, const void* q,
                         const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* seq_lens,
                         const int32_t* sel_indices, float k_scale, float v_scale,
                         float* out, void* stream);

/* Thread-local message of the last failure on this thread ("" if none). */
const char* dsa_decode_last_error(void);

/* ABI version of this header (major * 100 + minor). */
int dsa_decode_version(void);

#define DSA_DECODE_VERSION 400

#ifdef __cplusplus
}
#endif

#endif /* DSA_DECODE_H */
