/*
 * libpagedattn — attention over a paged KV cache for a mixed varlen batch,
 * written for AMD Instinct MI355X (gfx950, CDNA4).
 *
 * What is computed.  For every query token row r of sequence b, head h:
 *   out[r, h, :] = sum_t softmax_t(scale * q[r, h, :] . K_b[t, h / g, :]) * V_b[t, h / g, :]
 *   lse[r, h]    = ln sum_t exp(scale * q[r, h, :] . K_b[t, h / g, :])
 * over the visible keys t of that row, where K_b/V_b are gathered through the
 * block table (see pa_gather_kv).  Query i of a sequence with q_b query tokens
 * and seq_len L_b sits at position c_b + i, c_b = L_b - q_b, and with causal
 * masking sees keys 0 .. c_b + i (a decode, q_b = 1, sees all L_b keys).
 * Query head h reads KV head h / g, g = num_heads / num_kv_heads.
 *
 * Sources (cited by page title and section):
 *  - «FlashAttention y FlashInfer: los dos grandes backends de atención en
 *    GPU», §Responsabilidades: the forward takes Q as [num_tokens, num_heads,
 *    head_size], the paged KV cache and the metadata (query_start_loc,
 *    seq_lens, block table); the FlashInfer builder splits decodes from
 *    prefills and orders decodes first.  §Flujo de datos (get_kv_cache_shape
 *    listing): pool shape and the multiple-of-16 block size.
 *  - «El especialista del plato estrella: el backend de atención de vLLM»,
 *    §Por qué prefill y decode son problemas opuestos (decode is HBM-bound,
 *    prefill is compute-bound), §El truco del scheduler (both in one forward),
 *    §Cómo lee el backend el KV paginado (gather through the block table),
 *    §Qué aporta FlashInfer (cascade attention for a shared prefix).
 *  - «AttentionBackend: capa de abstracción de backends de atención»,
 *    §Flujo de datos (build(common_prefix_len, common_attn_metadata) and
 *    forward(..., kv_cache, attn_metadata, output) signatures), §Motivación de
 *    diseño and §Límites y fallos (LSE output, natural-log base, head-size and
 *    dtype limits).
 *
 * Conventions for every call:
 *  - Every function returns a pa_status and never aborts.  On error nothing is
 *    launched, outputs are untouched, and pa_last_error() (per calling thread)
 *    holds a message.
 *  - "host" pointers are ordinary CPU memory read during the call only.
 *    "device" pointers are GPU memory on the plan's device, owned by the caller.
 *  - Calls that launch work are asynchronous on the given HIP stream (NULL = the
 *    default stream); they neither allocate nor synchronise.
 *  - Element types: PA_BF16 (bfloat16, stored as 16-bit patterns) or PA_FP32.
 *    q and out share one element type; lse is always float32.  kv_cache has
 *    the same element type, or holds 8-bit e4m3 codes with K and V scales
 *    (pa_params.kv_dtype = PA_KV_FP8_E4M3, bf16 queries; see pa_forward_fp8).
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1, /* malformed sizes, metadata or pointers */
  PA_ERR_UNSUPPORTED = 2, /* well-formed but not built: head_size, dtype */
  PA_ERR_HIP = 3,         /* a HIP runtime call or kernel launch failed */
  PA_ERR_OOM = 4          /* host or device allocation failed */
} pa_status;

typedef enum pa_dtype { PA_BF16 = 0, PA_FP32 = 1 } pa_dtype;

/*
 * Element type of the paged pool.  PA_KV_FP8_E4M3: one byte per element, an
 * OCP 8-bit float with 4 exponent bits (bias 7) and 3 mantissa bits (largest
 * finite value 448, NaN only at 0x7F and 0xFF, no infinities); a K entry stands
 * for decode(code) * k_scale and a V entry for decode(code) * v_scale, with one
 * scale per tensor or one per KV head.  «FlashAttention y FlashInfer»,
 * §Motivación de diseño and §Límites y fallos: an fp8 (e4m3) KV cache with
 * per-head quantisation scales; the pages give no formula, this is the reading.
 */
typedef enum pa_kv_dtype { PA_KV_SAME = 0, PA_KV_FP8_E4M3 = 1 } pa_kv_dtype;

/*
 * Memory order of the pool («FlashAttention y FlashInfer», §Motivación de
 * diseño: two layouts NHD / HND chosen by get_kv_cache_stride_order).  The
 * logical shape is always (num_blocks, 2, bs, Hkv, d) (pa_kv_cache_shape).
 * PA_KV_NHD stores it in that order: the KV heads of one slot are adjacent.
 * PA_KV_HND stores (num_blocks, 2, Hkv, bs, d): one KV head's slots of a block
 * are adjacent (for one head, a block's bs rows of d elements are contiguous).
 */
typedef enum pa_kv_layout { PA_KV_NHD = 0, PA_KV_HND = 1 } pa_kv_layout;

/* Sizes of one batch.  All fields are read by pa_plan_create only. */
typedef struct pa_params {
  int32_t num_seqs;           /* B >= 0 */
  int32_t num_heads;          /* H >= 1, a multiple of num_kv_heads */
  int32_t num_kv_heads;       /* Hkv >= 1 */
  int32_t head_size;          /* d: 64 or 128 are built; others -> PA_ERR_UNSUPPORTED */
  int32_t block_size;         /* bs: a multiple of 16 (else PA_ERR_INVALID_ARG) */
  int32_t num_blocks;         /* pages in the pool; every used block id must be below it */
  int32_t max_blocks_per_seq; /* row stride of block_table */
  int32_t dtype;              /* pa_dtype */
  int32_t causal;             /* 1: key t visible to query i iff t <= c_b + i; 0: all L_b keys */
  int32_t common_prefix_len;  /* P: 0 = no cascade; else shared prefix tokens (see below) */
  int32_t kv_split_tokens;    /* 0 = automatic; else decode KV chunk per work item, multiple of 32
                                 (automatic: balanced work lists over the keys past the shared
                                 prefix, see pa_plan_info.num_decode_lists; beside prefills they
                                 take a share of the resident waves and the prefill the rest) */
  float scale;                /* softmax scale applied to q . k (positive, finite) */
  int32_t kv_dtype;           /* pa_kv_dtype: 0 = the pool has element type dtype; PA_KV_FP8_E4M3
                                 needs dtype PA_BF16 (else PA_ERR_UNSUPPORTED) */
  int32_t kv_layout;          /* pa_kv_layout: 0 = NHD, 1 = HND; block sizes up to 1024 and beyond
                                 (any multiple of 16) work with either */
  int32_t check_metadata;     /* 1: every forward first runs pa_plan_check_metadata on its device
                                 arrays (a debugging mode: it waits for the stream and cannot be
                                 captured into a graph); 0: the device arrays are trusted */
} pa_params;

/* Opaque, immutable schedule for one batch; reusable across layers and calls. */
typedef struct pa_plan pa_plan;

typedef struct pa_plan_info {
  int32_t num_seqs;
  int32_t num_tokens;           /* T = query_start_loc[B] */
  int32_t num_decodes;          /* sequences with exactly one query token */
  int32_t num_decode_tokens;
  int32_t num_prefills;         /* sequences with two or more query tokens */
  int32_t num_prefill_tokens;
  int32_t common_prefix_len;    /* P actually used (0 = cascade off) */
  int32_t num_prefix_blocks;    /* P / block_size */
  int32_t num_decode_items;     /* decode work items per KV head */
  int32_t num_prefill_items;    /* prefill work items per KV head and head group */
  int32_t num_prefix_items;     /* cascade prefix work items per KV head and head group */
  int32_t num_merge_rows;       /* token rows combined from several partial results */
  int32_t num_partials;         /* partial (out, lse) records in the workspace */
  int32_t kv_split_tokens;      /* decode KV chunk used (largest decode work item, keys) */
  int32_t prefill_rows_per_item; /* query positions per prefill work item */
  int32_t prefill_head_groups;  /* prefill work items per KV head and position block */
  int32_t num_decode_lists;     /* decode work lists: each is run by one group of waves (one
                                   wave per KV head) in order; one item per list unless balanced */
  int32_t decode_list_tokens;   /* balanced lists: the budget W of each list, in keys, where each of
                                   its items also counts decode_item_keys (every list but the last
                                   comes within 32 + decode_item_keys of its budget; see
                                   decode_list_xcd_budgets); else 0 */
  int64_t kv_tokens_read;       /* K/V token rows the schedule reads, summed over KV heads */
  int64_t prefix_tokens_read;   /* of which rows of the shared prefix (the prefix pass covers the
                                   decode rows; prefill rows read their whole context in their own
                                   items) */
  int64_t decode_tokens_read;   /* of which by decode work items */
  int64_t prefill_tokens_read;  /* of which by prefill work items */
  int64_t prefix_tokens_unique; /* distinct (KV head, prefix token) rows the prefix pass reads: P * Hkv
                                   (prefix_tokens_read counts each column group's read; groups of
                                   one KV head and chunk run together on one XCD and share its L2) */
  int32_t prefix_beside_decode; /* 1: the shared-prefix pass runs beside the decode on CUs of its
                                   own (one prefix workgroup per CU; the decode lists cover the
                                   others); 0: before it, or no prefix */
  int32_t decode_item_keys;     /* balanced lists: what one work item's start costs, in keys */
  int32_t decode_list_xcd_budgets; /* 1: list i's budget is W - W/128 for even i, W + W/128 for odd i
                                   (decodes alone, one workgroup per list, a 256-CU device: workgroups
                                   are dealt to the eight XCDs in turn, and lists on even XCDs run
                                   slower); 0: W for all */
} pa_plan_info;

/* Arrays a plan exposes through pa_plan_get_array. */
typedef enum pa_plan_array {
  PA_ARRAY_ORDER = 0,         /* int32[B]: decode-first stable order of sequence ids */
  PA_ARRAY_IS_DECODE = 1,     /* int32[B]: 1 if the sequence is a decode */
  PA_ARRAY_PREFIX_BLOCKS = 2, /* int32[P/bs]: the shared prefix's physical block ids */
  PA_ARRAY_ROW_PARTIALS = 3,  /* int32[T]: partial records combined for each row (0 = direct write) */
  PA_ARRAY_DECODE_LISTS = 4,  /* int32[num_decode_lists + 1]: first decode item of each list */
  PA_ARRAY_DECODE_SPANS = 5   /* int32[3 * num_decode_items]: (sequence, first key, end key) of each
                                 decode item, in schedule order */
} pa_plan_array;

/* Per-kernel timing gathered by pa_profile_start/stop. */
typedef struct pa_kernel_time {
  char name[48];     /* kernel family, e.g. "decode_bf16_d128" */
  int32_t launches;  /* launches recorded */
  double total_ms;   /* summed device time between HIP events around each launch */
  double min_ms;     /* shortest launch */
  double median_ms;  /* median launch (mean of the two middle ones for an even count) */
  double max_ms;     /* longest launch */
} pa_kernel_time;

/*
 * Shape of the paged pool: (num_blocks, 2, block_size, num_kv_heads, head_size),
 * dim 1 = 0 for K and 1 for V.  «FlashAttention y FlashInfer», §Flujo de datos
 * (get_kv_cache_shape listing).  shape_out: host int64[5].
 * Errors: block_size not a positive multiple of 16, or any size < 1 -> INVALID_ARG.
 */
pa_status pa_kv_cache_shape(int64_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                            int32_t head_size, int64_t shape_out[5]);

/*
 * Memory order of the pool's logical dimensions (blocks, K/V, slot, KV head,
 * head size), outermost first, for a pa_kv_layout: NHD -> {0, 1, 2, 3, 4},
 * HND -> {0, 1, 3, 2, 4} («FlashAttention y FlashInfer», §Motivación de
 * diseño, get_kv_cache_stride_order).  order_out: host int32[5].
 * Errors: INVALID_ARG (unknown layout, NULL order_out).
 */
pa_status pa_kv_cache_stride_order(int32_t layout, int32_t order_out[5]);

/*
 * Build the schedule for one batch (the metadata builder).  «AttentionBackend:
 * capa de abstracción», §Flujo de datos: build(common_prefix_len,
 * common_attn_metadata); «FlashAttention y FlashInfer», §Responsabilidades:
 * split decodes from prefills, order decodes first, schedule ahead of time.
 *
 *  params          host; sizes above.
 *  query_start_loc host int32[B+1]: 0 = qsl[0] < qsl[1] < ... (every q_b >= 1).
 *  seq_lens        host int32[B]: L_b >= q_b; ceil(L_b / bs) <= max_blocks_per_seq.
 *  block_table     host int32[B * max_blocks_per_seq] or NULL.  When given, every
 *                  used id (the first ceil(L_b / bs) of each row) is checked to be
 *                  in [0, num_blocks).  Required when common_prefix_len > 0.
 *  device          HIP device that will run the plan; < 0 builds a host-only plan
 *                  (metadata queries only, pa_forward rejects it).
 *  plan_out        receives the plan; release it with pa_plan_destroy.
 *
 * Cascade («El especialista del plato estrella», §Qué aporta FlashInfer): with
 * P = common_prefix_len > 0 the first P / bs block ids must be identical in every
 * row, P must be a multiple of bs, and P <= c_b for every sequence (the prefix
 * is context of all of them).  Violations -> INVALID_ARG.  The decode rows
 * attend to the prefix in one shared pass, merged with their own suffix by
 * LSE; prefill rows attend to their whole context (the result is the same
 * attention).
 * The plan copies its work lists and the metadata (for pa_plan_check_metadata)
 * to device memory it owns.
 * Errors: INVALID_ARG (any rule above, H % Hkv != 0, NULL pointers),
 * UNSUPPORTED (head_size, dtype), HIP / OOM (device copy).
 */
pa_status pa_plan_create(const pa_params* params, const int32_t* query_start_loc,
                         const int32_t* seq_lens, const int32_t* block_table, int device,
                         pa_plan** plan_out);

/* Counts and schedule figures of a plan.  info: host. */
pa_status pa_plan_get_info(const pa_plan* plan, pa_plan_info* info);

/*
 * Copy one of the plan's int32 arrays (pa_plan_array) into host memory dst of
 * `capacity` elements; *count (host, may be NULL) receives its length.
 * Errors: unknown array or capacity too small -> INVALID_ARG.
 */
pa_status pa_plan_get_array(const pa_plan* plan, int32_t which, int32_t* dst, int64_t capacity,
                            int64_t* count);

/* Bytes of device workspace pa_forward needs for this plan (0 is possible). */
size_t pa_plan_workspace_bytes(const pa_plan* plan);

/*
 * Compare device metadata with the host arrays the plan was built from
 * («AttentionBackend: capa de abstracción», §Flujo de datos: the forward takes
 * the metadata the builder produced; here the builder's copy drives the
 * schedule, so the caller's device arrays must describe the same batch).
 *  block_table     device int32[B * max_blocks_per_seq] or NULL (not compared).
 *                  The used ids (the first ceil(L_b / bs) of row b) must equal the
 *                  host table given to pa_plan_create; a plan made without one
 *                  checks that they lie in [0, num_blocks).
 *  query_start_loc device int32[B + 1] or NULL; must equal the plan's, entry for entry.
 *  seq_lens        device int32[B] or NULL; likewise.
 * Runs one small kernel on `stream` and waits for it (not capturable).  The
 * plan holds one result word: checks on one plan from several host threads
 * take turns (a lock held from the launch to the read of the result).
 * Errors: INVALID_ARG (host-only plan, misaligned arrays, any difference: the
 * message gives the count), HIP.
 */
pa_status pa_plan_check_metadata(const pa_plan* plan, const int32_t* block_table,
                                 const int32_t* query_start_loc, const int32_t* seq_lens, void* stream);

/*
 * Run attention for the planned batch.  «AttentionBackend: capa de abstracción»,
 * §Archivos clave: forward(layer, query, key, value, kv_cache, attn_metadata,
 * output); the new tokens' K/V are already in the pool (the cache write is a
 * separate step, «FlashAttention y FlashInfer», §Responsabilidades).
 *
 *  q           device [T, H, d], element type of the plan, 16-byte aligned.
 *  kv_cache    device [num_blocks, 2, bs, Hkv, d], same element type, 16-byte aligned.
 *  block_table device int32[B * max_blocks_per_seq]; the used ids must equal the
 *              host table given to (or implied by) the plan.
 *  query_start_loc, seq_lens  device int32[B + 1] and int32[B], or NULL: the
 *              batch's metadata (the attn_metadata of the pages' forward).  The
 *              schedule comes from the plan's own copy, so the kernels do not
 *              read them; with params.check_metadata = 1 they, and block_table,
 *              are compared with the plan's first (pa_plan_check_metadata).
 *  out         device [T, H, d], same element type, 16-byte aligned; fully written.
 *  lse         device float32[T, H] natural-log LSE, or NULL to skip it.
 *  workspace   device scratch of at least pa_plan_workspace_bytes(plan) bytes,
 *              16-byte aligned (NULL allowed when that is 0); contents need no
 *              initialisation.
 *  stream      hipStream_t (NULL = default stream).
 * Row order of out/lse is the caller's token order; the decode-first order only
 * affects the schedule.  The call is asynchronous and stream-ordered on
 * `stream`: when the plan holds both decode work and prefill work, the prefill
 * (and a shared-prefix pass, if any) runs on a side stream owned by the plan,
 * which first waits for `stream` and which `stream` waits for before the final
 * merge (event record/wait only, so the call can be captured into a graph);
 * otherwise every launch is on `stream`.  Host threads may share a plan: each
 * call needs its own workspace, calls on such a plan enqueue one at a time (a
 * lock held while they record the fork/join events), and their side-stream work
 * runs in the order they were made.
 * Errors: INVALID_ARG (host-only plan, NULL or misaligned pointers, small
 * workspace, metadata differing from the plan's when checked, a plan whose pool
 * holds e4m3 codes: those run through pa_forward_fp8), HIP (launch failure).
 * On error nothing is launched (a metadata check may have run).
 */
pa_status pa_forward(const pa_plan* plan, const void* q, const void* kv_cache,
                     const int32_t* block_table, const int32_t* query_start_loc,
                     const int32_t* seq_lens, void* out, float* lse, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * pa_forward for callers that cannot allocate device memory (code under graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * kernels, with the partial-result workspace in a static device array of
 * 64 MiB that the library holds on each device it runs on (until the process
 * ends) instead of caller memory.  The call itself allocates nothing; its first
 * call for a device looks the array's address up.
 *  Arguments as pa_forward, without workspace; the plan's pool holds q's
 *  element type (an e4m3 plan -> INVALID_ARG, as for pa_forward).
 * Every call on one device shares that device's array: calls that overlap in
 * time on one GPU (other streams, other threads) race on it and must be
 * serialised by the caller.  Nothing in the array needs clearing: every
 * partial record a forward reads is written earlier in the same forward.
 * Errors: as pa_forward; INVALID_ARG when pa_plan_workspace_bytes(plan)
 * exceeds 64 MiB (use pa_forward with a workspace); HIP.
 */
pa_status pa_forward_noalloc(const pa_plan* plan, const void* q, const void* kv_cache,
                             const int32_t* block_table, const int32_t* query_start_loc,
                             const int32_t* seq_lens, void* out, float* lse, void* stream);

/*
 * pa_forward over a pool of e4m3 codes (plan made with kv_dtype =
 * PA_KV_FP8_E4M3): the keys and values are decode(code) * k_scale and
 * decode(code) * v_scale («FlashAttention y FlashInfer», §Motivación de diseño
 * and §Límites y fallos: fp8 KV cache, per-head quantisation scales).
 *  q, out      device bf16 [T, H, d].
 *  kv_cache    device uint8 [num_blocks, 2, bs, Hkv, d], 16-byte aligned.
 *  k_scale, v_scale  device float32[num_scales]; num_scales is 1 (one scale for
 *              the tensor) or Hkv (one per KV head); read by the kernels, so
 *              they may change between calls without a new plan.  Positive and
 *              finite (not checked on the device).
 * Everything else as pa_forward.  Errors: INVALID_ARG (as pa_forward, a plan
 * without an e4m3 pool, NULL or misaligned scales, num_scales not 1 or Hkv,
 * misaligned pool), HIP.
 */
pa_status pa_forward_fp8(const pa_plan* plan, const void* q, const void* kv_cache,
                         const int32_t* block_table, const int32_t* query_start_loc,
                         const int32_t* seq_lens, const float* k_scale, const float* v_scale,
                         int32_t num_scales, void* out, float* lse, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * Combine two partial attentions over disjoint key sets by their LSE.
 * «AttentionBackend: capa de abstracción», §Motivación de diseño and §Límites y
 * fallos (partial softmax results combine through a natural-log LSE):
 *   lse = ln(e^lse_a + e^lse_b),  o = e^(lse_a - lse) o_a + e^(lse_b - lse) o_b.
 * A part with lse = -inf contributes nothing; both -inf gives o = 0, lse = -inf.
 *  o_a, o_b, o_out device [num_tokens, num_heads, head_size] of `dtype`,
 *                  aligned to 4 elements (8 bytes bf16, 16 bytes float32);
 *  lse_a, lse_b, lse_out device float32[num_tokens, num_heads] (lse_out may be NULL).
 * Errors: INVALID_ARG (sizes < 0, NULL or misaligned pointers), UNSUPPORTED
 * (dtype, head_size).
 */
pa_status pa_merge_states(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                          void* o_out, float* lse_out, int32_t num_tokens, int32_t num_heads,
                          int32_t head_size, int32_t dtype, void* stream);

/*
 * Write the new tokens' K and V rows into their pages: the cache update that
 * comes before attention and is an operation of its own, outside pa_forward
 * («FlashAttention y FlashInfer», §Responsabilidades).  Query token i of
 * sequence b is key position c_b + i, which lives in block
 * block_table[b][(c_b + i) / bs] at offset (c_b + i) % bs; its slot number is
 * block * bs + offset.
 *  key, value    device [num_tokens, num_kv_heads, head_size] of params->dtype,
 *                16-byte aligned.
 *  slot_mapping  device int64[num_tokens]; a negative slot skips the token, and
 *                so does a slot at or past num_blocks * block_size.
 *  kv_cache      device pool (num_blocks, 2, bs, Hkv, d) of params->dtype in the
 *                memory order params->kv_layout, 16-byte aligned, written in
 *                place; slots not named keep their contents.
 * Uses params->num_kv_heads, head_size, block_size, num_blocks, dtype and
 * kv_layout.  Two tokens with the same slot race.  Asynchronous on `stream`,
 * copies bit for bit.  Errors: INVALID_ARG (sizes, NULL or misaligned
 * pointers, unknown layout, an e4m3 pool: see pa_write_kv_fp8), UNSUPPORTED
 * (dtype, a head row that is not a whole number of 16-byte chunks), HIP.
 */
pa_status pa_write_kv(const void* key, const void* value, const int64_t* slot_mapping, int32_t num_tokens,
                      const pa_params* params, void* kv_cache, void* stream);

/*
 * pa_write_kv into a pool of e4m3 codes (params->kv_dtype = PA_KV_FP8_E4M3):
 * element x of a K row of KV head h is stored as the code nearest to the
 * float32 quotient x / k_scale[h] (ties to the even code, saturating at +-448;
 * NaN is stored as 0x7F), V likewise with v_scale.  The pages name the fp8
 * cache and its scales but not the rounding; this is the reading.
 *  key, value    device bf16 [num_tokens, num_kv_heads, head_size], 16-byte aligned.
 *  k_scale, v_scale  device float32[num_scales], num_scales 1 or num_kv_heads.
 *  kv_cache      device uint8 pool, 16-byte aligned, written in place.
 * Slots as in pa_write_kv.  Errors: INVALID_ARG (as pa_write_kv, a pool that
 * is not e4m3, NULL scales, num_scales), UNSUPPORTED (dtype other than bf16,
 * head_size not a multiple of 16), HIP.
 */
pa_status pa_write_kv_fp8(const void* key, const void* value, const int64_t* slot_mapping, int32_t num_tokens,
                          const pa_params* params, const float* k_scale, const float* v_scale,
                          int32_t num_scales, void* kv_cache, void* stream);

/*
 * Copy one sequence's K and V out of the pool, contiguous, bit for bit.
 * «El especialista del plato estrella», §Cómo lee el backend el KV paginado:
 * token t is slot t % bs of block block_table_row[t / bs].
 *  kv_cache        device pool of params->dtype (e4m3 codes when params->kv_dtype
 *                  is PA_KV_FP8_E4M3) in the memory order params->kv_layout,
 *                  16-byte aligned.
 *  block_table_row device int32[ceil(seq_len / bs)].
 *  k_out, v_out    device [seq_len, Hkv, d] each, the pool's element type,
 *                  16-byte aligned.
 * Uses params->block_size, num_kv_heads, head_size, dtype, kv_dtype, kv_layout.  The ids are not
 * checked on the device: they must be in [0, num_blocks).
 * Errors: INVALID_ARG (sizes, NULL or misaligned pointers), UNSUPPORTED (dtype).
 */
pa_status pa_gather_kv(const void* kv_cache, const int32_t* block_table_row, int32_t seq_len,
                       const pa_params* params, void* k_out, void* v_out, void* stream);

/* Release a plan (NULL is ignored).  Not while a forward using it is in flight. */
void pa_plan_destroy(pa_plan* plan);

/* Static text for a status code. */
const char* pa_status_string(pa_status status);

/* Message of the calling thread's last error ("" if none). */
const char* pa_last_error(void);

/*
 * Timing of the library's own launches on the calling thread.  After
 * pa_profile_start(max_launches), every launch made by this thread records a
 * HIP event before and after it, on the launch's stream, up to max_launches.
 * pa_profile_stop waits for the recorded events, sums device time per kernel
 * family into out (host, `capacity` entries; *count receives how many) with
 * the shortest, median and longest launch, and ends the session.  Errors: INVALID_ARG (no session / bad sizes), HIP.
 */
pa_status pa_profile_start(int32_t max_launches);
pa_status pa_profile_stop(pa_kernel_time* out, int32_t capacity, int32_t* count);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
