/*
 * pa.h -- C ABI of libpa.so: paged attention over a quantized, block-table
 * indexed KV cache, MXFP4 paged MQA logits, and the paged KV insert, for
 * AMD Instinct MI355X (gfx950).
 *
 * Conventions shared by every entry point
 *  - Pointers inside the argument structs, `workspace` and the buffers of
 *    pa_dequantize are DEVICE memory owned by the caller. The structs
 *    themselves are host memory and are only read during the call.
 *  - `stream` is a hipStream_t (NULL = the default stream). Every call only
 *    enqueues work on it: no allocation, no free, no host synchronisation,
 *    no read of device data by the host. Calls may be captured into a HIP
 *    graph.
 *  - Errors are returned as pa_status; nothing is enqueued when a call
 *    returns an error. pa_last_error() gives a message for the calling
 *    thread's last non-OK status.
 *  - Host-side checks (shapes, kinds, sizes) always run. Conditions that
 *    depend on device data (context lengths within [0, max_context_len],
 *    block ids of visible pages within [0, num_blocks) and, for attention,
 *    not the null block 0) are the caller's preconditions, as on the
 *    fp4_paged_mqa_logits API page (block_table / max_context_len
 *    parameters): violating them is undefined behaviour -- unless the
 *    environment variable PA_VALIDATE is set (to anything but "" or "0"):
 *    then paged_attn_fwd, paged_attn_fwd_noalloc, paged_attn_sparse and
 *    paged_mqa_logits first run a device check that reads only
 *    context_lens and the in-range table columns of visible pages, wait for
 *    it on the stream, and return PA_ERR_PRECONDITION (nothing else
 *    enqueued) naming the first violating sequence. The check is skipped
 *    while the stream is being captured into a graph, as the API page's
 *    validation is (max_context_len parameter). Its flags use 8 bytes of the
 *    workspace.
 *
 * Sources (titles of the pages these operations come from):
 *  [NULLPAD] "Stop grouped-page4 null-block padding from leaking E4M3 NaN"
 *  [FOLD]    "Normalize the PER_CHANNEL K scale folded into Q for paged XQA"
 *  [RELOC]   "Stabilize QSA page4 order under KV relocation"
 *  [INSERT]  "DeepSeek-V4.1 Q pad + fused KV insert" (the KV-only insert path)
 *  [FP4API]  "flashinfer.fp4_paged_mqa_logits" API documentation
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1,  /* a null pointer, a negative or inconsistent size */
  PA_ERR_UNSUPPORTED = 2,  /* valid, but a shape/kind the library has no kernel for */
  PA_ERR_PRECONDITION = 3, /* a documented precondition checked on the host failed */
  PA_ERR_WORKSPACE = 4,    /* workspace missing or smaller than *_workspace_size() */
  PA_ERR_HIP = 5           /* a HIP launch failed */
} pa_status;

typedef enum { PA_DT_F16 = 0, PA_DT_BF16 = 1, PA_DT_F32 = 2 } pa_dtype;

/* KV cache element kinds. E4M3 is OCP FP8 E4M3FN (bytes 0x7F/0xFF are NaN,
 * largest finite 448) [NULLPAD, Root cause]. INT8 is two's complement. INT4
 * packs two signed nibbles per byte, element 2j in the low nibble [FOLD,
 * Description: INT4 scale max|K|/7, INT8 max|K|/127]. */
typedef enum {
  PA_KV_F16 = 0,
  PA_KV_BF16 = 1,
  PA_KV_E4M3 = 2,
  PA_KV_INT8 = 3,
  PA_KV_INT4 = 4
} pa_kv_kind;

/* Scale of a cache plane: none (codes are values), one fp32 for the whole
 * tensor, or one fp32 per channel with shape [num_kv_heads, head_dim]
 * [FOLD, Cost: "1024 floats at H256"]. A dequantized value is
 * fp32(code) * scale. */
typedef enum {
  PA_SCALE_NONE = 0,
  PA_SCALE_PER_TENSOR = 1,
  PA_SCALE_PER_CHANNEL = 2
} pa_scale_mode;

/* ------------------------------------------------------------------------ */
/* paged_attn_fwd                                                            */
/* ------------------------------------------------------------------------ */

/*
 * out[b, i, h, :] = softmax(softmax_scale * q[b,i,h,:] . K_t) V_t over the
 * tokens t visible to query row i of sequence b, with K_t, V_t read through
 * block_table and dequantized. Decode is next_n = 1; multi-row verify /
 * short prefill is next_n > 1, where row i sits at position
 * context_lens[b] - next_n + i and, with `causal`, sees tokens t <= that
 * position.
 *
 * Layouts (all row-major, device memory):
 *   q, out       [batch, next_n, num_q_heads, head_dim], both of q_dtype: fp16
 *                (PA_DT_F16) or bf16 (PA_DT_BF16; q is widened to fp32 on load
 *                and converted to fp16 for the matrix cores -- exact for bf16
 *                values in fp16's normal range, |q| <= 65504 required -- and
 *                out is rounded to bf16 to nearest even)
 *   k_cache,
 *   v_cache      [num_blocks, block_size, num_kv_heads, row_bytes], row_bytes =
 *                head_dim * 2 (F16/BF16), head_dim (E4M3/INT8), head_dim / 2 (INT4)
 *   k_scale,
 *   v_scale      NULL (PA_SCALE_NONE), [1] or [num_kv_heads, head_dim] fp32
 *   block_table  [batch, max_blocks_per_seq] int32, physical block ids in
 *                logical order [FP4API, block_table parameter]
 *   context_lens [batch] int32, each in [0, max_context_len]
 * Query head h reads KV head h / (num_q_heads / num_kv_heads).
 *
 * Guarantees:
 *  - Only blocks holding visible tokens are read. Block 0 serves as the null
 *    block for table padding and is never read through padding entries;
 *    tail slots past a sequence's length are neutralised by select, so NaN
 *    bytes there cannot reach the output [NULLPAD, Fix].
 *  - A PER_CHANNEL K scale is folded into q as q * (k_scale / max|k_scale|)
 *    and max|k_scale| is applied to the scores once [FOLD, Approach]; no
 *    fp16 overflow can turn into inf * 0.
 *  - The reduction over tokens runs in logical token order and its split
 *    points depend only on shapes, so the output is bit-identical under any
 *    physical relocation of pages [RELOC, Summary].
 *  - A row with no visible token outputs +0.
 *
 * softmax_scale: 0 selects 1/sqrt(head_dim); otherwise it must be > 0.
 * Supported: head_dim 64/128/256 (INT4: 128/256), block_size 16/32,
 * next_n <= 4096 and next_n * num_q_heads / num_kv_heads <= 8192 query rows
 * per KV head (beyond 32 rows -- long verify, chunked prefill -- the rows are
 * processed in blocks of 32, each block walking only the tokens its last row
 * can see; the workspace grows with the number of blocks), q_dtype F16 or
 * BF16; KV kinds F16, BF16, E4M3, INT8, INT4. A BF16 cache is read through
 * fp16 for the matrix cores: exact for magnitudes in [2^-14, 65504], finite
 * magnitudes above become 65504, smaller ones keep fp16's subnormal
 * precision. Workspace: paged_attn_workspace_size(a) bytes, 256-byte aligned.
 */
typedef struct pa_attn_args {
  void* out;
  const void* q;
  pa_dtype q_dtype;
  const void* k_cache;
  const void* v_cache;
  pa_kv_kind kv_kind;
  const float* k_scale;
  pa_scale_mode k_scale_mode;
  const float* v_scale;
  pa_scale_mode v_scale_mode;
  const int32_t* block_table;
  const int32_t* context_lens;
  int32_t max_context_len;
  int32_t batch;
  int32_t next_n;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t max_blocks_per_seq;
  int64_t num_blocks;
  float softmax_scale;
  int32_t causal;
} pa_attn_args;

size_t paged_attn_workspace_size(const pa_attn_args* a);
pa_status paged_attn_fwd(const pa_attn_args* a, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * paged_attn_fwd_noalloc -- paged_attn_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments, kernels and result, with the
 * workspace taken from a scratch array the library holds in device memory
 * (paged_attn_noalloc_scratch_bytes() bytes per GPU, 32 MiB, kept until the
 * process ends) instead of a caller's buffer. Nothing is allocated or freed
 * by the call. Calls needing more workspace than the array holds (see
 * paged_attn_workspace_size) return PA_ERR_WORKSPACE and enqueue nothing.
 * The array is shared by every call on that GPU and keeps the last call's
 * contents (the kernels write every byte they read, so nothing needs
 * clearing); calls that overlap in time on one GPU -- on different streams
 * or from different threads -- race on it. The first call on a device
 * resolves the array's device address (hipGetSymbolAddress, no allocation).
 */
pa_status paged_attn_fwd_noalloc(const pa_attn_args* a, void* stream);
size_t paged_attn_noalloc_scratch_bytes(void);

/*
 * Test probe of the plan [RELOC, Summary: reduce in logical order, split
 * points that do not follow physical ids]: dumps what paged_attn_fwd's
 * attention kernel walks for these arguments. The work is a list of items --
 * (sequence, query row block, KV head group, block of `ts` logical tokens) in
 * that order -- placed on a cost line and cut into one contiguous range per
 * workgroup of the persistent grid; the probe runs the kernel's own range
 * computation in every workgroup and writes, for every item at its global
 * index g, items[g * 6 + {0..5}] = {workgroup, sequence, row block, head
 * group, first logical token, physical block of the item's first page}. It
 * also writes seq_first[b] (b < batch) = the first cost slot of sequence b
 * and seq_first[batch] = the slot total (what the merge kernel reads), and
 * *total = the number of items. Pages past a sequence's length are never
 * items, so the null block 0 never appears for a valid table.
 * `info` is HOST memory (int32[8], may be NULL when items is not) and
 * receives {workgroups, item capacity needed, ts, KV heads per item, run-start
 * cost in slots, row blocks, rows per block, head groups}; call with items =
 * NULL to get info only. items, seq_first and total are DEVICE memory; items
 * needs max_items >= the capacity, and entries past *total are not written.
 */
pa_status pa_plan(const pa_attn_args* a, int32_t* items, int64_t max_items, int32_t* seq_first,
                  int32_t* total, int32_t* info, void* stream);

/*
 * paged_attn_sparse -- selection-driven sparse paged attention, the QSA route
 * of [RELOC] (Summary and Fix: a physical-page union with per-row token masks,
 * walked in logical page order) with the unattended-row rule of [NULLPAD]
 * (Fix: rows that select nothing are written as zeros).
 *
 * sel: DEVICE int32 [batch, next_n, topk] logical token ids per query row
 *   (row i of sequence b attends to the distinct ids t of sel[b, i, :] with
 *   0 <= t < context_lens[b]; other ids, and repeats, add nothing). May be
 *   NULL when topk == 0.
 * The attention itself is the one of paged_attn_fwd restricted to each row's
 * selected set: scores are scale * q.k over the selected tokens only (no
 * causal rule: `causal` is ignored), softmax over them, and the values are
 * summed in ascending token order, so the output is bit-identical under any
 * physical relocation of pages. A row with an empty set outputs +0 and reads
 * no KV byte; KV bytes of unselected tokens are never part of a result (NaN
 * there cannot leak).
 * Supported: every KV kind and scale mode of paged_attn_fwd (a PER_CHANNEL K
 * scale is folded into q the same way), q_dtype F16 or BF16, next_n <= 4,
 * next_n * (num_q_heads / num_kv_heads) <= 32, max_blocks_per_seq <= 16384,
 * plus the shapes paged_attn_fwd supports.
 * Workspace: paged_attn_sparse_workspace_size(a, topk) bytes (0 when the
 * arguments are rejected); it holds the per-call union plan and split
 * partials, and its prior contents do not matter. Three kernels are enqueued
 * on `stream`: planner, attention, merge.
 */
size_t paged_attn_sparse_workspace_size(const pa_attn_args* a, int32_t topk);
pa_status paged_attn_sparse(const pa_attn_args* a, const int32_t* sel, int32_t topk,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Test probe of the sparse union planner: for each sequence b writes
 * count[b] = number of distinct logical pages that hold a selected token,
 * entries[(b * cap + e) * 2 + {0, 1}] = {block_table[b, page], page} for
 * e < count[b] in ascending page order, and
 * masks[(b * cap + e) * next_n + i] = bit (t % block_size) set for every
 * token t of page e that row i selected (all cap * next_n mask words of each
 * sequence are written; entries past count[b] are not). Pages beyond cap are
 * dropped from entries and masks but counted only up to cap. Buffers are
 * DEVICE memory; cap >= 1.
 */
pa_status pa_sparse_plan(const pa_attn_args* a, const int32_t* sel, int32_t topk,
                         int32_t* entries, uint32_t* masks, int32_t* count, int32_t cap,
                         void* stream);

/* ------------------------------------------------------------------------ */
/* paged_mqa_logits [FP4API]                                                 */
/* ------------------------------------------------------------------------ */

/* Element type of the logits output [FP4API, output_dtype] and of its
 * epilogue [FP4API, epi_dtype]. Zero is fp32, so a zero-initialised struct
 * keeps the fp32 contract. */
typedef enum { PA_LOGITS_F32 = 0, PA_LOGITS_F16 = 1, PA_LOGITS_BF16 = 2 } pa_logits_format;

/*
 * out[b*next_n + i, t] = sum over heads h (ascending, fp32 fma chain) of
 *   weights[b*next_n + i, h] * A(q[b,i,h,:] . k_t) with both operands MXFP4
 *   (E2M1 values, one UE8M0 scale per sf_vec_size elements), for
 *   t < context_lens[b]; -inf for context_lens[b] <= t < max_context_len.
 *   A is the identity, or with relu != 0 the rectifier max(., +0) (a variant
 *   the API page does not name). With epi_format fp16 / bf16 the head chain
 *   runs in that type [FP4API, epi_dtype; the page leaves the arithmetic
 *   open, the reading taken here]: the weight and A(S_h) are rounded to it
 *   (nearest even), each step is the fp32 fma of those and the running value,
 *   and the step's result is rounded to it again. The value is stored as
 *   out_format: fp32, or fp16 / bf16 rounded to nearest even (-inf stays
 *   -inf).
 * Rows >= batch*next_n and columns >= max_context_len are not written.
 *
 * Layouts:
 *   out       [>= batch*next_n, out_row_stride] of out_format, out_row_stride >=
 *             max_context_len
 *   q         [batch, next_n, num_heads, head_dim/2] uint8, element 2j in the low nibble
 *   sf_q      [batch, next_n, num_heads] int32, byte g scales elements [32g, 32g+32)
 *   kv_fused  [num_blocks, block_size, 1, head_dim/2 + head_dim/sf_vec_size] uint8; each
 *             block holds [block_size * head_dim/2 FP4 bytes][block_size * head_dim/32 SF
 *             bytes]. The SF tail is in token order, or with sf_interleaved != 0 in the
 *             interleaved order [FP4API, is_kv_sf_interleaved]: 4-byte slot k holds the
 *             scales of token (k % 4) * (block_size / 4) + k / 4.
 *   weights   [batch*next_n, num_heads] fp32
 *   block_table [batch, max_blocks_per_seq] int32 with max_blocks_per_seq >=
 *             round_up(max_context_len, 128) / block_size (checked on the host)
 * Supported: head_dim 128, sf_vec_size 32, block_size 64, num_heads 16, 32 or
 * 64, next_n 1..4, epi_format fp32 / fp16 / bf16. There is no schedule
 * argument: the grid follows max_context_len and each workgroup reads
 * context_lens itself, so nothing can go stale [FP4API, schedule_meta].
 * Workspace: paged_mqa_logits_workspace_size(a) bytes, used only for the
 * PA_VALIDATE flags; without PA_VALIDATE NULL, 0 is accepted.
 */
typedef struct pa_logits_args {
  void* out;
  int64_t out_row_stride;
  const uint8_t* q;
  const int32_t* sf_q;
  const uint8_t* kv_fused;
  const float* weights;
  const int32_t* context_lens;
  const int32_t* block_table;
  int32_t batch;
  int32_t next_n;
  int32_t num_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t max_blocks_per_seq;
  int64_t num_blocks;
  int32_t max_context_len;
  int32_t sf_vec_size;
  pa_logits_format out_format;
  pa_logits_format epi_format;
  int32_t sf_interleaved;
  int32_t relu;
} pa_logits_args;

size_t paged_mqa_logits_workspace_size(const pa_logits_args* a);
pa_status paged_mqa_logits(const pa_logits_args* a, void* workspace, size_t workspace_bytes,
                           void* stream);

/* ------------------------------------------------------------------------ */
/* pa_topk_select [RELOC] [FP4API]                                           */
/* ------------------------------------------------------------------------ */

/*
 * The top-k over indexer logits that gives each query row its token set
 * [RELOC, Investigation: the selected token ids of a query row; Upstream
 * check: top-k], joining paged_mqa_logits to paged_attn_sparse: for row
 * r = b * next_n + i, sel[r, :] holds the ids of the k largest logits[r, t]
 * over t < context_lens[b], in ascending id order, followed by -1 for the
 * positions left when context_lens[b] < k. Equal logits (+0 and -0 alike) go
 * to the lower token id, and NaN ranks below every number (the pages give no
 * tie rule; this is the reading taken). The result is exact: index work,
 * bit-identical to the oracle.
 *
 * Layouts: logits [>= batch * next_n, logits_row_stride] of logits_format
 *          (fp32 / fp16 / bf16: the output formats of paged_mqa_logits);
 *          context_lens [batch] int32, each in [0, logits_row_stride];
 *          sel [batch * next_n, k] int32 (= [batch, next_n, k], the sel
 *          argument of paged_attn_sparse with topk = k).
 * One workgroup per row; no workspace.
 */
typedef struct pa_topk_args {
  int32_t* sel;
  const void* logits;
  pa_logits_format logits_format;
  int64_t logits_row_stride;
  const int32_t* context_lens;
  int32_t batch;
  int32_t next_n;
  int32_t k;
} pa_topk_args;

pa_status pa_topk_select(const pa_topk_args* a, void* stream);

/* ------------------------------------------------------------------------ */
/* kv_insert_mxfp4 [FP4API] [INSERT]                                         */
/* ------------------------------------------------------------------------ */

/*
 * For each row i < num_tokens with i < num_slots and slot_mapping[i] >= 0, the
 * 128 values k[i, :] are quantized to MXFP4 and written to token position
 * slot % block_size of block slot / block_size of kv_fused (the layout of
 * paged_mqa_logits: [block_size * 64 FP4 bytes][block_size * 4 scale bytes]).
 * Rows without a slot are skipped and their destination left untouched
 * [INSERT, Design: the KV-only mode skips rows that have no slot]; so are rows
 * whose slot lies past num_blocks * block_size.
 *
 * Quantizer (the pages print none; the OCP Microscaling rule): per group of 32
 * values with largest magnitude amax, the UE8M0 scale byte is
 * floor(log2(amax)) - 2 + 127 clamped to [0, 254] (0 for an all-zero group),
 * and each value divided by 2^(byte - 127) is rounded to the nearest E2M1
 * value, ties to the even code, saturating at +-6; the sign bit is the
 * input's. Element 2j is the low nibble. The token's 4 scale bytes go to slot
 * pos in token order, or with sf_interleaved != 0 to the slot k with
 * (k % 4) * (block_size / 4) + k / 4 == pos [FP4API, is_kv_sf_interleaved].
 *
 * Layouts: k [num_tokens, 128] fp16 or bf16 (in_dtype); slot_mapping
 * [num_slots] int64; kv_fused [num_blocks, block_size, 1, 68] uint8.
 * Inputs must be finite. Supported: head_dim 128, sf_vec_size 32, block_size a
 * multiple of 4. Errors: status codes, nothing enqueued.
 */
typedef struct pa_mxfp4_insert_args {
  uint8_t* kv_fused;
  const void* k;
  pa_dtype in_dtype;
  const int64_t* slot_mapping;
  int64_t num_tokens;
  int64_t num_slots;
  int32_t head_dim;
  int32_t block_size;
  int64_t num_blocks;
  int32_t sf_vec_size;
  int32_t sf_interleaved;
} pa_mxfp4_insert_args;

pa_status kv_insert_mxfp4(const pa_mxfp4_insert_args* a, void* stream);

/* ------------------------------------------------------------------------ */
/* kv_insert [INSERT]                                                        */
/* ------------------------------------------------------------------------ */

/*
 * For each token row i < num_tokens with i < num_slots and slot_mapping[i] >= 0:
 * k_cache[slot / block_size, slot % block_size, hk, :] = Q(k[i, hk, :] / k_scale)
 * and likewise for v. Rows without a slot (i >= num_slots, or slot < 0) are
 * skipped and their destination bytes are left untouched [INSERT, Design: the
 * KV-only mode skips DP-padding rows that have no slot].
 * Rows whose slot lies at or past num_blocks * block_size are skipped too.
 * Q: E4M3 round-to-nearest-even saturating to +-448; INT8 / INT4 round to
 * nearest even clamped to +-127 / +-7; x / scale is an IEEE fp32 division of
 * the input value (fp16, or bf16 widened exactly to fp32).
 * F16 / BF16 caches take input of their own type, bits unchanged (scale mode
 * NONE).
 *
 * Layouts: k, v [num_tokens, num_kv_heads, head_dim] fp16 or bf16 (in_dtype);
 * slot_mapping [num_slots] int64; caches and scales as for paged_attn_fwd.
 */
typedef struct pa_insert_args {
  void* k_cache;
  void* v_cache;
  pa_kv_kind kv_kind;
  const void* k;
  const void* v;
  pa_dtype in_dtype;
  const int64_t* slot_mapping;
  int64_t num_tokens;
  int64_t num_slots;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int64_t num_blocks;
  const float* k_scale;
  pa_scale_mode k_scale_mode;
  const float* v_scale;
  pa_scale_mode v_scale_mode;
} pa_insert_args;

pa_status kv_insert(const pa_insert_args* a, void* stream);

/* ------------------------------------------------------------------------ */
/* probes and errors                                                         */
/* ------------------------------------------------------------------------ */

/*
 * Test probe of the cache codecs used by paged_attn_fwd: out[i] =
 * fp32(code_i) * scale, scale = scale[0] (PER_TENSOR), scale[i % channels]
 * (PER_CHANNEL) or 1 (NONE). `n` counts elements (INT4: two per byte). A BF16
 * code's value is the fp16 the attention kernels read it as (see
 * paged_attn_fwd).
 */
pa_status pa_dequantize(pa_kv_kind kind, const void* codes, int64_t n, const float* scale,
                        pa_scale_mode mode, int64_t channels, float* out, void* stream);

/*
 * Benchmark probe: reads `bytes` (a multiple of 16) of device memory at `src`
 * with 16-byte loads from `grid` workgroups of 256 threads, eight loads in
 * flight per thread, and writes one word per workgroup to sink[0 .. grid) so
 * the reads are live. Timing it gives the device's streaming-read rate.
 */
pa_status pa_read_probe(const void* src, int64_t bytes, uint32_t* sink, int32_t grid,
                        void* stream);

/* Message for the calling thread's last non-OK status ("" if none). */
const char* pa_last_error(void);

/*
 * Profiling hook for benchmarks: while set, every later paged_attn_fwd /
 * paged_attn_sparse / paged_mqa_logits / pa_topk_select / kv_insert_mxfp4 call
 * on the calling thread launches its dominant kernel (the attention ring or
 * prefill kernel, the logits kernel, the top-k kernel, the insert kernel)
 * with start_event and stop_event attached to that kernel's dispatch
 * (hipExtLaunchKernelGGL), so
 * the pair measures the kernel alone. Both are hipEvent_t handles owned by the
 * caller; pass NULL, NULL to clear. Returns PA_ERR_INVALID_ARG if exactly one
 * is NULL.
 */
pa_status pa_set_profile_events(void* start_event, void* stop_event);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
