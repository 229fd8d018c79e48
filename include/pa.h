/*
 * pa.h - paged GQA attention over a block-table KV cache, for AMD MI355X (gfx950).
 *
 * C ABI of libpa.so. Every entry point takes plain pointers and sizes; no
 * framework types cross this boundary. Three operations make up the path:
 *
 *   pa_store_kv        write new K/V rows into the paged pool through slot_mapping
 *                      (optionally quantising them to FP8 e4m3 or INT8 with
 *                      per-token-per-head scales); pa_rope_store_kv first applies the
 *                      rotary position embedding to q and k;
 *   pa_decode          one query token per sequence attends its whole cached context,
 *                      read block by block through block_tables, with an online
 *                      softmax; long contexts are split and merged by log-sum-exp;
 *                      pa_decode_step stores the step's new rows and attends in one;
 *   pa_varlen_prefill  a flat batch of query chunks (cu_seqlens) attends, causally, the
 *                      cached prefix plus the chunk itself, per sequence;
 *   pa_bm_*            a host block manager (allocation, prefix sharing, copy-on-
 *                      write) that produces block_tables and slots for the above.
 *
 * Sources (web pages; cited below by tag and section):
 *   [P1] lvyufeng.github.io/PocketLLM .../phase3_3_completion_summary
 *        "Phase 3.3 completion summary - Slot ID Threading and Batch API Integration"
 *   [P2] lvyufeng.github.io/PocketLLM .../cpp_engine_batching_phase3_1
 *        "cpp_engine Batching Implementation (Phase 3.1)"
 *   [P4] koas-w.github.io/posts/20260331-errorsandsolutions
 *        (milestone log, "KV Cache management", "hand-written Triton kernels",
 *         "errors encountered", types 1-5)
 *   [P5] happydog-intj.github.io/mini-vllm-tutorial/step14_7_batched_forward
 *        "step14_7 - Batched Forward" ("varlen batch", "cu_seqlens is only needed in
 *         attention", "comparison with vLLM")
 *
 * Conventions shared by all calls
 * --------------------------------
 *  - Every array argument of a kernel call is a DEVICE pointer owned by the caller. The
 *    library never allocates, frees or caches device memory and keeps no global
 *    mutable state: all addressing is passed explicitly on every call, as [P1] "design
 *    decisions / explicit parameter passing" argues against a hidden current slot (the
 *    host block manager keeps its state in the handle the caller creates). The one
 *    exception is pa_decode_noalloc's scratch array, a fixed block of device memory in
 *    the library's code object (per GPU), for callers that cannot pass a workspace.
 *  - Calls are asynchronous on `stream` (a hipStream_t passed as void*, NULL = the
 *    default stream). They return after enqueueing and never synchronise.
 *  - Element strides are in ELEMENTS, not bytes; the innermost (head_dim) stride is
 *    always 1. Passing strides is how non-contiguous K/V views are handled, the fix
 *    [P4] "errors, type 2" reports for its store kernel.
 *  - The KV pool layout is [num_blocks, block_size, kv_heads, head_dim], dense, the
 *    per-slot layout of [P2] "current KV cache structure" ([max_seq_len, kv_heads,
 *    head_dim]) cut into block_size-token blocks ([P4] "KV Cache management":
 *    16-token blocks). Physical token slot of logical position j of sequence s:
 *        slot = block_tables[s][j / block_size] * block_size + j % block_size.
 *  - GQA: query head h reads KV head h / (q_heads / kv_heads) (contiguous groups).
 *  - Indices: block_tables, context_lens, cu_seqlens are int32; slot_mapping is int64.
 *    Kernels use 64-bit element offsets, so pools may exceed 2^31 elements.
 *  - context_lens[s] counts every token already stored for sequence s, INCLUDING the
 *    tokens of the current step, which must be stored before attention runs ([P4]
 *    "errors, type 1": a context length one short hides the new token from itself).
 *  - Supported: block_size 16; head_dim 64 or 128; q_heads / kv_heads in 1..8.
 *    dtypes: (q F32, pool F32), (q BF16, pool BF16), (q BF16, pool FP8_E4M3 or INT8).
 *  - Validation happens on the host before any launch; a failing call launches
 *    nothing and returns a negative status. Device-data preconditions (block ids in
 *    range, 1 <= context_lens[s] <= max_context_len, n_s <= context_lens[s]) are the
 *    caller's contract; the kernels skip out-of-range block ids and slots rather than
 *    touch memory outside the pool, and the affected outputs are then unspecified.
 *    The PA_DEBUG_CHECKS build reports such violations (pa_debug_take_violation).
 *  - Concurrent calls on different streams are safe when their outputs (and
 *    workspaces) are disjoint.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. */
enum {
  PA_F32 = 0,      /* IEEE binary32 */
  PA_BF16 = 1,     /* bfloat16 */
  PA_FP8_E4M3 = 2, /* OCP e4m3fn codes (bias 7, max 448, no infinities), KV pools only */
  PA_INT8 = 3      /* symmetric int8 codes in [-127, 127], KV pools only */
};

/* Status codes. */
enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, bad stride, bad dtype combo */
  PA_ERR_UNSUPPORTED = -2, /* valid but not built: head_dim, block_size, group size */
  PA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than *_workspace_bytes() */
  PA_ERR_HIP = -4,         /* one of this call's kernel launches failed (each launch's own
                              status; an error pending from the caller's earlier HIP
                              calls is neither reported nor cleared) */
  PA_ERR_DEVICE_DATA = -5  /* PA_DEBUG_CHECKS build only: an earlier call's device-side
                              metadata broke its contract (pa_debug_take_violation) */
};

/* One layer's KV pool. Caller-owned, dense, persists across calls (it is the cache).
 *   k, v       [num_blocks, block_size, kv_heads, head_dim] of `dtype`
 *   k_scale,   [num_blocks, block_size, kv_heads] fp32; required iff dtype is
 *   v_scale    PA_FP8_E4M3 or PA_INT8 (per-token-per-head dequantisation scales, the
 *              k_scale/v_scale "used for FP8/INT8 quantisation" of [P2]), else NULL. */
typedef struct pa_kv_pool {
  void *k;
  void *v;
  float *k_scale;
  float *v_scale;
  int64_t num_blocks;
  int32_t block_size;
  int32_t kv_heads;
  int32_t head_dim;
  int32_t dtype;
} pa_kv_pool_t;

/* Human-readable name of a status code (static string, never NULL). */
const char *pa_status_string(int status);

/*
 * Debug build (libpa_debug.so, compiled with PA_DEBUG_CHECKS). The device-side
 * preconditions of the calls below are the caller's contract, and the release kernels
 * only make sure a broken one cannot take them outside their buffers (out-of-range
 * block ids and slots are skipped, lengths clamped; the affected outputs are then
 * unspecified) - the wrong-slot and context-length bugs [P4] "errors encountered"
 * types 1, 2 and 5 describe would pass silently. In the debug build every kernel call
 * first launches a check of the metadata it is about to use, on the same stream; the
 * first violation is recorded in a per-GPU word, and the call then runs as in the
 * release build (nothing faults). Every later call waits for its stream, reads the
 * word and, while a violation is recorded, returns PA_ERR_DEVICE_DATA and launches
 * nothing; pa_debug_take_violation reads and clears it. Debug calls synchronise and
 * cannot be captured in a graph.
 * Violations (code, and what `where` holds):
 */
enum {
  PA_VIOLATION_CONTEXT_LEN = 1, /* context_lens[s] outside [1, max_context_len] (decode) or
                                   [0, max_context_len] (varlen); where = s */
  PA_VIOLATION_BLOCK_ID = 2,    /* block_tables[s][j] outside [0, num_blocks) for a block the
                                   context uses (j < ceil(L/16)); where = s << 28 | j */
  PA_VIOLATION_SLOT = 3,        /* slot_mapping[t] >= num_blocks * block_size; where = t */
  PA_VIOLATION_CHUNK = 4,       /* varlen chunk longer than its context: n_s > L_s; where = s */
  PA_VIOLATION_CU_SEQLENS = 5,  /* cu_seqlens not 0 .. total_tokens non-decreasing, or a
                                   chunk longer than max_q_len; where = s */
  PA_VIOLATION_STEP_SLOT = 6,   /* pa_decode_step: slot_mapping[s] >= 0 but not the slot of
                                   position context_lens[s] - 1; where = s */
  PA_VIOLATION_POSITION = 7,    /* pa_rope_store_kv: positions[t] outside [0, max_position);
                                   where = t */
  PA_VIOLATION_DUP_SLOT = 8     /* a slot named twice in one call's slot_mapping (store, RoPE
                                   store, decode step; its rows would race); where = t, one
                                   of the tokens naming it (whichever the parallel check
                                   found second). Checked for calls of up to 2^19 tokens. */
};
/* 1 in the PA_DEBUG_CHECKS build, 0 in the release build. */
int32_t pa_debug_checks(void);
/* Waits for `stream`, then returns (and clears) the current GPU's recorded violation:
 * *code = 0 when there is none. Never fails with PA_ERR_DEVICE_DATA itself. */
int pa_debug_take_violation(void *stream, int32_t *code, int64_t *where);

/*
 * pa_store_kv - scatter new K/V rows into the pool through slot_mapping.
 *
 * Defined by [P4] "hand-written Triton kernels" (store_kvcache_kernel: a token x head
 * grid writes each new K/V row directly to its physical cache slot, with strides for
 * non-contiguous inputs) and [P2] "Step 3.4" (append of `rows` new K/V rows at an
 * offset into a slot's contiguous cache, the special case slot = slot_id*max_len+pos).
 *
 *   k, v            new rows, [num_tokens, kv_heads, head_dim] of src_dtype with
 *                   element strides (k_stride_tok, k_stride_head) and
 *                   (v_stride_tok, v_stride_head); innermost stride 1.
 *   slot_mapping    [num_tokens] int64 physical slots. slot < 0 means "skip this token"
 *                   (padding). Slots >= num_blocks*block_size are skipped too.
 *                   Two tokens with the same slot in one call is a contract violation.
 *   For t with a valid slot and every head g < kv_heads:
 *     pool->dtype == src_dtype (F32 or BF16): the row is copied bit for bit to
 *         pool->k[slot / block_size][slot % block_size][g][:] (same for v).
 *     pool->dtype == PA_FP8_E4M3 (src_dtype F32 or BF16): per row x (fp32 values),
 *         a = max_d |x_d|; scale = a / 448 (fp32, correctly rounded);
 *         code_d = e4m3fn(x_d / scale) with round-to-nearest-even and saturation to
 *         +-448; a == 0 gives scale 0 and all codes 0x00. Codes go to the pool, the
 *         scale to pool->k_scale[slot / block_size][slot % block_size][g] (same for v).
 *     pool->dtype == PA_INT8 (src_dtype F32 or BF16): the same with 127 in place of 448
 *         and code_d = x_d / scale rounded to the nearest integer, ties to even,
 *         clamped to [-127, 127] (two's complement bytes).
 *         Source values must be finite.
 *   Every byte of the pool not named by a valid slot is left untouched.
 *   num_tokens == 0 is a no-op returning PA_OK.
 */
int pa_store_kv(const pa_kv_pool_t *pool, const void *k, const void *v, int32_t src_dtype,
                int64_t num_tokens, int64_t k_stride_tok, int64_t k_stride_head,
                int64_t v_stride_tok, int64_t v_stride_head, const int64_t *slot_mapping,
                void *stream);

/*
 * pa_rope_store_kv - rotary position embedding of a step's new q and k rows, fused with
 * the store of the rotated k rows and of the v rows into the pool.
 *
 * Defined by [P4] "hand-written Triton kernels" (the fused RoPE + KV-cache store: q is
 * rotated and written back to a contiguous buffer, k and v go straight to their slots
 * through slot_mapping, no intermediate buffer) with [P4]'s table-driven real-valued
 * RoPE, numerically aligned with the HuggingFace model (milestone log), whose rotation
 * pairs dim i with dim i + D/2 of a head.
 * For token t, position p = positions[t], and each head row x (D = head_dim values) of
 * q (q_heads rows) and of k (kv_heads rows), with c_i = cos_table[p][i] and
 * s_i = sin_table[p][i] for i < D/2:
 *     r_i       = x_i * c_i - x_{i+D/2} * s_i
 *     r_{i+D/2} = x_{i+D/2} * c_i + x_i * s_i
 * in fp32 from the exact fp32 values of x, every product and every sum rounded to fp32
 * on its own (no fused multiply-add).
 *   q, q_out     [num_tokens, q_heads, head_dim] of src_dtype with element strides;
 *                q_out receives r rounded once (nearest even) to src_dtype; it may be
 *                q itself (same pointer and strides).
 *   k, v         [num_tokens, kv_heads, head_dim] of src_dtype, strided as in
 *                pa_store_kv. The rotated k rows (fp32 values r) and the v rows are
 *                stored as pa_store_kv stores rows with those values: rounded to a
 *                bf16 / fp32 pool (src_dtype must then equal the pool dtype), quantised
 *                to an FP8 / INT8 pool (with their scales).
 *   positions    [num_tokens] int64, each in [0, max_position) (an out-of-range value
 *                leaves that token's rows unspecified; the tables are never read
 *                outside their bounds).
 *   cos_table,   fp32 [max_position, head_dim / 2], row-major: the cosine / sine of the
 *   sin_table    rotation angle of pair i at position p (caller-built, any values).
 *   slot_mapping [num_tokens] int64; < 0 (or past the pool) stores nothing for that
 *                token; q is rotated for every token.
 * num_tokens == 0 is a no-op. Errors as pa_store_kv, plus q_heads not a positive
 * multiple of kv_heads and max_position <= 0 (PA_ERR_INVALID_ARG).
 */
int pa_rope_store_kv(const pa_kv_pool_t *pool, const void *q, int64_t q_stride_tok,
                     int64_t q_stride_head, int32_t q_heads, void *q_out,
                     int64_t q_out_stride_tok, int64_t q_out_stride_head, const void *k,
                     const void *v, int32_t src_dtype, int64_t num_tokens,
                     int64_t k_stride_tok, int64_t k_stride_head, int64_t v_stride_tok,
                     int64_t v_stride_head, const int64_t *positions, const float *cos_table,
                     const float *sin_table, int32_t max_position,
                     const int64_t *slot_mapping, void *stream);

/*
 * pa_decode_workspace_bytes - bytes of device workspace pa_decode needs for these
 * sizes and this split length (0 when no context can need more than one split):
 * 4096 bytes of arrival counters, then num_seqs*q_heads*max_splits*(head_dim+1) fp32
 * partials, with max_splits = ceil(max_context_len / split). Returns 0 for invalid
 * arguments as well; pa_decode then reports the error.
 */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t q_heads, int32_t kv_heads,
                                 int32_t head_dim, int32_t max_context_len,
                                 int32_t split_tokens);

/* Split length (tokens) pa_decode uses for split_tokens == 0 with this call shape: the
 * power of two in [32, 1024] nearest above num_seqs*kv_heads*max_context_len/2048, so
 * that a worst-case batch has about 2048 (sequence, KV head, split) work items. Returns
 * 0 for non-positive arguments. */
int32_t pa_decode_default_split_tokens(int32_t num_seqs, int32_t kv_heads,
                                       int32_t max_context_len);

/*
 * pa_decode - paged decode attention, one query row per sequence.
 *
 * Defined by [P4] "hand-written Triton kernels" (Decode_Paged_GQAAttention_Kernel:
 * reads the scattered KV blocks in place through block_table, online softmax, GQA
 * head mapping inside the kernel) with [P4] "errors, type 1" fixing what
 * context_lens counts. For sequence s, query head h, g = h / (q_heads/kv_heads),
 * L = context_lens[s]:
 *     out[s][h][:] = sum_{j<L} softmax_j(scale * q[s][h] . K_s[j][g]) * V_s[j][g][:]
 * where K_s[j] is the pool row at slot(s, j). FP8 and INT8 pools dequantise as
 * code * scale.
 *
 *   out          [num_seqs, q_heads, head_dim] of q_dtype, strides (out_stride_tok,
 *                out_stride_head); every element is written exactly once.
 *   q            [num_seqs, q_heads, head_dim] of q_dtype, strides (q_stride_tok,
 *                q_stride_head) (a [B, 1, Hq, D] view works unchanged).
 *   block_tables [num_seqs, max_blocks_per_seq] int32, row-major. Entries past
 *                ceil(L / block_size) may be loaded but are never used to address
 *                the pool, so they may hold any value.
 *   context_lens [num_seqs] int32, each in [1, max_context_len].
 *   max_context_len  host-side upper bound of context_lens (sizes the grid).
 *   scale        softmax scale, finite and > 0 (e.g. 1/sqrt(head_dim)).
 *   split_tokens tokens per split-K work item: a positive multiple of block_size, at
 *                most 1024, or 0 for pa_decode_default_split_tokens(num_seqs,
 *                kv_heads, max_context_len). With a given split length the split of
 *                sequence s depends only on context_lens[s], so its output bits do
 *                not depend on the rest of the batch; pass an explicit value to keep
 *                that when batch shapes vary.
 *   workspace    16-byte aligned device scratch of at least pa_decode_workspace_bytes(...)
 *                bytes for the same (num_seqs, q_heads, kv_heads, head_dim,
 *                max_context_len, split_tokens); may be NULL when that is 0. It holds
 *                arrival counters in its first 4096 bytes, which MUST be zero before
 *                the first call (zero-fill the workspace once when allocating it), and
 *                the split partials (o, lse) after them, written before they are read.
 *                Every call leaves the counters zero and writes no partial into them,
 *                so a workspace can be reused by any later call whose size fits.
 *                Two calls in flight must not share a workspace.
 * Split partials are merged by log-sum-exp in two levels, both in index order: each
 * group of 8 consecutive splits, then the groups. Small calls (at most 1024
 * (sequence, group, KV head) triples) run as one launch in which the last group of a
 * sequence to finish merges the others; larger ones as a persistent split launch plus
 * a merge launch. Both give identical bits.
 * Accumulation is fp32; out is rounded once (round-to-nearest-even) to q_dtype.
 */
int pa_decode(void *out, int64_t out_stride_tok, int64_t out_stride_head, const void *q,
              int64_t q_stride_tok, int64_t q_stride_head, int32_t q_dtype, int32_t num_seqs,
              int32_t q_heads, const pa_kv_pool_t *pool, const int32_t *block_tables,
              int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t max_context_len,
              float scale, int32_t split_tokens, void *workspace, size_t workspace_bytes,
              void *stream);

/*
 * pa_decode_noalloc - pa_decode for callers that cannot allocate device memory (code
 * under graph capture that must not allocate, tight serving loops, harnesses that
 * forbid allocation): the same call without the workspace arguments.
 *
 * Its split partials and counters live in a scratch array of PA_NOALLOC_SCRATCH_BYTES
 * that the library holds in device memory on every GPU it runs on, until the process
 * ends (looked up, and its counters cleared by a small kernel on `stream`, on the first
 * call on each device). The call allocates and frees nothing. Results are bit-identical
 * to pa_decode with the same arguments and split length.
 * Returns PA_ERR_WORKSPACE, launching nothing, when pa_decode_workspace_bytes(...) for
 * this call exceeds PA_NOALLOC_SCRATCH_BYTES (use pa_decode with a workspace, or a
 * longer split_tokens, then); other errors as pa_decode.
 * Every call on one GPU shares that GPU's array: calls that can overlap on one GPU
 * (different streams, or a graph replay beside an eager call) race and must not be
 * made; calls on one stream are ordered and safe.
 */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int pa_decode_noalloc(void *out, int64_t out_stride_tok, int64_t out_stride_head,
                      const void *q, int64_t q_stride_tok, int64_t q_stride_head,
                      int32_t q_dtype, int32_t num_seqs, int32_t q_heads,
                      const pa_kv_pool_t *pool, const int32_t *block_tables,
                      int32_t max_blocks_per_seq, const int32_t *context_lens,
                      int32_t max_context_len, float scale, int32_t split_tokens,
                      void *stream);

/*
 * pa_decode_step - one decode step of a layer: store each sequence's new K/V row, then
 * attend, with the same result as pa_store_kv followed by pa_decode.
 *
 * Defined by [P4] "KV Cache management" / "CUDA Graph" (a decode step writes the new
 * token's K/V to its slot through slot_mapping, then the paged decode kernel attends
 * the context including it; "errors, type 1": the context counts the new token).
 * Arguments are those of pa_decode plus the new rows of pa_store_kv with num_tokens =
 * num_seqs: row s of k_new / v_new ([num_seqs, kv_heads, head_dim] of src_dtype,
 * element strides, innermost stride 1) is sequence s's new token and slot_mapping[s]
 * (int64) its slot, or < 0 for a sequence without a new token this step.
 * Contract: a slot >= 0 must be the slot of position context_lens[s] - 1 (the new token
 * is the last token of the context). Otherwise the bytes written are still exactly
 * those of pa_store_kv, but that sequence's output is unspecified.
 * With bf16/fp32 pools and rows starting on 16 bytes, the store is folded into the
 * decode launch: small batches read the new token from k_new / v_new while its slot is
 * written; larger ones (the persistent schedule's dot-product items, at most 4096
 * sequences, q_heads / kv_heads <= 4 for bf16) store each sequence's row before the
 * items that read it. Otherwise a store launch runs first. Either way the output and
 * the pool bytes are identical to the two calls. Workspace as for pa_decode.
 */
int pa_decode_step(void *out, int64_t out_stride_tok, int64_t out_stride_head, const void *q,
                   int64_t q_stride_tok, int64_t q_stride_head, int32_t q_dtype,
                   int32_t num_seqs, int32_t q_heads, const pa_kv_pool_t *pool,
                   const void *k_new, const void *v_new, int32_t src_dtype,
                   int64_t k_stride_tok, int64_t k_stride_head, int64_t v_stride_tok,
                   int64_t v_stride_head, const int64_t *slot_mapping,
                   const int32_t *block_tables, int32_t max_blocks_per_seq,
                   const int32_t *context_lens, int32_t max_context_len, float scale,
                   int32_t split_tokens, void *workspace, size_t workspace_bytes,
                   void *stream);

/*
 * pa_varlen_prefill - causal attention for a flat batch of query chunks.
 *
 * Defined by [P5] "varlen batch" / "cu_seqlens is only needed in attention" (tokens of
 * all sequences concatenated, cu_seqlens [num_seqs+1] marks the boundaries, a token
 * attends only tokens of its own sequence, causally) and [P5]'s per-sequence attention
 * over the gathered cache with a start position, which a single varlen kernel reading
 * the paged pool through block_table replaces ("comparison with vLLM").
 * For sequence s: n_s = cu_seqlens[s+1] - cu_seqlens[s], L_s = context_lens[s] (the
 * chunk's K/V already stored), P_s = L_s - n_s. Query row i of the chunk (token
 * cu_seqlens[s] + i) sits at absolute position P_s + i and attends keys 0..P_s+i of
 * sequence s only:
 *     out[t][h][:] = sum_{j <= P_s+i} softmax_j(scale * q[t][h] . K_s[j][g]) V_s[j][g][:]
 *
 *   q, out       [total_tokens, q_heads, head_dim], strided as in pa_decode.
 *   cu_seqlens   [num_seqs+1] int32, cu[0] = 0, non-decreasing, cu[num_seqs] =
 *                total_tokens. n_s == 0 is allowed (no rows).
 *   max_q_len    host-side upper bound of n_s (sizes the grid).
 *   split_tokens keys per work item: 0 = 768, else a positive multiple of 64. A row
 *                tile whose visible keys exceed it is split into key chunks handled
 *                in parallel and merged by log-sum-exp; results depend bitwise only
 *                on this value and each sequence's own (n_s, context_lens[s]).
 *   workspace    16-byte aligned device scratch of at least pa_varlen_prefill_workspace_bytes(...)
 *                bytes for the same (total_tokens, q_heads, head_dim, max_context_len,
 *                split_tokens); contents on entry ignored. It holds the call's work
 *                list (built on the device from cu_seqlens and context_lens, longest
 *                items first, dealt to the persistent workgroups in a fixed order) and,
 *                when a row tile's keys exceed split_tokens, the per-chunk partials.
 *                Calls that share a workspace must be ordered (same stream);
 *                overlapping calls race.
 *   Other arguments as in pa_decode. A chunk of length 1 is a decode row.
 * Returns PA_ERR_UNSUPPORTED, with nothing launched, when total_tokens * q_heads, the
 * work-list bound, or the number of work items or merge workgroups (row tiles of 128
 * flattened rows times max(key chunks, 8) times kv_heads times num_seqs) reaches 2^31.
 * Supported dtypes: (q BF16, pool BF16). QK^T and PV run on the matrix cores with
 * bf16 operands (P rounded to bf16) and fp32 accumulation.
 */
size_t pa_varlen_prefill_workspace_bytes(int64_t total_tokens, int32_t q_heads,
                                         int32_t head_dim, int32_t max_context_len,
                                         int32_t split_tokens);

int pa_varlen_prefill(void *out, int64_t out_stride_tok, int64_t out_stride_head,
                      const void *q, int64_t q_stride_tok, int64_t q_stride_head,
                      int32_t q_dtype, const int32_t *cu_seqlens, int32_t num_seqs,
                      int64_t total_tokens, int32_t max_q_len, int32_t q_heads,
                      const pa_kv_pool_t *pool, const int32_t *block_tables,
                      int32_t max_blocks_per_seq, const int32_t *context_lens,
                      int32_t max_context_len, float scale, int32_t split_tokens,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * pa_copy_blocks - copy whole pool blocks: for i < num_pairs, block dst_blocks[i] of K
 * and of V (and the matching rows of k_scale / v_scale of a quantised pool) becomes a
 * copy of block src_blocks[i]. src_blocks / dst_blocks are int32 DEVICE arrays; a pair
 * with an id outside [0, num_blocks) is skipped. Used for the copy-on-write that
 * pa_bm_append_token reports. The destinations must be distinct and not also sources.
 */
int pa_copy_blocks(const pa_kv_pool_t *pool, const int32_t *src_blocks,
                   const int32_t *dst_blocks, int32_t num_pairs, void *stream);

/*
 * Block manager (host only; no device memory, no stream): hands out a pool's blocks to
 * sequences and builds the block_tables / context_lens / slot_mapping the kernels take.
 *
 * Defined by [P4] "KV Cache management" (one global pool of fixed-size blocks allocated
 * up front, blocks allocated and recycled per request, a logical -> physical block_table
 * per request that lives as long as the request) and the cross-request prefix sharing
 * [P2] plans after its per-slot prefix caches ("risk 3": RadixAttention-like sharing).
 * The policy is this library's (the pages fix none of it):
 *  - a new block is the lowest-numbered free block that holds no cached prefix; only
 *    when there is none is a cached free block evicted, least recently released first
 *    (ties: lowest number);
 *  - with prefix caching on, a block that becomes full is entered in a prefix index
 *    under a chained hash of (previous block's hash, its block_size token ids), unless
 *    that hash is already present;
 *  - pa_bm_add_sequence reuses indexed blocks for the new sequence's leading full blocks
 *    while they match (hash, parent hash and token ids all equal), never for the block
 *    of its last token, and reports how many leading tokens are already cached;
 *  - appending to a shared partial block first moves the sequence to a fresh copy
 *    (copy-on-write; the caller copies the device rows with pa_copy_blocks);
 *  - a released sequence returns its blocks last block first.
 * Every entry point returns PA_OK, PA_ERR_INVALID_ARG (null handle or pointer, unknown
 * or duplicate sequence id, out-of-range position, table too narrow) or
 * PA_ERR_WORKSPACE (not enough free blocks; nothing is changed). A handle is not
 * thread-safe.
 */
typedef struct pa_block_manager pa_block_manager_t;

/* num_blocks in [1, 2^31); block_size > 0 (the kernels take 16). NULL on bad input. */
pa_block_manager_t *pa_bm_create(int64_t num_blocks, int32_t block_size,
                                 int32_t prefix_caching);
void pa_bm_destroy(pa_block_manager_t *bm);
int64_t pa_bm_num_free_blocks(const pa_block_manager_t *bm);
/* Register a sequence with its num_tokens prompt token ids; *cached_tokens (may be
 * NULL) receives the number of leading tokens whose blocks were reused. */
int pa_bm_add_sequence(pa_block_manager_t *bm, int64_t seq_id, const int32_t *token_ids,
                       int64_t num_tokens, int64_t *cached_tokens);
/* Extend a sequence by one token: *slot receives its slot; *copy_src / *copy_dst the
 * block to copy for copy-on-write, or -1 / -1. */
int pa_bm_append_token(pa_block_manager_t *bm, int64_t seq_id, int32_t token_id,
                       int64_t *slot, int32_t *copy_src, int32_t *copy_dst);
/* New sequence child_id sharing all of parent_id's blocks. */
int pa_bm_fork(pa_block_manager_t *bm, int64_t parent_id, int64_t child_id);
int pa_bm_free_sequence(pa_block_manager_t *bm, int64_t seq_id);
/* Token count of a sequence, -1 if unknown. */
int64_t pa_bm_context_len(const pa_block_manager_t *bm, int64_t seq_id);
/* Host arrays: block_tables [num_seqs, max_blocks_per_seq] (-1 padded) and, unless NULL,
 * context_lens [num_seqs], for the given sequences in order. */
int pa_bm_block_tables(const pa_block_manager_t *bm, const int64_t *seq_ids, int32_t num_seqs,
                       int32_t max_blocks_per_seq, int32_t *block_tables,
                       int32_t *context_lens);
/* Host array slots [count]: the slots of positions first_pos .. first_pos + count - 1. */
int pa_bm_slots(const pa_block_manager_t *bm, int64_t seq_id, int64_t first_pos,
                int64_t count, int64_t *slots);
/* Sequences holding a block (0: free), -1 for a bad handle or id. */
int32_t pa_bm_block_refcount(const pa_block_manager_t *bm, int32_t block);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
