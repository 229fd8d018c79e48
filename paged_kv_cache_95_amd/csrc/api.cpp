// C ABI of libpa.so: argument validation, workspace sizing and dispatch.
//
// Validation runs entirely on the host and before any HIP call, so an invalid call
// launches nothing (and can be exercised without a GPU). No exception crosses the ABI.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "internal.h"

namespace {

using pa::kBlockSize;

constexpr int kMaxGroup = 8;
constexpr int kMaxSplitTokens = 1024;  // one wave keeps a split's block ids in its 64 lanes

bool pool_shape_ok(const pa_kv_pool_t* p, int* status) {
  if (!p || !p->k || !p->v) return *status = PA_ERR_INVALID_ARG, false;
  if (p->num_blocks <= 0 || p->block_size <= 0 || p->kv_heads <= 0 || p->head_dim <= 0)
    return *status = PA_ERR_INVALID_ARG, false;
  if (p->dtype != PA_F32 && p->dtype != PA_BF16 && p->dtype != PA_FP8_E4M3 &&
      p->dtype != PA_INT8)
    return *status = PA_ERR_INVALID_ARG, false;
  if ((p->dtype == PA_FP8_E4M3 || p->dtype == PA_INT8) && (!p->k_scale || !p->v_scale))
    return *status = PA_ERR_INVALID_ARG, false;
  if (p->block_size != kBlockSize) return *status = PA_ERR_UNSUPPORTED, false;
  if (p->head_dim != 64 && p->head_dim != 128) return *status = PA_ERR_UNSUPPORTED, false;
  return true;
}

bool q_dtype_ok(int q_dtype, int pool_dtype) {
  return (q_dtype == PA_F32 && pool_dtype == PA_F32) ||
         (q_dtype == PA_BF16 &&
          (pool_dtype == PA_BF16 || pool_dtype == PA_FP8_E4M3 || pool_dtype == PA_INT8));
}

// Split length used when the caller passes 0: aim at about 2048 (sequence, KV head,
// split) work items for the worst case of every context at max_context_len (eight
// waves per CU), as a power of two in [32, 1024] tokens. Small batches get short splits
// (more waves in flight for a latency-bound call), large ones long splits (fewer
// partials to merge, and fewer item starts: on the 256-sequence decode with contexts up
// to 32K, 1024-token splits took 1797 us against 1857 us at 512).
int effective_split(int split_tokens, int64_t num_seqs, int kv_heads, int max_context_len) {
  if (split_tokens != 0) return split_tokens;
  const int64_t want = num_seqs * kv_heads * (int64_t)max_context_len / 2048;
  int split = 32;
  while (split < 1024 && split < want) split <<= 1;
  return split;
}

// Source rows of pa_store_kv / pa_decode_step: dtype pairing and strides.
int check_store_rows(const pa_kv_pool_t* pool, int32_t src_dtype, int64_t k_stride_tok,
                     int64_t k_stride_head, int64_t v_stride_tok, int64_t v_stride_head) {
  const bool quant = pool->dtype == PA_FP8_E4M3 || pool->dtype == PA_INT8;
  const bool src_ok = quant ? (src_dtype == PA_BF16 || src_dtype == PA_F32)
                            : src_dtype == pool->dtype;
  if (!src_ok) return PA_ERR_INVALID_ARG;
  if (k_stride_tok < 0 || k_stride_head < 0 || v_stride_tok < 0 || v_stride_head < 0)
    return PA_ERR_INVALID_ARG;
  return PA_OK;
}

// Status of an entry point's launches: each launch reports its own status (see
// launch_kernel), so an error left pending by the caller's earlier HIP calls is neither
// attributed to this call nor cleared.
int launched(int status) { return status; }

// PA_DEBUG_CHECKS build: before a call launches, wait for its stream and refuse it while
// an earlier call's violation is recorded, then launch the check of this call's device
// metadata ahead of its kernels. The release build compiles these to nothing.
#ifdef PA_DEBUG_CHECKS
constexpr int kDebugBuild = 1;
#define PA_DEBUG_GATE(stream)                                           \
  do {                                                                  \
    const int gate_ = pa::debug_gate((hipStream_t)(stream));            \
    if (gate_ != PA_OK) return gate_;                                   \
  } while (0)
#define PA_DEBUG_CHECK(call)                                            \
  do {                                                                  \
    const int check_ = (call);                                          \
    if (check_ != PA_OK) return check_;                                 \
  } while (0)
#else
constexpr int kDebugBuild = 0;
#define PA_DEBUG_GATE(stream) \
  do {                        \
  } while (0)
#define PA_DEBUG_CHECK(call) \
  do {                       \
  } while (0)
#endif

}  // namespace

extern "C" {

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARG: return "PA_ERR_INVALID_ARG: invalid argument";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: shape or dtype not supported";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace missing or too small";
    case PA_ERR_HIP: return "PA_ERR_HIP: kernel launch failed";
    case PA_ERR_DEVICE_DATA:
      return "PA_ERR_DEVICE_DATA: an earlier call's device metadata broke its contract "
             "(pa_debug_take_violation)";
    default: return "unknown pa status";
  }
}

int32_t pa_decode_default_split_tokens(int32_t num_seqs, int32_t kv_heads,
                                       int32_t max_context_len) {
  if (num_seqs <= 0 || kv_heads <= 0 || max_context_len <= 0) return 0;
  return effective_split(0, num_seqs, kv_heads, max_context_len);
}

int32_t pa_debug_checks(void) { return kDebugBuild; }

int pa_debug_take_violation(void* stream, int32_t* code, int64_t* where) {
  if (!code || !where) return PA_ERR_INVALID_ARG;
#if PA_DEBUG_CHECKS
  return pa::debug_take((hipStream_t)stream, code, where);
#else
  // the release build runs no checks, so it never has a violation to report
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return PA_ERR_HIP;
  *code = 0;
  *where = 0;
  return PA_OK;
#endif
}


int pa_rope_store_kv(const pa_kv_pool_t* pool, const void* q, int64_t q_stride_tok,
                     int64_t q_stride_head, int32_t q_heads, void* q_out,
                     int64_t q_out_stride_tok, int64_t q_out_stride_head, const void* k,
                     const void* v, int32_t src_dtype, int64_t num_tokens,
                     int64_t k_stride_tok, int64_t k_stride_head, int64_t v_stride_tok,
                     int64_t v_stride_head, const int64_t* positions, const float* cos_table,
                     const float* sin_table, int32_t max_position,
                     const int64_t* slot_mapping, void* stream) {
  int status = PA_OK;
  if (!pool_shape_ok(pool, &status)) return status;
  if (num_tokens < 0 || q_heads <= 0 || q_heads % pool->kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (src_dtype != PA_BF16 && src_dtype != PA_F32) return PA_ERR_INVALID_ARG;
  status = check_store_rows(pool, src_dtype, k_stride_tok, k_stride_head, v_stride_tok,
                            v_stride_head);
  if (status != PA_OK) return status;
  if (q_stride_tok < 0 || q_stride_head < 0 || q_out_stride_tok < 0 || q_out_stride_head < 0 ||
      max_position <= 0)
    return PA_ERR_INVALID_ARG;
  if (num_tokens == 0) return PA_OK;
  if (!q || !q_out || !k || !v || !positions || !cos_table || !sin_table || !slot_mapping)
    return PA_ERR_INVALID_ARG;
  pa::RopeArgs a;
  a.kpool = pool->k;
  a.vpool = pool->v;
  a.kscale = pool->k_scale;
  a.vscale = pool->v_scale;
  a.num_blocks = pool->num_blocks;
  a.hkv = pool->kv_heads;
  a.q = q;
  a.q_st = q_stride_tok;
  a.q_sh = q_stride_head;
  a.q_heads = q_heads;
  a.q_out = q_out;
  a.qo_st = q_out_stride_tok;
  a.qo_sh = q_out_stride_head;
  a.k = k;
  a.k_st = k_stride_tok;
  a.k_sh = k_stride_head;
  a.v = v;
  a.v_st = v_stride_tok;
  a.v_sh = v_stride_head;
  a.num_tokens = num_tokens;
  a.positions = positions;
  a.cos_table = cos_table;
  a.sin_table = sin_table;
  a.max_position = max_position;
  a.slots = slot_mapping;
  PA_DEBUG_GATE(stream);
  PA_DEBUG_CHECK(pa::validate_tokens(*pool, slot_mapping, num_tokens, positions, max_position,
                                     (hipStream_t)stream));
  return launched(pa::launch_rope_store(*pool, a, src_dtype, (hipStream_t)stream));
}

int pa_copy_blocks(const pa_kv_pool_t* pool, const int32_t* src_blocks,
                   const int32_t* dst_blocks, int32_t num_pairs, void* stream) {
  int status = PA_OK;
  if (!pool_shape_ok(pool, &status)) return status;
  if (num_pairs < 0) return PA_ERR_INVALID_ARG;
  if (num_pairs == 0) return PA_OK;
  if (!src_blocks || !dst_blocks) return PA_ERR_INVALID_ARG;
  PA_DEBUG_GATE(stream);
  return launched(pa::launch_copy_blocks(*pool, src_blocks, dst_blocks, num_pairs,
                                         (hipStream_t)stream));
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t q_heads, int32_t kv_heads,
                                 int32_t head_dim, int32_t max_context_len,
                                 int32_t split_tokens) {
  if (num_seqs <= 0 || q_heads <= 0 || kv_heads <= 0 || head_dim <= 0 ||
      max_context_len <= 0 || split_tokens < 0)
    return 0;
  const int split = effective_split(split_tokens, num_seqs, kv_heads, max_context_len);
  const int64_t max_splits = ((int64_t)max_context_len + split - 1) / split;
  if (max_splits <= 1) return 0;
  return pa::kDecodeCounterBytes +
         (size_t)num_seqs * q_heads * max_splits * (head_dim + 1) * sizeof(float);
}

int pa_store_kv(const pa_kv_pool_t* pool, const void* k, const void* v, int32_t src_dtype,
                int64_t num_tokens, int64_t k_stride_tok, int64_t k_stride_head,
                int64_t v_stride_tok, int64_t v_stride_head, const int64_t* slot_mapping,
                void* stream) {
  int status = PA_OK;
  if (!pool_shape_ok(pool, &status)) return status;
  if (num_tokens < 0) return PA_ERR_INVALID_ARG;
  status = check_store_rows(pool, src_dtype, k_stride_tok, k_stride_head, v_stride_tok,
                            v_stride_head);
  if (status != PA_OK || num_tokens == 0) return status;
  if (!k || !v || !slot_mapping) return PA_ERR_INVALID_ARG;
  PA_DEBUG_GATE(stream);
  PA_DEBUG_CHECK(pa::validate_tokens(*pool, slot_mapping, num_tokens, nullptr, 0,
                                     (hipStream_t)stream));
  return launched(pa::launch_store(*pool, k, v, src_dtype, num_tokens, k_stride_tok,
                                   k_stride_head, v_stride_tok, v_stride_head, slot_mapping,
                                   (hipStream_t)stream));
}

}  // extern "C"

namespace {

// workspace: [arrival counters, fixed 4 KiB][o: num_seqs, q_heads, max_splits, D][lse];
// nullptr when the call needs none (every context fits one split).
void bind_decode_workspace(pa::DecodeArgs* a, void* workspace) {
  a->counters = workspace ? (unsigned*)workspace : nullptr;
  a->ws_o = workspace ? (float*)((char*)workspace + pa::kDecodeCounterBytes) : nullptr;
  a->ws_lse = workspace ? a->ws_o + (size_t)a->num_seqs * a->q_heads * a->max_splits * a->head_dim
                        : nullptr;
}

// Validation and argument block shared by pa_decode and pa_decode_step. Returns PA_OK
// with *nothing = true when there is no sequence to decode.
int prepare_decode(void* out, int64_t out_stride_tok, int64_t out_stride_head, const void* q,
                   int64_t q_stride_tok, int64_t q_stride_head, int32_t q_dtype,
                   int32_t num_seqs, int32_t q_heads, const pa_kv_pool_t* pool,
                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                   const int32_t* context_lens, int32_t max_context_len, float scale,
                   int32_t split_tokens, void* workspace, size_t workspace_bytes,
                   pa::DecodeArgs* a, bool* nothing) {
  *nothing = false;
  int status = PA_OK;
  if (!pool_shape_ok(pool, &status)) return status;
  if (num_seqs < 0 || q_heads <= 0 || q_heads % pool->kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (q_heads / pool->kv_heads > kMaxGroup) return PA_ERR_UNSUPPORTED;
  if (!q_dtype_ok(q_dtype, pool->dtype)) return PA_ERR_INVALID_ARG;
  if (out_stride_tok < 0 || out_stride_head < 0 || q_stride_tok < 0 || q_stride_head < 0)
    return PA_ERR_INVALID_ARG;
  if (split_tokens < 0 || split_tokens % kBlockSize != 0 || split_tokens > kMaxSplitTokens)
    return PA_ERR_INVALID_ARG;
  if (!(scale > 0.0f) || scale > 3.0e38f) return PA_ERR_INVALID_ARG;  // finite, positive
  if (num_seqs == 0) return *nothing = true, PA_OK;
  if (!out || !q || !block_tables || !context_lens) return PA_ERR_INVALID_ARG;
  if (max_blocks_per_seq <= 0 || max_context_len <= 0 ||
      (int64_t)max_context_len > (int64_t)max_blocks_per_seq * kBlockSize)
    return PA_ERR_INVALID_ARG;
  const int split = effective_split(split_tokens, num_seqs, pool->kv_heads, max_context_len);
  const int max_splits = (max_context_len + split - 1) / split;
  const size_t need = pa_decode_workspace_bytes(num_seqs, q_heads, pool->kv_heads,
                                                pool->head_dim, max_context_len, split);
  if (need > 0 && (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 15u) != 0))
    return PA_ERR_WORKSPACE;
  const int64_t grid = ((int64_t)num_seqs * max_splits * pool->kv_heads + 3) / 4;
  if (grid >= (int64_t)1 << 31 || (int64_t)num_seqs * q_heads >= (int64_t)1 << 31)
    return PA_ERR_UNSUPPORTED;

  a->out = out;
  a->out_st = out_stride_tok;
  a->out_sh = out_stride_head;
  a->q = q;
  a->q_st = q_stride_tok;
  a->q_sh = q_stride_head;
  a->num_seqs = num_seqs;
  a->q_heads = q_heads;
  a->block_tables = block_tables;
  a->max_blocks_per_seq = max_blocks_per_seq;
  a->context_lens = context_lens;
  a->max_context_len = max_context_len;
  a->scale = scale;
  a->split_tokens = split;
  a->max_splits = max_splits;
  a->head_dim = pool->head_dim;
  bind_decode_workspace(a, need > 0 ? workspace : nullptr);
  return PA_OK;
}

}  // namespace

extern "C" {

int pa_decode(void* out, int64_t out_stride_tok, int64_t out_stride_head, const void* q,
              int64_t q_stride_tok, int64_t q_stride_head, int32_t q_dtype, int32_t num_seqs,
              int32_t q_heads, const pa_kv_pool_t* pool, const int32_t* block_tables,
              int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t max_context_len,
              float scale, int32_t split_tokens, void* workspace, size_t workspace_bytes,
              void* stream) {
  pa::DecodeArgs a;
  bool nothing = false;
  const int st = prepare_decode(out, out_stride_tok, out_stride_head, q, q_stride_tok,
                                q_stride_head, q_dtype, num_seqs, q_heads, pool, block_tables,
                                max_blocks_per_seq, context_lens, max_context_len, scale,
                                split_tokens, workspace, workspace_bytes, &a, &nothing);
  if (st != PA_OK || nothing) return st;
  PA_DEBUG_GATE(stream);
  PA_DEBUG_CHECK(pa::validate_decode(*pool, block_tables, max_blocks_per_seq, context_lens,
                                     num_seqs, max_context_len, nullptr, (hipStream_t)stream));
  return launched(pa::launch_decode(*pool, a, (hipStream_t)stream));
}

int pa_decode_noalloc(void* out, int64_t out_stride_tok, int64_t out_stride_head,
                      const void* q, int64_t q_stride_tok, int64_t q_stride_head,
                      int32_t q_dtype, int32_t num_seqs, int32_t q_heads,
                      const pa_kv_pool_t* pool, const int32_t* block_tables,
                      int32_t max_blocks_per_seq, const int32_t* context_lens,
                      int32_t max_context_len, float scale, int32_t split_tokens,
                      void* stream) {
  pa::DecodeArgs a;
  bool nothing = false;
  // validated against the scratch array's size; its device address is looked up only
  // for a call that launches (a placeholder stands in for it until then)
  void* const placeholder = reinterpret_cast<void*>(uintptr_t{256});
  const int st = prepare_decode(out, out_stride_tok, out_stride_head, q, q_stride_tok,
                                q_stride_head, q_dtype, num_seqs, q_heads, pool, block_tables,
                                max_blocks_per_seq, context_lens, max_context_len, scale,
                                split_tokens, placeholder, pa::kNoallocScratchBytes, &a,
                                &nothing);
  if (st != PA_OK || nothing) return st;
  PA_DEBUG_GATE(stream);
  PA_DEBUG_CHECK(pa::validate_decode(*pool, block_tables, max_blocks_per_seq, context_lens,
                                     num_seqs, max_context_len, nullptr, (hipStream_t)stream));
  if (a.counters != nullptr) {
    void* scratch = nullptr;
    const int s2 = pa::noalloc_scratch(&scratch, (hipStream_t)stream);
    if (s2 != PA_OK) return s2;
    bind_decode_workspace(&a, scratch);
  }
  return launched(pa::launch_decode(*pool, a, (hipStream_t)stream));
}

int pa_decode_step(void* out, int64_t out_stride_tok, int64_t out_stride_head, const void* q,
                   int64_t q_stride_tok, int64_t q_stride_head, int32_t q_dtype,
                   int32_t num_seqs, int32_t q_heads, const pa_kv_pool_t* pool,
                   const void* k_new, const void* v_new, int32_t src_dtype,
                   int64_t k_stride_tok, int64_t k_stride_head, int64_t v_stride_tok,
                   int64_t v_stride_head, const int64_t* slot_mapping,
                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                   const int32_t* context_lens, int32_t max_context_len, float scale,
                   int32_t split_tokens, void* workspace, size_t workspace_bytes,
                   void* stream) {
  pa::DecodeArgs a;
  bool nothing = false;
  int st = prepare_decode(out, out_stride_tok, out_stride_head, q, q_stride_tok, q_stride_head,
                          q_dtype, num_seqs, q_heads, pool, block_tables, max_blocks_per_seq,
                          context_lens, max_context_len, scale, split_tokens, workspace,
                          workspace_bytes, &a, &nothing);
  if (st != PA_OK) return st;
  st = check_store_rows(pool, src_dtype, k_stride_tok, k_stride_head, v_stride_tok,
                        v_stride_head);
  if (st != PA_OK || nothing) return st;
  if (!k_new || !v_new || !slot_mapping) return PA_ERR_INVALID_ARG;
  pa::StepRows rows;
  rows.k = k_new;
  rows.v = v_new;
  rows.src_dtype = src_dtype;
  rows.k_st = k_stride_tok;
  rows.k_sh = k_stride_head;
  rows.v_st = v_stride_tok;
  rows.v_sh = v_stride_head;
  rows.slots = slot_mapping;
  PA_DEBUG_GATE(stream);
  PA_DEBUG_CHECK(pa::validate_decode(*pool, block_tables, max_blocks_per_seq, context_lens,
                                     num_seqs, max_context_len, slot_mapping,
                                     (hipStream_t)stream));
  PA_DEBUG_CHECK(pa::validate_tokens(*pool, slot_mapping, num_seqs, nullptr, 0,
                                     (hipStream_t)stream));
  return launched(pa::launch_decode_step(*pool, a, rows, (hipStream_t)stream));
}

size_t pa_varlen_prefill_workspace_bytes(int64_t total_tokens, int32_t q_heads,
                                         int32_t head_dim, int32_t max_context_len,
                                         int32_t split_tokens) {
  if (total_tokens <= 0 || q_heads <= 0 || head_dim <= 0 || max_context_len <= 0 ||
      split_tokens < 0 || split_tokens % 64 != 0)
    return 0;
  const int split = split_tokens == 0 ? pa::kPrefillDefaultSplit : split_tokens;
  const int64_t chunks = ((int64_t)max_context_len + split - 1) / split;
  // work list, then (several key chunks) the partials: o [T, Hq, chunks, D], lse
  const size_t plan = (size_t)(pa::kPfPlanHeaderBytes +
                               pa::prefill_plan_bound(total_tokens, q_heads, chunks) *
                                   pa::kPfPlanEntryBytes);
  if (chunks <= 1) return plan;
  return plan + (size_t)total_tokens * q_heads * chunks * (head_dim + 1) * sizeof(float);
}

int pa_varlen_prefill(void* out, int64_t out_stride_tok, int64_t out_stride_head,
                      const void* q, int64_t q_stride_tok, int64_t q_stride_head,
                      int32_t q_dtype, const int32_t* cu_seqlens, int32_t num_seqs,
                      int64_t total_tokens, int32_t max_q_len, int32_t q_heads,
                      const pa_kv_pool_t* pool, const int32_t* block_tables,
                      int32_t max_blocks_per_seq, const int32_t* context_lens,
                      int32_t max_context_len, float scale, int32_t split_tokens,
                      void* workspace, size_t workspace_bytes, void* stream) {
  int status = PA_OK;
  if (!pool_shape_ok(pool, &status)) return status;
  if (num_seqs < 0 || total_tokens < 0 || q_heads <= 0 || q_heads % pool->kv_heads != 0)
    return PA_ERR_INVALID_ARG;
  if (q_heads / pool->kv_heads > kMaxGroup) return PA_ERR_UNSUPPORTED;
  if (!q_dtype_ok(q_dtype, pool->dtype)) return PA_ERR_INVALID_ARG;
  if (pool->dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  if (out_stride_tok < 0 || out_stride_head < 0 || q_stride_tok < 0 || q_stride_head < 0)
    return PA_ERR_INVALID_ARG;
  if (!(scale > 0.0f) || scale > 3.0e38f) return PA_ERR_INVALID_ARG;  // finite, positive
  if (num_seqs == 0 || total_tokens == 0) return PA_OK;
  if (!out || !q || !cu_seqlens || !block_tables || !context_lens) return PA_ERR_INVALID_ARG;
  if (max_q_len <= 0 || max_blocks_per_seq <= 0 || max_context_len <= 0 ||
      max_q_len > max_context_len ||
      (int64_t)max_context_len > (int64_t)max_blocks_per_seq * kBlockSize)
    return PA_ERR_INVALID_ARG;
  if (split_tokens < 0 || split_tokens % 64 != 0) return PA_ERR_INVALID_ARG;
  const int split = split_tokens == 0 ? pa::kPrefillDefaultSplit : split_tokens;
  const int max_chunks = (max_context_len + split - 1) / split;
  const size_t need = pa_varlen_prefill_workspace_bytes(total_tokens, q_heads, pool->head_dim,
                                                        max_context_len, split);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 15u) != 0)
    return PA_ERR_WORKSPACE;
  const int64_t tiles = ((int64_t)max_q_len * (q_heads / pool->kv_heads) + 127) / 128;
  const int64_t plan_bound = pa::prefill_plan_bound(total_tokens, q_heads, max_chunks);
  // work items, the merge grid (at most 8 workgroups per row tile) and the work list
  if (tiles * std::max(max_chunks, 8) * pool->kv_heads * num_seqs >= (int64_t)1 << 31 ||
      total_tokens * q_heads >= (int64_t)1 << 31 || plan_bound >= (int64_t)1 << 31)
    return PA_ERR_UNSUPPORTED;

  pa::PrefillArgs a;
  a.out = out;
  a.out_st = out_stride_tok;
  a.out_sh = out_stride_head;
  a.q = q;
  a.q_st = q_stride_tok;
  a.q_sh = q_stride_head;
  a.cu_seqlens = cu_seqlens;
  a.num_seqs = num_seqs;
  a.total_tokens = total_tokens;
  a.max_q_len = max_q_len;
  a.q_heads = q_heads;
  a.block_tables = block_tables;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.context_lens = context_lens;
  a.max_context_len = max_context_len;
  a.scale = scale;
  a.split_keys = split;
  a.max_chunks = max_chunks;
  a.plan = workspace;
  a.plan_bound = plan_bound;
  const size_t plan_bytes = (size_t)(pa::kPfPlanHeaderBytes + plan_bound * pa::kPfPlanEntryBytes);
  a.ws_o = max_chunks > 1 ? (float*)((char*)workspace + plan_bytes) : nullptr;
  a.ws_lse = max_chunks > 1
                 ? a.ws_o + (size_t)total_tokens * q_heads * max_chunks * pool->head_dim
                 : nullptr;
  PA_DEBUG_GATE(stream);
  PA_DEBUG_CHECK(pa::validate_varlen(*pool, a, (hipStream_t)stream));
  return launched(pa::launch_prefill(*pool, a, (hipStream_t)stream));
}

}  // extern "C"
