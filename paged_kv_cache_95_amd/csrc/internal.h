// Internal launchers behind the C ABI (arguments already validated by api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pa.h"

namespace pa {

constexpr int kBlockSize = 16;

// Workgroups of `threads` threads of a kernel resident at once on the current device
// (CUs x workgroups per CU); the grid size of the persistent kernels.
template <typename K>
inline int64_t resident_workgroups(K kernel, int threads) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess ||
      cus <= 0 || per_cu <= 0)
    return 1024;
  return (int64_t)cus * per_cu;
}

int launch_store(const pa_kv_pool_t& pool, const void* k, const void* v, int src_dtype,
                 int64_t num_tokens, int64_t k_st, int64_t k_sh, int64_t v_st, int64_t v_sh,
                 const int64_t* slot_mapping, hipStream_t stream);

// Copy K/V blocks (and scales) src[i] -> dst[i], i < n (device arrays).
int launch_copy_blocks(const pa_kv_pool_t& pool, const int32_t* src, const int32_t* dst, int n,
                       hipStream_t stream);

struct DecodeArgs {
  void* out;
  int64_t out_st, out_sh;
  const void* q;
  int64_t q_st, q_sh;
  int num_seqs, q_heads;
  const int32_t* block_tables;
  int max_blocks_per_seq;
  const int32_t* context_lens;
  int max_context_len;
  float scale;
  int split_tokens;
  int max_splits;
  int head_dim;
  float* ws_o;    // [num_seqs, q_heads, max_splits, head_dim]
  float* ws_lse;  // [num_seqs, q_heads, max_splits]
  unsigned* counters;  // [num_seqs, kv_heads] used of kDecodeCounters, zero between calls
};

// The decode workspace starts with a fixed block of arrival counters (the single-launch
// schedule uses one per (sequence, KV head) and runs only when there are at most this
// many), so the same bytes are counters in every call and never hold partials.
constexpr int kDecodeCounters = 1024;
constexpr size_t kDecodeCounterBytes = kDecodeCounters * sizeof(unsigned);


int launch_decode(const pa_kv_pool_t& pool, const DecodeArgs& a, hipStream_t stream);

// Size of pa_decode_noalloc's per-device scratch array (the same value as
// PA_NOALLOC_SCRATCH_BYTES in pa.h).
constexpr size_t kNoallocScratchBytes = PA_NOALLOC_SCRATCH_BYTES;
// Device address of the current device's scratch array (looked up, and its counter
// block cleared by a kernel on `stream`, on the first call on that device).
int noalloc_scratch(void** ptr, hipStream_t stream);

// New rows of a decode step: row s of k / v ([num_seqs, kv_heads, head_dim] of src_dtype,
// element strides) is sequence s's newest token, to be stored at slots[s] (< 0: none).
struct StepRows {
  const void* k;
  const void* v;
  int src_dtype;
  int64_t k_st, k_sh, v_st, v_sh;
  const int64_t* slots;
};

// Store the step's rows, then decode; one launch when the single-launch schedule runs.
int launch_decode_step(const pa_kv_pool_t& pool, const DecodeArgs& a, const StepRows& rows,
                       hipStream_t stream);

// Fused RoPE + store of a step's new tokens (pa_rope_store_kv).
struct RopeArgs {
  void* kpool;
  void* vpool;
  float* kscale;
  float* vscale;
  int64_t num_blocks;
  int hkv;
  const void* q;
  int64_t q_st, q_sh;
  int q_heads;
  void* q_out;
  int64_t qo_st, qo_sh;
  const void* k;
  int64_t k_st, k_sh;
  const void* v;
  int64_t v_st, v_sh;
  int64_t num_tokens;
  const int64_t* positions;
  const float* cos_table;  // [max_position, head_dim / 2]
  const float* sin_table;
  int64_t max_position;
  const int64_t* slots;
};

int launch_rope_store(const pa_kv_pool_t& pool, const RopeArgs& a, int src_dtype,
                      hipStream_t stream);

struct PrefillArgs {
  void* out;
  int64_t out_st, out_sh;
  const void* q;
  int64_t q_st, q_sh;
  const int32_t* cu_seqlens;
  int num_seqs;
  int64_t total_tokens;
  int max_q_len, q_heads;
  const int32_t* block_tables;
  int max_blocks_per_seq;
  const int32_t* context_lens;
  int max_context_len;
  float scale;
  int split_keys;  // keys per work item, multiple of 64
  int max_chunks;  // ceil(max_context_len / split_keys)
  void* plan;      // work list: kPfPlanHeaderBytes of header, then plan_bound entries
  int64_t plan_bound;
  float* ws_o;     // [total_tokens, q_heads, max_chunks, head_dim] when max_chunks > 1
  float* ws_lse;   // [total_tokens, q_heads, max_chunks]
};

// Keys per prefill work item when the caller passes 0: on the varlen mixed step
// (16 chunks on prefixes up to 2048) 768 gave 63.0 us per call against 63.6 at 1024 and
// 64.6 at 896 (the longest items, which bound the call, against the extra partials).
constexpr int kPrefillDefaultSplit = 768;

// The prefill workspace starts with its work list: a header (entry count and the
// claim counter) and one 32-byte entry per (sequence, row tile, key chunk) that has
// work. Entries are at most one per 128 query rows (plus one per non-empty chunk) per
// key chunk, bounded without knowing the KV-head count by taking G <= q_heads.
constexpr int64_t kPfPlanHeaderBytes = 256;
constexpr int64_t kPfPlanEntryBytes = 32;
inline int64_t prefill_plan_bound(int64_t total_tokens, int64_t q_heads, int64_t max_chunks) {
  return ((total_tokens * q_heads + 127) / 128 + total_tokens) * max_chunks;
}

int launch_prefill(const pa_kv_pool_t& pool, const PrefillArgs& a, hipStream_t stream);

// Device-data checks (launched by the PA_DEBUG_CHECKS build of api.cpp only; the
// release build never calls them). Each records the first contract violation it sees
// in the current GPU's violation word.
int validate_decode(const pa_kv_pool_t& pool, const int32_t* block_tables, int max_blocks,
                    const int32_t* ctx, int num_seqs, int max_ctx, const int64_t* slots,
                    hipStream_t stream);
int validate_tokens(const pa_kv_pool_t& pool, const int64_t* slots, int64_t n,
                    const int64_t* positions, int64_t max_position, hipStream_t stream);
int validate_varlen(const pa_kv_pool_t& pool, const PrefillArgs& a, hipStream_t stream);
// Waits for `stream` and reads the violation word: PA_ERR_DEVICE_DATA while one is set.
int debug_gate(hipStream_t stream);
// Waits for `stream`, returns the recorded violation (code 0: none) and clears it.
int debug_take(hipStream_t stream, int32_t* code, int64_t* where);

}  // namespace pa
