// Internal launchers behind the C ABI (arguments already validated by api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pa.h"

namespace pa {

constexpr int kBlockSize = 16;

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
  float* ws_o;     // [total_tokens, q_heads, max_chunks, head_dim] when max_chunks > 1
  float* ws_lse;   // [total_tokens, q_heads, max_chunks]
};

constexpr int kPrefillDefaultSplit = 1024;

int launch_prefill(const pa_kv_pool_t& pool, const PrefillArgs& a, hipStream_t stream);

}  // namespace pa
