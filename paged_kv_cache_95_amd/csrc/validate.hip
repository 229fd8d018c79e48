// Device-data contract checks of the PA_DEBUG_CHECKS build of the library.
//
// The kernels of the path never read or write outside their buffers whatever the
// device-side metadata holds (block ids outside the pool and slots past it are
// skipped, context lengths are clamped to the host bound), but the affected outputs
// are then unspecified: a wrong slot or an off-by-one context length, the bugs the
// koas-w "errors and solutions" post lists first (types 1 and 2), would pass silently.
// In the debug build every kernel call first launches one of the small kernels below
// on the same stream. Each checks the metadata the call is about to use and records
// the first contract violation it sees in a per-device word (code in the top byte,
// where it happened below); the call itself then runs exactly as in the release
// build. The host reads the word before the next call (api.cpp).
#include <algorithm>
#include <mutex>

#include "common.h"
#include "internal.h"

namespace pa {

// The first violation recorded on this GPU since the word was last taken, or 0.
static __device__ __align__(8) unsigned long long violation_word = 0ull;

__device__ __forceinline__ void record(unsigned long long* w, int code, uint64_t where) {
  const unsigned long long v = ((unsigned long long)code << 56) | (where & ((1ull << 56) - 1));
  atomicCAS(w, 0ull, v);
}
__device__ __forceinline__ uint64_t seq_block(int s, int j) {
  return ((uint64_t)(uint32_t)s << 28) | (uint32_t)(j & ((1 << 28) - 1));
}

// One wave per sequence: 1 <= L <= max_ctx, the ids of blocks 0..ceil(L/16)-1 inside
// the pool, and (decode step) a new token's slot equal to the slot of position L - 1.
__global__ void __launch_bounds__(64) validate_decode_kernel(
    const int32_t* __restrict__ block_tables, int max_blocks, const int32_t* __restrict__ ctx,
    int max_ctx, int64_t num_blocks, const int64_t* __restrict__ slots,
    unsigned long long* w) {
  const int s = blockIdx.x, lane = threadIdx.x;
  const int L = ctx[s];
  if (L < 1 || L > max_ctx) {
    if (lane == 0) record(w, PA_VIOLATION_CONTEXT_LEN, (uint64_t)s);
    return;
  }
  const int32_t* row = block_tables + (int64_t)s * max_blocks;
  const int nblk = (L + kBlockSize - 1) / kBlockSize;  // <= max_blocks (host-checked bound)
  for (int j = lane; j < nblk; j += 64)
    if (row[j] < 0 || (int64_t)row[j] >= num_blocks)
      record(w, PA_VIOLATION_BLOCK_ID, seq_block(s, j));
  if (slots != nullptr && lane == 0) {
    const int64_t sl = slots[s];
    if (sl >= num_blocks * kBlockSize) {
      record(w, PA_VIOLATION_SLOT, (uint64_t)s);
    } else if (sl >= 0) {
      const int p = L - 1;
      const int64_t want = (int64_t)row[p / kBlockSize] * kBlockSize + p % kBlockSize;
      if (sl != want) record(w, PA_VIOLATION_STEP_SLOT, (uint64_t)s);
    }
  }
}

// Slots of one call seen so far, for the duplicate check: open addressing over
// kDupSlots entries (empty = -1), at most half full (longer calls skip the check).
constexpr int kDupSlots = 1 << 20;
constexpr int64_t kDupMaxTokens = kDupSlots / 2;
static __device__ __align__(16) unsigned long long dup_table[kDupSlots];

__global__ void __launch_bounds__(256) clear_dup_table_kernel(unsigned long long* t) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < kDupSlots; i += gridDim.x * 256) t[i] = ~0ull;
}

// Insert `slot` (>= 0); true when another token of the call inserted it first.
__device__ __forceinline__ bool dup_insert(unsigned long long* t, int64_t slot) {
  const unsigned long long key = (unsigned long long)slot;
  unsigned h = (unsigned)((key * 0x9E3779B97F4A7C15ull) >> 40) & (kDupSlots - 1);
  for (int probe = 0; probe < kDupSlots; ++probe) {  // ends: the table is at most half full
    const unsigned long long prev = atomicCAS(&t[h], ~0ull, key);
    if (prev == ~0ull) return false;
    if (prev == key) return true;
    h = (h + 1) & (kDupSlots - 1);
  }
  return false;
}

// One thread per token: slot_mapping[t] < num_blocks * 16 (negative = padding, legal);
// with positions, 0 <= positions[t] < max_position; with `dups`, no slot twice.
__global__ void __launch_bounds__(256) validate_tokens_kernel(
    const int64_t* __restrict__ slots, int64_t n, int64_t num_blocks,
    const int64_t* __restrict__ positions, int64_t max_position, unsigned long long* w,
    unsigned long long* dups) {
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n;
       t += (int64_t)gridDim.x * blockDim.x) {
    if (slots[t] >= num_blocks * kBlockSize) record(w, PA_VIOLATION_SLOT, (uint64_t)t);
    else if (dups != nullptr && slots[t] >= 0 && dup_insert(dups, slots[t]))
      record(w, PA_VIOLATION_DUP_SLOT, (uint64_t)t);
    if (positions != nullptr && (positions[t] < 0 || positions[t] >= max_position))
      record(w, PA_VIOLATION_POSITION, (uint64_t)t);
  }
}

// One wave per sequence of a varlen call: cu_seqlens starts at 0, never decreases and
// ends at total_tokens, every chunk is at most max_q_len long and fits its context
// (n_s <= L_s <= max_ctx), and the ids of blocks 0..ceil(L/16)-1 are inside the pool.
__global__ void __launch_bounds__(64) validate_varlen_kernel(
    const int32_t* __restrict__ cu, int num_seqs, int64_t total, int max_q_len,
    const int32_t* __restrict__ block_tables, int max_blocks, const int32_t* __restrict__ ctx,
    int max_ctx, int64_t num_blocks, unsigned long long* w) {
  const int s = blockIdx.x, lane = threadIdx.x;
  const int c0 = cu[s], c1 = cu[s + 1];
  const int n = c1 - c0;
  if ((s == 0 && c0 != 0) || c1 < c0 || (s == num_seqs - 1 && c1 != total) || n > max_q_len) {
    if (lane == 0) record(w, PA_VIOLATION_CU_SEQLENS, (uint64_t)s);
    return;
  }
  const int L = ctx[s];
  if (L < 0 || L > max_ctx) {
    if (lane == 0) record(w, PA_VIOLATION_CONTEXT_LEN, (uint64_t)s);
    return;
  }
  if (n > L) {
    if (lane == 0) record(w, PA_VIOLATION_CHUNK, (uint64_t)s);
    return;
  }
  const int32_t* row = block_tables + (int64_t)s * max_blocks;
  const int nblk = (L + kBlockSize - 1) / kBlockSize;
  for (int j = lane; j < nblk; j += 64)
    if (row[j] < 0 || (int64_t)row[j] >= num_blocks)
      record(w, PA_VIOLATION_BLOCK_ID, seq_block(s, j));
}

// Device addresses of the current device's violation word and duplicate table (looked
// up once per device, with that device current; host code never uses the variables'
// names as addresses).
static int debug_ptrs(unsigned long long** word, unsigned long long** dups) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static unsigned long long* words[kMaxDevices] = {};
  static unsigned long long* tables[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return PA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(mu);
  if (words[dev] == nullptr) {
    void* p = nullptr;
    void* t = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(violation_word)) != hipSuccess || p == nullptr ||
        hipGetSymbolAddress(&t, HIP_SYMBOL(dup_table)) != hipSuccess || t == nullptr)
      return PA_ERR_HIP;
    words[dev] = (unsigned long long*)p;
    tables[dev] = (unsigned long long*)t;
  }
  *word = words[dev];
  if (dups != nullptr) *dups = tables[dev];
  return PA_OK;
}
static int violation_ptr(unsigned long long** out) { return debug_ptrs(out, nullptr); }

static int read_word(hipStream_t stream, unsigned long long* w_dev, unsigned long long* value) {
  if (hipStreamSynchronize(stream) != hipSuccess) return PA_ERR_HIP;
  if (hipMemcpy(value, w_dev, sizeof(*value), hipMemcpyDeviceToHost) != hipSuccess)
    return PA_ERR_HIP;
  return PA_OK;
}

int debug_gate(hipStream_t stream) {
  unsigned long long* w = nullptr;
  unsigned long long v = 0;
  int st = violation_ptr(&w);
  if (st == PA_OK) st = read_word(stream, w, &v);
  if (st != PA_OK) return st;
  return v != 0 ? PA_ERR_DEVICE_DATA : PA_OK;
}

int debug_take(hipStream_t stream, int32_t* code, int64_t* where) {
  unsigned long long* w = nullptr;
  unsigned long long v = 0;
  int st = violation_ptr(&w);
  if (st == PA_OK) st = read_word(stream, w, &v);
  if (st != PA_OK) return st;
  if (v != 0) {
    const unsigned long long zero = 0;
    if (hipMemcpy(w, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess)
      return PA_ERR_HIP;
  }
  *code = (int32_t)(v >> 56);
  *where = (int64_t)(v & ((1ull << 56) - 1));
  return PA_OK;
}

int validate_decode(const pa_kv_pool_t& pool, const int32_t* block_tables, int max_blocks,
                    const int32_t* ctx, int num_seqs, int max_ctx, const int64_t* slots,
                    hipStream_t stream) {
  unsigned long long* w = nullptr;
  const int st = violation_ptr(&w);
  if (st != PA_OK) return st;
  const hipError_t e = launch_kernel(validate_decode_kernel, dim3(num_seqs), dim3(64), stream,
                                     block_tables, max_blocks, ctx, max_ctx, pool.num_blocks,
                                     slots, w);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int validate_tokens(const pa_kv_pool_t& pool, const int64_t* slots, int64_t n,
                    const int64_t* positions, int64_t max_position, hipStream_t stream) {
  unsigned long long* w = nullptr;
  unsigned long long* dups = nullptr;
  const int st = debug_ptrs(&w, &dups);
  if (st != PA_OK) return st;
  if (n > kDupMaxTokens) {
    dups = nullptr;  // too many tokens for the table: the duplicate check is skipped
  } else if (launch_kernel(clear_dup_table_kernel, dim3(1024), dim3(256), stream, dups) !=
             hipSuccess) {
    return PA_ERR_HIP;
  }
  const int64_t grid = std::min<int64_t>((n + 255) / 256, 4096);
  const hipError_t e = launch_kernel(validate_tokens_kernel, dim3((unsigned)grid), dim3(256),
                                     stream, slots, n, pool.num_blocks, positions, max_position, w,
                                     dups);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int validate_varlen(const pa_kv_pool_t& pool, const PrefillArgs& a, hipStream_t stream) {
  unsigned long long* w = nullptr;
  const int st = violation_ptr(&w);
  if (st != PA_OK) return st;
  const hipError_t e = launch_kernel(validate_varlen_kernel, dim3(a.num_seqs), dim3(64), stream,
                                     a.cu_seqlens, a.num_seqs, a.total_tokens, a.max_q_len,
                                     a.block_tables, a.max_blocks_per_seq, a.context_lens,
                                     a.max_context_len, pool.num_blocks, w);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace pa
