// pa_store_kv kernels: scatter new K/V rows into the paged pool through slot_mapping.
//
// Follows the store_kvcache_kernel of the koas-w "errors and solutions" post
// ("hand-written Triton kernels": token x head grid, rows written straight to their
// physical slot, strides for non-contiguous inputs) and the per-slot append of
// PocketLLM "cpp_engine Batching Implementation (Phase 3.1)" (Step 3.4). The FP8 and
// INT8 variants add the per-token-per-head absmax quantiser (the k_scale / v_scale that
// page lists "for FP8/INT8").
//
// Layout: pool [num_blocks, 16, Hkv, D]; the row of (slot, g) starts at element
// (slot * Hkv + g) * D, because block * 16 + offset == slot.
#include "common.h"
#include "internal.h"

namespace pa {

// ---------------------------------------------------------------- copy (f32 / bf16)
// One thread moves VB bytes (16 when every row start is 16-byte aligned, else the
// element size). Work item = (k|v, token, head, chunk), grid-stride.
template <int VB, int E>
__global__ void __launch_bounds__(256) store_copy_kernel(
    char* __restrict__ kpool, char* __restrict__ vpool, const char* __restrict__ ksrc,
    const char* __restrict__ vsrc, int64_t k_st, int64_t k_sh, int64_t v_st, int64_t v_sh,
    const int64_t* __restrict__ slot_mapping, int64_t num_tokens, int hkv, int row_bytes,
    int64_t num_slots) {
  const int chunks = row_bytes / VB;
  const int64_t per_side = num_tokens * hkv * chunks;
  const int64_t total = 2 * per_side;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const bool is_v = i >= per_side;
    const int64_t r = is_v ? i - per_side : i;
    const int64_t t = r / (hkv * chunks);
    const int rem = (int)(r - t * hkv * chunks);
    const int g = rem / chunks;
    const int c = rem - g * chunks;
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_slots) continue;
    const char* src = is_v ? vsrc + (t * v_st + g * v_sh) * E : ksrc + (t * k_st + g * k_sh) * E;
    char* dst = (is_v ? vpool : kpool) + (slot * hkv + g) * (int64_t)row_bytes;
    if constexpr (VB == 16) {
      *reinterpret_cast<uint4*>(dst + c * 16) = *reinterpret_cast<const uint4*>(src + c * 16);
    } else if constexpr (VB == 4) {
      *reinterpret_cast<uint32_t*>(dst + c * 4) = *reinterpret_cast<const uint32_t*>(src + c * 4);
    } else {
      *reinterpret_cast<uint16_t*>(dst + c * 2) = *reinterpret_cast<const uint16_t*>(src + c * 2);
    }
  }
}

// ---------------------------------------------------------------- quantise + store
// 16 lanes per (k|v, token, head) row, EPL = D/16 elements per lane; 16 rows per
// 256-thread block. absmax over the row via the 16-lane butterfly, scale = a / QMAX
// (correctly rounded fp32 divide; 448 for e4m3fn, 127 for int8), codes = the pool's
// encoding of x / scale (e4m3fn: round to nearest even with saturation; int8: nearest
// integer, ties to even, clamped to [-127, 127]).
template <int SRC, int D, int Q>
__global__ void __launch_bounds__(256) store_quant_kernel(
    uint8_t* __restrict__ kpool, uint8_t* __restrict__ vpool, float* __restrict__ kscale,
    float* __restrict__ vscale, const void* __restrict__ ksrc, const void* __restrict__ vsrc,
    int64_t k_st, int64_t k_sh, int64_t v_st, int64_t v_sh,
    const int64_t* __restrict__ slot_mapping, int64_t num_tokens, int hkv, int64_t num_slots) {
  constexpr int EPL = D / 16;
  const int sub = threadIdx.x & 15;
  const int64_t rows_per_side = num_tokens * hkv;
  const int64_t total_rows = 2 * rows_per_side;
  for (int64_t row = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 4; row < total_rows;
       row += ((int64_t)gridDim.x * blockDim.x) >> 4) {
    const bool is_v = row >= rows_per_side;
    const int64_t r = is_v ? row - rows_per_side : row;
    const int64_t t = r / hkv;
    const int g = (int)(r - t * hkv);
    const int64_t slot = slot_mapping[t];
    // all 16 lanes of a row see the same slot, so the skip is row-uniform and the
    // shuffles below only ever pair lanes that are both active
    if (slot < 0 || slot >= num_slots) continue;
    float x[EPL];
    const int64_t off = is_v ? t * v_st + g * v_sh : t * k_st + g * k_sh;
    if constexpr (SRC == kBF16) {
      const uint16_t* src = (const uint16_t*)(is_v ? vsrc : ksrc) + off + sub * EPL;
#pragma unroll
      for (int e = 0; e < EPL; ++e) x[e] = bf16_to_f32(src[e]);
    } else {
      const float* src = (const float*)(is_v ? vsrc : ksrc) + off + sub * EPL;
#pragma unroll
      for (int e = 0; e < EPL; ++e) x[e] = src[e];
    }
    float a = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) a = fmaxf(a, fabsf(x[e]));
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) a = fmaxf(a, __shfl_xor(a, m, 16));
    const float scale = a / kQMax<Q>;
    uint32_t words[EPL / 4];
#pragma unroll
    for (int w = 0; w < EPL / 4; ++w) {
      uint32_t word = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        uint32_t code = 0u;
        if (a != 0.0f) {
          const float y = x[4 * w + b] / scale;
          code = Q == kFP8 ? f32_to_e4m3fn(y) : f32_to_i8sym(y);
        }
        word |= code << (8 * b);
      }
      words[w] = word;
    }
    uint8_t* dst = (is_v ? vpool : kpool) + (slot * hkv + g) * (int64_t)D + sub * EPL;
    if constexpr (EPL == 8) {
      *reinterpret_cast<uint2*>(dst) = make_uint2(words[0], words[1]);
    } else {
      *reinterpret_cast<uint32_t*>(dst) = words[0];
    }
    if (sub == 0) (is_v ? vscale : kscale)[slot * hkv + g] = (a == 0.0f) ? 0.0f : scale;
  }
}

// ---------------------------------------------------------------- whole-block copy
// Copy-on-write helper: block dst[i] of K and V (and of the scales of a quantised pool)
// becomes a copy of block src[i]. 16-byte chunks, grid-stride; pairs with an id outside
// the pool are skipped.
__global__ void __launch_bounds__(256) copy_blocks_kernel(
    char* __restrict__ kpool, char* __restrict__ vpool, float* __restrict__ kscale,
    float* __restrict__ vscale, const int32_t* __restrict__ src, const int32_t* __restrict__ dst,
    int n, int64_t num_blocks, int64_t block_bytes, int scales_per_block) {
  const int64_t chunks = block_bytes / 16;
  const int64_t per_pair = 2 * chunks + 2 * scales_per_block;
  const int64_t total = (int64_t)n * per_pair;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int pair = (int)(i / per_pair);
    int64_t r = i - (int64_t)pair * per_pair;
    const int64_t sb = src[pair], db = dst[pair];
    if (sb < 0 || sb >= num_blocks || db < 0 || db >= num_blocks) continue;
    if (r < 2 * chunks) {
      char* pool = r < chunks ? kpool : vpool;
      const int64_t c = r < chunks ? r : r - chunks;
      *reinterpret_cast<uint4*>(pool + db * block_bytes + c * 16) =
          *reinterpret_cast<const uint4*>(pool + sb * block_bytes + c * 16);
    } else {
      r -= 2 * chunks;
      float* sc = r < scales_per_block ? kscale : vscale;
      const int64_t e = r < scales_per_block ? r : r - scales_per_block;
      sc[db * scales_per_block + e] = sc[sb * scales_per_block + e];
    }
  }
}

static int grid_for(int64_t work_items, int per_block) {
  int64_t blocks = (work_items + per_block - 1) / per_block;
  const int64_t cap = 256 * 64;  // 64 blocks per CU is plenty for a grid-stride loop
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  return (int)blocks;
}

int launch_store(const pa_kv_pool_t& pool, const void* k, const void* v, int src_dtype,
                 int64_t num_tokens, int64_t k_st, int64_t k_sh, int64_t v_st, int64_t v_sh,
                 const int64_t* slot_mapping, hipStream_t stream) {
  const int64_t num_slots = pool.num_blocks * pool.block_size;
  const int hkv = pool.kv_heads, D = pool.head_dim;
  if (pool.dtype == PA_FP8_E4M3 || pool.dtype == PA_INT8) {
    const int grid = grid_for(2 * num_tokens * hkv * 16, 256);
    hipError_t e = hipSuccess;
#define PA_QUANT_STORE(SRC, DD, Q)                                                          \
  e = launch_kernel(store_quant_kernel<SRC, DD, Q>, dim3(grid), dim3(256), stream,         \
                    (uint8_t*)pool.k, (uint8_t*)pool.v, pool.k_scale, pool.v_scale, k, v,  \
                    k_st, k_sh, v_st, v_sh, slot_mapping, num_tokens, hkv, num_slots)
#define PA_QUANT_STORE_Q(Q)                                                                 \
    if (src_dtype == PA_BF16 && D == 128) PA_QUANT_STORE(kBF16, 128, Q);                    \
    else if (src_dtype == PA_BF16 && D == 64) PA_QUANT_STORE(kBF16, 64, Q);                 \
    else if (src_dtype == PA_F32 && D == 128) PA_QUANT_STORE(kF32, 128, Q);                 \
    else if (src_dtype == PA_F32 && D == 64) PA_QUANT_STORE(kF32, 64, Q);                   \
    else return PA_ERR_UNSUPPORTED;
    if (pool.dtype == PA_FP8_E4M3) {
      PA_QUANT_STORE_Q(kFP8)
    } else {
      PA_QUANT_STORE_Q(kINT8)
    }
#undef PA_QUANT_STORE_Q
#undef PA_QUANT_STORE
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
  }
  const int E = pool.dtype == PA_F32 ? 4 : 2;
  const int row_bytes = D * E;
  auto al16 = [](const void* p) { return ((uintptr_t)p & 15u) == 0; };
  const bool vec16 = al16(k) && al16(v) && al16(pool.k) && al16(pool.v) &&
                     ((k_st * E) % 16 == 0) && ((k_sh * E) % 16 == 0) &&
                     ((v_st * E) % 16 == 0) && ((v_sh * E) % 16 == 0);
  auto copy = [&](auto kernel, int grid) {
    return launch_kernel(kernel, dim3(grid), dim3(256), stream, (char*)pool.k, (char*)pool.v,
                         (const char*)k, (const char*)v, k_st, k_sh, v_st, v_sh, slot_mapping,
                         num_tokens, hkv, row_bytes, num_slots);
  };
  hipError_t e;
  if (vec16) {
    const int grid = grid_for(2 * num_tokens * hkv * (row_bytes / 16), 256);
    e = E == 4 ? copy(store_copy_kernel<16, 4>, grid) : copy(store_copy_kernel<16, 2>, grid);
  } else {
    const int grid = grid_for(2 * num_tokens * hkv * (row_bytes / E), 256);
    e = E == 4 ? copy(store_copy_kernel<4, 4>, grid) : copy(store_copy_kernel<2, 2>, grid);
  }
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int launch_copy_blocks(const pa_kv_pool_t& pool, const int32_t* src, const int32_t* dst, int n,
                       hipStream_t stream) {
  const int E = pool.dtype == PA_F32 ? 4 : (pool.dtype == PA_BF16 ? 2 : 1);
  const int64_t block_bytes = (int64_t)pool.block_size * pool.kv_heads * pool.head_dim * E;
  const bool quant = pool.dtype == PA_FP8_E4M3 || pool.dtype == PA_INT8;
  const int spb = quant ? pool.block_size * pool.kv_heads : 0;
  const int grid = grid_for((int64_t)n * (2 * block_bytes / 16 + 2 * spb), 256);
  const hipError_t e = launch_kernel(copy_blocks_kernel, dim3(grid), dim3(256), stream,
                                     (char*)pool.k, (char*)pool.v, pool.k_scale, pool.v_scale,
                                     src, dst, n, pool.num_blocks, block_bytes, spb);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace pa
