// pa_rope_store_kv kernel: rotary position embedding of the new tokens' q and k, fused
// with the paged KV store of the rotated k and of v.
//
// Follows the fused RoPE + KV-cache store kernel of the koas-w "errors and solutions"
// post ("hand-written Triton kernels": q is rotated in registers and written back to a
// contiguous buffer, k and v go straight to their scattered cache slots through
// slot_mapping, no intermediate buffer) with the table-driven real-valued RoPE the post
// settles on, numerically aligned with the HuggingFace model: the pair (i, i + D/2) of a
// head is rotated by the angle whose cosine and sine are table[position][i].
//
// One row (token, head) of q, k or v per 16 lanes; lane l holds head dims
// [l*D/16, (l+1)*D/16) and reads its partner dims (d +- D/2, held by lane l^8) straight
// from memory. The rotation is done in fp32 with every product and every sum rounded on
// its own (no fused multiply-add), so its bits are fixed by the definition.
#include "common.h"
#include "internal.h"

namespace pa {

template <int SRC>
__device__ __forceinline__ float ld_src(const void* p, int64_t i) {
  if constexpr (SRC == kBF16) return bf16_to_f32(((const uint16_t*)p)[i]);
  else return ((const float*)p)[i];
}

// out = x * c - y * s (lower half) or x * c + y * s (upper half), each op rounded.
__device__ __forceinline__ float rot(float x, float y, float c, float s, bool upper) {
#pragma clang fp contract(off)
  const float xc = x * c;
  const float ys = y * s;
  return upper ? xc + ys : xc - ys;
}

template <int SRC, int D, int PT>
__global__ void __launch_bounds__(256) rope_store_kernel(RopeArgs a) {
  constexpr int EPL = D / 16;
  constexpr int HALF = D / 2;
  const int sub = threadIdx.x & 15;
  const bool upper = sub >= 8;
  const int d0 = sub * EPL;                 // this lane's first head dim
  const int dp = upper ? d0 - HALF : d0 + HALF;  // its partner dims
  const int dt = upper ? d0 - HALF : d0;    // table column
  const int rows_per_tok = a.q_heads + 2 * a.hkv;
  const int64_t total_rows = a.num_tokens * rows_per_tok;
  const int64_t num_slots = a.num_blocks * kBlockSize;
  for (int64_t row = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 4; row < total_rows;
       row += ((int64_t)gridDim.x * blockDim.x) >> 4) {
    const int64_t t = row / rows_per_tok;
    const int hr = (int)(row - t * rows_per_tok);
    const bool is_q = hr < a.q_heads;
    const bool is_k = !is_q && hr < a.q_heads + a.hkv;
    const int g = is_q ? hr : (is_k ? hr - a.q_heads : hr - a.q_heads - a.hkv);
    const int64_t slot = is_q ? 0 : a.slots[t];
    // row-uniform skip (all 16 lanes of a row share t), so the shuffles below only
    // pair lanes that are both active
    if (!is_q && (slot < 0 || slot >= num_slots)) continue;
    const void* src = is_q ? a.q : (is_k ? a.k : a.v);
    const int64_t off = is_q ? t * a.q_st + (int64_t)g * a.q_sh
                             : (is_k ? t * a.k_st + (int64_t)g * a.k_sh
                                     : t * a.v_st + (int64_t)g * a.v_sh);
    float x[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) x[e] = ld_src<SRC>(src, off + d0 + e);
    if (is_q || is_k) {
      // table row of this token's position (clamped: an out-of-range position is a
      // contract violation whose row is unspecified, never an out-of-bounds read)
      int64_t p = a.positions[t];
      p = p < 0 ? 0 : (p >= a.max_position ? a.max_position - 1 : p);
      const float* cs = a.cos_table + p * HALF + dt;
      const float* sn = a.sin_table + p * HALF + dt;
      float y[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) y[e] = ld_src<SRC>(src, off + dp + e);
#pragma unroll
      for (int e = 0; e < EPL; ++e) x[e] = rot(x[e], y[e], cs[e], sn[e], upper);
    }
    if (is_q) {
      const int64_t o = t * a.qo_st + (int64_t)g * a.qo_sh + d0;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        if constexpr (SRC == kBF16) ((uint16_t*)a.q_out)[o + e] = f32_to_bf16(x[e]);
        else ((float*)a.q_out)[o + e] = x[e];
      }
      continue;
    }
    char* pool = (char*)(is_k ? a.kpool : a.vpool);
    const int64_t prow = slot * a.hkv + g;  // (block * 16 + offset) * Hkv + g
    if constexpr (kQuant<PT>) {
      float amax = 0.0f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) amax = fmaxf(amax, fabsf(x[e]));
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 16));
      const float scale = amax / kQMax<PT>;
      uint8_t* dst = (uint8_t*)pool + prow * D + d0;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        uint32_t code = 0u;
        if (amax != 0.0f) {
          const float yq = x[e] / scale;
          code = PT == kFP8 ? f32_to_e4m3fn(yq) : f32_to_i8sym(yq);
        }
        dst[e] = (uint8_t)code;
      }
      if (sub == 0) (is_k ? a.kscale : a.vscale)[prow] = amax == 0.0f ? 0.0f : scale;
    } else if constexpr (PT == kBF16) {
      uint16_t* dst = (uint16_t*)pool + prow * D + d0;
#pragma unroll
      for (int e = 0; e < EPL; ++e) dst[e] = f32_to_bf16(x[e]);
    } else {
      float* dst = (float*)pool + prow * D + d0;
#pragma unroll
      for (int e = 0; e < EPL; ++e) dst[e] = x[e];
    }
  }
}

int launch_rope_store(const pa_kv_pool_t& pool, const RopeArgs& a, int src_dtype,
                      hipStream_t stream) {
  const int64_t rows = a.num_tokens * (a.q_heads + 2 * a.hkv);
  int64_t grid = (rows * 16 + 255) / 256;
  grid = grid < 1 ? 1 : (grid > 256 * 64 ? 256 * 64 : grid);
  const int D = pool.head_dim;
  hipError_t e = hipSuccess;
#define PA_ROPE(S, DD, P) \
  e = launch_kernel(rope_store_kernel<S, DD, P>, dim3((unsigned)grid), dim3(256), stream, a)
#define PA_ROPE_P(S, DD)                                                   \
  switch (pool.dtype) {                                                    \
    case PA_F32: PA_ROPE(S, DD, kF32); break;                              \
    case PA_BF16: PA_ROPE(S, DD, kBF16); break;                            \
    case PA_FP8_E4M3: PA_ROPE(S, DD, kFP8); break;                         \
    case PA_INT8: PA_ROPE(S, DD, kINT8); break;                            \
    default: return PA_ERR_UNSUPPORTED;                                    \
  }
  if (src_dtype == PA_BF16) {
    if (D == 128) { PA_ROPE_P(kBF16, 128) } else { PA_ROPE_P(kBF16, 64) }
  } else {
    if (D == 128) { PA_ROPE_P(kF32, 128) } else { PA_ROPE_P(kF32, 64) }
  }
#undef PA_ROPE_P
#undef PA_ROPE
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace pa
