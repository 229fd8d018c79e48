// pa_varlen_prefill kernel: causal attention for a flat batch of query chunks on top
// of their cached prefixes, read from the paged pool through block_tables.
//
// Semantics from the mini-vllm tutorial "step14_7 - Batched Forward" (tokens of all
// sequences concatenated, cu_seqlens marks the boundaries, attention is the only op
// that needs them, a chunk attends its cached prefix plus itself causally from its
// start position; one varlen kernel reading the paged pool replaces the per-sequence
// loop, "comparison with vLLM").
//
// Tiling (gfx950, v_mfma_f32_32x32x16_bf16, wave64):
//  * A workgroup owns 128 flattened query rows of one (sequence, KV head): row
//    m = i*G + hh is token i of the chunk and query head g*G + hh, so the G heads
//    that share a KV head share every K/V tile (read once per tile, not G times).
//    Each of the 4 waves owns 32 rows.
//  * Keys advance 64 at a time (four 16-token pool blocks gathered into LDS).
//  * S^T = K Q^T: A = K rows from LDS, B = the wave's Q rows held in registers, so
//    the accumulator gives every lane one query row (lane % 32) and 16 keys per
//    32-key tile; softmax statistics are lane-local plus one exchange with lane^32.
//  * O^T = V^T P^T: A = V^T from LDS, B = P straight from the S^T accumulator
//    (rounded to bf16). V is written to LDS transposed, with keys stored in the order
//    the accumulator holds them (bits 2 and 3 of the key index swapped within each
//    group of 16), so each A operand is one 16-byte LDS read.
//  * The causal mask is applied only on tiles that reach past the wave's first row.
//    Keys past the context are zero-filled in LDS (never multiplied in as garbage).
#include "common.h"
#include "internal.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kPfRows = 128;   // flattened rows per workgroup
constexpr int kPfKeys = 64;    // keys per iteration
constexpr int kKPad = 8;       // bf16 elements of padding per K row in LDS
constexpr int kVPad = 8;       // bf16 elements of padding per V^T row in LDS

__device__ __forceinline__ int vt_pos(int k) {
  // swap bits 2 and 3 of the key index (bits 0-1 and >= 4 unchanged)
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

template <int D, int G>
__global__ void __launch_bounds__(256) prefill_kernel(
    const uint16_t* __restrict__ kpool, const uint16_t* __restrict__ vpool, int64_t num_blocks,
    int hkv, uint16_t* __restrict__ out, int64_t out_st, int64_t out_sh,
    const uint16_t* __restrict__ q, int64_t q_st, int64_t q_sh,
    const int32_t* __restrict__ cu_seqlens, int64_t total_tokens, int tiles_per_seq,
    const int32_t* __restrict__ block_tables, int max_blocks_per_seq,
    const int32_t* __restrict__ context_lens, int max_context_len, float scale_log2) {
  constexpr int KROW = D + kKPad;             // LDS K row stride (elements)
  constexpr int VROW = kPfKeys + kVPad;       // LDS V^T row stride (elements)
  constexpr int CH = D / 8;                   // 16-byte chunks per K/V row
  constexpr int DSTEPS = D / 16;              // k-steps of the QK^T MFMA
  constexpr int DT = D / 32;                  // 32-wide d tiles of O^T
  constexpr float NEG_INF = -__builtin_huge_valf();
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kPfKeys * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VROW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hl = lane >> 5;     // which half of the wave (k-slot group of the MFMA)
  const int l32 = lane & 31;

  // blockIdx.x -> (tile, kv head, sequence); the last (longest) tiles of a chunk first
  const int mt = tiles_per_seq - 1 - (int)(blockIdx.x % tiles_per_seq);
  const int rest = blockIdx.x / tiles_per_seq;
  const int g = rest % hkv;
  const int s = rest / hkv;
  const int t_begin = cu_seqlens[s];
  const int t_end = cu_seqlens[s + 1];
  // chunks outside [0, total_tokens] break the cu_seqlens contract: skip them rather
  // than read or write outside q / out
  if (t_begin < 0 || t_end > total_tokens) return;
  const int n = t_end - t_begin;
  const int nrows = n * G;
  const int m0 = mt * kPfRows;
  if (m0 >= nrows) return;  // whole workgroup: no barrier reached yet
  // clamp to the host bound (<= max_blocks_per_seq * 16) so table reads stay in the row
  const int L = min(context_lens[s], max_context_len);
  const int P = L - n;
  const int m_last = min(m0 + kPfRows, nrows) - 1;
  const int kend = P + m_last / G + 1;  // keys [0, kend) are visible to some row here

  // ---- this wave's rows
  const int mw0 = m0 + 32 * wave;
  const bool wave_active = mw0 < nrows;
  const int my_m = mw0 + l32;
  const bool row_ok = my_m < nrows;
  const int my_tok = row_ok ? my_m / G : 0;
  const int my_hh = row_ok ? my_m % G : 0;
  const int my_limit = row_ok ? P + my_tok : -1;  // last visible key of this row
  const int wave_first_limit = P + mw0 / G;       // smallest limit among the wave's rows
  const int wave_last_limit = P + (min(mw0 + 31, nrows - 1)) / G;

  // ---- Q rows as the B operand: lane holds Q[row][16*st + 8*hl .. +8]
  bf16x8_t qreg[DSTEPS];
  {
    const uint16_t* qp = q + (int64_t)(t_begin + my_tok) * q_st + (int64_t)(g * G + my_hh) * q_sh;
#pragma unroll
    for (int st = 0; st < DSTEPS; ++st) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = 16 * st + 8 * hl + 2 * e;
        w[e] = row_ok ? ((uint32_t)qp[d] | ((uint32_t)qp[d + 1] << 16)) : 0u;
      }
      qreg[st] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
    }
  }

  f32x16_t oacc[DT];
#pragma unroll
  for (int dn = 0; dn < DT; ++dn)
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[dn][j] = 0.0f;
  float m_run = NEG_INF, l_run = 0.0f;

  const int32_t* bt_row = block_tables + (int64_t)s * max_blocks_per_seq;
  const int64_t tok_stride = (int64_t)hkv * D;  // elements between consecutive slots

  const int ntiles = (kend + kPfKeys - 1) / kPfKeys;
  for (int kt = 0; kt < ntiles; ++kt) {
    const int kbase = kt * kPfKeys;
    __syncthreads();
    // ---- gather K tile: row-major [key][d], 16 bytes per thread per step
#pragma unroll
    for (int it = 0; it < (kPfKeys * CH) / 256; ++it) {
      const int w = tid + 256 * it;
      const int key = w / CH, ch = w % CH;
      const int ka = kbase + key;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (ka < L) {
        const int bid = bt_row[ka >> 4];
        if ((unsigned)bid < (uint64_t)num_blocks) {
          const int64_t off = ((int64_t)bid * kBlockSize + (ka & 15)) * tok_stride + (int64_t)g * D + ch * 8;
          x = *reinterpret_cast<const uint4*>(kpool + off);
        }
      }
      *reinterpret_cast<uint4*>(&Ks[key * KROW + ch * 8]) = x;
    }
    // ---- gather V tile: four consecutive keys x 8 dims per thread, written transposed
    for (int w = tid; w < 16 * CH; w += 256) {
      const int kq = w / CH, ch = w % CH;
      uint4 rows[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ka = kbase + 4 * kq + r;
        rows[r] = make_uint4(0, 0, 0, 0);
        if (ka < L) {
          const int bid = bt_row[ka >> 4];
          if ((unsigned)bid < (uint64_t)num_blocks) {
            const int64_t off = ((int64_t)bid * kBlockSize + (ka & 15)) * tok_stride + (int64_t)g * D + ch * 8;
            rows[r] = *reinterpret_cast<const uint4*>(vpool + off);
          }
        }
      }
      const int pos = vt_pos(4 * kq);
      const uint32_t* r0 = &rows[0].x;
      const uint32_t* r1 = &rows[1].x;
      const uint32_t* r2 = &rows[2].x;
      const uint32_t* r3 = &rows[3].x;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint2 lo = make_uint2(__builtin_amdgcn_perm(r1[e], r0[e], 0x05040100u),
                                    __builtin_amdgcn_perm(r3[e], r2[e], 0x05040100u));
        const uint2 hi = make_uint2(__builtin_amdgcn_perm(r1[e], r0[e], 0x07060302u),
                                    __builtin_amdgcn_perm(r3[e], r2[e], 0x07060302u));
        *reinterpret_cast<uint2*>(&Vt[(ch * 8 + 2 * e) * VROW + pos]) = lo;
        *reinterpret_cast<uint2*>(&Vt[(ch * 8 + 2 * e + 1) * VROW + pos]) = hi;
      }
    }
    __syncthreads();
    if (!wave_active || kbase > wave_last_limit) continue;

    // ---- S^T = K Q^T for keys kbase + [0, 32) and + [32, 64)
    f32x16_t sacc[2];
#pragma unroll
    for (int nn = 0; nn < 2; ++nn) {
#pragma unroll
      for (int j = 0; j < 16; ++j) sacc[nn][j] = 0.0f;
#pragma unroll
      for (int st = 0; st < DSTEPS; ++st) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&Ks[(32 * nn + l32) * KROW + 16 * st + 8 * hl]);
        sacc[nn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[st], sacc[nn], 0, 0, 0);
      }
    }
    // ---- online softmax; lane holds keys kbase + 32nn + 8(j/4) + 4hl + j%4 of its row
    const bool need_mask = kbase + kPfKeys - 1 > wave_first_limit;
    float tmax = NEG_INF;
#pragma unroll
    for (int nn = 0; nn < 2; ++nn)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float x = sacc[nn][j] * scale_log2;
        if (need_mask) {
          const int key = kbase + 32 * nn + 8 * (j >> 2) + 4 * hl + (j & 3);
          x = key <= my_limit ? x : NEG_INF;
        }
        sacc[nn][j] = x;
        tmax = fmaxf(tmax, x);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    // rows past the chunk (my_limit = -1) see no key at all: keep them at zero
    const float m_use = m_new == NEG_INF ? 0.0f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float psum = 0.0f;
    bf16x8_t pb[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float pv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pv[i] = fast_exp2(sacc[t >> 1][8 * (t & 1) + i] - m_use);
        psum += pv[i];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[t][i] = (__bf16)pv[i];
    }
    l_run = fmaf(l_run, alpha, psum);
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
      for (int dn = 0; dn < DT; ++dn)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[dn][j] *= alpha;
    }
    // ---- O^T += V^T P^T
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int dn = 0; dn < DT; ++dn) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&Vt[(32 * dn + l32) * VROW + 16 * t + 8 * hl]);
        oacc[dn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[t], oacc[dn], 0, 0, 0);
      }
  }

  if (!row_ok) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  uint16_t* op = out + (int64_t)(t_begin + my_tok) * out_st + (int64_t)(g * G + my_hh) * out_sh;
#pragma unroll
  for (int dn = 0; dn < DT; ++dn)
#pragma unroll
    for (int jq = 0; jq < 4; ++jq) {
      const int d = 32 * dn + 8 * jq + 4 * hl;
      const uint32_t w0 = (uint32_t)f32_to_bf16(oacc[dn][4 * jq] * inv) |
                          ((uint32_t)f32_to_bf16(oacc[dn][4 * jq + 1] * inv) << 16);
      const uint32_t w1 = (uint32_t)f32_to_bf16(oacc[dn][4 * jq + 2] * inv) |
                          ((uint32_t)f32_to_bf16(oacc[dn][4 * jq + 3] * inv) << 16);
      op[d] = (uint16_t)w0;
      op[d + 1] = (uint16_t)(w0 >> 16);
      op[d + 2] = (uint16_t)w1;
      op[d + 3] = (uint16_t)(w1 >> 16);
    }
}

template <int D, int G>
static void launch_prefill_t(const pa_kv_pool_t& pool, const PrefillArgs& a, hipStream_t stream) {
  const int tiles = (int)(((int64_t)a.max_q_len * G + kPfRows - 1) / kPfRows);
  const int64_t grid = (int64_t)tiles * pool.kv_heads * a.num_seqs;
  prefill_kernel<D, G><<<(unsigned)grid, 256, 0, stream>>>(
      (const uint16_t*)pool.k, (const uint16_t*)pool.v, pool.num_blocks, pool.kv_heads,
      (uint16_t*)a.out, a.out_st, a.out_sh, (const uint16_t*)a.q, a.q_st, a.q_sh, a.cu_seqlens,
      a.total_tokens, tiles, a.block_tables, a.max_blocks_per_seq, a.context_lens,
      a.max_context_len, a.scale * kLog2e);
}

template <int D>
static int dispatch_pf_g(const pa_kv_pool_t& pool, const PrefillArgs& a, hipStream_t stream) {
  switch (a.q_heads / pool.kv_heads) {
    case 1: launch_prefill_t<D, 1>(pool, a, stream); return PA_OK;
    case 2: launch_prefill_t<D, 2>(pool, a, stream); return PA_OK;
    case 3: launch_prefill_t<D, 3>(pool, a, stream); return PA_OK;
    case 4: launch_prefill_t<D, 4>(pool, a, stream); return PA_OK;
    case 5: launch_prefill_t<D, 5>(pool, a, stream); return PA_OK;
    case 6: launch_prefill_t<D, 6>(pool, a, stream); return PA_OK;
    case 7: launch_prefill_t<D, 7>(pool, a, stream); return PA_OK;
    case 8: launch_prefill_t<D, 8>(pool, a, stream); return PA_OK;
    default: return PA_ERR_UNSUPPORTED;
  }
}

int launch_prefill(const pa_kv_pool_t& pool, const PrefillArgs& a, hipStream_t stream) {
  if (pool.dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  return pool.head_dim == 64 ? dispatch_pf_g<64>(pool, a, stream)
                             : dispatch_pf_g<128>(pool, a, stream);
}

}  // namespace pa
