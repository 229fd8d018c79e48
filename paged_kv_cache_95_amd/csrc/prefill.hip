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
//  * Long key ranges are split into chunks of split_keys keys handled by separate
//    workgroups (the critical path is otherwise the row tile with the longest prefix);
//    split tiles write (o, lse) partials and a small kernel merges them by
//    log-sum-exp. The next 64-key tile is fetched into registers while the current
//    one is multiplied.
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kPfRows = 128;   // flattened rows per workgroup
constexpr int kPfKeys = 64;    // keys per iteration
constexpr int kKPad = 8;       // bf16 elements of padding per K row in LDS
constexpr int kVPad = 8;       // bf16 elements of padding per V^T row in LDS
constexpr int kPfORow = 36;    // fp32 LDS row stride of the partial store staging (32 + 4)
constexpr float kPfLazyMax = 8.0f;  // log2 headroom of the lazily updated row max

__device__ __forceinline__ int vt_pos(int k) {
  // swap bits 2 and 3 of the key index (bits 0-1 and >= 4 unchanged)
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

struct PfArgs {
  const uint16_t* kpool;
  const uint16_t* vpool;
  int64_t num_blocks;
  int hkv;
  uint16_t* out;
  int64_t out_st, out_sh;
  const uint16_t* q;
  int64_t q_st, q_sh;
  const int32_t* cu_seqlens;
  int num_seqs;
  int64_t total_tokens;
  int tiles_per_seq;
  const int32_t* block_tables;
  int max_blocks_per_seq;
  const int32_t* context_lens;
  int max_context_len;
  float scale_log2;
  bool q_aligned;    // q rows start on 16 bytes
  bool out_aligned;  // out rows start on 8 bytes
  int q_heads;
  int split_keys;    // keys per work item (multiple of 64)
  int max_chunks;    // ceil(max_context_len / split_keys)
  char* plan;        // work list (header, then entries)
  int64_t plan_bound;
  float* ws_o;       // [total_tokens, q_heads, max_chunks, D] partials (max_chunks > 1)
  float* ws_lse;     // [total_tokens, q_heads, max_chunks]
};

// Work list written by prefill_plan_kernel at the start of the workspace: the number of
// entries, then the entries, costliest first. An entry is one (sequence, row tile, key
// chunk) with work; it stands for kv_heads work items (one per KV head).
struct PfPlanHeader {
  int32_t entries;
};
struct PfEntry {
  int32_t s, mt, chunk, t_begin;  // sequence, row tile, key chunk, first token
  int32_t n, L, cost, pad;        // chunk length, clamped context length, 64-key tiles
};
static_assert(sizeof(PfEntry) == kPfPlanEntryBytes, "entry size");
static_assert(sizeof(PfPlanHeader) <= kPfPlanHeaderBytes, "header size");

// x[i] for i in 0..3 as selects (a run-time index into a register array would put
// the array in scratch memory).
__device__ __forceinline__ int pick4(const int (&x)[4], int i) {
  return i == 0 ? x[0] : (i == 1 ? x[1] : (i == 2 ? x[2] : x[3]));
}

// One work item: 128 flattened query rows of (sequence, KV head g) against one key chunk.
// Called by every thread of the workgroup with the same arguments (its barriers are
// uniform); Ks / Vt are the workgroup's LDS tiles.
template <int D, int G>
__device__ __forceinline__ void prefill_item(const PfArgs& a, uint16_t* __restrict__ Ks,
                                             uint16_t* __restrict__ Vt, float* __restrict__ Os,
                                             const PfEntry& e, int g) {
  const uint16_t* __restrict__ kpool = a.kpool;
  const uint16_t* __restrict__ vpool = a.vpool;
  const int64_t num_blocks = a.num_blocks;
  const int hkv = a.hkv;
  const uint16_t* __restrict__ q = a.q;
  const int64_t q_st = a.q_st, q_sh = a.q_sh;
  const bool q_aligned = a.q_aligned, out_aligned = a.out_aligned;
  constexpr int KROW = D + kKPad;             // LDS K row stride (elements)
  constexpr int VROW = kPfKeys + kVPad;       // LDS V^T row stride (elements)
  constexpr int CH = D / 8;                   // 16-byte chunks per K/V row
  constexpr int DSTEPS = D / 16;              // k-steps of the QK^T MFMA
  constexpr int DT = D / 32;                  // 32-wide d tiles of O^T
  constexpr float NEG_INF = -__builtin_huge_valf();

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hl = lane >> 5;     // which half of the wave (k-slot group of the MFMA)
  const int l32 = lane & 31;

  // the plan only lists row tiles with rows and key chunks with keys
  const int s = e.s, mt = e.mt, chunk = e.chunk, t_begin = e.t_begin, n = e.n, L = e.L;
  const int nrows = n * G;
  const int m0 = mt * kPfRows;
  const int P = L - n;
  const int m_last = min(m0 + kPfRows, nrows) - 1;
  const int kend = P + m_last / G + 1;  // keys [0, kend) are visible to some row here
  // this work item's key range [k_lo, k_hi)
  const int nchunks = (kend + a.split_keys - 1) / a.split_keys;
  const int k_lo = chunk * a.split_keys;
  const int k_hi = min(kend, k_lo + a.split_keys);

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
      const int d0 = 16 * st + 8 * hl;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (row_ok && q_aligned) {
        x = *reinterpret_cast<const uint4*>(qp + d0);
      } else if (row_ok) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          w[e] = (uint32_t)qp[d0 + 2 * e] | ((uint32_t)qp[d0 + 2 * e + 1] << 16);
        x = make_uint4(w[0], w[1], w[2], w[3]);
      }
      qreg[st] = __builtin_bit_cast(bf16x8_t, x);
    }
  }

  f32x16_t oacc[DT];
#pragma unroll
  for (int dn = 0; dn < DT; ++dn)
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[dn][j] = 0.0f;
  float m_run = NEG_INF, l_run = 0.0f;

  const int32_t* bt_row = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  const int64_t tok_stride = (int64_t)hkv * D;  // elements between consecutive slots

  // K tile: row-major [key][d], 16 bytes per thread per step. V tile: four consecutive
  // keys x 8 dims per thread (written transposed). The next tile is fetched into
  // registers while the current one is computed, then stashed into LDS.
  constexpr int KIT = (kPfKeys * CH) / 256;   // K chunks per thread
  // V work items: 16 key quads x CH chunks, key quad fastest, so that one wave's
  // transposed LDS writes spread over the banks (chunk-fastest would put 8 lanes on
  // the same bank offset)
  const bool v_has = tid < 16 * CH;
  const int v_kq = tid & 15, v_ch = tid >> 4;
  uint4 kreg[KIT];
  uint4 vreg[4];
  // The 64 keys of tile kt are pool blocks kt*4 .. kt*4+3 of the sequence: four block
  // ids, the same for every thread, read as uniform (scalar) loads one tile ahead.
  // The 64 keys of tile kt are pool blocks kt*4 .. kt*4+3 of the sequence. Their ids
  // are read with vector loads (every lane reads the same address) two tiles ahead of
  // the fetch that uses them, so the table read never stalls a tile, and are moved to
  // scalar registers when used: the K addresses are then a scalar block base plus a
  // loop-invariant 32-bit lane offset.
  auto load_bids = [&](int kt, int (&raw)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kb = kt * 4 + i;
      raw[i] = kb * kBlockSize < L ? bt_row[kb] : -1;
    }
  };
  auto to_sgpr = [&](const int (&raw)[4], int (&bids)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = __builtin_amdgcn_readfirstlane(raw[i]);
      bids[i] = (unsigned)r < (uint64_t)num_blocks ? r : -1;
    }
  };
  const int64_t blk_stride = (int64_t)kBlockSize * tok_stride;  // elements per pool block
  // byte offsets, so that base + offset is a scalar base plus a zero-extended 32-bit
  // lane offset (the global load's scalar-base addressing)
  uint32_t koff[KIT];
#pragma unroll
  for (int it = 0; it < KIT; ++it) {
    const int w = tid + 256 * it;
    koff[it] = (uint32_t)(((w / CH) & 15) * tok_stride + g * D + (w % CH) * 8) * 2u;
  }
  const uint32_t voff = (uint32_t)(((4 * v_kq) & 15) * tok_stride + g * D + v_ch * 8);
  auto fetch = [&](int kt, const int (&bids)[4]) {
    const int kbase = kt * kPfKeys;
    // a tile fully inside the context with valid block ids (the common case) needs no
    // per-element guards
    const bool full = kbase + kPfKeys <= L && bids[0] >= 0 && bids[1] >= 0 &&
                      bids[2] >= 0 && bids[3] >= 0;
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
      const int key = (tid + 256 * it) / CH;
      // the block of K item `it` is the same for the whole wave
      const int blk = __builtin_amdgcn_readfirstlane(key >> 4);
      const int bid = pick4(bids, blk);
      const char* base = reinterpret_cast<const char*>(kpool + (int64_t)max(bid, 0) * blk_stride);
      if (full) {
        kreg[it] = *reinterpret_cast<const uint4*>(base + koff[it]);
      } else {
        kreg[it] = make_uint4(0, 0, 0, 0);
        if (kbase + key < L && bid >= 0) kreg[it] = *reinterpret_cast<const uint4*>(base + koff[it]);
      }
    }
    const int vbid = pick4(bids, v_kq >> 2);
    const uint16_t* vbase = vpool + (int64_t)max(vbid, 0) * blk_stride + voff;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ka = kbase + 4 * v_kq + r;
      if (full) {
        vreg[r] = v_has ? *reinterpret_cast<const uint4*>(vbase + r * tok_stride) : make_uint4(0, 0, 0, 0);
      } else {
        vreg[r] = make_uint4(0, 0, 0, 0);
        if (v_has && ka < L && vbid >= 0) vreg[r] = *reinterpret_cast<const uint4*>(vbase + r * tok_stride);
      }
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
      const int w = tid + 256 * it;
      const int key = w / CH, ch = w % CH;
      *reinterpret_cast<uint4*>(&Ks[key * KROW + ch * 8]) = kreg[it];
    }
    if (v_has) {
      const int pos = vt_pos(4 * v_kq);
      const uint32_t* r0 = &vreg[0].x;
      const uint32_t* r1 = &vreg[1].x;
      const uint32_t* r2 = &vreg[2].x;
      const uint32_t* r3 = &vreg[3].x;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint2 lo = make_uint2(__builtin_amdgcn_perm(r1[e], r0[e], 0x05040100u),
                                    __builtin_amdgcn_perm(r3[e], r2[e], 0x05040100u));
        const uint2 hi = make_uint2(__builtin_amdgcn_perm(r1[e], r0[e], 0x07060302u),
                                    __builtin_amdgcn_perm(r3[e], r2[e], 0x07060302u));
        *reinterpret_cast<uint2*>(&Vt[(v_ch * 8 + 2 * e) * VROW + pos]) = lo;
        *reinterpret_cast<uint2*>(&Vt[(v_ch * 8 + 2 * e + 1) * VROW + pos]) = hi;
      }
    }
  };

  const int kt0 = k_lo / kPfKeys;
  const int ntiles = (k_hi + kPfKeys - 1) / kPfKeys;
  const bf2 kOnesBf2 = {(__bf16)1.0f, (__bf16)1.0f};
  int raw_next[4];  // block ids of tile kt + 1, loaded during tile kt - 1
  if (kt0 < ntiles) {
    int raw0[4], b0[4];
    load_bids(kt0, raw0);
    to_sgpr(raw0, b0);
    fetch(kt0, b0);
    if (kt0 + 1 < ntiles) load_bids(kt0 + 1, raw_next);
  }
  for (int kt = kt0; kt < ntiles; ++kt) {
    const int kbase = kt * kPfKeys;
    __syncthreads();  // every wave is done reading the previous tile
    stash();
    __syncthreads();
    if (kt + 1 < ntiles) {
      int bn[4];
      to_sgpr(raw_next, bn);
      fetch(kt + 1, bn);
      if (kt + 2 < ntiles) load_bids(kt + 2, raw_next);
    }
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
    // raw scores: the (positive) scale is applied once, fused into the exponent
    if (need_mask) {
      // only the tiles that reach past the wave's first row (a uniform branch, so the
      // compares are not paid on the other tiles): key index relative to this lane's
      // limit, against the accumulator's compile-time key offsets
      const int lim = my_limit - kbase - 4 * hl;
#pragma unroll
      for (int nn = 0; nn < 2; ++nn)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (32 * nn + 8 * (j >> 2) + (j & 3) > lim) sacc[nn][j] = NEG_INF;
    }
    float tmax = NEG_INF;
#pragma unroll
    for (int nn = 0; nn < 2; ++nn)
#pragma unroll
      for (int j = 0; j < 16; ++j) tmax = fmaxf(tmax, sacc[nn][j]);
    tmax = xor32_max(tmax);
    const float sl2 = a.scale_log2;
    // The reference max m_run (log2 units) moves only when this tile's row max exceeds
    // it by more than kPfLazyMax: probabilities then stay below 2^kPfLazyMax and the
    // accumulators are rescaled on few tiles instead of on most (o / l is the same for
    // any reference). The first tile with a visible key always moves it.
    const float t2 = tmax * sl2;
    const float m_new = t2 > m_run + kPfLazyMax ? t2 : m_run;
    // rows past the chunk (my_limit = -1) see no key at all: keep them at zero
    const float m_use = m_new == NEG_INF ? 0.0f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    // the row sum is taken over the bf16-rounded probabilities that multiply V, two
    // per dot2
    float psum = 0.0f;
    bf16x8_t pb[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float pv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) pv[i] = fast_exp2(fmaf(sacc[t >> 1][8 * (t & 1) + i], sl2, -m_use));
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[t][i] = (__bf16)pv[i];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf2 pp = {pb[t][2 * i], pb[t][2 * i + 1]};
        psum = __builtin_amdgcn_fdot2_f32_bf16(pp, kOnesBf2, psum, false);
      }
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

  const float l_tot = xor32_sum(l_run);
  if (nchunks > 1) {
    if (!wave_active) return;
    // partial over this key chunk: normalised o and log2-sum-exp; a row that saw no
    // key here (all past its causal limit) gets lse = -inf and weighs nothing
    const bool any = l_tot > 0.0f;
    const float inv = any ? 1.0f / l_tot : 0.0f;
    const int64_t row = ((int64_t)(t_begin + my_tok) * a.q_heads + g * G + my_hh) * a.max_chunks + chunk;
    if (row_ok && hl == 0) a.ws_lse[row] = any ? m_run + __log2f(l_tot) : -__builtin_huge_valf();
    // A lane holds 16-byte pieces of one row, so storing them directly would touch 32
    // cache lines per instruction. Each 32-wide d slice goes through this wave's LDS
    // slice instead and leaves as whole 128-byte lines: lane l stores float4 l % 8 of
    // row 8 i + l / 8 (i = 0..3), eight lanes per line.
    float* os = Os + wave * (32 * kPfORow);
    const int rsub = lane >> 3, cq = lane & 7;
    float* dst[4];
    bool dst_ok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mw0 + 8 * i + rsub;
      dst_ok[i] = m < nrows;
      const int mm = dst_ok[i] ? m : mw0;
      const int64_t r = ((int64_t)(t_begin + mm / G) * a.q_heads + g * G + mm % G) * a.max_chunks + chunk;
      dst[i] = a.ws_o + r * D + 4 * cq;
    }
#pragma unroll
    for (int dn = 0; dn < DT; ++dn) {
      // the previous slice's LDS reads are done before this slice overwrites them
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int jq = 0; jq < 4; ++jq)
        *reinterpret_cast<float4*>(&os[l32 * kPfORow + 8 * jq + 4 * hl]) =
            make_float4(oacc[dn][4 * jq] * inv, oacc[dn][4 * jq + 1] * inv,
                        oacc[dn][4 * jq + 2] * inv, oacc[dn][4 * jq + 3] * inv);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 v = *reinterpret_cast<const float4*>(&os[(8 * i + rsub) * kPfORow + 4 * cq]);
        if (dst_ok[i]) *reinterpret_cast<float4*>(dst[i] + 32 * dn) = v;
      }
    }
    return;
  }
  if (!row_ok) return;
  const float inv = 1.0f / l_tot;
  uint16_t* op = a.out + (int64_t)(t_begin + my_tok) * a.out_st + (int64_t)(g * G + my_hh) * a.out_sh;
#pragma unroll
  for (int dn = 0; dn < DT; ++dn)
#pragma unroll
    for (int jq = 0; jq < 4; ++jq) {
      const int d = 32 * dn + 8 * jq + 4 * hl;
      const uint32_t w0 = (uint32_t)f32_to_bf16(oacc[dn][4 * jq] * inv) |
                          ((uint32_t)f32_to_bf16(oacc[dn][4 * jq + 1] * inv) << 16);
      const uint32_t w1 = (uint32_t)f32_to_bf16(oacc[dn][4 * jq + 2] * inv) |
                          ((uint32_t)f32_to_bf16(oacc[dn][4 * jq + 3] * inv) << 16);
      if (out_aligned) {
        *reinterpret_cast<uint2*>(op + d) = make_uint2(w0, w1);
      } else {
        op[d] = (uint16_t)w0;
        op[d + 1] = (uint16_t)(w0 >> 16);
        op[d + 2] = (uint16_t)w1;
        op[d + 3] = (uint16_t)(w1 >> 16);
      }
    }
}

// Persistent prefill: the grid holds at most the resident workgroups; the work items,
// sorted costliest first, are dealt to them in rounds, alternating direction from round
// to round (workgroup b takes item b in round 0, item 2*grid - 1 - b in round 1, ...),
// so that the workgroups with the longest first items get the shortest later ones.
// The assignment is static (no claim counter: one counter hit by every workgroup at
// once serialises). Items are independent, so the result does not depend on it.
template <int D, int G>
__global__ void __launch_bounds__(256, 2) prefill_kernel(PfArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kPfKeys * (D + kKPad)];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * (kPfKeys + kVPad)];
  __shared__ __attribute__((aligned(16))) float Os[(kPfRows / 32) * 32 * kPfORow];
  const PfPlanHeader* hdr = reinterpret_cast<const PfPlanHeader*>(a.plan);
  const PfEntry* entries = reinterpret_cast<const PfEntry*>(a.plan + kPfPlanHeaderBytes);
  const int64_t items = (int64_t)hdr->entries * a.hkv;
  const int64_t grid = gridDim.x, b = blockIdx.x;
  for (int64_t r = 0;; ++r) {
    const int64_t it = r * grid + ((r & 1) ? grid - 1 - b : b);
    if (it >= items) break;
    const int64_t ei = it / a.hkv;
    const PfEntry e = entries[ei];
    prefill_item<D, G>(a, Ks, Vt, Os, e, (int)(it - ei * a.hkv));
  }
}

// The work list. One workgroup: the sizes of the first kPfPlanSeqCache sequences are
// loaded once into LDS; every (sequence, row tile) pair contributes its key chunks
// (all but the last cover split_keys keys), counted into buckets by cost (64-key
// tiles, capped), then written costliest bucket first, so the persistent workgroups
// take the longest items first (longest-processing-time-first list scheduling).
constexpr int kPfPlanThreads = 1024;
constexpr int kPfPlanBuckets = 64;
constexpr int kPfPlanSeqCache = 4 * kPfPlanThreads;

__global__ void __launch_bounds__(kPfPlanThreads) prefill_plan_kernel(PfArgs a) {
  __shared__ int hist[kPfPlanBuckets];
  __shared__ int cursor[kPfPlanBuckets];
  __shared__ int c_begin[kPfPlanSeqCache], c_n[kPfPlanSeqCache], c_len[kPfPlanSeqCache];
  const int tid = threadIdx.x;
  const int G = a.q_heads / a.hkv;
  if (tid < kPfPlanBuckets) hist[tid] = 0;
  const int cached = min(a.num_seqs, kPfPlanSeqCache);
  {
    int tb[4], te[4], cl[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int s = tid + kPfPlanThreads * u;
      if (s < cached) {
        tb[u] = a.cu_seqlens[s];
        te[u] = a.cu_seqlens[s + 1];
        cl[u] = a.context_lens[s];
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int s = tid + kPfPlanThreads * u;
      if (s < cached) {
        c_begin[s] = tb[u];
        c_n[s] = te[u] - tb[u];
        c_len[s] = min(cl[u], a.max_context_len);
      }
    }
  }
  __syncthreads();
  const int64_t pairs = (int64_t)a.num_seqs * a.tiles_per_seq;
  const int S = a.split_keys;
  const int cost_full = S / kPfKeys;
  auto bucket = [](int cost) { return min(cost, kPfPlanBuckets - 1); };
  // (sequence, row tile) pair p: its entry template and number of chunks (0: no work)
  auto visit = [&](int64_t p, PfEntry& e, int& nch, int& cost_last) {
    const int s = (int)(p / a.tiles_per_seq);
    const int mt = (int)(p - (int64_t)s * a.tiles_per_seq);
    int tb, n, L;
    if (s < kPfPlanSeqCache) {
      tb = c_begin[s];
      n = c_n[s];
      L = c_len[s];
    } else {
      tb = a.cu_seqlens[s];
      n = a.cu_seqlens[s + 1] - tb;
      L = min(a.context_lens[s], a.max_context_len);
    }
    nch = 0;
    cost_last = 0;
    // chunks outside [0, total_tokens] break the cu_seqlens contract: no work for them
    if (tb < 0 || n <= 0 || (int64_t)tb + n > a.total_tokens) return;
    const int nrows = n * G;
    const int m0 = mt * kPfRows;
    if (m0 >= nrows) return;
    const int kend = L - n + (min(m0 + kPfRows, nrows) - 1) / G + 1;
    if (kend <= 0) return;  // context shorter than the chunk: nothing visible
    nch = (kend + S - 1) / S;
    const int k_lo = (nch - 1) * S;
    cost_last = (kend + kPfKeys - 1) / kPfKeys - k_lo / kPfKeys;
    e.s = s;
    e.mt = mt;
    e.t_begin = tb;
    e.n = n;
    e.L = L;
    e.pad = 0;
  };
  for (int64_t p = tid; p < pairs; p += kPfPlanThreads) {
    PfEntry e;
    int nch, cost_last;
    visit(p, e, nch, cost_last);
    if (nch > 1) atomicAdd(&hist[bucket(cost_full)], nch - 1);
    if (nch > 0) atomicAdd(&hist[bucket(cost_last)], 1);
  }
  __syncthreads();
  // exclusive scan of the buckets, costliest first, by the first wave (lane l holds
  // bucket kPfPlanBuckets - 1 - l); the counts sum to less than 2^31
  static_assert(kPfPlanBuckets == 64, "one bucket per lane");
  if (tid < 64) {
    const int b = kPfPlanBuckets - 1 - tid;
    const int c = hist[b];
    int incl = c;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d);
      if (tid >= d) incl += o;
    }
    cursor[b] = incl - c;
    if (tid == 63)
      reinterpret_cast<PfPlanHeader*>(a.plan)->entries = (int32_t)min((int64_t)incl, a.plan_bound);
  }
  __syncthreads();
  PfEntry* entries = reinterpret_cast<PfEntry*>(a.plan + kPfPlanHeaderBytes);
  for (int64_t p = tid; p < pairs; p += kPfPlanThreads) {
    PfEntry e;
    int nch, cost_last;
    visit(p, e, nch, cost_last);
    if (nch <= 0) continue;
    if (nch > 1) {
      const int pos = atomicAdd(&cursor[bucket(cost_full)], nch - 1);
      e.cost = cost_full;
      for (int c = 0; c < nch - 1; ++c) {
        if (pos + c >= a.plan_bound) break;
        e.chunk = c;
        entries[pos + c] = e;
      }
    }
    const int pos = atomicAdd(&cursor[bucket(cost_last)], 1);
    if (pos < a.plan_bound) {
      e.chunk = nch - 1;
      e.cost = cost_last;
      entries[pos] = e;
    }
  }
}

// Merge of the key-chunk partials. A thread takes kPfMergePieces 4-float pieces of a
// row: slice sl of the NS = D / (4 kPfMergePieces) slices holds the pieces at
// d = 4 sl + (D / kPfMergePieces) e, so each load instruction has the NS threads of a row
// read whole 128-byte lines of its partial. The prefill grid's row tiles are cut into
// parts of 256 / NS rows; one 256-thread workgroup per (part, row tile, KV head,
// sequence), one thread per (row, slice), slice fastest. Tiles with a single key chunk
// were written directly by the prefill kernel and their workgroups exit after one load
// of the sizes. Each thread runs an online log-sum-exp merge over the chunks, loading
// four chunks ahead.
constexpr int kPfMergePieces = 2;
template <int D>
constexpr int pf_merge_slices() { return D / (4 * kPfMergePieces); }
template <int D>
constexpr int pf_merge_rows() { return 256 / pf_merge_slices<D>(); }

template <int D>
__global__ void __launch_bounds__(256) prefill_merge_kernel(PfArgs a) {
  constexpr int E = kPfMergePieces;
  constexpr int NS = pf_merge_slices<D>();
  constexpr int ROWS = pf_merge_rows<D>();
  constexpr int PARTS = kPfRows / ROWS;
  constexpr float NEG_INF = -__builtin_huge_valf();
  const int part = (int)(blockIdx.x % PARTS);
  const int mt = (int)((blockIdx.x / PARTS) % a.tiles_per_seq);
  const int rest = (int)(blockIdx.x / PARTS / a.tiles_per_seq);
  const int g = rest % a.hkv;
  const int s = rest / a.hkv;
  const int G = a.q_heads / a.hkv;
  const int t_begin = a.cu_seqlens[s];
  const int t_end = a.cu_seqlens[s + 1];
  if (t_begin < 0 || t_end > a.total_tokens) return;
  const int n = t_end - t_begin;
  const int nrows = n * G;
  const int m0 = mt * kPfRows;
  if (m0 >= nrows) return;
  const int L = min(a.context_lens[s], a.max_context_len);
  const int m_last = min(m0 + kPfRows, nrows) - 1;
  const int kend = L - n + m_last / G + 1;
  const int nch = (kend + a.split_keys - 1) / a.split_keys;
  if (nch <= 1) return;  // written directly by the prefill kernel
  const int m = m0 + part * ROWS + (int)threadIdx.x / NS;
  if (m >= nrows) return;
  const int sl = (int)threadIdx.x % NS;
  const int tok = t_begin + m / G;
  const int h = g * G + m % G;
  const int64_t row0 = ((int64_t)tok * a.q_heads + h) * a.max_chunks;
  float mx = NEG_INF, den = 0.0f, acc[4 * E];
#pragma unroll
  for (int e = 0; e < 4 * E; ++e) acc[e] = 0.0f;
  constexpr int U = 4;
  for (int c0 = 0; c0 < nch; c0 += U) {
    float lse[U];
    float4 o[U][E];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = min(c0 + u, nch - 1);
      lse[u] = c0 + u < nch ? a.ws_lse[row0 + c] : NEG_INF;
      const float4* op = reinterpret_cast<const float4*>(a.ws_o + (row0 + c) * D + sl * 4);
#pragma unroll
      for (int e = 0; e < E; ++e) o[u][e] = op[e * NS];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // a chunk with no visible key (lse = -inf) weighs nothing
      const bool ok = lse[u] != NEG_INF;
      const float m_new = ok ? fmaxf(mx, lse[u]) : mx;
      const float f = ok ? fast_exp2(mx - m_new) : 1.0f;  // 0 while mx is -inf
      const float w = ok ? fast_exp2(lse[u] - m_new) : 0.0f;
      den = ok ? fmaf(den, f, w) : den;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        acc[4 * e] = ok ? fmaf(acc[4 * e], f, w * o[u][e].x) : acc[4 * e];
        acc[4 * e + 1] = ok ? fmaf(acc[4 * e + 1], f, w * o[u][e].y) : acc[4 * e + 1];
        acc[4 * e + 2] = ok ? fmaf(acc[4 * e + 2], f, w * o[u][e].z) : acc[4 * e + 2];
        acc[4 * e + 3] = ok ? fmaf(acc[4 * e + 3], f, w * o[u][e].w) : acc[4 * e + 3];
      }
      mx = m_new;
    }
  }
  const float inv = 1.0f / den;  // chunk 0 always holds key 0, so den > 0
  uint16_t* dst = a.out + (int64_t)tok * a.out_st + (int64_t)h * a.out_sh + sl * 4;
  uint32_t w[2 * E];
#pragma unroll
  for (int e = 0; e < 2 * E; ++e)
    w[e] = (uint32_t)f32_to_bf16(acc[2 * e] * inv) | ((uint32_t)f32_to_bf16(acc[2 * e + 1] * inv) << 16);
  if (a.out_aligned) {
#pragma unroll
    for (int e = 0; e < E; ++e) *reinterpret_cast<uint2*>(dst + e * (D / E)) = make_uint2(w[2 * e], w[2 * e + 1]);
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      dst[e * (D / E)] = (uint16_t)w[2 * e];
      dst[e * (D / E) + 1] = (uint16_t)(w[2 * e] >> 16);
      dst[e * (D / E) + 2] = (uint16_t)w[2 * e + 1];
      dst[e * (D / E) + 3] = (uint16_t)(w[2 * e + 1] >> 16);
    }
  }
}

template <int D, int G>
static int launch_prefill_t(const pa_kv_pool_t& pool, const PrefillArgs& pa_, hipStream_t stream) {
  PfArgs a;
  a.kpool = (const uint16_t*)pool.k;
  a.vpool = (const uint16_t*)pool.v;
  a.num_blocks = pool.num_blocks;
  a.hkv = pool.kv_heads;
  a.out = (uint16_t*)pa_.out;
  a.out_st = pa_.out_st;
  a.out_sh = pa_.out_sh;
  a.q = (const uint16_t*)pa_.q;
  a.q_st = pa_.q_st;
  a.q_sh = pa_.q_sh;
  a.cu_seqlens = pa_.cu_seqlens;
  a.num_seqs = pa_.num_seqs;
  a.total_tokens = pa_.total_tokens;
  a.tiles_per_seq = (int)(((int64_t)pa_.max_q_len * G + kPfRows - 1) / kPfRows);
  a.block_tables = pa_.block_tables;
  a.max_blocks_per_seq = pa_.max_blocks_per_seq;
  a.context_lens = pa_.context_lens;
  a.max_context_len = pa_.max_context_len;
  a.scale_log2 = pa_.scale * kLog2e;
  a.q_aligned = ((uintptr_t)pa_.q & 15u) == 0 && pa_.q_st % 8 == 0 && pa_.q_sh % 8 == 0;
  a.out_aligned = ((uintptr_t)pa_.out & 7u) == 0 && pa_.out_st % 4 == 0 && pa_.out_sh % 4 == 0;
  a.q_heads = pa_.q_heads;
  a.split_keys = pa_.split_keys;
  a.max_chunks = pa_.max_chunks;
  a.plan = (char*)pa_.plan;
  a.plan_bound = pa_.plan_bound;
  a.ws_o = pa_.ws_o;
  a.ws_lse = pa_.ws_lse;
  if (launch_kernel(prefill_plan_kernel, dim3(1), dim3(kPfPlanThreads), stream, a) != hipSuccess)
    return PA_ERR_HIP;
  // persistent: no more workgroups than fit at once, nor than there are work items
  const int64_t items = (int64_t)a.tiles_per_seq * a.max_chunks * pool.kv_heads * pa_.num_seqs;
  const int64_t grid = std::min(items, resident_workgroups(prefill_kernel<D, G>, 256));
  if (launch_kernel(prefill_kernel<D, G>, dim3((unsigned)grid), dim3(256), stream, a) != hipSuccess)
    return PA_ERR_HIP;
  if (a.max_chunks > 1 &&
      launch_kernel(prefill_merge_kernel<D>,
                    dim3((unsigned)((int64_t)(kPfRows / pf_merge_rows<D>()) * a.tiles_per_seq *
                                    pool.kv_heads * pa_.num_seqs)),
                    dim3(256), stream, a) != hipSuccess)
    return PA_ERR_HIP;
  return PA_OK;
}

template <int D>
static int dispatch_pf_g(const pa_kv_pool_t& pool, const PrefillArgs& a, hipStream_t stream) {
  switch (a.q_heads / pool.kv_heads) {
    case 1: return launch_prefill_t<D, 1>(pool, a, stream);
    case 2: return launch_prefill_t<D, 2>(pool, a, stream);
    case 3: return launch_prefill_t<D, 3>(pool, a, stream);
    case 4: return launch_prefill_t<D, 4>(pool, a, stream);
    case 5: return launch_prefill_t<D, 5>(pool, a, stream);
    case 6: return launch_prefill_t<D, 6>(pool, a, stream);
    case 7: return launch_prefill_t<D, 7>(pool, a, stream);
    case 8: return launch_prefill_t<D, 8>(pool, a, stream);
    default: return PA_ERR_UNSUPPORTED;
  }
}

int launch_prefill(const pa_kv_pool_t& pool, const PrefillArgs& a, hipStream_t stream) {
  if (pool.dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  return pool.head_dim == 64 ? dispatch_pf_g<64>(pool, a, stream)
                             : dispatch_pf_g<128>(pool, a, stream);
}

}  // namespace pa
