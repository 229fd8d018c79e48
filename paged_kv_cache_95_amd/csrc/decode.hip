// pa_decode kernels: paged GQA decode attention with split-K and a log-sum-exp merge.
//
// What is computed follows Decode_Paged_GQAAttention_Kernel of the koas-w "errors and
// solutions" post ("hand-written Triton kernels": KV read block by block in place
// through block_table, online softmax, GQA mapping inside the kernel). Splitting a
// long context into fixed-length pieces whose (lse, o) partials are merged by
// log-sum-exp is not on the pages; it is how one wave's worth of work is kept small
// enough to fill 256 CUs. The merge runs in the same launch: each split writes its
// normalised partial and log2-sum-exp, then counts its arrival on a per-(sequence,
// KV head) counter; the last arrival merges the group and resets the counter.
//
// Work item = (sequence s, KV head g, split i) = one wavefront, which serves all G
// query heads of the group, so every K/V byte is read once. Per 16-token block:
//
//   K side  lane = 16r + 4t + c holds token 4t + r of the block; c selects the
//           16-byte chunks c, c+4, ... of that token's row. Partial dots over those
//           chunks, a quad butterfly (DPP) finishes q.k for all G heads.
//   softmax each 16-lane DPP row r owns tokens {r, r+4, r+8, r+12} and keeps its own
//           running max / sum per head, so the per-block max is a 2-step row rotate;
//           the four rows are combined once per split, like split partials.
//   V side  lane = 16r + cv accumulates head dims [cv*D/16, (cv+1)*D/16) for the
//           row's four tokens; the probabilities reach it by row rotations of 4, 8
//           and 12 lanes, and the token each rotation delivers is found by rotating
//           the token index the same way.
//
// Loads are 16-byte per lane and each instruction covers whole 64-byte pieces of 16
// token rows (K) or four full rows (V); the next block is loaded while the current one
// is computed. Tokens past the context (the tail of the last block) are excluded by
// selects, never by multiplying with zero, so stale or NaN slots cannot leak in.
#include "common.h"
#include "internal.h"

namespace pa {

constexpr int kWaves = 4;  // wavefronts (independent work items) per 256-thread block

template <int KVT, int D>
struct Geom {
  static constexpr int E = ElemBytes<KVT>::value;
  static constexpr int ROW = D * E;      // bytes of one token row of one KV head
  static constexpr int NCH = ROW / 16;   // 16-byte chunks per row
  static constexpr int KCH = NCH / 4;    // chunks per K-lane
  static constexpr int EPC = 16 / E;     // elements per chunk
  static constexpr int EK = KCH * EPC;   // elements per K-lane (D / 4)
  static constexpr int EV = D / 16;      // elements per V-lane
  static constexpr int VB = EV * E;      // bytes per V-lane per token
  static constexpr int VW = VB / 4;      // dwords per V-lane per token
  static constexpr int QW = KVT == kF32 ? EK : EK / 2;  // query registers per head
};

template <int N>
__device__ __forceinline__ void load_dwords(const char* p, uint32_t (&w)[N]) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const uint4 x = reinterpret_cast<const uint4*>(p)[i];
      w[4 * i] = x.x; w[4 * i + 1] = x.y; w[4 * i + 2] = x.z; w[4 * i + 3] = x.w;
    }
  } else if constexpr (N == 2) {
    const uint2 x = *reinterpret_cast<const uint2*>(p);
    w[0] = x.x; w[1] = x.y;
  } else {
    static_assert(N == 1, "unsupported V width");
    w[0] = *reinterpret_cast<const uint32_t*>(p);
  }
}

template <int KVT, int D>
struct BlockBuf {
  using Gm = Geom<KVT, D>;
  uint32_t k[Gm::KCH * 4];
  uint32_t v[4][Gm::VW];
  float ks, vs;
  int nvalid;
};

template <int KVT, int D, int G>
struct DecodeState {
  using Gm = Geom<KVT, D>;
  float acc[G][Gm::EV];
  float m[G];  // running max of this lane's DPP row (log2 domain)
  float l[G];  // running sum of this lane's own token's weights
};

template <int KVT, int D, int G, bool MASKED>
__device__ __forceinline__ void process_block(const BlockBuf<KVT, D>& b, DecodeState<KVT, D, G>& st,
                                              const uint32_t (&qw)[G][Geom<KVT, D>::QW],
                                              float scale_log2, int tok_k, const int (&tok_v)[4]) {
  using Gm = Geom<KVT, D>;
  constexpr float NEG_INF = -__builtin_huge_valf();
  // ---- scores: partial dot over this lane's chunks, then the quad butterfly
  float s[G];
#pragma unroll
  for (int h = 0; h < G; ++h) s[h] = 0.0f;
  if constexpr (KVT == kBF16) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int w = 0; w < Gm::KCH * 4; ++w)
#pragma unroll
      for (int h = 0; h < G; ++h)
        s[h] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, qw[h][w]),
                                               __builtin_bit_cast(bf2, b.k[w]), s[h], false);
  } else if constexpr (KVT == kFP8) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int w = 0; w < Gm::KCH * 4; ++w) {
      float x0, x1, x2, x3;
      e4m3x2_to_f32(b.k[w], false, x0, x1);
      e4m3x2_to_f32(b.k[w], true, x2, x3);
      const uint32_t p0 = pack_bf16_exact(x0, x1), p1 = pack_bf16_exact(x2, x3);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        s[h] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, qw[h][2 * w]),
                                               __builtin_bit_cast(bf2, p0), s[h], false);
        s[h] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, qw[h][2 * w + 1]),
                                               __builtin_bit_cast(bf2, p1), s[h], false);
      }
    }
  } else {
#pragma unroll
    for (int w = 0; w < Gm::KCH * 4; ++w)
#pragma unroll
      for (int h = 0; h < G; ++h)
        s[h] = fmaf(__uint_as_float(qw[h][w]), __uint_as_float(b.k[w]), s[h]);
  }
  const float sc = KVT == kFP8 ? scale_log2 * b.ks : scale_log2;
  const bool valid_k = !MASKED || tok_k < b.nvalid;
  float p[G];
  bool rescale = false;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float x = s[h];
    x += dpp<kQuadXor1>(x);
    x += dpp<kQuadXor2>(x);
    x *= sc;
    if (MASKED) x = valid_k ? x : NEG_INF;
    float mb = fmaxf(x, dpp<kRowRor4>(x));
    mb = fmaxf(mb, dpp<kRowRor8>(mb));
    const float m_new = fmaxf(st.m[h], mb);
    float alpha, ph;
    if (MASKED) {
      // a row may have seen no valid token yet (m_new = -inf): keep it at zero
      alpha = m_new == NEG_INF ? 1.0f : fast_exp2(st.m[h] - m_new);
      ph = valid_k ? fast_exp2(x - m_new) : 0.0f;
    } else {
      alpha = fast_exp2(st.m[h] - m_new);
      ph = fast_exp2(x - m_new);
    }
    rescale |= alpha != 1.0f;
    st.l[h] = fmaf(st.l[h], alpha, ph);
    st.m[h] = m_new;
    p[h] = ph;
    if (__any(rescale)) {
      // alpha is uniform over the DPP row, and the V-lanes of row r own row r's acc
#pragma unroll
      for (int e = 0; e < Gm::EV; ++e) st.acc[h][e] *= alpha;
    }
    rescale = false;
  }
  if constexpr (KVT == kFP8) {
#pragma unroll
    for (int h = 0; h < G; ++h) p[h] = valid_k ? p[h] * b.vs : 0.0f;
  }
  // ---- V: four tokens of this row, delivered by row rotations
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    float pk[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (kk == 0) pk[h] = p[h];
      else if (kk == 1) pk[h] = dpp<kRowRor4>(p[h]);
      else if (kk == 2) pk[h] = dpp<kRowRor8>(p[h]);
      else pk[h] = dpp<kRowRor12>(p[h]);
    }
    const bool valid_v = !MASKED || tok_v[kk] < b.nvalid;
    float vf[Gm::EV];
    if constexpr (KVT == kBF16) {
#pragma unroll
      for (int w = 0; w < Gm::VW; ++w) {
        const uint32_t x = valid_v ? b.v[kk][w] : 0u;
        vf[2 * w] = bf16_lo(x);
        vf[2 * w + 1] = bf16_hi(x);
      }
    } else if constexpr (KVT == kFP8) {
#pragma unroll
      for (int w = 0; w < Gm::VW; ++w) {
        const uint32_t x = valid_v ? b.v[kk][w] : 0u;
        e4m3x2_to_f32(x, false, vf[4 * w], vf[4 * w + 1]);
        e4m3x2_to_f32(x, true, vf[4 * w + 2], vf[4 * w + 3]);
      }
    } else {
#pragma unroll
      for (int w = 0; w < Gm::VW; ++w) vf[w] = __uint_as_float(valid_v ? b.v[kk][w] : 0u);
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < Gm::EV; ++e) st.acc[h][e] = fmaf(pk[h], vf[e], st.acc[h][e]);
  }
}

template <int KVT, int D, int G, int QT>
__global__ void __launch_bounds__(64 * kWaves) decode_split_kernel(
    const char* __restrict__ kpool, const char* __restrict__ vpool,
    const float* __restrict__ kscale, const float* __restrict__ vscale, int64_t num_blocks,
    int hkv, void* __restrict__ out, int64_t out_st, int64_t out_sh,
    const void* __restrict__ q, int64_t q_st, int64_t q_sh, int num_seqs, int splits_per_row,
    const int32_t* __restrict__ block_tables, int max_blocks_per_seq,
    const int32_t* __restrict__ context_lens, int max_context_len, float scale_log2,
    int split_tokens, int max_splits, float* __restrict__ ws_o, float* __restrict__ ws_lse,
    int* __restrict__ counters) {
  using Gm = Geom<KVT, D>;
  constexpr float NEG_INF = -__builtin_huge_valf();
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // blockIdx.x -> (split group, kv head, sequence), split group fastest
  const int sg = blockIdx.x % splits_per_row;
  const int rest = blockIdx.x / splits_per_row;
  const int g = rest % hkv;
  const int s = rest / hkv;
  const int split = sg * kWaves + wave;
  // a context longer than the host bound would index past this sequence's workspace
  // rows and block-table row: clamp (contract violation, output then unspecified)
  const int L = min(context_lens[s], max_context_len);
  const int nsplit = L > 0 ? (L + split_tokens - 1) / split_tokens : 0;
  if (split >= nsplit) return;
  const int t0 = split * split_tokens;
  const int t1 = min(L, t0 + split_tokens);
  const int jb0 = t0 / kBlockSize;
  const int nblk = (t1 - t0 + kBlockSize - 1) / kBlockSize;

  // ---- lane geometry
  const int r = lane >> 4;
  const int tq = (lane >> 2) & 3;
  const int c = lane & 3;
  const int cv = lane & 15;
  const int tok_k = 4 * tq + r;
  int tok_v[4];
  tok_v[0] = tok_k;
  tok_v[1] = dpp_i<kRowRor4>(tok_k);
  tok_v[2] = dpp_i<kRowRor8>(tok_k);
  tok_v[3] = dpp_i<kRowRor12>(tok_k);

  // ---- query registers for the G heads of this group
  uint32_t qw[G][Gm::QW];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const int64_t qoff = (int64_t)s * q_st + (int64_t)(g * G + h) * q_sh;
#pragma unroll
    for (int i = 0; i < Gm::KCH; ++i) {
      const int d0 = (c + 4 * i) * Gm::EPC;
      if constexpr (QT == kF32) {
        const float* qp = (const float*)q + qoff + d0;
#pragma unroll
        for (int e = 0; e < Gm::EPC; ++e) qw[h][i * Gm::EPC + e] = __float_as_uint(qp[e]);
      } else {
        const uint16_t* qp = (const uint16_t*)q + qoff + d0;
#pragma unroll
        for (int e = 0; e < Gm::EPC / 2; ++e)
          qw[h][i * Gm::EPC / 2 + e] = (uint32_t)qp[2 * e] | ((uint32_t)qp[2 * e + 1] << 16);
      }
    }
  }

  // ---- block ids of this split: lane j holds entry jb0 + j (split <= 64 blocks)
  const int32_t* bt_row = block_tables + (int64_t)s * max_blocks_per_seq;
  const int bid_lane = lane < nblk ? bt_row[jb0 + lane] : 0;

  const int64_t blk_bytes = (int64_t)kBlockSize * hkv * Gm::ROW;
  const uint32_t kofs = (uint32_t)((tok_k * hkv + g) * Gm::ROW + c * 16);
  uint32_t vofs[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) vofs[kk] = (uint32_t)((tok_v[kk] * hkv + g) * Gm::ROW + cv * Gm::VB);
  const uint32_t sofs = (uint32_t)(tok_k * hkv + g);

  auto load = [&](BlockBuf<KVT, D>& b, int j) {
    const int bid_raw = __builtin_amdgcn_readlane(bid_lane, j);
    const bool ok = (unsigned)bid_raw < (uint64_t)num_blocks;
    const int64_t bid = ok ? bid_raw : 0;
    const int first = (jb0 + j) * kBlockSize;
    b.nvalid = ok ? min(kBlockSize, L - first) : 0;
    const char* kb = kpool + bid * blk_bytes + kofs;
#pragma unroll
    for (int i = 0; i < Gm::KCH; ++i) {
      const uint4 x = *reinterpret_cast<const uint4*>(kb + i * 64);
      b.k[4 * i] = x.x; b.k[4 * i + 1] = x.y; b.k[4 * i + 2] = x.z; b.k[4 * i + 3] = x.w;
    }
    const char* vb = vpool + bid * blk_bytes;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) load_dwords<Gm::VW>(vb + vofs[kk], b.v[kk]);
    if constexpr (KVT == kFP8) {
      const int64_t sb = bid * kBlockSize * hkv + sofs;
      b.ks = kscale[sb];
      b.vs = vscale[sb];
    } else {
      b.ks = b.vs = 1.0f;
    }
  };

  DecodeState<KVT, D, G> st;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    st.m[h] = NEG_INF;
    st.l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < Gm::EV; ++e) st.acc[h][e] = 0.0f;
  }
  auto process = [&](const BlockBuf<KVT, D>& b) {
    if (b.nvalid == kBlockSize)
      process_block<KVT, D, G, false>(b, st, qw, scale_log2, tok_k, tok_v);
    else
      process_block<KVT, D, G, true>(b, st, qw, scale_log2, tok_k, tok_v);
  };

  BlockBuf<KVT, D> A, B;
  load(A, 0);
  int j = 0;
  for (; j + 1 < nblk; j += 2) {
    load(B, j + 1);
    process(A);
    if (j + 2 < nblk) load(A, j + 2);
    process(B);
  }
  if (j < nblk) process(A);

  // ---- combine the four DPP rows: per head, rescale to the wave max and sum
  float inv_l[G], lse2[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float lr = st.l[h] + dpp<kRowRor4>(st.l[h]);
    lr += dpp<kRowRor8>(lr);  // sum over the row's four tokens
    float M = fmaxf(st.m[h], __shfl_xor(st.m[h], 16));
    M = fmaxf(M, __shfl_xor(M, 32));
    const float f = st.m[h] == NEG_INF ? 0.0f : fast_exp2(st.m[h] - M);
    lr *= f;
    lr += __shfl_xor(lr, 16);
    lr += __shfl_xor(lr, 32);
#pragma unroll
    for (int e = 0; e < Gm::EV; ++e) {
      float a = st.acc[h][e] * f;
      a += __shfl_xor(a, 16);
      a += __shfl_xor(a, 32);
      st.acc[h][e] = a;
    }
    inv_l[h] = 1.0f / lr;
    lse2[h] = M + __log2f(lr);
  }
  const int d0 = cv * Gm::EV;
  if (nsplit == 1) {
    if (lane < 16) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const int64_t o = (int64_t)s * out_st + (int64_t)(g * G + h) * out_sh + d0;
        if constexpr (QT == kF32) {
#pragma unroll
          for (int e = 0; e < Gm::EV; ++e) ((float*)out)[o + e] = st.acc[h][e] * inv_l[h];
        } else {
#pragma unroll
          for (int e = 0; e < Gm::EV; ++e)
            ((uint16_t*)out)[o + e] = f32_to_bf16(st.acc[h][e] * inv_l[h]);
        }
      }
    }
    return;
  }
  const int hq = hkv * G;
  if (lane < 16) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const int64_t row = ((int64_t)s * hq + g * G + h) * max_splits + split;
      float* wo = ws_o + row * D + d0;
#pragma unroll
      for (int e = 0; e < Gm::EV; ++e) wo[e] = st.acc[h][e] * inv_l[h];
      if (cv == 0) ws_lse[row] = lse2[h];
    }
  }
  // ---- the last split of (s, g) to finish merges the group's partials:
  // out = sum_i 2^(lse_i - M) o_i / sum_i 2^(lse_i - M), M = max_i lse_i.
  // Release our partials, count, and let only the last arrival read them back.
  __threadfence();
  int* counter = counters + (int64_t)s * hkv + g;
  int old = 0;
  if (lane == 0) old = atomicAdd(counter, 1);
  old = __shfl(old, 0);
  if (old != nsplit - 1) return;
  __threadfence();
  constexpr int PER = D / 64;
#pragma unroll 1
  for (int h = 0; h < G; ++h) {
    const int64_t row0 = ((int64_t)s * hq + g * G + h) * max_splits;
    // lse values are read with per-lane addresses (vector loads through the coherent
    // path), then broadcast with readlane
    float M = NEG_INF;
    for (int i0 = 0; i0 < nsplit; i0 += 64)
      if (i0 + lane < nsplit) M = fmaxf(M, ws_lse[row0 + i0 + lane]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.0f;
    float den = 0.0f;
    for (int i0 = 0; i0 < nsplit; i0 += 64) {
      const float w_lane = i0 + lane < nsplit ? fast_exp2(ws_lse[row0 + i0 + lane] - M) : 0.0f;
      const int cnt = min(64, nsplit - i0);
      for (int i = 0; i < cnt; ++i) {
        const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_lane), i));
        den += w;
        const float* o = ws_o + (row0 + i0 + i) * D;
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = fmaf(w, o[lane + 64 * e], acc[e]);
      }
    }
    const float inv = 1.0f / den;
    const int64_t base = (int64_t)s * out_st + (int64_t)(g * G + h) * out_sh;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int d = lane + 64 * e;
      if constexpr (QT == kF32) ((float*)out)[base + d] = acc[e] * inv;
      else ((uint16_t*)out)[base + d] = f32_to_bf16(acc[e] * inv);
    }
  }
  // every split of this group has arrived: leave the counter at zero for the next call
  if (lane == 0) *counter = 0;
}

template <int KVT, int D, int G, int QT>
static void launch_decode_t(const pa_kv_pool_t& pool, const DecodeArgs& a, hipStream_t stream) {
  const int splits_per_row = (a.max_splits + kWaves - 1) / kWaves;
  const int64_t grid = (int64_t)splits_per_row * pool.kv_heads * a.num_seqs;
  decode_split_kernel<KVT, D, G, QT><<<(unsigned)grid, 64 * kWaves, 0, stream>>>(
      (const char*)pool.k, (const char*)pool.v, pool.k_scale, pool.v_scale, pool.num_blocks,
      pool.kv_heads, a.out, a.out_st, a.out_sh, a.q, a.q_st, a.q_sh, a.num_seqs,
      splits_per_row, a.block_tables, a.max_blocks_per_seq, a.context_lens,
      a.max_context_len, a.scale * kLog2e, a.split_tokens, a.max_splits, a.ws_o, a.ws_lse,
      a.counters);
}

template <int KVT, int D, int QT>
static int dispatch_g(const pa_kv_pool_t& pool, const DecodeArgs& a, hipStream_t stream) {
  switch (a.q_heads / pool.kv_heads) {
    case 1: launch_decode_t<KVT, D, 1, QT>(pool, a, stream); return PA_OK;
    case 2: launch_decode_t<KVT, D, 2, QT>(pool, a, stream); return PA_OK;
    case 3: launch_decode_t<KVT, D, 3, QT>(pool, a, stream); return PA_OK;
    case 4: launch_decode_t<KVT, D, 4, QT>(pool, a, stream); return PA_OK;
    case 5: launch_decode_t<KVT, D, 5, QT>(pool, a, stream); return PA_OK;
    case 6: launch_decode_t<KVT, D, 6, QT>(pool, a, stream); return PA_OK;
    case 7: launch_decode_t<KVT, D, 7, QT>(pool, a, stream); return PA_OK;
    case 8: launch_decode_t<KVT, D, 8, QT>(pool, a, stream); return PA_OK;
    default: return PA_ERR_UNSUPPORTED;
  }
}

int launch_decode(const pa_kv_pool_t& pool, const DecodeArgs& a, hipStream_t stream) {
  const int D = pool.head_dim;
  switch (pool.dtype) {
    case PA_F32:
      return D == 64 ? dispatch_g<kF32, 64, kF32>(pool, a, stream)
                     : dispatch_g<kF32, 128, kF32>(pool, a, stream);
    case PA_BF16:
      return D == 64 ? dispatch_g<kBF16, 64, kBF16>(pool, a, stream)
                     : dispatch_g<kBF16, 128, kBF16>(pool, a, stream);
    case PA_FP8_E4M3:
      return D == 64 ? dispatch_g<kFP8, 64, kBF16>(pool, a, stream)
                     : dispatch_g<kFP8, 128, kBF16>(pool, a, stream);
    default:
      return PA_ERR_UNSUPPORTED;
  }
}

}  // namespace pa
