// pa_decode kernels: paged GQA decode attention with split-K and a log-sum-exp merge.
//
// What is computed follows Decode_Paged_GQAAttention_Kernel of the koas-w "errors and
// solutions" post ("hand-written Triton kernels": KV read block by block in place
// through block_table, online softmax, GQA mapping inside the kernel). Splitting a
// long context into fixed-length pieces whose (lse, o) partials are merged by
// log-sum-exp is not on the pages; it is how one wave's worth of work is kept small
// enough to fill 256 CUs. Each split writes its normalised partial and log2-sum-exp to
// the workspace; a second, small launch merges them.
//
// Work item = (sequence s, split i, KV head g) = one wavefront, which serves all G
// query heads of the group, so every K/V byte is read once; in the persistent and
// plain-grid schedules the KV heads of one split are neighbouring work items, so a
// pool block (all KV heads of 16 tokens) is fetched by one workgroup at about the same
// time. Two item bodies exist: the dot-product one described here (fp32 pools, and
// bf16 pools with G <= 4) and the matrix-core one further down (bf16 pools with G > 4,
// FP8, INT8).
// Dot-product item, lane = 16r + 8h + t (DPP row r, half h):
//
//   K side  the 8 lanes of a half-row share one token and each loads 16-byte chunks
//           t, t+8, ... of its row, so one load instruction covers whole 128-byte lines
//           of 8 tokens. Partial dots over those chunks, then quad and half-row
//           butterflies (DPP) give q.k for all G heads. Token of (set k, row r, half h)
//           = 8k + 2r + h, so row r owns tokens {2r, 2r+1, 8+2r, 9+2r}.
//   softmax each DPP row keeps its own running max / sum per head: the block max is a
//           local max over the two sets plus one row mirror; the four rows are
//           combined once per split, like split partials.
//   V side  lane 16r + c accumulates head dims [c*D/16, (c+1)*D/16) over the row's
//           four tokens, each read as a full row (16 lanes); the probabilities of the
//           other half-row's tokens arrive by a row mirror.
//
// A ring of block buffers keeps the next blocks' loads in flight while the current one
// is computed; KV loads are non-temporal (read once per call). Tokens past the context
// (the tail of the last block) are excluded by selects, never by multiplying with
// zero, so stale or NaN slots cannot leak in.
#include <algorithm>
#include <mutex>

#include "common.h"
#include "internal.h"

namespace pa {

constexpr int kWaves = 4;  // wavefronts (independent work items) per 256-thread block
// Most waves of any workgroup that runs decode_item (the persistent schedule's 8).
constexpr int kMaxItemWaves = 8;
constexpr int kRowMirror = 0x140;
constexpr int kHalfMirror = 0x141;

template <int KVT, int D>
struct Geom {
  static constexpr int E = ElemBytes<KVT>::value;
  static constexpr int ROW = D * E;                   // bytes of one token row, one KV head
  static constexpr int NCH = ROW / 16;                // 16-byte chunks per row
  static constexpr int KC = NCH >= 8 ? NCH / 8 : 1;   // chunks per K-lane per token
  static constexpr int EPC = 16 / E;                  // elements per chunk
  static constexpr int QW = 4 * KC;                  // query dwords per K-lane per head
  static constexpr int EV = D / 16;                   // elements per V-lane per token
  static constexpr int VB = EV * E;                   // bytes per V-lane per token
  static constexpr int VW = VB / 4;                   // dwords per V-lane per token
};

template <int N>
__device__ __forceinline__ void load_dwords(const char* p, uint32_t (&w)[N]) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const uint4 x = ld_stream16(p + 16 * i);
      w[4 * i] = x.x; w[4 * i + 1] = x.y; w[4 * i + 2] = x.z; w[4 * i + 3] = x.w;
    }
  } else if constexpr (N == 2) {
    const uint2 x = ld_stream8(p);
    w[0] = x.x; w[1] = x.y;
  } else {
    static_assert(N == 1, "unsupported V width");
    w[0] = ld_stream4(p);
  }
}

template <int KVT, int D>
struct BlockBuf {
  using Gm = Geom<KVT, D>;
  uint32_t k[2][Gm::KC * 4];  // [token set][dwords]
  uint32_t v[4][Gm::VW];      // [row token][dwords]
  int nvalid;
};

// Blocks kept in flight per wave: as many as the registers allow without losing a
// wave per SIMD.
template <int G>
struct RingDepth {
  static constexpr int value = G <= 4 ? 3 : 2;
};

template <int KVT, int D, int G>
struct DecodeState {
  using Gm = Geom<KVT, D>;
  float acc[G][Gm::EV];
  float m[G];  // running max of this lane's DPP row (log2 domain)
  float l[G];  // running sum over this lane's own K tokens (half of its DPP row's)
};

template <int KVT, int D, int G, bool MASKED>
__device__ __forceinline__ void process_block(const BlockBuf<KVT, D>& b, DecodeState<KVT, D, G>& st,
                                              const uint32_t (&qw)[G][Geom<KVT, D>::QW],
                                              float scale_log2, const int (&tok_k)[2],
                                              const int (&tok_v)[4]) {
  using Gm = Geom<KVT, D>;
  constexpr float NEG_INF = -__builtin_huge_valf();
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  // ---- scores of the two K tokens of this lane
  float s[2][G];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
#pragma unroll
    for (int h = 0; h < G; ++h) s[k][h] = 0.0f;
    if constexpr (KVT == kBF16) {
#pragma unroll
      for (int w = 0; w < Gm::KC * 4; ++w)
#pragma unroll
        for (int h = 0; h < G; ++h)
          s[k][h] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, qw[h][w]),
                                                    __builtin_bit_cast(bf2, b.k[k][w]), s[k][h],
                                                    false);
    } else {
#pragma unroll
      for (int w = 0; w < Gm::KC * 4; ++w)
#pragma unroll
        for (int h = 0; h < G; ++h)
          s[k][h] = fmaf(__uint_as_float(qw[h][w]), __uint_as_float(b.k[k][w]), s[k][h]);
    }
  }
  bool valid_k[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) valid_k[k] = !MASKED || tok_k[k] < b.nvalid;
  float p_own[2][G], p_oth[2][G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float x[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      float y = s[k][h];
      y += dpp<kQuadXor1>(y);
      y += dpp<kQuadXor2>(y);
      y += dpp<kHalfMirror>(y);
      y *= scale_log2;
      x[k] = MASKED ? (valid_k[k] ? y : NEG_INF) : y;
    }
    float mb = fmaxf(x[0], x[1]);
    mb = fmaxf(mb, dpp<kRowMirror>(mb));  // max over the row's four tokens
    const float m_new = fmaxf(st.m[h], mb);
    float alpha;
    if (MASKED) {
      // a row may have seen no valid token yet (m_new = -inf): keep it at zero
      alpha = m_new == NEG_INF ? 1.0f : fast_exp2(st.m[h] - m_new);
#pragma unroll
      for (int k = 0; k < 2; ++k) p_own[k][h] = valid_k[k] ? fast_exp2(x[k] - m_new) : 0.0f;
    } else {
      alpha = fast_exp2(st.m[h] - m_new);
#pragma unroll
      for (int k = 0; k < 2; ++k) p_own[k][h] = fast_exp2(x[k] - m_new);
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) p_oth[k][h] = dpp<kRowMirror>(p_own[k][h]);
    // sum over this lane's own two tokens; the half-row mirror is added once per item
    st.l[h] = fmaf(st.l[h], alpha, p_own[0][h] + p_own[1][h]);
    st.m[h] = m_new;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
      // alpha is uniform over the DPP row, and the V-lanes of row r own row r's acc
#pragma unroll
      for (int e = 0; e < Gm::EV; ++e) st.acc[h][e] *= alpha;
    }
  }
  // ---- V: the row's four tokens (own set 0, other set 0, own set 1, other set 1)
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const bool valid_v = !MASKED || tok_v[x] < b.nvalid;
    float vf[Gm::EV];
    if constexpr (KVT == kBF16) {
#pragma unroll
      for (int w = 0; w < Gm::VW; ++w) {
        const uint32_t y = valid_v ? b.v[x][w] : 0u;
        vf[2 * w] = bf16_lo(y);
        vf[2 * w + 1] = bf16_hi(y);
      }
    } else {
#pragma unroll
      for (int w = 0; w < Gm::VW; ++w) vf[w] = __uint_as_float(valid_v ? b.v[x][w] : 0u);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float pk = (x & 1) ? p_oth[x >> 1][h] : p_own[x >> 1][h];
#pragma unroll
      for (int e = 0; e < Gm::EV; ++e) st.acc[h][e] = fmaf(pk, vf[e], st.acc[h][e]);
    }
  }
}

struct SplitArgs {
  const char* kpool;
  const char* vpool;
  const float* kscale;
  const float* vscale;
  int64_t num_blocks;
  int hkv;
  void* out;
  int64_t out_st, out_sh;
  const void* q;
  int64_t q_st, q_sh;
  int num_seqs;
  const int32_t* block_tables;
  int max_blocks_per_seq;
  const int32_t* context_lens;
  int max_context_len;
  float scale_log2;
  int split_tokens;
  int max_splits;
  float* ws_o;       // [num_seqs, q_heads, max_splits, D] split (or group) partials
  float* ws_lse;     // [num_seqs, q_heads, max_splits]
  int group_splits;  // splits per level-1 merge group (GroupSplits<pool dtype>)
  int max_chunks;    // ceil(max_splits / group_splits): groups per sequence, at most
  unsigned* counters;  // [num_seqs, kv_heads] arrival counters, zero between calls
  // Decode step with the store folded in (single-launch schedule only; knew == nullptr
  // otherwise): row s of knew / vnew ([num_seqs, kv_heads, D] of the pool dtype, element
  // strides, 16-byte aligned rows) is sequence s's newest token, stored to slots[s].
  const char* knew;
  const char* vnew;
  int64_t knew_st, knew_sh, vnew_st, vnew_sh;
  const int64_t* slots;
  bool q_aligned;    // q rows start on 16-byte boundaries (base and strides)
  bool out_aligned;  // same for out
};

// Uniform read of call metadata that nothing writes during the launch, through the
// constant address space, so it is a scalar load (SGPR result, lgkmcnt): the vector
// loads issued around it are not waited for, and no readfirstlane is needed.
template <typename T>
__device__ __forceinline__ T ld_uniform(const T* p) {
  typedef const __attribute__((address_space(4))) T cT;
  return *(cT*)(uintptr_t)p;
}

// Context length as the kernels use it: clamped to the host bound, so a longer value
// (a contract violation) cannot index past the sequence's workspace rows or its
// block-table row; its output is then unspecified.
__device__ __forceinline__ int clamped_len(const SplitArgs& a, int s) {
  return min(a.context_lens[s], a.max_context_len);
}
__device__ __forceinline__ int num_splits(int L, int split_tokens) {
  return L > 0 ? (L + split_tokens - 1) / split_tokens : 0;
}

// Inputs of one work item that do not depend on its context length: the G query rows
// (as this lane's dot-product operands) and the block ids of the split (lane j holds
// entry jb0 + j; a split is at most 64 blocks). Issuing these before the length is
// known takes one dependent memory round trip off each item. Table entries past the
// context are loaded but never used for addressing.
template <int KVT, int D, int G>
struct ItemIn {
  uint32_t qw[G][Geom<KVT, D>::QW];
  int bid_lane;
};

// Block id of block `lane` of the split (one per lane, up to 64 blocks).
__device__ __forceinline__ int item_bid_lane(const SplitArgs& a, int s, int split, int lane) {
  const int jb0 = split * (a.split_tokens / kBlockSize);
  const int32_t* bt_row = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  return (lane < a.split_tokens / kBlockSize && jb0 + lane < a.max_blocks_per_seq)
             ? bt_row[jb0 + lane]
             : 0;
}

// The query rows of heads g*G .. g*G+G-1 of sequence s, in the dot-product body's lane
// layout.
template <int KVT, int D, int G, int QT>
__device__ __forceinline__ void load_item_q(const SplitArgs& a, int s, int g, int lane,
                                            uint32_t (&qw)[G][Geom<KVT, D>::QW]) {
  using Gm = Geom<KVT, D>;
  const int t8 = lane & 7;
  const bool k_lane = t8 < Gm::NCH;  // false only for rows shorter than 8 chunks
  // ---- query chunks t8 + 8j of the G heads (bf16 pairs, or fp32)
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const int64_t qoff = (int64_t)s * a.q_st + (int64_t)(g * G + h) * a.q_sh;
#pragma unroll
    for (int j = 0; j < Gm::KC; ++j) {
      const int d0 = (t8 + 8 * j) * Gm::EPC;
      if (a.q_aligned) {
        // rows start on 16 bytes: one or two 16-byte loads per chunk
        constexpr int QE = QT == kF32 ? 4 : 2;
        constexpr int N16 = Gm::EPC * QE / 16;
        const char* qp = (const char*)a.q + (qoff + d0) * QE;
#pragma unroll
        for (int v = 0; v < N16; ++v) {
          const uint4 x = k_lane ? *reinterpret_cast<const uint4*>(qp + 16 * v) : make_uint4(0, 0, 0, 0);
          qw[h][(N16 * j + v) * 4] = x.x;
          qw[h][(N16 * j + v) * 4 + 1] = x.y;
          qw[h][(N16 * j + v) * 4 + 2] = x.z;
          qw[h][(N16 * j + v) * 4 + 3] = x.w;
        }
        continue;
      }
      if constexpr (QT == kF32) {
        const float* qp = (const float*)a.q + qoff + d0;
#pragma unroll
        for (int e = 0; e < 4; ++e) qw[h][4 * j + e] = k_lane ? __float_as_uint(qp[e]) : 0u;
      } else {
        const uint16_t* qp = (const uint16_t*)a.q + qoff + d0;
        constexpr int PAIRS = Gm::EPC / 2;
#pragma unroll
        for (int e = 0; e < PAIRS; ++e)
          qw[h][PAIRS * j + e] =
              k_lane ? ((uint32_t)qp[2 * e] | ((uint32_t)qp[2 * e + 1] << 16)) : 0u;
      }
    }
  }
}

template <int KVT, int D, int G, int QT>
__device__ __forceinline__ void load_item_inputs(const SplitArgs& a, int s, int split, int g,
                                                 int lane, ItemIn<KVT, D, G>& in) {
  in.bid_lane = item_bid_lane(a, s, split, lane);
  load_item_q<KVT, D, G, QT>(a, s, g, lane, in.qw);
}

// Lane roles of the dot-product body for KV head g. Lane l works on DPP row r = l / 16:
// as a K-lane it holds 16-byte chunk t8 (+ 8j) of tokens tok_k[0..1] of the block, as
// a V-lane the head dims [cv * D/16, (cv + 1) * D/16) of the row's four tokens tok_v.
template <int KVT, int D>
struct DotLanes {
  int tok_k[2], tok_v[4];
  uint32_t kofs[2], vofs[4];
  int t8, cv;
  bool k_lane;  // false only for rows shorter than 8 chunks
  __device__ __forceinline__ void init(int hkv, int g, int lane) {
    using Gm = Geom<KVT, D>;
    const int r = lane >> 4;
    const int half = (lane >> 3) & 1;
    t8 = lane & 7;
    cv = lane & 15;
    k_lane = t8 < Gm::NCH;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      tok_k[k] = 8 * k + 2 * r + half;
      tok_v[2 * k] = tok_k[k];
      tok_v[2 * k + 1] = 8 * k + 2 * r + (half ^ 1);
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) kofs[k] = (uint32_t)((tok_k[k] * hkv + g) * Gm::ROW + t8 * 16);
#pragma unroll
    for (int x = 0; x < 4; ++x) vofs[x] = (uint32_t)((tok_v[x] * hkv + g) * Gm::ROW + cv * Gm::VB);
  }
};

// Request the K and V rows of pool block bid_raw (the context's tokens first .. first +
// 15) into b; an id outside the pool reads block 0 and marks no token valid. pnew: the
// block position of the step's new token (its row is read from krow_new / vrow_new), or
// outside [0, 16).
template <int KVT, int D>
__device__ __forceinline__ void dot_load(const SplitArgs& a, const DotLanes<KVT, D>& ln,
                                         BlockBuf<KVT, D>& b, int bid_raw, int first, int L,
                                         int pnew, const char* krow_new,
                                         const char* vrow_new) {
  using Gm = Geom<KVT, D>;
  const int64_t blk_bytes = (int64_t)kBlockSize * a.hkv * Gm::ROW;
  const bool ok = (unsigned)bid_raw < (uint64_t)a.num_blocks;
  const int64_t bid = ok ? bid_raw : 0;
  b.nvalid = ok ? min(kBlockSize, L - first) : 0;
  const char* kb = a.kpool + bid * blk_bytes;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const char* kp = ln.tok_k[k] == pnew ? krow_new + ln.t8 * 16 : kb + ln.kofs[k];
#pragma unroll
    for (int c = 0; c < Gm::KC; ++c) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (ln.k_lane) x = ld_stream16(kp + c * 128);
      b.k[k][4 * c] = x.x; b.k[k][4 * c + 1] = x.y; b.k[k][4 * c + 2] = x.z;
      b.k[k][4 * c + 3] = x.w;
    }
  }
  const char* vb = a.vpool + bid * blk_bytes;
#pragma unroll
  for (int x = 0; x < 4; ++x)
    load_dwords<Gm::VW>(ln.tok_v[x] == pnew ? vrow_new + ln.cv * Gm::VB : vb + ln.vofs[x], b.v[x]);
}

template <int KVT, int D, int G>
__device__ __forceinline__ void dot_state_init(DecodeState<KVT, D, G>& st) {
  constexpr float NEG_INF = -__builtin_huge_valf();
#pragma unroll
  for (int h = 0; h < G; ++h) {
    st.m[h] = NEG_INF;
    st.l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < Geom<KVT, D>::EV; ++e) st.acc[h][e] = 0.0f;
  }
}

// Combine the four DPP rows: per head, rescale to the wave max and sum; o = acc / l in
// lanes 0..15 (lane c: head dims c*D/16 ..), lse2 = log2 of the split's sum of exp2.
template <int KVT, int D, int G>
__device__ __forceinline__ void dot_finish(DecodeState<KVT, D, G>& st,
                                           float (&o)[G][Geom<KVT, D>::EV], float (&lse2)[G]) {
  using Gm = Geom<KVT, D>;
  constexpr float NEG_INF = -__builtin_huge_valf();
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float M = xor32_max(xor16_max(st.m[h]));
    const float f = st.m[h] == NEG_INF ? 0.0f : fast_exp2(st.m[h] - M);
    // l counts this lane's own tokens; the mirrored lane of the row holds the other two
    const float lr = xor32_sum(xor16_sum((st.l[h] + dpp<kRowMirror>(st.l[h])) * f));
#pragma unroll
    for (int e = 0; e < Gm::EV; ++e) st.acc[h][e] = xor32_sum(xor16_sum(st.acc[h][e] * f));
    const float inv_l = 1.0f / lr;
    lse2[h] = M + __log2f(lr);
#pragma unroll
    for (int e = 0; e < Gm::EV; ++e) o[h][e] = st.acc[h][e] * inv_l;
  }
}

// One work item (sequence s, split, kv head g) on one wavefront: the split's partial
// attention for the G heads of group g, normalised (o = sum p v / sum p) with its
// log2-sum-exp, in lanes 0..15 (lane c holds head dims [c*D/16, (c+1)*D/16)). A split
// past the context (possible in the fused schedule) yields lse2 = -inf.
// krow_new / vrow_new (may be null): the K / V row of the context's last token taken
// from the step's input instead of the pool, where a concurrent store is writing it.
__device__ __forceinline__ void balance_issue(int* progress, int done);

// BALANCE: progress is an LDS array with one entry per wave of an eight-wave workgroup
// whose waves w and w + 4 run items of equal length (see balance_issue).
template <int KVT, int D, int G, bool BALANCE = false>
__device__ __forceinline__ void item_partial(const SplitArgs& a, const ItemIn<KVT, D, G>& in,
                                             int split, int g, int L, int lane,
                                             float (&o)[G][Geom<KVT, D>::EV], float (&lse2)[G],
                                             const char* krow_new = nullptr,
                                             const char* vrow_new = nullptr,
                                             int* progress = nullptr) {
  static_assert(!kQuant<KVT>, "quantised pools take the matrix-core item");
  const int t0 = split * a.split_tokens;
  const int t1 = min(L, t0 + a.split_tokens);
  const int jb0 = t0 / kBlockSize;
  // wave-uniform (the split and the length are; the compiler cannot see it), so the
  // block loop below is a scalar loop
  const int nblk = __builtin_amdgcn_readfirstlane(t1 > t0 ? (t1 - t0 + kBlockSize - 1) / kBlockSize : 0);
  const int bid_lane = in.bid_lane;
  DotLanes<KVT, D> ln;
  ln.init(a.hkv, g, lane);

  auto load = [&](BlockBuf<KVT, D>& b, int j) {
    const int first = (jb0 + j) * kBlockSize;
    // position of the step's new token in this block (only the context's last block
    // has one in [0, 16)); lanes holding it read the input row instead of the pool
    const int pnew = krow_new != nullptr ? L - 1 - first : -1;
    dot_load<KVT, D>(a, ln, b, __builtin_amdgcn_readlane(bid_lane, j), first, L, pnew, krow_new,
                     vrow_new);
  };

  DecodeState<KVT, D, G> st;
  dot_state_init(st);
  auto process = [&](const BlockBuf<KVT, D>& b) {
    if (b.nvalid == kBlockSize)
      process_block<KVT, D, G, false>(b, st, in.qw, a.scale_log2, ln.tok_k, ln.tok_v);
    else
      process_block<KVT, D, G, true>(b, st, in.qw, a.scale_log2, ln.tok_k, ln.tok_v);
  };

  // ring of NB block buffers: block j + NB - 1 is requested before block j is used
  constexpr int NB = RingDepth<G>::value;
  BlockBuf<KVT, D> ring[NB];
  if (nblk > 0) {
    // every request is unconditional (past the last block, the last block is requested
    // again: its lines were just read), so the same loads are in flight on every path
    // and waiting for block j never waits for the blocks requested after it
#pragma unroll
    for (int p = 0; p < NB - 1; ++p) load(ring[p], min(p, nblk - 1));
    int j0 = 0;
    for (; j0 + NB <= nblk; j0 += NB) {
      if constexpr (BALANCE) balance_issue(progress, j0);
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        load(ring[(u + NB - 1) % NB], min(j0 + u + NB - 1, nblk - 1));
        process(ring[u]);
      }
    }
    if constexpr (BALANCE) __builtin_amdgcn_s_setprio(0);
    // fewer than NB blocks left: all of them requested already
#pragma unroll
    for (int u = 0; u < NB - 1; ++u)
      if (j0 + u < nblk) process(ring[u]);
  }
  dot_finish(st, o, lse2);
}

// ---------------------------------------------------------------- matrix-core item
// The same item (one KV head, G query heads, one split) for bf16 / FP8 / INT8 pools,
// with the two products of each 16-token block on the matrix cores: S = K Q^T on
// v_mfma_f32_16x16x32_bf16 (M = the block's 16 tokens, N = the G heads padded to 16,
// contraction over head_dim) and O += P V on v_mfma_f32_16x16x16_bf16 (M = heads,
// contraction over the 16 tokens, N = 16 head-dim slots per step). Only G of the 16
// head columns are used; the matrix cores are not the bound, the vector ALU was, and
// the per-block vector work drops to the code conversions and a 4-score softmax.
//
// Lane l (n = l % 16, kg = l / 16):
//  * K operand at step st: token n of the block, eight head dims starting at
//    mma_kdim<E>(st, kg); the Q operand holds the same dims of head n (zero for
//    n >= G). The order is chosen so that each K load instruction of a wave covers 64
//    contiguous bytes of every token row it touches.
//  * S (accumulator): tokens 4kg + i (i < 4) of head n. The softmax statistics of head
//    n are shared by the four lanes n + 16kg (lane-swap reductions).
//  * P operand: the same (head n, tokens 4kg + i): straight from S.
//  * V operand at step t: tokens 4kg + i, head dim (D/16)*n + t; a lane reads the
//    D/16 contiguous dims of its four tokens and builds one bf16 quad per step.
//  * O (accumulator) at step t: heads 4kg + i, dim (D/16)*n + t.
// The result goes through LDS (`stage`, this wave's [G][D] floats) into the layout of
// item_partial's output (lane c < 16: dims c*D/16 .. of every head), so the merges
// downstream are shared. Probabilities enter the PV product as bf16: for bf16 pools as a
// hi + lo pair (two products, P exact to ~2^-17, like the fp32 P of item_partial); for
// quantised pools once rounded, with the V scale folded in.
// Which item body a (pool dtype, group size) takes, in every schedule alike so that
// the schedules keep giving identical bits. Measured on bf16 calls that stream from
// HBM (256 sequences, contexts 1K-32K), the dot-product body, whose K loads cover
// whole 128-byte lines per instruction, is faster for small query groups (G = 4: 5.8
// against 5.5 TB/s; G = 1: 6.3 against 6.2), equal at G = 6, and slower at G = 8 (4.9
// against 5.0); at G = 6 the matrix cores also cut the latency-bound small-batch
// call (13.9 against 16.2 us at 8 sequences x 12/2 heads).
template <int KVT, int G>
struct MmaPath {
  static constexpr bool value = kQuant<KVT> || (KVT == kBF16 && G > 4);
};
constexpr float kMmaLazyMax = 8.0f;  // log2 headroom of the lazily moved reference max
// blocks in flight per wave: as many as fit in 256 registers with the wave count the
// kernels run at (a bf16 block buffer is twice a quantised one); the persistent kernel
// fits three for every dtype
template <int KVT>
struct MmaRing {
  static constexpr int value = kQuant<KVT> ? 3 : 2;
};

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// First of the eight head dims that lane group kg holds at QK step st (pools of E-byte
// elements): bf16 rows are read in 16-byte chunks 4*st + kg, 1-byte rows in 16-byte
// chunks 4*(st/2) + kg of which each step takes one half.
template <int E>
__device__ __forceinline__ int mma_kdim(int st, int kg) {
  return E == 2 ? 32 * st + 8 * kg : 64 * (st >> 1) + 16 * kg + 8 * (st & 1);
}

template <int D>
struct MmaIn {
  uint4 qb[D / 32];  // Q operand (bf16x8) of each QK step
  int bid_lane;      // block id of block `lane` of the split
};

template <int E, int D, int G>
__device__ __forceinline__ void load_mma_inputs(const SplitArgs& a, int s, int split, int g,
                                                int lane, MmaIn<D>& in) {
  const int jb0 = split * (a.split_tokens / kBlockSize);
  const int32_t* bt_row = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  in.bid_lane = (lane < a.split_tokens / kBlockSize && jb0 + lane < a.max_blocks_per_seq)
                    ? bt_row[jb0 + lane]
                    : 0;
  const int n = lane & 15, kg = lane >> 4;
#pragma unroll
  for (int st = 0; st < D / 32; ++st) in.qb[st] = make_uint4(0, 0, 0, 0);
  if (n < G) {
    const uint16_t* qp = (const uint16_t*)a.q + (int64_t)s * a.q_st +
                         (int64_t)(g * G + n) * a.q_sh;
#pragma unroll
    for (int st = 0; st < D / 32; ++st) {
      const int d0 = mma_kdim<E>(st, kg);
      if (a.q_aligned) {
        in.qb[st] = *reinterpret_cast<const uint4*>(qp + d0);
      } else {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          w[e] = (uint32_t)qp[d0 + 2 * e] | ((uint32_t)qp[d0 + 2 * e + 1] << 16);
        in.qb[st] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  }
}

template <int KVT, int D>
struct MmaBuf {
  static constexpr int E = ElemBytes<KVT>::value;
  static constexpr int KW = D / 4 * E / 4;     // dwords of K per lane (token n, D/4 dims)
  static constexpr int VW = D / 16 * E / 4;    // dwords of V per lane per token (D/16 dims)
  uint32_t k[KW];
  uint32_t v[4][VW > 0 ? VW : 1];
  float ks[4], vs[4];  // scales of tokens 4kg + i (quantised pools)
  int nvalid;
};

// Issue fairness between the two waves of a SIMD in the single-launch kernel (eight
// waves, wave w and w + 4 on one SIMD, equal work). The SIMD's arbiter favours the
// older wave, so without this wave w finished its split ~12 us before wave w + 4 on
// the 64 x 8192 FP8 decode and the SIMD ran its last stretch with one wave, exposing
// load latency. Each wave posts its block count in LDS; the one behind its partner
// raises its issue priority. Scheduling only: the arithmetic is unchanged.
__device__ __forceinline__ void balance_issue(int* progress, int done) {
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0)
    __hip_atomic_store(&progress[wave], done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  // At the first ring cycle both waves are at zero: nothing to balance, and the
  // partner may not have written its entry yet (until it does, LDS holds whatever an
  // earlier workgroup left there). The partner, started with this wave, writes it
  // before its first block load, so a later cycle reads a current entry; a late one
  // would only misplace one cycle's priority.
  if (done == 0) {
    __builtin_amdgcn_s_setprio(0);
    return;
  }
  // uniform, so that the branch is a scalar one (s_setprio ignores the exec mask)
  const int other = __builtin_amdgcn_readfirstlane(
      __hip_atomic_load(&progress[wave ^ 4], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
  if (done < other) __builtin_amdgcn_s_setprio(2);
  else __builtin_amdgcn_s_setprio(0);
}

// OUT_REGS = false: the normalised result is left in sw only ([G][D], the layout the
// single-launch kernel merges from), and o is not written.
template <int KVT, int D, int G, int NB = MmaRing<KVT>::value, bool OUT_REGS = true>
__device__ __forceinline__ void item_partial_mma(const SplitArgs& a, const MmaIn<D>& in,
                                                 int split, int g, int L, int lane,
                                                 float (&o)[G][D / 16], float (&lse2)[G],
                                                 float (&sw)[G][D],
                                                 const char* krow_new = nullptr,
                                                 const char* vrow_new = nullptr,
                                                 int* progress = nullptr) {
  using Bf = MmaBuf<KVT, D>;
  constexpr int E = Bf::E;
  constexpr int ROW = D * E;
  constexpr int QS = D / 32;  // QK steps
  constexpr int PS = D / 16;  // PV steps (head-dim slots per lane)
  constexpr int KB = D / 4 * E;  // K bytes per lane per token
  constexpr int VBY = D / 16 * E;
  constexpr float NEG_INF = -__builtin_huge_valf();
  static_assert(G <= 8, "two lane groups of O rows");
  // the split and the length are the same for the whole wave
  L = __builtin_amdgcn_readfirstlane(L);
  split = __builtin_amdgcn_readfirstlane(split);
  const int t0 = split * a.split_tokens;
  const int t1 = min(L, t0 + a.split_tokens);
  const int jb0 = t0 / kBlockSize;
  const int nblk = t1 > t0 ? (t1 - t0 + kBlockSize - 1) / kBlockSize : 0;
  const int n = lane & 15, kg = lane >> 4;
  const int64_t blk_bytes = (int64_t)kBlockSize * a.hkv * ROW;
  const uint32_t koff = (uint32_t)((n * a.hkv + g) * ROW + kg * 16);
  uint32_t voff[4], sofs[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    voff[r] = (uint32_t)(((4 * kg + r) * a.hkv + g) * ROW + n * VBY);
    sofs[r] = (uint32_t)((4 * kg + r) * a.hkv + g);
  }

  auto load = [&](Bf& b, int j) {
    const int bid_raw = __builtin_amdgcn_readlane(in.bid_lane, j);
    const bool ok = (unsigned)bid_raw < (uint64_t)a.num_blocks;
    const int64_t bid = ok ? bid_raw : 0;
    const int first = (jb0 + j) * kBlockSize;
    b.nvalid = ok ? min(kBlockSize, L - first) : 0;
    // block bases are wave-uniform (scalar registers); lane offsets are 32-bit, so the
    // loads use scalar-base addressing
    const char* kb = a.kpool + bid * blk_bytes;
    const char* vb = a.vpool + bid * blk_bytes;
    // the step's new token (context position L - 1) is read from the input row (only
    // the bf16 single-launch step folds the store in)
    const int pnew = !kQuant<KVT> && krow_new != nullptr ? L - 1 - first : -1;
    // 16-byte chunks kg, kg + 4, ... of the row (see mma_kdim)
    const char* kp = !kQuant<KVT> && n == pnew ? krow_new + kg * 16 : kb + koff;
#pragma unroll
    for (int c = 0; c < Bf::KW / 4; ++c) {
      const uint4 x = ld_stream16(kp + 64 * c);
      b.k[4 * c] = x.x; b.k[4 * c + 1] = x.y; b.k[4 * c + 2] = x.z; b.k[4 * c + 3] = x.w;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
      load_dwords<Bf::VW>(!kQuant<KVT> && 4 * kg + r == pnew ? vrow_new + n * VBY : vb + voff[r],
                          b.v[r]);
    if constexpr (kQuant<KVT>) {
      const char* ksb = reinterpret_cast<const char*>(a.kscale + bid * kBlockSize * a.hkv);
      const char* vsb = reinterpret_cast<const char*>(a.vscale + bid * kBlockSize * a.hkv);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        b.ks[r] = *reinterpret_cast<const float*>(ksb + 4 * sofs[r]);
        b.vs[r] = *reinterpret_cast<const float*>(vsb + 4 * sofs[r]);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) b.ks[r] = b.vs[r] = 1.0f;
    }
  };

  f32x4_t oacc[PS];
#pragma unroll
  for (int t = 0; t < PS; ++t) oacc[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = NEG_INF, l_run = 0.0f;  // of head n, over this lane's tokens (l)

  auto process = [&](const Bf& b) {
    // ---- S = K Q^T: lane gets tokens 4kg + i of head n
    f32x4_t sacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int st = 0; st < QS; ++st) {
      uint4 kk;
      if constexpr (KVT == kBF16) {
        kk = make_uint4(b.k[4 * st], b.k[4 * st + 1], b.k[4 * st + 2], b.k[4 * st + 3]);
      } else {
        const int w0 = 4 * (st >> 1) + 2 * (st & 1);
        kk = make_uint4(q8x2_to_bf16x2<KVT>(b.k[w0], false), q8x2_to_bf16x2<KVT>(b.k[w0], true),
                        q8x2_to_bf16x2<KVT>(b.k[w0 + 1], false),
                        q8x2_to_bf16x2<KVT>(b.k[w0 + 1], true));
      }
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kk),
                                                     __builtin_bit_cast(bf16x8_t, in.qb[st]),
                                                     sacc, 0, 0, 0);
    }
    // ---- online softmax of head n (log2 units, scale folded in)
    float x[4];
    bool valid[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      valid[i] = 4 * kg + i < b.nvalid;
      const float y = sacc[i] * (a.scale_log2 * b.ks[i]);
      x[i] = valid[i] ? y : NEG_INF;
    }
    const float mb = xor32_max(xor16_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]))));
    // reference max moved only past 2^kMmaLazyMax of headroom (o / l is the same for
    // any reference); a head that saw no valid token keeps m = -inf and zeros
    const float m_new = mb > m_run + kMmaLazyMax ? mb : m_run;
    const float m_use = m_new == NEG_INF ? 0.0f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = valid[i] ? fast_exp2(x[i] - m_use) : 0.0f;
    l_run = fmaf(l_run, alpha, (p[0] + p[1]) + (p[2] + p[3]));
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
      // O rows are heads 4kg + i: their factors come from lanes 4kg + i (n = head)
      float ah[8];
#pragma unroll
      for (int h = 0; h < 8; ++h) ah[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), h));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float f = kg == 0 ? ah[i] : ah[4 + i];
#pragma unroll
        for (int t = 0; t < PS; ++t) oacc[t][i] *= f;
      }
    }
    // P operand (V scales folded in for quantised pools; an invalid token's scale may be
    // anything, so its probability stays an exact 0 rather than 0 * scale)
    float pv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pv[i] = kQuant<KVT> ? (valid[i] ? p[i] * b.vs[i] : 0.0f) : p[i];
    const bf2 p01 = bf16x2_rne(pv[0], pv[1]);
    const bf2 p23 = bf16x2_rne(pv[2], pv[3]);
    const s16x4_t pa = __builtin_bit_cast(s16x4_t, make_uint2(__builtin_bit_cast(uint32_t, p01),
                                                              __builtin_bit_cast(uint32_t, p23)));
    s16x4_t pl;  // bf16 pools: the rounding residue of P, exact to ~2^-17 together
    if constexpr (KVT == kBF16) {
      const bf2 r01 = bf16x2_rne(pv[0] - (float)p01[0], pv[1] - (float)p01[1]);
      const bf2 r23 = bf16x2_rne(pv[2] - (float)p23[0], pv[3] - (float)p23[1]);
      pl = __builtin_bit_cast(s16x4_t, make_uint2(__builtin_bit_cast(uint32_t, r01),
                                                  __builtin_bit_cast(uint32_t, r23)));
    }
    // ---- O += P V: tokens of invalid rows are exact zeros (garbage could be NaN)
    uint32_t vw[4][D / 32];  // bf16 pairs of this lane's D/16 dims, per token
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (KVT == kBF16) {
#pragma unroll
        for (int w = 0; w < Bf::VW; ++w) vw[r][w] = valid[r] ? b.v[r][w] : 0u;
      } else {
        // codes -> bf16 pairs (exact)
#pragma unroll
        for (int w = 0; w < Bf::VW; ++w) {
          const uint32_t c = valid[r] ? b.v[r][w] : 0u;
          vw[r][2 * w] = q8x2_to_bf16x2<KVT>(c, false);
          vw[r][2 * w + 1] = q8x2_to_bf16x2<KVT>(c, true);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < PS; ++t) {
      // bf16 quad (tokens 4kg .. 4kg+3) of head dim slot t: one byte permute per pair
      const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
      const uint32_t lo = __builtin_amdgcn_perm(vw[1][t >> 1], vw[0][t >> 1], sel);
      const uint32_t hi = __builtin_amdgcn_perm(vw[3][t >> 1], vw[2][t >> 1], sel);
      const s16x4_t vb4 = __builtin_bit_cast(s16x4_t, make_uint2(lo, hi));
      oacc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb4, oacc[t], 0, 0, 0);
      if constexpr (KVT == kBF16)
        oacc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pl, vb4, oacc[t], 0, 0, 0);
    }
  };

  // ring of NB block buffers, requests unconditional (see item_partial)
  Bf ring[NB];

  if (nblk > 0) {
#pragma unroll
    for (int p = 0; p < NB - 1; ++p) load(ring[p], min(p, nblk - 1));
    int j0 = 0;
    for (; j0 + NB <= nblk; j0 += NB) {
      if (progress != nullptr) balance_issue(progress, j0);
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        load(ring[(u + NB - 1) % NB], min(j0 + u + NB - 1, nblk - 1));
        process(ring[u]);
      }
    }
    if (progress != nullptr) __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int u = 0; u < NB - 1; ++u)
      if (j0 + u < nblk) process(ring[u]);
  }

  // ---- per head n: totals over the four lane groups, then O rows normalised
  const float l_tot = xor32_sum(xor16_sum(l_run));
  const float lse = l_tot > 0.0f ? m_run + __log2f(l_tot) : NEG_INF;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * kg + i;
    const float f0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(inv), i));
    const float f1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(inv), 4 + i));
    const float f = kg == 0 ? f0 : f1;
    if (h < G) {
#pragma unroll
      for (int t = 0; t < PS; ++t) sw[h][PS * n + t] = oacc[t][i] * f;
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    lse2[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lse), h));
    if (OUT_REGS && lane < 16) {
#pragma unroll
      for (int e = 0; e < PS; ++e) o[h][e] = sw[h][PS * lane + e];
    }
  }
}

// Result of one item in the split-then-merge schedule: the final output row when the
// sequence has a single split, else the partial in the workspace. o and lse2 as the item
// bodies leave them (lanes 0..15).
// First row of the G split-partial rows of (sequence s, split, KV head g): rows are laid
// out [s][split][kv head][G].
__device__ __forceinline__ int64_t split_row(const SplitArgs& a, int s, int split, int g, int G) {
  return (((int64_t)s * a.max_splits + split) * a.hkv + g) * G;
}

template <int D, int G, int QT>
__device__ __forceinline__ void write_item_result(const SplitArgs& a, int s, int split, int g,
                                                  int nsplit, int lane,
                                                  const float (&o)[G][D / 16],
                                                  const float (&lse2)[G]) {
  constexpr int EV = D / 16;
  if (lane >= 16) return;
  const int cv = lane;
  const int d0 = cv * EV;
  if (nsplit == 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const int64_t off = (int64_t)s * a.out_st + (int64_t)(g * G + h) * a.out_sh + d0;
      if constexpr (QT == kF32) {
#pragma unroll
        for (int e = 0; e < EV; ++e) ((float*)a.out)[off + e] = o[h][e];
      } else {
        uint32_t w[EV / 2];
#pragma unroll
        for (int e = 0; e < EV / 2; ++e)
          w[e] = (uint32_t)f32_to_bf16(o[h][2 * e]) | ((uint32_t)f32_to_bf16(o[h][2 * e + 1]) << 16);
        uint16_t* op = (uint16_t*)a.out + off;
        bool stored = false;
        if constexpr (EV == 8) {
          if (a.out_aligned) {
            *reinterpret_cast<uint4*>(op) = make_uint4(w[0], w[1], w[2], w[3]);
            stored = true;
          }
        }
        if (!stored) {
#pragma unroll
          for (int e = 0; e < EV / 2; ++e) {
            op[2 * e] = (uint16_t)w[e];
            op[2 * e + 1] = (uint16_t)(w[e] >> 16);
          }
        }
      }
    }
    return;
  }
  // Split partials, rows [s][split][kv head][G] (o: D floats per row, lse: one), so an
  // item's G rows and the items of a persistent step (consecutive KV heads of one
  // split) are contiguous. o goes out with non-temporal stores: on the 256-sequence
  // decode the partials written through the caches slowed the whole read stream, 1776 us
  // per call against 1701 with non-temporal stores (bit-identical results).
  const int64_t row0 = split_row(a, s, split, g, G);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float* wo = a.ws_o + (row0 + h) * D + d0;
#pragma unroll
    for (int e = 0; e < EV; ++e) __builtin_nontemporal_store(o[h][e], wo + e);
  }
  // lanes 0 .. G-1 store the G lse values as one contiguous run (plain stores measured
  // a little faster than non-temporal ones here)
  float l = lse2[0];
#pragma unroll
  for (int h = 1; h < G; ++h) l = cv == h ? lse2[h] : l;
  if (cv < G) a.ws_lse[row0 + cv] = l;
}

template <int KVT, int D, int G, int QT, int NBM = MmaRing<KVT>::value>
__device__ __forceinline__ void decode_item(const SplitArgs& a, int s, int split, int g,
                                            int lane) {
  using Gm = Geom<KVT, D>;
  static_assert(Gm::EV == D / 16, "one output layout for both item bodies");
  float o[G][Gm::EV], lse2[G];
  int nsplit;
  if constexpr (MmaPath<KVT, G>::value) {
    __shared__ float stage[kMaxItemWaves][G][D];  // one slice per wave of the workgroup
    MmaIn<D> in;
    load_mma_inputs<ElemBytes<KVT>::value, D, G>(a, s, split, g, lane, in);
    const int L = clamped_len(a, s);
    nsplit = num_splits(L, a.split_tokens);
    item_partial_mma<KVT, D, G, NBM>(a, in, split, g, L, lane, o, lse2, stage[threadIdx.x >> 6]);
  } else {
    ItemIn<KVT, D, G> in;
    load_item_inputs<KVT, D, G, QT>(a, s, split, g, lane, in);
    const int L = clamped_len(a, s);
    nsplit = num_splits(L, a.split_tokens);
    item_partial<KVT, D, G>(a, in, split, g, L, lane, o, lse2);
  }
  write_item_result<D, G, QT>(a, s, split, g, nsplit, lane, o, lse2);
}

// One work item per wavefront over the full (sequence, max_splits, kv head) range, kv
// head fastest; items past a sequence's split count exit at once. Used when the batch
// is too large for the compact schedule below.
template <int KVT, int D, int G, int QT>
__global__ void __launch_bounds__(64 * kWaves) decode_split_kernel(SplitArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int g = (int)(item % a.hkv);
  const int64_t rest = item / a.hkv;
  const int split = (int)(rest % a.max_splits);
  const int s = (int)(rest / a.max_splits);
  if (s >= a.num_seqs) return;
  const int L = clamped_len(a, s);
  const int nsplit = num_splits(L, a.split_tokens);
  if (split >= nsplit) return;
  decode_item<KVT, D, G, QT>(a, s, split, g, lane);
}

// Compact persistent schedule. Every workgroup builds, in LDS, the same enumeration of
// exactly the existing (sequence, split, kv head) items (pair_order; kv head fastest,
// eight per workgroup step) and draws steps from a device-wide counter (without a
// workspace: the b-th contiguous share of the steps). Dispatching only real work
// matters for skewed batches: padding the grid to max_context_len would launch mostly
// empty workgroups. At most kMaxCompactSeqs sequences (the LDS tables).
constexpr int kMaxCompactSeqs = 4096;

// The single-launch schedule's workgroup: eight waves, in one unit or two. Quantised
// pools (128-byte head rows at two KV heads: half of each token's 256-byte record)
// take two units of four waves, so that both halves of a record are read by one CU at
// about the same time; other pools one unit of eight.
constexpr int kFusedWaves = 8;
template <int KVT>
struct FusedUnits {
  static constexpr int value = kQuant<KVT> ? 2 : 1;
};
// Partials are merged in groups of this many consecutive splits (a unit's waves; see
// the merge below), in both schedules alike.
template <int KVT>
struct GroupSplits {
  static constexpr int value = kFusedWaves / FusedUnits<KVT>::value;
};
constexpr int kMaxGroupSplits = kFusedWaves;
// Calls with at most this many single-launch workgroups take that schedule; larger
// ones the persistent split kernel plus a merge launch.
constexpr int64_t kFusedMaxWorkgroups = 1024;
// Words of the workspace's counter block: the single-launch schedule uses one per
// (sequence, KV head) when a sequence has two or more groups (the launch checks that
// they stay below the next two); the persistent schedule's work counter and leaver
// count use the last two.
constexpr int kCompactQueueWord = kDecodeCounters - 2;
constexpr int kCompactDoneWord = kDecodeCounters - 1;

template <int NWAVES>
__device__ __forceinline__ int block_exclusive_scan(int x, int* wave_sums, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wave_sums[wave] = incl;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < NWAVES; ++w) {
    const int v = wave_sums[w];
    before += w < wave ? v : 0;
    total += v;
  }
  __syncthreads();
  return before + incl - x;
}

// Waves (items) per workgroup step of the persistent schedule. Items are enumerated
// KV head fastest, so a step of eight holds all heads of a (sequence, split) at eight
// KV heads (pairs of heads at two): a CU reads whole token records of the pool, not
// halves of them, at the same occupancy as two four-wave workgroups.
constexpr int kCompactWaves = 8;
static_assert(kCompactWaves <= kMaxItemWaves && kWaves <= kMaxItemWaves, "decode_item's LDS slices");

// Order in which the persistent schedule hands out the (sequence, split) pairs: every
// full split first, sequence by sequence, then the sequences' shorter last splits from
// the longest to the shortest (kLenClasses classes of their block count, each class in
// sequence order). The shortest items are drawn last, so the workgroups run out of work
// at about the same time. The order changes no result: each split's partial is computed
// on its own and the merge takes them in split order.
// By the whole workgroup: cumf[s] = full splits of the sequences before s (s <=
// num_seqs), pseq[r] = the sequence of the r-th short split; full = the number of full
// splits. Returns the number of pairs. Ends with a barrier.
constexpr int kLenClasses = 8;
__device__ __forceinline__ int pair_order(const SplitArgs& a, int* cumf, short* pseq,
                                          int* wave_sums, int& full) {
  const int spb = a.split_tokens / kBlockSize;  // blocks of a full split
  // the first 64 * kCompactWaves lengths are read once and reused by every pass
  const int L0 = (int)threadIdx.x < a.num_seqs ? clamped_len(a, (int)threadIdx.x) : 0;
  auto len = [&](int base, int s) {
    return base == 0 ? L0 : (s < a.num_seqs ? clamped_len(a, s) : 0);
  };
  int carry = 0;
  for (int base = 0; base < a.num_seqs; base += 64 * kCompactWaves) {
    const int s = base + (int)threadIdx.x;
    const int L = len(base, s);
    const int n = L > 0 ? L / a.split_tokens : 0;
    int tot;
    const int ex = block_exclusive_scan<kCompactWaves>(n, wave_sums, tot);
    if (s < a.num_seqs) cumf[s] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) cumf[a.num_seqs] = carry;
  full = carry;
  int np = 0;
  for (int c = 0; c < kLenClasses; ++c) {
    for (int base = 0; base < a.num_seqs; base += 64 * kCompactWaves) {
      const int s = base + (int)threadIdx.x;
      const int L = len(base, s);
      const int rem = L > 0 ? L % a.split_tokens : 0;
      const int nb = (rem + kBlockSize - 1) / kBlockSize;  // 1 .. spb when rem > 0
      const bool mine = rem > 0 && (spb - nb) * kLenClasses / spb == c;
      int tot;
      const int ex = block_exclusive_scan<kCompactWaves>(mine ? 1 : 0, wave_sums, tot);
      if (mine) pseq[np + ex] = (short)s;
      np += tot;
    }
  }
  __syncthreads();
  return carry + np;
}

// Sequence of full split `pair`: the largest s with cum[s] <= pair (sequences without
// full splits have cum[s] == cum[s + 1]).
__device__ __forceinline__ int pair_sequence(const int* cum, int num_seqs, int pair) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cum[mid] <= pair) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <int KVT, int D, int G, int QT>
__global__ void __launch_bounds__(64 * kCompactWaves, 1)
    decode_compact_kernel(SplitArgs a) {
  __shared__ int cumf[kMaxCompactSeqs + 1];  // see pair_order
  __shared__ short pseq[kMaxCompactSeqs];
  __shared__ int wave_sums[kCompactWaves];
  __shared__ int progress[kCompactWaves];
  // (a scalar wave index makes the compiler spill the bf16 G = 4 item's registers)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (threadIdx.x < kCompactWaves) progress[threadIdx.x] = 0;
  int full = 0;
  const int pairs = pair_order(a, cumf, pseq, wave_sums, full);  // ends with a barrier
  const int64_t entries = (int64_t)pairs * a.hkv;
  if constexpr (!MmaPath<KVT, G>::value) {
    if (a.knew != nullptr && blockIdx.x == 0) {
      // decode step: a sequence without items (context length <= 0, outside the
      // contract) still gets its new rows stored, as pa_store_kv would store them
      using Gm = Geom<KVT, D>;
      for (int sq = (int)threadIdx.x; sq < a.num_seqs; sq += 64 * kCompactWaves) {
        const int64_t slot = a.slots[sq];
        if (clamped_len(a, sq) > 0 || slot < 0 || slot >= a.num_blocks * kBlockSize) continue;
        const int64_t base = (slot / kBlockSize) * kBlockSize * a.hkv * Gm::ROW +
                             (slot % kBlockSize) * a.hkv * Gm::ROW;
        for (int g = 0; g < a.hkv; ++g) {
          const char* kr = a.knew + ((int64_t)sq * a.knew_st + (int64_t)g * a.knew_sh) * Gm::E;
          const char* vr = a.vnew + ((int64_t)sq * a.vnew_st + (int64_t)g * a.vnew_sh) * Gm::E;
          for (int c = 0; c < Gm::NCH; ++c) {
            const int64_t off = base + (int64_t)g * Gm::ROW + c * 16;
            *reinterpret_cast<uint4*>(const_cast<char*>(a.kpool) + off) =
                *reinterpret_cast<const uint4*>(kr + c * 16);
            *reinterpret_cast<uint4*>(const_cast<char*>(a.vpool) + off) =
                *reinterpret_cast<const uint4*>(vr + c * 16);
          }
        }
      }
    }
  }
  const int64_t steps = (entries + kCompactWaves - 1) / kCompactWaves;
  // this wave's item of step st: (sequence, split, KV head), or none
  auto locate = [&](int64_t st, int& sq, int& split, int& g) {
    const int64_t e = st * kCompactWaves + wave;
    if (st >= steps || e >= entries) return false;
    g = (int)(e % a.hkv);
    const int pair = (int)(e / a.hkv);
    if (pair < full) {
      sq = pair_sequence(cumf, a.num_seqs, pair);
      split = pair - cumf[sq];
    } else {
      sq = pseq[pair - full];
      split = clamped_len(a, sq) / a.split_tokens;  // the last split
    }
    sq = __builtin_amdgcn_readfirstlane(sq);
    split = __builtin_amdgcn_readfirstlane(split);
    return true;
  };
  // the items of workgroup step st (one per wave); the dot-product items of a step have
  // equal lengths (same sequence and split) when the KV heads are a multiple of eight,
  // and the issue of each SIMD's two waves is balanced
  auto run_step = [&](int64_t st) {
    int sq = 0, split = 0, g = 0;
    if (!locate(st, sq, split, g)) return;
    if constexpr (MmaPath<KVT, G>::value) {
      decode_item<KVT, D, G, QT, 3>(a, sq, split, g, lane);
    } else {
      using Gm = Geom<KVT, D>;
      ItemIn<KVT, D, G> in;
      load_item_inputs<KVT, D, G, QT>(a, sq, split, g, lane, in);
      const int L = clamped_len(a, sq);
      const int nsplit = num_splits(L, a.split_tokens);
      // Decode step (a.knew set): the wave of the split holding the context's last token
      // copies that token's K and V rows of its head from the step's input into the
      // pool before its item's block loads (its query and block-id loads are already
      // out), then runs the item from the pool. Only this wave reads that row in the
      // launch, and its block loads follow the copy in the wave's memory order. slot <
      // 0: no new row, the pool holds the context.
      if (a.knew != nullptr && split == nsplit - 1) {
        const int64_t slot = ld_uniform(a.slots + sq);
        if (slot >= 0 && slot < a.num_blocks * kBlockSize && lane < 2 * Gm::NCH) {
          // lanes 0 .. NCH-1 copy the K row, the next NCH lanes the V row (16 bytes each)
          const bool is_v = lane >= Gm::NCH;
          const int chunk = is_v ? lane - Gm::NCH : lane;
          const char* src = is_v ? a.vnew + ((int64_t)sq * a.vnew_st + (int64_t)g * a.vnew_sh) * Gm::E
                                 : a.knew + ((int64_t)sq * a.knew_st + (int64_t)g * a.knew_sh) * Gm::E;
          const uint4 x = *reinterpret_cast<const uint4*>(src + chunk * 16);
          const int64_t off = (slot / kBlockSize) * kBlockSize * a.hkv * Gm::ROW +
                              ((slot % kBlockSize) * a.hkv + g) * Gm::ROW + chunk * 16;
          *reinterpret_cast<uint4*>(const_cast<char*>(is_v ? a.vpool : a.kpool) + off) = x;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
      float o[G][Gm::EV], lse2[G];
      item_partial<KVT, D, G, true>(a, in, split, g, L, lane, o, lse2, nullptr, nullptr,
                                    progress);
      write_item_result<D, G, QT>(a, sq, split, g, nsplit, lane, o, lse2);
      if (lane == 0)
        __hip_atomic_store(&progress[wave], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  };
  if (a.counters == nullptr) {
    // no workspace (every context fits one split): the b-th contiguous share of steps
    const int64_t first = (int64_t)blockIdx.x * steps / gridDim.x;
    const int64_t last = ((int64_t)blockIdx.x + 1) * steps / gridDim.x;
    for (int64_t st = first; st < last; ++st) run_step(st);
    return;
  }
  // Steps are handed out by a device-wide counter, so workgroups that drew short items
  // take more of them and the call ends with at most one step of imbalance. The next
  // step is drawn while the current one runs. The last workgroup to leave returns the
  // counters to zero for the next call.
  unsigned* queue = a.counters + kCompactQueueWord;
  unsigned* done = a.counters + kCompactDoneWord;
  __shared__ unsigned next_step;
  unsigned nxt = 0;
  if (threadIdx.x == 0) {
    nxt = __hip_atomic_fetch_add(queue, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    next_step = nxt;
  }
  __syncthreads();
  int64_t st = next_step;
  while (st < steps) {
    if (threadIdx.x == 0)
      nxt = __hip_atomic_fetch_add(queue, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    run_step(st);
    __syncthreads();  // every wave has read next_step for this round
    if (threadIdx.x == 0) next_step = nxt;
    __syncthreads();
    st = next_step;
  }
  if (threadIdx.x == 0) {
    const unsigned d = __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (d == gridDim.x - 1) {
      // every workgroup has drawn its last (out of range) step: reset for the next call
      __hip_atomic_store(queue, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---------------------------------------------------------------- log-sum-exp merge
// Partials are merged in two levels, in index order: the splits of each group of
// group_splits consecutive splits first (GroupSplits<pool dtype>: 4 for quantised
// pools, else 8), then the groups. Both schedules below follow
// exactly this order with the same float operations, so a sequence's output bits
// depend only on its own length and split_tokens, whichever schedule runs.
//   level 1 (group c):  M = max lse_i, den = sum 2^(lse_i - M), acc = sum 2^(lse_i - M) o_i
//                       (online, i ascending, splits with lse = -inf skipped);
//                       group partial o_c = acc * (1/den), lse_c = M + log2(den)
//   level 2:            the same online merge over the groups, out = acc * (1/den).
// A sequence with a single group writes level 1's acc * (1/den) directly.

struct Merge4 {
  float m, den, acc[4];
  __device__ __forceinline__ void init() {
    m = -__builtin_huge_valf();
    den = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = 0.0f;
  }
  // Branch-free so that a run of adds can consume operands loaded ahead of it; a
  // split or group with no token (lse = -inf, o undefined) leaves the state as is.
  __device__ __forceinline__ void add(float lse, const float4& o) {
    const bool ok = lse != -__builtin_huge_valf();
    const float m_new = ok ? fmaxf(m, lse) : m;
    const float f = ok ? fast_exp2(m - m_new) : 1.0f;  // 0 while m is -inf
    const float w = ok ? fast_exp2(lse - m_new) : 0.0f;
    den = ok ? fmaf(den, f, w) : den;
    acc[0] = ok ? fmaf(acc[0], f, w * o.x) : acc[0];
    acc[1] = ok ? fmaf(acc[1], f, w * o.y) : acc[1];
    acc[2] = ok ? fmaf(acc[2], f, w * o.z) : acc[2];
    acc[3] = ok ? fmaf(acc[3], f, w * o.w) : acc[3];
    m = m_new;
  }
};

// Four consecutive output elements (d multiple of 4) of row (s, qh), scaled by inv.
template <int QT>
__device__ __forceinline__ void store_out4(void* out, int64_t out_st, int64_t out_sh,
                                           bool out_aligned, int s, int qh, int d,
                                           const float (&v)[4], float inv) {
  const int64_t off = (int64_t)s * out_st + (int64_t)qh * out_sh + d;
  if constexpr (QT == kF32) {
    float* op = (float*)out + off;
    if (out_aligned) {
      *reinterpret_cast<float4*>(op) = make_float4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) op[e] = v[e] * inv;
    }
  } else {
    const uint32_t w0 = (uint32_t)f32_to_bf16(v[0] * inv) | ((uint32_t)f32_to_bf16(v[1] * inv) << 16);
    const uint32_t w1 = (uint32_t)f32_to_bf16(v[2] * inv) | ((uint32_t)f32_to_bf16(v[3] * inv) << 16);
    uint16_t* op = (uint16_t*)out + off;
    if (out_aligned) {
      *reinterpret_cast<uint2*>(op) = make_uint2(w0, w1);
    } else {
      op[0] = (uint16_t)w0;
      op[1] = (uint16_t)(w0 >> 16);
      op[2] = (uint16_t)w1;
      op[3] = (uint16_t)(w1 >> 16);
    }
  }
}

// Device-coherent (agent-scope, relaxed) accesses for the single-launch schedule's
// cross-workgroup exchange. On gfx950 these are plain vector loads and stores with the
// device-scope cache policy, which bypasses the non-coherent per-XCD L2 state, so no
// L2 writeback or invalidate is needed; ordering comes from waiting for the stores to
// complete before the arrival counter is incremented.
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The group partials of the single-launch schedule as a raw buffer (num_records = its
// byte size, so an access past it reads zeros / writes nothing), for 16-byte accesses
// with the cache policy of the agent-scope atomics above (sc1: coherent across XCDs).
// One such access replaces four dword atomics: on the 8-sequence Qwen-shaped step this
// took the layer from 13.8 to 12.9 us (13.0 with two 8-byte atomics instead), and the
// FP8 64 x 8192 decode from 61 to 58-59 us.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kBufCoherent = 16;  // buffer-op cache policy bit: sc1
constexpr int kBufDword3 = 0x00020000;  // gfx9 raw-buffer descriptor word 3
__device__ __forceinline__ __amdgpu_buffer_rsrc_t partial_rsrc(const SplitArgs& a, int g_len,
                                                               int d_len) {
  const int64_t bytes = (int64_t)a.num_seqs * a.hkv * g_len * a.max_splits * d_len * 4;
  const int n = (int)min(bytes, (int64_t)0x7fffffff);
  return __builtin_amdgcn_make_buffer_rsrc(a.ws_o, (short)0, n, kBufDword3);
}
__device__ __forceinline__ void st_dev4(__amdgpu_buffer_rsrc_t r, uint32_t off, float x, float y,
                                        float z, float w) {
  const u32x4_t v = {__float_as_uint(x), __float_as_uint(y), __float_as_uint(z), __float_as_uint(w)};
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kBufCoherent);
}
__device__ __forceinline__ float4 ld_dev4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kBufCoherent);
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                     __uint_as_float(v.w));
}

// Level 2 over the group partials 0..ngroups-1 of row0 (group stride = partial rows),
// read with device-coherent loads, sixteen groups' loads issued together.
template <int D>
__device__ __forceinline__ void merge_groups_coherent(__amdgpu_buffer_rsrc_t ws_o,
                                                      const float* ws_lse, int64_t row0,
                                                      int ngroups, int d, Merge4& mg) {
  constexpr int U = 16;
  for (int c0 = 0; c0 < ngroups; c0 += U) {
    float lse[U];
    float4 o[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u;
      lse[u] = -__builtin_huge_valf();
      o[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (c < ngroups) {  // uniform: no load is spent on a missing group
        const int64_t row = row0 + c;
        lse[u] = ld_dev(ws_lse + row);
        o[u] = ld_dev4(ws_o, (uint32_t)((row * D + d) * 4));
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) mg.add(lse[u], o[u]);
  }
}

// Merge launch of the split-then-merge schedule: one workgroup per (sequence, KV head);
// thread t owns column (head h = t / (D/4), dims 4*(t % (D/4)) .. +3) of the G query
// heads, runs level 1 over each group's split partials and folds each group result
// into level 2 as it goes.
constexpr int kMergeThreads = 256;

template <int D, int G, int QT>
__global__ void __launch_bounds__(kMergeThreads) decode_merge_kernel(SplitArgs a) {
  constexpr int D4 = D / 4;
  const int g = (int)(blockIdx.x % a.hkv);
  const int s = (int)(blockIdx.x / a.hkv);
  const int L = clamped_len(a, s);
  const int nsplit = num_splits(L, a.split_tokens);
  if (nsplit <= 1) return;  // written directly by the split kernel
  const int t = threadIdx.x;
  if (t >= G * D4) return;
  const int h = t / D4, d = 4 * (t % D4);
  const int qh = g * G + h;
  const int gs = a.group_splits;
  const int ngroups = (nsplit + gs - 1) / gs;
  Merge4 top;
  top.init();
  for (int c = 0; c < ngroups; ++c) {
    // level 1 over the (at most group_splits) splits of group c
    const int i0 = c * gs;
    const int n = min(gs, nsplit - i0);
    float lse[kMaxGroupSplits];
    float4 o[kMaxGroupSplits];
#pragma unroll
    for (int u = 0; u < kMaxGroupSplits; ++u) {
      const int64_t row = split_row(a, s, i0 + (u < n ? u : 0), g, G) + h;
      lse[u] = u < n ? a.ws_lse[row] : -__builtin_huge_valf();
      o[u] = *reinterpret_cast<const float4*>(a.ws_o + row * D + d);
    }
    Merge4 grp;
    grp.init();
#pragma unroll
    for (int u = 0; u < kMaxGroupSplits; ++u) grp.add(lse[u], o[u]);  // -inf past n: no-op
    if (ngroups == 1) {
      store_out4<QT>(a.out, a.out_st, a.out_sh, a.out_aligned, s, qh, d, grp.acc, 1.0f / grp.den);
      return;
    }
    // level 2, online over the groups as they complete
    const float inv = 1.0f / grp.den;
    const float4 og = make_float4(grp.acc[0] * inv, grp.acc[1] * inv, grp.acc[2] * inv,
                                  grp.acc[3] * inv);
    top.add(grp.m + __log2f(grp.den), og);
  }
  store_out4<QT>(a.out, a.out_st, a.out_sh, a.out_aligned, s, qh, d, top.acc, 1.0f / top.den);
}

// Single-launch schedule for small batches (latency bound: a handful of sequences
// whose whole KV fits in one pass of the GPU), on a plain grid. A workgroup is
// FusedUnits units of GroupSplits waves, each unit one (sequence, group of GroupSplits
// consecutive splits, KV head). With two units and an even KV-head count the units are
// the two heads of a head pair over the same splits, on alternating waves, so both
// halves of each token's K/V record are read by one CU at about the same time while
// the two waves sharing a SIMD (w, w + 4) are two splits of one head, whose loads
// arrive independently. On the FP8 64 x 8192 pools a read of the decode's bytes alone
// took 47.3 us with one head per workgroup and 42.7 us with head pairs (a plain
// streaming read of the same bytes: 42.3 us); the decode went from 56.2 to 54.3 us
// (with the pair on one SIMD instead: 60.6 us). With an odd head count the two units
// are two consecutive groups of one head. The item's query rows and block ids are requested before its
// context length is known, each unit merges its waves' partials in LDS (level 1), and
// a sequence with several groups publishes group partials to the workspace and counts
// arrivals on a per (sequence, KV head) counter; the last group to arrive merges them
// (level 2) and writes out, then returns the counter to zero. This replaces the merge
// launch and its dependent loads, which dominate the time of such small calls.
// STEP: a decode step (knew / vnew / slots set); a separate instantiation so that its
// loads are issued with the others, not behind a branch.
template <int KVT, int D, int G, int QT, bool STEP>
__global__ void __launch_bounds__(64 * kFusedWaves) decode_fused_kernel(SplitArgs a) {
  using Gm = Geom<KVT, D>;
  constexpr int NW = kFusedWaves;
  constexpr int NU = FusedUnits<KVT>::value;
  constexpr int UW = GroupSplits<KVT>::value;  // waves per unit
  constexpr int D4 = D / 4;
  static_assert(G * D4 <= 64 * UW, "one merge column per thread of a unit");
  __shared__ float part_o[NW][G][D];
  __shared__ float part_lse[NW][G];
  __shared__ unsigned arrival[2];
  __shared__ int progress[NW];  // blocks done per wave (issue fairness, see balance_issue)
  // Every kernel argument the launch uses, loaded up front: without this the compiler
  // loads them region by region behind divergent branches, and each region waited
  // for its own round trip to the argument segment before its memory requests.
  asm volatile("" ::"s"(a.kpool), "s"(a.vpool), "s"(a.q), "s"(a.block_tables),
               "s"(a.context_lens), "s"(a.slots), "s"(a.knew), "s"(a.vnew), "s"(a.out),
               "s"(a.max_blocks_per_seq), "s"(a.hkv), "s"(a.max_chunks), "s"(a.num_seqs),
               "s"(a.q_st), "s"(a.q_sh), "s"(a.max_context_len), "s"(a.split_tokens),
               "s"(a.num_blocks), "s"(a.knew_st), "s"(a.knew_sh), "s"(a.vnew_st),
               "s"(a.vnew_sh), "s"(a.counters), "s"(a.ws_o), "s"(a.ws_lse),
               "s"(a.scale_log2), "s"((int)a.q_aligned), "s"((int)a.out_aligned));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // with two units the item's unit alternates with the wave (the two units' waves of
  // one split sit on neighbouring SIMDs; the waves sharing a SIMD, w and w + 4, are two
  // splits of one unit, whose loads arrive independently)
  const int unit = NU == 2 ? wave & 1 : 0, wu = NU == 2 ? wave >> 1 : wave;
  // KV head (pair) slowest: consecutive workgroups go to different XCDs, so every XCD
  // gets the same mix of heads (with the head fastest, an XCD would only see heads
  // congruent to its index, and the FP8 64 x 8192 decode ran ~15% longer on KV head 1
  // than on head 0, which left the XCDs holding head 1 finishing last)
  // unit u is KV head g0 + u (head pairs) or group c0 + u (odd head counts)
  const bool pairs = NU == 2 && (a.hkv & 1) == 0;
  int s, g0, c0;
  if (NU == 1) {
    const int per_head = a.num_seqs * a.max_chunks;
    g0 = (int)blockIdx.x / per_head;
    const int rest = (int)blockIdx.x - g0 * per_head;
    c0 = rest % a.max_chunks;
    s = rest / a.max_chunks;
  } else if (pairs) {
    const int per_pair = a.num_seqs * a.max_chunks;
    const int p = (int)blockIdx.x / per_pair;
    const int rest = (int)blockIdx.x - p * per_pair;
    c0 = rest % a.max_chunks;
    s = rest / a.max_chunks;
    g0 = 2 * p;
  } else {
    const int nc2 = (a.max_chunks + 1) / 2;
    const int per_head = a.num_seqs * nc2;
    g0 = (int)blockIdx.x / per_head;
    const int rest = (int)blockIdx.x - g0 * per_head;
    c0 = 2 * (rest % nc2);
    s = rest / nc2;
  }
  const int g = pairs ? g0 + unit : g0;
  const int c = pairs ? c0 : c0 + unit;
  const int split = c * UW + wu;
  static_assert(NW == 8 && NU * UW == NW, "balance_issue pairs wave w with w + 4: two splits of one unit");
  if (lane == 0)
    __hip_atomic_store(&progress[wave], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  // the context length and the step's slot, then the item's inputs: every request is
  // out before the first of them is used (one round trip for all)
  const int L_raw = ld_uniform(a.context_lens + s);
  int64_t slot = STEP ? ld_uniform(a.slots + s) : -1;
  ItemIn<KVT, D, G> in;
  MmaIn<D> min_;
  if constexpr (MmaPath<KVT, G>::value)
    load_mma_inputs<ElemBytes<KVT>::value, D, G>(a, s, split, g, lane, min_);
  else load_item_inputs<KVT, D, G, QT>(a, s, split, g, lane, in);
  asm volatile("" ::"s"(L_raw), "s"(slot));  // the first use of either value
  const int L = min(L_raw, a.max_context_len);
  // Decode step: every wave reads the new K/V row from the input, not from the pool,
  // and the unit holding group 0 of (s, g) copies it into the pool (its first two
  // waves: K, then V; 16 bytes per lane).
  // The copy's load goes out with the item's inputs and its store after the item:
  // nothing in this launch reads that pool slot, and the item does not wait for it.
  const char* krow_new = nullptr;
  const char* vrow_new = nullptr;
  const bool copier = STEP && c == 0 && wu < 2 && lane < Gm::NCH;
  uint4 new_row = make_uint4(0, 0, 0, 0);
  if constexpr (STEP) {
    krow_new = a.knew + ((int64_t)s * a.knew_st + (int64_t)g * a.knew_sh) * Gm::E;
    vrow_new = a.vnew + ((int64_t)s * a.vnew_st + (int64_t)g * a.vnew_sh) * Gm::E;
    // every lane loads (a chunk of its wave's row: in bounds), so no branch separates
    // this load from the others
    static_assert((Gm::NCH & (Gm::NCH - 1)) == 0, "chunks per row: a power of two");
    new_row = *reinterpret_cast<const uint4*>(((wu & 1) ? vrow_new : krow_new) +
                                              (lane & (Gm::NCH - 1)) * 16);
  }
  if (slot < 0) krow_new = vrow_new = nullptr;  // no new row: the pool holds the context
  auto copy_new_row = [&]() {
    if (copier && slot >= 0 && slot < a.num_blocks * kBlockSize) {
      const int64_t off = (slot / kBlockSize) * kBlockSize * a.hkv * Gm::ROW +
                          ((slot % kBlockSize) * a.hkv + g) * Gm::ROW + lane * 16;
      char* dst = const_cast<char*>(wu == 0 ? a.kpool : a.vpool) + off;
      *reinterpret_cast<uint4*>(dst) = new_row;
    }
  };
  const int nsplit = num_splits(L, a.split_tokens);
  const int ngroups = (nsplit + UW - 1) / UW;
  if (c0 >= ngroups) {  // uniform over the workgroup, before any barrier
    copy_new_row();
    return;
  }
  // (two units, odd head counts) unit 1 may be past the last group: its waves run
  // empty items (splits past the context) through the barriers, and it publishes
  // nothing
  float o[G][Gm::EV], lse2[G];
  if constexpr (MmaPath<KVT, G>::value) {
    // Every wave's progress word is written before any wave reads its partner's (the
    // LDS may still hold an earlier workgroup's words). The wait covers LDS and scalar
    // memory only (the scalar loads were consumed above), so the item's vector loads
    // stay in flight; every wave of the workgroup reaches this barrier (the return
    // above is uniform over the workgroup).
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // the item leaves its result in part_o[wave] itself
    item_partial_mma<KVT, D, G, MmaRing<KVT>::value, false>(a, min_, split, g, L, lane, o, lse2,
                                                            part_o[wave], krow_new, vrow_new,
                                                            progress);
  } else {
    item_partial<KVT, D, G>(a, in, split, g, L, lane, o, lse2, krow_new, vrow_new);
    if (lane < 16) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < Gm::EV; ++e) part_o[wave][h][lane * Gm::EV + e] = o[h][e];
    }
  }
  copy_new_row();
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) part_lse[wave][h] = lse2[h];
  }
  __syncthreads();
  // merge: threads 256 mu .. 256 mu + 255 take unit mu, whose splits are waves mu + 2 i
  // (two units), or all threads the one unit (waves 0..7)
  const int mu = NU == 2 ? (int)threadIdx.x >> 8 : 0;
  const int t = NU == 2 ? (int)threadIdx.x & 255 : (int)threadIdx.x;
  const int mg = pairs ? g0 + mu : g0;
  const int mc = pairs || NU == 1 ? c0 : c0 + mu;
  const bool has = mc < ngroups;
  const bool col = t < G * D4;
  const int h = col ? t / D4 : 0, d = 4 * (t % D4);
  const int qh = mg * G + h;
  Merge4 grp;
  grp.init();
  if (col) {
    float lw[UW];
    float4 ow[UW];
#pragma unroll
    for (int w = 0; w < UW; ++w) {
      lw[w] = part_lse[mu + NU * w][h];
      ow[w] = *reinterpret_cast<const float4*>(&part_o[mu + NU * w][h][d]);
    }
#pragma unroll
    for (int w = 0; w < UW; ++w) grp.add(lw[w], ow[w]);
  }
  if (ngroups == 1) {  // then c == 0 for every unit that has work
    if (col && has) store_out4<QT>(a.out, a.out_st, a.out_sh, a.out_aligned, s, qh, d, grp.acc, 1.0f / grp.den);
    return;
  }
  const int64_t row0 = ((int64_t)s * a.hkv * G + qh) * a.max_splits;
  if (col && has) {
    const float inv = 1.0f / grp.den;
    st_dev4(partial_rsrc(a, G, D), (uint32_t)(((row0 + mc) * D + d) * 4), grp.acc[0] * inv,
            grp.acc[1] * inv, grp.acc[2] * inv, grp.acc[3] * inv);
    if (d == 0) st_dev(a.ws_lse + row0 + mc, grp.m + __log2f(grp.den));
  }
  // every thread's partial stores have completed before the arrival is counted
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  unsigned* counter = a.counters + ((int64_t)s * a.hkv + mg);
  if (t == 0 && has)
    arrival[mu] = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  // per unit from here on (no barrier follows)
  if (!has || arrival[mu] != (unsigned)(ngroups - 1)) return;
  if (col) {
    Merge4 top;
    top.init();
    merge_groups_coherent<D>(partial_rsrc(a, G, D), a.ws_lse, row0, ngroups, d, top);
    store_out4<QT>(a.out, a.out_st, a.out_sh, a.out_aligned, s, qh, d, top.acc, 1.0f / top.den);
  }
  if (t == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// step != nullptr: a decode step whose new rows are stored first (folded into the
// single-launch kernel when that schedule runs and the rows allow it, else a store
// launch ahead of the decode).
template <int KVT, int D, int G, int QT>
static int launch_decode_t(const pa_kv_pool_t& pool, const DecodeArgs& a, const StepRows* step,
                           hipStream_t stream) {
  SplitArgs sa;
  sa.kpool = (const char*)pool.k;
  sa.vpool = (const char*)pool.v;
  sa.kscale = pool.k_scale;
  sa.vscale = pool.v_scale;
  sa.num_blocks = pool.num_blocks;
  sa.hkv = pool.kv_heads;
  sa.out = a.out;
  sa.out_st = a.out_st;
  sa.out_sh = a.out_sh;
  sa.q = a.q;
  sa.q_st = a.q_st;
  sa.q_sh = a.q_sh;
  sa.num_seqs = a.num_seqs;
  sa.block_tables = a.block_tables;
  sa.max_blocks_per_seq = a.max_blocks_per_seq;
  sa.context_lens = a.context_lens;
  sa.max_context_len = a.max_context_len;
  sa.scale_log2 = a.scale * kLog2e;
  sa.split_tokens = a.split_tokens;
  sa.max_splits = a.max_splits;
  sa.ws_o = a.ws_o;
  sa.ws_lse = a.ws_lse;
  const int qe = QT == kF32 ? 4 : 2;
  auto al = [](const void* p, int64_t st, int64_t sh, int e) {
    return ((uintptr_t)p & 15u) == 0 && (st * e) % 16 == 0 && (sh * e) % 16 == 0;
  };
  sa.q_aligned = al(a.q, a.q_st, a.q_sh, qe);
  sa.out_aligned = al(a.out, a.out_st, a.out_sh, qe);
  sa.group_splits = GroupSplits<KVT>::value;
  sa.max_chunks = (a.max_splits + sa.group_splits - 1) / sa.group_splits;
  sa.counters = a.counters;
  sa.knew = sa.vnew = nullptr;
  sa.knew_st = sa.knew_sh = sa.vnew_st = sa.vnew_sh = 0;
  sa.slots = nullptr;
  // single-launch workgroups: (sequence, head, group); with two units (sequence, head
  // pair, group) or (sequence, head, two groups)
  const int64_t fused_groups =
      FusedUnits<KVT>::value == 1 ? (int64_t)a.num_seqs * pool.kv_heads * sa.max_chunks
      : pool.kv_heads % 2 == 0    ? (int64_t)a.num_seqs * (pool.kv_heads / 2) * sa.max_chunks
                                  : (int64_t)a.num_seqs * pool.kv_heads * ((sa.max_chunks + 1) / 2);
  // its arrival counters (one per (sequence, KV head), used when there are two or more
  // groups) stay below the persistent schedule's two words
  const bool fused = fused_groups <= kFusedMaxWorkgroups &&
                     (sa.max_chunks == 1 || (int64_t)a.num_seqs * pool.kv_heads <= kCompactQueueWord);
  // the persistent schedule's dot-product items fold the store in as well
  const bool fold = fused || (a.num_seqs <= kMaxCompactSeqs && !MmaPath<KVT, G>::value);
  if (step != nullptr && fold) {
    sa.knew = (const char*)step->k;
    sa.vnew = (const char*)step->v;
    sa.knew_st = step->k_st;
    sa.knew_sh = step->k_sh;
    sa.vnew_st = step->v_st;
    sa.vnew_sh = step->v_sh;
    sa.slots = step->slots;
  } else if (step != nullptr) {
    const int st = launch_store(pool, step->k, step->v, step->src_dtype, a.num_seqs, step->k_st,
                                step->k_sh, step->v_st, step->v_sh, step->slots, stream);
    if (st != PA_OK) return st;
  }
  if (fused) {
    const hipError_t e =
        sa.knew != nullptr
            ? launch_kernel(decode_fused_kernel<KVT, D, G, QT, true>, dim3((unsigned)fused_groups),
                            dim3(64 * kFusedWaves), stream, sa)
            : launch_kernel(decode_fused_kernel<KVT, D, G, QT, false>, dim3((unsigned)fused_groups),
                            dim3(64 * kFusedWaves), stream, sa);
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
  }
  const int64_t items = (int64_t)a.num_seqs * a.max_splits * pool.kv_heads;
  hipError_t e;
  if (a.num_seqs <= kMaxCompactSeqs) {
    const int64_t steps = (items + kCompactWaves - 1) / kCompactWaves;  // upper bound
    auto kern = decode_compact_kernel<KVT, D, G, QT>;
    const int64_t grid = std::min(steps, resident_workgroups(kern, 64 * kCompactWaves));
    e = launch_kernel(kern, dim3((unsigned)grid), dim3(64 * kCompactWaves), stream, sa);
  } else {
    const int64_t steps = (items + kWaves - 1) / kWaves;
    e = launch_kernel(decode_split_kernel<KVT, D, G, QT>, dim3((unsigned)steps),
                      dim3(64 * kWaves), stream, sa);
  }
  if (e == hipSuccess && a.max_splits > 1)
    e = launch_kernel(decode_merge_kernel<D, G, QT>,
                      dim3((unsigned)((int64_t)a.num_seqs * pool.kv_heads)), dim3(kMergeThreads),
                      stream, sa);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

template <int KVT, int D, int QT>
static int dispatch_g(const pa_kv_pool_t& pool, const DecodeArgs& a, const StepRows* step,
                      hipStream_t stream) {
  switch (a.q_heads / pool.kv_heads) {
    case 1: return launch_decode_t<KVT, D, 1, QT>(pool, a, step, stream);
    case 2: return launch_decode_t<KVT, D, 2, QT>(pool, a, step, stream);
    case 3: return launch_decode_t<KVT, D, 3, QT>(pool, a, step, stream);
    case 4: return launch_decode_t<KVT, D, 4, QT>(pool, a, step, stream);
    case 5: return launch_decode_t<KVT, D, 5, QT>(pool, a, step, stream);
    case 6: return launch_decode_t<KVT, D, 6, QT>(pool, a, step, stream);
    case 7: return launch_decode_t<KVT, D, 7, QT>(pool, a, step, stream);
    case 8: return launch_decode_t<KVT, D, 8, QT>(pool, a, step, stream);
    default: return PA_ERR_UNSUPPORTED;
  }
}

static int dispatch(const pa_kv_pool_t& pool, const DecodeArgs& a, const StepRows* step,
                    hipStream_t stream) {
  const int D = pool.head_dim;
  switch (pool.dtype) {
    case PA_F32:
      return D == 64 ? dispatch_g<kF32, 64, kF32>(pool, a, step, stream)
                     : dispatch_g<kF32, 128, kF32>(pool, a, step, stream);
    case PA_BF16:
      return D == 64 ? dispatch_g<kBF16, 64, kBF16>(pool, a, step, stream)
                     : dispatch_g<kBF16, 128, kBF16>(pool, a, step, stream);
    case PA_FP8_E4M3:
      return D == 64 ? dispatch_g<kFP8, 64, kBF16>(pool, a, step, stream)
                     : dispatch_g<kFP8, 128, kBF16>(pool, a, step, stream);
    case PA_INT8:
      return D == 64 ? dispatch_g<kINT8, 64, kBF16>(pool, a, step, stream)
                     : dispatch_g<kINT8, 128, kBF16>(pool, a, step, stream);
    default:
      return PA_ERR_UNSUPPORTED;
  }
}

int launch_decode(const pa_kv_pool_t& pool, const DecodeArgs& a, hipStream_t stream) {
  return dispatch(pool, a, nullptr, stream);
}

// ---------------------------------------------------------------- allocation-free decode
// The workspace of pa_decode_noalloc: one array per GPU, in the library's code object,
// held until the process ends. Host code never uses the array's name as an address
// (on the host it names a stand-in, not device memory): its device address is looked
// up once per device with hipGetSymbolAddress and that pointer is what the kernels get.
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

__global__ void zero_words_kernel(unsigned* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

constexpr int kMaxScratchDevices = 64;

int noalloc_scratch(void** ptr, hipStream_t stream) {
  static std::mutex mu;
  static void* dev_ptr[kMaxScratchDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_HIP;
  if (dev < 0 || dev >= kMaxScratchDevices) return PA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(mu);
  if (dev_ptr[dev] == nullptr) {
    void* p = nullptr;
    // with `dev` current: this device's copy of the array
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return PA_ERR_HIP;
    // the arrival / work counters at the start of a decode workspace must be zero before
    // its first use (every call leaves them zero again); a kernel, not a memset, so that
    // a first call under graph capture records an ordinary kernel node
    constexpr int words = (int)(kDecodeCounterBytes / sizeof(unsigned));
    if (launch_kernel(zero_words_kernel, dim3((words + 255) / 256), dim3(256), stream,
                      (unsigned*)p, words) != hipSuccess)
      return PA_ERR_HIP;
    dev_ptr[dev] = p;
  }
  *ptr = dev_ptr[dev];
  return PA_OK;
}

int launch_decode_step(const pa_kv_pool_t& pool, const DecodeArgs& a, const StepRows& rows,
                       hipStream_t stream) {
  // the store folds into the single-launch kernel for same-dtype rows that start on 16
  // bytes; a quantised pool (quantise-on-store) or other rows take a store launch first
  const int E = pool.dtype == PA_F32 ? 4 : 2;
  auto al = [&](const void* p, int64_t st, int64_t sh) {
    return ((uintptr_t)p & 15u) == 0 && (st * E) % 16 == 0 && (sh * E) % 16 == 0;
  };
  const bool foldable = pool.dtype != PA_FP8_E4M3 && pool.dtype != PA_INT8 &&
                        rows.src_dtype == pool.dtype &&
                        al(rows.k, rows.k_st, rows.k_sh) && al(rows.v, rows.v_st, rows.v_sh);
  if (!foldable) {
    const int st = launch_store(pool, rows.k, rows.v, rows.src_dtype, a.num_seqs, rows.k_st,
                                rows.k_sh, rows.v_st, rows.v_sh, rows.slots, stream);
    if (st != PA_OK) return st;
    return dispatch(pool, a, nullptr, stream);
  }
  return dispatch(pool, a, &rows, stream);
}

}  // namespace pa
