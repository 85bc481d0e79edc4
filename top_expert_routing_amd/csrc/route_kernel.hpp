// The gfx950 route kernel: score function, bias, group-limited top-k, top-k,
// weights and the per-block expert bitmask, for one token per cluster of LPT
// lanes (EPL experts per lane).
//
// Method (page title, section):
//   score function, pre/post-softmax order, group top-k, expert bias, scaling:
//     TransformerEngine Fused Router, Description + I/O Contract;
//   n_group / topk_group, routing bias, routed_scaling_factor, norm_topk_prob,
//   local experts: flashinfer trtllm_gen_routing, Parameters, Notes;
//   float32 sigmoid, selection by score + correction bias, unbiased weights:
//     MAX SigmoidTopKRouter, routing steps 2-4.
//
// Per token: the logits stream HBM -> VGPRs once (16-byte loads) and are kept
// raw in LDS as well; keys, group scores and a lower bound tau on the k-th key
// are formed in registers; the few keys >= tau are compacted into LDS as
// packed (key, index) words, ranked by counting, and the k best are emitted
// by rank, their score recomputed from the raw logit.  Per block of 64 tokens
// an LDS bitmask per expert records which tokens chose it; its popcounts are
// the block's counts row, added into a counting row shared by a group of
// blocks.
//
// One instance per (lanes per token, experts per lane, logits dtype, score
// variant); this header is included by one translation unit per variant.
#pragma once

#include "device_common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr float kInf = __builtin_huge_valf();

// Raw row slice of one lane: EPL logits as packed 32-bit words (two bf16 or
// one float32 per word), decoded later so that the loads can be issued before
// anything else.  Padded experts hold -inf.
template <int EPL, bool BF16>
struct RawRow {
  static constexpr int kWords = BF16 ? EPL / 2 : EPL;
  uint32_t w[kWords];
};

template <int EPL, bool BF16>
__device__ __forceinline__ void load_raw(RawRow<EPL, BF16>& r, const void* __restrict__ base,
                                         size_t row_elems, int e0, int E, bool vec, bool tv) {
  constexpr int NW = RawRow<EPL, BF16>::kWords;
  if (tv && vec && e0 + EPL <= E && NW % 4 == 0) {
    const u32x4* src = reinterpret_cast<const u32x4*>(
        static_cast<const char*>(base) + (row_elems + e0) * (BF16 ? 2 : 4));
#pragma unroll
    for (int v = 0; v < NW / 4; ++v) {
      const u32x4 q = __builtin_nontemporal_load(src + v);
      r.w[4 * v] = q.x; r.w[4 * v + 1] = q.y; r.w[4 * v + 2] = q.z; r.w[4 * v + 3] = q.w;
    }
  } else if constexpr (BF16) {
    const uint16_t* src = static_cast<const uint16_t*>(base) + row_elems;
#pragma unroll
    for (int i = 0; i < EPL; i += 2) {
      const int e = e0 + i;
      const uint32_t lo = e < E ? (tv ? (uint32_t)src[e] : 0u) : 0xFF80u;
      const uint32_t hi = e + 1 < E ? (tv ? (uint32_t)src[e + 1] : 0u) : 0xFF80u;
      r.w[i / 2] = lo | (hi << 16);
    }
  } else {
    const uint32_t* src = static_cast<const uint32_t*>(base) + row_elems;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = e0 + i;
      r.w[i] = e < E ? (tv ? src[e] : 0u) : 0xFF800000u;
    }
  }
}

template <int EPL, bool BF16>
__device__ __forceinline__ void decode_raw(const RawRow<EPL, BF16>& r, float (&x)[EPL]) {
  if constexpr (BF16) {
#pragma unroll
    for (int i = 0; i < EPL / 2; ++i) {
      x[2 * i] = bf16_lo(r.w[i]);
      x[2 * i + 1] = bf16_hi(r.w[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < EPL; ++i) x[i] = __uint_as_float(r.w[i]);
  }
}

// The cluster's row in LDS, dynamically indexable: for the softmax variant the
// raw logit words (two bf16 or one float32 per word; the logit is the score
// basis there), otherwise the float32 score basis of every expert -- except
// that the sigmoid variant with bfloat16 logits may keep the raw words too
// (`sig_raw`, half the LDS: a grid of several rounds of blocks then fits two
// blocks per CU) and recompute the sigmoid of the few experts it reads back.
template <int VAR, bool BF16>
constexpr bool kRawRow = VAR == kVarSoftmax;
template <int VAR, bool BF16>
constexpr bool kSigRawOk = VAR == kVarSigmoid && BF16;

// Expert e of the cluster lies in lane e / EPL, whose slice starts lpad
// padding words per earlier lane further on (see route_lane_pad).
template <int VAR, bool BF16, int EPL>
__device__ __forceinline__ float row_basis(const uint32_t* rowc, int e, bool sig_raw, int lpad) {
  rowc += lpad * (e / EPL);
  if constexpr (kRawRow<VAR, BF16> && BF16) {
    const uint32_t w = rowc[e >> 1];
    return (e & 1) ? bf16_hi(w) : bf16_lo(w);
  } else if constexpr (kSigRawOk<VAR, BF16>) {
    if (sig_raw) {
      const uint32_t w = rowc[e >> 1];
      return sigmoid_f32((e & 1) ? bf16_hi(w) : bf16_lo(w));      // sigmoid(-inf) = 0
    }
    return __uint_as_float(rowc[e]);
  } else {
    return __uint_as_float(rowc[e]);
  }
}

__device__ __forceinline__ float fast_rcp(float v) { return __builtin_amdgcn_rcpf(v); }

}  // namespace

// Weights of the selected experts (uniform per call):
//   plain      weight = score basis (sigmoid score, or the softmax probability
//              when a bias forced the probabilities to be formed first),
//              optionally renormalised over the k selected;
//   exact_pre  softmax over all E without renormalisation: exp(r - m) / sum;
//   soft_sel   softmax over the k selected (softmax after top-k, or softmax
//              before top-k renormalised, which is the same distribution).
enum { kEmitPlain = 0, kEmitExactPre = 1, kEmitSoftSel = 2 };

// Rank the cluster's C candidates by counting among the first T entries of its
// candidate list (entries C..T-1 hold 0, below every packed key).  Lane c
// ranks entries c, c + LPT, ...; the expert of rank n < k is recorded at
// position n of the selection list.
template <int LPT, int T>
__device__ __forceinline__ void rank_tier(const uint64_t* mycand, int C, int k, int lane_c,
                                          int* myselidx) {
  constexpr int CHUNK = T < 32 ? T : 32;
  uint64_t cv[CHUNK];
  if constexpr (T <= 32) {
#pragma unroll
    for (int i = 0; i < T; i += 2) {
      const u64x2 v = *reinterpret_cast<const u64x2*>(mycand + i);
      cv[i] = v.x;
      cv[i + 1] = v.y;
    }
  }
  constexpr int Q = (T + LPT - 1) / LPT;      // slots per lane
  if constexpr (T <= 32 && Q <= 8) {
    uint64_t mine[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) mine[q] = lane_c + q * LPT < T ? mycand[lane_c + q * LPT] : 0ull;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int j = lane_c + q * LPT;
      int rank = 0;
#pragma unroll
      for (int i = 0; i < T; ++i) rank += cv[i] > mine[q] ? 1 : 0;
      if (j < C && rank < k) myselidx[rank] = unpack_idx(mine[q]);
    }
    return;
  }
  for (int j = lane_c; j < C; j += LPT) {
    const uint64_t mine = mycand[j];
    int rank = 0;
    if constexpr (T <= 32) {
#pragma unroll
      for (int i = 0; i < T; ++i) rank += cv[i] > mine ? 1 : 0;
    } else {
      for (int i0 = 0; i0 < T; i0 += CHUNK) {
#pragma unroll
        for (int i = 0; i < CHUNK; i += 2) {
          const u64x2 v = *reinterpret_cast<const u64x2*>(mycand + i0 + i);
          rank += (v.x > mine ? 1 : 0) + (v.y > mine ? 1 : 0);
        }
      }
    }
    if (rank < k) myselidx[rank] = unpack_idx(mine);
  }
}

// Per-token values the emission needs.
struct EmitCtx {
  int32_t* ids;
  void* weights;
  bool weights_bf16, renorm, counting, pre;
  bool sig_raw;           // the row holds raw bfloat16 logits of the sigmoid variant
  int lpad;               // padding words per lane slice of the row
  int mode, k, loc_off, loc_n;
  float scale;
  uint64_t* hmask;
  int t, tl, lane_c;
  bool tv;
  float m, inv_s;
};

// Weights, ids and the block bitmask for the k selected, by rank: lane c
// handles ranks c, c + LPT, ... (contiguous stores across the cluster).  The
// score basis of each selected expert is recomputed from its raw logit.
template <int LPT, int EPL, bool BF16, int VAR>
__device__ __forceinline__ void emit_selected(const EmitCtx& c, const int* myselidx,
                                              const uint32_t* rowc) {
  const int k = c.k;
  if (k <= LPT) {                             // one rank per lane
    const bool v = c.lane_c < k;
    const int e = v ? myselidx[c.lane_c] : 0;
    const float r = row_basis<VAR, BF16, EPL>(rowc, e, c.sig_raw, c.lpad);
    float ref = 0.0f;
    if (c.mode == kEmitSoftSel) ref = cl_max<LPT>(v ? r : -kInf);
    float inv_den = c.inv_s;
    if (c.mode != kEmitExactPre)
      inv_den = fast_rcp(cl_sum<LPT>(v ? (c.mode == kEmitPlain ? r : exp_f32(r - ref)) : 0.0f));
    if (!c.tv || !v) return;
    float w;
    if (c.mode == kEmitPlain)
      w = c.renorm ? r * inv_den : r;
    else
      w = exp_f32(r - (c.mode == kEmitExactPre ? c.m : ref)) * inv_den;
    w *= c.scale;
    const size_t o = (size_t)c.t * k + c.lane_c;
    c.ids[o] = e;
    if (c.weights_bf16)
      static_cast<uint16_t*>(c.weights)[o] = (uint16_t)f32_to_bf16_rne(w);
    else
      static_cast<float*>(c.weights)[o] = w;
    if (c.counting) {
      const int el = e - c.loc_off;
      if (el >= 0 && el < c.loc_n) atomicOr(&c.hmask[el], 1ull << c.tl);
    }
    return;
  }
  constexpr int KQ = 4;
  if (k <= KQ * LPT) {                        // up to four ranks per lane, held in registers
    int e[KQ];
    float r[KQ];
#pragma unroll
    for (int q = 0; q < KQ; ++q) {
      const int n = c.lane_c + q * LPT;
      e[q] = n < k ? myselidx[n] : 0;
    }
#pragma unroll
    for (int q = 0; q < KQ; ++q)
      r[q] = row_basis<VAR, BF16, EPL>(rowc, e[q], c.sig_raw, c.lpad);
    float ref = 0.0f;
    if (c.mode == kEmitSoftSel) {
      float mx = -kInf;
#pragma unroll
      for (int q = 0; q < KQ; ++q) mx = c.lane_c + q * LPT < k ? fmaxf(mx, r[q]) : mx;
      ref = cl_max<LPT>(mx);
    }
    float inv_den = c.inv_s;
    if (c.mode != kEmitExactPre) {
      float part = 0.0f;
#pragma unroll
      for (int q = 0; q < KQ; ++q)
        if (c.lane_c + q * LPT < k) part += c.mode == kEmitPlain ? r[q] : exp_f32(r[q] - ref);
      inv_den = fast_rcp(cl_sum<LPT>(part));
    }
    if (!c.tv) return;
    const float sub = c.mode == kEmitExactPre ? c.m : ref;
#pragma unroll
    for (int q = 0; q < KQ; ++q) {
      const int n = c.lane_c + q * LPT;
      if (n < k) {
        float w;
        if (c.mode == kEmitPlain)
          w = c.renorm ? r[q] * inv_den : r[q];
        else
          w = exp_f32(r[q] - sub) * inv_den;
        w *= c.scale;
        const size_t o = (size_t)c.t * k + n;
        c.ids[o] = e[q];
        if (c.weights_bf16)
          static_cast<uint16_t*>(c.weights)[o] = (uint16_t)f32_to_bf16_rne(w);
        else
          static_cast<float*>(c.weights)[o] = w;
        if (c.counting) {
          const int el = e[q] - c.loc_off;
          if (el >= 0 && el < c.loc_n) atomicOr(&c.hmask[el], 1ull << c.tl);
        }
      }
    }
    return;
  }
  float ref = 0.0f;
  if (c.mode == kEmitSoftSel) {
    float mx = -kInf;
    for (int n = c.lane_c; n < k; n += LPT)
      mx = fmaxf(mx, row_basis<VAR, BF16, EPL>(rowc, myselidx[n], c.sig_raw, c.lpad));
    ref = cl_max<LPT>(mx);
  }
  float inv_den = c.inv_s;
  if (c.mode != kEmitExactPre) {
    float part = 0.0f;
    for (int n = c.lane_c; n < k; n += LPT) {
      const float r = row_basis<VAR, BF16, EPL>(rowc, myselidx[n], c.sig_raw, c.lpad);
      part += c.mode == kEmitPlain ? r : exp_f32(r - ref);
    }
    inv_den = fast_rcp(cl_sum<LPT>(part));
  }
  if (!c.tv) return;
  const float sub = c.mode == kEmitExactPre ? c.m : ref;
  for (int n = c.lane_c; n < k; n += LPT) {
    const int e = myselidx[n];
    const float r = row_basis<VAR, BF16, EPL>(rowc, e, c.sig_raw, c.lpad);
    float w;
    if (c.mode == kEmitPlain)
      w = c.renorm ? r * inv_den : r;
    else
      w = exp_f32(r - sub) * inv_den;
    w *= c.scale;
    const size_t o = (size_t)c.t * k + n;
    c.ids[o] = e;
    if (c.weights_bf16)
      static_cast<uint16_t*>(c.weights)[o] = (uint16_t)f32_to_bf16_rne(w);
    else
      static_cast<float*>(c.weights)[o] = w;
    if (c.counting) {
      const int el = e - c.loc_off;
      if (el >= 0 && el < c.loc_n) atomicOr(&c.hmask[el], 1ull << c.tl);
    }
  }
}

// Padded experts (e >= E) carry logit -inf and bias -inf, so their keys are
// -inf and no per-element validity masks are needed anywhere.
// The permutation of a call whose tokens all lie in this block (T <= 64), from
// the block's bitmask of which tokens chose each local expert (FlashInfer
// trtllm_gen_routing, Returns: the padded offsets, both index maps and the
// per-tile expert and row limit): counts are popcounts, the padded offsets a
// scan, and token t's slot for expert e is offset(e) + the number of lower
// tokens that chose e (stable by token).  po: LDS for loc_n + 1 ints and 8
// more (the scan's wave sums).
template <int BLOCK>
__device__ void permute_in_block(const RouteParams& p, const uint64_t* hmask, int* po) {
  const int tid = threadIdx.x;
  const int El = p.loc_n, k = p.k, tile = p.tile;
  __syncthreads();                                      // the bitmask and the ids are complete
  // exclusive scan of the padded sizes over the block, BLOCK experts a round
  int* scan_tmp = po + El + 1;                          // BLOCK / 64 ints
  int carry = 0;
  for (int e0 = 0; e0 < El; e0 += BLOCK) {             // uniform trip count
    const int e = e0 + tid;
    const int v = e < El ? ((__popcll(hmask[e]) + tile - 1) & ~(tile - 1)) : 0;
    int round_total;
    const int ex = block_excl_scan<BLOCK>(v, scan_tmp, round_total);
    if (e < El) po[e] = carry + ex;
    carry += round_total;
    if (e0 + BLOCK < El) __syncthreads();               // scan_tmp is written again
  }
  if (tid == 0) po[El] = carry;
  __syncthreads();
  // both index maps; every (token, choice) of the call is in this block
  for (int q = tid; q < p.T * k; q += BLOCK) {
    const int t = q / k;
    const int el = p.ids[q] - p.loc_off;
    int slot = -1;
    if (el >= 0 && el < El) {
      slot = po[el] + __popcll(hmask[el] & ((1ull << t) - 1ull));
      p.p2t[slot] = t;
    }
    p.e2p[q] = slot;
  }
  // per expert: count, padded offset, its tiles, the -1 padding of its last tile
  for (int e = tid; e < El; e += BLOCK) {
    const int seg = po[e], cnt = __popcll(hmask[e]);
    const int seg_end = seg + cnt;
    const int ntile = (po[e + 1] - seg) >> p.tile_shift;
    for (int j = 0; j < ntile; ++j) {
      const int c = (seg >> p.tile_shift) + j;
      p.batch_idx[c] = e;
      p.mn_limit[c] = min(seg + (j + 1) * tile, seg_end);
    }
    for (int s2 = seg_end; s2 < po[e + 1]; ++s2) p.p2t[s2] = -1;
    if (p.counts != nullptr) p.counts[e] = cnt;
    p.padded_offsets[e] = seg;
  }
  if (tid == 0) {
    const int total = po[El];
    p.padded_offsets[El] = total;
    *p.total_out = total;
    *p.nctas_out = total >> p.tile_shift;
  }
}

template <int LPT, int EPL, bool BF16, int VAR>
__global__ void __launch_bounds__(kRouteBlock<LPT>)
    __attribute__((amdgpu_waves_per_eu(kRouteMinWaves<LPT>))) route_kernel(RouteParams p) {
  constexpr int BLOCK = kRouteBlock<LPT>;
  constexpr int NCL = BLOCK / LPT;          // clusters (tokens in flight) per block
  constexpr int TPC = kTokensPerBlock / NCL;
  constexpr int EP = LPT * EPL;             // padded row length
  constexpr int WPL = RawRow<EPL, BF16>::kWords;
  constexpr bool kRaw = kRawRow<VAR, BF16>;
  const bool sig_raw = kSigRawOk<VAR, BF16> && p.sig_raw != 0;
  const int RWPL = (kRaw || sig_raw) ? WPL : EPL;   // row words per lane
  static_assert(TPC * NCL == kTokensPerBlock, "block shape");
  static_assert(EPL <= 32, "lane masks are 32-bit");
  constexpr bool kBias = VAR != kVarSoftmax;   // the softmax variant has no bias
  // tau from per-lane top four (ungrouped, 2..8 lanes per token): close to the
  // k-th key, so that few candidates remain to rank
  constexpr bool kRefineTau = LPT >= 2 && LPT <= 8;
  constexpr float kLowest = -3.402823466e38f;

  const int tid = threadIdx.x;
  const int lane_c = tid % LPT;
  const int cl = tid / LPT;
  const int e0 = lane_c * EPL;
  const int E = p.E, k = p.k;
  const int blk = xcd_block((int)blockIdx.x, (int)gridDim.x);   // XCD-contiguous order
  const bool pre = p.pre != 0;

  const RouteLds L = route_lds_layout(LPT, RWPL, EPL, p.hmask_len, p.cap, k,
                                      p.grouped ? p.n_group : 0);
  extern __shared__ __align__(16) unsigned char smem[];
  float* bias_s = reinterpret_cast<float*>(smem + L.bias);
  uint64_t* hmask = reinterpret_cast<uint64_t*>(smem + L.hmask);
  uint32_t* rowc = reinterpret_cast<uint32_t*>(smem + L.row) + cl * L.row_stride;
  const int lpad = route_lane_pad(LPT, RWPL);          // padded lane slices of the row
  constexpr int BPAD = route_lane_pad(LPT, EPL);       // and of the bias
  uint32_t* myrow = rowc + lane_c * (RWPL + lpad);
  uint64_t* mycand = reinterpret_cast<uint64_t*>(smem + L.cand) + cl * L.cand_stride;
  int* myselidx = reinterpret_cast<int*>(smem + L.sel_idx) + cl * L.sel_stride;
  uint64_t* mygs = reinterpret_cast<uint64_t*>(smem + L.gscore) + cl * L.gs_stride;

  // The bias is requested first (one block-wide pass into LDS), then the
  // first token's logits; the bias lands in LDS while the logits are in flight.
  // Its raw bits are loaded and decoded only after the logits are requested:
  // a value used inside the branch that loads it is awaited at once.
  uint32_t braw = 0u;
  const bool bias_here = kBias && tid < EP && tid < E && p.bias != nullptr;
  if (bias_here)
    braw = p.bias_bf16 ? (uint32_t)static_cast<const uint16_t*>(p.bias)[tid]
                       : __float_as_uint(static_cast<const float*>(p.bias)[tid]);
  RawRow<EPL, BF16> raw;
  {
    const int t = blk * kTokensPerBlock + cl;
    load_raw<EPL, BF16>(raw, p.logits, (size_t)t * E, e0, E, p.vec, t < p.T);
  }
  if constexpr (kBias) {
    const float bload = tid >= E ? -kInf
                        : !bias_here ? 0.0f
                        : p.bias_bf16 ? __uint_as_float(braw << 16) : __uint_as_float(braw);
    for (int e = tid; e < EP; e += BLOCK) {          // EP > BLOCK only for very wide rows
      float b = e == tid ? bload : (e >= E ? -kInf : 0.0f);
      if (e != tid && e < E && p.bias != nullptr)
        b = p.bias_bf16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(p.bias)[e])
                        : static_cast<const float*>(p.bias)[e];
      bias_s[e + BPAD * (e / EPL)] = b;
    }
  }
  const bool counting = p.super_rows != nullptr || p.fused;
  // the set of counting rows this call adds into (requested early, used last)
  const uint32_t hdr0 = p.super_rows != nullptr ? p.count_hdr[0] : 0u;
  const uint32_t cset = hdr0 & 1u;
  if (counting)
    for (int e = tid; e < p.loc_n; e += BLOCK) hmask[e] = 0;
  __syncthreads();
  float breg[EPL];
  if constexpr (kBias) {
#pragma unroll
    for (int i = 0; i < EPL; i += 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(bias_s + e0 + BPAD * lane_c + i);
      breg[i] = v.x; breg[i + 1] = v.y; breg[i + 2] = v.z; breg[i + 3] = v.w;
    }
  }

  const bool refine = !p.grouped && k <= 4 * LPT && k > 2;
  // softmax before top-k without a bias keys on the logits themselves (the
  // same order as the probabilities), but a group score sums probabilities:
  // grouped, it needs the token maximum m to form exp(x - m)
  const bool group_exp = VAR == kVarSoftmax && pre && p.grouped && p.topn > 1;
  const bool need_ms =
      VAR == kVarSigmoid ? false
                         : ((VAR == kVarSoftmax ? (pre && !p.renorm) : pre) || p.scores != nullptr ||
                            group_exp);
  const int mode = (VAR == kVarSigmoid || (VAR == kVarSoftmaxBias && pre))
                       ? kEmitPlain
                       : ((VAR == kVarSoftmax && pre && !p.renorm) ? kEmitExactPre : kEmitSoftSel);

  for (int it = 0; it < TPC; ++it) {
    const int tl = it * NCL + cl;               // token within the block
    const int t = blk * kTokensPerBlock + tl;
    const bool tv = t < p.T;
    if (kRaw || sig_raw) {                     // the raw row, dynamically indexable
      if constexpr (WPL % 4 == 0) {
#pragma unroll
        for (int v = 0; v < WPL; v += 4)
          *reinterpret_cast<u32x4*>(myrow + v) =
              u32x4{raw.w[v], raw.w[v + 1], raw.w[v + 2], raw.w[v + 3]};
      } else {
#pragma unroll
        for (int v = 0; v < WPL; ++v) myrow[v] = raw.w[v];
      }
    }
    float x[EPL];
    decode_raw<EPL, BF16>(raw, x);
    if (it + 1 < TPC) {                         // prefetch the cluster's next token
      const int tn = t + NCL;
      load_raw<EPL, BF16>(raw, p.logits, (size_t)tn * E, e0, E, p.vec, tn < p.T);
    }

    // ---- score basis r (kept in x) and selection key --------------------------
    float m = 0.0f, inv_s = 0.0f, ssum = 0.0f;
    if constexpr (VAR == kVarSigmoid) {
#pragma unroll
      for (int i = 0; i < EPL; ++i) x[i] = sigmoid_f32(x[i]);     // sigmoid(-inf) = 0
      if (p.scores != nullptr) {
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) part += x[i];
        ssum = cl_sum<LPT>(part);
      }
    } else {
      if (need_ms) {
        float mx = -kInf;
#pragma unroll
        for (int i = 0; i < EPL; ++i) mx = fmaxf(mx, x[i]);
        m = cl_max<LPT>(mx);
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) s += exp_f32(x[i] - m);     // exp(-inf) = 0
        inv_s = fast_rcp(cl_sum<LPT>(s));
      }
      if constexpr (VAR == kVarSoftmaxBias) {
        if (pre) {
#pragma unroll
          for (int i = 0; i < EPL; ++i) x[i] = exp_f32(x[i] - m) * inv_s;
        }
      }
    }
    if (!(kRaw || sig_raw)) {                  // the score basis, dynamically indexable
#pragma unroll
      for (int i = 0; i < EPL; i += 4)
        *reinterpret_cast<f32x4*>(myrow + i) = f32x4{x[i], x[i + 1], x[i + 2], x[i + 3]};
    }
    float key[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) key[i] = kBias ? x[i] + breg[i] : x[i];   // -inf if padded
    // top keys of the lane: four (sorted insertion with med3) when tau is
    // refined below, else two, as two interleaved chains merged at the end
    float m1, m2, m3 = -kInf, m4 = -kInf;
    if (kRefineTau && refine) {
      float a = -kInf, b = -kInf, c = -kInf, d = -kInf;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const float v = key[i];
        d = __builtin_amdgcn_fmed3f(c, d, v);
        c = __builtin_amdgcn_fmed3f(b, c, v);
        b = __builtin_amdgcn_fmed3f(a, b, v);
        a = fmaxf(a, v);
      }
      m1 = a; m2 = b; m3 = c; m4 = d;
    } else {
      float m1a = -kInf, m2a = -kInf, m1b = -kInf, m2b = -kInf;
#pragma unroll
      for (int i = 0; i < EPL; i += 2) {
        m2a = __builtin_amdgcn_fmed3f(m1a, m2a, key[i]);
        m1a = fmaxf(m1a, key[i]);
        m2b = __builtin_amdgcn_fmed3f(m1b, m2b, key[i + 1]);
        m1b = fmaxf(m1b, key[i + 1]);
      }
      m1 = fmaxf(m1a, m1b);
      m2 = fmaxf(fminf(m1a, m1b), fmaxf(m2a, m2b));
    }

    // ---- group-limited selection (a group spans p.lg whole lanes) ----------
    bool kept = m1 > -kInf;
    if (p.grouped) {
      float g1 = m1, g2 = m2;
      for (int o = 1; o < p.lg; o <<= 1) {
        const float a1 = __shfl_xor(g1, o, LPT);
        const float a2 = __shfl_xor(g2, o, LPT);
        const float n2 = fmaxf(fminf(g1, a1), fmaxf(g2, a2));
        g1 = fmaxf(g1, a1);
        g2 = n2;
      }
      // (softmax before top-k, keys = logits: the sum of the two largest
      // probabilities orders like exp(g1 - m) + exp(g2 - m), the common
      // normaliser dropped)
      const float gs = p.topn == 1 ? g1
                                   : (group_exp ? exp_f32(g1 - m) + exp_f32(g2 - m) : g1 + g2);
      const int myg = lane_c >> p.lg_shift;
      // group order as packed (score, group) words: slots n_group..LPT-1 hold 0
      const uint64_t gk = pack_key(gs, myg);
      if ((lane_c & (p.lg - 1)) == 0 && myg < p.n_group) mygs[myg] = gk;
      if (lane_c >= p.n_group) mygs[lane_c] = 0ull;
      wave_lds_sync();
      int rank = 0;
#pragma unroll
      for (int h = 0; h < LPT; h += 2) {        // n_group <= LPT
        const u64x2 v = *reinterpret_cast<const u64x2*>(mygs + h);
        rank += (v.x > gk ? 1 : 0) + (h + 1 < LPT && v.y > gk ? 1 : 0);
      }
      kept = kept && myg < p.n_group && rank < p.topk_group;
    }

    // ---- tau: a lower bound on the k-th eligible key ---------------------------
    float tau;
    if (kRefineTau && refine && LPT == 4) {
      // the k-th largest of the cluster's sixteen top-four keys (a subset of
      // the keys, so at most the k-th largest key) by two bitonic merges over
      // quad DPP moves: lanes l and l ^ 1 merge their sorted fours into one
      // sorted eight, lanes l and l ^ 2 then keep the larger (k <= 8) or the
      // smaller (k > 8) eight of the sixteen, sorted; every lane of the
      // cluster ends with the same value
      auto ce = [](float& hi, float& lo) {
        const float h = fmaxf(hi, lo), l = fminf(hi, lo);
        hi = h;
        lo = l;
      };
      const float a4[4] = {m1, m2, m3, m4};
      float pb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pb[i] = dpp_f<kDppXor1>(a4[i]);
      float s8[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s8[i] = fmaxf(a4[i], pb[3 - i]);
        s8[i + 4] = fminf(a4[i], pb[3 - i]);
      }
#pragma unroll
      for (int h = 0; h < 8; h += 4) {
        ce(s8[h], s8[h + 2]);
        ce(s8[h + 1], s8[h + 3]);
        ce(s8[h], s8[h + 1]);
        ce(s8[h + 2], s8[h + 3]);
      }
      float q8[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) q8[i] = dpp_f<kDppXor2>(s8[i]);
      float t8[8];
      const bool upper = k <= 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) t8[i] = upper ? fmaxf(s8[i], q8[7 - i]) : fminf(s8[i], q8[7 - i]);
#pragma unroll
      for (int i = 0; i < 4; ++i) ce(t8[i], t8[i + 4]);
#pragma unroll
      for (int h = 0; h < 8; h += 4) {
        ce(t8[h], t8[h + 2]);
        ce(t8[h + 1], t8[h + 3]);
        ce(t8[h], t8[h + 1]);
        ce(t8[h + 2], t8[h + 3]);
      }
      const int pos = (upper ? k : k - 8) - 1;
      tau = t8[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) tau = pos == i ? t8[i] : tau;
      if (!(tau > -kInf)) tau = kLowest;                  // fewer than k finite keys
    } else if (kRefineTau && refine) {
      // the k-th largest of the cluster's per-lane top four (a subset of the
      // keys, so at most the k-th largest key): each lane counts the values
      // >= each of its own; the largest own value with count >= k is a bound
      float* tv = reinterpret_cast<float*>(mycand);        // cluster scratch, LPT x 4
      *reinterpret_cast<f32x4*>(tv + 4 * lane_c) = f32x4{m1, m2, m3, m4};
      wave_lds_sync();
      const float mine[4] = {m1, m2, m3, m4};
      int cnt[4] = {0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < LPT; ++j) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(tv + 4 * j);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          cnt[q] += (v.x >= mine[q] ? 1 : 0) + (v.y >= mine[q] ? 1 : 0) +
                    (v.z >= mine[q] ? 1 : 0) + (v.w >= mine[q] ? 1 : 0);
      }
      float tl = -kInf;
#pragma unroll
      for (int q = 3; q >= 0; --q) tl = (mine[q] > -kInf && cnt[q] >= k) ? mine[q] : tl;
      tau = cl_max<LPT>(tl);
      if (!(tau > -kInf)) tau = kLowest;                  // fewer than k finite keys
      wave_lds_sync();                                     // scratch is reused below
    } else {
      const int cnt_l = kept ? (m1 > -kInf ? 1 : 0) + (m2 > -kInf ? 1 : 0) : 0;
      tau = cl_min<LPT>(cnt_l == 2 ? m2 : (cnt_l == 1 ? m1 : kInf));
      if (cl_sum_i<LPT>(cnt_l) < k) tau = kLowest;        // every finite key qualifies
    }
    // candidate bits: key[i] >= tau.  The sign bit of key[i] - tau marks the
    // keys below tau (-inf stays -inf; equal keys give +0); alignbit shifts it
    // in, top element first, so that bit i belongs to element i.  A zero tau
    // is taken as -0: then both -0 and +0 keys give +0 (x - x = +0, +0 - -0 =
    // +0) and count as equal to it.
    tau = tau == 0.0f ? -0.0f : tau;
    uint32_t below_hi = 0, below_lo = 0;
#pragma unroll
    for (int i = EPL / 2 - 1; i >= 0; --i) {
      below_hi = __builtin_amdgcn_alignbit(below_hi, __float_as_uint(key[i + EPL / 2] - tau), 31);
      below_lo = __builtin_amdgcn_alignbit(below_lo, __float_as_uint(key[i] - tau), 31);
    }
    const uint32_t below = (below_hi << (EPL / 2)) | below_lo;
    const uint32_t lane_bits = EPL == 32 ? 0xffffffffu : ((1u << EPL) - 1u);
    const uint32_t cmask = kept ? (~below & lane_bits) : 0u;
    const int pc = __builtin_popcount(cmask);
    const int coff = cl_excl_scan<LPT>(pc, lane_c);
    int C = cl_sum_i<LPT>(pc);

    if (C <= p.cap) {
      // compact the candidates, up to four set bits per round; the key is
      // formed again from the row (bit-identical to the register copy).  All
      // of a round's LDS reads are issued before its writes, and a round's
      // missing candidates write to the cluster's spare slot p.cap + 1 (never
      // ranked: the tier is at most the capacity) instead of branching, which
      // would put each read behind the previous write.
      uint32_t mm = cmask;
      int pos = coff;
      const int spare = p.cap + 1;
      while (mm) {
        int ii[4];
        bool hv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          hv[q] = mm != 0u;
          ii[q] = hv[q] ? __builtin_ctz(mm) : 0;
          mm &= hv[q] ? mm - 1u : mm;
        }
        float kk[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          kk[q] = row_basis<VAR, BF16, EPL>(rowc, e0 + ii[q], sig_raw, lpad);
          if constexpr (kBias) kk[q] += bias_s[e0 + BPAD * lane_c + ii[q]];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) mycand[hv[q] ? pos + q : spare] = pack_key(kk[q], e0 + ii[q]);
        pos += (int)hv[0] + (int)hv[1] + (int)hv[2] + (int)hv[3];
      }
    } else {
      // many keys tie at tau: k rounds of a cluster-wide maximum instead
      uint32_t taken = 0;
      for (int rr = 0; rr < k; ++rr) {
        uint64_t best = 0;
        if (kept) {
#pragma unroll
          for (int i = 0; i < EPL; ++i) {
            const uint64_t c = pack_key(key[i], e0 + i);
            best = (!((taken >> i) & 1u) && c > best) ? c : best;
          }
        }
        const uint64_t win = cl_max_u64<LPT>(best);
        const int wi = unpack_idx(win) - e0;
        if (wi >= 0 && wi < EPL) {
          taken |= 1u << wi;
          mycand[rr] = win;
        }
      }
      C = k;
    }
    // ranking tier: the smallest of 4, 8, 12, 16, 24, 32, 64 that holds every
    // cluster's list in this wavefront (uniform, so the wavefront takes one
    // path; the cost is about tier^2 / LPT compares per lane); the entries
    // between C and the tier are zeroed
    int tier;
    if (__ballot(C > 4) == 0ull) tier = 4;
    else if (__ballot(C > 8) == 0ull) tier = 8;
    else if (__ballot(C > 12) == 0ull) tier = 12;
    else if (__ballot(C > 16) == 0ull) tier = 16;
    else if (__ballot(C > 24) == 0ull) tier = 24;
    else if (__ballot(C > 32) == 0ull) tier = 32;
    else tier = 64;
    for (int j = C + lane_c; j < tier; j += LPT) mycand[j] = 0ull;
    wave_lds_sync();

    // ---- order the candidates, emit the top k ---------------------------------
    if (tier == 4) rank_tier<LPT, 4>(mycand, C, k, lane_c, myselidx);
    else if (tier == 8) rank_tier<LPT, 8>(mycand, C, k, lane_c, myselidx);
    else if (tier == 12) rank_tier<LPT, 12>(mycand, C, k, lane_c, myselidx);
    else if (tier == 16) rank_tier<LPT, 16>(mycand, C, k, lane_c, myselidx);
    else if (tier == 24) rank_tier<LPT, 24>(mycand, C, k, lane_c, myselidx);
    else if (tier == 32) rank_tier<LPT, 32>(mycand, C, k, lane_c, myselidx);
    else rank_tier<LPT, 64>(mycand, C, k, lane_c, myselidx);
    wave_lds_sync();
    {
      EmitCtx ec;
      ec.ids = p.ids;
      ec.weights = p.weights;
      ec.weights_bf16 = p.weights_bf16 != 0;
      ec.sig_raw = sig_raw;
      ec.lpad = lpad;
      ec.renorm = p.renorm != 0;
      ec.counting = counting;
      ec.pre = pre;
      ec.mode = mode;
      ec.k = k;
      ec.loc_off = p.loc_off;
      ec.loc_n = p.loc_n;
      ec.scale = p.scale;
      ec.hmask = hmask;
      ec.t = t;
      ec.tl = tl;
      ec.lane_c = lane_c;
      ec.tv = tv;
      ec.m = m;
      ec.inv_s = inv_s;
      emit_selected<LPT, EPL, BF16, VAR>(ec, myselidx, rowc);
    }
    // ---- full-E scores for the aux loss --------------------------------------------
    if (p.scores != nullptr) {
      const float inv_ss = VAR == kVarSigmoid ? fast_rcp(ssum) : 0.0f;
      float v[EPL];
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        if constexpr (VAR == kVarSigmoid) v[i] = x[i] * inv_ss;
        else if (VAR == kVarSoftmaxBias && pre) v[i] = x[i];
        else v[i] = exp_f32(x[i] - m) * inv_s;
      }
      // The wavefront's 64 / LPT tokens are consecutive, so their score rows
      // are one span of memory.  They pass through the wavefront's own rows in
      // LDS (free once the emission has read them), a chunk of tokens at a
      // time, so that each store instruction writes 64 consecutive 16-byte
      // pieces instead of 64 pieces one lane-slice apart.  Needs E % 4 == 0,
      // a 16-byte aligned scores array and room for one row (streaming stores:
      // nothing here reads them back); else each lane stores its slice.
      constexpr int TPW = 64 / LPT;
      const int chunk = ((E & 3) == 0 && p.scores_vec) ? (TPW * L.row_stride) / E : 0;
      if (chunk >= 1) {
        const int lw = tid & 63;
        const int tw = lw / LPT;                              // token within the wavefront
        const int tfirst = t - tw;
        float* stage = reinterpret_cast<float*>(smem + L.row) + (cl - tw) * L.row_stride;
        for (int c0 = 0; c0 < TPW; c0 += chunk) {
          wave_lds_sync();                                    // the rows, or the last chunk, are read
          if (tw >= c0 && tw < c0 + chunk) {
            float* dst = stage + (tw - c0) * E + e0;
#pragma unroll
            for (int i = 0; i < EPL; i += 4)
              if (e0 + i < E)
                *reinterpret_cast<f32x4*>(dst + i) = f32x4{v[i], v[i + 1], v[i + 2], v[i + 3]};
          }
          wave_lds_sync();
          const int ntok = min(chunk, TPW - c0);
          const int nval = max(0, min(ntok, p.T - (tfirst + c0)));   // tokens below T
          const f32x4* src = reinterpret_cast<const f32x4*>(stage);
          f32x4* out = reinterpret_cast<f32x4*>(p.scores + (size_t)(tfirst + c0) * E);
          for (int q = lw; q < nval * (E / 4); q += 64) __builtin_nontemporal_store(src[q], out + q);
        }
      } else if (tv) {
        // the row offset is formed here again (through an opaque copy of t)
        // rather than kept from the logit load across the whole token
        int to = t;
        asm volatile("" : "+v"(to));
        float* srow = p.scores + (size_t)to * E;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
          if (e0 + i < E) srow[e0 + i] = v[i];
      }
    }
    wave_lds_sync();
  }

  if (counting && p.super_rows != nullptr) {
    __syncthreads();
    int32_t* srow = p.super_rows + (size_t)cset * kCountSetInts +
                    (size_t)(blk / p.group_blocks) * p.loc_n;
    if (blk == 0 && tid == 0) {          // for this call's readers
      p.count_hdr[1] = cset | (hdr0 > 1u ? 2u : 0u);
      p.count_hdr[2 + cset] = (uint32_t)(p.num_super * p.loc_n);
    }
    for (int e = tid; e < p.loc_n; e += BLOCK) {
      const int c = __popcll(hmask[e]);
      if (p.hist != nullptr) p.hist[(size_t)blk * p.loc_n + e] = c;
      if (c != 0) atomicAdd(srow + e, c);
    }
  }
  if (p.fused) permute_in_block<BLOCK>(p, hmask, reinterpret_cast<int*>(smem + L.total));
}

template <int LPT, int EPL, bool BF16, int VAR>
hipError_t launch_route_inst(const RouteParams& p, int nb, hipStream_t s) {
  constexpr int BLOCK = kRouteBlock<LPT>;
  const bool raw_row = kRawRow<VAR, BF16> || (kSigRawOk<VAR, BF16> && p.sig_raw != 0);
  const size_t lds = route_lds_bytes(LPT, raw_row ? RawRow<EPL, BF16>::kWords : EPL,
                                     EPL, p.hmask_len, p.cap, p.k, p.grouped ? p.n_group : 0) +
                     (p.fused ? (((size_t)p.loc_n + 1) * 4 + 32 + 15) & ~(size_t)15 : 0);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&route_kernel<LPT, EPL, BF16, VAR>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  MOE_LAUNCH((route_kernel<LPT, EPL, BF16, VAR>), dim3(nb), dim3(BLOCK), lds, s, p);
  return hipGetLastError();
}

using RouteLaunchFn = hipError_t (*)(const RouteParams&, int, hipStream_t);

#define MOE_LPT_LIST(EPL, BF, VAR)                                                        \
  {launch_route_inst<1, EPL, BF, VAR>, launch_route_inst<2, EPL, BF, VAR>,                \
   launch_route_inst<4, EPL, BF, VAR>, launch_route_inst<8, EPL, BF, VAR>,                \
   launch_route_inst<16, EPL, BF, VAR>, launch_route_inst<32, EPL, BF, VAR>,              \
   launch_route_inst<64, EPL, BF, VAR>}

// Launch of one variant: table over (logits dtype, experts per lane 4..32,
// lanes per token 1..64).
template <int VAR>
hipError_t launch_route_variant(const RouteParams& p, int li, int ei, bool bf16, int nb,
                                hipStream_t s) {
  static const RouteLaunchFn table[2][4][7] = {
      {MOE_LPT_LIST(4, false, VAR), MOE_LPT_LIST(8, false, VAR), MOE_LPT_LIST(16, false, VAR),
       MOE_LPT_LIST(32, false, VAR)},
      {MOE_LPT_LIST(4, true, VAR), MOE_LPT_LIST(8, true, VAR), MOE_LPT_LIST(16, true, VAR),
       MOE_LPT_LIST(32, true, VAR)},
  };
  return table[bf16 ? 1 : 0][ei][li](p, nb, s);
}

#undef MOE_LPT_LIST

}  // namespace moe
