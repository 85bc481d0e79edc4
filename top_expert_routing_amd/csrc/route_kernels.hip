// gfx950 kernels for MoE top-k routing and the tile-padded permutation.
//
// Method (page title, section):
//   score function, pre/post-softmax order, group top-k, expert bias, scaling:
//     TransformerEngine Fused Router, Description + I/O Contract;
//   n_group / topk_group, routing bias, routed_scaling_factor, norm_topk_prob,
//   tile_tokens_dim, local experts, the permutation outputs and the
//   slot -> tile -> expert rule: flashinfer trtllm_gen_routing, Parameters,
//   Returns, Notes;
//   float32 sigmoid, selection by score + correction bias, unbiased weights:
//     MAX SigmoidTopKRouter, routing steps 2-4.
//
// Two launches per moe_route_permute call, both on the caller's stream:
//   route_kernel    one cluster of LPT lanes per token, EPL experts per lane.
//                   Logits stream HBM -> VGPRs once (16-byte loads); keys,
//                   group scores and a lower bound tau on the k-th key are
//                   formed in registers; the few keys >= tau are compacted
//                   into LDS and ranked by counting.  Per block of 64 tokens
//                   an LDS bitmask per expert records which tokens chose it;
//                   its popcounts are the block's histogram row.
//                   At its end each block writes its counts row and adds it
//                   into a counting row shared by a group of G blocks.
//   scatter_kernel  per block: expert totals and the block's base ranks from
//                   the counting rows plus the rows of earlier blocks of its
//                   group, padded offsets, the stable in-block rank (popcount
//                   of lower bits of the bitmask), slot = offset + base + rank;
//                   writes both index maps, the padding, and the per-tile
//                   expert / row limit.  The last block to finish reading the
//                   counting rows clears them for the next call.
// (moe_route with counts launches counts_kernel instead of scatter_kernel.)
// Integer additions commute, so the atomics leave no trace of their order:
// every output is a pure function of the input and two runs are bit-identical.
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

// Per-token values the emission needs.
struct EmitCtx {
  int32_t* ids;
  void* weights;
  bool weights_bf16, renorm, counting;
  int mode, k, loc_off, loc_n;
  float scale;
  uint64_t* hmask;
  int t, tl, lane_c;
  bool tv;
  float m, inv_s;
};

// Rank the cluster's C candidates by counting among the first T entries of its
// candidate list (entries C..T-1 hold 0, below every packed key).  Lane c
// ranks entries c, c + LPT, ...; a candidate of rank n < k is recorded at
// position n of the selection list.
template <int LPT, int T>
__device__ __forceinline__ void rank_tier(const uint64_t* mycand, const float* mycandr, int C,
                                          int k, int lane_c, int* myselidx, float* myselr) {
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
    if (rank < k) {
      myselidx[rank] = unpack_idx(mine);
      myselr[rank] = mycandr[j];
    }
  }
}

// Weights, ids and the block bitmask for the k selected, by rank: lane c
// handles ranks c, c + LPT, ... (contiguous stores across the cluster).
template <int LPT>
__device__ __forceinline__ void emit_selected(const EmitCtx& c, const int* myselidx,
                                              const float* myselr) {
  const int k = c.k;
  float ref = 0.0f;
  if (c.mode == kEmitSoftSel) {
    float mx = -__builtin_huge_valf();
    for (int n = c.lane_c; n < k; n += LPT) mx = fmaxf(mx, myselr[n]);
    ref = cl_max<LPT>(mx);
  }
  float inv_den = c.inv_s;
  if (c.mode != kEmitExactPre) {
    float part = 0.0f;
    for (int n = c.lane_c; n < k; n += LPT)
      part += c.mode == kEmitPlain ? myselr[n] : exp_f32(myselr[n] - ref);
    inv_den = fast_rcp(cl_sum<LPT>(part));
  }
  if (!c.tv) return;
  const float sub = c.mode == kEmitExactPre ? c.m : ref;
  for (int n = c.lane_c; n < k; n += LPT) {
    const float r = myselr[n];
    const int e = myselidx[n];
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

// One template instance per (lanes per token, experts per lane, logits dtype).
//
// Padded experts (e >= E) carry logit -inf and bias -inf, so their keys are
// -inf and no per-element validity masks are needed anywhere.
template <int LPT, int EPL, bool BF16>
__global__ void __launch_bounds__(kRouteBlock<LPT>) route_kernel(RouteParams p) {
  constexpr int BLOCK = kRouteBlock<LPT>;
  constexpr int NCL = BLOCK / LPT;          // clusters (tokens in flight) per block
  constexpr int TPC = kTokensPerBlock / NCL;
  constexpr int EP = LPT * EPL;             // padded row length
  constexpr int LSTR = EPL + 4;             // row floats per lane (+4 against bank conflicts)
  static_assert(TPC * NCL == kTokensPerBlock, "block shape");
  static_assert(EPL <= 32, "lane masks are 32-bit");
  constexpr float kLowest = -3.402823466e38f;

  const int tid = threadIdx.x;
  const int lane_c = tid % LPT;
  const int cl = tid / LPT;
  const int e0 = lane_c * EPL;
  const int E = p.E, k = p.k;
  const int blk = blockIdx.x;
  const bool has_bias = p.bias != nullptr;

  const RouteLds L = route_lds_layout(LPT, EPL, p.hmask_len, p.cap, k, p.grouped ? p.n_group : 0);
  extern __shared__ __align__(16) unsigned char smem[];
  float* bias_s = reinterpret_cast<float*>(smem + L.bias);
  uint64_t* hmask = reinterpret_cast<uint64_t*>(smem + L.hmask);
  float* myrow = reinterpret_cast<float*>(smem + L.row) + cl * L.row_stride + lane_c * LSTR;
  uint64_t* mycand = reinterpret_cast<uint64_t*>(smem + L.cand) + cl * L.cand_stride;
  float* mycandr = reinterpret_cast<float*>(smem + L.cand_r) + cl * L.cand_stride;
  int* myselidx = reinterpret_cast<int*>(smem + L.sel_idx) + cl * L.sel_stride;
  float* myselr = reinterpret_cast<float*>(smem + L.sel_r) + cl * L.sel_stride;
  float* mygs = reinterpret_cast<float*>(smem + L.gscore) + cl * L.gs_stride;

  // The bias is requested first (one block-wide pass into LDS), then the
  // first token's logits; the bias lands in LDS while the logits are in flight.
  float bload = 0.0f;
  const bool bthread = tid < EP;
  if (bthread) {
    if (tid >= E)
      bload = -kInf;
    else if (has_bias)
      bload = p.bias_bf16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(p.bias)[tid])
                          : static_cast<const float*>(p.bias)[tid];
  }
  RawRow<EPL, BF16> raw;
  {
    const int t = blk * kTokensPerBlock + cl;
    load_raw<EPL, BF16>(raw, p.logits, (size_t)t * E, e0, E, p.vec, t < p.T);
  }
  for (int e = tid; e < EP; e += BLOCK) {          // EP > BLOCK only for very wide rows
    float b = e == tid ? bload : (e >= E ? -kInf : 0.0f);
    if (e != tid && e < E && has_bias)
      b = p.bias_bf16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(p.bias)[e])
                      : static_cast<const float*>(p.bias)[e];
    bias_s[e] = b;
  }
  const bool counting = p.super_rows != nullptr;
  if (counting)
    for (int e = tid; e < p.loc_n; e += BLOCK) hmask[e] = 0;
  __syncthreads();
  float breg[EPL];
#pragma unroll
  for (int i = 0; i < EPL; i += 4) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(bias_s + e0 + i);
    breg[i] = v.x; breg[i + 1] = v.y; breg[i + 2] = v.z; breg[i + 3] = v.w;
  }

  const bool sigmoid = p.kind == kKindSigmoid;
  const bool pre = p.kind == kKindSoftmaxPre;
  const bool need_ms = !sigmoid && ((pre && (has_bias || !p.renorm)) || p.scores != nullptr);
  const int mode = (sigmoid || (pre && has_bias)) ? kEmitPlain
                   : ((pre && !p.renorm) ? kEmitExactPre : kEmitSoftSel);

  for (int it = 0; it < TPC; ++it) {
    const int tl = it * NCL + cl;               // token within the block
    const int t = blk * kTokensPerBlock + tl;
    const bool tv = t < p.T;
    float x[EPL];
    decode_raw<EPL, BF16>(raw, x);
    if (it + 1 < TPC) {                         // prefetch the cluster's next token
      const int tn = t + NCL;
      load_raw<EPL, BF16>(raw, p.logits, (size_t)tn * E, e0, E, p.vec, tn < p.T);
    }

    // ---- score basis r (kept in x) and selection key --------------------------
    float m = 0.0f, inv_s = 0.0f, ssum = 0.0f;
    if (sigmoid) {
#pragma unroll
      for (int i = 0; i < EPL; ++i) x[i] = sigmoid_f32(x[i]);     // sigmoid(-inf) = 0
      if (p.scores != nullptr) {
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) part += x[i];
        ssum = cl_sum<LPT>(part);
      }
    } else if (need_ms) {
      float mx = -kInf;
#pragma unroll
      for (int i = 0; i < EPL; ++i) mx = fmaxf(mx, x[i]);
      m = cl_max<LPT>(mx);
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) s += exp_f32(x[i] - m);     // exp(-inf) = 0
      inv_s = fast_rcp(cl_sum<LPT>(s));
      if (pre && has_bias) {
#pragma unroll
        for (int i = 0; i < EPL; ++i) x[i] = exp_f32(x[i] - m) * inv_s;
      }
    }
    float key[EPL];
    float m1 = -kInf, m2 = -kInf;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      key[i] = x[i] + breg[i];                  // -inf for padded experts
      m2 = __builtin_amdgcn_fmed3f(m1, m2, key[i]);
      m1 = fmaxf(m1, key[i]);
    }
    // the score basis, dynamically indexable by this lane
#pragma unroll
    for (int i = 0; i < EPL; i += 4)
      *reinterpret_cast<f32x4*>(myrow + i) = f32x4{x[i], x[i + 1], x[i + 2], x[i + 3]};

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
      const float gs = p.topn == 1 ? g1 : g1 + g2;
      const int myg = lane_c / p.lg;
      if (lane_c % p.lg == 0 && myg < p.n_group) mygs[myg] = gs;
      wave_lds_sync();
      int rank = 0;
#pragma unroll
      for (int h0 = 0; h0 < LPT; h0 += 4) {     // n_group <= LPT
        const f32x4 v = *reinterpret_cast<const f32x4*>(mygs + h0);
        const float gv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int u = 0; u < 4 && h0 + u < LPT; ++u) {
          const int h = h0 + u;
          rank += (h < p.n_group && (gv[u] > gs || (gv[u] == gs && h < myg))) ? 1 : 0;
        }
      }
      kept = kept && myg < p.n_group && rank < p.topk_group;
    }

    // ---- tau: a lower bound on the k-th eligible key ---------------------------
    const int cnt_l = kept ? (m1 > -kInf ? 1 : 0) + (m2 > -kInf ? 1 : 0) : 0;
    float tau = cl_min<LPT>(cnt_l == 2 ? m2 : (cnt_l == 1 ? m1 : kInf));
    if (cl_sum_i<LPT>(cnt_l) < k) tau = kLowest;          // every finite key qualifies
    // candidate bits: key[i] >= tau.  The sign bit of key[i] - tau marks the
    // keys below tau (-inf stays -inf; equal keys give +0); alignbit shifts it
    // in, top element first, so that bit i belongs to element i.
    uint32_t below = 0;
#pragma unroll
    for (int i = EPL - 1; i >= 0; --i)
      below = __builtin_amdgcn_alignbit(below, __float_as_uint(key[i] - tau), 31);
    const uint32_t lane_bits = EPL == 32 ? 0xffffffffu : ((1u << EPL) - 1u);
    const uint32_t cmask = kept ? (~below & lane_bits) : 0u;
    const int pc = __builtin_popcount(cmask);
    const int coff = cl_excl_scan<LPT>(pc, lane_c);
    int C = cl_sum_i<LPT>(pc);

    if (C <= p.cap) {
      // compact the candidates, two set bits per round
      uint32_t mm = cmask;
      int pos = coff;
      while (mm) {
        const int i0 = __builtin_ctz(mm);
        mm &= mm - 1u;
        const bool h1 = mm != 0u;
        const int i1 = h1 ? __builtin_ctz(mm) : i0;
        mm &= h1 ? mm - 1u : mm;
        const float r0 = myrow[i0], r1 = myrow[i1];
        const float b0 = bias_s[e0 + i0], b1 = bias_s[e0 + i1];
        mycand[pos] = pack_key(r0 + b0, e0 + i0);
        mycandr[pos] = r0;
        if (h1) {
          mycand[pos + 1] = pack_key(r1 + b1, e0 + i1);
          mycandr[pos + 1] = r1;
        }
        pos += h1 ? 2 : 1;
      }
    } else {
      // many keys tie at tau: k rounds of a cluster-wide maximum instead
      uint32_t taken = 0;
      for (int rr = 0; rr < k; ++rr) {
        uint64_t best = 0;
        float bestr = 0.0f;
        if (kept) {
#pragma unroll
          for (int i = 0; i < EPL; ++i) {
            const uint64_t c = pack_key(key[i], e0 + i);
            const bool take = !((taken >> i) & 1u) && c > best;
            best = take ? c : best;
            bestr = take ? x[i] : bestr;
          }
        }
        const uint64_t win = cl_max_u64<LPT>(best);
        const int wi = unpack_idx(win) - e0;
        if (wi >= 0 && wi < EPL) {
          taken |= 1u << wi;
          mycand[rr] = win;
          mycandr[rr] = bestr;
        }
      }
      C = k;
    }
    // ranking tier: the smallest of 4..64 that holds every cluster's list in
    // this wavefront (uniform, so the wavefront takes one path); the entries
    // between C and the tier are zeroed
    int tier;
    if (__ballot(C > 4) == 0ull) tier = 4;
    else if (__ballot(C > 8) == 0ull) tier = 8;
    else if (__ballot(C > 16) == 0ull) tier = 16;
    else if (__ballot(C > 32) == 0ull) tier = 32;
    else tier = 64;
    for (int j = C + lane_c; j < tier; j += LPT) mycand[j] = 0ull;
    wave_lds_sync();

    // ---- order the candidates, emit the top k ---------------------------------
    if (tier == 4) rank_tier<LPT, 4>(mycand, mycandr, C, k, lane_c, myselidx, myselr);
    else if (tier == 8) rank_tier<LPT, 8>(mycand, mycandr, C, k, lane_c, myselidx, myselr);
    else if (tier == 16) rank_tier<LPT, 16>(mycand, mycandr, C, k, lane_c, myselidx, myselr);
    else if (tier == 32) rank_tier<LPT, 32>(mycand, mycandr, C, k, lane_c, myselidx, myselr);
    else rank_tier<LPT, 64>(mycand, mycandr, C, k, lane_c, myselidx, myselr);
    wave_lds_sync();
    {
      EmitCtx ec;
      ec.ids = p.ids;
      ec.weights = p.weights;
      ec.weights_bf16 = p.weights_bf16 != 0;
      ec.renorm = p.renorm != 0;
      ec.counting = counting;
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
      emit_selected<LPT>(ec, myselidx, myselr);
    }
    if (tv) {
      // ---- full-E scores for the aux loss --------------------------------------------
      if (p.scores != nullptr) {
        float* srow = p.scores + (size_t)t * E;
        const float inv_ss = sigmoid ? fast_rcp(ssum) : 0.0f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
          if (e0 + i < E) {
            float v;
            if (sigmoid) v = x[i] * inv_ss;
            else if (pre && has_bias) v = x[i];
            else v = exp_f32(x[i] - m) * inv_s;
            srow[e0 + i] = v;
          }
        }
      }
    }
    wave_lds_sync();
  }

  if (counting) {
    __syncthreads();
    int32_t* srow = p.super_rows + (size_t)(blk / p.group_blocks) * p.loc_n;
    for (int e = tid; e < p.loc_n; e += BLOCK) {
      const int c = __popcll(hmask[e]);
      if (p.hist != nullptr) p.hist[(size_t)blk * p.loc_n + e] = c;
      if (c != 0) atomicAdd(srow + e, c);
    }
  }
}

// Per-expert totals of moe_route: sums the counting rows and clears them.
__global__ void counts_kernel(int32_t* __restrict__ super_rows, int num_super, int El,
                              int32_t* __restrict__ counts) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= El) return;
  int tot = 0;
  for (int r = 0; r < num_super; ++r) {
    int32_t* a = super_rows + (size_t)r * El + e;
    tot += *a;
    *a = 0;
  }
  counts[e] = tot;
}

// Scatter: one block per 64-token block of the route kernel.
//   1. expert totals and this block's base ranks from the counting rows (rows
//      of earlier groups) and the per-block counts of earlier blocks of its
//      own group; the block that finishes those reads last clears the rows;
//   2. padded offsets (a scan over the experts), the block's token bitmask per
//      expert, slot = offset + base + popcount of the lower token bits;
//   3. the tiles of the experts [b*El/nb, (b+1)*El/nb): expert, row limit and
//      the -1 padding of each segment's last tile.
constexpr int kScatterThreads = 256;
constexpr int kDoneLanes = 16;          // sub-counters of the block count
constexpr int kDoneStride = 64;         // 256 bytes apart: separate cache lines
constexpr int kScatterPairsPerThread = kTokensPerBlock * 64 / kScatterThreads;   // k <= 64

__global__ void __launch_bounds__(kScatterThreads) scatter_kernel(ScatterParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int last_block;
  const int El = p.El;
  uint64_t* msk = reinterpret_cast<uint64_t*>(smem);
  int* po = reinterpret_cast<int*>(msk + El);           // El + 1
  int* base = po + El + 1;                               // El
  int* cnt = base + El;                                  // El
  const int tid = threadIdx.x;
  const int blk = blockIdx.x;
  const int nb = gridDim.x;
  const int tile = p.tile;
  const int k = p.k;
  const int npairs = kTokensPerBlock * k;
  const int t0 = blk * kTokensPerBlock;
  const int valid_pairs = min(npairs, (p.T - t0) * k);

  // all global reads first
  int idv[kScatterPairsPerThread];
#pragma unroll
  for (int i = 0; i < kScatterPairsPerThread; ++i) {
    const int q = tid + i * kScatterThreads;
    idv[i] = q < valid_pairs ? p.ids[(size_t)t0 * k + q] - p.off : -1;
  }
  const int grp = blk / p.group_blocks;
  const int g0 = grp * p.group_blocks;
  for (int e = tid; e < El; e += kScatterThreads) {
    int tot = 0, pre = 0;
    // 16 counting rows and 16 per-block rows in flight at a time
    for (int r0 = 0; r0 < p.num_super || g0 + r0 < blk; r0 += 16) {
      int sv[16], hv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sv[i] = r0 + i < p.num_super ? p.super_rows[(size_t)(r0 + i) * El + e] : 0;
        hv[i] = g0 + r0 + i < blk ? p.hist[(size_t)(g0 + r0 + i) * El + e] : 0;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        tot += sv[i];
        pre += (r0 + i < grp ? sv[i] : 0) + hv[i];
      }
    }
    cnt[e] = tot;
    base[e] = pre;
    po[e] = (tot + tile - 1) / tile * tile;
    msk[e] = 0;
  }
  if (tid == 0) po[El] = 0;
  __syncthreads();
  // Every thread's counting-row reads have returned (their sums are in LDS):
  // count this block, on one of kDoneLanes sub-counters (blocks b = j mod
  // kDoneLanes) so that no address takes more than nb / kDoneLanes atomics;
  // the last block of each sub-counter then counts on the top counter.  The
  // return value is awaited only at the end, so that its latency overlaps the
  // rest of the block's work.
  const int dj = blk % kDoneLanes;
  const unsigned dn = (unsigned)((nb - dj + kDoneLanes - 1) / kDoneLanes);   // blocks of sub-counter dj
  unsigned done_before = 0u;
  if (tid == kScatterThreads - 64) done_before = atomicAdd(p.done + (dj + 1) * kDoneStride, 1u);

  // wave 0: exclusive scan of the padded sizes; everyone: token bitmasks
  if (tid < 64) {
    const int n = El + 1;
    const int per = (n + 63) / 64;
    const int lo = min(n, tid * per), hi = min(n, lo + per);
    int sum = 0;
    for (int i = lo; i < hi; ++i) sum += po[i];
    int incl = sum;
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o, 64);
      if (tid >= o) incl += u;
    }
    int run = incl - sum;
    for (int i = lo; i < hi; ++i) {
      const int v = po[i];
      po[i] = run;
      run += v;
    }
  }
#pragma unroll
  for (int i = 0; i < kScatterPairsPerThread; ++i) {
    const int q = tid + i * kScatterThreads;
    const int el = idv[i];
    if (el >= 0 && el < El) atomicOr(&msk[el], 1ull << (q / k));
  }
  __syncthreads();
  const int total = po[El];

#pragma unroll
  for (int i = 0; i < kScatterPairsPerThread; ++i) {
    const int q = tid + i * kScatterThreads;
    if (q >= valid_pairs) continue;
    const int tl = q / k;
    const int el = idv[i];
    int slot = -1;
    if (el >= 0 && el < El) {
      const uint64_t below = tl == 0 ? 0ull : (msk[el] & ((1ull << tl) - 1ull));
      slot = po[el] + base[el] + __popcll(below);
      p.p2t[slot] = t0 + tl;
    }
    p.e2p[(size_t)t0 * k + q] = slot;
  }

  // tiles of this block's experts
  const int e_lo = (int)((int64_t)blk * El / nb);
  const int e_hi = (int)((int64_t)(blk + 1) * El / nb);
  for (int e = e_lo; e < e_hi; ++e) {
    const int seg = po[e];
    const int seg_end = seg + cnt[e];
    const int ntile = (po[e + 1] - seg) / tile;
    for (int j = tid; j < ntile; j += kScatterThreads) {
      const int c = seg / tile + j;
      p.batch_idx[c] = e;
      p.mn_limit[c] = min(seg + (j + 1) * tile, seg_end);
    }
    for (int s2 = seg_end + tid; s2 < po[e + 1]; s2 += kScatterThreads) p.p2t[s2] = -1;
  }
  if (blk == 0) {
    for (int e = tid; e <= El; e += kScatterThreads) {
      p.padded_offsets[e] = po[e];
      if (e < El) p.counts[e] = cnt[e];
    }
    if (tid == 0) {
      *p.total_out = total;
      *p.nctas_out = total / tile;
    }
  }
  // the last block to finish reading the counting rows clears them
  if (tid == kScatterThreads - 64) {
    bool last = false;
    if (done_before == dn - 1u) {                  // last of its sub-counter
      p.done[(dj + 1) * kDoneStride] = 0u;         // nobody else touches it in this call
      const unsigned nsub = (unsigned)min(nb, kDoneLanes);
      last = atomicAdd(p.done, 1u) == nsub - 1u;
      if (last) p.done[0] = 0u;
    }
    last_block = last;
  }
  __syncthreads();
  if (last_block)
    for (int i = tid; i < p.num_super * El; i += kScatterThreads) p.super_rows[i] = 0;
}

// T = 0: the bookkeeping outputs still hold their defined values.
__global__ void empty_outputs_kernel(int32_t* counts, int El, int32_t* padded_offsets,
                                     int32_t* total, int32_t* nctas) {
  for (int e = threadIdx.x; e <= El; e += blockDim.x) {
    if (e < El && counts != nullptr) counts[e] = 0;
    if (padded_offsets != nullptr) padded_offsets[e] = 0;
  }
  if (threadIdx.x == 0) {
    if (total != nullptr) *total = 0;
    if (nctas != nullptr) *nctas = 0;
  }
}

// ---- host-side launchers -------------------------------------------------------------

template <int LPT, int EPL, bool BF16>
static hipError_t launch_route_inst(const RouteParams& p, int nb, hipStream_t s) {
  constexpr int BLOCK = kRouteBlock<LPT>;
  const size_t lds = route_lds_bytes(LPT, EPL, p.hmask_len, p.cap, p.k, p.grouped ? p.n_group : 0);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&route_kernel<LPT, EPL, BF16>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  MOE_LAUNCH((route_kernel<LPT, EPL, BF16>), dim3(nb), dim3(BLOCK), lds, s, p);
  return hipGetLastError();
}

size_t route_lds_bytes(int lpt, int epl, int hmask_len, int cap, int k, int n_group) {
  return route_lds_layout(lpt, epl, hmask_len, cap, k, n_group).total;
}

using LaunchFn = hipError_t (*)(const RouteParams&, int, hipStream_t);

#define MOE_LPT_LIST(EPL, BF)                                                                  \
  {launch_route_inst<1, EPL, BF>, launch_route_inst<2, EPL, BF>, launch_route_inst<4, EPL, BF>, \
   launch_route_inst<8, EPL, BF>, launch_route_inst<16, EPL, BF>,                             \
   launch_route_inst<32, EPL, BF>, launch_route_inst<64, EPL, BF>}

static const LaunchFn kRouteTable[2][4][7] = {
    {MOE_LPT_LIST(4, false), MOE_LPT_LIST(8, false), MOE_LPT_LIST(16, false),
     MOE_LPT_LIST(32, false)},
    {MOE_LPT_LIST(4, true), MOE_LPT_LIST(8, true), MOE_LPT_LIST(16, true),
     MOE_LPT_LIST(32, true)},
};

static int log2i(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

hipError_t launch_route(const RouteParams& p, int lpt, int epl, bool bf16, int nb, hipStream_t s) {
  const int ei = log2i(epl) - 2;   // 4 -> 0 ... 32 -> 3
  const int li = log2i(lpt);       // 1 -> 0 ... 64 -> 6
  return kRouteTable[bf16 ? 1 : 0][ei][li](p, nb, s);
}

hipError_t launch_counts(int32_t* super_rows, int num_super, int El, int32_t* counts,
                         hipStream_t s) {
  MOE_LAUNCH(counts_kernel, dim3((El + 255) / 256), dim3(256), 0, s, super_rows, num_super, El,
             counts);
  return hipGetLastError();
}

size_t scatter_lds_bytes(int El) { return (size_t)El * 8 + (size_t)(El + 1) * 4 + (size_t)El * 8; }

hipError_t launch_scatter(const ScatterParams& p, int nb, hipStream_t s) {
  MOE_LAUNCH(scatter_kernel, dim3(nb), dim3(kScatterThreads), scatter_lds_bytes(p.El), s, p);
  return hipGetLastError();
}

hipError_t launch_empty_outputs(int32_t* counts, int El, int32_t* padded_offsets, int32_t* total,
                                int32_t* nctas, hipStream_t s) {
  hipLaunchKernelGGL(empty_outputs_kernel, dim3(1), dim3(256), 0, s, counts, El, padded_offsets,
                     total, nctas);
  return hipGetLastError();
}

}  // namespace moe
