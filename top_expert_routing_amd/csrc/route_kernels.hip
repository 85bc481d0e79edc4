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
// Three launches per moe_route_permute call, all on the caller's stream:
//   route_kernel    one cluster of LPT lanes per token, EPL experts per lane.
//                   Logits stream HBM -> VGPRs once (16-byte loads); keys,
//                   group scores and a lower bound tau on the k-th key are
//                   formed in registers; the few keys >= tau are compacted
//                   into LDS and ranked by counting.  Per block of 64 tokens
//                   an LDS bitmask per expert records which tokens chose it;
//                   its popcounts are the block's histogram row.
//   scan_kernel     column-wise exclusive scan of the [blocks, experts]
//                   histogram -> per-(block, expert) base rank and per-expert
//                   totals (the expert_counts output).
//   scatter_kernel  per block: padded offsets from the totals, the stable
//                   in-block rank (popcount of lower bits of the bitmask),
//                   slot = offset + base + rank; writes both index maps, the
//                   padding, and the per-tile expert / row limit.
// No atomics on global memory; every output is a pure function of the input,
// so two runs are bit-identical.
#include "device_common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr float kInf = __builtin_huge_valf();

template <int EPL, bool BF16>
__device__ __forceinline__ void load_row(const void* __restrict__ base, size_t row_elems, int e0,
                                         int E, bool vec, bool tv, float (&x)[EPL]) {
  if (tv && vec && e0 + EPL <= E) {
    if constexpr (BF16) {
      const u32x4* src = reinterpret_cast<const u32x4*>(
          static_cast<const uint16_t*>(base) + row_elems + e0);
#pragma unroll
      for (int v = 0; v < EPL / 8; ++v) {
        const u32x4 q = __builtin_nontemporal_load(src + v);
        x[8 * v + 0] = bf16_lo(q.x); x[8 * v + 1] = bf16_hi(q.x);
        x[8 * v + 2] = bf16_lo(q.y); x[8 * v + 3] = bf16_hi(q.y);
        x[8 * v + 4] = bf16_lo(q.z); x[8 * v + 5] = bf16_hi(q.z);
        x[8 * v + 6] = bf16_lo(q.w); x[8 * v + 7] = bf16_hi(q.w);
      }
    } else {
      const f32x4* src = reinterpret_cast<const f32x4*>(
          static_cast<const float*>(base) + row_elems + e0);
#pragma unroll
      for (int v = 0; v < EPL / 4; ++v) {
        const f32x4 q = __builtin_nontemporal_load(src + v);
        x[4 * v + 0] = q.x; x[4 * v + 1] = q.y; x[4 * v + 2] = q.z; x[4 * v + 3] = q.w;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = e0 + i;
      float v = 0.0f;
      if (tv && e < E) {
        if constexpr (BF16)
          v = bf16_bits_to_f32(static_cast<const uint16_t*>(base)[row_elems + e]);
        else
          v = static_cast<const float*>(base)[row_elems + e];
      }
      x[i] = v;
    }
  }
}

}  // namespace

// One template instance per (lanes per token, experts per lane, logits dtype).
template <int LPT, int EPL, bool BF16>
__global__ void __launch_bounds__(kRouteBlock<LPT>) route_kernel(RouteParams p) {
  constexpr int BLOCK = kRouteBlock<LPT>;
  constexpr int NCL = BLOCK / LPT;          // clusters (tokens in flight) per block
  constexpr int TPC = kTokensPerBlock / NCL;
  constexpr int EP = LPT * EPL;             // padded row length
  static_assert(TPC * NCL == kTokensPerBlock, "block shape");
  static_assert(EPL <= 32, "lane masks are 32-bit");

  extern __shared__ __align__(16) unsigned char smem[];
  float* bias_s = reinterpret_cast<float*>(smem);
  uint64_t* hmask = reinterpret_cast<uint64_t*>(bias_s + EP);
  float* rowbuf = reinterpret_cast<float*>(hmask + p.hmask_len);
  uint64_t* cand = reinterpret_cast<uint64_t*>(rowbuf + NCL * EP);
  int* sel_idx = reinterpret_cast<int*>(cand + NCL * p.cap);
  float* sel_r = reinterpret_cast<float*>(sel_idx + NCL * p.k);

  const int tid = threadIdx.x;
  const int lane_c = tid % LPT;
  const int cl = tid / LPT;
  const int e0 = lane_c * EPL;
  const int E = p.E, k = p.k;
  const int blk = blockIdx.x;

  for (int e = tid; e < EP; e += BLOCK) {
    float b = 0.0f;
    if (p.bias != nullptr && e < E)
      b = p.bias_bf16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(p.bias)[e])
                      : static_cast<const float*>(p.bias)[e];
    bias_s[e] = b;
  }
  if (p.hist != nullptr)
    for (int e = tid; e < p.loc_n; e += BLOCK) hmask[e] = 0;
  __syncthreads();

  float breg[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) breg[i] = bias_s[e0 + i];

  const uint32_t vmask = e0 >= E ? 0u
                         : (e0 + EPL <= E ? (EPL == 32 ? 0xffffffffu : ((1u << EPL) - 1u))
                                          : ((1u << (E - e0)) - 1u));
  const int nvalid = __builtin_popcount(vmask);
  float* myrow = rowbuf + cl * EP;
  uint64_t* mycand = cand + cl * p.cap;
  int* myselidx = sel_idx + cl * k;
  float* myselr = sel_r + cl * k;

  const bool sigmoid = p.kind == kKindSigmoid;
  const bool pre = p.kind == kKindSoftmaxPre;
  const bool has_bias = p.bias != nullptr;
  const bool need_ms = !sigmoid && ((pre && (has_bias || !p.renorm)) || p.scores != nullptr);

  for (int it = 0; it < TPC; ++it) {
    const int tl = it * NCL + cl;               // token within the block
    const int t = blk * kTokensPerBlock + tl;
    const bool tv = t < p.T;
    float x[EPL];
    load_row<EPL, BF16>(p.logits, (size_t)t * E, e0, E, p.vec, tv, x);

    // ---- score basis r (kept in x) and selection key --------------------------
    float m = 0.0f, inv_s = 0.0f, ssum = 0.0f;
    if (sigmoid) {
      float part = 0.0f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        x[i] = sigmoid_f32(x[i]);
        part += ((vmask >> i) & 1u) ? x[i] : 0.0f;
      }
      if (p.scores != nullptr) ssum = cl_sum<LPT>(part);
    } else if (need_ms) {
      float mx = -kInf;
#pragma unroll
      for (int i = 0; i < EPL; ++i) mx = ((vmask >> i) & 1u) ? fmaxf(mx, x[i]) : mx;
      m = cl_max<LPT>(mx);
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) s += ((vmask >> i) & 1u) ? exp_f32(x[i] - m) : 0.0f;
      inv_s = 1.0f / cl_sum<LPT>(s);
      if (pre && has_bias) {
#pragma unroll
        for (int i = 0; i < EPL; ++i) x[i] = exp_f32(x[i] - m) * inv_s;
      }
    }
    float key[EPL];
    float m1 = -kInf, m2 = -kInf;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      key[i] = ((vmask >> i) & 1u) ? x[i] + breg[i] : -kInf;
      m2 = __builtin_amdgcn_fmed3f(m1, m2, key[i]);
      m1 = fmaxf(m1, key[i]);
    }

    // ---- group-limited selection (a group spans p.lg whole lanes) ----------
    bool kept = nvalid > 0;
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
      int rank = 0;
      for (int h = 0; h < p.n_group; ++h) {
        const float gh = __shfl(gs, h * p.lg, LPT);
        rank += (gh > gs || (gh == gs && h < myg)) ? 1 : 0;
      }
      kept = kept && myg < p.n_group && rank < p.topk_group;
    }

    // ---- tau: a lower bound on the k-th eligible key ---------------------------
    const int cnt_l = kept ? (nvalid < 2 ? nvalid : 2) : 0;
    float tau = cl_min<LPT>(cnt_l == 2 ? m2 : (cnt_l == 1 ? m1 : kInf));
    if (cl_sum_i<LPT>(cnt_l) < k) tau = -kInf;
    uint32_t cmask = 0;
    if (kept) {
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        cmask |= (((vmask >> i) & 1u) && key[i] >= tau) ? (1u << i) : 0u;
    }
    const int pc = __builtin_popcount(cmask);
    const int coff = cl_excl_scan<LPT>(pc, lane_c);
    int C = cl_sum_i<LPT>(pc);

#pragma unroll
    for (int i = 0; i < EPL; i += 4)
      *reinterpret_cast<float4*>(myrow + e0 + i) = make_float4(x[i], x[i + 1], x[i + 2], x[i + 3]);
    wave_lds_sync();

    if (C <= p.cap) {
      uint32_t mm = cmask;
      int pos = coff;
      while (mm) {
        const int i = __builtin_ctz(mm);
        mm &= mm - 1u;
        const int e = e0 + i;
        mycand[pos++] = pack_key(myrow[e] + bias_s[e], e);
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
            best = ((((vmask & ~taken) >> i) & 1u) && c > best) ? c : best;
          }
        }
        best = cl_max_u64<LPT>(best);
        const int wi = unpack_idx(best) - e0;
        if (wi >= 0 && wi < EPL) taken |= 1u << wi;
        if (lane_c == 0) mycand[rr] = best;
      }
      C = k;
    }
    wave_lds_sync();

    // ---- rank by counting: rank = number of candidates ordered before ------------
    for (int j = lane_c; j < C; j += LPT) {
      const uint64_t mine = mycand[j];
      int rank = 0;
      for (int i = 0; i < C; ++i) rank += mycand[i] > mine ? 1 : 0;
      if (rank < k) {
        const int e = unpack_idx(mine);
        myselidx[rank] = e;
        myselr[rank] = myrow[e];
      }
    }
    wave_lds_sync();

    // ---- weights -------------------------------------------------------------------
    const bool plain = sigmoid || (pre && has_bias);   // weight = basis (s or p)
    const bool exact_pre = pre && !has_bias && !p.renorm;
    float ref = 0.0f;
    if (!plain && !exact_pre) {
      float mx = -kInf;
      for (int j = lane_c; j < k; j += LPT) mx = fmaxf(mx, myselr[j]);
      ref = cl_max<LPT>(mx);
    }
    float part = 0.0f;
    for (int j = lane_c; j < k; j += LPT) {
      const float r = myselr[j];
      part += plain ? r : (exact_pre ? 0.0f : exp_f32(r - ref));
    }
    const float denom = cl_sum<LPT>(part);
    if (tv) {
      for (int j = lane_c; j < k; j += LPT) {
        const float r = myselr[j];
        float w;
        if (plain)
          w = p.renorm ? r / denom : r;
        else if (exact_pre)
          w = exp_f32(r - m) * inv_s;
        else
          w = exp_f32(r - ref) / denom;
        w *= p.scale;
        const int e = myselidx[j];
        p.ids[(size_t)t * k + j] = e;
        if (p.weights_bf16)
          static_cast<uint16_t*>(p.weights)[(size_t)t * k + j] = (uint16_t)f32_to_bf16_rne(w);
        else
          static_cast<float*>(p.weights)[(size_t)t * k + j] = w;
        if (p.hist != nullptr) {
          const int el = e - p.loc_off;
          if (el >= 0 && el < p.loc_n) atomicOr(&hmask[el], 1ull << tl);
        }
      }
      // ---- full-E scores for the aux loss --------------------------------------------
      if (p.scores != nullptr) {
        float* srow = p.scores + (size_t)t * E;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
          if ((vmask >> i) & 1u) {
            float v;
            if (sigmoid) v = x[i] / ssum;
            else if (pre && has_bias) v = x[i];
            else v = exp_f32(x[i] - m) * inv_s;
            srow[e0 + i] = v;
          }
        }
      }
    }
    wave_lds_sync();
  }

  if (p.hist != nullptr) {
    __syncthreads();
    for (int e = tid; e < p.loc_n; e += BLOCK)
      p.hist[(size_t)blk * p.loc_n + e] = __popcll(hmask[e]);
  }
}

// Column-wise exclusive scan of hist [nb][El] in place; totals -> counts[El].
// Block: 64 columns x 16 row chunks.
__global__ void __launch_bounds__(1024) scan_kernel(int32_t* __restrict__ hist, int nb, int El,
                                                    int32_t* __restrict__ counts) {
  __shared__ int part[16][64];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int col = blockIdx.x * 64 + lane;
  const int per = (nb + 15) / 16;
  const int r0 = w * per;
  const int r1 = min(nb, r0 + per);
  int s = 0;
  if (col < El)
    for (int r = r0; r < r1; ++r) s += hist[(size_t)r * El + col];
  part[w][lane] = s;
  __syncthreads();
  int pre = 0, tot = 0;
  for (int i = 0; i < 16; ++i) {
    const int v = part[i][lane];
    pre += i < w ? v : 0;
    tot += v;
  }
  if (col < El) {
    int run = pre;
    for (int r = r0; r < r1; ++r) {
      const size_t a = (size_t)r * El + col;
      const int v = hist[a];
      hist[a] = run;
      run += v;
    }
    if (w == 0) counts[col] = tot;
  }
}

// Exclusive scan of LDS array a[0..n) in place (n <= 8 * 256) with 256 threads;
// returns the total to every thread.  Uses tsum[256] scratch.
__device__ int block_excl_scan_256(int* a, int n, int* tsum) {
  const int tid = threadIdx.x;
  const int per = (n + 255) / 256;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  int s = 0;
  for (int i = lo; i < hi; ++i) s += a[i];
  tsum[tid] = s;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int v = tid >= o ? tsum[tid - o] : 0;
    __syncthreads();
    tsum[tid] += v;
    __syncthreads();
  }
  int run = tsum[tid] - s;
  const int total = tsum[255];
  __syncthreads();
  for (int i = lo; i < hi; ++i) {
    const int v = a[i];
    a[i] = run;
    run += v;
  }
  __syncthreads();
  return total;
}

__global__ void __launch_bounds__(256) scatter_kernel(ScatterParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int El = p.El;
  uint64_t* msk = reinterpret_cast<uint64_t*>(smem);
  int* po = reinterpret_cast<int*>(msk + El);          // El + 1
  int* base = po + El + 1;                              // El
  int* tsum = base + El;                                // 256
  const int tid = threadIdx.x;
  const int blk = blockIdx.x;
  const int tile = p.tile;

  for (int e = tid; e < El; e += 256) {
    const int c = p.counts[e];
    po[e] = (c + tile - 1) / tile * tile;
    msk[e] = 0;
    base[e] = p.excl[(size_t)blk * El + e];
  }
  if (tid == 0) po[El] = 0;
  __syncthreads();
  const int total = block_excl_scan_256(po, El + 1, tsum);  // po[El] = total
  const int ntiles = total / tile;

  const int k = p.k;
  const int npairs = kTokensPerBlock * k;
  const int t0 = blk * kTokensPerBlock;
  for (int q = tid; q < npairs; q += 256) {
    const int t = t0 + q / k;
    if (t < p.T) {
      const int el = p.ids[(size_t)t0 * k + q] - p.off;
      if (el >= 0 && el < El) atomicOr(&msk[el], 1ull << (q / k));
    }
  }
  __syncthreads();
  for (int q = tid; q < npairs; q += 256) {
    const int tl = q / k;
    const int t = t0 + tl;
    if (t >= p.T) continue;
    const size_t xi = (size_t)t0 * k + q;
    const int el = p.ids[xi] - p.off;
    int slot = -1;
    if (el >= 0 && el < El) {
      const uint64_t below = tl == 0 ? 0ull : (msk[el] & ((1ull << tl) - 1ull));
      slot = po[el] + base[el] + __popcll(below);
      p.p2t[slot] = t;
    }
    p.e2p[xi] = slot;
  }

  for (int c = blk * 256 + tid; c < ntiles; c += gridDim.x * 256) {
    const int pos = c * tile;
    int lo = 0, hi = El - 1;            // last e with po[e] <= pos
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (po[mid] <= pos) lo = mid; else hi = mid - 1;
    }
    const int seg_end = po[lo] + p.counts[lo];
    const int lim = min(pos + tile, seg_end);
    p.batch_idx[c] = lo;
    p.mn_limit[c] = lim;
    for (int s = max(pos, seg_end); s < pos + tile; ++s) p.p2t[s] = -1;
  }
  if (blk == 0) {
    for (int e = tid; e <= El; e += 256) p.padded_offsets[e] = po[e];
    if (tid == 0) {
      *p.total_out = total;
      *p.nctas_out = ntiles;
    }
  }
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
  const size_t lds = route_lds_bytes(LPT, EPL, p.hmask_len, p.cap, p.k);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&route_kernel<LPT, EPL, BF16>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((route_kernel<LPT, EPL, BF16>), dim3(nb), dim3(BLOCK), lds, s, p);
  return hipGetLastError();
}

size_t route_lds_bytes(int lpt, int epl, int hmask_len, int cap, int k) {
  const int block = lpt * 64 < 512 ? lpt * 64 : 512;
  const int ncl = block / lpt;
  const int ep = lpt * epl;
  return (size_t)ep * 4 + (size_t)hmask_len * 8 + (size_t)ncl * ep * 4 + (size_t)ncl * cap * 8 +
         (size_t)ncl * k * 8;
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

hipError_t launch_scan(int32_t* hist, int nb, int El, int32_t* counts, hipStream_t s) {
  hipLaunchKernelGGL(scan_kernel, dim3((El + 63) / 64), dim3(1024), 0, s, hist, nb, El, counts);
  return hipGetLastError();
}

size_t scatter_lds_bytes(int El) { return (size_t)El * 8 + (size_t)(El + 1) * 4 + (size_t)El * 4 + 256 * 4; }

hipError_t launch_scatter(const ScatterParams& p, int nb, hipStream_t s) {
  hipLaunchKernelGGL(scatter_kernel, dim3(nb), dim3(256), scatter_lds_bytes(p.El), s, p);
  return hipGetLastError();
}

hipError_t launch_empty_outputs(int32_t* counts, int El, int32_t* padded_offsets, int32_t* total,
                                int32_t* nctas, hipStream_t s) {
  hipLaunchKernelGGL(empty_outputs_kernel, dim3(1), dim3(256), 0, s, counts, El, padded_offsets,
                     total, nctas);
  return hipGetLastError();
}

}  // namespace moe
