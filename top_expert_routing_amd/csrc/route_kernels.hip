// gfx950 kernels for the tile-padded permutation and the per-expert counts;
// the route kernel itself is in route_kernel.hpp (one translation unit per
// score variant).
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
//                   expert / row limit.  Calls use two sets of counting rows
//                   in turn; the scatter blocks clear the set the previous
//                   call used, so no block has to find out that it was last.
// (moe_route with counts launches counts_kernel instead of scatter_kernel.)
// Integer additions commute, so the atomics leave no trace of their order:
// every output is a pure function of the input and two runs are bit-identical.
#include "device_common.hpp"
#include "kernels.hpp"

namespace moe {

// Per-expert totals of moe_route: sums the call's set of counting rows and
// clears it (each expert's rows are read by one thread only).  A count outside
// [0, T k] is reported as -1; a header that shows a dirty region makes every
// count -1 and clears both sets.
__global__ void counts_kernel(int32_t* __restrict__ super_rows, uint32_t* count_hdr,
                              int num_super, int El, int max_count, int32_t* __restrict__ counts) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  const uint32_t h1 = count_hdr[1];
  const bool dirty = (h1 >> 1) != 0u;
  if (e < El) {
    int32_t* rows = super_rows + (size_t)(h1 & 1u) * kCountSetInts;
    int tot = 0;
    for (int r = 0; r < num_super; ++r) {
      int32_t* a = rows + (size_t)r * El + e;
      tot += *a;
      *a = 0;
    }
    counts[e] = dirty || tot < 0 || tot > max_count ? -1 : tot;
  }
  if (dirty) {
    const int nt = gridDim.x * blockDim.x;
    for (int i = e; i < 2 * kCountSetInts; i += nt) super_rows[i] = 0;
    if (e == 0) {
      count_hdr[0] = 0u;
      count_hdr[2] = 0u;
      count_hdr[3] = 0u;
    }
  }
}

// Scatter: one block per R consecutive 64-token blocks of the route kernel
// (its sub-blocks; R divides the counting group size, so they share a group).
//   1. expert totals and the base rank of each sub-block from the call's set
//      of counting rows (rows of earlier groups), the per-block counts of
//      earlier blocks of the group and of the earlier sub-blocks; the blocks
//      clear the other set, which the previous call used, for the next call;
//   2. padded offsets (a scan over the experts), each sub-block's token
//      bitmask per expert, slot = offset + base + popcount of the lower token
//      bits;
//   3. the tiles of the experts b, b + nb, b + 2 nb, ...: expert, row limit
//      and the -1 padding of each segment's last tile.
// Every block reads the counting rows for the totals; R > 1 shares that read
// among R route blocks (large T, where those reads dominate).
constexpr int kScatterThreads = 256;

// NP = (token, choice) pairs per thread: 64 R k / kScatterThreads rounded up
// to a power of two.  The ids are loaded unconditionally (clamped index) so
// that all NP loads are in flight together.
// S = 2: the counting rows and per-block rows of an expert are split between
// two threads (every other row; El <= kScatterThreads / 2), so that up to 32
// counting rows and 32 per-block rows need one round of loads, not two.
template <int NP, int S, bool MULTI>
__global__ void __launch_bounds__(kScatterThreads) scatter_kernel(ScatterParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int El = p.El;
  const int R = MULTI ? p.sub_blocks : 1;
  uint64_t* msk = reinterpret_cast<uint64_t*>(smem);    // R El: sub-block r at r El
  int* po = reinterpret_cast<int*>(msk + R * El);       // El + 1
  int* base = po + El + 1;                               // R El
  int* cnt = base + R * El;                              // El
  const int tid = threadIdx.x;
  const int nb = gridDim.x;
  const int blk = xcd_block((int)blockIdx.x, nb);     // XCD-contiguous order
  const int tile = p.tile;
  const int k = p.k;
  const int b0 = blk * R;                                // first route block
  const int nsub = min(R, p.route_blocks - b0);
  const int npairs = kTokensPerBlock * R * k;
  const int t0 = b0 * kTokensPerBlock;
  const int valid_pairs = min(npairs, (p.T - t0) * k);

  // all global reads first (a block always holds a token: index 0 is in bounds)
  int idv[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int q = tid + i * kScatterThreads;
    idv[i] = p.ids[(size_t)t0 * k + (q < valid_pairs ? q : 0)];
  }
#pragma unroll
  for (int i = 0; i < NP; ++i)
    idv[i] = tid + i * kScatterThreads < valid_pairs ? idv[i] - p.off : -1;
  const int grp = b0 / p.group_blocks;
  const int g0 = grp * p.group_blocks;
  const uint32_t h1 = p.count_hdr[1];
  const uint32_t cset = h1 & 1u;                         // the set this call's route kernel used
  const int32_t* srows = p.super_rows + (size_t)cset * kCountSetInts;
  const uint32_t ext_other = p.count_hdr[2 + (1u - cset)];  // ints the previous user of the other touched
  const uint32_t ext_own = p.count_hdr[2 + cset];           // ints this call's route kernel touched
  int bad = 0;                                           // a count outside [0, T k]
  // per-sub-block counts of the block's own route blocks (the first needs none)
  auto own_rows = [&](int e, int pre) {
    base[e] = pre;
    for (int r = 1; r < R; ++r) {
      pre += r < nsub ? p.hist[(size_t)(b0 + r - 1) * El + e] : 0;
      base[r * El + e] = pre;
    }
  };
  if constexpr (S == 1) {
    for (int e = tid; e < El; e += kScatterThreads) {
      int tot = 0, pre = 0;
      // 16 counting rows and 16 per-block rows in flight at a time
      for (int r0 = 0; r0 < p.num_super || g0 + r0 < b0; r0 += 16) {
        int sv[16], hv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          sv[i] = r0 + i < p.num_super ? srows[(size_t)(r0 + i) * El + e] : 0;
          hv[i] = g0 + r0 + i < b0 ? p.hist[(size_t)(g0 + r0 + i) * El + e] : 0;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          tot += sv[i];
          pre += (r0 + i < grp ? sv[i] : 0) + hv[i];
        }
      }
      cnt[e] = tot;
      own_rows(e, pre);
      po[e] = (tot + tile - 1) & ~(tile - 1);
      for (int r = 0; r < R; ++r) msk[r * El + e] = 0;
      bad |= (tot < 0) | (tot > p.max_count);
    }
  } else {
    // thread h * El + e sums rows h, h + 2, ... of expert e; the second half's
    // sums reach the first half through LDS
    int* part = cnt + El;                                // 2 El: tot, pre of half 1
    const int h = tid >= El ? 1 : 0;
    const int e = tid - h * El;
    int tot = 0, pre = 0;
    if (e < El) {
      for (int r0 = h; r0 < p.num_super || g0 + r0 < b0; r0 += 32) {
        int sv[16], hv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = r0 + 2 * i;
          sv[i] = r < p.num_super ? srows[(size_t)r * El + e] : 0;
          hv[i] = g0 + r < b0 ? p.hist[(size_t)(g0 + r) * El + e] : 0;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = r0 + 2 * i;
          tot += sv[i];
          pre += (r < grp ? sv[i] : 0) + hv[i];
        }
      }
      if (h == 1) {
        part[e] = tot;
        part[El + e] = pre;
      }
    }
    __syncthreads();
    if (h == 0 && e < El) {
      tot += part[e];
      pre += part[El + e];
      cnt[e] = tot;
      own_rows(e, pre);
      po[e] = (tot + tile - 1) & ~(tile - 1);
      for (int r = 0; r < R; ++r) msk[r * El + e] = 0;
      bad |= (tot < 0) | (tot > p.max_count);
    }
  }
  if (tid == 0) po[El] = 0;
  __syncthreads();

  // token bitmasks (LDS atomics), then the exclusive scan of the padded sizes
  // over the block, 256 experts per round (wavefront scans in DPP moves).
  // Pair q is token q / k of the block: sub-block (q / k) / 64, bit (q / k) % 64.
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int q = tid + i * kScatterThreads;
    const int el = idv[i];
    const int tg = (int)((q * p.k_magic) >> 20);
    const int r = MULTI ? tg >> 6 : 0;                   // single: tg < 64
    if (el >= 0 && el < El) atomicOr(&msk[r * El + el], 1ull << (MULTI ? tg & 63 : tg));
  }
  int* scan_tmp = cnt + El;                              // kScatterThreads / 64 ints
  int carry = 0, neg = 0;
  for (int e0 = 0; e0 < El; e0 += kScatterThreads) {   // uniform trip count
    const int e = e0 + tid;
    const int v = e < El ? po[e] : 0;
    int round_total;
    const int ex = block_excl_scan<kScatterThreads>(v, scan_tmp, round_total);
    if (e < El) {
      po[e] = carry + ex;
      neg |= carry + ex < 0;                             // the running sum wrapped
    }
    carry += round_total;
    if (e0 + kScatterThreads < El) __syncthreads();     // scan_tmp is written again
  }
  if (tid == 0) po[El] = carry;
  const int wrapped = __syncthreads_or(neg | bad);          // or a count outside [0, T k]
  const int total = po[El];
  // A dirty counting region (see kCountSetInts): the permutation is not
  // written past the caller's arrays, the totals report -1 and both sets are
  // cleared.  Every term is uniform over the grid.
  const bool dirty = (h1 >> 1) != 0u || ext_other > (uint32_t)kCountSetInts ||
                     ext_own > (uint32_t)kCountSetInts || wrapped || total < 0 ||
                     total > p.max_padded;
  // The other set was used by the previous call and fully read by its
  // scatter: clear it (strided over the blocks) for the next call, which adds
  // into it; after a dirty region also the part of this call's set that its
  // route kernel did not touch (the touched part is cleared by the next call).
  {
    int32_t* other = p.super_rows + (size_t)(1u - cset) * kCountSetInts;
    const int n_other = dirty ? kCountSetInts : (int)ext_other;
    for (int i = blk * kScatterThreads + tid; i < n_other; i += nb * kScatterThreads) other[i] = 0;
    if (dirty) {
      int32_t* own = p.super_rows + (size_t)cset * kCountSetInts;
      const int from = ext_own > (uint32_t)kCountSetInts ? kCountSetInts : (int)ext_own;
      for (int i = from + blk * kScatterThreads + tid; i < kCountSetInts; i += nb * kScatterThreads)
        own[i] = 0;
    }
    if (blk == 0 && tid == 0) {
      p.count_hdr[0] = 1u - cset;
      if (dirty) p.count_hdr[2 + (1u - cset)] = 0u;   // that set is all zero now
    }
  }

#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int q = tid + i * kScatterThreads;
    if (q >= valid_pairs) continue;
    const int tg = (int)((q * p.k_magic) >> 20);
    const int tl = MULTI ? tg & 63 : tg;
    const int el = idv[i];
    int slot = -1;
    if (el >= 0 && el < El) {
      const int r = MULTI ? tg >> 6 : 0;
      const uint64_t below = tl == 0 ? 0ull : (msk[r * El + el] & ((1ull << tl) - 1ull));
      slot = po[el] + base[r * El + el] + __popcll(below);
      if ((unsigned)slot < (unsigned)p.max_padded) p.p2t[slot] = t0 + tg;
      else slot = -1;                                    // only with a dirty region
    }
    p.e2p[(size_t)t0 * k + q] = slot;
  }

  // tiles of this block's experts: b, b + nb, b + 2 nb, ... (no division);
  // with a clean region the offsets are non-decreasing and end at
  // total <= max_padded, so every tile and padding slot is in bounds
  for (int e = dirty ? El : blk; e < El; e += nb) {
    const int seg = po[e];
    const int seg_end = seg + cnt[e];
    const int ntile = (po[e + 1] - seg) >> p.tile_shift;
    for (int j = tid; j < ntile; j += kScatterThreads) {
      const int c = (seg >> p.tile_shift) + j;
      p.batch_idx[c] = e;
      p.mn_limit[c] = min(seg + (j + 1) * tile, seg_end);
    }
    for (int s2 = seg_end + tid; s2 < po[e + 1]; s2 += kScatterThreads) p.p2t[s2] = -1;
  }
  if (blk == 0) {
    for (int e = tid; e <= El; e += kScatterThreads) {
      p.padded_offsets[e] = po[e];
      if (e < El) p.counts[e] = dirty ? -1 : cnt[e];
    }
    if (tid == 0) {
      *p.total_out = dirty ? -1 : total;
      *p.nctas_out = dirty ? -1 : total >> p.tile_shift;
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

// Zero-fill of a 16-byte aligned region of n16 16-byte words (a kernel, so that
// it may be captured into a HIP graph where a memset node may not).
__global__ void zero_fill_kernel(u32x4* __restrict__ p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = u32x4{0u, 0u, 0u, 0u};
}

// ---- host-side launchers -------------------------------------------------------------

// Instances of the route kernel, one translation unit per score variant.
template <int VAR>
hipError_t launch_route_variant(const RouteParams& p, int li, int ei, bool bf16, int nb,
                                hipStream_t s);
extern template hipError_t launch_route_variant<kVarSigmoid>(const RouteParams&, int, int, bool,
                                                              int, hipStream_t);
extern template hipError_t launch_route_variant<kVarSoftmax>(const RouteParams&, int, int, bool,
                                                              int, hipStream_t);
extern template hipError_t launch_route_variant<kVarSoftmaxBias>(const RouteParams&, int, int,
                                                                  bool, int, hipStream_t);

size_t route_lds_bytes(int lpt, int rwpl, int epl, int hmask_len, int cap, int k, int n_group) {
  return route_lds_layout(lpt, rwpl, epl, hmask_len, cap, k, n_group).total;
}

static int log2i(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

hipError_t launch_route(const RouteParams& p, int lpt, int epl, bool bf16, int nb, hipStream_t s) {
  const int ei = log2i(epl) - 2;   // 4 -> 0 ... 32 -> 3
  const int li = log2i(lpt);       // 1 -> 0 ... 64 -> 6
  if (ei < 0 || ei > 3 || li > 6 || (4 << ei) != epl || (1 << li) != lpt)
    return hipErrorInvalidValue;
  switch (p.variant) {
    case kVarSigmoid: return launch_route_variant<kVarSigmoid>(p, li, ei, bf16, nb, s);
    case kVarSoftmax: return launch_route_variant<kVarSoftmax>(p, li, ei, bf16, nb, s);
    case kVarSoftmaxBias: return launch_route_variant<kVarSoftmaxBias>(p, li, ei, bf16, nb, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_counts(int32_t* super_rows, uint32_t* count_hdr, int num_super, int El,
                         int max_count, int32_t* counts, hipStream_t s) {
  MOE_LAUNCH(counts_kernel, dim3((El + 255) / 256), dim3(256), 0, s, super_rows, count_hdr,
             num_super, El, max_count, counts);
  return hipGetLastError();
}

// msk (R El u64), po (El + 1), base (R El), cnt (El), and the split
// partials (2 El), or the scan's wave sums
size_t scatter_lds_bytes(int El, int R) {
  return (size_t)R * El * 8 + (size_t)(El + 1) * 4 + (size_t)R * El * 4 + (size_t)El * 12 + 16;
}

template <int S, bool MULTI>
static void launch_scatter_s(const ScatterParams& p, int nb, hipStream_t s) {
  const size_t lds = scatter_lds_bytes(p.El, p.sub_blocks);
  const int np = (kTokensPerBlock * p.sub_blocks * p.k + kScatterThreads - 1) / kScatterThreads;
  const dim3 g(nb), b(kScatterThreads);
  if (np <= 1) MOE_LAUNCH((scatter_kernel<1, S, MULTI>), g, b, lds, s, p);
  else if (np <= 2) MOE_LAUNCH((scatter_kernel<2, S, MULTI>), g, b, lds, s, p);
  else if (np <= 4) MOE_LAUNCH((scatter_kernel<4, S, MULTI>), g, b, lds, s, p);
  else if (np <= 8) MOE_LAUNCH((scatter_kernel<8, S, MULTI>), g, b, lds, s, p);
  else MOE_LAUNCH((scatter_kernel<16, S, MULTI>), g, b, lds, s, p);
}

hipError_t launch_scatter(const ScatterParams& p, int nb, hipStream_t s) {
  // split the rows when an expert has more than 16 counting or per-block rows
  // to read and two threads per expert fit the block
  const int rows = p.num_super > p.group_blocks - 1 ? p.num_super : p.group_blocks - 1;
  const bool split = 2 * p.El <= kScatterThreads && rows > 16;
  if (p.sub_blocks > 1) {
    if (split) launch_scatter_s<2, true>(p, nb, s);
    else launch_scatter_s<1, true>(p, nb, s);
  } else {
    if (split) launch_scatter_s<2, false>(p, nb, s);
    else launch_scatter_s<1, false>(p, nb, s);
  }
  return hipGetLastError();
}

hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  const int blocks = (int)((n16 + 255) / 256 < 1024 ? (n16 + 255) / 256 : 1024);
  if (blocks > 0)
    hipLaunchKernelGGL(zero_fill_kernel, dim3(blocks), dim3(256), 0, s, static_cast<u32x4*>(p), n16);
  return hipGetLastError();
}

hipError_t launch_empty_outputs(int32_t* counts, int El, int32_t* padded_offsets, int32_t* total,
                                int32_t* nctas, hipStream_t s) {
  hipLaunchKernelGGL(empty_outputs_kernel, dim3(1), dim3(256), 0, s, counts, El, padded_offsets,
                     total, nctas);
  return hipGetLastError();
}

}  // namespace moe
