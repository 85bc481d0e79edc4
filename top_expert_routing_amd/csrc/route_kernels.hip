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
//                   expert / row limit.  The last block to finish reading the
//                   counting rows clears them for the next call.
// (moe_route with counts launches counts_kernel instead of scatter_kernel.)
// Integer additions commute, so the atomics leave no trace of their order:
// every output is a pure function of the input and two runs are bit-identical.
#include "device_common.hpp"
#include "kernels.hpp"

namespace moe {

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

// NP = (token, choice) pairs per thread: 64 k / kScatterThreads rounded up to
// a power of two (k <= 4, 8, 16, 32, 64).  The ids are loaded unconditionally
// (clamped index) so that all NP loads are in flight together.
// S = 2: the counting rows and per-block rows of an expert are split between
// two threads (every other row; El <= kScatterThreads / 2), so that up to 32
// counting rows and 32 per-block rows need one round of loads, not two.
template <int NP, int S>
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
  const int grp = blk / p.group_blocks;
  const int g0 = grp * p.group_blocks;
  if constexpr (S == 1) {
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
      po[e] = (tot + tile - 1) & ~(tile - 1);
      msk[e] = 0;
    }
  } else {
    // thread h * El + e sums rows h, h + 2, ... of expert e; the second half's
    // sums reach the first half through LDS
    int* part = cnt + El;                                // 2 El: tot, pre of half 1
    const int h = tid >= El ? 1 : 0;
    const int e = tid - h * El;
    int tot = 0, pre = 0;
    if (e < El) {
      for (int r0 = h; r0 < p.num_super || g0 + r0 < blk; r0 += 32) {
        int sv[16], hv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = r0 + 2 * i;
          sv[i] = r < p.num_super ? p.super_rows[(size_t)r * El + e] : 0;
          hv[i] = g0 + r < blk ? p.hist[(size_t)(g0 + r) * El + e] : 0;
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
      base[e] = pre;
      po[e] = (tot + tile - 1) & ~(tile - 1);
      msk[e] = 0;
    }
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
  for (int i = 0; i < NP; ++i) {
    const int q = tid + i * kScatterThreads;
    const int el = idv[i];
    if (el >= 0 && el < El) atomicOr(&msk[el], 1ull << ((q * p.k_magic) >> 20));
  }
  __syncthreads();
  const int total = po[El];

#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int q = tid + i * kScatterThreads;
    if (q >= valid_pairs) continue;
    const int tl = (int)((q * p.k_magic) >> 20);
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
      if (e < El) p.counts[e] = cnt[e];
    }
    if (tid == 0) {
      *p.total_out = total;
      *p.nctas_out = total >> p.tile_shift;
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

hipError_t launch_counts(int32_t* super_rows, int num_super, int El, int32_t* counts,
                         hipStream_t s) {
  MOE_LAUNCH(counts_kernel, dim3((El + 255) / 256), dim3(256), 0, s, super_rows, num_super, El,
             counts);
  return hipGetLastError();
}

// msk (El u64), po (El + 1), base, cnt (El each), and the split partials (2 El)
size_t scatter_lds_bytes(int El) { return (size_t)El * 8 + (size_t)(El + 1) * 4 + (size_t)El * 16; }

template <int S>
static void launch_scatter_s(const ScatterParams& p, int nb, hipStream_t s) {
  const size_t lds = scatter_lds_bytes(p.El);
  const int np = (kTokensPerBlock * p.k + kScatterThreads - 1) / kScatterThreads;
  if (np <= 1) MOE_LAUNCH((scatter_kernel<1, S>), dim3(nb), dim3(kScatterThreads), lds, s, p);
  else if (np <= 2) MOE_LAUNCH((scatter_kernel<2, S>), dim3(nb), dim3(kScatterThreads), lds, s, p);
  else if (np <= 4) MOE_LAUNCH((scatter_kernel<4, S>), dim3(nb), dim3(kScatterThreads), lds, s, p);
  else if (np <= 8) MOE_LAUNCH((scatter_kernel<8, S>), dim3(nb), dim3(kScatterThreads), lds, s, p);
  else MOE_LAUNCH((scatter_kernel<16, S>), dim3(nb), dim3(kScatterThreads), lds, s, p);
}

hipError_t launch_scatter(const ScatterParams& p, int nb, hipStream_t s) {
  // split the rows when an expert has more than 16 counting or per-block rows
  // to read and two threads per expert fit the block
  const int rows = p.num_super > p.group_blocks - 1 ? p.num_super : p.group_blocks - 1;
  if (2 * p.El <= kScatterThreads && rows > 16) launch_scatter_s<2>(p, nb, s);
  else launch_scatter_s<1>(p, nb, s);
  return hipGetLastError();
}

hipError_t launch_empty_outputs(int32_t* counts, int El, int32_t* padded_offsets, int32_t* total,
                                int32_t* nctas, hipStream_t s) {
  hipLaunchKernelGGL(empty_outputs_kernel, dim3(1), dim3(256), 0, s, counts, El, padded_offsets,
                     total, nctas);
  return hipGetLastError();
}

}  // namespace moe
