// Internal interface between the host library and the gfx950 kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Dispatch timestamps for the next single-kernel launch of this host thread.
// While a profiling caller sets them, the launchers go through
// hipExtLaunchKernel, which stamps the two events at the kernel's own start and
// end (the same clock a kernel trace reads); otherwise both are null.
struct LaunchStamp {
  hipEvent_t start = nullptr, stop = nullptr;
};
LaunchStamp& launch_stamp();

// Launch `kernel` on `s`, stamped when a profiling caller asked for it.
#define MOE_LAUNCH(kernel, grid, block, lds, s, ...)                                     \
  do {                                                                                   \
    const ::moe::LaunchStamp st_ = ::moe::launch_stamp();                                \
    if (st_.start != nullptr)                                                            \
      hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)(lds), s, st_.start, st_.stop, \
                            0u, __VA_ARGS__);                                            \
    else                                                                                 \
      hipLaunchKernelGGL(kernel, grid, block, lds, s, __VA_ARGS__);                      \
  } while (0)

constexpr int kTokensPerBlock = 64;   // tokens per route/scatter block (one u64 bitmask)

// Per-expert counting: each route block adds its counts into one of at most
// kMaxSuperRows rows (blocks [s*G, (s+1)*G) into row s).  The rows live at the
// start of the routing workspace in two sets that calls of moe_route_permute
// use in turn, so that no reader has to find out that it read them last: the
// scatter blocks of one call clear the set the previous call used.  A header
// of four words follows the sets:
//   hdr[0]  the set the next route kernel adds into,
//   hdr[1]  the set the current call's readers read, plus 2 when hdr[0] held
//           neither 0 nor 1 (written by route block 0),
//   hdr[2 + s]  how many ints of set s the call that last used it touched.
// A set is entirely zero whenever a route kernel starts adding into it.
// Every index taken from the region is masked or clamped into it, so a
// region that is not clean (never zeroed, or left by a launch that failed
// mid-call) cannot move an access out of bounds.  The readers treat a header
// out of range, a count outside [0, T k] or padded offsets that overflow as a
// dirty region: they report it (-1 totals or counts) and clear both sets.
constexpr int kMaxSuperRows = 64;
constexpr int kMaxCountExperts = 2048;
constexpr int kCountSetInts = kMaxSuperRows * kMaxCountExperts;

template <int LPT>
constexpr int kRouteBlock = (LPT * 64 < 512) ? LPT * 64 : 512;
// Wavefronts per SIMD the register allocation must allow: with up to 8 lanes
// per token the kernel fits in 128 VGPRs, so four wavefronts share a SIMD
// (a 65536-token call then runs in one round: 4096 wavefronts on 1024 SIMDs);
// wider clusters hold more per-lane state and are left unconstrained.
template <int LPT>
constexpr int kRouteMinWaves = LPT <= 8 ? 4 : 1;

// Score variants, one kernel instance each: sigmoid (bias optional), softmax
// without bias, softmax with bias (before or after top-k is a run-time flag).
enum { kVarSigmoid = 0, kVarSoftmax = 1, kVarSoftmaxBias = 2 };

struct RouteParams {
  const void* logits;
  const void* bias;       // nullable [E]
  int32_t* ids;           // [T, k]
  void* weights;          // [T, k] f32 or bf16
  float* scores;          // nullable [T, E]
  int32_t* super_rows;    // nullable: the two sets of counting rows (counting on when set)
  uint32_t* count_hdr;    // their header (see kCountSetInts)
  int32_t* hist;          // nullable [nb, loc_n]: per-block counts, for the permutation
  int group_blocks;       // blocks that add into one counting row
  int num_super;          // counting rows this call uses
  int T, E, k;
  int variant;            // kVar*
  int pre;                // softmax before top-k
  int bias_bf16;
  int weights_bf16;
  int grouped, n_group, topk_group, topn, lg, lg_shift;   // lg = 1 << lg_shift lanes per group
  int renorm;
  float scale;
  int vec;                // 16-byte vector loads of logits allowed
  int bias_vec;           // 16-byte aligned float32 bias
  int scores_vec;         // scores 16-byte aligned (16-byte stores of whole rows)
  int loc_off, loc_n;
  int hmask_len;          // LDS u64 words for the block bitmask (even)
  int cap;                // candidate list capacity per token (>= k)
  int sig_raw;            // sigmoid, bfloat16 logits: keep the raw logits in the LDS row
  // A call whose tokens fit one block (T <= 64) finishes the permutation in
  // the route kernel itself, from the block's LDS bitmask (no counting rows,
  // no scatter launch): set `fused` and these outputs.
  int fused;
  int tile, tile_shift;
  int32_t* e2p;           // [T k]
  int32_t* p2t;           // [max padded]
  int32_t* counts;        // [loc_n]
  int32_t* padded_offsets;   // [loc_n + 1]
  int32_t* total_out;
  int32_t* nctas_out;
  int32_t* batch_idx;     // [max tiles]
  int32_t* mn_limit;      // [max tiles]
};

struct ScatterParams {
  const int32_t* ids;
  int T, k, El, off, tile;
  int tile_shift;         // tile = 1 << tile_shift
  uint32_t k_magic;       // ceil(2^20 / k): (q * k_magic) >> 20 = q / k for q < 4096
  int32_t* super_rows;    // the two sets of counting rows, [num_super, El] used of each
  uint32_t* count_hdr;    // their header (see kCountSetInts)
  const int32_t* hist;    // [nb, El] per-block counts
  int group_blocks, num_super;
  int sub_blocks;         // route blocks per scatter block (divides group_blocks)
  int route_blocks;       // route blocks of the call
  int32_t* counts;        // out [El]
  int max_count;          // T k: no expert count exceeds it
  int max_padded;         // entries of p2t (moe_max_padded_tokens)
  int32_t* e2p;
  int32_t* p2t;
  int32_t* padded_offsets;
  int32_t* total_out;
  int32_t* nctas_out;
  int32_t* batch_idx;
  int32_t* mn_limit;
};

// Byte offsets of the route kernel's LDS regions (shared by host and device).
// Per cluster: the row (rwpl 32-bit words per lane: raw logits or float32
// score basis, padded so that the clusters of one wavefront fall on different
// LDS banks), the packed candidate keys, the experts of the selection by rank,
// and the packed group keys.
struct RouteLds {
  int bias, hmask, row, cand, sel_idx, gscore, total;
  int row_stride, cand_stride, sel_stride, gs_stride;   // in elements
};
// Padding words after each lane's slice of a cluster's LDS row (slices of
// `words` 32-bit words, lpt lanes).  When a cluster's row spans more than the
// 64 banks, lanes whose slices start a multiple of 64 words apart would hit
// the same banks with their 16-byte accesses; 4 words per lane spread them
// (and the rows of consecutive clusters follow directly).  Smaller rows keep
// the unpadded layout, whose clusters are offset by 4 words instead.
__host__ __device__ constexpr int route_lane_pad(int lpt, int words) {
  return lpt * words > 64 ? 4 : 0;
}

__host__ __device__ inline RouteLds route_lds_layout(int lpt, int rwpl, int epl, int hmask_len,
                                                    int cap, int k, int n_group) {
  RouteLds L{};
  const int block = lpt * 64 < 512 ? lpt * 64 : 512;
  const int ncl = block / lpt;
  const int lp = route_lane_pad(lpt, rwpl);
  L.row_stride = lp ? (lpt * (rwpl + lp) + 3) & ~3      // words, a multiple of 4
                    : ((lpt * rwpl + 3) & ~3) + 4;
  L.cand_stride = cap + 2;                     // even: 16-byte aligned rows
  L.sel_stride = k + 1;
  L.gs_stride = n_group > 0 ? ((lpt + 1) & ~1) : 0;   // u64 group keys, read two at a time
  int off = 0;
  auto take = [&](int bytes) { const int o = off; off += (bytes + 15) & ~15; return o; };
  L.bias = take(lpt * (epl + route_lane_pad(lpt, epl)) * 4);
  L.hmask = take(hmask_len * 8);
  L.row = take(ncl * L.row_stride * 4);
  L.cand = take(ncl * L.cand_stride * 8);
  L.sel_idx = take(ncl * L.sel_stride * 4);
  L.gscore = take(ncl * L.gs_stride * 8);
  L.total = off;
  return L;
}

size_t route_lds_bytes(int lpt, int rwpl, int epl, int hmask_len, int cap, int k, int n_group);
size_t scatter_lds_bytes(int El, int sub_blocks);
hipError_t launch_route(const RouteParams& p, int lpt, int epl, bool bf16, int nb, hipStream_t s);
hipError_t launch_counts(int32_t* super_rows, uint32_t* count_hdr, int num_super, int El,
                         int max_count, int32_t* counts, hipStream_t s);
hipError_t launch_scatter(const ScatterParams& p, int nb, hipStream_t s);
hipError_t launch_empty_outputs(int32_t* counts, int El, int32_t* padded_offsets, int32_t* total,
                                int32_t* nctas, hipStream_t s);
// Zero `bytes` (a multiple of 16) at the 16-byte aligned device address p.
hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t s);

// Backward of the routing outputs (see route_backward.hip).
enum { kBwdSigmoid = 0, kBwdSoftmaxPre = 1, kBwdSoftmaxPost = 2 };
struct RouteBwdParams {
  const void* logits;        // [T, E] f32 or bf16
  const int32_t* ids;        // [T, k] (with grad_weights)
  const float* grad_weights; // nullable [T, k]
  const float* grad_scores;  // nullable [T, E]
  float* grad_logits;        // [T, E]
  int T, E, k;
  int mode;                  // kBwd*
  int renorm;
  float scale;
};
hipError_t launch_route_backward(const RouteBwdParams& p, bool bf16, hipStream_t s);

// Token dispatch / combine (see dispatch.hip).
hipError_t launch_dispatch(const void* hidden, int64_t row_bytes, const int32_t* p2t,
                           const int32_t* total, int64_t max_rows, void* out, hipStream_t s);
hipError_t launch_combine(const void* expert_out, bool bf16, int T, int H, int k, const int32_t* e2p,
                          const void* weights, bool w_bf16, void* out, hipStream_t s);

// Dense [T, E] probs / routing map from the top-k outputs (see dense.hip).
hipError_t launch_dense(int T, int E, int k, const int32_t* ids, const void* weights, bool w_bf16,
                        float* probs, uint8_t* rmap, hipStream_t s);

struct FrontEndParams {
  const void* hidden;
  const void* gamma;
  const void* W;
  const void* rbias;      // nullable [E]
  int f16;                // 1: float16 inputs, 0: bfloat16
  int T, H, E, k;
  float eps;
  int act_sigmoid;
  void* normed;
  int32_t* ids;
  void* aff;
  void* workspace;        // sync region (failure line, r_t slots), partials [H / kchunk, T, E]
  int spin_limit;         // polls before a wait for r_t gives up
};
// Polls before a front-end wait gives up: far beyond any real wait (seconds).
constexpr int kFrontEndSpinLimit = 1 << 22;
// The front-end workspace starts with a synchronisation region of this many
// bytes: zero before the first call, zero again after every call.
constexpr int kFrontEndSyncBytes = 1024;
int front_end_kchunk(int H);
size_t front_end_workspace_bytes(int T, int H, int E);
hipError_t launch_front_end(const FrontEndParams& q, hipStream_t s);

// The aux-loss forward's workspace is one synchronisation region of this many
// bytes (a 64-bit partial slot per block, at most kAuxMaxBlocks blocks): zero
// before the first call, zero again after every call.  A forward whose summing
// block gave up waiting writes the loss as the float32 NaN kAuxTimeoutNaN.
constexpr int kAuxMaxBlocks = 2048;
constexpr int kAuxSyncBytes = kAuxMaxBlocks * 8;
constexpr uint32_t kAuxTimeoutNaN = 0x7fc0a0a0u;
constexpr int kAuxSpinLimit = 1 << 22;   // polls before the summing block gives up
int aux_fwd_blocks(int64_t rows, int E);
hipError_t launch_aux_fwd(const float* probs, const int32_t* counts, int64_t rows, int E,
                          double scale, void* sync, int nb, float* loss, int spin_limit,
                          hipStream_t s);
hipError_t launch_aux_bwd(const int32_t* counts, int64_t rows, int E, double scale,
                          const float* grad_loss, float* grad, hipStream_t s);

}  // namespace moe
