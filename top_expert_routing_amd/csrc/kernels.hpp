// Internal interface between the host library and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kTokensPerBlock = 64;   // tokens per route/scatter block (one u64 bitmask)

template <int LPT>
constexpr int kRouteBlock = (LPT * 64 < 512) ? LPT * 64 : 512;

enum { kKindSigmoid = 0, kKindSoftmaxPre = 1, kKindSoftmaxPost = 2 };

struct RouteParams {
  const void* logits;
  const void* bias;       // nullable [E]
  int32_t* ids;           // [T, k]
  void* weights;          // [T, k] f32 or bf16
  float* scores;          // nullable [T, E]
  int32_t* hist;          // nullable [nb, loc_n]
  int T, E, k;
  int kind;
  int bias_bf16;
  int weights_bf16;
  int grouped, n_group, topk_group, topn, lg;
  int renorm;
  float scale;
  int vec;                // 16-byte vector loads allowed
  int loc_off, loc_n;
  int hmask_len;          // LDS u64 words for the block bitmask (even)
  int cap;                // candidate list capacity per token (>= k)
};

struct ScatterParams {
  const int32_t* ids;
  int T, k, El, off, tile;
  const int32_t* counts;  // [El]
  const int32_t* excl;    // [nb, El] exclusive per-block base ranks
  int32_t* e2p;
  int32_t* p2t;
  int32_t* padded_offsets;
  int32_t* total_out;
  int32_t* nctas_out;
  int32_t* batch_idx;
  int32_t* mn_limit;
};

size_t route_lds_bytes(int lpt, int epl, int hmask_len, int cap, int k);
size_t scatter_lds_bytes(int El);
hipError_t launch_route(const RouteParams& p, int lpt, int epl, bool bf16, int nb, hipStream_t s);
hipError_t launch_scan(int32_t* hist, int nb, int El, int32_t* counts, hipStream_t s);
hipError_t launch_scatter(const ScatterParams& p, int nb, hipStream_t s);
hipError_t launch_empty_outputs(int32_t* counts, int El, int32_t* padded_offsets, int32_t* total,
                                int32_t* nctas, hipStream_t s);

int aux_fwd_blocks(int64_t rows, int E);
hipError_t launch_aux_fwd(const float* probs, const int32_t* counts, int64_t rows, int E,
                          double scale, double* partial, int nb, float* loss, hipStream_t s);
hipError_t launch_aux_bwd(const int32_t* counts, int64_t rows, int E, double scale,
                          const float* grad_loss, float* grad, hipStream_t s);

}  // namespace moe
