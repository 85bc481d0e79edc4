// gfx950 kernel for the dense [T, E] form of the top-k outputs
// (TransformerEngine Fused Router, I/O Contract: probs and routing_map of
// fused_topk_with_score_function): probs[t, e] = the weight of expert e if
// token t chose it, else 0; routing_map[t, e] = whether it did.
//
// A token per cluster of L lanes (L = 32 with J = 8 experts per lane for
// 128 < E <= 256, 32 x 4 for 64 < E <= 128, else the whole wavefront with
// J = 1, 2, 4, 8, 16 or 32, the least that holds E, for E <= 2048); lane l
// of a cluster writes experts [J l, J l + J) with
// one vector store per output; lanes j < k of a cluster read the token's j-th
// id and weight, and k readlanes (or cluster shuffles) bring each to the lane
// owning the expert; streaming stores.  Write-bound: T E (4 + 1) bytes.
#include "device_common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {
constexpr int kDenseThreads = 256;
}

template <int J, int L, bool VEC>
__global__ void __launch_bounds__(kDenseThreads)
    dense_kernel(int T, int E, int k, const int32_t* __restrict__ ids, const void* __restrict__ weights,
                 int w_bf16, float* __restrict__ probs, uint8_t* __restrict__ rmap) {
  const int lane_w = threadIdx.x & 63;
  const int t0 = (blockIdx.x * (kDenseThreads / 64) + (threadIdx.x >> 6)) * (64 / L);
  if (t0 >= T) return;                                  // whole wavefront leaves together
  const int lane = lane_w & (L - 1), cbase = lane_w & ~(L - 1);
  const int t = t0 + lane_w / L;
  const bool tv = t < T;
  int my_id = -1;
  float my_w = 0.0f;
  if (tv && lane < k) {
    my_id = ids[(size_t)t * k + lane];
    my_w = w_bf16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(weights)[(size_t)t * k + lane])
                  : static_cast<const float*>(weights)[(size_t)t * k + lane];
  }
  const int e0 = J * lane;
  float v[J];
  uint32_t sel = 0;
#pragma unroll
  for (int j = 0; j < J; ++j) v[j] = 0.0f;
  for (int i = 0; i < k; ++i) {
    int e;
    float w;
    if constexpr (L == 64) {
      e = __builtin_amdgcn_readlane(my_id, i);
      w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), i));
    } else {
      e = __shfl(my_id, cbase + i, 64);
      w = __shfl(my_w, cbase + i, 64);
    }
    if (e >= 0 && e < E && e / J == lane) {
#pragma unroll
      for (int j = 0; j < J; ++j)
        if (e % J == j) { v[j] = w; sel |= 1u << j; }
    }
  }
  if (!tv || e0 >= E) return;
  const size_t base = (size_t)t * E + e0;
  if constexpr (VEC && J >= 4) {
    if (probs != nullptr) {
#pragma unroll
      for (int h = 0; h < J / 4; ++h)
        __builtin_nontemporal_store(f32x4{v[4 * h], v[4 * h + 1], v[4 * h + 2], v[4 * h + 3]},
                                    reinterpret_cast<f32x4*>(probs + base) + h);
    }
    if (rmap != nullptr) {
      uint32_t b[J / 4];
#pragma unroll
      for (int h = 0; h < J / 4; ++h) b[h] = ((sel >> (4 * h)) & 1u) | ((sel >> (4 * h + 1)) & 1u) << 8 |
                                              ((sel >> (4 * h + 2)) & 1u) << 16 | ((sel >> (4 * h + 3)) & 1u) << 24;
      if constexpr (J == 4) {
        __builtin_nontemporal_store(b[0], reinterpret_cast<uint32_t*>(rmap + base));
      } else {
#pragma unroll
        for (int h = 0; h < J / 8; ++h)
          __builtin_nontemporal_store((uint64_t)b[2 * h] | ((uint64_t)b[2 * h + 1] << 32),
                                      reinterpret_cast<uint64_t*>(rmap + base) + h);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (e0 + j >= E) break;
      if (probs != nullptr) probs[base + j] = v[j];
      if (rmap != nullptr) rmap[base + j] = (uint8_t)((sel >> j) & 1u);
    }
  }
}

hipError_t launch_dense(int T, int E, int k, const int32_t* ids, const void* weights, bool w_bf16,
                        float* probs, uint8_t* rmap, hipStream_t s) {
  const int L = (E > 64 && E <= 256 && k <= 32) ? 32 : 64;
  const int J = L == 32 ? (E <= 128 ? 4 : 8)
              : E <= 64 ? 1 : E <= 128 ? 2 : E <= 256 ? 4 : E <= 512 ? 8 : E <= 1024 ? 16 : 32;
  const bool vec = J >= 4 && E % J == 0 && (uintptr_t)probs % 16 == 0 && (uintptr_t)rmap % 8 == 0;
  const int per_block = kDenseThreads / 64 * (64 / L);
  const dim3 grid((T + per_block - 1) / per_block);
#define MOE_DENSE(JJ, LL, V)                                                                     \
  MOE_LAUNCH((dense_kernel<JJ, LL, V>), grid, dim3(kDenseThreads), 0, s, T, E, k, ids, weights, \
             (int)w_bf16, probs, rmap)
  if (L == 32) {
    if (J == 4) { if (vec) MOE_DENSE(4, 32, true); else MOE_DENSE(4, 32, false); }
    else { if (vec) MOE_DENSE(8, 32, true); else MOE_DENSE(8, 32, false); }
    return hipGetLastError();
  }
  switch (J) {
    case 1: MOE_DENSE(1, 64, false); break;
    case 2: MOE_DENSE(2, 64, false); break;
    case 4: if (vec) MOE_DENSE(4, 64, true); else MOE_DENSE(4, 64, false); break;
    case 8: if (vec) MOE_DENSE(8, 64, true); else MOE_DENSE(8, 64, false); break;
    case 16: if (vec) MOE_DENSE(16, 64, true); else MOE_DENSE(16, 64, false); break;
    default: if (vec) MOE_DENSE(32, 64, true); else MOE_DENSE(32, 64, false); break;
  }
#undef MOE_DENSE
  return hipGetLastError();
}

}  // namespace moe
