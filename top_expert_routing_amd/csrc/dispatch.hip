// gfx950 kernels for token dispatch into expert (permuted) order and the
// weighted combine back into token order, either side of the grouped expert
// GEMM (Implementation:InternLM Lmdeploy Gemm MoeUtils, Description: dispatch
// and combine; the index maps are the routing's own, FlashInfer
// trtllm_gen_routing, Returns).
//
//   dispatch_kernel  one wavefront per permuted row p < total: the row of token
//                    permuted_idx_to_token_idx[p], copied bit for bit (zeros
//                    for a padding slot), 16-byte accesses, eight in flight
//                    per lane, streaming stores (the routed rows are not read
//                    back here; the token rows, read k times, stay cached).
//   combine_kernel   one wavefront per token: out[t] = sum_j w[t, j] *
//                    expert_out[expanded_idx_to_permuted_idx[t k + j]], one
//                    routed row at a time with up to 16 KiB of it requested
//                    together, summed in choice order in float32
//                    (deterministic), rounded once (bf16: RNE), streaming
//                    stores.
// Both are HBM-bound row movers.
#include "device_common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kMoveThreads = 256;   // 4 wavefronts, one row or token each
constexpr int kCopyInFlight = 8;    // 16-byte loads per lane per round

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

}  // namespace

// Rows of `row_bytes` bytes; VEC: rows and pointers 16-byte aligned.
template <bool VEC>
__global__ void __launch_bounds__(kMoveThreads)
    dispatch_kernel(const unsigned char* __restrict__ hidden, int64_t row_bytes,
                    const int32_t* __restrict__ p2t, const int32_t* __restrict__ total_ptr,
                    int64_t max_rows, unsigned char* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t p = (int64_t)blockIdx.x * (kMoveThreads / 64) + (threadIdx.x >> 6);
  const int64_t total = *total_ptr;
  if (p >= total || p >= max_rows) return;              // whole wavefront leaves together
  const int t = p2t[p];
  const unsigned char* src = hidden + (int64_t)(t < 0 ? 0 : t) * row_bytes;
  unsigned char* dst = out + p * row_bytes;
  if constexpr (VEC) {
    const int64_t nv = row_bytes / 16;
    for (int64_t v0 = 0; v0 < nv; v0 += 64 * kCopyInFlight) {
      u32x4 r[kCopyInFlight];
#pragma unroll
      for (int u = 0; u < kCopyInFlight; ++u) {
        const int64_t v = v0 + u * 64 + lane;
        r[u] = (t >= 0 && v < nv) ? reinterpret_cast<const u32x4*>(src)[v] : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < kCopyInFlight; ++u) {
        const int64_t v = v0 + u * 64 + lane;
        if (v < nv) __builtin_nontemporal_store(r[u], reinterpret_cast<u32x4*>(dst) + v);
      }
    }
  } else {
    for (int64_t b = lane; b < row_bytes; b += 64) dst[b] = t >= 0 ? src[b] : 0;
  }
}

// One wavefront per token; BF16: bfloat16 rows (8 elements per lane per slab),
// else float32 rows (4 per lane).  VEC: H a multiple of the lane width and
// 16-byte aligned rows.
#ifndef COMBINE_SLABS
#define COMBINE_SLABS 16
#endif

template <bool BF16, bool VEC>
__global__ void __launch_bounds__(kMoveThreads)
    combine_kernel(const void* __restrict__ expert_out, int T, int H, int k,
                   const int32_t* __restrict__ e2p, const void* __restrict__ weights, int w_bf16,
                   void* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kMoveThreads / 64) + (threadIdx.x >> 6);
  if (t >= T) return;                                   // whole wavefront leaves together
  // lane j < k holds choice j: its slot and weight, broadcast below
  int my_slot = -1;
  float my_w = 0.0f;
  if (lane < k) {
    my_slot = e2p[(size_t)t * k + lane];
    my_w = w_bf16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(weights)[(size_t)t * k + lane])
                  : static_cast<const float*>(weights)[(size_t)t * k + lane];
  }
  constexpr int EPL = BF16 ? 8 : 4;                     // elements per lane per slab
  if constexpr (VEC) {
    // One choice's row at a time, kSlabs 1 KiB column slabs of it requested
    // together: long contiguous reads of each routed row gather best (a
    // column strip of several rows at once measured slower)
    constexpr int kSlabs = COMBINE_SLABS;
    for (int c0 = 0; c0 < H; c0 += kSlabs * 64 * EPL) {
      float acc[kSlabs][EPL];
#pragma unroll
      for (int sl = 0; sl < kSlabs; ++sl)
#pragma unroll
        for (int i = 0; i < EPL; ++i) acc[sl][i] = 0.0f;
      // summed in choice order
      for (int j = 0; j < k; ++j) {
        const int slot = __builtin_amdgcn_readlane(my_slot, j);
        if (slot < 0) continue;                         // uniform: a dropped choice
        const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), j));
        u32x4 r[kSlabs];
#pragma unroll
        for (int sl = 0; sl < kSlabs; ++sl) {
          const int c = c0 + sl * 64 * EPL + lane * EPL;
          const size_t off = (size_t)slot * H + c;
          r[sl] = c < H ? __builtin_nontemporal_load(
                              BF16 ? reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(expert_out) + off)
                                   : reinterpret_cast<const u32x4*>(static_cast<const float*>(expert_out) + off))
                        : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int sl = 0; sl < kSlabs; ++sl) {
          if constexpr (BF16) {
            const uint32_t wv[4] = {r[sl].x, r[sl].y, r[sl].z, r[sl].w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
              acc[sl][2 * h] += wj * bf16_lo(wv[h]);
              acc[sl][2 * h + 1] += wj * bf16_hi(wv[h]);
            }
          } else {
            acc[sl][0] += wj * __uint_as_float(r[sl].x);
            acc[sl][1] += wj * __uint_as_float(r[sl].y);
            acc[sl][2] += wj * __uint_as_float(r[sl].z);
            acc[sl][3] += wj * __uint_as_float(r[sl].w);
          }
        }
      }
#pragma unroll
      for (int sl = 0; sl < kSlabs; ++sl) {
        const int c = c0 + sl * 64 * EPL + lane * EPL;
        if (c >= H) continue;
        if constexpr (BF16) {
          const u32x4 o{pack_bf16(acc[sl][0], acc[sl][1]), pack_bf16(acc[sl][2], acc[sl][3]),
                        pack_bf16(acc[sl][4], acc[sl][5]), pack_bf16(acc[sl][6], acc[sl][7])};
          __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + (size_t)t * H + c));
        } else {
          __builtin_nontemporal_store(f32x4{acc[sl][0], acc[sl][1], acc[sl][2], acc[sl][3]},
                                      reinterpret_cast<f32x4*>(static_cast<float*>(out) + (size_t)t * H + c));
        }
      }
    }
  } else {
    // any H: one element per lane per step, choices summed in order
    for (int c = lane; c < H; c += 64) {
      float acc = 0.0f;
      for (int j = 0; j < k; ++j) {
        const int slot = __builtin_amdgcn_readlane(my_slot, j);
        const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), j));
        if (slot < 0) continue;
        const size_t off = (size_t)slot * H + c;
        const float v = BF16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(expert_out)[off])
                             : static_cast<const float*>(expert_out)[off];
        acc += w * v;
      }
      if constexpr (BF16) static_cast<uint16_t*>(out)[(size_t)t * H + c] = (uint16_t)(pack_bf16(acc, 0.0f) & 0xffffu);
      else static_cast<float*>(out)[(size_t)t * H + c] = acc;
    }
  }
}

hipError_t launch_dispatch(const void* hidden, int64_t row_bytes, const int32_t* p2t,
                           const int32_t* total, int64_t max_rows, void* out, hipStream_t s) {
  const bool vec = row_bytes % 16 == 0 && (uintptr_t)hidden % 16 == 0 && (uintptr_t)out % 16 == 0;
  const dim3 grid((unsigned)((max_rows + kMoveThreads / 64 - 1) / (kMoveThreads / 64)));
  if (vec)
    MOE_LAUNCH(dispatch_kernel<true>, grid, dim3(kMoveThreads), 0, s,
               static_cast<const unsigned char*>(hidden), row_bytes, p2t, total, max_rows,
               static_cast<unsigned char*>(out));
  else
    MOE_LAUNCH(dispatch_kernel<false>, grid, dim3(kMoveThreads), 0, s,
               static_cast<const unsigned char*>(hidden), row_bytes, p2t, total, max_rows,
               static_cast<unsigned char*>(out));
  return hipGetLastError();
}

hipError_t launch_combine(const void* expert_out, bool bf16, int T, int H, int k, const int32_t* e2p,
                          const void* weights, bool w_bf16, void* out, hipStream_t s) {
  const int epl = bf16 ? 8 : 4;
  const bool vec = H % epl == 0 && (uintptr_t)expert_out % 16 == 0 && (uintptr_t)out % 16 == 0;
  const dim3 grid((T + kMoveThreads / 64 - 1) / (kMoveThreads / 64));
#define MOE_COMBINE(B, V)                                                                      \
  MOE_LAUNCH((combine_kernel<B, V>), grid, dim3(kMoveThreads), 0, s, expert_out, T, H, k, e2p, \
             weights, (int)w_bf16, out)
  if (bf16) {
    if (vec) MOE_COMBINE(true, true);
    else MOE_COMBINE(true, false);
  } else {
    if (vec) MOE_COMBINE(false, true);
    else MOE_COMBINE(false, false);
  }
#undef MOE_COMBINE
  return hipGetLastError();
}

}  // namespace moe
