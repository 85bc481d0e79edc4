// Device helpers shared by the gfx950 routing kernels: bf16 decode/encode,
// order-preserving key packing, sigmoid, and cluster (sub-wavefront) reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float32 -> bfloat16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Monotone map float -> uint32: a < b  <=>  ord(a) < ord(b) (for non-NaN,
// with -0 and +0 distinct; callers canonicalise -0 by adding +0.0f).
__device__ __forceinline__ uint32_t ord_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Selection order as one unsigned 64-bit integer: larger key first, then the
// lower expert index (its complement is larger).  Distinct experts never
// compare equal.
__device__ __forceinline__ uint64_t pack_key(float key, int idx) {
  return ((uint64_t)ord_key(key) << 32) | (uint64_t)(~(uint32_t)idx);
}
__device__ __forceinline__ int unpack_idx(uint64_t p) { return (int)(~(uint32_t)p); }

// Logistic sigmoid in float32: 1 / (1 + 2^(-x log2 e)) with the hardware
// exp2 and reciprocal (each about 1 ulp).
__device__ __forceinline__ float sigmoid_f32(float x) {
  float e = __builtin_amdgcn_exp2f(-x * 1.4426950408889634f);
  return __builtin_amdgcn_rcpf(1.0f + e);
}

// e^x for softmax terms, x <= 0.
__device__ __forceinline__ float exp_f32(float x) {
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// Intra-wavefront LDS hand-off: orders this lane's LDS writes before other
// lanes' later reads of the same wavefront.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Reductions over a cluster of W consecutive lanes (W a power of two <= 64).
template <int W>
__device__ __forceinline__ float cl_max(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, W));
  return v;
}
template <int W>
__device__ __forceinline__ float cl_min(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, W));
  return v;
}
template <int W>
__device__ __forceinline__ float cl_sum(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, W);
  return v;
}
template <int W>
__device__ __forceinline__ int cl_sum_i(int v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, W);
  return v;
}
template <int W>
__device__ __forceinline__ uint64_t cl_max_u64(uint64_t v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) {
    uint64_t w = __shfl_xor(v, o, W);
    v = w > v ? w : v;
  }
  return v;
}
// Exclusive prefix sum over the cluster (lane c gets sum of lanes < c).
template <int W>
__device__ __forceinline__ int cl_excl_scan(int v, int lane_c) {
  int incl = v;
#pragma unroll
  for (int o = 1; o < W; o <<= 1) {
    int u = __shfl_up(incl, o, W);
    if (lane_c >= o) incl += u;
  }
  return incl - v;
}

}  // namespace moe
