// gfx950 kernels for the fused decode front end (NKI "RMSNorm Router Top-K
// A2AV Kernel API Reference": Background, Parameters, Returns, Notes):
//
//   norm_kernel    one block per token: r_t = (mean_h x^2 + eps)^-1/2 in
//                  float32, normed = round(x * r_t * gamma) stored in the
//                  input dtype (RNE).
//   gemm_kernel    split-K router projection on MFMA: block (n-tile of 16
//                  experts, k-chunk) computes all T <= 128 tokens x 16 experts
//                  over its k-chunk with v_mfma_f32_16x16x32_{bf16,f16} and
//                  writes float32 partials [chunks, T, E].  A (normed) comes
//                  from global memory (shared by every n-tile through L2); the
//                  W tile is staged transposed in LDS.  The MFMA consumes
//                  exactly the stored normed values.
//   select_kernel  one wavefront per token: z = sum of the partials in chunk
//                  order (+ router bias) -- deterministic; top-k on the raw
//                  logits (lower index on ties); activation on the chosen
//                  experts only (sigmoid, or softmax over the k chosen);
//                  affinities [T, E] bf16 with zeros elsewhere.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

template <bool F16>
__device__ __forceinline__ float h2f(uint16_t b) {
  if constexpr (F16) return (float)__ushort_as_half(b);
  else return __uint_as_float((uint32_t)b << 16);
}

template <bool F16>
__device__ __forceinline__ uint16_t f2h(float v) {
  if constexpr (F16) return __half_as_ushort(__float2half_rn(v));
  else return (uint16_t)f32_to_bf16_rne(v);
}

constexpr int kNormThreads = 256;

}  // namespace

template <bool F16>
__global__ void __launch_bounds__(kNormThreads)
    norm_kernel(const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ gamma, int H,
                float eps, uint16_t* __restrict__ normed) {
  __shared__ float red[kNormThreads / 64];
  const int t = blockIdx.x;
  const uint16_t* x = hidden + (size_t)t * H;
  float ss = 0.0f;
  // H % 128 == 0: 16-byte vectors of 8 elements
  for (int v = threadIdx.x; v < H / 8; v += kNormThreads) {
    const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x) + v);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = h2f<F16>((uint16_t)(w[i] & 0xffffu));
      const float b = h2f<F16>((uint16_t)(w[i] >> 16));
      ss += a * a + b * b;
    }
  }
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int i = 0; i < kNormThreads / 64; ++i) tot += red[i];
  const float r = 1.0f / sqrtf(tot / (float)H + eps);
  uint16_t* y = normed + (size_t)t * H;
  for (int v = threadIdx.x; v < H / 8; v += kNormThreads) {
    const u32x4 q = reinterpret_cast<const u32x4*>(x)[v];
    const u32x4 g = reinterpret_cast<const u32x4*>(gamma)[v];
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    const uint32_t gw[4] = {g.x, g.y, g.z, g.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = h2f<F16>((uint16_t)(w[i] & 0xffffu)) * r * h2f<F16>((uint16_t)(gw[i] & 0xffffu));
      const float b = h2f<F16>((uint16_t)(w[i] >> 16)) * r * h2f<F16>((uint16_t)(gw[i] >> 16));
      o[i] = (uint32_t)f2h<F16>(a) | ((uint32_t)f2h<F16>(b) << 16);
    }
    reinterpret_cast<u32x4*>(y)[v] = u32x4{o[0], o[1], o[2], o[3]};
  }
}

constexpr int kGemmThreads = 256;   // 4 waves x 32 token rows
constexpr int kGemmN = 16;          // experts per block

template <bool F16>
__global__ void __launch_bounds__(kGemmThreads)
    gemm_kernel(const uint16_t* __restrict__ normed, const uint16_t* __restrict__ W, int T, int H,
                int E, int kc, float* __restrict__ partial) {
  extern __shared__ __align__(16) uint16_t wt[];         // [16][kc] transposed tile
  const int nt = blockIdx.x;                              // n-tile
  const int ch = blockIdx.y;                              // k-chunk
  const int n0 = nt * kGemmN, k0 = ch * kc;
  const int tid = threadIdx.x;
  // stage W[k0 : k0+kc, n0 : n0+16] transposed: 16-byte loads of 8 experts
  for (int v = tid; v < kc * 2; v += kGemmThreads) {
    const int kk = v >> 1, half = v & 1;
    const u32x4 q = *reinterpret_cast<const u32x4*>(W + (size_t)(k0 + kk) * E + n0 + half * 8);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      wt[(half * 8 + 2 * i) * kc + kk] = (uint16_t)(w[i] & 0xffffu);
      wt[(half * 8 + 2 * i + 1) * kc + kk] = (uint16_t)(w[i] >> 16);
    }
  }
  __syncthreads();
  const int lane = tid & 63, wv = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;          // k-group of 8
  f32x4v acc[2] = {f32x4v{0, 0, 0, 0}, f32x4v{0, 0, 0, 0}};
  const int rows[2] = {wv * 32 + col, wv * 32 + 16 + col};
  for (int kk = 0; kk < kc; kk += 32) {
    const u32x4 b = *reinterpret_cast<const u32x4*>(wt + col * kc + kk + grp * 8);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4 a = u32x4{0, 0, 0, 0};
      if (rows[s] < T)
        a = *reinterpret_cast<const u32x4*>(normed + (size_t)rows[s] * H + k0 + kk + grp * 8);
      if constexpr (F16)
        acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                       __builtin_bit_cast(f16x8, b), acc[s], 0, 0, 0);
      else
        acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                        __builtin_bit_cast(bf16x8, b), acc[s], 0, 0, 0);
    }
  }
  // D layout: lane holds column (lane & 15), rows 4 * (lane >> 4) + i
#pragma unroll
  for (int s = 0; s < 2; ++s) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wv * 32 + 16 * s + 4 * grp + i;
      if (row < T) partial[((size_t)ch * T + row) * E + n0 + col] = acc[s][i];
    }
  }
}

constexpr int kSelectThreads = 256;  // one wavefront per token
constexpr int kSelectMaxPerLane = 8; // E <= 512

template <bool F16>
__global__ void __launch_bounds__(kSelectThreads)
    select_kernel(const float* __restrict__ partial, int nchunks, const uint16_t* __restrict__ rbias,
                  int T, int E, int k, int act_sigmoid, int32_t* __restrict__ ids,
                  uint16_t* __restrict__ aff) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kSelectThreads / 64) + (threadIdx.x >> 6);
  if (t >= T) return;                                  // whole wavefront leaves together
  float z[kSelectMaxPerLane];
#pragma unroll
  for (int j = 0; j < kSelectMaxPerLane; ++j) {
    const int e = lane + 64 * j;
    float s = -__builtin_huge_valf();
    if (e < E) {
      s = 0.0f;
      for (int c = 0; c < nchunks; ++c) s += partial[((size_t)c * T + t) * E + e];
      if (rbias != nullptr) s += h2f<F16>(rbias[e]);
    }
    z[j] = s;
  }
  // top-k on the raw logits: k rounds of a wavefront-wide maximum of
  // (key, lower index first) packed into 64 bits
  uint32_t taken = 0;
  float zmax = 0.0f;
  for (int r = 0; r < k; ++r) {
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < kSelectMaxPerLane; ++j) {
      const int e = lane + 64 * j;
      const uint64_t c = pack_key(z[j] + 0.0f, e);
      best = (e < E && !((taken >> j) & 1u) && c > best) ? c : best;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const uint64_t w = __shfl_xor(best, o, 64);
      best = w > best ? w : best;
    }
    const int e = unpack_idx(best);
    if (lane == 0) ids[(size_t)t * k + r] = e;
    if ((e & 63) == lane) taken |= 1u << (e >> 6);
    if (r == 0) zmax = unord_key((uint32_t)(best >> 32));   // the largest logit
  }
  float my_aff_num[kSelectMaxPerLane];
  // activation on the chosen experts only
  float part = 0.0f;
#pragma unroll
  for (int j = 0; j < kSelectMaxPerLane; ++j) {
    my_aff_num[j] = 0.0f;
    if ((taken >> j) & 1u) {
      my_aff_num[j] = act_sigmoid ? sigmoid_f32(z[j]) : exp_f32(z[j] - zmax);
      part += my_aff_num[j];
    }
  }
  float denom = 1.0f;
  if (!act_sigmoid) {
    for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
    denom = part;
  }
  const float inv = 1.0f / denom;
#pragma unroll
  for (int j = 0; j < kSelectMaxPerLane; ++j) {
    const int e = lane + 64 * j;
    if (e < E) {
      const float v = ((taken >> j) & 1u) ? my_aff_num[j] * inv : 0.0f;
      aff[(size_t)t * E + e] = (uint16_t)f32_to_bf16_rne(v);
    }
  }
}

int front_end_kchunk(int H) {
  // 512, 256 or 128 elements per k-chunk, keeping at least ~14 chunks of work
  if (H % 512 == 0 && H / 512 >= 8) return 512;
  if (H % 256 == 0 && H / 256 >= 8) return 256;
  return 128;
}

hipError_t launch_front_end(const FrontEndParams& q, hipStream_t s) {
  const int kc = front_end_kchunk(q.H);
  const int nchunks = q.H / kc;
  if (q.f16) {
    hipLaunchKernelGGL(norm_kernel<true>, dim3(q.T), dim3(kNormThreads), 0, s,
                       (const uint16_t*)q.hidden, (const uint16_t*)q.gamma, q.H, q.eps,
                       (uint16_t*)q.normed);
  } else {
    hipLaunchKernelGGL(norm_kernel<false>, dim3(q.T), dim3(kNormThreads), 0, s,
                       (const uint16_t*)q.hidden, (const uint16_t*)q.gamma, q.H, q.eps,
                       (uint16_t*)q.normed);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = (size_t)kGemmN * kc * sizeof(uint16_t);
  dim3 grid(q.E / kGemmN, nchunks);
  if (q.f16)
    hipLaunchKernelGGL(gemm_kernel<true>, grid, dim3(kGemmThreads), lds, s,
                       (const uint16_t*)q.normed, (const uint16_t*)q.W, q.T, q.H, q.E, kc,
                       q.partial);
  else
    hipLaunchKernelGGL(gemm_kernel<false>, grid, dim3(kGemmThreads), lds, s,
                       (const uint16_t*)q.normed, (const uint16_t*)q.W, q.T, q.H, q.E, kc,
                       q.partial);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nb = (q.T + kSelectThreads / 64 - 1) / (kSelectThreads / 64);
  if (q.f16)
    hipLaunchKernelGGL(select_kernel<true>, dim3(nb), dim3(kSelectThreads), 0, s, q.partial,
                       nchunks, (const uint16_t*)q.rbias, q.T, q.E, q.k, q.act_sigmoid, q.ids,
                       (uint16_t*)q.aff);
  else
    hipLaunchKernelGGL(select_kernel<false>, dim3(nb), dim3(kSelectThreads), 0, s, q.partial,
                       nchunks, (const uint16_t*)q.rbias, q.T, q.E, q.k, q.act_sigmoid, q.ids,
                       (uint16_t*)q.aff);
  return hipGetLastError();
}

}  // namespace moe
