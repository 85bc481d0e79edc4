// gfx950 kernels for the fused decode front end (NKI "RMSNorm Router Top-K
// A2AV Kernel API Reference": Background, Parameters, Returns, Notes):
//
//   norm_kernel    one block per token: r_t = (mean_h x^2 + eps)^-1/2 in
//                  float32, normed = round(x * r_t * gamma) stored in the
//                  input dtype (RNE).
//   gemm_kernel    split-K router projection on MFMA: block (k-chunk, 64
//                  experts) computes all T <= 128 tokens x 64 experts over
//                  its k-chunk with v_mfma_f32_16x16x32_{bf16,f16} and writes
//                  float32 partials [chunks, T, E].  A (normed) comes from
//                  global memory into registers; the W tile is staged
//                  transposed in LDS.  The MFMA consumes exactly the stored
//                  normed values.
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
constexpr int kNormVecs = 8;        // H <= 16384: 16384 / 8 / 256 vectors per thread

}  // namespace

template <bool F16>
__global__ void __launch_bounds__(kNormThreads)
    norm_kernel(const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ gamma, int H,
                float eps, uint16_t* __restrict__ normed) {
  __shared__ float red[kNormThreads / 64];
  const int t = blockIdx.x;
  const uint16_t* x = hidden + (size_t)t * H;
  const int nv = H / 8;                                   // 16-byte vectors (H % 128 == 0)
  // every vector of the row and of gamma is requested before any is used
  u32x4 xv[kNormVecs], gv[kNormVecs];
#pragma unroll
  for (int j = 0; j < kNormVecs; ++j) {
    const int v = threadIdx.x + j * kNormThreads;
    xv[j] = v < nv ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x) + v)
                   : u32x4{0, 0, 0, 0};
    gv[j] = v < nv ? reinterpret_cast<const u32x4*>(gamma)[v] : u32x4{0, 0, 0, 0};
  }
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < kNormVecs; ++j) {
    const uint32_t w[4] = {xv[j].x, xv[j].y, xv[j].z, xv[j].w};
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
#pragma unroll
  for (int j = 0; j < kNormVecs; ++j) {
    const int v = threadIdx.x + j * kNormThreads;
    if (v >= nv) break;
    const uint32_t w[4] = {xv[j].x, xv[j].y, xv[j].z, xv[j].w};
    const uint32_t g[4] = {gv[j].x, gv[j].y, gv[j].z, gv[j].w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = h2f<F16>((uint16_t)(w[i] & 0xffffu)) * r * h2f<F16>((uint16_t)(g[i] & 0xffffu));
      const float b = h2f<F16>((uint16_t)(w[i] >> 16)) * r * h2f<F16>((uint16_t)(g[i] >> 16));
      o[i] = (uint32_t)f2h<F16>(a) | ((uint32_t)f2h<F16>(b) << 16);
    }
    reinterpret_cast<u32x4*>(y)[v] = u32x4{o[0], o[1], o[2], o[3]};
  }
}

constexpr int kGemmThreads = 256;   // 4 waves
constexpr int kGemmSteps = 16;      // 32-wide k steps of a chunk held in registers (kc <= 512)
constexpr int kXcds = 8;            // accelerator complex dies of the MI355X

// Tile shape of the projection: experts per block = 16 * MOE_FE_GEMM_NS,
// tokens per block = 64 * MOE_FE_GEMM_S, k-chunk = the largest multiple of 32
// up to MOE_FE_GEMM_KC_MAX (see front_end_kchunk).
#ifndef MOE_FE_GEMM_NS
#define MOE_FE_GEMM_NS 2
#endif
#ifndef MOE_FE_GEMM_S
#define MOE_FE_GEMM_S 1
#endif
#ifndef MOE_FE_GEMM_KC_MAX
#define MOE_FE_GEMM_KC_MAX 480
#endif

__host__ __device__ inline int gemm_tile_stride(int kc) { return kc + 8; }   // u16, padded

// Split-K router projection: block = (k-chunk, 16*NS experts, 64*S tokens).
// Wave w computes tokens [64*S*tb + 16*S*w, +16*S) x the block's experts with
// v_mfma_f32_16x16x32_{bf16,f16}.  A comes from global memory straight into
// registers, requested first.  The W tile is staged transposed in LDS
// ([16*NS][kc + 8]: the padding spreads the 16 columns an MFMA reads over the
// LDS banks); each thread transposes 8 k-rows x 8 experts in registers with
// byte permutes so that the LDS writes are 16 bytes wide.
template <bool F16, int NS, int S>
__global__ void __launch_bounds__(kGemmThreads)
    gemm_kernel(const uint16_t* __restrict__ normed, const uint16_t* __restrict__ W, int T, int H,
                int E, int kc, float* __restrict__ partial) {
  extern __shared__ __align__(16) uint16_t wt[];
  constexpr int kN = 16 * NS, kRows = 64 * S;
  const int ngroups = (E + kN - 1) / kN;
  const int ntb = (T + kRows - 1) / kRows;
  const int nchunks = H / kc;
  const int per_chunk = ngroups * ntb;
  // Blocks are dispatched to the 8 XCDs round-robin (block b on XCD b % 8).
  // When the chunk count is a multiple of 8, every block of chunk c runs on
  // XCD c % 8, so that the chunk's A rows and W tiles come into one L2 once.
  const int b = blockIdx.x;
  int ch, r;
  if (nchunks % kXcds == 0) {
    const int x = b % kXcds, i = b / kXcds;             // i-th block of XCD x
    ch = x + kXcds * (i / per_chunk);
    r = i % per_chunk;
  } else {
    ch = b / per_chunk;
    r = b % per_chunk;
  }
  const int ng = r / ntb, tb = r % ntb;
  const int n0 = ng * kN, k0 = ch * kc;
  const int nsub = min(NS, (E - n0) / 16);              // E % 16 == 0
  const int nw = nsub * 16;                             // experts in this block
  const int ts = gemm_tile_stride(kc);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;           // k-group of 8
  const int row0 = tb * kRows + wv * 16 * S;
  u32x4 av[kGemmSteps][S];
#pragma unroll
  for (int u = 0; u < kGemmSteps; ++u)
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int row = row0 + 16 * s + col;
      av[u][s] = (row < T && 32 * u < kc)
                     ? *reinterpret_cast<const u32x4*>(normed + (size_t)row * H + k0 + 32 * u +
                                                       grp * 8)
                     : u32x4{0, 0, 0, 0};
    }
  // W[k0 : k0+kc, n0 : n0+nw] -> wt[n][k]: 8 x 8 blocks, one per thread per round
  const int nb8 = (kc / 8) * (nw / 8);
  for (int q = tid; q < nb8; q += kGemmThreads) {
    const int kb = (q / (nw / 8)) * 8, nb = (q % (nw / 8)) * 8;
    u32x4 w8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      w8[i] = *reinterpret_cast<const u32x4*>(W + (size_t)(k0 + kb + i) * E + n0 + nb);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int wi = n >> 1;
      const uint32_t sel = (n & 1) ? 0x07060302u : 0x05040100u;   // high or low halves
      uint32_t o[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        o[j] = __builtin_amdgcn_perm(w8[2 * j + 1][wi], w8[2 * j][wi], sel);   // k = 2j, 2j+1
      *reinterpret_cast<u32x4*>(wt + (nb + n) * ts + kb) = u32x4{o[0], o[1], o[2], o[3]};
    }
  }
  __syncthreads();
  f32x4v acc[S][NS];
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int n = 0; n < NS; ++n) acc[s][n] = f32x4v{0, 0, 0, 0};
#pragma unroll
  for (int u = 0; u < kGemmSteps; ++u) {
    const int kk = 32 * u;
    if (kk >= kc) break;
#pragma unroll
    for (int n = 0; n < NS; ++n) {
      if (n >= nsub) break;
      const u32x4 bv = *reinterpret_cast<const u32x4*>(wt + (16 * n + col) * ts + kk + grp * 8);
#pragma unroll
      for (int s = 0; s < S; ++s) {
        if constexpr (F16)
          acc[s][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              __builtin_bit_cast(f16x8, av[u][s]), __builtin_bit_cast(f16x8, bv), acc[s][n], 0, 0, 0);
        else
          acc[s][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, av[u][s]), __builtin_bit_cast(bf16x8, bv), acc[s][n], 0, 0,
              0);
      }
    }
  }
  // D layout: lane holds column (lane & 15), rows 4 * (lane >> 4) + i
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int n = 0; n < NS; ++n) {
      if (n >= nsub) break;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = row0 + 16 * s + 4 * grp + i;
        if (row < T) partial[((size_t)ch * T + row) * E + n0 + 16 * n + col] = acc[s][n][i];
      }
    }
}

constexpr int kSelectThreads = 256;  // one wavefront per token

// One wavefront per token; J = ceil(E / 64) experts per lane (expert
// lane + 64 j).
template <bool F16, int J>
__global__ void __launch_bounds__(kSelectThreads)
    select_kernel(const float* __restrict__ partial, int nchunks, const uint16_t* __restrict__ rbias,
                  int T, int E, int k, int act_sigmoid, int32_t* __restrict__ ids,
                  uint16_t* __restrict__ aff) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kSelectThreads / 64) + (threadIdx.x >> 6);
  if (t >= T) return;                                  // whole wavefront leaves together
  // chunk partials, summed in chunk order: a per-chunk base and fixed
  // per-slot offsets, every load of the token requested before the sums
  const float* pt = partial + (size_t)t * E + lane;
  const size_t cstride = (size_t)T * E;
  float z[J];
#pragma unroll
  for (int j = 0; j < J; ++j) z[j] = 0.0f;
  constexpr int CU = 16;                               // chunks in flight
  for (int c0 = 0; c0 < nchunks; c0 += CU) {
    float pv[CU][J];
#pragma unroll
    for (int u = 0; u < CU; ++u) {
      const float* pc = pt + (size_t)(c0 + u) * cstride;
#pragma unroll
      for (int j = 0; j < J; ++j)
        pv[u][j] = (c0 + u < nchunks && lane + 64 * j < E) ? pc[64 * j] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < CU; ++u)
#pragma unroll
      for (int j = 0; j < J; ++j)
        if (c0 + u < nchunks) z[j] += pv[u][j];
  }
  uint64_t pk[J];                                      // (key, lower index first); 0 = taken
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int e = lane + 64 * j;
    if (e < E) {
      if (rbias != nullptr) z[j] += h2f<F16>(rbias[e]);
      pk[j] = pack_key(z[j] + 0.0f, e);
    } else {
      z[j] = -__builtin_huge_valf();
      pk[j] = 0ull;
    }
  }
  // top-k on the raw logits: k rounds of a wavefront-wide maximum
  uint32_t taken = 0;
  float zmax = 0.0f;
  for (int r = 0; r < k; ++r) {
    uint64_t m[J];
#pragma unroll
    for (int j = 0; j < J; ++j) m[j] = pk[j];
#pragma unroll
    for (int w = 1; w < J; w <<= 1)                    // tree over the lane's slots
#pragma unroll
      for (int j = 0; j + w < J; j += 2 * w) m[j] = m[j + w] > m[j] ? m[j + w] : m[j];
    const uint64_t best = wave_max_u64(m[0]);
    const int e = unpack_idx(best);
    if (lane == 0) ids[(size_t)t * k + r] = e;
    if ((e & 63) == lane) {
      taken |= 1u << (e >> 6);
#pragma unroll
      for (int j = 0; j < J; ++j) pk[j] = j == (e >> 6) ? 0ull : pk[j];
    }
    if (r == 0) zmax = unord_key((uint32_t)(best >> 32));   // the largest logit
  }
  float num[J];
  // activation on the chosen experts only
  float part = 0.0f;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    num[j] = 0.0f;
    if ((taken >> j) & 1u) {
      num[j] = act_sigmoid ? sigmoid_f32(z[j]) : exp_f32(z[j] - zmax);
      part += num[j];
    }
  }
  float denom = 1.0f;
  if (!act_sigmoid) {
    for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
    denom = part;
  }
  const float inv = 1.0f / denom;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int e = lane + 64 * j;
    if (e < E) {
      const float v = ((taken >> j) & 1u) ? num[j] * inv : 0.0f;
      aff[(size_t)t * E + e] = (uint16_t)f32_to_bf16_rne(v);
    }
  }
}

int front_end_kchunk(int H) {
  // The largest multiple of 32 (one MFMA k step), at most MOE_FE_GEMM_KC_MAX
  // (<= 480: a padded 64-expert W tile then fits in 64 KiB of LDS), that
  // divides H into a multiple of 8 chunks (one group of blocks per XCD);
  // else the largest that divides H into at least 8 chunks; else 128
  // (H % 128 == 0).
  static_assert(MOE_FE_GEMM_KC_MAX <= 480 && MOE_FE_GEMM_KC_MAX % 32 == 0, "k-chunk bound");
  for (int kc = MOE_FE_GEMM_KC_MAX; kc >= 128; kc -= 32)
    if (H % kc == 0 && (H / kc) % kXcds == 0) return kc;
  for (int kc = MOE_FE_GEMM_KC_MAX; kc >= 128; kc -= 32)
    if (H % kc == 0 && H / kc >= 8) return kc;
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
  constexpr int kNS = MOE_FE_GEMM_NS, kS = MOE_FE_GEMM_S;
  static_assert((kNS == 1 || kNS == 2 || kNS == 4) && (kS == 1 || kS == 2), "gemm tile shape");
  const size_t lds = (size_t)16 * kNS * gemm_tile_stride(kc) * sizeof(uint16_t);
  const int blocks = ((q.E + 16 * kNS - 1) / (16 * kNS)) * ((q.T + 64 * kS - 1) / (64 * kS)) *
                     nchunks;
  if (q.f16)
    hipLaunchKernelGGL((gemm_kernel<true, kNS, kS>), dim3(blocks), dim3(kGemmThreads), lds, s,
                       (const uint16_t*)q.normed, (const uint16_t*)q.W, q.T, q.H, q.E, kc,
                       q.partial);
  else
    hipLaunchKernelGGL((gemm_kernel<false, kNS, kS>), dim3(blocks), dim3(kGemmThreads), lds, s,
                       (const uint16_t*)q.normed, (const uint16_t*)q.W, q.T, q.H, q.E, kc,
                       q.partial);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nb = (q.T + kSelectThreads / 64 - 1) / (kSelectThreads / 64);
  const int J = (q.E + 63) / 64;                     // E <= 512
#define MOE_SELECT(F, JJ)                                                                       \
  hipLaunchKernelGGL((select_kernel<F, JJ>), dim3(nb), dim3(kSelectThreads), 0, s, q.partial,  \
                     nchunks, (const uint16_t*)q.rbias, q.T, q.E, q.k, q.act_sigmoid, q.ids,    \
                     (uint16_t*)q.aff)
  if (q.f16) {
    if (J <= 1) MOE_SELECT(true, 1);
    else if (J <= 2) MOE_SELECT(true, 2);
    else if (J <= 4) MOE_SELECT(true, 4);
    else MOE_SELECT(true, 8);
  } else {
    if (J <= 1) MOE_SELECT(false, 1);
    else if (J <= 2) MOE_SELECT(false, 2);
    else if (J <= 4) MOE_SELECT(false, 4);
    else MOE_SELECT(false, 8);
  }
#undef MOE_SELECT
  return hipGetLastError();
}

}  // namespace moe
