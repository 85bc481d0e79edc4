// gfx950 kernel for the backward of the routing outputs with respect to the
// router logits (TransformerEngine Fused Router, Description: the fused top-k
// with score function op and the scores-for-aux-loss op each have a
// backward).  The gradient is that of the forward with the chosen experts
// held fixed -- the top-k choice passes no gradient and the expert bias, used
// only to choose, receives none:
//
//   weights  w' = scale * w;  sigmoid: w = s_sel (or s_sel / sum s_sel);
//            softmax before top-k: w = p_sel (or p_sel / sum p_sel), p over E;
//            softmax after top-k: w = softmax of the chosen logits
//   scores   sigmoid: s / sum_E s;  softmax: softmax over E
//
//   grad_logits = d/dx ( sum_j g_j w'_j + sum_e h_e scores_e )
//
// A token per cluster of L lanes (L = 8/16 with four experts per lane for
// E <= 32/64, L = 16 with eight for E <= 128 (E a multiple of 8, k <= 16),
// L = 32 with eight for E <= 256,
// else the whole wavefront with J = 1, 2, 4, 8, 16 or 32 per lane, the least
// that holds E, for E <= 2048);
// lane l of a cluster holds experts [J l, J l + J): the logits row, the score
// gradient row and the output row move with one vector access per lane; the
// chosen experts' weight gradients reach their owner lanes by readlane (or a
// cluster shuffle); per-token sums are cluster reductions.  HBM-bound: per
// token it reads the logits row (+ the score gradient row) and k ids and
// weight gradients, and writes one float32 row.
#include "device_common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kBwdThreads = 256;
constexpr float kNegInf = -__builtin_huge_valf();

// reductions over the L lanes of one token
template <int L>
__device__ __forceinline__ float wsum(float v) { return cl_sum<L>(v); }
template <int L>
__device__ __forceinline__ float wmax(float v) { return cl_max<L>(v); }

// J consecutive elements at p (VEC: one vector access, p aligned to its size)
template <int J, bool VEC>
__device__ __forceinline__ void load_f32(const float* p, int n_valid, float (&v)[J]) {
  if constexpr (VEC && J >= 4) {
#pragma unroll
    for (int h = 0; h < J / 4; ++h) {
      const f32x4 q = reinterpret_cast<const f32x4*>(p)[h];
      v[4 * h] = q.x; v[4 * h + 1] = q.y; v[4 * h + 2] = q.z; v[4 * h + 3] = q.w;
    }
  } else if constexpr (VEC && J == 2) {
    const float2 q = *reinterpret_cast<const float2*>(p);
    v[0] = q.x; v[1] = q.y;
  } else {
#pragma unroll
    for (int j = 0; j < J; ++j) v[j] = j < n_valid ? p[j] : 0.0f;
  }
}

template <int J, bool VEC>
__device__ __forceinline__ void load_bf16(const uint16_t* p, int n_valid, float (&v)[J]) {
  if constexpr (VEC && J % 8 == 0) {
#pragma unroll
    for (int c = 0; c < J / 8; ++c) {
      const u32x4 q = reinterpret_cast<const u32x4*>(p)[c];
      const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) { v[8 * c + 2 * h] = bf16_lo(w[h]); v[8 * c + 2 * h + 1] = bf16_hi(w[h]); }
    }
  } else if constexpr (VEC && J == 4) {
    const uint2 q = *reinterpret_cast<const uint2*>(p);
    v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x); v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
  } else if constexpr (VEC && J == 2) {
    const uint32_t q = *reinterpret_cast<const uint32_t*>(p);
    v[0] = bf16_lo(q); v[1] = bf16_hi(q);
  } else {
#pragma unroll
    for (int j = 0; j < J; ++j) v[j] = j < n_valid ? bf16_bits_to_f32(p[j]) : 0.0f;
  }
}

template <int J, bool VEC>
__device__ __forceinline__ void store_f32(float* p, int n_valid, const float (&v)[J]) {
  if constexpr (VEC && J >= 4) {
#pragma unroll
    for (int h = 0; h < J / 4; ++h)
      __builtin_nontemporal_store(f32x4{v[4 * h], v[4 * h + 1], v[4 * h + 2], v[4 * h + 3]},
                                  reinterpret_cast<f32x4*>(p) + h);
  } else if constexpr (VEC && J == 2) {
    *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
  } else {
#pragma unroll
    for (int j = 0; j < J; ++j)
      if (j < n_valid) p[j] = v[j];
  }
}

}  // namespace

// One token's inputs, read before any token of the wavefront is computed.  The
// loads are unconditional, so that they are all in flight together (a load in
// a branch is awaited where the branch joins): t is a valid token (clusters
// past T read token T - 1 and store nothing), lanes past E read the row start,
// lanes j >= k read choice k - 1 and drop it.  HW / HS: weight / score
// gradients are given.
template <bool BF16, int J, bool VEC, bool HW, bool HS>
__device__ __forceinline__ void load_token(const RouteBwdParams& p, int t, int lane_c, int e0, int nv,
                                           float (&x)[J], float (&h)[J], int& my_id,
                                           float& my_g) {
  const int E = p.E, k = p.k;
  my_id = -1;
  my_g = 0.0f;
  if constexpr (HW) {
    const size_t q = (size_t)t * k + (lane_c < k ? lane_c : k - 1);
    my_id = p.ids[q];
    my_g = p.grad_weights[q];
  }
  const size_t row = (size_t)t * E + (nv > 0 ? e0 : 0);
  if constexpr (BF16)
    load_bf16<J, VEC>(static_cast<const uint16_t*>(p.logits) + row, nv, x);
  else
    load_f32<J, VEC>(static_cast<const float*>(p.logits) + row, nv, x);
#pragma unroll
  for (int j = 0; j < J; ++j) h[j] = 0.0f;
  if constexpr (HS) {
    load_f32<J, VEC>(p.grad_scores + row, nv, h);
#pragma unroll
    for (int j = 0; j < J; ++j)
      if (j >= nv) h[j] = 0.0f;                          // lanes past E read the row start
  }
  if constexpr (HW) {
    if (lane_c >= k) {
      my_id = -1;
      my_g = 0.0f;
    }
    my_g *= p.scale;
  }
}

// One token's gradient row, from its inputs; stored with streaming stores.
template <int J, int L, bool VEC, bool HW, bool HS>
__device__ __forceinline__ void token_grad(const RouteBwdParams& p, int t, bool tv, int lane, int e0,
                                           int nv, float (&x)[J], const float (&h)[J], int my_id,
                                           float my_g) {
  const int lane_c = lane & (L - 1), cbase = lane & ~(L - 1);
  const int E = p.E, k = p.k;
#pragma unroll
  for (int j = 0; j < J; ++j)
    if (j >= nv) x[j] = kNegInf;                        // outside E: no softmax mass
  float dx[J];
#pragma unroll
  for (int j = 0; j < J; ++j) dx[j] = 0.0f;

  const bool sigmoid = p.mode == kBwdSigmoid;
  // sigmoid scores s (0 outside E) and their derivative s (1 - s), formed as
  // e s^2 (e = exp(-x)) where s >= 1/2, so that 1 - s is not a cancellation
  float s[J], ds[J];
  if (sigmoid) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const float e = exp_f32(-x[j]);
      s[j] = j < nv ? __builtin_amdgcn_rcpf(1.0f + e) : 0.0f;
      ds[j] = j < nv ? (s[j] >= 0.5f ? e * s[j] * s[j] : s[j] * (1.0f - s[j])) : 0.0f;
    }
  }
  float pz[J];                                           // softmax over E (0 outside E)
  if (!sigmoid && (p.mode == kBwdSoftmaxPre || HS)) {
    float m = kNegInf;
#pragma unroll
    for (int j = 0; j < J; ++j) m = fmaxf(m, x[j]);
    m = wmax<L>(m);
    float z = 0.0f;
#pragma unroll
    for (int j = 0; j < J; ++j) { pz[j] = exp_f32(x[j] - m); z += pz[j]; }
    const float inv = 1.0f / wsum<L>(z);
#pragma unroll
    for (int j = 0; j < J; ++j) pz[j] *= inv;
  }

  if constexpr (HW) {
    // the chosen experts' scaled weight gradients, at their owner lanes
    float g[J];
    uint32_t sel = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) g[j] = 0.0f;
    for (int i = 0; i < k; ++i) {
      int e;
      float gi;
      if constexpr (L == 64) {                           // one token per wavefront: uniform
        e = __builtin_amdgcn_readlane(my_id, i);
        gi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_g), i));
      } else {                                           // the cluster's lane i
        e = __shfl(my_id, cbase + i, 64);
        gi = __shfl(my_g, cbase + i, 64);
      }
      if (e >= 0 && e < E && e / J == lane_c) {
#pragma unroll
        for (int j = 0; j < J; ++j)
          if (e % J == j) { g[j] = gi; sel |= 1u << j; }
      }
    }
    if (sigmoid) {
      float gs_[J];
      if (p.renorm) {                                    // w = s / S over the chosen
        float S = 0.0f, gs = 0.0f;
#pragma unroll
        for (int j = 0; j < J; ++j)
          if ((sel >> j) & 1u) { S += s[j]; gs += g[j] * s[j]; }
        S = wsum<L>(S);
        gs = wsum<L>(gs);
        const float invS = 1.0f / S, c = gs * invS;      // c = sum_j g_j w_j
#pragma unroll
        for (int j = 0; j < J; ++j) gs_[j] = (g[j] - c) * invS;
      } else {
#pragma unroll
        for (int j = 0; j < J; ++j) gs_[j] = g[j];
      }
#pragma unroll
      for (int j = 0; j < J; ++j)
        if ((sel >> j) & 1u) dx[j] += gs_[j] * ds[j];
    } else if (p.mode == kBwdSoftmaxPre) {
      float dp[J];
      if (p.renorm) {                                    // w = p_sel / S
        float S = 0.0f, gp = 0.0f;
#pragma unroll
        for (int j = 0; j < J; ++j)
          if ((sel >> j) & 1u) { S += pz[j]; gp += g[j] * pz[j]; }
        S = wsum<L>(S);
        gp = wsum<L>(gp);
        const float invS = 1.0f / S, c = gp * invS;
#pragma unroll
        for (int j = 0; j < J; ++j) dp[j] = ((sel >> j) & 1u) ? (g[j] - c) * invS : 0.0f;
      } else {
#pragma unroll
        for (int j = 0; j < J; ++j) dp[j] = g[j];         // zero where not chosen
      }
      float c2 = 0.0f;                                   // softmax Jacobian, transposed
#pragma unroll
      for (int j = 0; j < J; ++j) c2 += pz[j] * dp[j];
      c2 = wsum<L>(c2);
#pragma unroll
      for (int j = 0; j < J; ++j) dx[j] += pz[j] * (dp[j] - c2);
    } else {                                             // softmax of the chosen logits
      float ms = kNegInf;
#pragma unroll
      for (int j = 0; j < J; ++j)
        if ((sel >> j) & 1u) ms = fmaxf(ms, x[j]);
      ms = wmax<L>(ms);
      float w[J], zs = 0.0f;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        w[j] = ((sel >> j) & 1u) ? exp_f32(x[j] - ms) : 0.0f;
        zs += w[j];
      }
      const float invz = 1.0f / wsum<L>(zs);
      float c = 0.0f;
#pragma unroll
      for (int j = 0; j < J; ++j) { w[j] *= invz; c += w[j] * g[j]; }
      c = wsum<L>(c);
#pragma unroll
      for (int j = 0; j < J; ++j)
        if ((sel >> j) & 1u) dx[j] += w[j] * (g[j] - c);
    }
  }

  if constexpr (HS) {
    if (sigmoid) {                                       // q = s / sum_E s
      float Z = 0.0f;
#pragma unroll
      for (int j = 0; j < J; ++j) Z += s[j];
      Z = wsum<L>(Z);
      const float invZ = 1.0f / Z;
      float c = 0.0f;
#pragma unroll
      for (int j = 0; j < J; ++j) c += h[j] * s[j];
      c = wsum<L>(c) * invZ;                                // sum_e h_e q_e
#pragma unroll
      for (int j = 0; j < J; ++j) dx[j] += ds[j] * (h[j] - c) * invZ;
    } else {                                             // q = softmax over E
      float c = 0.0f;
#pragma unroll
      for (int j = 0; j < J; ++j) c += h[j] * pz[j];
      c = wsum<L>(c);
#pragma unroll
      for (int j = 0; j < J; ++j) dx[j] += pz[j] * (h[j] - c);
    }
  }
  if (tv && nv > 0) store_f32<J, VEC>(p.grad_logits + (size_t)t * E + e0, nv, dx);
}

// A token per cluster of L lanes (64 / L tokens per wavefront): token
// (4 b + w) (64 / L) + lane / L.  Clusters past T compute but store nothing.
template <bool BF16, int J, int L, bool VEC, bool HW, bool HS>
__global__ void __launch_bounds__(kBwdThreads) route_bwd_kernel(RouteBwdParams p) {
  constexpr int kTpw = 64 / L;
  const int lane = threadIdx.x & 63;
  const int t0 = (blockIdx.x * (kBwdThreads / 64) + (threadIdx.x >> 6)) * kTpw;
  if (t0 >= p.T) return;                                 // whole wavefront leaves together
  const int t = t0 + lane / L;
  const bool tv = t < p.T;
  const int e0 = J * (lane & (L - 1));
  const int nv = min(J, max(0, p.E - e0));               // this lane's experts
  float x[J], h[J], g;
  int id;
  load_token<BF16, J, VEC, HW, HS>(p, tv ? t : p.T - 1, lane & (L - 1), e0, nv, x, h, id, g);
  token_grad<J, L, VEC, HW, HS>(p, t, tv, lane, e0, nv, x, h, id, g);
}

template <bool BF16, int J, int L, bool VEC>
static void launch_bwd_v(const RouteBwdParams& p, dim3 grid, hipStream_t s) {
  const bool hw = p.grad_weights != nullptr, hs = p.grad_scores != nullptr;   // one at least
  if (hw && hs) MOE_LAUNCH((route_bwd_kernel<BF16, J, L, VEC, true, true>), grid, dim3(kBwdThreads), 0, s, p);
  else if (hw) MOE_LAUNCH((route_bwd_kernel<BF16, J, L, VEC, true, false>), grid, dim3(kBwdThreads), 0, s, p);
  else MOE_LAUNCH((route_bwd_kernel<BF16, J, L, VEC, false, true>), grid, dim3(kBwdThreads), 0, s, p);
}

template <bool BF16, int J, int L>
static hipError_t launch_bwd_j(const RouteBwdParams& p, bool vec, hipStream_t s) {
  const int per_block = kBwdThreads / 64 * (64 / L);
  const dim3 grid((p.T + per_block - 1) / per_block);
  if (vec) launch_bwd_v<BF16, J, L, true>(p, grid, s);
  else launch_bwd_v<BF16, J, L, false>(p, grid, s);
  return hipGetLastError();
}

hipError_t launch_route_backward(const RouteBwdParams& p, bool bf16, hipStream_t s) {
  // lanes per token: four experts per lane (16-byte float32 accesses) while a
  // token's k choices still fit its lanes, eight per lane over 16 lanes for
  // 64 < E <= 128 (E = 128, k = 8: 23 -> 19 us against four over 32), eight
  // over 32 lanes up to E = 256; else the whole wavefront
  const bool wide16 = p.E > 64 && p.E <= 128 && p.E % 8 == 0 && p.k <= 16;
  const int L = (p.E <= 32 && p.k <= 8) ? 8 : ((p.E <= 64 && p.k <= 16) || wide16) ? 16
              : (p.E <= 256 && p.k <= 32) ? 32 : 64;
  const int J = wide16 ? 8 : L < 32 ? 4 : L == 32 ? (p.E <= 128 ? 4 : 8)
              : p.E <= 64 ? 1 : p.E <= 128 ? 2 : p.E <= 256 ? 4 : p.E <= 512 ? 8
              : p.E <= 1024 ? 16 : 32;                                  // E <= 2048
  // vector accesses when every lane's J elements are whole and aligned
  const int esz = bf16 ? 2 : 4;
  const bool vec = J > 1 && p.E % J == 0 &&
                   (uintptr_t)p.logits % (J * esz) == 0 && (uintptr_t)p.grad_logits % (J * 4) == 0 &&
                   (p.grad_scores == nullptr || (uintptr_t)p.grad_scores % (J * 4) == 0);
  if (L == 8) return bf16 ? launch_bwd_j<true, 4, 8>(p, vec, s) : launch_bwd_j<false, 4, 8>(p, vec, s);
  if (L == 16 && J == 8) return bf16 ? launch_bwd_j<true, 8, 16>(p, vec, s) : launch_bwd_j<false, 8, 16>(p, vec, s);
  if (L == 16) return bf16 ? launch_bwd_j<true, 4, 16>(p, vec, s) : launch_bwd_j<false, 4, 16>(p, vec, s);
  if (L == 32 && J == 4)
    return bf16 ? launch_bwd_j<true, 4, 32>(p, vec, s) : launch_bwd_j<false, 4, 32>(p, vec, s);
  if (L == 32) return bf16 ? launch_bwd_j<true, 8, 32>(p, vec, s) : launch_bwd_j<false, 8, 32>(p, vec, s);
  switch (J) {
    case 1: return bf16 ? launch_bwd_j<true, 1, 64>(p, false, s) : launch_bwd_j<false, 1, 64>(p, false, s);
    case 2: return bf16 ? launch_bwd_j<true, 2, 64>(p, vec, s) : launch_bwd_j<false, 2, 64>(p, vec, s);
    case 4: return bf16 ? launch_bwd_j<true, 4, 64>(p, vec, s) : launch_bwd_j<false, 4, 64>(p, vec, s);
    case 8: return bf16 ? launch_bwd_j<true, 8, 64>(p, vec, s) : launch_bwd_j<false, 8, 64>(p, vec, s);
    case 16: return bf16 ? launch_bwd_j<true, 16, 64>(p, vec, s) : launch_bwd_j<false, 16, 64>(p, vec, s);
    default: return bf16 ? launch_bwd_j<true, 32, 64>(p, vec, s) : launch_bwd_j<false, 32, 64>(p, vec, s);
  }
}

}  // namespace moe
