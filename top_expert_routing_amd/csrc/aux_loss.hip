// gfx950 kernels for the MoE load-balancing aux loss (TransformerEngine Fused
// Router, Description: FusedAuxLoss forward and backward from probs and
// tokens-per-expert; Signature: fused_moe_aux_loss(probs, tokens_per_expert,
// total_num_tokens, num_experts, topk, coeff)).
//
//   loss            = C * sum_{t,e} probs[t, e] * c_e,  C = coeff*E/(topk*T_tot^2)
//   grad_probs[t,e] = g * C * c_e
//
// Forward: each block reduces a contiguous row range of probs into one partial
// (the dot with c needs no per-column state: every element contributes
// probs * c_col), partials are summed in block order by one block in float64,
// so the result is deterministic.  Backward: a broadcast write.  Both stream
// probs / grad_probs with 16-byte accesses: HBM-bound.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {
constexpr int kAuxBlock = 256;
constexpr int kAuxMaxE = 2048;
constexpr int kAuxUnroll = 8;   // 16-byte loads in flight per thread (32 KiB per block)
}

__global__ void __launch_bounds__(kAuxBlock)
    aux_fwd_partial_kernel(const float* __restrict__ probs, const int32_t* __restrict__ counts,
                           int64_t rows, int E, int64_t rows_per_block, int vec,
                           double* __restrict__ partial) {
  __shared__ __align__(16) float cs[kAuxMaxE];
  __shared__ float red[kAuxBlock / 64];
  for (int e = threadIdx.x; e < E; e += kAuxBlock) cs[e] = (float)counts[e];
  __syncthreads();
  const int64_t r0 = (int64_t)blockIdx.x * rows_per_block;
  const int64_t r1 = r0 + rows_per_block < rows ? r0 + rows_per_block : rows;
  const int64_t begin = r0 * E, end = r1 * E;
  float acc = 0.0f;
  if (vec) {
    // E % 4 == 0 and probs 16-byte aligned: element groups of 4 share a row.
    // kAuxUnroll groups per thread are requested before any is used.
    const int64_t stride = (int64_t)kAuxBlock * 4;
    const int step = (int)(stride % E);
    int64_t i = begin + threadIdx.x * 4;
    int col = (int)(i % E);
    for (; i < end; i += stride * kAuxUnroll) {
      f32x4 v[kAuxUnroll];
#pragma unroll
      for (int u = 0; u < kAuxUnroll; ++u)
        v[u] = i + u * stride < end
                   ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(probs + i + u * stride))
                                    : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int u = 0; u < kAuxUnroll; ++u) {
        const f32x4 c = *reinterpret_cast<const f32x4*>(cs + col);   // col % 4 == 0
        acc += v[u].x * c.x + v[u].y * c.y + v[u].z * c.z + v[u].w * c.w;
        col += step;
        if (col >= E) col -= E;
      }
    }
  } else {
    for (int64_t i = begin + threadIdx.x; i < end; i += kAuxBlock)
      acc += probs[i] * cs[(int)(i % E)];
  }
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double s = 0.0;
    for (int w = 0; w < kAuxBlock / 64; ++w) s += (double)red[w];
    partial[blockIdx.x] = s;
  }
}

__global__ void __launch_bounds__(256)
    aux_fwd_final_kernel(const double* __restrict__ partial, int nparts, double scale,
                         float* __restrict__ loss) {
  __shared__ double s[4];
  // each thread sums a contiguous run, then a fixed butterfly per wavefront and
  // the four wavefront sums in order: the same order on every run
  const int per = (nparts + 255) / 256;
  const int lo = threadIdx.x * per;
  double a = 0.0;
  for (int i = lo; i < lo + per && i < nparts; ++i) a += partial[i];
  for (int o = 32; o > 0; o >>= 1) a += __shfl_xor(a, o, 64);
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = a;
  __syncthreads();
  if (threadIdx.x == 0) *loss = (float)((((s[0] + s[1]) + s[2]) + s[3]) * scale);
}

__global__ void __launch_bounds__(kAuxBlock)
    aux_bwd_kernel(const int32_t* __restrict__ counts, int64_t rows, int E, double scale,
                   const float* __restrict__ grad_loss, int vec, float* __restrict__ grad) {
  __shared__ float v[kAuxMaxE];
  const double g = grad_loss != nullptr ? (double)*grad_loss : 1.0;
  for (int e = threadIdx.x; e < E; e += kAuxBlock) v[e] = (float)(g * scale * (double)counts[e]);
  __syncthreads();
  const int64_t n = rows * E;
  const int64_t tid = (int64_t)blockIdx.x * kAuxBlock + threadIdx.x;
  const int64_t nthreads = (int64_t)gridDim.x * kAuxBlock;
  if (vec) {
    const int64_t stride = nthreads * 4;
    int col = (int)((tid * 4) % E);
    const int step = (int)(stride % E);
    for (int64_t i = tid * 4; i < n; i += stride) {
      f32x4 q;
      q.x = v[col]; q.y = v[col + 1]; q.z = v[col + 2]; q.w = v[col + 3];
      __builtin_nontemporal_store(q, reinterpret_cast<f32x4*>(grad + i));
      col += step;
      while (col >= E) col -= E;
    }
  } else {
    for (int64_t i = tid; i < n; i += nthreads) grad[i] = v[(int)(i % E)];
  }
}

int aux_fwd_blocks(int64_t rows, int E) {
  // about 32 KiB of probs per block, at most 2048 blocks
  int64_t rpb = (8192 + E - 1) / E;
  if (rpb < 1) rpb = 1;
  int64_t nb = (rows + rpb - 1) / rpb;
  if (nb > 2048) nb = 2048;
  if (nb < 1) nb = 1;
  return (int)nb;
}

hipError_t launch_aux_fwd(const float* probs, const int32_t* counts, int64_t rows, int E,
                          double scale, double* partial, int nb, float* loss, hipStream_t s) {
  const int64_t rpb = (rows + nb - 1) / nb;
  const int vec = (E % 4 == 0) && ((uintptr_t)probs % 16 == 0);
  hipLaunchKernelGGL(aux_fwd_partial_kernel, dim3(nb), dim3(kAuxBlock), 0, s, probs, counts,
                     rows, E, rpb < 1 ? (int64_t)1 : rpb, vec, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(aux_fwd_final_kernel, dim3(1), dim3(256), 0, s, partial, nb, scale, loss);
  return hipGetLastError();
}

hipError_t launch_aux_bwd(const int32_t* counts, int64_t rows, int E, double scale,
                          const float* grad_loss, float* grad, hipStream_t s) {
  const int vec = (E % 4 == 0) && ((uintptr_t)grad % 16 == 0);
  const int64_t n = rows * E;
  // sixteen 16-byte stores per thread (eight or four measured slower)
  int64_t nb = (n + (int64_t)kAuxBlock * 4 * 16 - 1) / ((int64_t)kAuxBlock * 4 * 16);
  if (nb > 4096) nb = 4096;
  if (nb < 1) nb = 1;
  MOE_LAUNCH(aux_bwd_kernel, dim3((unsigned)nb), dim3(kAuxBlock), 0, s, counts, rows, E, scale,
             grad_loss, vec, grad);
  return hipGetLastError();
}

}  // namespace moe
