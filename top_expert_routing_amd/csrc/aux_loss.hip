// gfx950 kernels for the MoE load-balancing aux loss (TransformerEngine Fused
// Router, Description: FusedAuxLoss forward and backward from probs and
// tokens-per-expert; Signature: fused_moe_aux_loss(probs, tokens_per_expert,
// total_num_tokens, num_experts, topk, coeff)).
//
//   loss            = C * sum_{t,e} probs[t, e] * c_e,  C = coeff*E/(topk*T_tot^2)
//   grad_probs[t,e] = g * C * c_e
//
// Forward, one launch: each block reduces a contiguous row range of probs into
// one float64 partial (the dot with c needs no per-column state: every element
// contributes probs * c_col) and publishes it; the block with the highest
// index, dispatched last, also waits for every other partial and sums them in
// block order, so the result does not depend on the order of arrival.
// Backward: a broadcast write.  Both stream probs / grad_probs with 16-byte
// accesses: HBM-bound.
//
// The hand-off needs no counter and no release fence (an agent-scope release
// writes back the XCD's whole L2, once per block; same-address device atomics
// from every block serialise): a partial slot is its own ready flag.  The
// slots are zero between calls; a block stores the bitwise complement of its
// partial (NaN made canonical first, so the stored word is never zero) with
// one device-scope 64-bit store, and the summing block polls the slots with
// device-scope loads (coherent across the XCDs' L2 caches) until none is
// zero, then returns them to zero.  Only the summing block waits, and every
// block it waits for was dispatched before it and never waits, so every wait
// ends; the poll is still bounded (kAuxSpinLimit polls), and one that runs out
// writes the loss as kAuxTimeoutNaN and leaves the slots as they are.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {
constexpr int kAuxBlock = 256;
constexpr int kAuxMaxE = 2048;
// 16-byte loads in flight per thread: four (16 KiB per block), two rounds of
// them per block (32 KiB).  Measured at 65536 x 128: 8.9 us, against 9.5 us
// for eight loads and one round, 10.9 us for four loads and one round (2048
// blocks: the summing block polls twice the slots) and 9.3 us for eight loads
// and two rounds.
constexpr int kAuxUnroll = 4;
constexpr int kAuxMaxRun = kAuxMaxBlocks / kAuxBlock;   // slots per summing thread
static_assert(kAuxMaxBlocks * 8 <= kAuxSyncBytes, "partial slots exceed the sync region");
}

__device__ __forceinline__ unsigned long long encode_partial(double s) {
  const unsigned long long b = s != s ? 0x7ff8000000000000ull   // canonical NaN
                                      : (unsigned long long)__double_as_longlong(s);
  return ~b;
}

__global__ void __launch_bounds__(kAuxBlock)
    aux_fwd_kernel(const float* __restrict__ probs, const int32_t* __restrict__ counts,
                   int64_t rows, int E, int64_t rows_per_block, int vec, double scale,
                   unsigned long long* __restrict__ slots, float* __restrict__ loss, int spin_limit) {
  static_assert(kAuxBlock == 256, "the final sum assumes four wavefronts");
  __shared__ __align__(16) float cs[kAuxMaxE];
  __shared__ float red[kAuxBlock / 64];
  __shared__ double red4[kAuxBlock / 64];
  __shared__ unsigned long long own;
  __shared__ int timed_out;
  const int64_t r0 = (int64_t)blockIdx.x * rows_per_block;
  const int64_t r1 = r0 + rows_per_block < rows ? r0 + rows_per_block : rows;
  const int64_t begin = r0 * E, end = r1 * E;
  float acc = 0.0f;
  if (vec) {
    // E % 4 == 0 and probs 16-byte aligned: element groups of 4 share a row.
    // kAuxUnroll groups per thread are requested before any is used; the
    // first ones before the counts are staged in LDS, so that their latency
    // and the counts' overlap.
    const int64_t stride = (int64_t)kAuxBlock * 4;
    int64_t i = begin + threadIdx.x * 4;
    f32x4 v[kAuxUnroll];
#pragma unroll
    for (int u = 0; u < kAuxUnroll; ++u)
      v[u] = i + u * stride < end
                 ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(probs + i + u * stride))
                                  : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int e = threadIdx.x; e < E; e += kAuxBlock) cs[e] = (float)counts[e];
    if (threadIdx.x == 0) timed_out = 0;
    const int step = (int)(stride % E);
    int col = (int)(i % E);
    __syncthreads();
    for (;;) {
#pragma unroll
      for (int u = 0; u < kAuxUnroll; ++u) {
        const f32x4 c = *reinterpret_cast<const f32x4*>(cs + col);   // col % 4 == 0
        acc += v[u].x * c.x + v[u].y * c.y + v[u].z * c.z + v[u].w * c.w;
        col += step;
        if (col >= E) col -= E;
      }
      i += stride * kAuxUnroll;
      if (i >= end) break;
#pragma unroll
      for (int u = 0; u < kAuxUnroll; ++u)
        v[u] = i + u * stride < end
                   ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(probs + i + u * stride))
                                    : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  } else {
    for (int e = threadIdx.x; e < E; e += kAuxBlock) cs[e] = (float)counts[e];
    if (threadIdx.x == 0) timed_out = 0;
    __syncthreads();
    for (int64_t i = begin + threadIdx.x; i < end; i += kAuxBlock)
      acc += probs[i] * cs[(int)(i % E)];
  }
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  const int nb = (int)gridDim.x;
  const bool summer = (int)blockIdx.x == nb - 1;
  if (threadIdx.x == 0) {
    double s = 0.0;
    for (int w = 0; w < kAuxBlock / 64; ++w) s += (double)red[w];
    if (summer) own = encode_partial(s);
    else __hip_atomic_store(slots + blockIdx.x, encode_partial(s), __ATOMIC_RELAXED,
                            __HIP_MEMORY_SCOPE_AGENT);
  }
  if (!summer) return;
  __syncthreads();
  // each thread polls a contiguous run of the other blocks' slots; all its
  // loads are in flight at once (clamped indices), reloaded until none is zero
  const int per = (nb + kAuxBlock - 1) / kAuxBlock;
  const int lo = threadIdx.x * per;
  const int n_mine = max(0, min(per, nb - 1 - lo));   // slot nb - 1 is `own`
  unsigned long long v[kAuxMaxRun] = {};
  bool ready = n_mine == 0;
  for (int spin = 0; !ready && spin < spin_limit; ++spin) {
#pragma unroll
    for (int u = 0; u < kAuxMaxRun; ++u)
      v[u] = __hip_atomic_load(slots + min(lo + u, nb - 1), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    ready = true;
#pragma unroll
    for (int u = 0; u < kAuxMaxRun; ++u)
      if (u < n_mine && v[u] == 0ull) ready = false;
    if (!ready) __builtin_amdgcn_s_sleep(2);
  }
  if (!ready) timed_out = 1;
  // the fixed-order sum: each thread its run, a butterfly per wavefront, the
  // four wavefront sums in order
  double a = 0.0;
#pragma unroll
  for (int u = 0; u < kAuxMaxRun; ++u) {
    if (u < per && lo + u < nb) {
      const unsigned long long w = lo + u == nb - 1 ? own : v[u];
      a += __longlong_as_double((long long)~w);
    }
  }
  for (int o = 32; o > 0; o >>= 1) a += __shfl_xor(a, o, 64);
  if ((threadIdx.x & 63) == 0) red4[threadIdx.x >> 6] = a;
  __syncthreads();
  if (timed_out) {
    if (threadIdx.x == 0) *loss = __uint_as_float(kAuxTimeoutNaN);
    return;
  }
  // every slot read: return them to zero for the next call (the summing
  // block's own slot too, which it never wrote: that repairs a dirty one)
  for (int u = 0; u < n_mine; ++u)
    __hip_atomic_store(slots + lo + u, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (threadIdx.x == 0)
    __hip_atomic_store(slots + nb - 1, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (threadIdx.x == 0) *loss = (float)((((red4[0] + red4[1]) + red4[2]) + red4[3]) * scale);
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
  // about 32 KiB of probs per block, at most kAuxMaxBlocks blocks
  int64_t rpb = (8192 + E - 1) / E;
  if (rpb < 1) rpb = 1;
  int64_t nb = (rows + rpb - 1) / rpb;
  if (nb > kAuxMaxBlocks) nb = kAuxMaxBlocks;
  if (nb < 1) nb = 1;
  return (int)nb;
}

hipError_t launch_aux_fwd(const float* probs, const int32_t* counts, int64_t rows, int E,
                          double scale, void* sync, int nb, float* loss, int spin_limit,
                          hipStream_t s) {
  const int64_t rpb = (rows + nb - 1) / nb;
  const int vec = (E % 4 == 0) && ((uintptr_t)probs % 16 == 0);
  MOE_LAUNCH(aux_fwd_kernel, dim3(nb), dim3(kAuxBlock), 0, s, probs, counts, rows, E,
             rpb < 1 ? (int64_t)1 : rpb, vec, scale, static_cast<unsigned long long*>(sync),
             loss, spin_limit);
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
