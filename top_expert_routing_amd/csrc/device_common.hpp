// Device helpers shared by the gfx950 routing kernels: bf16 decode/encode,
// order-preserving key packing, sigmoid, and cluster (sub-wavefront) reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

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

// Inverse of ord_key.
__device__ __forceinline__ float unord_key(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// Selection order as one unsigned 64-bit integer: larger key first, then the
// lower expert index (its complement is larger).  Distinct experts never
// compare equal.  -0 is folded into +0 first (x + 0.0f), so that two zero keys
// are equal and the index decides between them.
__device__ __forceinline__ uint64_t pack_key(float key, int idx) {
  return ((uint64_t)ord_key(key + 0.0f) << 32) | (uint64_t)(~(uint32_t)idx);
}
__device__ __forceinline__ int unpack_idx(uint64_t p) { return (int)(~(uint32_t)p); }

// The MI355X dispatches the blocks of a 1-D grid to its 8 XCDs round-robin
// (block b on XCD b % 8), and each XCD has its own L2.  This maps the launch
// index to a logical block so that every XCD takes one contiguous range of
// logical blocks (a bijection on [0, nb)): neighbouring logical blocks then
// share an L2, so lines that consecutive blocks both write (a p2t segment
// filled in token order) are written back from one XCD, and rows that a range
// of blocks reads (a counting group) are fetched into one L2.
__device__ __forceinline__ int xcd_block(int b, int nb) {
  const int x = b & 7, i = b >> 3;
  const int per = nb >> 3, extra = nb & 7;
  return x * per + (x < extra ? x : extra) + i;
}

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

// ---- cross-lane primitives -------------------------------------------------------
// DPP controls (gfx9 encoding): quad permutes, mirrors inside a 16-lane row and
// row shifts.  A DPP move is one VALU op; no LDS round trip.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i inside each 8 lanes
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i inside each 16 lanes
constexpr int kDppRowShr = 0x110;     // + d: lane i reads lane i-d of its row (0 outside)
constexpr int kDppRowShl = 0x100;     // + d: lane i reads lane i+d of its row (0 outside)

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, true);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// Butterfly-style all-reduce over clusters of W consecutive lanes (W a power of
// two <= 64).  W <= 16 uses DPP (quad permutes, then half-row and row mirrors:
// after reducing inside quads, the mirror partner always lies in the other
// half); W >= 32 adds ds_bpermute steps.
template <int W, class T, class Op>
__device__ __forceinline__ T cl_reduce(T v, Op op) {
  if constexpr (W >= 2) {
    if constexpr (sizeof(T) == 8) v = op(v, dpp_u64<kDppXor1>(v));
    else if constexpr (__is_same(T, float)) v = op(v, dpp_f<kDppXor1>(v));
    else v = op(v, dpp_i<kDppXor1>(v));
  }
  if constexpr (W >= 4) {
    if constexpr (sizeof(T) == 8) v = op(v, dpp_u64<kDppXor2>(v));
    else if constexpr (__is_same(T, float)) v = op(v, dpp_f<kDppXor2>(v));
    else v = op(v, dpp_i<kDppXor2>(v));
  }
  if constexpr (W >= 8) {
    if constexpr (sizeof(T) == 8) v = op(v, dpp_u64<kDppHalfMirror>(v));
    else if constexpr (__is_same(T, float)) v = op(v, dpp_f<kDppHalfMirror>(v));
    else v = op(v, dpp_i<kDppHalfMirror>(v));
  }
  if constexpr (W >= 16) {
    if constexpr (sizeof(T) == 8) v = op(v, dpp_u64<kDppMirror>(v));
    else if constexpr (__is_same(T, float)) v = op(v, dpp_f<kDppMirror>(v));
    else v = op(v, dpp_i<kDppMirror>(v));
  }
  if constexpr (W >= 32) v = op(v, __shfl_xor(v, 16, 64));
  if constexpr (W >= 64) v = op(v, __shfl_xor(v, 32, 64));
  return v;
}

template <int W>
__device__ __forceinline__ float cl_max(float v) {
  return cl_reduce<W>(v, [](float a, float b) { return fmaxf(a, b); });
}
template <int W>
__device__ __forceinline__ float cl_min(float v) {
  return cl_reduce<W>(v, [](float a, float b) { return fminf(a, b); });
}
template <int W>
__device__ __forceinline__ float cl_sum(float v) {
  return cl_reduce<W>(v, [](float a, float b) { return a + b; });
}
template <int W>
__device__ __forceinline__ int cl_sum_i(int v) {
  return cl_reduce<W>(v, [](int a, int b) { return a + b; });
}
template <int W>
__device__ __forceinline__ uint64_t cl_max_u64(uint64_t v) {
  return cl_reduce<W>(v, [](uint64_t a, uint64_t b) { return a > b ? a : b; });
}

// Wavefront-wide maximum of an unsigned 64-bit value, uniform in every lane:
// DPP inside each 16-lane row, then row_bcast:15 (rows 1 and 3 take the last
// lane of the row before) and row_bcast:31 (rows 2 and 3 take lane 31); lane
// 63 ends with the maximum, which is read into scalar registers.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_u64_keep(uint64_t x) {   // disabled rows keep x
  const int lo = __builtin_amdgcn_update_dpp((int)(uint32_t)x, (int)(uint32_t)x, CTRL, ROW_MASK,
                                             0xF, false);
  const int hi = __builtin_amdgcn_update_dpp((int)(uint32_t)(x >> 32), (int)(uint32_t)(x >> 32),
                                             CTRL, ROW_MASK, 0xF, false);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = cl_max_u64<16>(v);
  uint64_t t = dpp_u64_keep<0x142, 0xA>(v);    // row_bcast:15 into rows 1 and 3
  v = t > v ? t : v;
  t = dpp_u64_keep<0x143, 0xC>(v);             // row_bcast:31 into rows 2 and 3
  v = t > v ? t : v;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// Value of lane (lane ^ D) for D in {1, 2, 4, 8} (inside a 16-lane row).  For
// D = 4 and 8 both row shifts are executed by every lane, then selected.
template <int D>
__device__ __forceinline__ uint64_t xor_lane_u64(uint64_t v, int lane) {
  if constexpr (D == 1) {
    return dpp_u64<kDppXor1>(v);
  } else if constexpr (D == 2) {
    return dpp_u64<kDppXor2>(v);
  } else {
    const uint64_t up = dpp_u64<kDppRowShl + D>(v);    // lane + D
    const uint64_t dn = dpp_u64<kDppRowShr + D>(v);    // lane - D
    return (lane & D) ? dn : up;
  }
}

// Bitonic sort, descending, of NS unsigned 64-bit values held S = NS / LPT per
// lane by a cluster of LPT lanes (LPT <= 16): element n = lane * S + s.
// Pairs closer than S are compared inside a lane, farther ones across lanes
// with DPP moves.
template <int LPT, int NS>
__device__ __forceinline__ void bitonic_desc(uint64_t (&v)[NS / LPT], int lane_c) {
  constexpr int S = NS / LPT;
  static_assert(S >= 1 && S * LPT == NS, "slots");
#pragma unroll
  for (int size = 2; size <= NS; size <<= 1) {
#pragma unroll
    for (int d = size >> 1; d >= 1; d >>= 1) {
      if (d < S) {
#pragma unroll
        for (int s = 0; s < S; ++s) {
          const int t = s ^ d;
          if (t > s) {
            const int n = lane_c * S + s;
            const bool desc = size == NS || (n & size) == 0;
            const uint64_t a = v[s], b = v[t];
            const bool sw = desc ? (a < b) : (a > b);
            v[s] = sw ? b : a;
            v[t] = sw ? a : b;
          }
        }
      } else {
#pragma unroll
        for (int s = 0; s < S; ++s) {
          uint64_t o;
          const int D = d / S;
          if (D == 1) o = xor_lane_u64<1>(v[s], lane_c);
          else if (D == 2) o = xor_lane_u64<2>(v[s], lane_c);
          else if (D == 4) o = xor_lane_u64<4>(v[s], lane_c);
          else o = xor_lane_u64<8>(v[s], lane_c);
          const int n = lane_c * S + s;
          const bool desc = size == NS || (n & size) == 0;
          const bool lower = (n & d) == 0;
          const bool keep_max = lower == desc;
          v[s] = keep_max ? (o > v[s] ? o : v[s]) : (o < v[s] ? o : v[s]);
        }
      }
    }
  }
}

// Inclusive prefix sum over the 64 lanes of a wavefront (lane i gets the sum
// of lanes 0..i), all in DPP moves: shifts by 1, 2, 4, 8 inside each 16-lane
// row (lanes without a source add 0), then row_bcast:15 adds row 0's total to
// row 1 and row 2's to row 3, and row_bcast:31 adds lanes 0..31's total to
// rows 2 and 3.  Every lane executes every move.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr + 1, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr + 2, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr + 4, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr + 8, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31 -> rows 2, 3
  return v;
}

// Exclusive prefix sum of one value per thread over a block of THREADS
// threads (a multiple of 64), in thread order; `total` gets the block's sum.
// tmp: LDS for THREADS / 64 ints.  Contains one block barrier; the caller
// places another before tmp is written again (a further round).
template <int THREADS>
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) tmp[w] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < THREADS / 64; ++i) {
    const int s = tmp[i];
    before += i < w ? s : 0;
    tot += s;
  }
  total = tot;
  return before + incl - v;
}

// Exclusive prefix sum over the cluster (lane c gets the sum of lanes < c).
template <int W>
__device__ __forceinline__ int cl_excl_scan(int v, int lane_c) {
  int incl = v;
  if constexpr (W <= 16) {
    // Every lane must execute each DPP move (a lane reading a source lane that
    // is switched off gets 0), so the shifted value is formed unconditionally
    // and only then masked by the cluster position.
    if constexpr (W >= 2) { const int u = dpp_i<kDppRowShr + 1>(incl); incl += lane_c >= 1 ? u : 0; }
    if constexpr (W >= 4) { const int u = dpp_i<kDppRowShr + 2>(incl); incl += lane_c >= 2 ? u : 0; }
    if constexpr (W >= 8) { const int u = dpp_i<kDppRowShr + 4>(incl); incl += lane_c >= 4 ? u : 0; }
    if constexpr (W >= 16) { const int u = dpp_i<kDppRowShr + 8>(incl); incl += lane_c >= 8 ? u : 0; }
  } else {
#pragma unroll
    for (int o = 1; o < W; o <<= 1) {
      const int u = __shfl_up(incl, o, W);
      if (lane_c >= o) incl += u;
    }
  }
  return incl - v;
}

}  // namespace moe
