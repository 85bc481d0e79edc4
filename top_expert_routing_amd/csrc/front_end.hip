// gfx950 kernels for the fused decode front end (NKI "RMSNorm Router Top-K
// A2AV Kernel API Reference": Background, Parameters, Returns, Notes).
//
// norm_gemm_kernel: one launch whose blocks take two roles in block-index
// order.
//   rms blocks     [0, T): one per token: r_t = (mean_h x^2 + eps)^-1/2 in
//                  float32; r_t is published first, then
//                  normed = round((x * gamma) * r_t) is stored in the input
//                  dtype (RNE).
//   gemm blocks    split-K router projection on MFMA: block (k-chunk, 16*NS
//                  experts, 64*S tokens) reads raw hidden and gamma, stages
//                  the W tile transposed in LDS while the rms blocks run,
//                  then waits for its tokens' r_t, forms exactly the normed
//                  values the rms blocks store and runs
//                  v_mfma_f32_16x16x32_{bf16,f16}, writing float32 partials
//                  [chunks, T, E].
// A gemm block waits only for rms blocks, which have lower indices and never
// wait: blocks are dispatched in index order on each XCD, so every wait ends.
// r_t is its own ready flag: the workspace slot is zero between calls and
// r_t > 0, so a gemm lane polls its token's slot (a device-scope load, coherent
// across the XCDs' L2 caches) until it is non-zero.  The poll is bounded by a
// spin limit: one that runs out sets the failure word, and the call then
// writes -1 into topk_ids instead of hanging; the last select block to have
// read the word counts the call and clears the word again.
//
// select_kernel: one wavefront per token, after the projection: z = sum of
// the partials in chunk order (+ router bias) -- deterministic; top-k on the
// raw logits (lower index on ties); activation on the chosen experts only
// (sigmoid, or softmax over the k chosen); affinities [T, E] bf16 with zeros
// elsewhere.  It also returns the token's r_t slot to zero.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

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

// The normalisation of one packed pair, in two steps: xg = x * gamma (float32,
// formed before r_t is known), then round(xg * r_t) into the input dtype.
// Wherever normed values are formed, the same two steps are used, so the
// stored values and the MFMA operands agree bit for bit.  bfloat16 rounds
// with gfx950's packed convert (v_cvt_pk_bf16_f32, round to nearest even).
template <bool F16>
__device__ __forceinline__ f32x2v xg_pair(uint32_t w, uint32_t g) {
  return f32x2v{h2f<F16>((uint16_t)(w & 0xffffu)) * h2f<F16>((uint16_t)(g & 0xffffu)),
                h2f<F16>((uint16_t)(w >> 16)) * h2f<F16>((uint16_t)(g >> 16))};
}
template <bool F16>
__device__ __forceinline__ uint32_t round_pair(f32x2v xg, float r) {
  const float lo = xg.x * r, hi = xg.y * r;
  if constexpr (F16)
    return (uint32_t)f2h<F16>(lo) | ((uint32_t)f2h<F16>(hi) << 16);
  else
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{lo, hi}, bf16x2));
}

constexpr int kThreads = 256;       // every role: 4 wavefronts
constexpr int kNormVecs = 8;        // H <= 16384: 16384 / 8 / 256 vectors per thread
constexpr int kXcds = 8;            // accelerator complex dies of the MI355X

}  // namespace

// Tile shape of the projection: experts per block = 16 * MOE_FE_GEMM_NS,
// tokens per block = 64 * MOE_FE_GEMM_S, k-chunk one of 128, 256, 384 or 448
// (a compile-time count of 32-wide MFMA steps; see front_end_kchunk).
#ifndef MOE_FE_GEMM_NS
#define MOE_FE_GEMM_NS 2
#endif
#ifndef MOE_FE_GEMM_S
#define MOE_FE_GEMM_S 1
#endif
constexpr int kNS = MOE_FE_GEMM_NS, kS = MOE_FE_GEMM_S;
static_assert((kNS == 1 || kNS == 2 || kNS == 4) && (kS == 1 || kS == 2), "gemm tile shape");
constexpr int kTileRows = 64 * kS;  // tokens per gemm block (one completion counter each)

// Workspace: the synchronisation region -- a failure line of 256 bytes and
// the r_t slots [128] -- then the float32 partials [H / kc, T, E].  The
// failure line holds three words: [0] set when a wait gave up, [1] the number
// of calls whose wait gave up (never cleared here: the caller's to read), [2]
// the select blocks that have read [0] in such a call.  Only [1] may be
// non-zero between calls.  Nothing clears [0] while the projection runs (a
// clear there could race with a give-up and lose it): it is set by the
// projection and read, counted and cleared by the selection, which runs after
// it in stream order.
constexpr int kFailBytes = 256;
static_assert(kFailBytes + 128 * 4 <= kFrontEndSyncBytes, "sync region");

__host__ __device__ inline int gemm_tile_stride(int kc) { return kc + 8; }   // u16, padded

namespace {

struct FeArgs {
  const uint16_t* hidden;
  const uint16_t* gamma;
  const uint16_t* W;
  const uint16_t* rbias;
  int T, H, E, kc;
  float eps;
  uint16_t* normed;
  uint32_t* fail;     // failure word
  uint32_t* rstd;     // [T] float32 bits, 0 = not yet written
  float* partial;     // [H / kc, T, E]
  int gemm_begin, gemm_blocks;
  int spin_limit;     // polls before a wait gives up
};

// r_t crosses blocks inside one launch: it is stored and loaded with
// device-scope accesses (sc1), which are coherent across the XCDs' L2 caches
// on their own: no whole-cache write-back or invalidation is needed.
__device__ __forceinline__ void st_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Poll one word until it is non-zero; 0 when the spin limit ran out.
__device__ __forceinline__ uint32_t poll_nonzero(const uint32_t* p, int spin_limit) {
  for (int i = 0; i < spin_limit; ++i) {
    const uint32_t v = ld_dev(p);
    if (v != 0u) return v;
    __builtin_amdgcn_s_sleep(2);
  }
  return 0u;
}

// A wait ran out: record it (the select kernel reads, counts and clears it).
__device__ __forceinline__ void mark_failed(const FeArgs& a) {
  st_dev(a.fail, 1u);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// rms role: one block per token.
template <bool F16>
__device__ void rms_role(const FeArgs& a, int t, float* red) {
  const int H = a.H;
  const uint16_t* x = a.hidden + (size_t)t * H;
  const int nv = H / 8;                                   // 16-byte vectors (H % 128 == 0)
  // every vector of the row and of gamma is requested before any is used
  u32x4 xv[kNormVecs], gv[kNormVecs];
#pragma unroll
  for (int j = 0; j < kNormVecs; ++j) {
    const int v = threadIdx.x + j * kThreads;
    xv[j] = v < nv ? reinterpret_cast<const u32x4*>(x)[v] : u32x4{0, 0, 0, 0};
    gv[j] = v < nv ? reinterpret_cast<const u32x4*>(a.gamma)[v] : u32x4{0, 0, 0, 0};
  }
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < kNormVecs; ++j) {
    const uint32_t w[4] = {xv[j].x, xv[j].y, xv[j].z, xv[j].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = h2f<F16>((uint16_t)(w[i] & 0xffffu));
      const float hi = h2f<F16>((uint16_t)(w[i] >> 16));
      ss += lo * lo + hi * hi;
    }
  }
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) tot += red[i];
  const float r = 1.0f / sqrtf(tot / (float)H + a.eps);
  if (threadIdx.x == 0) st_dev(a.rstd + t, __float_as_uint(r));   // r > 0: never 0 bits
  uint16_t* y = a.normed + (size_t)t * H;
#pragma unroll
  for (int j = 0; j < kNormVecs; ++j) {
    const int v = threadIdx.x + j * kThreads;
    if (v >= nv) break;
    const uint32_t w[4] = {xv[j].x, xv[j].y, xv[j].z, xv[j].w};
    const uint32_t g[4] = {gv[j].x, gv[j].y, gv[j].z, gv[j].w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = round_pair<F16>(xg_pair<F16>(w[i], g[i]), r);
    __builtin_nontemporal_store(u32x4{o[0], o[1], o[2], o[3]}, reinterpret_cast<u32x4*>(y) + v);
  }
}

// gemm role: block b of the projection.  Wave w computes tokens
// [64*S*tb + 16*S*w, +16*S) x the block's experts.  The raw hidden rows come
// from global memory straight into registers, requested first; gamma's chunk
// and the W tile are staged in LDS (W transposed, [16*NS][kc + 8]: the padding
// spreads the 16 columns an MFMA reads over the LDS banks; each thread
// transposes 8 k-rows x 8 experts in registers with byte permutes so that the
// LDS writes are 16 bytes wide).  Then each lane polls its token's r_t and
// normalises in registers exactly as the rms blocks do.
template <bool F16, int STEPS>
__device__ void gemm_role(const FeArgs& a, int b, uint16_t* wt, uint16_t* gl) {
  constexpr int kN = 16 * kNS;
  constexpr int kc = 32 * STEPS;
  const int T = a.T, H = a.H, E = a.E;
  const int ngroups = (E + kN - 1) / kN;
  const int ntb = (T + kTileRows - 1) / kTileRows;
  const int nchunks = H / kc;
  const int per_chunk = ngroups * ntb;
  // Blocks are dispatched to the 8 XCDs round-robin (block b on XCD b % 8;
  // the gemm range starts at a multiple of 8).  When the chunk count is a
  // multiple of 8, every block of chunk c runs on XCD c % 8, so that the
  // chunk's hidden rows and W tiles come into one L2 once.
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
  const int nsub = min(kNS, (E - n0) / 16);             // E % 16 == 0
  const int nw = nsub * 16;                             // experts in this block
  const int ts = gemm_tile_stride(kc);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;           // k-group of 8
  const int row0 = tb * kTileRows + wv * 16 * kS;
  // Every global read is issued before any is awaited (a load under a branch,
  // or one whose value goes straight to LDS, is awaited at once, and with it
  // every older load): the hidden rows (rows past T read row T - 1; their
  // products are never stored: an MFMA output row depends on its own input
  // row only), gamma into registers, then the W tile.
  u32x4 av[STEPS][kS];
#pragma unroll
  for (int u = 0; u < STEPS; ++u)
#pragma unroll
    for (int s = 0; s < kS; ++s) {
      const int row = min(row0 + 16 * s + col, T - 1);
      av[u][s] = *reinterpret_cast<const u32x4*>(a.hidden + (size_t)row * H + k0 + 32 * u + grp * 8);
    }
  static_assert(kc / 8 <= kThreads, "gamma: one 16-byte piece per thread");
  const u32x4 gv = reinterpret_cast<const u32x4*>(a.gamma + k0)[tid < kc / 8 ? tid : 0];
  // W[k0 : k0+kc, n0 : n0+nw] -> wt[n][k]: 8 x 8 blocks, one per thread per round
  const int nb8 = (kc / 8) * (nw / 8);
  for (int q = tid; q < nb8; q += kThreads) {
    const int kb = (q / (nw / 8)) * 8, nb = (q % (nw / 8)) * 8;
    u32x4 w8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      w8[i] = *reinterpret_cast<const u32x4*>(a.W + (size_t)(k0 + kb + i) * E + n0 + nb);
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
  if (tid < kc / 8) reinterpret_cast<u32x4*>(gl)[tid] = gv;
  __syncthreads();                                      // W tile and gamma staged
  // x * gamma while r_t is on its way
  f32x2v xg[STEPS][kS][4];
#pragma unroll
  for (int u = 0; u < STEPS; ++u) {
    const u32x4 g8 = *reinterpret_cast<const u32x4*>(gl + 32 * u + grp * 8);
#pragma unroll
    for (int s = 0; s < kS; ++s) {
      xg[u][s][0] = xg_pair<F16>(av[u][s].x, g8.x);
      xg[u][s][1] = xg_pair<F16>(av[u][s].y, g8.y);
      xg[u][s][2] = xg_pair<F16>(av[u][s].z, g8.z);
      xg[u][s][3] = xg_pair<F16>(av[u][s].w, g8.w);
    }
  }
  // keep the products here, ahead of the wait (the compiler would otherwise
  // sink them past the poll, onto the path after r_t arrives)
#pragma unroll
  for (int u = 0; u < STEPS; ++u)
#pragma unroll
    for (int s = 0; s < kS; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(xg[u][s][i].x), "+v"(xg[u][s][i].y));
  float rr[kS];
#pragma unroll
  for (int s = 0; s < kS; ++s) {
    const int row = row0 + 16 * s + col;
    uint32_t bits = 0u;
    if (row < T) {
      bits = poll_nonzero(a.rstd + row, a.spin_limit);
      if (bits == 0u) mark_failed(a);
    }
    rr[s] = __uint_as_float(bits);
  }
#pragma unroll
  for (int u = 0; u < STEPS; ++u)
#pragma unroll
    for (int s = 0; s < kS; ++s)
      av[u][s] = u32x4{round_pair<F16>(xg[u][s][0], rr[s]), round_pair<F16>(xg[u][s][1], rr[s]),
                       round_pair<F16>(xg[u][s][2], rr[s]), round_pair<F16>(xg[u][s][3], rr[s])};
  f32x4v acc[kS][kNS];
#pragma unroll
  for (int s = 0; s < kS; ++s)
#pragma unroll
    for (int n = 0; n < kNS; ++n) acc[s][n] = f32x4v{0, 0, 0, 0};
  // Every n-subtile is computed (rows of the W tile past the block's experts
  // hold stale LDS data, whose sums are never stored): no branch between the
  // LDS reads and the MFMAs.
#pragma unroll
  for (int u = 0; u < STEPS; ++u) {
    const int kk = 32 * u;
#pragma unroll
    for (int n = 0; n < kNS; ++n) {
      const u32x4 bv = *reinterpret_cast<const u32x4*>(wt + (16 * n + col) * ts + kk + grp * 8);
#pragma unroll
      for (int s = 0; s < kS; ++s) {
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
  for (int s = 0; s < kS; ++s)
#pragma unroll
    for (int n = 0; n < kNS; ++n) {
      if (n >= nsub) break;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = row0 + 16 * s + 4 * grp + i;
        if (row < T) a.partial[((size_t)ch * T + row) * E + n0 + 16 * n + col] = acc[s][n][i];
      }
    }
}

// Lane `l`'s value (l uniform) in every lane.  The readlane builtin returns a
// signed int: each half is taken as uint32 before it is widened.
__device__ __forceinline__ uint64_t read_u64(uint64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

// Top-2 of a 16-lane row, in every lane of the row: (a1 >= a2) merged with
// the partner's pair over the same DPP pattern as a row reduction (quad
// permutes, then half-row and row mirrors: each partner holds a disjoint set).
template <int CTRL>
__device__ __forceinline__ void top2_step(uint64_t& a1, uint64_t& a2) {
  const uint64_t b1 = dpp_u64<CTRL>(a1), b2 = dpp_u64<CTRL>(a2);
  const uint64_t hi = a1 > b1 ? a1 : b1, lo = a1 > b1 ? b1 : a1;
  const uint64_t m2 = a2 > b2 ? a2 : b2;
  a1 = hi;
  a2 = lo > m2 ? lo : m2;
}

// Top-k (k <= 8) of the keys a wavefront holds (J per lane, 0 = no expert)
// by a threshold: tau = the smallest of the four rows' second-largest lane
// maxima, so at least 8 keys are >= tau; the candidates (keys >= tau) are
// compacted into LDS and each is ranked against the others.  Writes ids[0..k)
// and returns the k-th largest key; returns 0 (nothing written) when there
// are more than 64 candidates.
template <int J>
__device__ __forceinline__ uint64_t topk_threshold(const uint64_t (&pk)[J], int k, int lane,
                                                   uint64_t* cand, int32_t* ids, bool failed,
                                                   uint64_t& top) {
  uint64_t a1 = pk[0];
#pragma unroll
  for (int j = 1; j < J; ++j) a1 = pk[j] > a1 ? pk[j] : a1;
  uint64_t a2 = 0ull;
  top2_step<kDppXor1>(a1, a2);
  top2_step<kDppXor2>(a1, a2);
  top2_step<kDppHalfMirror>(a1, a2);
  top2_step<kDppMirror>(a1, a2);
  uint64_t tau = ~0ull;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint64_t v = read_u64(a2, 16 * r);
    tau = v < tau ? v : tau;
  }
  if (tau == 0ull) tau = 1ull;                         // a row without two keys: every key
  int n = 0;
#pragma unroll
  for (int j = 0; j < J; ++j) n += __popcll(__ballot(pk[j] >= tau));
  if (n > 64) return 0ull;
  int base = 0;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const bool c = pk[j] >= tau;
    const uint64_t m = __ballot(c);
    if (c) cand[base + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u))] = pk[j];
    base += __popcll(m);
  }
  wave_lds_sync();
  const uint64_t x = lane < n ? cand[lane] : 0ull;
  int rank = 0;
  int i = 0;
  for (; i + 8 <= n; i += 8) {                         // eight LDS reads in flight
    uint64_t c[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) c[q] = cand[i + q];
#pragma unroll
    for (int q = 0; q < 8; ++q) rank += c[q] > x ? 1 : 0;
  }
  for (; i < n; ++i) rank += cand[i] > x ? 1 : 0;
  if (lane < n && rank < k) ids[rank] = failed ? -1 : unpack_idx(x);
  const uint64_t mk = __ballot(lane < n && rank == k - 1);
  const uint64_t m0 = __ballot(lane < n && rank == 0);
  const int lk = __builtin_ctzll(mk), l0 = __builtin_ctzll(m0);
  top = read_u64(x, l0);
  return read_u64(x, lk);
}

}  // namespace

template <bool F16, int STEPS>
__global__ void __launch_bounds__(kThreads) norm_gemm_kernel(FeArgs a) {
  extern __shared__ __align__(16) uint16_t lds[];
  __shared__ float red[kThreads / 64];
  const int b = blockIdx.x;
  // The select blocks' reader count starts every call at zero, whatever a
  // region that was not clean held (only select blocks touch it, and they run
  // after this launch).
  if (b == 0 && threadIdx.x == 0) st_dev(a.fail + 2, 0u);
  if (b < a.T) rms_role<F16>(a, b, red);
  else if (b >= a.gemm_begin) gemm_role<F16, STEPS>(a, b - a.gemm_begin, lds + 8 + 32 * STEPS, lds);
}

// J consecutive floats (J in {1, 2, 4, 8}; p aligned to 4 J bytes).
template <int J>
__device__ __forceinline__ void load_floats(const float* p, float (&v)[J]) {
  if constexpr (J == 1) {
    v[0] = *p;
  } else if constexpr (J == 2) {
    const f32x2v q = *reinterpret_cast<const f32x2v*>(p);
    v[0] = q.x;
    v[1] = q.y;
  } else {
#pragma unroll
    for (int h = 0; h < J / 4; ++h) {
      const f32x4v q = reinterpret_cast<const f32x4v*>(p)[h];
      v[4 * h] = q.x;
      v[4 * h + 1] = q.y;
      v[4 * h + 2] = q.z;
      v[4 * h + 3] = q.w;
    }
  }
}

// J consecutive bf16 values (p aligned to 2 J bytes).
template <int J>
__device__ __forceinline__ void store_bf16(uint16_t* p, const float (&v)[J]) {
  if constexpr (J == 1) {
    *p = (uint16_t)f32_to_bf16_rne(v[0]);
  } else {
    uint32_t w[J / 2];
#pragma unroll
    for (int h = 0; h < J / 2; ++h)
      w[h] = f32_to_bf16_rne(v[2 * h]) | (f32_to_bf16_rne(v[2 * h + 1]) << 16);
    if constexpr (J == 2) *reinterpret_cast<uint32_t*>(p) = w[0];
    else if constexpr (J == 4) *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
    else *reinterpret_cast<u32x4*>(p) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// One wavefront per token, one token per block (the reads of a CU are bounded
// by its own outstanding requests, so the tokens spread over as many CUs as
// possible); J = ceil(E / 64) experts per lane, consecutive (expert
// J * lane + j), so that each chunk's partials arrive in one vector load per
// lane.
template <bool F16, int J>
__global__ void __launch_bounds__(64)
    select_kernel(const float* __restrict__ partial, int nchunks, const uint16_t* __restrict__ rbias,
                  int T, int E, int k, int act_sigmoid, uint32_t* __restrict__ rstd,
                  uint32_t* __restrict__ fail, int32_t* __restrict__ ids,
                  uint16_t* __restrict__ aff) {
  __shared__ uint64_t cand_lds[64];
  const int lane = threadIdx.x;
  const int t = blockIdx.x;
  const int e0 = J * lane;
  const bool owner = e0 < E;                           // E % J == 0: whole vectors
  // the failure word and the router bias first: their latency overlaps the
  // partials'
  const bool failed = *fail != 0u;
  float bias[J];
#pragma unroll
  for (int j = 0; j < J; ++j) bias[j] = (owner && rbias != nullptr) ? h2f<F16>(rbias[e0 + j]) : 0.0f;
  // chunk partials, summed in chunk order, every load of the token requested
  // before the sums
  const float* pt = partial + (size_t)t * E + e0;
  const size_t cstride = (size_t)T * E;
  float z[J];
#pragma unroll
  for (int j = 0; j < J; ++j) z[j] = 0.0f;
  constexpr int CU = 16;                               // chunks in flight
  for (int c0 = 0; c0 < nchunks; c0 += CU) {
    float pv[CU][J];
#pragma unroll
    for (int u = 0; u < CU; ++u) {
      if (owner && c0 + u < nchunks) {
        load_floats<J>(pt + (size_t)(c0 + u) * cstride, pv[u]);
      } else {
#pragma unroll
        for (int j = 0; j < J; ++j) pv[u][j] = 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < CU; ++u)
#pragma unroll
      for (int j = 0; j < J; ++j)
        if (c0 + u < nchunks) z[j] += pv[u][j];
  }
  if (lane == 0) rstd[t] = 0u;                         // back to "not yet written"
  uint64_t pk[J];                                      // (key, lower index first); 0 = none
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if (owner) {
      if (rbias != nullptr) z[j] += bias[j];
      pk[j] = pack_key(z[j] + 0.0f, e0 + j);
    } else {
      z[j] = -__builtin_huge_valf();
      pk[j] = 0ull;
    }
  }
  // top-k on the raw logits: a threshold and a ranking of the candidates, or
  // (k > 8, or more than 64 candidates) k rounds of a wavefront-wide maximum
  uint32_t taken = 0;
  float zmax = 0.0f;
  uint64_t top = 0ull;
  const uint64_t kth = k <= 8 ? topk_threshold<J>(pk, k, lane, cand_lds,
                                                  ids + (size_t)t * k, failed, top)
                              : 0ull;
  if (kth != 0ull) {
#pragma unroll
    for (int j = 0; j < J; ++j) taken |= (pk[j] >= kth ? 1u : 0u) << j;
    zmax = unord_key((uint32_t)(top >> 32));           // the largest logit
  }
  for (int r = 0; kth == 0ull && r < k; ++r) {
    uint64_t m[J];
#pragma unroll
    for (int j = 0; j < J; ++j) m[j] = pk[j];
#pragma unroll
    for (int w = 1; w < J; w <<= 1)                    // tree over the lane's slots
#pragma unroll
      for (int j = 0; j + w < J; j += 2 * w) m[j] = m[j + w] > m[j] ? m[j + w] : m[j];
    const uint64_t best = wave_max_u64(m[0]);
    const int e = unpack_idx(best);
    if (lane == 0) ids[(size_t)t * k + r] = failed ? -1 : e;
    if (e / J == lane) {
      taken |= 1u << (e % J);
#pragma unroll
      for (int j = 0; j < J; ++j) pk[j] = j == e % J ? 0ull : pk[j];
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
  if (owner) {
    float v[J];
#pragma unroll
    for (int j = 0; j < J; ++j) v[j] = ((taken >> j) & 1u) ? num[j] * inv : 0.0f;
    store_bf16<J>(aff + (size_t)t * E + e0, v);
  }
  // a call whose wait gave up: the last select block to have read the failure
  // word counts the call, once, and clears the word (nothing of this runs
  // otherwise)
  if (failed && lane == 0) {
    const uint32_t seen =
        __hip_atomic_fetch_add(fail + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (seen == (uint32_t)T - 1u) {
      __hip_atomic_fetch_add(fail + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      st_dev(fail + 2, 0u);
      st_dev(fail, 0u);
    }
  }
}

int front_end_kchunk(int H) {
  // One of the compiled chunk lengths (MFMA steps of 32): the largest that
  // divides H into a multiple of 8 chunks (one group of blocks per XCD); else
  // the largest that divides H into at least 8 chunks; else 128 (H % 128 == 0).
  static constexpr int kChunks[] = {448, 384, 256, 128};
  for (int kc : kChunks)
    if (H % kc == 0 && (H / kc) % kXcds == 0) return kc;
  for (int kc : kChunks)
    if (H % kc == 0 && H / kc >= 8) return kc;
  return 128;
}

size_t front_end_workspace_bytes(int T, int H, int E) {
  const int nchunks = H / front_end_kchunk(H);
  return (size_t)kFrontEndSyncBytes + (size_t)nchunks * T * E * sizeof(float);
}

hipError_t launch_front_end(const FrontEndParams& q, hipStream_t s) {
  FeArgs a{};
  a.hidden = (const uint16_t*)q.hidden;
  a.gamma = (const uint16_t*)q.gamma;
  a.W = (const uint16_t*)q.W;
  a.rbias = (const uint16_t*)q.rbias;
  a.T = q.T;
  a.H = q.H;
  a.E = q.E;
  a.kc = front_end_kchunk(q.H);
  a.eps = q.eps;
  a.normed = (uint16_t*)q.normed;
  char* ws = static_cast<char*>(q.workspace);
  a.fail = reinterpret_cast<uint32_t*>(ws);
  a.rstd = reinterpret_cast<uint32_t*>(ws + kFailBytes);
  a.partial = reinterpret_cast<float*>(ws + kFrontEndSyncBytes);
  a.spin_limit = q.spin_limit;
  const int nchunks = q.H / a.kc;
  a.gemm_begin = (q.T + kXcds - 1) / kXcds * kXcds;   // keeps b % 8 for the XCD mapping
  a.gemm_blocks = ((q.E + 16 * kNS - 1) / (16 * kNS)) * ((q.T + kTileRows - 1) / kTileRows) * nchunks;
  const size_t lds = (size_t)(8 + a.kc + 16 * kNS * gemm_tile_stride(a.kc)) * sizeof(uint16_t);
  const dim3 grid1(a.gemm_begin + a.gemm_blocks);
#define MOE_NG(F, ST) hipLaunchKernelGGL((norm_gemm_kernel<F, ST>), grid1, dim3(kThreads), lds, s, a)
  switch (a.kc / 32) {
    case 14: if (q.f16) MOE_NG(true, 14); else MOE_NG(false, 14); break;
    case 12: if (q.f16) MOE_NG(true, 12); else MOE_NG(false, 12); break;
    case 8: if (q.f16) MOE_NG(true, 8); else MOE_NG(false, 8); break;
    default: if (q.f16) MOE_NG(true, 4); else MOE_NG(false, 4); break;
  }
#undef MOE_NG
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int J = (q.E + 63) / 64;                     // E <= 512
#define MOE_SELECT(F, JJ)                                                                     \
  hipLaunchKernelGGL((select_kernel<F, JJ>), dim3(q.T), dim3(64), 0, s, a.partial, nchunks,  \
                     a.rbias, q.T, q.E, q.k, q.act_sigmoid, a.rstd, a.fail, q.ids,         \
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
