// Host side of the C ABI declared in include/moe_route.h: argument validation,
// workspace sizing, kernel-shape selection and launches.  Validation runs
// before anything is enqueued; on error nothing is written.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "kernels.hpp"
#include "moe_route.h"

namespace moe {
LaunchStamp& launch_stamp() {
  static thread_local LaunchStamp st;
  return st;
}
}  // namespace moe

namespace {

thread_local char g_msg[512] = "";
thread_local int32_t g_hip_err = 0;

moe_status fail(moe_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof g_msg, fmt, ap);
  va_end(ap);
  return st;
}

moe_status hip_fail(hipError_t e, const char* what) {
  g_hip_err = (int32_t)e;
  return fail(MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

void clear_error() {
  g_msg[0] = '\0';
  g_hip_err = 0;
}

// ---- profiling aid: HIP events around each launch while enabled ------------------
struct ProfRecord {
  int kind;
  hipEvent_t start, stop;
};
struct Profiler {
  std::mutex mu;
  std::atomic<bool> on{false};
  std::vector<ProfRecord> pending;
  std::vector<hipEvent_t> pool;
  double total_ms[MOE_KERNEL_KINDS] = {};
  int64_t launches[MOE_KERNEL_KINDS] = {};
};
Profiler& profiler() {
  static Profiler* p = new Profiler();   // never destroyed: events may outlive exit order
  return *p;
}
hipEvent_t take_event(Profiler& P) {
  if (!P.pool.empty()) {
    hipEvent_t e = P.pool.back();
    P.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// While profiling is on, a launch group `f` is timed with two events: for a
// single kernel they are stamped by the dispatch itself (kernel start and
// end); a group of several kernels is bracketed by event records instead.
template <class F>
hipError_t launch_with_profile(int kind, hipStream_t stream, F&& f, bool single_kernel = true) {
  Profiler& P = profiler();
  if (!P.on.load(std::memory_order_relaxed)) return f();
  std::lock_guard<std::mutex> lk(P.mu);
  hipEvent_t a = take_event(P), b = take_event(P);
  if (a == nullptr || b == nullptr) return f();
  hipError_t e;
  if (single_kernel) {
    moe::LaunchStamp& st = moe::launch_stamp();
    st.start = a;
    st.stop = b;
    e = f();
    st = moe::LaunchStamp{};
    if (e != hipSuccess) return e;
  } else {
    e = hipEventRecord(a, stream);
    if (e != hipSuccess) return e;
    e = f();
    if (e != hipSuccess) return e;
    e = hipEventRecord(b, stream);
    if (e != hipSuccess) return e;
  }
  P.pending.push_back({kind, a, b});
  return hipSuccess;
}

bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }
int log2_exact(int v) {   // v a power of two
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}
int next_pow2(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}
size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

constexpr int kMaxExperts = 2048;
constexpr int kMaxTopK = 64;

bool grouping_on(const moe_route_args& a) {
  return a.n_group > 1 && a.topk_group > 0 && a.topk_group < a.n_group;
}

// Shape of the route kernel for one call: lanes per token and experts per lane.
struct Shape {
  int lpt = 0, epl = 0, lg = 1;
};

bool pick_shape(const moe_route_args& a, Shape* s) {
  const int E = a.num_experts;
  if (!grouping_on(a)) {
    // ungrouped: 32 experts per lane once rows are long enough, fewer lanes
    // per token for short rows so that a wavefront carries many tokens
    int epl = E <= 32 ? 8 : (E <= 64 ? 16 : 32);
    int lpt = next_pow2((E + epl - 1) / epl);
    if (lpt > 64) return false;
    s->lpt = lpt;
    s->epl = epl;
    s->lg = 1;
    return true;
  }
  const int gsz = E / a.n_group;
  for (int epl : {32, 16, 8, 4}) {
    if (gsz % epl) continue;
    const int lg = gsz / epl;
    const int lpt = next_pow2((E + epl - 1) / epl);
    if (!is_pow2(lg) || lg > lpt || lpt > 64) continue;
    s->lpt = lpt;
    s->epl = epl;
    s->lg = lg;
    return true;
  }
  return false;
}

moe_status validate_route(const moe_route_args* a, Shape* shape) {
  if (a == nullptr) return fail(MOE_EINVAL, "args is NULL");
  if (a->num_tokens < 0) return fail(MOE_EINVAL, "num_tokens < 0");
  if (a->num_experts < 1) return fail(MOE_EINVAL, "num_experts < 1");
  if (a->num_experts > kMaxExperts)
    return fail(MOE_EUNSUPPORTED, "num_experts > %d", kMaxExperts);
  if (a->top_k < 1 || a->top_k > a->num_experts)
    return fail(MOE_EINVAL, "top_k must be in [1, num_experts]");
  if (a->top_k > kMaxTopK) return fail(MOE_EUNSUPPORTED, "top_k > %d", kMaxTopK);
  if (a->score_fn != MOE_SOFTMAX && a->score_fn != MOE_SIGMOID)
    return fail(MOE_EINVAL, "score_fn must be MOE_SOFTMAX or MOE_SIGMOID");
  if (a->logits_dtype != MOE_F32 && a->logits_dtype != MOE_BF16)
    return fail(MOE_EINVAL, "logits_dtype must be MOE_F32 or MOE_BF16");
  if (a->bias_dtype != MOE_F32 && a->bias_dtype != MOE_BF16)
    return fail(MOE_EINVAL, "bias_dtype must be MOE_F32 or MOE_BF16");
  if (a->weights_dtype != MOE_F32 && a->weights_dtype != MOE_BF16)
    return fail(MOE_EINVAL, "weights_dtype must be MOE_F32 or MOE_BF16");
  if (!std::isfinite(a->routed_scaling_factor))
    return fail(MOE_EINVAL, "routed_scaling_factor is not finite");
  if (a->n_group < 0 || a->topk_group < 0) return fail(MOE_EINVAL, "negative group parameter");
  if (a->n_group > 1 && a->topk_group > a->n_group)
    return fail(MOE_EINVAL, "topk_group > n_group");
  if (grouping_on(*a)) {
    if (a->num_experts % a->n_group)
      return fail(MOE_EINVAL, "num_experts %% n_group != 0");
    const int gsz = a->num_experts / a->n_group;
    if (a->group_score_topn < 1 || a->group_score_topn > gsz)
      return fail(MOE_EINVAL, "group_score_topn must be in [1, E / n_group]");
    if (a->top_k > a->topk_group * gsz)
      return fail(MOE_EINVAL, "top_k exceeds the experts of the kept groups");
    if (a->group_score_topn > 2)
      return fail(MOE_EUNSUPPORTED, "group_score_topn > 2");
  }
  if (!pick_shape(*a, shape))
    return fail(MOE_EUNSUPPORTED,
                "no kernel shape for E=%d, n_group=%d: the group size must be a multiple of 4 "
                "whose lane count is a power of two",
                a->num_experts, a->n_group);
  return MOE_OK;
}

int num_blocks(int T) { return (T + moe::kTokensPerBlock - 1) / moe::kTokensPerBlock; }

// Routing workspace: [counting rows, two sets | their header][per-block
// counts].  The first region has a fixed size (two sets of kMaxSuperRows rows
// of up to kMaxExperts, a 256-byte header), so that it lies at the same place
// whatever the call's sizes; it must be zero before the first call and every
// call leaves it ready for the next (kernels.hpp: kCountSetInts).
static_assert(kMaxExperts == moe::kMaxCountExperts, "counting rows hold every expert");
constexpr size_t kCountRowsBytes = (size_t)moe::kCountSetInts * sizeof(int32_t);   // one set
constexpr size_t kCountRegionBytes = 2 * kCountRowsBytes + 256;   // two sets + their header
static_assert(kCountRegionBytes % 256 == 0, "the per-block counts follow 256-byte aligned");

struct CountPlan {
  int nb = 0, group_blocks = 1, num_super = 1;
  int sub_blocks = 1;   // route blocks per scatter block
};
// Route blocks per scatter block: every scatter block reads the counting rows
// (about 2 sqrt(nb) rows of E_loc counts) for its totals, so at large nb
// those reads dominate and one scatter block serves several route blocks.
// Limits: a scatter block's pairs fit the k_magic division (R k <= 64) and
// its LDS (two R E_loc arrays) stays within 64 KiB.
int scatter_sub_blocks(int nb, int k, int loc_n) {
  int r = nb >= 2048 ? 4 : (nb >= 1024 ? 2 : 1);
  while (r > 1 && ((int64_t)r * k > 64 || moe::scatter_lds_bytes(loc_n, r) > 64 * 1024)) r >>= 1;
  return r;
}
// sub_blocks > 1: the group size is a multiple of it, so that the route blocks
// of one scatter block share a counting group.
CountPlan count_plan(int T, int sub_blocks = 1) {
  CountPlan c;
  c.nb = num_blocks(T);
  c.sub_blocks = sub_blocks;
  int g = 1;
  while ((int64_t)g * g < c.nb) ++g;                 // ~sqrt(nb) blocks per row
  const int gmin = (c.nb + moe::kMaxSuperRows - 1) / moe::kMaxSuperRows;
  c.group_blocks = g > gmin ? g : gmin;
  if (c.group_blocks < 1) c.group_blocks = 1;
  c.group_blocks = (c.group_blocks + sub_blocks - 1) / sub_blocks * sub_blocks;
  c.num_super = (c.nb + c.group_blocks - 1) / c.group_blocks;
  return c;
}

size_t route_ws_bytes(const moe_route_args& a, int loc_n, bool permute) {
  return kCountRegionBytes +
         (permute ? align256((size_t)num_blocks(a.num_tokens) * loc_n * sizeof(int32_t)) : 0);
}
int32_t* ws_count_rows(void* ws) { return static_cast<int32_t*>(ws); }
// Polls before a front-end wait gives up.  MOE_ROUTE_FRONT_END_SPIN_LIMIT (an
// integer in [0, the default]) lowers it, read on every call: a limit of 0
// makes every wait give up at once, which exercises the give-up path (-1 ids,
// the failure count) with every kernel still ending normally.  Values outside
// [0, the default] leave the default.
int spin_limit_from_env(const char* name, int dflt) {
  const char* v = std::getenv(name);
  if (v == nullptr || *v == '\0') return dflt;
  char* end = nullptr;
  const long n = std::strtol(v, &end, 10);
  if (*end != '\0' || n < 0 || n > dflt) return dflt;
  return (int)n;
}
int front_end_spin_limit() {
  return spin_limit_from_env("MOE_ROUTE_FRONT_END_SPIN_LIMIT", moe::kFrontEndSpinLimit);
}
// The same for the aux-loss forward's final wait (MOE_ROUTE_AUX_SPIN_LIMIT):
// a limit of 0 makes the summing block give up at once (the loss is the
// timeout NaN; the workspace is left dirty).
int aux_spin_limit() { return spin_limit_from_env("MOE_ROUTE_AUX_SPIN_LIMIT", moe::kAuxSpinLimit); }

uint32_t* ws_count_hdr(void* ws) {
  return reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + 2 * kCountRowsBytes);
}
int32_t* ws_hist(void* ws) {
  return reinterpret_cast<int32_t*>(static_cast<char*>(ws) + kCountRegionBytes);
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Compute units of the current device (cached per device; 0 if unknown).
int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

moe::RouteParams make_params(const moe_route_args& a, const Shape& sh, const void* logits,
                             const void* bias, int32_t* ids, void* weights, float* scores,
                             int32_t* super_rows, uint32_t* count_hdr, int32_t* hist,
                             int group_blocks, int num_super, int loc_off, int loc_n) {
  moe::RouteParams p{};
  p.count_hdr = count_hdr;
  p.num_super = num_super;
  p.logits = logits;
  p.bias = bias;
  p.ids = ids;
  p.weights = weights;
  p.scores = scores;
  p.super_rows = super_rows;
  p.hist = hist;
  p.group_blocks = group_blocks;
  p.T = a.num_tokens;
  p.E = a.num_experts;
  p.k = a.top_k;
  p.variant = a.score_fn == MOE_SIGMOID
                  ? moe::kVarSigmoid
                  : (bias != nullptr ? moe::kVarSoftmaxBias : moe::kVarSoftmax);
  p.pre = a.score_fn == MOE_SOFTMAX && a.use_pre_softmax != 0;
  p.bias_bf16 = a.bias_dtype == MOE_BF16;
  p.weights_bf16 = a.weights_dtype == MOE_BF16;
  p.grouped = grouping_on(a);
  p.n_group = a.n_group;
  p.topk_group = a.topk_group;
  p.topn = a.group_score_topn;
  p.lg = sh.lg;
  p.lg_shift = log2_exact(sh.lg);
  p.renorm = a.renormalize != 0;
  p.scale = a.routed_scaling_factor;
  const size_t esz = a.logits_dtype == MOE_BF16 ? 2 : 4;
  p.vec = ((size_t)a.num_experts * esz) % 16 == 0 && aligned(logits, 16) &&
          (sh.epl * esz) % 16 == 0;
  p.bias_vec = bias != nullptr && aligned(bias, 16);
  p.scores_vec = scores != nullptr && aligned(scores, 16);
  p.loc_off = loc_off;
  p.loc_n = loc_n;
  p.hmask_len = super_rows != nullptr ? (loc_n + 1) & ~1 : 0;
  p.cap = a.top_k <= 32 ? 32 : 64;
  // sigmoid of bfloat16 logits with more blocks than one round on the device:
  // raw logits in the LDS row (half its size; two blocks fit a CU, so one
  // block's logit loads overlap the other's work)
  const int cus = device_cu_count();
  p.sig_raw = a.score_fn == MOE_SIGMOID && a.logits_dtype == MOE_BF16 && cus > 0 &&
              num_blocks(a.num_tokens) > cus;
  return p;
}

moe_status launch_route_checked(const moe::RouteParams& p, const Shape& sh, bool bf16,
                                hipStream_t stream) {
  const int rwpl =
      ((p.variant == moe::kVarSoftmax || p.sig_raw) && bf16) ? sh.epl / 2 : sh.epl;
  const size_t lds = moe::route_lds_bytes(sh.lpt, rwpl, sh.epl, p.hmask_len, p.cap, p.k,
                                          p.grouped ? p.n_group : 0) +
                     (p.fused ? (((size_t)p.loc_n + 1) * 4 + 32 + 15) & ~(size_t)15 : 0);
  if (lds > 160 * 1024)
    return fail(MOE_EUNSUPPORTED, "route kernel needs %zu bytes of LDS", lds);
  hipError_t e = launch_with_profile(MOE_KERNEL_ROUTE, stream, [&] {
    return moe::launch_route(p, sh.lpt, sh.epl, bf16, num_blocks(p.T), stream);
  });
  if (e != hipSuccess) return hip_fail(e, "route_kernel launch");
  return MOE_OK;
}

// Scratch of moe_route_permute: the caller's workspace.
struct CallerWorkspace {
  void* ptr;
  size_t bytes;
  moe_status get(size_t need, void** ws, hipStream_t) {
    if (ptr == nullptr || bytes < need) return fail(MOE_EWORKSPACE, "workspace needs %zu bytes", need);
    if (!aligned(ptr, 256)) return fail(MOE_EINVAL, "workspace must be 256-byte aligned");
    *ws = ptr;
    return MOE_OK;
  }
};

// Scratch of moe_route_permute_noalloc: a file-scope device array of fixed
// size, one instance on every device the library runs on.  Host code never
// uses the array's name as an address (on the host it is a stand-in symbol):
// the device address comes from hipGetSymbolAddress, taken once per device
// with that device current, and only that address is passed to kernels.
// Its counting region must be zero on entry to a call and every completed
// call leaves it zero; a zero-fill kernel runs before the first call on a
// device and after a call on it failed to launch (the region may then be
// dirty).  Every call on one device shares the array: calls that overlap on
// one device race.
constexpr size_t kScratchBytes = (size_t)8 << 20;
static_assert(kScratchBytes > kCountRegionBytes, "scratch holds the counting region");
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kScratchMaxDevices = 64;
struct ScratchState {
  std::mutex mu;
  void* ptr[kScratchMaxDevices] = {};
  bool dirty[kScratchMaxDevices] = {};
};
ScratchState& scratch_state() {
  static ScratchState* s = new ScratchState();
  return *s;
}

struct StaticScratch {
  int device = -1;
  moe_status get(size_t need, void** ws, hipStream_t stream) {
    if (need > kScratchBytes)
      return fail(MOE_EUNSUPPORTED,
                  "this call needs %zu bytes of scratch; moe_route_permute_noalloc holds %zu "
                  "(use moe_route_permute with a workspace)",
                  need, kScratchBytes);
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kScratchMaxDevices)
      return fail(MOE_EUNSUPPORTED, "device index %d >= %d", dev, kScratchMaxDevices);
    ScratchState& S = scratch_state();
    std::lock_guard<std::mutex> lk(S.mu);
    if (S.ptr[dev] == nullptr) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
      if (p == nullptr || !aligned(p, 256)) return fail(MOE_EHIP, "scratch address not aligned");
      S.ptr[dev] = p;
      S.dirty[dev] = true;
    }
    device = dev;
    if (S.dirty[dev]) {
      e = moe::launch_zero_fill(S.ptr[dev], kCountRegionBytes, stream);
      if (e != hipSuccess) return hip_fail(e, "scratch zero-fill launch");
      S.dirty[dev] = false;
    }
    *ws = S.ptr[dev];
    return MOE_OK;
  }
};

// moe_route_permute with its scratch from `wsp` (the caller's workspace or the
// library's static scratch), asked for only after every argument is validated.
template <class WS>
moe_status route_permute_impl(const moe_route_args* args, int32_t tile, int32_t loc_off,
                              int32_t loc_n, const void* logits, const void* bias,
                              int32_t* topk_ids, void* topk_weights, float* scores,
                              int32_t* expert_counts, int32_t* padded_offsets,
                              int32_t* total_num_padded_tokens, int32_t* num_non_exiting_ctas,
                              int32_t* e2p, int32_t* p2t, int32_t* batch_idx, int32_t* mn_limit,
                              WS& wsp, hipStream_t stream) {
  Shape sh;
  moe_status st = validate_route(args, &sh);
  if (st != MOE_OK) return st;
  const moe_route_args& a = *args;
  const int T = a.num_tokens, E = a.num_experts;
  if (!is_pow2(tile) || tile > 1024)
    return fail(MOE_EINVAL, "tile_tokens_dim must be a power of two in [1, 1024]");
  if (loc_off < 0 || loc_n < 1 || (int64_t)loc_off + loc_n > E)
    return fail(MOE_EINVAL, "local experts [off, off + n) must lie inside [0, E)");
  if (expert_counts == nullptr || padded_offsets == nullptr ||
      total_num_padded_tokens == nullptr || num_non_exiting_ctas == nullptr)
    return fail(MOE_EINVAL, "bookkeeping outputs are required");
  if ((int64_t)T * a.top_k + (int64_t)loc_n * (tile - 1) > INT32_MAX)
    return fail(MOE_EUNSUPPORTED, "padded token count exceeds int32");
  if (T == 0) {
    hipError_t e = moe::launch_empty_outputs(expert_counts, loc_n, padded_offsets,
                                             total_num_padded_tokens, num_non_exiting_ctas,
                                             stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "empty_outputs launch");
  }
  if (logits == nullptr || topk_ids == nullptr || topk_weights == nullptr || e2p == nullptr ||
      p2t == nullptr || batch_idx == nullptr || mn_limit == nullptr)
    return fail(MOE_EINVAL, "a required pointer is NULL");
  if (a.weights_dtype == MOE_F32 && !aligned(topk_weights, 4))
    return fail(MOE_EINVAL, "topk_weights must be 4-byte aligned");
  const size_t need = route_ws_bytes(a, loc_n, true);
  void* workspace = nullptr;
  st = wsp.get(need, &workspace, stream);
  if (st != MOE_OK) return st;
  const CountPlan cp = count_plan(T, scatter_sub_blocks(num_blocks(T), a.top_k, loc_n));
  int32_t* rows = ws_count_rows(workspace);
  int32_t* hist = ws_hist(workspace);

  if (cp.nb == 1) {
    // every token in one route block: the route kernel finishes the
    // permutation from its own bitmask (no counting rows, no second launch)
    moe::RouteParams p = make_params(a, sh, logits, bias, topk_ids, topk_weights, scores, nullptr,
                                     nullptr, nullptr, cp.group_blocks, cp.num_super, loc_off,
                                     loc_n);
    p.fused = 1;
    p.hmask_len = (loc_n + 1) & ~1;                     // the bitmask, without counting rows
    p.tile = tile;
    p.tile_shift = log2_exact(tile);
    p.e2p = e2p;
    p.p2t = p2t;
    p.counts = expert_counts;
    p.padded_offsets = padded_offsets;
    p.total_out = total_num_padded_tokens;
    p.nctas_out = num_non_exiting_ctas;
    p.batch_idx = batch_idx;
    p.mn_limit = mn_limit;
    return launch_route_checked(p, sh, a.logits_dtype == MOE_BF16, stream);
  }
  const moe::RouteParams p = make_params(a, sh, logits, bias, topk_ids, topk_weights, scores,
                                         rows, ws_count_hdr(workspace), hist, cp.group_blocks,
                                         cp.num_super, loc_off, loc_n);
  st = launch_route_checked(p, sh, a.logits_dtype == MOE_BF16, stream);
  if (st != MOE_OK) return st;

  moe::ScatterParams q{};
  q.ids = topk_ids;
  q.T = T;
  q.k = a.top_k;
  q.El = loc_n;
  q.off = loc_off;
  q.tile = tile;
  q.tile_shift = log2_exact(tile);
  q.k_magic = (uint32_t)(((1u << 20) + (uint32_t)a.top_k - 1u) / (uint32_t)a.top_k);
  q.super_rows = rows;
  q.hist = hist;
  q.count_hdr = ws_count_hdr(workspace);
  q.group_blocks = cp.group_blocks;
  q.num_super = cp.num_super;
  q.sub_blocks = cp.sub_blocks;
  q.route_blocks = cp.nb;
  q.counts = expert_counts;
  q.max_count = T * a.top_k;
  q.max_padded = (int)moe_max_padded_tokens(T, a.top_k, loc_n, tile);
  q.e2p = e2p;
  q.p2t = p2t;
  q.padded_offsets = padded_offsets;
  q.total_out = total_num_padded_tokens;
  q.nctas_out = num_non_exiting_ctas;
  q.batch_idx = batch_idx;
  q.mn_limit = mn_limit;
  hipError_t e = launch_with_profile(MOE_KERNEL_SCATTER, stream,
                                     [&] {
                                       return moe::launch_scatter(
                                           q, (cp.nb + cp.sub_blocks - 1) / cp.sub_blocks, stream);
                                     });
  if (e != hipSuccess) return hip_fail(e, "scatter_kernel launch");
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_EINVAL: return "MOE_EINVAL: invalid argument";
    case MOE_EUNSUPPORTED: return "MOE_EUNSUPPORTED: outside the implemented limits";
    case MOE_EWORKSPACE: return "MOE_EWORKSPACE: workspace too small";
    case MOE_EHIP: return "MOE_EHIP: HIP launch failed";
  }
  return "unknown moe_status";
}

const char* moe_last_error_message(void) { return g_msg; }

moe_status moe_profile_begin(void) {
  clear_error();
  Profiler& P = profiler();
  std::lock_guard<std::mutex> lk(P.mu);
  for (auto& r : P.pending) {
    P.pool.push_back(r.start);
    P.pool.push_back(r.stop);
  }
  P.pending.clear();
  for (int i = 0; i < MOE_KERNEL_KINDS; ++i) {
    P.total_ms[i] = 0.0;
    P.launches[i] = 0;
  }
  P.on.store(true);
  return MOE_OK;
}

moe_status moe_profile_end(void) {
  profiler().on.store(false);
  return MOE_OK;
}

moe_status moe_profile_read(int32_t kind, double* total_ms, int64_t* launches) {
  clear_error();
  if (kind < 0 || kind >= MOE_KERNEL_KINDS || total_ms == nullptr || launches == nullptr)
    return fail(MOE_EINVAL, "invalid kernel kind or NULL output");
  Profiler& P = profiler();
  std::lock_guard<std::mutex> lk(P.mu);
  std::vector<ProfRecord> keep;
  for (auto& r : P.pending) {
    if (r.kind != kind) {
      keep.push_back(r);
      continue;
    }
    hipError_t e = hipEventSynchronize(r.stop);
    float ms = 0.0f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess) return hip_fail(e, "profile event");
    P.total_ms[kind] += ms;
    P.launches[kind] += 1;
    P.pool.push_back(r.start);
    P.pool.push_back(r.stop);
  }
  P.pending.swap(keep);
  *total_ms = P.total_ms[kind];
  *launches = P.launches[kind];
  return MOE_OK;
}
int32_t moe_last_hip_error(void) { return g_hip_err; }

int64_t moe_max_padded_tokens(int32_t T, int32_t k, int32_t loc_n, int32_t tile) {
  if (T < 0 || k < 1 || loc_n < 1 || !is_pow2(tile)) return -1;
  return (int64_t)T * k + (int64_t)loc_n * (tile - 1);
}

int64_t moe_max_tiles(int32_t T, int32_t k, int32_t loc_n, int32_t tile) {
  const int64_t m = moe_max_padded_tokens(T, k, loc_n, tile);
  return m < 0 ? -1 : m / tile;
}

size_t moe_route_count_region_bytes(void) { return kCountRegionBytes; }

size_t moe_route_workspace_size(const moe_route_args* a, int32_t tile, int32_t loc_n) {
  (void)tile;
  if (a == nullptr || a->num_tokens < 0 || loc_n < 1) return 0;
  return route_ws_bytes(*a, loc_n, true);
}

moe_status moe_route(const moe_route_args* args, const void* logits, const void* bias,
                     int32_t* topk_ids, void* topk_weights, float* scores,
                     int32_t* expert_counts, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
  clear_error();
  Shape sh;
  moe_status st = validate_route(args, &sh);
  if (st != MOE_OK) return st;
  const moe_route_args& a = *args;
  const int T = a.num_tokens, E = a.num_experts;
  if (T == 0) {
    if (expert_counts == nullptr) return MOE_OK;
    hipError_t e = moe::launch_empty_outputs(expert_counts, E, nullptr, nullptr, nullptr, stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "empty_outputs launch");
  }
  if (logits == nullptr || topk_ids == nullptr || topk_weights == nullptr)
    return fail(MOE_EINVAL, "logits, topk_ids and topk_weights are required");
  if (a.weights_dtype == MOE_F32 && !aligned(topk_weights, 4))
    return fail(MOE_EINVAL, "topk_weights must be 4-byte aligned");
  int32_t* rows = nullptr;
  uint32_t* hdr = nullptr;
  const CountPlan cp = count_plan(T);
  if (expert_counts != nullptr) {
    const size_t need = route_ws_bytes(a, E, false);
    if (workspace == nullptr || workspace_bytes < need)
      return fail(MOE_EWORKSPACE, "workspace needs %zu bytes", need);
    if (!aligned(workspace, 256)) return fail(MOE_EINVAL, "workspace must be 256-byte aligned");
    rows = ws_count_rows(workspace);
    hdr = ws_count_hdr(workspace);
  }
  const moe::RouteParams p = make_params(a, sh, logits, bias, topk_ids, topk_weights, scores,
                                         rows, hdr, nullptr, cp.group_blocks, cp.num_super, 0, E);
  st = launch_route_checked(p, sh, a.logits_dtype == MOE_BF16, stream);
  if (st != MOE_OK) return st;
  if (rows != nullptr) {
    hipError_t e = launch_with_profile(MOE_KERNEL_COUNTS, stream, [&] {
      return moe::launch_counts(rows, hdr, cp.num_super, E, T * a.top_k, expert_counts, stream);
    });
    if (e != hipSuccess) return hip_fail(e, "counts_kernel launch");
  }
  return MOE_OK;
}

moe_status moe_route_permute(const moe_route_args* args, int32_t tile, int32_t loc_off,
                             int32_t loc_n, const void* logits, const void* bias,
                             int32_t* topk_ids, void* topk_weights, float* scores,
                             int32_t* expert_counts, int32_t* padded_offsets,
                             int32_t* total_num_padded_tokens, int32_t* num_non_exiting_ctas,
                             int32_t* e2p, int32_t* p2t, int32_t* batch_idx, int32_t* mn_limit,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  clear_error();
  CallerWorkspace ws{workspace, workspace_bytes};
  return route_permute_impl(args, tile, loc_off, loc_n, logits, bias, topk_ids, topk_weights,
                            scores, expert_counts, padded_offsets, total_num_padded_tokens,
                            num_non_exiting_ctas, e2p, p2t, batch_idx, mn_limit, ws, stream);
}

moe_status moe_route_permute_noalloc(const moe_route_args* args, int32_t tile, int32_t loc_off,
                                     int32_t loc_n, const void* logits, const void* bias,
                                     int32_t* topk_ids, void* topk_weights, float* scores,
                                     int32_t* expert_counts, int32_t* padded_offsets,
                                     int32_t* total_num_padded_tokens,
                                     int32_t* num_non_exiting_ctas, int32_t* e2p, int32_t* p2t,
                                     int32_t* batch_idx, int32_t* mn_limit, hipStream_t stream) {
  clear_error();
  StaticScratch ws;
  const moe_status st = route_permute_impl(
      args, tile, loc_off, loc_n, logits, bias, topk_ids, topk_weights, scores, expert_counts,
      padded_offsets, total_num_padded_tokens, num_non_exiting_ctas, e2p, p2t, batch_idx,
      mn_limit, ws, stream);
  if (st == MOE_EHIP && ws.device >= 0) scratch_state().dirty[ws.device] = true;
  return st;
}

size_t moe_route_permute_noalloc_max_scratch_bytes(void) { return kScratchBytes; }

size_t moe_aux_loss_workspace_size(int64_t rows, int32_t num_experts) {
  if (rows < 0 || num_experts < 1) return 0;
  return moe::kAuxSyncBytes;
}

size_t moe_aux_loss_sync_region_bytes(void) { return moe::kAuxSyncBytes; }

moe_status moe_aux_loss(const float* probs, const int32_t* tokens_per_expert, int64_t rows,
                        int64_t total_num_tokens, int32_t E, int32_t top_k, float coeff,
                        float* loss, const float* grad_loss, float* grad_probs, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  clear_error();
  if (rows < 0) return fail(MOE_EINVAL, "rows < 0");
  if (total_num_tokens < 1) return fail(MOE_EINVAL, "total_num_tokens < 1");
  if (E < 1) return fail(MOE_EINVAL, "num_experts < 1");
  if (E > 2048) return fail(MOE_EUNSUPPORTED, "num_experts > 2048");
  if (top_k < 1 || top_k > E) return fail(MOE_EINVAL, "top_k must be in [1, num_experts]");
  if (!std::isfinite(coeff)) return fail(MOE_EINVAL, "coeff is not finite");
  if (loss == nullptr && grad_probs == nullptr)
    return fail(MOE_EINVAL, "neither loss nor grad_probs requested");
  if (tokens_per_expert == nullptr) return fail(MOE_EINVAL, "tokens_per_expert is NULL");
  if (rows * (int64_t)E > ((int64_t)1 << 40)) return fail(MOE_EUNSUPPORTED, "probs too large");
  const double scale =
      (double)coeff * E / ((double)top_k * (double)total_num_tokens * (double)total_num_tokens);
  if (loss != nullptr) {
    if (rows > 0 && probs == nullptr) return fail(MOE_EINVAL, "probs is NULL");
    const size_t need = moe_aux_loss_workspace_size(rows, E);
    if (workspace == nullptr || workspace_bytes < need)
      return fail(MOE_EWORKSPACE, "workspace needs %zu bytes", need);
  }
  if (loss != nullptr) {
    const int nb = moe::aux_fwd_blocks(rows, E);
    hipError_t e = launch_with_profile(MOE_KERNEL_AUX_FWD, stream, [&] {
      return moe::launch_aux_fwd(probs, tokens_per_expert, rows, E, scale, workspace, nb, loss,
                                 aux_spin_limit(), stream);
    });
    if (e != hipSuccess) return hip_fail(e, "aux forward launch");
  }
  if (grad_probs != nullptr && rows > 0) {
    hipError_t e = launch_with_profile(MOE_KERNEL_AUX_BWD, stream, [&] {
      return moe::launch_aux_bwd(tokens_per_expert, rows, E, scale, grad_loss, grad_probs,
                                 stream);
    });
    if (e != hipSuccess) return hip_fail(e, "aux backward launch");
  }
  return MOE_OK;
}

moe_status moe_route_backward(const moe_route_args* args, const void* logits,
                              const int32_t* topk_ids, const float* grad_weights,
                              const float* grad_scores, float* grad_logits, hipStream_t stream) {
  clear_error();
  if (args == nullptr) return fail(MOE_EINVAL, "args is NULL");
  const moe_route_args& a = *args;
  if (a.num_tokens < 0) return fail(MOE_EINVAL, "num_tokens < 0");
  if (a.num_experts < 1) return fail(MOE_EINVAL, "num_experts < 1");
  if (a.num_experts > kMaxExperts) return fail(MOE_EUNSUPPORTED, "num_experts > %d", kMaxExperts);
  if (a.top_k < 1 || a.top_k > a.num_experts)
    return fail(MOE_EINVAL, "top_k must be in [1, num_experts]");
  if (a.top_k > kMaxTopK) return fail(MOE_EUNSUPPORTED, "top_k > %d", kMaxTopK);
  if (a.score_fn != MOE_SOFTMAX && a.score_fn != MOE_SIGMOID)
    return fail(MOE_EINVAL, "score_fn must be MOE_SOFTMAX or MOE_SIGMOID");
  if (a.logits_dtype != MOE_F32 && a.logits_dtype != MOE_BF16)
    return fail(MOE_EINVAL, "logits_dtype must be MOE_F32 or MOE_BF16");
  if (!std::isfinite(a.routed_scaling_factor))
    return fail(MOE_EINVAL, "routed_scaling_factor is not finite");
  if (grad_weights == nullptr && grad_scores == nullptr)
    return fail(MOE_EINVAL, "one of grad_weights / grad_scores is required");
  if (a.num_tokens == 0) return MOE_OK;
  if (logits == nullptr || grad_logits == nullptr)
    return fail(MOE_EINVAL, "logits and grad_logits are required");
  if (grad_weights != nullptr && topk_ids == nullptr)
    return fail(MOE_EINVAL, "topk_ids is required with grad_weights");
  const int esz = a.logits_dtype == MOE_BF16 ? 2 : 4;
  if (!aligned(logits, esz) || !aligned(grad_logits, 4) || !aligned(grad_scores, 4) ||
      !aligned(grad_weights, 4) || !aligned(topk_ids, 4))
    return fail(MOE_EINVAL, "misaligned pointer");
  moe::RouteBwdParams p{};
  p.logits = logits;
  p.ids = topk_ids;
  p.grad_weights = grad_weights;
  p.grad_scores = grad_scores;
  p.grad_logits = grad_logits;
  p.T = a.num_tokens;
  p.E = a.num_experts;
  p.k = a.top_k;
  p.mode = a.score_fn == MOE_SIGMOID ? moe::kBwdSigmoid
                                     : (a.use_pre_softmax ? moe::kBwdSoftmaxPre : moe::kBwdSoftmaxPost);
  p.renorm = a.renormalize != 0;
  p.scale = a.routed_scaling_factor;
  hipError_t e = launch_with_profile(MOE_KERNEL_ROUTE_BWD, stream, [&] {
    return moe::launch_route_backward(p, a.logits_dtype == MOE_BF16, stream);
  });
  if (e != hipSuccess) return hip_fail(e, "route_bwd_kernel launch");
  return MOE_OK;
}

moe_status moe_topk_to_dense(int32_t T, int32_t E, int32_t k, const int32_t* ids, const void* weights,
                             int32_t weights_dtype, float* probs, uint8_t* rmap, hipStream_t stream) {
  clear_error();
  if (T < 0 || E < 1) return fail(MOE_EINVAL, "T >= 0 and E >= 1");
  if (E > kMaxExperts) return fail(MOE_EUNSUPPORTED, "E > %d", kMaxExperts);
  if (k < 1 || k > E) return fail(MOE_EINVAL, "top_k must be in [1, E]");
  if (k > kMaxTopK) return fail(MOE_EUNSUPPORTED, "top_k > %d", kMaxTopK);
  if (weights_dtype != MOE_F32 && weights_dtype != MOE_BF16)
    return fail(MOE_EINVAL, "weights_dtype must be MOE_F32 or MOE_BF16");
  if (probs == nullptr && rmap == nullptr) return fail(MOE_EINVAL, "one of probs / routing_map is required");
  if (T == 0) return MOE_OK;
  if (ids == nullptr || weights == nullptr) return fail(MOE_EINVAL, "topk_ids and topk_weights are required");
  if (!aligned(ids, 4) || !aligned(probs, 4) || !aligned(weights, weights_dtype == MOE_BF16 ? 2 : 4))
    return fail(MOE_EINVAL, "misaligned pointer");
  hipError_t e = launch_with_profile(MOE_KERNEL_DENSE, stream, [&] {
    return moe::launch_dense(T, E, k, ids, weights, weights_dtype == MOE_BF16, probs, rmap, stream);
  });
  if (e != hipSuccess) return hip_fail(e, "dense_kernel launch");
  return MOE_OK;
}

moe_status moe_dispatch(const void* hidden, int32_t dtype, int32_t T, int32_t H,
                        const int32_t* p2t, const int32_t* total, int64_t max_padded, void* out,
                        hipStream_t stream) {
  clear_error();
  if (dtype != MOE_F32 && dtype != MOE_BF16) return fail(MOE_EINVAL, "dtype must be MOE_F32 or MOE_BF16");
  if (T < 0 || H < 1 || max_padded < 0) return fail(MOE_EINVAL, "T >= 0, H >= 1, max_padded_tokens >= 0");
  if (T == 0 || max_padded == 0) return MOE_OK;
  if (hidden == nullptr || p2t == nullptr || total == nullptr || out == nullptr)
    return fail(MOE_EINVAL, "a required pointer is NULL");
  const int esz = dtype == MOE_BF16 ? 2 : 4;
  if (!aligned(hidden, esz) || !aligned(out, esz) || !aligned(p2t, 4) || !aligned(total, 4))
    return fail(MOE_EINVAL, "misaligned pointer");
  hipError_t e = launch_with_profile(MOE_KERNEL_DISPATCH, stream, [&] {
    return moe::launch_dispatch(hidden, (int64_t)H * esz, p2t, total, max_padded, out, stream);
  });
  if (e != hipSuccess) return hip_fail(e, "dispatch_kernel launch");
  return MOE_OK;
}

moe_status moe_combine(const void* expert_out, int32_t dtype, int32_t T, int32_t H, int32_t top_k,
                       const int32_t* e2p, const void* weights, int32_t weights_dtype, void* out,
                       hipStream_t stream) {
  clear_error();
  if (dtype != MOE_F32 && dtype != MOE_BF16) return fail(MOE_EINVAL, "dtype must be MOE_F32 or MOE_BF16");
  if (weights_dtype != MOE_F32 && weights_dtype != MOE_BF16)
    return fail(MOE_EINVAL, "weights_dtype must be MOE_F32 or MOE_BF16");
  if (T < 0 || H < 1) return fail(MOE_EINVAL, "T >= 0 and H >= 1");
  if (top_k < 1) return fail(MOE_EINVAL, "top_k >= 1");
  if (top_k > kMaxTopK) return fail(MOE_EUNSUPPORTED, "top_k > %d", kMaxTopK);
  if (T == 0) return MOE_OK;
  if (expert_out == nullptr || e2p == nullptr || weights == nullptr || out == nullptr)
    return fail(MOE_EINVAL, "a required pointer is NULL");
  const int esz = dtype == MOE_BF16 ? 2 : 4;
  if (!aligned(expert_out, esz) || !aligned(out, esz) || !aligned(e2p, 4) ||
      !aligned(weights, weights_dtype == MOE_BF16 ? 2 : 4))
    return fail(MOE_EINVAL, "misaligned pointer");
  hipError_t e = launch_with_profile(MOE_KERNEL_COMBINE, stream, [&] {
    return moe::launch_combine(expert_out, dtype == MOE_BF16, T, H, top_k, e2p, weights,
                               weights_dtype == MOE_BF16, out, stream);
  });
  if (e != hipSuccess) return hip_fail(e, "combine_kernel launch");
  return MOE_OK;
}

size_t rmsnorm_gate_route_workspace_size(int32_t T, int32_t H, int32_t E) {
  if (T < 1 || H < 128 || H % 128 || E < 1) return 0;
  return align256(moe::front_end_workspace_bytes(T, H, E));
}

size_t rmsnorm_gate_route_sync_region_bytes(void) { return moe::kFrontEndSyncBytes; }

int32_t rmsnorm_gate_route_sum_depth(int32_t H) {
  if (H < 128 || H % 128 || H > 16384) return -1;
  const int kc = moe::front_end_kchunk(H);
  return kc / 32 + H / kc + 32 + 1;
}

moe_status rmsnorm_gate_route(const void* hidden, const void* gamma, const void* router_weights,
                              const void* router_bias, int32_t dtype, int32_t T, int32_t H,
                              int32_t E, float eps, int32_t top_k, int32_t act_fn, void* normed,
                              int32_t* topk_ids, void* affinities, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  clear_error();
  if (dtype != MOE_BF16 && dtype != MOE_F16) return fail(MOE_EINVAL, "dtype must be MOE_BF16 or MOE_F16");
  if (T < 1) return fail(MOE_EINVAL, "T must be >= 1");
  if (T > 128) return fail(MOE_EINVAL, "T must be <= 128 (single-tile decode front end)");
  if (H < 128 || H % 128) return fail(MOE_EINVAL, "H must be a positive multiple of 128");
  if (H > 16384) return fail(MOE_EUNSUPPORTED, "H > 16384");
  if (E < 1) return fail(MOE_EINVAL, "E must be >= 1");
  if (E % 16 || E > 512) return fail(MOE_EUNSUPPORTED, "E must be a multiple of 16, at most 512");
  if (top_k < 1 || top_k > E) return fail(MOE_EINVAL, "top_k must be in [1, E]");
  if (top_k > 64) return fail(MOE_EUNSUPPORTED, "top_k > 64");
  if (act_fn != MOE_SOFTMAX && act_fn != MOE_SIGMOID) return fail(MOE_EINVAL, "act_fn must be MOE_SOFTMAX or MOE_SIGMOID");
  if (!std::isfinite(eps) || eps < 0.0f) return fail(MOE_EINVAL, "eps must be finite and >= 0");
  if (hidden == nullptr || gamma == nullptr || router_weights == nullptr || normed == nullptr ||
      topk_ids == nullptr || affinities == nullptr)
    return fail(MOE_EINVAL, "a required pointer is NULL");
  if (!aligned(hidden, 16) || !aligned(gamma, 16) || !aligned(router_weights, 16) ||
      !aligned(normed, 16) || !aligned(affinities, 2) || (router_bias && !aligned(router_bias, 2)))
    return fail(MOE_EINVAL, "hidden, gamma, router_weights and normed must be 16-byte aligned");
  const size_t need = rmsnorm_gate_route_workspace_size(T, H, E);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(MOE_EWORKSPACE, "workspace needs %zu bytes", need);
  if (!aligned(workspace, 256)) return fail(MOE_EINVAL, "workspace must be 256-byte aligned");
  moe::FrontEndParams q{};
  q.hidden = hidden;
  q.gamma = gamma;
  q.W = router_weights;
  q.rbias = router_bias;
  q.f16 = dtype == MOE_F16;
  q.T = T;
  q.H = H;
  q.E = E;
  q.k = top_k;
  q.eps = eps;
  q.act_sigmoid = act_fn == MOE_SIGMOID;
  q.normed = normed;
  q.ids = topk_ids;
  q.aff = affinities;
  q.workspace = workspace;
  q.spin_limit = front_end_spin_limit();
  hipError_t e = launch_with_profile(
      MOE_KERNEL_FRONT_END, stream, [&] { return moe::launch_front_end(q, stream); },
      /*single_kernel=*/false);
  if (e != hipSuccess) return hip_fail(e, "front end launch");
  return MOE_OK;
}

}  // extern "C"
