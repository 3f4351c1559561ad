// Host side of the C ABI declared in include/moe.h: plan creation and
// validation, workspace layout, the launch sequence of one forward call, the
// readers of routing / intermediate buffers, and optional per-stage timing.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <cstdlib>
#include <mutex>
#include <new>
#include <vector>

#include "kernels.h"
#include "moe.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxTopK = 16;
constexpr int kMaxExperts = 1024;
// Decode-sized batches (mean tokens per routed expert at most this) take the
// weight-streaming kernels under MOE_PATH_AUTO.  At the GLM-5 shape the streaming
// path is faster up to 128 tokens (4 per expert) and the MFMA path from 192 (6).
constexpr int kStreamMaxMeanTokens = 5;
// Split-K target: enough blocks for two per compute unit on 256 CUs.
constexpr int kTargetBlocks = 512;
constexpr int kComputeUnits = 256;  // MI355X
// Partial sums the router top-k and the shared-expert consumers add per value.
constexpr int kMaxRouterSplits = 16;
constexpr int kMaxSharedSplits = 16;

enum Stage {
  kStNorm = 0,
  kStRouter,
  kStTopk,
  kStScan,
  kStScatter,
  kStGateUp,
  kStSharedGateUp,
  kStSharedAct,
  kStDown,
  kStSharedDown,
  kStCombine,
  kStFused,  // the whole forward in the fused decode kernel
  kNumStages
};
const char* const kStageNames[kNumStages] = {
    "rmsnorm",       "router_logits",   "router_topk", "permute_scan", "permute_scatter",
    "expert_gate_up", "shared_gate_up", "shared_act",  "expert_down",  "shared_down",
    "combine",        "fused_decode"};
// Largest batch the fused decode kernel takes.
constexpr int64_t kFusedMaxTokens = 64;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Split {
  int splits;
  int kt_per;
};

// Split-K factor for a dense K-contiguous product of M rows, N columns, K depth:
// at least two K tiles per split and at most max_splits partial sums for the
// consumer to add.  The 128-row kernel asks for about kTargetBlocks blocks.  The
// 256-row kernel holds a compute unit alone: with fewer tiles than compute
// units it splits K to fill one wave of them.  With more it splits only a deep
// product (K of 128 tiles or more) whose last wave would be at most half full, in
// two: the partial sums cost HBM traffic twice, in the product and in its
// consumer.  (A 384-tile product split in two fills its last wave: at K = 12288,
// the dense block's down product at 4096 tokens, the block is 1.7 % faster; at
// K = 2048, the MoE block's shared down product, the step is slower.)
// The 64-row kernel, one block per compute unit too and bound by its weight
// stream, takes the split count with the fewest K-steps on the busiest of `cus`
// compute units, a split's partial sums (M x 128 fp32 per tile, written and read
// again) counting as 4M / 64 K-steps of weight traffic spread over all of them.
Split nt_split(int64_t M, int64_t N, int64_t K, int tm, int tn, int tk, int max_splits,
               int cus = kComputeUnits) {
  const int64_t tiles = std::max<int64_t>(1, cdiv(M, tm) * cdiv(N, tn));
  const int64_t nkt = K / tk;
  const int64_t smax = std::max<int64_t>(1, std::min<int64_t>(max_splits, nkt / 2));
  int64_t s = 1;
  if (tm == kNtBigTile) {
    if (tiles < kComputeUnits)
      s = std::min<int64_t>(smax, cdiv(kComputeUnits, tiles));
    else if (nkt >= 128 && tiles % kComputeUnits != 0 &&
             tiles % kComputeUnits <= kComputeUnits / 2)
      s = std::min<int64_t>(smax, 2);
  } else if (tm == kNtSkinnyRows) {
    double best = 0.0;
    for (int64_t c = 1; c <= smax; ++c) {
      const double est = (double)cdiv(tiles * c, cus) * (double)cdiv(nkt, c) +
                         4.0 * (double)std::min<int64_t>(M, tm) / tk * (double)(tiles * c) /
                             cus;
      if (c == 1 || est < best) {
        best = est;
        s = c;
      }
    }
  } else {
    s = std::min<int64_t>(smax, std::max<int64_t>(1, cdiv(kTargetBlocks, tiles)));
  }
  const int64_t per = cdiv(nkt, s);
  return Split{(int)cdiv(nkt, per), (int)per};
}

struct Layout {
  size_t h, logits, topk_idx, topk_w, chunk_cnt, counts, offsets, hdr, active, mtiles,
      perm_token, row_of, pass_base, s_parts, act, y, sh_gu, act_s, sh_dn, sync,
      total;
  // bytes of the split-K partial-sum regions (router logits, shared gate/up, shared down)
  size_t logits_bytes, sh_gu_bytes, sh_dn_bytes;
};

struct EventPair {
  int stage;
  hipEvent_t a, b;
};

}  // namespace

// Side stream of the shared expert on one device, with the fork and join events.
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kMaxSideDevices = 64;

struct moe_plan {
  moe_config_t cfg;
  size_t es;  // bytes per element of D
  Layout lay;
  // stage timing: events are made by moe_set_stage_timing, never by a forward call
  std::mutex tmu;
  int32_t timing_mask = 0;
  int64_t timed_calls = 0;
  std::vector<EventPair> pending;
  std::vector<hipEvent_t> pool;
  // shared-expert side stream of the device current at plan creation (made there,
  // never by a forward call); smu is held from a call's fork until its join is
  // enqueued
  std::mutex smu;
  SideStream side[kMaxSideDevices];
};

namespace {

bool use_mfma(const moe_plan* p, int64_t T, int k) {
  if (p->cfg.dtype != MOE_DTYPE_BF16) return false;
  if (p->cfg.path == MOE_PATH_STREAM || p->cfg.path == MOE_PATH_FUSED) return false;
  if (p->cfg.path == MOE_PATH_MFMA) return true;
  return T * k > (int64_t)kStreamMaxMeanTokens * p->cfg.n_experts;
}

// The fused decode kernel: bf16 MoE plans under MOE_PATH_FUSED, for calls of at
// most kFusedMaxTokens tokens (larger calls of such a plan take the streaming
// kernels).  AUTO does not pick it: its grid barriers cost more than the launch
// gaps of the multi-kernel path at every decode batch size measured.
bool use_fused(const moe_plan* p, int64_t T, int k) {
  (void)k;
  return p->cfg.path == MOE_PATH_FUSED && p->cfg.dtype == MOE_DTYPE_BF16 &&
         p->cfg.n_experts > 0 && T <= kFusedMaxTokens;
}

// Compute units the shared expert's 64-row products are sized for when they run on
// the side stream beside the routing steps: a quarter of the chip, so that the
// routing kernels (one to a few blocks each, on the critical path) find free
// compute units at once instead of waiting for a wave of the shared expert's
// blocks (GLM-5 decode: 1 token 0.169 -> 0.159 ms, 2 tokens 0.250 -> 0.241 ms;
// with half the chip 0.161 ms, with an eighth 0.172 ms).
constexpr int kSideCUs = kComputeUnits / 4;

// Compute units the shared expert's split-K is chosen for in a call of T tokens
// and top-k k: kSideCUs when the call forks it onto the side stream (streaming
// kernels), else the whole chip.
int shared_cus(const moe_plan* p, int64_t T, int k) {
  return p->cfg.n_experts > 0 && p->cfg.shared_inter > 0 && !use_mfma(p, T, k) &&
                 !use_fused(p, T, k)
             ? kSideCUs
             : kComputeUnits;
}

// Tile sizes of the dense K-contiguous products of T rows for this plan's dtype.
void nt_tiles(const moe_plan* p, int64_t T, int* tm, int* tn, int* tk) {
  if (p->cfg.dtype == MOE_DTYPE_BF16) {
    mfma_nt_tile(T, tm, tn, tk);
  } else {
    *tm = *tn = *tk = kFmaTile;
  }
}

// Largest split-K partial buffer (in fp32 elements) over every T <= Tmax.  The
// 64-row kernel's split count depends on the row count itself (its estimate
// counts the partial sums' traffic, 4 min(M, 64) / 64 K-steps per split), and not
// monotonically, so every T up to kExactRows is evaluated.  From there on the
// split count depends only on the tile count, which is constant between
// multiples of the row tile (128 or 256 rows), where the buffer is largest: the
// multiples of 32 and Tmax itself cover the rest.
// For the shared expert's products (shared = true) both compute-unit counts of
// shared_cus are evaluated.
constexpr int64_t kExactRows = 512;
size_t max_partial_elems(const moe_plan* p, int64_t Tmax, int64_t N, int64_t K, int max_splits,
                         bool shared) {
  size_t best = 0;
  const int64_t top = std::max<int64_t>(Tmax, 1);
  auto at = [&](int64_t T) {
    int tm, tn, tk;
    nt_tiles(p, T, &tm, &tn, &tk);
    for (int cus : {kComputeUnits, kSideCUs}) {
      if (cus != kComputeUnits && !shared) break;
      const Split s = nt_split(T, N, K, tm, tn, tk, max_splits, cus);
      best = std::max(best, (size_t)s.splits * (size_t)T * (size_t)N);
    }
  };
  for (int64_t T = 1; T <= std::min(top, kExactRows); ++T) at(T);
  for (int64_t T = kExactRows + 32; T < top; T += 32) at(T);
  at(top);
  return best;
}

void make_layout(moe_plan* p) {
  const moe_config_t& c = p->cfg;
  const int64_t T = std::max<int64_t>(c.max_tokens, 1);
  const int64_t A = T * c.max_top_k;
  const int64_t nch = cdiv(T, kChunkTokens);
  const size_t es = p->es;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(std::max<size_t>(bytes, 1));
    return at;
  };
  Layout& L = p->lay;
  L.h = take((size_t)T * c.dim * es);
  L.logits_bytes = max_partial_elems(p, T, c.n_experts, c.dim, kMaxRouterSplits, false) * 4;
  L.logits = take(L.logits_bytes);
  L.topk_idx = take((size_t)A * 4);
  L.topk_w = take((size_t)A * 4);
  L.chunk_cnt = take((size_t)nch * c.n_experts * 4);
  L.counts = take((size_t)c.n_experts * 4);
  L.offsets = take((size_t)(c.n_experts + 1) * 4);
  L.hdr = take(sizeof(RouteHeader));
  L.active = take((size_t)c.n_experts * 4);
  L.mtiles = take((size_t)(cdiv(A, kGroupBM) + std::min<int64_t>(c.n_experts, A)) * sizeof(int2));
  L.perm_token = take((size_t)A * 4);
  L.row_of = take((size_t)A * 4);
  L.pass_base = take((size_t)(c.n_experts + 1) * 4);
  L.s_parts = c.n_experts > 0 && c.path != MOE_PATH_MFMA
                  ? take((size_t)kStreamMaxBlocks * 2 *
                         stream_slot_floats(c.dtype == MOE_DTYPE_BF16 ? kBF16 : kF32,
                                            c.moe_inter, c.dim) * 4)
                  : 0;
  L.act = take((size_t)A * c.moe_inter * es);
  L.y = take((size_t)A * c.dim * es);
  if (c.shared_inter > 0) {
    L.sh_gu_bytes =
        max_partial_elems(p, T, 2 * (int64_t)c.shared_inter, c.dim, kMaxSharedSplits, true) * 4;
    L.sh_gu = take(L.sh_gu_bytes);
    L.act_s = take((size_t)T * c.shared_inter * es);
    L.sh_dn_bytes = max_partial_elems(p, T, c.dim, c.shared_inter, kMaxSharedSplits, true) * 4;
    L.sh_dn = take(L.sh_dn_bytes);
  } else {
    L.sh_gu = L.act_s = L.sh_dn = 0;
    L.sh_gu_bytes = L.sh_dn_bytes = 0;
  }
  L.sync = take((size_t)kFusedSyncWords * 4);
  L.total = off;
}

// The split-K partial sums a call of T rows writes fit the regions the plan sized
// for max_tokens (WORKSPACE_TOO_SMALL otherwise; checked before anything is
// enqueued, so a sizing mistake can never write past a region).
moe_status_t check_splits(const moe_plan* p, int64_t T, int k) {
  const moe_config_t& c = p->cfg;
  if (T <= 0) return MOE_SUCCESS;
  int tm, tn, tk;
  nt_tiles(p, T, &tm, &tn, &tk);
  const int scus = shared_cus(p, T, k);
  auto fits = [&](int64_t N, int64_t K, int max_splits, size_t bytes, int cus) {
    const Split s = nt_split(T, N, K, tm, tn, tk, max_splits, cus);
    return (size_t)s.splits * (size_t)T * (size_t)N * 4 <= bytes;
  };
  if (c.n_experts > 0 &&
      !fits(c.n_experts, c.dim, kMaxRouterSplits, p->lay.logits_bytes, kComputeUnits))
    return MOE_ERROR_WORKSPACE_TOO_SMALL;
  if (c.shared_inter > 0 &&
      (!fits(2 * (int64_t)c.shared_inter, c.dim, kMaxSharedSplits, p->lay.sh_gu_bytes, scus) ||
       !fits(c.dim, c.shared_inter, kMaxSharedSplits, p->lay.sh_dn_bytes, scus)))
    return MOE_ERROR_WORKSPACE_TOO_SMALL;
  return MOE_SUCCESS;
}

bool misaligned(const void* ptr) { return ((uintptr_t)ptr & 15u) != 0; }

// MOE_DEBUG_SYNC=1 in the environment (read at every forward call): each stage is
// followed by a synchronisation of its stream, so that a kernel that fails is
// reported by the call that launched it, as MOE_ERROR_HIP.  Debug only: it
// serialises the forward, and a stream under graph capture cannot be synchronised.
bool debug_sync() {
  const char* v = getenv("MOE_DEBUG_SYNC");
  return v && v[0] == '1' && v[1] == 0;
}

// Calls whose selected stages the event pool made by moe_set_stage_timing covers
// (two events per stage and call); a call made while the pool is short is not
// timed and not counted.
constexpr int kTimedCallsMax = 128;

int popcount32(uint32_t v) { return __builtin_popcount(v); }

hipEvent_t get_event(moe_plan* p) {
  if (p->pool.empty()) return nullptr;
  hipEvent_t e = p->pool.back();
  p->pool.pop_back();
  return e;
}

// Stage timing of one forward call: returns the selected stages, with the timing
// state locked until the call returns, or 0 (unlocked) when timing is off or the
// event pool cannot cover every selected stage of the call.
int32_t begin_timing(moe_plan* p, std::unique_lock<std::mutex>& lk) {
  lk = std::unique_lock<std::mutex>(p->tmu);
  const int32_t m = p->timing_mask;
  if (m == 0 || p->pool.size() < (size_t)2 * popcount32((uint32_t)m)) {
    lk.unlock();
    return 0;
  }
  ++p->timed_calls;
  return m;
}

// Makes the side stream (non-blocking, at the default priority) and its fork and
// join events on the current device.  Failure (no device) leaves none: calls then
// run the shared expert in order on their own stream.
void make_side_stream(moe_plan* p) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxSideDevices) return;
  SideStream& sd = p->side[dev];
  hipStream_t st = nullptr;
  hipEvent_t f = nullptr, j = nullptr;
  if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess) return;
  if (hipEventCreateWithFlags(&f, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&j, hipEventDisableTiming) != hipSuccess) {
    if (f) (void)hipEventDestroy(f);
    (void)hipStreamDestroy(st);
    return;
  }
  sd.stream = st, sd.fork = f, sd.join = j;
}

// The side stream of the current device, or nullptr when the plan has none there.
SideStream* side_stream(moe_plan* p) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxSideDevices) return nullptr;
  SideStream& sd = p->side[dev];
  return sd.stream ? &sd : nullptr;
}

}  // namespace

// Workspace of moe_block_forward_static: one static buffer in every GPU's memory,
// held from the library's load on that GPU until the process ends.  In host code
// `scratch` only names a host-side stand-in; kernels get the device address that
// hipGetSymbolAddress returns for the current device (static_workspace below).
static __device__ __align__(256) unsigned char scratch[MOE_STATIC_WORKSPACE_BYTES];

namespace {

std::mutex g_scratch_mu;
void* g_scratch[kMaxSideDevices];  // device address of `scratch` per device, once resolved

// Device address of `scratch` on the current device, resolved once per device
// (with that device current) and kept.
hipError_t static_workspace(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxSideDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress((void**)&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_SUCCESS: return "success";
    case MOE_ERROR_INVALID_VALUE: return "invalid value";
    case MOE_ERROR_NOT_SUPPORTED: return "not supported";
    case MOE_ERROR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_ERROR_MISALIGNED: return "pointer not 16-byte aligned";
    case MOE_ERROR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* moe_stage_name(int32_t stage) {
  if (stage < 0 || stage >= kNumStages) return nullptr;
  return kStageNames[stage];
}

moe_status_t moe_plan_create(const moe_config_t* cfg, moe_plan_t* plan, size_t* workspace_bytes) {
  if (!cfg || !plan || !workspace_bytes) return MOE_ERROR_INVALID_VALUE;
  *plan = nullptr;
  if (cfg->struct_size != sizeof(moe_config_t)) return MOE_ERROR_INVALID_VALUE;
  // n_experts == 0: a dense block (its MLP is the shared_inter-wide SwiGLU; no router)
  const bool dense = cfg->n_experts == 0;
  if (cfg->dim <= 0 || cfg->n_experts < 0 || cfg->shared_inter < 0 || cfg->max_tokens < 0 ||
      !(cfg->eps > 0.0f) || !isfinite(cfg->eps) || cfg->flags != 0)
    return MOE_ERROR_INVALID_VALUE;
  if (dense ? (cfg->moe_inter != 0 || cfg->max_top_k != 0 || cfg->shared_inter == 0)
            : (cfg->moe_inter <= 0 || cfg->max_top_k < 1 || cfg->max_top_k > cfg->n_experts))
    return MOE_ERROR_INVALID_VALUE;
  if (cfg->dtype != MOE_DTYPE_F32 && cfg->dtype != MOE_DTYPE_BF16) return MOE_ERROR_NOT_SUPPORTED;
  if (cfg->path < MOE_PATH_AUTO || cfg->path > MOE_PATH_FUSED) return MOE_ERROR_INVALID_VALUE;
  if ((cfg->path == MOE_PATH_MFMA || cfg->path == MOE_PATH_FUSED) && cfg->dtype != MOE_DTYPE_BF16)
    return MOE_ERROR_NOT_SUPPORTED;
  if (cfg->dim % 64 || cfg->moe_inter % 64 || cfg->shared_inter % 64 ||
      cfg->n_experts > kMaxExperts || cfg->max_top_k > kMaxTopK)
    return MOE_ERROR_NOT_SUPPORTED;
  // 32-bit row indices inside the kernels
  if (cfg->max_tokens > (int64_t)1 << 26 || (int64_t)cfg->max_tokens * cfg->max_top_k >= INT32_MAX)
    return MOE_ERROR_NOT_SUPPORTED;
  moe_plan* p = new (std::nothrow) moe_plan();
  if (!p) return MOE_ERROR_INVALID_VALUE;
  p->cfg = *cfg;
  p->es = cfg->dtype == MOE_DTYPE_BF16 ? 2 : 4;
  make_layout(p);
  // the streaming path runs the shared expert on a side stream
  if (!dense && cfg->shared_inter > 0 && cfg->path != MOE_PATH_MFMA) make_side_stream(p);
  // set-up of moe_block_forward_static on this device, so that its calls (under graph
  // capture, say) do no more than look the address up; without a device this fails
  // and the entry point retries on its first call
  if (!dense) {
    void* unused = nullptr;
    if (static_workspace(&unused) != hipSuccess) (void)hipGetLastError();
  }
  *plan = p;
  *workspace_bytes = p->lay.total;
  return MOE_SUCCESS;
}

moe_status_t moe_plan_destroy(moe_plan_t p) {
  if (!p) return MOE_SUCCESS;
  for (auto& ev : p->pending) {
    (void)hipEventDestroy(ev.a);
    (void)hipEventDestroy(ev.b);
  }
  for (auto e : p->pool) (void)hipEventDestroy(e);
  for (auto& sd : p->side) {
    if (sd.fork) (void)hipEventDestroy(sd.fork);
    if (sd.join) (void)hipEventDestroy(sd.join);
    if (sd.stream) (void)hipStreamDestroy(sd.stream);
  }
  delete p;
  return MOE_SUCCESS;
}

int32_t moe_plan_path(moe_plan_t p, int64_t num_tokens, int32_t top_k) {
  if (!p) return -1;
  if (p->cfg.n_experts == 0)  // dense plan: the family of its K-contiguous products
    return p->cfg.dtype == MOE_DTYPE_BF16 ? MOE_PATH_MFMA : MOE_PATH_STREAM;
  if (use_fused(p, num_tokens, top_k)) return MOE_PATH_FUSED;
  return use_mfma(p, num_tokens, top_k) ? MOE_PATH_MFMA : MOE_PATH_STREAM;
}

moe_status_t moe_plan_check(moe_plan_t p, int64_t T, int32_t k) {
  if (!p) return MOE_ERROR_INVALID_VALUE;
  const moe_config_t& c = p->cfg;
  if (T < 0 || T > c.max_tokens) return MOE_ERROR_INVALID_VALUE;
  if (c.n_experts == 0 ? k != 0 : (k < 1 || k > c.max_top_k || k > c.n_experts))
    return MOE_ERROR_INVALID_VALUE;
  return check_splits(p, T, k);
}

moe_status_t moe_set_stage_timing(moe_plan_t p, int32_t stage_mask) {
  if (!p || stage_mask < 0 || stage_mask >= (1 << kNumStages)) return MOE_ERROR_INVALID_VALUE;
  std::lock_guard<std::mutex> g(p->tmu);
  // events for kTimedCallsMax calls, beside those still pending
  const size_t want = (size_t)2 * popcount32((uint32_t)stage_mask) * kTimedCallsMax;
  while (p->pool.size() < want) {
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return MOE_ERROR_HIP;
    p->pool.push_back(e);
  }
  p->timing_mask = stage_mask;
  return MOE_SUCCESS;
}

moe_status_t moe_stage_times(moe_plan_t p, double* ms, int64_t* calls) {
  if (!p || !ms) return MOE_ERROR_INVALID_VALUE;
  std::lock_guard<std::mutex> g(p->tmu);
  for (int i = 0; i < MOE_MAX_STAGES; ++i) ms[i] = 0.0;
  for (auto& ev : p->pending) {
    float t = 0.f;
    if (hipEventElapsedTime(&t, ev.a, ev.b) != hipSuccess) return MOE_ERROR_HIP;
    ms[ev.stage] += t;
  }
  for (auto& ev : p->pending) {
    p->pool.push_back(ev.a);
    p->pool.push_back(ev.b);
  }
  p->pending.clear();
  if (calls) *calls = p->timed_calls;
  p->timed_calls = 0;
  return MOE_SUCCESS;
}

moe_status_t moe_block_forward(moe_plan_t p, void* workspace, size_t workspace_bytes,
                               void* stream, int64_t T, const void* x, const void* norm_w,
                               const void* router_w, const float* corr_bias, const void* gate_up,
                               const void* down, const void* shared_gate, const void* shared_up,
                               const void* shared_down, int32_t k, float routed_scale,
                               void* out) {
  if (!p) return MOE_ERROR_INVALID_VALUE;
  const moe_config_t& c = p->cfg;
  if (c.n_experts == 0) return MOE_ERROR_NOT_SUPPORTED;  // dense plan: moe_dense_block_forward
  if (T < 0 || T > c.max_tokens) return MOE_ERROR_INVALID_VALUE;
  if (k < 1 || k > c.max_top_k || k > c.n_experts) return MOE_ERROR_INVALID_VALUE;
  if (!isfinite(routed_scale)) return MOE_ERROR_INVALID_VALUE;
  if (T == 0) return MOE_SUCCESS;  // nothing is read or written
  if (!workspace || !x || !norm_w || !router_w || !corr_bias || !gate_up || !down || !out)
    return MOE_ERROR_INVALID_VALUE;
  const bool has_shared = c.shared_inter > 0;
  if (has_shared && (!shared_gate || !shared_up || !shared_down)) return MOE_ERROR_INVALID_VALUE;
  if (misaligned(workspace) || misaligned(x) || misaligned(norm_w) || misaligned(router_w) ||
      misaligned(corr_bias) || misaligned(gate_up) || misaligned(down) || misaligned(out) ||
      (has_shared && (misaligned(shared_gate) || misaligned(shared_up) || misaligned(shared_down))))
    return MOE_ERROR_MISALIGNED;
  if (workspace_bytes < p->lay.total) return MOE_ERROR_WORKSPACE_TOO_SMALL;
  {
    const moe_status_t st = check_splits(p, T, k);
    if (st != MOE_SUCCESS) return st;
  }

  hipStream_t s = (hipStream_t)stream;
  const Layout& L = p->lay;
  char* ws = (char*)workspace;
  void* h = ws + L.h;
  float* logits = (float*)(ws + L.logits);
  int32_t* topk_idx = (int32_t*)(ws + L.topk_idx);
  float* topk_w = (float*)(ws + L.topk_w);
  int32_t* chunk_cnt = (int32_t*)(ws + L.chunk_cnt);
  int32_t* counts = (int32_t*)(ws + L.counts);
  int32_t* offsets = (int32_t*)(ws + L.offsets);
  RouteHeader* hdr = (RouteHeader*)(ws + L.hdr);
  int32_t* active = (int32_t*)(ws + L.active);
  int2* mtiles = (int2*)(ws + L.mtiles);
  int32_t* perm_token = (int32_t*)(ws + L.perm_token);
  int32_t* row_of = (int32_t*)(ws + L.row_of);
  int32_t* pass_base = (int32_t*)(ws + L.pass_base);
  float* s_parts = (float*)(ws + L.s_parts);
  void* act = ws + L.act;
  void* y = ws + L.y;
  float* sh_gu = (float*)(ws + L.sh_gu);
  void* act_s = ws + L.act_s;
  float* sh_dn = (float*)(ws + L.sh_dn);

  const int dt = c.dtype == MOE_DTYPE_BF16 ? kBF16 : kF32;
  const int E = c.n_experts, d = c.dim, I = c.moe_inter, Is = c.shared_inter;
  const int64_t A = T * k;
  const int nchunks = (int)cdiv(T, kChunkTokens);
  const bool mfma = use_mfma(p, T, k);
  int tm, tn, tk;
  nt_tiles(p, T, &tm, &tn, &tk);

  std::unique_lock<std::mutex> tlock;
  const int32_t tmask = begin_timing(p, tlock);
  hipError_t err = hipSuccess;
  hipStream_t cs = s;  // stream the stages below are enqueued on
  const bool dbg = debug_sync();
  auto stage = [&](int st, auto&& fn) {
    if (err != hipSuccess) return;
    EventPair ev{st, nullptr, nullptr};
    const bool timing = (tmask >> st) & 1;
    if (timing) {
      ev.a = get_event(p);
      ev.b = get_event(p);
      if (!ev.a || !ev.b) {
        err = hipErrorOutOfMemory;
        return;
      }
      err = hipEventRecord(ev.a, cs);
      if (err != hipSuccess) return;
    }
    err = fn();
    if (err == hipSuccess && dbg) err = hipStreamSynchronize(cs);
    if (timing) {
      const hipError_t e2 = hipEventRecord(ev.b, cs);
      if (err == hipSuccess) err = e2;
      p->pending.push_back(ev);
    }
  };
  auto nt = [&](const void* Aop, int64_t lda, const void* B1, const void* B2, int64_t ldb,
                int n_split, float* outp, int64_t N, int64_t K, const Split& sp) {
    NtArgs a{Aop, lda, B1, B2, ldb, n_split, outp, (int)T, (int)N, (int)K, sp.splits, sp.kt_per};
    return dt == kBF16 ? launch_mfma_nt(a, cs) : launch_fma_nt(dt, a, cs);
  };
  const Split rsplit = nt_split(T, E, d, tm, tn, tk, kMaxRouterSplits);
  const int scus = shared_cus(p, T, k);
  const Split sdsplit =
      has_shared ? nt_split(T, d, Is, tm, tn, tk, kMaxSharedSplits, scus) : Split{0, 0};
  const Split sgsplit =
      has_shared ? nt_split(T, 2 * (int64_t)Is, d, tm, tn, tk, kMaxSharedSplits, scus)
                 : Split{0, 0};

  if (use_fused(p, T, k)) {
    FusedArgs f{};
    f.x = (const bf16*)x, f.norm_w = (const bf16*)norm_w, f.router_w = (const bf16*)router_w;
    f.corr_bias = corr_bias, f.gate_up = (const bf16*)gate_up, f.down = (const bf16*)down;
    f.sg = (const bf16*)shared_gate, f.su = (const bf16*)shared_up, f.sd = (const bf16*)shared_down;
    f.out = (bf16*)out;
    f.T = T, f.d = d, f.E = E, f.I = I, f.Is = Is, f.k = k, f.eps = c.eps, f.rs = routed_scale;
    f.h = (bf16*)h, f.logits = logits, f.topk_idx = topk_idx, f.topk_w = topk_w;
    f.chunk_cnt = chunk_cnt, f.counts = counts, f.offsets = offsets, f.hdr = hdr, f.active = active;
    f.perm_token = perm_token, f.row_of = row_of, f.act = (bf16*)act, f.y = (bf16*)y;
    f.pass_base = pass_base, f.parts = s_parts;
    f.sh_gu = sh_gu, f.act_s = (bf16*)act_s, f.sh_dn = sh_dn;
    f.r_splits = rsplit.splits, f.r_kper = rsplit.kt_per;
    f.sg_splits = sgsplit.splits, f.sg_kper = sgsplit.kt_per;
    f.sd_splits = sdsplit.splits, f.sd_kper = sdsplit.kt_per;
    f.sync = (uint32_t*)(ws + L.sync);
    int blocks = 0;
    if (fused_decode_blocks(&blocks) != hipSuccess) {
      (void)hipGetLastError();
      return MOE_ERROR_NOT_SUPPORTED;  // no cooperative launch on this device
    }
    stage(kStFused, [&] { return launch_fused_decode(f, blocks, s); });
    return err == hipSuccess ? MOE_SUCCESS : MOE_ERROR_HIP;
  }
  stage(kStNorm, [&] { return launch_rmsnorm(dt, x, d, norm_w, h, d, T, d, c.eps, s); });
  // The shared expert depends only on h.  With the streaming expert kernels (small
  // batches, latency-bound routing steps) it runs on a side stream, forked here and
  // joined before the combine, beside the router, the routing steps and the routed
  // experts; with the MFMA kernels its GEMMs would hold the compute units the
  // routing steps wait for, so it runs in order after the routed experts.
  std::unique_lock<std::mutex> slock(p->smu, std::defer_lock);
  SideStream* side = nullptr;
  // With one K split the 256-row kernel forms silu(gate) * up itself.
  const bool fused_act = dt == kBF16 && has_shared && nt_swiglu_fused(T, sgsplit.splits);
  auto shared_branch = [&] {
    stage(kStSharedGateUp, [&] {
      if (fused_act) {
        NtArgs a{h, d, shared_gate, shared_up, d, Is, nullptr, (int)T, 2 * Is, d, 1, sgsplit.kt_per};
        return launch_mfma_nt_swiglu(a, act_s, cs);
      }
      return nt(h, d, shared_gate, shared_up, d, Is, sh_gu, 2 * (int64_t)Is, d, sgsplit);
    });
    if (!fused_act)
      stage(kStSharedAct,
            [&] { return launch_swiglu_finalize(dt, sh_gu, sgsplit.splits, T, Is, act_s, cs); });
    stage(kStSharedDown, [&] {
      return nt(act_s, Is, shared_down, shared_down, Is, d, sh_dn, d, Is, sdsplit);
    });
  };
  auto fork_shared = [&] {
    if (!has_shared || err != hipSuccess) return;
    slock.lock();
    side = side_stream(p);
    if (side) {
      err = hipEventRecord(side->fork, s);
      if (err == hipSuccess) err = hipStreamWaitEvent(side->stream, side->fork, 0);
      cs = side->stream;
      shared_branch();
      if (err == hipSuccess) err = hipEventRecord(side->join, side->stream);
      cs = s;
    } else {
      slock.unlock();
    }
  };
  // Small batches: per-token selection blocks, then the whole permutation in one
  // block; otherwise chunked selection with histograms, scans and the scatter.
  const bool small_route = T * k <= kRouteSmallMax && E <= 1024;
  // A few bf16 tokens on the streaming path: the shared expert runs in extra blocks
  // of the router's split-K product and of those two one-block launches, on the
  // compute units they leave idle, instead of on the side stream (whose kernels the
  // routing launches and the routed gate_up would wait behind).
  const bool shared_small = has_shared && !mfma && dt == kBF16 && small_route &&
                            T <= kSharedSmallTokens;
  // act_s columns [0, split) beside the router product, [split, Is) beside the
  // selection (two fifths and three fifths: at 1-4 GLM-5 tokens 0.4-0.8 % faster
  // than a quarter or 55 %, 1-2.5 % faster than all beside the selection); the down
  // product beside the permutation
  SharedSmall sh_r{}, sh_t{}, sh_p{};
  const int rblocks = (int)cdiv(E, kMfmaBN) * rsplit.splits;
  if (shared_small) {
    const int split = rblocks < kComputeUnits ? (int)((int64_t)Is * 2 / 5 / 8 * 8) : 0;
    const SharedSmall base{(const bf16*)h, (const bf16*)shared_gate, (const bf16*)shared_up,
                           (const bf16*)shared_down, (bf16*)act_s, sh_dn, (int)T, d, Is, 0, 0, 0};
    sh_r = base;
    sh_r.blocks = kComputeUnits - rblocks, sh_r.col0 = 0, sh_r.col1 = split;
    if (split == 0) sh_r.T = 0;
    sh_t = base;
    sh_t.blocks = kComputeUnits - (int)T, sh_t.col0 = split, sh_t.col1 = Is;
    sh_p = base;
    sh_p.blocks = kComputeUnits - 1, sh_p.col0 = sh_p.col1 = 0;
  }
  if (!mfma && !shared_small) fork_shared();
  stage(kStRouter, [&] {
    if (sh_r.T > 0) {
      NtArgs a{h, d, router_w, router_w, d, (int)E, logits, (int)T, (int)E, (int)d,
               rsplit.splits, rsplit.kt_per};
      return launch_mfma_nt_shared(a, sh_r, cs);
    }
    return nt(h, d, router_w, router_w, d, E, logits, E, d, rsplit);
  });
  stage(kStTopk, [&] {
    return small_route ? launch_topk_small(logits, rsplit.splits, corr_bias, T, E, k,
                                           routed_scale, topk_idx, topk_w, sh_t, s)
                       : launch_topk(logits, rsplit.splits, corr_bias, T, E, k, routed_scale,
                                     topk_idx, topk_w, chunk_cnt, s);
  });
  stage(kStScan, [&] {
    return small_route ? launch_route_small(topk_idx, T, E, k, counts, offsets, hdr, active,
                                            mtiles, pass_base, perm_token, row_of, sh_p, s)
                       : launch_scan(chunk_cnt, nchunks, E, counts, offsets, hdr, active, mtiles,
                                     pass_base, s);
  });
  if (!small_route)
    stage(kStScatter, [&] {
      return launch_scatter(topk_idx, chunk_cnt, offsets, T, E, k, perm_token, row_of, s);
    });
  GroupArgs g{counts, offsets, hdr, active, mtiles, perm_token, pass_base, E, d, I};
  const StreamFix fx{s_parts, stream_slot_floats(dt, I, d), 0};
  // the gate_up's K split keeps its range sums in the streaming part-sum region
  const ColKSplit ks{s_parts, A,
                     L.s_parts != 0 && col_ksplit_floats(A, I) <=
                                           (int64_t)kStreamMaxBlocks * 2 * fx.slot_floats};
  const int max_mtiles = (int)(cdiv(A, kGroupBM) + std::min<int64_t>(E, A));
  stage(kStGateUp, [&] {
    return mfma ? launch_mfma_gate_up(g, max_mtiles, A, h, gate_up, act, s)
                : launch_stream_gate_up(dt, g, fx, A, ks, h, gate_up, act, s);
  });
  stage(kStDown, [&] {
    return mfma ? launch_mfma_down(g, max_mtiles, act, down, y, s)
                : launch_stream_down(dt, g, fx, A, ks, act, down, y, s);
  });
  if (side) {
    const hipError_t e2 = hipStreamWaitEvent(s, side->join, 0);
    if (err == hipSuccess) err = e2;
    slock.unlock();
  } else if (has_shared && !shared_small) {
    shared_branch();  // the shared expert runs in order on s
  }
  stage(kStCombine, [&] {
    return launch_combine(dt, x, sh_dn, has_shared ? (shared_small ? 1 : sdsplit.splits) : 0, y,
                          topk_w, row_of, T, d, k, out, s);
  });
  return err == hipSuccess ? MOE_SUCCESS : MOE_ERROR_HIP;
}

moe_status_t moe_block_forward_static(moe_plan_t p, void* stream, int64_t T, const void* x,
                                      const void* norm_w, const void* router_w,
                                      const float* corr_bias, const void* gate_up,
                                      const void* down, const void* shared_gate,
                                      const void* shared_up, const void* shared_down, int32_t k,
                                      float routed_scale, void* out) {
  if (!p) return MOE_ERROR_INVALID_VALUE;
  if (p->lay.total > MOE_STATIC_WORKSPACE_BYTES) return MOE_ERROR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  if (static_workspace(&ws) != hipSuccess) return MOE_ERROR_HIP;
  return moe_block_forward(p, ws, MOE_STATIC_WORKSPACE_BYTES, stream, T, x, norm_w, router_w,
                           corr_bias, gate_up, down, shared_gate, shared_up, shared_down, k,
                           routed_scale, out);
}

moe_status_t moe_dense_block_forward(moe_plan_t p, void* workspace, size_t workspace_bytes,
                                     void* stream, int64_t T, const void* x, const void* norm_w,
                                     const void* gate, const void* up, const void* down,
                                     void* out) {
  if (!p) return MOE_ERROR_INVALID_VALUE;
  const moe_config_t& c = p->cfg;
  if (c.n_experts != 0) return MOE_ERROR_NOT_SUPPORTED;  // MoE plan: moe_block_forward
  if (T < 0 || T > c.max_tokens) return MOE_ERROR_INVALID_VALUE;
  if (T == 0) return MOE_SUCCESS;  // nothing is read or written
  if (!workspace || !x || !norm_w || !gate || !up || !down || !out) return MOE_ERROR_INVALID_VALUE;
  if (misaligned(workspace) || misaligned(x) || misaligned(norm_w) || misaligned(gate) ||
      misaligned(up) || misaligned(down) || misaligned(out))
    return MOE_ERROR_MISALIGNED;
  if (workspace_bytes < p->lay.total) return MOE_ERROR_WORKSPACE_TOO_SMALL;
  {
    const moe_status_t st = check_splits(p, T, 0);
    if (st != MOE_SUCCESS) return st;
  }

  hipStream_t s = (hipStream_t)stream;
  const Layout& L = p->lay;
  char* ws = (char*)workspace;
  void* h = ws + L.h;
  float* sh_gu = (float*)(ws + L.sh_gu);
  void* act_s = ws + L.act_s;
  float* sh_dn = (float*)(ws + L.sh_dn);
  const int dt = c.dtype == MOE_DTYPE_BF16 ? kBF16 : kF32;
  const int d = c.dim, Id = c.shared_inter;
  int tm, tn, tk;
  nt_tiles(p, T, &tm, &tn, &tk);
  const Split gsplit = nt_split(T, 2 * (int64_t)Id, d, tm, tn, tk, kMaxSharedSplits);
  const Split dsplit = nt_split(T, d, Id, tm, tn, tk, kMaxSharedSplits);
  auto nt = [&](const void* Aop, int64_t lda, const void* B1, const void* B2, int64_t ldb,
                int n_split, float* outp, int64_t N, int64_t K, const Split& sp) {
    NtArgs a{Aop, lda, B1, B2, ldb, n_split, outp, (int)T, (int)N, (int)K, sp.splits, sp.kt_per};
    return dt == kBF16 ? launch_mfma_nt(a, s) : launch_fma_nt(dt, a, s);
  };

  std::unique_lock<std::mutex> tlock;
  const int32_t tmask = begin_timing(p, tlock);
  hipError_t err = hipSuccess;
  const bool dbg = debug_sync();
  auto stage = [&](int st, auto&& fn) {
    if (err != hipSuccess) return;
    EventPair ev{st, nullptr, nullptr};
    const bool timing = (tmask >> st) & 1;
    if (timing) {
      ev.a = get_event(p);
      ev.b = get_event(p);
      if (!ev.a || !ev.b) {
        err = hipErrorOutOfMemory;
        return;
      }
      err = hipEventRecord(ev.a, s);
      if (err != hipSuccess) return;
    }
    err = fn();
    if (err == hipSuccess && dbg) err = hipStreamSynchronize(s);
    if (timing) {
      const hipError_t e2 = hipEventRecord(ev.b, s);
      if (err == hipSuccess) err = e2;
      p->pending.push_back(ev);
    }
  };
  // h = RMSNorm(x); act = silu(h gate^T) * (h up^T); out = x + act down^T
  stage(kStNorm, [&] { return launch_rmsnorm(dt, x, d, norm_w, h, d, T, d, c.eps, s); });
  // With one K split the 256-row kernel forms silu(gate) * up itself.
  const bool fused_act = dt == kBF16 && nt_swiglu_fused(T, gsplit.splits);
  stage(kStSharedGateUp, [&] {
    if (fused_act) {
      NtArgs a{h, d, gate, up, d, Id, nullptr, (int)T, 2 * Id, d, 1, gsplit.kt_per};
      return launch_mfma_nt_swiglu(a, act_s, s);
    }
    return nt(h, d, gate, up, d, Id, sh_gu, 2 * (int64_t)Id, d, gsplit);
  });
  if (!fused_act)
    stage(kStSharedAct, [&] { return launch_swiglu_finalize(dt, sh_gu, gsplit.splits, T, Id, act_s, s); });
  stage(kStSharedDown, [&] { return nt(act_s, Id, down, down, Id, d, sh_dn, d, Id, dsplit); });
  stage(kStCombine, [&] {
    return launch_combine(dt, x, sh_dn, dsplit.splits, nullptr, nullptr, nullptr, T, d, 0, out, s);
  });
  return err == hipSuccess ? MOE_SUCCESS : MOE_ERROR_HIP;
}

namespace {
// [p, p + bytes) and [q, q + bytes2) overlap
bool overlaps(const void* p, size_t bytes, const void* q, size_t bytes2) {
  const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
  return a < b + bytes2 && b < a + bytes;
}

moe_status_t pack_args_ok(int32_t dtype, int32_t dim, int32_t inter, const void* const* in, int n_in,
                          const size_t* in_bytes, void* const* out, int n_out,
                          const size_t* out_bytes) {
  if (dtype != MOE_DTYPE_F32 && dtype != MOE_DTYPE_BF16) return MOE_ERROR_NOT_SUPPORTED;
  if (dim <= 0 || inter <= 0 || dim > (1 << 20) || inter > (1 << 20)) return MOE_ERROR_INVALID_VALUE;
  if (dim % 64 || inter % 64) return MOE_ERROR_NOT_SUPPORTED;
  for (int i = 0; i < n_in; ++i)
    if (!in[i]) return MOE_ERROR_INVALID_VALUE;
  for (int i = 0; i < n_out; ++i)
    if (!out[i]) return MOE_ERROR_INVALID_VALUE;
  for (int i = 0; i < n_in; ++i)
    if (misaligned(in[i])) return MOE_ERROR_MISALIGNED;
  for (int i = 0; i < n_out; ++i)
    if (misaligned(out[i])) return MOE_ERROR_MISALIGNED;
  for (int i = 0; i < n_out; ++i) {
    for (int j = 0; j < n_in; ++j)
      if (overlaps(out[i], out_bytes[i], in[j], in_bytes[j])) return MOE_ERROR_INVALID_VALUE;
    for (int j = 0; j < i; ++j)
      if (overlaps(out[i], out_bytes[i], out[j], out_bytes[j])) return MOE_ERROR_INVALID_VALUE;
  }
  return MOE_SUCCESS;
}
}  // namespace

moe_status_t moe_pack_expert(void* stream, int32_t dtype, int32_t dim, int32_t inter,
                             const void* gate, const void* up, const void* down, void* gate_up,
                             void* down_packed) {
  const size_t es = dtype == MOE_DTYPE_BF16 ? 2 : 4, n = (size_t)dim * (size_t)inter * es;
  const void* in[3] = {gate, up, down};
  const size_t in_b[3] = {n, n, n};
  void* out[2] = {gate_up, down_packed};
  const size_t out_b[2] = {2 * n, n};
  const moe_status_t st = pack_args_ok(dtype, dim, inter, in, 3, in_b, out, 2, out_b);
  if (st != MOE_SUCCESS) return st;
  // gate_up[i][n] = gate[n][i], gate_up[i][I + n] = up[n][i], down_packed[n][m] = down[m][n]
  TransposeBatch b{};
  b.count = 3;
  b.src[0] = gate, b.dst[0] = gate_up, b.rows[0] = inter, b.cols[0] = dim;
  b.ld_src[0] = dim, b.ld_dst[0] = 2 * (int64_t)inter;
  b.src[1] = up, b.dst[1] = (char*)gate_up + (size_t)inter * es, b.rows[1] = inter, b.cols[1] = dim;
  b.ld_src[1] = dim, b.ld_dst[1] = 2 * (int64_t)inter;
  b.src[2] = down, b.dst[2] = down_packed, b.rows[2] = dim, b.cols[2] = inter;
  b.ld_src[2] = inter, b.ld_dst[2] = dim;
  const hipError_t e = launch_transpose(dtype == MOE_DTYPE_BF16 ? kBF16 : kF32, b, (hipStream_t)stream);
  return e == hipSuccess ? MOE_SUCCESS : MOE_ERROR_HIP;
}

moe_status_t moe_unpack_expert(void* stream, int32_t dtype, int32_t dim, int32_t inter,
                               const void* gate_up, const void* down_packed, void* gate, void* up,
                               void* down) {
  const size_t es = dtype == MOE_DTYPE_BF16 ? 2 : 4, n = (size_t)dim * (size_t)inter * es;
  const void* in[2] = {gate_up, down_packed};
  const size_t in_b[2] = {2 * n, n};
  void* out[3] = {gate, up, down};
  const size_t out_b[3] = {n, n, n};
  const moe_status_t st = pack_args_ok(dtype, dim, inter, in, 2, in_b, out, 3, out_b);
  if (st != MOE_SUCCESS) return st;
  // gate[n][i] = gate_up[i][n], up[n][i] = gate_up[i][I + n], down[m][n] = down_packed[n][m]
  TransposeBatch b{};
  b.count = 3;
  b.src[0] = gate_up, b.dst[0] = gate, b.rows[0] = dim, b.cols[0] = inter;
  b.ld_src[0] = 2 * (int64_t)inter, b.ld_dst[0] = dim;
  b.src[1] = (const char*)gate_up + (size_t)inter * es, b.dst[1] = up, b.rows[1] = dim;
  b.cols[1] = inter, b.ld_src[1] = 2 * (int64_t)inter, b.ld_dst[1] = dim;
  b.src[2] = down_packed, b.dst[2] = down, b.rows[2] = inter, b.cols[2] = dim;
  b.ld_src[2] = dim, b.ld_dst[2] = inter;
  const hipError_t e = launch_transpose(dtype == MOE_DTYPE_BF16 ? kBF16 : kF32, b, (hipStream_t)stream);
  return e == hipSuccess ? MOE_SUCCESS : MOE_ERROR_HIP;
}

size_t moe_buffer_bytes(moe_plan_t p, int64_t T, int32_t k, int32_t which) {
  if (!p || T < 0 || T > p->cfg.max_tokens) return 0;
  const moe_config_t& c = p->cfg;
  if (c.n_experts == 0) {  // dense plan: h and the MLP activation, k must be 0
    if (k != 0) return 0;
    if (which == MOE_BUF_H) return (size_t)T * c.dim * p->es;
    if (which == MOE_BUF_SHARED_ACT) return (size_t)T * c.shared_inter * p->es;
    return 0;
  }
  if (k < 1 || k > c.max_top_k) return 0;
  const int64_t A = T * k;
  switch (which) {
    case MOE_BUF_H: return (size_t)T * c.dim * p->es;
    case MOE_BUF_OFFSETS: return (size_t)(c.n_experts + 1) * 4;
    case MOE_BUF_PERM_TOKEN: return (size_t)A * 4;
    case MOE_BUF_ROW_OF: return (size_t)A * 4;
    case MOE_BUF_ACT: return (size_t)A * c.moe_inter * p->es;
    case MOE_BUF_Y: return (size_t)A * c.dim * p->es;
    case MOE_BUF_SHARED_ACT: return (size_t)T * c.shared_inter * p->es;
    case MOE_BUF_FUSED_ERROR: return 4;
  }
  return 0;
}

moe_status_t moe_rmsnorm(void* stream, int32_t dtype, int64_t rows, int32_t width, float eps,
                         const void* x, int64_t x_stride, const void* weight, void* out,
                         int64_t out_stride) {
  if (dtype != MOE_DTYPE_F32 && dtype != MOE_DTYPE_BF16) return MOE_ERROR_NOT_SUPPORTED;
  const int64_t es = dtype == MOE_DTYPE_BF16 ? 2 : 4, vec = 16 / es;
  if (rows < 0 || rows > INT32_MAX || width <= 0 || width > (1 << 24) || width % vec ||
      x_stride < width || out_stride < width || x_stride % vec || out_stride % vec ||
      !(eps > 0.0f) || !isfinite(eps))
    return MOE_ERROR_INVALID_VALUE;
  if (rows == 0) return MOE_SUCCESS;
  if (!x || !weight || !out) return MOE_ERROR_INVALID_VALUE;
  if (misaligned(x) || misaligned(weight) || misaligned(out)) return MOE_ERROR_MISALIGNED;
  // out may be x itself (same stride); any other overlap of the two row ranges is rejected
  const uintptr_t x0 = (uintptr_t)x, x1 = x0 + (uintptr_t)(((rows - 1) * x_stride + width) * es);
  const uintptr_t o0 = (uintptr_t)out, o1 = o0 + (uintptr_t)(((rows - 1) * out_stride + width) * es);
  const bool overlap = x0 < o1 && o0 < x1;
  if (overlap && !(x0 == o0 && x_stride == out_stride)) return MOE_ERROR_INVALID_VALUE;
  const hipError_t e = moe::launch_rmsnorm(dtype == MOE_DTYPE_BF16 ? moe::kBF16 : moe::kF32, x,
                                           x_stride, weight, out, out_stride, rows, width, eps,
                                           (hipStream_t)stream);
  return e == hipSuccess ? MOE_SUCCESS : MOE_ERROR_HIP;
}

moe_status_t moe_calib_hbm_read(void* stream, const void* src, size_t bytes, int32_t blocks,
                                void* sink) {
  if (!src || !sink || bytes == 0 || bytes % 16 || blocks < 1 || blocks > 65536)
    return MOE_ERROR_INVALID_VALUE;
  if (misaligned(src) || ((uintptr_t)sink & 3u)) return MOE_ERROR_MISALIGNED;
  const hipError_t e = launch_calib_read(src, bytes, blocks, (uint32_t*)sink, (hipStream_t)stream);
  return e == hipSuccess ? MOE_SUCCESS : MOE_ERROR_HIP;
}

moe_status_t moe_calib_mfma(void* stream, int32_t iters, int32_t blocks, void* sink,
                            double* flops) {
  if (!sink || !flops || iters < 1 || blocks < 1 || blocks > 65536) return MOE_ERROR_INVALID_VALUE;
  if ((uintptr_t)sink & 3u) return MOE_ERROR_MISALIGNED;
  const hipError_t e = launch_calib_mfma(iters, blocks, (float*)sink, flops, (hipStream_t)stream);
  return e == hipSuccess ? MOE_SUCCESS : MOE_ERROR_HIP;
}

moe_status_t moe_read_buffer(moe_plan_t p, const void* workspace, void* stream, int64_t T,
                             int32_t k, int32_t which, void* dst, size_t dst_bytes) {
  if (!p || !workspace || !dst) return MOE_ERROR_INVALID_VALUE;
  if (which < 0 || which >= MOE_BUF_COUNT) return MOE_ERROR_INVALID_VALUE;
  if (T < 0 || T > p->cfg.max_tokens) return MOE_ERROR_INVALID_VALUE;
  if (p->cfg.n_experts == 0) {  // dense plan: k = 0; only h and the MLP activation exist
    if (k != 0 || (which != MOE_BUF_H && which != MOE_BUF_SHARED_ACT)) return MOE_ERROR_INVALID_VALUE;
  } else if (k < 1 || k > p->cfg.max_top_k) {
    return MOE_ERROR_INVALID_VALUE;
  }
  const size_t bytes = moe_buffer_bytes(p, T, k, which);
  if (dst_bytes < bytes) return MOE_ERROR_INVALID_VALUE;
  if (bytes == 0) return MOE_SUCCESS;
  const Layout& L = p->lay;
  size_t off = 0;
  switch (which) {
    case MOE_BUF_H: off = L.h; break;
    case MOE_BUF_OFFSETS: off = L.offsets; break;
    case MOE_BUF_PERM_TOKEN: off = L.perm_token; break;
    case MOE_BUF_ROW_OF: off = L.row_of; break;
    case MOE_BUF_ACT: off = L.act; break;
    case MOE_BUF_Y: off = L.y; break;
    case MOE_BUF_SHARED_ACT: off = L.act_s; break;
    case MOE_BUF_FUSED_ERROR: off = L.sync + 8; break;
  }
  const hipError_t e = hipMemcpyAsync(dst, (const char*)workspace + off, bytes,
                                      hipMemcpyDeviceToDevice, (hipStream_t)stream);
  return e == hipSuccess ? MOE_SUCCESS : MOE_ERROR_HIP;
}

moe_status_t moe_read_routing(moe_plan_t p, const void* workspace, void* stream, int64_t T,
                              int32_t k, int32_t* topk_idx, float* topk_w, int32_t* counts) {
  if (p && p->cfg.n_experts == 0) return MOE_ERROR_NOT_SUPPORTED;  // dense plan: no routing
  if (!p || !workspace) return MOE_ERROR_INVALID_VALUE;
  if (T < 0 || T > p->cfg.max_tokens || k < 1 || k > p->cfg.max_top_k) return MOE_ERROR_INVALID_VALUE;
  const Layout& L = p->lay;
  const char* ws = (const char*)workspace;
  hipStream_t s = (hipStream_t)stream;
  const size_t ab = (size_t)T * k * 4;
  hipError_t e = hipSuccess;
  if (topk_idx && ab) e = hipMemcpyAsync(topk_idx, ws + L.topk_idx, ab, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess && topk_w && ab)
    e = hipMemcpyAsync(topk_w, ws + L.topk_w, ab, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess && counts)
    e = hipMemcpyAsync(counts, ws + L.counts, (size_t)p->cfg.n_experts * 4,
                       hipMemcpyDeviceToDevice, s);
  return e == hipSuccess ? MOE_SUCCESS : MOE_ERROR_HIP;
}

}  // extern "C"
