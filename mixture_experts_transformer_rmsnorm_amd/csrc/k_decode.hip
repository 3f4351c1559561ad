// Fused decode forward: the whole sublayer for a decode-sized batch in one
// persistent launch (after a one-block reset of its counters).
//
// The work is a list of items in a fixed order, grouped in phases:
//   norm      RMSNorm of 8 rows per item
//   router    router logits, one 128 x 128 x K-range MFMA tile per item (split-K partials)
//   topk      selection for one chunk of 16 tokens (+ the chunk's expert histogram)
//   scan      per-expert counts, segment offsets, active-expert list (one item)
//   scatter   stable permutation of one chunk
//   sh_gu     shared expert gate/up, MFMA tiles
//   gu        routed gate/up + SwiGLU, one (expert, column slice) per item, weights streamed
//   sh_act    shared expert SwiGLU of 8 tokens per item
//   sh_dn     shared expert down, MFMA tiles
//   dn        routed down, one (expert, column slice) per item
//   combine   weighted combine + residual for 4 tokens per item
// Each block takes the next item from a global ticket counter.  An item waits, before
// it starts, until the items it reads from are done: a phase counter reaching the
// phase's item count, or (dn) the counter of its expert's gu items.  Items are
// handed out in list order and every dependency points to earlier items, so the
// earliest unfinished item always has its inputs: a waiting block never waits on
// an item that has not been handed to a running block, and the launch completes
// whatever the number of resident blocks.  Each wait is also bounded; a wait that
// runs out sets an error word (the item then proceeds, so the launch still ends).
//
// Memory ordering: a finished item's threads issue an agent-scope release fence
// (their stores reach the level every XCD reads) before one thread adds to the
// counter; a waiting item's thread polls with agent-scope loads, and every thread
// issues an agent-scope acquire fence after the block barrier.
#include <type_traits>

#include "common.h"
#include "dev_nt.h"
#include "dev_small.h"
#include "dev_stream.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kGuCL = 32, kDnCL = 64;  // stream shapes of the gate/up and down items
constexpr uint32_t kSpinLimit = 1u << 22;

struct FusedSmem {
  union {
    NtSmem nt;
    float red[StreamShape<bf16, kGuCL, true>::RG * kStreamMaxMT *
              StreamShape<bf16, kGuCL, true>::RED_COLS];
    int hist[1024];
    int s_idx[kChunkTokens * 16];
    int scan[1024 + 256];
    double rms[4];
  } u;
  int ticket;
};
static_assert(StreamShape<bf16, kDnCL, false>::RG * StreamShape<bf16, kDnCL, false>::RED_COLS <=
                  StreamShape<bf16, kGuCL, true>::RG * StreamShape<bf16, kGuCL, true>::RED_COLS,
              "the down items' reduction fits the union");

// Thread 0 polls *ctr (agent-scope loads, no cache maintenance per poll) until it
// reaches target (bounded); the caller then synchronises the block and every
// thread issues the acquire fence.
__device__ __forceinline__ void wait_for(const uint32_t* ctr, uint32_t target, uint32_t* err) {
  if (threadIdx.x != 0) return;
  for (uint32_t it = 0; it < kSpinLimit; ++it) {
    if (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) return;
    __builtin_amdgcn_s_sleep(4);
  }
  __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Scan item: per expert, exclusive prefix of the chunk histograms over the chunks
// (in place) and the total; then the segment offsets (exclusive scan of the totals
// over experts, in expert order) and the list of active experts.  256 threads.
__device__ void scan_item(int32_t* __restrict__ chunk_cnt, int nchunks, int E,
                          int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                          RouteHeader* __restrict__ hdr, int32_t* __restrict__ active, int* sm) {
  int* s_cnt = sm;          // [E] totals
  int* s_part = sm + 1024;  // [256] per-thread partial sums (count, active) packed
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int carry = 0;
    for (int c = 0; c < nchunks; ++c) {
      const int v = chunk_cnt[(int64_t)c * E + e];
      chunk_cnt[(int64_t)c * E + e] = carry;
      carry += v;
    }
    counts[e] = carry;
    s_cnt[e] = carry;
  }
  __syncthreads();
  // each thread owns a contiguous run of experts
  const int per = (E + 255) / 256;
  const int e0 = min(E, (int)threadIdx.x * per), e1 = min(E, e0 + per);
  int sum = 0, act = 0;
  for (int e = e0; e < e1; ++e) {
    sum += s_cnt[e];
    act += s_cnt[e] > 0 ? 1 : 0;
  }
  // inclusive scan of (sum, act) over the 256 threads (sum < 2^20, act <= 1024)
  s_part[threadIdx.x] = (sum << 11) | act;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int v = threadIdx.x >= off ? s_part[threadIdx.x - off] : 0;
    __syncthreads();
    s_part[threadIdx.x] += v;
    __syncthreads();
  }
  const int excl = threadIdx.x ? s_part[threadIdx.x - 1] : 0;
  int off = excl >> 11, a = excl & 2047;
  for (int e = e0; e < e1; ++e) {
    offsets[e] = off;
    off += s_cnt[e];
    if (s_cnt[e] > 0) active[a++] = e;
  }
  if (threadIdx.x == 255) {
    offsets[E] = s_part[255] >> 11;
    hdr->n_active = s_part[255] & 2047;
    hdr->n_mtiles = 0;
  }
  __syncthreads();
}

template <int Q>
__device__ __attribute__((noinline)) void topk_item(const float* logits, int splits,
                                                    const float* bias, int64_t T, int E, int k,
                                                    float rs, int32_t* idx, float* w,
                                                    int32_t* chunk_cnt, int64_t chunk, int* hist) {
  topk_chunk<Q, 4>(logits, splits, bias, T, E, k, rs, idx, w, chunk_cnt, chunk, hist);
}

// The heavy item kinds are separate functions, so that each is register-allocated
// on its own rather than all together inside one switch.
__device__ __attribute__((noinline)) void nt_item(NtArgs a, int n_tile, int z, NtSmem* sm) {
  nt_tile_128(a, n_tile, 0, z, *sm);
}

template <int CL, bool GU>
__device__ __attribute__((noinline)) void stream_work(GroupArgs g, const bf16* A, const bf16* W,
                                                      bf16* out, int e, int slice, float* red) {
  stream_item<bf16, CL, GU>(g, A, W, out, e, slice, red);
}

}  // namespace

__global__ __launch_bounds__(256, 2) void fused_reset_kernel(uint32_t* sync, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) sync[i] = 0u;
}

__global__ __launch_bounds__(256, 2) void fused_decode_kernel(FusedArgs f) {
  __shared__ __attribute__((aligned(16))) FusedSmem sm;
  uint32_t* queue = f.sync;
  uint32_t* err = f.sync + 1;
  uint32_t* done = f.sync + 2;                 // [kFusedPhases]
  uint32_t* gu_done = f.sync + 2 + kFusedPhases;  // [E]
  const int total = f.start[kFusedPhases];
  const int E = f.E;
  GroupArgs g{f.counts, f.offsets, f.hdr, f.active, nullptr, f.perm_token, nullptr, f.E, f.d, f.I};
  const int gu_slices = stream_slices<bf16, kGuCL, true>(f.I, f.d);
  const int dn_slices = stream_slices<bf16, kDnCL, false>(f.I, f.d);

  for (;;) {
    if (threadIdx.x == 0) sm.ticket = (int)atomicAdd(queue, 1u);
    __syncthreads();
    const int item = sm.ticket;
    __syncthreads();
    if (item >= total) break;
    int ph = 0;
    while (item >= f.start[ph + 1]) ++ph;
    const int i = item - f.start[ph];
    auto phase_count = [&](int p) { return (uint32_t)(f.start[p + 1] - f.start[p]); };

    // ---- dependencies
    switch (ph) {
      case kPhRouter:
      case kPhShGu: wait_for(done + kPhNorm, phase_count(kPhNorm), err); break;
      case kPhTopk: wait_for(done + kPhRouter, phase_count(kPhRouter), err); break;
      case kPhScan: wait_for(done + kPhTopk, phase_count(kPhTopk), err); break;
      case kPhScatter: wait_for(done + kPhScan, phase_count(kPhScan), err); break;
      case kPhGu: wait_for(done + kPhScatter, phase_count(kPhScatter), err); break;
      case kPhShAct: wait_for(done + kPhShGu, phase_count(kPhShGu), err); break;
      case kPhShDn: wait_for(done + kPhShAct, phase_count(kPhShAct), err); break;
      case kPhDn: wait_for(gu_done + i / dn_slices, (uint32_t)gu_slices, err); break;
      case kPhCombine:
        wait_for(done + kPhDn, phase_count(kPhDn), err);
        wait_for(done + kPhShDn, phase_count(kPhShDn), err);
        break;
      default: break;
    }
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

    // ---- the item
    switch (ph) {
      case kPhNorm: {
        const int64_t r1 = min<int64_t>(f.T, (int64_t)(i + 1) * 8);
        for (int64_t r = (int64_t)i * 8; r < r1; ++r)
          rms_block_row<bf16>(f.x + r * f.d, f.norm_w, f.h + r * f.d, f.d, f.eps, sm.u.rms);
        break;
      }
      case kPhRouter: {
        const int n_tiles = (E + kNtBN - 1) / kNtBN;
        NtArgs a{f.h, f.d, f.router_w, f.router_w, f.d, E, f.logits, (int)f.T, E, f.d,
                 f.r_splits, f.r_kper};
        nt_item(a, i % n_tiles, i / n_tiles, &sm.u.nt);
        break;
      }
      case kPhTopk: {
        const int q = (E + kWave - 1) / kWave;
#define MOE_TOPK_ITEM(QQ)                                                                       \
  topk_item<QQ>(f.logits, f.r_splits, f.corr_bias, f.T, E, f.k, f.rs, f.topk_idx, f.topk_w,       \
                f.chunk_cnt, i, sm.u.hist)
        if (q <= 1) MOE_TOPK_ITEM(1);
        else if (q <= 2) MOE_TOPK_ITEM(2);
        else if (q <= 4) MOE_TOPK_ITEM(4);
        else if (q <= 8) MOE_TOPK_ITEM(8);
        else MOE_TOPK_ITEM(16);
#undef MOE_TOPK_ITEM
        break;
      }
      case kPhScan:
        scan_item(f.chunk_cnt, (int)((f.T + kChunkTokens - 1) / kChunkTokens), E, f.counts,
                  f.offsets, f.hdr, f.active, sm.u.scan);
        break;
      case kPhScatter:
        scatter_chunk(f.topk_idx, f.chunk_cnt, f.offsets, f.T, E, f.k, f.perm_token, f.row_of, i,
                      sm.u.s_idx);
        break;
      case kPhShGu: {
        const int n_tiles = (2 * f.Is + kNtBN - 1) / kNtBN;
        NtArgs a{f.h, f.d, f.sg, f.su, f.d, f.Is, f.sh_gu, (int)f.T, 2 * f.Is, f.d, f.sg_splits,
                 f.sg_kper};
        nt_item(a, i % n_tiles, i / n_tiles, &sm.u.nt);
        break;
      }
      case kPhGu: {
        const int e = i / gu_slices;
        if (f.counts[e] > 0)
          stream_work<kGuCL, true>(g, f.h, f.gate_up, f.act, e, i % gu_slices, sm.u.red);
        break;
      }
      case kPhShAct: {
        const int64_t t1 = min<int64_t>(f.T, (int64_t)(i + 1) * 8);
        const int nv = f.Is / 4;
        for (int64_t t = (int64_t)i * 8; t < t1; ++t)
          for (int n4 = threadIdx.x; n4 < nv; n4 += blockDim.x)
            swiglu_vec<bf16>(f.sh_gu, f.sg_splits, f.T, f.Is, f.act_s, t, n4);
        break;
      }
      case kPhShDn: {
        const int n_tiles = (f.d + kNtBN - 1) / kNtBN;
        NtArgs a{f.act_s, f.Is, f.sd, f.sd, f.Is, f.d, f.sh_dn, (int)f.T, f.d, f.Is, f.sd_splits,
                 f.sd_kper};
        nt_item(a, i % n_tiles, i / n_tiles, &sm.u.nt);
        break;
      }
      case kPhDn: {
        const int e = i / dn_slices;
        if (f.counts[e] > 0)
          stream_work<kDnCL, false>(g, f.act, f.down, f.y, e, i % dn_slices, sm.u.red);
        break;
      }
      case kPhCombine: {
        const int64_t t1 = min<int64_t>(f.T, (int64_t)(i + 1) * 4);
        const int nv = f.d / 8;
        for (int64_t t = (int64_t)i * 4; t < t1; ++t)
          for (int v = threadIdx.x; v < nv; v += blockDim.x)
            combine_vec<bf16>(f.x, f.sh_dn, f.sd_splits, f.y, f.topk_w, f.row_of, f.T, f.d, f.k,
                              f.out, t, v * 8);
        break;
      }
      default: break;
    }

    // ---- publish
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (threadIdx.x == 0) {
      __hip_atomic_fetch_add(done + ph, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      if (ph == kPhGu) __hip_atomic_fetch_add(gu_done + i / gu_slices, 1u, __ATOMIC_RELEASE,
                                              __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

int fused_item_counts(const FusedArgs& f, int* counts) {
  const int nchunks = (int)((f.T + kChunkTokens - 1) / kChunkTokens);
  counts[kPhNorm] = (int)((f.T + 7) / 8);
  counts[kPhRouter] = ((f.E + kNtBN - 1) / kNtBN) * f.r_splits;
  counts[kPhTopk] = nchunks;
  counts[kPhScan] = 1;
  counts[kPhScatter] = nchunks;
  counts[kPhShGu] = ((2 * f.Is + kNtBN - 1) / kNtBN) * f.sg_splits;
  counts[kPhGu] = f.E * stream_slices<bf16, kGuCL, true>(f.I, f.d);
  counts[kPhShAct] = (int)((f.T + 7) / 8);
  counts[kPhShDn] = ((f.d + kNtBN - 1) / kNtBN) * f.sd_splits;
  counts[kPhDn] = f.E * stream_slices<bf16, kDnCL, false>(f.I, f.d);
  counts[kPhCombine] = (int)((f.T + 3) / 4);
  int total = 0;
  for (int p = 0; p < kFusedPhases; ++p) total += counts[p];
  return total;
}

hipError_t launch_fused_decode(FusedArgs f, int grid, hipStream_t s) {
  int counts[kFusedPhases];
  fused_item_counts(f, counts);
  f.start[0] = 0;
  for (int p = 0; p < kFusedPhases; ++p) f.start[p + 1] = f.start[p] + counts[p];
  fused_reset_kernel<<<1, 256, 0, s>>>(f.sync, kFusedSyncWords(f.E));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  fused_decode_kernel<<<dim3((unsigned)grid), 256, 0, s>>>(f);
  return hipGetLastError();
}

}  // namespace moe
