// Fused decode forward: the whole sublayer for a decode-sized batch (at most 64
// tokens) in one launch of one block per compute unit, all resident at once
// (cooperative launch).  The phases run in order, separated by grid barriers:
//
//   1  RMSNorm, one token row per block
//   2  router logits (128 x 128 MFMA tiles over K ranges, split-K partials) and the
//      shared expert's gate/up product (same tiles)
//   3  top-k selection, 16 tokens per block (with per-chunk expert histograms);
//      the shared expert's SwiGLU, one token per block
//   4  one block: per-expert counts, segment offsets, active-expert list and
//      streaming-pass prefix, then the stable scatter of every chunk; the other
//      blocks: the shared expert's down product
//   5  routed gate/up + SwiGLU, the weight stream split into equal row ranges
//      over all blocks (the Stream-K split of the stand-alone streaming kernel)
//   6  the gate/up items cut between blocks, finished (only when some item is cut)
//   7  routed down, the same way
//   8  the down items cut between blocks, finished (only when some item is cut)
//   9  weighted combine + shared output + residual, one token per block
//
// The item bodies are the device functions of the stand-alone kernels
// (dev_small.h, dev_nt.h, dev_stream.h).  Every block runs every phase's loop
// (`for (i = block; i < items; i += blocks)`, bounds from the arguments) and
// every barrier, so the barriers inside item bodies are reached by all waves of
// a block; values that steer control flow and are computed inside the launch
// (the routing's pass count, the active-expert count) reach every thread of a
// block from one read by thread 0 through LDS.
//
// Grid barrier: after a block barrier, wave 0 issues an agent-scope release fence
// for the block, then thread 0 adds 1 to a cumulative arrival counter
// (acquire-release, agent scope); the block that brings it to blocks x (barriers
// passed + 1) publishes the next generation number (release); the others' thread
// 0 polls the generation word.  Wave 0 then issues an agent-scope acquire fence
// before a block barrier lets the other waves read.  Each wait is bounded by
// wall-clock time (1 s of the 100 MHz constant clock): a wait that runs out, or
// that sees the error flag already set, sets the flag, and its block leaves the
// kernel at once, so every wait of every block ends and the launch completes;
// the caller reads the flag (MOE_BUF_FUSED_ERROR).  A block passes a barrier only
// when every block has arrived, i.e. after all of the previous phase's writes.
#include <algorithm>

#include "common.h"
#include "dev_nt.h"
#include "dev_small.h"
#include "dev_stream.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kFT = 256;  // threads per block
// Dynamic LDS asked for beside the kernel's own (about 78 KiB), so that no compute
// unit can hold two blocks and the dispatcher puts one on each.
constexpr unsigned kLdsPad = 8192;
constexpr uint64_t kWaitTicks = 100000000ull;  // 1 s of s_memrealtime (100 MHz)

struct FusedSmem {
  union {
    NtSmem nt;
    int hist[1024];
    int s_idx[kChunkTokens * 16];
    int scan[1024 + 2 * 256];
    double rms[4];
  } u;
  int s_pass[kMaxStreamExperts + 1];
  int bcast[2];
};

// Grid barrier (see the file comment); returns false when the block must leave.
__device__ __forceinline__ bool grid_barrier(uint32_t* sync, uint32_t blocks, uint32_t& gen,
                                             int* bcast) {
  // Wave 0's fences act for the block: after the block barrier every wave's stores
  // have reached this XCD's L2, which the release writes back; the acquire
  // invalidates this compute unit's L1 and the L2's lines before any wave reads.
  __syncthreads();
  if (threadIdx.x < kWave) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  if (threadIdx.x == 0) {
    const uint32_t target = gen + 1;
    int ok = __hip_atomic_load(sync + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u;
    if (ok) {
      const uint32_t arrived =
          __hip_atomic_fetch_add(sync, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      if (arrived == blocks * target - 1u) {
        __hip_atomic_store(sync + 1, target, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        while (__hip_atomic_load(sync + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
          if (__hip_atomic_load(sync + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u ||
              __builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks) {
            ok = 0;
            break;
          }
          __builtin_amdgcn_s_sleep(2);
        }
      }
    }
    if (!ok) __hip_atomic_fetch_or(sync + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bcast[0] = ok;
  }
  if (threadIdx.x < kWave) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  __syncthreads();
  gen += 1;
  const bool ok = bcast[0] != 0;
  __syncthreads();  // bcast is written again at the next barrier
  return ok;
}

// Routing summary of the whole batch (one block of 256 threads): per expert,
// exclusive prefix of the chunk histograms over the chunks (in place) and the
// total; then the segment offsets (exclusive scan of the totals over experts),
// the list of active experts, the first streaming pass of each active expert
// (passes of up to kStreamMaxMT tokens) and the header.
__device__ void scan_item(int32_t* __restrict__ chunk_cnt, int nchunks, int E,
                          int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                          RouteHeader* __restrict__ hdr, int32_t* __restrict__ active,
                          int32_t* __restrict__ pass_base, int* sm) {
  int* s_cnt = sm;                                      // [E] totals
  unsigned long long* s_part = (unsigned long long*)(sm + 1024);  // [256] packed sums
  for (int e = threadIdx.x; e < E; e += kFT) {
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
  // each thread owns a contiguous run of experts; its (count, active, passes)
  // sums are packed in 16-bit fields (each total is at most 64 x 16 assignments
  // or 1024 experts), then scanned over the threads
  const int per = (E + kFT - 1) / kFT;
  const int e0 = min(E, (int)threadIdx.x * per), e1 = min(E, e0 + per);
  unsigned long long sum = 0, act = 0, pas = 0;
  for (int e = e0; e < e1; ++e) {
    sum += (unsigned)s_cnt[e];
    act += s_cnt[e] > 0 ? 1u : 0u;
    pas += (unsigned)(s_cnt[e] + kStreamMaxMT - 1) / kStreamMaxMT;
  }
  s_part[threadIdx.x] = (sum << 32) | (act << 16) | pas;
  __syncthreads();
  for (int off = 1; off < kFT; off <<= 1) {
    const unsigned long long v = threadIdx.x >= (unsigned)off ? s_part[threadIdx.x - off] : 0ull;
    __syncthreads();
    s_part[threadIdx.x] += v;
    __syncthreads();
  }
  const unsigned long long excl = threadIdx.x ? s_part[threadIdx.x - 1] : 0ull;
  int off = (int)(excl >> 32), a = (int)((excl >> 16) & 0xffff), p = (int)(excl & 0xffff);
  for (int e = e0; e < e1; ++e) {
    offsets[e] = off;
    off += s_cnt[e];
    if (s_cnt[e] > 0) {
      active[a] = e;
      pass_base[a] = p;
      ++a;
      p += (s_cnt[e] + kStreamMaxMT - 1) / kStreamMaxMT;
    }
  }
  if (threadIdx.x == kFT - 1) {
    const unsigned long long tot = s_part[kFT - 1];
    const int na = (int)((tot >> 16) & 0xffff), np = (int)(tot & 0xffff);
    offsets[E] = (int)(tot >> 32);
    hdr->n_active = na;
    hdr->n_mtiles = 0;
    hdr->n_passes = np;
    pass_base[na] = np;
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
// on its own rather than all together.
__device__ __attribute__((noinline)) void nt_item(NtArgs a, int n_tile, int z, NtSmem* sm) {
  nt_tile_128(a, n_tile, 0, z, *sm);
}

template <bool GU>
__device__ __attribute__((noinline)) void stream_part(GroupArgs g, StreamFix fx, const int* s_pass,
                                                      int n_active, const bf16* A, const bf16* W,
                                                      bf16* out, int b, int blocks) {
  rs_block<bf16, GU, kFT>(g, fx, s_pass, n_active, A, W, out, b, blocks);
}

template <bool GU>
__device__ __attribute__((noinline)) void stream_fix(GroupArgs g, StreamFix fx, const int* s_pass,
                                                     int n_active, bf16* out, int b, int blocks) {
  rs_fixup_block<bf16, GU, kFT>(g, fx, s_pass, n_active, out, b, blocks, threadIdx.x);
}

// Whether the streaming phase of this geometry cuts items between blocks (the
// same answer in every block: it depends on the pass count and the block count).
template <bool GU>
__device__ __forceinline__ bool stream_cuts(const GroupArgs& g, int n_passes, int blocks) {
  const RsGeom<bf16, GU, kFT> G(g, n_passes, blocks);
  return G.R.hblocks == 0;
}

}  // namespace

__global__ __launch_bounds__(64) void fused_reset_kernel(uint32_t* sync) {
  if (threadIdx.x < kFusedSyncWords) sync[threadIdx.x] = 0u;
}

__global__ __launch_bounds__(kFT, 1) void fused_decode_kernel(FusedArgs f) {
  __shared__ __attribute__((aligned(16))) FusedSmem sm;
  const int G = gridDim.x, b = blockIdx.x;
  const int E = f.E;
  uint32_t gen = 0;
  GroupArgs g{f.counts, f.offsets, f.hdr, f.active, nullptr, f.perm_token, f.pass_base, f.E, f.d, f.I};
  const StreamFix fx{f.parts, 0, G};
  const int nchunks = (int)((f.T + kChunkTokens - 1) / kChunkTokens);
  auto barrier = [&]() { return grid_barrier(f.sync, (uint32_t)G, gen, sm.bcast); };

  // 1: RMSNorm
  for (int64_t t = b; t < f.T; t += G)
    rms_block_row<bf16>(f.x + t * f.d, f.norm_w, f.h + t * f.d, f.d, f.eps, sm.u.rms);
  if (!barrier()) return;

  // 2: router logits and the shared gate/up product, 128 x 128 tiles per K range
  {
    const int rn = (E + kNtBN - 1) / kNtBN, rt = rn * f.r_splits;
    const int sn = (2 * f.Is + kNtBN - 1) / kNtBN, st = f.Is > 0 ? sn * f.sg_splits : 0;
    for (int i = b; i < rt + st; i += G) {
      if (i < rt) {
        NtArgs a{f.h, f.d, f.router_w, f.router_w, f.d, E, f.logits, (int)f.T, E, f.d,
                 f.r_splits, f.r_kper};
        nt_item(a, i % rn, i / rn, &sm.u.nt);
      } else {
        const int j = i - rt;
        NtArgs a{f.h, f.d, f.sg, f.su, f.d, f.Is, f.sh_gu, (int)f.T, 2 * f.Is, f.d, f.sg_splits,
                 f.sg_kper};
        nt_item(a, j % sn, j / sn, &sm.u.nt);
      }
    }
  }
  if (!barrier()) return;

  // 3: selection per chunk of 16 tokens; the shared expert's SwiGLU per token
  {
    const int act_items = f.Is > 0 ? (int)f.T : 0;
    const int q = (E + kWave - 1) / kWave;
    for (int i = b; i < nchunks + act_items; i += G) {
      if (i < nchunks) {
#define MOE_TOPK_ITEM(QQ)                                                                       \
  topk_item<QQ>(f.logits, f.r_splits, f.corr_bias, f.T, E, f.k, f.rs, f.topk_idx, f.topk_w,       \
                f.chunk_cnt, i, sm.u.hist)
        if (q <= 1) MOE_TOPK_ITEM(1);
        else if (q <= 2) MOE_TOPK_ITEM(2);
        else if (q <= 4) MOE_TOPK_ITEM(4);
        else if (q <= 8) MOE_TOPK_ITEM(8);
        else MOE_TOPK_ITEM(16);
#undef MOE_TOPK_ITEM
      } else {
        const int64_t t = i - nchunks;
        for (int n4 = threadIdx.x; n4 < f.Is / 4; n4 += kFT)
          swiglu_vec<bf16>(f.sh_gu, f.sg_splits, f.T, f.Is, f.act_s, t, n4);
      }
    }
  }
  if (!barrier()) return;

  // 4: the routing summary and the scatter (one block); the shared down product
  {
    const int dn = (f.d + kNtBN - 1) / kNtBN, dt = f.Is > 0 ? dn * f.sd_splits : 0;
    for (int i = b; i < 1 + dt; i += G) {
      if (i == 0) {
        scan_item(f.chunk_cnt, nchunks, E, f.counts, f.offsets, f.hdr, f.active, f.pass_base,
                  sm.u.scan);
        for (int c = 0; c < nchunks; ++c)
          scatter_chunk(f.topk_idx, f.chunk_cnt, f.offsets, f.T, E, f.k, f.perm_token, f.row_of, c,
                        sm.u.s_idx);
      } else {
        const int j = i - 1;
        NtArgs a{f.act_s, f.Is, f.sd, f.sd, f.Is, f.d, f.sh_dn, (int)f.T, f.d, f.Is, f.sd_splits,
                 f.sd_kper};
        nt_item(a, j % dn, j / dn, &sm.u.nt);
      }
    }
  }
  if (!barrier()) return;

  // the routing's active experts and passes, read once per block
  if (threadIdx.x == 0) sm.bcast[1] = f.hdr->n_active;
  __syncthreads();
  const int n_active = sm.bcast[1];
  for (int i = threadIdx.x; i <= n_active; i += kFT) sm.s_pass[i] = f.pass_base[i];
  __syncthreads();
  const int n_passes = sm.s_pass[n_active];

  // 5-6: routed gate/up + SwiGLU
  stream_part<true>(g, fx, sm.s_pass, n_active, f.h, f.gate_up, f.act, b, G);
  if (!barrier()) return;
  if (stream_cuts<true>(g, n_passes, G)) {
    stream_fix<true>(g, fx, sm.s_pass, n_active, f.act, b, G);
    if (!barrier()) return;
  }

  // 7-8: routed down
  stream_part<false>(g, fx, sm.s_pass, n_active, f.act, f.down, f.y, b, G);
  if (!barrier()) return;
  if (stream_cuts<false>(g, n_passes, G)) {
    stream_fix<false>(g, fx, sm.s_pass, n_active, f.y, b, G);
    if (!barrier()) return;
  }

  // 9: combine + residual
  for (int64_t t = b; t < f.T; t += G)
    for (int v = threadIdx.x; v < f.d / 8; v += kFT)
      combine_vec<bf16>(f.x, f.sh_dn, f.Is > 0 ? f.sd_splits : 0, f.y, f.topk_w, f.row_of, f.T,
                        f.d, f.k, f.out, t, v * 8);
}

hipError_t fused_decode_blocks(int* blocks) {
  int dev = 0, cus = 0, coop = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fused_decode_kernel, kFT, kLdsPad);
  if (e != hipSuccess) return e;
  if (!coop || per_cu < 1 || cus < 1) return hipErrorNotSupported;
  *blocks = std::min(cus, kStreamMaxBlocks);
  return hipSuccess;
}

hipError_t launch_fused_decode(const FusedArgs& f, int blocks, hipStream_t s) {
  if (blocks < 1 || blocks > kStreamMaxBlocks) return hipErrorInvalidValue;
  fused_reset_kernel<<<1, 64, 0, s>>>(f.sync);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  FusedArgs a = f;
  void* args[] = {&a};
  return hipLaunchCooperativeKernel((const void*)fused_decode_kernel, dim3((unsigned)blocks),
                                    dim3(kFT), args, kLdsPad, s);
}

}  // namespace moe
