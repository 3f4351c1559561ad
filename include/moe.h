/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE feed-forward sublayer library.
 *
 * One call, moe_block_forward, runs the post-attention half of a GLM-style MoE
 * block on one GPU:
 *
 *   h   = RMSNorm(x) * norm_w                    (fp32 math, cast back, gain)
 *   s   = sigmoid(h . router_w^T)                (one score per routed expert)
 *   sel = top_k experts by s + corr_bias         (bias used for selection only)
 *   w_j = routed_scale * s_sel_j / sum_j s_sel_j
 *   out = x + shared(h) + sum_j w_j * expert_sel_j(h)
 *
 * with every expert a SwiGLU MLP down(silu(gate h) * up h).
 *
 * Sources (web pages, cited by title and section):
 *  - "GLM-5 · Input features" (OpenModelAtlas), excerpts "rmsnorm"
 *    (GlmMoeDsaRMSNorm: float32 normalisation by the root mean square, cast back
 *    to the input dtype, then the per-feature gain; epsilon default 1e-6),
 *    "block" (GlmMoeDsaDecoderLayer: out = residual + mlp(norm(residual))) and
 *    "mlp" (GlmMoeDsaMLP: the SwiGLU form, bias-free linear maps).
 *  - "nemo_automodel.components.models.glm4_moe.state_dict_adapter",
 *    class Glm4MoeStateDictAdapter:
 *    the grouped native expert layout gate_and_up_projs [n_experts, dim,
 *    2*moe_inter_dim] and down_projs [n_experts, moe_inter_dim, dim], and the
 *    shared expert's separate gate/up/down nn.Linear weights.
 *  - "GLM-5 · MoE transformer block", Parameters table and note: one
 *    correction-bias value per expert, held by the router as a buffer.
 *  The router rule (sigmoid, bias for selection only, renormalised unbiased
 *  scores times routed_scale) is not printed on the pages; it is the workload
 *  definition this library implements.
 *
 * Conventions
 *  - All tensors are row-major, contiguous, in device memory, 16-byte aligned.
 *  - D = the plan's dtype (fp32 or bfloat16) for x, out, norm_w, router_w,
 *    gate_up, down and shared_*; corr_bias is always fp32.
 *  - Layouts (T = num_tokens, d = dim, E = n_experts, I = moe_inter,
 *    Is = shared_inter, k = top_k):
 *      x, out        [T, d]        D
 *      norm_w        [d]           D
 *      router_w      [E, d]        D   (nn.Linear [out, in])
 *      corr_bias     [E]           fp32
 *      gate_up       [E, d, 2I]    D   columns [0, I) gate, [I, 2I) up
 *      down          [E, I, d]     D
 *      shared_gate   [Is, d]       D   (nn.Linear [out, in])
 *      shared_up     [Is, d]       D
 *      shared_down   [d, Is]       D
 *  - Ownership: the caller allocates and owns every tensor and the workspace.
 *    The library never allocates device memory, frees, or synchronises inside
 *    moe_block_forward.  A plan's configuration is immutable after creation and
 *    one plan may serve several threads.  A MoE plan with a shared expert whose
 *    path is not MFMA also owns one non-blocking side stream and two events on
 *    the device current at moe_plan_create (made there, released by
 *    moe_plan_destroy; a forward call creates no HIP object): on the STREAM path
 *    from 5 tokens (and for fp32 plans) the shared expert runs there, forked from
 *    and joined back to the call's stream, so the call stays ordered on its
 *    stream (and can be captured into a graph); calls on another device run it in
 *    order on their own stream.  At 1-4 bf16 tokens it runs inside the router,
 *    selection and permutation launches on the call's stream.
 *    Concurrent calls on one plan serialise only their host-side enqueueing.
 *    A workspace serves one call in flight at a time; later calls on the same
 *    stream may reuse it.
 *  - Aliasing: out may alias x (in-place residual); no other aliasing.
 *  - Errors: arguments are validated synchronously before anything is
 *    enqueued; on error nothing is written and a status is returned.  Device
 *    faults surface at the caller's next synchronisation.  Inputs must be
 *    finite; NaN/Inf behaviour is unspecified.
 *  - Debugging: with MOE_DEBUG_SYNC=1 in the environment (read at every call),
 *    moe_block_forward and moe_dense_block_forward synchronise their stream
 *    after each stage, so a kernel that fails is reported as MOE_ERROR_HIP by
 *    the call that launched it.  It serialises the call and must not be set
 *    while a stream is being captured into a graph.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

#if defined(__GNUC__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

typedef enum {
  MOE_SUCCESS = 0,
  MOE_ERROR_INVALID_VALUE = 1,       /* null pointer, bad size, top_k, num_tokens, scale */
  MOE_ERROR_NOT_SUPPORTED = 2,       /* shape / dtype / path outside what the kernels handle */
  MOE_ERROR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes below the plan's requirement */
  MOE_ERROR_MISALIGNED = 4,          /* a pointer not 16-byte aligned */
  MOE_ERROR_HIP = 5                  /* a HIP launch or copy returned an error */
} moe_status_t;

typedef enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 } moe_dtype_t;

/* Kernel family for the expert matmuls.
 *  AUTO:   STREAM when the mean tokens per routed expert, T*k/E, is at most 5
 *          (decode-sized batches, where the expert weights are streamed once from
 *          HBM), MFMA otherwise.  fp32 plans always use STREAM.
 *  STREAM: weight-streaming FMA kernels (any dtype).
 *  MFMA:   LDS-tiled bf16 matrix-core kernels (bf16 only).
 *  FUSED:  the whole forward in one launch (bf16 only) for calls of at most 64
 *          tokens: one block per compute unit, all resident at once (cooperative
 *          launch), the steps separated by grid barriers; larger calls of a FUSED
 *          plan take the STREAM kernels.  Forward returns NOT_SUPPORTED on a device
 *          without cooperative launch.  AUTO does not pick it (slower than the
 *          multi-kernel path at the batch sizes measured). */
typedef enum {
  MOE_PATH_AUTO = 0,
  MOE_PATH_STREAM = 1,
  MOE_PATH_MFMA = 2,
  MOE_PATH_FUSED = 3
} moe_path_t;

typedef struct {
  uint32_t struct_size;  /* sizeof(moe_config_t) */
  int32_t dim;           /* d: multiple of 64 */
  int64_t max_tokens;    /* largest num_tokens a forward call may pass (>= 0) */
  int32_t n_experts;     /* E: 1..1024; 0 makes a dense-block plan (see below) */
  int32_t moe_inter;     /* I: multiple of 64 (0 for a dense-block plan) */
  int32_t shared_inter;  /* Is: 0 (no shared expert) or a multiple of 64; for a
                            dense-block plan, the MLP width (> 0) */
  int32_t max_top_k;     /* 1..min(E, 16) (0 for a dense-block plan) */
  int32_t dtype;         /* moe_dtype_t */
  int32_t path;          /* moe_path_t */
  float eps;             /* RMSNorm epsilon (> 0) */
  uint32_t flags;        /* reserved, must be 0 */
} moe_config_t;

typedef struct moe_plan* moe_plan_t;

/* Validate *cfg and create a plan; *workspace_bytes receives the device
 * workspace size every moe_block_forward call with this plan needs.
 * Returns INVALID_VALUE for null pointers or out-of-range fields,
 * NOT_SUPPORTED for shapes/dtypes/paths the kernels do not handle. */
MOE_API moe_status_t moe_plan_create(const moe_config_t* cfg, moe_plan_t* plan, size_t* workspace_bytes);

/* Whether a forward call with num_tokens / top_k fits the plan: the host-side
 * size checks of moe_block_forward (top_k = 0 for a dense-block plan), with no
 * pointer argument and no device work.  INVALID_VALUE for num_tokens outside
 * [0, max_tokens] or top_k outside its range; WORKSPACE_TOO_SMALL if a
 * split-K partial-sum region sized at plan creation could not hold the call's
 * partial sums (forward calls return the same status before enqueueing
 * anything); MOE_SUCCESS otherwise. */
MOE_API moe_status_t moe_plan_check(moe_plan_t plan, int64_t num_tokens, int32_t top_k);

/* Destroy a plan (NULL is accepted). */
MOE_API moe_status_t moe_plan_destroy(moe_plan_t plan);

/* Enqueue the whole sublayer on `stream` (a hipStream_t; NULL = default stream).
 * num_tokens in [0, max_tokens]; 0 is a successful no-op that reads no pointer
 * (they may then be NULL).  top_k in [1, min(E, max_top_k)].  routed_scale
 * finite.  Shared pointers may be NULL only when the plan's shared_inter is 0.
 * Returns asynchronously. */
MOE_API moe_status_t moe_block_forward(moe_plan_t plan, void* workspace, size_t workspace_bytes,
                               void* stream, int64_t num_tokens, const void* x, const void* norm_w,
                               const void* router_w, const float* corr_bias, const void* gate_up,
                               const void* down, const void* shared_gate, const void* shared_up,
                               const void* shared_down, int32_t top_k, float routed_scale,
                               void* out);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): moe_block_forward with
 * its workspace taken from a static buffer of MOE_STATIC_WORKSPACE_BYTES (128 MiB)
 * that the library holds in each GPU's memory from its load on that GPU until
 * the process ends; the caller passes no workspace.  The call allocates nothing
 * (no hipMalloc, no allocating library routine); its first call on a device
 * that no plan was created on looks the buffer's address up once.
 *  - Arguments, layouts, errors and results as for moe_block_forward;
 *    WORKSPACE_TOO_SMALL when the plan's workspace_bytes exceeds
 *    MOE_STATIC_WORKSPACE_BYTES (the GLM-5 decode plan for 64 tokens needs
 *    about 122 MiB and fits; prefill-sized plans do not).
 *  - Every call on one GPU, from any plan or thread, shares that GPU's buffer,
 *    which keeps the last call's contents (the kernels need nothing zeroed):
 *    calls that overlap in time on one GPU (on different streams, or from
 *    several host threads without ordering) race and give wrong results.  Order
 *    them on one stream. */
#define MOE_STATIC_WORKSPACE_BYTES ((size_t)128 << 20)
MOE_API moe_status_t moe_block_forward_static(moe_plan_t plan, void* stream, int64_t num_tokens,
                                              const void* x, const void* norm_w,
                                              const void* router_w, const float* corr_bias,
                                              const void* gate_up, const void* down,
                                              const void* shared_gate, const void* shared_up,
                                              const void* shared_down, int32_t top_k,
                                              float routed_scale, void* out);

/* Dense block: the blocks in front of the first MoE block use a dense SwiGLU MLP
 * instead of the MoE ("GLM-5 · Input features", excerpt block: the first
 * first_k_dense_replace blocks; excerpt mlp: GlmMoeDsaMLP, down(silu(gate x) *
 * up x) with bias-free nn.Linear maps).  Per token t:
 *
 *   h   = RMSNorm(x) * norm_w          (as in moe_block_forward)
 *   out = x + down(silu(h . gate^T) * (h . up^T))
 *
 * The plan comes from moe_plan_create with n_experts = 0, moe_inter = 0,
 * max_top_k = 0 and shared_inter = Id, the MLP width (a multiple of 64).
 * Layouts (row-major, contiguous, device memory, 16-byte aligned, dtype D):
 *   x, out [T, d]; norm_w [d]; gate, up [Id, d]; down [d, Id]  (nn.Linear [out, in]).
 * num_tokens in [0, max_tokens]; 0 is a successful no-op that reads no pointer.
 * out may alias x.  Errors, ownership, workspace and stage timing as for
 * moe_block_forward (stages rmsnorm, shared_gate_up, shared_act, shared_down,
 * combine).  A dense plan passed to moe_block_forward, or a MoE plan passed
 * here, returns NOT_SUPPORTED.  For a dense plan, moe_read_buffer and
 * moe_buffer_bytes take top_k = 0 and serve MOE_BUF_H and MOE_BUF_SHARED_ACT (the
 * MLP activation); moe_read_routing returns NOT_SUPPORTED. */
MOE_API moe_status_t moe_dense_block_forward(moe_plan_t plan, void* workspace, size_t workspace_bytes,
                                             void* stream, int64_t num_tokens, const void* x,
                                             const void* norm_w, const void* gate, const void* up,
                                             const void* down, void* out);

/* Expert weight layout conversion ("nemo_automodel.components.models.glm4_moe.state_dict_adapter",
 * class Glm4MoeStateDictAdapter: HF checkpoints keep each expert's gate_proj, up_proj and
 * down_proj as separate nn.Linear weights; the native grouped layout stacks them
 * as gate_and_up_projs [n_experts, dim, 2*moe_inter_dim] and down_projs
 * [n_experts, moe_inter_dim, dim]).  One expert per call (d = dim, I = inter):
 *
 *   moe_pack_expert:   gate [I, d], up [I, d], down [d, I]   (HF, nn.Linear [out, in])
 *                      -> gate_up [d, 2I]: gate_up[i][n] = gate[n][i], gate_up[i][I+n] = up[n][i]
 *                         down_packed [I, d]: down_packed[n][m] = down[m][n]
 *   moe_unpack_expert: the inverse.
 *
 * gate_up / down_packed are expert e's slices of the grouped tensors
 * (gate_and_up_projs + e*d*2I, down_projs + e*I*d elements).  Bits are moved, not
 * converted.  dtype is moe_dtype_t; dim and inter are multiples of 64
 * (NOT_SUPPORTED otherwise); pointers are 16-byte aligned device memory
 * (MISALIGNED); no output may overlap an input or another output
 * (INVALID_VALUE).  Enqueued on `stream`; returns asynchronously. */
MOE_API moe_status_t moe_pack_expert(void* stream, int32_t dtype, int32_t dim, int32_t inter,
                                     const void* gate, const void* up, const void* down,
                                     void* gate_up, void* down_packed);
MOE_API moe_status_t moe_unpack_expert(void* stream, int32_t dtype, int32_t dim, int32_t inter,
                                       const void* gate_up, const void* down_packed, void* gate,
                                       void* up, void* down);

/* Copy the routing of the last forward call that used `workspace` into caller
 * buffers (device memory), enqueued on `stream`:
 *   topk_idx [num_tokens, top_k] int32  experts in (key desc, index asc) order
 *   topk_w   [num_tokens, top_k] fp32   weights in the same order
 *   counts   [E] int32                  tokens routed to each expert
 * Any destination may be NULL.  num_tokens/top_k must be those of that call. */
MOE_API moe_status_t moe_read_routing(moe_plan_t plan, const void* workspace, void* stream,
                              int64_t num_tokens, int32_t top_k, int32_t* topk_idx, float* topk_w,
                              int32_t* counts);

/* Standalone RMSNorm, the same operation as the sublayer's first step, for the
 * block's other norms ("GLM-5 · Input features", excerpt rmsnorm: fp32
 * normalisation by the root mean square over the last dimension, cast back to
 * the input dtype, then the per-feature gain; excerpt block: the norm in front
 * of attention, width dim; "GLM-5 · MoE transformer block", Parameters: the MLA
 * latent norms, query latent width 2048, and the per-head query/key norms):
 *
 *   out[r, i] = D(weight[i] * D(x[r, i] * rsqrt(mean_i x[r, i]^2 + eps)))
 *
 * for r < rows, i < width.  x row r starts at x + r * x_stride elements, out
 * row r at out + r * out_stride (strides in elements, >= width), so a norm over
 * the leading columns of a wider row (a latent that shares its row with other
 * features) needs no copy.  Per-head norms pass rows = tokens * heads and
 * width = the head dimension.
 *  dtype     moe_dtype_t of x, weight and out (D).
 *  width     a multiple of 16 / sizeof(D) (8 for bf16, 4 for fp32), <= 2^24.
 *  strides   multiples of 16 / sizeof(D); pointers 16-byte aligned device memory.
 *  weight    [width] D.
 *  eps       > 0 and finite.
 * out may be x itself (same stride); any other overlap is INVALID_VALUE.
 * rows == 0 is a successful no-op that reads no pointer.  Enqueued on `stream`
 * (a hipStream_t; NULL = default stream); returns asynchronously; the caller
 * owns every buffer. */
MOE_API moe_status_t moe_rmsnorm(void* stream, int32_t dtype, int64_t rows, int32_t width, float eps,
                                 const void* x, int64_t x_stride, const void* weight, void* out,
                                 int64_t out_stride);

/* Measurement kernels: the attainable peaks of this GPU, for reporting the
 * sublayer's kernels against them beside the published peaks.
 *  moe_calib_hbm_read: reads `bytes` (a multiple of 16) of device buffer src
 *    (16-byte aligned), each of `blocks` blocks of 1024 lanes an equal contiguous
 *    share, with 16-byte nontemporal loads.  sink: 4 bytes of device memory,
 *    written only for a data pattern that real buffers do not produce.
 *  moe_calib_mfma: `blocks` blocks of 8 waves, each wave `iters` rounds of four
 *    independent v_mfma_f32_32x32x16_bf16 on register operands; *flops (host)
 *    receives the FLOPs enqueued; sink as above.
 * Both enqueue on `stream` and return asynchronously; the caller times them
 * (events around the call).  INVALID_VALUE / MISALIGNED for bad arguments. */
MOE_API moe_status_t moe_calib_hbm_read(void* stream, const void* src, size_t bytes, int32_t blocks,
                                        void* sink);
MOE_API moe_status_t moe_calib_mfma(void* stream, int32_t iters, int32_t blocks, void* sink,
                                    double* flops);

/* Intermediate buffers of the last forward call (tests, diagnostics). */
typedef enum {
  MOE_BUF_H = 0,          /* [T, d] D: normalised input */
  MOE_BUF_OFFSETS = 1,    /* [E + 1] int32: expert segment offsets in the permuted order */
  MOE_BUF_PERM_TOKEN = 2, /* [T*k] int32: token of each permuted row */
  MOE_BUF_ROW_OF = 3,     /* [T, k] int32: permuted row of assignment (t, j) */
  MOE_BUF_ACT = 4,        /* [T*k, I] D: silu(gate) * up per permuted row */
  MOE_BUF_Y = 5,          /* [T*k, d] D: routed expert output per permuted row */
  MOE_BUF_SHARED_ACT = 6, /* [T, Is] D: shared expert silu(gate) * up */
  MOE_BUF_FUSED_ERROR = 7, /* [1] uint32: error word of the last fused decode launch: 0, or
                              nonzero if a grid-barrier wait ran out of time (1 s) and the
                              launch ended early (outputs then undefined) */
  MOE_BUF_COUNT = 8
} moe_buffer_t;

/* Copy intermediate buffer `which` of the last forward call into `dst` (device
 * memory, dst_bytes >= the buffer's size for num_tokens/top_k), on `stream`. */
MOE_API moe_status_t moe_read_buffer(moe_plan_t plan, const void* workspace, void* stream,
                             int64_t num_tokens, int32_t top_k, int32_t which, void* dst,
                             size_t dst_bytes);

/* Size in bytes of intermediate buffer `which` for num_tokens/top_k (0 if invalid). */
MOE_API size_t moe_buffer_bytes(moe_plan_t plan, int64_t num_tokens, int32_t top_k, int32_t which);

/* Path the plan takes for num_tokens/top_k (MOE_PATH_STREAM, MOE_PATH_MFMA or
 * MOE_PATH_FUSED); for
 * a dense-block plan, MFMA for bf16 and STREAM (the fp32 FMA products) for fp32. */
MOE_API int32_t moe_plan_path(moe_plan_t plan, int64_t num_tokens, int32_t top_k);

/* Per-stage GPU timing.  stage_mask selects stages (bit s = stage s, see
 * moe_stage_name; 0 disables).  While set, moe_block_forward records a HIP
 * event before and after each selected stage's kernels on the stream they run
 * on (the call's stream, or the side stream for the shared-expert stages);
 * after the caller synchronises, moe_stage_times returns the elapsed
 * milliseconds summed per stage since the last read in ms[stage] and the number
 * of timed calls in *calls.  moe_set_stage_timing makes the events (enough for
 * 128 calls between two reads; HIP if they cannot be made); a forward call made
 * while too few are left is neither timed nor counted.  A stage whose work another stage's kernel does
 * records nothing: bf16 shared_act when the shared (or dense) gate/up product
 * runs at 256 rows or more in one K split and forms silu(gate) * up itself
 * (its time is in shared_gate_up); the three shared-expert stages at 1-4 bf16
 * tokens on the STREAM path (their time is in router_logits, router_topk and
 * permute_scan).  Timing state is the only mutable part of a
 * plan and is meant for one thread. */
#define MOE_MAX_STAGES 16
MOE_API moe_status_t moe_set_stage_timing(moe_plan_t plan, int32_t stage_mask);
MOE_API moe_status_t moe_stage_times(moe_plan_t plan, double* ms /*[MOE_MAX_STAGES]*/,
                                     int64_t* calls);
MOE_API const char* moe_stage_name(int32_t stage);

MOE_API const char* moe_status_string(moe_status_t status);
MOE_API int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
