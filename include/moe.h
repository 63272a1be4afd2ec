/*
 * moe.h - C ABI of the routed mixture-of-experts FFN layer for AMD Instinct MI355X (gfx950).
 *
 * One layer of a GLM-5.3-Flash-class model's routed experts: router scoring and top-k
 * selection, grouping of the picks per expert, the SwiGLU expert FFN on block-scaled
 * 4-bit weights (MXFP4, and NVFP4 as a variant) dequantised on the fly, and the
 * route-weighted combine.  Each step is one entry point; moe_layer chains them.
 *
 * Sources (web pages, cited by title and section):
 *  [Maya]     "Project Maya: GLM-5.3-Flash on two 2017 GPUs, and what the 40 tok/s is made of"
 *  [Strata]   Strata-GLM on an RTX 4090 (indrasmirror.au blog)
 *  [windlass] windlass README (GLM-5.2 MXFP4 engine)
 *  [HotCache] "A hot expert cache made a 181 GiB model faster on one 96 GiB GPU"
 *
 * Conventions shared by every entry point
 *  - Memory: every pointer argument is caller-owned DEVICE memory unless a comment says
 *    "host".  The library never allocates, frees or synchronises; scratch space is the
 *    caller's workspace (see moe_workspace_bytes).
 *  - Streams: every call enqueues asynchronous work on `stream` and returns; the results
 *    are ready after the caller synchronises that stream.  Calls contain no host-device
 *    synchronisation, so they can be captured in a HIP graph.
 *  - Errors: arguments are validated on the host BEFORE anything is launched, so an
 *    error return means no work was enqueued.  MOE_ERR_HIP reports a launch failure
 *    (hipGetLastError); faults inside kernels surface at the caller's next
 *    synchronisation.  No entry point prints, exits or throws.
 *  - T = 0 (no tokens) is a valid no-op.
 *  - Activations x, residual and y share the dtype shape->act_dtype (fp32 or bf16),
 *    row-major [T][d_model].
 *  - State: the library holds none between calls (timing hooks travel with the call that
 *    uses them, see moe_layer_observed).  Concurrent calls are safe when they use distinct
 *    workspaces and outputs.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;
typedef struct ihipStream_t *hipStream_t;
struct ihipEvent_t;
typedef struct ihipEvent_t *hipEvent_t;

#define MOE_ABI_VERSION 2

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID = 1,      /* bad argument: null pointer, bad enum, inconsistent sizes */
    MOE_ERR_UNSUPPORTED = 2,  /* valid but outside the kernels' limits (see each call)    */
    MOE_ERR_WORKSPACE = 3,    /* workspace smaller than moe_workspace_bytes               */
    MOE_ERR_HIP = 4           /* a kernel launch failed                                   */
} moe_status;

typedef enum { MOE_DT_F32 = 0, MOE_DT_BF16 = 1 } moe_dtype;

/* Weight formats ([windlass]: GLM-5.2 MXFP4; [HotCache] "The wall: one PCIe transfer per
 * token": NVFP4).  Both store E2M1 values (OCP FP4: 1 sign, 2 exponent, 1 mantissa bit),
 * two per byte, element 2i in the LOW nibble and 2i+1 in the high nibble, with one scale
 * per block of consecutive elements along each row's reduction dimension:
 *   MOE_WF_MXFP4: blocks of 32, E8M0 scale byte (2^(b-127); 0xFF = NaN block);
 *   MOE_WF_NVFP4: blocks of 16, E4M3FN scale byte, times one fp32 scale per tensor. */
typedef enum { MOE_WF_MXFP4 = 0, MOE_WF_NVFP4 = 1 } moe_wformat;

/* Layer shape.  top_k of n_experts per token ([Maya] "What is in the 96.5 GB": 8 of 288).
 * routed_scaling multiplies the routed sum ([windlass], negative controls: the model's
 * routed_scaling_factor); 1.0 leaves the normalised route weights as they are.
 *
 * renorm_skip ([Strata] "Uncensoring without touching the weights", --renorm-skip): 0 turns it
 *   off.  Otherwise a pick whose normalised weight is below renorm_skip is dropped cleanly (no
 *   expert is computed for it; topk_idx -1, topk_w 0) and the kept weights are renormalised,
 *   w_j = sigmoid(l_j) / sum over kept j' of sigmoid(l_j').  Weights fall with rank, so the
 *   dropped picks are a tail of the rank order; rank 0 is always kept.  0 <= renorm_skip < 1.
 * n_shared ([Maya] "What is in the 96.5 GB": the shared experts sit beside the routed ones):
 *   0 or 1.  With 1, the expert table holds n_experts + 1 entries and entry n_experts is the
 *   shared expert, which every token passes through with weight 1, outside routed_scaling:
 *   y[t] = routed_scaling * sum_j w[t,j] o[t,j] + o_shared[t] (+ residual[t]).
 * act_quant: MOE_AQ_EXACT (0) computes with the activations as given (the default).
 *   MOE_AQ_MXFP8 (1, MXFP4 weights only) opts into quantising the FFN inputs x and h to one
 *   E4M3 value per element with one power-of-two scale 2^(floor(log2 amax) - 7) per block of 32
 *   consecutive elements (amax = the block's largest magnitude; exponent at least -126), the
 *   operand format of the FP4 x FP8 matrix cores: half the matrix-core work of the exact mode,
 *   at the precision of that quantiser (an analogue of [Maya] "A V100 has no BF16 and no FP8",
 *   activations quantised on the fly to 8 bits).  The router always sees x exactly. */
typedef enum { MOE_AQ_EXACT = 0, MOE_AQ_MXFP8 = 1 } moe_act_quant;

typedef struct {
    int32_t d_model;
    int32_t d_ff;
    int32_t n_experts;
    int32_t top_k;
    int32_t wformat;      /* moe_wformat   */
    int32_t act_dtype;    /* moe_dtype     */
    float routed_scaling;
    float renorm_skip;    /* 0: off        */
    int32_t n_shared;     /* 0 or 1        */
    int32_t act_quant;    /* moe_act_quant */
} moe_shape;

/* One expert's weights: gate and up are [d_ff][d_model], down is [d_model][d_ff], each as
 * packed codes q[rows][K/2] plus scales s[rows][K/B] (K = the row length, B = block size).
 * The table of n_experts (+ n_shared) entries lives in DEVICE memory ([Maya] "Three tiers and
 * the rules between them": the router looks its experts up in a device table).  Code pointers
 * must be 16-byte aligned.  The *_ts fields are the NVFP4 tensor scales (ignored for MXFP4). */
typedef struct {
    const uint8_t *gate_q, *up_q, *down_q;
    const uint8_t *gate_s, *up_s, *down_s;
    float gate_ts, up_ts, down_ts, reserved;
} moe_expert;

/* Limits: 1 <= top_k <= n_experts <= 1024; d_model and d_ff multiples of 128; T <= 65536.
 * Anything else returns MOE_ERR_UNSUPPORTED (or MOE_ERR_INVALID for nonsense). */

/* ABI version of the loaded library (MOE_ABI_VERSION of the headers it was built with). */
int moe_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char *moe_status_string(moe_status status);

/* Bytes in one expert's canonical blob: [gate_q | up_q | down_q | gate_s | up_s | down_s],
 * plus, for NVFP4, the three fp32 tensor scales (gate, up, down), padded to 256 bytes.
 * This is the packed fixed-stride expert layout ([windlass] build steps: experts repacked
 * per layer with a fixed stride, verified as 6 sub-tensors).  Returns 0 for a bad shape. */
size_t moe_blob_stride(const moe_shape *shape);

/* ---------------------------------------------------------------------------------------
 * Workspace.  Every entry point that takes `ws` uses it for its intermediates; a workspace
 * of moe_workspace_bytes(shape, T) bytes serves every call with that shape and at most T
 * tokens.  Calls that overlap in time need distinct workspaces.
 *
 * The first 4 bytes (offset MOE_WS_STATUS_OFFSET) are a status word: the kernels OR error
 * bits into it and nothing clears it except moe_workspace_init.  After a call, a caller that
 * wants to know reads it (4 bytes, device memory, after synchronising the stream):
 *   MOE_WS_ROUTE_TIMEOUT  the few-token router (moe_layer, T <= 16) gave up waiting for its
 *                         logits.  That call's topk_idx are -1, its topk_w and y NaN.
 *   MOE_WS_BAD_EXPERT_ID  an expert id outside [0, n_experts) other than -1 reached the
 *                         permute; that pick was left out (pick_pos -1).
 * While the status word is nonzero, moe_layer with T <= 16 refuses to route (topk_idx -1,
 * topk_w and y NaN): its logit hand-over slots may hold stale values after a timeout.
 * --------------------------------------------------------------------------------------- */
#define MOE_WS_STATUS_OFFSET 0
#define MOE_WS_ROUTE_TIMEOUT 0x1u
#define MOE_WS_BAD_EXPERT_ID 0x2u

/* Bytes of workspace the entry points need for T tokens (moe_layer needs the most; every
 * other call needs no more).  Returns 0 for a bad shape or T. */
size_t moe_workspace_bytes(const moe_shape *shape, int32_t T);

/* Prepare a workspace before its first use, or again after a nonzero status: clears the status
 * word and the few-token router's logit hand-over slots with a fill kernel on `stream` (so it
 * can be captured in a graph; no memset node).  A workspace that is all zero bytes is already
 * prepared with poll_limit 0.  poll_limit: 0 for the default (2^20 polls, far beyond any
 * launch); n > 0 lets the few-token router poll its hand-over slots at most n times; n < 0 makes
 * it give up at once, without polling (a test of the failure path: every kernel still ends
 * normally).  ws_bytes must cover moe_workspace_bytes(shape, T). */
moe_status moe_workspace_init(const moe_shape *shape, int32_t T, void *ws, size_t ws_bytes,
                              int32_t poll_limit, hipStream_t stream);

/* Fill a DEVICE expert table from n_experts + n_shared blobs laid out at base + e * stride
 * (stride >= moe_blob_stride, a multiple of 16; base 16-byte aligned); blob n_experts is the
 * shared expert when n_shared = 1.  For NVFP4 the tensor scales are read from the blobs on the
 * device.  table: [n_experts + n_shared] moe_expert in device memory. */
moe_status moe_fill_table(const moe_shape *shape, const void *base, size_t stride,
                          moe_expert *table, hipStream_t stream);

/* Router ([Maya] "What is in the 96.5 GB": one F32 router per layer; "Three tiers ...":
 * routed on the device).  For each token t:
 *   l[t,e]   = sum_i x[t,i] * w_router[e,i] (+ logit_bias[e]), accumulated in fp64 (each
 *              product is exact in fp64), so the selection is that of the fp64 logits;
 *   topk_idx = the top_k experts by (l descending, expert index ascending) - ties go to the
 *              lower index ([Maya] "Steady speed with depth": the radix select breaks ties
 *              by the lower index) - written in that order; a NaN logit ranks last;
 *   topk_w   = sigmoid(l_sel) / sum_j sigmoid(l_sel)  (renormalised over the kept experts,
 *              [Strata] "Uncensoring without touching the weights"); with renorm_skip, the
 *              dropped picks get topk_idx -1 and topk_w 0 and the sum runs over the kept ones.
 * x: [T][d_model] act_dtype; w_router: [n_experts][d_model] fp32; logit_bias: [n_experts]
 * fp32 or NULL; topk_idx: [T][top_k] int32; topk_w: [T][top_k] fp32. */
moe_status moe_route(const moe_shape *shape, const void *x, int32_t T, const float *w_router,
                     const float *logit_bias, int32_t *topk_idx, float *topk_w, void *ws,
                     size_t ws_bytes, hipStream_t stream);

/* Group the T*top_k picks (pick p = t*top_k + j) by expert, on the device ([HotCache] "A
 * gather kernel that reads wide": the expert list stays on the GPU): a counting sort,
 * stable in pick order.
 * expert_offsets: [n_experts+1], picks of expert e are sorted positions
 *   [expert_offsets[e], expert_offsets[e+1]);  sorted_pick: [T*top_k] pick id at each
 *   sorted position;  pick_pos: [T*top_k] sorted position of each pick (inverse).
 * A pick with expert id -1 (dropped by renorm_skip) takes no position: pick_pos -1, and the
 *   sorted positions past expert_offsets[n_experts] hold -1.  Any other id outside
 *   [0, n_experts) is refused the same way and sets MOE_WS_BAD_EXPERT_ID in the workspace's
 *   status word when a workspace is given.
 * ws / ws_bytes: NULL, or the workspace of moe_workspace_bytes(shape, T) bytes (less is
 *   MOE_ERR_WORKSPACE).  With it, 4096 or more picks are sorted by one workgroup per 1024 picks,
 *   whose per-block expert counts it holds; without it one workgroup sorts them all.  The
 *   result is the same either way. */
moe_status moe_permute(const moe_shape *shape, const int32_t *topk_idx, int32_t T,
                       int32_t *expert_offsets, int32_t *sorted_pick, int32_t *pick_pos,
                       void *ws, size_t ws_bytes, hipStream_t stream);

/* Copy the n experts listed in d_list (device int32 expert ids) from the blobs referenced by
 * d_table into `staging` (n * moe_blob_stride bytes, 256-byte aligned) with wide loads, and
 * write a table for the staged copies into d_staged_table ([n] device moe_expert) -
 * the device-list gather of [HotCache] "A gather kernel that reads wide" and "Prefill in
 * groups of 64 experts".  Entry i of d_staged_table describes expert d_list[i]. */
moe_status moe_gather_experts(const moe_shape *shape, const moe_expert *d_table,
                              const int32_t *d_list, int32_t n, void *staging,
                              moe_expert *d_staged_table, hipStream_t stream);

/* Expert FFN for every pick ([Maya] "What is in the 96.5 GB": an expert is gate, up and
 * down): with W dequantised on the fly from its block-scaled codes,
 *   o_i = W_down,e (silu(W_gate,e x_t) * (W_up,e x_t)),  silu(g) = g * sigmoid(g),
 * for each sorted position i < expert_offsets[n_experts] with pick p = sorted_pick[i], token
 * t = p / top_k, and e the expert whose range [expert_offsets[e], expert_offsets[e+1]) holds i.
 * With n_shared = 1, rows T*top_k + t (t < T) are the shared expert's o for token t.
 * o: [T*top_k + T*n_shared][d_model] fp32, row i = sorted position i (rows of positions past
 * expert_offsets[n_experts] and below T*top_k are not written).  MXFP4 weights enter the scaled
 * FP4 matrix cores as they are; NVFP4 weights are dequantised in registers to bf16 (code x E4M3
 * block scale is exact in bf16), the tensor scales applied to the fp32 sums. */
moe_status moe_expert_ffn(const moe_shape *shape, const moe_expert *d_table, const void *x,
                          int32_t T, const int32_t *expert_offsets, const int32_t *sorted_pick,
                          float *o, void *ws, size_t ws_bytes, hipStream_t stream);

/* Route-weighted combine: y[t] = routed_scaling * sum_j topk_w[t,j] * o[pick_pos[t*k+j]]
 * (+ o[T*k + t] with n_shared = 1) (+ residual[t]), summed over j in order (picks with
 * pick_pos -1 left out), rounded once to act_dtype (nearest-even).
 * residual: [T][d_model] act_dtype or NULL; y: [T][d_model] act_dtype. */
moe_status moe_combine(const moe_shape *shape, const float *o, const float *topk_w,
                       const int32_t *pick_pos, int32_t T, const void *residual, void *y,
                       hipStream_t stream);

/* The whole layer: moe_route, moe_permute, moe_expert_ffn and moe_combine on the stream,
 * with the intermediates in the workspace (prepared by moe_workspace_init or zero-filled).
 * For MXFP4 with T <= 16 (and T * top_k <= 512, top_k <= 64) the layer runs as three launches:
 * the router fused with the grouping, the tile records and the activation split; the gate/up
 * GEMM; and the down GEMM fused with the combine.  topk_idx_out / topk_w_out ([T][top_k],
 * device) are optional copies of the routing.  y may not alias x; it may alias residual.
 * staging: NULL, or (NVFP4 only) a device buffer of min(n_experts, 64) * moe_blob_stride bytes,
 * 16-byte aligned: the distinct selected experts are then copied into it 64 at a time by a
 * device-resident list (moe_gather_experts' copy), and each group's tiles read the staged copies
 * ("A hot expert cache made a 181 GiB model faster ...", sections "A gather kernel that reads
 * wide" and "Prefill in groups of 64 experts").  A non-NULL staging with MXFP4 is
 * MOE_ERR_INVALID. */
moe_status moe_layer(const moe_shape *shape, const void *x, int32_t T, const float *w_router,
                     const float *logit_bias, const moe_expert *d_table, void *staging,
                     const void *residual, void *y, int32_t *topk_idx_out, float *topk_w_out,
                     void *ws, size_t ws_bytes, hipStream_t stream);

/* Per-call observation of the kernels a call enqueues (measuring each step where it runs, as the
 * pages write a measurement next to each design rule: [Maya] "Three tiers and the rules between
 * them").  Both hooks are optional and run on the calling host thread, for that call only.
 *  trace_hook(trace_user, kernel, 0, stream) right before each kernel is enqueued and
 *    (..., 1, stream) right after; `kernel` is a static name ("router_logits", "topk",
 *    "route_small", "act_split", "permute", "plan", "gemm_gate_up", "gemm_down",
 *    "down_combine", "combine", "stage_plan", "gather").
 *  event_hook(event_user, kernel, &start, &stop) right before each kernel is enqueued, with
 *    start = stop = NULL.  If it sets both to HIP events it created, the kernel is launched with
 *    hipExtLaunchKernel, which records them when the kernel itself starts and ends (the dispatch
 *    timestamps a profiler reads), so hipEventElapsedTime(start, stop) is that kernel's duration
 *    without launch gaps.  Do not set events while the stream is being captured. */
typedef void (*moe_trace_hook)(void *user, const char *kernel, int phase, hipStream_t stream);
typedef void (*moe_event_hook)(void *user, const char *kernel, hipEvent_t *start, hipEvent_t *stop);
typedef struct {
    moe_trace_hook trace_hook;
    void *trace_user;
    moe_event_hook event_hook;
    void *event_user;
} moe_observer;

/* moe_layer with an observer (NULL: exactly moe_layer). */
moe_status moe_layer_observed(const moe_shape *shape, const void *x, int32_t T, const float *w_router,
                              const float *logit_bias, const moe_expert *d_table, void *staging,
                              const void *residual, void *y, int32_t *topk_idx_out, float *topk_w_out,
                              void *ws, size_t ws_bytes, hipStream_t stream, const moe_observer *observer);

/* moe_layer for callers that cannot allocate device memory - code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc - with the same arguments minus the staging buffer
 * and the workspace.  Its intermediates live in a scratch array inside the library: 32 MiB of
 * device memory per GPU the library runs on, held until the process ends.  Shapes and token counts
 * whose moe_workspace_bytes-style layout needs more (at d_model 4096, d_ff 2048, 288 experts: more
 * than 64 tokens) return MOE_ERR_WORKSPACE.  The call allocates nothing: no hipMalloc, no hipFree,
 * no allocating library routine; its first call on a device clears the array's status word and
 * hand-over slots with a fill kernel on `stream`.  Every call on one GPU shares that GPU's array:
 * calls that overlap in time on one GPU race (run them on one stream, or serialise them).  The
 * array's status word cannot be read by the caller; a router timeout shows as idx -1 and NaN y,
 * and the array then refuses to route for the rest of the process. */
moe_status moe_layer_noalloc(const moe_shape *shape, const void *x, int32_t T, const float *w_router,
                             const float *logit_bias, const moe_expert *d_table, const void *residual,
                             void *y, int32_t *topk_idx_out, float *topk_w_out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
