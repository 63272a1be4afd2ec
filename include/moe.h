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
 *  - Thread safety: the library holds no state; concurrent calls are safe when they
 *    use distinct workspaces and outputs.
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

#define MOE_ABI_VERSION 1

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
 * routed_scaling_factor); 1.0 leaves the normalised route weights as they are. */
typedef struct {
    int32_t d_model;
    int32_t d_ff;
    int32_t n_experts;
    int32_t top_k;
    int32_t wformat;      /* moe_wformat */
    int32_t act_dtype;    /* moe_dtype   */
    float routed_scaling;
} moe_shape;

/* One expert's weights: gate and up are [d_ff][d_model], down is [d_model][d_ff], each as
 * packed codes q[rows][K/2] plus scales s[rows][K/B] (K = the row length, B = block size).
 * The table of n_experts entries lives in DEVICE memory ([Maya] "Three tiers and the rules
 * between them": the router looks its experts up in a device table).  Code pointers must be
 * 16-byte aligned.  The *_ts fields are the NVFP4 tensor scales (ignored for MXFP4). */
typedef struct {
    const uint8_t *gate_q, *up_q, *down_q;
    const uint8_t *gate_s, *up_s, *down_s;
    float gate_ts, up_ts, down_ts, reserved;
} moe_expert;

/* Limits: 1 <= top_k <= n_experts <= 1024; d_model and d_ff multiples of 128; d_ff a
 * multiple of 32 rows per output tile as well (always true then); T <= 65536.
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

/* Bytes of workspace the entry points need for T tokens (moe_layer needs the most; every
 * other call needs no more).  Returns 0 for a bad shape or T.  A workspace must be zero-filled
 * once before its first use (a memset at allocation): for T <= 16, moe_layer hands the router
 * logits over through slots in it that every call leaves at zero again.  Calls that overlap in
 * time need distinct workspaces. */
size_t moe_workspace_bytes(const moe_shape *shape, int32_t T);

/* Fill a DEVICE expert table from n_experts blobs laid out at base + e * stride (stride >=
 * moe_blob_stride, a multiple of 16; base 16-byte aligned).  For NVFP4 the tensor scales are
 * read from the blobs on the device.  table: [n_experts] moe_expert in device memory. */
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
 *              [Strata] "Uncensoring without touching the weights").
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
 * Expert ids in topk_idx must be in [0, n_experts).
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
 * for each sorted position i with pick p = sorted_pick[i], token t = p / top_k, and e the
 * expert whose range [expert_offsets[e], expert_offsets[e+1]) holds i.
 * o: [T*top_k][d_model] fp32, row i = sorted position i.  MXFP4 weights enter the scaled FP4
 * matrix cores as they are; NVFP4 weights are dequantised in registers to bf16 (code x E4M3
 * block scale is exact in bf16), the tensor scales applied to the fp32 sums. */
moe_status moe_expert_ffn(const moe_shape *shape, const moe_expert *d_table, const void *x,
                          int32_t T, const int32_t *expert_offsets, const int32_t *sorted_pick,
                          float *o, void *ws, size_t ws_bytes, hipStream_t stream);

/* Route-weighted combine: y[t] = routed_scaling * sum_j topk_w[t,j] * o[pick_pos[t*k+j]]
 * (+ residual[t]), summed over j in order, rounded once to act_dtype (nearest-even).
 * residual: [T][d_model] act_dtype or NULL; y: [T][d_model] act_dtype. */
moe_status moe_combine(const moe_shape *shape, const float *o, const float *topk_w,
                       const int32_t *pick_pos, int32_t T, const void *residual, void *y,
                       hipStream_t stream);

/* Tracing hook.  When set (non-NULL), every entry point calls hook(user, kernel, 0, stream)
 * right before it enqueues each of its kernels and hook(user, kernel, 1, stream) right after,
 * on the calling host thread; `kernel` is a static name ("router_logits", "topk",
 * "act_split", "permute", "plan", "gemm_gate_up", "gemm_down", "combine", "fill_table",
 * "gather").  A hook may record HIP events on `stream` to time one kernel in place (inside
 * stream capture those become graph nodes).  This is the only process-wide state in the
 * library; setting it while other threads are inside the library is a race.  Measuring each
 * step where it runs follows the pages' practice of writing the measurement next to each design
 * rule ("Project Maya ...", section "Three tiers and the rules between them"). */
typedef void (*moe_trace_hook)(void *user, const char *kernel, int phase, hipStream_t stream);
void moe_set_trace_hook(moe_trace_hook hook, void *user);

/* Kernel timing hook.  When set, every entry point calls hook(user, kernel, &start, &stop) right
 * before it enqueues each kernel (same names as the tracing hook), with start = stop = NULL.
 * If the hook sets both to HIP events it created, the kernel is enqueued with
 * hipExtLaunchKernel, which records them when the kernel itself starts and ends (the dispatch
 * timestamps a profiler reads), so hipEventElapsedTime(start, stop) is the kernel's duration
 * without any launch gap.  Leave them NULL to launch normally.  Do not set events while the
 * stream is being captured.  Process-wide, like the tracing hook. */
typedef void (*moe_event_hook)(void *user, const char *kernel, hipEvent_t *start, hipEvent_t *stop);
void moe_set_event_hook(moe_event_hook hook, void *user);

/* The whole layer: moe_route, moe_permute, moe_expert_ffn and moe_combine on the stream,
 * with the intermediates in the workspace (zero-filled before its first use).  For MXFP4 with
 * T <= 16 (and T * top_k <= 512, top_k <= 64) the layer runs as three launches: the router fused
 * with the grouping, the tile records and the activation split; the gate/up GEMM; and the down
 * GEMM fused with the combine.  topk_idx_out / topk_w_out ([T][top_k], device) are optional
 * copies of the routing.  y may not alias x; it may alias residual.
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

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
