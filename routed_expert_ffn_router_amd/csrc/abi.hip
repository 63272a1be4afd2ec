// Host side of the C ABI: argument validation (before any launch), workspace layout and the
// launch sequence of each entry point.
#include <math.h>
#include <string.h>

#include <mutex>

#include "moe_internal.h"

namespace moe {

constexpr int kSmallTokens = 16;   // moe_layer's fused three-launch path

// The observer of the call in progress on this thread (moe_layer_observed), null otherwise: it
// lives only for the duration of that call, so the library keeps no state between calls.
static thread_local const moe_observer* t_obs = nullptr;
static thread_local hipEvent_t t_launch_ev[2] = {nullptr, nullptr};

struct ObserverScope {
    explicit ObserverScope(const moe_observer* o) { t_obs = o; }
    ~ObserverScope() {
        t_obs = nullptr;
        t_launch_ev[0] = t_launch_ev[1] = nullptr;
    }
};

void trace(const char* kernel, int phase, hipStream_t st) {
    t_launch_ev[0] = t_launch_ev[1] = nullptr;
    if (!t_obs) return;
    if (t_obs->trace_hook) t_obs->trace_hook(t_obs->trace_user, kernel, phase, st);
    if (phase == 0 && t_obs->event_hook) {
        t_obs->event_hook(t_obs->event_user, kernel, &t_launch_ev[0], &t_launch_ev[1]);
        if (!t_launch_ev[0] || !t_launch_ev[1]) t_launch_ev[0] = t_launch_ev[1] = nullptr;
    }
}

hipEvent_t launch_event(int which) { return t_launch_ev[which]; }

static size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// activation terms per value: the opt-in MXFP8 mode takes one (the quantised value itself); the
// exact mode two for bf16 and four for fp32 activations (their residuals are exact)
int act_terms(const moe_shape* s) {
    if (s->act_quant == MOE_AQ_MXFP8) return 1;
    return s->act_dtype == MOE_DT_BF16 ? 2 : 4;
}

WsLayout ws_layout(const moe_shape* s, int32_t T, bool slots_for_any_shape) {
    WsLayout L;
    memset(&L, 0, sizeof L);
    const size_t E = s->n_experts, k = s->top_k, d = s->d_model, f = s->d_ff;
    const size_t P = (size_t)T * k;
    L.nt = act_terms(s);
    const bool nv = s->wformat == MOE_WF_NVFP4;
    const int variant = gemm_variant(s, T);
    size_t tt = (size_t)gemm_tile_tokens(variant, L.nt);
    // the fused few-token path tiles with the smaller few-token tile: bound for both
    if (T <= kSmallTokens && (size_t)gemm_tile_tokens(0, L.nt) < tt) tt = (size_t)gemm_tile_tokens(0, L.nt);
    if (nv) tt = kNvTilePicks;
    // routed tiles, then the shared expert's T picks (positions P .. P + T - 1)
    const size_t Pall = P + (s->n_shared ? (size_t)T : 0);
    L.max_tiles = (int)((E < P ? E : P) + P / tt + 1 + (s->n_shared ? (size_t)T / tt + 1 : 0));
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t at = o; o += align256(bytes); return at; };
    // status word and poll limit (MOE_WS_STATUS_OFFSET = 0), then the fused router's logit
    // hand-over: the same bytes in the layout of every T, used by nothing else, so that calls with
    // different T on one workspace keep them
    L.hdr = take(kWsHeaderBytes);
    L.slots = take(8 * (size_t)kSmallTokens * (slots_for_any_shape ? (size_t)kMaxExperts : E));
    // write-only scratch of the one-token router's warm-up pass
    const size_t sink_rec = sizeof(TileDesc) * (size_t)L.max_tiles, sink_slots = 8 * (E + 1);
    L.sink = take(sink_rec > sink_slots ? sink_rec : sink_slots);
    L.logits = take(8 * (size_t)T * E * (size_t)logits_splits(s, T));   // partial slices of the tiled router
    L.idx = take(4 * P);
    L.w = take(4 * P);
    L.offsets = take(4 * (E + 1));
    L.sorted_pick = take(4 * P);
    L.pick_pos = take(4 * P);
    L.perm_blocks = take(4 * ((P + 1023) / 1024) * E);
    L.tiles = take(8 * (size_t)L.max_tiles);
    L.ntiles = take(4);
    L.desc = take(sizeof(TileDesc) * (size_t)L.max_tiles);
    if (nv) {
        // bf16 terms: x as two terms when it is fp32, h always as two
        L.xq = take((size_t)T * 2 * d * 2);
        L.xs = take(0);
        L.hq = take(Pall * 2 * f * 2);
        L.hs = take(0);
    } else {
        L.xq = take((size_t)T * L.nt * d);
        L.xs = take((size_t)T * L.nt * d / 32);
        L.hq = take(Pall * L.nt * f);
        L.hs = take(Pall * L.nt * f / 32);
    }
    L.o = take(4 * Pall * d);
    if (nv) {
        L.stage_table = take(sizeof(moe_expert) * (E + s->n_shared));   // the shared expert's entry last
        L.stage_list = take(4 * E);
        L.stage_n = take(4);
        L.stage_ranges = take(8 * ((E + kStageGroup - 1) / kStageGroup));
    }
    L.total = o;
    return L;
}

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

static moe_status check_shape(const moe_shape* s) {
    if (!s) return MOE_ERR_INVALID;
    if (s->d_model <= 0 || s->d_ff <= 0 || s->n_experts <= 0 || s->top_k <= 0) return MOE_ERR_INVALID;
    if (s->top_k > s->n_experts) return MOE_ERR_INVALID;
    if (s->wformat != MOE_WF_MXFP4 && s->wformat != MOE_WF_NVFP4) return MOE_ERR_INVALID;
    if (s->act_dtype != MOE_DT_F32 && s->act_dtype != MOE_DT_BF16) return MOE_ERR_INVALID;
    if (!isfinite(s->routed_scaling)) return MOE_ERR_INVALID;
    if (!isfinite(s->renorm_skip) || s->renorm_skip < 0.0f || s->renorm_skip >= 1.0f) return MOE_ERR_INVALID;
    if (s->n_shared != 0 && s->n_shared != 1) return MOE_ERR_INVALID;
    if (s->act_quant != MOE_AQ_EXACT && s->act_quant != MOE_AQ_MXFP8) return MOE_ERR_INVALID;
    if (s->act_quant == MOE_AQ_MXFP8 && s->wformat != MOE_WF_MXFP4) return MOE_ERR_UNSUPPORTED;
    if (s->renorm_skip > 0.0f && s->top_k > 64) return MOE_ERR_UNSUPPORTED;
    if (s->n_experts > 1024) return MOE_ERR_UNSUPPORTED;
    if (s->d_model % 128 != 0 || s->d_ff % 128 != 0) return MOE_ERR_UNSUPPORTED;
    if ((long long)s->d_model * s->d_ff > (1LL << 30)) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

static moe_status check_T(const moe_shape* s, int32_t T) {
    if (T < 0) return MOE_ERR_INVALID;
    if (T > 65536) return MOE_ERR_UNSUPPORTED;
    (void)s;
    return MOE_OK;
}

static moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

#define MOE_TRY(expr)                              \
    do {                                           \
        moe_status st_ = (expr);                   \
        if (st_ != MOE_OK) return st_;             \
    } while (0)
#define MOE_HIP(expr)                              \
    do {                                           \
        if ((expr) != hipSuccess) return MOE_ERR_HIP; \
    } while (0)

static GemmArgs gemm_args(const moe_shape* s, const moe_expert* table, int32_t T, const int32_t* sorted_pick,
                          const int32_t* offsets, uint8_t* ws, const WsLayout& L, float* o) {
    GemmArgs a;
    a.table = table;
    a.d = s->d_model;
    a.f = s->d_ff;
    a.E = s->n_experts;
    a.k = s->top_k;
    a.P = T * s->top_k;
    a.Pall = a.P + (s->n_shared ? T : 0);
    a.sorted_pick = sorted_pick;
    a.tiles = (const int32_t*)(ws + L.tiles);
    a.ntiles = (const int32_t*)(ws + L.ntiles);
    a.offsets = offsets;
    a.desc = (const TileDesc*)(ws + L.desc);
    a.max_tiles = L.max_tiles;
    a.aq = ws + L.xq;
    a.as = ws + L.xs;
    a.hq = ws + L.hq;
    a.hs = ws + L.hs;
    a.o = o;
    a.tile_range = nullptr;
    return a;
}

// NVFP4: plan tiles of kNvTilePicks picks, bf16 terms of an fp32 x, then gate/up and down on the
// bf16 matrix cores; with staging, the distinct experts are first copied into the staging buffer
// kStageGroup at a time and each group's tiles run from the staged copies
// planned: the tile plan is already in the workspace (the fused router wrote it)
static moe_status run_ffn_nv(const moe_shape* s, const moe_expert* table, const void* x, int32_t T,
                             const int32_t* offsets, const int32_t* sorted_pick, float* o, uint8_t* ws,
                             const WsLayout& L, void* staging, hipStream_t st, bool planned = false) {
    const int tt = nv_tile_picks(s, T);
    int32_t* tiles = (int32_t*)(ws + L.tiles);
    int32_t* ntiles = (int32_t*)(ws + L.ntiles);
    if (!planned) MOE_HIP(launch_plan(s, offsets, T, tt, tiles, ntiles, st));
    const bool bf = s->act_dtype == MOE_DT_BF16;
    const int NT = bf ? 1 : 2;      // bf16 terms of x and of h: one with bf16 activations, two with fp32
    if (!bf) MOE_HIP(launch_bf16_terms((const float*)x, T, s->d_model, (uint16_t*)(ws + L.xq), st));
    GemmArgs a = gemm_args(s, table, T, sorted_pick, offsets, ws, L, o);
    // the few-token router's tile records name the table's experts: used in place only
    if (!planned || staging) a.desc = nullptr;
    const uint8_t* xin = bf ? (const uint8_t*)x : ws + L.xq;
    if (!staging) {
        a.aq = xin;
        MOE_HIP(launch_nv_gemm(a, true, NT, tt, L.max_tiles, st));
        a.aq = ws + L.hq;
        MOE_HIP(launch_nv_gemm(a, false, NT, tt, L.max_tiles, st));
        return MOE_OK;
    }
    int32_t* list = (int32_t*)(ws + L.stage_list);
    int32_t* nlist = (int32_t*)(ws + L.stage_n);
    int32_t* ranges = (int32_t*)(ws + L.stage_ranges);
    moe_expert* staged = (moe_expert*)(ws + L.stage_table);
    MOE_HIP(launch_stage_plan(s, offsets, tt, ntiles, list, nlist, ranges, table, staged, st));
    const size_t stride = moe_blob_stride(s);
    const long long P = (long long)T * s->top_k;
    const long long distinct = P < s->n_experts ? P : s->n_experts;
    const int groups = (int)((distinct + kStageGroup - 1) / kStageGroup);
    a.table = staged;
    for (int g = 0; g < groups; ++g) {
        MOE_HIP(launch_gather_group(s, table, list, nlist, g, (uint8_t*)staging, stride, staged, st));
        a.tile_range = ranges + 2 * g;
        a.aq = xin;
        MOE_HIP(launch_nv_gemm(a, true, NT, tt, L.max_tiles, st));
        a.aq = ws + L.hq;
        MOE_HIP(launch_nv_gemm(a, false, NT, tt, L.max_tiles, st));
    }
    return MOE_OK;
}

// sequence shared by moe_expert_ffn and moe_layer (general token counts)
static moe_status run_ffn(const moe_shape* s, const moe_expert* table, const void* x, int32_t T,
                          const int32_t* offsets, const int32_t* sorted_pick, float* o, uint8_t* ws,
                          const WsLayout& L, hipStream_t st) {
    if (s->wformat == MOE_WF_NVFP4) return run_ffn_nv(s, table, x, T, offsets, sorted_pick, o, ws, L, nullptr, st);
    const int variant = gemm_variant(s, T);
    const int NT = L.nt;
    const int tt = gemm_tile_tokens(variant, NT);
    MOE_HIP(launch_plan(s, offsets, T, tt, (int32_t*)(ws + L.tiles), (int32_t*)(ws + L.ntiles), st));
    const int SS1 = act_super_step(s->d_model, variant);
    MOE_HIP(launch_act_split(s, x, T, s->d_model, SS1, NT, ws + L.xq, ws + L.xs, st));
    GemmArgs a = gemm_args(s, table, T, sorted_pick, offsets, ws, L, o);
    MOE_HIP(launch_gemm_gateup(a, NT, variant, L.max_tiles, st));
    a.aq = ws + L.hq;
    a.as = ws + L.hs;
    MOE_HIP(launch_gemm_down(a, NT, variant, L.max_tiles, st));
    return MOE_OK;
}

}  // namespace moe

namespace moe {

// ---------------------------------------------------------------------------------------------
// moe_layer_noalloc's scratch: a device array of the library, one copy per GPU, for callers that
// cannot allocate.  Host code never passes the array's name to a kernel or a copy (in host code it
// is a stand-in, not a device address): each device's address comes from hipGetSymbolAddress,
// taken once per device with that device current, and the kernels receive that address.
// ---------------------------------------------------------------------------------------------
constexpr size_t kScratchBytes = (size_t)32 << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
static std::mutex g_scratch_mu;
static uint8_t* g_scratch_ptr[kMaxDevices] = {};

// the current device's scratch address; the first call on a device also clears the array's status
// word and logit hand-over slots (a fill kernel on `st`, ahead of the layer's kernels)
static moe_status device_scratch(hipStream_t st, uint8_t** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
        const size_t end = kWsHeaderBytes + 8 * (size_t)kSmallTokens * kMaxExperts;   // header + slots
        static_assert(kWsHeaderBytes + 8 * (size_t)kSmallTokens * kMaxExperts <= kScratchBytes, "slots fit");
        if (launch_ws_init((uint32_t*)p, end / 4, 0, st) != hipSuccess) return MOE_ERR_HIP;
        g_scratch_ptr[dev] = (uint8_t*)p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

static moe_status check_layer_args(const moe_shape* s, const void* x, const float* w_router,
                                   const moe_expert* d_table, const void* staging, const void* residual,
                                   const void* y) {
    if (!x || !w_router || !d_table || !y) return MOE_ERR_INVALID;
    if (!aligned(x, 16) || !aligned(y, 16) || !aligned(w_router, 16) || (residual && !aligned(residual, 16)) ||
        (staging && !aligned(staging, 16)))
        return MOE_ERR_INVALID;
    if (x == y) return MOE_ERR_INVALID;
    if (staging && s->wformat != MOE_WF_NVFP4) return MOE_ERR_INVALID;      // staging is the NVFP4 gather path
    return MOE_OK;
}

static moe_status layer_launches(const moe_shape* s, const void* x, int32_t T, const float* w_router,
                                 const float* logit_bias, const moe_expert* d_table, void* staging,
                                 const void* residual, void* y, int32_t* topk_idx_out, float* topk_w_out,
                                 uint8_t* w8, const WsLayout& L, hipStream_t stream);

}  // namespace moe

using namespace moe;

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(moe_status status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported shape or size";
        case MOE_ERR_WORKSPACE: return "workspace too small";
        case MOE_ERR_HIP: return "HIP launch failed";
    }
    return "unknown status";
}

size_t moe_blob_stride(const moe_shape* s) {
    if (check_shape(s) != MOE_OK) return 0;
    const size_t B = s->wformat == MOE_WF_MXFP4 ? 32 : 16;
    const size_t fd = (size_t)s->d_model * s->d_ff;
    size_t n = 3 * (fd / 2) + 3 * (fd / B);
    if (s->wformat == MOE_WF_NVFP4) n = (n + 12 + 255) / 256 * 256;
    return n;
}

size_t moe_workspace_bytes(const moe_shape* s, int32_t T) {
    if (check_shape(s) != MOE_OK || check_T(s, T) != MOE_OK) return 0;
    return ws_layout(s, T).total;
}

moe_status moe_workspace_init(const moe_shape* s, int32_t T, void* ws, size_t ws_bytes, int32_t poll_limit,
                              hipStream_t stream) {
    MOE_TRY(check_shape(s));
    MOE_TRY(check_T(s, T));
    if (!ws) return MOE_ERR_INVALID;
    if (!aligned(ws, 256)) return MOE_ERR_INVALID;
    const WsLayout L = ws_layout(s, T);
    if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    // the header and the hand-over slots are the workspace's first bytes (one range)
    const size_t end = L.slots + 8 * (size_t)kSmallTokens * s->n_experts;
    return hip_status(launch_ws_init((uint32_t*)ws, end / 4, poll_limit, stream));
}

moe_status moe_fill_table(const moe_shape* s, const void* base, size_t stride, moe_expert* table,
                          hipStream_t stream) {
    MOE_TRY(check_shape(s));
    if (!base || !table) return MOE_ERR_INVALID;
    if (!aligned(base, 16) || stride % 16 != 0 || stride < moe_blob_stride(s)) return MOE_ERR_INVALID;
    return hip_status(launch_fill_table(s, (const uint8_t*)base, stride, table, stream));
}

moe_status moe_route(const moe_shape* s, const void* x, int32_t T, const float* w_router,
                     const float* logit_bias, int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
    MOE_TRY(check_shape(s));
    MOE_TRY(check_T(s, T));
    if (T == 0) return MOE_OK;
    if (!x || !w_router || !topk_idx || !topk_w || !ws) return MOE_ERR_INVALID;
    if (!aligned(x, 16) || !aligned(w_router, 16) || !aligned(ws, 256)) return MOE_ERR_INVALID;
    const WsLayout L = ws_layout(s, T);
    if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    uint8_t* w8 = (uint8_t*)ws;
    double* logits = (double*)(w8 + L.logits);
    MOE_HIP(launch_router_logits(s, x, T, w_router, logit_bias, logits, stream));
    MOE_HIP(launch_topk(s, logits, T, topk_idx, topk_w, stream));
    return MOE_OK;
}

moe_status moe_permute(const moe_shape* s, const int32_t* topk_idx, int32_t T, int32_t* expert_offsets,
                       int32_t* sorted_pick, int32_t* pick_pos, void* ws, size_t ws_bytes, hipStream_t stream) {
    MOE_TRY(check_shape(s));
    MOE_TRY(check_T(s, T));
    if (!topk_idx || !expert_offsets || !sorted_pick || !pick_pos) return MOE_ERR_INVALID;
    if (T == 0) return MOE_OK;
    int32_t* bcnt = nullptr;         // with a workspace, many picks are sorted by many workgroups
    uint32_t* status = nullptr;
    if (ws) {
        if (!aligned(ws, 256)) return MOE_ERR_INVALID;
        const WsLayout L = ws_layout(s, T);
        if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
        bcnt = (int32_t*)((uint8_t*)ws + L.perm_blocks);
        status = (uint32_t*)((uint8_t*)ws + L.hdr);
    }
    return hip_status(launch_permute(s, topk_idx, T, expert_offsets, sorted_pick, pick_pos, bcnt, status, stream));
}

moe_status moe_gather_experts(const moe_shape* s, const moe_expert* d_table, const int32_t* d_list, int32_t n,
                              void* staging, moe_expert* d_staged_table, hipStream_t stream) {
    MOE_TRY(check_shape(s));
    if (n < 0) return MOE_ERR_INVALID;
    if (n == 0) return MOE_OK;
    if (!d_table || !d_list || !staging || !d_staged_table) return MOE_ERR_INVALID;
    if (!aligned(staging, 256)) return MOE_ERR_INVALID;
    const size_t stride = (moe_blob_stride(s) + 255) / 256 * 256;
    return hip_status(launch_gather(s, d_table, d_list, n, (uint8_t*)staging, stride, d_staged_table, stream));
}

moe_status moe_expert_ffn(const moe_shape* s, const moe_expert* d_table, const void* x, int32_t T,
                          const int32_t* expert_offsets, const int32_t* sorted_pick, float* o, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
    MOE_TRY(check_shape(s));
    MOE_TRY(check_T(s, T));
    if (T == 0) return MOE_OK;
    if (!d_table || !x || !expert_offsets || !sorted_pick || !o || !ws) return MOE_ERR_INVALID;
    if (!aligned(x, 16) || !aligned(o, 16) || !aligned(ws, 256)) return MOE_ERR_INVALID;
    const WsLayout L = ws_layout(s, T);
    if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    return run_ffn(s, d_table, x, T, expert_offsets, sorted_pick, o, (uint8_t*)ws, L, stream);
}

moe_status moe_combine(const moe_shape* s, const float* o, const float* topk_w, const int32_t* pick_pos,
                       int32_t T, const void* residual, void* y, hipStream_t stream) {
    MOE_TRY(check_shape(s));
    MOE_TRY(check_T(s, T));
    if (T == 0) return MOE_OK;
    if (!o || !topk_w || !pick_pos || !y) return MOE_ERR_INVALID;
    if (!aligned(o, 16) || !aligned(y, 16) || (residual && !aligned(residual, 16))) return MOE_ERR_INVALID;
    return hip_status(launch_combine(s, o, topk_w, pick_pos, T, residual, y, stream));
}

moe_status moe_layer(const moe_shape* s, const void* x, int32_t T, const float* w_router,
                     const float* logit_bias, const moe_expert* d_table, void* staging, const void* residual,
                     void* y, int32_t* topk_idx_out, float* topk_w_out, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
    return moe_layer_observed(s, x, T, w_router, logit_bias, d_table, staging, residual, y, topk_idx_out,
                              topk_w_out, ws, ws_bytes, stream, nullptr);
}

moe_status moe_layer_observed(const moe_shape* s, const void* x, int32_t T, const float* w_router,
                              const float* logit_bias, const moe_expert* d_table, void* staging,
                              const void* residual, void* y, int32_t* topk_idx_out, float* topk_w_out, void* ws,
                              size_t ws_bytes, hipStream_t stream, const moe_observer* observer) {
    ObserverScope scope(observer);
    MOE_TRY(check_shape(s));
    MOE_TRY(check_T(s, T));
    if (T == 0) return MOE_OK;
    if (!ws) return MOE_ERR_INVALID;
    MOE_TRY(check_layer_args(s, x, w_router, d_table, staging, residual, y));
    if (!aligned(ws, 256)) return MOE_ERR_INVALID;
    const WsLayout L = ws_layout(s, T);
    if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    return layer_launches(s, x, T, w_router, logit_bias, d_table, staging, residual, y, topk_idx_out, topk_w_out,
                          (uint8_t*)ws, L, stream);
}

moe_status moe_layer_noalloc(const moe_shape* s, const void* x, int32_t T, const float* w_router,
                             const float* logit_bias, const moe_expert* d_table, const void* residual, void* y,
                             int32_t* topk_idx_out, float* topk_w_out, hipStream_t stream) {
    MOE_TRY(check_shape(s));
    MOE_TRY(check_T(s, T));
    if (T == 0) return MOE_OK;
    MOE_TRY(check_layer_args(s, x, w_router, d_table, nullptr, residual, y));
    // every shape lays out the array with hand-over slots for the largest expert count, so that
    // calls of different shapes never find another region's bytes in their slots
    const WsLayout L = ws_layout(s, T, /*slots_for_any_shape=*/true);
    if (L.total > kScratchBytes) return MOE_ERR_WORKSPACE;     // beyond the library's scratch array
    uint8_t* ws = nullptr;
    MOE_TRY(device_scratch(stream, &ws));
    return layer_launches(s, x, T, w_router, logit_bias, d_table, nullptr, residual, y, topk_idx_out, topk_w_out, ws,
                          L, stream);
}

}  // extern "C"

namespace moe {

// moe_layer's launch sequence on a validated, large enough workspace
static moe_status layer_launches(const moe_shape* s, const void* x, int32_t T, const float* w_router,
                                 const float* logit_bias, const moe_expert* d_table, void* staging,
                                 const void* residual, void* y, int32_t* topk_idx_out, float* topk_w_out,
                                 uint8_t* w8, const WsLayout& L, hipStream_t stream) {
    const bool nv = s->wformat == MOE_WF_NVFP4;
    int32_t* idx = topk_idx_out ? topk_idx_out : (int32_t*)(w8 + L.idx);
    float* w = topk_w_out ? topk_w_out : (float*)(w8 + L.w);
    double* logits = (double*)(w8 + L.logits);
    int32_t* offsets = (int32_t*)(w8 + L.offsets);
    int32_t* sorted_pick = (int32_t*)(w8 + L.sorted_pick);
    int32_t* pick_pos = (int32_t*)(w8 + L.pick_pos);
    float* o = (float*)(w8 + L.o);
    if ((!nv || !staging) && T <= kSmallTokens && s->top_k <= 64 &&
        (long long)T * (s->top_k + s->n_shared) <= kMaxFusedPicks && s->d_model <= 8192) {
        // few tokens: fused router (logits, top-k, permute, plan, activation split), the gate/up
        // GEMM, and the down GEMM fused with the weighted combine: three launches per layer
        // (NVFP4: the fused router, its two GEMMs and the combine)
        const int NT = L.nt;
        const int variant = 0;
        RouteSmallArgs r;
        r.x = x;
        r.T = T;
        r.d = s->d_model;
        r.E = s->n_experts;
        r.k = s->top_k;
        r.wr = w_router;
        r.bias = logit_bias;
        r.logits = logits;
        r.hdr = (uint32_t*)(w8 + L.hdr);
        r.slots = (unsigned long long*)(w8 + L.slots);
        r.sink = w8 + L.sink;
        r.idx = idx;
        r.w = w;
        r.offsets = offsets;
        r.sorted_pick = sorted_pick;
        r.pick_pos = pick_pos;
        r.tiles = (int32_t*)(w8 + L.tiles);
        r.ntiles = (int32_t*)(w8 + L.ntiles);
        r.desc = (TileDesc*)(w8 + L.desc);
        r.table = d_table;
        r.max_tiles = L.max_tiles;
        r.tt = gemm_tile_tokens(variant, NT);
        r.xq = w8 + L.xq;
        r.xs = w8 + L.xs;
        r.ss1 = super_step(s->d_model, ksplit_for(s->d_model, variant));
        r.split = nv ? 0 : 1;
        r.tau = s->renorm_skip;
        r.shared = s->n_shared;
        if (nv) {
            r.tt = nv_tile_picks(s, T);
            MOE_HIP(launch_route_small(s, r, stream));
            MOE_TRY(run_ffn_nv(s, d_table, x, T, offsets, sorted_pick, o, w8, L, nullptr, stream, true));
            MOE_HIP(launch_combine(s, o, w, pick_pos, T, residual, y, stream));
            return MOE_OK;
        }
        const bool dec = decode_gemm_ok(s);
        if (dec) r.ss1 = 4;   // x terms in chunks of 512: the layout k_mx_gateup_dec reads
        MOE_HIP(launch_route_small(s, r, stream));
        GemmArgs a = gemm_args(s, d_table, T, sorted_pick, offsets, w8, L, o);
        if (dec) MOE_HIP(launch_gateup_dec(a, NT, L.max_tiles, stream));
        else MOE_HIP(launch_gemm_gateup(a, NT, variant, L.max_tiles, stream));
        a.aq = w8 + L.hq;
        a.as = w8 + L.hs;
        CombineArgs c;
        c.T = T;
        c.shared = s->n_shared;
        c.P = T * s->top_k;
        c.w = w;
        c.pick_pos = pick_pos;
        c.residual = residual;
        c.y = y;
        c.scaling = s->routed_scaling;
        if (dec) MOE_HIP(launch_down_dec(s, a, c, NT, stream));
        else MOE_HIP(launch_down_combine(s, a, c, NT, stream));
        return MOE_OK;
    }
    MOE_HIP(launch_router_logits(s, x, T, w_router, logit_bias, logits, stream));
    MOE_HIP(launch_topk(s, logits, T, idx, w, stream));
    MOE_HIP(launch_permute(s, idx, T, offsets, sorted_pick, pick_pos, (int32_t*)(w8 + L.perm_blocks),
                           (uint32_t*)(w8 + L.hdr), stream));
    if (nv) MOE_TRY(run_ffn_nv(s, d_table, x, T, offsets, sorted_pick, o, w8, L, staging, stream));
    else MOE_TRY(run_ffn(s, d_table, x, T, offsets, sorted_pick, o, w8, L, stream));
    MOE_HIP(launch_combine(s, o, w, pick_pos, T, residual, y, stream));
    return MOE_OK;
}

}  // namespace moe
