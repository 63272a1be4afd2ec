// Router: fp64-accumulated logits, wavefront top-k with normalised sigmoid weights, and the
// split of activations into scaled fp8 terms for the matrix cores.
//
// Router semantics follow "Project Maya ..." (section "What is in the 96.5 GB": an F32 router
// per layer, 8 of 288 experts per token), with ties to the lower expert index as in the same
// page's section "Steady speed with depth" (the radix select keeps the old order, ties broken
// by the lower index), and weights renormalised over the kept experts (Strata-GLM blog,
// "Uncensoring without touching the weights").  Sigmoid scoring is the reading taken where the
// pages name no score function.
#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------------------------------------
// logits, few tokens: one wave per expert row, all T (<= 8) tokens at once.  Each product
// x*w (bf16 or fp32 times fp32) is exact in fp64 and fma() rounds once per term, so every
// partial sum is the fp64 sum of exact products, as in the plain definition.
// ---------------------------------------------------------------------------------------------
template <typename XT>
__global__ __launch_bounds__(256) void k_logits_gemv(const XT* __restrict__ x, int T, int d,
                                                     const float* __restrict__ wr,
                                                     const float* __restrict__ bias, int E,
                                                     double* __restrict__ logits) {
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (e >= E) return;
#pragma unroll 1
    for (int t = 0; t < T; ++t) {
        const double v = wave_logit(x + (size_t)t * d, d, wr + (size_t)e * d);
        if (lane == 0) logits[(size_t)t * E + e] = bias ? v + (double)bias[e] : v;
    }
}

// Router logits on the fp64 matrix cores (V_MFMA_F64_16X16X4_F64), for T > 8.  Products of
// bf16 (or fp32) x and fp32 Wr are exact in fp64 and summed in fp64, so the top-k decides on the
// same numbers as a sequential fp64 sum up to the last bits.  A workgroup (4 waves) owns 32
// tokens x 64 experts and one K slice of the split; wave w computes tokens 16 (w & 1) + [0, 16)
// against experts 32 (w >> 1) + [0, 32) as two 16x16 blocks.  Operand layout (measured): lane l
// supplies row or column l % 16 at K = l / 16; result register r of lane l is row 4 r + l / 16,
// column l % 16.  The K slice is staged through LDS 64 columns at a time as fp32.  Slice z's
// partial sums go to part[z][t][e]; slice 0 also adds the bias.  The top-k sums the slices in
// order z = 0, 1, ...
constexpr int kLgTok = 32, kLgExp = 64, kLgK = 64;

template <typename XT>
__global__ __launch_bounds__(256) void k_logits_mfma(const XT* __restrict__ x, int T, int d,
                                                      const float* __restrict__ wr, const float* __restrict__ bias,
                                                      int E, int kslice, double* __restrict__ part) {
    __shared__ float xs[2][kLgTok][kLgK + 1];
    __shared__ float ws[2][kLgExp][kLgK + 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t0 = blockIdx.x * kLgTok, e0 = blockIdx.y * kLgExp, z = blockIdx.z;
    const int kb = z * kslice;
    typedef double d4 __attribute__((ext_vector_type(4)));
    d4 acc[2] = {d4{0, 0, 0, 0}, d4{0, 0, 0, 0}};
    const int tr = (wave & 1) * 16 + (lane & 15);        // A row (token) of this lane
    const int ec = (wave >> 1) * 32 + (lane & 15);       // B column (expert) of block 0
    const int kl = lane >> 4;
    // staging: x 32 x 64 (8 consecutive per thread), Wr 64 x 64 (4 float4 per thread); rows past
    // the end re-read the last row (their results are not stored)
    const int xr = tid >> 3, xc = (tid & 7) * 8;
    const XT* xsrc = x + (size_t)min(t0 + xr, T - 1) * d + kb + xc;
    const float* wsrc[4];
    int wrow[4], wcol[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = i * 256 + tid;
        wrow[i] = q >> 4;
        wcol[i] = (q & 15) * 4;
        wsrc[i] = wr + (size_t)min(e0 + wrow[i], E - 1) * d + kb + wcol[i];
    }
    float4 xv0, xv1, wv[4];
    auto load_chunk = [&](int k0) {
        xv0 = load_act4(xsrc + k0, 0);
        xv1 = load_act4(xsrc + k0, 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) wv[i] = *(const float4*)(wsrc[i] + k0);
    };
    auto store_chunk = [&](int buf) {
        float* xd = &xs[buf][xr][xc];
        xd[0] = xv0.x; xd[1] = xv0.y; xd[2] = xv0.z; xd[3] = xv0.w;
        xd[4] = xv1.x; xd[5] = xv1.y; xd[6] = xv1.z; xd[7] = xv1.w;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float* wd = &ws[buf][wrow[i]][wcol[i]];
            wd[0] = wv[i].x; wd[1] = wv[i].y; wd[2] = wv[i].z; wd[3] = wv[i].w;
        }
    };
    const int nch = kslice / kLgK;
    load_chunk(0);
    store_chunk(0);
    __syncthreads();
    for (int ch = 0; ch < nch; ++ch) {
        const int buf = ch & 1;
        if (ch + 1 < nch) load_chunk((ch + 1) * kLgK);
#pragma unroll 4
        for (int kk = 0; kk < kLgK; kk += 4) {
            const double a = (double)xs[buf][tr][kk + kl];
            const double b0 = (double)ws[buf][ec][kk + kl];
            const double b1 = (double)ws[buf][ec + 16][kk + kl];
            acc[0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b0, acc[0], 0, 0, 0);
            acc[1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b1, acc[1], 0, 0, 0);
        }
        if (ch + 1 < nch) store_chunk(buf ^ 1);
        __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = t0 + (wave & 1) * 16 + 4 * r + (lane >> 4);
            const int e = e0 + (wave >> 1) * 32 + 16 * j + (lane & 15);
            if (t < T && e < E) {
                double v = acc[j][r];
                if (z == 0 && bias) v += (double)bias[e];
                part[((size_t)z * T + t) * E + e] = v;
            }
        }
}

// K slices for the tiled router: enough workgroups to cover the chip, slices of >= 128 columns
int logits_splits(const moe_shape* s, int T) {
    if (T <= 8) return 1;
    const long long tiles = (long long)((T + kLgTok - 1) / kLgTok) * ((s->n_experts + kLgExp - 1) / kLgExp);
    int S = 1;
    while (tiles * S < 512 && s->d_model % (2 * S * 128) == 0 && S < 64) S *= 2;
    return S;
}

hipError_t launch_router_logits(const moe_shape* s, const void* x, int T, const float* wr,
                                const float* bias, double* logits, hipStream_t st) {
    trace("router_logits", 0, st);
    const int d = s->d_model, E = s->n_experts;
    const bool bf = s->act_dtype == MOE_DT_BF16;
    if (T <= 8) {
        dim3 grid((E + 3) / 4);
        if (bf)
            MOE_LAUNCH((k_logits_gemv<uint16_t>), grid, dim3(256), 0, st,
                               (const uint16_t*)x, T, d, wr, bias, E, logits);
        else
            MOE_LAUNCH((k_logits_gemv<float>), grid, dim3(256), 0, st,
                               (const float*)x, T, d, wr, bias, E, logits);
    } else {
        const int S = logits_splits(s, T);
        dim3 grid((T + kLgTok - 1) / kLgTok, (E + kLgExp - 1) / kLgExp, S);
        if (bf)
            MOE_LAUNCH((k_logits_mfma<uint16_t>), grid, dim3(256), 0, st, (const uint16_t*)x, T, d, wr, bias, E,
                       d / S, logits);
        else
            MOE_LAUNCH((k_logits_mfma<float>), grid, dim3(256), 0, st, (const float*)x, T, d, wr, bias, E, d / S,
                       logits);
    }
    trace("router_logits", 1, st);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// top-k: one wave per token.  Each lane holds up to 16 logits (E <= 1024), sorted; k rounds each
// take the wave's best head under the order (logit descending, index ascending, NaN last).
// ---------------------------------------------------------------------------------------------
// The order is carried by an integer key per logit: larger logit, larger key; -0 and +0 share
// one; a NaN has key 0, below every number.  Keys are compared as (key, expert index): equal
// keys mean equal logits, and then the lower index ranks first.
__device__ __forceinline__ unsigned long long logit_key(double v) {
    unsigned long long b = (unsigned long long)__double_as_longlong(v);
    b = (b == 0x8000000000000000ull) ? 0ull : b;
    const unsigned long long k = (b >> 63) ? ~b : (b | 0x8000000000000000ull);
    return __builtin_isnan(v) ? 0ull : k;
}
// the logit of a key (keys of numbers; key 0 gives a NaN)
__device__ __forceinline__ double key_logit(unsigned long long k) {
    const unsigned long long b = (k >> 63) ? (k & 0x7fffffffffffffffull) : ~k;
    return __longlong_as_double((long long)b);
}

// Wave reductions of the top-k rounds, latency-bound: each of the six steps (xor 1, xor 2,
// half-row mirror, row mirror, then row broadcasts 15 and 31 into the upper rows) is one VALU
// op reading its permuted operand through DPP, after which lane 63 holds the result of the whole
// wave.  The s_nop 1 before each step covers the DPP read of a VGPR written just before.  All
// 64 lanes must be active.
#define MOE_WAVE_REDUCE_DPP(op)                                                             \
    "s_nop 1\n\t" op " %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"     \
    "s_nop 1\n\t" op " %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"     \
    "s_nop 1\n\t" op " %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"          \
    "s_nop 1\n\t" op " %0, %0, %0 row_mirror row_mask:0xf bank_mask:0xf\n\t"               \
    "s_nop 1\n\t" op " %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"             \
    "s_nop 1\n\t" op " %0, %0, %0 row_bcast:31 row_mask:0xc bank_mask:0xf\n\t"             \
    "s_nop 1"
// largest value of the wave (in every lane)
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    asm volatile(MOE_WAVE_REDUCE_DPP("v_max_u32_dpp") : "+v"(v));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
// smallest value of the wave (in every lane)
__device__ __forceinline__ int wave_min_i32(int v) {
    asm volatile(MOE_WAVE_REDUCE_DPP("v_min_i32_dpp") : "+v"(v));
    return __builtin_amdgcn_readlane(v, 63);
}
#undef MOE_WAVE_REDUCE_DPP

// Top-k of one token's E logits by one wave (E <= 64 * S, k <= E), written in rank order to
// idx[0..k).  w[j] = sigmoid(l_j) / sum_j' sigmoid(l_j'), the sum taken in rank order.  Lane l
// holds experts l + 64 s, sorted by (key, index).  A round takes the lanes whose head has the
// largest upper key half (a 32-bit wave max); when that is one lane, its head is the best.
// Otherwise the lower key half decides among them, and for equal keys (equal logits) the lower
// expert index.  All 64 lanes must call it; lane j%64 stores entry j.
template <int S>
__device__ __forceinline__ void topk_load(const double* __restrict__ l, int E, double (&lv)[S]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int s = 0; s < S; ++s) {          // all loads together, none behind a branch
        const int e = lane + 64 * s;
        lv[s] = l[e < E ? e : E - 1];
    }
}

// The k rounds; lane j (j < min(k, 64)) returns the key of pick j.
template <int S>
__device__ __forceinline__ unsigned long long topk_rounds(const double (&lv)[S], int E, int k, int32_t* idx) {
    const int lane = threadIdx.x & 63;
    constexpr int kNone = 0x7fff;          // slot of an exhausted entry: index past every expert
    // keys and slots (expert = lane + 64 * slot) of this lane's entries; slots past E hold key 0
    // and rank after every expert, and k <= E keeps them from being taken
    unsigned long long key[S];
    int slot[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const bool ok = lane + 64 * s < E;
        key[s] = ok ? logit_key(lv[s]) : 0ull;
        slot[s] = ok ? s : kNone;
    }
    // rank order within the lane (odd-even transposition sort, S passes)
#pragma unroll
    for (int pass = 0; pass < S; ++pass) {
#pragma unroll
        for (int s = pass & 1; s + 1 < S; s += 2) {
            const bool sw = (key[s + 1] > key[s]) | ((key[s + 1] == key[s]) & (slot[s + 1] < slot[s]));
            const unsigned long long k0 = key[s], k1 = key[s + 1];
            const int s0 = slot[s], s1 = slot[s + 1];
            key[s] = sw ? k1 : k0;
            key[s + 1] = sw ? k0 : k1;
            slot[s] = sw ? s1 : s0;
            slot[s + 1] = sw ? s0 : s1;
        }
    }
    // k rounds: the winning lane shifts its list up by one
    unsigned long long my_key = 0ull;
    for (int j = 0; j < k; ++j) {
        const uint32_t hk = (uint32_t)(key[0] >> 32);
        const uint32_t mh = wave_max_u32(hk);
        const unsigned long long c1 = __ballot(hk == mh);
        int wl;
        if (__popcll(c1) == 1) {
            wl = __builtin_ctzll(c1);
        } else {                            // equal upper halves: the lower half, then the index
            const bool in1 = (c1 >> lane) & 1ull;
            const uint32_t lk = (uint32_t)key[0];
            const uint32_t ml = wave_max_u32(in1 ? lk : 0u);
            const unsigned long long c2 = c1 & __ballot(lk == ml);
            if (__popcll(c2) == 1) {
                wl = __builtin_ctzll(c2);
            } else {
                const bool in2 = (c2 >> lane) & 1ull;
                wl = wave_min_i32(in2 ? lane + 64 * slot[0] : 0x7fffffff) & 63;
            }
        }
        const int c = wl + 64 * __builtin_amdgcn_readlane(slot[0], wl);
        const uint32_t wlo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)key[0], wl);
        const uint32_t whi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(key[0] >> 32), wl);
        const bool win = wl == lane;
#pragma unroll
        for (int s = 0; s + 1 < S; ++s) {
            key[s] = win ? key[s + 1] : key[s];
            slot[s] = win ? slot[s + 1] : slot[s];
        }
        key[S - 1] = win ? 0ull : key[S - 1];
        slot[S - 1] = win ? kNone : slot[S - 1];
        if ((j & 63) == lane) {
            idx[j] = c;
            my_key = ((unsigned long long)whi << 32) | wlo;
        }
    }
    return my_key;
}

__device__ __forceinline__ double sigmoid64(double z) { return 1.0 / (1.0 + exp(-z)); }

// The weights of the k picks idx[0..k) (rank order) of one token, by one wave: lane j holds
// pick j's key (from topk_rounds).  sig: the sigmoid of every expert's logit, computed
// beforehand, or null (each lane computes its pick's: of the selected logit, where a -0 comes
// back as +0, with the same sigmoid).  The sum is taken in rank order.
__device__ __forceinline__ void topk_weights(unsigned long long my_key, const double* __restrict__ l,
                                             const int32_t* idx, int k, float* w, const double* sig) {
    const int lane = threadIdx.x & 63;
    double sg = 0.0;
    if (lane < k) sg = sig ? sig[idx[lane]] : sigmoid64(key_logit(my_key));
    double ssum = 0.0;
    for (int j = 0; j < k && j < 64; ++j) ssum += readlane_f64(sg, j);
    for (int j = 64; j < k; ++j) ssum += sig ? sig[idx[j]] : sigmoid64(l[idx[j]]);   // k > 64 only
    if (lane < k) w[lane] = (float)(sg / ssum);
    for (int j = lane + 64; j < k; j += 64) w[j] = (float)((sig ? sig[idx[j]] : sigmoid64(l[idx[j]])) / ssum);
}

template <int S>
__device__ void topk_select(const double (&lv)[S], const double* __restrict__ l, int E, int k, int32_t* idx,
                            float* w) {
    const unsigned long long my_key = topk_rounds<S>(lv, E, k, idx);
    topk_weights(my_key, l, idx, k, w, nullptr);
}

template <int S>
__device__ void wave_topk(const double* __restrict__ l, int E, int k, int32_t* idx, float* w) {
    double lv[S];
    topk_load<S>(l, E, lv);
    topk_select<S>(lv, l, E, k, idx, w);
}

// one wave per token; the logits are the sum, in slice order, of nsplit partial slices
// [nsplit][T][E] (nsplit = 1: the logits themselves)
template <int S>
__global__ __launch_bounds__(256) void k_topk(const double* __restrict__ logits, int T, int E, int k, int nsplit,
                                              int32_t* __restrict__ idx, float* __restrict__ wout) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const double* l = logits + (size_t)t * E;
    double lv[S];
    topk_load<S>(l, E, lv);
    // slices 1.. in groups of 4: a group's loads are all in flight before its sums, in order
    for (int z0 = 1; z0 < nsplit; z0 += 4) {
        double pz[4][S];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int z = z0 + j < nsplit ? z0 + j : z0;     // past the end: re-read, not added
            topk_load<S>(l + (size_t)z * T * E, E, pz[j]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (z0 + j < nsplit) {
#pragma unroll
                for (int s = 0; s < S; ++s) lv[s] += pz[j][s];
            }
    }
    if (nsplit > 1 && k > 64) {
        // the weights of picks past 64 re-read l[idx]: store the summed logits over slice 0
        double* lw = const_cast<double*>(l);
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int s = 0; s < S; ++s)
            if (lane + 64 * s < E) lw[lane + 64 * s] = lv[s];
        __threadfence_block();
    }
    topk_select<S>(lv, l, E, k, idx + (size_t)t * k, wout + (size_t)t * k);
}

hipError_t launch_topk(const moe_shape* s, const double* logits, int T, int32_t* idx, float* w,
                       hipStream_t st) {
    trace("topk", 0, st);
    dim3 grid((T + 3) / 4);
    const int nsplit = logits_splits(s, T);
    if (s->n_experts <= 320)
        MOE_LAUNCH(k_topk<5>, grid, dim3(256), 0, st, logits, T, s->n_experts, s->top_k, nsplit, idx, w);
    else
        MOE_LAUNCH(k_topk<16>, grid, dim3(256), 0, st, logits, T, s->n_experts, s->top_k, nsplit, idx, w);
    trace("topk", 1, st);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// fused router for few tokens (T <= 16), one launch per layer: every workgroup computes the fp64
// logits of 4 experts (a wave each; rows longer than 4096: 2 experts, two waves each); the last
// workgroup to finish (device-scope counter) does the top-k, the grouping and the tile records,
// then resets the counter to zero for the next launch, while the others split x into fp8 terms
// (when the GEMMs read them).
// ---------------------------------------------------------------------------------------------
constexpr int kSmallT = 16;

// RW router rows per workgroup: 4 (a wave per row) or 2 (two waves per row, each with half of
// it, for long rows).  NC = float4 chunks per lane of a wave's part of a row (d / (4 / RW) <= 256
// NC, d a multiple of 8).  Every load is issued without a condition (reads past the part re-read
// its last four elements and are not used), so that no branch separates them and all of a
// wave's loads are in flight together.
template <typename XT, int NT, int S, int NC, int RW>
__global__ __launch_bounds__(256) void k_route_small(RouteSmallArgs a) {
    const XT* __restrict__ x = (const XT*)a.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, tid = threadIdx.x;
    const int T = a.T, d = a.d, E = a.E, k = a.k;
    // 1. issue the loads of this wave's part of its router row.  Lane l reads elements 256 u +
    // 4 l .. +3 of the part; reads past it are clamped to its last four and not used.
    constexpr int WPR = 4 / RW;
    static_assert(RW * WPR == 4, "four waves per workgroup");
    const int e = blockIdx.x * RW + wave / WPR, part = wave % WPR;
    const int pl = d / WPR;
    auto at = [&](int u) { return min(u * 256 + lane * 4, pl - 4); };
    auto used = [&](int u) { return u * 256 + lane * 4 < pl; };
    float4 w4[NC];
    const float* row = a.wr + (size_t)(e < E ? e : 0) * d + (size_t)part * pl;
#pragma unroll
    for (int u = 0; u < NC; ++u) w4[u] = *(const float4*)(row + at(u));
    // 2. logits, fp64 accumulation of exact products (the parts of a row added in order)
    __shared__ double s_part[4][kSmallT];
    if (e < E) {
#pragma unroll 1
        for (int t = 0; t < T; ++t) {
            const XT* xt = x + (size_t)t * d + (size_t)part * pl;
            float4 x4[NC];
#pragma unroll
            for (int u = 0; u < NC; ++u) x4[u] = load_act4(xt, at(u));
            double acc = 0.0;
#pragma unroll
            for (int u = 0; u < NC; ++u) {
                double p = fma((double)x4[u].x, (double)w4[u].x, acc);
                p = fma((double)x4[u].y, (double)w4[u].y, p);
                p = fma((double)x4[u].z, (double)w4[u].z, p);
                p = fma((double)x4[u].w, (double)w4[u].w, p);
                acc = used(u) ? p : acc;
            }
            acc = wave_sum_f64(acc);
            if constexpr (WPR == 1) {
                if (lane == 0) a.logits[(size_t)t * E + e] = a.bias ? acc + (double)a.bias[e] : acc;
            } else {
                if (lane == 0) s_part[wave][t] = acc;
            }
        }
    }
    if constexpr (WPR == 2) {
        __syncthreads();
        if (tid < RW * T) {
            const int j = tid % RW, t = tid / RW, ej = blockIdx.x * RW + j;
            if (ej < E) {
                const double v = s_part[2 * j][t] + s_part[2 * j + 1][t];
                a.logits[(size_t)t * E + ej] = a.bias ? v + (double)a.bias[ej] : v;
            }
        }
    }

    // the last workgroup to arrive finishes the routing.  The barrier orders every wave's logit
    // stores before thread 0's device-scope release, which writes back the L2 once per workgroup
    // (a fence in every thread would write it back once per wave, and a few hundred write-backs
    // per launch cost microseconds); one atomic per workgroup counts arrivals, and only the last
    // workgroup's thread 0 acquires (one L2 invalidate).  The others, in arrival order, then
    // split x into fp8 terms for the gate/up GEMM while the last one routes.
    __shared__ int s_ticket;
    const int G = (int)gridDim.x;
    __syncthreads();
    if (tid == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        s_ticket = (int)__hip_atomic_fetch_add(a.counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (s_ticket == G - 1) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
    const int ticket = s_ticket;
    if (ticket != G - 1) {
        if (a.split) split_rows_lanewise<XT, NT>(x, T, d, a.ss1, a.xq, a.xs, ticket, G - 1);
        return;
    }
    if (G == 1 && a.split) split_rows_lanewise<XT, NT>(x, T, d, a.ss1, a.xq, a.xs, 0, 1);

    __shared__ int32_t s_idx[kMaxFusedPicks];
    __shared__ float s_w[kMaxFusedPicks];
    __shared__ int32_t s_sorted[kMaxFusedPicks];    // sorted position -> pick
    __shared__ uint8_t s_start[kMaxFusedPicks];     // sorted position starts a tile
    const int P = T * k, tt = a.tt;
    // the routed tokens' logits (up to four per wave) and, for E <= kTabLds, the whole expert
    // table are requested in one round, the logits first; the table goes to LDS while the
    // top-k runs
    constexpr int kTabLds = 320, kTabRounds = (kTabLds * 4 + 255) / 256;
    constexpr bool tab_lds = S <= 5;
    __shared__ uint4 s_tab[tab_lds ? kTabLds * 4 : 1];
    constexpr int J = tab_lds ? kSmallT / 4 : 1;     // tokens whose logits are preloaded per wave
    double lv[J][S];
    if (wave < T) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int t = wave + 4 * j;
            topk_load<S>(a.logits + (size_t)(t < T ? t : T - 1) * E, E, lv[j]);
        }
    }
    uint4 tab[tab_lds ? kTabRounds : 1];
    if constexpr (tab_lds) {
#pragma unroll
        for (int r = 0; r < kTabRounds; ++r) {
            const int g = r * 256 + tid;
            tab[r] = ((const uint4*)a.table)[g < 4 * E ? g : 4 * E - 1];
        }
    }
    if constexpr (tab_lds) {
#pragma unroll
        for (int r = 0; r < kTabRounds; ++r) asm volatile("" ::"v"(tab[r].x), "v"(tab[r].y), "v"(tab[r].z), "v"(tab[r].w));
#pragma unroll
        for (int r = 0; r < kTabRounds; ++r) {
            const int g = r * 256 + tid;
            if (g < 4 * E) s_tab[g] = tab[r];
        }
    }
    if (T == 1 && tab_lds) {
        // one token: wave 0 runs the rounds while the other three waves take the sigmoid of every
        // expert's logit, so that the weights need only the sum and the divisions
        __shared__ double s_sig[kTabLds];
        unsigned long long my_key = 0ull;
        if (wave == 0) {
            my_key = topk_rounds<S>(lv[0], E, k, s_idx);
        } else {
            for (int e = tid - 64; e < E; e += 192) s_sig[e] = sigmoid64(a.logits[e]);
        }
        __syncthreads();
        if (wave == 0) topk_weights(my_key, a.logits, s_idx, k, s_w, s_sig);
    } else if (wave < T) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int t = wave + 4 * j;
            if (t < T) topk_select<S>(lv[j], a.logits + (size_t)t * E, E, k, s_idx + t * k, s_w + t * k);
        }
        for (int t = wave + 4 * J; t < T; t += 4)
            wave_topk<S>(a.logits + (size_t)t * E, E, k, s_idx + t * k, s_w + t * k);
    }
    __syncthreads();
    // the expert-table entry of expert e into a tile record: four 16-byte moves, from the LDS copy
    // of the table when there is one
    auto put_expert = [&](TileDesc* D, int e) {
        const uint4* src = tab_lds ? &s_tab[4 * e] : (const uint4*)(a.table + e);
        uint4* dst = (uint4*)&D->ex;
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i] = src[i];
    };
    // an empty record still names a real expert (the first pick's), so that a stray read of its
    // pointers stays inside the weights
    auto put_empty = [&](int id) {
        TileDesc* D = a.desc + id;
        put_expert(D, s_idx[0]);
        D->i0 = 0;
        D->ntok = 0;
        D->e = s_idx[0];
    };
    // the expert offsets: the number of picks of lower experts
    auto put_offsets = [&]() {
        for (int e = tid; e <= E; e += 256) {
            int lower = 0;
#pragma unroll 8
            for (int q = 0; q < P; ++q) lower += s_idx[q] < e;
            a.offsets[e] = lower;
        }
    };
    if (T == 1) {
        // one token: its k experts are distinct, so each pick is a tile of its own, and its
        // sorted position is the number of picks of lower experts (what the grouping below
        // gives in this case, without its scans)
        for (int p = tid; p < k; p += 256) {
            const int e = s_idx[p];
            int pos = 0;
#pragma unroll 8
            for (int q = 0; q < k; ++q) pos += s_idx[q] < e;
            TileDesc* D = a.desc + pos;
            put_expert(D, e);
            D->i0 = pos;
            D->ntok = 1;
            D->e = e;
            D->pad0 = 0;
#pragma unroll
            for (int c = 0; c < kDescTokens; ++c) D->tok[c] = 0;
            a.tiles[2 * pos] = e;
            a.tiles[2 * pos + 1] = pos;
            a.idx[p] = e;
            a.w[p] = s_w[p];
            a.pick_pos[p] = pos;
            a.sorted_pick[pos] = p;
        }
        put_offsets();
        for (int id = k + tid; id < a.max_tiles; id += 256) put_empty(id);
        if (tid == 0) {
            *a.ntiles = k;
            *a.counter = 0u;
        }
        return;
    }
    // Grouping without atomics or scans (P <= 512, two picks per thread): a pick's sorted
    // position is the number of picks of lower experts plus its rank among the picks of its own
    // expert; it starts a tile when that rank is a multiple of tt.
    int pos[2], rank[2], cnt[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int p = tid + 256 * u;
        pos[u] = -1;
        if (p < P) {
            const int e = s_idx[p];
            int lower = 0, before = 0, same = 0;
#pragma unroll 8
            for (int q = 0; q < P; ++q) {
                const int eq = s_idx[q];
                lower += eq < e;
                same += eq == e;
                before += (eq == e) & (q < p);
            }
            pos[u] = lower + before;
            rank[u] = before;
            cnt[u] = same;
            s_sorted[pos[u]] = p;
            s_start[pos[u]] = (before % tt) == 0;
            a.idx[p] = e;
            a.w[p] = s_w[p];
            a.pick_pos[p] = pos[u];
            a.sorted_pick[pos[u]] = p;
        }
    }
    put_offsets();
    __syncthreads();
    // tiles: numbered by sorted position of their first pick
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        if (pos[u] >= 0 && s_start[pos[u]]) {
            int id = 0;
#pragma unroll 8
            for (int q = 0; q < pos[u]; ++q) id += s_start[q];
            const int ntok = min(tt, cnt[u] - rank[u]);
            TileDesc* D = a.desc + id;
            put_expert(D, s_idx[tid + 256 * u]);
            D->i0 = pos[u];
            D->ntok = ntok;
            D->e = s_idx[s_sorted[pos[u]]];
            D->pad0 = 0;
            for (int c = 0; c < kDescTokens; ++c) D->tok[c] = c < ntok ? s_sorted[pos[u] + c] / k : 0;
            a.tiles[2 * id] = D->e;
            a.tiles[2 * id + 1] = pos[u];
        }
    }
    // the tile count, and empty records up to max_tiles
    int nt = 0;
#pragma unroll 8
    for (int q = 0; q < P; ++q) nt += s_start[q];
    for (int id = nt + tid; id < a.max_tiles; id += 256) put_empty(id);
    if (tid == 0) {
        *a.ntiles = nt;
        *a.counter = 0u;
    }
}

hipError_t launch_route_small(const moe_shape* s, const RouteSmallArgs& a, hipStream_t st) {
    trace("route_small", 0, st);
    // rows up to 4096: a wave per row; longer (up to 8192): two waves per row
    const int RW = s->d_model <= 4096 ? 4 : 2;
    dim3 grid((s->n_experts + RW - 1) / RW);
    const bool bf = s->act_dtype == MOE_DT_BF16;
#define MOE_RS(XT, N, R)                                                                                \
    do {                                                                                                \
        if (s->n_experts <= 320) MOE_LAUNCH((k_route_small<XT, N, 5, 16, R>), grid, dim3(256), 0, st, a); \
        else MOE_LAUNCH((k_route_small<XT, N, 16, 16, R>), grid, dim3(256), 0, st, a);              \
    } while (0)
    // activation terms: 2 for bf16 activations, 4 for fp32 (act_terms)
    if (bf) {
        if (RW == 4) MOE_RS(uint16_t, 2, 4);
        else MOE_RS(uint16_t, 2, 2);
    } else {
        if (RW == 4) MOE_RS(float, 4, 4);
        else MOE_RS(float, 4, 2);
    }
#undef MOE_RS
    trace("route_small", 1, st);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// activation split: 32 lanes per natural 32-element block of one row
// ---------------------------------------------------------------------------------------------
// Four consecutive elements per thread, eight lanes per block: the block maximum takes three DPP
// steps (xor 1, xor 2, half-row mirror), each term's four codes are one dword.
template <typename XT, int NT>
__global__ __launch_bounds__(256) void k_act_split(const XT* __restrict__ x, int rows, int K, int SS,
                                                   uint8_t* __restrict__ q, uint8_t* __restrict__ sc) {
    const size_t n4 = (size_t)rows * (K / 4);
    const size_t g = (size_t)blockIdx.x * 256 + threadIdx.x;     // 4-element group
    const bool ok = g < n4;                                      // uniform per 8-lane block
    const size_t gg = ok ? g : 0;
    const int row = (int)(gg / (K / 4)), c4 = (int)(gg % (K / 4));
    const int blk = c4 >> 3, j = c4 & 7;                         // block, group within it
    const float4 v4 = load_act4(x, (size_t)row * K + (size_t)c4 * 4);
    float v[4] = {v4.x, v4.y, v4.z, v4.w};
    const int groups = K / 32;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        float m = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
        m = fmaxf(m, __uint_as_float(dpp_u32<kDppXor1, 0xF>(__float_as_uint(m), __float_as_uint(m))));
        m = fmaxf(m, __uint_as_float(dpp_u32<kDppXor2, 0xF>(__float_as_uint(m), __float_as_uint(m))));
        m = fmaxf(m, __uint_as_float(dpp_u32<kDppHalfMirror, 0xF>(__float_as_uint(m), __float_as_uint(m))));
        const int S = split_exponent(m);
        const float scale = pow2f(S);
        uint32_t w = fp8x2_encode<false>(0u, v[0], v[1], scale);
        w = fp8x2_encode<true>(w, v[2], v[3], scale);
        if (t + 1 < NT) {
            const v2f_t lo = fp8x2_decode<false>(w, scale), hi = fp8x2_decode<true>(w, scale);
            v[0] -= lo[0];
            v[1] -= lo[1];
            v[2] -= hi[0];
            v[3] -= hi[1];
        }
        if (ok) {
            uint8_t* base = q + ((size_t)row * NT + t) * K;
            const int i = 4 * j;                                   // element index in the block
            *(uint32_t*)(base + act_half_offset(SS, blk, i >> 4) + (i & 15)) = w;
            if (j == 0) sc[((size_t)row * NT + t) * groups + blk] = (uint8_t)(S + 127);
        }
    }
}

hipError_t launch_act_split(const moe_shape* s, const void* x, int rows, int K, int SS, int NT,
                            uint8_t* q, uint8_t* sc, hipStream_t st) {
    trace("act_split", 0, st);
    const size_t n = (size_t)rows * (K / 4);           // 4-element groups, one per thread
    dim3 grid((unsigned)((n + 255) / 256));
    const bool bf = s->act_dtype == MOE_DT_BF16;
#define MOE_SPLIT(XT, N)                                                                    \
    MOE_LAUNCH((k_act_split<XT, N>), grid, dim3(256), 0, st, (const XT*)x, rows, K, SS, q, sc)
    if (bf && NT == 2) MOE_SPLIT(uint16_t, 2);
    else if (bf && NT == 4) MOE_SPLIT(uint16_t, 4);
    else if (!bf && NT == 2) MOE_SPLIT(float, 2);
    else MOE_SPLIT(float, 4);
#undef MOE_SPLIT
    trace("act_split", 1, st);
    return hipGetLastError();
}

}  // namespace moe
