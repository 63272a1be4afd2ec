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

// ---------------------------------------------------------------------------------------------
// logits, many tokens: 64 tokens x 64 experts per workgroup, K in chunks of 16 through LDS,
// 4 x 4 outputs per thread, fp64 FMA.
// ---------------------------------------------------------------------------------------------
template <typename XT>
__global__ __launch_bounds__(256) void k_logits_tiled(const XT* __restrict__ x, int T, int d,
                                                      const float* __restrict__ wr,
                                                      const float* __restrict__ bias, int E,
                                                      double* __restrict__ logits) {
    constexpr int TT = 64, TE = 64, KC = 16;
    __shared__ double xs[KC][TT + 1];
    __shared__ double ws[KC][TE + 1];
    const int t0 = blockIdx.x * TT, e0 = blockIdx.y * TE;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    double acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
    for (int k0 = 0; k0 < d; k0 += KC) {
        // 64 rows x 16 k for both operands: 1024 elements each, 4 per thread
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            int idx = threadIdx.x + u * 256;
            int r = idx >> 4, kk = idx & 15;
            int t = t0 + r, e = e0 + r;
            xs[kk][r] = (t < T) ? load_act_f64(x, (size_t)t * d + k0 + kk) : 0.0;
            ws[kk][r] = (e < E) ? (double)wr[(size_t)e * d + k0 + kk] : 0.0;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) {
            double xa[4], wb[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) xa[a] = xs[kk][ty + 16 * a];
#pragma unroll
            for (int b = 0; b < 4; ++b) wb[b] = ws[kk][tx + 16 * b];
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b) acc[a][b] = fma(xa[a], wb[b], acc[a][b]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        int t = t0 + ty + 16 * a;
        if (t >= T) continue;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            int e = e0 + tx + 16 * b;
            if (e < E) logits[(size_t)t * E + e] = bias ? acc[a][b] + (double)bias[e] : acc[a][b];
        }
    }
}

hipError_t launch_router_logits(const moe_shape* s, const void* x, int T, const float* wr,
                                const float* bias, double* logits, hipStream_t st) {
    trace("router_logits", 0, st);
    const int d = s->d_model, E = s->n_experts;
    const bool bf = s->act_dtype == MOE_DT_BF16;
    if (T <= 8) {
        dim3 grid((E + 3) / 4);
        if (bf)
            hipLaunchKernelGGL((k_logits_gemv<uint16_t>), grid, dim3(256), 0, st,
                               (const uint16_t*)x, T, d, wr, bias, E, logits);
        else
            hipLaunchKernelGGL((k_logits_gemv<float>), grid, dim3(256), 0, st,
                               (const float*)x, T, d, wr, bias, E, logits);
    } else {
        dim3 grid((T + 63) / 64, (E + 63) / 64);
        if (bf)
            hipLaunchKernelGGL((k_logits_tiled<uint16_t>), grid, dim3(256), 0, st,
                               (const uint16_t*)x, T, d, wr, bias, E, logits);
        else
            hipLaunchKernelGGL((k_logits_tiled<float>), grid, dim3(256), 0, st,
                               (const float*)x, T, d, wr, bias, E, logits);
    }
    trace("router_logits", 1, st);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// top-k: one wave per token.  Each lane holds up to 16 logits (E <= 1024); k rounds of a
// wave arg-max under the order (logit descending, index ascending, NaN last).
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ bool ranks_before(double la, int a, double lb, int b) {
    const bool na = isnan(la), nb = isnan(lb);
    if (na || nb) return (na && nb) ? (a < b) : nb;
    if (la != lb) return la > lb;
    return a < b;
}

// Order-preserving 64-bit key of a logit: a larger logit has a larger key, -0 and +0 share a
// key, and a NaN gets key 0 (below every number).
__device__ __forceinline__ unsigned long long logit_key(double v) {
    if (isnan(v)) return 0ull;
    unsigned long long b = (unsigned long long)__double_as_longlong(v);
    if (b == 0x8000000000000000ull) b = 0ull;
    return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

__device__ __forceinline__ double key_to_logit(unsigned long long key) {
    const unsigned long long b = (key >> 63) ? (key & 0x7fffffffffffffffull) : ~key;
    return __longlong_as_double((long long)b);
}

// Top-k of one token's E logits by one wave (E <= 64 * S), written in rank order to idx[0..k):
// rank order is (logit descending, expert index ascending), a NaN ranks after every number.
// w[j] = sigmoid(l_j) / sum_j' sigmoid(l_j'), the sum taken in rank order.  Each lane keeps its
// S logits as order-preserving keys; a round takes every lane's best remaining key (first
// maximum in slot order = lowest index) and a DPP arg-max across the wave.  All 64 lanes must
// call it; lane j%64 stores entries j.
template <int S>
__device__ void wave_topk(const double* __restrict__ l, int E, int k, int32_t* idx, float* w) {
    const int lane = threadIdx.x & 63;
    unsigned long long key[S];
    uint32_t avail = 0;
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int e = lane + 64 * s;
        key[s] = (e < E) ? logit_key(l[e]) : 0ull;
        if (e < E) avail |= 1u << s;
    }
    unsigned long long my_key = 0ull;
    for (int j = 0; j < k; ++j) {
        unsigned long long bk = 0ull;
        int be = 0x7fffffff;
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const bool ok = (avail >> s) & 1u;
            if (ok && (be == 0x7fffffff || key[s] > bk)) { bk = key[s]; be = lane + 64 * s; }
        }
        wave_argmax(bk, be);
        if ((be & 63) == lane) avail &= ~(1u << (be >> 6));
        if ((j & 63) == lane) {
            idx[j] = be;
            if (j < 64) my_key = bk;
        }
    }
    // weights: every lane's sigmoid in parallel (from the selected key), the sum in rank order
    const double sg = (lane < k) ? 1.0 / (1.0 + exp(-key_to_logit(my_key))) : 0.0;
    double ssum = 0.0;
    for (int j = 0; j < k && j < 64; ++j) ssum += readlane_f64(sg, j);
    for (int j = 64; j < k; ++j) ssum += 1.0 / (1.0 + exp(-l[idx[j]]));   // k > 64 only
    if (lane < k) w[lane] = (float)(sg / ssum);
    for (int j = lane + 64; j < k; j += 64) w[j] = (float)((1.0 / (1.0 + exp(-l[idx[j]]))) / ssum);
}

template <int S>
__global__ __launch_bounds__(256) void k_topk(const double* __restrict__ logits, int T, int E, int k,
                                              int32_t* __restrict__ idx, float* __restrict__ wout) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    wave_topk<S>(logits + (size_t)t * E, E, k, idx + (size_t)t * k, wout + (size_t)t * k);
}

hipError_t launch_topk(const moe_shape* s, const double* logits, int T, int32_t* idx, float* w,
                       hipStream_t st) {
    trace("topk", 0, st);
    dim3 grid((T + 3) / 4);
    if (s->n_experts <= 320)
        hipLaunchKernelGGL(k_topk<5>, grid, dim3(256), 0, st, logits, T, s->n_experts, s->top_k, idx, w);
    else
        hipLaunchKernelGGL(k_topk<16>, grid, dim3(256), 0, st, logits, T, s->n_experts, s->top_k, idx, w);
    trace("topk", 1, st);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// fused router for few tokens (T <= 16), one launch per layer: every workgroup computes the fp64
// logits of 4 experts (one wave each) and splits part of x into fp8 terms; the last workgroup to
// finish (device-scope counter) does the top-k, the permute, and the grouped-GEMM tile plan,
// then resets the counter to zero for the next launch.
// ---------------------------------------------------------------------------------------------
constexpr int kSmallT = 16;
constexpr int kRouteRowChunks = 32;   // float4 per lane: router rows of up to 8192

// exclusive scan over 256 threads; returns this thread's prefix, *total = sum (LDS scratch[4])
__device__ int block_scan_256(int v, int* scratch, int* total) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
    }
    if (lane == 63) scratch[wv] = incl;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        if (w < wv) base += scratch[w];
        tot += scratch[w];
    }
    __syncthreads();
    *total = tot;
    return base + incl - v;
}

template <typename XT, int NT, int S>
__global__ __launch_bounds__(256) void k_route_small(RouteSmallArgs a) {
    const XT* __restrict__ x = (const XT*)a.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, tid = threadIdx.x;
    const int T = a.T, d = a.d, E = a.E, k = a.k;
    // 1. issue the loads of this wave's whole router row (d <= 8192: up to 32 float4 per lane)
    const int e = blockIdx.x * 4 + wave;
    const int nw = d / 256;
    float4 w4[kRouteRowChunks];
    const float* row = a.wr + (size_t)(e < E ? e : 0) * d;
#pragma unroll
    for (int u = 0; u < kRouteRowChunks; ++u)
        w4[u] = (u < nw) ? *(const float4*)(row + u * 256 + lane * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
    // 2. while they are in flight, split x into fp8 terms for the gate/up GEMM
    split_rows_lanewise<XT, NT>(x, T, d, a.ss1, a.xq, a.xs, blockIdx.x, gridDim.x);
    // 3. logits, fp64 accumulation of exact products
    if (e < E) {
#pragma unroll 1
        for (int t = 0; t < T; ++t) {
            const XT* xt = x + (size_t)t * d;
            double acc = 0.0;
#pragma unroll
            for (int u = 0; u < kRouteRowChunks; ++u) {
                if (u < nw) {
                    const float4 x4 = load_act4(xt, u * 256 + lane * 4);
                    acc = fma((double)x4.x, (double)w4[u].x, acc);
                    acc = fma((double)x4.y, (double)w4[u].y, acc);
                    acc = fma((double)x4.z, (double)w4[u].z, acc);
                    acc = fma((double)x4.w, (double)w4[u].w, acc);
                }
            }
            acc = wave_sum_f64(acc);
            if (lane == 0) a.logits[(size_t)t * E + e] = a.bias ? acc + (double)a.bias[e] : acc;
        }
    }

    // the last workgroup to arrive finishes the routing
    __shared__ int s_last;
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = (atomicAdd(a.counter, 1u) == gridDim.x - 1);
    __syncthreads();
    if (!s_last) return;
    __threadfence();

    __shared__ int32_t s_idx[kSmallT * 64];
    __shared__ float s_w[kSmallT * 64];
    __shared__ int s_cnt[1024];
    __shared__ int s_off[1024];
    __shared__ int scratch[4];
    const int P = T * k;
    for (int i = tid; i < E; i += 256) s_cnt[i] = 0;
    for (int t = wave; t < T; t += 4) wave_topk<S>(a.logits + (size_t)t * E, E, k, s_idx + t * k, s_w + t * k);
    __syncthreads();
    for (int p = tid; p < P; p += 256) {
        a.idx[p] = s_idx[p];
        a.w[p] = s_w[p];
        atomicAdd(&s_cnt[s_idx[p]], 1);
    }
    __syncthreads();
    // offsets: exclusive scan of the counts, 4 experts per thread
    int c4[4], sum4 = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int ee = tid * 4 + u;
        c4[u] = ee < E ? s_cnt[ee] : 0;
        sum4 += c4[u];
    }
    int total;
    int run = block_scan_256(sum4, scratch, &total);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int ee = tid * 4 + u;
        if (ee < E) {
            s_off[ee] = run;
            a.offsets[ee] = run;
        }
        run += c4[u];
    }
    if (tid == 0) a.offsets[E] = total;
    __syncthreads();
    // stable positions: rank of pick p among the earlier picks of its expert
    for (int p = tid; p < P; p += 256) {
        const int ep = s_idx[p];
        int r = 0;
        for (int q = 0; q < p; ++q) r += (s_idx[q] == ep);
        const int pos = s_off[ep] + r;
        a.sorted_pick[pos] = p;
        a.pick_pos[p] = pos;
    }
    // tile plan: ceil(count / tt) tiles per expert
    int n4[4], nsum = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        n4[u] = (c4[u] + a.tt - 1) / a.tt;
        nsum += n4[u];
    }
    int first = block_scan_256(nsum, scratch, &total);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int ee = tid * 4 + u;
        for (int j = 0; j < n4[u]; ++j) {
            a.tiles[2 * (first + j)] = ee;
            a.tiles[2 * (first + j) + 1] = s_off[ee] + j * a.tt;
        }
        first += n4[u];
    }
    if (tid == 0) {
        *a.ntiles = total;
        *a.counter = 0u;
    }
}

hipError_t launch_route_small(const moe_shape* s, const RouteSmallArgs& a, hipStream_t st) {
    trace("route_small", 0, st);
    dim3 grid((s->n_experts + 3) / 4);
    const bool bf = s->act_dtype == MOE_DT_BF16;
    const int NT = act_terms(s);
#define MOE_RS(XT, N)                                                                                \
    do {                                                                                             \
        if (s->n_experts <= 320) hipLaunchKernelGGL((k_route_small<XT, N, 5>), grid, dim3(256), 0, st, a); \
        else hipLaunchKernelGGL((k_route_small<XT, N, 16>), grid, dim3(256), 0, st, a);              \
    } while (0)
    if (bf && NT == 2) MOE_RS(uint16_t, 2);
    else if (bf) MOE_RS(uint16_t, 4);
    else if (NT == 2) MOE_RS(float, 2);
    else MOE_RS(float, 4);
#undef MOE_RS
    trace("route_small", 1, st);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// activation split: 32 lanes per natural 32-element block of one row
// ---------------------------------------------------------------------------------------------
template <typename XT, int NT>
__global__ __launch_bounds__(256) void k_act_split(const XT* __restrict__ x, int rows, int K, int SS,
                                                   uint8_t* __restrict__ q, uint8_t* __restrict__ sc) {
    split_rows_lanewise<XT, NT>(x, rows, K, SS, q, sc, blockIdx.x, gridDim.x);
}

hipError_t launch_act_split(const moe_shape* s, const void* x, int rows, int K, int SS, int NT,
                            uint8_t* q, uint8_t* sc, hipStream_t st) {
    trace("act_split", 0, st);
    const size_t n = (size_t)rows * (K / 32);          // 32-element blocks, 8 per workgroup
    dim3 grid((unsigned)((n + 7) / 8));
    const bool bf = s->act_dtype == MOE_DT_BF16;
#define MOE_SPLIT(XT, N)                                                                    \
    hipLaunchKernelGGL((k_act_split<XT, N>), grid, dim3(256), 0, st, (const XT*)x, rows, K, SS, q, sc)
    if (bf && NT == 2) MOE_SPLIT(uint16_t, 2);
    else if (bf && NT == 4) MOE_SPLIT(uint16_t, 4);
    else if (!bf && NT == 2) MOE_SPLIT(float, 2);
    else MOE_SPLIT(float, 4);
#undef MOE_SPLIT
    trace("act_split", 1, st);
    return hipGetLastError();
}

}  // namespace moe
