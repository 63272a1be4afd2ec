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
template <typename XT, int TMAX>
__global__ __launch_bounds__(256) void k_logits_gemv(const XT* __restrict__ x, int T, int d,
                                                     const float* __restrict__ wr,
                                                     const float* __restrict__ bias, int E,
                                                     double* __restrict__ logits) {
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (e >= E) return;
    double acc[TMAX];
#pragma unroll
    for (int t = 0; t < TMAX; ++t) acc[t] = 0.0;
    const float* row = wr + (size_t)e * d;
    for (int i = lane * 4; i < d; i += 256) {
        float4 w4 = *(const float4*)(row + i);
        const double w0 = w4.x, w1 = w4.y, w2 = w4.z, w3 = w4.w;
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
            if (t < T) {
                const size_t b = (size_t)t * d + i;
                acc[t] = fma(load_act_f64(x, b + 0), w0, acc[t]);
                acc[t] = fma(load_act_f64(x, b + 1), w1, acc[t]);
                acc[t] = fma(load_act_f64(x, b + 2), w2, acc[t]);
                acc[t] = fma(load_act_f64(x, b + 3), w3, acc[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
        double v = acc[t];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
        if (lane == 0 && t < T) logits[(size_t)t * E + e] = bias ? v + (double)bias[e] : v;
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
            hipLaunchKernelGGL((k_logits_gemv<uint16_t, 8>), grid, dim3(256), 0, st,
                               (const uint16_t*)x, T, d, wr, bias, E, logits);
        else
            hipLaunchKernelGGL((k_logits_gemv<float, 8>), grid, dim3(256), 0, st,
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

__global__ __launch_bounds__(256) void k_topk(const double* __restrict__ logits, int T, int E, int k,
                                              int32_t* __restrict__ idx, float* __restrict__ wout) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const double* l = logits + (size_t)t * E;
    double v[16];
    uint32_t taken = 0;
#pragma unroll
    for (int s = 0; s < 16; ++s) {
        int e = lane + 64 * s;
        v[s] = (e < E) ? l[e] : 0.0;
        if (e >= E) taken |= 1u << s;
    }
    double ssum = 0.0;
    for (int j = 0; j < k; ++j) {
        // local best
        double bv = 0.0;
        int be = -1;
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            if (taken & (1u << s)) continue;
            int e = lane + 64 * s;
            if (be < 0 || ranks_before(v[s], e, bv, be)) { bv = v[s]; be = e; }
        }
        // wave reduction
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            double ov = __shfl_xor(bv, off);
            int oe = __shfl_xor(be, off);
            if (oe >= 0 && (be < 0 || ranks_before(ov, oe, bv, be))) { bv = ov; be = oe; }
        }
        if ((be & 63) == lane) taken |= 1u << (be >> 6);
        if (lane == 0) idx[(size_t)t * k + j] = be;
        ssum += 1.0 / (1.0 + exp(-bv));
    }
    // weights: sigmoid(l_sel) / sum, in fp64, written in rank order (lane 0 reads back the ids
    // it wrote itself)
    if (lane == 0) {
        for (int j = 0; j < k; ++j) {
            int e = idx[(size_t)t * k + j];
            double s = 1.0 / (1.0 + exp(-l[e]));
            wout[(size_t)t * k + j] = (float)(s / ssum);
        }
    }
}

hipError_t launch_topk(const moe_shape* s, const double* logits, int T, int32_t* idx, float* w,
                       hipStream_t st) {
    trace("topk", 0, st);
    dim3 grid((T + 3) / 4);
    hipLaunchKernelGGL(k_topk, grid, dim3(256), 0, st, logits, T, s->n_experts, s->top_k, idx, w);
    trace("topk", 1, st);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// activation split: one thread per natural 32-element block of one row
// ---------------------------------------------------------------------------------------------
template <typename XT, int NT>
__global__ __launch_bounds__(256) void k_act_split(const XT* __restrict__ x, int rows, int K, int SS,
                                                   uint8_t* __restrict__ q, uint8_t* __restrict__ sc) {
    const int groups = K / 32;
    const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (gid >= (size_t)rows * groups) return;
    const int row = (int)(gid / groups), blk = (int)(gid % groups);
    float v[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) v[e] = load_act(x, (size_t)row * K + blk * 32 + e);
    uint32_t codes[NT][8];
    int S[NT];
    split_terms<NT>(v, codes, S, [](float a) { return a; });
    const int o0 = act_half_offset(SS, blk, 0), o1 = act_half_offset(SS, blk, 1);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        uint8_t* base = q + ((size_t)row * NT + t) * K;
        *(uint4*)(base + o0) = make_uint4(codes[t][0], codes[t][1], codes[t][2], codes[t][3]);
        *(uint4*)(base + o1) = make_uint4(codes[t][4], codes[t][5], codes[t][6], codes[t][7]);
        sc[((size_t)row * NT + t) * groups + blk] = (uint8_t)(S[t] + 127);
    }
}

hipError_t launch_act_split(const moe_shape* s, const void* x, int rows, int K, int SS, int NT,
                            uint8_t* q, uint8_t* sc, hipStream_t st) {
    trace("act_split", 0, st);
    const size_t n = (size_t)rows * (K / 32);
    dim3 grid((unsigned)((n + 255) / 256));
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
