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
// tokens x 96 experts (288 = 3 x 96, no idle columns) and one K slice of the split; wave w computes
// tokens 16 (w & 1) + [0, 16) against experts 48 (w >> 1) + [0, 48) as three 16x16 blocks.  Operand layout (measured): lane l
// supplies row or column l % 16 at K = l / 16; result register r of lane l is row 4 r + l / 16,
// column l % 16.  Within each group of 16 K values, the four MFMAs j = 0..3 take K = 4 (l / 16) + j
// (each K once), so a lane reads its four values with one 16-byte LDS load.  The K slice is staged
// through LDS 64 columns at a time as fp32, rows padded to 68 floats (16-byte aligned).  Slice z's
// partial sums go to part[z][t][e]; slice 0 also adds the bias.  The top-k sums the slices in
// order z = 0, 1, ...
constexpr int kLgTok = 32, kLgExp = 96, kLgK = 64;

template <typename XT>
__global__ __launch_bounds__(256) void k_logits_mfma(const XT* __restrict__ x, int T, int d,
                                                      const float* __restrict__ wr, const float* __restrict__ bias,
                                                      int E, int kslice, double* __restrict__ part) {
    __shared__ __align__(16) float xs[2][kLgTok][kLgK + 4];
    __shared__ __align__(16) float ws[2][kLgExp][kLgK + 4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t0 = blockIdx.x * kLgTok, e0 = blockIdx.y * kLgExp, z = blockIdx.z;
    const int kb = z * kslice;
    typedef double d4 __attribute__((ext_vector_type(4)));
    constexpr int NB = kLgExp / 32;                      // 16-expert blocks per wave
    d4 acc[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[j] = d4{0, 0, 0, 0};
    const int tr = (wave & 1) * 16 + (lane & 15);        // A row (token) of this lane
    const int ec = (wave >> 1) * (kLgExp / 2) + (lane & 15);   // B column (expert) of block 0
    const int kl = lane >> 4;
    // staging: x 32 x 64 (8 consecutive per thread), Wr kLgExp x 64 (kLgExp / 16 float4 per thread);
    // rows past the end re-read the last row (their results are not stored)
    constexpr int NW = kLgExp / 16;
    const int xr = tid >> 3, xc = (tid & 7) * 8;
    const XT* xsrc = x + (size_t)min(t0 + xr, T - 1) * d + kb + xc;
    const float* wsrc[NW];
    int wrow[NW], wcol[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int q = i * 256 + tid;
        wrow[i] = q >> 4;
        wcol[i] = (q & 15) * 4;
        wsrc[i] = wr + (size_t)min(e0 + wrow[i], E - 1) * d + kb + wcol[i];
    }
    float4 xv0, xv1, wv[NW];
    auto load_chunk = [&](int k0) {
        xv0 = load_act4(xsrc + k0, 0);
        xv1 = load_act4(xsrc + k0, 4);
#pragma unroll
        for (int i = 0; i < NW; ++i) wv[i] = *(const float4*)(wsrc[i] + k0);
    };
    auto store_chunk = [&](int buf) {
        float* xd = &xs[buf][xr][xc];
        xd[0] = xv0.x; xd[1] = xv0.y; xd[2] = xv0.z; xd[3] = xv0.w;
        xd[4] = xv1.x; xd[5] = xv1.y; xd[6] = xv1.z; xd[7] = xv1.w;
#pragma unroll
        for (int i = 0; i < NW; ++i) {
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
#pragma unroll
        for (int kk = 0; kk < kLgK; kk += 16) {
            const float4 a4 = *(const float4*)&xs[buf][tr][kk + 4 * kl];
            float4 b4[NB];
#pragma unroll
            for (int jb = 0; jb < NB; ++jb) b4[jb] = *(const float4*)&ws[buf][ec + 16 * jb][kk + 4 * kl];
            const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
#pragma unroll
                for (int jb = 0; jb < NB; ++jb) {
                    const float bv = j == 0 ? b4[jb].x : j == 1 ? b4[jb].y : j == 2 ? b4[jb].z : b4[jb].w;
                    acc[jb] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)av[j], (double)bv, acc[jb], 0, 0, 0);
                }
            }
        }
        if (ch + 1 < nch) store_chunk(buf ^ 1);
        __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = t0 + (wave & 1) * 16 + 4 * r + (lane >> 4);
            const int e = e0 + (wave >> 1) * (kLgExp / 2) + 16 * j + (lane & 15);
            if (t < T && e < E) {
                double v = acc[j][r];
                if (z == 0 && bias) v += (double)bias[e];
                part[((size_t)z * T + t) * E + e] = v;
            }
        }
}

// K slices for the tiled router: enough workgroups for the chip's two per CU, slices of >= 128
// columns.  (At 4096 tokens: four slices, 1536 workgroups, three full rounds; with two, 768
// workgroups left the second round half empty: 216 against 202 us)
int logits_splits(const moe_shape* s, int T) {
    if (T <= 8) return 1;
    const long long tiles = (long long)((T + kLgTok - 1) / kLgTok) * ((s->n_experts + kLgExp - 1) / kLgExp);
    int S = 1;
    while (tiles * S < 1024 && s->d_model % (2 * S * 128) == 0 && S < 64) S *= 2;
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
// largest value of each 16-lane row, in every lane of the row (the first four steps above: the
// mirrors leave the row's maximum in all of its lanes)
__device__ __forceinline__ uint32_t row_max_u32(uint32_t v) {
    asm volatile("s_nop 1\n\tv_max_u32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
                 "s_nop 1\n\tv_max_u32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
                 "s_nop 1\n\tv_max_u32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
                 "s_nop 1\n\tv_max_u32_dpp %0, %0, %0 row_mirror row_mask:0xf bank_mask:0xf\n\t"
                 "s_nop 1"
                 : "+v"(v));
    return v;
}

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

// The k rounds over the keys kv (lane l: experts l + 64 s; entries past E are ignored); lane j
// (j < min(k, 64)) returns the key of pick j.
template <int S>
__device__ __forceinline__ unsigned long long topk_rounds(const unsigned long long (&kv)[S], int E, int k,
                                                          int32_t* idx) {
    const int lane = threadIdx.x & 63;
    constexpr int kNone = 0x7fff;          // slot of an exhausted entry: index past every expert
    // keys and slots (expert = lane + 64 * slot) of this lane's entries; slots past E hold key 0
    // and rank after every expert, and k <= E keeps them from being taken
    unsigned long long key[S];
    int slot[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const bool ok = lane + 64 * s < E;
        key[s] = ok ? kv[s] : 0ull;
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

// The same top-k (k <= 8) in one pass instead of k dependent rounds.  Lane l holds experts l + 64 s
// (unsorted).  Every 16-lane row offers its two best entries by upper key half (the lane with the
// row's best, the lowest such lane, offers its second); t, the least of these eight offers, has at
// least k distinct entries at or above it, so every pick has upper half >= t.  (When a row offers
// padding, t is 0 and every expert qualifies.)  The qualifying entries (usually a dozen or two)
// are packed into cand (128 entries of LDS owned by this wave: 64 candidates, then a discard area
// that the other lanes write to, so that the writes need no branch), and candidate c's rank is the
// number of candidates ahead of it under (key descending, index ascending): a total order, so
// ranks 0..k-1 are the picks.  Sixteen candidates are ranked at a time: lane l takes candidate
// 16 b + l % 16 and counts a quarter of the others, and the four lanes l ^ 16 s add their counts.
// Writes idx[0..k) and returns, in lane j < k, the key of pick j; returns false (writing nothing)
// when more than 64 entries qualify.  kv: the keys (entries past E are ignored).
template <int S>
__device__ __forceinline__ bool topk_pass(const unsigned long long (&kv)[S], int E, int k, int32_t* idx, uint4* cand,
                                          unsigned long long* rk, unsigned long long& my_key) {
    const int lane = threadIdx.x & 63;
    unsigned long long key[S];
    uint32_t b1 = 0u, b2 = 0u;              // the lane's two largest upper halves
#pragma unroll
    for (int s = 0; s < S; ++s) {
        key[s] = lane + 64 * s < E ? kv[s] : 0ull;
        const uint32_t h = (uint32_t)(key[s] >> 32);
        b2 = max(b2, min(b1, h));
        b1 = max(b1, h);
    }
    const uint32_t m1 = row_max_u32(b1);
    const uint32_t rowbits = (uint32_t)(__ballot(b1 == m1) >> (lane & 48)) & 0xffffu;
    const bool first = b1 == m1 && (rowbits & ((1u << (lane & 15)) - 1u)) == 0u;
    const uint32_t m2 = row_max_u32(first ? b2 : b1);
    const uint32_t t = min(min((uint32_t)__builtin_amdgcn_readlane((int)m2, 0), (uint32_t)__builtin_amdgcn_readlane((int)m2, 16)),
                           min((uint32_t)__builtin_amdgcn_readlane((int)m2, 32), (uint32_t)__builtin_amdgcn_readlane((int)m2, 48)));
    unsigned long long cm[S];
    int base[S], C = 0;
#pragma unroll
    for (int s = 0; s < S; ++s) {
        cm[s] = __ballot(lane + 64 * s < E && (uint32_t)(key[s] >> 32) >= t);
        base[s] = C;
        C += __popcll(cm[s]);
    }
    if (C > 64) return false;
    const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const bool in = (cm[s] >> lane) & 1ull;
        cand[in ? base[s] + __popcll(cm[s] & below) : 64 + lane] =
            make_uint4((uint32_t)key[s], (uint32_t)(key[s] >> 32), (uint32_t)(lane + 64 * s), 0u);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");    // the wave's LDS writes land in order
    for (int b = 0; 16 * b < C; ++b) {
        const int c = 16 * b + (lane & 15);
        const int cc = c < C ? c : 0;
        const uint4 me = cand[cc];
        const unsigned long long mk = ((unsigned long long)me.y << 32) | me.x;
        int part = 0;
#pragma unroll 4
        for (int j0 = 0; j0 < C; j0 += 4) {
            const int j = j0 + (lane >> 4);
            const uint4 o = cand[j < C ? j : cc];           // past C: itself, which never counts
            const unsigned long long ok_ = ((unsigned long long)o.y << 32) | o.x;
            part += (ok_ > mk) | ((ok_ == mk) & (o.z < me.z));
        }
        const auto r16 = __builtin_amdgcn_permlane16_swap((uint32_t)part, (uint32_t)part, false, false);
        const uint32_t p2 = r16[0] + r16[1];
        const auto r32 = __builtin_amdgcn_permlane32_swap(p2, p2, false, false);
        const int rank = (int)(r32[0] + r32[1]);
        if (lane < 16 && c < C && rank < k) {
            idx[rank] = (int32_t)me.z;
            rk[rank] = mk;
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    my_key = lane < k ? rk[lane] : 0ull;
    return true;
}

__device__ __forceinline__ double sigmoid64(double z) { return 1.0 / (1.0 + exp(-z)); }

// The weights of the k picks idx[0..k) (rank order) of one token, by one wave: lane j holds
// pick j's key (from topk_rounds).  sig: the sigmoid of every expert's logit, computed
// beforehand, or null (each lane computes its pick's: of the selected logit, where a -0 comes
// back as +0, with the same sigmoid).  The sum is taken in rank order.
// Renorm-skip (tau > 0, k <= 64; the Strata-GLM blog, "Uncensoring without touching the
// weights"): a pick after the first whose weight is below tau is dropped - idx -1 (written by the
// lane that holds that pick), weight 0 - and the kept weights are renormalised over the kept
// picks' sigmoids, summed in rank order.  The decision is taken on the fp64 weight.
__device__ __forceinline__ void topk_weights(unsigned long long my_key, const double* __restrict__ l,
                                             int32_t* idx, int k, float* w, const double* sig, float tau) {
    const int lane = threadIdx.x & 63;
    double sg = 0.0;
    if (lane < k) sg = sig ? sig[idx[lane]] : sigmoid64(key_logit(my_key));
    double ssum = 0.0;
    for (int j = 0; j < k && j < 64; ++j) ssum += readlane_f64(sg, j);
    if (tau > 0.0f) {
        const bool drop = lane > 0 && lane < k && sg / ssum < (double)tau;
        const unsigned long long dm = __ballot(drop);
        double kept = 0.0;
        for (int j = 0; j < k; ++j)
            if (!((dm >> j) & 1ull)) kept += readlane_f64(sg, j);
        if (lane < k) {
            w[lane] = drop ? 0.0f : (float)(sg / kept);
            if (drop) idx[lane] = -1;
        }
        return;
    }
    for (int j = 64; j < k; ++j) ssum += sig ? sig[idx[j]] : sigmoid64(l[idx[j]]);   // k > 64 only
    if (lane < k) w[lane] = (float)(sg / ssum);
    for (int j = lane + 64; j < k; j += 64) w[j] = (float)((sig ? sig[idx[j]] : sigmoid64(l[idx[j]])) / ssum);
}

// (topk_rounds has lane j % 64 write idx[j]: the lane that topk_weights has drop pick j)
template <int S>
__device__ void topk_select(const double (&lv)[S], const double* __restrict__ l, int E, int k, int32_t* idx,
                            float* w, float tau) {
    unsigned long long kv[S];
#pragma unroll
    for (int s = 0; s < S; ++s) kv[s] = logit_key(lv[s]);
    const unsigned long long my_key = topk_rounds<S>(kv, E, k, idx);
    topk_weights(my_key, l, idx, k, w, nullptr, tau);
}

// one wave per token; the logits are the sum, in slice order, of nsplit partial slices
// [nsplit][T][E] (nsplit = 1: the logits themselves)
template <int S>
__global__ __launch_bounds__(256) void k_topk(const double* __restrict__ logits, int T, int E, int k, int nsplit,
                                              float tau, int32_t* __restrict__ idx, float* __restrict__ wout) {
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
    topk_select<S>(lv, l, E, k, idx + (size_t)t * k, wout + (size_t)t * k, tau);
}

hipError_t launch_topk(const moe_shape* s, const double* logits, int T, int32_t* idx, float* w,
                       hipStream_t st) {
    trace("topk", 0, st);
    dim3 grid((T + 3) / 4);
    const int nsplit = logits_splits(s, T);
    if (s->n_experts <= 320)
        MOE_LAUNCH(k_topk<5>, grid, dim3(256), 0, st, logits, T, s->n_experts, s->top_k, nsplit, s->renorm_skip, idx,
                   w);
    else
        MOE_LAUNCH(k_topk<16>, grid, dim3(256), 0, st, logits, T, s->n_experts, s->top_k, nsplit, s->renorm_skip, idx,
                   w);
    trace("topk", 1, st);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// fused router for few tokens (T <= 16), one launch per layer.  Every workgroup but the last
// computes the fp64 logits of RW experts and then splits its share of x into fp8 terms (when the
// GEMMs read them); the last workgroup waits for the logits and does the top-k, the grouping and
// the tile records.
//
// Hand-over without a counter: each logit goes to its own 8-byte slot as the complement of its
// order key (logit_key), written with a device-scope store (through to the coherent level, no
// fence).  No key is all ones (that would be a NaN's natural key, and NaNs take key 0), so a slot
// reads zero exactly until its logit is there.  The routing workgroup polls its tokens' slots with
// device-scope loads until none is zero, and zeroes them again for the next launch.  Workgroups
// start in index order, so every row workgroup has started before the routing workgroup waits;
// the wait is bounded all the same.
// ---------------------------------------------------------------------------------------------
constexpr int kSmallT = 16;

// Routing refused (the status word was already nonzero, or the wait for the logits gave up):
// record a timeout in the status word (only if it was clean), and leave outputs that fail loudly
// downstream: idx -1 and w NaN, so that y is NaN.  Several tokens: no tile, positions 0 (in bounds
// for every reader).  One token: the pass runs on stand-in picks (real experts, so the GEMMs stay
// in bounds) with the NaN weights.
__device__ __forceinline__ void report_timeout(uint32_t* status) {
    __hip_atomic_fetch_or(status, MOE_WS_ROUTE_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void put_slot(unsigned long long* p, double v) {
    __hip_atomic_store(p, ~logit_key(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long get_slot(const unsigned long long* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void clear_slot(unsigned long long* p) {
    __hip_atomic_store(p, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// a stand-in key for expert e (distinct, scattered like real logits), for the warm-up pass
__device__ __forceinline__ unsigned long long dummy_key(int e) {
    return ((unsigned long long)(uint32_t)(e + 1) * 0x9e3779b97f4a7c15ull) | 0x8000000000000000ull;
}

// RW router rows per workgroup, 4 / RW waves per row, each with an equal part of it.  NC = float4
// chunks per lane of a wave's part (d / (4 / RW) <= 256 NC, d a multiple of 8).  Every load is
// issued without a condition (reads past the part re-read its last four elements and are not
// used), so that no branch separates them and all of a wave's loads are in flight together.
// PLAIN: no renorm-skip and no shared expert, known at compile time, so that the one-token tail (a
// chain of dependent steps, each worth tens of nanoseconds) carries none of their bookkeeping.
template <typename XT, int NT, int S, int NC, int RW, bool PLAIN>
__global__ __launch_bounds__(256) void k_route_small(RouteSmallArgs a) {
    const XT* __restrict__ x = (const XT*)a.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, tid = threadIdx.x;
    const int T = a.T, d = a.d, E = a.E, k = a.k;
    const int Gr = (int)gridDim.x - 1;          // row workgroups; the last workgroup routes
    if ((int)blockIdx.x < Gr) {
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
        // 2. logits, fp64 accumulation of exact products (the parts of a row added in order), TB
        // tokens at a time so that their loads are in flight together (past T: the last token
        // again, not stored); one token alone does no extra work
        __shared__ double s_part[4][kSmallT];
        auto logits = [&](auto tb) {
            constexpr int TB = decltype(tb)::value;
#pragma unroll 1
            for (int t0 = 0; t0 < T; t0 += TB) {
                float4 x4[TB][NC];
#pragma unroll
                for (int b = 0; b < TB; ++b) {
                    const XT* xt = x + (size_t)min(t0 + b, T - 1) * d + (size_t)part * pl;
#pragma unroll
                    for (int u = 0; u < NC; ++u) x4[b][u] = load_act4(xt, at(u));
                }
                double acc[TB];
#pragma unroll
                for (int b = 0; b < TB; ++b) {
                    acc[b] = 0.0;
#pragma unroll
                    for (int u = 0; u < NC; ++u) {
                        double p = fma((double)x4[b][u].x, (double)w4[u].x, acc[b]);
                        p = fma((double)x4[b][u].y, (double)w4[u].y, p);
                        p = fma((double)x4[b][u].z, (double)w4[u].z, p);
                        p = fma((double)x4[b][u].w, (double)w4[u].w, p);
                        acc[b] = used(u) ? p : acc[b];
                    }
                }
#pragma unroll
                for (int b = 0; b < TB; ++b) acc[b] = wave_sum_f64(acc[b]);
#pragma unroll
                for (int b = 0; b < TB; ++b) {
                    const int t = t0 + b;
                    if (t < T && lane == 0) {
                        if constexpr (WPR == 1)
                            put_slot(a.slots + (size_t)t * E + e, a.bias ? acc[b] + (double)a.bias[e] : acc[b]);
                        else
                            s_part[wave][t] = acc[b];
                    }
                }
            }
        };
        if (e < E) {
            if (T == 1)
                logits(std::integral_constant<int, 1>{});
            else
                logits(std::integral_constant<int, 4>{});
        }
        if constexpr (WPR > 1) {
            __syncthreads();
            if (tid < RW * T) {
                const int j = tid % RW, t = tid / RW, ej = blockIdx.x * RW + j;
                if (ej < E) {
                    double v = s_part[WPR * j][t];
#pragma unroll
                    for (int q = 1; q < WPR; ++q) v += s_part[WPR * j + q][t];
                    put_slot(a.slots + (size_t)t * E + ej, a.bias ? v + (double)a.bias[ej] : v);
                }
            }
        }
        // 3. this workgroup's share of the split of x into fp8 terms for the gate/up GEMM
        if (a.split) split_rows_lanewise<XT, NT>(x, T, d, a.ss1, a.xq, a.xs, blockIdx.x, Gr);
        return;
    }

    // the routing workgroup
    __shared__ int32_t s_idx[kMaxFusedPicks];
    __shared__ float s_w[kMaxFusedPicks];
    __shared__ uint32_t s_tm[64 * S];               // per expert: the tokens that picked it
    __shared__ uint32_t s_off[64 * S];              // per expert: picks and tiles of lower experts
    __shared__ uint32_t s_wsum[4];
    __shared__ uint4 s_cand[4][128];                // top-k candidates, per wave
    __shared__ unsigned long long s_rk[4][8];       // keys of the picks in rank order, per wave
    const int P = T * k, tt = a.tt;
    const float tau = PLAIN ? 0.0f : a.tau;        // renorm-skip threshold
    const int shared = PLAIN ? 0 : a.shared;       // a shared expert (table entry E)
    // for E <= kTabLds the whole expert table is kept in LDS
    constexpr int kTabLds = 320, kTabRounds = (kTabLds * 4 + 255) / 256;
    constexpr bool tab_lds = S <= 5;
    __shared__ uint4 s_tab[tab_lds ? kTabLds * 4 : 1];
    // the expert-table entry of expert e into a tile record: four 16-byte moves, from the LDS copy
    // of the table when there is one
    // (the shared expert, entry E, always from memory; the LDS copy holds the routed experts.  Two
    // branches, so that the LDS path stays LDS loads rather than generic ones)
    auto put_expert = [&](TileDesc* D, int e) {
        uint4* dst = (uint4*)&D->ex;
        if (tab_lds && (PLAIN || e < E)) {
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[i] = s_tab[4 * e + i];
        } else {
            const uint4* src = (const uint4*)(a.table + e);
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[i] = src[i];
        }
    };
    // an empty record still names a real expert (the first pick's, or expert 0), so that a stray
    // read of its pointers stays inside the weights
    auto put_empty = [&](TileDesc* desc, int id, int e) {
        TileDesc* D = desc + id;
        put_expert(D, e);
        D->i0 = 0;
        D->ntok = 0;
        D->e = e;
    };
    // the shared expert's tiles (table entry E): tokens c tt .. of tile c, at sorted positions
    // P + c tt .., record ids first, first + 1, ...; nothing without a shared expert
    auto put_shared = [&](TileDesc* desc, int32_t* tiles, int first, int thread, int nthreads) {
        const int tt = a.tt, nsh = shared ? (T + tt - 1) / tt : 0;
        for (int c = thread; c < nsh; c += nthreads) {
            TileDesc* D = desc + first + c;
            const int ntok = min(tt, T - c * tt);
            put_expert(D, E);
            D->i0 = P + c * tt;
            D->ntok = ntok;
            D->e = E;
            D->pad0 = 0;
#pragma unroll
            for (int j = 0; j < kDescTokens; ++j) D->tok[j] = j < ntok ? c * tt + j : 0;
            tiles[2 * (first + c)] = E;
            tiles[2 * (first + c) + 1] = P + c * tt;
        }
        return nsh;
    };
    // the outputs of a refused routing (see report_timeout), by all 256 threads
    auto put_refused = [&](TileDesc* desc, int32_t* idx, float* wout, int32_t* pick_pos, int32_t* sorted_pick,
                           int32_t* offsets, int32_t* ntiles) {
        for (int p = tid; p < P; p += 256) {
            idx[p] = -1;
            wout[p] = __builtin_nan("");
            pick_pos[p] = 0;
            sorted_pick[p] = 0;
        }
        for (int e = tid; e <= E; e += 256) offsets[e] = 0;
        for (int id = tid; id < a.max_tiles; id += 256) put_empty(desc, id, 0);
        if (tid == 0) *ntiles = 0;
    };
    // the status word and the poll limit (< 0: no polls), written only by earlier launches.  Vector
    // loads, issued next to the first poll of the slots so that they cost no wait of their own (a
    // scalar load in flight would make every LDS wait of the tail wait for it too)
    auto poll_limit_of = [](uint32_t plim) { return plim == 0u ? kPollLimitDefault : (int)plim; };
    __shared__ int s_fail[4];                                           // per wave: its wait gave up

    if (T == 1 && tab_lds) {
        // One token (the decode step).  The expert table is requested first.  While the row
        // workgroups still stream the router, the whole tail below runs once on stand-in keys with
        // every output pointed at a.sink, so that the real pass, which starts by polling the
        // slots, then runs from a warm instruction cache.  Wave 0 polls, picks and writes the
        // records; waves 1-3 meanwhile take the sigmoid of every logit into LDS and zero the slots;
        // then wave 1 writes the weights and waves 2-3 the offsets and the empty records.
        __shared__ unsigned long long s_key[kTabLds];
        __shared__ double s_sig[kTabLds];
        // the table in five named pieces (an array held across the pass loop would go to scratch)
        static_assert(kTabRounds == 5, "five rounds of table loads");
        const uint4* tsrc = (const uint4*)a.table;
        auto tload = [&](int r) { const int g = r * 256 + tid; return tsrc[g < 4 * E ? g : 4 * E - 1]; };
        auto tstore = [&](int r, const uint4& v) { const int g = r * 256 + tid; if (g < 4 * E) s_tab[g] = v; };
        const uint4 tab0 = tload(0), tab1 = tload(1), tab2 = tload(2), tab3 = tload(3), tab4 = tload(4);
#pragma unroll 1
        for (int pass = 0; pass < 2; ++pass) {
            int live = pass;
            asm volatile("" : "+s"(live));      // opaque: one copy of the code serves both passes
            TileDesc* const desc = live ? a.desc : (TileDesc*)a.sink;
            int32_t* const tiles = live ? a.tiles : (int32_t*)a.sink;
            int32_t* const idx = live ? a.idx : (int32_t*)a.sink;
            float* const wout = live ? a.w : (float*)a.sink;
            int32_t* const pick_pos = live ? a.pick_pos : (int32_t*)a.sink;
            int32_t* const sorted_pick = live ? a.sorted_pick : (int32_t*)a.sink;
            int32_t* const offsets = live ? a.offsets : (int32_t*)a.sink;
            int32_t* const ntiles = live ? a.ntiles : (int32_t*)a.sink;
            unsigned long long* const slots = live ? a.slots : (unsigned long long*)a.sink;
            unsigned long long kv[S];
#pragma unroll
            for (int s = 0; s < S; ++s) kv[s] = 0ull;
            bool refused = false;       // (wave 0) the wait gave up, or the workspace was refused
            if (live) {
                tstore(0, tab0);
                tstore(1, tab1);
                tstore(2, tab2);
                tstore(3, tab3);
                tstore(4, tab4);
            }
            if (wave == 0) {
                if (live) {
                    // poll the slots (lane l: experts l + 64 s) until none is zero, at most
                    // poll_limit times; none at all on a workspace whose status is already set.
                    // The reads of a round are all issued before its tests.  The status word and
                    // the poll limit (one 8-byte read: the header is 256-byte aligned) are read
                    // in every round beside the slots: read once before the loop, they cost a
                    // round trip of their own before the first poll.
                    uint32_t st0 = 0u;
                    bool got = false;
                    for (int it = 0;; ++it) {
                        bool miss = false;
#pragma unroll
                        for (int s = 0; s < S; ++s) {
                            const unsigned long long v = get_slot(a.slots + min(lane + 64 * s, E - 1));
                            kv[s] = ~v;
                            miss |= (lane + 64 * s < E) & (v == 0ull);
                        }
                        const unsigned long long h = get_slot((const unsigned long long*)a.hdr);
                        st0 = (uint32_t)h;
                        if ((st0 != 0u) | (it >= poll_limit_of((uint32_t)(h >> 32)))) break;
                        if (__ballot(miss) == 0ull) {
                            got = true;
                            break;
                        }
                    }
                    if (!got) {
                        // the pass still runs: its picks come from the stand-in keys, its weights
                        // from key 0 (a NaN logit, below), and the indices it writes are -1
#pragma unroll
                        for (int s = 0; s < S; ++s) kv[s] = dummy_key(lane + 64 * s);
                        if (lane == 0 && st0 == 0u) report_timeout(a.hdr);
                    }
                    refused = !got;
                } else {
                    // a branch of its own (the asm keeps it one), so that the warm-up pass does
                    // not wait for the poll in flight
                    asm volatile("" ::: "memory");
#pragma unroll
                    for (int s = 0; s < S; ++s) kv[s] = dummy_key(lane + 64 * s);
                }
                // the keys whose sigmoids make the weights: after a refusal key 0 for every expert,
                // whose logit is a NaN, so that every weight and y are NaN
#pragma unroll
                for (int s = 0; s < S; ++s)
                    if (lane + 64 * s < E) s_key[lane + 64 * s] = refused ? 0ull : kv[s];
            }
            lds_barrier();
            if (wave == 0) {
                unsigned long long my_key = 0ull;
                if (k > 8 || !topk_pass<S>(kv, E, k, s_idx, s_cand[0], s_rk[0], my_key))
                    my_key = topk_rounds<S>(kv, E, k, s_idx);
            } else {
                for (int e = tid - 64; e < E; e += 192) {
                    s_sig[e] = sigmoid64(key_logit(s_key[e]));
                    clear_slot(slots + e);
                }
            }
            lds_barrier();
            if constexpr (PLAIN) {
                // every pick stays.  Records: the token's experts are distinct, so pick p is a tile of
                // its own at sorted position = the number of picks of lower experts (what the grouping
                // below gives in this case)
                if (wave == 0) {
                    const int p = lane;
                    const int e = p < k ? s_idx[p] : 0;
                    int pos = 0;
                    for (int q = 0; q < k; ++q) pos += __builtin_amdgcn_readlane(e, q) < e;
                    if (p < k) {
                        TileDesc* D = desc + pos;
                        put_expert(D, e);
                        D->i0 = pos;
                        D->ntok = 1;
                        D->e = e;
                        D->pad0 = 0;
#pragma unroll
                        for (int c = 0; c < kDescTokens; ++c) D->tok[c] = 0;
                        tiles[2 * pos] = e;
                        tiles[2 * pos + 1] = pos;
                        idx[p] = refused ? -1 : e;
                        pick_pos[p] = pos;
                        sorted_pick[pos] = p;
                    }
                } else if (wave == 1) {
                    // the weights, the sum in rank order
                    const int p = lane;
                    const double sg = p < k ? s_sig[s_idx[p]] : 0.0;
                    double ssum = 0.0;
                    for (int j = 0; j < k; ++j) ssum += readlane_f64(sg, j);
                    if (p < k) wout[p] = (float)(sg / ssum);
                } else {
                    // the expert offsets (picks of lower experts), the empty records, the tile count
                    for (int e = tid - 128; e <= E; e += 128) {
                        int lower = 0;
#pragma unroll 8
                        for (int q = 0; q < k; ++q) lower += s_idx[q] < e;
                        offsets[e] = lower;
                    }
                    for (int id = k + tid - 128; id < a.max_tiles; id += 128) put_empty(desc, id, s_idx[0]);
                    if (tid == 128) *ntiles = k;
                }
                lds_barrier();      // the real pass rewrites what this one read from LDS
                continue;
            }
            // the picks that stay (bit j: pick j), the same in every wave: all k, or with renorm-skip
            // those not dropped (rank 0 and every pick whose fp64 weight is not below tau)
            unsigned long long km = k >= 64 ? ~0ull : ((1ull << k) - 1ull);
            double sg = 0.0, ssum = 0.0;
            if (wave == 1 || tau > 0.0f) {        // (wave 1 always: it writes the weights)
                if (lane < k) sg = s_sig[s_idx[lane]];
                for (int j = 0; j < k; ++j) ssum += readlane_f64(sg, j);
            }
            if (tau > 0.0f) km = __ballot(lane < k && !(lane > 0 && sg / ssum < (double)tau));
            const int nkept = __popcll(km);
            if (wave == 0) {
                // the records: the token's kept experts are distinct, so kept pick p is a tile of
                // its own at sorted position = the number of kept picks of lower experts (what the
                // grouping below gives in this case)
                const int p = lane;
                const int e = p < k ? s_idx[p] : 0;
                const bool kept = (km >> p) & 1ull;
                int pos = 0;
                // (bitwise tests, not &&: no branch may separate the reads, so they go out together)
                for (int q = 0; q < k; ++q) pos += (int)((km >> q) & 1ull) & (int)(__builtin_amdgcn_readlane(e, q) < e);
                if (kept) {
                    TileDesc* D = desc + pos;
                    put_expert(D, e);
                    D->i0 = pos;
                    D->ntok = 1;
                    D->e = e;
                    D->pad0 = 0;
#pragma unroll
                    for (int c = 0; c < kDescTokens; ++c) D->tok[c] = 0;
                    tiles[2 * pos] = e;
                    tiles[2 * pos + 1] = pos;
                    idx[p] = refused ? -1 : e;
                    pick_pos[p] = pos;
                    sorted_pick[pos] = p;
                } else if (p < k) {          // dropped: no expert, no position
                    idx[p] = -1;
                    pick_pos[p] = -1;
                    sorted_pick[p] = -1;     // positions nkept .. k - 1 (p >= nkept for a dropped pick)
                }
                put_shared(desc, tiles, nkept, lane, 64);
            } else if (wave == 1) {
                // the weights, the sums in rank order (over the kept picks)
                const int p = lane;
                double kept_sum = ssum;
                if (nkept < k) {
                    kept_sum = 0.0;
                    for (int j = 0; j < k; ++j)
                        if ((km >> j) & 1ull) kept_sum += readlane_f64(sg, j);
                }
                if (p < k) wout[p] = ((km >> p) & 1ull) ? (float)(sg / kept_sum) : 0.0f;
            } else {
                // the expert offsets (kept picks of lower experts), the empty records, the tile count
                for (int e = tid - 128; e <= E; e += 128) {
                    int lower = 0;
#pragma unroll 8
                    for (int q = 0; q < k; ++q) lower += (int)((km >> q) & 1ull) & (int)(s_idx[q] < e);
                    offsets[e] = lower;
                }
                const int nall = nkept + (shared ? 1 : 0);      // one token: one shared tile
                for (int id = nall + tid - 128; id < a.max_tiles; id += 128) put_empty(desc, id, s_idx[0]);
                if (tid == 128) *ntiles = nall;
            }
            lds_barrier();      // the real pass rewrites what this one read from LDS
        }
        return;
    }

    if constexpr (tab_lds) {
        uint4 tab[kTabRounds];
#pragma unroll
        for (int r = 0; r < kTabRounds; ++r) {
            const int g = r * 256 + tid;
            tab[r] = ((const uint4*)a.table)[g < 4 * E ? g : 4 * E - 1];
        }
#pragma unroll
        for (int r = 0; r < kTabRounds; ++r) {
            const int g = r * 256 + tid;
            if (g < 4 * E) s_tab[g] = tab[r];
        }
    }
    for (int e = tid; e < E; e += 256) s_tm[e] = 0u;   // (the barrier after the top-k orders these)
    // wave w routes tokens w, w + 4, ...; J of them per round of polls (lane l: experts l + 64 s).
    // Every poll load is issued without a condition (indices past T or E re-read the last slot
    // and are not used), so that all of them are in flight together.
    constexpr int J = tab_lds ? kSmallT / 4 : 1;
    const uint32_t st0 = gload4(&a.hdr[0]);
    const int poll_limit = poll_limit_of(gload4(&a.hdr[1]));
    bool gave_up = st0 != 0u;      // a workspace whose status is set is not routed on
    for (int t0 = wave; t0 < T && !gave_up; t0 += 4 * J) {
        unsigned long long kv[J][S];
        bool got = false;
        for (int it = 0; it < poll_limit; ++it) {
            bool miss = false;
#pragma unroll
            for (int j = 0; j < J; ++j)
#pragma unroll
                for (int s = 0; s < S; ++s) {
                    const int t = t0 + 4 * j, e = lane + 64 * s;
                    const unsigned long long v = get_slot(a.slots + (size_t)min(t, T - 1) * E + min(e, E - 1));
                    kv[j][s] = ~v;
                    miss |= (t < T) & (e < E) & (v == 0ull);
                }
            if (__ballot(miss) == 0ull) {
                got = true;
                break;
            }
        }
        if (!got) {
            gave_up = true;
            if (lane == 0) report_timeout(a.hdr);
            break;
        }
#pragma unroll
        for (int j = 0; j < J; ++j)
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const int t = t0 + 4 * j, e = lane + 64 * s;
                if (t < T && e < E) clear_slot(a.slots + (size_t)t * E + e);
            }
        // the round's tokens one after another in a rolled loop: one copy of the top-k code, warm in
        // the instruction cache after the first token (the keys are taken out of kv by selects, so
        // that kv stays in registers)
#pragma unroll 1
        for (int j = 0; j < J; ++j) {
            const int t = t0 + 4 * j;
            if (t >= T) break;
            unsigned long long cur[S];
#pragma unroll
            for (int s = 0; s < S; ++s) {
                cur[s] = kv[0][s];
#pragma unroll
                for (int jj = 1; jj < J; ++jj) cur[s] = j == jj ? kv[jj][s] : cur[s];
            }
            unsigned long long my_key = 0ull;
            if (k > 8 || !topk_pass<S>(cur, E, k, s_idx + t * k, s_cand[wave], s_rk[wave], my_key))
                my_key = topk_rounds<S>(cur, E, k, s_idx + t * k);
            topk_weights(my_key, nullptr, s_idx + t * k, k, s_w + t * k, nullptr, tau);
        }
    }
    if (lane == 0) s_fail[wave] = gave_up ? 1 : 0;
    lds_barrier();
    if (s_fail[0] | s_fail[1] | s_fail[2] | s_fail[3]) {
        put_refused(a.desc, a.idx, a.w, a.pick_pos, a.sorted_pick, a.offsets, a.ntiles);
        return;
    }
    // Grouping, without a pass over the picks per pick (P <= 512, T <= 16).  A token picks an
    // expert at most once, so each expert's picks are a set of tokens: a bit mask (dropped picks, id
    // -1, are in none).  A pick's sorted position is the number of kept picks of lower experts plus
    // the number of earlier tokens of its own expert, and it starts a tile when that number is a
    // multiple of tt.  One exclusive scan over the experts gives both per-expert prefixes: picks
    // (the expert offsets) in the low 16 bits, tiles (the first record id) in the high 16 bits.
    for (int p = tid; p < P; p += 256) {
        const int e = s_idx[p];
        if (e >= 0) atomicOr(&s_tm[e], 1u << (p / k));
    }
    lds_barrier();
    const int Q = (E + 255) / 256, e0 = tid * Q;        // Q <= 4 consecutive experts per thread
    uint32_t cnt[4], own = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t n = (i < Q && e0 + i < E) ? (uint32_t)__popc(s_tm[e0 + i]) : 0u;
        cnt[i] = n | (((n + tt - 1) / tt) << 16);
        own += cnt[i];
    }
    uint32_t inc = own;                                  // inclusive scan over the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t v = (uint32_t)__shfl_up((int)inc, o);
        inc += lane >= o ? v : 0u;
    }
    if (lane == 63) s_wsum[wave] = inc;
    lds_barrier();
    const uint32_t total = s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3];
    uint32_t ex = inc - own;
    for (int w = 0; w < wave; ++w) ex += s_wsum[w];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (i < Q && e0 + i < E) {
            s_off[e0 + i] = ex;
            a.offsets[e0 + i] = (int32_t)(ex & 0xffffu);
        }
        ex += cnt[i];
    }
    const int Pv = (int)(total & 0xffffu);              // kept picks
    if (tid == 0) a.offsets[E] = Pv;
    lds_barrier();
    for (int p = tid; p < P; p += 256) {
        const int e = s_idx[p];
        if (e < 0) {                                     // dropped: no expert, no position
            a.idx[p] = -1;
            a.w[p] = 0.0f;
            a.pick_pos[p] = -1;
            continue;
        }
        const int t = p / k;
        const uint32_t m = s_tm[e], o = s_off[e];
        const int before = __popc(m & ((1u << t) - 1u)), pos = (int)(o & 0xffffu) + before;
        a.idx[p] = e;
        a.w[p] = s_w[p];
        a.pick_pos[p] = pos;
        a.sorted_pick[pos] = p;
        if (before % tt == 0) {
            // a tile: this expert's tokens from t on (t is its first), at most tt of them
            const int id = (int)(o >> 16) + before / tt, ntok = min(tt, __popc(m) - before);
            TileDesc* D = a.desc + id;
            put_expert(D, e);
            D->i0 = pos;
            D->ntok = ntok;
            D->e = e;
            D->pad0 = 0;
            uint32_t mm = m >> t;
#pragma unroll
            for (int c = 0; c < kDescTokens; ++c) {
                D->tok[c] = c < ntok ? t + __builtin_ctz(mm | 0x80000000u) : 0;
                mm &= mm - 1u;
            }
            a.tiles[2 * id] = e;
            a.tiles[2 * id + 1] = pos;
        }
    }
    if (tau > 0.0f)
        for (int i = Pv + tid; i < P; i += 256) a.sorted_pick[i] = -1;
    // the tile count (the shared expert's tiles after the routed ones), and empty records up to
    // max_tiles
    int nt = (int)(total >> 16);
    nt += put_shared(a.desc, a.tiles, nt, tid, 256);
    for (int id = nt + tid; id < a.max_tiles; id += 256) put_empty(a.desc, id, s_idx[0]);
    if (tid == 0) *a.ntiles = nt;
}

hipError_t launch_route_small(const moe_shape* s, const RouteSmallArgs& a, hipStream_t st) {
    trace("route_small", 0, st);
    // one router row per workgroup, a quarter per wave (about 4 KB per wave at d = 4096), so the
    // rows spread over the whole chip; the routing workgroup last
    dim3 grid(s->n_experts + 1);
    const bool bf = s->act_dtype == MOE_DT_BF16;
    const bool lng = s->d_model > 4096;
    const bool plain = s->renorm_skip == 0.0f && s->n_shared == 0;
#define MOE_RS_P(XT, N, PL)                                                                              \
    do {                                                                                                 \
        if (s->n_experts <= 320) {                                                                       \
            if (lng) MOE_LAUNCH((k_route_small<XT, N, 5, 8, 1, PL>), grid, dim3(256), 0, st, a);        \
            else MOE_LAUNCH((k_route_small<XT, N, 5, 4, 1, PL>), grid, dim3(256), 0, st, a);            \
        } else {                                                                                         \
            if (lng) MOE_LAUNCH((k_route_small<XT, N, 16, 8, 1, PL>), grid, dim3(256), 0, st, a);       \
            else MOE_LAUNCH((k_route_small<XT, N, 16, 4, 1, PL>), grid, dim3(256), 0, st, a);           \
        }                                                                                                \
    } while (0)
#define MOE_RS(XT, N)                                                                                    \
    do {                                                                                                 \
        if (plain) MOE_RS_P(XT, N, true);                                                                \
        else MOE_RS_P(XT, N, false);                                                                     \
    } while (0)
    // activation terms (act_terms): 1 in the MXFP8 mode, else 2 for bf16 activations, 4 for fp32
    const int nt = act_terms(s);
    if (nt == 1) {
        if (bf) MOE_RS(uint16_t, 1);
        else MOE_RS(float, 1);
    } else if (bf) {
        MOE_RS(uint16_t, 2);
    } else {
        MOE_RS(float, 4);
    }
#undef MOE_RS
#undef MOE_RS_P
    trace("route_small", 1, st);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// activation split: 32 lanes per natural 32-element block of one row
// ---------------------------------------------------------------------------------------------
// Eight consecutive elements per thread (one 16-byte load of bf16), four lanes per block: the block
// maximum takes two DPP steps within the lane quad (xor 1, xor 2), and each term's eight codes are
// one 8-byte store.  (Four elements per thread, eight lanes and three DPP steps took 28 us for a
// 4096-token chunk.)
template <typename XT, int NT>
__global__ __launch_bounds__(256) void k_act_split(const XT* __restrict__ x, int rows, int K, int SS,
                                                   uint8_t* __restrict__ q, uint8_t* __restrict__ sc) {
    const size_t n8 = (size_t)rows * (K / 8);
    const size_t g = (size_t)blockIdx.x * 256 + threadIdx.x;     // 8-element group
    const bool ok = g < n8;                                      // uniform per 4-lane block
    const size_t gg = ok ? g : 0;
    const int row = (int)(gg / (K / 8)), c8 = (int)(gg % (K / 8));
    const int blk = c8 >> 2, j = c8 & 3;                         // block, group within it
    const size_t e0 = (size_t)row * K + (size_t)c8 * 8;
    const float4 va = load_act4(x, e0), vb = load_act4(x, e0 + 4);
    float v[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
    const int groups = K / 32;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
        m = fmaxf(m, __uint_as_float(dpp_u32<kDppXor1, 0xF>(__float_as_uint(m), __float_as_uint(m))));
        m = fmaxf(m, __uint_as_float(dpp_u32<kDppXor2, 0xF>(__float_as_uint(m), __float_as_uint(m))));
        const int S = split_exponent(m);
        const float scale = pow2f(S);
        uint32_t w[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            w[h] = fp8x2_encode<false>(0u, v[4 * h], v[4 * h + 1], scale);
            w[h] = fp8x2_encode<true>(w[h], v[4 * h + 2], v[4 * h + 3], scale);
        }
        if (t + 1 < NT) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const v2f_t lo = fp8x2_decode<false>(w[h], scale), hi = fp8x2_decode<true>(w[h], scale);
                v[4 * h] -= lo[0];
                v[4 * h + 1] -= lo[1];
                v[4 * h + 2] -= hi[0];
                v[4 * h + 3] -= hi[1];
            }
        }
        if (ok) {
            uint8_t* base = q + ((size_t)row * NT + t) * K;
            const int i = 8 * j;                                   // element index in the block
            *(uint2*)(base + act_half_offset(SS, blk, i >> 4) + (i & 15)) = make_uint2(w[0], w[1]);
            if (j == 0) sc[((size_t)row * NT + t) * groups + blk] = (uint8_t)(S + 127);
        }
    }
}

hipError_t launch_act_split(const moe_shape* s, const void* x, int rows, int K, int SS, int NT,
                            uint8_t* q, uint8_t* sc, hipStream_t st) {
    trace("act_split", 0, st);
    const size_t n = (size_t)rows * (K / 8);           // 8-element groups, one per thread
    dim3 grid((unsigned)((n + 255) / 256));
    const bool bf = s->act_dtype == MOE_DT_BF16;
#define MOE_SPLIT(XT, N)                                                                    \
    MOE_LAUNCH((k_act_split<XT, N>), grid, dim3(256), 0, st, (const XT*)x, rows, K, SS, q, sc)
    if (bf && NT == 1) MOE_SPLIT(uint16_t, 1);
    else if (bf && NT == 2) MOE_SPLIT(uint16_t, 2);
    else if (bf && NT == 4) MOE_SPLIT(uint16_t, 4);
    else if (!bf && NT == 1) MOE_SPLIT(float, 1);
    else if (!bf && NT == 2) MOE_SPLIT(float, 2);
    else MOE_SPLIT(float, 4);
#undef MOE_SPLIT
    trace("act_split", 1, st);
    return hipGetLastError();
}

}  // namespace moe
