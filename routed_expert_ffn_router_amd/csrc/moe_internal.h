// Internal declarations of the routed-MoE HIP library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------------------------
// element formats (device side)
// ---------------------------------------------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <typename XT>
__device__ __forceinline__ float load_act(const XT* p, size_t i);
template <>
__device__ __forceinline__ float load_act<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_act<uint16_t>(const uint16_t* p, size_t i) { return bf16_bits_to_f32(p[i]); }

template <typename XT>
__device__ __forceinline__ double load_act_f64(const XT* p, size_t i) { return (double)load_act<XT>(p, i); }

template <typename XT>
__device__ __forceinline__ void store_act(XT* p, size_t i, float v);
template <>
__device__ __forceinline__ void store_act<float>(float* p, size_t i, float v) { p[i] = v; }
template <>
__device__ __forceinline__ void store_act<uint16_t>(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16_bits(v); }

// E4M3FN code (sign | exponent<<3 | mantissa) of v, round to nearest even, saturating to
// +-448.  v must be finite.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
    uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
    float a = fabsf(v);
    uint32_t code;
    if (a >= 0.015625f) {                       // normal range (>= 2^-6)
        int e;
        float m = frexpf(a, &e);                // a = m * 2^e, m in [0.5, 1)
        float q = rintf((2.0f * m - 1.0f) * 8.0f);
        int E = e - 1;
        int mi = (int)q;
        if (mi == 8) { mi = 0; E += 1; }
        int biased = E + 7;
        code = (biased > 15 || (biased == 15 && mi == 7)) ? 0x7Eu : (uint32_t)((biased << 3) | mi);
    } else {
        code = (uint32_t)rintf(a * 512.0f);     // subnormal step 2^-9; 8 -> 0x08 = 2^-6
    }
    return sign | code;
}

__device__ __forceinline__ float e4m3_decode(uint32_t c) {
    uint32_t e = (c >> 3) & 15u, m = c & 7u;
    float mag = e ? ldexpf(1.0f + (float)m * 0.125f, (int)e - 7) : ldexpf((float)m * 0.125f, -6);
    return (c & 0x80u) ? -mag : mag;
}

// ---------------------------------------------------------------------------------------------
// activation "terms": x (or h) is written as a sum of NT fp8 E4M3 terms, each with one
// power-of-two scale per natural block of 32 consecutive elements, so the FP4 weights can be
// contracted on the scaled FP4 x FP8 matrix cores.  The byte order follows the FP8 operand of
// V_MFMA_SCALE_F32_16X16X128_F8F6F4 as measured on gfx950: the scale supplied by lane group b
// covers K block b, while the codes held by lane group g are the halves
// [16(g%2), 16(g%2)+16) of K blocks g/2 and g/2 + 2.  For a vector of length K in chunks of
// CK = 128*SS elements (SS MFMAs per chunk), natural block beta = B*SS + h of chunk c
// (B in 0..3, h in 0..SS-1) has its scale byte at c*4*SS + beta, and its two 16-element halves
// are stored in the 32-byte group q = (2*(B%2) + half)*SS + h of the chunk, at byte offset
// 16*(B/2) inside the group.
// ---------------------------------------------------------------------------------------------

// byte offset (within a K-long code row) of half `half` (0/1) of natural block `blk`
__device__ __forceinline__ int act_half_offset(int SS, int blk, int half) {
    const int c = blk / (4 * SS), beta = blk % (4 * SS);
    const int B = beta / SS, h = beta % SS;
    const int q = (2 * (B & 1) + half) * SS + h;
    return c * 128 * SS + q * 32 + 16 * (B >> 1);
}

__device__ __forceinline__ int split_exponent(float amax) {
    if (!(amax > 0.0f)) return 0;
    int e;
    frexpf(amax, &e);
    int S = e - 1 - 7;                      // |v| / 2^S < 256 <= 448
    return S < -127 ? -127 : (S > 127 ? 127 : S);
}

// Split n values (registers) of one block into NT terms: code bytes packed 4 per word,
// exponents S[t]; residuals are exact.  `amax_reduce` combines the per-lane max across the
// lanes that share the block (identity when one thread holds the whole block).
template <int NT, int N, typename Reduce>
__device__ __forceinline__ void split_terms(float (&v)[N], uint32_t (&codes)[NT][N / 4], int (&S)[NT],
                                            Reduce amax_reduce) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < N; ++i) amax = fmaxf(amax, fabsf(v[i]));
        S[t] = split_exponent(amax_reduce(amax));
#pragma unroll
        for (int i = 0; i < N / 4; ++i) codes[t][i] = 0;
#pragma unroll
        for (int i = 0; i < N; ++i) {
            uint32_t c = e4m3_encode(ldexpf(v[i], -S[t]));
            v[i] -= ldexpf(e4m3_decode(c), S[t]);
            codes[t][i >> 2] |= c << (8 * (i & 3));
        }
    }
}

// ---------------------------------------------------------------------------------------------
// launchers (one per kernel family); all return hipGetLastError() of their launch
// ---------------------------------------------------------------------------------------------

// tracing hook (set through moe_set_trace_hook); every launcher brackets its launch with these
void trace(const char* kernel, int phase, hipStream_t st);

struct WsLayout {
    size_t logits, idx, w, offsets, sorted_pick, pick_pos, tiles, ntiles, xq, xs, hq, hs, o, total;
    int nt;        // activation terms
    int max_tiles;
};

int act_terms(const moe_shape* s);
int super_step(int K, int ksplit);
WsLayout ws_layout(const moe_shape* s, int32_t T);

hipError_t launch_router_logits(const moe_shape* s, const void* x, int T, const float* wr,
                                const float* bias, double* logits, hipStream_t st);
hipError_t launch_topk(const moe_shape* s, const double* logits, int T, int32_t* idx, float* w,
                       hipStream_t st);
hipError_t launch_act_split(const moe_shape* s, const void* x, int rows, int K, int SS, int NT,
                            uint8_t* q, uint8_t* sc, hipStream_t st);
hipError_t launch_permute(const moe_shape* s, const int32_t* idx, int T, int32_t* offsets,
                          int32_t* sorted_pick, int32_t* pick_pos, hipStream_t st);
hipError_t launch_plan(const moe_shape* s, const int32_t* offsets, int tile_tokens, int32_t* tiles,
                       int32_t* ntiles, hipStream_t st);

struct GemmArgs {
    const moe_expert* table;
    int d, f, E, k, P;
    const int32_t* sorted_pick;
    const int32_t* tiles;     // [max_tiles][2] = (expert, first sorted position)
    const int32_t* ntiles;
    const int32_t* offsets;
    const uint8_t* aq;        // activation terms (x terms by token / h terms by sorted position)
    const uint8_t* as;
    uint8_t* hq;              // gate/up output: h terms
    uint8_t* hs;
    float* o;                 // down output [P][d]
};

// variant: 0 = few tokens per expert (16 columns per tile, K split over the 4 waves when
// possible); 1 = many tokens per expert (128 columns per tile)
int gemm_variant(const moe_shape* s, int T);
int gemm_tile_tokens(int variant, int NT);
hipError_t launch_gemm_gateup(const GemmArgs& a, int NT, int variant, int max_tiles, hipStream_t st);
hipError_t launch_gemm_down(const GemmArgs& a, int NT, int variant, int max_tiles, hipStream_t st);

hipError_t launch_combine(const moe_shape* s, const float* o, const float* w, const int32_t* pick_pos,
                          int T, const void* residual, void* y, hipStream_t st);
hipError_t launch_fill_table(const moe_shape* s, const uint8_t* base, size_t stride,
                             moe_expert* table, hipStream_t st);
hipError_t launch_gather(const moe_shape* s, const moe_expert* table, const int32_t* list, int n,
                         uint8_t* staging, size_t stride, moe_expert* staged, hipStream_t st);

}  // namespace moe
