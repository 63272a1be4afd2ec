// Internal declarations of the routed-MoE HIP library (gfx950 only).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <utility>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------------------------
// wave reductions on DPP lane permutations (quad_perm xor 1 / xor 2, row half-mirror, row
// mirror, row broadcast 15 / 31), which avoid the LDS round trip of a shuffle; the result is
// complete in lane 63 and broadcast with readlane.  Fixed combination order: deterministic.
// ---------------------------------------------------------------------------------------------
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
constexpr int kDppBcast15 = 0x142, kDppBcast31 = 0x143;

template <int CTRL, int ROWMASK>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROWMASK, 0xF, false);
}

template <int CTRL, int ROWMASK>
__device__ __forceinline__ double dpp_add_f64(double v) {
    const unsigned long long b = (unsigned long long)__double_as_longlong(v);
    const uint32_t lo = dpp_u32<CTRL, ROWMASK>(0u, (uint32_t)b), hi = dpp_u32<CTRL, ROWMASK>(0u, (uint32_t)(b >> 32));
    return v + __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
    const unsigned long long b = (unsigned long long)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), lane);
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// sum over the 64 lanes of a wave, returned in every lane
__device__ __forceinline__ double wave_sum_f64(double v) {
    v = dpp_add_f64<kDppXor1, 0xF>(v);
    v = dpp_add_f64<kDppXor2, 0xF>(v);
    v = dpp_add_f64<kDppHalfMirror, 0xF>(v);
    v = dpp_add_f64<kDppMirror, 0xF>(v);
    v = dpp_add_f64<kDppBcast15, 0xA>(v);
    v = dpp_add_f64<kDppBcast31, 0xC>(v);
    return readlane_f64(v, 63);
}

// maximum over each 16-lane row, returned in every lane of the row
__device__ __forceinline__ float row16_max(float m) {
    m = fmaxf(m, __uint_as_float(dpp_u32<kDppXor1, 0xF>(__float_as_uint(m), __float_as_uint(m))));
    m = fmaxf(m, __uint_as_float(dpp_u32<kDppXor2, 0xF>(__float_as_uint(m), __float_as_uint(m))));
    m = fmaxf(m, __uint_as_float(dpp_u32<kDppHalfMirror, 0xF>(__float_as_uint(m), __float_as_uint(m))));
    m = fmaxf(m, __uint_as_float(dpp_u32<kDppMirror, 0xF>(__float_as_uint(m), __float_as_uint(m))));
    return m;
}

// value of lane l ^ 16 and of lane l ^ 32 (gfx950 permlane swaps: no LDS round trip)
__device__ __forceinline__ float max_xor16(float m) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float m) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// sum over lanes l and l ^ 1 (and l ^ 2 for NT = 4): the NT adjacent columns of one token (NT = 1:
// the column itself)
template <int NT>
__device__ __forceinline__ float sum_adjacent(float v) {
    if constexpr (NT >= 2) v += __uint_as_float(dpp_u32<kDppXor1, 0xF>(0u, __float_as_uint(v)));
    if constexpr (NT == 4) v += __uint_as_float(dpp_u32<kDppXor2, 0xF>(0u, __float_as_uint(v)));
    return v;
}

// A matrix-core instruction reads its operands from all 64 lanes.  When its result is used only
// inside a lane-dependent branch (a store by the lanes that hold valid columns), the compiler may
// sink the MFMAs into that branch, where they run with the other lanes switched off and take no
// operands from them.  Consuming each accumulator here, in every lane and outside any such
// branch, keeps them in front of it.  (No instruction is emitted.)
template <typename V>
__device__ __forceinline__ void mfma_results_here(const V& acc) {
    asm volatile("" ::"v"(acc));
}

// loads through global-address-space pointers: global_load rather than flat_load (pointers read
// from memory are generic otherwise, and a flat load also holds up LDS waits)
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 gload16(const void* p) {
    const u32x4_t v = *(__attribute__((address_space(1))) const u32x4_t*)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 gload8(const void* p) {
    const u32x2_t v = *(__attribute__((address_space(1))) const u32x2_t*)p;
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t gload4(const void* p) {
    return *(__attribute__((address_space(1))) const uint32_t*)p;
}
__device__ __forceinline__ int32_t gload_i32(const void* p) {
    return *(__attribute__((address_space(1))) const int32_t*)p;
}
// A load of wave-uniform data through the scalar path (s_load into SGPRs): it does not queue
// behind the vector memory requests of the CU.  Only for data that no wave writes during the
// kernel (the scalar cache is invalidated when a kernel starts), at a wave-uniform address.
template <typename T>
__device__ __forceinline__ T sload(const T* p) {
    return *(const __attribute__((address_space(4))) T*)p;
}

// Workgroup barrier for LDS hand-over: this wave's LDS operations done, then s_barrier.  Unlike
// __syncthreads it does not wait for global loads in flight (the workgroup-scope fence would).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);                  // lgkmcnt(0), vmcnt and expcnt unchanged
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------------------------
// direct global -> LDS loads (global_load_lds) for the stage rings of the many-picks GEMMs
// ---------------------------------------------------------------------------------------------
typedef const __attribute__((address_space(1))) void* dma_src_t;
typedef __attribute__((address_space(3))) void* dma_dst_t;
// lane l's 16 (4) bytes at src land at lds + 16 l (4 l); lds must be the same in every lane
__device__ __forceinline__ void dma16(const uint8_t* src, uint8_t* lds) {
    __builtin_amdgcn_global_load_lds((dma_src_t)src, (dma_dst_t)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const uint8_t* src, uint8_t* lds) {
    __builtin_amdgcn_global_load_lds((dma_src_t)src, (dma_dst_t)lds, 4, 0, 0);
}
// wait until at most N vector-memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// workgroup barrier for the stage ring: this wave's LDS reads are complete and the compiler
// moves no memory access across it.  Unlike __syncthreads it does not wait for this wave's
// direct loads still in flight (they target other stages; each is waited for with wait_vm
// before the barrier that publishes its stage).
__device__ __forceinline__ void ring_barrier() { lds_barrier(); }

// compile-time step positions of the unrolled ring loops
template <int Q>
struct StepPos {
    static constexpr int value = Q;
};
// f(StepPos<B>), f(StepPos<B + 1>), ... in order, for each index of the sequence
template <int B, typename F, int... I>
__device__ __forceinline__ void for_steps(F&& f, std::integer_sequence<int, I...>) {
    (f(StepPos<B + I>{}), ...);
}

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

// four consecutive activations starting at a multiple of 4
template <typename XT>
__device__ __forceinline__ float4 load_act4(const XT* p, size_t i);
template <>
__device__ __forceinline__ float4 load_act4<float>(const float* p, size_t i) { return *(const float4*)(p + i); }
template <>
__device__ __forceinline__ float4 load_act4<uint16_t>(const uint16_t* p, size_t i) {
    const uint2 u = *(const uint2*)(p + i);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}

// Router logit of one expert row for token t, fp64 accumulation of exact products, in every
// lane of the wave.  The row is read in chunks of 8 float4 per lane with all loads of a chunk
// issued together; loops over chunks and tokens stay rolled to keep the code small.
template <typename XT>
__device__ __forceinline__ double wave_logit(const XT* __restrict__ xt, int d, const float* __restrict__ row) {
    const int lane = threadIdx.x & 63;
    double acc = 0.0;
#pragma unroll 1
    for (int base = 0; base < d; base += 256 * 8) {
        float4 w4[8], x4[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = base + u * 256 + lane * 4;
            w4[u] = (i < d) ? *(const float4*)(row + i) : make_float4(0.f, 0.f, 0.f, 0.f);
            x4[u] = (i < d) ? load_act4(xt, i) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            acc = fma((double)x4[u].x, (double)w4[u].x, acc);
            acc = fma((double)x4[u].y, (double)w4[u].y, acc);
            acc = fma((double)x4[u].z, (double)w4[u].z, acc);
            acc = fma((double)x4[u].w, (double)w4[u].w, acc);
        }
    }
    return wave_sum_f64(acc);
}

template <typename XT>
__device__ __forceinline__ void store_act(XT* p, size_t i, float v);
template <>
__device__ __forceinline__ void store_act<float>(float* p, size_t i, float v) { p[i] = v; }
template <>
__device__ __forceinline__ void store_act<uint16_t>(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16_bits(v); }

// E4M3FN codes on the gfx950 conversion unit.  V_CVT_SCALEF32_PK_FP8_F32 writes the codes of
// round-to-nearest-even(a / scale) and (b / scale) into the low (HI = false) or high 16 bits of
// `old`; V_CVT_SCALEF32_PK_F32_FP8 returns code * scale for the two codes of the selected half.
// For a power-of-two scale (a normal float) and |v| / scale <= 448 both are exact
// (checked against a software encoder on gfx950).
typedef short v2i16_t __attribute__((ext_vector_type(2)));
typedef float v2f_t __attribute__((ext_vector_type(2)));

template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_encode(uint32_t old, float a, float b, float scale) {
    v2i16_t o;
    o[0] = (short)(old & 0xffffu);
    o[1] = (short)(old >> 16);
    const v2i16_t r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, a, b, scale, HI);
    return (uint32_t)(uint16_t)r[0] | ((uint32_t)(uint16_t)r[1] << 16);
}

template <bool HI>
__device__ __forceinline__ v2f_t fp8x2_decode(uint32_t codes, float scale) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(codes, scale, HI);
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

// exponent S of a term: |v| / 2^S < 256 <= 448 for every v of the block (amax = max |v|),
// clamped at -126 so that 2^S is a normal float (also for an all-zero block)
__device__ __forceinline__ int split_exponent(float amax) {
    const int be = (int)((__float_as_uint(amax) >> 23) & 0xffu);
    return be - 134 < -126 ? -126 : be - 134;
}

__device__ __forceinline__ float pow2f(int S) { return __uint_as_float((uint32_t)(S + 127) << 23); }

// Split n values (registers) of one block into NT terms: code bytes packed 4 per word,
// exponents S[t]; residuals are exact.  `amax_reduce` combines the per-lane max across the
// lanes that share the block (identity when one thread holds the whole block).
template <int NT, int N, typename Reduce>
__device__ __forceinline__ void split_terms(float (&v)[N], uint32_t (&codes)[NT][N / 4], int (&S)[NT],
                                            Reduce amax_reduce) {
    static_assert(N % 4 == 0, "values come in words of four codes");
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < N; ++i) amax = fmaxf(amax, fabsf(v[i]));
        S[t] = split_exponent(amax_reduce(amax));
        const float sc = pow2f(S[t]);
#pragma unroll
        for (int i = 0; i < N / 4; ++i) {
            uint32_t w = fp8x2_encode<false>(0u, v[4 * i], v[4 * i + 1], sc);
            w = fp8x2_encode<true>(w, v[4 * i + 2], v[4 * i + 3], sc);
            codes[t][i] = w;
            if (t + 1 < NT) {       // the last term's residual is not needed
                const v2f_t lo = fp8x2_decode<false>(w, sc), hi = fp8x2_decode<true>(w, sc);
                v[4 * i] -= lo[0];
                v[4 * i + 1] -= lo[1];
                v[4 * i + 2] -= hi[0];
                v[4 * i + 3] -= hi[1];
            }
        }
    }
}

// The same split with one element per lane: 32 lanes (half a wave) share a block, the block
// maximum comes from xor-shuffles, and lanes 4i..4i+3 pack their four code bytes into one word.
// Rows [0, T) of x (length d) are covered by the threads of workgroups wg, wg + nwg, ...
template <typename XT, int NT>
__device__ __forceinline__ void split_rows_lanewise(const XT* __restrict__ x, int T, int d, int SS,
                                                    uint8_t* __restrict__ q, uint8_t* __restrict__ sc,
                                                    int wg, int nwg) {
    const int lane = threadIdx.x & 63;
    const int i = lane & 31;
    const int groups = d / 32;
    const size_t nblk = (size_t)T * groups;
    const size_t per_wg = (blockDim.x / 32);
    for (size_t b0 = (size_t)wg * per_wg; b0 < nblk; b0 += (size_t)nwg * per_wg) {
        const size_t blk_all = b0 + (threadIdx.x >> 5);
        const bool ok = blk_all < nblk;          // uniform per 32-lane half
        const int row = ok ? (int)(blk_all / groups) : 0, blk = ok ? (int)(blk_all % groups) : 0;
        float v = ok ? load_act(x, (size_t)row * d + blk * 32 + i) : 0.0f;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float m = max_xor16(row16_max(fabsf(v)));
            const int S = split_exponent(m);
            const float scale = pow2f(S);
            const uint32_t c = fp8x2_encode<false>(0u, v, 0.0f, scale) & 0xffu;
            if (t + 1 < NT) v -= fp8x2_decode<false>(c, scale)[0];
            uint32_t word = c << (8 * (i & 3));
            word |= dpp_u32<kDppXor1, 0xF>(word, word);
            word |= dpp_u32<kDppXor2, 0xF>(word, word);
            if (ok && (i & 3) == 0) {
                const int half = i >> 4;
                uint8_t* base = q + ((size_t)row * NT + t) * d;
                *(uint32_t*)(base + act_half_offset(SS, blk, half) + (i & 15)) = word;
            }
            if (ok && i == 0) sc[((size_t)row * NT + t) * groups + blk] = (uint8_t)(S + 127);
        }
    }
}

// ---------------------------------------------------------------------------------------------
// launchers (one per kernel family); all return hipGetLastError() of their launch
// ---------------------------------------------------------------------------------------------

// every launcher brackets its launch with these: they call the hooks of the observer of the call in
// progress (moe_layer_observed), if any
void trace(const char* kernel, int phase, hipStream_t st);

// timing events for the launch being enqueued (from the observer's event hook, at trace phase 0;
// null when there is none): every launch goes through MOE_LAUNCH, which hands them to hipExtLaunchKernel
hipEvent_t launch_event(int which);
#define MOE_LAUNCH(kernel, grid, block, shm, st, ...)                                                  \
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)(shm), st, ::moe::launch_event(0),            \
                          ::moe::launch_event(1), 0, __VA_ARGS__)

// One grouped-GEMM tile of the few-token path, written by the fused router: the expert's
// table entry, the tile's first sorted position and pick count (0 = no tile), and the token
// row of each of its picks, so that a GEMM workgroup's set-up is a single 128-byte read.
constexpr int kDescTokens = 8;            // tokens per few-token tile at most (16 / terms)
struct TileDesc {
    moe_expert ex;
    int32_t i0, ntok, e, pad0;
    int32_t tok[kDescTokens];
    int32_t pad1[4];
};
static_assert(sizeof(TileDesc) == 128, "tile record is 128 bytes");

// workspace header: word 0 = status (MOE_WS_* error bits, sticky), word 1 = poll limit of the
// few-token router (0: kPollLimitDefault; < 0: no polls)
constexpr size_t kWsHeaderBytes = 256;
constexpr int kMaxExperts = 1024;
constexpr int kPollLimitDefault = 1 << 20;

struct WsLayout {
    size_t hdr, slots, sink, logits, idx, w, offsets, sorted_pick, pick_pos, perm_blocks, tiles, ntiles, desc, xq, xs,
        hq, hs, o;
    size_t stage_table, stage_list, stage_n, stage_ranges;   // NVFP4 staging (moe_layer)
    size_t total;
    int nt;        // activation terms
    int max_tiles;
};

int act_terms(const moe_shape* s);
int logits_splits(const moe_shape* s, int T);   // K slices of the tiled router (1 for T <= 8)
int super_step(int K, int ksplit);
int act_super_step(int K, int variant);
// slots_for_any_shape: hand-over slots sized for kMaxExperts (a workspace shared by every shape)
WsLayout ws_layout(const moe_shape* s, int32_t T, bool slots_for_any_shape = false);

hipError_t launch_router_logits(const moe_shape* s, const void* x, int T, const float* wr,
                                const float* bias, double* logits, hipStream_t st);
hipError_t launch_topk(const moe_shape* s, const double* logits, int T, int32_t* idx, float* w,
                       hipStream_t st);
hipError_t launch_act_split(const moe_shape* s, const void* x, int rows, int K, int SS, int NT,
                            uint8_t* q, uint8_t* sc, hipStream_t st);
// bcnt: per-block expert counts ([ceil(T * top_k / 1024)][n_experts] int32) or null (one workgroup);
// status: the workspace's status word (MOE_WS_BAD_EXPERT_ID) or null
hipError_t launch_permute(const moe_shape* s, const int32_t* idx, int T, int32_t* offsets,
                          int32_t* sorted_pick, int32_t* pick_pos, int32_t* bcnt, uint32_t* status,
                          hipStream_t st);
// zero words [0, nwords) of a workspace, except word 1 := poll_limit
hipError_t launch_ws_init(uint32_t* ws, size_t nwords, int32_t poll_limit, hipStream_t st);
// tiles of the routed experts' ranges, then (n_shared) the shared expert's: positions [P, P + T)
hipError_t launch_plan(const moe_shape* s, const int32_t* offsets, int T, int tile_tokens, int32_t* tiles,
                       int32_t* ntiles, hipStream_t st);

// fused few-token router (route + permute + plan + activation split); T <= 16, P <= 1024
struct RouteSmallArgs {
    uint32_t* hdr;            // workspace header: status word, poll limit
    const void* x;
    int T, d, E, k;
    const float* wr;
    const float* bias;
    double* logits;
    unsigned long long* slots;  // [T][E] logit hand-over, zero before the launch; the launch leaves it zero
    void* sink;               // write-only scratch for the one-token warm-up pass: >= 8 (E + 1) bytes and
                              // >= max_tiles records
    int32_t* idx;
    float* w;
    int32_t* offsets;
    int32_t* sorted_pick;
    int32_t* pick_pos;
    int32_t* tiles;
    int32_t* ntiles;
    TileDesc* desc;           // [max_tiles]; entries past the last tile get ntok = 0
    const moe_expert* table;
    int max_tiles;
    int tt;                   // tokens per GEMM tile
    uint8_t* xq;
    uint8_t* xs;
    int ss1;                  // MFMAs per chunk of the gate/up GEMM (activation layout)
    int split;                // 1: the other workgroups split x into fp8 terms (MXFP4); 0: not
    float tau;                // renorm-skip threshold (0: off)
    int shared;               // 1: a shared expert (table entry E) at sorted positions T * k + t
};
hipError_t launch_route_small(const moe_shape* s, const RouteSmallArgs& a, hipStream_t st);

// Sorted positions: [0, P) are the routed picks (P = T * k), grouped by expert through the offsets;
// with a shared expert, [P, P + T) are its picks, token t at position P + t, and its table entry is E.
struct GemmArgs {
    const moe_expert* table;
    int d, f, E, k, P;
    int Pall;                 // P + T with a shared expert, else P
    const int32_t* sorted_pick;
    const int32_t* tiles;     // [max_tiles][2] = (expert, first sorted position)
    const int32_t* ntiles;
    const int32_t* offsets;
    const TileDesc* desc;     // few-token kernels: [max_tiles] tile records
    int max_tiles;
    const uint8_t* aq;        // activation terms (x terms by token / h terms by sorted position)
    const uint8_t* as;
    uint8_t* hq;              // gate/up output: h terms
    uint8_t* hs;
    float* o;                 // down output [P][d]
    const int32_t* tile_range;  // NVFP4 staged groups: [t0, t1) of the tiles to run, or null (all)
};

// end of expert e's range of sorted positions (the shared expert, e = E: P + T)
__device__ __forceinline__ int range_end(const GemmArgs& a, int e) { return e < a.E ? a.offsets[e + 1] : a.Pall; }
// token of sorted position i: a routed pick's through sorted_pick, the shared expert's i - P
__device__ __forceinline__ int pos_token(const GemmArgs& a, int i) {
    return i < a.P ? a.sorted_pick[i] / a.k : i - a.P;
}

// picks whose per-row outputs the fused down+combine kernel keeps in LDS (P = T * top_k)
constexpr int kMaxFusedPicks = 512;
constexpr int kMaxDecSlices = 2;          // d_ff / 1024 K slices kept in LDS by the down kernel

struct CombineArgs {
    int T;
    int shared;               // 1: add the shared expert's output (sorted position P + t), unscaled
    int P;
    const float* w;           // [T][k] route weights
    const int32_t* pick_pos;  // [T][k] sorted position of each pick
    const void* residual;     // [T][d] or null
    void* y;                  // [T][d]
    float scaling;
};

// variant: 0 = few tokens per expert (16 columns per tile, K split over the 4 waves when
// possible); 1 = many tokens per expert (128 columns per tile); 2 = between (64 columns per tile)
int gemm_variant(const moe_shape* s, int T);
int gemm_tile_tokens(int variant, int NT);
hipError_t launch_gemm_gateup(const GemmArgs& a, int NT, int variant, int max_tiles, hipStream_t st);
hipError_t launch_gemm_down(const GemmArgs& a, int NT, int variant, int max_tiles, hipStream_t st);
hipError_t launch_down_combine(const moe_shape* s, const GemmArgs& a, const CombineArgs& c, int NT,
                               hipStream_t st);
int ksplit_for(int K, int variant);
// few-token GEMMs with 16 small waves per workgroup (d_model / 4 a multiple of 512, d_ff a
// multiple of 1024 and at most 2048)
bool decode_gemm_ok(const moe_shape* s);
hipError_t launch_gateup_dec(const GemmArgs& a, int NT, int max_tiles, hipStream_t st);
hipError_t launch_down_dec(const moe_shape* s, const GemmArgs& a, const CombineArgs& c, int NT, hipStream_t st);

// NVFP4 (gemm_nv.hip): bf16 terms of fp32 activations, and the grouped GEMMs
constexpr int kNvTilePicks = 4;          // few picks per expert
constexpr int kNvTilePicksMany = 64;     // many picks per expert: the LDS-tiled GEMM's tile
int nv_tile_picks(const moe_shape* s, int T);
constexpr int kStageGroup = 64;           // experts staged per group (NVFP4 layer with staging)
hipError_t launch_bf16_terms(const float* x, int rows, int K, uint16_t* terms, hipStream_t st);
hipError_t launch_nv_gemm(const GemmArgs& a, bool gateup, int NT, int tile_picks, int max_tiles,
                          hipStream_t st);
// the distinct experts of a plan, in groups of kStageGroup, with each group's tile range
// (with a shared expert, its table entry is copied to staged[E]: it is read in place)
hipError_t launch_stage_plan(const moe_shape* s, const int32_t* offsets, int tt, const int32_t* ntiles,
                             int32_t* list, int32_t* nlist, int32_t* ranges, const moe_expert* table,
                             moe_expert* staged, hipStream_t st);
hipError_t launch_gather_group(const moe_shape* s, const moe_expert* table, const int32_t* list,
                               const int32_t* nlist, int group, uint8_t* staging, size_t stride,
                               moe_expert* staged_by_expert, hipStream_t st);

hipError_t launch_combine(const moe_shape* s, const float* o, const float* w, const int32_t* pick_pos,
                          int T, const void* residual, void* y, hipStream_t st);   // (s->n_shared: + o[T k + t])
hipError_t launch_fill_table(const moe_shape* s, const uint8_t* base, size_t stride,
                             moe_expert* table, hipStream_t st);
hipError_t launch_gather(const moe_shape* s, const moe_expert* table, const int32_t* list, int n,
                         uint8_t* staging, size_t stride, moe_expert* staged, hipStream_t st);

}  // namespace moe
