// Grouped expert GEMMs on the gfx950 scaled matrix cores, MXFP4 weights.
//
// Each expert is a gate, an up and a down projection ("Project Maya ...", section "What is in
// the 96.5 GB": one expert blob holds gate, up and down), run as a SwiGLU FFN.  The packed
// E2M1 weights and their E8M0 block scales go from HBM straight into
// V_MFMA_SCALE_F32_16X16X128_F8F6F4 as the FP4 operand with its per-lane block scale, so no
// instruction is spent dequantising them.  The activations (x for gate/up, the SwiGLU output h
// for down) are the FP8 operand, written beforehand as a sum of NT scaled E4M3 terms; each
// MFMA column is one (token, term) pair and the terms are summed in the epilogue.
//
// Operand layout of the 16x16x128 scaled MFMA (measured on gfx950): lane l of the FP4 operand
// holds row l%16 and 32 consecutive K of one 32-block (16 bytes, element 2i in the low
// nibble); the result holds row 4*(l/16)+r, column l%16 in register r; the FP8 operand holds
// column l%16 with its codes in split halves of two K blocks, while the scale of lane group b
// applies to K block b (act_half_offset in the internal header gives the byte order).
//
// Work decomposition: a tile is up to TT consecutive sorted picks of one expert (planned on the
// device); a wave owns 32 weight rows (two 16-row MFMA tiles).  With KSPLIT = 4 the four waves
// of a workgroup split K and reduce through LDS (few tokens per expert: decode); with
// KSPLIT = 1 they own four different row groups (many tokens per expert: prefill).
#include "moe_internal.h"

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

template <int SS>
__device__ __forceinline__ uint32_t load_scale_word(const uint8_t* p) {
    if constexpr (SS == 4) return *(const uint32_t*)p;
    else if constexpr (SS == 2) return *(const uint16_t*)p;
    else return *p;
}

__device__ __forceinline__ v4f mfma_fp4_fp8(const uint4& a, const uint4& b0, const uint4& b1, v4f c,
                                            int sa, int sb) {
    v8i A = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
    v8i B = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, c, 4, 0, 0, sa, 0, sb);
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

template <int NT, int NTN, int KSPLIT, int SS, bool GATEUP>
__global__ __launch_bounds__(256) void k_mx_gemm(GemmArgs a, int ss2) {
    constexpr int NA = GATEUP ? 4 : 2;      // A fragments per MFMA step
    constexpr int TT = 16 * NTN / NT;       // tokens per tile
    const int tile = blockIdx.x;
    if (tile >= *a.ntiles) return;
    const int e = a.tiles[2 * tile], i0 = a.tiles[2 * tile + 1];
    const int ntok = min(TT, a.offsets[e + 1] - i0);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int li = lane & 15, lg = lane >> 4;
    const int K = GATEUP ? a.d : a.f;
    const int rows_out = GATEUP ? a.f : a.d;
    (void)rows_out;
    const moe_expert ex = a.table[e];

    // row group owned by this wave
    const int rg = (KSPLIT == 4) ? blockIdx.y : (blockIdx.y * 4 + wave);
    const int T0 = 32 * rg, T1 = T0 + 16;  // one natural 32-row block of the output
    const int kw = (KSPLIT == 4) ? wave : 0;
    const int kspan = K / KSPLIT;
    const int nss = kspan / (128 * SS);
    const int kss0 = kw * nss;  // first super-step of this wave

    // A fragment pointers (this lane's row, its first K block of the super-step)
    const uint8_t* aq[NA];
    const uint8_t* as[NA];
    {
        const uint8_t* mq0 = GATEUP ? ex.gate_q : ex.down_q;
        const uint8_t* ms0 = GATEUP ? ex.gate_s : ex.down_s;
        const uint8_t* mq1 = GATEUP ? ex.up_q : ex.down_q;
        const uint8_t* ms1 = GATEUP ? ex.up_s : ex.down_s;
#pragma unroll
        for (int f = 0; f < NA; ++f) {
            const int row = ((f & 1) ? T1 : T0) + li;
            const uint8_t* mq = (f < 2) ? mq0 : mq1;
            const uint8_t* ms = (f < 2) ? ms0 : ms1;
            aq[f] = mq + (size_t)row * (K / 2) + lg * 16 * SS + (size_t)kss0 * 64 * SS;
            as[f] = ms + (size_t)row * (K / 32) + lg * SS + (size_t)kss0 * 4 * SS;
        }
    }
    // B column pointers
    const uint8_t* bq[NTN];
    const uint8_t* bs[NTN];
    bool bval[NTN];
#pragma unroll
    for (int n = 0; n < NTN; ++n) {
        const int tc = n * (16 / NT) + li / NT, t = li % NT;
        bval[n] = tc < ntok;
        int arow = 0;
        if (bval[n]) arow = GATEUP ? a.sorted_pick[i0 + tc] / a.k : (i0 + tc);
        bq[n] = a.aq + ((size_t)arow * NT + t) * K + lg * 32 * SS + (size_t)kss0 * 128 * SS;
        bs[n] = a.as + ((size_t)arow * NT + t) * (K / 32) + lg * SS + (size_t)kss0 * 4 * SS;
    }

    v4f acc[NA][NTN];
#pragma unroll
    for (int f = 0; f < NA; ++f)
#pragma unroll
        for (int n = 0; n < NTN; ++n) acc[f][n] = v4f{0.f, 0.f, 0.f, 0.f};

    for (int s = 0; s < nss; ++s) {
        uint4 A[NA][SS];
        uint32_t sa[NA];
#pragma unroll
        for (int f = 0; f < NA; ++f) {
            const uint4* p = (const uint4*)(aq[f] + (size_t)s * 64 * SS);
#pragma unroll
            for (int h = 0; h < SS; ++h) A[f][h] = p[h];
            sa[f] = load_scale_word<SS>(as[f] + (size_t)s * 4 * SS);
        }
        uint32_t sb[NTN];
#pragma unroll
        for (int n = 0; n < NTN; ++n) sb[n] = bval[n] ? load_scale_word<SS>(bs[n] + (size_t)s * 4 * SS) : 0x7f7f7f7fu;
#pragma unroll
        for (int h = 0; h < SS; ++h) {
#pragma unroll
            for (int n = 0; n < NTN; ++n) {
                uint4 b0 = make_uint4(0, 0, 0, 0), b1 = b0;
                if (bval[n]) {
                    const uint4* p = (const uint4*)(bq[n] + (size_t)s * 128 * SS + 32 * h);
                    b0 = p[0];
                    b1 = p[1];
                }
                const int sbv = (int)((sb[n] >> (8 * h)) & 0xffu);
#pragma unroll
                for (int f = 0; f < NA; ++f)
                    acc[f][n] = mfma_fp4_fp8(A[f][h], b0, b1, acc[f][n], (int)((sa[f] >> (8 * h)) & 0xffu), sbv);
            }
        }
    }

    if constexpr (KSPLIT == 4) {
        __shared__ float red[3][NA * NTN * 4][64];
        if (wave > 0) {
#pragma unroll
            for (int f = 0; f < NA; ++f)
#pragma unroll
                for (int n = 0; n < NTN; ++n)
#pragma unroll
                    for (int r = 0; r < 4; ++r) red[wave - 1][(f * NTN + n) * 4 + r][lane] = acc[f][n][r];
        }
        __syncthreads();
        if (wave > 0) return;
#pragma unroll
        for (int w = 0; w < 3; ++w)
#pragma unroll
            for (int f = 0; f < NA; ++f)
#pragma unroll
                for (int n = 0; n < NTN; ++n)
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[f][n][r] += red[w][(f * NTN + n) * 4 + r][lane];
    }

    // sum the NT terms of each token (adjacent columns)
#pragma unroll
    for (int f = 0; f < NA; ++f)
#pragma unroll
        for (int n = 0; n < NTN; ++n)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float v = acc[f][n][r];
                v += __shfl_xor(v, 1);
                if (NT == 4) v += __shfl_xor(v, 2);
                acc[f][n][r] = v;
            }

    if constexpr (GATEUP) {
        // h = silu(g) * u for rows T0..T0+31, split into NT terms with one exponent per term
        // (the 32 rows are one natural block of h's reduction dimension in the down GEMM)
        const int f = a.f;
        const int o0 = act_half_offset(ss2, rg, 0) + 4 * lg, o1 = act_half_offset(ss2, rg, 1) + 4 * lg;
#pragma unroll
        for (int n = 0; n < NTN; ++n) {
            float v[8];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                v[r] = silu(acc[0][n][r]) * acc[2][n][r];
                v[4 + r] = silu(acc[1][n][r]) * acc[3][n][r];
            }
            uint32_t codes[NT][2];
            int S[NT];
            split_terms<NT>(v, codes, S, [](float m) {
                m = fmaxf(m, __shfl_xor(m, 16));
                return fmaxf(m, __shfl_xor(m, 32));
            });
            const int tc = n * (16 / NT) + li / NT, tme = li % NT;
            if (tc < ntok) {
                const size_t pos = (size_t)i0 + tc;
                uint32_t w0 = codes[0][0], w1 = codes[0][1];
                int Sme = S[0];
#pragma unroll
                for (int t = 1; t < NT; ++t)
                    if (t == tme) { w0 = codes[t][0]; w1 = codes[t][1]; Sme = S[t]; }
                uint8_t* dst = a.hq + (pos * NT + tme) * (size_t)f;
                *(uint32_t*)(dst + o0) = w0;
                *(uint32_t*)(dst + o1) = w1;
                if (lg == 0) a.hs[(pos * NT + tme) * (size_t)(f / 32) + rg] = (uint8_t)(Sme + 127);
            }
        }
    } else {
#pragma unroll
        for (int n = 0; n < NTN; ++n) {
            const int tc = n * (16 / NT) + li / NT;
            if (tc < ntok && (li % NT) == 0) {
                float* dst = a.o + ((size_t)i0 + tc) * a.d;
                *(float4*)(dst + T0 + 4 * lg) = make_float4(acc[0][n][0], acc[0][n][1], acc[0][n][2], acc[0][n][3]);
                *(float4*)(dst + T1 + 4 * lg) = make_float4(acc[1][n][0], acc[1][n][1], acc[1][n][2], acc[1][n][3]);
            }
        }
    }
}

int gemm_variant(const moe_shape* s, int T) {
    const long long P = (long long)T * s->top_k;
    return (P <= 8LL * s->n_experts) ? 0 : 1;
}

int gemm_tile_tokens(int variant, int NT) { return (variant == 0 ? 16 : 128) / NT; }

int super_step(int K, int ksplit) {
    const int span = K / ksplit;
    if (span % 512 == 0) return 4;
    if (span % 256 == 0) return 2;
    return 1;
}

static int ksplit_for(int K, int variant) { return (variant == 0 && (K / 4) % 128 == 0) ? 4 : 1; }

template <bool GATEUP, int NT, int NTN>
static hipError_t launch_one(const GemmArgs& a, int ksplit, int SS, int ss2, dim3 grid, hipStream_t st) {
#define MOE_GEMM(KS, S)                                                                                  \
    hipLaunchKernelGGL((k_mx_gemm<NT, NTN, KS, S, GATEUP>), grid, dim3(256), 0, st, a, ss2)
    if (ksplit == 4) {
        if (SS == 4) MOE_GEMM(4, 4);
        else if (SS == 2) MOE_GEMM(4, 2);
        else MOE_GEMM(4, 1);
    } else {
        if (SS == 4) MOE_GEMM(1, 4);
        else if (SS == 2) MOE_GEMM(1, 2);
        else MOE_GEMM(1, 1);
    }
#undef MOE_GEMM
    return hipGetLastError();
}

template <bool GATEUP>
static hipError_t launch_gemm(const GemmArgs& a, int NT, int variant, int max_tiles, hipStream_t st) {
    const int K = GATEUP ? a.d : a.f;
    const int rows = GATEUP ? a.f : a.d;
    const int ks = ksplit_for(K, variant);
    const int SS = super_step(K, ks);
    const int ss2 = super_step(a.f, ksplit_for(a.f, variant));
    dim3 grid(max_tiles, (rows / 32) / (ks == 4 ? 1 : 4));
    if (variant == 0) {
        if (NT == 2) return launch_one<GATEUP, 2, 1>(a, ks, SS, ss2, grid, st);
        return launch_one<GATEUP, 4, 1>(a, ks, SS, ss2, grid, st);
    }
    if (NT == 2) return launch_one<GATEUP, 2, 8>(a, ks, SS, ss2, grid, st);
    return launch_one<GATEUP, 4, 8>(a, ks, SS, ss2, grid, st);
}

hipError_t launch_gemm_gateup(const GemmArgs& a, int NT, int variant, int max_tiles, hipStream_t st) {
    trace("gemm_gate_up", 0, st);
    hipError_t e = launch_gemm<true>(a, NT, variant, max_tiles, st);
    trace("gemm_gate_up", 1, st);
    return e;
}

hipError_t launch_gemm_down(const GemmArgs& a, int NT, int variant, int max_tiles, hipStream_t st) {
    trace("gemm_down", 0, st);
    hipError_t e = launch_gemm<false>(a, NT, variant, max_tiles, st);
    trace("gemm_down", 1, st);
    return e;
}

}  // namespace moe
