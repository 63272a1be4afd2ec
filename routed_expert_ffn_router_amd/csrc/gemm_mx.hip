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
// KSPLIT = 1 they own four different row groups (many tokens per expert: prefill).  The K loop
// issues every load of a chunk of CH super-steps before its MFMAs, so each wave keeps
// CH * 64 * SS bytes per weight fragment in flight.
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

// acc[f][n] += A_f x B_n over nss super-steps (SS MFMAs each), CH super-steps per load burst.
// aq/as: per-lane pointers to this lane's first weight block/scale; bq/bs: activation columns.
template <int NA, int NTN, int SS, int CH>
__device__ __forceinline__ void mx_accumulate(const uint8_t* const (&aq)[NA], const uint8_t* const (&as)[NA],
                                              const uint8_t* const (&bq)[NTN], const uint8_t* const (&bs)[NTN],
                                              const bool (&bval)[NTN], int nss, v4f (&acc)[NA][NTN]) {
    for (int s0 = 0; s0 < nss; s0 += CH) {
        uint4 A[CH][NA][SS];
        uint32_t sa[CH][NA];
        uint4 B[CH][NTN][SS][2];
        uint32_t sb[CH][NTN];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            if (s0 + c >= nss) break;
            const size_t s = (size_t)(s0 + c);
#pragma unroll
            for (int f = 0; f < NA; ++f) {
                const uint4* p = (const uint4*)(aq[f] + s * 64 * SS);
#pragma unroll
                for (int h = 0; h < SS; ++h) A[c][f][h] = p[h];
                sa[c][f] = load_scale_word<SS>(as[f] + s * 4 * SS);
            }
#pragma unroll
            for (int n = 0; n < NTN; ++n) {
                if (bval[n]) {
                    const uint4* p = (const uint4*)(bq[n] + s * 128 * SS);
#pragma unroll
                    for (int h = 0; h < SS; ++h) {
                        B[c][n][h][0] = p[2 * h];
                        B[c][n][h][1] = p[2 * h + 1];
                    }
                    sb[c][n] = load_scale_word<SS>(bs[n] + s * 4 * SS);
                } else {
#pragma unroll
                    for (int h = 0; h < SS; ++h) B[c][n][h][0] = B[c][n][h][1] = make_uint4(0, 0, 0, 0);
                    sb[c][n] = 0x7f7f7f7fu;
                }
            }
        }
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            if (s0 + c >= nss) break;
#pragma unroll
            for (int h = 0; h < SS; ++h)
#pragma unroll
                for (int n = 0; n < NTN; ++n) {
                    const int sbv = (int)((sb[c][n] >> (8 * h)) & 0xffu);
#pragma unroll
                    for (int f = 0; f < NA; ++f)
                        acc[f][n] = mfma_fp4_fp8(A[c][f][h], B[c][n][h][0], B[c][n][h][1], acc[f][n],
                                                 (int)((sa[c][f] >> (8 * h)) & 0xffu), sbv);
                }
        }
    }
}

// sum the NT adjacent (token, term) columns of each token
template <int NA, int NTN, int NT>
__device__ __forceinline__ void sum_terms(v4f (&acc)[NA][NTN]) {
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
}

template <int NT, int NTN, int KSPLIT, int SS, bool GATEUP>
__global__ __launch_bounds__(256) void k_mx_gemm(GemmArgs a, int ss2) {
    constexpr int NA = GATEUP ? 4 : 2;      // A fragments per MFMA step
    constexpr int TT = 16 * NTN / NT;       // tokens per tile
    constexpr int CH = GATEUP ? 1 : 2;
    const int tile = blockIdx.x;
    if (tile >= *a.ntiles) return;
    const int e = a.tiles[2 * tile], i0 = a.tiles[2 * tile + 1];
    const int ntok = min(TT, a.offsets[e + 1] - i0);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int li = lane & 15, lg = lane >> 4;
    const int K = GATEUP ? a.d : a.f;
    const moe_expert ex = a.table[e];

    // row group owned by this wave: one natural 32-row block of the output
    const int rg = (KSPLIT == 4) ? blockIdx.y : (blockIdx.y * 4 + wave);
    const int T0 = 32 * rg, T1 = T0 + 16;
    const int kw = (KSPLIT == 4) ? wave : 0;
    const int nss = (K / KSPLIT) / (128 * SS);
    const int kss0 = kw * nss;  // first super-step of this wave

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
    mx_accumulate<NA, NTN, SS, CH>(aq, as, bq, bs, bval, nss, acc);

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
    sum_terms<NA, NTN, NT>(acc);

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

// ---------------------------------------------------------------------------------------------
// down projection fused with the weighted combine, for few picks (P <= kMaxFusedPicks): one
// workgroup owns 16 output rows of every pick; its eight waves take the tiles in turn, park each
// pick's 16 outputs in LDS, and the workgroup then forms
//   y[t][r] = scaling * sum_j w[t,j] * o[pick_pos[t*k+j]][r] (+ residual[t][r])
// in rank order j, rounded once to the output dtype.
// ---------------------------------------------------------------------------------------------
template <typename XT, int NT, int SS>
__global__ __launch_bounds__(512) void k_mx_down_combine(GemmArgs a, CombineArgs c) {
    constexpr int NTN = 1, TT = 16 / NT, CH = 4;
    __shared__ float o_lds[kMaxFusedPicks][16];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int li = lane & 15, lg = lane >> 4;
    const int r0 = blockIdx.x * 16;
    const int K = a.f;
    const int nss = K / (128 * SS);
    const int ntiles = *a.ntiles;
    for (int tile = wave; tile < ntiles; tile += 8) {
        const int e = a.tiles[2 * tile], i0 = a.tiles[2 * tile + 1];
        const int ntok = min(TT, a.offsets[e + 1] - i0);
        const moe_expert ex = a.table[e];
        const uint8_t* const aq[1] = {ex.down_q + (size_t)(r0 + li) * (K / 2) + lg * 16 * SS};
        const uint8_t* const as[1] = {ex.down_s + (size_t)(r0 + li) * (K / 32) + lg * SS};
        const int tc = li / NT, t = li % NT;
        const bool bval[1] = {tc < ntok};
        const size_t arow = bval[0] ? (size_t)(i0 + tc) : 0;
        const uint8_t* const bq[1] = {a.aq + (arow * NT + t) * K + lg * 32 * SS};
        const uint8_t* const bs[1] = {a.as + (arow * NT + t) * (K / 32) + lg * SS};
        v4f acc[1][1] = {{v4f{0.f, 0.f, 0.f, 0.f}}};
        mx_accumulate<1, NTN, SS, CH>(aq, as, bq, bs, bval, nss, acc);
        sum_terms<1, NTN, NT>(acc);
        if (tc < ntok && t == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) o_lds[i0 + tc][4 * lg + r] = acc[0][0][r];
        }
    }
    __syncthreads();
    const int k = a.k;
    for (int q = threadIdx.x; q < c.T * 16; q += 512) {
        const int tok = q >> 4, r = q & 15;
        float accv = 0.f;
        for (int j = 0; j < k; ++j) {
            const int p = tok * k + j;
            accv = fmaf(c.w[p], o_lds[c.pick_pos[p]][r], accv);
        }
        float v = accv * c.scaling;
        const size_t off = (size_t)tok * a.d + r0 + r;
        if (c.residual) v += load_act((const XT*)c.residual, off);
        store_act((XT*)c.y, off, v);
    }
}

// ---------------------------------------------------------------------------------------------
// few-token ("decode") GEMMs: each wave streams one 16-row tile of one matrix over part of K
// (8-16 KB), the K parts are reduced through LDS in a fixed order, and workgroups are kept to
// eight waves of at most 128 VGPRs so that two of them share a CU and one's epilogue overlaps
// the other's loads.
// ---------------------------------------------------------------------------------------------
constexpr int kDecKSlice = 1024;          // K elements per wave (512 bytes of codes per row)

// gate/up for one tile of picks and one 32-row block: eight waves, wave w = (16-row tile
// f = w/2: gate rows 0-15, gate 16-31, up 0-15, up 16-31; K half ks = w%2).  512 threads and at
// most 128 VGPRs per wave let two workgroups share a CU, so one workgroup's epilogue overlaps
// the other's loads.
template <int NT>
__global__ __launch_bounds__(512, 2) void k_mx_gateup_dec(GemmArgs a, int ss2) {
    constexpr int SS = 4, TT = 16 / NT;
    const int tile = blockIdx.x;
    if (tile >= *a.ntiles) return;
    const int e = a.tiles[2 * tile], i0 = a.tiles[2 * tile + 1];
    const int ntok = min(TT, a.offsets[e + 1] - i0);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int li = lane & 15, lg = lane >> 4;
    const int f = wave >> 1, ks = wave & 1;
    const int K = a.d;
    const int rg = blockIdx.y;
    const int row = 32 * rg + 16 * (f & 1) + li;
    const int nss = (K / 2) / (128 * SS);
    const int kss0 = ks * nss;
    const moe_expert ex = a.table[e];
    const uint8_t* mq = (f >= 2) ? ex.up_q : ex.gate_q;
    const uint8_t* ms = (f >= 2) ? ex.up_s : ex.gate_s;
    const uint8_t* const aq[1] = {mq + (size_t)row * (K / 2) + lg * 16 * SS + (size_t)kss0 * 64 * SS};
    const uint8_t* const as[1] = {ms + (size_t)row * (K / 32) + lg * SS + (size_t)kss0 * 4 * SS};
    const int tc = li / NT, t = li % NT;
    const bool bval[1] = {tc < ntok};
    const size_t arow = bval[0] ? (size_t)(a.sorted_pick[i0 + tc] / a.k) : 0;
    const uint8_t* const bq[1] = {a.aq + (arow * NT + t) * K + lg * 32 * SS + (size_t)kss0 * 128 * SS};
    const uint8_t* const bs[1] = {a.as + (arow * NT + t) * (K / 32) + lg * SS + (size_t)kss0 * 4 * SS};
    v4f acc[1][1] = {{v4f{0.f, 0.f, 0.f, 0.f}}};
    mx_accumulate<1, 1, SS, 2>(aq, as, bq, bs, bval, nss, acc);

    __shared__ float4 part[8][64];
    part[wave][lane] = make_float4(acc[0][0][0], acc[0][0][1], acc[0][0][2], acc[0][0][3]);
    __syncthreads();
    if (wave > 0) return;
    // wave 0: add the two K halves of each 16-row tile, then SwiGLU and the split of the block
    v4f gu[4][1];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float4 p0 = part[2 * q][lane], p1 = part[2 * q + 1][lane];
        gu[q][0] = v4f{p0.x + p1.x, p0.y + p1.y, p0.z + p1.z, p0.w + p1.w};
    }
    sum_terms<4, 1, NT>(gu);
    float v[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        v[r] = silu(gu[0][0][r]) * gu[2][0][r];
        v[4 + r] = silu(gu[1][0][r]) * gu[3][0][r];
    }
    uint32_t codes[NT][2];
    int S[NT];
    split_terms<NT>(v, codes, S, [](float mm) {
        mm = fmaxf(mm, __shfl_xor(mm, 16));
        return fmaxf(mm, __shfl_xor(mm, 32));
    });
    if (tc < ntok) {
        const size_t pos = (size_t)i0 + tc;
        uint32_t w0 = codes[0][0], w1 = codes[0][1];
        int Sme = S[0];
#pragma unroll
        for (int q = 1; q < NT; ++q)
            if (q == t) { w0 = codes[q][0]; w1 = codes[q][1]; Sme = S[q]; }
        uint8_t* dst = a.hq + (pos * NT + t) * (size_t)a.f;
        *(uint32_t*)(dst + act_half_offset(ss2, rg, 0) + 4 * lg) = w0;
        *(uint32_t*)(dst + act_half_offset(ss2, rg, 1) + 4 * lg) = w1;
        if (lg == 0) a.hs[(pos * NT + t) * (size_t)(a.f / 32) + rg] = (uint8_t)(Sme + 127);
    }
}

// down projection + weighted combine for few picks: workgroup = 16 output rows; its 16 waves
// take (tile, K slice) units in turn (K slice = kDecKSlice of d_ff; eight waves per workgroup), park each unit's 16 outputs
// per pick in LDS, and the workgroup sums slices and picks in a fixed order.
template <typename XT, int NT>
__global__ __launch_bounds__(512, 2) void k_mx_down_dec(GemmArgs a, CombineArgs c) {
    constexpr int SS = 4, TT = 16 / NT;
    __shared__ float o_part[kMaxDecSlices][kMaxFusedPicks][16];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int li = lane & 15, lg = lane >> 4;
    const int r0 = blockIdx.x * 16;
    const int K = a.f;
    const int nsl = K / kDecKSlice;
    const int nss = kDecKSlice / (128 * SS);
    const int units = *a.ntiles * nsl;
    for (int unit = wave; unit < units; unit += 8) {
        const int tile = unit / nsl, ks = unit % nsl;
        const int e = a.tiles[2 * tile], i0 = a.tiles[2 * tile + 1];
        const int ntok = min(TT, a.offsets[e + 1] - i0);
        const moe_expert ex = a.table[e];
        const int kss0 = ks * nss;
        const uint8_t* const aq[1] = {ex.down_q + (size_t)(r0 + li) * (K / 2) + lg * 16 * SS + (size_t)kss0 * 64 * SS};
        const uint8_t* const as[1] = {ex.down_s + (size_t)(r0 + li) * (K / 32) + lg * SS + (size_t)kss0 * 4 * SS};
        const int tc = li / NT, t = li % NT;
        const bool bval[1] = {tc < ntok};
        const size_t arow = bval[0] ? (size_t)(i0 + tc) : 0;
        const uint8_t* const bq[1] = {a.aq + (arow * NT + t) * K + lg * 32 * SS + (size_t)kss0 * 128 * SS};
        const uint8_t* const bs[1] = {a.as + (arow * NT + t) * (K / 32) + lg * SS + (size_t)kss0 * 4 * SS};
        v4f acc[1][1] = {{v4f{0.f, 0.f, 0.f, 0.f}}};
        mx_accumulate<1, 1, SS, 2>(aq, as, bq, bs, bval, nss, acc);
        sum_terms<1, 1, NT>(acc);
        if (tc < ntok && t == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) o_part[ks][i0 + tc][4 * lg + r] = acc[0][0][r];
        }
    }
    __syncthreads();
    const int k = a.k;
    for (int q = threadIdx.x; q < c.T * 16; q += 512) {
        const int tok = q >> 4, r = q & 15;
        float accv = 0.f;
        for (int j = 0; j < k; ++j) {
            const int p = tok * k + j;
            const int pos = c.pick_pos[p];
            float o = 0.f;
            for (int sl = 0; sl < nsl; ++sl) o += o_part[sl][pos][r];
            accv = fmaf(c.w[p], o, accv);
        }
        float v = accv * c.scaling;
        const size_t off = (size_t)tok * a.d + r0 + r;
        if (c.residual) v += load_act((const XT*)c.residual, off);
        store_act((XT*)c.y, off, v);
    }
}

bool decode_gemm_ok(const moe_shape* s) {
    return (s->d_model / 2) % 512 == 0 && s->d_ff % kDecKSlice == 0 && s->d_ff / kDecKSlice <= kMaxDecSlices;
}

hipError_t launch_gateup_dec(const GemmArgs& a, int NT, int max_tiles, hipStream_t st) {
    trace("gemm_gate_up", 0, st);
    const int ss2 = 4;   // h terms in chunks of 512: the layout k_mx_down_dec reads
    dim3 grid(max_tiles, a.f / 32);
    if (NT == 2) hipLaunchKernelGGL(k_mx_gateup_dec<2>, grid, dim3(512), 0, st, a, ss2);
    else hipLaunchKernelGGL(k_mx_gateup_dec<4>, grid, dim3(512), 0, st, a, ss2);
    trace("gemm_gate_up", 1, st);
    return hipGetLastError();
}

hipError_t launch_down_dec(const moe_shape* s, const GemmArgs& a, const CombineArgs& c, int NT, hipStream_t st) {
    trace("down_combine", 0, st);
    dim3 grid(a.d / 16);
    const bool bf = s->act_dtype == MOE_DT_BF16;
    if (bf) {
        if (NT == 2) hipLaunchKernelGGL((k_mx_down_dec<uint16_t, 2>), grid, dim3(512), 0, st, a, c);
        else hipLaunchKernelGGL((k_mx_down_dec<uint16_t, 4>), grid, dim3(512), 0, st, a, c);
    } else {
        if (NT == 2) hipLaunchKernelGGL((k_mx_down_dec<float, 2>), grid, dim3(512), 0, st, a, c);
        else hipLaunchKernelGGL((k_mx_down_dec<float, 4>), grid, dim3(512), 0, st, a, c);
    }
    trace("down_combine", 1, st);
    return hipGetLastError();
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

int ksplit_for(int K, int variant) { return (variant == 0 && (K / 4) % 128 == 0) ? 4 : 1; }

template <bool GATEUP, int NT, int NTN, int KS>
static hipError_t launch_one(const GemmArgs& a, int SS, int ss2, dim3 grid, hipStream_t st) {
    if (SS == 4) hipLaunchKernelGGL((k_mx_gemm<NT, NTN, KS, 4, GATEUP>), grid, dim3(256), 0, st, a, ss2);
    else if (SS == 2) hipLaunchKernelGGL((k_mx_gemm<NT, NTN, KS, 2, GATEUP>), grid, dim3(256), 0, st, a, ss2);
    else hipLaunchKernelGGL((k_mx_gemm<NT, NTN, KS, 1, GATEUP>), grid, dim3(256), 0, st, a, ss2);
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
        if (ks == 4) return NT == 2 ? launch_one<GATEUP, 2, 1, 4>(a, SS, ss2, grid, st)
                                    : launch_one<GATEUP, 4, 1, 4>(a, SS, ss2, grid, st);
        return NT == 2 ? launch_one<GATEUP, 2, 1, 1>(a, SS, ss2, grid, st)
                       : launch_one<GATEUP, 4, 1, 1>(a, SS, ss2, grid, st);
    }
    return NT == 2 ? launch_one<GATEUP, 2, 8, 1>(a, SS, ss2, grid, st)
                   : launch_one<GATEUP, 4, 8, 1>(a, SS, ss2, grid, st);
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

hipError_t launch_down_combine(const moe_shape* s, const GemmArgs& a, const CombineArgs& c, int NT,
                               hipStream_t st) {
    trace("down_combine", 0, st);
    // the h terms were written in the few-token down GEMM's layout (chunks of d_ff / 4)
    const int SS = super_step(a.f, ksplit_for(a.f, 0));
    dim3 grid(a.d / 16);
    const bool bf = s->act_dtype == MOE_DT_BF16;
#define MOE_DC(XT, N, S) hipLaunchKernelGGL((k_mx_down_combine<XT, N, S>), grid, dim3(512), 0, st, a, c)
#define MOE_DC_SS(XT, N) \
    do { if (SS == 4) MOE_DC(XT, N, 4); else if (SS == 2) MOE_DC(XT, N, 2); else MOE_DC(XT, N, 1); } while (0)
    if (bf) {
        if (NT == 2) MOE_DC_SS(uint16_t, 2);
        else MOE_DC_SS(uint16_t, 4);
    } else {
        if (NT == 2) MOE_DC_SS(float, 2);
        else MOE_DC_SS(float, 4);
    }
#undef MOE_DC_SS
#undef MOE_DC
    trace("down_combine", 1, st);
    return hipGetLastError();
}

}  // namespace moe
