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
    if constexpr (SS == 4) return gload4(p);
    else if constexpr (SS == 2) return *(__attribute__((address_space(1))) const uint16_t*)p;
    else return *(__attribute__((address_space(1))) const uint8_t*)p;
}

__device__ __forceinline__ v4f mfma_fp4_fp8(const uint4& a, const uint4& b0, const uint4& b1, v4f c,
                                            int sa, int sb) {
    v8i A = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
    v8i B = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, c, 4, 0, 0, sa, 0, sb);
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }


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
                const uint8_t* p = aq[f] + s * 64 * SS;
#pragma unroll
                for (int h = 0; h < SS; ++h) A[c][f][h] = gload16(p + 16 * h);
                sa[c][f] = load_scale_word<SS>(as[f] + s * 4 * SS);
            }
#pragma unroll
            for (int n = 0; n < NTN; ++n) {
                if (bval[n]) {
                    const uint8_t* p = bq[n] + s * 128 * SS;
#pragma unroll
                    for (int h = 0; h < SS; ++h) {
                        B[c][n][h][0] = gload16(p + 32 * h);
                        B[c][n][h][1] = gload16(p + 32 * h + 16);
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
            for (int r = 0; r < 4; ++r) acc[f][n][r] = sum_adjacent<NT>(acc[f][n][r]);
}

template <int NT, int NTN, int KSPLIT, int SS, bool GATEUP>
__global__ __launch_bounds__(256) void k_mx_gemm(GemmArgs a, int ss2, int nrg) {
    // output rows per row group: 32 (gate/up: the same 32 rows of gate and of up); down with K split
    // four ways 64, so that a workgroup streams as many weight bytes as a gate/up one (with 32, twice
    // the workgroups each brought half the bytes, and down ran at about 70% of gate/up's rate)
    constexpr int RB = (GATEUP || KSPLIT != 4) ? 32 : 64;
    constexpr int NA = GATEUP ? 4 : RB / 16;  // A fragments per MFMA step
    // tokens per tile: the tile's columns, at most the tokens a few-token tile record holds
    constexpr int TT = (16 * NTN / NT) < kDescTokens ? 16 * NTN / NT : kDescTokens;
    constexpr int CH = NA == 4 ? 1 : 2;      // super-steps per load burst: 16 weight loads per lane either way
    // workgroup -> (tile, row group gy of nrg): XCD x = id % 8 takes row groups x, x + 8, .. and,
    // within each, the tiles in order, so that the tiles of one expert (consecutive) read the same
    // weight rows on one XCD at about the same time and share its L2 (with the tiles as the grid's
    // fast dimension they landed on different XCDs, and HBM served each tile's weights again:
    // 1.15x / 1.24x the algorithmic bytes for gate/up / down in a skewed 64-token batch)
    const int g = blockIdx.x, j = g >> 3;
    const int gy = (g & 7) + 8 * (j / a.max_tiles), tile = j % a.max_tiles;
    if (gy >= nrg || tile >= *a.ntiles) return;
    const int e = a.tiles[2 * tile], i0 = a.tiles[2 * tile + 1];
    const int ntok = min(TT, range_end(a, e) - i0);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int li = lane & 15, lg = lane >> 4;
    const int K = GATEUP ? a.d : a.f;
    const moe_expert ex = a.table[e];

    // row group owned by this wave: one natural 32-row block of the output
    const int rg = (KSPLIT == 4) ? gy : (gy * 4 + wave);
    const int T0 = RB * rg, T1 = T0 + 16;
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
            // gate/up: gate rows T0, T1 then up rows T0, T1; down: rows T0 + 16 f
            const int row = GATEUP ? ((f & 1) ? T1 : T0) + li : T0 + 16 * f + li;
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
        if (bval[n]) arow = GATEUP ? pos_token(a, i0 + tc) : (i0 + tc);
        bq[n] = a.aq + ((size_t)arow * NT + t) * K + lg * 32 * SS + (size_t)kss0 * 128 * SS;
        bs[n] = a.as + ((size_t)arow * NT + t) * (K / 32) + lg * SS + (size_t)kss0 * 4 * SS;
    }

    v4f acc[NA][NTN];
#pragma unroll
    for (int f = 0; f < NA; ++f)
#pragma unroll
        for (int n = 0; n < NTN; ++n) acc[f][n] = v4f{0.f, 0.f, 0.f, 0.f};
    mx_accumulate<NA, NTN, SS, CH>(aq, as, bq, bs, bval, nss, acc);
#pragma unroll
    for (int f = 0; f < NA; ++f)
#pragma unroll
        for (int n = 0; n < NTN; ++n) mfma_results_here(acc[f][n]);

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
            split_terms<NT>(v, codes, S, [](float m) { return max_xor32(max_xor16(m)); });
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
#pragma unroll
                for (int f = 0; f < NA; ++f)
                    *(float4*)(dst + T0 + 16 * f + 4 * lg) =
                        make_float4(acc[f][n][0], acc[f][n][1], acc[f][n][2], acc[f][n][3]);
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
    constexpr int NTN = 1, TT = (16 / NT) < kDescTokens ? 16 / NT : kDescTokens, CH = 4;
    __shared__ float o_lds[kMaxFusedPicks][16];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int li = lane & 15, lg = lane >> 4;
    const int r0 = blockIdx.x * 16;
    const int K = a.f;
    const int nss = K / (128 * SS);
    const int ntiles = *a.ntiles;
    for (int tile = wave; tile < ntiles; tile += 8) {
        const int e = a.tiles[2 * tile], i0 = a.tiles[2 * tile + 1];
        const int ntok = min(TT, range_end(a, e) - i0);
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
        mfma_results_here(acc[0][0]);
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
            const int pos = c.pick_pos[p];
            if (pos >= 0) accv = fmaf(c.w[p], o_lds[pos][r], accv);   // (a dropped pick has none)
        }
        float v = accv * c.scaling;
        if (c.shared) v += o_lds[c.P + tok][r];                            // the shared expert, unscaled
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
// f = w/2: gate rows 0-15, gate 16-31, up 0-15, up 16-31; K half ks = w%2).  Every wave issues
// all of its weight loads (16 MFMAs' worth, 64 VGPRs) at once; the tile's x terms are staged in
// LDS by the whole workgroup meanwhile, so the FP8 operand costs no registers.  512 threads and
// at most 128 VGPRs per wave (four waves per SIMD: the second launch bound) let two workgroups
// share a CU, so one's epilogue overlaps the other's loads.
constexpr int kDecCols = 16;              // MFMA columns: (token, term) pairs of a tile
constexpr int kDecMaxD = 4096;            // d_model staged per column
constexpr int kDecSteps = 16;             // MFMAs per wave (K / 2 = 2048 at d_model 4096)

template <int NT>
__global__ __launch_bounds__(512, 4) void k_mx_gateup_dec(GemmArgs a, int ss2, int nwg) {
    constexpr int SS = 4, NSS = kDecSteps / SS;
    __shared__ __align__(16) uint8_t b_lds[kDecCols][kDecMaxD + 16];
    __shared__ __align__(16) uint8_t bs_lds[kDecCols][kDecMaxD / 32];
    __shared__ float4 part[8][64];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int li = lane & 15, lg = lane >> 4;
    const int f = wave >> 1, ks = wave & 1;
    const int K = a.d;
    const int nss = (K / 2) / (128 * SS);     // super-steps of this wave (<= NSS)
    // (tile, 32-row block) pairs p = tile * nrg + rg, taken by the workgroups in turn; the grid
    // never exceeds the pairs of max_tiles tiles, so the first record read is always in bounds
    const int nrg = a.f / 32;
    // a tile record's fields, read on the scalar path (the vector path would queue them behind the
    // weight loads of the other workgroup on this CU)
    struct Rec {
        const uint8_t *gq, *uq, *gs, *us;
        int i0, ntok, tk[kDescTokens];
    };
    static_assert(kDescTokens == 8, "token fields of a tile record");
    auto load_rec = [&](int tile) {
        const TileDesc* D = a.desc + tile;
        Rec r;
        r.gq = sload(&D->ex.gate_q);
        r.uq = sload(&D->ex.up_q);
        r.gs = sload(&D->ex.gate_s);
        r.us = sload(&D->ex.up_s);
        r.i0 = sload(&D->i0);
        r.ntok = sload(&D->ntok);
#pragma unroll
        for (int j = 0; j < kDescTokens; ++j) r.tk[j] = sload(&D->tok[j]);
        return r;
    };
    // the first pair's record and the tile count in one round trip (all requested before the
    // first wait); each later pair's record is requested at the start of the pair before it
    int pair = blockIdx.x;                                // nwg = grid size, passed as an argument
    const int32_t* ntp = a.ntiles;
    asm volatile("" : "+s"(ntp));     // read with the record in one round trip, not hoisted ahead of it
    const int ntile_count = sload(ntp);
    Rec rec = load_rec(__builtin_amdgcn_readfirstlane(pair / nrg));
    asm volatile("" ::"s"(ntile_count), "s"(rec.gq), "s"(rec.uq), "s"(rec.gs), "s"(rec.us), "s"(rec.i0),
                 "s"(rec.ntok), "s"(rec.tk[0]), "s"(rec.tk[1]), "s"(rec.tk[2]), "s"(rec.tk[3]), "s"(rec.tk[4]),
                 "s"(rec.tk[5]), "s"(rec.tk[6]), "s"(rec.tk[7]));
    for (;;) {
    const int tile = __builtin_amdgcn_readfirstlane(pair / nrg), rg = __builtin_amdgcn_readfirstlane(pair % nrg);
    if (tile >= ntile_count) break;
    // the next pair's record, requested now and used by the next pass (none when this pair is the
    // workgroup's last: one pair per workgroup with one token)
    const bool more = pair + nwg < ntile_count * nrg;
    Rec nrec = rec;
    if (more) nrec = load_rec(__builtin_amdgcn_readfirstlane((pair + nwg) / nrg));
    const uint8_t* const gq = rec.gq;
    const uint8_t* const uq = rec.uq;
    const uint8_t* const gs = rec.gs;
    const uint8_t* const us = rec.us;
    const int i0 = rec.i0;
    const int ntok = rec.ntok;
    const int tk0 = rec.tk[0], tk1 = rec.tk[1], tk2 = rec.tk[2], tk3 = rec.tk[3];
    const int tk4 = rec.tk[4], tk5 = rec.tk[5], tk6 = rec.tk[6], tk7 = rec.tk[7];
    const int row = 32 * rg + 16 * (f & 1) + li;
    const int kss0 = ks * nss;
    // 1. the tile's x terms (ncol columns of K code bytes and K/32 scale bytes) are staged in LDS,
    // one 16-byte chunk per thread and round; the token of this thread's first chunk is read
    // before the weights are requested
    const int ncol = ntok * NT;
    const int nchunk = ncol * (K / 16), ntotal = nchunk + ncol * (K / 512);
    auto chunk_col = [&](int g, int& off) {
        const bool data = g < nchunk;
        const int per = data ? K / 16 : K / 512;
        const int gg = data ? g : g - nchunk;
        off = (gg % per) * 16;
        return gg / per;
    };
    auto chunk_src = [&](int g, int tok, int c, int off) -> const uint8_t* {
        const size_t tokrow = (size_t)tok * NT + c % NT;
        return g < nchunk ? a.aq + tokrow * K + off : a.as + tokrow * (K / 32) + off;
    };
    auto chunk_dst = [&](int g, int c, int off) -> uint4* {
        return g < nchunk ? (uint4*)&b_lds[c][off] : (uint4*)&bs_lds[c][off];
    };
    // token of a chunk's column: tok[c / NT] of the record
    auto chunk_tok = [&](int c) {
        const int ti = c / NT;
        const int a01 = (ti & 1) ? tk1 : tk0, a23 = (ti & 1) ? tk3 : tk2;
        const int a45 = (ti & 1) ? tk5 : tk4, a67 = (ti & 1) ? tk7 : tk6;
        const int a03 = (ti & 2) ? a23 : a01, a47 = (ti & 2) ? a67 : a45;
        return (ti & 4) ? a47 : a03;
    };
    const int g0 = tid < ntotal ? tid : ntotal - 1;
    int off0;
    const int c0 = chunk_col(g0, off0);
    const int tok0 = chunk_tok(c0);
    const uint4 xv0 = gload16(chunk_src(g0, tok0, c0, off0));
    __builtin_amdgcn_sched_barrier(0);       // keep it ahead of the weight loads
    // 2. this wave's weights: all loads at once (super-steps past nss re-read the last one), after
    // the x-term chunk, so that storing that chunk waits only for it
    const uint8_t* mq = (f >= 2) ? uq : gq;
    const uint8_t* ms = (f >= 2) ? us : gs;
    const uint8_t* aq = (mq + (size_t)row * (K / 2) + lg * 16 * SS + (size_t)kss0 * 64 * SS);
    const uint8_t* as = (ms + (size_t)row * (K / 32) + lg * SS + (size_t)kss0 * 4 * SS);
    uint4 A[NSS][SS];
    uint32_t sa[NSS];
#pragma unroll
    for (int q = 0; q < NSS; ++q) {
        const int qq = q < nss ? q : nss - 1;
#pragma unroll
        for (int h = 0; h < SS; ++h) A[q][h] = gload16(aq + (size_t)qq * 64 * SS + 16 * h);
        sa[q] = gload4(as + (size_t)qq * 4 * SS);
    }
    // 3. the x-term chunks to LDS
    if (tid < ntotal) *chunk_dst(g0, c0, off0) = xv0;
    for (int g = tid + 512; g < ntotal; g += 512) {      // more than 512 chunks: tiles of many picks
        int off;
        const int c = chunk_col(g, off);
        const int tok = chunk_tok(c);
        const uint4 v = gload16(chunk_src(g, tok, c, off));
        *chunk_dst(g, c, off) = v;
    }
    lds_barrier();
    // 4. MFMAs, FP8 operand from LDS, one super-step's operands read before its MFMAs (columns
    // past the tile read its last column; their results are not used).  The barrier above does
    // not wait for the weights: each super-step's MFMAs start when its own weights are in.
    const int col = li < ncol ? li : ncol - 1;
    const uint8_t* bl = &b_lds[col][(size_t)kss0 * 128 * SS + lg * 32 * SS];
    const uint8_t* bsl = &bs_lds[col][kss0 * 4 * SS + lg * SS];
    v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < NSS; ++q) {
        if (q < nss) {
            const uint32_t sb = *(const uint32_t*)(bsl + q * 4 * SS);
            uint4 B[SS][2];
#pragma unroll
            for (int h = 0; h < SS; ++h) {
                B[h][0] = *(const uint4*)(bl + q * 128 * SS + 32 * h);
                B[h][1] = *(const uint4*)(bl + q * 128 * SS + 32 * h + 16);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int h = 0; h < SS; ++h)
                acc = mfma_fp4_fp8(A[q][h], B[h][0], B[h][1], acc, (int)((sa[q] >> (8 * h)) & 0xffu),
                                   (int)((sb >> (8 * h)) & 0xffu));
        }
    }

    part[wave][lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    __syncthreads();
    if (wave == 0) {
    // wave 0: add the two K halves of each 16-row tile, then SwiGLU and the split of the block
    // (the other waves go on to the next pair; its LDS fill barrier waits for this wave)
    const int tc = li / NT, t = li % NT;
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
    split_terms<NT>(v, codes, S, [](float mm) { return max_xor32(max_xor16(mm)); });
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
    if (!more) break;
    pair += nwg;
    rec = nrec;
    }
}

// down projection + weighted combine for few picks: workgroup = 16 output rows; its sixteen
// waves take (tile, K slice) units in turn (K slice = kDecKSlice of d_ff), park each unit's 16
// outputs per pick in LDS, and the workgroup sums slices and picks in a fixed order.  A wave has
// one unit in flight at a time (its loads, then its MFMAs), so sixteen waves rather than eight
// keep twice the bytes in flight per CU (at most 128 VGPRs, four waves per SIMD).
// PLAIN: no renorm-skip and no shared expert (known at compile time): every pick has a position,
// so the combine carries no test for dropped picks and no shared row (about 0.5 us of its tail)
constexpr int kDownDecWaves = 16;
// tile records the kernel keeps in LDS: the most a few-token layer plans (picks of at most
// kMaxFusedPicks, tiles of at least 4 picks, one ragged tile per expert and the shared expert's)
constexpr int kDownDecMaxTiles = 648;
template <typename XT, int NT, bool PLAIN>
__global__ __launch_bounds__(64 * kDownDecWaves) void k_mx_down_dec(GemmArgs a, CombineArgs c) {
    constexpr int SS = 4;
    __shared__ float o_part[kMaxDecSlices][kMaxFusedPicks][16];
    // the fields of the tile records that the units read, staged once (one round trip for the
    // workgroup), instead of two dependent loads of the record per unit
    __shared__ const uint8_t* s_dq[kDownDecMaxTiles];
    __shared__ const uint8_t* s_ds[kDownDecMaxTiles];
    __shared__ int s_i0[kDownDecMaxTiles], s_nt[kDownDecMaxTiles];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int li = lane & 15, lg = lane >> 4;
    const int r0 = blockIdx.x * 16;
    const int K = a.f;
    const int nsl = K / kDecKSlice;
    const int nss = kDecKSlice / (128 * SS);
    const int units = a.max_tiles * nsl;          // (max_tiles <= kDownDecMaxTiles: checked at launch)
    for (int t = threadIdx.x; t < a.max_tiles; t += 64 * kDownDecWaves) {
        const TileDesc* D = a.desc + t;
        s_dq[t] = D->ex.down_q;
        s_ds[t] = D->ex.down_s;
        s_i0[t] = D->i0;
        s_nt[t] = D->ntok;
    }
    __syncthreads();
    for (int unit = wave; unit < units; unit += kDownDecWaves) {
        const int tile = unit / nsl, ks = unit % nsl;
        const int ntok = s_nt[tile];
        if (ntok == 0) continue;
        const int i0 = s_i0[tile];
        const int kss0 = ks * nss;
        const uint8_t* const aq[1] = {s_dq[tile] + (size_t)(r0 + li) * (K / 2) + lg * 16 * SS + (size_t)kss0 * 64 * SS};
        const uint8_t* const as[1] = {s_ds[tile] + (size_t)(r0 + li) * (K / 32) + lg * SS + (size_t)kss0 * 4 * SS};
        const int tc = li / NT, t = li % NT;
        const bool bval[1] = {tc < ntok};
        const size_t arow = bval[0] ? (size_t)(i0 + tc) : 0;
        const uint8_t* const bq[1] = {a.aq + (arow * NT + t) * K + lg * 32 * SS + (size_t)kss0 * 128 * SS};
        const uint8_t* const bs[1] = {a.as + (arow * NT + t) * (K / 32) + lg * SS + (size_t)kss0 * 4 * SS};
        v4f acc[1][1] = {{v4f{0.f, 0.f, 0.f, 0.f}}};
        mx_accumulate<1, 1, SS, 2>(aq, as, bq, bs, bval, nss, acc);
        mfma_results_here(acc[0][0]);
        sum_terms<1, 1, NT>(acc);
        if (tc < ntok && t == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) o_part[ks][i0 + tc][4 * lg + r] = acc[0][0][r];
        }
    }
    __syncthreads();
    const int k = a.k;
    for (int q = threadIdx.x; q < c.T * 16; q += 64 * kDownDecWaves) {
        const int tok = q >> 4, r = q & 15;
        float accv = 0.f;
        for (int j = 0; j < k; ++j) {
            const int p = tok * k + j;
            const int pos = c.pick_pos[p];
            if (!PLAIN && pos < 0) continue;        // a dropped pick
            float o = 0.f;
            for (int sl = 0; sl < nsl; ++sl) o += o_part[sl][pos][r];
            accv = fmaf(c.w[p], o, accv);
        }
        float v = accv * c.scaling;
        if (!PLAIN && c.shared) {                        // the shared expert, unscaled
            float o = 0.f;
            for (int sl = 0; sl < nsl; ++sl) o += o_part[sl][c.P + tok][r];
            v += o;
        }
        const size_t off = (size_t)tok * a.d + r0 + r;
        if (c.residual) v += load_act((const XT*)c.residual, off);
        store_act((XT*)c.y, off, v);
    }
}

// down projection + weighted combine for very few picks (P * NT <= 32, d_ff <= 2048): one
// workgroup of 16 output rows per CU.  Round trip 1 fetches the tile records and the combine's
// inputs.  Then waves 4-7 request the weights of their two (tile, K slice) units at once, while
// waves 0-3 first stage every pick's h terms in LDS and only then request theirs: a wave cannot
// get past a long run of load instructions until the CU's memory pipeline has taken them, so an
// LDS store placed after its weight requests would wait for most of the weight stream.  Each wave
// waits for the staged h terms (an LDS counter, not a barrier) just before its MFMAs.
constexpr int kDownLdsCols = 32;
constexpr int kDownMaxF = 2048;
constexpr int kDownMaxTiles = 32;
constexpr int kDownFillThreads = 256;      // waves 0-3 stage the h terms
constexpr int kDownFillRounds =
    (kDownLdsCols * (kDownMaxF / 16 + kDownMaxF / 512) + kDownFillThreads - 1) / kDownFillThreads;

template <typename XT, int NT, bool PLAIN>
__global__ __launch_bounds__(512, 2) void k_mx_down_dec_lds(GemmArgs a, CombineArgs c) {
    constexpr int SS = 4, NSS = kDecKSlice / (128 * SS);
    constexpr int MAXP = kDownLdsCols / NT;
    __shared__ __align__(16) uint8_t b_lds[kDownLdsCols][kDownMaxF + 16];
    __shared__ __align__(16) uint8_t bs_lds[kDownLdsCols][kDownMaxF / 32];
    __shared__ __align__(16) TileDesc d_lds[kDownMaxTiles];
    __shared__ float o_part[kMaxDecSlices][MAXP][16];
    __shared__ float s_wq[MAXP];
    __shared__ int s_posq[MAXP];
    __shared__ int s_staged;                        // filler waves done with the h terms
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int li = lane & 15, lg = lane >> 4;
    const int r0 = blockIdx.x * 16;
    const int K = a.f;
    const int nsl = K / kDecKSlice;
    const int P = a.P, ncols = a.Pall * NT;         // picks; h columns (with the shared expert's)
    // 1. tile records (16-byte chunks, one per thread), this thread's pick weight and position,
    // and the residual of the output it will write (thread q = tid writes token q/16, row
    // r0 + q%16): one round trip
    const int nd = a.max_tiles * 8;
    const uint4 dv = gload16((const uint8_t*)a.desc + (size_t)(tid < nd ? tid : nd - 1) * 16);
    const int pq = tid < P ? tid : P - 1;
    const float wq = c.w[pq];
    const int posq = c.pick_pos[pq];
    const int oq = tid < c.T * 16 ? tid : c.T * 16 - 1;
    const size_t yoff = (size_t)(oq >> 4) * a.d + r0 + (oq & 15);
    const XT* rsrc = c.residual ? (const XT*)c.residual : (const XT*)c.y;   // read, used only with a residual
    const float resq = load_act(rsrc, yoff);
    asm volatile("" ::"v"(dv.x), "v"(dv.y), "v"(dv.z), "v"(dv.w), "v"(wq), "v"(posq), "v"(resq));
    if (tid < nd) *((uint4*)&d_lds[0] + tid) = dv;
    if (tid < P) {
        s_wq[tid] = wq;
        s_posq[tid] = posq;
    }
    if (tid == 0) s_staged = 0;
    __syncthreads();
    // 2. every pick's h codes and scales (first P*NT rows of the h terms), by waves 0-3: all
    // requests of a wave first, then its LDS stores (only the rounds that hold chunks; the round
    // count is uniform)
    const int nb = ncols * (K / 16), ntot = nb + ncols * (K / 512);
    const bool filler = wave < kDownFillThreads / 64;
    auto stage_h = [&]() {
        uint4 v[kDownFillRounds];
#pragma unroll
        for (int r = 0; r < kDownFillRounds; ++r) {
            if (r * kDownFillThreads < ntot) {
                int g = r * kDownFillThreads + tid;
                g = g < ntot ? g : ntot - 1;
                // one address by selects, one load: no branch between the loads of the round
                const uintptr_t base = g < nb ? (uintptr_t)a.aq : (uintptr_t)a.as;
                const int gi = g < nb ? g : g - nb;
                v[r] = gload16((const void*)(base + (size_t)gi * 16));
            }
        }
#pragma unroll
        for (int r = 0; r < kDownFillRounds; ++r) {
            const int g = r * kDownFillThreads + tid;
            if (g < nb) {
                const int col = g / (K / 16);
                *(uint4*)&b_lds[col][(g % (K / 16)) * 16] = v[r];
            } else if (g < ntot) {
                const int gg = g - nb, col = gg / (K / 512);
                *(uint4*)&bs_lds[col][(gg % (K / 512)) * 16] = v[r];
            }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);            // this wave's LDS stores are done
        asm volatile("" ::: "memory");
        if (lane == 0) atomicAdd(&s_staged, 1);
    };
    // the staged h terms: wait until the four filler waves have counted themselves in (an atomic
    // read: a volatile one would also wait for this wave's weight loads)
    auto wait_h = [&]() {
        while (__hip_atomic_load(&s_staged, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < kDownFillThreads / 64)
            __builtin_amdgcn_s_sleep(1);
        asm volatile("" ::: "memory");
    };
    // 3. the weights of this wave's first two units (tile, K slice): u0 = wave, u1 = wave + 8
    const int units = a.max_tiles * nsl;
    const int tc = li / NT, t = li % NT;
    auto unit_ok = [&](int u) { return u < units && d_lds[u / nsl].ntok > 0; };
    // loads of units u0 and u0 + 8, issued without a condition (so that the h terms above can be
    // waited for alone): a unit without a tile re-reads the other one's weights, or unit 0's when
    // neither has one (every record, an empty one too, names a real expert)
    auto load_units = [&](int u0, uint4 (&A)[2][NSS][SS], uint32_t (&sa)[2][NSS], bool& ok0, bool& ok1,
                          int (&us)[2]) {
        const int u1 = u0 + 8;
        ok0 = unit_ok(u0);
        ok1 = unit_ok(u1);
        us[1] = ok1 ? u1 : (ok0 ? u0 : 0);
        us[0] = ok0 ? u0 : us[1];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const TileDesc& D = d_lds[us[j] / nsl];
            const int kss0 = (us[j] % nsl) * NSS;
            const uint8_t* aq = D.ex.down_q + (size_t)(r0 + li) * (K / 2) + lg * 16 * SS + (size_t)kss0 * 64 * SS;
            const uint8_t* as = D.ex.down_s + (size_t)(r0 + li) * (K / 32) + lg * SS + (size_t)kss0 * 4 * SS;
#pragma unroll
            for (int q = 0; q < NSS; ++q) {
#pragma unroll
                for (int h = 0; h < SS; ++h) A[j][q][h] = gload16(aq + (size_t)q * 64 * SS + 16 * h);
                sa[j][q] = gload4(as + (size_t)q * 4 * SS);
            }
        }
    };
    auto run_units = [&](const uint4 (&A)[2][NSS][SS], const uint32_t (&sa)[2][NSS], bool ok0, bool ok1,
                         const int (&us)[2]) {
        if (!ok0 && !ok1) return;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if (!(j == 0 ? ok0 : ok1)) continue;
            const TileDesc& D = d_lds[us[j] / nsl];
            const int ks = us[j] % nsl, kss0 = ks * NSS;
            const int ntok = D.ntok, i0 = D.i0;
            const int colp = i0 + (tc < ntok ? tc : ntok - 1);
            const uint8_t* bl = &b_lds[colp * NT + t][(size_t)kss0 * 128 * SS + lg * 32 * SS];
            const uint8_t* bsl = &bs_lds[colp * NT + t][kss0 * 4 * SS + lg * SS];
            v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < NSS; ++q) {
                const uint32_t sb = *(const uint32_t*)(bsl + q * 4 * SS);
                uint4 B[SS][2];
#pragma unroll
                for (int h = 0; h < SS; ++h) {
                    B[h][0] = *(const uint4*)(bl + q * 128 * SS + 32 * h);
                    B[h][1] = *(const uint4*)(bl + q * 128 * SS + 32 * h + 16);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int h = 0; h < SS; ++h)
                    acc = mfma_fp4_fp8(A[j][q][h], B[h][0], B[h][1], acc, (int)((sa[j][q] >> (8 * h)) & 0xffu),
                                       (int)((sb >> (8 * h)) & 0xffu));
            }
            mfma_results_here(acc);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = sum_adjacent<NT>(acc[r]);
            if (tc < ntok && t == 0) {
#pragma unroll
                for (int r = 0; r < 4; ++r) o_part[ks][i0 + tc][4 * lg + r] = acc[r];
            }
        }
    };
    uint4 A[2][NSS][SS];
    uint32_t sa[2][NSS];
    bool ok0, ok1;
    int us[2];
    if (filler) stage_h();
    __builtin_amdgcn_sched_barrier(0);
    load_units(wave, A, sa, ok0, ok1, us);
    __builtin_amdgcn_sched_barrier(0);
    // 4. the MFMAs of the first units, once the h terms are staged (each unit's MFMAs start when
    // its own weights are in)
    wait_h();
    run_units(A, sa, ok0, ok1, us);
    for (int u0 = wave + 16; u0 < units; u0 += 16) {      // more than sixteen units: further pairs
        if (!unit_ok(u0) && !unit_ok(u0 + 8)) continue;       // (none of them holds a tile)
        load_units(u0, A, sa, ok0, ok1, us);
        run_units(A, sa, ok0, ok1, us);
    }
    __syncthreads();
    // 5. y[t][r] = scaling * sum_j w[t,j] * (sum over K slices of o) (+ residual), rank order j
    // (every pick's position and weight read first, then every partial, then the sums: two LDS
    // round trips instead of two per pick)
    const int k = a.k;
    if (tid < c.T * 16) {
        const int tok = tid >> 4, r = tid & 15;
        int pos[MAXP];
        float wgt[MAXP], o[MAXP];
#pragma unroll
        for (int j = 0; j < MAXP; ++j) {
            const int p = tok * k + (j < k ? j : 0);
            pos[j] = s_posq[p];
            wgt[j] = s_wq[p];
        }
        static_assert(kMaxDecSlices == 2, "the K slices of a down unit are added below");
#pragma unroll
        for (int j = 0; j < MAXP; ++j) {
            const int pj = (PLAIN || pos[j] >= 0) ? pos[j] : 0;                 // a dropped pick: -1
            const float p0 = o_part[0][pj][r], p1 = o_part[1][pj][r];           // slice 1 read even
            o[j] = nsl > 1 ? p0 + p1 : p0;                                     // when unused
        }
        float accv = 0.f;
#pragma unroll
        for (int j = 0; j < MAXP; ++j)
            if (j < k && (PLAIN || pos[j] >= 0)) accv = fmaf(wgt[j], o[j], accv);
        float val = accv * c.scaling;
        if (!PLAIN && c.shared) {                        // the shared expert, unscaled
            const float s0 = o_part[0][c.P + tok][r], s1 = o_part[1][c.P + tok][r];
            val += nsl > 1 ? s0 + s1 : s0;
        }
        if (c.residual) val += resq;
        store_act((XT*)c.y, yoff, val);
    }
}

bool decode_gemm_ok(const moe_shape* s) {
    return (s->d_model / 2) % 512 == 0 && s->d_model <= kDecMaxD && s->d_ff % kDecKSlice == 0 &&
           s->d_ff / kDecKSlice <= kMaxDecSlices;
}

// compute units of the current device (cached per device)
static int device_cus() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

hipError_t launch_gateup_dec(const GemmArgs& a, int NT, int max_tiles, hipStream_t st) {
    trace("gemm_gate_up", 0, st);
    const int ss2 = 4;   // h terms in chunks of 512: the layout k_mx_down_dec reads
    // two workgroups per CU, each taking (tile, row block) pairs in turn
    const long long pairs = (long long)max_tiles * (a.f / 32);
    dim3 grid((unsigned)(pairs < 2LL * device_cus() ? pairs : 2LL * device_cus()));
    if (NT == 1) MOE_LAUNCH(k_mx_gateup_dec<1>, grid, dim3(512), 0, st, a, ss2, (int)grid.x);
    else if (NT == 2) MOE_LAUNCH(k_mx_gateup_dec<2>, grid, dim3(512), 0, st, a, ss2, (int)grid.x);
    else MOE_LAUNCH(k_mx_gateup_dec<4>, grid, dim3(512), 0, st, a, ss2, (int)grid.x);
    trace("gemm_gate_up", 1, st);
    return hipGetLastError();
}

hipError_t launch_down_dec(const moe_shape* s, const GemmArgs& a, const CombineArgs& c, int NT, hipStream_t st) {
    trace("down_combine", 0, st);
    dim3 grid(a.d / 16);
    const bool bf = s->act_dtype == MOE_DT_BF16;
    const bool plain = s->renorm_skip == 0.0f && s->n_shared == 0;
    const bool lds = a.Pall * NT <= kDownLdsCols && a.f <= kDownMaxF && a.max_tiles <= kDownMaxTiles;
#define MOE_DD(K, XT, N, PL) MOE_LAUNCH((K<XT, N, PL>), grid, dim3(512), 0, st, a, c)
#define MOE_DD_NT(K, XT, PL)                                                                  \
    do {                                                                                      \
        if (NT == 1) MOE_DD(K, XT, 1, PL);                                                    \
        else if (NT == 2) MOE_DD(K, XT, 2, PL);                                               \
        else MOE_DD(K, XT, 4, PL);                                                            \
    } while (0)
#define MOE_DD_PL(K, XT)                                                                      \
    do {                                                                                      \
        if (plain) MOE_DD_NT(K, XT, true);                                                    \
        else MOE_DD_NT(K, XT, false);                                                         \
    } while (0)
    if (lds) {
        if (bf) MOE_DD_PL(k_mx_down_dec_lds, uint16_t);
        else MOE_DD_PL(k_mx_down_dec_lds, float);
    } else {
        if (a.max_tiles > kDownDecMaxTiles) return hipErrorInvalidValue;     // (its records are kept in LDS)
#undef MOE_DD
#define MOE_DD(K, XT, N, PL) MOE_LAUNCH((K<XT, N, PL>), grid, dim3(64 * kDownDecWaves), 0, st, a, c)
        if (bf) MOE_DD_PL(k_mx_down_dec, uint16_t);
        else MOE_DD_PL(k_mx_down_dec, float);
    }
#undef MOE_DD_PL
#undef MOE_DD_NT
#undef MOE_DD
    trace("down_combine", 1, st);
    return hipGetLastError();
}

int gemm_variant(const moe_shape* s, int T) {
    const long long P = (long long)T * s->top_k, E = s->n_experts;
    const int NT = act_terms(s);
    // few-pick tiles up to 5/8 of a tile's picks per expert on average (measured crossover at d_model
    // 4096, d_ff 2048, 288 experts: between 4.4 and 5.3 picks per expert), then the 64-column tile
    // up to its picks per expert, then the 128-column tile
    if (8 * P <= 5LL * gemm_tile_tokens(0, NT) * E) return 0;
    return P <= (long long)(64 / NT) * E ? 2 : 1;
}

// picks per tile: the MFMA columns over the terms per value; a few-token tile also at most the
// tokens its tile record holds
int gemm_tile_tokens(int variant, int NT) {
    if (variant == 0) return 16 / NT < kDescTokens ? 16 / NT : kDescTokens;
    return (variant == 2 ? 64 : 128) / NT;
}

// activation layout super-step for the variant: the LDS-tiled many-picks GEMM reads chunks of 128
int act_super_step(int K, int variant) { return variant >= 1 ? 1 : super_step(K, ksplit_for(K, variant)); }

int super_step(int K, int ksplit) {
    const int span = K / ksplit;
    if (span % 512 == 0) return 4;
    if (span % 256 == 0) return 2;
    return 1;
}

int ksplit_for(int K, int variant) { return (variant == 0 && (K / 4) % 128 == 0) ? 4 : 1; }

template <bool GATEUP, int NT, int NTN, int KS>
static hipError_t launch_one(const GemmArgs& a, int SS, int ss2, int nrg, hipStream_t st) {
    // eight XCD lanes of (row groups / 8, rounded up) x max_tiles workgroups
    const dim3 grid((unsigned)(8LL * a.max_tiles * ((nrg + 7) / 8)));
    if (SS == 4) MOE_LAUNCH((k_mx_gemm<NT, NTN, KS, 4, GATEUP>), grid, dim3(256), 0, st, a, ss2, nrg);
    else if (SS == 2) MOE_LAUNCH((k_mx_gemm<NT, NTN, KS, 2, GATEUP>), grid, dim3(256), 0, st, a, ss2, nrg);
    else MOE_LAUNCH((k_mx_gemm<NT, NTN, KS, 1, GATEUP>), grid, dim3(256), 0, st, a, ss2, nrg);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// many picks per expert ("prefill"): an LDS-tiled grouped GEMM fed by direct global->LDS loads.
// A workgroup (4 waves, 2 x 2) owns one tile of up to 128 / NT picks (128 MFMA columns) and one
// block of 256 weight rows: for gate/up the same 128 row indices of gate and of up (so SwiGLU
// needs no exchange), for down 256 rows.  K advances 128 at a time through a ring of four LDS
// stages that global_load_lds fills (no register round trip) four steps before they are
// consumed; the fragments of step s + 1 are read from LDS into a second register set while the
// MFMAs of step s run.  Wave (wm, wn) computes 128 weight rows x 64 columns (32 MFMAs per step).
//
// The vector L1 serves a load one lane quad at a time, so every direct load has consecutive
// lanes read consecutive bytes: 4 lanes per 64-byte weight-row chunk, 8 lanes per 128-byte
// activation chunk.  In LDS a chunk keeps its row, with its 16-byte units XOR-swizzled so that
// the MFMA fragment reads (16 rows or columns at one unit each) meet no bank conflict.  The
// scale words (one per row and step) are loaded four steps at a time, consecutive lanes taking
// consecutive words of a row, into a ring of two slots.  Workgroups are spread over the 8 XCDs
// by tile range, with the row block fastest, so one XCD's L2 serves a tile's activations to all
// its row blocks and the tiles of one expert run together.
//
// Stage layout (bytes): weight row r (0..255) at 64 r, its 16-byte part p in slot p ^ swz_a(r
// % 16); activation column c (0..127) at 16384 + 128 c, unit u in slot u ^ swz_b(c % 16).
// Scale slot layout: row r's words of steps 4m..4m+3 at 16 r + 4 (step % 4); column c's at
// 4096 + 16 c.
// ---------------------------------------------------------------------------------------------
constexpr int kPfRows = 256, kPfCols = 128;
constexpr int kPfA = 0, kPfB = 16384, kPfStage = 32768;
constexpr int kScA = 0, kScB = 4096, kScSlot = 6144;
// NCF = MFMA column fragments per wave: 4 (128 columns per workgroup) or 2 (64 columns, the
// narrow tile for 8-32 picks per expert: half the MFMAs and B-side LDS work per step, the same
// weight bytes)
template <int NCF> constexpr int pf_loads() { return 4 + NCF; }       // direct loads per wave and stage
template <int NCF> constexpr int sc_loads() { return 4 + NCF / 2; }   // per wave and group of four steps

__device__ __forceinline__ int swz_a(int r) { return ((r >> 2) ^ (r >> 1)) & 3; }
__device__ __forceinline__ int swz_b(int c) { return ((c >> 1) ^ ((c & 1) << 2)) & 7; }


struct PfFrags {
    uint4 a[8];
    uint4 b[4][2];
    int sa[8];
    int sb[4];
};

// fragments of one step: stg = its stage, sc = its scale slot, w = the step's index in its group
template <bool GATEUP, int NCF>
__device__ __forceinline__ void pf_read(const uint8_t* stg, const uint8_t* sc, int w, PfFrags& fr, int wm,
                                        int wn, int lane) {
    const int lg = lane >> 4, li = lane & 15;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int fa = GATEUP ? ((j >> 2) * 8 + wm * 4 + (j & 3)) : (wm * 8 + j);
        fr.a[j] = *(const uint4*)(stg + kPfA + (fa * 16 + li) * 64 + ((lg ^ swz_a(li)) * 16));
        fr.sa[j] = sc[kScA + (fa * 16 + li) * 16 + w * 4 + lg];      // scale byte of K block lg
    }
#pragma unroll
    for (int n = 0; n < NCF; ++n) {
        const int col = (wn * NCF + n) * 16 + li;
        const uint8_t* cp = stg + kPfB + col * 128;
        fr.b[n][0] = *(const uint4*)(cp + (((2 * lg) ^ swz_b(li)) * 16));
        fr.b[n][1] = *(const uint4*)(cp + (((2 * lg + 1) ^ swz_b(li)) * 16));
        fr.sb[n] = sc[kScB + col * 16 + w * 4 + lg];
    }
}

template <int NCF>
__device__ __forceinline__ void pf_mfma(const PfFrags& fr, v4f (&acc)[8][NCF]) {
#pragma unroll
    for (int n = 0; n < NCF; ++n)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc[j][n] = mfma_fp4_fp8(fr.a[j], fr.b[n][0], fr.b[n][1], acc[j][n], fr.sa[j], fr.sb[n]);
}


// FULL: 0, or the step count K / 128 that this instance runs as straight-line code; NCF: column
// fragments per wave (above)
template <int NT, bool GATEUP, int FULL, int NCF>
__global__ __launch_bounds__(256, 1) void k_mx_pf(GemmArgs a, int ss2, int tiles_per_xcd_cap) {
    __shared__ __align__(16) uint8_t stg0[kPfStage];
    __shared__ __align__(16) uint8_t stg1[kPfStage];
    __shared__ __align__(16) uint8_t stg2[kPfStage];
    __shared__ __align__(16) uint8_t stg3[kPfStage];
    __shared__ __align__(16) uint8_t scr0[kScSlot];
    __shared__ __align__(16) uint8_t scr1[kScSlot];
    constexpr int TT = 32 * NCF / NT;                   // picks per tile
    constexpr int PL = pf_loads<NCF>(), SL = sc_loads<NCF>();
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int li = lane & 15, lg = lane >> 4;
    const int wm = wave & 1, wn = wave >> 1;
    const int K = GATEUP ? a.d : a.f;
    const int rows = GATEUP ? a.f : a.d;                 // output rows (h rows / d)
    const int MT = GATEUP ? a.f / 128 : (a.d + kPfRows - 1) / kPfRows;
    // workgroup -> (tile, row block): XCD x = id % 8 takes tiles [x * TPX, (x + 1) * TPX)
    const int nt = *a.ntiles;
    const int g = blockIdx.x, xcd = g & 7, sidx = g >> 3;
    const int mblk = sidx % MT, tq = sidx / MT;
    const int TPX = (nt + 7) >> 3;
    if (tq >= TPX || tq >= tiles_per_xcd_cap) return;
    const int tile = xcd * TPX + tq;
    if (tile >= nt) return;
    const int e = a.tiles[2 * tile], i0 = a.tiles[2 * tile + 1];
    const int ntok = min(TT, range_end(a, e) - i0);
    const moe_expert ex = a.table[e];

    // tile row r (0..255) -> weight row; down rows past d re-read row d - 1 (not stored)
    auto a_row_ptr = [&](int r, bool scale) -> const uint8_t* {
        int mr;
        const uint8_t* base;
        if (GATEUP) {
            mr = mblk * 128 + (r & 127);
            base = (r < 128) ? (scale ? ex.gate_s : ex.gate_q) : (scale ? ex.up_s : ex.up_q);
        } else {
            mr = min(mblk * kPfRows + r, a.d - 1);
            base = scale ? ex.down_s : ex.down_q;
        }
        return base + (size_t)mr * (scale ? K / 32 : K / 2);
    };
    // tile column c (0..32 NCF - 1) = (pick c / NT, term c % NT); columns past the tile re-read column 0
    auto b_col_ptr = [&](int c, bool scale) -> const uint8_t* {
        const int tc = c / NT, t = c % NT;
        const int tcc = tc < ntok ? tc : 0;
        const size_t arow = GATEUP ? (size_t)pos_token(a, i0 + tcc) : (size_t)(i0 + tcc);
        return scale ? a.as + (arow * NT + t) * (size_t)(K / 32) : a.aq + (arow * NT + t) * (size_t)K;
    };
    // this wave's direct loads: weight rows 64 w .. 64 w + 63 (4 instructions of 16 rows, a
    // lane quad per row), activation columns 8 NCF w .. 8 NCF w + 8 NCF - 1 (NCF instructions of
    // 8 columns, 8 lanes per column); scale words of the same rows (4 instructions) and columns
    // (NCF / 2)
    const uint8_t* srcA[4];
    const uint8_t* srcB[NCF];
    const uint8_t* srcAs[4];
    const uint8_t* srcBs[NCF / 2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = (wave * 4 + j) * 16 + (lane >> 2);
        srcA[j] = a_row_ptr(r, false) + (((lane & 3) ^ swz_a(r & 15)) * 16);
        if (j < NCF) {
            const int c = (wave * NCF + j) * 8 + (lane >> 3);
            srcB[j] = b_col_ptr(c, false) + (((lane & 7) ^ swz_b(c & 15)) * 16);
        }
        srcAs[j] = a_row_ptr(r, true);
    }
#pragma unroll
    for (int j = 0; j < NCF / 2; ++j) srcBs[j] = b_col_ptr((wave * (NCF / 2) + j) * 16 + (lane >> 2), true);
    const int nsteps = K / 128, last = nsteps - 1;

    auto issue = [&](int st, uint8_t* stg) {
        const size_t oa = (size_t)st * 64, ob = (size_t)st * 128;
#pragma unroll
        for (int j = 0; j < 4; ++j) dma16(srcA[j] + oa, stg + kPfA + (wave * 4 + j) * 1024);
#pragma unroll
        for (int j = 0; j < NCF; ++j) dma16(srcB[j] + ob, stg + kPfB + (wave * NCF + j) * 1024);
    };
    // scale words of steps 4m .. 4m + 3 (past the last step: the last step's) into slot sc
    auto issue_scales = [&](int m, uint8_t* sc) {
        const size_t ow = (size_t)min(4 * m + (lane & 3), last) * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) dma4(srcAs[j] + ow, sc + kScA + (wave * 4 + j) * 256);
#pragma unroll
        for (int j = 0; j < NCF / 2; ++j) dma4(srcBs[j] + ow, sc + kScB + (wave * (NCF / 2) + j) * 256);
    };

    v4f acc[8][NCF];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int n = 0; n < NCF; ++n) acc[j][n] = v4f{0.f, 0.f, 0.f, 0.f};
    PfFrags fr0, fr1;
    // Every step issues one stage, clamped to the last: past the end the ring is refilled with
    // copies of the last stage that no step reads.  The scale group of steps 4m.. rides with
    // stage 4m.  Before step s reads stage s + 1, the loads of stages s + 2 and s + 3 (and of
    // the one scale group among them, if any) may still be in flight.
    issue(0, stg0);
    issue_scales(0, scr0);
    issue(min(1, last), stg1);
    issue(min(2, last), stg2);
    issue(min(3, last), stg3);
    wait_vm<3 * PL>();                                       // stage 0 and its scales complete
    ring_barrier();
    pf_read<GATEUP, NCF>(stg0, scr0, 0, fr0, wm, wn, lane);

    // buffers by compile-time index (distinct arrays, so the compiler sees that a direct load
    // into one never feeds a read of another)
    auto stage_buf = [&](auto i) -> uint8_t* {
        constexpr int I = decltype(i)::value;
        if constexpr (I == 0) return stg0;
        else if constexpr (I == 1) return stg1;
        else if constexpr (I == 2) return stg2;
        else return stg3;
    };
    auto scale_buf = [&](auto i) -> uint8_t* {
        if constexpr (decltype(i)::value == 0) return scr0;
        else return scr1;
    };
    // step s (s % 8 == Q): stage s is in registers; wait for stage s + 1, refill stage s's
    // buffer with step s + 4 (and, opening a group of four, the scale slot of the next group),
    // read stage s + 1 into the other register set (past the end: unused values), run the
    // MFMAs of step s
    auto step = [&](int s, auto pos) {
        constexpr int Q = decltype(pos)::value;
        PfFrags& cur = (Q & 1) ? fr1 : fr0;
        PfFrags& nxt = (Q & 1) ? fr0 : fr1;
        wait_vm<2 * PL + (((Q & 3) == 1 || (Q & 3) == 2) ? SL : 0)>();
        ring_barrier();                                      // also: every wave has stage s in registers
        __builtin_amdgcn_sched_barrier(0);
        issue(min(s + 4, last), stage_buf(StepPos<Q & 3>{}));
        if constexpr ((Q & 3) == 0) issue_scales((s >> 2) + 1, scale_buf(StepPos<((Q >> 2) + 1) & 1>{}));
        pf_read<GATEUP, NCF>(stage_buf(StepPos<(Q + 1) & 3>{}), scale_buf(StepPos<((Q + 1) >> 2) & 1>{}),
                             (Q + 1) & 3, nxt, wm, wn, lane);
        pf_mfma<NCF>(cur, acc);
        // schedule: the step's direct loads (NV) and its 28 LDS reads of step s + 1 go between the
        // 32 MFMAs of step s, one MFMA, one direct load and one LDS read at a time, so that their
        // issue hides under the matrix core's work (with one wave per SIMD nothing else would);
        // the MFMAs do not wait for those reads, and no MFMA of step s + 1 is hoisted above the
        // next barrier
        constexpr int NV = PL + ((Q & 3) == 0 ? SL : 0);
        if constexpr (NCF == 4) {
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
#pragma unroll
            for (int i = 0; i < 28 - NV; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        } else {
            // 16 MFMAs, 22 LDS reads: the first 14 MFMAs each take one or two reads (and the
            // direct loads, one each, from the first), the last two none
            constexpr int NMF = 8 * NCF, NDS = 16 + 3 * NCF, SLOTS = NMF - 2, D2 = NDS - SLOTS;
            static_assert(D2 >= 0 && D2 <= SLOTS && NV <= SLOTS, "one or two LDS reads per MFMA slot");
#pragma unroll
            for (int i = 0; i < D2; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (i < NV) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
#pragma unroll
            for (int i = D2; i < SLOTS; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (i < NV) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, NMF - SLOTS, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    // The K extents of the workload (d_model 4096 for gate/up, d_ff 2048 for down) run as straight-
    // line code: with a loop, the allocator moves accumulators across the back edge, and each such
    // move waits for the MFMA that writes its source (several hundred cycles).
    if constexpr (FULL > 0) {
        for_steps<0>([&](auto i) { step(decltype(i)::value, StepPos<decltype(i)::value % 8>{}); },
                     std::make_integer_sequence<int, FULL>{});
        wait_vm<0>();
    } else {
    int s = 0;
    for (; s + 8 <= nsteps; s += 8) {
        step(s, StepPos<0>{});
        step(s + 1, StepPos<1>{});
        step(s + 2, StepPos<2>{});
        step(s + 3, StepPos<3>{});
        step(s + 4, StepPos<4>{});
        step(s + 5, StepPos<5>{});
        step(s + 6, StepPos<6>{});
        step(s + 7, StepPos<7>{});
    }
    if (s < nsteps) step(s, StepPos<0>{});
    if (s + 1 < nsteps) step(s + 1, StepPos<1>{});
    if (s + 2 < nsteps) step(s + 2, StepPos<2>{});
    if (s + 3 < nsteps) step(s + 3, StepPos<3>{});
    if (s + 4 < nsteps) step(s + 4, StepPos<4>{});
    if (s + 5 < nsteps) step(s + 5, StepPos<5>{});
    if (s + 6 < nsteps) step(s + 6, StepPos<6>{});
    wait_vm<0>();                                            // no direct load outlives the workgroup
    }

    // columns: n * 16 + li of this wave's 16 NCF = (pick tc, term t)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int n = 0; n < NCF; ++n) mfma_results_here(acc[j][n]);
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int n = 0; n < NCF; ++n)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[j][n][r] = sum_adjacent<NT>(acc[j][n][r]);
    const int t = li % NT;
    if constexpr (GATEUP) {
        // h = silu(g) u for the wave's 64 row indices (two natural blocks of h), each split into
        // NT terms with one exponent per term and block
#pragma unroll
        for (int n = 0; n < NCF; ++n)
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                float v[8];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    v[r] = silu(acc[2 * b][n][r]) * acc[4 + 2 * b][n][r];
                    v[4 + r] = silu(acc[2 * b + 1][n][r]) * acc[5 + 2 * b][n][r];
                }
                uint32_t codes[NT][2];
                int S[NT];
                split_terms<NT>(v, codes, S, [](float mm) { return max_xor32(max_xor16(mm)); });
                const int rg = (mblk * 128 + wm * 64) / 32 + b;
                const int tc = (wn * 16 * NCF + n * 16 + li) / NT;
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
    } else {
#pragma unroll
        for (int n = 0; n < NCF; ++n) {
            const int tc = (wn * 16 * NCF + n * 16 + li) / NT;
            if (tc < ntok && t == 0) {
                float* dst = a.o + ((size_t)i0 + tc) * a.d;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int row = mblk * kPfRows + wm * 128 + 16 * j + 4 * lg;
                    if (row < rows)
                        *(float4*)(dst + row) = make_float4(acc[j][n][0], acc[j][n][1], acc[j][n][2], acc[j][n][3]);
                }
            }
        }
    }
}

template <bool GATEUP, int NCF>
static hipError_t launch_pf(const GemmArgs& a, int NT, int max_tiles, hipStream_t st) {
    const int MT = GATEUP ? a.f / 128 : (a.d + kPfRows - 1) / kPfRows;
    const int cap = (max_tiles + 7) / 8;
    dim3 grid((unsigned)(8 * cap * MT));
    // the workload's K (d_model 4096 for gate/up, d_ff 2048 for down) takes the straight-line instance
    constexpr int kFull = GATEUP ? 32 : 16;
    const bool full = (GATEUP ? a.d : a.f) == 128 * kFull;
    if (NT == 1) {
        // (single-term down runs the looped instance: the straight-line one spills at K = 2048)
        if (full && GATEUP) MOE_LAUNCH((k_mx_pf<1, true, 32, NCF>), grid, dim3(256), 0, st, a, 1, cap);
        else MOE_LAUNCH((k_mx_pf<1, GATEUP, 0, NCF>), grid, dim3(256), 0, st, a, 1, cap);
    } else if (NT == 2) {
        if (full) MOE_LAUNCH((k_mx_pf<2, GATEUP, kFull, NCF>), grid, dim3(256), 0, st, a, 1, cap);
        else MOE_LAUNCH((k_mx_pf<2, GATEUP, 0, NCF>), grid, dim3(256), 0, st, a, 1, cap);
    } else {
        if (full) MOE_LAUNCH((k_mx_pf<4, GATEUP, kFull, NCF>), grid, dim3(256), 0, st, a, 1, cap);
        else MOE_LAUNCH((k_mx_pf<4, GATEUP, 0, NCF>), grid, dim3(256), 0, st, a, 1, cap);
    }
    return hipGetLastError();
}

template <bool GATEUP>
static hipError_t launch_gemm(const GemmArgs& a, int NT, int variant, int max_tiles, hipStream_t st) {
    const int K = GATEUP ? a.d : a.f;
    const int rows = GATEUP ? a.f : a.d;
    const int ks = ksplit_for(K, variant);
    const int SS = super_step(K, ks);
    const int ss2 = super_step(a.f, ksplit_for(a.f, variant));
    // row groups of 32 rows (64 for down with K split four ways: k_mx_gemm's RB)
    const int nrg = ks == 4 ? rows / (GATEUP ? 32 : 64) : (rows / 32) / 4;
    if (variant == 0) {
        if (a.max_tiles != max_tiles) return hipErrorInvalidValue;     // (the kernel maps by a.max_tiles)
        if (ks == 4) return NT == 1 ? launch_one<GATEUP, 1, 1, 4>(a, SS, ss2, nrg, st)
                          : NT == 2 ? launch_one<GATEUP, 2, 1, 4>(a, SS, ss2, nrg, st)
                                    : launch_one<GATEUP, 4, 1, 4>(a, SS, ss2, nrg, st);
        return NT == 1 ? launch_one<GATEUP, 1, 1, 1>(a, SS, ss2, nrg, st)
             : NT == 2 ? launch_one<GATEUP, 2, 1, 1>(a, SS, ss2, nrg, st)
                       : launch_one<GATEUP, 4, 1, 1>(a, SS, ss2, nrg, st);
    }
    return variant == 2 ? launch_pf<GATEUP, 2>(a, NT, max_tiles, st) : launch_pf<GATEUP, 4>(a, NT, max_tiles, st);
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
#define MOE_DC(XT, N, S) MOE_LAUNCH((k_mx_down_combine<XT, N, S>), grid, dim3(512), 0, st, a, c)
#define MOE_DC_SS(XT, N) \
    do { if (SS == 4) MOE_DC(XT, N, 4); else if (SS == 2) MOE_DC(XT, N, 2); else MOE_DC(XT, N, 1); } while (0)
    if (bf) {
        if (NT == 1) MOE_DC_SS(uint16_t, 1);
        else if (NT == 2) MOE_DC_SS(uint16_t, 2);
        else MOE_DC_SS(uint16_t, 4);
    } else {
        if (NT == 1) MOE_DC_SS(float, 1);
        else if (NT == 2) MOE_DC_SS(float, 2);
        else MOE_DC_SS(float, 4);
    }
#undef MOE_DC_SS
#undef MOE_DC
    trace("down_combine", 1, st);
    return hipGetLastError();
}

}  // namespace moe
