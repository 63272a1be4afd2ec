// Grouped expert GEMMs for NVFP4 weights: E2M1 codes with one E4M3 scale per 16 elements along
// each row and one fp32 scale per weight tensor ("A hot expert cache made a 181 GiB model
// faster ...", section "The wall: one PCIe transfer per token": the NVFP4 build of the model).
//
// The scaled FP4 matrix cores take only power-of-two scales per 32 elements, so an NVFP4 weight
// is dequantised in registers instead: V_CVT_SCALEF32_PK_F32_FP4 decodes two codes, an fp32
// multiply applies the E4M3 block scale, and the product is rounded to bf16.  That product is
// exact in bf16 (at most 2 + 4 significant bits), so the bf16 matrix cores
// (V_MFMA_F32_16X16X32_BF16) see the weights exactly;
// the tensor scale multiplies the fp32 accumulator.  Activations are the bf16 operand, NT terms
// of each value, each term one MFMA column: with bf16 activations x as it is and the SwiGLU output
// h rounded to bf16 (NT = 1); with fp32 activations x and h as two bf16 terms (hi = bf16(v),
// lo = bf16(v - hi)), which keep fp32-level accuracy (NT = 2).
//
// K order of one MFMA: lane l supplies 8 consecutive K of row (A) or column (B) l % 16; any
// assignment of K to lane groups works when both operands share it (measured on gfx950).  Here a
// super-step covers 128 K of a row (64 code bytes): lane group g takes elements [32g, 32g + 32)
// (16 code bytes, two NVFP4 blocks) and MFMA h of the super-step its elements [8h, 8h + 8).
//
// Work decomposition: a tile is up to 8 consecutive sorted picks of one expert; a workgroup of
// four waves owns one tile and one 32-row block of the output and splits K four ways, the partial
// sums reduced through LDS in a fixed order.
#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float v4f_nv __attribute__((ext_vector_type(4)));


// 8 codes (one dword, element 2i in the low nibble of byte i) x block scale -> 8 bf16.  The
// conversion unit's scale operand acts as a power of two only, so codes are converted at scale 1
// and multiplied by the E4M3 block scale in fp32 (exact: at most 2 + 4 significant bits), then
// rounded to bf16 (exact as well).
__device__ __forceinline__ bf16x8_t nv_dequant8(uint32_t codes, float scale) {
    bf16x8_t r;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const v2f_t v = b == 0 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0)
                      : b == 1 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1)
                      : b == 2 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2)
                               : __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3);
        r[2 * b] = (__bf16)(v[0] * scale);
        r[2 * b + 1] = (__bf16)(v[1] * scale);
    }
    return r;
}

// two E4M3 scale bytes (low byte first) -> two floats (exact)
__device__ __forceinline__ v2f_t e4m3x2_to_f32(uint32_t two) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(two, 1.0f, false);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) {
    bf16x8_t r;
    __builtin_memcpy(&r, &v, 16);
    return r;
}

__device__ __forceinline__ uint16_t bf16_rne(float f) { return f32_to_bf16_bits(f); }

// h value v of row `row` as NT bf16 terms of a pick's [NT][f] block: bf16(v), and with NT = 2 also
// bf16(v - bf16(v))
template <int NT>
__device__ __forceinline__ void put_h_terms(uint16_t* hb, int f, int row, float v) {
    const uint16_t hi = bf16_rne(v);
    hb[row] = hi;
    if constexpr (NT == 2) hb[f + row] = bf16_rne(v - bf16_bits_to_f32(hi));
}

// bf16 terms of fp32 activations: hi = bf16(v), lo = bf16(v - hi); layout [rows][2][K]
__global__ __launch_bounds__(256) void k_bf16_terms(const float* __restrict__ x, size_t n, int K,
                                                   uint16_t* __restrict__ terms) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const float v = x[i];
    const uint16_t hi = bf16_rne(v);
    const uint16_t lo = bf16_rne(v - bf16_bits_to_f32(hi));
    const size_t r = i / K, c = i % K;
    terms[(r * 2) * K + c] = hi;
    terms[(r * 2 + 1) * K + c] = lo;
}

hipError_t launch_bf16_terms(const float* x, int rows, int K, uint16_t* terms, hipStream_t st) {
    trace("act_split", 0, st);
    const size_t n = (size_t)rows * K;
    MOE_LAUNCH(k_bf16_terms, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, x, n, K, terms);
    trace("act_split", 1, st);
    return hipGetLastError();
}

// NT: bf16 terms per activation (1: bf16 x read in place; 2: hi/lo terms); TTP: picks per tile
// (MFMA columns = TTP * NT, in NCF 16-column fragments).  GATEUP: the gate and up rows of one
// 32-row block, SwiGLU, and h as NT bf16 terms; else the down rows, o in fp32.
template <int NT, bool GATEUP, int TTP>
__global__ __launch_bounds__(256) void k_nv_gemm(GemmArgs a, int nrg) {
    constexpr int NA = GATEUP ? 4 : 2;      // 16-row fragments: gate lo/hi, up lo/hi (or down lo/hi)
    constexpr int NCF = (TTP * NT + 15) / 16;
    // workgroup -> (tile, 32-row block rg of nrg): XCD x = id % 8 takes blocks x, x + 8, .. and,
    // within each, the tiles in order, so that the tiles of one expert read the same weight rows on
    // one XCD at about the same time, from its L2
    const int g = blockIdx.x, j = g >> 3;
    const int rg = (g & 7) + 8 * (j / a.max_tiles), tile = j % a.max_tiles;
    int t0 = 0, t1 = *a.ntiles;
    if (a.tile_range) {
        t0 = a.tile_range[0];
        t1 = a.tile_range[1];
    }
    if (rg >= nrg || tile < t0 || tile >= t1) return;
    const int e = a.tiles[2 * tile], i0 = a.tiles[2 * tile + 1];
    const int ntok = min(TTP, range_end(a, e) - i0);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int li = lane & 15, lg = lane >> 4;
    const int K = GATEUP ? a.d : a.f;
    const moe_expert ex = a.table[e];
    const int T0 = 32 * rg;
    const int NS = K / 128;                  // super-steps of the row, shared out over the 4 waves
    const int s0 = (wave * NS) / 4, nss = ((wave + 1) * NS) / 4 - s0;

    // weights: fragment f = rows T0 + 16 (f & 1) + li of gate (f < 2) or up (f >= 2)
    const uint8_t* aq[NA];
    const uint8_t* as[NA];
#pragma unroll
    for (int f = 0; f < NA; ++f) {
        const int row = T0 + 16 * (f & 1) + li;
        const uint8_t* mq = GATEUP ? (f < 2 ? ex.gate_q : ex.up_q) : ex.down_q;
        const uint8_t* ms = GATEUP ? (f < 2 ? ex.gate_s : ex.up_s) : ex.down_s;
        aq[f] = mq + (size_t)row * (K / 2) + (size_t)s0 * 64 + lg * 16;
        as[f] = ms + (size_t)row * (K / 16) + (size_t)s0 * 8 + lg * 2;
    }
    // activations: column n * 16 + li = (pick tc, term t); columns past the tile read the tile's
    // first pick (their results are not used)
    const uint16_t* bp[NCF];
#pragma unroll
    for (int n = 0; n < NCF; ++n) {
        const int c = n * 16 + li, tc = c / NT, t = c % NT;
        const int tcc = tc < ntok ? tc : 0;
        const size_t arow = GATEUP ? (size_t)pos_token(a, i0 + tcc) : (size_t)(i0 + tcc);
        bp[n] = (const uint16_t*)a.aq + (arow * NT + t) * (size_t)K + (size_t)s0 * 128 + lg * 32;
    }

    v4f_nv acc[NA][NCF];
#pragma unroll
    for (int f = 0; f < NA; ++f)
#pragma unroll
        for (int n = 0; n < NCF; ++n) acc[f][n] = v4f_nv{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < nss; ++s) {
        uint4 A[NA];
        uint32_t sc[NA];
#pragma unroll
        for (int f = 0; f < NA; ++f) {
            A[f] = gload16(aq[f] + (size_t)s * 64);
            sc[f] = *(__attribute__((address_space(1))) const uint16_t*)(as[f] + (size_t)s * 8);
        }
        uint4 B[NCF][4];
#pragma unroll
        for (int n = 0; n < NCF; ++n)
#pragma unroll
            for (int h = 0; h < 4; ++h) B[n][h] = gload16(bp[n] + (size_t)s * 128 + 8 * h);
#pragma unroll
        for (int f = 0; f < NA; ++f) {
            const v2f_t bs = e4m3x2_to_f32(sc[f]);
            const uint32_t w[4] = {A[f].x, A[f].y, A[f].z, A[f].w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const bf16x8_t af = nv_dequant8(w[h], h < 2 ? bs[0] : bs[1]);
#pragma unroll
                for (int n = 0; n < NCF; ++n)
                    acc[f][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, as_bf16x8(B[n][h]), acc[f][n], 0, 0, 0);
            }
        }
    }
#pragma unroll
    for (int f = 0; f < NA; ++f)
#pragma unroll
        for (int n = 0; n < NCF; ++n) mfma_results_here(acc[f][n]);
    // K quarters summed through LDS in wave order
    __shared__ float red[3][NA * NCF * 4][64];
    if (wave > 0) {
#pragma unroll
        for (int f = 0; f < NA; ++f)
#pragma unroll
            for (int n = 0; n < NCF; ++n)
#pragma unroll
                for (int r = 0; r < 4; ++r) red[wave - 1][(f * NCF + n) * 4 + r][lane] = acc[f][n][r];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 0; w < 3; ++w)
#pragma unroll
        for (int f = 0; f < NA; ++f)
#pragma unroll
            for (int n = 0; n < NCF; ++n)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[f][n][r] += red[w][(f * NCF + n) * 4 + r][lane];
    if constexpr (NT == 2) {
#pragma unroll
        for (int f = 0; f < NA; ++f)
#pragma unroll
            for (int n = 0; n < NCF; ++n)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[f][n][r] = sum_adjacent<2>(acc[f][n][r]);
    }
#pragma unroll
    for (int n = 0; n < NCF; ++n) {
        const int c = n * 16 + li, tc = c / NT, t = c % NT;
        if (tc >= ntok || t != 0) continue;
        const size_t pos = (size_t)i0 + tc;
        if constexpr (GATEUP) {
            // h = silu(g) u for rows T0 + 4 lg + r (half 0) and T0 + 16 + 4 lg + r (half 1), as NT
            // bf16 terms [P][NT][f]
            uint16_t* hb = (uint16_t*)a.hq + pos * NT * (size_t)a.f;
#pragma unroll
            for (int half = 0; half < 2; ++half)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float g = acc[half][n][r] * ex.gate_ts, u = acc[2 + half][n][r] * ex.up_ts;
                    const int row = T0 + 16 * half + 4 * lg + r;
                    put_h_terms<NT>(hb, a.f, row, g / (1.0f + __expf(-g)) * u);
                }
        } else {
            float* dst = a.o + pos * (size_t)a.d + T0 + 4 * lg;
            *(float4*)dst = make_float4(acc[0][n][0] * ex.down_ts, acc[0][n][1] * ex.down_ts,
                                        acc[0][n][2] * ex.down_ts, acc[0][n][3] * ex.down_ts);
            *(float4*)(dst + 16) = make_float4(acc[1][n][0] * ex.down_ts, acc[1][n][1] * ex.down_ts,
                                               acc[1][n][2] * ex.down_ts, acc[1][n][3] * ex.down_ts);
        }
    }
}

// Many picks per expert: an LDS-tiled version.  A workgroup (4 waves) owns one tile of up to
// kNvTilePicksMany picks (64 * NT columns) and 128 weight rows (gate/up: the same 64 row indices
// of gate and up).  K advances 128 at a time through double-buffered LDS: the global loads of step
// s + 1 are in flight while step s computes.  Each wave decodes its two 16-row weight fragments
// once per step (32 bf16 per lane each) and runs them against every column fragment of the tile,
// so that each decode feeds twice the MFMAs of a 2 x 2 split of the waves.  Workgroups are spread
// over the 8 XCDs by tile range, row block fastest.
constexpr int kNvPfRows = 128, kNvPfBStride = 272;   // bf16 column: 256 bytes per step + pad

template <int NT, bool GATEUP>
__global__ __launch_bounds__(256) void k_nv_pf(GemmArgs a, int tiles_per_xcd_cap) {
    constexpr int BN = kNvTilePicksMany * NT;       // columns of the tile
    constexpr int NCF = BN / 16;                     // column fragments per wave (the whole tile)
    __shared__ __align__(16) uint8_t lA[2][kNvPfRows][64];
    __shared__ __align__(16) uint8_t lAs[2][kNvPfRows][8];
    __shared__ __align__(16) uint8_t lB[2][BN * kNvPfBStride];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int li = lane & 15, lg = lane >> 4;
    const int K = GATEUP ? a.d : a.f;
    const int MT = GATEUP ? a.f / 64 : a.d / 128;
    int t_lo = 0, t_hi = *a.ntiles;
    if (a.tile_range) {
        t_lo = a.tile_range[0];
        t_hi = a.tile_range[1];
    }
    const int nt = t_hi - t_lo;
    const int g = blockIdx.x, xcd = g & 7, sidx = g >> 3;
    const int mblk = sidx % MT, tq = sidx / MT;
    const int TPX = (nt + 7) >> 3;
    if (nt <= 0 || tq >= TPX || tq >= tiles_per_xcd_cap) return;
    const int tile = t_lo + xcd * TPX + tq;
    if (tile >= t_hi) return;
    const int e = a.tiles[2 * tile], i0 = a.tiles[2 * tile + 1];
    const int ntok = min(kNvTilePicksMany, range_end(a, e) - i0);
    const moe_expert ex = a.table[e];

    auto a_row = [&](int r, bool scale) -> const uint8_t* {
        int mr;
        const uint8_t* base;
        if (GATEUP) {
            mr = mblk * 64 + (r & 63);
            base = (r < 64) ? (scale ? ex.gate_s : ex.gate_q) : (scale ? ex.up_s : ex.up_q);
        } else {
            mr = mblk * 128 + r;
            base = scale ? ex.down_s : ex.down_q;
        }
        return base + (size_t)mr * (scale ? K / 16 : K / 2);
    };
    auto b_col = [&](int c) -> const uint8_t* {
        const int tc = c / NT, t = c % NT;
        const int tcc = tc < ntok ? tc : 0;
        const size_t arow = GATEUP ? (size_t)pos_token(a, i0 + tcc) : (size_t)(i0 + tcc);
        return a.aq + (arow * NT + t) * (size_t)K * 2;
    };
    // staging: A codes (2 chunks per thread), A scales (threads < 64: 16 bytes = two rows' 8),
    // B (BN * 16 chunks of 16 bytes: BN / 16 per thread)
    constexpr int NBC = BN * 16 / 256;
    const uint8_t* srcA[2];
    int dstA[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int q = i * 256 + tid, r = q >> 2, part = q & 3;
        srcA[i] = a_row(r, false) + part * 16;
        dstA[i] = r * 64 + part * 16;
    }
    const int sq = tid & 63;
    const uint8_t* srcS0 = a_row(2 * sq, true);
    const uint8_t* srcS1 = a_row(2 * sq + 1, true);
    const uint8_t* srcB[NBC];
    int dstB[NBC];
#pragma unroll
    for (int i = 0; i < NBC; ++i) {
        const int q = i * 256 + tid, c = q >> 4, part = q & 15;
        srcB[i] = b_col(c) + part * 16;
        dstB[i] = c * kNvPfBStride + part * 16;
    }
    uint4 vA[2], vB[NBC];
    uint2 vS0, vS1;
    auto load_step = [&](int st) {
#pragma unroll
        for (int i = 0; i < 2; ++i) vA[i] = gload16(srcA[i] + (size_t)st * 64);
        vS0 = gload8(srcS0 + (size_t)st * 8);
        vS1 = gload8(srcS1 + (size_t)st * 8);
#pragma unroll
        for (int i = 0; i < NBC; ++i) vB[i] = gload16(srcB[i] + (size_t)st * 256);
    };
    auto store_step = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 2; ++i) *(uint4*)(&lA[buf][0][0] + dstA[i]) = vA[i];
        if (tid < 64) {
            *(uint2*)&lAs[buf][2 * sq][0] = vS0;
            *(uint2*)&lAs[buf][2 * sq + 1][0] = vS1;
        }
#pragma unroll
        for (int i = 0; i < NBC; ++i) *(uint4*)(&lB[buf][0] + dstB[i]) = vB[i];
    };

    // wave w decodes two 16-row fragments (gate/up: rows 16 w .. of gate and of up; down: rows
    // 32 w ..) once per step and runs them against every column fragment of the tile, so that a
    // decoded fragment feeds 4 NCF MFMAs
    int arow[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) arow[f] = GATEUP ? (f * 64 + wave * 16 + li) : (wave * 32 + f * 16 + li);
    v4f_nv acc[2][NCF];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int n = 0; n < NCF; ++n) acc[f][n] = v4f_nv{0.f, 0.f, 0.f, 0.f};
    const int nsteps = K / 128;
    load_step(0);
    store_step(0);
    __syncthreads();
    for (int st = 0; st < nsteps; ++st) {
        const int buf = st & 1;
        if (st + 1 < nsteps) load_step(st + 1);
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            const uint4 codes = *(const uint4*)&lA[buf][arow[f]][lg * 16];
            const v2f_t bs = e4m3x2_to_f32(*(const uint16_t*)&lAs[buf][arow[f]][2 * lg]);
            const uint32_t w[4] = {codes.x, codes.y, codes.z, codes.w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const bf16x8_t af = nv_dequant8(w[h], h < 2 ? bs[0] : bs[1]);
#pragma unroll
                for (int n = 0; n < NCF; ++n) {
                    const int col = n * 16 + li;
                    const uint4 bv = *(const uint4*)&lB[buf][col * kNvPfBStride + (lg * 32 + 8 * h) * 2];
                    acc[f][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, as_bf16x8(bv), acc[f][n], 0, 0, 0);
                }
            }
        }
        if (st + 1 < nsteps) store_step(buf ^ 1);
        __syncthreads();
    }
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int n = 0; n < NCF; ++n) mfma_results_here(acc[f][n]);
    if constexpr (NT == 2) {
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int n = 0; n < NCF; ++n)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[f][n][r] = sum_adjacent<2>(acc[f][n][r]);
    }
#pragma unroll
    for (int n = 0; n < NCF; ++n) {
        const int c = n * 16 + li, tc = c / NT, t = c % NT;
        if (tc >= ntok || t != 0) continue;
        const size_t pos = (size_t)i0 + tc;
        if constexpr (GATEUP) {
            uint16_t* hb = (uint16_t*)a.hq + pos * NT * (size_t)a.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float gv = acc[0][n][r] * ex.gate_ts, uv = acc[1][n][r] * ex.up_ts;
                const int row = mblk * 64 + wave * 16 + 4 * lg + r;
                put_h_terms<NT>(hb, a.f, row, gv / (1.0f + __expf(-gv)) * uv);
            }
        } else {
            float* dst = a.o + pos * (size_t)a.d + mblk * 128 + wave * 32 + 4 * lg;
#pragma unroll
            for (int f = 0; f < 2; ++f)
                *(float4*)(dst + 16 * f) = make_float4(acc[f][n][0] * ex.down_ts, acc[f][n][1] * ex.down_ts,
                                                       acc[f][n][2] * ex.down_ts, acc[f][n][3] * ex.down_ts);
        }
    }
}

// The same tile for single-term activations (bf16 x in place, h as one bf16 term), fed by a ring
// of four LDS stages that global_load_lds fills three steps ahead, with no register round trip.
// A stage holds one 128-K step: the rows' code bytes, the tile's activation columns and the rows'
// E4M3 scale bytes.  While the MFMAs of step s run, the fragments of step s + 1 are read from LDS
// and decoded into a second register set.  Consecutive lanes read consecutive bytes (4 lanes per
// 64-byte row chunk, 16 per 256-byte column chunk): the vector L1 serves a load one lane quad at a
// time.  In LDS the rows' 16-byte parts are XOR-swizzled (no bank conflicts, measured); the
// columns' units are XOR-swizzled by column, which leaves 4 conflict cycles per column read
// (measured) that cost no time: the kernel ran as fast with the column reads taken out.
// Like the register-staged kernel, this one is bound by its loads, more by the cache lines a step
// requests than by its bytes (the decode, the MFMAs or the column reads, each taken out, changed
// the time by at most 7%).  Against it: 5% faster at K = 6144 (48 steps); at K = 2048 slower, one
// workgroup per CU leaving the ring's fill and drain exposed, so short K stays there.
//
// Stage layout (bytes): row r (0..127) at 64 r, its 16-byte part p in slot p ^ swz_a(r % 16);
// column c (0..63) at 8192 + 256 c, its 16-byte unit u in slot u ^ (c % 16); row r's 8 scale
// bytes at 24576 + 8 r.
constexpr int kNrA = 0, kNrB = 8192, kNrS = 24576, kNrStage = 25600;
constexpr int kNrLoads = 7;      // direct loads per wave and stage: 2 code, 4 activation, 1 scale
constexpr int kNrMinK = 4096;    // shortest K that takes the ring

__device__ __forceinline__ int swz_rows(int r) { return ((r >> 2) ^ (r >> 1)) & 3; }

// the fragments of one step: two decoded 16-row weight fragments (4 MFMAs of 32 K each) and the
// tile's four 16-column activation fragments
struct NrFrags {
    bf16x8_t a[2][4];
    uint4 b[4][4];
};

template <bool GATEUP>
__global__ __launch_bounds__(256, 1) void k_nv_pf_ring(GemmArgs a, int tiles_per_xcd_cap) {
    constexpr int NSTG = 4;                          // stages in the ring
    __shared__ __align__(16) uint8_t stg0[kNrStage];
    __shared__ __align__(16) uint8_t stg1[kNrStage];
    __shared__ __align__(16) uint8_t stg2[kNrStage];
    __shared__ __align__(16) uint8_t stg3[kNrStage];
    constexpr int BN = kNvTilePicksMany;             // columns of the tile (one term per pick)
    constexpr int NCF = BN / 16;
    static_assert(kNrB == 128 * 64 && kNrS == kNrB + BN * 256 && kNrStage == kNrS + 128 * 8, "stage layout");
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int li = lane & 15, lg = lane >> 4;
    const int K = GATEUP ? a.d : a.f;
    const int MT = GATEUP ? a.f / 64 : a.d / 128;
    int t_lo = 0, t_hi = *a.ntiles;
    if (a.tile_range) {
        t_lo = a.tile_range[0];
        t_hi = a.tile_range[1];
    }
    const int nt = t_hi - t_lo;
    const int g = blockIdx.x, xcd = g & 7, sidx = g >> 3;
    const int mblk = sidx % MT, tq = sidx / MT;
    const int TPX = (nt + 7) >> 3;
    if (nt <= 0 || tq >= TPX || tq >= tiles_per_xcd_cap) return;
    const int tile = t_lo + xcd * TPX + tq;
    if (tile >= t_hi) return;
    const int e = a.tiles[2 * tile], i0 = a.tiles[2 * tile + 1];
    const int ntok = min(kNvTilePicksMany, range_end(a, e) - i0);
    const moe_expert ex = a.table[e];

    // tile row r (0..127) -> weight row (gate/up: rows 0..63 gate, 64..127 up, same indices)
    auto a_row = [&](int r, bool scale) -> const uint8_t* {
        int mr;
        const uint8_t* base;
        if (GATEUP) {
            mr = mblk * 64 + (r & 63);
            base = (r < 64) ? (scale ? ex.gate_s : ex.gate_q) : (scale ? ex.up_s : ex.up_q);
        } else {
            mr = mblk * 128 + r;
            base = scale ? ex.down_s : ex.down_q;
        }
        return base + (size_t)mr * (scale ? K / 16 : K / 2);
    };
    // tile column c (0..63) = pick c; columns past the tile re-read column 0
    auto b_col = [&](int c) -> const uint8_t* {
        const int tcc = c < ntok ? c : 0;
        const size_t arow = GATEUP ? (size_t)pos_token(a, i0 + tcc) : (size_t)(i0 + tcc);
        return a.aq + arow * (size_t)K * 2;
    };
    // this wave's direct loads: rows 32 w .. 32 w + 31 (two instructions of 16 rows, a lane quad
    // per row), columns 16 w .. 16 w + 15 (four instructions of 4 columns, 16 lanes per column),
    // and the scale bytes of rows 32 w .. (one instruction, two lanes of 4 bytes per row)
    const uint8_t* srcA[2];
    const uint8_t* srcB[4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int r = (wave * 2 + j) * 16 + (lane >> 2);
        srcA[j] = a_row(r, false) + (((lane & 3) ^ swz_rows(r & 15)) * 16);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = (wave * 4 + j) * 4 + (lane >> 4);
        srcB[j] = b_col(c) + (((lane & 15) ^ (c & 15)) * 16);
    }
    const uint8_t* srcS = a_row(wave * 32 + (lane >> 1), true) + (lane & 1) * 4;
    const int nsteps = K / 128, last = nsteps - 1;
    auto issue = [&](int st, uint8_t* stg) {
        const size_t oa = (size_t)st * 64, ob = (size_t)st * 256, os = (size_t)st * 8;
#pragma unroll
        for (int j = 0; j < 2; ++j) dma16(srcA[j] + oa, stg + kNrA + (wave * 2 + j) * 1024);
#pragma unroll
        for (int j = 0; j < 4; ++j) dma16(srcB[j] + ob, stg + kNrB + (wave * 4 + j) * 1024);
        dma4(srcS + os, stg + kNrS + wave * 256);
    };

    // wave w's two 16-row fragments (gate/up: rows 16 w .. of gate and of up; down: rows 32 w ..)
    int arow[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) arow[f] = GATEUP ? (f * 64 + wave * 16 + li) : (wave * 32 + f * 16 + li);
    // fragments of the step in stage stg: code parts and scale pairs first, then the columns;
    // each lane group takes K [32 lg, 32 lg + 32) of the step, MFMA h its [8 h, 8 h + 8)
    auto read_step = [&](const uint8_t* stg, NrFrags& fr) {
        uint4 codes[2];
        uint32_t sp[2];
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            codes[f] = *(const uint4*)(stg + kNrA + arow[f] * 64 + ((lg ^ swz_rows(li)) * 16));
            sp[f] = *(const uint16_t*)(stg + kNrS + arow[f] * 8 + 2 * lg);
        }
#pragma unroll
        for (int n = 0; n < NCF; ++n)
#pragma unroll
            for (int h = 0; h < 4; ++h)
                fr.b[n][h] = *(const uint4*)(stg + kNrB + (n * 16 + li) * 256 + (((lg * 4 + h) ^ li) * 16));
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            const v2f_t bs = e4m3x2_to_f32(sp[f]);
            const uint32_t w[4] = {codes[f].x, codes[f].y, codes[f].z, codes[f].w};
#pragma unroll
            for (int h = 0; h < 4; ++h) fr.a[f][h] = nv_dequant8(w[h], h < 2 ? bs[0] : bs[1]);
        }
    };
    v4f_nv acc[2][NCF];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int n = 0; n < NCF; ++n) acc[f][n] = v4f_nv{0.f, 0.f, 0.f, 0.f};
    auto run_step = [&](const NrFrags& fr) {
#pragma unroll
        for (int h = 0; h < 4; ++h)
#pragma unroll
            for (int f = 0; f < 2; ++f)
#pragma unroll
                for (int n = 0; n < NCF; ++n)
                    acc[f][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr.a[f][h], as_bf16x8(fr.b[n][h]), acc[f][n],
                                                                        0, 0, 0);
    };
    auto stage_buf = [&](auto i) -> uint8_t* {
        constexpr int I = decltype(i)::value;
        if constexpr (I == 0) return stg0;
        else if constexpr (I == 1) return stg1;
        else if constexpr (I == 2) return stg2;
        else return stg3;
    };

    NrFrags fr0, fr1;
    // every step issues one stage, clamped to the last (past the end the ring is refilled with
    // copies of the last stage that no step reads); before step s reads stage s + 1, the loads of
    // stages s + 2 and s + 3 may still be in flight
    for_steps<0>([&](auto i) { issue(min(decltype(i)::value, last), stage_buf(i)); },
                 std::make_integer_sequence<int, NSTG>{});
    wait_vm<(NSTG - 1) * kNrLoads>();
    ring_barrier();
    read_step(stg0, fr0);
    // step s (s % 8 == Q): stage s is in registers; wait for stage s + 1, refill stage s's buffer
    // with step s + 4, read and decode stage s + 1 into the other register set (past the end:
    // unused values), run the MFMAs of step s
    auto step = [&](int s, auto pos) {
        constexpr int Q = decltype(pos)::value;
        NrFrags& cur = (Q & 1) ? fr1 : fr0;
        NrFrags& nxt = (Q & 1) ? fr0 : fr1;
        wait_vm<(NSTG - 2) * kNrLoads>();
        ring_barrier();                        // also: every wave has stage s in registers
        __builtin_amdgcn_sched_barrier(0);
        issue(min(s + NSTG, last), stage_buf(StepPos<Q % NSTG>{}));
        read_step(stage_buf(StepPos<(Q + 1) % NSTG>{}), nxt);
        run_step(cur);
        // schedule: the code and scale reads of step s + 1 first, then its column reads and
        // direct loads one at a time between the MFMAs of step s, the decode's arithmetic beside
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
#pragma unroll
        for (int i = 0; i < kNrLoads; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
#pragma unroll
        for (int i = 0; i < 32 - 16 - kNrLoads; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    // eight steps per loop iteration: two turns of the ring, four of the register-set pairs
    constexpr int U = 8;
    int s = 0;
    for (; s + U <= nsteps; s += U)
        for_steps<0>([&](auto i) { step(s + decltype(i)::value, i); }, std::make_integer_sequence<int, U>{});
    for_steps<0>([&](auto i) { if (s + decltype(i)::value < nsteps) step(s + decltype(i)::value, i); },
                 std::make_integer_sequence<int, U - 1>{});
    wait_vm<0>();                              // no direct load outlives the workgroup

#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int n = 0; n < NCF; ++n) mfma_results_here(acc[f][n]);
#pragma unroll
    for (int n = 0; n < NCF; ++n) {
        const int tc = n * 16 + li;
        if (tc >= ntok) continue;
        const size_t pos = (size_t)i0 + tc;
        if constexpr (GATEUP) {
            uint16_t* hb = (uint16_t*)a.hq + pos * (size_t)a.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float gv = acc[0][n][r] * ex.gate_ts, uv = acc[1][n][r] * ex.up_ts;
                const int row = mblk * 64 + wave * 16 + 4 * lg + r;
                put_h_terms<1>(hb, a.f, row, gv / (1.0f + __expf(-gv)) * uv);
            }
        } else {
            float* dst = a.o + pos * (size_t)a.d + mblk * 128 + wave * 32 + 4 * lg;
#pragma unroll
            for (int f = 0; f < 2; ++f)
                *(float4*)(dst + 16 * f) = make_float4(acc[f][n][0] * ex.down_ts, acc[f][n][1] * ex.down_ts,
                                                       acc[f][n][2] * ex.down_ts, acc[f][n][3] * ex.down_ts);
        }
    }
}

// Few picks per expert ("decode"): a workgroup of 8 waves owns one tile (up to kNvTilePicks
// picks) and one block of output rows: the same 16 row indices of gate and of up, or 32 down
// rows.  Wave w takes the 16-row fragment w / 4 over the K quarter w % 4 and requests all of its
// code and scale loads at once (NSW super-steps of 128 K at most); the tile's activation columns
// are staged in LDS meanwhile (their first chunks requested before the weights), so the bf16
// operand costs no registers.  Two workgroups share a CU, so one's MFMAs overlap the other's
// loads.  The K quarters are summed through LDS in quarter order by wave 0, which also runs the
// epilogue.  K is at most 512 NSW (so that a quarter has at most NSW super-steps) and a tile
// has at most NCOL / NT picks (the launch guarantees it: a tile holds at most one pick per
// token).
constexpr int kNvDecMaxK = 8192;

template <int NT, bool GATEUP, int NSW, int NCOL>
__global__ __launch_bounds__(512) void k_nv_dec(GemmArgs a) {
    constexpr int KMAX = 512 * NSW;
    constexpr int CST = KMAX * 2 + 16;               // column stride in LDS (bf16, padded)
    __shared__ __align__(16) uint8_t b_lds[NCOL * CST];
    __shared__ v4f_nv part[8][64];
    __shared__ __align__(16) uint8_t s_sc[8][16][128];   // per wave: its rows' scale bytes of its K quarter
    __shared__ int s_staged;                              // filler waves done with the columns
    static_assert(NSW * 8 <= 128 && NSW % 4 == 0, "a K quarter's scale bytes: 8 per super-step and row");
    static_assert(kNvTilePicks <= 4 && kDescTokens >= 4, "a tile's tokens: the first four of its record");
    const int tile = blockIdx.x;
    if constexpr (NCOL <= 2) {
        if (threadIdx.x == 0) s_staged = 0;
        __syncthreads();
    }
    // the tile: with the few-token router's records (a.desc set), the tile count and the record
    // (the expert's pointers and tensor scales, first position, pick count and tokens) in one
    // round trip on the scalar path; else the tile count, the tile's list entry and the tile range
    // together, then the expert table and the end of the expert's range
    moe_expert ex;
    int i0, ntok, tk[4] = {0, 0, 0, 0};
    if (a.desc) {
        const TileDesc* D = a.desc + tile;         // tile < max_tiles: always a written record
        const int32_t* ntp = a.ntiles;
        asm volatile("" : "+s"(ntp));     // read with the record in one round trip
        const int ntile_count = sload(ntp);
        if (GATEUP) {
            ex.gate_q = sload(&D->ex.gate_q);
            ex.up_q = sload(&D->ex.up_q);
            ex.gate_s = sload(&D->ex.gate_s);
            ex.up_s = sload(&D->ex.up_s);
            ex.gate_ts = sload(&D->ex.gate_ts);
            ex.up_ts = sload(&D->ex.up_ts);
            ex.down_q = ex.down_s = nullptr;
            ex.down_ts = 0.0f;
        } else {
            ex.down_q = sload(&D->ex.down_q);
            ex.down_s = sload(&D->ex.down_s);
            ex.down_ts = sload(&D->ex.down_ts);
            ex.gate_q = ex.up_q = ex.gate_s = ex.up_s = nullptr;
            ex.gate_ts = ex.up_ts = 0.0f;
        }
        i0 = sload(&D->i0);
        const int dn = sload(&D->ntok);
#pragma unroll
        for (int j = 0; j < 4; ++j) tk[j] = sload(&D->tok[j]);
        // all of them requested before the first wait
        asm volatile("" ::"s"(ntile_count), "s"(ex.gate_q), "s"(ex.up_q), "s"(ex.down_q), "s"(ex.gate_s),
                     "s"(ex.up_s), "s"(ex.down_s), "s"(ex.gate_ts), "s"(ex.up_ts), "s"(ex.down_ts), "s"(i0),
                     "s"(dn), "s"(tk[0]), "s"(tk[1]), "s"(tk[2]), "s"(tk[3]));
        if (tile >= ntile_count) return;
        ntok = min(min(kNvTilePicks, NCOL / NT), dn);
    } else {
        // (the list entry is read with the count: tile < max_tiles keeps it in bounds, and it is
        // used only for a tile in range)
        const int ntile_count = sload(a.ntiles);
        const int e = sload(&a.tiles[2 * tile]);
        i0 = sload(&a.tiles[2 * tile + 1]);
        int t0 = 0, t1 = ntile_count;
        if (a.tile_range) {
            t0 = sload(a.tile_range);
            t1 = sload(a.tile_range + 1);
        }
        if (tile < t0 || tile >= t1) return;
        ex = a.table[e];
        const int end = e < a.E ? sload(a.offsets + e + 1) : a.Pall;
        ntok = min(min(kNvTilePicks, NCOL / NT), end - i0);
    }
    // token of the tile's pick tc (gate/up columns): the record's, else through sorted_pick
    auto tile_token = [&](int tc) -> int {
        if (a.desc) return tc == 0 ? tk[0] : tc == 1 ? tk[1] : tc == 2 ? tk[2] : tk[3];
        return pos_token(a, i0 + tc);
    };
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int li = lane & 15, lg = lane >> 4;
    const int f = wave >> 2, kq = wave & 3;
    const int K = GATEUP ? a.d : a.f;
    const int cst = K * 2 + 16;
    const int T0 = (GATEUP ? 16 : 32) * blockIdx.y;
    const int NS = K / 128, s0 = (kq * NS) / 4, nss = ((kq + 1) * NS) / 4 - s0;
    // 1. activation columns c = (pick c / NT, term c % NT), K bf16 each, as 16-byte chunks.  With
    // at most two columns (ALL_FIRST) every round is requested before the weights, and so are the
    // scale bytes (step 2), so that the LDS stores below wait for them alone and the barrier after
    // them need not wait for the weights: each super-step's MFMAs then start when its own weights
    // are in.  With more columns the first round goes first and the rest follow the weights.
    const int ncol = ntok * NT, cpc = K / 8, nchunk = ncol * cpc;
    constexpr bool ALL_FIRST = NCOL <= 2;
    constexpr int RF = ALL_FIRST ? (NCOL * (KMAX / 8) + 511) / 512 : 1;     // rounds requested first
    // with at most two columns their bases are found once (one token-index round trip for all
    // rounds, not one per round)
    const uint8_t* colb[2] = {a.aq, a.aq};
    if constexpr (ALL_FIRST) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int cc = c < ncol ? c : ncol - 1, tc = cc / NT, t = cc % NT;
            const size_t arow = GATEUP ? (size_t)tile_token(tc) : (size_t)(i0 + tc);
            colb[c] = a.aq + (arow * NT + t) * (size_t)K * 2;
        }
    }
    auto chunk_src = [&](int g) -> const uint8_t* {
        if constexpr (ALL_FIRST) {
            return colb[g >= cpc ? 1 : 0] + (size_t)(g % cpc) * 16;
        } else {
            const int c = g / cpc, tc = c / NT, t = c % NT;
            const size_t arow = GATEUP ? (size_t)tile_token(tc) : (size_t)(i0 + tc);
            return a.aq + ((arow * NT + t) * (size_t)K + (size_t)(g % cpc) * 8) * 2;
        }
    };
    // (every round's load is issued, without a branch; chunks past the columns re-read the last).
    // With at most two columns, waves 0-3 stage them in LDS before requesting anything else and
    // count themselves in; waves 4-7 go straight to their scales and weights.  (A wave cannot get
    // past a long run of load instructions until the CU's memory pipeline has taken them, so
    // columns stored after the weight requests would hold every wave's MFMAs for most of the
    // stream.)
    constexpr int RS = ALL_FIRST ? 2 * RF : 1;        // rounds of 256 threads
    if constexpr (ALL_FIRST) {
        if (wave < 4) {
            uint4 cv[RS];
#pragma unroll
            for (int r = 0; r < RS; ++r) {
                const int g = tid + 256 * r;
                cv[r] = gload16(chunk_src(g < nchunk ? g : nchunk - 1));
            }
#pragma unroll
            for (int r = 0; r < RS; ++r) {
                const int g = tid + 256 * r;
                if (g < nchunk) *(uint4*)(b_lds + (size_t)(g / cpc) * cst + (size_t)(g % cpc) * 16) = cv[r];
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);        // this wave's LDS stores are done
            asm volatile("" ::: "memory");
            if (lane == 0) atomicAdd(&s_staged, 1);
        }
    }
    uint4 vx[ALL_FIRST ? 1 : RF];
    if constexpr (!ALL_FIRST) {
#pragma unroll
        for (int r = 0; r < RF; ++r) {
            const int g = tid + 512 * r;
            vx[r] = gload16(chunk_src(g < nchunk ? g : nchunk - 1));
        }
    }
    __builtin_amdgcn_sched_barrier(0);     // requested in this order: columns, scales, weights
    // 2. the scale bytes of this wave's quarter, 8 per super-step and row: lane (li, lg) loads
    // those of super-steps lg, lg + 4, .. of row li (past nss: super-step nss - 1 again, not
    // used), one 8-byte load each, for LDS with the columns
    const int row = GATEUP ? T0 + li : T0 + 16 * f + li;
    const uint8_t* mq = GATEUP ? (f == 0 ? ex.gate_q : ex.up_q) : ex.down_q;
    const uint8_t* ms = GATEUP ? (f == 0 ? ex.gate_s : ex.up_s) : ex.down_s;
    const uint8_t* srow = ms + (size_t)row * (K / 16) + (size_t)s0 * 8;
    uint2 S2[NSW / 4];
#pragma unroll
    for (int i = 0; i < NSW / 4; ++i) {
        const int q = 4 * i + lg, qq = q < nss ? q : (nss > 0 ? nss - 1 : 0);
        S2[i] = gload8(srow + (size_t)qq * 8);
    }
    __builtin_amdgcn_sched_barrier(0);
    // 3. this wave's weights: row of fragment f (gate: f = 0, up: f = 1; down: rows 16 f ..),
    // super-steps s0 .. s0 + nss (past nss: re-read; a quarter without steps, K < 512, re-reads
    // step s0, which is inside the row)
    const uint8_t* aq = mq + (size_t)row * (K / 2) + (size_t)s0 * 64 + lg * 16;
    uint4 A[NSW];
#pragma unroll
    for (int q = 0; q < NSW; ++q) {
        const int qq = q < nss ? q : (nss > 0 ? nss - 1 : 0);
        A[q] = gload16(aq + (size_t)qq * 64);
    }
    // 4. the columns and scale bytes into LDS (further rounds, for many columns, after the weights).
    // Their registers are taken here, in straight-line code, so that the wait for them counts the
    // weight loads issued since and leaves those in flight
    if constexpr (!ALL_FIRST) {
#pragma unroll
        for (int r = 0; r < RF; ++r) asm volatile("" ::"v"(vx[r].x), "v"(vx[r].y), "v"(vx[r].z), "v"(vx[r].w));
    }
#pragma unroll
    for (int i = 0; i < NSW / 4; ++i) asm volatile("" ::"v"(S2[i].x), "v"(S2[i].y));
    if constexpr (!ALL_FIRST) {
#pragma unroll
        for (int r = 0; r < RF; ++r) {
            const int g = tid + 512 * r;
            if (g < nchunk) *(uint4*)(b_lds + (size_t)(g / cpc) * cst + (size_t)(g % cpc) * 16) = vx[r];
        }
    }
#pragma unroll
    for (int i = 0; i < NSW / 4; ++i) *(uint2*)&s_sc[wave][li][8 * (4 * i + lg)] = S2[i];
    if constexpr (ALL_FIRST) {
        // the staged columns (an atomic read: a volatile one would also wait for the weights); this
        // wave's own scale bytes are read back by itself, in order
        __builtin_amdgcn_s_waitcnt(0xC07F);
        while (__hip_atomic_load(&s_staged, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < 4)
            __builtin_amdgcn_s_sleep(1);
        asm volatile("" ::: "memory");
    } else {
        for (int g = tid + 512; g < nchunk; g += 512)
            *(uint4*)(b_lds + (size_t)(g / cpc) * cst + (size_t)(g % cpc) * 16) = gload16(chunk_src(g));
        __syncthreads();
    }
    // 5. MFMAs: lane group lg takes K [32 lg, 32 lg + 32) of a super-step, MFMA h its [8h, 8h + 8);
    // columns past the tile read its last column (their results are not used)
    const int col = li < ncol ? li : ncol - 1;
    const uint8_t* bl = b_lds + (size_t)col * cst + (size_t)s0 * 256 + lg * 64;
    v4f_nv acc = v4f_nv{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < NSW; ++q) {
        if (q < nss) {
            const v2f_t bs = e4m3x2_to_f32(*(const uint16_t*)&s_sc[wave][li][8 * q + 2 * lg]);
            const uint32_t w[4] = {A[q].x, A[q].y, A[q].z, A[q].w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const bf16x8_t af = nv_dequant8(w[h], h < 2 ? bs[0] : bs[1]);
                const uint4 b = *(const uint4*)(bl + (size_t)q * 256 + 16 * h);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, as_bf16x8(b), acc, 0, 0, 0);
            }
        }
    }
    // 6. K quarters summed in quarter order by wave 0, then the epilogue
    mfma_results_here(acc);
    part[wave][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
    v4f_nv r4[2];
#pragma unroll
    for (int ff = 0; ff < 2; ++ff) {
        r4[ff] = part[4 * ff][lane];
#pragma unroll
        for (int k2 = 1; k2 < 4; ++k2) r4[ff] += part[4 * ff + k2][lane];
        if constexpr (NT == 2) {
#pragma unroll
            for (int r = 0; r < 4; ++r) r4[ff][r] = sum_adjacent<2>(r4[ff][r]);
        }
    }
    const int tc = li / NT, t = li % NT;
    if (tc >= ntok || t != 0) return;
    const size_t pos = (size_t)i0 + tc;
    if constexpr (GATEUP) {
        // h = silu(g) u for rows T0 + 4 lg + r, as NT bf16 terms [P][NT][f]
        uint16_t* hb = (uint16_t*)a.hq + pos * NT * (size_t)a.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float g = r4[0][r] * ex.gate_ts, u = r4[1][r] * ex.up_ts;
            put_h_terms<NT>(hb, a.f, T0 + 4 * lg + r, g / (1.0f + __expf(-g)) * u);
        }
    } else {
#pragma unroll
        for (int ff = 0; ff < 2; ++ff) {
            float* dst = a.o + pos * (size_t)a.d + T0 + 16 * ff + 4 * lg;
            *(float4*)dst = make_float4(r4[ff][0] * ex.down_ts, r4[ff][1] * ex.down_ts, r4[ff][2] * ex.down_ts,
                                        r4[ff][3] * ex.down_ts);
        }
    }
}

int nv_tile_picks(const moe_shape* s, int T) {
    return (long long)T * s->top_k > 8LL * s->n_experts ? kNvTilePicksMany : kNvTilePicks;
}

hipError_t launch_nv_gemm(const GemmArgs& a, bool gateup, int NT, int tile_picks, int max_tiles, hipStream_t st) {
    const char* name = gateup ? "gemm_gate_up" : "gemm_down";
    trace(name, 0, st);
    const int rows = gateup ? a.f : a.d;
    // few-pick tiles: eight XCD lanes of (32-row blocks / 8, rounded up) x max_tiles workgroups
    const int nrg = rows / 32;
    const dim3 grid((unsigned)(8LL * max_tiles * ((nrg + 7) / 8)));
#define MOE_NV(N, G, P)                                                                     \
    do {                                                                                    \
        if (a.max_tiles != max_tiles) return hipErrorInvalidValue;                          \
        MOE_LAUNCH((k_nv_gemm<N, G, P>), grid, dim3(256), 0, st, a, nrg);                   \
    } while (0)
    if (tile_picks == kNvTilePicksMany) {
        const int MT = gateup ? a.f / 64 : a.d / 128;
        const int cap = (max_tiles + 7) / 8;
        dim3 g2((unsigned)(8 * cap * MT));
        // single-term activations and a long K (at least kNrMinK): the ring-fed kernel, one
        // workgroup per CU; else the register-staged one, whose smaller LDS lets workgroups share a
        // CU and hide each other's start and end (which a short K does not amortise)
        const bool ring = NT == 1 && (gateup ? a.d : a.f) >= kNrMinK;
        if (!gateup && ring) MOE_LAUNCH((k_nv_pf_ring<false>), g2, dim3(256), 0, st, a, cap);
        else if (!gateup && NT == 1) MOE_LAUNCH((k_nv_pf<1, false>), g2, dim3(256), 0, st, a, cap);
        else if (!gateup) MOE_LAUNCH((k_nv_pf<2, false>), g2, dim3(256), 0, st, a, cap);
        else if (ring) MOE_LAUNCH((k_nv_pf_ring<true>), g2, dim3(256), 0, st, a, cap);
        else if (NT == 1) MOE_LAUNCH((k_nv_pf<1, true>), g2, dim3(256), 0, st, a, cap);
        else MOE_LAUNCH((k_nv_pf<2, true>), g2, dim3(256), 0, st, a, cap);
    } else if ((gateup ? a.d : a.f) <= kNvDecMaxK) {
        // LDS columns: a tile holds at most one pick per token, so min(tile picks, T) * NT;
        // super-steps per K quarter: 4 (K <= 2048), 12 (K <= 6144) or 16
        const int K = gateup ? a.d : a.f;
        const bool narrow = (long long)(a.P / a.k < kNvTilePicks ? a.P / a.k : kNvTilePicks) * NT <= 2;
        const int nsw = K <= 2048 ? 4 : (K <= 6144 ? 12 : 16);
        dim3 g3(max_tiles, rows / (gateup ? 16 : 32));
#define MOE_NVD(N, G, S, NC) MOE_LAUNCH((k_nv_dec<N, G, S, NC>), g3, dim3(512), 0, st, a)
#define MOE_NVD_S(N, G, NC)                                                                 \
        do {                                                                                \
            if (nsw == 4) MOE_NVD(N, G, 4, NC);                                             \
            else if (nsw == 12) MOE_NVD(N, G, 12, NC);                                      \
            else MOE_NVD(N, G, 16, NC);                                                     \
        } while (0)
#define MOE_NVD2(N, G)                                                                      \
        do {                                                                                \
            if (narrow) MOE_NVD_S(N, G, 2);                                                 \
            else MOE_NVD_S(N, G, 2 * kNvTilePicks);                                         \
        } while (0)
        if (!gateup && NT == 1) MOE_NVD2(1, false);
        else if (!gateup) MOE_NVD2(2, false);
        else if (NT == 1) MOE_NVD2(1, true);
        else MOE_NVD2(2, true);
#undef MOE_NVD2
#undef MOE_NVD_S
#undef MOE_NVD
    } else {
        if (!gateup && NT == 1) MOE_NV(1, false, kNvTilePicks);
        else if (!gateup) MOE_NV(2, false, kNvTilePicks);
        else if (NT == 1) MOE_NV(1, true, kNvTilePicks);
        else MOE_NV(2, true, kNvTilePicks);
    }
#undef MOE_NV
    trace(name, 1, st);
    return hipGetLastError();
}

}  // namespace moe
