// Permute: group the picks by expert on the device (a counting sort, stable in pick order), and
// plan the grouped-GEMM tiles from the per-expert offsets.  The expert list never leaves the
// GPU ("A hot expert cache made a 181 GiB model faster ...", section "A gather kernel that reads
// wide": a device-resident list lets the CPU stay out of the step).
#include "moe_internal.h"

namespace moe {

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / 64;
constexpr int kPermMultiBlocks = 4;    // blocks of picks from which the sort spreads over workgroups

// Block-wide exclusive scan of one int per thread (1024 threads).  Returns the exclusive
// prefix; *total receives the sum.  Uses `scratch` (kPermWaves ints) in LDS.
__device__ int block_excl_scan(int v, int* scratch, int* total) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
    }
    if (lane == 63) scratch[wv] = incl;
    __syncthreads();
    int wbase = 0, tot = 0;
    for (int w = 0; w < kPermWaves; ++w) {
        int s = scratch[w];
        if (w < wv) wbase += s;
        tot += s;
    }
    __syncthreads();
    *total = tot;
    return wbase + incl - v;
}

// Rank of this lane's pick among the lanes of its wave holding the same expert id (ballots over
// the id's 10 bits; ids are below 1024), and their number in *n.  Lanes with e < 0 take part in no
// group.
__device__ __forceinline__ int wave_peer_rank(int e, int lane, int* n) {
    unsigned long long peers = __ballot(e >= 0);
#pragma unroll
    for (int b = 0; b < 10; ++b) {
        unsigned long long m = __ballot((e >> b) & 1);
        peers &= ((e >> b) & 1) ? m : ~m;
    }
    const unsigned long long lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    *n = __popcll(peers);
    return __popcll(peers & lt_mask);
}

// An expert id outside [0, E): -1 is a dropped pick (renorm_skip), anything else an error that
// sets MOE_WS_BAD_EXPERT_ID in the status word (when there is one).  Either way the pick takes no
// sorted position: pick_pos -1, and the positions past offsets[E] hold -1.
__device__ __forceinline__ bool bad_expert_id(int e, int E) { return e < -1 || e >= E; }

__device__ __forceinline__ void report_bad_ids(bool any_bad, uint32_t* status) {
    if (any_bad && status) __hip_atomic_fetch_or(status, MOE_WS_BAD_EXPERT_ID, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
}

// One workgroup of 1024 threads.  LDS: counts and running cursors per expert, and per-wave
// counts of the current chunk (for the stable rank across waves).
__global__ __launch_bounds__(kPermThreads) void k_permute(const int32_t* __restrict__ idx, int P, int E,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ sorted_pick,
                                                          int32_t* __restrict__ pick_pos,
                                                          uint32_t* __restrict__ status) {
    __shared__ int cnt[1024];
    __shared__ int run[1024];
    __shared__ int wcnt[kPermWaves][1024];
    __shared__ int scratch[kPermWaves];
    __shared__ int s_bad;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    for (int e = tid; e < 1024; e += kPermThreads) cnt[e] = 0;
    for (int i = tid; i < kPermWaves * 1024; i += kPermThreads) (&wcnt[0][0])[i] = 0;
    if (tid == 0) s_bad = 0;
    __syncthreads();
    bool bad = false;
    for (int p = tid; p < P; p += kPermThreads) {
        int e = idx[p];
        if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
        bad |= bad_expert_id(e, E);
    }
    if (bad) s_bad = 1;
    __syncthreads();
    int total;
    int excl = block_excl_scan(tid < E ? cnt[tid] : 0, scratch, &total);
    if (tid < E) {
        offsets[tid] = excl;
        run[tid] = excl;
    }
    if (tid == 0) {
        offsets[E] = total;
        report_bad_ids(s_bad != 0, status);
    }
    for (int i = total + tid; i < P; i += kPermThreads) sorted_pick[i] = -1;
    __syncthreads();
    for (int base = 0; base < P; base += kPermThreads) {
        const int p = base + tid;
        int e = (p < P) ? idx[p] : -1;
        if (e >= E || e < 0) {
            if (p < P) pick_pos[p] = -1;
            e = -1;
        }
        int n;
        const int rank = wave_peer_rank(e, lane, &n);
        if (e >= 0 && rank == 0) wcnt[wv][e] = n;
        __syncthreads();
        if (e >= 0) {
            int pos = run[e] + rank;
            for (int w = 0; w < wv; ++w) pos += wcnt[w][e];
            sorted_pick[pos] = p;
            pick_pos[p] = pos;
        }
        __syncthreads();
        if (e >= 0 && rank == 0) {
            atomicAdd(&run[e], n);
            wcnt[wv][e] = 0;
        }
        __syncthreads();
    }
}

// Many picks: the same counting sort over blocks of kPermThreads picks, one workgroup per block.
// (1) per-block counts per expert; (2) one workgroup turns them, expert by expert, into each
// block's first position relative to the expert's offset, and scans the totals into the offsets;
// (3) each block places its picks at offset + block start + rank within the block, which is the
// single-workgroup order (stable in pick order).  bcnt: [nblk][E] int32 in the workspace.
__global__ __launch_bounds__(kPermThreads) void k_perm_count(const int32_t* __restrict__ idx, int P, int E,
                                                             int32_t* __restrict__ bcnt, uint32_t* __restrict__ status) {
    __shared__ int cnt[1024];
    const int tid = threadIdx.x;
    cnt[tid] = 0;
    __syncthreads();
    const int p = blockIdx.x * kPermThreads + tid;
    bool bad = false;
    if (p < P) {
        const int e = idx[p];
        if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
        bad = bad_expert_id(e, E);
    }
    report_bad_ids(__syncthreads_or(bad) && tid == 0, status);
    if (tid < E) bcnt[(size_t)blockIdx.x * E + tid] = cnt[tid];
}

__global__ __launch_bounds__(kPermThreads) void k_perm_scan(int nblk, int E, int P, int32_t* __restrict__ bcnt,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ sorted_pick) {
    __shared__ int scratch[kPermWaves];
    const int e = threadIdx.x;
    int run = 0;
    if (e < E) {
        for (int b0 = 0; b0 < nblk; b0 += 8) {      // eight blocks' loads in flight at once
            int c[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) c[i] = (b0 + i < nblk) ? bcnt[(size_t)(b0 + i) * E + e] : 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (b0 + i < nblk) bcnt[(size_t)(b0 + i) * E + e] = run;
                run += c[i];
            }
        }
    }
    int total;
    const int excl = block_excl_scan(e < E ? run : 0, scratch, &total);
    if (e < E) offsets[e] = excl;
    if (e == 0) offsets[E] = total;
    for (int i = total + e; i < P; i += kPermThreads) sorted_pick[i] = -1;   // positions of no pick
}

__global__ __launch_bounds__(kPermThreads) void k_perm_scatter(const int32_t* __restrict__ idx, int P, int E,
                                                               const int32_t* __restrict__ bcnt,
                                                               const int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ sorted_pick,
                                                               int32_t* __restrict__ pick_pos) {
    __shared__ int wcnt[kPermWaves][1024];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int p = blockIdx.x * kPermThreads + tid;
    int e = (p < P) ? idx[p] : -1;
    if (e >= E || e < 0) {
        if (p < P) pick_pos[p] = -1;
        e = -1;
    }
    for (int i = tid; i < kPermWaves * 1024; i += kPermThreads) (&wcnt[0][0])[i] = 0;
    int n;
    const int rank = wave_peer_rank(e, lane, &n);
    __syncthreads();
    if (e >= 0 && rank == 0) wcnt[wv][e] = n;
    __syncthreads();
    if (e >= 0) {
        int pos = offsets[e] + bcnt[(size_t)blockIdx.x * E + e] + rank;
        for (int w = 0; w < wv; ++w) pos += wcnt[w][e];
        sorted_pick[pos] = p;
        pick_pos[p] = pos;
    }
}

hipError_t launch_permute(const moe_shape* s, const int32_t* idx, int T, int32_t* offsets,
                          int32_t* sorted_pick, int32_t* pick_pos, int32_t* bcnt, uint32_t* status, hipStream_t st) {
    trace("permute", 0, st);
    const int P = T * s->top_k;
    const int nblk = (P + kPermThreads - 1) / kPermThreads;
    if (bcnt && nblk >= kPermMultiBlocks) {
        MOE_LAUNCH(k_perm_count, dim3(nblk), dim3(kPermThreads), 0, st, idx, P, s->n_experts, bcnt, status);
        MOE_LAUNCH(k_perm_scan, dim3(1), dim3(kPermThreads), 0, st, nblk, s->n_experts, P, bcnt, offsets,
                   sorted_pick);
        MOE_LAUNCH(k_perm_scatter, dim3(nblk), dim3(kPermThreads), 0, st, idx, P, s->n_experts, bcnt, offsets,
                   sorted_pick, pick_pos);
    } else {
        MOE_LAUNCH(k_permute, dim3(1), dim3(kPermThreads), 0, st, idx, P, s->n_experts, offsets,
                   sorted_pick, pick_pos, status);
    }
    trace("permute", 1, st);
    return hipGetLastError();
}

// Tiles of at most `tt` consecutive sorted positions of one expert: tiles[i] = (expert, first); then
// the shared expert's (table entry E) over positions [P, P + Tsh), Tsh = T with a shared expert, else 0.
__global__ __launch_bounds__(kPermThreads) void k_plan(const int32_t* __restrict__ offsets, int E, int tt, int P,
                                                       int Tsh, int32_t* __restrict__ tiles,
                                                       int32_t* __restrict__ ntiles) {
    __shared__ int scratch[kPermWaves];
    const int e = threadIdx.x;
    int n = 0, o0 = 0;
    if (e < E) {
        o0 = offsets[e];
        n = offsets[e + 1] - o0;
    }
    const int nt = (n + tt - 1) / tt;
    int total;
    const int first = block_excl_scan(nt, scratch, &total);
    for (int j = 0; j < nt; ++j) {
        tiles[2 * (first + j)] = e;
        tiles[2 * (first + j) + 1] = o0 + j * tt;
    }
    const int nsh = (Tsh + tt - 1) / tt;
    for (int j = threadIdx.x; j < nsh; j += kPermThreads) {
        tiles[2 * (total + j)] = E;
        tiles[2 * (total + j) + 1] = P + j * tt;
    }
    if (e == 0) *ntiles = total + nsh;
}

// workspace preparation: the header (status 0, poll limit) and the hand-over slots (0)
__global__ __launch_bounds__(256) void k_ws_init(uint32_t* __restrict__ ws, size_t nwords, int32_t poll_limit) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < nwords; i += (size_t)gridDim.x * 256)
        ws[i] = i == 1 ? (uint32_t)poll_limit : 0u;
}

hipError_t launch_ws_init(uint32_t* ws, size_t nwords, int32_t poll_limit, hipStream_t st) {
    trace("ws_init", 0, st);
    const size_t blocks = (nwords + 255) / 256;
    MOE_LAUNCH(k_ws_init, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0, st, ws, nwords, poll_limit);
    trace("ws_init", 1, st);
    return hipGetLastError();
}

hipError_t launch_plan(const moe_shape* s, const int32_t* offsets, int T, int tile_tokens, int32_t* tiles,
                       int32_t* ntiles, hipStream_t st) {
    trace("plan", 0, st);
    MOE_LAUNCH(k_plan, dim3(1), dim3(kPermThreads), 0, st, offsets, s->n_experts, tile_tokens, T * s->top_k,
               s->n_shared ? T : 0, tiles, ntiles);
    trace("plan", 1, st);
    return hipGetLastError();
}

// The distinct experts of a tile plan in ascending order, cut into groups of kStageGroup, with
// each group's tile range [first tile of its first expert, first tile of the next group): the
// tiles of a plan are ordered by expert, so a group's tiles are contiguous.  Unused groups (up
// to max_groups) get an empty range.
__global__ __launch_bounds__(kPermThreads) void k_stage_plan(const int32_t* __restrict__ offsets, int E, int tt,
                                                             const int32_t* __restrict__ ntiles,
                                                             int32_t* __restrict__ list, int32_t* __restrict__ nlist,
                                                             int32_t* __restrict__ ranges, int max_groups,
                                                             const moe_expert* __restrict__ table,
                                                             moe_expert* __restrict__ staged, int shared) {
    __shared__ int scratch[kPermWaves];
    const int e = threadIdx.x;
    const int cnt = e < E ? offsets[e + 1] - offsets[e] : 0;
    const int active = cnt > 0 ? 1 : 0;
    int total_tiles, n;
    const int first_tile = block_excl_scan((cnt + tt - 1) / tt, scratch, &total_tiles);
    const int pos = block_excl_scan(active, scratch, &n);
    const int G = kStageGroup;
    const int groups = (n + G - 1) / G;
    for (int g = e; g < max_groups; g += kPermThreads) {
        if (g >= groups) {
            ranges[2 * g] = 0;
            ranges[2 * g + 1] = 0;
        }
    }
    if (active) {
        list[pos] = e;
        if (pos % G == 0) {
            ranges[2 * (pos / G)] = first_tile;
            if (pos > 0) ranges[2 * (pos / G - 1) + 1] = first_tile;
        }
    }
    if (e == 0) {
        *nlist = n;
        // the last group's range runs to the end of the plan, the shared expert's tiles included
        if (n > 0) ranges[2 * (groups - 1) + 1] = *ntiles;
        if (shared) staged[E] = table[E];       // the shared expert is read in place
    }
}

hipError_t launch_stage_plan(const moe_shape* s, const int32_t* offsets, int tt, const int32_t* ntiles,
                             int32_t* list, int32_t* nlist, int32_t* ranges, const moe_expert* table,
                             moe_expert* staged, hipStream_t st) {
    trace("stage_plan", 0, st);
    const int max_groups = (s->n_experts + kStageGroup - 1) / kStageGroup;
    MOE_LAUNCH(k_stage_plan, dim3(1), dim3(kPermThreads), 0, st, offsets, s->n_experts, tt, ntiles, list, nlist,
               ranges, max_groups, table, staged, s->n_shared);
    trace("stage_plan", 1, st);
    return hipGetLastError();
}

}  // namespace moe
