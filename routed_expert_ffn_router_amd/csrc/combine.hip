// Route-weighted combine, expert-table fill and the device-list expert gather.
#include "moe_internal.h"

namespace moe {

// y[t] = s * sum_j w[t,j] * o[pick_pos[t*k+j]] (+ residual[t]); one thread per 4 columns,
// the k terms summed in rank order in fp32 (picks with pick_pos -1 left out), rounded once to the
// output dtype.
// With a shared expert (shared = 1) its output, row T k + t of o, is added after the scaling.
template <typename XT>
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ o, const float* __restrict__ w,
                                                 const int32_t* __restrict__ pick_pos, int T, int k, int d,
                                                 float scaling, int shared, const XT* __restrict__ residual,
                                                 XT* __restrict__ y) {
    const int t = blockIdx.y;
    const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (c >= d) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    // eight picks at a time: their positions and weights, then all eight partial loads, then the
    // sums in rank order (so the loads are in flight together, not one round trip per pick).  A
    // pick without an expert (dropped or refused, position -1), or past k, reads row 0 and adds
    // nothing.
    for (int j0 = 0; j0 < k; j0 += 8) {
        int pos[8];
        float wj[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int j = j0 + i;
            pos[i] = j < k ? pick_pos[(size_t)t * k + j] : -1;
            wj[i] = j < k ? w[(size_t)t * k + j] : 0.0f;
        }
        float4 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = *(const float4*)(o + (size_t)(pos[i] >= 0 ? pos[i] : 0) * d + c);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const bool use = pos[i] >= 0;
            acc.x = use ? fmaf(wj[i], v[i].x, acc.x) : acc.x;
            acc.y = use ? fmaf(wj[i], v[i].y, acc.y) : acc.y;
            acc.z = use ? fmaf(wj[i], v[i].z, acc.z) : acc.z;
            acc.w = use ? fmaf(wj[i], v[i].w, acc.w) : acc.w;
        }
    }
    float r[4] = {acc.x * scaling, acc.y * scaling, acc.z * scaling, acc.w * scaling};
    if (shared) {
        const float4 v = *(const float4*)(o + ((size_t)T * k + t) * d + c);
        r[0] += v.x;
        r[1] += v.y;
        r[2] += v.z;
        r[3] += v.w;
    }
    const size_t b = (size_t)t * d + c;
    if (residual) {
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] += load_act(residual, b + i);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) store_act(y, b + i, r[i]);
}

hipError_t launch_combine(const moe_shape* s, const float* o, const float* w, const int32_t* pick_pos,
                          int T, const void* residual, void* y, hipStream_t st) {
    trace("combine", 0, st);
    const int d = s->d_model;
    dim3 grid((d / 4 + 255) / 256, T);
    if (s->act_dtype == MOE_DT_BF16)
        MOE_LAUNCH(k_combine<uint16_t>, grid, dim3(256), 0, st, o, w, pick_pos, T, s->top_k, d,
                   s->routed_scaling, s->n_shared, (const uint16_t*)residual, (uint16_t*)y);
    else
        MOE_LAUNCH(k_combine<float>, grid, dim3(256), 0, st, o, w, pick_pos, T, s->top_k, d,
                   s->routed_scaling, s->n_shared, (const float*)residual, (float*)y);
    trace("combine", 1, st);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// expert table from fixed-stride blobs [gate_q | up_q | down_q | gate_s | up_s | down_s | ts]
// ---------------------------------------------------------------------------------------------
struct BlobSizes {
    size_t nq, ns;
};

static BlobSizes blob_sizes(const moe_shape* s) {
    const size_t B = s->wformat == MOE_WF_MXFP4 ? 32 : 16;
    const size_t fd = (size_t)s->d_model * s->d_ff;
    return {fd / 2, fd / B};
}

__global__ void k_fill_table(const uint8_t* __restrict__ base, size_t stride, int E, size_t nq, size_t ns,
                             int nv, moe_expert* __restrict__ table) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= E) return;
    const uint8_t* b = base + (size_t)e * stride;
    moe_expert m;
    m.gate_q = b;
    m.up_q = b + nq;
    m.down_q = b + 2 * nq;
    m.gate_s = b + 3 * nq;
    m.up_s = b + 3 * nq + ns;
    m.down_s = b + 3 * nq + 2 * ns;
    m.gate_ts = m.up_ts = m.down_ts = 1.0f;
    m.reserved = 0.0f;
    if (nv) {
        const float* ts = (const float*)(b + 3 * nq + 3 * ns);
        m.gate_ts = ts[0];
        m.up_ts = ts[1];
        m.down_ts = ts[2];
    }
    table[e] = m;
}

hipError_t launch_fill_table(const moe_shape* s, const uint8_t* base, size_t stride, moe_expert* table,
                             hipStream_t st) {
    trace("fill_table", 0, st);
    const BlobSizes z = blob_sizes(s);
    const int n = s->n_experts + s->n_shared;       // the shared expert's entry last
    MOE_LAUNCH(k_fill_table, dim3((n + 255) / 256), dim3(256), 0, st, base, stride, n, z.nq, z.ns,
               (int)(s->wformat == MOE_WF_NVFP4), table);
    trace("fill_table", 1, st);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// gather: copy the listed experts into contiguous staging with 16-byte loads ("A hot expert
// cache ...", section "A gather kernel that reads wide": wide reads from a device-resident list)
// ---------------------------------------------------------------------------------------------
// copy one expert's six sub-tensors into dst (its canonical blob) with 16-byte loads; returns the
// staged table entry
__device__ moe_expert gather_one(const moe_expert& src, uint8_t* dst, size_t nq, size_t ns, size_t stride) {
    const size_t n16 = (3 * nq + 3 * ns) / 16;
    auto src_of = [&](size_t off) -> const uint8_t* {
        if (off < nq) return src.gate_q + off;
        if (off < 2 * nq) return src.up_q + (off - nq);
        if (off < 3 * nq) return src.down_q + (off - 2 * nq);
        if (off < 3 * nq + ns) return src.gate_s + (off - 3 * nq);
        if (off < 3 * nq + 2 * ns) return src.up_s + (off - 3 * nq - ns);
        return src.down_s + (off - 3 * nq - 2 * ns);
    };
    // four 16-byte units per thread and round, all loaded before any is stored, so that each
    // thread keeps four loads in flight; units past the end re-read the last one and are not stored
    const size_t G = (size_t)gridDim.x * 256;
    for (size_t u = (size_t)blockIdx.x * 256 + threadIdx.x; u < n16; u += 4 * G) {
        uint4 v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const size_t ui = u + i * G < n16 ? u + i * G : n16 - 1;
            v[i] = gload16(src_of(ui * 16));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (u + i * G < n16) *(uint4*)(dst + (u + i * G) * 16) = v[i];
    }
    moe_expert m;
    m.gate_q = dst;
    m.up_q = dst + nq;
    m.down_q = dst + 2 * nq;
    m.gate_s = dst + 3 * nq;
    m.up_s = dst + 3 * nq + ns;
    m.down_s = dst + 3 * nq + 2 * ns;
    m.gate_ts = src.gate_ts;
    m.up_ts = src.up_ts;
    m.down_ts = src.down_ts;
    m.reserved = 0.0f;
    if (blockIdx.x == 0 && threadIdx.x == 0 && stride >= 3 * nq + 3 * ns + 12) {
        float* ts = (float*)(dst + 3 * nq + 3 * ns);
        ts[0] = src.gate_ts;
        ts[1] = src.up_ts;
        ts[2] = src.down_ts;
    }
    return m;
}

__global__ __launch_bounds__(256) void k_gather(const moe_expert* __restrict__ table,
                                                const int32_t* __restrict__ list, int n, size_t nq,
                                                size_t ns, size_t stride, uint8_t* __restrict__ staging,
                                                moe_expert* __restrict__ staged) {
    const int i = blockIdx.y;
    const moe_expert m = gather_one(table[list[i]], staging + (size_t)i * stride, nq, ns, stride);
    if (blockIdx.x == 0 && threadIdx.x == 0) staged[i] = m;
}

// group `group` of the distinct-expert list: expert list[group * G + i] goes to staging slot i and
// its staged entry to staged_by_expert[expert] (the table the grouped GEMMs read)
__global__ __launch_bounds__(256) void k_gather_group(const moe_expert* __restrict__ table,
                                                      const int32_t* __restrict__ list,
                                                      const int32_t* __restrict__ nlist, int group, size_t nq,
                                                      size_t ns, size_t stride, uint8_t* __restrict__ staging,
                                                      moe_expert* __restrict__ staged_by_expert) {
    const int i = blockIdx.y;
    const int li = group * kStageGroup + i;
    if (li >= *nlist) return;
    const int e = list[li];
    const moe_expert m = gather_one(table[e], staging + (size_t)i * stride, nq, ns, stride);
    if (blockIdx.x == 0 && threadIdx.x == 0) staged_by_expert[e] = m;
}

hipError_t launch_gather_group(const moe_shape* s, const moe_expert* table, const int32_t* list,
                               const int32_t* nlist, int group, uint8_t* staging, size_t stride,
                               moe_expert* staged_by_expert, hipStream_t st) {
    trace("gather", 0, st);
    const BlobSizes z = blob_sizes(s);
    const int G = s->n_experts < kStageGroup ? s->n_experts : kStageGroup;
    MOE_LAUNCH(k_gather_group, dim3(64, G), dim3(256), 0, st, table, list, nlist, group, z.nq, z.ns, stride, staging,
               staged_by_expert);
    trace("gather", 1, st);
    return hipGetLastError();
}

hipError_t launch_gather(const moe_shape* s, const moe_expert* table, const int32_t* list, int n,
                         uint8_t* staging, size_t stride, moe_expert* staged, hipStream_t st) {
    trace("gather", 0, st);
    const BlobSizes z = blob_sizes(s);
    dim3 grid(64, n);
    MOE_LAUNCH(k_gather, grid, dim3(256), 0, st, table, list, n, z.nq, z.ns, stride, staging, staged);
    trace("gather", 1, st);
    return hipGetLastError();
}

}  // namespace moe
