/*
 * Plain fp64 CPU oracle of the routed mixture-of-experts FFN layer.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
 * cpu_baseline leg load this library.  It shares no code, header, table or
 * constant with the HIP library; the only thing both sides share is the byte
 * layout of their inputs (the expert blob, documented below and in the C ABI
 * header), which each side decodes with its own code.
 *
 * Every function is the plain definition, written for a reader to check by eye:
 * fp64 everywhere, loops in the obvious order, no blocking, no fusion.  OpenMP
 * only splits independent output elements across threads; it changes no sum's
 * order.
 *
 * What it follows (pages are cited by title and section):
 *  - top-8 of 288 experts per token, one router per layer with F32 weights
 *    ("Project Maya: GLM-5.3-Flash on two 2017 GPUs ...", section "What is in the
 *    96.5 GB", the tensor-size table; Strata-GLM blog, "Why GLM-5.3-Flash");
 *  - an expert is a gate, an up and a down projection ("Project Maya", "What is
 *    in the 96.5 GB"), combined as a SwiGLU FFN;
 *  - route weights renormalised over the kept experts (Strata-GLM blog,
 *    "Uncensoring without touching the weights", the --renorm-skip fix);
 *  - a routed scaling factor on the routed sum (windlass README, the negative
 *    controls paragraph, routed_scaling_factor 2.5 vs 1.0);
 *  - MXFP4 weights (windlass README, GLM-5.2 MXFP4) and NVFP4 weights ("A hot
 *    expert cache made a 181 GiB model faster ...", "The wall: one PCIe transfer
 *    per token");
 *  - ties in a top-k go to the lower index ("Project Maya", section "Steady speed
 *    with depth", the radix-select replacement keeps the old order, ties broken
 *    by the lower pool index).
 * Readings where the pages are silent (E2M1/E8M0/E4M3 per the OCP formats,
 * nibble order, block axis, sigmoid scoring, SwiGLU form) are listed in the
 * design notes; each is pinned by a CPU test against something other than this
 * file.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define WF_MXFP4 0
#define WF_NVFP4 1

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------------------------------- */
/* element formats                                                                           */
/* ---------------------------------------------------------------------------------------- */

/* E2M1 (OCP MX): 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit, no inf/NaN.
 * Normal (e > 0): 2^(e-1) * (1 + m/2).  Subnormal (e = 0): 0.5 * m. */
double oracle_e2m1(unsigned code) {
    code &= 0xFu;
    unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
    double mag = e ? ldexp(1.0 + 0.5 * (double)m, (int)e - 1) : 0.5 * (double)m;
    return s ? -mag : mag;
}

/* E8M0 (OCP MX scale): 2^(b - 127) for b = 0..254, NaN for 255; no zero, no sign. */
double oracle_e8m0(unsigned b) {
    b &= 0xFFu;
    if (b == 255u) return NAN;
    return ldexp(1.0, (int)b - 127);
}

/* E4M3FN (OCP FP8): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; subnormals;
 * S.1111.111 is NaN; no infinity; largest finite 448. */
double oracle_e4m3(unsigned b) {
    b &= 0xFFu;
    unsigned s = b >> 7, e = (b >> 3) & 0xFu, m = b & 7u;
    if (e == 15u && m == 7u) return NAN;
    double mag = e ? ldexp(1.0 + (double)m / 8.0, (int)e - 7) : ldexp((double)m / 8.0, -6);
    return s ? -mag : mag;
}

/* Dequantise a [rows][K] weight matrix stored as packed E2M1 codes q[rows][K/2]
 * (element 2i in the low nibble, 2i+1 in the high nibble) with one scale per block
 * of B consecutive elements along K: E8M0 for MXFP4 (B = 32), E4M3 times the fp32
 * tensor scale ts for NVFP4 (B = 16).  Returns 0, or -1 on a bad format. */
int oracle_dequant(const uint8_t *q, const uint8_t *s, double ts, int64_t rows, int64_t K,
                   int wformat, double *out) {
    if (wformat != WF_MXFP4 && wformat != WF_NVFP4) return -1;
    const int64_t B = (wformat == WF_MXFP4) ? 32 : 16;
    if (K % B != 0) return -1;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t i = 0; i < K; ++i) {
            unsigned byte = q[r * (K / 2) + i / 2];
            unsigned code = (i % 2 == 0) ? (byte & 0xFu) : (byte >> 4);
            unsigned sb = s[r * (K / B) + i / B];
            double scale = (wformat == WF_MXFP4) ? oracle_e8m0(sb) : oracle_e4m3(sb) * ts;
            out[r * K + i] = oracle_e2m1(code) * scale;
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------------------- */
/* the opt-in MXFP8 activation quantiser (an analogue of the on-the-fly 8-bit activations of */
/* "Project Maya", section "A V100 has no BF16 and no FP8")                                   */
/* ---------------------------------------------------------------------------------------- */

/* The E4M3FN value nearest to v, ties to the even code, for |v| < 448 (no saturation needed
 * here): below 2^-6 the subnormal grid m * 2^-9, else 8 steps per binade [2^e, 2^(e+1)).
 * Exact in fp64: every step is a power of two and rint() rounds half to even. */
double oracle_e4m3_round(double v) {
    double a = fabs(v), q;
    if (a < ldexp(1.0, -6)) {
        q = ldexp(rint(ldexp(a, 9)), -9);
    } else {
        int ex;
        frexp(a, &ex);                          /* a = m * 2^ex, m in [0.5, 1): binade 2^(ex - 1) */
        double step = ldexp(1.0, ex - 1 - 3);
        q = rint(a / step) * step;
    }
    return v < 0 ? -q : q;
}

/* Quantise n values (n a multiple of 32) in place, block by block of 32: with amax the block's
 * largest magnitude, the scale is 2^S with S = floor(log2 amax) - 7 (at least -126; -126 for an
 * all-zero block), so every |v| / 2^S < 256; each value becomes E4M3(v / 2^S) * 2^S. */
void oracle_quant_mxfp8(double *v, int64_t n) {
    for (int64_t b = 0; b < n; b += 32) {
        double amax = 0.0;
        for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs(v[b + i]));
        int S = -126;
        if (amax > 0.0) {
            int ex;
            frexp(amax, &ex);                   /* floor(log2 amax) = ex - 1 */
            S = ex - 1 - 7;
            if (S < -126) S = -126;
        }
        for (int i = 0; i < 32; ++i) v[b + i] = ldexp(oracle_e4m3_round(ldexp(v[b + i], -S)), S);
    }
}

/* ---------------------------------------------------------------------------------------- */
/* expert blob: [gate_q | up_q | down_q | gate_s | up_s | down_s] (+ 3 fp32 tensor scales,  */
/* padded to 256 bytes, for NVFP4).  gate/up are [f][d], down is [d][f]; blocks run along   */
/* the reduction dimension of each row.                                                       */
/* ---------------------------------------------------------------------------------------- */

typedef struct {
    const uint8_t *gate_q, *up_q, *down_q, *gate_s, *up_s, *down_s;
    double gate_ts, up_ts, down_ts;
} oracle_expert_view;

int64_t oracle_blob_stride(int d, int f, int wformat) {
    int64_t B = (wformat == WF_MXFP4) ? 32 : 16;
    int64_t n = 3 * ((int64_t)f * d / 2) + 3 * ((int64_t)f * d / B);
    if (wformat == WF_NVFP4) n = (n + 12 + 255) / 256 * 256;
    return n;
}

static void view_blob(const uint8_t *blob, int d, int f, int wformat, oracle_expert_view *v) {
    int64_t B = (wformat == WF_MXFP4) ? 32 : 16;
    int64_t nq = (int64_t)f * d / 2, ns = (int64_t)f * d / B;
    v->gate_q = blob;
    v->up_q = blob + nq;
    v->down_q = blob + 2 * nq;
    v->gate_s = blob + 3 * nq;
    v->up_s = blob + 3 * nq + ns;
    v->down_s = blob + 3 * nq + 2 * ns;
    v->gate_ts = v->up_ts = v->down_ts = 1.0;
    if (wformat == WF_NVFP4) {
        float ts[3];
        memcpy(ts, blob + 3 * nq + 3 * ns, sizeof ts);
        v->gate_ts = ts[0];
        v->up_ts = ts[1];
        v->down_ts = ts[2];
    }
}

/* ---------------------------------------------------------------------------------------- */
/* router: logits, top-k, normalised sigmoid weights                                         */
/* ---------------------------------------------------------------------------------------- */

/* Is expert a ranked before expert b?  Larger logit first, lower index on equal
 * logits; a NaN logit ranks after every number (NaNs among themselves by index). */
static int ranks_before(double la, int a, double lb, int b) {
    int na = isnan(la), nb = isnan(lb);
    if (na || nb) {
        if (na && nb) return a < b;
        return nb;
    }
    if (la != lb) return la > lb;
    return a < b;
}

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* x: [T][d] fp64 (the layer input, converted exactly); w_router: [E][d] fp32;
 * bias: [E] fp32 or NULL, added to the logit before selection.
 * Outputs: logits [T][E] (may be NULL), idx [T][k] in rank order, w [T][k] with
 * w = sigmoid(l_sel) / sum sigmoid(l_sel).
 * renorm_skip (Strata-GLM blog, "Uncensoring without touching the weights": an expert skipped
 * for its tiny routing weight is dropped cleanly and the remaining weights are renormalised):
 * 0 leaves the picks as they are.  Otherwise every pick after the first whose weight above is
 * below renorm_skip is dropped - idx -1, w 0 - and each kept pick's weight becomes
 * sigmoid(l) / (sum of sigmoid(l) over the kept picks, in rank order).
 * Returns 0, or -1 on bad sizes. */
int oracle_route(const double *x, int T, int d, const float *w_router, const float *bias,
                 int E, int k, double renorm_skip, double *logits, int32_t *idx, double *w) {
    if (T < 0 || d <= 0 || E <= 0 || k < 1 || k > E) return -1;
    #pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        double *l = (double *)malloc(sizeof(double) * (size_t)E);
        char *taken = (char *)calloc((size_t)E, 1);
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int i = 0; i < d; ++i)
                acc += x[(int64_t)t * d + i] * (double)w_router[(int64_t)e * d + i];
            if (bias) acc += (double)bias[e];
            l[e] = acc;
            if (logits) logits[(int64_t)t * E + e] = acc;
        }
        double ssum = 0.0;
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || ranks_before(l[e], e, l[best], best)) best = e;
            }
            taken[best] = 1;
            idx[(int64_t)t * k + j] = best;
            ssum += sigmoid(l[best]);
        }
        for (int j = 0; j < k; ++j)
            w[(int64_t)t * k + j] = sigmoid(l[idx[(int64_t)t * k + j]]) / ssum;
        if (renorm_skip > 0.0) {
            double kept = 0.0;
            for (int j = 0; j < k; ++j) {
                int64_t p = (int64_t)t * k + j;
                if (j > 0 && w[p] < renorm_skip) idx[p] = -1;
                else kept += sigmoid(l[idx[p]]);
            }
            for (int j = 0; j < k; ++j) {
                int64_t p = (int64_t)t * k + j;
                w[p] = idx[p] < 0 ? 0.0 : sigmoid(l[idx[p]]) / kept;
            }
        }
        free(l);
        free(taken);
    }
    return 0;
}

/* ---------------------------------------------------------------------------------------- */
/* permute: counting sort of the picks by expert, stable in pick order (p = t*k + j)         */
/* A dropped pick (expert id -1) takes no position: pick_pos -1; sorted positions past the   */
/* last kept pick hold -1.  Any other id outside [0, E) is an error (-1).                    */
/* ---------------------------------------------------------------------------------------- */

int oracle_permute(const int32_t *idx, int T, int k, int E, int32_t *offsets,
                   int32_t *sorted_pick, int32_t *pick_pos) {
    int64_t P = (int64_t)T * k;
    int32_t *cursor = (int32_t *)calloc((size_t)E + 1, sizeof(int32_t));
    for (int e = 0; e <= E; ++e) offsets[e] = 0;
    for (int64_t p = 0; p < P; ++p) {
        if (idx[p] == -1) continue;
        if (idx[p] < 0 || idx[p] >= E) { free(cursor); return -1; }
        offsets[idx[p] + 1] += 1;
    }
    for (int e = 0; e < E; ++e) offsets[e + 1] += offsets[e];
    for (int64_t i = offsets[E]; i < P; ++i) sorted_pick[i] = -1;
    for (int64_t p = 0; p < P; ++p) {
        int e = idx[p];
        if (e == -1) {
            pick_pos[p] = -1;
            continue;
        }
        int32_t pos = offsets[e] + cursor[e]++;
        sorted_pick[pos] = (int32_t)p;
        pick_pos[p] = pos;
    }
    free(cursor);
    return 0;
}

/* ---------------------------------------------------------------------------------------- */
/* expert FFN: for every pick, o = W_down (silu(W_gate x) * (W_up x)), silu(g) = g*sigmoid(g) */
/* ---------------------------------------------------------------------------------------- */

/* blobs[e]: host pointer to expert e's blob (NULL allowed for experts that receive
 * no pick).  o: [T*k][d], row i belongs to pick sorted_pick[i].  act_quant 1: the FFN's
 * inputs x and h are quantised first (oracle_quant_mxfp8; the opt-in activation mode), 0: used
 * as they are.  Returns 0, -1 on a bad argument, -2 if a routed expert has no blob. */
int oracle_expert_ffn(const uint8_t *const *blobs, int d, int f, int E, int wformat, int act_quant,
                      const double *x, int T, int k, const int32_t *offsets,
                      const int32_t *sorted_pick, double *o) {
    if (d <= 0 || f <= 0 || E <= 0 || k < 1) return -1;
    (void)T;
    double *Wg = (double *)malloc(sizeof(double) * (size_t)f * d);
    double *Wu = (double *)malloc(sizeof(double) * (size_t)f * d);
    double *Wd = (double *)malloc(sizeof(double) * (size_t)d * f);
    double *h = (double *)malloc(sizeof(double) * (size_t)f);
    double *xq = (double *)malloc(sizeof(double) * (size_t)d);
    int rc = 0;
    for (int e = 0; e < E && rc == 0; ++e) {
        if (offsets[e + 1] == offsets[e]) continue;
        if (!blobs[e]) { rc = -2; break; }
        oracle_expert_view v;
        view_blob(blobs[e], d, f, wformat, &v);
        oracle_dequant(v.gate_q, v.gate_s, v.gate_ts, f, d, wformat, Wg);
        oracle_dequant(v.up_q, v.up_s, v.up_ts, f, d, wformat, Wu);
        oracle_dequant(v.down_q, v.down_s, v.down_ts, d, f, wformat, Wd);
        for (int32_t i = offsets[e]; i < offsets[e + 1]; ++i) {
            int t = sorted_pick[i] / k;
            const double *xt = x + (int64_t)t * d;
            if (act_quant) {
                memcpy(xq, xt, sizeof(double) * (size_t)d);
                oracle_quant_mxfp8(xq, d);
                xt = xq;
            }
            #pragma omp parallel for schedule(static)
            for (int r = 0; r < f; ++r) {
                double g = 0.0, u = 0.0;
                for (int c = 0; c < d; ++c) {
                    g += Wg[(int64_t)r * d + c] * xt[c];
                    u += Wu[(int64_t)r * d + c] * xt[c];
                }
                h[r] = g * sigmoid(g) * u;
            }
            if (act_quant) oracle_quant_mxfp8(h, f);
            #pragma omp parallel for schedule(static)
            for (int c = 0; c < d; ++c) {
                double acc = 0.0;
                for (int r = 0; r < f; ++r) acc += Wd[(int64_t)c * f + r] * h[r];
                o[(int64_t)i * d + c] = acc;
            }
        }
    }
    free(Wg);
    free(Wu);
    free(Wd);
    free(h);
    free(xq);
    return rc;
}

/* ---------------------------------------------------------------------------------------- */
/* combine: y[t] = scaling * sum_j w[t,j] * o[pick_pos[t*k+j]] (+ o_shared[t])              */
/* (+ residual[t]), dropped picks (pick_pos -1) left out.  o_shared: the shared expert's    */
/* output per token ("Project Maya", "What is in the 96.5 GB": shared experts beside the    */
/* routed ones), added with weight 1 outside the routed scaling, or NULL.                   */
/* ---------------------------------------------------------------------------------------- */

int oracle_combine(const double *o, const double *w, const int32_t *pick_pos, int T, int k,
                   int d, double scaling, const double *o_shared, const double *residual,
                   double *y) {
    if (T < 0 || k < 1 || d <= 0) return -1;
    #pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int j = 0; j < k; ++j) {
                int32_t pos = pick_pos[(int64_t)t * k + j];
                if (pos < 0) continue;                  /* a dropped pick */
                acc += w[(int64_t)t * k + j] * o[(int64_t)pos * d + c];
            }
            acc *= scaling;
            if (o_shared) acc += o_shared[(int64_t)t * d + c];
            if (residual) acc += residual[(int64_t)t * d + c];
            y[(int64_t)t * d + c] = acc;
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------------------- */
/* whole layer = route, permute, expert FFN, combine                                         */
/* ---------------------------------------------------------------------------------------- */

/* shared_blob: the shared expert's blob, or NULL for none.  Its output for every token is that
 * expert's FFN of the token: the expert FFN above with one expert taking every token once. */
int oracle_layer(const double *x, int T, int d, int f, int E, int k, int wformat, int act_quant,
                 double scaling, double renorm_skip, const float *w_router, const float *bias,
                 const uint8_t *const *blobs, const uint8_t *shared_blob, const double *residual,
                 double *y, int32_t *idx_out, double *w_out, double *logits_out) {
    if (T == 0) return 0;
    int64_t P = (int64_t)T * k;
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)P);
    double *w = (double *)malloc(sizeof(double) * (size_t)P);
    int32_t *offsets = (int32_t *)malloc(sizeof(int32_t) * ((size_t)E + 1));
    int32_t *sorted_pick = (int32_t *)malloc(sizeof(int32_t) * (size_t)P);
    int32_t *pick_pos = (int32_t *)malloc(sizeof(int32_t) * (size_t)P);
    double *o = (double *)malloc(sizeof(double) * (size_t)P * d);
    double *o_shared = NULL;
    int rc = oracle_route(x, T, d, w_router, bias, E, k, renorm_skip, logits_out, idx, w);
    if (rc == 0) rc = oracle_permute(idx, T, k, E, offsets, sorted_pick, pick_pos);
    if (rc == 0) rc = oracle_expert_ffn(blobs, d, f, E, wformat, act_quant, x, T, k, offsets, sorted_pick, o);
    if (rc == 0 && shared_blob) {
        /* one expert, every token: offsets {0, T}, token t at position t */
        int32_t sh_off[2] = {0, T};
        int32_t *sh_pick = (int32_t *)malloc(sizeof(int32_t) * (size_t)T);
        for (int t = 0; t < T; ++t) sh_pick[t] = t;
        o_shared = (double *)malloc(sizeof(double) * (size_t)T * d);
        const uint8_t *sh_blobs[1] = {shared_blob};
        rc = oracle_expert_ffn(sh_blobs, d, f, 1, wformat, act_quant, x, T, 1, sh_off, sh_pick, o_shared);
        free(sh_pick);
    }
    if (rc == 0) rc = oracle_combine(o, w, pick_pos, T, k, d, scaling, o_shared, residual, y);
    if (rc == 0 && idx_out) memcpy(idx_out, idx, sizeof(int32_t) * (size_t)P);
    if (rc == 0 && w_out) memcpy(w_out, w, sizeof(double) * (size_t)P);
    free(idx);
    free(w);
    free(offsets);
    free(sorted_pick);
    free(pick_pos);
    free(o);
    free(o_shared);
    return rc;
}
