/*
 * moe_oracle.c — CPU oracle for the MoE expert layer (TEST INFRASTRUCTURE ONLY).
 *
 * Plain loops in the order the pages describe the layer; fp64 arithmetic except the fp32
 * router-logit chain. OpenMP only splits independent tokens/rows across threads; no loop is
 * blocked, fused or reordered. See moe_oracle.h for the page passages each function follows.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static inline float bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* element i of a tensor of dtype dt, widened exactly */
static inline float elf(const void* p, int dt, int64_t i) {
    return dt == ORC_F32 ? ((const float*)p)[i] : bf16_to_f32(((const uint16_t*)p)[i]);
}
static inline double eld(const void* p, int dt, int64_t i) { return (double)elf(p, dt, i); }

static int bad_dt(int dt) { return dt != ORC_F32 && dt != ORC_BF16; }

#ifdef _OPENMP
#include <omp.h>
void orc_set_threads(int n) {
    if (n > 0) omp_set_num_threads(n);
}
int orc_max_threads(void) { return omp_get_max_threads(); }
#else
void orc_set_threads(int n) { (void)n; }
int orc_max_threads(void) { return 1; }
#endif

static double silu(double z) { return z / (1.0 + exp(-z)); }
static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* ------------------------------------------------------------------------------------------ */
/* Router logits: gate applied to the token, in fp32 ("FP32 softmax" consumes fp32 logits).    */
/* Four fixed blocks of the hidden dimension, each an fmaf chain from 0 in ascending h, then the */
/* four partial sums added in block order: ((c0 + c1) + c2) + c3. Block b covers                */
/* [b*HB, min((b+1)*HB, H)), HB = 128 * ceil(H / 512); an empty block contributes +0.0.         */
int orc_router_logit_block(int64_t H) { return (int)(128 * ((H + 511) / 512)); }

int orc_router_logits(const void* x, const void* w_gate, int dt, int64_t T, int64_t H, int64_t E,
                      float* logits) {
    if (!x || !w_gate || !logits || bad_dt(dt) || T < 0 || H < 0 || E < 1) return -1;
    const int64_t hb = orc_router_logit_block(H);
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t e = 0; e < E; ++e) {
            float total = 0.0f;
            for (int64_t b = 0; b < 4; ++b) {
                float acc = 0.0f;
                for (int64_t h = b * hb; h < (b + 1) * hb && h < H; ++h)
                    acc = fmaf(elf(x, dt, t * H + h), elf(w_gate, dt, h * E + e), acc);
                total = b == 0 ? acc : total + acc;
            }
            logits[t * E + e] = total;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* Top-k selection and weight normalisation.                                                  */
typedef struct {
    float l;
    int32_t e;
} scored;

/* total order: larger logit first, then lower expert index */
static int by_logit_desc(const void* a, const void* b) {
    const scored* p = (const scored*)a;
    const scored* q = (const scored*)b;
    if (p->l > q->l) return -1;
    if (p->l < q->l) return 1;
    return (p->e > q->e) - (p->e < q->e);
}

int orc_router_topk(const float* logits, int64_t T, int64_t E, int64_t k, int renorm,
                    int32_t* topk_idx, double* topk_w) {
    if (!logits || !topk_idx || !topk_w || T < 0 || E < 1 || k < 1 || k > E) return -1;
#pragma omp parallel
    {
        scored* s = (scored*)malloc(sizeof(scored) * (size_t)E);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            const float* l = logits + t * E;
            for (int64_t e = 0; e < E; ++e) {
                s[e].l = l[e];
                s[e].e = (int32_t)e;
            }
            qsort(s, (size_t)E, sizeof(scored), by_logit_desc);
            double m = (double)s[0].l;
            double den = 0.0;
            if (renorm) {
                for (int64_t j = 0; j < k; ++j) den += exp((double)s[j].l - m);
            } else {
                for (int64_t e = 0; e < E; ++e) den += exp((double)l[e] - m);
            }
            for (int64_t j = 0; j < k; ++j) {
                topk_idx[t * k + j] = s[j].e;
                topk_w[t * k + j] = exp((double)s[j].l - m) / den;
            }
        }
        free(s);
    }
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* Router statistics: the full softmax per token, its mean over tokens, and the expert load.   */
int orc_router_stats(const float* logits, const int32_t* topk_idx, int64_t T, int64_t E, int64_t k,
                     double* probs, double* mean_prob, int64_t* load) {
    if (!logits || !topk_idx || !mean_prob || !load || T < 0 || E < 1 || k < 1) return -1;
    for (int64_t e = 0; e < E; ++e) {
        mean_prob[e] = 0.0;
        load[e] = 0;
    }
    double* p = (double*)malloc(sizeof(double) * (size_t)E);
    for (int64_t t = 0; t < T; ++t) {
        const float* l = logits + t * E;
        double m = (double)l[0];
        for (int64_t e = 1; e < E; ++e)
            if ((double)l[e] > m) m = (double)l[e];
        double den = 0.0;
        for (int64_t e = 0; e < E; ++e) {
            p[e] = exp((double)l[e] - m);
            den += p[e];
        }
        for (int64_t e = 0; e < E; ++e) {
            p[e] /= den;
            mean_prob[e] += p[e];
            if (probs) probs[t * E + e] = p[e];
        }
        for (int64_t j = 0; j < k; ++j) {
            const int32_t e = topk_idx[t * k + j];
            if (e >= 0 && e < E) load[e] += 1;
        }
    }
    free(p);
    if (T > 0)
        for (int64_t e = 0; e < E; ++e) mean_prob[e] /= (double)T;
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* Permute plan: rows grouped by expert, tokens ascending inside each expert.                  */
int orc_permute_plan(const int32_t* topk_idx, int64_t T, int64_t k, int64_t E, int32_t* counts,
                     int32_t* offsets, int32_t* row_of_slot, int32_t* slot_of_row) {
    if (!topk_idx || !counts || !offsets || !row_of_slot || !slot_of_row || T < 0 || k < 1 || E < 1)
        return -1;
    const int64_t N = T * k;
    /* a slot whose index lies outside [0, E) names no expert: it is sent nowhere, so it is not
     * counted and gets no row (row_of_slot = -1); the rows of the valid slots follow in order */
    for (int64_t e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t s = 0; s < N; ++s)
        if (topk_idx[s] >= 0 && topk_idx[s] < E) counts[topk_idx[s]] += 1;
    offsets[0] = 0;
    for (int64_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    for (int64_t s = 0; s < N; ++s) {
        row_of_slot[s] = -1;
        slot_of_row[s] = -1;
    }
    /* rows expert by expert; inside an expert, tokens ascending and, should a token name the same
     * expert in several slots, those slots in ascending order */
    int64_t row = 0;
    for (int64_t e = 0; e < E; ++e)
        for (int64_t t = 0; t < T; ++t)
            for (int64_t j = 0; j < k; ++j)
                if (topk_idx[t * k + j] == e) {
                    row_of_slot[t * k + j] = (int32_t)row;
                    slot_of_row[row] = (int32_t)(t * k + j);
                    ++row;
                }
    return 0;
}

int orc_permute_rows(const void* x, int64_t elem_bytes, int64_t H, const int32_t* slot_of_row,
                     int64_t k, int64_t N, void* x_perm) {
    if (!x || !slot_of_row || !x_perm || elem_bytes < 1 || H < 0 || k < 1 || N < 0) return -1;
    const size_t rb = (size_t)(elem_bytes * H);
    for (int64_t r = 0; r < N; ++r)
        if (slot_of_row[r] < 0) return -2; /* only rows that exist (below offsets[E]) are copied */
    for (int64_t r = 0; r < N; ++r) {
        int64_t t = slot_of_row[r] / k;
        memcpy((char*)x_perm + (size_t)r * rb, (const char*)x + (size_t)t * rb, rb);
    }
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* One expert's SwiGLU FFN on one row (fp64). gu/dn point at the expert's block of the fused   */
/* weights: gu [H, 2I] row-major (gate columns 0..I-1, up columns I..2I-1), dn [I, H].         */
static void ffn_row(const double* xr, int dt, const void* gu, int64_t gu_off, const void* dn,
                    int64_t dn_off, int64_t H, int64_t I, double* g, double* u, double* a,
                    double* y) {
    for (int64_t i = 0; i < I; ++i) g[i] = u[i] = 0.0;
    for (int64_t h = 0; h < H; ++h) {
        const double xh = xr[h];
        const int64_t base = gu_off + h * 2 * I;
        for (int64_t i = 0; i < I; ++i) {
            g[i] += xh * eld(gu, dt, base + i);
            u[i] += xh * eld(gu, dt, base + I + i);
        }
    }
    for (int64_t i = 0; i < I; ++i) a[i] = silu(g[i]) * u[i];
    for (int64_t c = 0; c < H; ++c) y[c] = 0.0;
    for (int64_t i = 0; i < I; ++i) {
        const double ai = a[i];
        const int64_t base = dn_off + i * H;
        for (int64_t c = 0; c < H; ++c) y[c] += ai * eld(dn, dt, base + c);
    }
}

static int64_t expert_of_row(const int32_t* offsets, int64_t E, int64_t r) {
    for (int64_t e = 0; e < E; ++e)
        if (offsets[e] <= r && r < offsets[e + 1]) return e;
    return -1;
}

int orc_expert_rows(const void* x_perm, int dt, int64_t H, int64_t I, int64_t E,
                    const int32_t* offsets, const void* gate_up, const void* down,
                    const int64_t* rows, int64_t nrows, double* y_out, double* a_out, double* gu_out) {
    if (!x_perm || !offsets || !gate_up || !down || !rows || !y_out || bad_dt(dt) || H < 1 || I < 1 ||
        E < 1 || nrows < 0)
        return -1;
    for (int64_t n = 0; n < nrows; ++n)
        if (expert_of_row(offsets, E, rows[n]) < 0) return -2;
#pragma omp parallel
    {
        double* xr = (double*)malloc(sizeof(double) * (size_t)H);
        double* g = (double*)malloc(sizeof(double) * (size_t)I);
        double* u = (double*)malloc(sizeof(double) * (size_t)I);
        double* a = (double*)malloc(sizeof(double) * (size_t)I);
#pragma omp for schedule(dynamic, 1)
        for (int64_t n = 0; n < nrows; ++n) {
            const int64_t r = rows[n];
            const int64_t e = expert_of_row(offsets, E, r);
            for (int64_t h = 0; h < H; ++h) xr[h] = eld(x_perm, dt, r * H + h);
            ffn_row(xr, dt, gate_up, e * H * 2 * I, down, e * I * H, H, I, g, u, a, y_out + n * H);
            if (a_out) memcpy(a_out + n * I, a, sizeof(double) * (size_t)I);
            if (gu_out) {
                memcpy(gu_out + n * 2 * I, g, sizeof(double) * (size_t)I);
                memcpy(gu_out + n * 2 * I + I, u, sizeof(double) * (size_t)I);
            }
        }
        free(xr);
        free(g);
        free(u);
        free(a);
    }
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* Unpermute + gate-weighted combine.                                                          */
int orc_combine(const void* y, int dt, int64_t H, int64_t k, const int32_t* row_of_slot,
                const float* topk_w, const void* residual, const int64_t* tokens, int64_t ntok,
                double* out) {
    if (!y || !row_of_slot || !topk_w || !tokens || !out || bad_dt(dt) || H < 1 || k < 1 || ntok < 0)
        return -1;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < ntok; ++n) {
        const int64_t t = tokens[n];
        double* o = out + n * H;
        for (int64_t c = 0; c < H; ++c) o[c] = residual ? eld(residual, dt, t * H + c) : 0.0;
        for (int64_t j = 0; j < k; ++j) {
            const double w = (double)topk_w[t * k + j];
            const int64_t r = row_of_slot[t * k + j];
            if (r < 0) continue; /* a dropped slot contributes nothing */
            for (int64_t c = 0; c < H; ++c) o[c] += w * eld(y, dt, r * H + c);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* Whole layer per token: sum over the token's k experts of gate weight x expert FFN.          */
int orc_moe_forward_tokens(const void* x, int dt, int64_t H, int64_t I, int64_t E, int64_t k,
                           const int32_t* topk_idx, const double* topk_w, const void* gate_up,
                           const void* down, const void* shared_gate_up, const void* shared_down,
                           int64_t Is, const int64_t* tokens, int64_t ntok, double* out) {
    if (!x || !topk_idx || !topk_w || !gate_up || !down || !tokens || !out || bad_dt(dt) || H < 1 ||
        I < 1 || E < 1 || k < 1 || ntok < 0)
        return -1;
    if (shared_gate_up && (!shared_down || Is < 1)) return -1;
    const int64_t Imax = (shared_gate_up && Is > I) ? Is : I;
#pragma omp parallel
    {
        double* xr = (double*)malloc(sizeof(double) * (size_t)H);
        double* y = (double*)malloc(sizeof(double) * (size_t)H);
        double* g = (double*)malloc(sizeof(double) * (size_t)Imax);
        double* u = (double*)malloc(sizeof(double) * (size_t)Imax);
        double* a = (double*)malloc(sizeof(double) * (size_t)Imax);
#pragma omp for schedule(dynamic, 1)
        for (int64_t n = 0; n < ntok; ++n) {
            const int64_t t = tokens[n];
            double* o = out + n * H;
            for (int64_t h = 0; h < H; ++h) xr[h] = eld(x, dt, t * H + h);
            for (int64_t c = 0; c < H; ++c) o[c] = 0.0;
            for (int64_t j = 0; j < k; ++j) {
                const int64_t e = topk_idx[t * k + j];
                if (e < 0 || e >= E) continue;
                ffn_row(xr, dt, gate_up, e * H * 2 * I, down, e * I * H, H, I, g, u, a, y);
                const double w = topk_w[t * k + j];
                for (int64_t c = 0; c < H; ++c) o[c] += w * y[c];
            }
            if (shared_gate_up) {
                ffn_row(xr, dt, shared_gate_up, 0, shared_down, 0, H, Is, g, u, a, y);
                for (int64_t c = 0; c < H; ++c) o[c] += y[c];
            }
        }
        free(xr);
        free(y);
        free(g);
        free(u);
        free(a);
    }
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* Backward.                                                                                   */
int orc_combine_bwd(const void* d_out, int dt, const void* y, int dt_y, int64_t H, int64_t k,
                    const int32_t* row_of_slot, const float* topk_w, const int64_t* tokens,
                    int64_t ntok, double* d_y_slots, double* d_w) {
    if (!d_out || !y || !row_of_slot || !topk_w || !tokens || bad_dt(dt) || bad_dt(dt_y) || H < 1 || k < 1 ||
        ntok < 0)
        return -1;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < ntok; ++n) {
        const int64_t t = tokens[n];
        for (int64_t j = 0; j < k; ++j) {
            const double w = (double)topk_w[t * k + j];
            const int64_t r = row_of_slot[t * k + j];
            double dot = 0.0;
            for (int64_t c = 0; c < H; ++c) {
                const double go = eld(d_out, dt, t * H + c);
                /* a dropped slot (no row) takes no part in the combine: zero gradients */
                if (d_y_slots) d_y_slots[(n * k + j) * H + c] = r < 0 ? 0.0 : w * go;
                if (r >= 0) dot += go * eld(y, dt_y, r * H + c);
            }
            if (d_w) d_w[n * k + j] = dot;
        }
    }
    return 0;
}

/* Backward of one expert FFN row; accumulates nothing, returns per-row results. */
static void ffn_row_bwd(const double* xr, const double* dyr, int dt, const void* gu, int64_t gu_off,
                        const void* dn, int64_t dn_off, int64_t H, int64_t I, double* g, double* u,
                        double* da, double* dg, double* du, double* dx) {
    for (int64_t i = 0; i < I; ++i) g[i] = u[i] = 0.0;
    for (int64_t h = 0; h < H; ++h) {
        const double xh = xr[h];
        const int64_t base = gu_off + h * 2 * I;
        for (int64_t i = 0; i < I; ++i) {
            g[i] += xh * eld(gu, dt, base + i);
            u[i] += xh * eld(gu, dt, base + I + i);
        }
    }
    /* da_i = sum_c dy_c * down[i, c] */
    for (int64_t i = 0; i < I; ++i) {
        double s = 0.0;
        const int64_t base = dn_off + i * H;
        for (int64_t c = 0; c < H; ++c) s += dyr[c] * eld(dn, dt, base + c);
        da[i] = s;
    }
    for (int64_t i = 0; i < I; ++i) {
        const double sg = sigmoid(g[i]);
        dg[i] = da[i] * u[i] * sg * (1.0 + g[i] * (1.0 - sg));
        du[i] = da[i] * g[i] * sg;
    }
    /* dx_h = sum_i dg_i gate_up[h, i] + du_i gate_up[h, I+i] */
    for (int64_t h = 0; h < H; ++h) {
        double s = 0.0;
        const int64_t base = gu_off + h * 2 * I;
        for (int64_t i = 0; i < I; ++i) s += dg[i] * eld(gu, dt, base + i) + du[i] * eld(gu, dt, base + I + i);
        dx[h] = s;
    }
}

int orc_expert_rows_bwd(const void* x_perm, const void* d_y, int dt, int dt_dy, int64_t H, int64_t I,
                        int64_t E, const int32_t* offsets, const void* gate_up, const void* down,
                        const int64_t* rows, int64_t nrows, double* d_x_out, double* d_gu_out) {
    if (!x_perm || !d_y || !offsets || !gate_up || !down || !rows || !d_x_out || bad_dt(dt) || bad_dt(dt_dy) || H < 1 ||
        I < 1 || E < 1 || nrows < 0)
        return -1;
    for (int64_t n = 0; n < nrows; ++n)
        if (expert_of_row(offsets, E, rows[n]) < 0) return -2;
#pragma omp parallel
    {
        double* xr = (double*)malloc(sizeof(double) * (size_t)H);
        double* dyr = (double*)malloc(sizeof(double) * (size_t)H);
        double* g = (double*)malloc(sizeof(double) * (size_t)I);
        double* u = (double*)malloc(sizeof(double) * (size_t)I);
        double* da = (double*)malloc(sizeof(double) * (size_t)I);
        double* dg = (double*)malloc(sizeof(double) * (size_t)I);
        double* du = (double*)malloc(sizeof(double) * (size_t)I);
#pragma omp for schedule(dynamic, 1)
        for (int64_t n = 0; n < nrows; ++n) {
            const int64_t r = rows[n];
            const int64_t e = expert_of_row(offsets, E, r);
            for (int64_t h = 0; h < H; ++h) {
                xr[h] = eld(x_perm, dt, r * H + h);
                dyr[h] = eld(d_y, dt_dy, r * H + h);
            }
            ffn_row_bwd(xr, dyr, dt, gate_up, e * H * 2 * I, down, e * I * H, H, I, g, u, da, dg, du,
                        d_x_out + n * H);
            if (d_gu_out) {
                memcpy(d_gu_out + n * 2 * I, dg, sizeof(double) * (size_t)I);
                memcpy(d_gu_out + n * 2 * I + I, du, sizeof(double) * (size_t)I);
            }
        }
        free(xr);
        free(dyr);
        free(g);
        free(u);
        free(da);
        free(dg);
        free(du);
    }
    return 0;
}

int orc_expert_weight_grads(const void* x_perm, const void* d_y, int dt, int dt_dy, int64_t H, int64_t I,
                            int64_t E, const int32_t* offsets, const void* gate_up,
                            const void* down, int64_t e, double* d_gate_up_e, double* d_down_e) {
    if (!x_perm || !d_y || !offsets || !gate_up || !down || !d_gate_up_e || !d_down_e || bad_dt(dt) || bad_dt(dt_dy) ||
        H < 1 || I < 1 || e < 0 || e >= E)
        return -1;
    const int64_t r0 = offsets[e], r1 = offsets[e + 1];
    const int64_t n = r1 - r0 > 0 ? r1 - r0 : 0;
    /* per-row activations of this expert first (rows are independent) */
    double* A = (double*)calloc((size_t)(n * I + 1), sizeof(double));
    double* DG = (double*)calloc((size_t)(n * 2 * I + 1), sizeof(double));
#pragma omp parallel
    {
        double* xr = (double*)malloc(sizeof(double) * (size_t)H);
        double* dyr = (double*)malloc(sizeof(double) * (size_t)H);
        double* g = (double*)malloc(sizeof(double) * (size_t)I);
        double* u = (double*)malloc(sizeof(double) * (size_t)I);
        double* da = (double*)malloc(sizeof(double) * (size_t)I);
        double* dx = (double*)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(dynamic, 1)
        for (int64_t q = 0; q < n; ++q) {
            const int64_t r = r0 + q;
            for (int64_t h = 0; h < H; ++h) {
                xr[h] = eld(x_perm, dt, r * H + h);
                dyr[h] = eld(d_y, dt_dy, r * H + h);
            }
            ffn_row_bwd(xr, dyr, dt, gate_up, e * H * 2 * I, down, e * I * H, H, I, g, u, da,
                        DG + q * 2 * I, DG + q * 2 * I + I, dx);
            for (int64_t i = 0; i < I; ++i) A[q * I + i] = silu(g[i]) * u[i];
        }
        free(xr);
        free(dyr);
        free(g);
        free(u);
        free(da);
        free(dx);
    }
    /* d_gate_up_e[h, c] = sum over the expert's rows (ascending) of x[r, h] * (dg|du)[r, c] */
#pragma omp parallel for schedule(static)
    for (int64_t h = 0; h < H; ++h) {
        double* o = d_gate_up_e + h * 2 * I;
        for (int64_t c = 0; c < 2 * I; ++c) o[c] = 0.0;
        for (int64_t q = 0; q < n; ++q) {
            const double xh = eld(x_perm, dt, (r0 + q) * H + h);
            for (int64_t c = 0; c < 2 * I; ++c) o[c] += xh * DG[q * 2 * I + c];
        }
    }
    /* d_down_e[i, c] = sum over rows of a[r, i] * d_y[r, c] */
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < I; ++i) {
        double* o = d_down_e + i * H;
        for (int64_t c = 0; c < H; ++c) o[c] = 0.0;
        for (int64_t q = 0; q < n; ++q) {
            const double ai = A[q * I + i];
            for (int64_t c = 0; c < H; ++c) o[c] += ai * eld(d_y, dt_dy, (r0 + q) * H + c);
        }
    }
    free(A);
    free(DG);
    return 0;
}

/* The same weight gradients restricted to a few intermediate units i (columns i and I+i of
 * d_gate_up_e, row i of d_down_e): each unit's entries depend only on that unit's pre-activations,
 * so they can be computed one unit at a time over all rows of the expert. Rows ascending. */
int orc_expert_weight_grads_units(const void* x_perm, const void* d_y, int dt, int dt_dy, int64_t H, int64_t I,
                                  int64_t E, const int32_t* offsets, const void* gate_up,
                                  const void* down, int64_t e, const int64_t* units, int64_t nunits,
                                  double* d_gate_up_cols, double* d_down_rows) {
    if (!x_perm || !d_y || !offsets || !gate_up || !down || !units || !d_gate_up_cols || !d_down_rows ||
        bad_dt(dt) || bad_dt(dt_dy) || H < 1 || I < 1 || e < 0 || e >= E || nunits < 0)
        return -1;
    for (int64_t q = 0; q < nunits; ++q)
        if (units[q] < 0 || units[q] >= I) return -2;
    const int64_t r0 = offsets[e], r1 = offsets[e + 1];
    const int64_t gu_off = e * H * 2 * I, dn_off = e * I * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < nunits; ++q) {
        const int64_t i = units[q];
        double* dgc = d_gate_up_cols + q * 2 * H; /* [H] gate column, then [H] up column */
        double* duc = dgc + H;
        double* ddr = d_down_rows + q * H;
        for (int64_t h = 0; h < H; ++h) dgc[h] = duc[h] = ddr[h] = 0.0;
        for (int64_t r = r0; r < r1; ++r) {
            double g = 0.0, u = 0.0, da = 0.0;
            for (int64_t h = 0; h < H; ++h) {
                const double xh = eld(x_perm, dt, r * H + h);
                g += xh * eld(gate_up, dt, gu_off + h * 2 * I + i);
                u += xh * eld(gate_up, dt, gu_off + h * 2 * I + I + i);
            }
            for (int64_t c = 0; c < H; ++c) da += eld(d_y, dt_dy, r * H + c) * eld(down, dt, dn_off + i * H + c);
            const double sg = sigmoid(g);
            const double dg = da * u * sg * (1.0 + g * (1.0 - sg));
            const double du = da * g * sg;
            const double a = silu(g) * u;
            for (int64_t h = 0; h < H; ++h) {
                const double xh = eld(x_perm, dt, r * H + h);
                dgc[h] += xh * dg;
                duc[h] += xh * du;
                ddr[h] += a * eld(d_y, dt_dy, r * H + h);
            }
        }
    }
    return 0;
}

int orc_permute_bwd(const void* d_x_perm, int dt, int64_t H, int64_t k, const int32_t* row_of_slot,
                    const void* d_x_add, const int64_t* tokens, int64_t ntok, double* d_x) {
    if (!d_x_perm || !row_of_slot || !tokens || !d_x || bad_dt(dt) || H < 1 || k < 1 || ntok < 0) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < ntok; ++n) {
        const int64_t t = tokens[n];
        double* o = d_x + n * H;
        for (int64_t c = 0; c < H; ++c) o[c] = d_x_add ? eld(d_x_add, dt, t * H + c) : 0.0;
        for (int64_t j = 0; j < k; ++j) {
            const int64_t r = row_of_slot[t * k + j];
            if (r < 0) continue; /* a dropped slot was never copied */
            for (int64_t c = 0; c < H; ++c) o[c] += eld(d_x_perm, dt, r * H + c);
        }
    }
    return 0;
}

int orc_router_topk_bwd(const float* logits, const int32_t* topk_idx, const double* d_w,
                        int64_t T, int64_t E, int64_t k, int renorm, double* d_logits) {
    if (!logits || !topk_idx || !d_w || !d_logits || T < 0 || E < 1 || k < 1 || k > E) return -1;
#pragma omp parallel
    {
        double* p = (double*)malloc(sizeof(double) * (size_t)E);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            const float* l = logits + t * E;
            const int32_t* S = topk_idx + t * k;
            double* dl = d_logits + t * E;
            double m = (double)l[S[0]];
            for (int64_t e = 0; e < E; ++e)
                if ((double)l[e] > m) m = (double)l[e];
            double den = 0.0;
            if (renorm) {
                for (int64_t j = 0; j < k; ++j) den += exp((double)l[S[j]] - m);
            } else {
                for (int64_t e = 0; e < E; ++e) den += exp((double)l[e] - m);
            }
            for (int64_t e = 0; e < E; ++e) p[e] = exp((double)l[e] - m) / den;
            double s = 0.0;
            for (int64_t j = 0; j < k; ++j) s += p[S[j]] * d_w[t * k + j];
            if (renorm) {
                for (int64_t e = 0; e < E; ++e) dl[e] = 0.0;
                for (int64_t j = 0; j < k; ++j) dl[S[j]] = p[S[j]] * (d_w[t * k + j] - s);
            } else {
                for (int64_t e = 0; e < E; ++e) dl[e] = -p[e] * s;
                for (int64_t j = 0; j < k; ++j) dl[S[j]] += p[S[j]] * d_w[t * k + j];
            }
        }
        free(p);
    }
    return 0;
}

int orc_router_logits_bwd(const void* x, const void* w_gate, int dt, const double* d_logits,
                          int64_t T, int64_t H, int64_t E, double* d_w_gate, double* d_x) {
    if (!x || !w_gate || !d_logits || bad_dt(dt) || T < 0 || H < 1 || E < 1) return -1;
    if (d_w_gate) {
#pragma omp parallel for schedule(static)
        for (int64_t h = 0; h < H; ++h)
            for (int64_t e = 0; e < E; ++e) {
                double s = 0.0;
                for (int64_t t = 0; t < T; ++t) s += eld(x, dt, t * H + h) * d_logits[t * E + e];
                d_w_gate[h * E + e] = s;
            }
    }
    if (d_x) {
#pragma omp parallel for schedule(static)
        for (int64_t t = 0; t < T; ++t)
            for (int64_t h = 0; h < H; ++h) {
                double s = 0.0;
                for (int64_t e = 0; e < E; ++e) s += d_logits[t * E + e] * eld(w_gate, dt, h * E + e);
                d_x[t * H + h] = s;
            }
    }
    return 0;
}
