/*
 * Plain fp64 CPU oracle for scaled dot-product attention and its exact gradient.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the package's smoke() check and
 * the CPU-baseline leg of the benchmark may load this library. The product path
 * (the HIP kernels and their C ABI) never calls it, shares no code, header,
 * table or helper with it, and must fail loudly when its own library is missing.
 *
 * What it computes follows "Scheduling Data to Compute: Hierarchical Data
 * Pipelining for LLM Training on AMD GPUs" (Rao et al.), section 2.1, Eq. (1):
 * O = softmax(Q K^T * scale) V, one row of Q at a time, written out naively in
 * double precision with no tiling, no fusion and no reordering. The backward
 * pass is the exact gradient of Eq. (1); the same section's Table 3 lists the
 * two products it contains (dQ = dS K and dK = dS^T Q). Readings of the page
 * where it is silent:
 *   - scale is an argument (the page uses 1/sqrt(d));
 *   - causal: key j is visible to query i iff j <= i (query and key lengths equal);
 *   - sliding window W > 0 (causal only): key j is visible to query i iff
 *     i - W < j <= i, the band of the W most recent keys: the sliding window
 *     every query of the page's compressed sparse attention sees (Table 7,
 *     W = 128; the cr0 kernels of section 3.1.1 attend to it alone);
 *     W = 0 means no window;
 *   - grouped-query attention: query head hq reads key/value head hq / (Hq/Hkv);
 *   - lse_i = m_i + ln(sum_j exp(s_ij - m_i)), natural log; subtracting the row
 *     maximum m_i is an exact rescaling, not an approximation;
 *   - dK and dV of a key/value head are summed over every query head that reads it;
 *   - Eq. (1) gives queries and keys d columns and values d_v: here D and Dv.
 *     V, O, dO and dV have Dv columns, Q, K, dQ and dK have D.
 *
 * Layout: contiguous [B][H][S][D] (Dv for V, O, dO, dV); inputs are bf16 bit
 * patterns (uint16), widened exactly to double; every output is double.
 * All functions return 0 on success and a negative value on bad arguments
 * (-5: a window that is negative, or set without causal).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

typedef struct {
    const uint16_t *q, *k, *v, *dout;
    int B, Hq, Hkv, S, D, Dv, G, causal, window;
    double scale;
} ctx_t;

static double widen(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static int check_args(int B, int Hq, int Hkv, int S, int D, int Dv, int causal, int window) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || S <= 0 || D <= 0 || Dv <= 0) return -1;
    if (Hq % Hkv != 0) return -2;
    if (window < 0 || (window > 0 && !causal)) return -5;
    return 0;
}

/* Element offset of a row: `width` is D for Q, K, dQ, dK and Dv for V, O, dO, dV. */
static size_t qrow_off(const ctx_t* c, int b, int hq, int i, int width) {
    return (((size_t)b * c->Hq + hq) * c->S + i) * (size_t)width;
}
static size_t kvrow_off(const ctx_t* c, int b, int hkv, int j, int width) {
    return (((size_t)b * c->Hkv + hkv) * c->S + j) * (size_t)width;
}

static double dot_bf16(const uint16_t* x, const uint16_t* y, int D) {
    double s = 0.0;
    for (int d = 0; d < D; ++d) s += widen(x[d]) * widen(y[d]);
    return s;
}

/* Query row i sees the keys first_key(i) .. last_key(i); key j is seen by the
 * query rows first_query(j) .. last_query(j). */
static int first_key(const ctx_t* c, int i) {
    return (c->window > 0 && i - c->window + 1 > 0) ? i - c->window + 1 : 0;
}
static int last_key(const ctx_t* c, int i) { return c->causal ? i : c->S - 1; }
static int first_query(const ctx_t* c, int j) { return c->causal ? j : 0; }
static int last_query(const ctx_t* c, int j) {
    return (c->window > 0 && j + c->window - 1 < c->S - 1) ? j + c->window - 1 : c->S - 1;
}

/*
 * One query row of Eq. (1): scores s_j = scale * q_i . k_j over the visible
 * keys, their softmax P_j, and optionally O_i = sum_j P_j v_j and
 * lse_i = m + ln(l). If dout is set, also the row's backward quantities:
 * dP_j = dO_i . v_j, delta_i = sum_j P_j dP_j, dS_j = P_j (dP_j - delta_i),
 * dQ_i = scale * sum_j dS_j k_j.  `p` and `dp` are caller scratch of length S,
 * indexed by key.
 */
static void one_row(const ctx_t* c, int b, int hq, int i, double* p, double* dp,
                    double* o_out, double* lse_out, double* delta_out, double* dq_out) {
    const int D = c->D, Dv = c->Dv, j0 = first_key(c, i), j1 = last_key(c, i), hkv = hq / c->G;
    const uint16_t* qi = c->q + qrow_off(c, b, hq, i, D);
    double m = -INFINITY;
    for (int j = j0; j <= j1; ++j) {
        p[j] = c->scale * dot_bf16(qi, c->k + kvrow_off(c, b, hkv, j, D), D);
        if (p[j] > m) m = p[j];
    }
    double l = 0.0;
    for (int j = j0; j <= j1; ++j) {
        p[j] = exp(p[j] - m);
        l += p[j];
    }
    for (int j = j0; j <= j1; ++j) p[j] /= l;
    if (lse_out) *lse_out = m + log(l);
    if (o_out) {
        for (int d = 0; d < Dv; ++d) o_out[d] = 0.0;
        for (int j = j0; j <= j1; ++j) {
            const uint16_t* vj = c->v + kvrow_off(c, b, hkv, j, Dv);
            for (int d = 0; d < Dv; ++d) o_out[d] += p[j] * widen(vj[d]);
        }
    }
    if (c->dout && (delta_out || dq_out)) {
        const uint16_t* doi = c->dout + qrow_off(c, b, hq, i, Dv);
        double delta = 0.0;
        for (int j = j0; j <= j1; ++j) {
            dp[j] = dot_bf16(doi, c->v + kvrow_off(c, b, hkv, j, Dv), Dv);
            delta += p[j] * dp[j];
        }
        if (delta_out) *delta_out = delta;
        if (dq_out) {
            for (int d = 0; d < D; ++d) dq_out[d] = 0.0;
            for (int j = j0; j <= j1; ++j) {
                const double ds = p[j] * (dp[j] - delta);
                const uint16_t* kj = c->k + kvrow_off(c, b, hkv, j, D);
                for (int d = 0; d < D; ++d) dq_out[d] += c->scale * ds * widen(kj[d]);
            }
        }
    }
}

/*
 * Gradient of one key/value row j of head group (b, hkv): for every query head
 * hq that reads this group and every query row i that sees key j,
 *   P_ij = exp(scale q_i.k_j - lse_i),  dP_ij = dO_i . v_j,
 *   dV_j += P_ij dO_i,   dK_j += scale * P_ij (dP_ij - delta_i) q_i.
 * lse and delta are the per-row values of one_row for the group's query heads,
 * indexed [g][i] with g = hq - hkv*G.
 */
static void one_key(const ctx_t* c, int b, int hkv, int j, const double* lse,
                    const double* delta, double* dk_out, double* dv_out) {
    const int D = c->D, Dv = c->Dv, S = c->S, i0 = first_query(c, j), i1 = last_query(c, j);
    const uint16_t* kj = c->k + kvrow_off(c, b, hkv, j, D);
    const uint16_t* vj = c->v + kvrow_off(c, b, hkv, j, Dv);
    for (int d = 0; d < D; ++d) dk_out[d] = 0.0;
    for (int d = 0; d < Dv; ++d) dv_out[d] = 0.0;
    for (int g = 0; g < c->G; ++g) {
        const int hq = hkv * c->G + g;
        for (int i = i0; i <= i1; ++i) {
            const uint16_t* qi = c->q + qrow_off(c, b, hq, i, D);
            const uint16_t* doi = c->dout + qrow_off(c, b, hq, i, Dv);
            const double pij = exp(c->scale * dot_bf16(qi, kj, D) - lse[(size_t)g * S + i]);
            const double dpij = dot_bf16(doi, vj, Dv);
            const double ds = pij * (dpij - delta[(size_t)g * S + i]);
            for (int d = 0; d < Dv; ++d) dv_out[d] += pij * widen(doi[d]);
            for (int d = 0; d < D; ++d) dk_out[d] += c->scale * ds * widen(qi[d]);
        }
    }
}

static void init_ctx(ctx_t* c, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                     const uint16_t* dout, int B, int Hq, int Hkv, int S, int D, int Dv,
                     int causal, int window, double scale) {
    c->q = q; c->k = k; c->v = v; c->dout = dout;
    c->B = B; c->Hq = Hq; c->Hkv = Hkv; c->S = S; c->D = D; c->Dv = Dv; c->G = Hq / Hkv;
    c->causal = causal ? 1 : 0;
    c->window = window;
    c->scale = scale;
}

int oracle_num_threads(void) { return omp_get_max_threads(); }

/* Forward over every row: o [B][Hq][S][Dv], lse [B][Hq][S]. */
int oracle_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, double* o,
                    double* lse, int B, int Hq, int Hkv, int S, int D, int Dv, int causal,
                    int window, double scale) {
    int rc = check_args(B, Hq, Hkv, S, D, Dv, causal, window);
    if (rc) return rc;
    ctx_t c;
    init_ctx(&c, q, k, v, NULL, B, Hq, Hkv, S, D, Dv, causal, window, scale);
    const long long rows = (long long)B * Hq * S;
#pragma omp parallel
    {
        double* p = (double*)malloc(sizeof(double) * (size_t)S);
#pragma omp for schedule(dynamic, 16)
        for (long long r = 0; r < rows; ++r) {
            const int i = (int)(r % S), bh = (int)(r / S);
            one_row(&c, bh / Hq, bh % Hq, i, p, NULL, o + (size_t)r * Dv, lse + r, NULL, NULL);
        }
        free(p);
    }
    return 0;
}

/* Forward for selected rows only; rows[n] are flat indices (b*Hq + hq)*S + i.
 * o_rows [n][Dv], lse_rows [n]. */
int oracle_attn_fwd_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const int64_t* rows, int64_t n, double* o_rows, double* lse_rows,
                         int B, int Hq, int Hkv, int S, int D, int Dv, int causal, int window,
                         double scale) {
    int rc = check_args(B, Hq, Hkv, S, D, Dv, causal, window);
    if (rc) return rc;
    for (int64_t t = 0; t < n; ++t)
        if (rows[t] < 0 || rows[t] >= (int64_t)B * Hq * S) return -3;
    ctx_t c;
    init_ctx(&c, q, k, v, NULL, B, Hq, Hkv, S, D, Dv, causal, window, scale);
#pragma omp parallel
    {
        double* p = (double*)malloc(sizeof(double) * (size_t)S);
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < n; ++t) {
            const int64_t r = rows[t];
            const int i = (int)(r % S), bh = (int)(r / S);
            one_row(&c, bh / Hq, bh % Hq, i, p, NULL, o_rows + (size_t)t * Dv, lse_rows + t,
                    NULL, NULL);
        }
        free(p);
    }
    return 0;
}

/* Per-row lse and delta for every query head of group (b, hkv): [G][S] each. */
static void group_row_stats(const ctx_t* c, int b, int hkv, double* lse, double* delta) {
    const int S = c->S, G = c->G;
#pragma omp parallel
    {
        double* p = (double*)malloc(sizeof(double) * (size_t)S);
        double* dp = (double*)malloc(sizeof(double) * (size_t)S);
#pragma omp for schedule(dynamic, 8)
        for (long long r = 0; r < (long long)G * S; ++r) {
            const int g = (int)(r / S), i = (int)(r % S);
            one_row(c, b, hkv * G + g, i, p, dp, NULL, lse + r, delta + r, NULL);
        }
        free(p);
        free(dp);
    }
}

/* Full backward: dq [B][Hq][S][D]; dk [B][Hkv][S][D], dv [B][Hkv][S][Dv] (summed over the group). */
int oracle_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    const uint16_t* dout, double* dq, double* dk, double* dv, int B, int Hq,
                    int Hkv, int S, int D, int Dv, int causal, int window, double scale) {
    int rc = check_args(B, Hq, Hkv, S, D, Dv, causal, window);
    if (rc) return rc;
    ctx_t c;
    init_ctx(&c, q, k, v, dout, B, Hq, Hkv, S, D, Dv, causal, window, scale);
    const int G = c.G;
    const long long rows = (long long)B * Hq * S;
    double* lse = (double*)malloc(sizeof(double) * (size_t)rows);
    double* delta = (double*)malloc(sizeof(double) * (size_t)rows);
    if (!lse || !delta) { free(lse); free(delta); return -4; }
#pragma omp parallel
    {
        double* p = (double*)malloc(sizeof(double) * (size_t)S);
        double* dp = (double*)malloc(sizeof(double) * (size_t)S);
#pragma omp for schedule(dynamic, 16)
        for (long long r = 0; r < rows; ++r) {
            const int i = (int)(r % S), bh = (int)(r / S);
            one_row(&c, bh / Hq, bh % Hq, i, p, dp, NULL, lse + r, delta + r,
                    dq + (size_t)r * D);
        }
        free(p);
        free(dp);
    }
    const long long keys = (long long)B * Hkv * S;
#pragma omp parallel for schedule(dynamic, 16)
    for (long long r = 0; r < keys; ++r) {
        const int j = (int)(r % S), bh = (int)(r / S);
        const int b = bh / Hkv, hkv = bh % Hkv;
        /* the group's query heads are hkv*G .. hkv*G+G-1, contiguous in [Hq] */
        const size_t base = ((size_t)b * Hq + (size_t)hkv * G) * S;
        one_key(&c, b, hkv, j, lse + base, delta + base, dk + (size_t)r * D, dv + (size_t)r * Dv);
    }
    free(lse);
    free(delta);
    return 0;
}

/*
 * Backward for selected rows only. qrows[nq]: flat query rows (b*Hq+hq)*S+i,
 * giving dq_rows [nq][D]. kvrows[nkv]: flat key rows (b*Hkv+hkv)*S+j, giving
 * dk_rows [nkv][D] and dv_rows [nkv][Dv]. Every query row of each group that a selected key
 * belongs to is visited once for its lse and delta.
 */
int oracle_attn_bwd_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const uint16_t* dout, const int64_t* qrows, int64_t nq, double* dq_rows,
                         const int64_t* kvrows, int64_t nkv, double* dk_rows, double* dv_rows,
                         int B, int Hq, int Hkv, int S, int D, int Dv, int causal, int window,
                         double scale) {
    int rc = check_args(B, Hq, Hkv, S, D, Dv, causal, window);
    if (rc) return rc;
    for (int64_t t = 0; t < nq; ++t)
        if (qrows[t] < 0 || qrows[t] >= (int64_t)B * Hq * S) return -3;
    for (int64_t t = 0; t < nkv; ++t)
        if (kvrows[t] < 0 || kvrows[t] >= (int64_t)B * Hkv * S) return -3;
    ctx_t c;
    init_ctx(&c, q, k, v, dout, B, Hq, Hkv, S, D, Dv, causal, window, scale);
    const int G = c.G;
#pragma omp parallel
    {
        double* p = (double*)malloc(sizeof(double) * (size_t)S);
        double* dp = (double*)malloc(sizeof(double) * (size_t)S);
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < nq; ++t) {
            const int64_t r = qrows[t];
            const int i = (int)(r % S), bh = (int)(r / S);
            one_row(&c, bh / Hq, bh % Hq, i, p, dp, NULL, NULL, NULL, dq_rows + (size_t)t * D);
        }
        free(p);
        free(dp);
    }
    if (nkv == 0) return 0;
    double* lse = (double*)malloc(sizeof(double) * (size_t)G * S);
    double* delta = (double*)malloc(sizeof(double) * (size_t)G * S);
    if (!lse || !delta) { free(lse); free(delta); return -4; }
    /* visit groups in the order they first appear; recompute stats per group */
    int64_t done_group = -1;
    for (int64_t t = 0; t < nkv; ++t) {
        const int64_t grp = kvrows[t] / S;
        if (grp == done_group) continue;
        const int b = (int)(grp / Hkv), hkv = (int)(grp % Hkv);
        group_row_stats(&c, b, hkv, lse, delta);
        done_group = grp;
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t u = t; u < nkv; ++u) {
            if (kvrows[u] / S != grp) continue;
            one_key(&c, b, hkv, (int)(kvrows[u] % S), lse, delta, dk_rows + (size_t)u * D,
                    dv_rows + (size_t)u * Dv);
        }
    }
    free(lse);
    free(delta);
    return 0;
}

/* ------------------------------------------------------------------------------
 * Sparse attention over per-token index lists.
 *
 * The page's compressed sparse attention (section 2.1; Table 7 for its shapes)
 * gives every query token a top-k list of key/value row indices: a sliding
 * window of recent tokens plus rows of a compressed pool. The forward gathers
 * the listed rows, scores them and streams their values into the output; the
 * backward gathers the same rows for dQ, forms one dK/dV contribution per
 * (token, list slot) and reduces those by the inverse of the index map.
 * Readings of the page where it is silent:
 *   - idx is [B][S][topk] int32, shared by every query head of a token; entry s
 *     of token i names row idx[b][i][s] of the N key/value rows of each K/V head
 *     (k, v: [B][Hkv][N][D]); an entry outside [0, N) is an empty slot;
 *   - attention runs over slots: Eq. (1) with the scores of token i's non-empty
 *     slots, so a row listed twice counts twice; the lists carry any causal or
 *     window structure, nothing else masks;
 *   - a token with no non-empty slot gets O = 0, lse = -inf, dQ = 0 and adds
 *     nothing to dK/dV;
 *   - query heads map to K/V heads as in the dense functions (hq / (Hq/Hkv)).
 * -------------------------------------------------------------------------- */
typedef struct {
    const uint16_t *q, *k, *v, *dout;
    const int32_t* idx;
    int B, Hq, Hkv, S, N, D, G, topk;
    double scale;
} sctx_t;

static int check_sparse(int B, int Hq, int Hkv, int S, int N, int D, int topk) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || S <= 0 || N <= 0 || D <= 0 || topk <= 0) return -1;
    if (Hq % Hkv != 0) return -2;
    return 0;
}

/* Key/value row of slot s of token i, or -1 for an empty slot. */
static int slot_row(const sctx_t* c, int b, int i, int s) {
    const int32_t j = c->idx[((size_t)b * c->S + i) * c->topk + s];
    return (j >= 0 && j < c->N) ? (int)j : -1;
}

static const uint16_t* sq_row(const sctx_t* c, const uint16_t* base, int b, int hq, int i) {
    return base + (((size_t)b * c->Hq + hq) * c->S + i) * (size_t)c->D;
}
static const uint16_t* skv_row(const sctx_t* c, const uint16_t* base, int b, int hkv, int j) {
    return base + (((size_t)b * c->Hkv + hkv) * c->N + j) * (size_t)c->D;
}

/*
 * One query row over its token's slots: p[s] = softmax_s(scale q_i . k_idx[s]) on
 * non-empty slots (0 on empty ones), optionally O_i, lse_i, and with dout the
 * backward quantities dP_s = dO_i . v_idx[s], delta_i = sum_s p_s dP_s and
 * dQ_i = scale sum_s p_s (dP_s - delta_i) k_idx[s]. p and dp: caller scratch of
 * length topk. Returns the number of non-empty slots.
 */
static int sparse_row(const sctx_t* c, int b, int hq, int i, double* p, double* dp, double* o_out,
                      double* lse_out, double* delta_out, double* dq_out) {
    const int D = c->D, hkv = hq / c->G;
    const uint16_t* qi = sq_row(c, c->q, b, hq, i);
    double m = -INFINITY;
    int n = 0;
    for (int s = 0; s < c->topk; ++s) {
        const int j = slot_row(c, b, i, s);
        if (j < 0) { p[s] = 0.0; continue; }
        p[s] = c->scale * dot_bf16(qi, skv_row(c, c->k, b, hkv, j), D);
        if (p[s] > m) m = p[s];
        ++n;
    }
    if (o_out) for (int d = 0; d < D; ++d) o_out[d] = 0.0;
    if (dq_out) for (int d = 0; d < D; ++d) dq_out[d] = 0.0;
    if (n == 0) {
        if (lse_out) *lse_out = -INFINITY;
        if (delta_out) *delta_out = 0.0;
        return 0;
    }
    double l = 0.0;
    for (int s = 0; s < c->topk; ++s) {
        if (slot_row(c, b, i, s) < 0) continue;
        p[s] = exp(p[s] - m);
        l += p[s];
    }
    for (int s = 0; s < c->topk; ++s)
        if (slot_row(c, b, i, s) >= 0) p[s] /= l;
    if (lse_out) *lse_out = m + log(l);
    if (o_out) {
        for (int s = 0; s < c->topk; ++s) {
            const int j = slot_row(c, b, i, s);
            if (j < 0) continue;
            const uint16_t* vj = skv_row(c, c->v, b, hkv, j);
            for (int d = 0; d < D; ++d) o_out[d] += p[s] * widen(vj[d]);
        }
    }
    if (c->dout && (delta_out || dq_out)) {
        const uint16_t* doi = sq_row(c, c->dout, b, hq, i);
        double delta = 0.0;
        for (int s = 0; s < c->topk; ++s) {
            const int j = slot_row(c, b, i, s);
            if (j < 0) { dp[s] = 0.0; continue; }
            dp[s] = dot_bf16(doi, skv_row(c, c->v, b, hkv, j), D);
            delta += p[s] * dp[s];
        }
        if (delta_out) *delta_out = delta;
        if (dq_out) {
            for (int s = 0; s < c->topk; ++s) {
                const int j = slot_row(c, b, i, s);
                if (j < 0) continue;
                const double ds = p[s] * (dp[s] - delta);
                const uint16_t* kj = skv_row(c, c->k, b, hkv, j);
                for (int d = 0; d < D; ++d) dq_out[d] += c->scale * ds * widen(kj[d]);
            }
        }
    }
    return n;
}

static void init_sctx(sctx_t* c, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const uint16_t* dout, const int32_t* idx, int B, int Hq, int Hkv, int S,
                      int N, int D, int topk, double scale) {
    c->q = q; c->k = k; c->v = v; c->dout = dout; c->idx = idx;
    c->B = B; c->Hq = Hq; c->Hkv = Hkv; c->S = S; c->N = N; c->D = D; c->G = Hq / Hkv;
    c->topk = topk;
    c->scale = scale;
}

/* Sparse forward for the flat query rows rows[0..n) ((b*Hq + hq)*S + i), or for
 * every row when rows is NULL: o [n][D] (or [B][Hq][S][D]), lse [n]. */
int oracle_sparse_fwd_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const int32_t* idx, const int64_t* rows, int64_t n, double* o,
                           double* lse, int B, int Hq, int Hkv, int S, int N, int D, int topk,
                           double scale) {
    int rc = check_sparse(B, Hq, Hkv, S, N, D, topk);
    if (rc) return rc;
    if (!rows) n = (int64_t)B * Hq * S;
    for (int64_t t = 0; rows && t < n; ++t)
        if (rows[t] < 0 || rows[t] >= (int64_t)B * Hq * S) return -3;
    sctx_t c;
    init_sctx(&c, q, k, v, NULL, idx, B, Hq, Hkv, S, N, D, topk, scale);
#pragma omp parallel
    {
        double* p = (double*)malloc(sizeof(double) * (size_t)topk);
#pragma omp for schedule(dynamic, 16)
        for (int64_t t = 0; t < n; ++t) {
            const int64_t r = rows ? rows[t] : t;
            const int i = (int)(r % S), bh = (int)(r / S);
            sparse_row(&c, bh / Hq, bh % Hq, i, p, NULL, o + (size_t)t * D, lse + t, NULL, NULL);
        }
        free(p);
    }
    return 0;
}

/* Per-row lse and delta of every query row: [B][Hq][S] each. */
static void sparse_row_stats(const sctx_t* c, double* lse, double* delta) {
    const long long rows = (long long)c->B * c->Hq * c->S;
#pragma omp parallel
    {
        double* p = (double*)malloc(sizeof(double) * (size_t)c->topk);
        double* dp = (double*)malloc(sizeof(double) * (size_t)c->topk);
#pragma omp for schedule(dynamic, 16)
        for (long long r = 0; r < rows; ++r) {
            const int i = (int)(r % c->S), bh = (int)(r / c->S);
            sparse_row(c, bh / c->Hq, bh % c->Hq, i, p, dp, NULL, lse + r, delta + r, NULL);
        }
        free(p);
        free(dp);
    }
}

/*
 * dK and dV of key/value row j of head group (b, hkv): the contributions of every
 * (token i, slot s) whose entry names row j, taken in token order through the
 * inverse of the index map (ent[0..ne): flat i*topk + s of batch b), each summed
 * over the group's query heads:
 *   P = exp(scale q.k_j - lse),  dV_j += P dO,  dK_j += scale P (dO.v_j - delta) q.
 */
static void sparse_key(const sctx_t* c, int b, int hkv, int j, const int64_t* ent, int64_t ne,
                       const double* lse, const double* delta, double* dk_out, double* dv_out) {
    const int D = c->D, S = c->S;
    const uint16_t* kj = skv_row(c, c->k, b, hkv, j);
    const uint16_t* vj = skv_row(c, c->v, b, hkv, j);
    for (int d = 0; d < D; ++d) { dk_out[d] = 0.0; dv_out[d] = 0.0; }
    for (int64_t e = 0; e < ne; ++e) {
        const int i = (int)(ent[e] / c->topk);
        for (int g = 0; g < c->G; ++g) {
            const int hq = hkv * c->G + g;
            const size_t r = ((size_t)b * c->Hq + hq) * S + i;
            const uint16_t* qi = sq_row(c, c->q, b, hq, i);
            const uint16_t* doi = sq_row(c, c->dout, b, hq, i);
            const double pij = exp(c->scale * dot_bf16(qi, kj, D) - lse[r]);
            const double ds = pij * (dot_bf16(doi, vj, D) - delta[r]);
            for (int d = 0; d < D; ++d) {
                dv_out[d] += pij * widen(doi[d]);
                dk_out[d] += c->scale * ds * widen(qi[d]);
            }
        }
    }
}

/* Inverse of batch b's index map: for each row j, the entries naming it, in
 * increasing flat order i*topk + s. start [N+1], ent [count of non-empty slots]. */
static int64_t* invert_map(const sctx_t* c, int b, int64_t* start) {
    const int N = c->N;
    for (int j = 0; j <= N; ++j) start[j] = 0;
    for (int64_t e = 0; e < (int64_t)c->S * c->topk; ++e) {
        const int j = slot_row(c, b, (int)(e / c->topk), (int)(e % c->topk));
        if (j >= 0) start[j + 1]++;
    }
    for (int j = 0; j < N; ++j) start[j + 1] += start[j];
    int64_t* ent = (int64_t*)malloc(sizeof(int64_t) * (size_t)(start[N] > 0 ? start[N] : 1));
    int64_t* fill = (int64_t*)malloc(sizeof(int64_t) * (size_t)N);
    if (!ent || !fill) { free(ent); free(fill); return NULL; }
    for (int j = 0; j < N; ++j) fill[j] = start[j];
    for (int64_t e = 0; e < (int64_t)c->S * c->topk; ++e) {
        const int j = slot_row(c, b, (int)(e / c->topk), (int)(e % c->topk));
        if (j >= 0) ent[fill[j]++] = e;
    }
    free(fill);
    return ent;
}

/*
 * Sparse backward. dq_rows gets dQ of the flat query rows qrows[0..nq) (every
 * row, [B][Hq][S][D], when qrows is NULL); dk_rows, dv_rows get dK, dV of the flat
 * key/value rows kvrows[0..nkv) ((b*Hkv + hkv)*N + j; every row, [B][Hkv][N][D],
 * when kvrows is NULL). Every query row's lse and delta are computed first.
 */
int oracle_sparse_bwd_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const uint16_t* dout, const int32_t* idx, const int64_t* qrows,
                           int64_t nq, double* dq_rows, const int64_t* kvrows, int64_t nkv,
                           double* dk_rows, double* dv_rows, int B, int Hq, int Hkv, int S,
                           int N, int D, int topk, double scale) {
    int rc = check_sparse(B, Hq, Hkv, S, N, D, topk);
    if (rc) return rc;
    if (!qrows) nq = (int64_t)B * Hq * S;
    if (!kvrows) nkv = (int64_t)B * Hkv * N;
    for (int64_t t = 0; qrows && t < nq; ++t)
        if (qrows[t] < 0 || qrows[t] >= (int64_t)B * Hq * S) return -3;
    for (int64_t t = 0; kvrows && t < nkv; ++t)
        if (kvrows[t] < 0 || kvrows[t] >= (int64_t)B * Hkv * N) return -3;
    sctx_t c;
    init_sctx(&c, q, k, v, dout, idx, B, Hq, Hkv, S, N, D, topk, scale);
#pragma omp parallel
    {
        double* p = (double*)malloc(sizeof(double) * (size_t)topk);
        double* dp = (double*)malloc(sizeof(double) * (size_t)topk);
#pragma omp for schedule(dynamic, 16)
        for (int64_t t = 0; t < nq; ++t) {
            const int64_t r = qrows ? qrows[t] : t;
            const int i = (int)(r % S), bh = (int)(r / S);
            sparse_row(&c, bh / Hq, bh % Hq, i, p, dp, NULL, NULL, NULL, dq_rows + (size_t)t * D);
        }
        free(p);
        free(dp);
    }
    if (nkv == 0) return 0;
    const size_t nrows = (size_t)B * Hq * S;
    double* lse = (double*)malloc(sizeof(double) * nrows);
    double* delta = (double*)malloc(sizeof(double) * nrows);
    int64_t* start = (int64_t*)malloc(sizeof(int64_t) * ((size_t)N + 1));
    if (!lse || !delta || !start) { free(lse); free(delta); free(start); return -4; }
    sparse_row_stats(&c, lse, delta);
    for (int b = 0; b < B; ++b) {
        int64_t* ent = invert_map(&c, b, start);
        if (!ent) { free(lse); free(delta); free(start); return -4; }
#pragma omp parallel for schedule(dynamic, 4)
        for (int64_t t = 0; t < nkv; ++t) {
            const int64_t r = kvrows ? kvrows[t] : t;
            const int j = (int)(r % N), bh = (int)(r / N);
            if (bh / Hkv != b) continue;
            sparse_key(&c, b, bh % Hkv, j, ent + start[j], start[j + 1] - start[j], lse, delta,
                       dk_rows + (size_t)t * D, dv_rows + (size_t)t * D);
        }
        free(ent);
    }
    free(lse);
    free(delta);
    free(start);
    return 0;
}
