/*
 * plx_oracle.c -- plain fp64 CPU oracle for the Parallax attention forward.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path links, loads or calls
 * this file; only the tests, the smoke check and the bench's CPU-baseline leg
 * use it. It shares no code, header or constant with the HIP library.
 *
 * What it computes (per batch b, head h, query i, over the visible keys
 * j = 0 .. n-1; causal prefill: n = i+1; decode: n = clamp(seqlens[b], 0, L_max)):
 *
 *   Central equation [Resumen Tecnico: Parallax - Atencion Lineal Local
 *   Parametrizada, section "Mecanismo Central"]: the output is the softmax
 *   attention output minus the KV covariance applied to the probe,
 *       o_i = o_SA_i - Sigma_KV^(i) rho_i .
 *   The covariance is the softmax-weighted one [Parallax: Parameterized Local
 *   Linear Attention for Language Modeling (agihunt review), method paragraph]:
 *       p_ij = exp(a_ij) / sum_j exp(a_ij),  a_ij = scale * <q_i, k_j>
 *       kbar = sum_j p_ij k_j,  vbar = sum_j p_ij v_j  (= o_SA_i)
 *       Sigma_KV^(i) = sum_j p_ij (v_j - vbar)(k_j - kbar)^T     (d_v x d_qk)
 *   with the boundary amplification factor fixed at zero (same section).
 *
 *   Six-step form [Parallax (paper.rainbus.top summary), section "方法步骤详情"
 *   (method steps)]: w_ij = exp score, omega_i = normaliser, p_ij softmax weight;
 *   t_ij = <rho_i, k_j> probe inner product, tbar_i = sum_j p_ij t_ij;
 *   corrected weight s_ij = p_ij (1 - (t_ij - tbar_i)); outputs
 *   O1 = sum_j p_ij v_j, O2 = sum_j p_ij t_ij v_j; combine o = (1 + tbar) O1 - O2.
 *
 *   Streaming form (same section, last sentences; agihunt review hardware
 *   paragraph): keys are visited block by block with one running max and one
 *   rescale factor shared by both branches; per block S1 = scores, S2 = probe
 *   products, P1 = exp(S1 - m), P2 = P1 * S2, and O1, O2 accumulate together.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   - population weighting (no Bessel factor) for Sigma_KV, centred on both sides;
 *   - the score scale applies to q.k only; t is unscaled;
 *   - causal prefill: key j visible to query i iff j <= i;
 *   - decode: the query sees cache rows [0, seqlens[b]); seqlens <= 0 gives o = 0,
 *     seqlens > L_max is clamped to L_max.
 *
 * Layouts (all row-major, contiguous, fp64):
 *   prefill q, k, rho: [B][H][T][dqk]   v, o: [B][H][T][dv]
 *   decode  q, rho: [B][H][dqk]  k: [B][H][L_max][dqk]  v: [B][H][L_max][dv]
 *           o: [B][H][dv]      seqlens: int32 [B]
 * Return value: 0 on success, -1 on a bad argument or allocation failure.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double dot(const double* x, const double* y, int n) {
    double s = 0.0;
    for (int e = 0; e < n; ++e) s += x[e] * y[e];
    return s;
}

/* Softmax weights p_j over n keys (a_j = scale <q, k_j>). */
static void softmax_weights(const double* q, const double* K, int n, int dqk, double scale,
                            double* p) {
    double m = -INFINITY;
    for (int j = 0; j < n; ++j) {
        p[j] = scale * dot(q, K + (size_t)j * dqk, dqk);
        if (p[j] > m) m = p[j];
    }
    double omega = 0.0;
    for (int j = 0; j < n; ++j) {
        p[j] = exp(p[j] - m);
        omega += p[j];
    }
    for (int j = 0; j < n; ++j) p[j] /= omega;
}

/*
 * F1 -- the definition: o = vbar - Sigma_KV rho with Sigma_KV formed explicitly.
 * scratch: n + dqk + dv + dv*dqk doubles.
 */
static void row_cov(const double* q, const double* rho, const double* K, const double* V,
                    int n, int dqk, int dv, double scale, double* o, double* scratch) {
    if (n <= 0) {
        for (int c = 0; c < dv; ++c) o[c] = 0.0;
        return;
    }
    double* p = scratch;
    double* kbar = p + n;
    double* vbar = kbar + dqk;
    double* sigma = vbar + dv; /* [dv][dqk] */
    softmax_weights(q, K, n, dqk, scale, p);
    for (int e = 0; e < dqk; ++e) kbar[e] = 0.0;
    for (int c = 0; c < dv; ++c) vbar[c] = 0.0;
    for (int j = 0; j < n; ++j) {
        for (int e = 0; e < dqk; ++e) kbar[e] += p[j] * K[(size_t)j * dqk + e];
        for (int c = 0; c < dv; ++c) vbar[c] += p[j] * V[(size_t)j * dv + c];
    }
    memset(sigma, 0, sizeof(double) * (size_t)dv * dqk);
    for (int j = 0; j < n; ++j) {
        const double* kj = K + (size_t)j * dqk;
        const double* vj = V + (size_t)j * dv;
        for (int c = 0; c < dv; ++c) {
            double wv = p[j] * (vj[c] - vbar[c]);
            double* srow = sigma + (size_t)c * dqk;
            for (int e = 0; e < dqk; ++e) srow[e] += wv * (kj[e] - kbar[e]);
        }
    }
    for (int c = 0; c < dv; ++c) o[c] = vbar[c] - dot(sigma + (size_t)c * dqk, rho, dqk);
}

/* F2 -- corrected weights s_j = p_j (1 - (t_j - tbar)), o = sum_j s_j v_j.
 * scratch: 2n doubles. */
static void row_sweighted(const double* q, const double* rho, const double* K,
                          const double* V, int n, int dqk, int dv, double scale, double* o,
                          double* scratch) {
    for (int c = 0; c < dv; ++c) o[c] = 0.0;
    if (n <= 0) return;
    double* p = scratch;
    double* t = p + n;
    softmax_weights(q, K, n, dqk, scale, p);
    double tbar = 0.0;
    for (int j = 0; j < n; ++j) {
        t[j] = dot(rho, K + (size_t)j * dqk, dqk);
        tbar += p[j] * t[j];
    }
    for (int j = 0; j < n; ++j) {
        double s = p[j] * (1.0 - (t[j] - tbar));
        for (int c = 0; c < dv; ++c) o[c] += s * V[(size_t)j * dv + c];
    }
}

/* Running state of the streaming form for keys [j0, j1): max m, normaliser l,
 * beta = sum P2 (un-normalised tbar), O1 and O2 accumulators (un-normalised). */
typedef struct {
    double m, l, beta;
    double* O1;
    double* O2;
} stream_state;

static void state_init(stream_state* st, int dv) {
    st->m = -INFINITY;
    st->l = 0.0;
    st->beta = 0.0;
    for (int c = 0; c < dv; ++c) st->O1[c] = st->O2[c] = 0.0;
}

/* Fold keys [j0, j1) into the state, one block at a time (block >= 1). */
static void state_consume(stream_state* st, const double* q, const double* rho,
                          const double* K, const double* V, int j0, int j1, int block,
                          int dqk, int dv, double scale, double* S1, double* S2) {
    for (int b0 = j0; b0 < j1; b0 += block) {
        int b1 = b0 + block < j1 ? b0 + block : j1;
        int nb = b1 - b0;
        double mb = -INFINITY;
        for (int j = 0; j < nb; ++j) {
            S1[j] = scale * dot(q, K + (size_t)(b0 + j) * dqk, dqk);
            S2[j] = dot(rho, K + (size_t)(b0 + j) * dqk, dqk);
            if (S1[j] > mb) mb = S1[j];
        }
        double mnew = st->m > mb ? st->m : mb;
        double alpha = (st->m == -INFINITY) ? 0.0 : exp(st->m - mnew);
        st->l *= alpha;
        st->beta *= alpha;
        for (int c = 0; c < dv; ++c) {
            st->O1[c] *= alpha;
            st->O2[c] *= alpha;
        }
        for (int j = 0; j < nb; ++j) {
            double P1 = exp(S1[j] - mnew);
            double P2 = P1 * S2[j];
            const double* vj = V + (size_t)(b0 + j) * dv;
            st->l += P1;
            st->beta += P2;
            for (int c = 0; c < dv; ++c) {
                st->O1[c] += P1 * vj[c];
                st->O2[c] += P2 * vj[c];
            }
        }
        st->m = mnew;
    }
}

/* Fold state `src` into `dst` (both over disjoint key sets): one rescale each. */
static void state_merge(stream_state* dst, const stream_state* src, int dv) {
    if (src->m == -INFINITY) return;
    double mnew = dst->m > src->m ? dst->m : src->m;
    double fd = (dst->m == -INFINITY) ? 0.0 : exp(dst->m - mnew);
    double fs = exp(src->m - mnew);
    dst->l = fd * dst->l + fs * src->l;
    dst->beta = fd * dst->beta + fs * src->beta;
    for (int c = 0; c < dv; ++c) {
        dst->O1[c] = fd * dst->O1[c] + fs * src->O1[c];
        dst->O2[c] = fd * dst->O2[c] + fs * src->O2[c];
    }
    dst->m = mnew;
}

/* Step 6: o = (1 + tbar) O1 - O2 with the normalised O1 = O1/l, O2 = O2/l, tbar = beta/l. */
static void state_finish(const stream_state* st, int dv, double* o) {
    if (st->l == 0.0) {
        for (int c = 0; c < dv; ++c) o[c] = 0.0;
        return;
    }
    double tbar = st->beta / st->l;
    for (int c = 0; c < dv; ++c) o[c] = (1.0 + tbar) * (st->O1[c] / st->l) - st->O2[c] / st->l;
}

/* F3 -- streaming over blocks of `block` keys, optionally split into `splits`
 * contiguous chunks whose partial states are merged at the end.
 * scratch: 2*block + 4*dv doubles. */
static void row_stream(const double* q, const double* rho, const double* K, const double* V,
                       int n, int dqk, int dv, double scale, int block, int splits, double* o,
                       double* scratch) {
    double* S1 = scratch;
    double* S2 = S1 + block;
    stream_state acc = {0, 0, 0, S2 + block, S2 + block + dv};
    stream_state part = {0, 0, 0, S2 + block + 2 * dv, S2 + block + 3 * dv};
    state_init(&acc, dv);
    if (n <= 0) {
        state_finish(&acc, dv, o);
        return;
    }
    if (splits < 1) splits = 1;
    int chunk = (n + splits - 1) / splits;
    for (int s = 0; s < splits; ++s) {
        int j0 = s * chunk, j1 = (s + 1) * chunk < n ? (s + 1) * chunk : n;
        if (j0 >= j1) continue;
        state_init(&part, dv);
        state_consume(&part, q, rho, K, V, j0, j1, block, dqk, dv, scale, S1, S2);
        state_merge(&acc, &part, dv);
    }
    state_finish(&acc, dv, o);
}

/* ------------------------------------------------------------------ drivers */

enum { FORM_COV = 0, FORM_SWEIGHTED = 1, FORM_STREAM = 2 };

static size_t scratch_doubles(int form, int n, int dqk, int dv, int block) {
    if (form == FORM_COV) return (size_t)n + dqk + dv + (size_t)dv * dqk;
    if (form == FORM_SWEIGHTED) return 2 * (size_t)n;
    return 2 * (size_t)block + 4 * (size_t)dv;
}

static void run_row(int form, const double* q, const double* rho, const double* K,
                    const double* V, int n, int dqk, int dv, double scale, int block,
                    int splits, double* o, double* scratch) {
    if (form == FORM_COV)
        row_cov(q, rho, K, V, n, dqk, dv, scale, o, scratch);
    else if (form == FORM_SWEIGHTED)
        row_sweighted(q, rho, K, V, n, dqk, dv, scale, o, scratch);
    else
        row_stream(q, rho, K, V, n, dqk, dv, scale, block, splits, o, scratch);
}

/* Causal prefill over a list of rows r = (b*H + h)*T + i (all rows if rows == NULL).
 * Output row k of `o` belongs to the k-th listed row ([nrows][dv]); with rows == NULL
 * `o` is the full [B][H][T][dv] tensor. */
int plx_oracle_prefill(int form, int B, int H, int T, int dqk, int dv, const double* q,
                       const double* k, const double* v, const double* rho, double scale,
                       int block, int splits, const int64_t* rows, int64_t nrows, double* o) {
    if (B < 0 || H < 0 || T < 0 || dqk < 1 || dv < 1 || block < 1 || form < 0 || form > 2)
        return -1;
    int64_t total = rows ? nrows : (int64_t)B * H * T;
    int bad = 0;
#pragma omp parallel
    {
        double* scratch = (double*)malloc(sizeof(double) * scratch_doubles(form, T, dqk, dv, block));
        if (!scratch) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < total; ++r) {
            if (!scratch) continue;
            int64_t row = rows ? rows[r] : r;
            if (row < 0 || row >= (int64_t)B * H * T) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            int64_t bh = row / T;
            int i = (int)(row % T);
            const double* Kb = k + (size_t)bh * T * dqk;
            const double* Vb = v + (size_t)bh * T * dv;
            run_row(form, q + (size_t)row * dqk, rho + (size_t)row * dqk, Kb, Vb, i + 1, dqk, dv,
                    scale, block, splits, o + (size_t)r * dv, scratch);
        }
        free(scratch);
    }
    return bad ? -1 : 0;
}

/* Decode: one query row per (b, h) against cache rows [0, clamp(seqlens[b], 0, L_max)). */
int plx_oracle_decode(int form, int B, int H, int L_max, int dqk, int dv, const double* q,
                      const double* rho, const double* k, const double* v,
                      const int32_t* seqlens, double scale, int block, int splits, double* o) {
    if (B < 0 || H < 0 || L_max < 0 || dqk < 1 || dv < 1 || block < 1 || form < 0 || form > 2)
        return -1;
    int bad = 0;
#pragma omp parallel
    {
        double* scratch =
            (double*)malloc(sizeof(double) * scratch_doubles(form, L_max, dqk, dv, block));
        if (!scratch) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
            if (!scratch) continue;
            int b = (int)(bh / H);
            int n = seqlens[b];
            if (n < 0) n = 0;
            if (n > L_max) n = L_max;
            run_row(form, q + (size_t)bh * dqk, rho + (size_t)bh * dqk,
                    k + (size_t)bh * L_max * dqk, v + (size_t)bh * L_max * dv, n, dqk, dv, scale,
                    block, splits, o + (size_t)bh * dv, scratch);
        }
        free(scratch);
    }
    return bad ? -1 : 0;
}

/* Threads the OpenMP loops above will use (reported next to CPU timings). */
#ifdef _OPENMP
#include <omp.h>
#endif
int plx_oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
