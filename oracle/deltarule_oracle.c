/*
 * deltarule_oracle.c -- fp64 CPU oracle for the gated delta-rule recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product: only
 * the test suite and the smoke check load it.  It shares no code, header,
 * table or helper with the HIP library.
 *
 * What it computes (one (b,h) head at a time, all arithmetic in double; row
 * vectors q_t, k_t in R^{d_k}, v_t in R^{d_v}, a d_k x d_v state):
 *
 *   forward   S_0 = S_in
 *             S_t = a_t (I - beta_t k_t^T k_t) S_{t-1} + beta_t k_t^T v_t
 *             o_t = q_t S_t,   S_out = S_T
 *
 * written as the delta update it is: with the decayed state read at the key,
 *             u_t = beta_t (v_t - a_t k_t S_{t-1})
 *             S_t = a_t S_{t-1} + k_t^T u_t.
 *
 * Source.  StateFlow trains Gated DeltaNet models (the gptget summary,
 * "Experimental design"); the pages name the model but do not write its
 * recurrence.  This is the gated delta rule in the d_k x d_v orientation of
 * the linear recurrence S_t = a_t S_{t-1} + k_t^T v_t that the rest of the
 * layer uses: the erase term (I - beta k^T k) acts on the key dimension, so
 * that reading the new state at the written key gives back v_t when
 * |k_t| = 1 and beta_t = 1.
 *
 * Backward, hand-derived, for L = sum_t <dO_t, o_t> + <dS_out, S_T>, with
 * G_t the gradient of L with respect to S_t (it includes q_t^T dO_t):
 *   G_T     = dS_out + q_T^T dO_T
 *   du_t    = k_t G_t
 *   dv_t    = beta_t du_t
 *   dk_t    = u_t G_t^T - a_t beta_t du_t S_{t-1}^T
 *   dbeta_t = < du_t, v_t - a_t k_t S_{t-1} >
 *   da_t    = < G_t, S_{t-1} > - beta_t < du_t, k_t S_{t-1} >
 *   G_{t-1} = a_t (G_t - beta_t k_t^T du_t) + q_{t-1}^T dO_{t-1}
 *   dq_t    = dO_t S_t^T,   dS_in = a_1 (G_1 - beta_1 k_1^T du_1)
 * The reverse sweep needs S_{t-1}; the transition is not invertible (with
 * beta |k|^2 = 1 it is a projection), so S is checkpointed every CK tokens
 * in the forward sweep and each block is re-run before it is walked back.
 *
 * Layouts: activations [B,H,T,d] with element strides (sb, sh, st), feature
 * index contiguous.  beta is read as beta[b*bb + h*bh + t*bt]; the decay as
 * a[b*ab + h*ah + t*at] (at = 0: per head; a == NULL: a_t = 1).  States are
 * contiguous [B,H,d_k,d_v].  NULL S_in / dS_out mean zeros; NULL outputs
 * are skipped.  Parallel over (b,h) with OpenMP; each head's arithmetic
 * order is fixed, so the result does not depend on the thread count or on
 * how the sequence is split.
 *
 * Return value: 0 on success, -1 on a bad argument or allocation failure.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define CK 64

typedef struct {
    int64_t sb, sh, st;
} dstride;

static inline const double* row(const double* base, dstride s, int b, int h, int64_t t)
{
    return base + b * s.sb + h * s.sh + t * s.st;
}

static inline double scal(const double* p, int64_t sb, int64_t sh, int64_t st, int b, int h,
                          int64_t t, double dflt)
{
    return p ? p[b * sb + h * sh + t * st] : dflt;
}

/* One step: S <- a S + k^T u with u = beta (v - a k S).  u (d_v) is returned. */
static void step(double* S, int dk, int dv, const double* k, const double* v, double a,
                 double beta, double* u)
{
    for (int j = 0; j < dv; ++j) {
        double ks = 0.0;
        for (int i = 0; i < dk; ++i)
            ks += k[i] * S[(int64_t)i * dv + j];
        u[j] = beta * (v[j] - a * ks);
    }
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            S[(int64_t)i * dv + j] = a * S[(int64_t)i * dv + j] + k[i] * u[j];
}

int delta_fwd(int B, int H, int64_t T, int dk, int dv,
              const double* q, int64_t qsb, int64_t qsh, int64_t qst,
              const double* k, int64_t ksb, int64_t ksh, int64_t kst,
              const double* v, int64_t vsb, int64_t vsh, int64_t vst,
              const double* beta, int64_t bsb, int64_t bsh, int64_t bst,
              const double* a, int64_t ab, int64_t ah, int64_t at,
              const double* S_in, double* o, int64_t osb, int64_t osh, int64_t ost,
              double* S_out, int nthreads)
{
    if (B < 0 || H < 0 || T < 0 || dk <= 0 || dv <= 0 || !k || !v || !beta || (o && !q))
        return -1;
    const dstride qs = {qsb, qsh, qst}, ks = {ksb, ksh, kst}, vs = {vsb, vsh, vst},
                  os = {osb, osh, ost};
    const int64_t sd = (int64_t)dk * dv;
    int rc = 0;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
    {
        double* S = (double*)malloc((size_t)(sd + dv) * sizeof(double));
        if (!S) {
#pragma omp atomic write
            rc = -1;
        } else {
            double* u = S + sd;
#pragma omp for schedule(dynamic, 1)
            for (int bh = 0; bh < B * H; ++bh) {
                const int b = bh / H, h = bh % H;
                if (S_in)
                    memcpy(S, S_in + (int64_t)bh * sd, (size_t)sd * sizeof(double));
                else
                    memset(S, 0, (size_t)sd * sizeof(double));
                for (int64_t t = 0; t < T; ++t) {
                    step(S, dk, dv, row(k, ks, b, h, t), row(v, vs, b, h, t),
                         scal(a, ab, ah, at, b, h, t, 1.0), scal(beta, bsb, bsh, bst, b, h, t, 0.0),
                         u);
                    if (o) {
                        const double* qt = row(q, qs, b, h, t);
                        double* ot = o + b * os.sb + h * os.sh + t * os.st;
                        for (int j = 0; j < dv; ++j) {
                            double acc = 0.0;
                            for (int i = 0; i < dk; ++i)
                                acc += qt[i] * S[(int64_t)i * dv + j];
                            ot[j] = acc;
                        }
                    }
                }
                if (S_out)
                    memcpy(S_out + (int64_t)bh * sd, S, (size_t)sd * sizeof(double));
            }
            free(S);
        }
    }
    return rc;
}

/* Backward for one head; scratch holds (T/CK + CK + 1) states, G and 3 rows. */
static void delta_bwd_head(int b, int h, int64_t T, int dk, int dv,
                           const double* q, dstride qs, const double* k, dstride ks,
                           const double* v, dstride vs,
                           const double* beta, int64_t bsb, int64_t bsh, int64_t bst,
                           const double* a, int64_t ab, int64_t ah, int64_t at,
                           const double* S_in, const double* dO, dstride dos,
                           const double* dS_out,
                           double* dq, dstride dqs, double* dk_, dstride dks,
                           double* dv_, dstride dvs, double* dS_in,
                           double* dbeta, int64_t dbb, int64_t dbh, int64_t dbt,
                           double* da, int64_t dab, int64_t dah, int64_t dat,
                           double* ckpt, double* blk, double* G, double* u, double* du,
                           double* kS)
{
    const int64_t sd = (int64_t)dk * dv;
    const int64_t nck = (T + CK - 1) / CK;
    /* forward sweep: checkpoints (state before token c*CK) and dq_t = dO_t S_t^T */
    double* S = blk; /* a running state; blk is reused by the reverse sweep */
    if (S_in)
        memcpy(S, S_in, (size_t)sd * sizeof(double));
    else
        memset(S, 0, (size_t)sd * sizeof(double));
    for (int64_t t = 0; t < T; ++t) {
        if (t % CK == 0)
            memcpy(ckpt + (t / CK) * sd, S, (size_t)sd * sizeof(double));
        step(S, dk, dv, row(k, ks, b, h, t), row(v, vs, b, h, t),
             scal(a, ab, ah, at, b, h, t, 1.0), scal(beta, bsb, bsh, bst, b, h, t, 0.0), u);
        if (dq) {
            double* dqt = dq + b * dqs.sb + h * dqs.sh + t * dqs.st;
            const double* dOt = dO ? row(dO, dos, b, h, t) : NULL;
            for (int i = 0; i < dk; ++i) {
                double acc = 0.0;
                if (dOt)
                    for (int j = 0; j < dv; ++j)
                        acc += dOt[j] * S[(int64_t)i * dv + j];
                dqt[i] = acc;
            }
        }
    }
    /* reverse sweep */
    if (dS_out)
        memcpy(G, dS_out, (size_t)sd * sizeof(double));
    else
        memset(G, 0, (size_t)sd * sizeof(double));
    for (int64_t c = nck - 1; c >= 0; --c) {
        const int64_t t0 = c * CK, t1 = (t0 + CK < T) ? t0 + CK : T;
        /* blk + (t - t0) * sd = S_{t-1} for t in [t0, t1) */
        memcpy(blk, ckpt + c * sd, (size_t)sd * sizeof(double));
        for (int64_t t = t0; t + 1 < t1; ++t) {
            memcpy(blk + (t - t0 + 1) * sd, blk + (t - t0) * sd, (size_t)sd * sizeof(double));
            step(blk + (t - t0 + 1) * sd, dk, dv, row(k, ks, b, h, t), row(v, vs, b, h, t),
                 scal(a, ab, ah, at, b, h, t, 1.0), scal(beta, bsb, bsh, bst, b, h, t, 0.0), u);
        }
        for (int64_t t = t1 - 1; t >= t0; --t) {
            const double* Sp = blk + (t - t0) * sd;      /* S_{t-1} */
            const double* qt = row(q, qs, b, h, t);
            const double* kt = row(k, ks, b, h, t);
            const double* vt = row(v, vs, b, h, t);
            const double at_ = scal(a, ab, ah, at, b, h, t, 1.0);
            const double bt_ = scal(beta, bsb, bsh, bst, b, h, t, 0.0);
            /* G_t gains q_t^T dO_t */
            if (dO) {
                const double* dOt = row(dO, dos, b, h, t);
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j)
                        G[(int64_t)i * dv + j] += qt[i] * dOt[j];
            }
            /* kS = k_t S_{t-1}, u = beta (v - a kS), du = k_t G_t */
            for (int j = 0; j < dv; ++j) {
                double s1 = 0.0, s2 = 0.0;
                for (int i = 0; i < dk; ++i) {
                    s1 += kt[i] * Sp[(int64_t)i * dv + j];
                    s2 += kt[i] * G[(int64_t)i * dv + j];
                }
                kS[j] = s1;
                u[j] = bt_ * (vt[j] - at_ * s1);
                du[j] = s2;
            }
            if (dv_) {
                double* dvt = dv_ + b * dvs.sb + h * dvs.sh + t * dvs.st;
                for (int j = 0; j < dv; ++j)
                    dvt[j] = bt_ * du[j];
            }
            if (dk_) {
                double* dkt = dk_ + b * dks.sb + h * dks.sh + t * dks.st;
                for (int i = 0; i < dk; ++i) {
                    double s1 = 0.0, s2 = 0.0;
                    for (int j = 0; j < dv; ++j) {
                        s1 += u[j] * G[(int64_t)i * dv + j];
                        s2 += du[j] * Sp[(int64_t)i * dv + j];
                    }
                    dkt[i] = s1 - at_ * bt_ * s2;
                }
            }
            if (dbeta) {
                double acc = 0.0;
                for (int j = 0; j < dv; ++j)
                    acc += du[j] * (vt[j] - at_ * kS[j]);
                dbeta[b * dbb + h * dbh + t * dbt] = acc;
            }
            if (da) {
                double g1 = 0.0, g2 = 0.0;
                for (int64_t e = 0; e < sd; ++e)
                    g1 += G[e] * Sp[e];
                for (int j = 0; j < dv; ++j)
                    g2 += du[j] * kS[j];
                da[b * dab + h * dah + t * dat] = g1 - bt_ * g2;
            }
            /* G_{t-1} (before its own q term) = a_t (G_t - beta_t k_t^T du_t) */
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j)
                    G[(int64_t)i * dv + j] = at_ * (G[(int64_t)i * dv + j] - bt_ * kt[i] * du[j]);
        }
    }
    if (dS_in)
        memcpy(dS_in, G, (size_t)sd * sizeof(double));
}

int delta_bwd(int B, int H, int64_t T, int dk, int dv,
              const double* q, int64_t qsb, int64_t qsh, int64_t qst,
              const double* k, int64_t ksb, int64_t ksh, int64_t kst,
              const double* v, int64_t vsb, int64_t vsh, int64_t vst,
              const double* beta, int64_t bsb, int64_t bsh, int64_t bst,
              const double* a, int64_t ab, int64_t ah, int64_t at,
              const double* S_in,
              const double* dO, int64_t dosb, int64_t dosh, int64_t dost,
              const double* dS_out,
              double* dq, int64_t dqsb, int64_t dqsh, int64_t dqst,
              double* dk_, int64_t dksb, int64_t dksh, int64_t dkst,
              double* dv_, int64_t dvsb, int64_t dvsh, int64_t dvst,
              double* dS_in,
              double* dbeta, int64_t dbb, int64_t dbh, int64_t dbt,
              double* da, int64_t dab, int64_t dah, int64_t dat,
              int nthreads)
{
    if (B < 0 || H < 0 || T < 0 || dk <= 0 || dv <= 0 || !q || !k || !v || !beta ||
        (da && !a))
        return -1;
    const dstride qs = {qsb, qsh, qst}, ks = {ksb, ksh, kst}, vs = {vsb, vsh, vst},
                  dos = {dosb, dosh, dost}, dqs = {dqsb, dqsh, dqst},
                  dks = {dksb, dksh, dkst}, dvs = {dvsb, dvsh, dvst};
    const int64_t sd = (int64_t)dk * dv;
    const int64_t nck = (T + CK - 1) / CK;
    int rc = 0;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
    {
        const size_t n = (size_t)((nck + CK + 2) * sd + 3 * dv);
        double* buf = (double*)malloc(n * sizeof(double));
        if (!buf) {
#pragma omp atomic write
            rc = -1;
        } else {
            double* ckpt = buf;
            double* blk = ckpt + nck * sd;
            double* G = blk + (CK + 1) * sd;
            double* u = G + sd;
            double* du = u + dv;
            double* kS = du + dv;
#pragma omp for schedule(dynamic, 1)
            for (int bh = 0; bh < B * H; ++bh) {
                const int b = bh / H, h = bh % H;
                delta_bwd_head(b, h, T, dk, dv, q, qs, k, ks, v, vs, beta, bsb, bsh, bst,
                               a, ab, ah, at, S_in ? S_in + (int64_t)bh * sd : NULL, dO, dos,
                               dS_out ? dS_out + (int64_t)bh * sd : NULL, dq, dqs, dk_, dks,
                               dv_, dvs, dS_in ? dS_in + (int64_t)bh * sd : NULL,
                               dbeta, dbb, dbh, dbt, da, dab, dah, dat,
                               ckpt, blk, G, u, du, kS);
            }
            free(buf);
        }
    }
    return rc;
}
