/*
 * linrec_oracle.c -- fp64 CPU oracle for the decayed linear recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product: only
 * the test suite, the smoke check and the benchmark's CPU-baseline leg load
 * it.  It shares no code, header, table or helper with the HIP library.
 *
 * What it computes (one (b,h) head at a time, all arithmetic in double):
 *
 *   forward   S_0 = S_in
 *             S_t = a_t * S_{t-1} + k_t^T v_t        (d_k x d_v state)
 *             o_t = q_t S_t                           (row vector times state)
 *             S_out = S_T
 *
 *   backward  for L = sum_t <dO_t, o_t> + <dS_out, S_T>:
 *             dq_t = dO_t S_t^T                       (forward sweep)
 *             G_t  = q_t^T dO_t + carry,  carry starts at dS_out
 *             dk_t = v_t G_t^T,  dv_t = k_t G_t,  carry <- a_t G_t
 *             dS_in = carry after t = 1               (reverse sweep)
 *             (optional) da_t = <G_t, S_{t-1}>_F
 *
 * Sources.  The recurrence is the linear-attention / linear-recurrence form
 * that all three pages build on: a d x d memory state accumulated over
 * sub-sequences with the backward pass run over stored states (Sequence
 * Accumulation and Beyond, "Approach"), boundary states and gradients carried
 * from chunk to chunk (StateFlow, Abstract), and the right-product form of
 * linear attention (Linear Attention Sequence Parallelism, abstract).  The
 * pages do not write the formula out; the readings taken where they are
 * silent are: o_t uses S_t (token t sees its own k_t^T v_t), no scale,
 * normaliser or feature map, and S_in is multiplied by the first token's
 * decay (S_0 = S_in), which is what makes any split of the sequence exact.
 *
 * The backward is the hand-derived adjoint of the forward.  It keeps O(d^2)
 * memory per head: the reverse sweep never inverts S <- (S - k^T v)/a, which
 * would amplify rounding by 1/a per step.
 *
 * Layouts: every activation is [B,H,T,d] with explicit element strides
 * (sb, sh, st; the feature index is contiguous).  The decay is read as
 * a[b*ab + h*ah + t*at]; at = 0 gives a per-head constant, a == NULL gives
 * a_t = 1.  States are contiguous [B,H,d_k,d_v].  NULL S_in / dS_out mean
 * zeros; NULL outputs are skipped.  Parallel over (b,h) with OpenMP; each
 * head's arithmetic order is fixed, so results do not depend on the thread
 * count or on how the sequence is split.
 *
 * Return value: 0 on success, -1 on a bad argument (nothing written).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int64_t sb, sh, st;
} ostride;

static inline double decay_at(const double* a, int64_t ab, int64_t ah, int64_t at,
                              int b, int h, int64_t t)
{
    return a ? a[b * ab + h * ah + t * at] : 1.0;
}

static int check_dims(int B, int H, int64_t T, int dk, int dv)
{
    return (B < 0 || H < 0 || T < 0 || dk <= 0 || dv <= 0) ? -1 : 0;
}

/* Forward sweep for one head: S <- a_t S + k_t^T v_t, o_t = q_t S. */
static void fwd_head(int b, int h, int64_t T, int dk, int dv,
                     const double* q, ostride qs, const double* k, ostride ks,
                     const double* v, ostride vs,
                     const double* a, int64_t ab, int64_t ah, int64_t at,
                     const double* S_in, double* o, ostride os, double* S_out,
                     double* S /* scratch dk*dv */)
{
    const int64_t sd = (int64_t)dk * dv;
    if (S_in)
        memcpy(S, S_in, (size_t)sd * sizeof(double));
    else
        memset(S, 0, (size_t)sd * sizeof(double));

    const double* qh = q ? q + b * qs.sb + h * qs.sh : NULL;
    const double* kh = k + b * ks.sb + h * ks.sh;
    const double* vh = v + b * vs.sb + h * vs.sh;
    double* oh = o ? o + b * os.sb + h * os.sh : NULL;

    for (int64_t t = 0; t < T; ++t) {
        const double at_ = decay_at(a, ab, ah, at, b, h, t);
        const double* kt = kh + t * ks.st;
        const double* vt = vh + t * vs.st;
        for (int i = 0; i < dk; ++i) {
            double* Si = S + (int64_t)i * dv;
            const double ki = kt[i];
            for (int j = 0; j < dv; ++j)
                Si[j] = at_ * Si[j] + ki * vt[j];
        }
        if (oh) {
            const double* qt = qh + t * qs.st;
            double* ot = oh + t * os.st;
            for (int j = 0; j < dv; ++j)
                ot[j] = 0.0;
            for (int i = 0; i < dk; ++i) {
                const double* Si = S + (int64_t)i * dv;
                const double qi = qt[i];
                for (int j = 0; j < dv; ++j)
                    ot[j] += qi * Si[j];
            }
        }
    }
    if (S_out)
        memcpy(S_out, S, (size_t)sd * sizeof(double));
}

int oracle_fwd(int B, int H, int64_t T, int dk, int dv,
               const double* q, int64_t qsb, int64_t qsh, int64_t qst,
               const double* k, int64_t ksb, int64_t ksh, int64_t kst,
               const double* v, int64_t vsb, int64_t vsh, int64_t vst,
               const double* a, int64_t ab, int64_t ah, int64_t at,
               const double* S_in, double* o, int64_t osb, int64_t osh, int64_t ost,
               double* S_out, int nthreads)
{
    if (check_dims(B, H, T, dk, dv) || !k || !v || (o && !q))
        return -1;
    const ostride qs = {qsb, qsh, qst}, ks = {ksb, ksh, kst}, vs = {vsb, vsh, vst},
                  os = {osb, osh, ost};
    const int64_t sd = (int64_t)dk * dv;
    const int nh = B * H;
    int rc = 0;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
    {
        double* S = (double*)malloc((size_t)sd * sizeof(double));
        if (!S) {
#pragma omp atomic write
            rc = -1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int bh = 0; bh < nh; ++bh) {
                const int b = bh / H, h = bh % H;
                fwd_head(b, h, T, dk, dv, q, qs, k, ks, v, vs, a, ab, ah, at,
                         S_in ? S_in + (int64_t)bh * sd : NULL, o, os,
                         S_out ? S_out + (int64_t)bh * sd : NULL, S);
            }
            free(S);
        }
    }
    return rc;
}

/*
 * Backward for one head.  Two sweeps, O(d_k d_v) memory:
 *   forward sweep rebuilds S_t and writes dq_t = dO_t S_t^T;
 *   reverse sweep carries G from dS_out back to dS_in.
 * When da is requested the reverse sweep also needs S_{t-1}; it is rebuilt
 * per token by a forward re-sweep from a checkpoint every `ck` tokens, so
 * memory stays O((T/ck + ck) d^2) without inverting the recurrence.
 */
static void bwd_head(int b, int h, int64_t T, int dk, int dv,
                     const double* q, ostride qs, const double* k, ostride ks,
                     const double* v, ostride vs,
                     const double* a, int64_t ab, int64_t ah, int64_t at,
                     const double* S_in, const double* dO, ostride dos,
                     const double* dS_out,
                     double* dq, ostride dqs, double* dk_, ostride dks,
                     double* dv_, ostride dvs, double* dS_in,
                     double* da, int64_t dab, int64_t dah, int64_t dat,
                     double* S, double* G)
{
    const int64_t sd = (int64_t)dk * dv;
    const double* qh = q + b * qs.sb + h * qs.sh;
    const double* kh = k + b * ks.sb + h * ks.sh;
    const double* vh = v + b * vs.sb + h * vs.sh;
    const double* dOh = dO ? dO + b * dos.sb + h * dos.sh : NULL;

    /* forward sweep: dq_t = dO_t S_t^T, i.e. dq_t[i] = sum_j dO_t[j] S_t[i][j] */
    if (dq) {
        double* dqh = dq + b * dqs.sb + h * dqs.sh;
        if (S_in)
            memcpy(S, S_in, (size_t)sd * sizeof(double));
        else
            memset(S, 0, (size_t)sd * sizeof(double));
        for (int64_t t = 0; t < T; ++t) {
            const double at_ = decay_at(a, ab, ah, at, b, h, t);
            const double* kt = kh + t * ks.st;
            const double* vt = vh + t * vs.st;
            double* dqt = dqh + t * dqs.st;
            for (int i = 0; i < dk; ++i) {
                double* Si = S + (int64_t)i * dv;
                const double ki = kt[i];
                double acc = 0.0;
                for (int j = 0; j < dv; ++j) {
                    Si[j] = at_ * Si[j] + ki * vt[j];
                    if (dOh)
                        acc += dOh[t * dos.st + j] * Si[j];
                }
                dqt[i] = acc;
            }
        }
    }

    /* optional checkpoints of S_{t-1} for da: S before token c*ck */
    const int64_t ck = 256;
    const int64_t nck = da ? (T + ck - 1) / ck : 0;
    double* cks = NULL;
    double* Sprev = NULL;
    if (da) {
        cks = (double*)malloc((size_t)(nck * sd + (ck + 1) * sd) * sizeof(double));
        Sprev = cks + nck * sd; /* (ck+1) states: S_{c*ck-1} .. for one block */
        if (S_in)
            memcpy(S, S_in, (size_t)sd * sizeof(double));
        else
            memset(S, 0, (size_t)sd * sizeof(double));
        for (int64_t t = 0; t < T; ++t) {
            if (t % ck == 0)
                memcpy(cks + (t / ck) * sd, S, (size_t)sd * sizeof(double));
            const double at_ = decay_at(a, ab, ah, at, b, h, t);
            const double* kt = kh + t * ks.st;
            const double* vt = vh + t * vs.st;
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j)
                    S[(int64_t)i * dv + j] = at_ * S[(int64_t)i * dv + j] + kt[i] * vt[j];
        }
    }

    /* reverse sweep: G_t = q_t^T dO_t + carry; carry <- a_t G_t */
    if (dS_out)
        memcpy(G, dS_out, (size_t)sd * sizeof(double));
    else
        memset(G, 0, (size_t)sd * sizeof(double));
    double* dkh = dk_ ? dk_ + b * dks.sb + h * dks.sh : NULL;
    double* dvh = dv_ ? dv_ + b * dvs.sb + h * dvs.sh : NULL;
    int64_t blk = -1;
    for (int64_t t = T - 1; t >= 0; --t) {
        if (da && t / ck != blk) {
            /* rebuild S_{t'-1} for every t' of this checkpoint block */
            blk = t / ck;
            const int64_t t0 = blk * ck, t1 = (t0 + ck < T) ? t0 + ck : T;
            memcpy(Sprev, cks + blk * sd, (size_t)sd * sizeof(double));
            for (int64_t u = t0; u < t1 - 1; ++u) {
                const double au = decay_at(a, ab, ah, at, b, h, u);
                const double* ku = kh + u * ks.st;
                const double* vu = vh + u * vs.st;
                double* src = Sprev + (u - t0) * sd;
                double* dst = src + sd;
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j)
                        dst[(int64_t)i * dv + j] = au * src[(int64_t)i * dv + j] + ku[i] * vu[j];
            }
        }
        const double at_ = decay_at(a, ab, ah, at, b, h, t);
        const double* qt = qh + t * qs.st;
        const double* kt = kh + t * ks.st;
        const double* vt = vh + t * vs.st;
        if (dOh) {
            const double* dOt = dOh + t * dos.st;
            for (int i = 0; i < dk; ++i) {
                double* Gi = G + (int64_t)i * dv;
                const double qi = qt[i];
                for (int j = 0; j < dv; ++j)
                    Gi[j] += qi * dOt[j];
            }
        }
        if (dkh) {
            double* dkt = dkh + t * dks.st;
            for (int i = 0; i < dk; ++i) {
                const double* Gi = G + (int64_t)i * dv;
                double acc = 0.0;
                for (int j = 0; j < dv; ++j)
                    acc += Gi[j] * vt[j];
                dkt[i] = acc;
            }
        }
        if (dvh) {
            double* dvt = dvh + t * dvs.st;
            for (int j = 0; j < dv; ++j)
                dvt[j] = 0.0;
            for (int i = 0; i < dk; ++i) {
                const double* Gi = G + (int64_t)i * dv;
                const double ki = kt[i];
                for (int j = 0; j < dv; ++j)
                    dvt[j] += ki * Gi[j];
            }
        }
        if (da) {
            const double* Sp = Sprev + (t - blk * ck) * sd;
            double acc = 0.0;
            for (int64_t e = 0; e < sd; ++e)
                acc += G[e] * Sp[e];
            da[b * dab + h * dah + t * dat] = acc;
        }
        for (int64_t e = 0; e < sd; ++e)
            G[e] *= at_;
    }
    if (dS_in)
        memcpy(dS_in, G, (size_t)sd * sizeof(double));
    free(cks);
}

int oracle_bwd(int B, int H, int64_t T, int dk, int dv,
               const double* q, int64_t qsb, int64_t qsh, int64_t qst,
               const double* k, int64_t ksb, int64_t ksh, int64_t kst,
               const double* v, int64_t vsb, int64_t vsh, int64_t vst,
               const double* a, int64_t ab, int64_t ah, int64_t at,
               const double* S_in,
               const double* dO, int64_t dosb, int64_t dosh, int64_t dost,
               const double* dS_out,
               double* dq, int64_t dqsb, int64_t dqsh, int64_t dqst,
               double* dk_, int64_t dksb, int64_t dksh, int64_t dkst,
               double* dv_, int64_t dvsb, int64_t dvsh, int64_t dvst,
               double* dS_in,
               double* da, int64_t dab, int64_t dah, int64_t dat,
               int nthreads)
{
    if (check_dims(B, H, T, dk, dv) || !q || !k || !v || (da && !a))
        return -1;
    const ostride qs = {qsb, qsh, qst}, ks = {ksb, ksh, kst}, vs = {vsb, vsh, vst},
                  dos = {dosb, dosh, dost}, dqs = {dqsb, dqsh, dqst},
                  dks = {dksb, dksh, dkst}, dvs = {dvsb, dvsh, dvst};
    const int64_t sd = (int64_t)dk * dv;
    const int nh = B * H;
    int rc = 0;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
    {
        double* buf = (double*)malloc((size_t)(2 * sd) * sizeof(double));
        if (!buf) {
#pragma omp atomic write
            rc = -1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int bh = 0; bh < nh; ++bh) {
                const int b = bh / H, h = bh % H;
                bwd_head(b, h, T, dk, dv, q, qs, k, ks, v, vs, a, ab, ah, at,
                         S_in ? S_in + (int64_t)bh * sd : NULL, dO, dos,
                         dS_out ? dS_out + (int64_t)bh * sd : NULL,
                         dq, dqs, dk_, dks, dv_, dvs,
                         dS_in ? dS_in + (int64_t)bh * sd : NULL,
                         da, dab, dah, dat, buf, buf + sd);
            }
            free(buf);
        }
    }
    return rc;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
