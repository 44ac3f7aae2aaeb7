/*
 * The C oracles (oracle/linrec_oracle.c, oracle/deltarule_oracle.c) under
 * AddressSanitizer and UndefinedBehaviorSanitizer.  Built and run by
 * tests/test_sanitizers.py.  Inputs are small and strided (padded token and
 * head strides, odd d_k and d_v, T across the oracles' 256-token checkpoint
 * blocks); the checks are the ones any memory error would disturb: a split
 * into two pieces with the state and its gradient carried between them gives
 * bitwise the unsplit result, T = 0 returns the carried state unchanged, and
 * bad dimensions are refused.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_fwd(int B, int H, int64_t T, int dk, int dv, const double* q, int64_t qsb, int64_t qsh,
               int64_t qst, const double* k, int64_t ksb, int64_t ksh, int64_t kst, const double* v,
               int64_t vsb, int64_t vsh, int64_t vst, const double* a, int64_t ab, int64_t ah, int64_t at,
               const double* S_in, double* o, int64_t osb, int64_t osh, int64_t ost, double* S_out,
               int nthreads);
int oracle_bwd(int B, int H, int64_t T, int dk, int dv, const double* q, int64_t qsb, int64_t qsh,
               int64_t qst, const double* k, int64_t ksb, int64_t ksh, int64_t kst, const double* v,
               int64_t vsb, int64_t vsh, int64_t vst, const double* a, int64_t ab, int64_t ah, int64_t at,
               const double* S_in, const double* dO, int64_t dosb, int64_t dosh, int64_t dost,
               const double* dS_out, double* dq, int64_t dqsb, int64_t dqsh, int64_t dqst, double* dk_,
               int64_t dksb, int64_t dksh, int64_t dkst, double* dv_, int64_t dvsb, int64_t dvsh,
               int64_t dvst, double* dS_in, double* da, int64_t dab, int64_t dah, int64_t dat,
               int nthreads);
int delta_fwd(int B, int H, int64_t T, int dk, int dv, const double* q, int64_t qsb, int64_t qsh,
              int64_t qst, const double* k, int64_t ksb, int64_t ksh, int64_t kst, const double* v,
              int64_t vsb, int64_t vsh, int64_t vst, const double* beta, int64_t bsb, int64_t bsh,
              int64_t bst, const double* a, int64_t ab, int64_t ah, int64_t at, const double* S_in,
              double* o, int64_t osb, int64_t osh, int64_t ost, double* S_out, int nthreads);
int delta_bwd(int B, int H, int64_t T, int dk, int dv, const double* q, int64_t qsb, int64_t qsh,
              int64_t qst, const double* k, int64_t ksb, int64_t ksh, int64_t kst, const double* v,
              int64_t vsb, int64_t vsh, int64_t vst, const double* beta, int64_t bsb, int64_t bsh,
              int64_t bst, const double* a, int64_t ab, int64_t ah, int64_t at, const double* S_in,
              const double* dO, int64_t dosb, int64_t dosh, int64_t dost, const double* dS_out, double* dq,
              int64_t dqsb, int64_t dqsh, int64_t dqst, double* dk_, int64_t dksb, int64_t dksh,
              int64_t dkst, double* dv_, int64_t dvsb, int64_t dvsh, int64_t dvst, double* dS_in,
              double* dbeta, int64_t dbb, int64_t dbh, int64_t dbt, double* da, int64_t dab, int64_t dah,
              int64_t dat, int nthreads);

enum { B = 2, H = 3, T = 300, CUT = 100, DK = 5, DV = 7, PADT = 3 };

static int failures = 0;
#define EXPECT(cond, what)                                             \
    do {                                                               \
        if (!(cond)) {                                                 \
            fprintf(stderr, "FAIL %s:%d %s\n", __FILE__, __LINE__, what); \
            ++failures;                                                \
        }                                                              \
    } while (0)

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double uniform(void)
{
    rng = rng * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(rng >> 11) / 9007199254740992.0;
}

/* [B][H][T][d] with token stride d + PADT and head stride T * (d + PADT) + 5 */
typedef struct {
    double* p;
    int64_t sb, sh, st;
} act;

static act make_act(int d, int fill)
{
    act x;
    x.st = d + PADT;
    x.sh = (int64_t)T * x.st + 5;
    x.sb = H * x.sh + 11;
    const size_t n = (size_t)(B * x.sb);
    x.p = (double*)calloc(n, sizeof(double));
    if (fill)
        for (int b = 0; b < B; ++b)
            for (int h = 0; h < H; ++h)
                for (int t = 0; t < T; ++t)
                    for (int i = 0; i < d; ++i)
                        x.p[b * x.sb + h * x.sh + t * x.st + i] = 2.0 * uniform() - 1.0;
    return x;
}

static act shift(act x, int t0)
{
    act y = x;
    y.p += (int64_t)t0 * x.st;
    return y;
}

static int same(const double* x, const double* y, size_t n)
{
    return memcmp(x, y, n * sizeof(double)) == 0;
}

static void linear_checks(const double* a, int64_t ab, int64_t ah, int64_t at, const char* name)
{
    act q = make_act(DK, 1), k = make_act(DK, 1), v = make_act(DV, 1), dO = make_act(DV, 1);
    act o1 = make_act(DV, 0), o2 = make_act(DV, 0);
    act dq1 = make_act(DK, 0), dk1 = make_act(DK, 0), dv1 = make_act(DV, 0);
    act dq2 = make_act(DK, 0), dk2 = make_act(DK, 0), dv2 = make_act(DV, 0);
    const size_t sd = (size_t)B * H * DK * DV;
    double *S_in = malloc(sd * 8), *S_mid = malloc(sd * 8), *S1 = malloc(sd * 8), *S2 = malloc(sd * 8);
    double *dS_out = malloc(sd * 8), *dS_mid = malloc(sd * 8), *G1 = malloc(sd * 8), *G2 = malloc(sd * 8);
    double *da1 = calloc((size_t)B * H * T, 8), *da2 = calloc((size_t)B * H * T, 8);
    for (size_t i = 0; i < sd; ++i) {
        S_in[i] = 0.1 * (2.0 * uniform() - 1.0);
        dS_out[i] = 2.0 * uniform() - 1.0;
    }
    const int wantda = a != NULL;
    EXPECT(oracle_fwd(B, H, T, DK, DV, q.p, q.sb, q.sh, q.st, k.p, k.sb, k.sh, k.st, v.p, v.sb, v.sh, v.st, a,
                      ab, ah, at, S_in, o1.p, o1.sb, o1.sh, o1.st, S1, 2) == 0, name);
    EXPECT(oracle_fwd(B, H, CUT, DK, DV, q.p, q.sb, q.sh, q.st, k.p, k.sb, k.sh, k.st, v.p, v.sb, v.sh, v.st,
                      a, ab, ah, at, S_in, o2.p, o2.sb, o2.sh, o2.st, S_mid, 2) == 0, name);
    act q2 = shift(q, CUT), k2 = shift(k, CUT), v2 = shift(v, CUT), o2b = shift(o2, CUT), dO2 = shift(dO, CUT);
    const double* a2 = a ? a + (int64_t)CUT * at : NULL;
    EXPECT(oracle_fwd(B, H, T - CUT, DK, DV, q2.p, q.sb, q.sh, q.st, k2.p, k.sb, k.sh, k.st, v2.p, v.sb, v.sh,
                      v.st, a2, ab, ah, at, S_mid, o2b.p, o2.sb, o2.sh, o2.st, S2, 2) == 0, name);
    EXPECT(same(o1.p, o2.p, (size_t)(B * o1.sb)), "fwd split: o");
    EXPECT(same(S1, S2, sd), "fwd split: S_out");

    EXPECT(oracle_bwd(B, H, T, DK, DV, q.p, q.sb, q.sh, q.st, k.p, k.sb, k.sh, k.st, v.p, v.sb, v.sh, v.st, a,
                      ab, ah, at, S_in, dO.p, dO.sb, dO.sh, dO.st, dS_out, dq1.p, dq1.sb, dq1.sh, dq1.st, dk1.p,
                      dk1.sb, dk1.sh, dk1.st, dv1.p, dv1.sb, dv1.sh, dv1.st, G1, wantda ? da1 : NULL,
                      (int64_t)H * T, T, 1, 2) == 0, name);
    act dq2b = shift(dq2, CUT), dk2b = shift(dk2, CUT), dv2b = shift(dv2, CUT);
    EXPECT(oracle_bwd(B, H, T - CUT, DK, DV, q2.p, q.sb, q.sh, q.st, k2.p, k.sb, k.sh, k.st, v2.p, v.sb, v.sh,
                      v.st, a2, ab, ah, at, S_mid, dO2.p, dO.sb, dO.sh, dO.st, dS_out, dq2b.p, dq2.sb, dq2.sh,
                      dq2.st, dk2b.p, dk2.sb, dk2.sh, dk2.st, dv2b.p, dv2.sb, dv2.sh, dv2.st, dS_mid,
                      wantda ? da2 + CUT : NULL, (int64_t)H * T, T, 1, 2) == 0, name);
    EXPECT(oracle_bwd(B, H, CUT, DK, DV, q.p, q.sb, q.sh, q.st, k.p, k.sb, k.sh, k.st, v.p, v.sb, v.sh, v.st,
                      a, ab, ah, at, S_in, dO.p, dO.sb, dO.sh, dO.st, dS_mid, dq2.p, dq2.sb, dq2.sh, dq2.st,
                      dk2.p, dk2.sb, dk2.sh, dk2.st, dv2.p, dv2.sb, dv2.sh, dv2.st, G2, wantda ? da2 : NULL,
                      (int64_t)H * T, T, 1, 2) == 0, name);
    EXPECT(same(dq1.p, dq2.p, (size_t)(B * dq1.sb)), "bwd split: dq");
    EXPECT(same(dk1.p, dk2.p, (size_t)(B * dk1.sb)), "bwd split: dk");
    EXPECT(same(dv1.p, dv2.p, (size_t)(B * dv1.sb)), "bwd split: dv");
    EXPECT(same(G1, G2, sd), "bwd split: dS_in");
    if (wantda) {
        /* the decay gradient of the later piece depends on dS_out only
           through the carried gradient; the split regroups no sum */
        double worst = 0.0;
        for (size_t i = 0; i < (size_t)B * H * T; ++i)
            worst = fmax(worst, fabs(da1[i] - da2[i]) / (1.0 + fabs(da1[i])));
        EXPECT(worst < 1e-12, "bwd split: da");
    }
    /* T = 0: the carried states pass through */
    EXPECT(oracle_fwd(B, H, 0, DK, DV, q.p, q.sb, q.sh, q.st, k.p, k.sb, k.sh, k.st, v.p, v.sb, v.sh, v.st, a,
                      ab, ah, at, S_in, NULL, 0, 0, 0, S2, 1) == 0, name);
    EXPECT(same(S_in, S2, sd), "T = 0 forward");
    free(q.p); free(k.p); free(v.p); free(dO.p); free(o1.p); free(o2.p);
    free(dq1.p); free(dk1.p); free(dv1.p); free(dq2.p); free(dk2.p); free(dv2.p);
    free(S_in); free(S_mid); free(S1); free(S2); free(dS_out); free(dS_mid); free(G1); free(G2);
    free(da1); free(da2);
}

static void delta_checks(const double* a, int64_t ab, int64_t ah, int64_t at, const char* name)
{
    act q = make_act(DK, 1), k = make_act(DK, 1), v = make_act(DV, 1), dO = make_act(DV, 1);
    act o1 = make_act(DV, 0), o2 = make_act(DV, 0);
    act dq1 = make_act(DK, 0), dk1 = make_act(DK, 0), dv1 = make_act(DV, 0);
    act dq2 = make_act(DK, 0), dk2 = make_act(DK, 0), dv2 = make_act(DV, 0);
    /* keys of norm about 1 keep I - beta k^T k a contraction */
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int t = 0; t < T; ++t) {
                double* r = k.p + b * k.sb + h * k.sh + t * k.st;
                double n2 = 0.0;
                for (int i = 0; i < DK; ++i)
                    n2 += r[i] * r[i];
                for (int i = 0; i < DK; ++i)
                    r[i] /= sqrt(n2);
            }
    const size_t nb = (size_t)B * H * T, sd = (size_t)B * H * DK * DV;
    double* beta = malloc(nb * 8);
    for (size_t i = 0; i < nb; ++i)
        beta[i] = uniform();
    double *S_in = malloc(sd * 8), *S_mid = malloc(sd * 8), *S1 = malloc(sd * 8), *S2 = malloc(sd * 8);
    double *dS_out = malloc(sd * 8), *dS_mid = malloc(sd * 8), *G1 = malloc(sd * 8), *G2 = malloc(sd * 8);
    double *db1 = calloc(nb, 8), *db2 = calloc(nb, 8), *da1 = calloc(nb, 8), *da2 = calloc(nb, 8);
    for (size_t i = 0; i < sd; ++i) {
        S_in[i] = 0.1 * (2.0 * uniform() - 1.0);
        dS_out[i] = 2.0 * uniform() - 1.0;
    }
    const int wantda = a != NULL;
    const int64_t bsb = (int64_t)H * T, bsh = T;
    EXPECT(delta_fwd(B, H, T, DK, DV, q.p, q.sb, q.sh, q.st, k.p, k.sb, k.sh, k.st, v.p, v.sb, v.sh, v.st, beta,
                     bsb, bsh, 1, a, ab, ah, at, S_in, o1.p, o1.sb, o1.sh, o1.st, S1, 2) == 0, name);
    EXPECT(delta_fwd(B, H, CUT, DK, DV, q.p, q.sb, q.sh, q.st, k.p, k.sb, k.sh, k.st, v.p, v.sb, v.sh, v.st,
                     beta, bsb, bsh, 1, a, ab, ah, at, S_in, o2.p, o2.sb, o2.sh, o2.st, S_mid, 2) == 0, name);
    act q2 = shift(q, CUT), k2 = shift(k, CUT), v2 = shift(v, CUT), o2b = shift(o2, CUT), dO2 = shift(dO, CUT);
    const double* a2 = a ? a + (int64_t)CUT * at : NULL;
    EXPECT(delta_fwd(B, H, T - CUT, DK, DV, q2.p, q.sb, q.sh, q.st, k2.p, k.sb, k.sh, k.st, v2.p, v.sb, v.sh,
                     v.st, beta + CUT, bsb, bsh, 1, a2, ab, ah, at, S_mid, o2b.p, o2.sb, o2.sh, o2.st, S2, 2) == 0,
           name);
    EXPECT(same(o1.p, o2.p, (size_t)(B * o1.sb)), "delta fwd split: o");
    EXPECT(same(S1, S2, sd), "delta fwd split: S_out");

    EXPECT(delta_bwd(B, H, T, DK, DV, q.p, q.sb, q.sh, q.st, k.p, k.sb, k.sh, k.st, v.p, v.sb, v.sh, v.st, beta,
                     bsb, bsh, 1, a, ab, ah, at, S_in, dO.p, dO.sb, dO.sh, dO.st, dS_out, dq1.p, dq1.sb, dq1.sh,
                     dq1.st, dk1.p, dk1.sb, dk1.sh, dk1.st, dv1.p, dv1.sb, dv1.sh, dv1.st, G1, db1, bsb, bsh, 1,
                     wantda ? da1 : NULL, bsb, bsh, 1, 2) == 0, name);
    act dq2b = shift(dq2, CUT), dk2b = shift(dk2, CUT), dv2b = shift(dv2, CUT);
    EXPECT(delta_bwd(B, H, T - CUT, DK, DV, q2.p, q.sb, q.sh, q.st, k2.p, k.sb, k.sh, k.st, v2.p, v.sb, v.sh,
                     v.st, beta + CUT, bsb, bsh, 1, a2, ab, ah, at, S_mid, dO2.p, dO.sb, dO.sh, dO.st, dS_out,
                     dq2b.p, dq2.sb, dq2.sh, dq2.st, dk2b.p, dk2.sb, dk2.sh, dk2.st, dv2b.p, dv2.sb, dv2.sh,
                     dv2.st, dS_mid, db2 + CUT, bsb, bsh, 1, wantda ? da2 + CUT : NULL, bsb, bsh, 1, 2) == 0,
           name);
    EXPECT(delta_bwd(B, H, CUT, DK, DV, q.p, q.sb, q.sh, q.st, k.p, k.sb, k.sh, k.st, v.p, v.sb, v.sh, v.st,
                     beta, bsb, bsh, 1, a, ab, ah, at, S_in, dO.p, dO.sb, dO.sh, dO.st, dS_mid, dq2.p, dq2.sb,
                     dq2.sh, dq2.st, dk2.p, dk2.sb, dk2.sh, dk2.st, dv2.p, dv2.sb, dv2.sh, dv2.st, G2, db2, bsb,
                     bsh, 1, wantda ? da2 : NULL, bsb, bsh, 1, 2) == 0, name);
    EXPECT(same(dq1.p, dq2.p, (size_t)(B * dq1.sb)), "delta bwd split: dq");
    EXPECT(same(dk1.p, dk2.p, (size_t)(B * dk1.sb)), "delta bwd split: dk");
    EXPECT(same(dv1.p, dv2.p, (size_t)(B * dv1.sb)), "delta bwd split: dv");
    EXPECT(same(G1, G2, sd), "delta bwd split: dS_in");
    double worst = 0.0;
    for (size_t i = 0; i < nb; ++i) {
        worst = fmax(worst, fabs(db1[i] - db2[i]) / (1.0 + fabs(db1[i])));
        if (wantda)
            worst = fmax(worst, fabs(da1[i] - da2[i]) / (1.0 + fabs(da1[i])));
    }
    EXPECT(worst < 1e-12, "delta bwd split: dbeta, da");
    free(q.p); free(k.p); free(v.p); free(dO.p); free(o1.p); free(o2.p);
    free(dq1.p); free(dk1.p); free(dv1.p); free(dq2.p); free(dk2.p); free(dv2.p);
    free(beta); free(S_in); free(S_mid); free(S1); free(S2); free(dS_out); free(dS_mid); free(G1); free(G2);
    free(db1); free(db2); free(da1); free(da2);
}

int main(void)
{
    /* per-token gate, per-head decay, no decay */
    double* tok = malloc((size_t)B * H * T * 8);
    for (int i = 0; i < B * H * T; ++i)
        tok[i] = 0.9 + 0.1 * uniform();
    double head[H];
    for (int h = 0; h < H; ++h)
        head[h] = 1.0 - pow(2.0, -(5.0 + 8.0 * h / H));
    linear_checks(tok, (int64_t)H * T, T, 1, "linear, token decay");
    linear_checks(head, 0, 1, 0, "linear, head decay");
    linear_checks(NULL, 0, 0, 0, "linear, no decay");
    delta_checks(tok, (int64_t)H * T, T, 1, "delta, token decay");
    delta_checks(NULL, 0, 0, 0, "delta, no decay");
    /* bad dimensions are refused */
    double x = 0.0;
    EXPECT(oracle_fwd(B, H, T, 0, DV, &x, 0, 0, 0, &x, 0, 0, 0, &x, 0, 0, 0, NULL, 0, 0, 0, NULL, NULL, 0, 0, 0,
                      NULL, 1) != 0, "d_k = 0");
    EXPECT(delta_fwd(B, H, -1, DK, DV, &x, 0, 0, 0, &x, 0, 0, 0, &x, 0, 0, 0, &x, 0, 0, 0, NULL, 0, 0, 0, NULL,
                     NULL, 0, 0, 0, NULL, 1) != 0, "T < 0");
    free(tok);
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle checks passed\n");
    return 0;
}
