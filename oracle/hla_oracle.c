/*
 * hla_oracle.c -- plain fp64 CPU oracle for masked second-order
 * Higher-order Linear Attention (HLA).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the bench's CPU
 * baseline use it.  It shares no code, header, table or helper with the HIP
 * library; the two meet only through the seeded input generators.
 *
 * What it computes (all in double precision, one head at a time):
 *
 *   Prefix summaries, updated once per token t (paperlayer.ai page, sec. 3 and
 *   3.1; gist.science page, "Methodik" item 1):
 *     S_t = g S_{t-1} + k_t k_t^T           key second moment      (d x d)
 *     C_t = g C_{t-1} + q_t v_t^T           query-value accumulator (d x dv)
 *     m_t = g m_{t-1} + q_t                 query mass              (d)
 *   Cross summaries that remove the "future" pairs (key index after query
 *   index) from the naive product S_t C_t (gist.science page, "Methodik" 1,
 *   "Strenge Kausalitaet"):
 *     G_t = g^2 G_{t-1} + g k_t (k_t^T C_{t-1})                      (d x dv)
 *     h_t = g^2 h_{t-1} + g k_t (k_t . m_{t-1})                      (d)
 *   i.e. G_t = sum_{j < i <= t} g^(2t-i-j) k_i (k_i . q_j) v_j^T.
 *   Output (gist.science page, "Ausgangsformulierung"; paperlayer.ai page,
 *   sec. 5.1 for the ridge and the unnormalized default):
 *     a_t   = (S_t + lambda I) q_t
 *     num_t = a_t^T C_t - q_t^T G_t
 *     den_t = a_t . m_t - q_t . h_t         (the same with every v_j = 1)
 *     out_t = num_t, or num_t / den_t when normalize is set.
 *   g is the fixed per-head exponential decay (paperlayer.ai page, sec. 4.3);
 *   S, C, m decay by g per token, G and h by g^2, and the cross term carries
 *   one factor g, so that q_t^T(S_t C_t - G_t) keeps exactly the pairs
 *   i <= j <= t with weight g^(2t-i-j).
 *
 *   Segment composition (paperlayer.ai page, sec. 4.2: masked semidirect
 *   product on (S, C, m, G, h); gist.science page, "Assoziative Operatoren",
 *   cross term S_B C_A), earlier segment a, later segment b, rho = g^len:
 *     S = rho_b S_a + S_b        C = rho_b C_a + C_b       m = rho_b m_a + m_b
 *     G = rho_b^2 G_a + G_b + rho_b S_b C_a
 *     h = rho_b^2 h_a + h_b + rho_b S_b m_a
 *     rho = rho_a rho_b
 *
 * Layouts are row-major and contiguous: q, k [B,H,n,d], v [B,H,n,dv],
 * out [B,H,n,dv], den [B,H,n]; states indexed by b*H+h: S [BH,d,d],
 * C and G [BH,d,dv], m and h [BH,d], rho [BH].
 */
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    double *S, *C, *m, *G, *h, *rho;
} ora_state;

/* One token of the serial recurrence.  State is updated in place.
 * r (dv) and a (d) are scratch. */
static void ora_step(int d, int dv, double g, double lam,
                     const double *q, const double *k, const double *v,
                     double *S, double *C, double *m, double *G, double *h,
                     double *r, double *a, double *num, double *den)
{
    int i, j;
    double s = 0.0, g2 = g * g, dn;

    /* r = k^T C_{t-1}, s = k . m_{t-1}  (exclusive prefix, before the delta) */
    for (j = 0; j < dv; ++j) r[j] = 0.0;
    for (i = 0; i < d; ++i) {
        const double ki = k[i];
        const double *Ci = C + (size_t)i * dv;
        for (j = 0; j < dv; ++j) r[j] += ki * Ci[j];
        s += ki * m[i];
    }
    /* cross summaries: G, h */
    for (i = 0; i < d; ++i) {
        double *Gi = G + (size_t)i * dv;
        const double gk = g * k[i];
        for (j = 0; j < dv; ++j) Gi[j] = g2 * Gi[j] + gk * r[j];
        h[i] = g2 * h[i] + gk * s;
    }
    /* token delta into the prefix moments (inclusive state) */
    for (i = 0; i < d; ++i) {
        double *Si = S + (size_t)i * d;
        double *Ci = C + (size_t)i * dv;
        for (j = 0; j < d; ++j) Si[j] = g * Si[j] + k[i] * k[j];
        for (j = 0; j < dv; ++j) Ci[j] = g * Ci[j] + q[i] * v[j];
        m[i] = g * m[i] + q[i];
    }
    /* a = (S_t + lambda I) q_t */
    for (i = 0; i < d; ++i) {
        const double *Si = S + (size_t)i * d;
        double acc = 0.0;
        for (j = 0; j < d; ++j) acc += Si[j] * q[j];
        a[i] = acc + lam * q[i];
    }
    /* num = a^T C_t - q^T G_t ; den = a . m_t - q . h_t */
    for (j = 0; j < dv; ++j) num[j] = 0.0;
    dn = 0.0;
    for (i = 0; i < d; ++i) {
        const double *Ci = C + (size_t)i * dv;
        const double *Gi = G + (size_t)i * dv;
        const double ai = a[i], qi = q[i];
        for (j = 0; j < dv; ++j) num[j] += ai * Ci[j] - qi * Gi[j];
        dn += ai * m[i] - qi * h[i];
    }
    *den = dn;
}

typedef struct {
    int B, H, n, d, dv, normalize;
    const double *q, *k, *v, *gamma;
    double lam;
    ora_state init;          /* S == NULL means zero state */
    double *out, *den;       /* den may be NULL */
    ora_state fin;           /* S == NULL means not returned */
    int next;                /* work counter */
} fwd_job;

static void fwd_head(fwd_job *J, int bh)
{
    const int d = J->d, dv = J->dv, n = J->n;
    const double g = J->gamma ? J->gamma[bh % J->H] : 1.0;
    const size_t sd = (size_t)d * d, sc = (size_t)d * dv;
    double *buf = (double *)calloc(sd + 2 * sc + 2 * (size_t)d + (size_t)dv + (size_t)d + (size_t)dv, sizeof(double));
    double *S = buf, *C = S + sd, *G = C + sc, *m = G + sc, *h = m + d;
    double *r = h + d, *a = r + dv, *num = a + d;
    double rho = 1.0, dn;
    int t, j;

    if (J->init.S) {
        memcpy(S, J->init.S + bh * sd, sd * sizeof(double));
        memcpy(C, J->init.C + bh * sc, sc * sizeof(double));
        memcpy(G, J->init.G + bh * sc, sc * sizeof(double));
        memcpy(m, J->init.m + (size_t)bh * d, (size_t)d * sizeof(double));
        memcpy(h, J->init.h + (size_t)bh * d, (size_t)d * sizeof(double));
        if (J->init.rho) rho = J->init.rho[bh];
    }
    for (t = 0; t < n; ++t) {
        const size_t tok = (size_t)bh * n + t;
        ora_step(d, dv, g, J->lam, J->q + tok * d, J->k + tok * d, J->v + tok * dv,
                 S, C, m, G, h, r, a, num, &dn);
        for (j = 0; j < dv; ++j)
            J->out[tok * dv + j] = J->normalize ? num[j] / dn : num[j];
        if (J->den) J->den[tok] = dn;
        rho *= g;
    }
    if (J->fin.S) {
        memcpy(J->fin.S + bh * sd, S, sd * sizeof(double));
        memcpy(J->fin.C + bh * sc, C, sc * sizeof(double));
        memcpy(J->fin.G + bh * sc, G, sc * sizeof(double));
        memcpy(J->fin.m + (size_t)bh * d, m, (size_t)d * sizeof(double));
        memcpy(J->fin.h + (size_t)bh * d, h, (size_t)d * sizeof(double));
        if (J->fin.rho) J->fin.rho[bh] = rho;
    }
    free(buf);
}

static void *fwd_worker(void *arg)
{
    fwd_job *J = (fwd_job *)arg;
    const int total = J->B * J->H;
    for (;;) {
        int bh = __atomic_fetch_add(&J->next, 1, __ATOMIC_RELAXED);
        if (bh >= total) break;
        fwd_head(J, bh);
    }
    return NULL;
}

static void run_pool(void *(*fn)(void *), void *job, int threads, int units)
{
    pthread_t *tid;
    int i, nt = threads < 1 ? 1 : threads;
    if (nt > units) nt = units;
    if (nt <= 1) { fn(job); return; }
    tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nt);
    for (i = 0; i < nt; ++i) pthread_create(&tid[i], NULL, fn, job);
    for (i = 0; i < nt; ++i) pthread_join(tid[i], NULL);
    free(tid);
}

/* Serial-recurrence forward over every (b, h).  Returns 0, or -1 on a bad
 * size.  gamma: [H] or NULL (no decay).  init_* / fin_*: all NULL or all set
 * (the rho pointers may be NULL on their own).  den may be NULL. */
int hla_oracle_forward(int B, int H, int n, int d, int dv,
                       const double *q, const double *k, const double *v,
                       const double *gamma, double lam, int normalize,
                       const double *iS, const double *iC, const double *im,
                       const double *iG, const double *ih, const double *irho,
                       double *out, double *den,
                       double *fS, double *fC, double *fm, double *fG, double *fh,
                       double *frho, int threads)
{
    fwd_job J;
    if (B < 1 || H < 1 || n < 0 || d < 1 || dv < 1) return -1;
    memset(&J, 0, sizeof(J));
    J.B = B; J.H = H; J.n = n; J.d = d; J.dv = dv; J.normalize = normalize;
    J.q = q; J.k = k; J.v = v; J.gamma = gamma; J.lam = lam;
    J.init.S = (double *)iS; J.init.C = (double *)iC; J.init.m = (double *)im;
    J.init.G = (double *)iG; J.init.h = (double *)ih; J.init.rho = (double *)irho;
    J.out = out; J.den = den;
    J.fin.S = fS; J.fin.C = fC; J.fin.m = fm; J.fin.G = fG; J.fin.h = fh; J.fin.rho = frho;
    J.next = 0;
    run_pool(fwd_worker, &J, threads, B * H);
    return 0;
}

/* One decode step for N independent states (state index b*H+h): the same
 * per-token update as the forward, applied in place.  gamma: [H] or NULL. */
int hla_oracle_decode(int B, int H, int d, int dv,
                      const double *q, const double *k, const double *v,
                      const double *gamma, double lam, int normalize,
                      double *S, double *C, double *m, double *G, double *h, double *rho,
                      double *out, double *den, int threads)
{
    /* A decode step is a forward of length 1 that starts from and returns
     * to the same state; forward reads init fully before writing fin. */
    if (B < 1 || H < 1 || d < 1 || dv < 1) return -1;
    return hla_oracle_forward(B, H, 1, d, dv, q, k, v, gamma, lam, normalize,
                              S, C, m, G, h, rho, out, den,
                              S, C, m, G, h, rho, threads);
}

/* Masked semidirect-product composition of `count` segment pairs (earlier a,
 * later b).  rho pointers may be NULL (meaning 1); r_rho may be NULL (not
 * written). */
int hla_oracle_compose(int count, int d, int dv,
                       const double *aS, const double *aC, const double *am,
                       const double *aG, const double *ah, const double *arho,
                       const double *bS, const double *bC, const double *bm,
                       const double *bG, const double *bh, const double *brho,
                       double *rS, double *rC, double *rm, double *rG, double *rh,
                       double *rrho)
{
    int p, i, j, l;
    const size_t sd = (size_t)d * d, sc = (size_t)d * dv;
    if (count < 0 || d < 1 || dv < 1) return -1;
    for (p = 0; p < count; ++p) {
        const double ra = arho ? arho[p] : 1.0, rb = brho ? brho[p] : 1.0;
        const double *Sa = aS + p * sd, *Ca = aC + p * sc, *ma = am + (size_t)p * d;
        const double *Ga = aG + p * sc, *ha = ah + (size_t)p * d;
        const double *Sb = bS + p * sd, *Cb = bC + p * sc, *mb = bm + (size_t)p * d;
        const double *Gb = bG + p * sc, *hb = bh + (size_t)p * d;
        double *S = rS + p * sd, *C = rC + p * sc, *m = rm + (size_t)p * d;
        double *G = rG + p * sc, *h = rh + (size_t)p * d;
        for (i = 0; i < d; ++i) {
            for (j = 0; j < d; ++j) S[i * d + j] = rb * Sa[i * d + j] + Sb[i * d + j];
            for (j = 0; j < dv; ++j) {
                double cross = 0.0;
                for (l = 0; l < d; ++l) cross += Sb[i * d + l] * Ca[(size_t)l * dv + j];
                C[(size_t)i * dv + j] = rb * Ca[(size_t)i * dv + j] + Cb[(size_t)i * dv + j];
                G[(size_t)i * dv + j] = rb * rb * Ga[(size_t)i * dv + j] + Gb[(size_t)i * dv + j] + rb * cross;
            }
            {
                double cross = 0.0;
                for (l = 0; l < d; ++l) cross += Sb[i * d + l] * ma[l];
                m[i] = rb * ma[i] + mb[i];
                h[i] = rb * rb * ha[i] + hb[i] + rb * cross;
            }
        }
        if (rrho) rrho[p] = ra * rb;
    }
    return 0;
}
