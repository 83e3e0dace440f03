/*
 * higher_oracle.c -- plain fp64 CPU oracle for the two other operators of
 * Higher-order Linear Attention: the asymmetric variant (AHLA) and masked
 * third-order HLA.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the bench's CPU
 * baseline use it.  It shares no code, header, table or helper with the HIP
 * library.
 *
 * Both operators are read with the masking principle of the second-order
 * case: every attention factor is causal (a key index never after the query
 * index it meets, diagonal included), and the output at t uses tokens <= t
 * only.
 *
 * AHLA (paperlayer.ai page, sec. 6 and 6.1-6.3; gist.science page,
 * "Methodik" item 2): the left-cascaded product Q (K^T Q)(K^T V), masked:
 *   num_t = sum_{j<=t} sum_{i<=j} g^(t-i) (q_t . k_j)(q_j . k_i) v_i
 *   den_t = the same with every v_i = 1.
 * Streaming summaries (P^KV, m^K, E, n), each decayed by g per token:
 *   P_t = g P + k_t v_t^T          (d x dv)     m_t = g m + k_t     (d)
 *   y_t = P_t^T q_t                              yd_t = q_t . m_t
 *   E_t = g E + k_t y_t^T          (d x dv)     n_t = g n + yd_t k_t (d)
 *   num_t = E_t^T q_t,   den_t = q_t . n_t
 * O(d dv) work and state per token.  Segment composition (earlier a, later
 * b, rho = g^len), which needs the segment sum R = sum_j k_j q_j^T (d x d,
 * not decayed: the O(d^2) chunk memory of sec. 6.1):
 *   P = rho_b P_a + P_b      m = rho_b m_a + m_b
 *   E = rho_b E_a + E_b + rho_b R_b P_a
 *   n = rho_b n_a + n_b + rho_b R_b m_a
 *   R = R_a + R_b            rho = rho_a rho_b
 *
 * Third order (paperlayer.ai page, sec. 7 and 7.1-7.3; gist.science page,
 * "Methodik" item 3 and "Scans dritter Ordnung"): the product A A^T A V with
 * A = Q K^T, masked at every factor:
 *   num_t = sum_{j<=t} sum_{i<=j} sum_{l<=j} (q_t . k_i)(k_i . q_j)(q_j . k_l) v_l
 *   den_t = the same with every v_l = 1.
 * No decay (the pages state the third-order scan exactly for g = 1).
 * Streaming state (S^K, P^KV, m^K, F, Fd):
 *   S_t = S + k k^T,  P_t = P + k v^T,  m_t = m + k
 *   a_t = S_t q_t,  y_t = P_t^T q_t,  yd_t = q_t . m_t
 *   F_t = F + a_t y_t^T,   Fd_t = Fd + yd_t a_t
 *   num_t = F_t^T q_t,   den_t = q_t . Fd_t
 * (F_t equals the naive product S_t S^Q_t P_t with S^Q = sum q q^T, minus
 * the pairs with i > j, minus those with l > j, plus those with both: the
 * three corrections the pages count.)  Segment composition needs, besides
 * the streaming state from zero, S^Q = sum q q^T, M = sum_j S_j q_j q_j^T,
 * N = sum_j q_j y_j^T and Nd = sum_j yd_j q_j (segment-local S_j, y_j):
 *   S = S_a + S_b,  P = P_a + P_b,  m = m_a + m_b,  SQ = SQ_a + SQ_b
 *   F  = F_a + F_b + S_a SQ_b P_a + S_a N_b + M_b P_a
 *   Fd = Fd_a + Fd_b + S_a SQ_b m_a + S_a Nd_b + M_b m_a
 *   M  = M_a + M_b + S_a SQ_b,  N = N_a + N_b + SQ_b P_a,  Nd = Nd_a + Nd_b + SQ_b m_a
 *
 * Layouts: q, k [B,H,n,d], v [B,H,n,dv], out [B,H,n,dv], den [B,H,n]; states
 * indexed by b*H+h, row-major.
 */
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- AHLA */

typedef struct {
    double *P, *m, *E, *n, *R, *rho;
} ahla_state;

/* one token; P, m, E, n (and R when given) updated in place; y (dv) scratch */
static void ahla_step(int d, int dv, double g, const double *q, const double *k, const double *v,
                      double *P, double *m, double *E, double *n, double *R, double *y,
                      double *num, double *den)
{
    int i, j;
    double yd = 0.0, dn = 0.0;
    for (i = 0; i < d; ++i) {
        double *Pi = P + (size_t)i * dv;
        for (j = 0; j < dv; ++j) Pi[j] = g * Pi[j] + k[i] * v[j];
        m[i] = g * m[i] + k[i];
    }
    for (j = 0; j < dv; ++j) y[j] = 0.0;
    for (i = 0; i < d; ++i) {
        const double *Pi = P + (size_t)i * dv;
        for (j = 0; j < dv; ++j) y[j] += q[i] * Pi[j];
        yd += q[i] * m[i];
    }
    for (i = 0; i < d; ++i) {
        double *Ei = E + (size_t)i * dv;
        for (j = 0; j < dv; ++j) Ei[j] = g * Ei[j] + k[i] * y[j];
        n[i] = g * n[i] + yd * k[i];
    }
    if (R)
        for (i = 0; i < d; ++i)
            for (j = 0; j < d; ++j) R[(size_t)i * d + j] += k[i] * q[j];
    for (j = 0; j < dv; ++j) num[j] = 0.0;
    for (i = 0; i < d; ++i) {
        const double *Ei = E + (size_t)i * dv;
        for (j = 0; j < dv; ++j) num[j] += q[i] * Ei[j];
        dn += q[i] * n[i];
    }
    *den = dn;
}

typedef struct {
    int B, H, n, d, dv, normalize;
    const double *q, *k, *v, *gamma;
    ahla_state init;         /* P == NULL: zero state */
    double *out, *den;
    ahla_state fin;          /* P == NULL: not returned; R may be NULL */
    int next;
    pthread_mutex_t mu;
} ahla_job;

static void ahla_head(ahla_job *J, int bh)
{
    const int d = J->d, dv = J->dv, n = J->n;
    const double g = J->gamma ? J->gamma[bh % J->H] : 1.0;
    const size_t sc = (size_t)d * dv;
    double *buf = (double *)calloc(2 * sc + 2 * (size_t)d + (size_t)d * d + 2 * (size_t)dv, sizeof(double));
    double *P = buf, *E = P + sc, *m = E + sc, *nn = m + d, *R = nn + d, *y = R + (size_t)d * d, *num = y + dv;
    double rho = 1.0, dn;
    int t, j;
    if (J->init.P) {
        memcpy(P, J->init.P + bh * sc, sc * sizeof(double));
        memcpy(E, J->init.E + bh * sc, sc * sizeof(double));
        memcpy(m, J->init.m + (size_t)bh * d, (size_t)d * sizeof(double));
        memcpy(nn, J->init.n + (size_t)bh * d, (size_t)d * sizeof(double));
        if (J->init.rho) rho = J->init.rho[bh];
    }
    for (t = 0; t < n; ++t) {
        const size_t tok = (size_t)bh * n + t;
        ahla_step(d, dv, g, J->q + tok * d, J->k + tok * d, J->v + tok * dv, P, m, E, nn,
                  J->fin.R ? R : NULL, y, num, &dn);
        for (j = 0; j < dv; ++j) J->out[tok * dv + j] = J->normalize ? num[j] / dn : num[j];
        if (J->den) J->den[tok] = dn;
        rho *= g;
    }
    if (J->fin.P) {
        memcpy(J->fin.P + bh * sc, P, sc * sizeof(double));
        memcpy(J->fin.E + bh * sc, E, sc * sizeof(double));
        memcpy(J->fin.m + (size_t)bh * d, m, (size_t)d * sizeof(double));
        memcpy(J->fin.n + (size_t)bh * d, nn, (size_t)d * sizeof(double));
        if (J->fin.R) memcpy(J->fin.R + (size_t)bh * d * d, R, (size_t)d * d * sizeof(double));
        if (J->fin.rho) J->fin.rho[bh] = rho;
    }
    free(buf);
}

static void *ahla_worker(void *arg)
{
    ahla_job *J = (ahla_job *)arg;
    for (;;) {
        int bh;
        pthread_mutex_lock(&J->mu);
        bh = J->next++;
        pthread_mutex_unlock(&J->mu);
        if (bh >= J->B * J->H) break;
        ahla_head(J, bh);
    }
    return NULL;
}

/* fin.R, when given, receives sum_j k_j q_j^T over this call's tokens. */
int hla_oracle_ahla_forward(int B, int H, int n, int d, int dv, const double *q, const double *k,
                            const double *v, const double *gamma, int normalize,
                            double *iP, double *im, double *iE, double *in_, double *irho,
                            double *out, double *den,
                            double *fP, double *fm, double *fE, double *fn, double *fR, double *frho,
                            int threads)
{
    ahla_job J;
    pthread_t th[64];
    int i, nt;
    if (B < 1 || H < 1 || n < 0 || d < 1 || dv < 1) return 1;
    memset(&J, 0, sizeof(J));
    J.B = B; J.H = H; J.n = n; J.d = d; J.dv = dv; J.normalize = normalize;
    J.q = q; J.k = k; J.v = v; J.gamma = gamma;
    J.init.P = iP; J.init.m = im; J.init.E = iE; J.init.n = in_; J.init.rho = irho;
    J.out = out; J.den = den;
    J.fin.P = fP; J.fin.m = fm; J.fin.E = fE; J.fin.n = fn; J.fin.R = fR; J.fin.rho = frho;
    pthread_mutex_init(&J.mu, NULL);
    nt = threads < 1 ? 1 : (threads > 64 ? 64 : threads);
    for (i = 0; i < nt; ++i) pthread_create(&th[i], NULL, ahla_worker, &J);
    for (i = 0; i < nt; ++i) pthread_join(th[i], NULL);
    pthread_mutex_destroy(&J.mu);
    return 0;
}

/* a then b, batched over N segment pairs; r must not alias a or b */
int hla_oracle_ahla_compose(int N, int d, int dv,
                            const double *Pa, const double *ma, const double *Ea, const double *na,
                            const double *Ra, const double *rhoa,
                            const double *Pb, const double *mb, const double *Eb, const double *nb,
                            const double *Rb, const double *rhob,
                            double *P, double *m, double *E, double *n, double *R, double *rho)
{
    int s, i, j, l;
    const size_t sc = (size_t)d * dv, sd = (size_t)d * d;
    if (N < 0 || d < 1 || dv < 1) return 1;
    for (s = 0; s < N; ++s) {
        const double rb = rhob[s];
        for (i = 0; i < d; ++i) {
            double cn = 0.0;
            for (l = 0; l < d; ++l) cn += Rb[s * sd + (size_t)i * d + l] * ma[(size_t)s * d + l];
            m[(size_t)s * d + i] = rb * ma[(size_t)s * d + i] + mb[(size_t)s * d + i];
            n[(size_t)s * d + i] = rb * na[(size_t)s * d + i] + nb[(size_t)s * d + i] + rb * cn;
            for (j = 0; j < dv; ++j) {
                double cross = 0.0;
                for (l = 0; l < d; ++l) cross += Rb[s * sd + (size_t)i * d + l] * Pa[s * sc + (size_t)l * dv + j];
                P[s * sc + (size_t)i * dv + j] = rb * Pa[s * sc + (size_t)i * dv + j] + Pb[s * sc + (size_t)i * dv + j];
                E[s * sc + (size_t)i * dv + j] = rb * Ea[s * sc + (size_t)i * dv + j] + Eb[s * sc + (size_t)i * dv + j] + rb * cross;
            }
            for (j = 0; j < d; ++j) R[s * sd + (size_t)i * d + j] = Ra[s * sd + (size_t)i * d + j] + Rb[s * sd + (size_t)i * d + j];
        }
        rho[s] = rhoa[s] * rb;
    }
    return 0;
}

/* ---------------------------------------------------------- third order */

typedef struct {
    double *S, *P, *m, *F, *Fd;   /* streaming state */
    double *SQ, *M, *N, *Nd;      /* segment aggregates (composition only) */
} ho3_state;

static void ho3_step(int d, int dv, const double *q, const double *k, const double *v,
                     double *S, double *P, double *m, double *F, double *Fd,
                     double *SQ, double *M, double *N, double *Nd,
                     double *a, double *y, double *num, double *den)
{
    int i, j;
    double yd = 0.0, dn = 0.0;
    for (i = 0; i < d; ++i) {
        double *Si = S + (size_t)i * d, *Pi = P + (size_t)i * dv;
        for (j = 0; j < d; ++j) Si[j] += k[i] * k[j];
        for (j = 0; j < dv; ++j) Pi[j] += k[i] * v[j];
        m[i] += k[i];
    }
    for (j = 0; j < dv; ++j) y[j] = 0.0;
    for (i = 0; i < d; ++i) {
        const double *Si = S + (size_t)i * d, *Pi = P + (size_t)i * dv;
        double acc = 0.0;
        for (j = 0; j < d; ++j) acc += Si[j] * q[j];
        a[i] = acc;
        for (j = 0; j < dv; ++j) y[j] += q[i] * Pi[j];
        yd += q[i] * m[i];
    }
    for (i = 0; i < d; ++i) {
        double *Fi = F + (size_t)i * dv;
        for (j = 0; j < dv; ++j) Fi[j] += a[i] * y[j];
        Fd[i] += yd * a[i];
    }
    if (SQ) {
        for (i = 0; i < d; ++i) {
            for (j = 0; j < d; ++j) {
                SQ[(size_t)i * d + j] += q[i] * q[j];
                M[(size_t)i * d + j] += a[i] * q[j];
            }
            for (j = 0; j < dv; ++j) N[(size_t)i * dv + j] += q[i] * y[j];
            Nd[i] += yd * q[i];
        }
    }
    for (j = 0; j < dv; ++j) num[j] = 0.0;
    for (i = 0; i < d; ++i) {
        const double *Fi = F + (size_t)i * dv;
        for (j = 0; j < dv; ++j) num[j] += q[i] * Fi[j];
        dn += q[i] * Fd[i];
    }
    *den = dn;
}

typedef struct {
    int B, H, n, d, dv, normalize;
    const double *q, *k, *v;
    ho3_state init;          /* S == NULL: zero state (aggregates never read) */
    double *out, *den;
    ho3_state fin;           /* S == NULL: not returned; SQ == NULL: no aggregates */
    int next;
    pthread_mutex_t mu;
} ho3_job;

static void ho3_head(ho3_job *J, int bh)
{
    const int d = J->d, dv = J->dv, n = J->n;
    const size_t sd = (size_t)d * d, sc = (size_t)d * dv;
    double *buf = (double *)calloc(3 * sd + 3 * sc + 4 * (size_t)d + 2 * (size_t)dv, sizeof(double));
    double *S = buf, *SQ = S + sd, *M = SQ + sd, *P = M + sd, *F = P + sc, *N = F + sc;
    double *m = N + sc, *Fd = m + d, *Nd = Fd + d, *a = Nd + d, *y = a + d, *num = y + dv;
    double dn;
    int t, j;
    const int agg = J->fin.SQ != NULL;
    if (J->init.S) {
        memcpy(S, J->init.S + bh * sd, sd * sizeof(double));
        memcpy(P, J->init.P + bh * sc, sc * sizeof(double));
        memcpy(F, J->init.F + bh * sc, sc * sizeof(double));
        memcpy(m, J->init.m + (size_t)bh * d, (size_t)d * sizeof(double));
        memcpy(Fd, J->init.Fd + (size_t)bh * d, (size_t)d * sizeof(double));
    }
    for (t = 0; t < n; ++t) {
        const size_t tok = (size_t)bh * n + t;
        ho3_step(d, dv, J->q + tok * d, J->k + tok * d, J->v + tok * dv, S, P, m, F, Fd,
                 agg ? SQ : NULL, M, N, Nd, a, y, num, &dn);
        for (j = 0; j < dv; ++j) J->out[tok * dv + j] = J->normalize ? num[j] / dn : num[j];
        if (J->den) J->den[tok] = dn;
    }
    if (J->fin.S) {
        memcpy(J->fin.S + bh * sd, S, sd * sizeof(double));
        memcpy(J->fin.P + bh * sc, P, sc * sizeof(double));
        memcpy(J->fin.F + bh * sc, F, sc * sizeof(double));
        memcpy(J->fin.m + (size_t)bh * d, m, (size_t)d * sizeof(double));
        memcpy(J->fin.Fd + (size_t)bh * d, Fd, (size_t)d * sizeof(double));
        if (agg) {
            memcpy(J->fin.SQ + bh * sd, SQ, sd * sizeof(double));
            memcpy(J->fin.M + bh * sd, M, sd * sizeof(double));
            memcpy(J->fin.N + bh * sc, N, sc * sizeof(double));
            memcpy(J->fin.Nd + (size_t)bh * d, Nd, (size_t)d * sizeof(double));
        }
    }
    free(buf);
}

static void *ho3_worker(void *arg)
{
    ho3_job *J = (ho3_job *)arg;
    for (;;) {
        int bh;
        pthread_mutex_lock(&J->mu);
        bh = J->next++;
        pthread_mutex_unlock(&J->mu);
        if (bh >= J->B * J->H) break;
        ho3_head(J, bh);
    }
    return NULL;
}

/* The aggregates (fSQ, fM, fN, fNd) are only defined for a call from the zero
 * state: returned only when iS is NULL (error otherwise). */
int hla_oracle_ho3_forward(int B, int H, int n, int d, int dv, const double *q, const double *k,
                           const double *v, int normalize,
                           double *iS, double *iP, double *im, double *iF, double *iFd,
                           double *out, double *den,
                           double *fS, double *fP, double *fm, double *fF, double *fFd,
                           double *fSQ, double *fM, double *fN, double *fNd, int threads)
{
    ho3_job J;
    pthread_t th[64];
    int i, nt;
    if (B < 1 || H < 1 || n < 0 || d < 1 || dv < 1) return 1;
    if (iS && fSQ) return 1;
    memset(&J, 0, sizeof(J));
    J.B = B; J.H = H; J.n = n; J.d = d; J.dv = dv; J.normalize = normalize;
    J.q = q; J.k = k; J.v = v;
    J.init.S = iS; J.init.P = iP; J.init.m = im; J.init.F = iF; J.init.Fd = iFd;
    J.out = out; J.den = den;
    J.fin.S = fS; J.fin.P = fP; J.fin.m = fm; J.fin.F = fF; J.fin.Fd = fFd;
    J.fin.SQ = fSQ; J.fin.M = fM; J.fin.N = fN; J.fin.Nd = fNd;
    pthread_mutex_init(&J.mu, NULL);
    nt = threads < 1 ? 1 : (threads > 64 ? 64 : threads);
    for (i = 0; i < nt; ++i) pthread_create(&th[i], NULL, ho3_worker, &J);
    for (i = 0; i < nt; ++i) pthread_join(th[i], NULL);
    pthread_mutex_destroy(&J.mu);
    return 0;
}

/* Xab = X_a (d x dv) + the sum over l of A(i, l) B(l, j) for a batch entry */
static void mat_acc(int d, int cols, const double *A, const double *Bm, double *out)
{
    int i, j, l;
    for (i = 0; i < d; ++i)
        for (j = 0; j < cols; ++j) {
            double acc = 0.0;
            for (l = 0; l < d; ++l) acc += A[(size_t)i * d + l] * Bm[(size_t)l * cols + j];
            out[(size_t)i * cols + j] += acc;
        }
}

/* a then b, batched over N segment pairs, every one of the nine parts;
 * r must not alias a or b. */
int hla_oracle_ho3_compose(int N, int d, int dv,
                           const double *Sa, const double *Pa, const double *ma, const double *Fa,
                           const double *Fda, const double *SQa, const double *Ma, const double *Na,
                           const double *Nda,
                           const double *Sb, const double *Pb, const double *mb, const double *Fb,
                           const double *Fdb, const double *SQb, const double *Mb, const double *Nb,
                           const double *Ndb,
                           double *S, double *P, double *m, double *F, double *Fd, double *SQ, double *M,
                           double *Nn, double *Nd)
{
    int s;
    size_t e;
    const size_t sd = (size_t)d * d, sc = (size_t)d * dv;
    double *T = (double *)malloc(sd * sizeof(double));   /* S_a SQ_b */
    if (!T || N < 0 || d < 1 || dv < 1) {
        free(T);
        return 1;
    }
    for (s = 0; s < N; ++s) {
        const double *sa = Sa + s * sd, *sqb = SQb + s * sd, *mbb = Mb + s * sd;
        const double *pa = Pa + s * sc, *vma = ma + (size_t)s * d;
        memset(T, 0, sd * sizeof(double));
        mat_acc(d, d, sa, sqb, T);
        for (e = 0; e < sd; ++e) {
            S[s * sd + e] = sa[e] + Sb[s * sd + e];
            SQ[s * sd + e] = SQa[s * sd + e] + sqb[e];
            M[s * sd + e] = Ma[s * sd + e] + mbb[e] + T[e];
        }
        for (e = 0; e < sc; ++e) {
            P[s * sc + e] = pa[e] + Pb[s * sc + e];
            F[s * sc + e] = Fa[s * sc + e] + Fb[s * sc + e];
            Nn[s * sc + e] = Na[s * sc + e] + Nb[s * sc + e];
        }
        for (e = 0; e < (size_t)d; ++e) {
            m[(size_t)s * d + e] = vma[e] + mb[(size_t)s * d + e];
            Fd[(size_t)s * d + e] = Fda[(size_t)s * d + e] + Fdb[(size_t)s * d + e];
            Nd[(size_t)s * d + e] = Nda[(size_t)s * d + e] + Ndb[(size_t)s * d + e];
        }
        /* F += S_a SQ_b P_a + S_a N_b + M_b P_a ;  Fd likewise with m_a, Nd_b */
        mat_acc(d, dv, T, pa, F + s * sc);
        mat_acc(d, dv, sa, Nb + s * sc, F + s * sc);
        mat_acc(d, dv, mbb, pa, F + s * sc);
        mat_acc(d, 1, T, vma, Fd + (size_t)s * d);
        mat_acc(d, 1, sa, Ndb + (size_t)s * d, Fd + (size_t)s * d);
        mat_acc(d, 1, mbb, vma, Fd + (size_t)s * d);
        /* N += SQ_b P_a ; Nd += SQ_b m_a */
        mat_acc(d, dv, sqb, pa, Nn + s * sc);
        mat_acc(d, 1, sqb, vma, Nd + (size_t)s * d);
    }
    free(T);
    return 0;
}
