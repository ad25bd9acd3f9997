/*
 * oracle.c -- plain fp64 CPU oracle for kernelized linear attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or
 * calls this file: only the tests, the package smoke check and the
 * CPU-baseline leg of the benchmark use it.  It shares no code, header,
 * table or constant with the HIP library; every number it needs is written
 * here from the definitions on the pages:
 *
 *   [KZ]  "The Kernel Zoo: Performers, Fast Weight Programmers, and the
 *          Capacity-Approximation Tradeoff in Linear Attention" (prathamp.com)
 *   [RF]  "Reassociate a feature-map kernel without claiming exact softmax"
 *          (study.greatitself.com)
 *   [LA]  "Linear attention & kernelized approximations" (interactive chapter)
 *   [PF]  "Performer -- Random Feature Softmax Approximation" (lizeman.github.io)
 *
 * Everything is computed token by token, in the order the definitions give,
 * in IEEE double precision (built with -ffp-contract=off, no fast-math).
 * There is no chunking, blocking or reordering: chunk length and segment
 * count are properties of the GPU path only.
 *
 * Layouts (all row-major, contiguous):
 *   x, q, k   [BH, N, d]      v, out  [BH, N, dv]
 *   omega     [r, d]          phi     [BH, N, r]
 *   S         [BH, r, dv]     z       [BH, r]
 * BH is the flattened batch*heads count; heads are independent.
 *
 * Return value: 0 on success, -1 on an invalid argument.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Feature-map kinds and readout modes (the oracle's own numbering). */
#define ORC_PHI_IDENTITY 0
#define ORC_PHI_ELU1 1
#define ORC_PHI_FAVOR 2
#define ORC_PHI_DPFP 3
#define ORC_NORM_ATTN 0
#define ORC_NORM_NONE 1

typedef struct {
    int phi;        /* one of ORC_PHI_*                                   */
    int r;          /* feature dimension                                  */
    int nu;         /* DPFP shift count                                   */
    int sum_norm;   /* 1: divide each feature vector by its (clamped) sum */
    int norm;       /* ORC_NORM_ATTN or ORC_NORM_NONE                     */
    double scale;   /* x <- scale * x before the map                      */
    double eps;     /* lower clamp of denominators                        */
} orc_cfg;

/* Feature dimension implied by the kind ([KZ] sec. 2.5 table, sec. 6.3,
 * sec. 4.2): identity and ELU+1 keep d, DPFP-nu gives 2*d*nu, FAVOR+ gives
 * one feature per row of omega. */
static int orc_expected_r(const orc_cfg *c, long d, long r_omega)
{
    switch (c->phi) {
    case ORC_PHI_IDENTITY:
    case ORC_PHI_ELU1:
        return (int)d;
    case ORC_PHI_FAVOR:
        return (int)r_omega;
    case ORC_PHI_DPFP:
        return (int)(2 * d * c->nu);
    default:
        return -1;
    }
}

static int orc_check(const orc_cfg *c, long d)
{
    if (c->phi < ORC_PHI_IDENTITY || c->phi > ORC_PHI_DPFP) return -1;
    if (c->norm != ORC_NORM_ATTN && c->norm != ORC_NORM_NONE) return -1;
    if (!(c->eps > 0.0)) return -1;
    if (c->r <= 0 || d <= 0) return -1;
    if (c->phi == ORC_PHI_DPFP && (c->nu < 1 || c->nu > 2 * d - 1)) return -1;
    if (orc_expected_r(c, d, c->r) != c->r) return -1;
    return 0;
}

/*
 * phi(x) for one vector x of length d, written to out[r].
 * work must hold at least max(d, 2d) doubles.
 *
 *  identity ([KZ] sec. 1.3, [LA] step 2):  phi(x) = x
 *  ELU+1    ([KZ] running example, [PF] sec. 1):  phi(x)_i = elu(x_i) + 1,
 *           elu(a) = a for a > 0, exp(a) - 1 otherwise (alpha = 1)
 *  FAVOR+   ([KZ] sec. 4.2 boxed map and sec. 5.4; [PF] sketch):
 *           phi(x)_i = exp(omega_i . x - ||x||^2 / 2) / sqrt(m)
 *  DPFP-nu  ([KZ] sec. 6.3): kt = relu([x, -x]) in R^{2d};
 *           block s (s = 1..nu) holds kt_i * kt_{(i+s) mod 2d}, i < 2d
 *  sum normalisation ([KZ] sec. 7.2): phi <- phi / sum_j phi_j, with the
 *           sum clamped below by eps so that an all-zero map stays zero.
 * The input is first multiplied by cfg->scale (1 for the pages' worked
 * examples; d^-1/4 puts the 1/sqrt(d) softmax temperature into q and k,
 * as [KZ] sec. 3.3 says it can be absorbed).
 */
static void orc_phi(const orc_cfg *c, const double *x, long d,
                    const double *omega, double *out, double *work)
{
    double *u = work; /* scaled input */
    for (long i = 0; i < d; ++i) u[i] = c->scale * x[i];

    if (c->phi == ORC_PHI_IDENTITY) {
        for (long i = 0; i < d; ++i) out[i] = u[i];
    } else if (c->phi == ORC_PHI_ELU1) {
        for (long i = 0; i < d; ++i) {
            double elu = u[i] > 0.0 ? u[i] : expm1(u[i]);
            out[i] = elu + 1.0;
        }
    } else if (c->phi == ORC_PHI_FAVOR) {
        double sq = 0.0;
        for (long i = 0; i < d; ++i) sq += u[i] * u[i];
        double inv_sqrt_m = 1.0 / sqrt((double)c->r);
        for (long f = 0; f < c->r; ++f) {
            double dot = 0.0;
            for (long i = 0; i < d; ++i) dot += omega[f * d + i] * u[i];
            out[f] = exp(dot - 0.5 * sq) * inv_sqrt_m;
        }
    } else { /* DPFP */
        long two_d = 2 * d;
        double *kt = work + d;
        for (long i = 0; i < d; ++i) {
            kt[i] = u[i] > 0.0 ? u[i] : 0.0;
            kt[d + i] = -u[i] > 0.0 ? -u[i] : 0.0;
        }
        for (long s = 1; s <= c->nu; ++s)
            for (long i = 0; i < two_d; ++i)
                out[(s - 1) * two_d + i] = kt[i] * kt[(i + s) % two_d];
    }

    if (c->sum_norm) {
        double sum = 0.0;
        for (long f = 0; f < c->r; ++f) sum += out[f];
        double den = sum > c->eps ? sum : c->eps;
        for (long f = 0; f < c->r; ++f) out[f] /= den;
    }
}

/* Readout of one query against summaries (S, z) ([RF] first paragraph;
 * [KZ] sec. 5.4 ratio; [PF] sketch clamp):
 *   num = phi(q)^T S,  den = phi(q) . z,
 *   out = num / max(den, eps)  (ATTN)   or   out = num  (NONE). */
static void orc_readout(const orc_cfg *c, const double *pq, const double *S,
                        const double *z, long dv, double *out)
{
    double den = 0.0;
    for (long f = 0; f < c->r; ++f) den += pq[f] * z[f];
    for (long n = 0; n < dv; ++n) {
        double num = 0.0;
        for (long f = 0; f < c->r; ++f) num += pq[f] * S[f * dv + n];
        if (c->norm == ORC_NORM_ATTN) {
            double dd = den > c->eps ? den : c->eps;
            out[n] = num / dd;
        } else {
            out[n] = num;
        }
    }
}

/* One additive fast-weight write ([KZ] sec. 1.2-1.3):
 *   S <- S + phi(k) v^T,  z <- z + phi(k). */
static void orc_write(const orc_cfg *c, const double *pk, const double *v,
                      long dv, double *S, double *z)
{
    for (long f = 0; f < c->r; ++f) {
        for (long n = 0; n < dv; ++n) S[f * dv + n] += pk[f] * v[n];
        z[f] += pk[f];
    }
}

int orc_feature_dim(int phi, int nu, long d, long r_omega)
{
    orc_cfg c;
    memset(&c, 0, sizeof c);
    c.phi = phi;
    c.nu = nu;
    return orc_expected_r(&c, d, r_omega);
}

int orc_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* phi for every row of x [BH, N, d] -> out [BH, N, r]. */
int orc_featuremap(int phi, int r, int nu, int sum_norm, double scale,
                   double eps, const double *x, long BH, long N, long d,
                   const double *omega, double *out)
{
    orc_cfg c = {phi, r, nu, sum_norm, ORC_NORM_ATTN, scale, eps};
    if (orc_check(&c, d) || BH < 0 || N < 0) return -1;
    if (phi == ORC_PHI_FAVOR && !omega) return -1;
    long rows = BH * N;
#pragma omp parallel
    {
        double *work = (double *)malloc(sizeof(double) * 3 * (size_t)d);
#pragma omp for schedule(static)
        for (long i = 0; i < rows; ++i)
            orc_phi(&c, x + i * d, d, omega, out + i * (long)r, work);
        free(work);
    }
    return 0;
}

/*
 * Bidirectional reassociated form ([RF] first paragraph; [PF] sec. 2 step 5;
 * [LA] "build the state once"):
 *   S = sum_j phi(k_j) v_j^T,  z = sum_j phi(k_j),
 *   out_i = readout(phi(q_i), S, z).
 * S_out / z_out may be NULL.
 */
int orc_bidir(int phi, int r, int nu, int sum_norm, int norm, double scale,
              double eps, const double *q, const double *k, const double *v,
              long BH, long N, long d, long dv, const double *omega,
              double *out, double *S_out, double *z_out)
{
    orc_cfg c = {phi, r, nu, sum_norm, norm, scale, eps};
    if (orc_check(&c, d) || BH < 0 || N < 0 || dv <= 0) return -1;
    if (phi == ORC_PHI_FAVOR && !omega) return -1;
#pragma omp parallel
    {
        double *work = (double *)malloc(sizeof(double) * 3 * (size_t)d);
        double *pk = (double *)malloc(sizeof(double) * (size_t)r);
        double *pq = (double *)malloc(sizeof(double) * (size_t)r);
        double *S = (double *)malloc(sizeof(double) * (size_t)r * dv);
        double *z = (double *)malloc(sizeof(double) * (size_t)r);
#pragma omp for schedule(dynamic, 1)
        for (long bh = 0; bh < BH; ++bh) {
            memset(S, 0, sizeof(double) * (size_t)r * dv);
            memset(z, 0, sizeof(double) * (size_t)r);
            for (long j = 0; j < N; ++j) {
                orc_phi(&c, k + (bh * N + j) * d, d, omega, pk, work);
                orc_write(&c, pk, v + (bh * N + j) * dv, dv, S, z);
            }
            for (long i = 0; i < N; ++i) {
                orc_phi(&c, q + (bh * N + i) * d, d, omega, pq, work);
                orc_readout(&c, pq, S, z, dv, out + (bh * N + i) * dv);
            }
            if (S_out) memcpy(S_out + bh * (long)r * dv, S, sizeof(double) * (size_t)r * dv);
            if (z_out) memcpy(z_out + bh * (long)r, z, sizeof(double) * (size_t)r);
        }
        free(work); free(pk); free(pq); free(S); free(z);
    }
    return 0;
}

/*
 * Causal prefix-sum recurrence ([KZ] sec. 1.3 and sec. 5.4; [RF] causal
 * paragraph; [PF] sec. 2 step 5): starting from (S, z) = 0 -- the empty fast
 * weight memory W(0) = 0 of [KZ] sec. 1.2 -- or from the caller's state when
 * state_in is set, for t = 1..N in order:
 *   S <- S + phi(k_t) v_t^T,  z <- z + phi(k_t)      (write first)
 *   out_t = readout(phi(q_t), S, z)                   (then read)
 * so query t sees keys 1..t.  S and z are in/out: on return they hold the
 * state after the last token.
 */
int orc_causal(int phi, int r, int nu, int sum_norm, int norm, double scale,
               double eps, const double *q, const double *k, const double *v,
               long BH, long N, long d, long dv, const double *omega,
               int state_in, double *S, double *z, double *out)
{
    orc_cfg c = {phi, r, nu, sum_norm, norm, scale, eps};
    if (orc_check(&c, d) || BH < 0 || N < 0 || dv <= 0 || !S || !z) return -1;
    if (phi == ORC_PHI_FAVOR && !omega) return -1;
#pragma omp parallel
    {
        double *work = (double *)malloc(sizeof(double) * 3 * (size_t)d);
        double *pk = (double *)malloc(sizeof(double) * (size_t)r);
        double *pq = (double *)malloc(sizeof(double) * (size_t)r);
#pragma omp for schedule(dynamic, 1)
        for (long bh = 0; bh < BH; ++bh) {
            double *Sh = S + bh * (long)r * dv;
            double *zh = z + bh * (long)r;
            if (!state_in) {
                memset(Sh, 0, sizeof(double) * (size_t)r * dv);
                memset(zh, 0, sizeof(double) * (size_t)r);
            }
            for (long t = 0; t < N; ++t) {
                orc_phi(&c, k + (bh * N + t) * d, d, omega, pk, work);
                orc_write(&c, pk, v + (bh * N + t) * dv, dv, Sh, zh);
                orc_phi(&c, q + (bh * N + t) * d, d, omega, pq, work);
                orc_readout(&c, pq, Sh, zh, dv, out + (bh * N + t) * dv);
            }
        }
        free(work); free(pk); free(pq);
    }
    return 0;
}

/* Single-token decode step ([KZ] sec. 1.2 steps 2-3): one iteration of the
 * causal recurrence on the caller's (S, z), for q, k, v [BH, d] / [BH, dv]. */
int orc_decode(int phi, int r, int nu, int sum_norm, int norm, double scale,
               double eps, const double *q, const double *k, const double *v,
               long BH, long d, long dv, const double *omega, double *S,
               double *z, double *out)
{
    return orc_causal(phi, r, nu, sum_norm, norm, scale, eps, q, k, v, BH, 1,
                      d, dv, omega, 1, S, z, out);
}

/*
 * Explicit N x N form ([LA] "the naive way: rescan every key"; [KZ] opening
 * paragraph, left-hand side of the associativity identity):
 *   A_ij = phi(q_i) . phi(k_j)        (only j <= i when causal)
 *   num_i = sum_j A_ij v_j,  den_i = sum_j A_ij
 * plus, when state_in is set, the contribution phi(q_i)^T S0 and phi(q_i).z0
 * of a carried-in state.  Output as in orc_readout.  Quadratic in N: for
 * small cases only.
 */
int orc_explicit(int phi, int r, int nu, int sum_norm, int norm, double scale,
                 double eps, int causal, const double *q, const double *k,
                 const double *v, long BH, long N, long d, long dv,
                 const double *omega, int state_in, const double *S0,
                 const double *z0, double *out)
{
    orc_cfg c = {phi, r, nu, sum_norm, norm, scale, eps};
    if (orc_check(&c, d) || BH < 0 || N < 0 || dv <= 0) return -1;
    if (phi == ORC_PHI_FAVOR && !omega) return -1;
    if (state_in && (!S0 || !z0)) return -1;
#pragma omp parallel
    {
        double *work = (double *)malloc(sizeof(double) * 3 * (size_t)d);
        double *pq = (double *)malloc(sizeof(double) * (size_t)r);
        double *pk = (double *)malloc(sizeof(double) * (size_t)r * (N > 0 ? N : 1));
        double *num = (double *)malloc(sizeof(double) * (size_t)dv);
#pragma omp for schedule(dynamic, 1)
        for (long bh = 0; bh < BH; ++bh) {
            for (long j = 0; j < N; ++j)
                orc_phi(&c, k + (bh * N + j) * d, d, omega, pk + j * (long)r, work);
            for (long i = 0; i < N; ++i) {
                orc_phi(&c, q + (bh * N + i) * d, d, omega, pq, work);
                double den = 0.0;
                for (long n = 0; n < dv; ++n) num[n] = 0.0;
                long jmax = causal ? i + 1 : N;
                for (long j = 0; j < jmax; ++j) {
                    double a = 0.0;
                    for (long f = 0; f < r; ++f) a += pq[f] * pk[j * (long)r + f];
                    for (long n = 0; n < dv; ++n) num[n] += a * v[(bh * N + j) * dv + n];
                    den += a;
                }
                if (state_in) {
                    const double *Sh = S0 + bh * (long)r * dv;
                    const double *zh = z0 + bh * (long)r;
                    for (long f = 0; f < r; ++f) {
                        for (long n = 0; n < dv; ++n) num[n] += pq[f] * Sh[f * dv + n];
                        den += pq[f] * zh[f];
                    }
                }
                double *o = out + (bh * N + i) * dv;
                for (long n = 0; n < dv; ++n) {
                    if (norm == ORC_NORM_ATTN) {
                        double dd = den > eps ? den : eps;
                        o[n] = num[n] / dd;
                    } else {
                        o[n] = num[n];
                    }
                }
            }
        }
        free(work); free(pq); free(pk); free(num);
    }
    return 0;
}

/*
 * Orthogonal random features ([PF] sec. 2 step 4; [KZ] sec. 5.1-5.3):
 * omega [r, d] from ceil(r/d) independent blocks.  Block b takes the rows of
 * the d x d Gaussian matrix gauss[b] in order and applies Gram-Schmidt:
 * subtract from each row its projections on the earlier (orthonormal) rows,
 * then divide by its norm.  Row f of the block is then scaled to the length
 * of the independent Gaussian vector len_gauss[f] (chi(d)-distributed,
 * [PF] sec. 2 step 4), or to sqrt(d) when len_gauss is NULL (the fixed
 * length of [KZ] sec. 5.3).  The last block keeps its first r - (b*d) rows.
 *   gauss      [ceil(r/d), d, d]     len_gauss  [ceil(r/d) * d, d] or NULL
 */
int orc_orf(const double *gauss, const double *len_gauss, long r, long d, double *omega)
{
    if (!gauss || !omega || r < 0 || d < 1)
        return -1;
    const long nblk = (r + d - 1) / d;
    double *e = (double *)malloc((size_t)(d * d) * sizeof(double));
    if (!e)
        return -1;
    for (long b = 0; b < nblk; ++b) {
        const double *g = gauss + b * d * d;
        for (long i = 0; i < d; ++i) {
            double *ei = e + i * d;
            for (long k = 0; k < d; ++k)
                ei[k] = g[i * d + k];
            for (long j = 0; j < i; ++j) {
                const double *ej = e + j * d;
                double dot = 0.0;
                for (long k = 0; k < d; ++k)
                    dot += g[i * d + k] * ej[k];
                for (long k = 0; k < d; ++k)
                    ei[k] -= dot * ej[k];
            }
            double nrm = 0.0;
            for (long k = 0; k < d; ++k)
                nrm += ei[k] * ei[k];
            nrm = sqrt(nrm);
            for (long k = 0; k < d; ++k)
                ei[k] /= nrm;
        }
        for (long i = 0; i < d && b * d + i < r; ++i) {
            const long f = b * d + i;
            double len = sqrt((double)d);
            if (len_gauss) {
                double s = 0.0;
                for (long k = 0; k < d; ++k)
                    s += len_gauss[f * d + k] * len_gauss[f * d + k];
                len = sqrt(s);
            }
            for (long k = 0; k < d; ++k)
                omega[f * d + k] = e[i * d + k] * len;
        }
    }
    free(e);
    return 0;
}

/*
 * Backward pass: the gradients of a loss L with respect to q, k and v given
 * dL/dout ([RF] par. 6 asks for gradient error to be evaluated; the
 * derivatives are the chain rule through the definitions above).  With
 * D_i = max(den_i, eps):
 *   ATTN: dnum_i = dout_i / D_i,  dden_i = -(dout_i . out_i) / D_i when
 *         den_i > eps (0 where the clamp holds D_i fixed)
 *   NONE: dnum_i = dout_i,        dden_i = 0
 *   dphi(q_i) = S_i dnum_i + z_i dden_i      (S_i, z_i: what query i read)
 *   dphi(k_j) = sum over the queries i that see key j of
 *               phi(q_i) (dnum_i . v_j + dden_i)
 *   dv_j      = sum over the same i of dnum_i (phi(q_i) . phi(k_j))
 * and dx = scale * J_phi(u)^T dphi at u = scale * x, J_phi from the map's
 * definition (orc_phi_backward).
 */

/* dx = scale * J_phi(u)^T dphi for one vector x (u = scale * x).
 * work must hold at least 3d + 2r doubles. */
static void orc_phi_backward(const orc_cfg *c, const double *x, long d, const double *omega,
                             const double *dphi, double *dx, double *work)
{
    double *u = work;                 /* d */
    double *kt = work + d;            /* 2d (DPFP) */
    double *p = work + 3 * d;         /* r: the map before sum normalisation */
    double *dp = work + 3 * d + c->r; /* r */
    for (long i = 0; i < d; ++i) u[i] = c->scale * x[i];
    long r = c->r;

    /* the map before normalisation */
    if (c->phi == ORC_PHI_IDENTITY) {
        for (long i = 0; i < d; ++i) p[i] = u[i];
    } else if (c->phi == ORC_PHI_ELU1) {
        for (long i = 0; i < d; ++i) p[i] = (u[i] > 0.0 ? u[i] : expm1(u[i])) + 1.0;
    } else if (c->phi == ORC_PHI_FAVOR) {
        double sq = 0.0;
        for (long i = 0; i < d; ++i) sq += u[i] * u[i];
        for (long f = 0; f < r; ++f) {
            double dot = 0.0;
            for (long i = 0; i < d; ++i) dot += omega[f * d + i] * u[i];
            p[f] = exp(dot - 0.5 * sq) / sqrt((double)r);
        }
    } else {
        for (long i = 0; i < d; ++i) {
            kt[i] = u[i] > 0.0 ? u[i] : 0.0;
            kt[d + i] = -u[i] > 0.0 ? -u[i] : 0.0;
        }
        long two_d = 2 * d;
        for (long s = 1; s <= c->nu; ++s)
            for (long i = 0; i < two_d; ++i)
                p[(s - 1) * two_d + i] = kt[i] * kt[(i + s) % two_d];
    }

    /* through the sum normalisation phi = p / max(sum p, eps) */
    if (c->sum_norm) {
        double sum = 0.0;
        for (long f = 0; f < r; ++f) sum += p[f];
        double den = sum > c->eps ? sum : c->eps;
        double dot = 0.0; /* dphi . phi */
        for (long f = 0; f < r; ++f) dot += dphi[f] * (p[f] / den);
        for (long f = 0; f < r; ++f)
            dp[f] = (dphi[f] - (sum > c->eps ? dot : 0.0)) / den;
    } else {
        for (long f = 0; f < r; ++f) dp[f] = dphi[f];
    }

    /* through the map */
    double *du = dx;
    if (c->phi == ORC_PHI_IDENTITY) {
        for (long i = 0; i < d; ++i) du[i] = dp[i];
    } else if (c->phi == ORC_PHI_ELU1) {
        for (long i = 0; i < d; ++i) du[i] = dp[i] * (u[i] > 0.0 ? 1.0 : exp(u[i]));
    } else if (c->phi == ORC_PHI_FAVOR) {
        /* d p_f / d u = p_f (omega_f - u) */
        double w = 0.0;
        for (long f = 0; f < r; ++f) w += dp[f] * p[f];
        for (long i = 0; i < d; ++i) {
            double s = 0.0;
            for (long f = 0; f < r; ++f) s += dp[f] * p[f] * omega[f * d + i];
            du[i] = s - w * u[i];
        }
    } else {
        long two_d = 2 * d;
        double *dkt = p; /* p is no longer needed */
        for (long m = 0; m < two_d; ++m) dkt[m] = 0.0;
        for (long s = 1; s <= c->nu; ++s)
            for (long i = 0; i < two_d; ++i) {
                double g = dp[(s - 1) * two_d + i];
                dkt[i] += g * kt[(i + s) % two_d];
                dkt[(i + s) % two_d] += g * kt[i];
            }
        for (long i = 0; i < d; ++i)
            du[i] = (u[i] > 0.0 ? dkt[i] : 0.0) - (-u[i] > 0.0 ? dkt[d + i] : 0.0);
    }
    for (long i = 0; i < d; ++i) dx[i] = c->scale * du[i];
}

/* dnum, dden of one query from its readout inputs and dout. */
static void orc_readout_backward(const orc_cfg *c, const double *pq, const double *S,
                                 const double *z, long dv, const double *dout, double *dnum,
                                 double *dden)
{
    double den = 0.0;
    for (long f = 0; f < c->r; ++f) den += pq[f] * z[f];
    if (c->norm == ORC_NORM_ATTN) {
        double D = den > c->eps ? den : c->eps;
        double go = 0.0; /* dout . out */
        for (long n = 0; n < dv; ++n) {
            double num = 0.0;
            for (long f = 0; f < c->r; ++f) num += pq[f] * S[f * dv + n];
            go += dout[n] * (num / D);
            dnum[n] = dout[n] / D;
        }
        *dden = den > c->eps ? -go / D : 0.0;
    } else {
        for (long n = 0; n < dv; ++n) dnum[n] = dout[n];
        *dden = 0.0;
    }
}

/* dphi(q) = S dnum + z dden */
static void orc_dphi_q(const orc_cfg *c, const double *S, const double *z, long dv,
                       const double *dnum, double dden, double *dpq)
{
    for (long f = 0; f < c->r; ++f) {
        double s = z[f] * dden;
        for (long n = 0; n < dv; ++n) s += S[f * dv + n] * dnum[n];
        dpq[f] = s;
    }
}

/* key side from the accumulated G = sum phi(q_i) dnum_i^T, g = sum phi(q_i) dden_i */
static void orc_key_grads(const orc_cfg *c, const double *G, const double *g, const double *pk,
                          const double *v, long dv, double *dpk, double *dvj)
{
    for (long f = 0; f < c->r; ++f) {
        double s = g[f];
        for (long n = 0; n < dv; ++n) s += G[f * dv + n] * v[n];
        dpk[f] = s;
    }
    for (long n = 0; n < dv; ++n) {
        double s = 0.0;
        for (long f = 0; f < c->r; ++f) s += G[f * dv + n] * pk[f];
        dvj[n] = s;
    }
}

/* Gradients of the bidirectional form (every query sees every key). */
int orc_bidir_backward(int phi, int r, int nu, int sum_norm, int norm, double scale, double eps,
                       const double *q, const double *k, const double *v, const double *dout,
                       long BH, long N, long d, long dv, const double *omega, double *dq,
                       double *dk, double *dvo)
{
    orc_cfg c = {phi, r, nu, sum_norm, norm, scale, eps};
    if (orc_check(&c, d) || BH < 0 || N < 0 || dv <= 0) return -1;
    if (phi == ORC_PHI_FAVOR && !omega) return -1;
#pragma omp parallel
    {
        double *work = (double *)malloc(sizeof(double) * (3 * (size_t)d + 2 * (size_t)r));
        double *pk = (double *)malloc(sizeof(double) * (size_t)r);
        double *pq = (double *)malloc(sizeof(double) * (size_t)r);
        double *dp = (double *)malloc(sizeof(double) * (size_t)r);
        double *S = (double *)malloc(sizeof(double) * (size_t)r * dv);
        double *z = (double *)malloc(sizeof(double) * (size_t)r);
        double *G = (double *)malloc(sizeof(double) * (size_t)r * dv);
        double *g = (double *)malloc(sizeof(double) * (size_t)r);
        double *dnum = (double *)malloc(sizeof(double) * (size_t)dv);
#pragma omp for schedule(dynamic, 1)
        for (long bh = 0; bh < BH; ++bh) {
            memset(S, 0, sizeof(double) * (size_t)r * dv);
            memset(z, 0, sizeof(double) * (size_t)r);
            memset(G, 0, sizeof(double) * (size_t)r * dv);
            memset(g, 0, sizeof(double) * (size_t)r);
            for (long j = 0; j < N; ++j) {
                orc_phi(&c, k + (bh * N + j) * d, d, omega, pk, work);
                orc_write(&c, pk, v + (bh * N + j) * dv, dv, S, z);
            }
            for (long i = 0; i < N; ++i) {
                double dden;
                orc_phi(&c, q + (bh * N + i) * d, d, omega, pq, work);
                orc_readout_backward(&c, pq, S, z, dv, dout + (bh * N + i) * dv, dnum, &dden);
                orc_dphi_q(&c, S, z, dv, dnum, dden, dp);
                orc_phi_backward(&c, q + (bh * N + i) * d, d, omega, dp, dq + (bh * N + i) * d, work);
                for (long f = 0; f < r; ++f) {
                    for (long n = 0; n < dv; ++n) G[f * dv + n] += pq[f] * dnum[n];
                    g[f] += pq[f] * dden;
                }
            }
            for (long j = 0; j < N; ++j) {
                orc_phi(&c, k + (bh * N + j) * d, d, omega, pk, work);
                orc_key_grads(&c, G, g, pk, v + (bh * N + j) * dv, dv, dp, dvo + (bh * N + j) * dv);
                orc_phi_backward(&c, k + (bh * N + j) * d, d, omega, dp, dk + (bh * N + j) * d, work);
            }
        }
        free(work); free(pk); free(pq); free(dp); free(S); free(z); free(G); free(g); free(dnum);
    }
    return 0;
}

/* Gradients of the causal recurrence from zero state: a forward sweep
 * (query i reads the state after key i) gives dq and stores phi(q_i),
 * dnum_i, dden_i; a backward sweep accumulates G, g over the queries
 * i >= j that see key j. */
int orc_causal_backward(int phi, int r, int nu, int sum_norm, int norm, double scale, double eps,
                        const double *q, const double *k, const double *v, const double *dout,
                        long BH, long N, long d, long dv, const double *omega, double *dq,
                        double *dk, double *dvo)
{
    orc_cfg c = {phi, r, nu, sum_norm, norm, scale, eps};
    if (orc_check(&c, d) || BH < 0 || N < 0 || dv <= 0) return -1;
    if (phi == ORC_PHI_FAVOR && !omega) return -1;
#pragma omp parallel
    {
        double *work = (double *)malloc(sizeof(double) * (3 * (size_t)d + 2 * (size_t)r));
        double *pk = (double *)malloc(sizeof(double) * (size_t)r);
        double *dp = (double *)malloc(sizeof(double) * (size_t)r);
        double *S = (double *)malloc(sizeof(double) * (size_t)r * dv);
        double *z = (double *)malloc(sizeof(double) * (size_t)r);
        double *PQ = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1) * r);
        double *DN = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1) * dv);
        double *DD = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
#pragma omp for schedule(dynamic, 1)
        for (long bh = 0; bh < BH; ++bh) {
            memset(S, 0, sizeof(double) * (size_t)r * dv);
            memset(z, 0, sizeof(double) * (size_t)r);
            for (long t = 0; t < N; ++t) {
                orc_phi(&c, k + (bh * N + t) * d, d, omega, pk, work);
                orc_write(&c, pk, v + (bh * N + t) * dv, dv, S, z);
                double *pq = PQ + t * r;
                orc_phi(&c, q + (bh * N + t) * d, d, omega, pq, work);
                orc_readout_backward(&c, pq, S, z, dv, dout + (bh * N + t) * dv, DN + t * dv, DD + t);
                orc_dphi_q(&c, S, z, dv, DN + t * dv, DD[t], dp);
                orc_phi_backward(&c, q + (bh * N + t) * d, d, omega, dp, dq + (bh * N + t) * d, work);
            }
            /* S, z reused as G, g */
            memset(S, 0, sizeof(double) * (size_t)r * dv);
            memset(z, 0, sizeof(double) * (size_t)r);
            for (long t = N - 1; t >= 0; --t) {
                const double *pq = PQ + t * r;
                for (long f = 0; f < r; ++f) {
                    for (long n = 0; n < dv; ++n) S[f * dv + n] += pq[f] * DN[t * dv + n];
                    z[f] += pq[f] * DD[t];
                }
                orc_phi(&c, k + (bh * N + t) * d, d, omega, pk, work);
                orc_key_grads(&c, S, z, pk, v + (bh * N + t) * dv, dv, dp, dvo + (bh * N + t) * dv);
                orc_phi_backward(&c, k + (bh * N + t) * d, d, omega, dp, dk + (bh * N + t) * d, work);
            }
        }
        free(work); free(pk); free(dp); free(S); free(z); free(PQ); free(DN); free(DD);
    }
    return 0;
}
