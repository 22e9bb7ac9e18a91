/*
 * oracle.c -- plain fp64 CPU oracle for multi-scale retention (MSR).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or constant with the HIP library under
 * retnet_scale_retention_amd/csrc, and it includes nothing from there.
 *
 * Every routine is a direct, slow transcription of what the pages define,
 * written as loops over tokens and channels with no blocking or fusion:
 *
 *   rotation   -- theta_shift(x) = x*cos + rotate_every_two(x)*sin
 *                 (jsqmd.com "From RoPE to Retention", section 2, the
 *                 theta_shift snippet; K gets the conjugate rotation, which
 *                 for a real dot product is the same rotation, see
 *                 oracle_rotate below)
 *   scale      -- scores divided by sqrt(d_k) (same page, section 5,
 *                 "normalisation strategy")
 *   decay mask -- D[n][m] = gamma^(n-m) for n >= m, else 0 (same page,
 *                 section 3; aiqz.cc RetNet tutorial, "retention score and
 *                 exponential decay")
 *   parallel   -- O = (Q K^T (.) D) V (jsqmd.com section 4.1; aiqz.cc
 *                 "parallel representation")
 *   recurrent  -- S_n = gamma S_{n-1} + K_n^T V_n, O_n = Q_n S_n (jsqmd.com
 *                 section 4.2; aiqz.cc "recurrent representation")
 *   chunkwise  -- intra-chunk parallel product + decayed cross-chunk state,
 *                 state discounted by gamma^b per chunk (jsqmd.com section
 *                 4.3; aiqz.cc "chunkwise recurrence"; b99b.cn QbitAI
 *                 article, the three forms)
 *   GroupNorm  -- one group per head over its d_v channels, per token
 *                 (jsqmd.com section 5; b99b.cn, retention features)
 *   row-normalised decay (optional) -- each row of D divided by its sum
 *                 (jsqmd.com section 5, one of the score normalisations it
 *                 lists, no formula given)
 *
 * Readings where the pages are silent or garbled (the same readings the GPU
 * library implements, each justified in the design notes):
 *   - rotate_every_two maps the pair (x[2i], x[2i+1]) to (-x[2i+1], x[2i]);
 *     the angle of pair i at absolute position p is p * theta[i].
 *   - Q and K get the same real rotation; the real dot product of the two
 *     rotated vectors depends only on the position difference, which is the
 *     relative-position property the conjugate pairing is there to give.
 *   - The 1/sqrt(d_k) scale is folded into the rotated K, so the carried
 *     state holds scaled keys.  scale is a parameter here.
 *   - The decay includes the diagonal (gamma^0 = 1 for m == n).
 *   - With an incoming state S_in the parallel output gains
 *     gamma^(n+1) q_n S_in and the outgoing state is
 *     gamma^T S_in + sum_m gamma^(T-1-m) k_m^T v_m.
 *   - GroupNorm: biased variance, no affine, y = (x - mean)/sqrt(var + eps).
 *   - Row-normalised decay: the row of the token at absolute position p
 *     sums its decay weights over every position from 0 to p (the incoming
 *     state stands for the positions before pos0), i.e. sum_{j=0}^{p}
 *     gamma^j, and the row's output is divided by that sum before GroupNorm.
 *
 * Layouts (row-major, fp64): q, k [B][T][H][dk]; v, o [B][T][H][dv];
 * state [B][H][dk][dv].  Pairs (b, h) are independent and are spread over
 * OpenMP threads; within a pair every loop runs in the order written.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int B, T, H, dk, dv;
    const double *gamma; /* [H] decay per head, 0 < gamma <= 1 */
    const double *theta; /* [dk/2] rotation frequency per channel pair */
    double scale;        /* multiplies the rotated K (d_k^-0.5 by default) */
    double eps;          /* GroupNorm epsilon */
    int64_t pos0;        /* absolute position of token 0 */
    int rotate;          /* 0 => no rotation */
    int groupnorm;       /* 0 => raw retention output, no GroupNorm */
    int rownorm;         /* 1 => row-normalised decay */
} oracle_problem;

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static size_t idx_tok(const oracle_problem *p, int b, int t, int h, int d)
{
    return (((size_t)b * p->T + t) * p->H + h) * (size_t)d;
}

/* theta_shift on one d_k vector at absolute position pos:
 * y[2i]   = x[2i]  *cos(pos*theta_i) - x[2i+1]*sin(pos*theta_i)
 * y[2i+1] = x[2i+1]*cos(pos*theta_i) + x[2i]  *sin(pos*theta_i)            */
static void rotate_vec(const oracle_problem *p, const double *x, int64_t pos,
                       double factor, double *y)
{
    for (int i = 0; i < p->dk / 2; i++) {
        double a = x[2 * i], c = x[2 * i + 1];
        if (p->rotate) {
            double phi = (double)pos * p->theta[i];
            double cs = cos(phi), sn = sin(phi);
            y[2 * i] = (a * cs - c * sn) * factor;
            y[2 * i + 1] = (c * cs + a * sn) * factor;
        } else {
            y[2 * i] = a * factor;
            y[2 * i + 1] = c * factor;
        }
    }
}

/* Rotated (and, for K, scaled) copy of one pair's tokens: out[T][dk]. */
static void rotated_pair(const oracle_problem *p, const double *x, int b, int h,
                         double factor, double *out)
{
    for (int t = 0; t < p->T; t++)
        rotate_vec(p, x + idx_tok(p, b, t, h, p->dk), p->pos0 + t, factor,
                   out + (size_t)t * p->dk);
}

static double dot(const double *a, const double *b, int n)
{
    double s = 0.0;
    for (int i = 0; i < n; i++) s += a[i] * b[i];
    return s;
}

/* GroupNorm of one head's d_v outputs of one token, in place. */
static void groupnorm_row(double *x, int n, double eps)
{
    double mean = 0.0, var = 0.0;
    for (int j = 0; j < n; j++) mean += x[j];
    mean /= n;
    for (int j = 0; j < n; j++) var += (x[j] - mean) * (x[j] - mean);
    var /= n;
    double inv = 1.0 / sqrt(var + eps);
    for (int j = 0; j < n; j++) x[j] = (x[j] - mean) * inv;
}

void oracle_groupnorm(int rows, int n, double eps, double *x)
{
    for (int r = 0; r < rows; r++) groupnorm_row(x + (size_t)r * n, n, eps);
}

/* Rotation of a whole [B][T][H][d] tensor (d == dk), times factor. */
void oracle_rotate(const oracle_problem *p, const double *x, double factor, double *y)
{
    for (int b = 0; b < p->B; b++)
        for (int t = 0; t < p->T; t++)
            for (int h = 0; h < p->H; h++)
                rotate_vec(p, x + idx_tok(p, b, t, h, p->dk), p->pos0 + t, factor,
                           y + idx_tok(p, b, t, h, p->dk));
}

typedef struct {
    double *qr, *kr, *acc;
} scratch;

static int scratch_alloc(const oracle_problem *p, scratch *s)
{
    s->qr = malloc(sizeof(double) * (size_t)p->T * p->dk);
    s->kr = malloc(sizeof(double) * (size_t)p->T * p->dk);
    s->acc = malloc(sizeof(double) * (size_t)p->dv);
    return s->qr && s->kr && s->acc;
}

static void scratch_free(scratch *s)
{
    free(s->qr);
    free(s->kr);
    free(s->acc);
}

/* Sum of the decay weights of the row at absolute position pos: the
 * weights gamma^(pos - m) of every position m = 0 .. pos, added one by one. */
static double decay_row_sum(double g, int64_t pos)
{
    double s = 0.0;
    for (int64_t m = 0; m <= pos; m++) s += pow(g, (double)(pos - m));
    return s;
}

/* The finished output row of token t: the optional row normalisation of the
 * decay (a factor on the whole row, state term included), then GroupNorm. */
static void finish_row(const oracle_problem *p, double *row, int64_t pos, int h)
{
    if (p->rownorm) {
        const double r = decay_row_sum(p->gamma[h], pos);
        for (int j = 0; j < p->dv; j++) row[j] /= r;
    }
    if (p->groupnorm) groupnorm_row(row, p->dv, p->eps);
}

static void store_output(const oracle_problem *p, double *o, int b, int t, int h,
                         const double *acc)
{
    double *dst = o + idx_tok(p, b, t, h, p->dv);
    memcpy(dst, acc, sizeof(double) * p->dv);
    finish_row(p, dst, p->pos0 + t, h);
}

/*
 * Parallel form, the plain definition:
 *   O_raw[n] = sum_{m<=n} gamma^(n-m) (q~_n . k~_m) v_m + gamma^(n+1) q~_n S_in
 *   S_out    = gamma^T S_in + sum_m gamma^(T-1-m) k~_m^T v_m
 * Terms with m > n are never formed (they are multiplied by D = 0).
 * o or s_out may be NULL to skip that result; s_in NULL means zeros.
 */
static void parallel_pair(const oracle_problem *p, int b, int h, const double *q,
                          const double *k, const double *v, const double *s_in,
                          double *o, double *s_out, scratch *s)
{
    const int T = p->T, dk = p->dk, dv = p->dv;
    const double g = p->gamma[h];
    const size_t st = ((size_t)b * p->H + h) * (size_t)dk * dv;
    rotated_pair(p, q, b, h, 1.0, s->qr);
    rotated_pair(p, k, b, h, p->scale, s->kr);
    if (o) {
        for (int n = 0; n < T; n++) {
            for (int j = 0; j < dv; j++) s->acc[j] = 0.0;
            for (int m = 0; m <= n; m++) {
                double w = pow(g, n - m) * dot(s->qr + (size_t)n * dk, s->kr + (size_t)m * dk, dk);
                const double *vm = v + idx_tok(p, b, m, h, dv);
                for (int j = 0; j < dv; j++) s->acc[j] += w * vm[j];
            }
            if (s_in) {
                double gn = pow(g, n + 1);
                for (int j = 0; j < dv; j++) {
                    double r = 0.0;
                    for (int i = 0; i < dk; i++) r += s->qr[(size_t)n * dk + i] * s_in[st + (size_t)i * dv + j];
                    s->acc[j] += gn * r;
                }
            }
            store_output(p, o, b, n, h, s->acc);
        }
    }
    if (s_out) {
        for (int i = 0; i < dk; i++)
            for (int j = 0; j < dv; j++) {
                double r = s_in ? pow(g, T) * s_in[st + (size_t)i * dv + j] : 0.0;
                for (int m = 0; m < T; m++)
                    r += pow(g, T - 1 - m) * s->kr[(size_t)m * dk + i] * v[idx_tok(p, b, m, h, dv) + j];
                s_out[st + (size_t)i * dv + j] = r;
            }
    }
}

/*
 * Recurrent form: S_t = gamma S_{t-1} + k~_t^T v_t ; o_t = q~_t S_t.
 * The output reads the state after this token's update.
 */
static void recurrent_pair(const oracle_problem *p, int b, int h, const double *q,
                           const double *k, const double *v, const double *s_in,
                           double *o, double *s_out, double *S, scratch *s)
{
    const int T = p->T, dk = p->dk, dv = p->dv;
    const double g = p->gamma[h];
    const size_t st = ((size_t)b * p->H + h) * (size_t)dk * dv;
    rotated_pair(p, q, b, h, 1.0, s->qr);
    rotated_pair(p, k, b, h, p->scale, s->kr);
    for (size_t e = 0; e < (size_t)dk * dv; e++) S[e] = s_in ? s_in[st + e] : 0.0;
    for (int t = 0; t < T; t++) {
        const double *kt = s->kr + (size_t)t * dk, *qt = s->qr + (size_t)t * dk;
        const double *vt = v + idx_tok(p, b, t, h, dv);
        for (int i = 0; i < dk; i++)
            for (int j = 0; j < dv; j++) S[(size_t)i * dv + j] = g * S[(size_t)i * dv + j] + kt[i] * vt[j];
        for (int j = 0; j < dv; j++) {
            double r = 0.0;
            for (int i = 0; i < dk; i++) r += qt[i] * S[(size_t)i * dv + j];
            s->acc[j] = r;
        }
        if (o) store_output(p, o, b, t, h, s->acc);
    }
    if (s_out) memcpy(s_out + st, S, sizeof(double) * (size_t)dk * dv);
}

/*
 * Chunkwise-recurrent form with chunk size c (c divides T).  For chunk i
 * with local token index j (0 <= j < c) and the state S_{i-1} entering it:
 *   O[j]  = sum_{t<=j} gamma^(j-t) (q~_j . k~_t) v_t       (intra-chunk)
 *         + xi_j (q~_j S_{i-1}),      xi_j   = gamma^(j+1)  (cross-chunk)
 *   S_i   = gamma^c S_{i-1} + sum_t zeta_t k~_t^T v_t,
 *                                     zeta_t = gamma^(c-1-t)
 */
static void chunkwise_pair(const oracle_problem *p, int c, int b, int h, const double *q,
                           const double *k, const double *v, const double *s_in,
                           double *o, double *s_out, double *S, double *Snew, scratch *s)
{
    const int T = p->T, dk = p->dk, dv = p->dv;
    const double g = p->gamma[h];
    const size_t st = ((size_t)b * p->H + h) * (size_t)dk * dv;
    rotated_pair(p, q, b, h, 1.0, s->qr);
    rotated_pair(p, k, b, h, p->scale, s->kr);
    for (size_t e = 0; e < (size_t)dk * dv; e++) S[e] = s_in ? s_in[st + e] : 0.0;
    for (int c0 = 0; c0 < T; c0 += c) {
        for (int j = 0; j < c; j++) {
            const double *qj = s->qr + (size_t)(c0 + j) * dk;
            for (int x = 0; x < dv; x++) s->acc[x] = 0.0;
            for (int t = 0; t <= j; t++) {
                double w = pow(g, j - t) * dot(qj, s->kr + (size_t)(c0 + t) * dk, dk);
                const double *vt = v + idx_tok(p, b, c0 + t, h, dv);
                for (int x = 0; x < dv; x++) s->acc[x] += w * vt[x];
            }
            double xi = pow(g, j + 1);
            for (int x = 0; x < dv; x++) {
                double r = 0.0;
                for (int i = 0; i < dk; i++) r += qj[i] * S[(size_t)i * dv + x];
                s->acc[x] += xi * r;
            }
            if (o) store_output(p, o, b, c0 + j, h, s->acc);
        }
        double gc = pow(g, c);
        for (int i = 0; i < dk; i++)
            for (int x = 0; x < dv; x++) {
                double r = gc * S[(size_t)i * dv + x];
                for (int t = 0; t < c; t++)
                    r += pow(g, c - 1 - t) * s->kr[(size_t)(c0 + t) * dk + i] *
                         v[idx_tok(p, b, c0 + t, h, dv) + x];
                Snew[(size_t)i * dv + x] = r;
            }
        memcpy(S, Snew, sizeof(double) * (size_t)dk * dv);
    }
    if (s_out) memcpy(s_out + st, S, sizeof(double) * (size_t)dk * dv);
}

/* Form selector shared by the exported entry points below. */
enum { FORM_PARALLEL = 0, FORM_RECURRENT = 1, FORM_CHUNKWISE = 2 };

static int run_form(const oracle_problem *p, int form, int chunk, const double *q,
                    const double *k, const double *v, const double *s_in, double *o,
                    double *s_out)
{
    if (p->B < 0 || p->T < 0 || p->H <= 0 || p->dk <= 0 || p->dv <= 0 || (p->dk & 1)) return -1;
    if (form == FORM_CHUNKWISE && (chunk <= 0 || p->T % chunk != 0)) return -2;
    const int pairs = p->B * p->H;
    int failed = 0;
#pragma omp parallel reduction(| : failed)
    {
        scratch s;
        size_t sz = sizeof(double) * (size_t)p->dk * p->dv;
        double *S = malloc(sz), *Snew = malloc(sz);
        if (!scratch_alloc(p, &s) || !S || !Snew) {
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int pr = 0; pr < pairs; pr++) {
                int b = pr / p->H, h = pr % p->H;
                if (form == FORM_PARALLEL)
                    parallel_pair(p, b, h, q, k, v, s_in, o, s_out, &s);
                else if (form == FORM_RECURRENT)
                    recurrent_pair(p, b, h, q, k, v, s_in, o, s_out, S, &s);
                else
                    chunkwise_pair(p, chunk, b, h, q, k, v, s_in, o, s_out, S, Snew, &s);
            }
        }
        scratch_free(&s);
        free(S);
        free(Snew);
    }
    return failed ? -3 : 0;
}

int oracle_parallel(const oracle_problem *p, const double *q, const double *k,
                    const double *v, const double *s_in, double *o, double *s_out)
{
    return run_form(p, FORM_PARALLEL, 0, q, k, v, s_in, o, s_out);
}

int oracle_recurrent(const oracle_problem *p, const double *q, const double *k,
                     const double *v, const double *s_in, double *o, double *s_out)
{
    return run_form(p, FORM_RECURRENT, 0, q, k, v, s_in, o, s_out);
}

int oracle_chunkwise(const oracle_problem *p, int chunk, const double *q, const double *k,
                     const double *v, const double *s_in, double *o, double *s_out)
{
    return run_form(p, FORM_CHUNKWISE, chunk, q, k, v, s_in, o, s_out);
}

/*
 * Selected output rows of the parallel definition for a single pair
 * (the problem must have B == H == 1): o_rows[r] = O[rows[r]], GroupNorm
 * applied if enabled.  Used to check single outputs of sequences too long
 * for the full quadratic oracle.
 */
int oracle_parallel_rows(const oracle_problem *p, int nrows, const int64_t *rows,
                         const double *q, const double *k, const double *v,
                         const double *s_in, double *o_rows)
{
    if (p->B != 1 || p->H != 1 || (p->dk & 1)) return -1;
    const int dk = p->dk, dv = p->dv;
    const double g = p->gamma[0];
    int failed = 0;
#pragma omp parallel reduction(| : failed)
    {
        double *qr = malloc(sizeof(double) * dk), *kr = malloc(sizeof(double) * dk);
        double *acc = malloc(sizeof(double) * dv);
        if (!qr || !kr || !acc) {
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int r = 0; r < nrows; r++) {
                int64_t n = rows[r];
                if (n < 0 || n >= p->T) continue;
                rotate_vec(p, q + (size_t)n * dk, p->pos0 + n, 1.0, qr);
                for (int j = 0; j < dv; j++) acc[j] = 0.0;
                for (int64_t m = 0; m <= n; m++) {
                    rotate_vec(p, k + (size_t)m * dk, p->pos0 + m, p->scale, kr);
                    double w = pow(g, (double)(n - m)) * dot(qr, kr, dk);
                    for (int j = 0; j < dv; j++) acc[j] += w * v[(size_t)m * dv + j];
                }
                if (s_in) {
                    double gn = pow(g, (double)(n + 1));
                    for (int j = 0; j < dv; j++) {
                        double s = 0.0;
                        for (int i = 0; i < dk; i++) s += qr[i] * s_in[(size_t)i * dv + j];
                        acc[j] += gn * s;
                    }
                }
                finish_row(p, acc, p->pos0 + n, 0);
                memcpy(o_rows + (size_t)r * dv, acc, sizeof(double) * dv);
            }
        }
        free(qr);
        free(kr);
        free(acc);
    }
    return failed ? -3 : 0;
}
