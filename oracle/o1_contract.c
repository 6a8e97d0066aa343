/*
 * O1 -- contract oracle for the Mamba-3 MIMO backward first stage
 * (mamba_mimo_bwd_fwd). TEST INFRASTRUCTURE ONLY: nothing in the product
 * path may include, link or call this file. It shares no code with the HIP
 * library.
 *
 * Source of the method: the Triton-Ascend mamba_mimo_bwd_fwd pull request
 * page, "BF16-boundary PyTorch reference" section (bias, qk_dot, rotation,
 * PsiV, discretisation, chunk loop, gating branches), and its operator
 * document ("inputs and outputs" tables and constraints).
 *
 * Plain, slow, token-by-token loops. Every intermediate the pages keep as an
 * fp32 tensor is rounded to fp32 (RF) and every place the pages round to
 * bf16 is rounded to bf16 round-to-nearest-even (RB). Dot products and sums
 * accumulate in double and are rounded once at the end, which is at least as
 * accurate as any fp32 summation order. Three modes:
 *   0  the bf16 contract above;
 *   1  exact: both roundings are the identity and every quantity is carried
 *      in double -- the chunked algorithm in exact arithmetic, used to check
 *      the algebra against an unchunked recurrence;
 *   2  fp32 intermediates: the same page's FP32 reference -- every
 *      intermediate stays fp32 (no bf16 rounding of q, k, PsiV, the
 *      projections, dt, the causal block, the state, y, the diagonal chain or
 *      the dz chain) and only the outputs are cast to their dtypes (states,
 *      qk_dot and dz to bf16). That reference writes the look-ahead weight as
 *      dt[t+1] * (1 - sigmoid(trap[t+1])), followed here.
 *
 * All tensors are dense row-major in the operator's own layouts:
 *   dout   [B,S,H,P] (reduce_o) or [B,S,R,H,P] (non-reduced)
 *   q, k   [B,S,R,G,N]      v, z [B,S,H,P]
 *   q_bias, k_bias [H,R,N]   mimo_v, mimo_o, mimo_z [H,R,P]
 *   angles [B,S,H,W]         da_cs, da_cs_rev, dt, trap [B,H,S]
 * (W = N / rotary_dim_divisor rotated column pairs: columns [0,W) pair with
 * [N/2, N/2+W))
 *   d [H]                    segsum [B,H,nc,C,C]
 * outputs
 *   dmimo_o, dmimo_z [B,H,R,P]   states [B,H,nc,N,P]
 *   dz [B,S,H,P]                 qk_dot [B,H,S,R,R]
 *
 * o1_fwd runs the same chunk walk without dout and returns the layer output
 * the backward differentiates (inferred from the gating branches of the
 * BF16-boundary reference: dmimo_o, dz and dmimo_z are the gradients of
 * sum(o * dout) with respect to mimo_o, z and mimo_z):
 *   reduced (mimo_o given)  o[b,t,h,p]   = bf16( sum_r (y * bf16(mimo_o)) * silu(pz) )
 *   not reduced             o[b,t,r,h,p] = bf16( y * silu(pz) )
 * with silu(pz) = pz * sigmoid(pz), pz = z * mimo_z, and the silu factor left
 * out without z. The rank sum runs in rank order in fp32.
 * Every array is double; in contract mode the caller passes values that are
 * exactly representable in the pages' dtypes (bf16 or fp32) and gets back
 * values representable in the output dtypes.
 *
 * Tail chunk: only real tokens are visited. The pages zero-pad the last
 * chunk; padded tokens have PsiV = 0 (v = 0), so they add nothing to the
 * intra-chunk term or to the state, and their output rows meet dout = 0 and
 * z = 0 in every sum, so visiting them changes no result.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static int g_mode = 0;   /* 0 contract, 1 exact, 2 fp32 intermediates */

/* fp32 rounding of a double (identity in exact mode). */
static inline double RF(double x) { return g_mode == 1 ? x : (double)(float)x; }

/* bf16 round-to-nearest-even of an fp32 value, from the IEEE-754 binary
 * encoding: keep the upper 16 bits, rounding on the lower 16 with ties to
 * the even upper half. NaN stays NaN. */
static inline double RB(double xd) {
    if (g_mode == 1) return xd;
    float f = (float)xd;
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) {
        u = (u | 0x00400000u) & 0xffff0000u;
    } else {
        uint32_t lsb = (u >> 16) & 1u;
        u = (u + 0x7fffu + lsb) & 0xffff0000u;
    }
    memcpy(&f, &u, 4);
    return (double)f;
}

/* The contract's bf16 roundings of intermediate values, one id per place the
 * BF16-boundary reference rounds. Tests may switch single places off (their
 * value then stays fp32) to check which outputs each one reaches. */
enum {
    R_Q_BIAS, R_K_BIAS, R_Q0, R_K0, R_QK, R_QROT, R_KROT, R_MIMO_V, R_PSI,
    R_DT_G, R_DT_B, R_BETA, R_FACTOR, R_KT, R_KAP, R_A, R_SB,
    R_DPROD, R_DSUM, R_DGAM, R_Y, R_MIMO_O, R_G_IN, R_G_OUT, R_G_NR, R_DZ,
    R_COUNT
};
static uint64_t g_skip = 0;   /* bit i set: rounding place i is left out (contract mode only) */

/* A bf16 rounding of an intermediate value at place `site`: the contract's RB,
 * fp32 in mode 2 or where the place is switched off. RB itself is kept for the
 * outputs, which are bf16 in every mode but exact. */
static inline double RBI_(int site, double x) {
    if (g_mode == 2 || ((g_skip >> site) & 1u)) return RF(x);
    return RB(x);
}
#define RBI(site, x) RBI_(R_##site, (x))

static inline double EXP(double x) { return RF(exp(x)); }
static inline double SIG(double x) { return RF(1.0 / (1.0 + exp(-x))); }

typedef struct {
    int64_t B, S, H, G, R, N, P, C, W;
    int reduce_o, has_z, has_d;
    const double *dout, *q, *k, *v, *q_bias, *k_bias, *mimo_v, *mimo_o, *z, *mimo_z;
    const double *angles, *da_cs, *da_cs_rev, *dt, *trap, *d, *segsum;
    double *dmimo_o, *states, *dz, *dmimo_z, *qk_dot;
    int fwd;     /* layer output instead of the gradients */
    double *o;   /* [B,S,H,P] reduced, [B,S,R,H,P] otherwise */
} o1_args;

/* One (batch, head) pair: the whole sequence, chunk by chunk. */
static void o1_head(const o1_args *a, int64_t b, int64_t h) {
    const int64_t S = a->S, H = a->H, G = a->G, R = a->R, N = a->N, P = a->P, C = a->C;
    const int64_t W = a->W, M = N / 2, nc = (S + C - 1) / C;
    const int64_t g = h / (H / G);

    double *q0 = malloc(sizeof(double) * C * R * N);   /* biased q, before rotation  */
    double *k0 = malloc(sizeof(double) * C * R * N);
    double *qr = malloc(sizeof(double) * C * R * N);   /* rotated q                  */
    double *kt = malloc(sizeof(double) * C * R * N);   /* rotated, factor-scaled k   */
    double *kap = malloc(sizeof(double) * C * R * N);  /* kt * exp(da_cs_rev)        */
    double *psi = malloc(sizeof(double) * C * R * P);
    double *y = malloc(sizeof(double) * C * R * P);
    double *qk = malloc(sizeof(double) * C * R * R);
    double *gam = malloc(sizeof(double) * C);
    double *St = calloc(N * P, sizeof(double));        /* fp32 recurrent state       */
    double *Sb = malloc(sizeof(double) * N * P);       /* its bf16 copy              */
    double *acc = malloc(sizeof(double) * (N > P ? N : P));
    double *dmo = calloc(R * P, sizeof(double));
    double *dmz = calloc(R * P, sizeof(double));
    double *A = malloc(sizeof(double) * C * R);        /* one row of the causal block */

    for (int64_t c = 0; c < nc; ++c) {
        const int64_t c0 = c * C;
        const int64_t cl = (S - c0 < C) ? (S - c0) : C;   /* real tokens in chunk */

        /* entry state of chunk c */
        for (int64_t i = 0; i < N * P; ++i) Sb[i] = RBI(SB, St[i]);
        if (a->states) {
            double *st_out = a->states + (((b * H + h) * nc + c) * N) * P;
            for (int64_t i = 0; i < N * P; ++i) st_out[i] = RB(St[i]);
        }

        /* per-token preparation */
        for (int64_t t = 0; t < cl; ++t) {
            const int64_t T = c0 + t;
            for (int64_t r = 0; r < R; ++r) {
                const double *qs = a->q + (((b * S + T) * R + r) * G + g) * N;
                const double *ks = a->k + (((b * S + T) * R + r) * G + g) * N;
                const double *qb = a->q_bias + (h * R + r) * N;
                const double *kb = a->k_bias + (h * R + r) * N;
                double *q0r = q0 + (t * R + r) * N, *k0r = k0 + (t * R + r) * N;
                for (int64_t n = 0; n < N; ++n) {
                    q0r[n] = RBI(Q0, RF(qs[n] + RBI(Q_BIAS, qb[n])));
                    k0r[n] = RBI(K0, RF(ks[n] + RBI(K_BIAS, kb[n])));
                }
            }
            /* same-token rank-by-rank dot of the biased, unrotated q and k */
            for (int64_t r = 0; r < R; ++r)
                for (int64_t s2 = 0; s2 < R; ++s2) {
                    double sum = 0.0;
                    const double *x = q0 + (t * R + r) * N, *w = k0 + (t * R + s2) * N;
                    for (int64_t n = 0; n < N; ++n) sum += x[n] * w[n];
                    qk[(t * R + r) * R + s2] = RBI(QK, RF(sum));
                    if (a->qk_dot) a->qk_dot[(((b * H + h) * S + T) * R + r) * R + s2] = RB(RF(sum));
                }
            /* partial rotate-half: columns [0,W) pair with [M, M+W) */
            const double *th = a->angles + ((b * S + T) * H + h) * W;
            for (int64_t r = 0; r < R; ++r) {
                double *q0r = q0 + (t * R + r) * N, *k0r = k0 + (t * R + r) * N;
                double *qrr = qr + (t * R + r) * N, *ktr = kt + (t * R + r) * N;
                for (int64_t n = 0; n < N; ++n) { qrr[n] = q0r[n]; ktr[n] = k0r[n]; }
                for (int64_t n = 0; n < W; ++n) {
                    const double cs = RF(cos(th[n])), sn = RF(sin(th[n]));
                    qrr[n] = RBI(QROT, RF(RF(cs * q0r[n]) - RF(sn * q0r[M + n])));
                    qrr[M + n] = RBI(QROT, RF(RF(sn * q0r[n]) + RF(cs * q0r[M + n])));
                    ktr[n] = RBI(KROT, RF(RF(cs * k0r[n]) - RF(sn * k0r[M + n])));
                    ktr[M + n] = RBI(KROT, RF(RF(sn * k0r[n]) + RF(cs * k0r[M + n])));
                }
            }
            /* PsiV = v * bf16(mimo_v) */
            for (int64_t r = 0; r < R; ++r)
                for (int64_t p = 0; p < P; ++p)
                    psi[(t * R + r) * P + p] =
                        RBI(PSI, RF(a->v[((b * S + T) * H + h) * P + p] * RBI(MIMO_V, a->mimo_v[(h * R + r) * P + p])));
            /* trapezoidal discretisation: gamma (fp32), beta from the next token, factor (bf16) */
            const int64_t ih = (b * H + h) * S;
            const double gamma = RF(RBI(DT_G, a->dt[ih + T]) * SIG(a->trap[ih + T]));
            double beta = 0.0;
            if (T + 1 < S) {
                const double w = g_mode == 2 ? RF(1.0 - SIG(a->trap[ih + T + 1])) : SIG(-a->trap[ih + T + 1]);
                beta = RBI(BETA, RF(RBI(DT_B, a->dt[ih + T + 1]) * w));
            }
            const double factor = RBI(FACTOR, RF(gamma + beta));
            gam[t] = gamma;
            const double erev = EXP(a->da_cs_rev[ih + T]);
            for (int64_t r = 0; r < R; ++r)
                for (int64_t n = 0; n < N; ++n) {
                    double *ktr = kt + (t * R + r) * N;
                    ktr[n] = RBI(KT, RF(ktr[n] * factor));
                    kap[(t * R + r) * N + n] = RBI(KAP, RF(ktr[n] * erev));
                }
        }

        /* outputs of the chunk */
        const int64_t ih = (b * H + h) * S;
        const double *seg = a->segsum + ((b * H + h) * nc + c) * C * C;
        for (int64_t t = 0; t < cl; ++t) {
            const double ecs = EXP(a->da_cs[ih + c0 + t]);
            for (int64_t r = 0; r < R; ++r) {
                const double *qrow = qr + (t * R + r) * N;
                /* causal row: earlier tokens only, the same token is excluded */
                for (int64_t j = 0; j < t; ++j) {
                    const double es = EXP(seg[t * C + j]);
                    for (int64_t s2 = 0; s2 < R; ++s2) {
                        double sum = 0.0;
                        const double *krow = kt + (j * R + s2) * N;
                        for (int64_t n = 0; n < N; ++n) sum += qrow[n] * krow[n];
                        A[j * R + s2] = RBI(A, RF(RF(sum) * es));
                    }
                }
                for (int64_t p = 0; p < P; ++p) acc[p] = 0.0;
                for (int64_t n = 0; n < N; ++n) {       /* inter: q_rot . bf16(state) */
                    const double qv = qrow[n];
                    const double *sr = Sb + n * P;
                    for (int64_t p = 0; p < P; ++p) acc[p] += qv * sr[p];
                }
                for (int64_t p = 0; p < P; ++p) {
                    const double inter = RF(RF(acc[p]) * ecs);
                    double isum = 0.0;                       /* intra */
                    for (int64_t j = 0; j < t; ++j)
                        for (int64_t s2 = 0; s2 < R; ++s2) isum += A[j * R + s2] * psi[(j * R + s2) * P + p];
                    const double intra = RF(isum);
                    /* diagonal: rank-ordered bf16 products and sums, then times gamma */
                    double dg = 0.0;
                    for (int64_t s2 = 0; s2 < R; ++s2) {
                        const double prod = RBI(DPROD, RF(qk[(t * R + r) * R + s2] * psi[(t * R + s2) * P + p]));
                        dg = RBI(DSUM, RF(dg + prod));
                    }
                    dg = RBI(DGAM, RF(dg * gam[t]));
                    double o = RF(RF(inter + intra) + dg);
                    if (a->has_d) o = RF(o + RF(a->d[h] * psi[(t * R + r) * P + p]));
                    y[(t * R + r) * P + p] = RBI(Y, o);
                }
            }
        }

        /* state update: decay at the chunk's last real token plus kappa^T PsiV */
        {
            const double dl = EXP(a->da_cs[ih + c0 + cl - 1]);
            for (int64_t n = 0; n < N; ++n) {
                for (int64_t p = 0; p < P; ++p) acc[p] = 0.0;
                for (int64_t t = 0; t < cl; ++t)
                    for (int64_t r = 0; r < R; ++r) {
                        const double kv = kap[(t * R + r) * N + n];
                        const double *pr = psi + (t * R + r) * P;
                        for (int64_t p = 0; p < P; ++p) acc[p] += kv * pr[p];
                    }
                for (int64_t p = 0; p < P; ++p) St[n * P + p] = RF(RF(St[n * P + p] * dl) + RF(acc[p]));
            }
        }

        /* layer output */
        if (a->fwd) {
            for (int64_t t = 0; t < cl; ++t) {
                const int64_t T = c0 + t;
                for (int64_t p = 0; p < P; ++p) {
                    const int64_t ivp = ((b * S + T) * H + h) * P + p;
                    double oacc = 0.0;
                    for (int64_t r = 0; r < R; ++r) {
                        double val = y[(t * R + r) * P + p];
                        if (a->reduce_o) val = RF(val * RBI(MIMO_O, a->mimo_o[(h * R + r) * P + p]));
                        if (a->has_z) {
                            const double pz = RF(a->z[ivp] * a->mimo_z[(h * R + r) * P + p]);
                            val = RF(val * RF(pz * SIG(pz)));
                        }
                        if (a->reduce_o)
                            oacc = RF(oacc + val);
                        else
                            a->o[(((b * S + T) * R + r) * H + h) * P + p] = RB(val);
                    }
                    if (a->reduce_o) a->o[ivp] = RB(oacc);
                }
            }
            continue;
        }

        /* gating branches */
        for (int64_t t = 0; t < cl; ++t) {
            const int64_t T = c0 + t;
            for (int64_t p = 0; p < P; ++p) {
                const int64_t ivp = ((b * S + T) * H + h) * P + p;   /* [B,S,H,P] index */
                double dzacc = 0.0;
                for (int64_t r = 0; r < R; ++r) {
                    const double yv = y[(t * R + r) * P + p];
                    double pz = 0.0, sg = 0.0, silu = 0.0, G = 0.0;
                    if (a->has_z) {
                        pz = RF(a->z[ivp] * a->mimo_z[(h * R + r) * P + p]);
                        sg = SIG(pz);
                        silu = RF(pz * sg);
                    }
                    if (a->reduce_o) {
                        const double dv = a->dout[ivp];
                        if (a->has_z) {
                            dmo[r * P + p] += RF(RF(yv * silu) * dv);
                            G = RBI(G_OUT, RF(RBI(G_IN, RF(dv * RBI(MIMO_O, a->mimo_o[(h * R + r) * P + p]))) * yv));
                        } else {
                            dmo[r * P + p] += RF(yv * dv);
                        }
                    } else if (a->has_z) {
                        const double dv = a->dout[(((b * S + T) * R + r) * H + h) * P + p];
                        G = RBI(G_NR, RF(dv * yv));
                    }
                    if (a->has_z) {
                        const double gz = RF(RF(G * sg) * RF(1.0 + RF(pz * SIG(-pz))));
                        dzacc = RBI(DZ, RF(dzacc + RF(gz * a->mimo_z[(h * R + r) * P + p])));
                        dmz[r * P + p] += RF(gz * a->z[ivp]);
                    }
                }
                if (a->has_z) a->dz[ivp] = RB(dzacc);
            }
        }
    }
    for (int64_t i = 0; i < R * P && !a->fwd; ++i) {
        if (a->reduce_o) a->dmimo_o[(b * H + h) * R * P + i] = RF(dmo[i]);
        if (a->has_z) a->dmimo_z[(b * H + h) * R * P + i] = RF(dmz[i]);
    }
    free(q0); free(k0); free(qr); free(kt); free(kap); free(psi); free(y); free(qk); free(gam);
    free(St); free(Sb); free(acc); free(dmo); free(dmz); free(A);
}

/* Entry point. Returns 0, or -1 for an invalid shape. */
int o1_bwd_fwd(int64_t B, int64_t S, int64_t H, int64_t G, int64_t R, int64_t N, int64_t P,
               int64_t C, int64_t W, int mode, int reduce_o, int has_z, int has_d,
               const double *dout, const double *q, const double *k, const double *v,
               const double *q_bias, const double *k_bias, const double *mimo_v,
               const double *mimo_o, const double *z, const double *mimo_z,
               const double *angles, const double *da_cs, const double *da_cs_rev,
               const double *dt, const double *trap, const double *d, const double *segsum,
               double *dmimo_o, double *states, double *dz, double *dmimo_z, double *qk_dot) {
    if (B < 1 || S < 1 || H < 1 || G < 1 || R < 1 || N < 2 || P < 1 || C < 1) return -1;
    if (H % G || N % 2 || W < 0 || 2 * W > N || mode < 0 || mode > 2) return -1;
    g_mode = mode;
    o1_args a = {B, S, H, G, R, N, P, C, W, reduce_o, has_z, has_d,
                 dout, q, k, v, q_bias, k_bias, mimo_v, mimo_o, z, mimo_z,
                 angles, da_cs, da_cs_rev, dt, trap, d, segsum,
                 dmimo_o, states, dz, dmimo_z, qk_dot, 0, NULL};
    int64_t nbh = B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < nbh; ++i) o1_head(&a, i / H, i % H);
    return 0;
}

/* Test hook: leave out the bf16 roundings whose bits are set in `mask` (ids
 * from the enum above) in later contract-mode runs; 0 restores the contract.
 * Returns the number of rounding places. */
int o1_set_skip(uint64_t mask) {
    g_skip = mask;
    return R_COUNT;
}

/* bf16 rounding exposed for the oracle's own unit tests. */
void o1_round_bf16(const float *x, float *y, int64_t n) {
    int save = g_mode;
    g_mode = 0;
    for (int64_t i = 0; i < n; ++i) y[i] = (float)RB((double)x[i]);
    g_mode = save;
}

/* Layer output (see the header comment): the chunk walk of o1_bwd_fwd without
 * dout. states may be NULL. Returns 0, or -1 for an invalid shape. */
int o1_fwd(int64_t B, int64_t S, int64_t H, int64_t G, int64_t R, int64_t N, int64_t P,
           int64_t C, int64_t W, int mode, int reduce_o, int has_z, int has_d,
           const double *q, const double *k, const double *v,
           const double *q_bias, const double *k_bias, const double *mimo_v,
           const double *mimo_o, const double *z, const double *mimo_z,
           const double *angles, const double *da_cs, const double *da_cs_rev,
           const double *dt, const double *trap, const double *d, const double *segsum,
           double *o, double *states) {
    if (B < 1 || S < 1 || H < 1 || G < 1 || R < 1 || N < 2 || P < 1 || C < 1) return -1;
    if (H % G || N % 2 || W < 0 || 2 * W > N || mode < 0 || mode > 2) return -1;
    g_mode = mode;
    o1_args a = {B, S, H, G, R, N, P, C, W, reduce_o, has_z, has_d,
                 NULL, q, k, v, q_bias, k_bias, mimo_v, mimo_o, z, mimo_z,
                 angles, da_cs, da_cs_rev, dt, trap, d, segsum,
                 NULL, states, NULL, NULL, NULL, 1, o};
    int64_t nbh = B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < nbh; ++i) o1_head(&a, i / H, i % H);
    return 0;
}
