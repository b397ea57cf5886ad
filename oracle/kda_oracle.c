/*
 * kda_oracle.c -- plain fp64 CPU oracle for Kimi Delta Attention (KDA).
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke entry and the bench's
 * cpu_baseline leg may load or call this code.  It shares nothing with the
 * HIP path: no header, no helper, no table.
 *
 * What it computes (readings of the pages, stated once here):
 *
 *   The pages name a "delta-rule recurrence" with a per-channel ("channel-wise")
 *   decay gate and an "exact recurrent FP32-state oracle":
 *     - Pure KDA 300M on Primus guide, section "Overview" (delta-rule
 *       recurrence; decay gate f_a -> f_b with learnable A_log and dt_bias
 *       through softplus);
 *     - openkimi README, section "What is implemented" (exact recurrent
 *       fp32-state oracle; fused Q/K norm, decay gate and beta) and the
 *       paragraph on FlashQLA (KDA's decay is channel-wise, not scalar);
 *     - torchtitan PR #4347, "Verification" (the recurrent state resets at
 *       every document offset; a packed row equals the separate runs).
 *   The plainest reading, used here: per sequence and head, with state
 *   S in R^{dk x dv} starting at h0 (or 0), for every token t
 *       a    = exp(g_t)                         (dk, per channel)
 *       S'   = Diag(a) S                        (decay first)
 *       r    = v_t - S'^T k_t                   (prediction error, dv)
 *       S    = S' + beta_t k_t r^T              (= (I - b k k^T) S' + b k v^T)
 *       o_t  = scale * S^T q_t                  (read after the write)
 *   and hT = S after the last token of the sequence.
 *
 * Layout: token-major rows x[t][h][c], t over the concatenation of all
 * sequences; sequence n covers tokens [seg_start[n], seg_start[n]+seg_len[n]).
 * A dense batch [B,T,H,d] is the same memory with seg_start[n] = n*T.
 * States h0/hT/dh0/dhT are [N][H][dk][dv].
 *
 * The backward is derived by hand from the recurrence above (reverse-mode,
 * one token at a time); S_{t-1} is recomputed from a checkpoint taken every
 * CKPT tokens, which repeats the same fp64 operations and so reproduces the
 * forward's states exactly.
 *
 * The chunked form (kdo_chunked_forward) writes out, in fp64, the algebraic
 * rewrite of the same recurrence over chunks of C tokens (in-chunk Gram
 * matrices, unit-lower-triangular inverse, w and u, state passing, output).
 * It is used only to show that the result does not depend on C.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define CKPT 64

static inline const double* row(const double* x, int64_t t, int h, int H, int d) {
    return x + ((size_t)t * H + h) * d;
}
static inline double* rowm(double* x, int64_t t, int h, int H, int d) {
    return x + ((size_t)t * H + h) * d;
}

/* One step of the recurrence on S (dk x dv, row-major), in place.  If o is
 * non-null it receives scale * S^T q after the update. */
static void token_step(int dk, int dv, double* S, const double* q, const double* k,
                       const double* v, const double* g, double beta, double scale,
                       double* o, double* r /* scratch dv */) {
    for (int c = 0; c < dk; ++c) {
        const double a = exp(g[c]);
        for (int j = 0; j < dv; ++j) S[c * dv + j] *= a;
    }
    for (int j = 0; j < dv; ++j) {
        double p = 0.0;
        for (int c = 0; c < dk; ++c) p += S[c * dv + j] * k[c];
        r[j] = v[j] - p;
    }
    for (int c = 0; c < dk; ++c)
        for (int j = 0; j < dv; ++j) S[c * dv + j] += beta * k[c] * r[j];
    if (o) {
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int c = 0; c < dk; ++c) acc += S[c * dv + j] * q[c];
            o[j] = scale * acc;
        }
    }
}

static int pick_threads(int nthreads) {
#ifdef _OPENMP
    return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/* Forward: o [Ttot][H][dv], hT [N][H][dk][dv] (nullable), h0 nullable (zero). */
void kdo_forward(int N, const int64_t* seg_start, const int64_t* seg_len, int H, int dk,
                 int dv, const double* q, const double* k, const double* v, const double* g,
                 const double* beta, double scale, const double* h0, double* o, double* hT,
                 int nthreads) {
    const int nt = pick_threads(nthreads);
    const int64_t pairs = (int64_t)N * H;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int64_t p = 0; p < pairs; ++p) {
        const int n = (int)(p / H), h = (int)(p % H);
        double* S = (double*)calloc((size_t)dk * dv, sizeof(double));
        double* r = (double*)malloc(sizeof(double) * dv);
        if (h0) memcpy(S, h0 + (size_t)p * dk * dv, sizeof(double) * dk * dv);
        for (int64_t t = seg_start[n]; t < seg_start[n] + seg_len[n]; ++t) {
            token_step(dk, dv, S, row(q, t, h, H, dk), row(k, t, h, H, dk), row(v, t, h, H, dv),
                       row(g, t, h, H, dk), beta[(size_t)t * H + h], scale,
                       rowm(o, t, h, H, dv), r);
        }
        if (hT) memcpy(hT + (size_t)p * dk * dv, S, sizeof(double) * dk * dv);
        free(S);
        free(r);
    }
}

/* One decode step for B independent sequences: h [B][H][dk][dv] updated in
 * place; q,k,g [B][H][dk], v [B][H][dv], beta [B][H]; o [B][H][dv]. */
void kdo_step(int B, int H, int dk, int dv, const double* q, const double* k, const double* v,
              const double* g, const double* beta, double scale, double* h, double* o,
              int nthreads) {
    const int nt = pick_threads(nthreads);
    const int64_t pairs = (int64_t)B * H;
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t p = 0; p < pairs; ++p) {
        double* r = (double*)malloc(sizeof(double) * dv);
        token_step(dk, dv, h + (size_t)p * dk * dv, q + (size_t)p * dk, k + (size_t)p * dk,
                   v + (size_t)p * dv, g + (size_t)p * dk, beta[p], scale, o + (size_t)p * dv, r);
        free(r);
    }
}

/*
 * Backward of kdo_forward.  Inputs as the forward plus d_o [Ttot][H][dv] and
 * dhT [N][H][dk][dv] (nullable = 0).  Outputs dq, dk_, dg [Ttot][H][dk],
 * dv_ [Ttot][H][dv], dbeta [Ttot][H], dh0 [N][H][dk][dv] (nullable).
 *
 * Per token, going backwards with D = dL/dS_t (after the write):
 *   D    += scale q_t do_t^T            dq_t  = scale S_t do_t
 *   dbeta = k^T D r                     dr    = beta D^T k        dv_t = dr
 *   dk    = beta D r - S' dr            dS'   = D - k dr^T
 *   dg    = a (.) rowsum(dS' (.) S_{t-1})                       D    = Diag(a) dS'
 * and dh0 = D after the first token.
 */
void kdo_backward(int N, const int64_t* seg_start, const int64_t* seg_len, int H, int dk,
                  int dv, const double* q, const double* k, const double* v, const double* g,
                  const double* beta, double scale, const double* h0, const double* d_o,
                  const double* dhT, double* dq, double* dk_, double* dv_, double* dg,
                  double* dbeta, double* dh0, int nthreads) {
    const int nt = pick_threads(nthreads);
    const int64_t pairs = (int64_t)N * H;
    const size_t SZ = (size_t)dk * dv;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int64_t p = 0; p < pairs; ++p) {
        const int n = (int)(p / H), h = (int)(p % H);
        const int64_t t0 = seg_start[n], L = seg_len[n];
        const int64_t nck = (L + CKPT - 1) / CKPT;
        /* checkpoints: state before tokens t0 + i*CKPT, i = 0..nck-1 */
        double* ck = (double*)calloc((size_t)(nck > 0 ? nck : 1) * SZ, sizeof(double));
        double* blk = (double*)malloc(sizeof(double) * (CKPT + 1) * SZ); /* S before each token, and after the last */
        double* S = (double*)calloc(SZ, sizeof(double));
        double* D = (double*)calloc(SZ, sizeof(double));
        double* Sp = (double*)malloc(sizeof(double) * SZ);
        double* r = (double*)malloc(sizeof(double) * dv);
        double* dr = (double*)malloc(sizeof(double) * dv);
        double* a = (double*)malloc(sizeof(double) * dk);
        if (h0) memcpy(S, h0 + (size_t)p * SZ, sizeof(double) * SZ);
        for (int64_t i = 0; i < nck; ++i) {
            memcpy(ck + (size_t)i * SZ, S, sizeof(double) * SZ);
            const int64_t te = (i + 1) * CKPT < L ? (i + 1) * CKPT : L;
            for (int64_t tt = i * CKPT; tt < te; ++tt) {
                const int64_t t = t0 + tt;
                token_step(dk, dv, S, NULL, row(k, t, h, H, dk), row(v, t, h, H, dv),
                           row(g, t, h, H, dk), beta[(size_t)t * H + h], scale, NULL, r);
            }
        }
        if (dhT) memcpy(D, dhT + (size_t)p * SZ, sizeof(double) * SZ);
        for (int64_t i = nck - 1; i >= 0; --i) {
            const int64_t tb = i * CKPT;
            const int64_t te = (i + 1) * CKPT < L ? (i + 1) * CKPT : L;
            /* recompute the states inside this block */
            memcpy(blk, ck + (size_t)i * SZ, sizeof(double) * SZ);
            for (int64_t tt = tb; tt < te; ++tt) {
                const int64_t t = t0 + tt;
                double* nxt = blk + (size_t)(tt - tb + 1) * SZ;
                memcpy(nxt, blk + (size_t)(tt - tb) * SZ, sizeof(double) * SZ);
                token_step(dk, dv, nxt, NULL, row(k, t, h, H, dk), row(v, t, h, H, dv),
                           row(g, t, h, H, dk), beta[(size_t)t * H + h], scale, NULL, r);
            }
            for (int64_t tt = te - 1; tt >= tb; --tt) {
                const int64_t t = t0 + tt;
                const double* Sprev = blk + (size_t)(tt - tb) * SZ;
                const double* Scur = blk + (size_t)(tt - tb + 1) * SZ;
                const double* qt = row(q, t, h, H, dk);
                const double* kt = row(k, t, h, H, dk);
                const double* vt = row(v, t, h, H, dv);
                const double* gt = row(g, t, h, H, dk);
                const double* dot = row(d_o, t, h, H, dv);
                const double bt = beta[(size_t)t * H + h];
                double* dqt = rowm(dq, t, h, H, dk);
                double* dkt = rowm(dk_, t, h, H, dk);
                double* dvt = rowm(dv_, t, h, H, dv);
                double* dgt = rowm(dg, t, h, H, dk);
                /* output read: o_t = scale S_t^T q_t */
                for (int c = 0; c < dk; ++c) {
                    double acc = 0.0;
                    for (int j = 0; j < dv; ++j) {
                        D[c * dv + j] += scale * qt[c] * dot[j];
                        acc += Scur[c * dv + j] * dot[j];
                    }
                    dqt[c] = scale * acc;
                }
                /* rebuild S' and r of this token */
                for (int c = 0; c < dk; ++c) {
                    a[c] = exp(gt[c]);
                    for (int j = 0; j < dv; ++j) Sp[c * dv + j] = a[c] * Sprev[c * dv + j];
                }
                for (int j = 0; j < dv; ++j) {
                    double pj = 0.0;
                    for (int c = 0; c < dk; ++c) pj += Sp[c * dv + j] * kt[c];
                    r[j] = vt[j] - pj;
                }
                /* write S = S' + beta k r^T */
                double db = 0.0;
                for (int c = 0; c < dk; ++c)
                    for (int j = 0; j < dv; ++j) db += kt[c] * D[c * dv + j] * r[j];
                dbeta[(size_t)t * H + h] = db;
                for (int j = 0; j < dv; ++j) {
                    double acc = 0.0;
                    for (int c = 0; c < dk; ++c) acc += D[c * dv + j] * kt[c];
                    dr[j] = bt * acc;
                    dvt[j] = dr[j];
                }
                for (int c = 0; c < dk; ++c) {
                    double acc1 = 0.0, acc2 = 0.0;
                    for (int j = 0; j < dv; ++j) {
                        acc1 += D[c * dv + j] * r[j];
                        acc2 += Sp[c * dv + j] * dr[j];
                    }
                    dkt[c] = bt * acc1 - acc2;
                }
                /* dS' = D - k dr^T ; decay S' = Diag(a) S_{t-1} */
                for (int c = 0; c < dk; ++c) {
                    double acc = 0.0;
                    for (int j = 0; j < dv; ++j) {
                        const double dsp = D[c * dv + j] - kt[c] * dr[j];
                        acc += dsp * Sprev[c * dv + j];
                        D[c * dv + j] = a[c] * dsp;
                    }
                    dgt[c] = a[c] * acc;
                }
            }
        }
        if (dh0) memcpy(dh0 + (size_t)p * SZ, D, sizeof(double) * SZ);
        free(ck); free(blk); free(S); free(D); free(Sp); free(r); free(dr); free(a);
    }
}

/* ---------------------------------------------------------------------------
 * Gate preparation and its backward (Primus guide "Overview": decay gate with
 * learnable A_log and dt_bias through softplus; openkimi README "What is
 * implemented": fused Q/K norm, decay gate and beta).
 *   l2norm:  x^ = x (|x|^2 + eps)^(-1/2) per token and head
 *   gate:    g  = -exp(A_log[h]) * softplus(f + dt_bias[h][c])
 *   beta:    beta = sigmoid(b)
 * softplus(x) = log1p(exp(x)) for x <= 20, x above (the usual threshold).
 * ------------------------------------------------------------------------- */
static double softplus(double x) { return x > 20.0 ? x : log1p(exp(x)); }
static double dsoftplus(double x) { return x > 20.0 ? 1.0 : 1.0 / (1.0 + exp(-x)); }
static double sigm(double x) { return 1.0 / (1.0 + exp(-x)); }

void kdo_l2norm_fwd(int64_t rows, int d, double eps, const double* x, double* y) {
    for (int64_t i = 0; i < rows; ++i) {
        double ss = 0.0;
        for (int c = 0; c < d; ++c) ss += x[i * d + c] * x[i * d + c];
        const double rr = 1.0 / sqrt(ss + eps);
        for (int c = 0; c < d; ++c) y[i * d + c] = x[i * d + c] * rr;
    }
}

void kdo_l2norm_bwd(int64_t rows, int d, double eps, const double* x, const double* dy,
                    double* dx) {
    for (int64_t i = 0; i < rows; ++i) {
        double ss = 0.0, xd = 0.0;
        for (int c = 0; c < d; ++c) {
            ss += x[i * d + c] * x[i * d + c];
            xd += x[i * d + c] * dy[i * d + c];
        }
        const double rr = 1.0 / sqrt(ss + eps);
        for (int c = 0; c < d; ++c)
            dx[i * d + c] = rr * dy[i * d + c] - rr * rr * rr * xd * x[i * d + c];
    }
}

/* f [Ttot][H][dk] -> g [Ttot][H][dk] */
void kdo_gate_fwd(int64_t Ttot, int H, int dk, const double* f, const double* A_log,
                  const double* dt_bias, double* g) {
    for (int64_t t = 0; t < Ttot; ++t)
        for (int h = 0; h < H; ++h)
            for (int c = 0; c < dk; ++c) {
                const size_t i = ((size_t)t * H + h) * dk + c;
                g[i] = -exp(A_log[h]) * softplus(f[i] + dt_bias[h * dk + c]);
            }
}

/* dg -> df, and the token sums dA_log [H], ddt_bias [H][dk] */
void kdo_gate_bwd(int64_t Ttot, int H, int dk, const double* f, const double* A_log,
                  const double* dt_bias, const double* dg, double* df, double* dA_log,
                  double* ddt_bias) {
    for (int h = 0; h < H; ++h) {
        dA_log[h] = 0.0;
        for (int c = 0; c < dk; ++c) ddt_bias[h * dk + c] = 0.0;
    }
    for (int64_t t = 0; t < Ttot; ++t)
        for (int h = 0; h < H; ++h)
            for (int c = 0; c < dk; ++c) {
                const size_t i = ((size_t)t * H + h) * dk + c;
                const double x = f[i] + dt_bias[h * dk + c];
                const double e = exp(A_log[h]);
                const double gi = -e * softplus(x);
                df[i] = dg[i] * (-e) * dsoftplus(x);
                ddt_bias[h * dk + c] += df[i];
                dA_log[h] += dg[i] * gi;
            }
}

void kdo_sigmoid_fwd(int64_t n, const double* b, double* beta) {
    for (int64_t i = 0; i < n; ++i) beta[i] = sigm(b[i]);
}

void kdo_sigmoid_bwd(int64_t n, const double* b, const double* dbeta, double* db) {
    for (int64_t i = 0; i < n; ++i) {
        const double s = sigm(b[i]);
        db[i] = dbeta[i] * s * (1.0 - s);
    }
}

/* ---------------------------------------------------------------------------
 * Chunked forward in fp64 (used to show chunk-size invariance).
 * For each chunk of L <= C tokens of a sequence, with h the state entering it:
 *   G_t      = sum_{s<=t in chunk} g_s                       (per channel)
 *   Akk[t,s] = beta_t sum_c k_tc k_sc exp(G_tc - G_sc),  s < t
 *   Aqk[t,s] = sum_c q_tc k_sc exp(G_tc - G_sc),         s <= t
 *   T        = (I + Akk)^{-1}                                (unit lower)
 *   w        = T Diag(beta) (exp(G) (.) K),  u = T Diag(beta) V
 *   vn       = u - w h
 *   o        = scale ((exp(G) (.) Q) h + Aqk vn)
 *   h       <- Diag(exp(G_L)) h + (K (.) exp(G_L - G))^T vn
 * ------------------------------------------------------------------------- */
void kdo_chunked_forward(int N, const int64_t* seg_start, const int64_t* seg_len, int H, int dk,
                         int dv, const double* q, const double* k, const double* v,
                         const double* g, const double* beta, double scale, const double* h0,
                         int C, double* o, double* hT, int nthreads) {
    const int nt = pick_threads(nthreads);
    const int64_t pairs = (int64_t)N * H;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int64_t p = 0; p < pairs; ++p) {
        const int n = (int)(p / H), h = (int)(p % H);
        double* S = (double*)calloc((size_t)dk * dv, sizeof(double));
        double* G = (double*)malloc(sizeof(double) * C * dk);
        double* A = (double*)malloc(sizeof(double) * C * C);
        double* Aq = (double*)malloc(sizeof(double) * C * C);
        double* Tm = (double*)malloc(sizeof(double) * C * C);
        double* w = (double*)malloc(sizeof(double) * C * dk);
        double* u = (double*)malloc(sizeof(double) * C * dv);
        double* vn = (double*)malloc(sizeof(double) * C * dv);
        double* Sn = (double*)malloc(sizeof(double) * dk * dv);
        if (h0) memcpy(S, h0 + (size_t)p * dk * dv, sizeof(double) * dk * dv);
        for (int64_t c0 = 0; c0 < seg_len[n]; c0 += C) {
            const int L = (int)((seg_len[n] - c0) < C ? (seg_len[n] - c0) : C);
            const int64_t tb = seg_start[n] + c0;
#define Q_(t, c) row(q, tb + (t), h, H, dk)[c]
#define K_(t, c) row(k, tb + (t), h, H, dk)[c]
#define V_(t, j) row(v, tb + (t), h, H, dv)[j]
#define B_(t) beta[(size_t)(tb + (t)) * H + h]
            for (int c = 0; c < dk; ++c) {
                double acc = 0.0;
                for (int t = 0; t < L; ++t) {
                    acc += row(g, tb + t, h, H, dk)[c];
                    G[t * dk + c] = acc;
                }
            }
            for (int t = 0; t < L; ++t)
                for (int s = 0; s < L; ++s) {
                    double ak = 0.0, aq = 0.0;
                    if (s <= t)
                        for (int c = 0; c < dk; ++c) {
                            const double e = exp(G[t * dk + c] - G[s * dk + c]);
                            ak += K_(t, c) * K_(s, c) * e;
                            aq += Q_(t, c) * K_(s, c) * e;
                        }
                    A[t * C + s] = (s < t) ? B_(t) * ak : 0.0;
                    Aq[t * C + s] = (s <= t) ? aq : 0.0;
                }
            /* T = (I + A)^{-1}: forward substitution column by column */
            for (int s = 0; s < L; ++s)
                for (int t = 0; t < L; ++t) {
                    if (t < s) { Tm[t * C + s] = 0.0; continue; }
                    double x = (t == s) ? 1.0 : 0.0;
                    for (int m = s; m < t; ++m) x -= A[t * C + m] * Tm[m * C + s];
                    Tm[t * C + s] = x;
                }
            for (int t = 0; t < L; ++t) {
                for (int c = 0; c < dk; ++c) {
                    double acc = 0.0;
                    for (int s = 0; s <= t; ++s)
                        acc += Tm[t * C + s] * B_(s) * exp(G[s * dk + c]) * K_(s, c);
                    w[t * dk + c] = acc;
                }
                for (int j = 0; j < dv; ++j) {
                    double acc = 0.0;
                    for (int s = 0; s <= t; ++s) acc += Tm[t * C + s] * B_(s) * V_(s, j);
                    u[t * dv + j] = acc;
                }
            }
            for (int t = 0; t < L; ++t)
                for (int j = 0; j < dv; ++j) {
                    double acc = u[t * dv + j];
                    for (int c = 0; c < dk; ++c) acc -= w[t * dk + c] * S[c * dv + j];
                    vn[t * dv + j] = acc;
                }
            for (int t = 0; t < L; ++t)
                for (int j = 0; j < dv; ++j) {
                    double acc = 0.0;
                    for (int c = 0; c < dk; ++c) acc += exp(G[t * dk + c]) * Q_(t, c) * S[c * dv + j];
                    for (int s = 0; s <= t; ++s) acc += Aq[t * C + s] * vn[s * dv + j];
                    rowm(o, tb + t, h, H, dv)[j] = scale * acc;
                }
            for (int c = 0; c < dk; ++c)
                for (int j = 0; j < dv; ++j) {
                    double acc = exp(G[(L - 1) * dk + c]) * S[c * dv + j];
                    for (int s = 0; s < L; ++s)
                        acc += K_(s, c) * exp(G[(L - 1) * dk + c] - G[s * dk + c]) * vn[s * dv + j];
                    Sn[c * dv + j] = acc;
                }
            memcpy(S, Sn, sizeof(double) * dk * dv);
#undef Q_
#undef K_
#undef V_
#undef B_
        }
        if (hT) memcpy(hT + (size_t)p * dk * dv, S, sizeof(double) * dk * dv);
        free(S); free(G); free(A); free(Aq); free(Tm); free(w); free(u); free(vn); free(Sn);
    }
}

int kdo_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
