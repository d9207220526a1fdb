/*
 * oracle.c -- plain, slow, double-precision CPU reference for the multi-head
 * LSTM / GRU recurrence with a block-diagonal recurrent matrix.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library.  It shares no
 * code, header, table or helper with the GPU library and includes nothing
 * from it.
 *
 * What it follows:
 *   - FlashRNN (arXiv 2412.07752), abstract: traditional LSTM and GRU cells
 *     processed strictly sequentially in time, extended by splitting the
 *     hidden state into several small independent RNNs ("heads") that run
 *     side by side, as with Transformer heads.
 *   - "Re-examining RNNs from a GPU programming perspective" (blog.hotdry.top,
 *     2025-09-21), the paragraph on head-wise splitting: each head owns its
 *     own smaller recurrent matrix, so the full recurrent matrix is
 *     block-diagonal and heads never exchange data.
 *   The pages print no cell equations; the cells are the textbook
 *   forget-gate LSTM (no peepholes) with gate order i, f, z, o and the
 *   reset-after GRU with gate order r, z, n (the form whose recurrent part
 *   is a single h_{t-1} R product per step, with no separate recurrent bias).
 *
 * Layouts (row-major, all double):
 *   x      [T][B][Din]             W   [Din][NH][G][Dh]   (column (n*G+g)*Dh+j)
 *   R      [NH][Dh][G*Dh]          b   [NH][G][Dh]
 *   h0,c0  [B][NH*Dh]              h_seq, c_seq, dh_seq  [T][B][NH*Dh]  (h_1..h_T)
 *   gate-space arrays (dA, dGx, dS) [T][B][NH*G*Dh]
 *
 * Every (batch row b, head n) pair is an independent chain.  `chain_mask`
 * ([B][NH] bytes, NULL = all) restricts the work to some chains; outputs of
 * the other chains are left untouched.  Parallelism (OpenMP) runs only over
 * independent chains or independent output elements; every sum is taken in
 * the plain index order written below, so 1 and N threads give identical
 * bits.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define LSTM_G 4
#define GRU_G 3

static double sigm(double a) { return 1.0 / (1.0 + exp(-a)); }

static int chain_on(const unsigned char *mask, int b, int n, int NH) {
    return mask == NULL || mask[(size_t)b * NH + n] != 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Input projection of one (t, b) row restricted to head n:
 *   gx[g*Dh + j] = bias[(n*G+g)*Dh + j] + sum_{k=0..Din-1} x[t][b][k] * W[k][(n*G+g)*Dh + j]
 * (FlashRNN abstract: the input part of every gate is a dense projection of
 * x_t, independent of the recurrence, so all T rows can be formed up front.)
 */
static void input_proj_head(int Din, int N, int G, int Dh, int n,
                            const double *xrow, const double *W,
                            const double *bias, double *gx) {
    const int GD = G * Dh;
    const size_t c0 = (size_t)n * GD;
    for (int c = 0; c < GD; ++c) gx[c] = bias ? bias[c0 + c] : 0.0;
    for (int k = 0; k < Din; ++k) {
        const double xv = xrow[k];
        const double *wr = W + (size_t)k * N + c0;
        for (int c = 0; c < GD; ++c) gx[c] += xv * wr[c];
    }
}

/* s[c] = sum_{m=0..Dh-1} h[m] * Rn[m][c]  (one head's block of R). */
static void rec_proj(int Dh, int GD, const double *h, const double *Rn, double *s) {
    for (int c = 0; c < GD; ++c) s[c] = 0.0;
    for (int m = 0; m < Dh; ++m) {
        const double hv = h[m];
        const double *rr = Rn + (size_t)m * GD;
        for (int c = 0; c < GD; ++c) s[c] += hv * rr[c];
    }
}

/* ------------------------------------------------------------------ LSTM */

/*
 * One LSTM chain forward.  Per step (textbook forget-gate LSTM):
 *   A = Gx_t + h_{t-1} R_n
 *   i = sigma(A_i), f = sigma(A_f), z = tanh(A_z), o = sigma(A_o)
 *   c_t = f*c_{t-1} + i*z ;  h_t = o*tanh(c_t)
 * Optionally keeps the activated gates [T][G*Dh] and c_t, h_t [T][Dh] for
 * the backward pass.
 */
static void lstm_chain_fwd(int T, int B, int Din, int NH, int Dh, int b, int n,
                           const double *x, const double *W, const double *R,
                           const double *bias, const double *h0, const double *c0,
                           double *h_seq, double *c_seq, double *hT, double *cT,
                           double *keep_gates, double *keep_c, double *keep_h) {
    const int G = LSTM_G, GD = G * Dh, H = NH * Dh, N = NH * GD;
    const double *Rn = R + (size_t)n * Dh * GD;
    double *hp = malloc(sizeof(double) * Dh), *cp = malloc(sizeof(double) * Dh);
    double *a = malloc(sizeof(double) * GD), *s = malloc(sizeof(double) * GD);
    for (int j = 0; j < Dh; ++j) {
        hp[j] = h0 ? h0[(size_t)b * H + n * Dh + j] : 0.0;
        cp[j] = c0 ? c0[(size_t)b * H + n * Dh + j] : 0.0;
    }
    for (int t = 0; t < T; ++t) {
        input_proj_head(Din, N, G, Dh, n, x + ((size_t)t * B + b) * Din, W, bias, a);
        rec_proj(Dh, GD, hp, Rn, s);
        for (int c = 0; c < GD; ++c) a[c] += s[c];
        for (int j = 0; j < Dh; ++j) {
            const double ig = sigm(a[j]), fg = sigm(a[Dh + j]);
            const double zg = tanh(a[2 * Dh + j]), og = sigm(a[3 * Dh + j]);
            const double c = fg * cp[j] + ig * zg;
            const double h = og * tanh(c);
            if (keep_gates) {
                double *kg = keep_gates + (size_t)t * GD;
                kg[j] = ig; kg[Dh + j] = fg; kg[2 * Dh + j] = zg; kg[3 * Dh + j] = og;
            }
            cp[j] = c;
            hp[j] = h;
        }
        const size_t o = ((size_t)t * B + b) * H + (size_t)n * Dh;
        for (int j = 0; j < Dh; ++j) {
            if (h_seq) h_seq[o + j] = hp[j];
            if (c_seq) c_seq[o + j] = cp[j];
            if (keep_c) keep_c[(size_t)t * Dh + j] = cp[j];
            if (keep_h) keep_h[(size_t)t * Dh + j] = hp[j];
        }
    }
    for (int j = 0; j < Dh; ++j) {
        if (hT) hT[(size_t)b * H + n * Dh + j] = hp[j];
        if (cT) cT[(size_t)b * H + n * Dh + j] = cp[j];
    }
    free(hp); free(cp); free(a); free(s);
}

int oracle_lstm_fwd(int T, int B, int Din, int NH, int Dh,
                    const double *x, const double *W, const double *R,
                    const double *bias, const double *h0, const double *c0,
                    const unsigned char *chain_mask,
                    double *h_seq, double *c_seq, double *hT, double *cT) {
    if (T < 0 || B <= 0 || Din <= 0 || NH <= 0 || Dh <= 0) return -1;
    const int nchains = B * NH;
#pragma omp parallel for schedule(dynamic, 1)
    for (int ch = 0; ch < nchains; ++ch) {
        const int b = ch / NH, n = ch % NH;
        if (!chain_on(chain_mask, b, n, NH)) continue;
        lstm_chain_fwd(T, B, Din, NH, Dh, b, n, x, W, R, bias, h0, c0,
                       h_seq, c_seq, hT, cT, NULL, NULL, NULL);
    }
    return 0;
}

/*
 * LSTM backpropagation through time for the loss
 *   L = sum_{t,b,k} dh_seq[t][b][k] * h_t[b][k] + dhT . h_T + dcT . c_T
 * (dhT, dcT may be NULL = 0).  Reverse-time chain rule of the forward above:
 *   dh  = dh_seq[t] + dh_next            tc = tanh(c_t)
 *   dA_o = dh*tc*o*(1-o)                 dc = dc_next + dh*o*(1-tc^2)
 *   dA_i = dc*z*i*(1-i)                  dA_z = dc*i*(1-z^2)
 *   dA_f = dc*c_{t-1}*f*(1-f)            dc_next <- dc*f
 *   dh_next[m] <- sum_c dA[c] * R_n[m][c]
 * Writes the per-step gate gradients dA [T][B][N] of the active chains,
 * dh0/dc0 (the carries left after t = 0) and, if asked, the forward's h_seq.
 */
int oracle_lstm_bptt(int T, int B, int Din, int NH, int Dh,
                     const double *x, const double *W, const double *R,
                     const double *bias, const double *h0, const double *c0,
                     const double *dh_seq, const double *dhT, const double *dcT,
                     const unsigned char *chain_mask,
                     double *dA, double *dh0, double *dc0, double *h_seq_out) {
    if (T <= 0 || B <= 0 || Din <= 0 || NH <= 0 || Dh <= 0) return -1;
    const int G = LSTM_G, GD = G * Dh, H = NH * Dh, N = NH * GD;
    const int nchains = B * NH;
#pragma omp parallel for schedule(dynamic, 1)
    for (int ch = 0; ch < nchains; ++ch) {
        const int b = ch / NH, n = ch % NH;
        if (!chain_on(chain_mask, b, n, NH)) continue;
        const double *Rn = R + (size_t)n * Dh * GD;
        double *gates = malloc(sizeof(double) * (size_t)T * GD);
        double *cs = malloc(sizeof(double) * (size_t)T * Dh);
        double *hs = malloc(sizeof(double) * (size_t)T * Dh);
        lstm_chain_fwd(T, B, Din, NH, Dh, b, n, x, W, R, bias, h0, c0,
                       h_seq_out, NULL, NULL, NULL, gates, cs, hs);
        double *dhn = malloc(sizeof(double) * Dh), *dcn = malloc(sizeof(double) * Dh);
        double *d = malloc(sizeof(double) * GD);
        for (int j = 0; j < Dh; ++j) {
            dhn[j] = dhT ? dhT[(size_t)b * H + n * Dh + j] : 0.0;
            dcn[j] = dcT ? dcT[(size_t)b * H + n * Dh + j] : 0.0;
        }
        for (int t = T - 1; t >= 0; --t) {
            const double *g = gates + (size_t)t * GD;
            for (int j = 0; j < Dh; ++j) {
                const double ig = g[j], fg = g[Dh + j], zg = g[2 * Dh + j], og = g[3 * Dh + j];
                const double ct = cs[(size_t)t * Dh + j];
                const double cprev = t > 0 ? cs[(size_t)(t - 1) * Dh + j]
                                           : (c0 ? c0[(size_t)b * H + n * Dh + j] : 0.0);
                const double dh = dh_seq[((size_t)t * B + b) * H + n * Dh + j] + dhn[j];
                const double tc = tanh(ct);
                const double dc = dcn[j] + dh * og * (1.0 - tc * tc);
                d[j] = dc * zg * ig * (1.0 - ig);
                d[Dh + j] = dc * cprev * fg * (1.0 - fg);
                d[2 * Dh + j] = dc * ig * (1.0 - zg * zg);
                d[3 * Dh + j] = dh * tc * og * (1.0 - og);
                dcn[j] = dc * fg;
            }
            for (int m = 0; m < Dh; ++m) {
                double acc = 0.0;
                const double *rr = Rn + (size_t)m * GD;
                for (int c = 0; c < GD; ++c) acc += d[c] * rr[c];
                dhn[m] = acc;
            }
            double *out = dA + ((size_t)t * B + b) * N + (size_t)n * GD;
            for (int c = 0; c < GD; ++c) out[c] = d[c];
        }
        for (int j = 0; j < Dh; ++j) {
            if (dh0) dh0[(size_t)b * H + n * Dh + j] = dhn[j];
            if (dc0) dc0[(size_t)b * H + n * Dh + j] = dcn[j];
        }
        free(gates); free(cs); free(hs); free(dhn); free(dcn); free(d);
    }
    return 0;
}

/* ------------------------------------------------------------------- GRU */

/*
 * One GRU chain forward (reset-after form, gate order r, z, n):
 *   S = h_{t-1} R_n           (one recurrent product per step)
 *   r = sigma(Gx_r + S_r), u = sigma(Gx_z + S_z)
 *   nn = tanh(Gx_n + r*S_n)   (the bias is part of Gx; no separate recurrent bias)
 *   h_t = (1-u)*nn + u*h_{t-1}
 * Optionally keeps r, u, nn [T][3*Dh], S_n [T][Dh] and h_t [T][Dh].
 */
static void gru_chain_fwd(int T, int B, int Din, int NH, int Dh, int b, int n,
                          const double *x, const double *W, const double *R,
                          const double *bias, const double *h0,
                          double *h_seq, double *hT,
                          double *keep_gates, double *keep_sn, double *keep_h) {
    const int G = GRU_G, GD = G * Dh, H = NH * Dh, N = NH * GD;
    const double *Rn = R + (size_t)n * Dh * GD;
    double *hp = malloc(sizeof(double) * Dh), *hn = malloc(sizeof(double) * Dh);
    double *a = malloc(sizeof(double) * GD), *s = malloc(sizeof(double) * GD);
    for (int j = 0; j < Dh; ++j) hp[j] = h0 ? h0[(size_t)b * H + n * Dh + j] : 0.0;
    for (int t = 0; t < T; ++t) {
        input_proj_head(Din, N, G, Dh, n, x + ((size_t)t * B + b) * Din, W, bias, a);
        rec_proj(Dh, GD, hp, Rn, s);
        for (int j = 0; j < Dh; ++j) {
            const double rg = sigm(a[j] + s[j]);
            const double ug = sigm(a[Dh + j] + s[Dh + j]);
            const double ng = tanh(a[2 * Dh + j] + rg * s[2 * Dh + j]);
            if (keep_gates) {
                double *kg = keep_gates + (size_t)t * GD;
                kg[j] = rg; kg[Dh + j] = ug; kg[2 * Dh + j] = ng;
            }
            if (keep_sn) keep_sn[(size_t)t * Dh + j] = s[2 * Dh + j];
            hn[j] = (1.0 - ug) * ng + ug * hp[j];
        }
        for (int j = 0; j < Dh; ++j) hp[j] = hn[j];
        if (h_seq) {
            const size_t o = ((size_t)t * B + b) * H + (size_t)n * Dh;
            for (int j = 0; j < Dh; ++j) h_seq[o + j] = hp[j];
        }
        if (keep_h)
            for (int j = 0; j < Dh; ++j) keep_h[(size_t)t * Dh + j] = hp[j];
    }
    if (hT)
        for (int j = 0; j < Dh; ++j) hT[(size_t)b * H + n * Dh + j] = hp[j];
    free(hp); free(hn); free(a); free(s);
}

int oracle_gru_fwd(int T, int B, int Din, int NH, int Dh,
                   const double *x, const double *W, const double *R,
                   const double *bias, const double *h0,
                   const unsigned char *chain_mask, double *h_seq, double *hT) {
    if (T < 0 || B <= 0 || Din <= 0 || NH <= 0 || Dh <= 0) return -1;
    const int nchains = B * NH;
#pragma omp parallel for schedule(dynamic, 1)
    for (int ch = 0; ch < nchains; ++ch) {
        const int b = ch / NH, n = ch % NH;
        if (!chain_on(chain_mask, b, n, NH)) continue;
        gru_chain_fwd(T, B, Din, NH, Dh, b, n, x, W, R, bias, h0, h_seq, hT,
                      NULL, NULL, NULL);
    }
    return 0;
}

/*
 * GRU backpropagation through time for L = sum dh_seq . h_t + dhT . h_T
 * (dhT may be NULL = 0).  Chain rule of the forward above, per step:
 *   dh = dh_seq[t] + dh_next
 *   dnn = dh*(1-u)   du = dh*(h_{t-1} - nn)   (direct part to h_{t-1}: dh*u)
 *   dGx_n = dnn*(1-nn^2)      dS_n = dGx_n * r
 *   dGx_r = dS_r = dGx_n*S_n*r*(1-r)
 *   dGx_z = dS_z = du*u*(1-u)
 *   dh_next[m] <- dh[m]*u[m] + sum_c dS[c] * R_n[m][c]
 * dGx (input side: feeds dx, dW, db) and dS (recurrent side: feeds dR)
 * differ only in the n gate.  Both are written [T][B][N] for the active
 * chains, with dh0 the carry left after t = 0.
 */
int oracle_gru_bptt(int T, int B, int Din, int NH, int Dh,
                    const double *x, const double *W, const double *R,
                    const double *bias, const double *h0,
                    const double *dh_seq, const double *dhT,
                    const unsigned char *chain_mask,
                    double *dGx, double *dS, double *dh0, double *h_seq_out) {
    if (T <= 0 || B <= 0 || Din <= 0 || NH <= 0 || Dh <= 0) return -1;
    const int G = GRU_G, GD = G * Dh, H = NH * Dh, N = NH * GD;
    const int nchains = B * NH;
#pragma omp parallel for schedule(dynamic, 1)
    for (int ch = 0; ch < nchains; ++ch) {
        const int b = ch / NH, n = ch % NH;
        if (!chain_on(chain_mask, b, n, NH)) continue;
        const double *Rn = R + (size_t)n * Dh * GD;
        double *gates = malloc(sizeof(double) * (size_t)T * GD);
        double *sn = malloc(sizeof(double) * (size_t)T * Dh);
        double *hs = malloc(sizeof(double) * (size_t)T * Dh);
        gru_chain_fwd(T, B, Din, NH, Dh, b, n, x, W, R, bias, h0, h_seq_out, NULL,
                      gates, sn, hs);
        double *dhn = malloc(sizeof(double) * Dh), *dd = malloc(sizeof(double) * Dh);
        double *dgx = malloc(sizeof(double) * GD), *ds = malloc(sizeof(double) * GD);
        for (int j = 0; j < Dh; ++j) dhn[j] = dhT ? dhT[(size_t)b * H + n * Dh + j] : 0.0;
        for (int t = T - 1; t >= 0; --t) {
            const double *g = gates + (size_t)t * GD;
            for (int j = 0; j < Dh; ++j) {
                const double rg = g[j], ug = g[Dh + j], ng = g[2 * Dh + j];
                const double hprev = t > 0 ? hs[(size_t)(t - 1) * Dh + j]
                                           : (h0 ? h0[(size_t)b * H + n * Dh + j] : 0.0);
                const double dh = dh_seq[((size_t)t * B + b) * H + n * Dh + j] + dhn[j];
                const double dnn = dh * (1.0 - ug);
                const double du = dh * (hprev - ng);
                const double dan = dnn * (1.0 - ng * ng);
                const double dar = dan * sn[(size_t)t * Dh + j] * rg * (1.0 - rg);
                const double dau = du * ug * (1.0 - ug);
                dgx[j] = dar; dgx[Dh + j] = dau; dgx[2 * Dh + j] = dan;
                ds[j] = dar;  ds[Dh + j] = dau;  ds[2 * Dh + j] = dan * rg;
                dd[j] = dh * ug;
            }
            for (int m = 0; m < Dh; ++m) {
                double acc = dd[m];
                const double *rr = Rn + (size_t)m * GD;
                for (int c = 0; c < GD; ++c) acc += ds[c] * rr[c];
                dhn[m] = acc;
            }
            const size_t o = ((size_t)t * B + b) * N + (size_t)n * GD;
            for (int c = 0; c < GD; ++c) {
                if (dGx) dGx[o + c] = dgx[c];
                if (dS) dS[o + c] = ds[c];
            }
        }
        if (dh0)
            for (int j = 0; j < Dh; ++j) dh0[(size_t)b * H + n * Dh + j] = dhn[j];
        free(gates); free(sn); free(hs); free(dhn); free(dd); free(dgx); free(ds);
    }
    return 0;
}

/* ------------------------------------------------ parameter gradients */

/*
 * Gradients of the parameters and of x from the per-step gate gradients.
 * With A = x W + b + h_{t-1} R (block-diagonal), the chain rule gives
 *   db[c]        = sum_{t,b} dG[t][b][c]
 *   dW[k][c]     = sum_{t,b} x[t][b][k] * dG[t][b][c]
 *   dx[t][b][k]  = sum_c dG[t][b][c] * W[k][c]
 *   dR[n][m][c]  = sum_{t,b} h_{t-1}[b][n*Dh+m] * dS[t][b][n*G*Dh+c]
 * where dG is the input-side gradient (dA for the LSTM, dGx for the GRU) and
 * dS the recurrent-side one (dA again for the LSTM).  Any output may be NULL.
 */
int oracle_param_grads(int T, int B, int Din, int NH, int Dh, int G,
                       const double *x, const double *W, const double *h0,
                       const double *h_seq, const double *dG, const double *dS,
                       double *dx, double *dW, double *dR, double *db) {
    if (T <= 0 || B <= 0 || Din <= 0 || NH <= 0 || Dh <= 0 || G <= 0) return -1;
    const int GD = G * Dh, H = NH * Dh, N = NH * GD;
    const long M = (long)T * B;
    if (db) {
#pragma omp parallel for
        for (int c = 0; c < N; ++c) {
            double s = 0.0;
            for (long m = 0; m < M; ++m) s += dG[(size_t)m * N + c];
            db[c] = s;
        }
    }
    if (dW) {
#pragma omp parallel for
        for (int k = 0; k < Din; ++k) {
            double *row = dW + (size_t)k * N;
            for (int c = 0; c < N; ++c) row[c] = 0.0;
            for (long m = 0; m < M; ++m) {
                const double xv = x[(size_t)m * Din + k];
                const double *g = dG + (size_t)m * N;
                for (int c = 0; c < N; ++c) row[c] += xv * g[c];
            }
        }
    }
    if (dx) {
#pragma omp parallel for
        for (long m = 0; m < M; ++m) {
            const double *g = dG + (size_t)m * N;
            for (int k = 0; k < Din; ++k) {
                const double *w = W + (size_t)k * N;
                double s = 0.0;
                for (int c = 0; c < N; ++c) s += g[c] * w[c];
                dx[(size_t)m * Din + k] = s;
            }
        }
    }
    if (dR) {
#pragma omp parallel for
        for (int nm = 0; nm < NH * Dh; ++nm) {
            const int n = nm / Dh, mm = nm % Dh;
            double *row = dR + ((size_t)n * Dh + mm) * GD;
            for (int c = 0; c < GD; ++c) row[c] = 0.0;
            for (int t = 0; t < T; ++t)
                for (int b = 0; b < B; ++b) {
                    const double hv = t > 0 ? h_seq[((size_t)(t - 1) * B + b) * H + n * Dh + mm]
                                            : (h0 ? h0[(size_t)b * H + n * Dh + mm] : 0.0);
                    const double *s = dS + ((size_t)t * B + b) * N + (size_t)n * GD;
                    for (int c = 0; c < GD; ++c) row[c] += hv * s[c];
                }
        }
    }
    return 0;
}

/*
 * The same four sums at chosen entries only (for full-size spot checks):
 *   kind 0: db[c]            idx = {c}
 *   kind 1: dW[k][c]         idx = {k, c}
 *   kind 2: dx[m][k]         idx = {m, k}     (m = t*B + b)
 *   kind 3: dR[n][mm][c]     idx = {n, mm, c}
 * idx holds 3 longs per entry (unused ones ignored).
 */
int oracle_param_grad_entries(int T, int B, int Din, int NH, int Dh, int G, int kind,
                              long nent, const long *idx,
                              const double *x, const double *W, const double *h0,
                              const double *h_seq, const double *dG, const double *dS,
                              double *out) {
    const int GD = G * Dh, H = NH * Dh, N = NH * GD;
    const long M = (long)T * B;
#pragma omp parallel for
    for (long e = 0; e < nent; ++e) {
        const long i0 = idx[3 * e], i1 = idx[3 * e + 1], i2 = idx[3 * e + 2];
        double s = 0.0;
        if (kind == 0) {
            for (long m = 0; m < M; ++m) s += dG[(size_t)m * N + i0];
        } else if (kind == 1) {
            for (long m = 0; m < M; ++m) s += x[(size_t)m * Din + i0] * dG[(size_t)m * N + i1];
        } else if (kind == 2) {
            for (int c = 0; c < N; ++c) s += dG[(size_t)i0 * N + c] * W[(size_t)i1 * N + c];
        } else {
            for (int t = 0; t < T; ++t)
                for (int b = 0; b < B; ++b) {
                    const double hv = t > 0 ? h_seq[((size_t)(t - 1) * B + b) * H + i0 * Dh + i1]
                                            : (h0 ? h0[(size_t)b * H + i0 * Dh + i1] : 0.0);
                    s += hv * dS[((size_t)t * B + b) * N + (size_t)i0 * GD + i2];
                }
        }
        out[e] = s;
    }
    return 0;
}

/* ------------------------------------------------- input projection */

/*
 * The input projection on its own, at chosen rows (rows = NULL: all M rows):
 *   gx[e][c] = b[c] + sum_{k=0..K-1} x[rows[e]][k] * W[k][c]
 * x [M][K], W [K][N], gx [nrows][N].
 */
int oracle_input_proj(long M, int K, int N, const double *x, const double *W,
                      const double *bias, long nrows, const long *rows, double *gx) {
    if (M <= 0 || K <= 0 || N <= 0) return -1;
    const long R = rows ? nrows : M;
    if (rows)
        for (long e = 0; e < nrows; ++e)
            if (rows[e] < 0 || rows[e] >= M) return -1;
#pragma omp parallel for
    for (long e = 0; e < R; ++e) {
        const long m = rows ? rows[e] : e;
        double *o = gx + (size_t)e * N;
        for (int c = 0; c < N; ++c) o[c] = bias ? bias[c] : 0.0;
        for (int k = 0; k < K; ++k) {
            const double xv = x[(size_t)m * K + k];
            const double *w = W + (size_t)k * N;
            for (int c = 0; c < N; ++c) o[c] += xv * w[c];
        }
    }
    return 0;
}
