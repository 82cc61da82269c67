/*
 * wtconv_oracle.c -- plain, slow, fp64 CPU oracle of the WTConv layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header or constant with the
 * HIP library.
 *
 * What it computes (source: "Fast and Memory-Efficient Wavelet Convolutions
 * via I/O-Aware Reformulation", Aflalo, Finder, Amoyal, Treister, Freifeld,
 * arXiv 2608.10805, as summarised on gist.science/pt, "Resumo Tecnico",
 * sections "Metodologia" and "Principais Contribuicoes"; the 2x2 Haar filter
 * matrices with their factor 1/2 are those of the cybasar.com WTConv
 * tutorial, section 3):
 *
 *   The unfused operator, one intermediate tensor per stage, exactly as the
 *   reference sequence of framework ops does it:
 *     A0 = X
 *     for l = 1..L:   (S_LL, S_LH, S_HL, S_HH)^l = H(A^{l-1});  A^l = S^l_LL
 *                     Y^l_s = gamma[l,c,s] * conv_{K[l,c,s]}(S^l_s)
 *     R^{L+1} = 0
 *     for l = L..1:   R^l = H^T(Y^l_LL + R^{l+1}, Y^l_LH, Y^l_HL, Y^l_HH)
 *     y = beta[c] * (conv_{Kb[c]}(X) + bias[c]) + R^1
 *   conv is a k x k cross-correlation with 'same' zero padding (k odd).
 *   H is the stride-2 2x2 Haar analysis with filters
 *     LL = 1/2 [[1, 1],[ 1, 1]]    LH = 1/2 [[1,-1],[ 1,-1]]
 *     HL = 1/2 [[1, 1],[-1,-1]]    HH = 1/2 [[1,-1],[-1, 1]]
 *   (rows index y, columns index x) and H^T is its transpose (the stride-2
 *   transposed convolution with the same filters).
 *
 *   The backward is the reverse-mode adjoint of that sequence, taken op by
 *   op with every forward intermediate kept in memory: adjoint of a
 *   correlation is a scatter with the same kernel, adjoint of H is H^T and
 *   vice versa.  Parameter gradients are summed per plane, then over the
 *   batch in ascending b, so results do not depend on the thread count.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   subband order (LL, LH, HL, HH); base conv carries a bias, wavelet convs
 *   do not; scales beta[C], gamma[L,C,4] multiply after the conv; each level
 *   zero-pads its own coefficient grid.
 *
 * Grids with an odd side: the tutorial's analysis is a stride-2 convolution
 * with TensorFlow's 'SAME' padding (cybasar.com, section 3), which for an
 * odd side appends one zero row (column) at the end, so level l has
 * ceil(h_{l-1}/2) rows.  H^T is the transpose of that map: the transposed
 * stride-2 convolution cropped back to the h_{l-1} rows of the finer grid.
 *
 * Layouts (all contiguous, row-major):
 *   x, y, dy, dx : [B][C][H][W]
 *   w_base       : [C][k][k]      b_base, s_base : [C]
 *   w_wav        : [L][C][4][k][k]  s_wav : [L][C][4]
 *
 * Precision: fp64 throughout, no intermediate rounding.
 */
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* The four 2x2 analysis filters, [s][row][col], with the factor 1/2. */
static const double HAAR[4][2][2] = {
    {{0.5, 0.5}, {0.5, 0.5}},    /* LL */
    {{0.5, -0.5}, {0.5, -0.5}},  /* LH: difference along x */
    {{0.5, 0.5}, {-0.5, -0.5}},  /* HL: difference along y */
    {{0.5, -0.5}, {-0.5, 0.5}},  /* HH: diagonal */
};

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads of the calls that follow (n >= 1; timing only, results do not
 * depend on it). */
void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* out[i][j] = sum_{u,v} K[u][v] * z[i+u-p][j+v-p], zero outside z. */
static void conv_same(const double* z, int h, int w, const double* K, int k,
                      double* out) {
    int p = k / 2;
    for (int i = 0; i < h; ++i)
        for (int j = 0; j < w; ++j) {
            double acc = 0.0;
            for (int u = 0; u < k; ++u) {
                int ii = i + u - p;
                if (ii < 0 || ii >= h) continue;
                for (int v = 0; v < k; ++v) {
                    int jj = j + v - p;
                    if (jj < 0 || jj >= w) continue;
                    acc += K[u * k + v] * z[ii * w + jj];
                }
            }
            out[i * w + j] = acc;
        }
}

/* Adjoint of conv_same with respect to z: dz += scatter of dout through K. */
static void conv_same_adj_input(const double* dout, int h, int w,
                                const double* K, int k, double* dz) {
    int p = k / 2;
    for (int i = 0; i < h; ++i)
        for (int j = 0; j < w; ++j) {
            double g = dout[i * w + j];
            for (int u = 0; u < k; ++u) {
                int ii = i + u - p;
                if (ii < 0 || ii >= h) continue;
                for (int v = 0; v < k; ++v) {
                    int jj = j + v - p;
                    if (jj < 0 || jj >= w) continue;
                    dz[ii * w + jj] += K[u * k + v] * g;
                }
            }
        }
}

/* Gradient of conv_same with respect to K: dK[u][v] += sum dout * z-shift. */
static void conv_same_adj_kernel(const double* dout, const double* z, int h,
                                 int w, int k, double* dK) {
    int p = k / 2;
    for (int u = 0; u < k; ++u)
        for (int v = 0; v < k; ++v) {
            double acc = 0.0;
            for (int i = 0; i < h; ++i) {
                int ii = i + u - p;
                if (ii < 0 || ii >= h) continue;
                for (int j = 0; j < w; ++j) {
                    int jj = j + v - p;
                    if (jj < 0 || jj >= w) continue;
                    acc += dout[i * w + j] * z[ii * w + jj];
                }
            }
            dK[u * k + v] += acc;
        }
}

/* Rows (columns) of the next coarser grid. */
static int half_up(int n) { return (n + 1) / 2; }

/* H: z is h x w; sub[s] is ceil(h/2) x ceil(w/2).  Taps past the end of z
   read zero (the appended row / column of an odd side). */
static void haar_analysis(const double* z, int h, int w, double* sub[4]) {
    int h2 = half_up(h), w2 = half_up(w);
    for (int s = 0; s < 4; ++s)
        for (int i = 0; i < h2; ++i)
            for (int j = 0; j < w2; ++j) {
                double acc = 0.0;
                for (int a = 0; a < 2; ++a)
                    for (int b = 0; b < 2; ++b) {
                        int r = 2 * i + a, q = 2 * j + b;
                        if (r < h && q < w) acc += HAAR[s][a][b] * z[r * w + q];
                    }
                sub[s][i * w2 + j] = acc;
            }
}

/* H^T: z (h x w) = transposed stride-2 conv of the four subbands
   (ceil(h/2) x ceil(w/2)), cropped to h x w. */
static void haar_synthesis(double* const sub[4], int h, int w, double* z) {
    int h2 = half_up(h), w2 = half_up(w);
    memset(z, 0, sizeof(double) * (size_t)h * w);
    for (int s = 0; s < 4; ++s)
        for (int i = 0; i < h2; ++i)
            for (int j = 0; j < w2; ++j) {
                double c = sub[s][i * w2 + j];
                for (int a = 0; a < 2; ++a)
                    for (int b = 0; b < 2; ++b) {
                        int r = 2 * i + a, q = 2 * j + b;
                        if (r < h && q < w) z[r * w + q] += HAAR[s][a][b] * c;
                    }
            }
}

/* Per-plane working set: every forward intermediate of the cascade. */
typedef struct {
    int L, H, W;
    double* base;      /* conv_Kb(X), H x W */
    double* S[8][4];   /* S^l_s, level l = 1..L (index l-1) */
    double* Y[8][4];   /* gamma * conv(S^l_s) */
    double* CS[8][4];  /* conv(S^l_s), kept for the gamma gradient */
    double* R[9];      /* R^l at level l-1 resolution, l = 1..L+1 */
    double* T[8];      /* Y^l_LL + R^{l+1} */
} plane_ws;

/* Side of level l's grid: l halvings, each rounded up. */
static int lvl_h(int H, int l) {
    for (int m = 0; m < l; ++m) H = half_up(H);
    return H;
}

static void ws_alloc(plane_ws* ws, int L, int H, int W) {
    ws->L = L; ws->H = H; ws->W = W;
    ws->base = (double*)calloc((size_t)H * W, sizeof(double));
    for (int l = 1; l <= L; ++l) {
        size_t n = (size_t)lvl_h(H, l) * lvl_h(W, l);
        for (int s = 0; s < 4; ++s) {
            ws->S[l - 1][s] = (double*)calloc(n, sizeof(double));
            ws->Y[l - 1][s] = (double*)calloc(n, sizeof(double));
            ws->CS[l - 1][s] = (double*)calloc(n, sizeof(double));
        }
        ws->T[l - 1] = (double*)calloc(n, sizeof(double));
    }
    for (int l = 1; l <= L + 1; ++l) {
        size_t n = (size_t)lvl_h(H, l - 1) * lvl_h(W, l - 1);
        ws->R[l - 1] = (double*)calloc(n, sizeof(double));
    }
}

static void ws_free(plane_ws* ws) {
    free(ws->base);
    for (int l = 1; l <= ws->L; ++l) {
        for (int s = 0; s < 4; ++s) {
            free(ws->S[l - 1][s]); free(ws->Y[l - 1][s]); free(ws->CS[l - 1][s]);
        }
        free(ws->T[l - 1]);
    }
    for (int l = 1; l <= ws->L + 1; ++l) free(ws->R[l - 1]);
}

/* Forward of one (b, c) plane; keeps every intermediate in ws. */
static void plane_forward(plane_ws* ws, const double* X, int c, int C, int k,
                          const double* w_base, const double* b_base,
                          const double* s_base, const double* w_wav,
                          const double* s_wav, double* y) {
    int L = ws->L, H = ws->H, W = ws->W, kk = k * k;
    /* analysis cascade on the raw LL, one subband conv per (l, s) */
    const double* A = X;
    for (int l = 1; l <= L; ++l) {
        int hp = lvl_h(H, l - 1), wp = lvl_h(W, l - 1);
        int hl = lvl_h(H, l), wl = lvl_h(W, l);
        haar_analysis(A, hp, wp, ws->S[l - 1]);
        for (int s = 0; s < 4; ++s) {
            const double* K = w_wav + (((size_t)(l - 1) * C + c) * 4 + s) * kk;
            double g = s_wav[((size_t)(l - 1) * C + c) * 4 + s];
            conv_same(ws->S[l - 1][s], hl, wl, K, k, ws->CS[l - 1][s]);
            for (int t = 0; t < hl * wl; ++t)
                ws->Y[l - 1][s][t] = g * ws->CS[l - 1][s][t];
        }
        A = ws->S[l - 1][0];
    }
    /* synthesis cascade, deepest level first */
    {
        double* Rz = ws->R[L];  /* R^{L+1} = 0 */
        memset(Rz, 0, sizeof(double) * (size_t)lvl_h(H, L) * lvl_h(W, L));
    }
    for (int l = L; l >= 1; --l) {
        int hl = lvl_h(H, l), wl = lvl_h(W, l);
        for (int t = 0; t < hl * wl; ++t)
            ws->T[l - 1][t] = ws->Y[l - 1][0][t] + ws->R[l][t];
        double* sub[4] = {ws->T[l - 1], ws->Y[l - 1][1], ws->Y[l - 1][2],
                          ws->Y[l - 1][3]};
        haar_synthesis(sub, lvl_h(H, l - 1), lvl_h(W, l - 1), ws->R[l - 1]);
    }
    /* scaled base path plus the reconstruction */
    conv_same(X, H, W, w_base + (size_t)c * kk, k, ws->base);
    double beta = s_base[c], bias = b_base[c];
    for (int t = 0; t < H * W; ++t)
        y[t] = beta * (ws->base[t] + bias) + ws->R[0][t];
}

int oracle_fwd(int B, int C, int H, int W, int L, int k, const double* x,
               const double* w_base, const double* b_base,
               const double* s_base, const double* w_wav,
               const double* s_wav, double* y) {
    if (B < 0 || C < 0 || H < 0 || W < 0 || L < 1 || L > 8 || k < 1 ||
        (k % 2) == 0)
        return -1;
    long nplanes = (long)B * C;
    size_t hw = (size_t)H * W;
#pragma omp parallel
    {
        plane_ws ws;
        ws_alloc(&ws, L, H, W);
#pragma omp for schedule(dynamic, 1)
        for (long pl = 0; pl < nplanes; ++pl) {
            int c = (int)(pl % C);
            plane_forward(&ws, x + pl * hw, c, C, k, w_base, b_base, s_base,
                          w_wav, s_wav, y + pl * hw);
        }
        ws_free(&ws);
    }
    return 0;
}

/*
 * Backward.  Given dy = dLoss/dy, returns dx and the gradients of every
 * parameter tensor (overwritten, not accumulated).
 */
int oracle_bwd(int B, int C, int H, int W, int L, int k, const double* x,
               const double* dy, const double* w_base, const double* b_base,
               const double* s_base, const double* w_wav, const double* s_wav,
               double* dx, double* dw_base, double* db_base, double* ds_base,
               double* dw_wav, double* ds_wav) {
    if (B < 0 || C < 0 || H < 0 || W < 0 || L < 1 || L > 8 || k < 1 ||
        (k % 2) == 0)
        return -1;
    int kk = k * k;
    long nplanes = (long)B * C;
    size_t hw = (size_t)H * W;
    /* per-plane parameter-gradient slots, summed over b afterwards */
    size_t per = (size_t)kk + 2 + (size_t)L * 4 * kk + (size_t)L * 4;
    double* part = (double*)calloc((size_t)(nplanes > 0 ? nplanes : 1) * per,
                                   sizeof(double));
    if (!part) return -3;
#pragma omp parallel
    {
        plane_ws ws;
        ws_alloc(&ws, L, H, W);
        double* y = (double*)malloc(sizeof(double) * (hw ? hw : 1));
        double* dT = (double*)malloc(sizeof(double) * (hw ? hw : 1));
        double* dR = (double*)malloc(sizeof(double) * (hw ? hw : 1));
        double* dA = (double*)malloc(sizeof(double) * (hw ? hw : 1));
        double* dAn = (double*)malloc(sizeof(double) * (hw ? hw : 1));
        double* dSub[4];
        double* dSc[4];
        for (int s = 0; s < 4; ++s) {
            dSub[s] = (double*)malloc(sizeof(double) * (hw ? hw : 1));
            dSc[s] = (double*)malloc(sizeof(double) * (hw ? hw : 1));
        }
        double* dSll = (double*)malloc(sizeof(double) * (hw ? hw : 1));
        /* dS^l_s from the conv adjoints, kept per level for the analysis
           backward (which runs deepest level first) */
        double* dS[8][4];
        for (int l = 1; l <= L; ++l)
            for (int s = 0; s < 4; ++s)
                dS[l - 1][s] = (double*)calloc(
                    (size_t)lvl_h(H, l) * lvl_h(W, l) + 1, sizeof(double));

#pragma omp for schedule(dynamic, 1)
        for (long pl = 0; pl < nplanes; ++pl) {
            int c = (int)(pl % C);
            const double* X = x + pl * hw;
            const double* G = dy + pl * hw;
            double* P = part + (size_t)pl * per;
            double* pKb = P;
            double* pbias = P + kk;
            double* pbeta = P + kk + 1;
            double* pK = P + kk + 2;
            double* pg = P + kk + 2 + (size_t)L * 4 * kk;
            plane_forward(&ws, X, c, C, k, w_base, b_base, s_base, w_wav,
                          s_wav, y);
            double beta = s_base[c], bias = b_base[c];
            const double* Kb = w_base + (size_t)c * kk;
            double* dX = dx + pl * hw;

            /* y = beta * (base + bias) + R^1 */
            double sb = 0.0, sg = 0.0;
            for (size_t t = 0; t < hw; ++t) {
                sb += G[t] * (ws.base[t] + bias);
                sg += G[t];
            }
            *pbeta = sb;
            *pbias = beta * sg;
            for (size_t t = 0; t < hw; ++t) dT[t] = beta * G[t];
            conv_same_adj_kernel(dT, X, H, W, k, pKb);
            memset(dX, 0, sizeof(double) * hw);
            conv_same_adj_input(dT, H, W, Kb, k, dX);
            memcpy(dR, G, sizeof(double) * hw); /* dR^1 = dy */

            /* synthesis cascade backward: l = 1..L */
            for (int l = 1; l <= L; ++l) {
                int hp = lvl_h(H, l - 1), wp = lvl_h(W, l - 1);
                int hl = lvl_h(H, l), wl = lvl_h(W, l);
                /* R^l = H^T(T^l, Y_LH, Y_HL, Y_HH) -> d(...) = H(dR^l) */
                haar_analysis(dR, hp, wp, dSub);
                /* T^l = Y^l_LL + R^{l+1}: both receive dSub[0] */
                /* Y^l_s = gamma * CS^l_s,  CS = conv_K(S) */
                for (int s = 0; s < 4; ++s) {
                    const double* K =
                        w_wav + (((size_t)(l - 1) * C + c) * 4 + s) * kk;
                    double g = s_wav[((size_t)(l - 1) * C + c) * 4 + s];
                    double acc = 0.0;
                    for (int t = 0; t < hl * wl; ++t)
                        acc += dSub[s][t] * ws.CS[l - 1][s][t];
                    pg[(size_t)(l - 1) * 4 + s] = acc;
                    for (int t = 0; t < hl * wl; ++t) dSc[s][t] = g * dSub[s][t];
                    conv_same_adj_kernel(dSc[s], ws.S[l - 1][s], hl, wl, k,
                                         pK + ((size_t)(l - 1) * 4 + s) * kk);
                    memset(dS[l - 1][s], 0, sizeof(double) * (size_t)hl * wl);
                    conv_same_adj_input(dSc[s], hl, wl, K, k, dS[l - 1][s]);
                }
                memcpy(dR, dSub[0], sizeof(double) * (size_t)hl * wl);
            }

            /* analysis cascade backward: l = L..1.
               S^l = H(A^{l-1}); A^l = S^l_LL feeds level l+1. */
            memset(dA, 0, sizeof(double) * hw); /* dA^L = 0 */
            for (int l = L; l >= 1; --l) {
                int hp = lvl_h(H, l - 1), wp = lvl_h(W, l - 1);
                int hl = lvl_h(H, l), wl = lvl_h(W, l);
                for (int t = 0; t < hl * wl; ++t)
                    dSll[t] = dS[l - 1][0][t] + dA[t];
                double* sub[4] = {dSll, dS[l - 1][1], dS[l - 1][2],
                                  dS[l - 1][3]};
                haar_synthesis(sub, hp, wp, dAn);
                memcpy(dA, dAn, sizeof(double) * (size_t)hp * wp);
            }
            for (size_t t = 0; t < hw; ++t) dX[t] += dA[t];
        }
        for (int l = 1; l <= L; ++l)
            for (int s = 0; s < 4; ++s) free(dS[l - 1][s]);
        for (int s = 0; s < 4; ++s) { free(dSub[s]); free(dSc[s]); }
        free(dSll); free(dA); free(dAn); free(dR); free(dT); free(y);
        ws_free(&ws);
    }
    /* fixed-order reduction over the batch */
    for (int c = 0; c < C; ++c) {
        double* dKb = dw_base + (size_t)c * kk;
        for (int t = 0; t < kk; ++t) dKb[t] = 0.0;
        db_base[c] = 0.0;
        ds_base[c] = 0.0;
        for (int l = 0; l < L; ++l)
            for (int s = 0; s < 4; ++s) {
                double* dK = dw_wav + (((size_t)l * C + c) * 4 + s) * kk;
                for (int t = 0; t < kk; ++t) dK[t] = 0.0;
                ds_wav[((size_t)l * C + c) * 4 + s] = 0.0;
            }
        for (int b = 0; b < B; ++b) {
            const double* P = part + ((size_t)b * C + c) * per;
            for (int t = 0; t < kk; ++t) dKb[t] += P[t];
            db_base[c] += P[kk];
            ds_base[c] += P[kk + 1];
            for (int l = 0; l < L; ++l)
                for (int s = 0; s < 4; ++s) {
                    double* dK = dw_wav + (((size_t)l * C + c) * 4 + s) * kk;
                    const double* pK = P + kk + 2 + ((size_t)l * 4 + s) * kk;
                    for (int t = 0; t < kk; ++t) dK[t] += pK[t];
                    ds_wav[((size_t)l * C + c) * 4 + s] +=
                        P[kk + 2 + (size_t)L * 4 * kk + (size_t)l * 4 + s];
                }
        }
    }
    free(part);
    return 0;
}

/* Test hooks: the single-level building blocks, exposed so that the test
   suite can pin them on their own (z is h x w, sub is
   4 x ceil(h/2) x ceil(w/2)). */
int oracle_haar_analysis(int h, int w, const double* z, double* sub) {
    if (h < 0 || w < 0) return -2;
    size_t q = (size_t)half_up(h) * half_up(w);
    double* s4[4] = {sub, sub + q, sub + 2 * q, sub + 3 * q};
    haar_analysis(z, h, w, s4);
    return 0;
}

int oracle_haar_synthesis(int h, int w, const double* sub, double* z) {
    if (h < 0 || w < 0) return -2;
    size_t q = (size_t)half_up(h) * half_up(w);
    double* s4[4] = {(double*)sub, (double*)sub + q, (double*)sub + 2 * q,
                     (double*)sub + 3 * q};
    haar_synthesis(s4, h, w, z);
    return 0;
}
