/*
 * avq_oracle.c -- plain CPU oracle for the AVQ-Attention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the bench's CPU-baseline
 * leg use it.  It shares no code with the HIP library.
 *
 * Source: "AVQ-Attention: Adaptive Vector-Quantized Attention" (van den Dool,
 * Forre, Habibian, Asano, Welling; arXiv 2607.12789v1), cited below by section,
 * equation and algorithm.  Every function is written for a reader checking it
 * against the paper by eye: plain loops, no blocking, no fusion.
 *
 * Precision.  Everything is computed in double on the inputs widened
 * exactly (bf16 and fp32 values are exact doubles): the value sums, the
 * attention outputs, and the two places where floating point decides an
 * integer -- the nearest codeword (Sec. 4.2, Alg. 1) and the top-P parent
 * choice (Eq. 7, Alg. 2).  The paper fixes no precision; double is the
 * plainest reading of "the exact result".  Separate functions report how far
 * each decision is from a tie (used to draw inputs whose decisions do not
 * depend on the rounding of any implementation).
 *
 * Layouts (all row-major, contiguous):
 *   K, V, Q    [B*H][N][d]      token rows of head h of batch b at bh = b*H + h
 *   cb         [H][Mt][d]       Mt = M0*(1+C); rows 0..M0-1 are the parents,
 *                               the C children of parent m are rows
 *                               M0 + m*C ... M0 + m*C + C-1 (Alg. 1 input)
 *   vsum       [B*H][Mt][d]     aggregated values (Eq. 3)
 *   counts     [B*H][Mt]        key counts (Eq. 3)
 *   query tiles: tile t of a head holds queries t*bq ... min(N, (t+1)*bq)-1
 *
 * Pins (tests/oracle_pins.py checks each function against what the paper and
 * the mathematics fix, not against itself):
 *   avqo_assign               generator ground truth, keys equal to codewords,
 *                             hand-built ties, brute force on small inputs
 *   avqo_aggregate            column sums, parent/child count relations
 *   avqo_importance           two-parent closed form; w >= 0, w = 0 iff n = 0,
 *                             sum of w over a tile = its query count
 *   avqo_importance_tiled_f64 first codeword tile holds |I| * N_seen / N of the
 *                             mass; one-codeword tiles: w_0 = |I| n_0 / N; the
 *                             last tile's parents get the exact Eq. 7 values
 *   avqo_select               hand cases with ties, brute-force sort
 *   avqo_attention_*          the three output forms agree; keys = parents and
 *                             keys = children give exact softmax; linearity,
 *                             convex hull; far-away empty child changes nothing
 *   avqo_exact_attention      equal keys, a two-key closed form, keys = parents
 *   avqo_key_margins,
 *   avqo_tile_margin(s)       hand-computed tie distances
 *   avqo_codebook_update_f64  the constraint holds exactly; the children solve
 *                             the weighted least-squares problem (against an
 *                             independent KKT solve and against feasible
 *                             perturbations); N_c times the displacement is
 *                             the same for every child; equal masses shift
 *                             every child alike; decay 0 gives the cell means
 *                             of the keys; massless children take the residual
 * No function is left unpinned.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <float.h>

#define ORACLE_OK 0
#define ORACLE_ERR (-1)

static int64_t mt_of(int M0, int C) { return (int64_t)M0 * (1 + C); }
static int ntiles(int N, int bq) { return (N + bq - 1) / bq; }

/* ------------------------------------------------------------------------ */
/* Sec. 4.2 / Alg. 1: two-level assignment of every key.
 * Eq. 2 distance ||C_a - K_j||^2.  Step 1: nearest parent among the M0 parents;
 * on equal distances the lowest index wins (first minimum).  Step 2: scan the C
 * children of that parent in order, keeping a child only when it is strictly
 * closer than the best child so far; the key moves to the best child only when
 * that child is strictly closer than the parent.
 * Outputs: parent[bh*N + j] = chosen parent row; row[bh*N + j] = final row
 * (the child row if the key moved, else the parent row). */
static double dist2(const double* k, const double* c, int d) {
    double acc = 0.0;
    for (int t = 0; t < d; ++t) {
        double diff = k[t] - c[t];
        acc += diff * diff;
    }
    return acc;
}

int avqo_assign(int B, int H, int N, int d, int M0, int C,
                const double* K, const double* cb, int32_t* parent, int32_t* row) {
    if (B < 0 || H < 0 || N < 0 || d < 1 || M0 < 1 || C < 0) return ORACLE_ERR;
    const int64_t Mt = mt_of(M0, C);
    const int BH = B * H;
#pragma omp parallel for schedule(static)
    for (int bh = 0; bh < BH; ++bh) {
        const int h = bh % H;
        const double* cbh = cb + (int64_t)h * Mt * d;
        for (int j = 0; j < N; ++j) {
            const double* k = K + ((int64_t)bh * N + j) * d;
            int a = 0;
            double dbest = dist2(k, cbh, d);
            for (int m = 1; m < M0; ++m) {
                double dm = dist2(k, cbh + (int64_t)m * d, d);
                if (dm < dbest) { dbest = dm; a = m; }
            }
            int64_t c0 = M0 + (int64_t)a * C;
            double dchild = INFINITY;
            int64_t cstar = c0;
            for (int c = 0; c < C; ++c) {
                double dc = dist2(k, cbh + (c0 + c) * d, d);
                if (dc < dchild) { dchild = dc; cstar = c0 + c; }
            }
            parent[(int64_t)bh * N + j] = a;
            row[(int64_t)bh * N + j] = (C > 0 && dchild < dbest) ? (int32_t)cstar : a;
        }
    }
    return ORACLE_OK;
}

/* Eq. 3 with Alg. 1 (the scatter after each assignment level): every key adds its value and a count of one
 * to its parent row (a parent holds its whole cluster); a key that moved also
 * adds them to its child row. */
int avqo_aggregate(int B, int H, int N, int d, int M0, int C,
                   const double* V, const int32_t* parent, const int32_t* row,
                   double* vsum, int32_t* counts) {
    if (B < 0 || H < 0 || N < 0 || d < 1 || M0 < 1 || C < 0) return ORACLE_ERR;
    const int64_t Mt = mt_of(M0, C);
    const int BH = B * H;
#pragma omp parallel for schedule(static)
    for (int bh = 0; bh < BH; ++bh) {
        double* vs = vsum + (int64_t)bh * Mt * d;
        int32_t* ct = counts + (int64_t)bh * Mt;
        memset(vs, 0, sizeof(double) * Mt * d);
        memset(ct, 0, sizeof(int32_t) * Mt);
        for (int j = 0; j < N; ++j) {
            const double* v = V + ((int64_t)bh * N + j) * d;
            int64_t a = parent[(int64_t)bh * N + j];
            int64_t r = row[(int64_t)bh * N + j];
            for (int t = 0; t < d; ++t) vs[a * d + t] += v[t];
            ct[a] += 1;
            if (r != a) {
                for (int t = 0; t < d; ++t) vs[r * d + t] += v[t];
                ct[r] += 1;
            }
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Eq. 7 with Alg. 2 (the parent pass and the importance), one query tile:
 * importance w[M0] of the parents for the queries Qt[nq][d]:
 *   s_ij = scale * Q_i . C_j over the parents j,
 *   m_i  = max of s_ij over the parents with n_j > 0 (Eq. 18),
 *   A_ij = exp(s_ij - m_i), set to zero where n_j = 0 (Sec. D),
 *   Z_i  = sum_j A_ij n_j,
 *   w_j  = sum_{i in tile} A_ij n_j / Z_i.
 * s: scratch of M0 doubles. */
static double dotd(const double* a, const double* b, int d) {
    double acc = 0.0;
    for (int t = 0; t < d; ++t) acc += a[t] * b[t];
    return acc;
}

static void importance_tile(int nq, int d, int M0, const double* Qt, const double* cbh,
                            const int32_t* n, double scale, double* s, double* w) {
    for (int j = 0; j < M0; ++j) w[j] = 0.0;
    for (int i = 0; i < nq; ++i) {
        const double* q = Qt + (int64_t)i * d;
        double m = -INFINITY;
        for (int j = 0; j < M0; ++j) {
            s[j] = scale * dotd(q, cbh + (int64_t)j * d, d);
            if (n[j] > 0 && s[j] > m) m = s[j];
        }
        double Z = 0.0;
        for (int j = 0; j < M0; ++j)
            if (n[j] > 0) Z += exp(s[j] - m) * n[j];
        for (int j = 0; j < M0; ++j)
            if (n[j] > 0) w[j] += exp(s[j] - m) * n[j] / Z;
    }
}

/* Eq. 7 for every query tile of every (batch, head): w [BH][T][M0]. */
int avqo_importance(int B, int H, int N, int d, int M0, int C,
                    const double* Q, const double* cb, const int32_t* counts,
                    int bq, double scale, double* w) {
    if (B < 0 || H < 0 || N < 0 || d < 1 || M0 < 1 || C < 0 || bq < 1) return ORACLE_ERR;
    const int64_t Mt = mt_of(M0, C);
    const int BH = B * H, T = ntiles(N, bq);
#pragma omp parallel for schedule(static)
    for (int bh = 0; bh < BH; ++bh) {
        const int h = bh % H;
        double* s = (double*)malloc(sizeof(double) * M0);
        for (int t = 0; t < T; ++t) {
            const int i0 = t * bq, i1 = (t + 1) * bq < N ? (t + 1) * bq : N;
            importance_tile(i1 - i0, d, M0, Q + ((int64_t)bh * N + i0) * d,
                            cb + (int64_t)h * Mt * d, counts + (int64_t)bh * Mt, scale, s,
                            w + ((int64_t)bh * T + t) * M0);
        }
        free(s);
    }
    return ORACLE_OK;
}

/* Alg. 2, the parent choice: the P parents of largest importance.  Equal importances are
 * ordered by the lower parent index.  The chosen set is written ascending.
 * w: [R][M0] (R = BH*T rows), sel: [R][P]. */
int avqo_select(int64_t R, int M0, int P, const double* w, int32_t* sel) {
    if (P < 0 || P > M0) return ORACLE_ERR;
    for (int64_t r = 0; r < R; ++r) {
        const double* wr = w + r * M0;
        int32_t* out = sel + r * P;
        int k = 0;
        /* parent j is chosen iff fewer than P parents precede it in the order
         * (larger w first, then lower index) */
        for (int j = 0; j < M0; ++j) {
            int ahead = 0;
            for (int jj = 0; jj < M0; ++jj)
                if (wr[jj] > wr[j] || (wr[jj] == wr[j] && jj < j)) ++ahead;
            if (ahead < P) out[k++] = j;
        }
        if (k != P) return ORACLE_ERR;
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* helper for the output forms */
static int in_sel(const int32_t* sel, int P, int p) {
    for (int k = 0; k < P; ++k) if (sel[k] == p) return 1;
    return 0;
}

/* O3 -- Alg. 2 as written, in double: parent pass with the masked stable max,
 * then for each selected parent: child logits, online-max merge, parent logit
 * recovered as the mean of its C child logits (Eq. 8), correcting weights
 * dA = exp(s_c - m) - exp(s_p - m) zeroed for empty children (Eq. 9, Sec. D),
 * accumulator update (Sec. C, Eq. 17); finally Y = x / z.
 * sel: [BH][T][P] ascending (from avqo_select).  Y: [BH][N][d]. */
int avqo_attention_alg2(int B, int H, int N, int d, int M0, int C,
                        const double* Q, const double* cb, const double* vsum,
                        const int32_t* counts, const int32_t* sel, int P,
                        int bq, double scale, double* Y) {
    if (B < 0 || H < 0 || N < 0 || d < 1 || M0 < 1 || C < 0 || bq < 1 || P < 0 || P > M0) return ORACLE_ERR;
    if (C == 0 && P > 0) return ORACLE_ERR; /* a flat codebook has no children to refine with */
    const int64_t Mt = mt_of(M0, C);
    const int BH = B * H, T = ntiles(N, bq);
#pragma omp parallel for schedule(static)
    for (int bh = 0; bh < BH; ++bh) {
        const int h = bh % H;
        const double* cbh = cb + (int64_t)h * Mt * d;
        const double* vs = vsum + (int64_t)bh * Mt * d;
        const int32_t* n = counts + (int64_t)bh * Mt;
        double* s = (double*)malloc(sizeof(double) * (M0 > C ? M0 : C));
        double* x = (double*)malloc(sizeof(double) * d);
        for (int i = 0; i < N; ++i) {
            const int t = i / bq;
            const int32_t* S = sel + ((int64_t)bh * T + t) * P;
            const double* q = Q + ((int64_t)bh * N + i) * d;
            /* the parent pass */
            double m = -INFINITY;
            for (int j = 0; j < M0; ++j) {
                s[j] = scale * dotd(q, cbh + (int64_t)j * d, d);
                if (n[j] > 0 && s[j] > m) m = s[j];
            }
            double z = 0.0;
            for (int u = 0; u < d; ++u) x[u] = 0.0;
            for (int j = 0; j < M0; ++j) {
                double A = n[j] > 0 ? exp(s[j] - m) : 0.0;
                for (int u = 0; u < d; ++u) x[u] += A * vs[(int64_t)j * d + u];
                z += A * n[j];
            }
            /* the refinement over the selected parents' children */
            for (int k = 0; k < P; ++k) {
                const int64_t c0 = M0 + (int64_t)S[k] * C;
                double mnew = m;
                for (int c = 0; c < C; ++c) {
                    s[c] = scale * dotd(q, cbh + (c0 + c) * d, d);
                    if (n[c0 + c] > 0 && s[c] > mnew) mnew = s[c];
                }
                const double resc = exp(m - mnew);
                for (int u = 0; u < d; ++u) x[u] *= resc;
                z *= resc;
                m = mnew;
                double sp = 0.0;
                for (int c = 0; c < C; ++c) sp += s[c];
                sp /= C;
                for (int c = 0; c < C; ++c) {
                    double dA = n[c0 + c] > 0 ? exp(s[c] - m) - exp(sp - m) : 0.0;
                    for (int u = 0; u < d; ++u) x[u] += dA * vs[(c0 + c) * d + u];
                    z += dA * n[c0 + c];
                }
            }
            double* y = Y + ((int64_t)bh * N + i) * d;
            for (int u = 0; u < d; ++u) y[u] = x[u] / z;
        }
        free(s);
        free(x);
    }
    return ORACLE_OK;
}

/* O2 -- Eq. 4 over the codebook each query tile actually uses (Sec. C, Eq. 15):
 * unselected parents keep (C_j, Vsum_j, n_j); a selected parent p keeps only
 * the keys that did not move, (C_p, Vsum_p - sum_c Vsum_c, n_p - sum_c n_c);
 * its children enter as (C_pc, Vsum_pc, n_pc).  Codewords with no keys are left
 * out.  Y_i = sum_a exp(s_ia - M) Vsum_a / sum_a exp(s_ia - M) n_a. */
int avqo_attention_substituted(int B, int H, int N, int d, int M0, int C,
                               const double* Q, const double* cb, const double* vsum,
                               const int32_t* counts, const int32_t* sel, int P,
                               int bq, double scale, double* Y) {
    if (B < 0 || H < 0 || N < 0 || d < 1 || M0 < 1 || C < 0 || bq < 1 || P < 0 || P > M0) return ORACLE_ERR;
    if (C == 0 && P > 0) return ORACLE_ERR; /* a flat codebook has no children to refine with */
    const int64_t Mt = mt_of(M0, C);
    const int BH = B * H, T = ntiles(N, bq);
    const int64_t Muse = M0 + (int64_t)P * C;
#pragma omp parallel for schedule(static)
    for (int bh = 0; bh < BH; ++bh) {
        const int h = bh % H;
        const double* cbh = cb + (int64_t)h * Mt * d;
        const double* vs = vsum + (int64_t)bh * Mt * d;
        const int32_t* n = counts + (int64_t)bh * Mt;
        /* the substituted codebook of the current tile */
        const double** cw = (const double**)malloc(sizeof(double*) * Muse);
        double* vv = (double*)malloc(sizeof(double) * Muse * d);
        double* nn = (double*)malloc(sizeof(double) * Muse);
        double* sa = (double*)malloc(sizeof(double) * Muse);
        for (int t = 0; t < T; ++t) {
            const int32_t* S = sel + ((int64_t)bh * T + t) * P;
            int64_t a = 0;
            for (int j = 0; j < M0; ++j) {
                cw[a] = cbh + (int64_t)j * d;
                for (int u = 0; u < d; ++u) vv[a * d + u] = vs[(int64_t)j * d + u];
                nn[a] = n[j];
                if (in_sel(S, P, j)) {
                    const int64_t c0 = M0 + (int64_t)j * C;
                    for (int c = 0; c < C; ++c) {
                        for (int u = 0; u < d; ++u) vv[a * d + u] -= vs[(c0 + c) * d + u];
                        nn[a] -= n[c0 + c];
                    }
                }
                ++a;
            }
            for (int k = 0; k < P; ++k) {
                const int64_t c0 = M0 + (int64_t)S[k] * C;
                for (int c = 0; c < C; ++c) {
                    cw[a] = cbh + (c0 + c) * d;
                    for (int u = 0; u < d; ++u) vv[a * d + u] = vs[(c0 + c) * d + u];
                    nn[a] = n[c0 + c];
                    ++a;
                }
            }
            const int i_end = (t + 1) * bq < N ? (t + 1) * bq : N;
            for (int i = t * bq; i < i_end; ++i) {
                const double* q = Q + ((int64_t)bh * N + i) * d;
                double M = -INFINITY;
                for (int64_t b2 = 0; b2 < Muse; ++b2) {
                    sa[b2] = scale * dotd(q, cw[b2], d);
                    if (nn[b2] > 0 && sa[b2] > M) M = sa[b2];
                }
                double* y = Y + ((int64_t)bh * N + i) * d;
                double z = 0.0;
                for (int u = 0; u < d; ++u) y[u] = 0.0;
                for (int64_t b2 = 0; b2 < Muse; ++b2) {
                    if (!(nn[b2] > 0)) continue;
                    double e = exp(sa[b2] - M);
                    for (int u = 0; u < d; ++u) y[u] += e * vv[b2 * d + u];
                    z += e * nn[b2];
                }
                for (int u = 0; u < d; ++u) y[u] /= z;
            }
        }
        free(cw); free(vv); free(nn); free(sa);
    }
    return ORACLE_OK;
}

/* O1 -- quantized-key attention by brute force (Eq. 1 with Eq. 2's K-hat and
 * the regrouping argument of Sec. 3.2): for query i in tile t, key j is
 * represented by its child codeword if it moved to a child of a parent selected
 * for tile t, else by its parent codeword; then ordinary softmax attention over
 * all N keys with the original values.  O(N^2 d). */
int avqo_attention_quantized_keys(int B, int H, int N, int d, int M0, int C,
                                  const double* Q, const double* V, const double* cb,
                                  const int32_t* parent, const int32_t* row,
                                  const int32_t* sel, int P, int bq, double scale,
                                  double* Y) {
    if (B < 0 || H < 0 || N < 0 || d < 1 || M0 < 1 || C < 0 || bq < 1 || P < 0 || P > M0) return ORACLE_ERR;
    const int64_t Mt = mt_of(M0, C);
    const int BH = B * H, T = ntiles(N, bq);
#pragma omp parallel for schedule(static)
    for (int bh = 0; bh < BH; ++bh) {
        const int h = bh % H;
        const double* cbh = cb + (int64_t)h * Mt * d;
        double* s = (double*)malloc(sizeof(double) * (N > 0 ? N : 1));
        for (int i = 0; i < N; ++i) {
            const int t = i / bq;
            const int32_t* S = sel + ((int64_t)bh * T + t) * P;
            const double* q = Q + ((int64_t)bh * N + i) * d;
            double M = -INFINITY;
            for (int j = 0; j < N; ++j) {
                int32_t a = parent[(int64_t)bh * N + j];
                int32_t r = row[(int64_t)bh * N + j];
                int32_t khat = (r != a && in_sel(S, P, a)) ? r : a;
                s[j] = scale * dotd(q, cbh + (int64_t)khat * d, d);
                if (s[j] > M) M = s[j];
            }
            double* y = Y + ((int64_t)bh * N + i) * d;
            double z = 0.0;
            for (int u = 0; u < d; ++u) y[u] = 0.0;
            for (int j = 0; j < N; ++j) {
                double e = exp(s[j] - M);
                const double* v = V + ((int64_t)bh * N + j) * d;
                for (int u = 0; u < d; ++u) y[u] += e * v[u];
                z += e;
            }
            for (int u = 0; u < d; ++u) y[u] /= z;
        }
        free(s);
    }
    return ORACLE_OK;
}

/* Eq. 1 with the 1/sqrt(d)-style scale of Sec. 3.1: exact softmax attention,
 * queries rows [i0, i1) of every head only (so a sample of queries can be
 * checked at large N).  Y: [BH][i1-i0][d]. */
int avqo_exact_attention(int BH, int N, int d, const double* Q, const double* K,
                         const double* V, double scale, int i0, int i1, double* Y) {
    if (BH < 0 || N < 0 || d < 1 || i0 < 0 || i1 < i0 || i1 > N) return ORACLE_ERR;
    const int R = i1 - i0;
#pragma omp parallel for schedule(static)
    for (int bh = 0; bh < BH; ++bh) {
        double* s = (double*)malloc(sizeof(double) * (N > 0 ? N : 1));
        for (int i = i0; i < i1; ++i) {
            const double* q = Q + ((int64_t)bh * N + i) * d;
            double M = -INFINITY;
            for (int j = 0; j < N; ++j) {
                s[j] = scale * dotd(q, K + ((int64_t)bh * N + j) * d, d);
                if (s[j] > M) M = s[j];
            }
            double* y = Y + ((int64_t)bh * R + (i - i0)) * d;
            double z = 0.0;
            for (int u = 0; u < d; ++u) y[u] = 0.0;
            for (int j = 0; j < N; ++j) {
                double e = exp(s[j] - M);
                const double* v = V + ((int64_t)bh * N + j) * d;
                for (int u = 0; u < d; ++u) y[u] += e * v[u];
                z += e;
            }
            for (int u = 0; u < d; ++u) y[u] /= z;
        }
        free(s);
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Distance from a tie, in double (used to draw inputs whose discrete results
 * do not depend on rounding).  For each key, with D = 1 + ||k||^2:
 *   gap of the parent choice      (second smallest - smallest parent distance)/D
 *   gap of the move decision      |best child distance - parent distance| / D
 *   gap of the child choice       (second smallest - smallest child distance)/D
 * and margin = the smallest of those that exist (inf if none).  Two codewords
 * that are the same vector tie exactly for every key, in every precision and
 * summation order, and the comparison rules decide such a tie; those pairs
 * are left out (e.g. with C = 1, Eq. 5 makes the only child equal its
 * parent). */
static int same_vec(const double* a, const double* b, int d) {
    for (int t = 0; t < d; ++t) if (a[t] != b[t]) return 0;
    return 1;
}

int avqo_key_margins(int B, int H, int N, int d, int M0, int C,
                     const double* K, const double* cb, double* margin) {
    if (B < 0 || H < 0 || N < 0 || d < 1 || M0 < 1 || C < 0) return ORACLE_ERR;
    const int64_t Mt = mt_of(M0, C);
    const int BH = B * H;
#pragma omp parallel for schedule(static)
    for (int bh = 0; bh < BH; ++bh) {
        const int h = bh % H;
        const double* cbh = cb + (int64_t)h * Mt * d;
        for (int j = 0; j < N; ++j) {
            const double* k = K + ((int64_t)bh * N + j) * d;
            const double D = 1.0 + dotd(k, k, d);
            double b1 = INFINITY, b2 = INFINITY;
            int a = -1, a2 = -1;
            for (int m = 0; m < M0; ++m) {
                double dm = dist2(k, cbh + (int64_t)m * d, d);
                if (dm < b1) { b2 = b1; a2 = a; b1 = dm; a = m; }
                else if (dm < b2) { b2 = dm; a2 = m; }
            }
            double mg = INFINITY;
            if (a2 >= 0 && !same_vec(cbh + (int64_t)a * d, cbh + (int64_t)a2 * d, d)) mg = (b2 - b1) / D;
            if (C > 0) {
                const double* pa = cbh + (int64_t)a * d;
                double c1 = INFINITY, c2 = INFINITY;
                int i1 = -1, i2 = -1;
                for (int c = 0; c < C; ++c) {
                    const int64_t rowc = M0 + (int64_t)a * C + c;
                    double dc = dist2(k, cbh + rowc * d, d);
                    if (dc < c1) { c2 = c1; i2 = i1; c1 = dc; i1 = (int)rowc; }
                    else if (dc < c2) { c2 = dc; i2 = (int)rowc; }
                }
                if (!same_vec(cbh + (int64_t)i1 * d, pa, d)) {
                    double g2 = fabs(c1 - b1) / D;
                    if (g2 < mg) mg = g2;
                }
                if (i2 >= 0 && !same_vec(cbh + (int64_t)i1 * d, cbh + (int64_t)i2 * d, d)) {
                    double g3 = (c2 - c1) / D;
                    if (g3 < mg) mg = g3;
                }
            }
            margin[(int64_t)bh * N + j] = mg;
        }
    }
    return ORACLE_OK;
}

/* Gap of the top-P choice of one tile, in double: with the importances sorted
 * in decreasing order w(1) >= w(2) >= ..., returns
 * (w(P) - w(P+1)) / max(1, w(P)) when 0 < P < M0 and w(P+1) > 0, else inf
 * (a tie among parents with w = 0 is exact on every side and is broken by the
 * lower index). */
double avqo_tile_margin(int nq, int d, int M0, const double* Qt, const double* cbh,
                        const int32_t* n, int P, double scale) {
    if (P <= 0 || P >= M0 || nq <= 0) return INFINITY;
    double* s = (double*)malloc(sizeof(double) * M0);
    double* w = (double*)malloc(sizeof(double) * M0);
    importance_tile(nq, d, M0, Qt, cbh, n, scale, s, w);
    /* P-th and (P+1)-th largest by selection */
    double wp = 0.0, wq = 0.0;
    for (int j = 0; j < M0; ++j) {
        int ahead = 0;
        for (int jj = 0; jj < M0; ++jj) if (w[jj] > w[j] || (w[jj] == w[j] && jj < j)) ++ahead;
        if (ahead == P - 1) wp = w[j];
        if (ahead == P) wq = w[j];
    }
    free(s); free(w);
    if (!(wq > 0.0)) return INFINITY;
    return (wp - wq) / (wp > 1.0 ? wp : 1.0);
}

/* avqo_tile_margin for every tile of every (batch, head): out[BH][T]. */
int avqo_tile_margins(int B, int H, int N, int d, int M0, int C,
                      const double* Q, const double* cb, const int32_t* counts,
                      int bq, int P, double scale, double* out) {
    if (B < 0 || H < 0 || N < 0 || d < 1 || M0 < 1 || C < 0 || bq < 1) return ORACLE_ERR;
    const int64_t Mt = mt_of(M0, C);
    const int BH = B * H, T = ntiles(N, bq);
#pragma omp parallel for schedule(dynamic)
    for (int r = 0; r < BH * T; ++r) {
        const int bh = r / T, t = r % T, h = bh % H;
        const int i0 = t * bq, i1 = (t + 1) * bq < N ? (t + 1) * bq : N;
        out[r] = avqo_tile_margin(i1 - i0, d, M0, Q + ((int64_t)bh * N + i0) * d,
                                  cb + (int64_t)h * Mt * d, counts + (int64_t)bh * Mt, P, scale);
    }
    return ORACLE_OK;
}

/* App. B, Eq. 13-14: importance with the approximate tiled denominator, in
 * double.  The parents are visited in tiles of `tile` consecutive codewords
 * (tile J holds parents J*tile ... min(M0, (J+1)*tile) - 1).  After tile J:
 *   N_seen(J) = sum of n_j over the parents of the tiles t <= J,
 *   Z~_i(J)   = N / N_seen(J) * sum over t <= J of Z_i(t),
 *               Z_i(t) = sum over j in t of A_ij n_j,
 *   w_j       = sum over the queries i of the tile of A_ij n_j / Z~_i(J), j in J,
 * with N the sum of n_j over all parents, A_ij = exp(s_ij - m_i), m_i the
 * running maximum over the non-empty parents seen so far (the ratio A / Z~
 * does not depend on it), A_ij = 0 where n_j = 0, and w_j = 0 while
 * N_seen(J) = 0.  With one tile (tile >= M0) this is Eq. 7.  w: [BH][T][M0]. */
int avqo_importance_tiled_f64(int B, int H, int N, int d, int M0, int C,
                              const double* Q, const double* cb, const int32_t* counts,
                              int bq, double scale, int tile, double* w) {
    if (B < 0 || H < 0 || N < 0 || d < 1 || M0 < 1 || C < 0 || bq < 1 || tile < 1) return ORACLE_ERR;
    const int64_t Mt = mt_of(M0, C);
    const int BH = B * H, T = ntiles(N, bq);
#pragma omp parallel for schedule(static)
    for (int bh = 0; bh < BH; ++bh) {
        const int h = bh % H;
        const double* cbh = cb + (int64_t)h * Mt * d;
        const int32_t* n = counts + (int64_t)bh * Mt;
        double* s = (double*)malloc(sizeof(double) * M0);
        double ntot = 0.0;
        for (int j = 0; j < M0; ++j) ntot += n[j];
        for (int t = 0; t < T; ++t) {
            double* wt = w + ((int64_t)bh * T + t) * M0;
            for (int j = 0; j < M0; ++j) wt[j] = 0.0;
            const int i_end = (t + 1) * bq < N ? (t + 1) * bq : N;
            for (int i = t * bq; i < i_end; ++i) {
                const double* q = Q + ((int64_t)bh * N + i) * d;
                for (int j = 0; j < M0; ++j) s[j] = scale * dotd(q, cbh + (int64_t)j * d, d);
                double m = -INFINITY, zacc = 0.0, nseen = 0.0;
                for (int j0 = 0; j0 < M0; j0 += tile) {
                    const int j1 = j0 + tile < M0 ? j0 + tile : M0;
                    double mt = m;
                    for (int j = j0; j < j1; ++j) {
                        nseen += n[j];
                        if (n[j] > 0 && s[j] > mt) mt = s[j];
                    }
                    if (mt > m) {  /* new stabiliser: rescale what is accumulated */
                        zacc = m == -INFINITY ? 0.0 : zacc * exp(m - mt);
                        m = mt;
                    }
                    for (int j = j0; j < j1; ++j)
                        if (n[j] > 0) zacc += exp(s[j] - m) * n[j];
                    if (nseen > 0.0) {
                        const double zt = ntot / nseen * zacc;  /* Eq. 13 */
                        for (int j = j0; j < j1; ++j)
                            if (n[j] > 0) wt[j] += exp(s[j] - m) * n[j] / zt;  /* Eq. 14 */
                    }
                }
            }
        }
        free(s);
    }
    return ORACLE_OK;
}

/* App. A, Eq. 11 and Eq. 12: one codebook-update step (training), per head.
 *
 * ksum [B*H][Mt][d], counts [B*H][Mt]: the keys of this batch summed per
 *   codeword and counted, parents over their whole cell and children over the
 *   keys that moved to them (the aggregation of Eq. 3 with the keys in place
 *   of the values; Fig. 2 steps 3 and 4).
 * S [H][Mt][d], Nm [H][Mt]: the EMA statistics (S_x, N_x), updated in place
 *   by Eq. 11 with the batch's sums over all b of the head (one codebook per
 *   head, Sec. 4.1): S <- decay S + (1 - decay) sum k, N <- decay N + (1 -
 *   decay) |{k}|.
 * cb [H][Mt][d]: the codeword positions, updated in place.  A parent moves to
 *   its mean M_p = S_p / N_p (it keeps its position while N_p = 0).  Its
 *   children move to the solution of the mass-weighted least-squares problem
 *   of App. A (minimise sum_c N_c |M_c - C_pc|^2 subject to the mean of the
 *   children being the new parent): Eq. 12, C_pc = M_c - delta / (N_c sigma)
 *   with M_c = S_c / N_c, delta = sum_c M_c - C C_p, sigma = sum_c 1 / N_c.
 *   A child with N_c = 0 has no mean: its current position stands for M_c,
 *   and, having no mass, it takes the whole residual -- the limit of Eq. 12
 *   as its N_c goes to zero: each of the |Z| massless children moves by
 *   -delta / |Z| and the others keep their means.
 */
int avqo_codebook_update_f64(int B, int H, int d, int M0, int C, const double* ksum, const int32_t* counts,
                             double decay, double* S, double* Nm, double* cb) {
  if (B < 0 || H < 0 || d < 1 || M0 < 1 || C < 0 || !(decay >= 0.0 && decay <= 1.0)) return ORACLE_ERR;
  const int64_t Mt = mt_of(M0, C);
  double* kb = (double*)malloc(sizeof(double) * (size_t)d);
  double* M = (double*)malloc(sizeof(double) * (size_t)(C > 0 ? C : 1) * (size_t)d);
  double* delta = (double*)malloc(sizeof(double) * (size_t)d);
  if (!kb || !M || !delta) { free(kb); free(M); free(delta); return ORACLE_ERR; }
  for (int h = 0; h < H; ++h) {
    double* Sh = S + (int64_t)h * Mt * d;
    double* Nh = Nm + (int64_t)h * Mt;
    double* cbh = cb + (int64_t)h * Mt * d;
    /* Eq. 11 for every codeword of the head */
    for (int64_t x = 0; x < Mt; ++x) {
      double cnt = 0.0;
      for (int t = 0; t < d; ++t) kb[t] = 0.0;
      for (int b = 0; b < B; ++b) {
        const int64_t bh = (int64_t)b * H + h;
        cnt += (double)counts[bh * Mt + x];
        for (int t = 0; t < d; ++t) kb[t] += ksum[(bh * Mt + x) * d + t];
      }
      for (int t = 0; t < d; ++t) Sh[x * d + t] = decay * Sh[x * d + t] + (1.0 - decay) * kb[t];
      Nh[x] = decay * Nh[x] + (1.0 - decay) * cnt;
    }
    for (int p = 0; p < M0; ++p) {
      /* the parent: its unconstrained mean, no constraint */
      if (Nh[p] > 0.0)
        for (int t = 0; t < d; ++t) cbh[(int64_t)p * d + t] = Sh[(int64_t)p * d + t] / Nh[p];
      if (C == 0) continue;
      /* the children: unconstrained means, then Eq. 12 */
      const int64_t c0 = M0 + (int64_t)p * C;
      int zeros = 0;
      double sigma = 0.0;
      for (int c = 0; c < C; ++c) {
        const double n = Nh[c0 + c];
        for (int t = 0; t < d; ++t)
          M[c * d + t] = n > 0.0 ? Sh[(c0 + c) * d + t] / n : cbh[(c0 + c) * d + t];
        if (n > 0.0) sigma += 1.0 / n; else ++zeros;
      }
      for (int t = 0; t < d; ++t) {
        double sm = 0.0;
        for (int c = 0; c < C; ++c) sm += M[c * d + t];
        delta[t] = sm - (double)C * cbh[(int64_t)p * d + t];
      }
      for (int c = 0; c < C; ++c) {
        const double n = Nh[c0 + c];
        double share;                      /* the part of delta this child takes */
        if (zeros == 0) share = 1.0 / (n * sigma);
        else share = n > 0.0 ? 0.0 : 1.0 / zeros;
        for (int t = 0; t < d; ++t) cbh[(c0 + c) * d + t] = M[c * d + t] - share * delta[t];
      }
    }
  }
  free(kb); free(M); free(delta);
  return ORACLE_OK;
}

int avqo_version(void) { return 1; }
