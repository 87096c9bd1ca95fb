/*
 * Plain fp64 CPU oracle for the gate-first sparse FFN forward pass.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may call, link or load
 * this file; only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark do. It shares no code, header, table or helper with the HIP
 * library.
 *
 * What it computes, and where the pages define it:
 *
 *   Gated FFN, one token (page "Model casting: compute the gate, then skip most
 *   of the FFN", section "What an FFN actually computes"):
 *       y = W2 (A(W1 x) (.) (W3 x)),  W1, W3 in R^{H x D},  W2 in R^{D x H}.
 *   W2 is passed transposed, W2T[i][j] = W2[j][i], so unit i's column of W2 is
 *   the row W2T[i].
 *
 *   Gate first, skip the dead units (same section, and section "The 3x ceiling,
 *   and why W1 is always on"): if A(W1 x)_i = 0 then row i of W3 and column i
 *   of W2 are not needed; the skip is exact, not an approximation.
 *
 *   R-S+ (section "Model casting: make sparsity a target"): x*sigmoid(x) for
 *   x >= 0 and 0 for x < 0. ReLU is max(0, x).
 *
 *   LoPA gate (section "LoPA Gating: moving the ceiling"): the gate
 *   pre-activation is U (V x) with U in R^{H' x r}, V in R^{r x D}
 *   (orc_ffn_lopa). The full form the paper trains (same section, and the
 *   paper card's Figure 6 and Table 4) is orc_ffn_lopa_full:
 *       z = G x + U RMSNorm(V x),   a_i = A(z_i) * A(u_i)  (double activation)
 *   with G the tiled identity, (G x)_i = x_{i mod D} (Figure 6 (c)), and
 *   RMSNorm(t) = t / sqrt(mean_m t_m^2 + eps). The pages give neither eps nor
 *   a gain: eps = 1e-6 and unit gain are this oracle's reading. With double
 *   activation a live unit whose A(u_i) is 0 contributes nothing, and its W2
 *   column is skipped (the s_gated skip of the paper card's Table 5).
 *
 * Arithmetic: every input is widened exactly to double (bf16 bit patterns by a
 * 16-bit shift into an fp32, fp32 directly). Every dot product is a plain
 * ascending loop. The live set is L = {i : z_i > 0}: strict, decided on z, so
 * R-S+(0) = 0 and a live unit never has h_i = 0 from a positive z's rounding.
 * y starts at +0.0 and accumulates a_i * W2T[i][j] in ascending i.
 *
 * Dense and sparse modes visit the same units in the same order; a dead unit
 * contributes a_i = h_i * u_i = +-0, and adding +-0 to a sum that started at
 * +0.0 never changes it, so the two modes are bitwise equal.
 *
 * OpenMP splits only independent outputs (rows i of the gate and of W3, and
 * column ranges of y), never a sum, so results do not depend on the thread
 * count.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_BF16 = 0, ORC_F32 = 1, ORC_F64 = 2 };
enum { ORC_RELU = 0, ORC_RSPLUS = 1 };
enum { ORC_G_TILED = 1, ORC_RMSNORM = 2, ORC_DOUBLE_ACT = 4 };
#define ORC_RMS_EPS 1e-6

static double elem(const void *p, int dtype, size_t idx) {
    if (dtype == ORC_BF16) {
        uint32_t u = (uint32_t)((const uint16_t *)p)[idx] << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    if (dtype == ORC_F32) return (double)((const float *)p)[idx];
    return ((const double *)p)[idx];
}

/* A(z): ReLU or R-S+. */
double orc_activation(int act, double z) {
    if (act == ORC_RELU) return z > 0.0 ? z : 0.0;
    if (z >= 0.0) return z / (1.0 + exp(-z)); /* z * sigmoid(z) */
    return 0.0;
}

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void orc_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* row . vector over n entries, ascending index. */
static double dot_row(const void *M, int dtype, size_t row, int n, const double *v) {
    double s = 0.0;
    size_t base = row * (size_t)n;
    for (int j = 0; j < n; ++j) s += elem(M, dtype, base + (size_t)j) * v[j];
    return s;
}

/*
 * Back half shared by standard and LoPA gating, given the gate
 * pre-activation z[H]: h = A(z), L = {z > 0}, u_i = W3_i . x, a_i = h_i u_i,
 * y = sum_i a_i W2T_i.  dense != 0 visits every unit, else only L.
 * double_act != 0: a_i = h_i * A(u_i), and in sparse mode the units with
 * a_i == 0 are left out of the W2 pass (their terms are exact zeros).
 * Returns k = |L|; writes L (ascending) into live_idx when non-null, and the
 * number of units that enter the W2 pass into *k2_out when non-null.
 */
static int back_half2(int D, int H, int act, int dtype, const double *x, const double *z,
                      const void *W3, const void *W2T, int dense, int double_act, double *y,
                      double *a_out, int32_t *live_idx, int32_t *k2_out) {
    int k = 0;
    for (int i = 0; i < H; ++i)
        if (z[i] > 0.0) {
            if (live_idx) live_idx[k] = i;
            ++k;
        }
    /* the units visited, ascending */
    int n_vis = dense ? H : k;
    int32_t *vis = (int32_t *)malloc((size_t)(n_vis > 0 ? n_vis : 1) * sizeof(int32_t));
    double *a = (double *)malloc((size_t)(n_vis > 0 ? n_vis : 1) * sizeof(double));
    if (!vis || !a) {
        free(vis);
        free(a);
        return -1;
    }
    int m = 0;
    for (int i = 0; i < H; ++i)
        if (dense || z[i] > 0.0) vis[m++] = i;

#pragma omp parallel for schedule(static)
    for (int q = 0; q < n_vis; ++q) {
        int i = vis[q];
        double h = orc_activation(act, z[i]);
        double u = dot_row(W3, dtype, (size_t)i, D, x);
        a[q] = h * (double_act ? orc_activation(act, u) : u);
    }
    if (a_out)
        for (int q = 0; q < n_vis; ++q) a_out[q] = a[q];
    /* s_gated: with double activation, sparse mode drops the units whose a_i is 0 */
    if (double_act && !dense) {
        int w = 0;
        for (int q = 0; q < n_vis; ++q)
            if (a[q] != 0.0) {
                vis[w] = vis[q];
                a[w] = a[q];
                ++w;
            }
        n_vis = w;
    }
    if (k2_out) {
        int c = 0;
        for (int q = 0; q < n_vis; ++q)
            if (z[vis[q]] > 0.0 && (!double_act || a[q] != 0.0)) ++c;
        *k2_out = c;
    }

    /* y_j = sum over visited i (ascending) of a_i * W2T[i][j]; columns split across threads */
#pragma omp parallel for schedule(static)
    for (int j = 0; j < D; ++j) y[j] = 0.0;
    const int JB = 256;
#pragma omp parallel for schedule(static)
    for (int j0 = 0; j0 < D; j0 += JB) {
        int j1 = j0 + JB < D ? j0 + JB : D;
        for (int q = 0; q < n_vis; ++q) {
            size_t base = (size_t)vis[q] * (size_t)D;
            double aq = a[q];
            for (int j = j0; j < j1; ++j) y[j] += aq * elem(W2T, dtype, base + (size_t)j);
        }
    }
    free(vis);
    free(a);
    return k;
}

static int back_half(int D, int H, int act, int dtype, const double *x, const double *z,
                     const void *W3, const void *W2T, int dense, double *y, double *a_out,
                     int32_t *live_idx) {
    return back_half2(D, H, act, dtype, x, z, W3, W2T, dense, 0, y, a_out, live_idx, NULL);
}

static double *widen(const void *v, int dtype, size_t n) {
    double *out = (double *)malloc((n > 0 ? n : 1) * sizeof(double));
    if (!out) return NULL;
    for (size_t j = 0; j < n; ++j) out[j] = elem(v, dtype, j);
    return out;
}

/*
 * Standard gating, one token.
 *   x [D], W1/W3/W2T [H x D] row-major, all of `dtype`.
 *   y [D] (out), z [H] (out, nullable), a [H or k] (out, nullable: a_i for the
 *   visited units), live_idx [H] (out, nullable, ascending). Returns k or < 0.
 */
int orc_ffn_standard(int D, int H, int act, int dtype, const void *x, const void *W1,
                     const void *W3, const void *W2T, int dense, double *y, double *z_out,
                     double *a_out, int32_t *live_idx) {
    if (D <= 0 || H < 0) return -2;
    double *xd = widen(x, dtype, (size_t)D);
    double *z = (double *)malloc((size_t)(H > 0 ? H : 1) * sizeof(double));
    if (!xd || !z) {
        free(xd);
        free(z);
        return -1;
    }
#pragma omp parallel for schedule(static)
    for (int i = 0; i < H; ++i) z[i] = dot_row(W1, dtype, (size_t)i, D, xd);
    if (z_out) memcpy(z_out, z, (size_t)H * sizeof(double));
    int k = back_half(D, H, act, dtype, xd, z, W3, W2T, dense, y, a_out, live_idx);
    free(xd);
    free(z);
    return k;
}

/*
 * LoPA gating, one token: t = V x (r entries), z = U t, then the same back
 * half.  V [r x D], U [H x r]; t_out [r] nullable.
 */
int orc_ffn_lopa(int D, int H, int r, int act, int dtype, const void *x, const void *V,
                 const void *U, const void *W3, const void *W2T, int dense, double *y,
                 double *z_out, double *t_out, double *a_out, int32_t *live_idx) {
    if (D <= 0 || H < 0 || r <= 0) return -2;
    double *xd = widen(x, dtype, (size_t)D);
    double *t = (double *)malloc((size_t)r * sizeof(double));
    double *z = (double *)malloc((size_t)(H > 0 ? H : 1) * sizeof(double));
    if (!xd || !t || !z) {
        free(xd);
        free(t);
        free(z);
        return -1;
    }
#pragma omp parallel for schedule(static)
    for (int m = 0; m < r; ++m) t[m] = dot_row(V, dtype, (size_t)m, D, xd);
#pragma omp parallel for schedule(static)
    for (int i = 0; i < H; ++i) z[i] = dot_row(U, dtype, (size_t)i, r, t);
    if (t_out) memcpy(t_out, t, (size_t)r * sizeof(double));
    if (z_out) memcpy(z_out, z, (size_t)H * sizeof(double));
    int k = back_half(D, H, act, dtype, xd, z, W3, W2T, dense, y, a_out, live_idx);
    free(xd);
    free(t);
    free(z);
    return k;
}

/*
 * Batches: the FFN is a per-token function, so a batch of T tokens is T
 * independent single-token evaluations (x [T x D], y [T x D]; live_idx
 * [T x H] holds each token's ascending list, live_count [T] its k). Whether a
 * GPU batch reads the union of the live sets once or each token's list on its
 * own changes only data movement, never these values.
 */
/*
 * Full LoPA gate (flags: ORC_G_TILED | ORC_RMSNORM | ORC_DOUBLE_ACT), one token,
 * in the order of the pages: t = V x; t <- t / sqrt(mean(t^2) + eps) when
 * RMSNORM; z_i = (G x)_i + U_i . t with (G x)_i = x_{i mod D} when G_TILED;
 * then the back half with double activation when DOUBLE_ACT. t_out receives
 * the (normalised) t. *k2_out: units that enter the W2 pass (sparse mode).
 */
int orc_ffn_lopa_full(int D, int H, int r, int act, int dtype, unsigned flags, const void *x,
                      const void *V, const void *U, const void *W3, const void *W2T, int dense,
                      double *y, double *z_out, double *t_out, double *a_out, int32_t *live_idx,
                      int32_t *k2_out) {
    if (D <= 0 || H < 0 || r <= 0) return -2;
    if (flags & ~(unsigned)(ORC_G_TILED | ORC_RMSNORM | ORC_DOUBLE_ACT)) return -3;
    double *xd = widen(x, dtype, (size_t)D);
    double *t = (double *)malloc((size_t)r * sizeof(double));
    double *z = (double *)malloc((size_t)(H > 0 ? H : 1) * sizeof(double));
    if (!xd || !t || !z) {
        free(xd);
        free(t);
        free(z);
        return -1;
    }
#pragma omp parallel for schedule(static)
    for (int m = 0; m < r; ++m) t[m] = dot_row(V, dtype, (size_t)m, D, xd);
    if (flags & ORC_RMSNORM) {
        double ss = 0.0;
        for (int m = 0; m < r; ++m) ss += t[m] * t[m];
        double inv = 1.0 / sqrt(ss / (double)r + ORC_RMS_EPS);
        for (int m = 0; m < r; ++m) t[m] *= inv;
    }
#pragma omp parallel for schedule(static)
    for (int i = 0; i < H; ++i) {
        double g = (flags & ORC_G_TILED) ? xd[i % D] : 0.0;
        z[i] = g + dot_row(U, dtype, (size_t)i, r, t);
    }
    if (t_out) memcpy(t_out, t, (size_t)r * sizeof(double));
    if (z_out) memcpy(z_out, z, (size_t)H * sizeof(double));
    int k = back_half2(D, H, act, dtype, xd, z, W3, W2T, dense, (flags & ORC_DOUBLE_ACT) ? 1 : 0,
                       y, a_out, live_idx, k2_out);
    free(xd);
    free(t);
    free(z);
    return k;
}
