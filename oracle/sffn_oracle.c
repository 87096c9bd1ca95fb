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
 *   pre-activation is U (V x) with U in R^{H' x r}, V in R^{r x D}. The
 *   fixed G term, the RMSNorm between the factors and the double activation are
 *   not part of this gate form (the workload specifies ReLU(U(Vx))).
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
 * Returns k = |L|; writes L (ascending) into live_idx when non-null.
 */
static int back_half(int D, int H, int act, int dtype, const double *x, const double *z,
                     const void *W3, const void *W2T, int dense, double *y,
                     double *a_out, int32_t *live_idx) {
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
        a[q] = h * u;
    }
    if (a_out)
        for (int q = 0; q < n_vis; ++q) a_out[q] = a[q];

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
int orc_ffn_standard_batch(int T, int D, int H, int act, int dtype, const void *x,
                           const void *W1, const void *W3, const void *W2T, int dense,
                           double *y, double *z_out, int32_t *live_idx, int32_t *live_count) {
    size_t esz = dtype == ORC_BF16 ? 2 : (dtype == ORC_F32 ? 4 : 8);
    for (int t = 0; t < T; ++t) {
        int k = orc_ffn_standard(D, H, act, dtype, (const char *)x + (size_t)t * D * esz, W1, W3,
                                 W2T, dense, y + (size_t)t * D,
                                 z_out ? z_out + (size_t)t * H : NULL, NULL,
                                 live_idx ? live_idx + (size_t)t * H : NULL);
        if (k < 0) return k;
        if (live_count) live_count[t] = k;
    }
    return 0;
}

int orc_ffn_lopa_batch(int T, int D, int H, int r, int act, int dtype, const void *x,
                       const void *V, const void *U, const void *W3, const void *W2T, int dense,
                       double *y, double *z_out, int32_t *live_idx, int32_t *live_count) {
    size_t esz = dtype == ORC_BF16 ? 2 : (dtype == ORC_F32 ? 4 : 8);
    for (int t = 0; t < T; ++t) {
        int k = orc_ffn_lopa(D, H, r, act, dtype, (const char *)x + (size_t)t * D * esz, V, U, W3,
                             W2T, dense, y + (size_t)t * D, z_out ? z_out + (size_t)t * H : NULL,
                             NULL, NULL, live_idx ? live_idx + (size_t)t * H : NULL);
        if (k < 0) return k;
        if (live_count) live_count[t] = k;
    }
    return 0;
}
