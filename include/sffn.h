/*
 * sffn.h - C ABI of the gate-first sparse FFN forward pass for AMD MI355X
 * (gfx950). Library: libsffn.so, built from activation_sparse_gated_amd/csrc.
 *
 * The operation (page "Model casting: compute the gate, then skip most of the
 * FFN", sections "What an FFN actually computes" and "The 3x ceiling, and why
 * W1 is always on"): for each token x in R^D,
 *
 *     z = W1 x                     gate pre-activation, H entries
 *     h = A(z)                     A = ReLU, or R-S+ (x*sigmoid(x) for x >= 0,
 *                                  0 below; section "Model casting: make
 *                                  sparsity a target")
 *     L = { i : z_i > 0 }          the live hidden units
 *     y = W2 (h (.) W3 x) = sum_{i in L} h_i (W3_i . x) W2[:, i]
 *
 * Only the rows of W3 and the columns of W2 of live units are read; the result
 * is exact, not an approximation. Under LoPA gating (section "LoPA Gating:
 * moving the ceiling") the gate pre-activation is z = U (V x) with a rank-r
 * factorisation, U in R^{H x r}, V in R^{r x D}; H is then the widened
 * hidden size H'.
 *
 * Layout (all row-major, element type given by the handle's dtype):
 *   x    [T x D]   tokens, one row per token
 *   W1   [H x D]   gate; row i belongs to hidden unit i
 *   W3   [H x D]   up projection; row i belongs to hidden unit i
 *   W2T  [H x D]   the down projection W2 (D x H) stored TRANSPOSED, so that
 *                  unit i's column of W2 is the contiguous row W2T[i]
 *   V    [r x D], U [H x r]   LoPA factors
 *   y    [T x D]   fp32 output, overwritten
 * Requirements: D % 8 == 0, D <= 8192; 1 <= H <= 1<<20; LoPA: r % 8 == 0 and
 * 8 <= r <= 2048; 0 <= T <= max_tokens (at most 64, or 8192 for bf16
 * standard-gating handles: union and dense calls with T > 64 run as MFMA
 * GEMMs with the unit products rounded to bf16 (above 1024 tokens the down
 * projection is one hipBLASLt GEMM over every unit: the products of units
 * dead for every token are exact zeros), and those with 5..64 tokens
 * multiply them as two bf16 parts, about 16 significant bits, on MFMA); every
 * pointer 16-byte aligned and a device pointer (hipMalloc or torch CUDA
 * tensors). T == 0 is a no-op.
 *
 * Ownership: the caller owns every tensor. The library borrows them only for
 * the work it enqueues and keeps no pointer between calls, so the same handle
 * can be used with different weight buffers on every call. The handle owns its
 * device scratch (per-token unit products and LoPA rank vectors), allocated
 * once in sffn_create and freed in sffn_destroy.
 *
 * Streams and errors: `stream` is a hipStream_t passed as void* (NULL = the
 * default stream). Arguments are checked synchronously before anything is
 * enqueued; the forward calls never synchronise the host. A launch failure is
 * reported from hipGetLastError; a device fault surfaces at the caller's next
 * synchronisation. One handle must not be used from two streams or threads at
 * once. No C++ exception crosses this ABI.
 */
#ifndef SFFN_H
#define SFFN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct sffn_handle sffn_handle;
typedef int sffn_status;

enum {
    SFFN_OK = 0,
    SFFN_INVALID_ARGUMENT = -1, /* null pointer, bad size, misalignment, T > max_tokens */
    SFFN_UNSUPPORTED = -2,      /* unknown activation, dtype, mode or flag */
    SFFN_OUT_OF_MEMORY = -3,    /* scratch allocation failed in sffn_create */
    SFFN_HIP_ERROR = -4,        /* a HIP runtime call or launch failed */
    SFFN_INTERNAL = -5          /* unexpected internal failure */
};

enum { SFFN_ACT_RELU = 0, SFFN_ACT_RSPLUS = 1 };
/* Weight storage. SFFN_I8: weight-only int8, symmetric per stored row: the
 * weight is q[i][j] * scale[i] with q int8 and one fp32 scale per row (the
 * pages report int8 weight-only models and kernels, paper card Table 17 and
 * Figure 9; the scheme is this library's reading). x stays bf16 and every
 * product and sum is fp32. Forward calls: the _i8 ones (standard gating with
 * r == 0, LoPA with r > 0). */
/* SFFN_I4: weight-only int4 with one fp32 scale per 128 columns of a row
 * (one scale per row would round nearly every weight of a row with a large
 * bias-like entry to zero); codes in [-8, 7], packed two per byte, column 2j
 * in the low nibble. D % 128 == 0. Standard gating: W1, W3, W2T in int4.
 * LoPA (r > 0, r % 16 == 0): W3 and W2T in int4, the low-rank gate V, U in
 * int8 rows as for SFFN_I8 (a U row's bias-like first column rules out one
 * scale per row in int4, and r need not be a multiple of 128). Forward calls:
 * the _i4 ones. */
enum { SFFN_BF16 = 0, SFFN_F32 = 1, SFFN_I8 = 2, SFFN_I4 = 3 };
/* How a batch of T tokens moves data; never changes the result.
 * PER_TOKEN: each token reads the W3 rows and W2T rows of its own live set
 *            (bf16 standard-gating batches above 64 tokens, where nearly every
 *            unit is live for some token, run as UNION; live lists stay per
 *            token).
 * UNION:     the union of the tokens' live sets is read once and each row is
 *            applied to the tokens for which it is live (batched decode: the
 *            pages note the speedup is quoted at batch size 1 and erodes as
 *            the batch grows, since the union fills up). */
enum { SFFN_MODE_PER_TOKEN = 0, SFFN_MODE_UNION = 1 };

/* Gate options of LoPA handles (r > 0): the full LoPA gate of page "Model
 * casting: compute the gate, then skip most of the FFN", section "LoPA
 * Gating: moving the ceiling", z = G x + U RMSNorm(V x), with the double
 * activation described there. Bits of sffn_create's `flags`.
 *   G_TILED     add (G x)_i = x_{i mod D}: the fixed tiled-identity term
 *               (paper card Figure 6 (c)); it reads no weight bytes.
 *   RMSNORM     normalise the rank vector t = V x to t / sqrt(mean(t^2) + 1e-6)
 *               before U (eps and the unit gain are this library's reading:
 *               the pages give neither).
 *   DOUBLE_ACT  a_i = A(z_i) * A(W3_i . x) instead of A(z_i) * (W3_i . x); a
 *               live unit whose A(W3_i . x) is 0 contributes nothing and its
 *               W2T row is not read (the s_gated skip of the paper card's
 *               Table 5). The live set is still {i : z_i > 0}. */
enum { SFFN_FLAG_G_TILED = 1u, SFFN_FLAG_RMSNORM = 2u, SFFN_FLAG_DOUBLE_ACT = 4u };

/*
 * Create a handle for one FFN shape.
 *   D, H        model width and hidden width (H' for LoPA handles)
 *   r           LoPA rank; 0 for a standard-gating handle
 *   max_tokens  largest T any forward call on this handle will pass (1..64;
 *               1..8192 for SFFN_BF16 handles with r == 0)
 *   act         SFFN_ACT_RELU or SFFN_ACT_RSPLUS
 *   dtype       SFFN_BF16 (weights and x as bf16 bit patterns; products in
 *               fp32), SFFN_F32, SFFN_I8 (int8 weights with per-row
 *               scales, x bf16; needs D % 16 == 0 and r % 16 == 0), or
 *               SFFN_I4 (int4 weights with per-128-column scales, x bf16;
 *               needs D % 128 == 0, and r % 16 == 0 for LoPA)
 *   flags       0, or for LoPA handles any of SFFN_FLAG_G_TILED,
 *               SFFN_FLAG_RMSNORM, SFFN_FLAG_DOUBLE_ACT (other bits, or any
 *               bit on a standard handle: SFFN_UNSUPPORTED)
 * On success *out receives the handle. Allocates device scratch on the
 * current device: about min(max_tokens, 64) * (H + r) floats plus
 * max_tokens * H bytes, and for max_tokens > 64 also H * 256 ceil(max_tokens /
 * 256) bf16 unit products; for max_tokens > 1024 also a hipBLASLt handle and its
 * 64 MiB workspace (SFFN_HIP_ERROR if the library cannot create the handle).
 */
sffn_status sffn_create(sffn_handle **out, int D, int H, int r, int max_tokens, int act,
                        int dtype, unsigned flags);

/*
 * Launch plan. sffn_create fixes it from the shape alone (no environment
 * variable or other outside input takes part): the kernel of each step, its
 * block shape and the unit-range splits of the down passes, with the constants
 * chosen from measured sweeps on MI355X. It chooses data movement only, never
 * the mathematics: results differ between plans only by rounding (summation
 * order, and where a path rounds the unit products for its MFMA operands, as
 * described under Requirements). sffn_create also clears the scratch that must
 * start zeroed, on a private stream it waits for; it never synchronises the
 * whole device.
 */

/* Frees the handle and its scratch. NULL is ignored. The caller must make sure
 * no work using the handle is still pending (synchronise the stream first). */
void sffn_destroy(sffn_handle *h);

/*
 * Dense comparator: y = W2 (A(W1 x) (.) W3 x) over all H units, reading every
 * row of W1, W3 and W2T (page "Model casting: compute the gate, then skip most
 * of the FFN", section "What an FFN actually computes"). Standard-gating
 * handles only.
 */
sffn_status sffn_forward_dense(sffn_handle *h, const void *x, const void *W1, const void *W3,
                               const void *W2T, float *y, int T, void *stream);

/*
 * Gate-first sparse forward, standard gating (sections "The 3x ceiling, and
 * why W1 is always on" and "Compute the gate first, then skip the dead
 * units"): all of W1 is read; W3 rows and W2T rows are read only for live
 * units.
 *   mode        SFFN_MODE_PER_TOKEN or SFFN_MODE_UNION
 *   live_count  nullable device int32 [T]: k_t = |L_t| per token
 *   live_idx    nullable device int32 [T x H]: token t's live units in
 *               live_idx[t*H : t*H + k_t] (ascending); entries past k_t are
 *               unspecified. live_count and live_idx must be both set or both
 *               NULL.
 */
sffn_status sffn_forward_sparse(sffn_handle *h, const void *x, const void *W1, const void *W3,
                                const void *W2T, float *y, int T, int mode, int32_t *live_count,
                                int32_t *live_idx, void *stream);

/*
 * The batch-1 sparse forward of sffn_forward_sparse (standard gating, bf16
 * weights, fp32 accumulation) for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. It takes no handle and allocates nothing: the unit products
 * handed from the gate kernel to the down kernel live in a static device array
 * of the library (16384 floats, 64 KiB, one per GPU until the process ends).
 * The T tokens of x run one after another through the same kernels as the
 * handle path, each on its own live set; the output is the same up to the
 * summation order of the down pass.
 *   x [T x D] bf16, W1, W3, W2T [H x D] bf16 (W2 stored transposed), y [T x D]
 *   fp32 (overwritten): device pointers, 16-byte aligned, owned by the caller.
 *   D a positive multiple of 8, at most 4096; H in [1, 16384]; T >= 0 (0 is a
 *   no-op); act SFFN_ACT_RELU or SFFN_ACT_RSPLUS; stream a hipStream_t.
 * Errors: SFFN_INVALID_ARGUMENT for a size beyond these limits (H above 16384
 * says so) or a bad pointer, SFFN_UNSUPPORTED for an unknown activation, both
 * before any launch; sffn_last_error(NULL) gives the message. Calls that
 * overlap on one GPU (concurrent streams, or host threads) share the static
 * array and race: serialise them.
 */
sffn_status sffn_forward_sparse_noalloc(const void *x, const void *W1, const void *W3,
                                        const void *W2T, float *y, int D, int H, int T, int act,
                                        void *stream);

/*
 * Gate-first sparse forward, LoPA gating without the fixed G term:
 * z = U (V x), then the same skip as sffn_forward_sparse. The rank vector
 * V x is kept in fp32 up to the live test. LoPA handles (r > 0) only.
 */
sffn_status sffn_forward_lopa(sffn_handle *h, const void *x, const void *V, const void *U,
                              const void *W3, const void *W2T, float *y, int T, int mode,
                              int32_t *live_count, int32_t *live_idx, void *stream);

/*
 * Gate-first sparse forward and the dense comparator with weight-only int8
 * weights (SFFN_I8 handles): as sffn_forward_sparse / sffn_forward_dense, with
 * W1, W3, W2T int8 [H x D] row-major (16-byte aligned) and W1_scale, W3_scale,
 * W2T_scale fp32 [H] (4-byte aligned): weight (i, j) of each matrix is
 * q[i][j] * scale[i]. x is bf16 [T x D], y fp32 [T x D]. Calls with 2..64
 * tokens, in either mode and dense, read every weight code once for the batch:
 * one gate pass (VALU for 2 tokens; from 3 tokens MFMA on exactly decoded codes,
 * with the W1 and W3 rows staged together) computes the W3 dots of the units live
 * for some token; then the union's W2T rows
 * are read once (union, dense) or each token's own live rows are gathered
 * (per-token lists). Errors as for the other forward calls; a non-int8 handle
 * gives SFFN_INVALID_ARGUMENT.
 */
/*
 * Gate-first sparse forward and the dense comparator with weight-only int4
 * weights (SFFN_I4 handles): as the _i8 calls, with W1, W3, W2T packed int4
 * [H x D/2] bytes (16-byte aligned) and W1_scale, W3_scale, W2T_scale fp32
 * [H x D/128] (4-byte aligned): weight (i, j) is code(i, j) * scale[i][j / 128].
 * x bf16 [T x D], y fp32 [T x D]; batches of 2..64 tokens read every code
 * once per call, as for int8. Errors as for the other forward calls; a non-int4
 * handle gives SFFN_INVALID_ARGUMENT.
 */
sffn_status sffn_forward_sparse_i4(sffn_handle *h, const void *x, const void *W1,
                                   const float *W1_scale, const void *W3, const float *W3_scale,
                                   const void *W2T, const float *W2T_scale, float *y, int T,
                                   int mode, int32_t *live_count, int32_t *live_idx,
                                   void *stream);
sffn_status sffn_forward_dense_i4(sffn_handle *h, const void *x, const void *W1,
                                  const float *W1_scale, const void *W3, const float *W3_scale,
                                  const void *W2T, const float *W2T_scale, float *y, int T,
                                  void *stream);

/*
 * LoPA gating with weight-only int8 weights (SFFN_I8 handles with r > 0, r a
 * multiple of 16): as sffn_forward_lopa, with V int8 [r x D], U int8 [H x r],
 * W3 and W2T int8 [H x D] (row-major, 16-byte aligned) and one fp32 scale per
 * stored row of each (V_scale [r], U_scale [H], W3_scale [H], W2T_scale [H],
 * 4-byte aligned): t = V x is exact in fp32 on the dequantised rows, the gate
 * options of the handle (G, RMSNorm, double activation) apply as for bf16.
 * Batches of 5..64 tokens (without RMSNorm) read every code once per call on
 * MFMA, in either mode; batches of 2..4 tokens (D <= 4096), and larger ones
 * with RMSNorm, read the weights once per group of 2..4 consecutive tokens;
 * other calls run token by token. Errors as for the other forward calls; a
 * non-int8 or r == 0 handle gives SFFN_INVALID_ARGUMENT.
 */
sffn_status sffn_forward_lopa_i8(sffn_handle *h, const void *x, const void *V,
                                 const float *V_scale, const void *U, const float *U_scale,
                                 const void *W3, const float *W3_scale, const void *W2T,
                                 const float *W2T_scale, float *y, int T, int mode,
                                 int32_t *live_count, int32_t *live_idx, void *stream);

/*
 * LoPA gating with int4 up and down weights (SFFN_I4 handles with r > 0, r a
 * multiple of 16): as sffn_forward_lopa_i8 for V int8 [r x D] and U int8
 * [H x r] with one fp32 scale per stored row (V_scale [r], U_scale [H]), and
 * W3, W2T packed int4 [H x D/2] bytes with W3_scale, W2T_scale fp32
 * [H x D/128] as for sffn_forward_sparse_i4. The gate options of the handle
 * apply as for bf16; batches are planned as for sffn_forward_lopa_i8. Errors as
 * for the other forward calls; a non-int4 or r == 0 handle gives
 * SFFN_INVALID_ARGUMENT.
 */
sffn_status sffn_forward_lopa_i4(sffn_handle *h, const void *x, const void *V,
                                 const float *V_scale, const void *U, const float *U_scale,
                                 const void *W3, const float *W3_scale, const void *W2T,
                                 const float *W2T_scale, float *y, int T, int mode,
                                 int32_t *live_count, int32_t *live_idx, void *stream);

sffn_status sffn_forward_sparse_i8(sffn_handle *h, const void *x, const void *W1,
                                   const float *W1_scale, const void *W3, const float *W3_scale,
                                   const void *W2T, const float *W2T_scale, float *y, int T,
                                   int mode, int32_t *live_count, int32_t *live_idx,
                                   void *stream);
sffn_status sffn_forward_dense_i8(sffn_handle *h, const void *x, const void *W1,
                                  const float *W1_scale, const void *W3, const float *W3_scale,
                                  const void *W2T, const float *W2T_scale, float *y, int T,
                                  void *stream);

/*
 * Sparse expert FFNs inside a top-K mixture of experts (K = 1 or 2), the
 * generalisation named in section "Where it generalizes" of page "Model
 * casting: compute the gate, then skip most of the FFN": every expert is a
 * gate-first sparse FFN of the handle's shape (bf16, standard gating), and
 *   y[t] = sum_k gate[t*K + k] * FFN_{route[t*K + k]}(x[t])   (k ascending).
 *   E              number of experts (1..1024)
 *   W1, W3, W2T    HOST arrays of E device pointers: expert e's weights, each
 *                  [H x D] bf16, 16-byte aligned (only routed experts are read)
 *   route, gate    HOST arrays [T x K]: expert index in [0, E) and weight of
 *                  each (token, k); read during the call only
 *   dense          0: each expert runs the sparse forward over the tokens routed
 *                  to it as one batch in union mode; 1: the dense comparator
 * x bf16 [T x D], y fp32 [T x D] (overwritten); T <= max_tokens. Uses the
 * handle's scratch, so calls on one handle must not overlap. Errors as for
 * the other forward calls (a route entry outside [0, E): INVALID_ARGUMENT).
 */
sffn_status sffn_forward_moe(sffn_handle *h, const void *x, int E, const void *const *W1,
                             const void *const *W3, const void *const *W2T, int K,
                             const int32_t *route, const float *gate, float *y, int T, int dense,
                             void *stream);

/* Message of the last failure on this handle; with NULL, the calling thread's
 * last failure that had no handle (e.g. in sffn_create). Never NULL. */
const char *sffn_last_error(const sffn_handle *h);

/* Name of a status code. Never NULL. */
const char *sffn_status_string(sffn_status s);

/* ABI version of the library (this header: 1). */
int sffn_abi_version(void);

/*
 * Instrumentation, for measuring the kernels' own durations. enable = 0 turns
 * it off; enable = N > 0 times the forward calls 0, N, 2N, ... counted from
 * this call (N = 1: every call): each kernel such a call enqueues is launched
 * with a start/stop event pair recorded at the kernel's own begin and end, and
 * the other calls launch as usual, so a long stream of calls keeps the GPU as
 * busy as it is untimed. sffn_timing_read
 * synchronises with those events and returns, for kernel kind `kind`, the
 * summed duration in milliseconds and the number of launches since the last
 * reset (reset != 0 clears the totals of every kind after reading). Kinds are
 * numbered 0 .. sffn_kernel_kinds()-1 and named by sffn_kernel_name. Each timed
 * launch holds two events until the next sffn_timing_read folds them into the
 * totals and returns them to the handle's pool, so a long timed run should be
 * read now and then. Timing adds events between launches, so it is off by
 * default and must stay off during stream capture. Like the forward calls,
 * these two must not run on one handle from two threads at once.
 */
sffn_status sffn_timing_enable(sffn_handle *h, int enable);
sffn_status sffn_timing_read(sffn_handle *h, int kind, double *total_ms, int64_t *launches,
                             int reset);
int sffn_kernel_kinds(void);
const char *sffn_kernel_name(int kind);

#ifdef __cplusplus
}
#endif

#endif /* SFFN_H */
