// Device kernels of the gate-first sparse FFN forward pass, written for CDNA4
// (gfx950: 64-wide wavefronts, 256 CUs in 8 XCDs, HBM3E).
//
// The method (page "Model casting: compute the gate, then skip most of the
// FFN", sections "What an FFN actually computes" and "The 3x ceiling, and why
// W1 is always on"): compute the gate z = W1 x first, keep the units with
// z_i > 0, and read row i of W3 and column i of W2 (row i of W2T) only for
// those. LoPA (section "LoPA Gating: moving the ceiling") replaces W1 x by
// U (V x).
//
// Work split, per forward call:
//   k_rank_proj        LoPA only: t = V x, fp32 rank vector per token.
//   k_gate_up_sparse   row-split over hidden units. Each block owns up to 64
//                      consecutive units: it streams their gate rows (W1, or
//                      U against t), applies the live test z > 0 on the fp32
//                      accumulator, compacts the live units into an LDS list
//                      with a wavefront ballot + lane prefix (mbcnt), then
//                      reads only the live W3 rows and writes the unit
//                      products a_i = A(z_i) (W3_i . x) (0 for dead units).
//   k_gate_up_dense    dense comparator: W1 and W3 rows read together for
//                      every unit (the merged gate/up pass of the FFN tutorial,
//                      section 9.2 case 3).
//   k_down             column-split over D. Each block owns a slice of y,
//                      compacts the nonzero a_i into LDS (ballot + prefix) and
//                      accumulates a_i * W2T[i, slice]. W2T rows are
//                      contiguous, so each live unit's slice is one coalesced
//                      run of 16-byte loads; no block shares an output, so
//                      there are no atomics and no second reduction pass.
//   k_live_list        only when the caller asks for the live sets: ascending
//                      per-token index lists from the live flags.
//
// Weights are streamed with nontemporal 16-byte loads; every product is
// accumulated in fp32.
#include <hip/hip_runtime.h>
#include <type_traits>
#include <stdint.h>

namespace sffn {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;
constexpr int MAXT = 64;          // largest token batch
constexpr int K1_THREADS = 256;   // gate/up blocks: 4 waves
constexpr int K1_WAVES = K1_THREADS / WAVE;
constexpr int K1_MAX_ROWS = 64;   // units per gate/up block (one per lane of wave 0)
constexpr int K2_THREADS = 512;   // down blocks: 8 waves
constexpr int K2_WAVES = K2_THREADS / WAVE;
constexpr int K2_CAP = 2048;      // live units compacted per pass of a down block

// bf16 weights are carried as raw uint16 bit patterns.
template <typename WT> struct Elem;
template <> struct Elem<uint16_t> {
    __device__ static inline float get1(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
    static constexpr int VEC = 8;  // elements per 16-byte load
    __device__ static inline float get(const u32x4& v, int k) {
        uint32_t w = v[k >> 1];
        return (k & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
    }
};
template <> struct Elem<float> {
    __device__ static inline float get1(float v) { return v; }
    static constexpr int VEC = 4;
    __device__ static inline float get(const u32x4& v, int k) { return __uint_as_float(v[k]); }
};

__device__ inline u32x4 load_stream(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ inline u32x4 load_cached(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ inline float wave_sum(float v) {
#pragma unroll
    for (int o = WAVE / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
    return v;
}

// Full LoPA gate options (page "Model casting: compute the gate, then skip
// most of the FFN", section "LoPA Gating: moving the ceiling"; paper card
// Figure 6 (c) and Table 5): z = G x + U RMSNorm(V x) with (G x)_i = x_{i mod D},
// and double activation a_i = A(z_i) A(u_i). eps and a unit gain are this
// library's reading (the pages give neither).
constexpr unsigned LOPA_G_TILED = 1u, LOPA_RMSNORM = 2u, LOPA_DOUBLE_ACT = 4u;
constexpr float RMS_EPS = 1e-6f;

// A(z): ReLU, or R-S+ = z * sigmoid(z) for z >= 0 and 0 below.
__device__ inline float activation(int act, float z) {
    if (act == 0) return z > 0.0f ? z : 0.0f;
    return z >= 0.0f ? z / (1.0f + expf(-z)) : 0.0f;
}

// ---------------------------------------------------------------------------
// Register tile of one D-long row: lane l holds columns c*64*VEC + l*VEC + [0, VEC)
// for chunk c < NC. D % 8 == 0, so a chunk is wholly inside or wholly outside D.
template <typename WT, int NC>
struct RowTile {
    static constexpr int VEC = Elem<WT>::VEC;
    static constexpr int CW = WAVE * VEC;
    u32x4 v[NC];

    __device__ inline void load(const WT* row, int D, int lane, bool valid, bool stream) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int col = c * CW + lane * VEC;
            if (valid && col < D)
                v[c] = stream ? load_stream(row + col) : load_cached(row + col);
            else
                v[c] = u32x4{0u, 0u, 0u, 0u};
        }
    }
};

template <typename WT, int NC>
struct XTile {
    static constexpr int VEC = Elem<WT>::VEC;
    float f[NC][VEC];

    __device__ inline void load(const WT* x, int D, int lane) {
        RowTile<WT, NC> t;
        t.load(x, D, lane, true, false);
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int k = 0; k < VEC; ++k) f[c][k] = Elem<WT>::get(t.v[c], k);
    }
    __device__ inline float dot(const RowTile<WT, NC>& w) const {
        float s = 0.0f;
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int k = 0; k < VEC; ++k) s = fmaf(Elem<WT>::get(w.v[c], k), f[c][k], s);
        return s;
    }
};

// ---------------------------------------------------------------------------
// Back half of a gate/up block, once z_lds[t * 64 + rloc] holds the gate
// pre-activations of this block's `nrows` units for T tokens:
// compaction of the live (unit, token) pairs into an LDS list, then the W3
// rows of the live units only.
//   per-token mode: one list entry per live (unit, token) pair; the W3 row is
//                   read once per entry.
//   union mode:     one entry per unit live for any token, with a token mask;
//                   the W3 row is read once and applied to each live token.
template <typename WT, int NC>
__device__ void compact_and_up(const float* z_lds, uint32_t* list, uint64_t* masks, int* n_list,
                               const WT* __restrict__ x, const WT* __restrict__ W3,
                               float* __restrict__ a_out, uint8_t* __restrict__ live_out,
                               int row0, int nrows, int D, int H, int T, int act, int union_mode,
                               int double_act) {
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    if (wave == 0) {
        // wave 0: lane = unit within the block
        const bool in = lane < nrows;
        const int row = row0 + lane;
        int base = 0;
        uint64_t tokmask = 0;
        for (int t = 0; t < T; ++t) {
            const bool live = in && z_lds[t * K1_MAX_ROWS + lane] > 0.0f;
            if (in) {
                if (live_out) live_out[(size_t)t * H + row] = live ? 1 : 0;
                if (!live) a_out[(size_t)t * H + row] = 0.0f;
            }
            if (live) tokmask |= (uint64_t)1 << t;
            if (!union_mode) {
                const uint64_t m = __ballot(live);
                const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                          __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
                if (live) list[base + pos] = (uint32_t)lane | ((uint32_t)t << 16);
                base += __popcll(m);
            }
        }
        if (union_mode) {
            const bool any = tokmask != 0;
            const uint64_t m = __ballot(any);
            const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
            if (any) {
                list[pos] = (uint32_t)lane;
                masks[pos] = tokmask;
            }
            base = __popcll(m);
        }
        if (lane == 0) *n_list = base;
    }
    __syncthreads();
    const int n = *n_list;
    XTile<WT, NC> xt;
    int xtok = -1;
    for (int e = wave; e < n; e += K1_WAVES) {
        const uint32_t ent = list[e];
        const int rloc = (int)(ent & 0xffffu);
        const int row = row0 + rloc;
        uint64_t m = union_mode ? masks[e] : ((uint64_t)1 << (ent >> 16));
        RowTile<WT, NC> w3;
        w3.load(W3 + (size_t)row * D, D, lane, true, true);
        while (m) {
            const int t = __builtin_ctzll(m);
            m &= m - 1;
            if (t != xtok) {
                xt.load(x + (size_t)t * D, D, lane);
                xtok = t;
            }
            const float u = wave_sum(xt.dot(w3));
            const float h = activation(act, z_lds[t * K1_MAX_ROWS + rloc]);
            if (lane == 0) a_out[(size_t)t * H + row] = h * (double_act ? activation(act, u) : u);
        }
    }
}

// Standard gate: z = W1 x for this block's units, then compact_and_up.
template <typename WT, int NC>
__global__ __launch_bounds__(K1_THREADS) void k_gate_up_sparse(
    const WT* __restrict__ x, const WT* __restrict__ W1, const WT* __restrict__ W3,
    float* __restrict__ a_out, uint8_t* __restrict__ live_out, int D, int H, int T, int act,
    int union_mode, int rows_per_wave) {
    __shared__ float z_lds[MAXT * K1_MAX_ROWS];
    __shared__ uint32_t list[MAXT * K1_MAX_ROWS];
    __shared__ uint64_t masks[K1_MAX_ROWS];
    __shared__ int n_list;
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int rows_per_block = rows_per_wave * K1_WAVES;
    const int row0 = blockIdx.x * rows_per_block;
    const int nrows = min(rows_per_block, H - row0);

    XTile<WT, NC> xt;
    int xtok = -1;
    for (int q = 0; q < rows_per_wave; q += 2) {
        // two gate rows in flight per wave
        const int ra = wave * rows_per_wave + q, rb = ra + 1;
        const bool va = q < rows_per_wave && ra < nrows;
        const bool vb = q + 1 < rows_per_wave && rb < nrows;
        RowTile<WT, NC> wa, wb;
        wa.load(W1 + (size_t)(row0 + ra) * D, D, lane, va, true);
        wb.load(W1 + (size_t)(row0 + rb) * D, D, lane, vb, true);
        for (int t = 0; t < T; ++t) {
            if (t != xtok) {
                xt.load(x + (size_t)t * D, D, lane);
                xtok = t;
            }
            const float za = wave_sum(xt.dot(wa));
            const float zb = wave_sum(xt.dot(wb));
            if (lane == 0) {
                if (va) z_lds[t * K1_MAX_ROWS + ra] = za;
                if (vb) z_lds[t * K1_MAX_ROWS + rb] = zb;
            }
        }
    }
    __syncthreads();
    compact_and_up<WT, NC>(z_lds, list, masks, &n_list, x, W3, a_out, live_out, row0, nrows, D,
                           H, T, act, union_mode, 0);
}

// LoPA gate: z = U t with t = V x in fp32 (t_in [T x r]), then compact_and_up.
// NR = register chunks of a U row (r <= NR * 64 * VEC).
template <typename WT, int NC, int NR>
__global__ __launch_bounds__(K1_THREADS) void k_gate_up_lopa(
    const WT* __restrict__ x, const float* __restrict__ t_in, const WT* __restrict__ U,
    const WT* __restrict__ W3, float* __restrict__ a_out, uint8_t* __restrict__ live_out, int D,
    int H, int r, int T, int act, int union_mode, int rows_per_wave, unsigned flags) {
    __shared__ float z_lds[MAXT * K1_MAX_ROWS];
    __shared__ uint32_t list[MAXT * K1_MAX_ROWS];
    __shared__ uint64_t masks[K1_MAX_ROWS];
    __shared__ int n_list;
    __shared__ float inv_rms[MAXT];
    constexpr int VEC = Elem<WT>::VEC;
    constexpr int CW = WAVE * VEC;
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int rows_per_block = rows_per_wave * K1_WAVES;
    const int row0 = blockIdx.x * rows_per_block;
    const int nrows = min(rows_per_block, H - row0);
    // RMSNorm of each token's rank vector: 1 / sqrt(mean t^2 + eps), one wave per token
    for (int t = wave; t < T; t += K1_WAVES) {
        float ss = 0.0f;
        for (int m = lane; m < r; m += WAVE) {
            const float tv = t_in[(size_t)t * r + m];
            ss = fmaf(tv, tv, ss);
        }
        ss = wave_sum(ss);
        if (lane == 0) inv_rms[t] = (flags & LOPA_RMSNORM) ? 1.0f / sqrtf(ss / (float)r + RMS_EPS) : 1.0f;
    }
    __syncthreads();

    for (int q = 0; q < rows_per_wave; q += 2) {
        const int ra = wave * rows_per_wave + q, rb = ra + 1;
        const bool va = q < rows_per_wave && ra < nrows;
        const bool vb = q + 1 < rows_per_wave && rb < nrows;
        RowTile<WT, NR> ua, ub;
        ua.load(U + (size_t)(row0 + ra) * r, r, lane, va, true);
        ub.load(U + (size_t)(row0 + rb) * r, r, lane, vb, true);
        for (int t = 0; t < T; ++t) {
            float sa = 0.0f, sb = 0.0f;
#pragma unroll
            for (int c = 0; c < NR; ++c) {
                const int col = c * CW + lane * VEC;
                if (col < r) {
                    const float* tp = t_in + (size_t)t * r + col;
#pragma unroll
                    for (int k = 0; k < VEC; ++k) {
                        const float tv = tp[k];
                        sa = fmaf(Elem<WT>::get(ua.v[c], k), tv, sa);
                        sb = fmaf(Elem<WT>::get(ub.v[c], k), tv, sb);
                    }
                }
            }
            sa = wave_sum(sa) * inv_rms[t];
            sb = wave_sum(sb) * inv_rms[t];
            if (flags & LOPA_G_TILED) {  // (G x)_i = x_{i mod D}
                if (va) sa += Elem<WT>::get1(x[(size_t)t * D + (row0 + ra) % D]);
                if (vb) sb += Elem<WT>::get1(x[(size_t)t * D + (row0 + rb) % D]);
            }
            if (lane == 0) {
                if (va) z_lds[t * K1_MAX_ROWS + ra] = sa;
                if (vb) z_lds[t * K1_MAX_ROWS + rb] = sb;
            }
        }
    }
    __syncthreads();
    compact_and_up<WT, NC>(z_lds, list, masks, &n_list, x, W3, a_out, live_out, row0, nrows, D,
                           H, T, act, union_mode, (flags & LOPA_DOUBLE_ACT) ? 1 : 0);
}

// LoPA rank projection t = V x: one V row per wave-iteration, fp32 out [T x r].
template <typename WT, int NC>
__global__ __launch_bounds__(K1_THREADS) void k_rank_proj(const WT* __restrict__ x,
                                                          const WT* __restrict__ V,
                                                          float* __restrict__ t_out, int D, int r,
                                                          int T, int rows_per_wave) {
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int m0 = (blockIdx.x * K1_WAVES + wave) * rows_per_wave;
    XTile<WT, NC> xt;
    int xtok = -1;
    for (int q = 0; q < rows_per_wave; ++q) {
        const int m = m0 + q;
        if (m >= r) break;
        RowTile<WT, NC> v;
        v.load(V + (size_t)m * D, D, lane, true, true);
        for (int t = 0; t < T; ++t) {
            if (t != xtok) {
                xt.load(x + (size_t)t * D, D, lane);
                xtok = t;
            }
            const float s = wave_sum(xt.dot(v));
            if (lane == 0) t_out[(size_t)t * r + m] = s;
        }
    }
}

// Dense comparator, first half: a_i = A(W1_i . x) (W3_i . x) for every unit.
template <typename WT, int NC>
__global__ __launch_bounds__(K1_THREADS) void k_gate_up_dense(
    const WT* __restrict__ x, const WT* __restrict__ W1, const WT* __restrict__ W3,
    float* __restrict__ a_out, int D, int H, int T, int act, int rows_per_wave) {
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int r0 = (blockIdx.x * K1_WAVES + wave) * rows_per_wave;
    XTile<WT, NC> xt;
    int xtok = -1;
    for (int q = 0; q < rows_per_wave; ++q) {
        const int row = r0 + q;
        if (row >= H) break;
        RowTile<WT, NC> w1, w3;
        w1.load(W1 + (size_t)row * D, D, lane, true, true);
        w3.load(W3 + (size_t)row * D, D, lane, true, true);
        for (int t = 0; t < T; ++t) {
            if (t != xtok) {
                xt.load(x + (size_t)t * D, D, lane);
                xtok = t;
            }
            const float z = wave_sum(xt.dot(w1));
            const float u = wave_sum(xt.dot(w3));
            if (lane == 0) a_out[(size_t)t * H + row] = activation(act, z) * u;
        }
    }
}

// ---------------------------------------------------------------------------
// Down projection, column-split: block -> slice of LPR*VEC columns of y.
// Blocks are dispatched round-robin over the 8 XCDs; the slice index is
// remapped so that consecutive slices (which share 128-byte lines of W2T) run
// on the same XCD and its L2.
template <typename WT, int LPR, int TC>
__global__ __launch_bounds__(K2_THREADS) void k_down(const float* __restrict__ a,
                                                     const WT* __restrict__ W2T,
                                                     float* __restrict__ y, int D, int H, int T,
                                                     int union_mode, int dense) {
    constexpr int VEC = Elem<WT>::VEC;
    constexpr int CB = LPR * VEC;       // columns per block
    constexpr int RPI = WAVE / LPR;     // rows covered by one wave-wide load
    constexpr int PER_THREAD = K2_CAP / K2_THREADS;
    __shared__ int list[K2_CAP];
    __shared__ float alds[TC][K2_CAP];
    __shared__ int wcount[PER_THREAD][K2_WAVES];
    __shared__ float red[K2_WAVES][TC][CB];

    const int nslices = (D + CB - 1) / CB;
    const int per_xcd = (nslices + 7) / 8;
    const int slice = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (slice >= nslices) return;
    const int col0 = slice * CB;
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int sub = lane % LPR;           // which 16 bytes of the row slice
    const int grp = lane / LPR;           // which row of the wave-wide load
    const int col = col0 + sub * VEC;
    const bool col_ok = col < D;
    const int tstep = union_mode ? TC : 1;

    for (int t0 = 0; t0 < T; t0 += tstep) {
        const int tn = min(tstep, T - t0);
        float acc[TC][VEC];
#pragma unroll
        for (int tc = 0; tc < TC; ++tc)
#pragma unroll
            for (int k = 0; k < VEC; ++k) acc[tc][k] = 0.0f;

        for (int r0 = 0; r0 < H; r0 += K2_CAP) {
            // compaction of the nonzero unit products of rows [r0, r0 + K2_CAP)
            uint64_t mk[PER_THREAD];
            bool pk[PER_THREAD];
#pragma unroll
            for (int p = 0; p < PER_THREAD; ++p) {
                const int row = r0 + p * K2_THREADS + threadIdx.x;
                bool keep = false;
                if (row < H) {
                    if (dense) {
                        keep = true;
                    } else {
                        for (int tc = 0; tc < tn; ++tc)
                            keep |= a[(size_t)(t0 + tc) * H + row] != 0.0f;
                    }
                }
                pk[p] = keep;
                mk[p] = __ballot(keep);
                if (lane == 0) wcount[p][wave] = __popcll(mk[p]);
            }
            __syncthreads();
            int n = 0;
#pragma unroll
            for (int p = 0; p < PER_THREAD; ++p) {
                int off = n;
                for (int w = 0; w < K2_WAVES; ++w) {
                    if (w == wave) off = n;
                    n += wcount[p][w];
                }
                if (pk[p]) {
                    const int pos = off + __builtin_amdgcn_mbcnt_hi(
                                              (uint32_t)(mk[p] >> 32),
                                              __builtin_amdgcn_mbcnt_lo((uint32_t)mk[p], 0));
                    const int row = r0 + p * K2_THREADS + threadIdx.x;
                    list[pos] = row;
                    for (int tc = 0; tc < tn; ++tc) alds[tc][pos] = a[(size_t)(t0 + tc) * H + row];
                }
            }
            __syncthreads();
            // accumulate: each wave-wide load covers RPI live rows
            for (int e0 = wave * RPI; e0 < n; e0 += K2_WAVES * RPI * 4) {
                u32x4 w[4];
                int ee[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    ee[u] = e0 + u * K2_WAVES * RPI + grp;
                    if (ee[u] < n && col_ok)
                        w[u] = load_stream(W2T + (size_t)list[ee[u]] * D + col);
                    else
                        w[u] = u32x4{0u, 0u, 0u, 0u};
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if (ee[u] < n) {
#pragma unroll
                        for (int tc = 0; tc < TC; ++tc) {
                            if (tc < tn) {
                                const float av = alds[tc][ee[u]];
#pragma unroll
                                for (int k = 0; k < VEC; ++k)
                                    acc[tc][k] = fmaf(av, Elem<WT>::get(w[u], k), acc[tc][k]);
                            }
                        }
                    }
                }
            }
            __syncthreads();
        }
        // reduce over the RPI row groups of each wave, then over waves
#pragma unroll
        for (int tc = 0; tc < TC; ++tc)
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                float v = acc[tc][k];
                for (int o = LPR; o < WAVE; o <<= 1) v += __shfl_xor(v, o, WAVE);
                acc[tc][k] = v;
            }
        if (grp == 0) {
#pragma unroll
            for (int tc = 0; tc < TC; ++tc)
#pragma unroll
                for (int k = 0; k < VEC; ++k) red[wave][tc][sub * VEC + k] = acc[tc][k];
        }
        __syncthreads();
        for (int i = threadIdx.x; i < tn * CB; i += K2_THREADS) {
            const int tc = i / CB, c = i % CB;
            float s = 0.0f;
            for (int w = 0; w < K2_WAVES; ++w) s += red[w][tc][c];
            if (col0 + c < D) y[(size_t)(t0 + tc) * D + col0 + c] = s;
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Batch-1 bf16 fast path.
//
// 64-lane sum with DPP: quad swaps, half-row and row mirrors give every lane
// its 16-lane row sum; row_bcast15/31 fold the four rows into lane 63.
__device__ inline float wave_sum_dpp(float v) {
    int t;
    t = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
    v += __int_as_float(t);
    t = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
    v += __int_as_float(t);
    t = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false);  // row_half_mirror
    v += __int_as_float(t);
    t = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false);  // row_mirror
    v += __int_as_float(t);
    t = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false);  // row_bcast:15
    v += __int_as_float(t);
    t = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false);  // row_bcast:31
    v += __int_as_float(t);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// sum over a 16-byte chunk pair of bf16x2 products, accumulated in fp32.
// The vector elements are copied to scalars before the bit cast: a bit cast of
// an element lvalue of an ext_vector_type reads element 0 with this compiler.
__device__ inline float dot2_chunk(const u32x4& w, const u32x4& x, float s) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t wq = w[q], xq = x[q];
        s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wq),
                                            __builtin_bit_cast(bf16x2, xq), s, false);
    }
    return s;
}

// Gate and gathered up projection for one token, bf16. Each wave owns one
// unit and issues all of its W1 loads before any arithmetic; the grid is sized
// so every block is resident at once, so the whole of W1 is requested in one
// round. A wave reads the W3 row of its unit as soon as the unit's z is known
// to be live (no block-wide compaction or barrier, so a live unit's W3 round
// trip never waits for another wave's W1 row; with one 5 KB row per wave the
// first z values are known early, and the W3 reads of those units overlap the
// rest of the W1 stream). y_zero (nullable): D floats this grid clears for a
// down pass that accumulates.
template <int NC>
__global__ __launch_bounds__(K1_THREADS) void k_gate_up_t1(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W1,
    const uint16_t* __restrict__ W3, float* __restrict__ a_out, uint8_t* __restrict__ live_out,
    float* __restrict__ y_zero, int D, int H, int act) {
    constexpr int CW = WAVE * 8;
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int unit = blockIdx.x * K1_WAVES + wave;
    const bool in = unit < H;

    u32x4 w[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int col = c * CW + lane * 8;
        w[c] = (in && col < D) ? load_stream(W1 + (size_t)unit * D + col) : u32x4{0u, 0u, 0u, 0u};
    }
    u32x4 xv[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int col = c * CW + lane * 8;
        xv[c] = col < D ? load_cached(x + col) : u32x4{0u, 0u, 0u, 0u};
    }
    if (y_zero) {
        for (int j = blockIdx.x * K1_THREADS + threadIdx.x; j < D; j += gridDim.x * K1_THREADS)
            y_zero[j] = 0.0f;
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) s = dot2_chunk(w[c], xv[c], s);
    const float z = wave_sum_dpp(s);
    const bool live = in && z > 0.0f;
    if (lane == 0 && in) {
        if (live_out) live_out[unit] = live ? 1 : 0;
        if (!live) a_out[unit] = 0.0f;
    }
    if (!live) return;  // wave-uniform
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int col = c * CW + lane * 8;
        w[c] = col < D ? load_stream(W3 + (size_t)unit * D + col) : u32x4{0u, 0u, 0u, 0u};
    }
    float su = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) su = dot2_chunk(w[c], xv[c], su);
    const float u = wave_sum_dpp(su);
    if (lane == 0) a_out[unit] = activation(act, z) * u;
}

// LoPA batch-1 bf16: rank projection t = V x (fp32 out), one V row per wave,
// products of bf16 pairs accumulated in fp32. Also clears y for a down pass
// that accumulates.
template <int NC>
__global__ __launch_bounds__(K1_THREADS) void k_rank_proj_t1(const uint16_t* __restrict__ x,
                                                             const uint16_t* __restrict__ V,
                                                             float* __restrict__ t_out,
                                                             float* __restrict__ y_zero, int D,
                                                             int r) {
    constexpr int CW = WAVE * 8;
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int m = blockIdx.x * K1_WAVES + wave;
    u32x4 w[NC], xv[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int col = c * CW + lane * 8;
        w[c] = (m < r && col < D) ? load_stream(V + (size_t)m * D + col) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int col = c * CW + lane * 8;
        xv[c] = col < D ? load_cached(x + col) : u32x4{0u, 0u, 0u, 0u};
    }
    if (y_zero) {
        for (int j = blockIdx.x * K1_THREADS + threadIdx.x; j < D; j += gridDim.x * K1_THREADS)
            y_zero[j] = 0.0f;
    }
    float sacc = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) sacc = dot2_chunk(w[c], xv[c], sacc);
    sacc = wave_sum_dpp(sacc);
    if (lane == 0 && m < r) t_out[m] = sacc;
}

// LoPA batch-1 bf16 gate: z_i = U_i . t with t in fp32 (U rows widened exactly
// from bf16), then, as in k_gate_up_t1, each wave reads the W3 rows of its own
// live units. x is read only by waves with a live unit, together with their W3
// rows (the gate itself needs only t), which keeps the L2 free for the U stream.
// NR = 16-byte register chunks of a U row (r <= NR * 512); RW units per wave.
template <int NC, int NR, int RW>
__global__ __launch_bounds__(K1_THREADS) void k_gate_up_lopa_t1(
    const uint16_t* __restrict__ x, const float* __restrict__ t_in,
    const uint16_t* __restrict__ U, const uint16_t* __restrict__ W3, float* __restrict__ a_out,
    uint8_t* __restrict__ live_out, int D, int H, int r, int act, unsigned flags) {
    constexpr int CW = WAVE * 8;
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int unit0 = (blockIdx.x * K1_WAVES + wave) * RW;

    u32x4 u[RW][NR];
#pragma unroll
    for (int q = 0; q < RW; ++q) {
#pragma unroll
        for (int c = 0; c < NR; ++c) {
            const int col = c * CW + lane * 8;
            u[q][c] = (unit0 + q < H && col < r) ? load_stream(U + (size_t)(unit0 + q) * r + col)
                                                 : u32x4{0u, 0u, 0u, 0u};
        }
    }
    float tv[NR][8];
#pragma unroll
    for (int c = 0; c < NR; ++c) {
        const int col = c * CW + lane * 8;
        if (col < r) {
            const float4 a = *reinterpret_cast<const float4*>(t_in + col);
            const float4 b = *reinterpret_cast<const float4*>(t_in + col + 4);
            tv[c][0] = a.x; tv[c][1] = a.y; tv[c][2] = a.z; tv[c][3] = a.w;
            tv[c][4] = b.x; tv[c][5] = b.y; tv[c][6] = b.z; tv[c][7] = b.w;
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) tv[c][k] = 0.0f;
        }
    }
    float inv = 1.0f;  // RMSNorm of t: every wave sees all of t
    if (flags & LOPA_RMSNORM) {
        float ss = 0.0f;
#pragma unroll
        for (int c = 0; c < NR; ++c)
#pragma unroll
            for (int k = 0; k < 8; ++k) ss = fmaf(tv[c][k], tv[c][k], ss);
        inv = 1.0f / sqrtf(wave_sum_dpp(ss) / (float)r + RMS_EPS);
    }
    float z[RW];
    bool live[RW];
    bool any = false;
#pragma unroll
    for (int q = 0; q < RW; ++q) {
        const int unit = unit0 + q;
        const bool in = unit < H;
        float s = 0.0f;
#pragma unroll
        for (int c = 0; c < NR; ++c)
#pragma unroll
            for (int k = 0; k < 8; ++k) s = fmaf(Elem<uint16_t>::get(u[q][c], k), tv[c][k], s);
        // (G x)_i = x_{i mod D} when G is on
        const float gx = ((flags & LOPA_G_TILED) && in) ? Elem<uint16_t>::get1(x[unit % D]) : 0.0f;
        z[q] = wave_sum_dpp(s) * inv + gx;
        live[q] = in && z[q] > 0.0f;
        any = any || live[q];
        if (lane == 0 && in) {
            if (live_out) live_out[unit] = live[q] ? 1 : 0;
            if (!live[q]) a_out[unit] = 0.0f;
        }
    }
    if (!any) return;  // wave-uniform
    // the wave's live units: x and all W3 loads first (wave-uniform branches)
    u32x4 xv[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int col = c * CW + lane * 8;
        xv[c] = col < D ? load_cached(x + col) : u32x4{0u, 0u, 0u, 0u};
    }
    u32x4 w3[RW][NC];
#pragma unroll
    for (int q = 0; q < RW; ++q) {
        if (!live[q]) continue;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int col = c * CW + lane * 8;
            w3[q][c] = col < D ? load_stream(W3 + (size_t)(unit0 + q) * D + col) : u32x4{0u, 0u, 0u, 0u};
        }
    }
#pragma unroll
    for (int q = 0; q < RW; ++q) {
        if (!live[q]) continue;
        float s = 0.0f;
#pragma unroll
        for (int c = 0; c < NC; ++c) s = dot2_chunk(w3[q][c], xv[c], s);
        const float uu = wave_sum_dpp(s);
        const float g3 = (flags & LOPA_DOUBLE_ACT) ? activation(act, uu) : uu;
        if (lane == 0) a_out[unit0 + q] = activation(act, z[q]) * g3;
    }
}

// Wave-local compaction of the units a down pass visits: `m` marks the ones
// still to visit among 64 consecutive units (bit b = unit b). One round takes
// the next RPI * UF of them in ascending order, the g-th of every RPI going to
// lane group g; bit[u] = -1 once they run out. Every step is wave-uniform
// (scalar bit scans), so no LDS list, prefix sum or barrier is needed.
template <int RPI, int UF>
__device__ inline void next_live_bits(uint64_t& m, int grp, int (&bit)[UF]) {
#pragma unroll
    for (int u = 0; u < UF; ++u) {
        int b = -1;
#pragma unroll
        for (int g = 0; g < RPI; ++g) {
            const int bg = m ? (int)__builtin_ctzll(m) : -1;
            m &= m - 1;  // stays 0 once empty
            if (g == grp) b = bg;
        }
        bit[u] = b;
    }
}

// Wave-local compaction for the batch-1 down passes. A wave holds the products
// of 64 consecutive units, one per lane; `m` marks the ones still to visit
// (bit b = the unit of lane b). One round takes the next RPI * UF of them in
// ascending order, the g-th of every RPI going to lane group g, so all row
// loads of a round are issued together. A unit's product is read from its own
// lane with a wave-uniform lane index: no LDS list, prefix sum or barrier sits
// between the products and the row loads. bit[u] = -1 once the units run out.
template <int RPI, int UF>
__device__ inline void next_live_round(uint64_t& m, float ar, int grp, int (&bit)[UF],
                                       float (&av)[UF]) {
#pragma unroll
    for (int u = 0; u < UF; ++u) {
        int b = -1;
        float v = 0.0f;
#pragma unroll
        for (int g = 0; g < RPI; ++g) {
            const int bg = m ? (int)__builtin_ctzll(m) : -1;
            m &= m - 1;  // stays 0 once empty
            const float vg = bg >= 0 ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ar), bg))
                                     : 0.0f;
            if (g == grp) {
                b = bg;
                v = vg;
            }
        }
        bit[u] = b;
        av[u] = v;
    }
}

// next_live_round over the PMAX groups of 64 units a wave holds (products ar[p],
// marks m[p]), taken in ascending order across the groups, so a round's row loads
// span group boundaries and a wave with several groups pays one round trip per
// RPI * UF units rather than one per group (used by the int8 and int4 downs, whose
// rounds take 32 units; the bf16 plan splits the units so that a wave holds one
// group). off[u] = 64 p + bit (the unit's offset within the wave's units), -1 once
// they run out.
template <int PMAX, int RPI, int UF>
__device__ inline void next_live_round_multi(uint64_t (&m)[PMAX], const float (&ar)[PMAX],
                                             int grp, int (&off)[UF], float (&av)[UF]) {
#pragma unroll
    for (int u = 0; u < UF; ++u) {
        int o = -1;
        float v = 0.0f;
#pragma unroll
        for (int g = 0; g < RPI; ++g) {
            int og = -1;
            float vg = 0.0f;
#pragma unroll
            for (int q = 0; q < PMAX; ++q) {
                if (og < 0 && m[q]) {
                    const int b = (int)__builtin_ctzll(m[q]);
                    m[q] &= m[q] - 1;
                    og = q * WAVE + b;
                    vg = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ar[q]), b));
                }
            }
            if (g == grp) {
                o = og;
                v = vg;
            }
        }
        off[u] = o;
        av[u] = v;
    }
}

template <int PMAX>
__device__ inline bool any_bits(const uint64_t (&m)[PMAX]) {
    uint64_t a = 0;
#pragma unroll
    for (int q = 0; q < PMAX; ++q) a |= m[q];
    return a != 0;
}

// Column slice of y for the XCD-contiguous order of the down grids: the blocks
// dispatched to one XCD (block index mod 8) take consecutive slices.
__device__ inline int xcd_slice(int bx, int nslices) {
    const int per_xcd = (nslices + 7) / 8;
    return (bx & 7) * per_xcd + (bx >> 3);
}

// Down projection for one token: y[slice] = sum_i a_i W2T[i, slice].
// Grid = (column slices of 256 columns: 32 lanes x 8 bf16, XCD-contiguous) x
// (row splits S). Wave w of a block owns the 64 * PMAX consecutive units
// h0 + 64 * (w * PMAX + p) + lane of its split; all of its products are loaded
// in one round, then its nonzero ones (every unit when dense) are visited by
// next_live_round, two W2T row slices per wave instruction and 8 per lane in
// flight. The 8 waves' slices are summed in LDS; with S > 1 the block adds its
// slice to y (cleared by the gate pass), with S == 1 it stores.
constexpr int KD_THREADS = 512;
constexpr int KD_WAVES = KD_THREADS / WAVE;
template <int PMAX>
__global__ __launch_bounds__(KD_THREADS) void k_down_t1(const float* __restrict__ a,
                                                        const uint16_t* __restrict__ W2T,
                                                        float* __restrict__ y, int D, int H,
                                                        int splits, int dense) {
    constexpr int LPR = 32;
    constexpr int VEC = 8;
    constexpr int CB = LPR * VEC;
    constexpr int RPI = WAVE / LPR;
    constexpr int UF = 8;
    __shared__ float red[KD_WAVES][CB];

    const int slice = xcd_slice(blockIdx.x, (D + CB - 1) / CB);
    if (slice * CB >= D) return;
    const int col0 = slice * CB;
    const int hs = (H + splits - 1) / splits;
    const int h0 = blockIdx.y * hs;
    const int h1 = min(H, h0 + hs);
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int sub = lane % LPR, grp = lane / LPR;
    const int col = col0 + sub * VEC;
    const bool col_ok = col < D;

    float ar[PMAX];
#pragma unroll
    for (int p = 0; p < PMAX; ++p) {
        const int row = h0 + (wave * PMAX + p) * WAVE + lane;
        ar[p] = row < h1 ? a[row] : 0.0f;
    }
    float acc[VEC];
#pragma unroll
    for (int k = 0; k < VEC; ++k) acc[k] = 0.0f;
#pragma unroll
    for (int p = 0; p < PMAX; ++p) {
        const int base = h0 + (wave * PMAX + p) * WAVE;
        uint64_t m = __ballot(base + lane < h1 && (dense || ar[p] != 0.0f));
        while (m) {
            int bit[UF];
            float av[UF];
            next_live_round<RPI, UF>(m, ar[p], grp, bit, av);
            u32x4 wv[UF];
#pragma unroll
            for (int u = 0; u < UF; ++u)
                wv[u] = (bit[u] >= 0 && col_ok) ? load_stream(W2T + (size_t)(base + bit[u]) * D + col)
                                                : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int u = 0; u < UF; ++u)
#pragma unroll
                for (int k = 0; k < VEC; ++k) acc[k] = fmaf(av[u], Elem<uint16_t>::get(wv[u], k), acc[k]);
        }
    }
#pragma unroll
    for (int k = 0; k < VEC; ++k) {
        float v = acc[k];
        for (int o = LPR; o < WAVE; o <<= 1) v += __shfl_xor(v, o, WAVE);
        acc[k] = v;
    }
    if (grp == 0) {
#pragma unroll
        for (int k = 0; k < VEC; ++k) red[wave][sub * VEC + k] = acc[k];
    }
    __syncthreads();
    for (int c = threadIdx.x; c < CB; c += KD_THREADS) {
        float s = 0.0f;
#pragma unroll
        for (int w2 = 0; w2 < KD_WAVES; ++w2) s += red[w2][c];
        if (col0 + c < D) {
            if (splits > 1)
                atomicAdd(y + col0 + c, s);
            else
                y[col0 + c] = s;
        }
    }
}

// Down projection of a batch with per-token live lists: y_t[slice] =
// sum_{i in L_t} a[i][t] W2T[i, slice]. Grid = (column slices, row splits,
// tokens): the blocks of token t compact the units of their split that are
// live for t (bit t of umask, wave-local as in k_down_t1) and gather only those
// W2T row slices, with the products a[i][t] from the unit-major batch buffer
// (row stride tp); a row live for several tokens is fetched by each of their
// blocks (from HBM the first time, from the caches after). y (T x D) is
// cleared by the gate pass.
template <int PMAX>
__global__ __launch_bounds__(KD_THREADS) void k_down_pt(const float* __restrict__ a_rm,
                                                        const uint64_t* __restrict__ umask,
                                                        const uint16_t* __restrict__ W2T,
                                                        float* __restrict__ y, int D, int H, int tp,
                                                        int splits) {
    constexpr int LPR = 32;
    constexpr int VEC = 8;
    constexpr int CB = LPR * VEC;
    constexpr int RPI = WAVE / LPR;
    constexpr int UF = 8;
    __shared__ float red[KD_WAVES][CB];

    const int slice = xcd_slice(blockIdx.x, (D + CB - 1) / CB);
    if (slice * CB >= D) return;
    const int t = blockIdx.z;
    const int col0 = slice * CB;
    const int hs = (H + splits - 1) / splits;
    const int h0 = blockIdx.y * hs;
    const int h1 = min(H, h0 + hs);
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int sub = lane % LPR, grp = lane / LPR;
    const int col = col0 + sub * VEC;
    const bool col_ok = col < D;

    uint64_t mk[PMAX];
#pragma unroll
    for (int p = 0; p < PMAX; ++p) {
        const int row = h0 + (wave * PMAX + p) * WAVE + lane;
        mk[p] = __ballot(row < h1 && ((umask[row] >> t) & 1ull));
    }
    float acc[VEC];
#pragma unroll
    for (int k = 0; k < VEC; ++k) acc[k] = 0.0f;
#pragma unroll
    for (int p = 0; p < PMAX; ++p) {
        const int base = h0 + (wave * PMAX + p) * WAVE;
        uint64_t m = mk[p];
        while (m) {
            int bit[UF];
            next_live_bits<RPI, UF>(m, grp, bit);
            u32x4 wv[UF];
            float av[UF];
#pragma unroll
            for (int u = 0; u < UF; ++u) {
                const bool ok = bit[u] >= 0;
                const size_t row = (size_t)(base + (ok ? bit[u] : 0));
                wv[u] = (ok && col_ok) ? load_stream(W2T + row * D + col) : u32x4{0u, 0u, 0u, 0u};
                av[u] = ok ? a_rm[row * tp + t] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < UF; ++u)
#pragma unroll
                for (int k = 0; k < VEC; ++k) acc[k] = fmaf(av[u], Elem<uint16_t>::get(wv[u], k), acc[k]);
        }
    }
#pragma unroll
    for (int k = 0; k < VEC; ++k) {
        float v = acc[k];
        for (int o = LPR; o < WAVE; o <<= 1) v += __shfl_xor(v, o, WAVE);
        acc[k] = v;
    }
    if (grp == 0) {
#pragma unroll
        for (int k = 0; k < VEC; ++k) red[wave][sub * VEC + k] = acc[k];
    }
    __syncthreads();
    float* yt = y + (size_t)t * D;
    for (int c = threadIdx.x; c < CB; c += KD_THREADS) {
        float s = 0.0f;
#pragma unroll
        for (int w2 = 0; w2 < KD_WAVES; ++w2) s += red[w2][c];
        if (col0 + c < D) atomicAdd(yt + col0 + c, s);
    }
}

// ---------------------------------------------------------------------------
// Batch-1 dense comparator in one pass: one block per group of consecutive
// units (about one block per two CUs). Each wave reads the W1, W3 and W2T rows
// of its units together (the merged gate/up pass of the FFN tutorial, section
// 9.2 case 3, with the down rows in the same round), so the dense FFN costs one
// streaming pass over its 3HD weights. Each lane keeps the slice of y that
// matches its slice of x in registers; the waves' slices are summed in LDS and
// the block writes one partial y of D floats; k_reduce_partials adds the
// partials.
constexpr int KF_THREADS = 512;
constexpr int KF_WAVES = KF_THREADS / WAVE;
constexpr int KF_DMAX = 4096;

template <int NC>
__device__ inline void axpy_chunks(float (&acc)[NC][8], float a, const u32x4 (&w)[NC]) {
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[c][k] = fmaf(a, Elem<uint16_t>::get(w[c], k), acc[c][k]);
}

template <int NC>
__device__ inline void load_row(u32x4 (&w)[NC], const uint16_t* row, int D, int lane, bool ok) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int col = c * WAVE * 8 + lane * 8;
        w[c] = (ok && col < D) ? load_stream(row + col) : u32x4{0u, 0u, 0u, 0u};
    }
}

template <int NC>
__device__ inline float dot_row(const u32x4 (&w)[NC], const u32x4 (&xv)[NC]) {
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) s = dot2_chunk(w[c], xv[c], s);
    return s;
}

template <int NC, int RW>
__global__ __launch_bounds__(KF_THREADS) void k_ffn_dense_t1(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W1,
    const uint16_t* __restrict__ W3, const uint16_t* __restrict__ W2T,
    float* __restrict__ part, int D, int H, int rows_per_block, int act) {
    extern __shared__ float ywave[];  // [KF_WAVES][D]: each wave's slice of y
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int row0 = blockIdx.x * rows_per_block;
    const int nrows = min(rows_per_block, H - row0);

    u32x4 xv[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int col = c * WAVE * 8 + lane * 8;
        xv[c] = col < D ? load_cached(x + col) : u32x4{0u, 0u, 0u, 0u};
    }
    float acc[NC][8];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[c][k] = 0.0f;

    // every unit: W1, W3 and W2T rows together, one unit at a time per wave
    for (int r = 0; r < RW; ++r) {
        const int rl = wave * RW + r;
        const bool ok = rl < nrows;
        const size_t off = (size_t)(row0 + rl) * D;
        u32x4 w1[NC], w3[NC], w2[NC];
        load_row<NC>(w1, W1 + off, D, lane, ok);
        load_row<NC>(w3, W3 + off, D, lane, ok);
        load_row<NC>(w2, W2T + off, D, lane, ok);
        const float z = wave_sum_dpp(dot_row<NC>(w1, xv));
        const float u = wave_sum_dpp(dot_row<NC>(w3, xv));
        const float a = ok ? activation(act, z) * u : 0.0f;
        axpy_chunks<NC>(acc, a, w2);
    }
    // each wave stores its y slice to LDS (16-byte stores, conflict-free), then
    // every thread sums 8 columns over the waves and writes the partial
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int col = c * WAVE * 8 + lane * 8;
        if (col < D) {
            float4* dst = reinterpret_cast<float4*>(ywave + (size_t)wave * D + col);
            dst[0] = make_float4(acc[c][0], acc[c][1], acc[c][2], acc[c][3]);
            dst[1] = make_float4(acc[c][4], acc[c][5], acc[c][6], acc[c][7]);
        }
    }
    __syncthreads();
    float* pb = part + (size_t)blockIdx.x * D;
    for (int j = threadIdx.x * 8; j < D; j += KF_THREADS * 8) {
        float4 s0 = make_float4(0.f, 0.f, 0.f, 0.f), s1 = s0;
        for (int w2 = 0; w2 < KF_WAVES; ++w2) {
            const float4* src = reinterpret_cast<const float4*>(ywave + (size_t)w2 * D + j);
            const float4 a0 = src[0], a1 = src[1];
            s0.x += a0.x; s0.y += a0.y; s0.z += a0.z; s0.w += a0.w;
            s1.x += a1.x; s1.y += a1.y; s1.z += a1.z; s1.w += a1.w;
        }
        reinterpret_cast<float4*>(pb + j)[0] = s0;
        reinterpret_cast<float4*>(pb + j)[1] = s1;
    }
}

// y = sum over the nb partials. Block: 64 columns; thread (pg, cq) adds the
// partials pg, pg + 16, ... of columns 4cq .. 4cq+3 (16-byte loads, all issued
// before any use), then the 16 partial groups are summed in LDS.
constexpr int KR_THREADS = 256;
__global__ __launch_bounds__(KR_THREADS) void k_reduce_partials(const float* __restrict__ part,
                                                                float* __restrict__ y, int D,
                                                                int nb) {
    __shared__ float red[16][64];
    const int cq = threadIdx.x & 15, pg = threadIdx.x >> 4;
    const int c = blockIdx.x * 64 + cq * 4;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    if (c < D) {
        constexpr int U = 16;
        for (int b0 = pg; b0 < nb; b0 += 16 * U) {
            float4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int b = b0 + u * 16;
                v[u] = b < nb ? *reinterpret_cast<const float4*>(part + (size_t)b * D + c)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                s.x += v[u].x; s.y += v[u].y; s.z += v[u].z; s.w += v[u].w;
            }
        }
    }
    red[pg][cq * 4 + 0] = s.x;
    red[pg][cq * 4 + 1] = s.y;
    red[pg][cq * 4 + 2] = s.z;
    red[pg][cq * 4 + 3] = s.w;
    __syncthreads();
    if (threadIdx.x < 64) {
        float t = 0.0f;
#pragma unroll
        for (int g = 0; g < 16; ++g) t += red[g][threadIdx.x];
        const int col = blockIdx.x * 64 + threadIdx.x;
        if (col < D) y[col] = t;
    }
}

// ---------------------------------------------------------------------------
// Batch-1 path with weight-only int8 weights: W[i][j] = q[i][j] * scale[i]
// (symmetric, one fp32 scale per stored row; x stays bf16, every product and
// sum is fp32). A lane's 16-byte piece holds 16 columns; a wave covers 1024
// columns per chunk.

// 16 int8 weights against 16 fp32 inputs, accumulated in fp32
__device__ inline float dot16_i8(const u32x4& w, const float* xv, float s) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t wq = w[q];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int v = (int)(wq << (24 - 8 * b)) >> 24;  // sign-extended byte b
            s = fmaf((float)v, xv[4 * q + b], s);
        }
    }
    return s;
}

// 16 bf16 of x (32 bytes at col) as 8 bf16 pairs, and their fp32 sum; zeros past D
struct X16 {
    u32x4 v[2];
    float sum;
};
__device__ inline X16 load_x16(const uint16_t* __restrict__ x, int col, int D) {
    X16 r;
    r.v[0] = col < D ? load_cached(x + col) : u32x4{0u, 0u, 0u, 0u};
    r.v[1] = col < D ? load_cached(x + col + 8) : u32x4{0u, 0u, 0u, 0u};
    r.sum = 0.0f;  // one bf16 dot2 against (1, 1) per pair
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t xq = r.v[h][q];
            r.sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xq),
                                                    __builtin_bit_cast(bf16x2, 0x3F803F80u), r.sum, false);
        }
    return r;
}

// 16 int8 weights against 16 bf16 x values, fp32 sum. A weight q becomes q + 128
// (byte ^ 0x80), converted exactly to fp32 and packed two at a time as bf16 (its
// 8 significant bits hold 0..255), so one bf16 dot2 takes two weights; the
// 128 * sum(x) this adds is taken off at the end.
__device__ inline float dot16_i8x(const u32x4& w, const X16& xv, float s) {
    float sp = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t wq = w[q] ^ 0x80808080u;
        const uint32_t f0 = __float_as_uint((float)(wq & 0xffu));
        const uint32_t f1 = __float_as_uint((float)((wq >> 8) & 0xffu));
        const uint32_t f2 = __float_as_uint((float)((wq >> 16) & 0xffu));
        const uint32_t f3 = __float_as_uint((float)(wq >> 24));
        const uint32_t p01 = __builtin_amdgcn_perm(f1, f0, 0x07060302u);  // bf16 of f0, f1
        const uint32_t p23 = __builtin_amdgcn_perm(f3, f2, 0x07060302u);
        const u32x4 xq = xv.v[q >> 1];
        const uint32_t x01 = xq[2 * (q & 1)], x23 = xq[2 * (q & 1) + 1];
        sp = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p01),
                                             __builtin_bit_cast(bf16x2, x01), sp, false);
        sp = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p23),
                                             __builtin_bit_cast(bf16x2, x23), sp, false);
    }
    return s + fmaf(-128.0f, xv.sum, sp);
}

// Gate and gathered up projection, int8 weights: z_i = s1_i (q1_i . x); for a
// live unit u_i = s3_i (q3_i . x) and the unit product is stored pre-multiplied
// by the W2T row scale, a_i * s2_i, so the down pass reads only q2. DENSE
// visits every unit. One unit per wave; all W1 loads are issued first.
// y_zero (nullable): D floats this grid clears for a down pass that accumulates.
template <int NC, bool DENSE>
__global__ __launch_bounds__(K1_THREADS) void k_gate_up_t1_i8(
    const uint16_t* __restrict__ x, const int8_t* __restrict__ W1, const float* __restrict__ s1,
    const int8_t* __restrict__ W3, const float* __restrict__ s3, const float* __restrict__ s2,
    float* __restrict__ a_out, uint8_t* __restrict__ live_out, float* __restrict__ y_zero, int D,
    int H, int act) {
    constexpr int CW = WAVE * 16;
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int unit = blockIdx.x * K1_WAVES + wave;
    const bool in = unit < H;
    u32x4 w[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int col = c * CW + lane * 16;
        w[c] = (in && col < D) ? load_stream(W1 + (size_t)unit * D + col) : u32x4{0u, 0u, 0u, 0u};
    }
    u32x4 w3[NC];
    if (DENSE) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int col = c * CW + lane * 16;
            w3[c] = (in && col < D) ? load_stream(W3 + (size_t)unit * D + col) : u32x4{0u, 0u, 0u, 0u};
        }
    }
    const float sc1 = in ? s1[unit] : 0.0f;
    const float sc3 = in ? s3[unit] : 0.0f;
    const float sc2 = in ? s2[unit] : 0.0f;
    X16 xv[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) xv[c] = load_x16(x, c * CW + lane * 16, D);
    if (y_zero) {
        for (int j = blockIdx.x * K1_THREADS + threadIdx.x; j < D; j += gridDim.x * K1_THREADS)
            y_zero[j] = 0.0f;
    }
    float sz = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) sz = dot16_i8x(w[c], xv[c], sz);
    const float z = wave_sum_dpp(sz) * sc1;
    const bool live = in && z > 0.0f;
    if (!in) return;
    if (lane == 0 && live_out) live_out[unit] = live ? 1 : 0;
    if (!DENSE && !live) {
        if (lane == 0) a_out[unit] = 0.0f;
        return;
    }
    if (!DENSE) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int col = c * CW + lane * 16;
            w3[c] = col < D ? load_stream(W3 + (size_t)unit * D + col) : u32x4{0u, 0u, 0u, 0u};
        }
    }
    float su = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) su = dot16_i8x(w3[c], xv[c], su);
    const float u = wave_sum_dpp(su) * sc3;
    if (lane == 0) a_out[unit] = activation(act, z) * u * sc2;
}

// LoPA rank projection, int8 V rows: t_m = sV_m (qV_m . x), one row per wave.
// y_zero (nullable): D floats this grid clears for a down pass that accumulates.
template <int NC>
__global__ __launch_bounds__(K1_THREADS) void k_rank_proj_t1_i8(
    const uint16_t* __restrict__ x, const int8_t* __restrict__ V, const float* __restrict__ sV,
    float* __restrict__ t_out, float* __restrict__ y_zero, int D, int r) {
    constexpr int CW = WAVE * 16;
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int m = blockIdx.x * K1_WAVES + wave;
    u32x4 w[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int col = c * CW + lane * 16;
        w[c] = (m < r && col < D) ? load_stream(V + (size_t)m * D + col) : u32x4{0u, 0u, 0u, 0u};
    }
    X16 xv[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) xv[c] = load_x16(x, c * CW + lane * 16, D);
    if (y_zero) {
        for (int j = blockIdx.x * K1_THREADS + threadIdx.x; j < D; j += gridDim.x * K1_THREADS)
            y_zero[j] = 0.0f;
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) s = dot16_i8x(w[c], xv[c], s);
    s = wave_sum_dpp(s);
    if (lane == 0 && m < r) t_out[m] = s * sV[m];
}

// Sum over the 16 lanes of a lane group (lanes 16g .. 16g + 15).
__device__ inline float group16_sum(float v) {
    v += __shfl_xor(v, 8, 16);
    v += __shfl_xor(v, 4, 16);
    v += __shfl_xor(v, 2, 16);
    v += __shfl_xor(v, 1, 16);
    return v;
}

// LoPA gate and gathered up projection, int8 U and W3 rows. Gate: UPW units
// per wave, 64 / UPW lanes per unit (a U row of r int8 is NR pieces of 16
// bytes per lane of the group):
// z_i = sU_i (qU_i . t) (t through RMSNorm when asked) + (G x)_i when asked.
// Up projection: the wave's live units one after another, 64 lanes each:
// u_i = s3_i (q3_i . x), through A as well under double activation. The stored
// product is pre-multiplied by the W2T row scale s2_i.
// Sum over the N lanes of a lane group (lanes N g .. N g + N - 1), N a power of two.
template <int N>
__device__ inline float group_sum(float v) {
#pragma unroll
    for (int o = N / 2; o >= 1; o /= 2) v += __shfl_xor(v, o, N);
    return v;
}

constexpr int KLQ_UPW = 4;  // units per wave in the gate phase
template <int NC, int NR, int UPW>
__global__ __launch_bounds__(K1_THREADS) void k_gate_up_lopa_t1_i8(
    const uint16_t* __restrict__ x, const float* __restrict__ t_in,
    const int8_t* __restrict__ U, const float* __restrict__ sU, const int8_t* __restrict__ W3,
    const float* __restrict__ s3, const float* __restrict__ s2, float* __restrict__ a_out,
    uint8_t* __restrict__ live_out, int D, int H, int r, int act, unsigned flags) {
    constexpr int CW = WAVE * 16;  // columns of one full-wave chunk of an int8 row
    constexpr int LPU = WAVE / UPW;  // lanes per unit in the gate phase
    constexpr int PB = LPU * 16;     // bytes of U row per piece
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int sub = lane % LPU, grp = lane / LPU;
    const int base = (blockIdx.x * K1_WAVES + wave) * UPW;
    const int unit = base + grp;
    const bool in = unit < H;
    u32x4 u[NR];
#pragma unroll
    for (int c = 0; c < NR; ++c) {
        const int col = c * PB + sub * 16;
        u[c] = (in && col < r) ? load_stream(U + (size_t)unit * r + col) : u32x4{0u, 0u, 0u, 0u};
    }
    float tv[NR][16];
#pragma unroll
    for (int c = 0; c < NR; ++c) {
        const int col = c * PB + sub * 16;
        if (col < r) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 a = *reinterpret_cast<const float4*>(t_in + col + 4 * q);
                tv[c][4 * q] = a.x; tv[c][4 * q + 1] = a.y; tv[c][4 * q + 2] = a.z; tv[c][4 * q + 3] = a.w;
            }
        } else {
#pragma unroll
            for (int k = 0; k < 16; ++k) tv[c][k] = 0.0f;
        }
    }
    const float su_ = in ? sU[unit] : 0.0f;
    const float gx = ((flags & LOPA_G_TILED) && in) ? Elem<uint16_t>::get1(x[unit % D]) : 0.0f;
    float inv = 1.0f;  // RMSNorm of t: every lane group sees all of t
    if (flags & LOPA_RMSNORM) {
        float ss = 0.0f;
#pragma unroll
        for (int c = 0; c < NR; ++c)
#pragma unroll
            for (int k = 0; k < 16; ++k) ss = fmaf(tv[c][k], tv[c][k], ss);
        inv = 1.0f / sqrtf(group_sum<LPU>(ss) / (float)r + RMS_EPS);
    }
    float sz = 0.0f;
#pragma unroll
    for (int c = 0; c < NR; ++c) sz = dot16_i8(u[c], tv[c], sz);
    const float z = group_sum<LPU>(sz) * su_ * inv + gx;
    const bool live = in && z > 0.0f;
    if (in && sub == 0) {
        if (live_out) live_out[unit] = live ? 1 : 0;
        if (!live) a_out[unit] = 0.0f;
    }
    uint64_t m = __ballot(live && sub == 0);
    // x only for waves with a live unit (about a fifth of them): its loads go out with
    // the first W3 row's
    X16 xv[NC];
    if (m) {
#pragma unroll
        for (int c = 0; c < NC; ++c) xv[c] = load_x16(x, c * CW + lane * 16, D);
    }
    while (m) {
        const int g = __builtin_ctzll(m) / LPU;
        m &= m - 1;
        const int ul = base + g;
        const float zl = __shfl(z, LPU * g);
        u32x4 w3[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int col = c * CW + lane * 16;
            w3[c] = col < D ? load_stream(W3 + (size_t)ul * D + col) : u32x4{0u, 0u, 0u, 0u};
        }
        float s = 0.0f;
#pragma unroll
        for (int c = 0; c < NC; ++c) s = dot16_i8x(w3[c], xv[c], s);
        const float uu = wave_sum_dpp(s) * s3[ul];
        const float g3 = (flags & LOPA_DOUBLE_ACT) ? activation(act, uu) : uu;
        if (lane == 0) a_out[ul] = activation(act, zl) * g3 * s2[ul];
    }
}

// Sum over the 4 row groups (16 lanes each) of a wave as a reduce-scatter
// (lanes 32 and 16 apart): each lane ends with 4 whole columns of its 16 in
// acc[0..3] (12 shuffles instead of 32), then stores them to its wave's row of
// red at the columns it owns.
__device__ inline void rowgroup4_reduce_scatter(float (&acc)[16], float* red_row, int lane) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        const int o = 32 >> st, half = 8 >> st;
        const bool upper = (lane & o) != 0;
#pragma unroll
        for (int k = 0; k < half; ++k) {
            const float lo = acc[k], hi = acc[k + half];
            const float keep = upper ? hi : lo;
            acc[k] = keep + __shfl_xor(upper ? lo : hi, o, WAVE);
        }
    }
    const int sub = lane % 16;
    const int cpart = 8 * ((lane >> 5) & 1) + 4 * ((lane >> 4) & 1);
#pragma unroll
    for (int k = 0; k < 4; ++k) red_row[sub * 16 + cpart + k] = acc[k];
}

// Down projection, int8 W2T rows: y[slice] = sum_i a'_i q2[i, slice] with
// a'_i = a_i s2_i from the gate pass. As k_down_t1 (wave-local compaction),
// with column slices of 16 lanes x 16 int8 columns = 256 columns, so a wave
// instruction covers 4 rows and a lane keeps 8 rows in flight.
template <int PMAX>
__global__ __launch_bounds__(KD_THREADS) void k_down_t1_i8(const float* __restrict__ a,
                                                           const int8_t* __restrict__ W2T,
                                                           float* __restrict__ y, int D, int H,
                                                           int splits, int dense) {
    constexpr int LPR = 16;
    constexpr int CB = LPR * 16;
    constexpr int RPI = WAVE / LPR;
    constexpr int UF = 8;
    __shared__ float red[KD_WAVES][CB];

    const int slice = xcd_slice(blockIdx.x, (D + CB - 1) / CB);
    if (slice * CB >= D) return;
    const int col0 = slice * CB;
    const int hs = (H + splits - 1) / splits;
    const int h0 = blockIdx.y * hs;
    const int h1 = min(H, h0 + hs);
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int sub = lane % LPR, grp = lane / LPR;
    const int col = col0 + sub * 16;
    const bool col_ok = col < D;

    float ar[PMAX];
#pragma unroll
    for (int p = 0; p < PMAX; ++p) {
        const int row = h0 + (wave * PMAX + p) * WAVE + lane;
        ar[p] = row < h1 ? a[row] : 0.0f;
    }
    float acc[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) acc[k] = 0.0f;
    uint64_t mk[PMAX];
#pragma unroll
    for (int p = 0; p < PMAX; ++p) {
        const int base = h0 + (wave * PMAX + p) * WAVE;
        mk[p] = __ballot(base + lane < h1 && (dense || ar[p] != 0.0f));
    }
    const int wbase = h0 + wave * PMAX * WAVE;
    while (any_bits(mk)) {
        int off[UF];
        float av[UF];
        next_live_round_multi<PMAX, RPI, UF>(mk, ar, grp, off, av);
        u32x4 wv[UF];
#pragma unroll
        for (int u = 0; u < UF; ++u)
            wv[u] = (off[u] >= 0 && col_ok) ? load_stream(W2T + (size_t)(wbase + off[u]) * D + col)
                                            : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int u = 0; u < UF; ++u) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t wq = wv[u][q];
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    acc[4 * q + b] = fmaf(av[u], (float)((int)(wq << (24 - 8 * b)) >> 24), acc[4 * q + b]);
            }
        }
    }
    static_assert(LPR == 16, "two halving exchanges over 4 row groups");
    rowgroup4_reduce_scatter(acc, red[wave], lane);
    __syncthreads();
    for (int c = threadIdx.x; c < CB; c += KD_THREADS) {
        float s = 0.0f;
#pragma unroll
        for (int w2 = 0; w2 < KD_WAVES; ++w2) s += red[w2][c];
        if (col0 + c < D) {
            if (splits > 1)
                atomicAdd(y + col0 + c, s);
            else
                y[col0 + c] = s;
        }
    }
}

// ---------------------------------------------------------------------------
// Weight-only int4, batch 1: codes packed two per byte (column 2j in the low
// nibble, two's complement), one fp32 scale per 128 columns of a row. A lane's
// 16-byte load holds 32 codes of one 128-column group, so its partial dot
// product takes one scale.
constexpr int I4_GROUP = 128;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 32 bf16 of x (64 bytes at col) as 16 bf16 pairs, and their fp32 sum; zeros past D
struct X32 {
    u32x4 v[4];
    float sum;
};
__device__ inline X32 load_x32(const uint16_t* __restrict__ x, int col, int D) {
    X32 r;
    r.sum = 0.0f;  // one bf16 dot2 against (1, 1) per pair
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        r.v[q] = col < D ? load_cached(x + col + 8 * q) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t xq = r.v[q][k];
            r.sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xq),
                                                    __builtin_bit_cast(bf16x2, 0x3F803F80u), r.sum, false);
        }
    }
    return r;
}

// sum over 32 int4 codes (16 bytes) times x. A code n (two's complement
// nibble u) becomes the bf16 128 + (u ^ 8) = n + 136 exactly: the nibble goes
// into the low mantissa bits of 128.0 (0x4300). One byte permute places the
// codes of columns 2b and 2b + 1 side by side, so a bf16 dot2 takes two
// codes against two x values; the 136 * sum(x) this adds is taken off once.
__device__ inline float dot32_i4(const u32x4& w, const X32& xv) {
    float s = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t wq = w[q] ^ 0x88888888u;
        const uint32_t lo = wq & 0x0F0F0F0Fu;         // byte b: column 2b (offset binary)
        const uint32_t hi = (wq >> 4) & 0x0F0F0F0Fu;  // byte b: column 2b + 1
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            // bytes: lo.b, 0, hi.b, 0 (selector 0x0c gives a zero byte)
            const uint32_t sel = (uint32_t)b | (0x0cu << 8) | ((4u + b) << 16) | (0x0cu << 24);
            const uint32_t pair = __builtin_amdgcn_perm(hi, lo, sel) | 0x43004300u;
            const uint32_t xp = xv.v[q][b];  // x of columns 8q + 2b, 8q + 2b + 1
            s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair),
                                                __builtin_bit_cast(bf16x2, xp), s, false);
        }
    }
    return fmaf(-136.0f, xv.sum, s);
}

// Gate and gathered up projection, int4 weights: z_i = sum_g s1_ig (q1_i,g . x_g);
// for a live unit u_i likewise with W3, and a_i = A(z_i) u_i (the W2T scales
// vary along D, so the down pass applies them). DENSE visits every unit. One
// unit per wave; all W1 loads are issued first.
template <int NC, bool DENSE>
__global__ __launch_bounds__(K1_THREADS) void k_gate_up_t1_i4(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ W1, const float* __restrict__ s1,
    const uint8_t* __restrict__ W3, const float* __restrict__ s3, float* __restrict__ a_out,
    uint8_t* __restrict__ live_out, float* __restrict__ y_zero, int D, int H, int act) {
    constexpr int CW = WAVE * 32;  // columns of one chunk
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int unit = blockIdx.x * K1_WAVES + wave;
    const bool in = unit < H;
    const int G = D / I4_GROUP;
    const size_t rb = (size_t)D / 2;  // bytes per row
    u32x4 w[NC], w3[NC];
    float sc1[NC], sc3[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int col = c * CW + lane * 32;
        const bool ok = in && col < D;
        w[c] = ok ? load_stream(W1 + (size_t)unit * rb + col / 2) : u32x4{0u, 0u, 0u, 0u};
        sc1[c] = ok ? s1[(size_t)unit * G + col / I4_GROUP] : 0.0f;
        if (DENSE) {
            w3[c] = ok ? load_stream(W3 + (size_t)unit * rb + col / 2) : u32x4{0u, 0u, 0u, 0u};
            sc3[c] = ok ? s3[(size_t)unit * G + col / I4_GROUP] : 0.0f;
        }
    }
    X32 xv[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) xv[c] = load_x32(x, c * CW + lane * 32, D);
    if (y_zero) {
        for (int j = blockIdx.x * K1_THREADS + threadIdx.x; j < D; j += gridDim.x * K1_THREADS)
            y_zero[j] = 0.0f;
    }
    float sz = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) sz = fmaf(sc1[c], dot32_i4(w[c], xv[c]), sz);
    const float z = wave_sum_dpp(sz);
    const bool live = in && z > 0.0f;
    if (!in) return;
    if (lane == 0 && live_out) live_out[unit] = live ? 1 : 0;
    if (!DENSE && !live) {
        if (lane == 0) a_out[unit] = 0.0f;
        return;
    }
    if (!DENSE) {  // the live unit's W3 row and its group scales
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int col = c * CW + lane * 32;
            w3[c] = col < D ? load_stream(W3 + (size_t)unit * rb + col / 2) : u32x4{0u, 0u, 0u, 0u};
            sc3[c] = col < D ? s3[(size_t)unit * G + col / I4_GROUP] : 0.0f;
        }
    }
    float su = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) su = fmaf(sc3[c], dot32_i4(w3[c], xv[c]), su);
    const float u = wave_sum_dpp(su);
    if (lane == 0) a_out[unit] = activation(act, z) * u;
}

// LoPA gate with int8 U rows and gathered up projection with group-scaled int4
// W3 rows. The gate is that of k_gate_up_lopa_t1_i8 (four units per wave, 16
// lanes per unit: z_i = sU_i (qU_i . t), t through RMSNorm when asked, plus
// (G x)_i when asked); each live unit of the wave then takes the whole wave for
// its W3 row: u_i = sum_g s3_ig (q3_i,g . x_g), through A as well under double
// activation, and a_i = A(z_i) g(u_i) (the down pass applies the W2T group
// scales). NC chunks of 2048 columns, NR pieces of 256 int8 of a U row.
template <int NC, int NR>
__global__ __launch_bounds__(K1_THREADS) void k_gate_up_lopa_t1_i4(
    const uint16_t* __restrict__ x, const float* __restrict__ t_in,
    const int8_t* __restrict__ U, const float* __restrict__ sU, const uint8_t* __restrict__ W3,
    const float* __restrict__ s3, float* __restrict__ a_out, uint8_t* __restrict__ live_out,
    int D, int H, int r, int act, unsigned flags) {
    constexpr int CW = WAVE * 32;  // columns of one full-wave chunk of an int4 row
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int sub = lane & 15, grp = lane >> 4;
    const int base = (blockIdx.x * K1_WAVES + wave) * KLQ_UPW;
    const int unit = base + grp;
    const bool in = unit < H;
    const int G = D / I4_GROUP;
    const size_t rb = (size_t)D / 2;  // bytes per int4 row
    u32x4 u[NR];
#pragma unroll
    for (int c = 0; c < NR; ++c) {
        const int col = c * 256 + sub * 16;
        u[c] = (in && col < r) ? load_stream(U + (size_t)unit * r + col) : u32x4{0u, 0u, 0u, 0u};
    }
    float tv[NR][16];
#pragma unroll
    for (int c = 0; c < NR; ++c) {
        const int col = c * 256 + sub * 16;
        if (col < r) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 a = *reinterpret_cast<const float4*>(t_in + col + 4 * q);
                tv[c][4 * q] = a.x; tv[c][4 * q + 1] = a.y; tv[c][4 * q + 2] = a.z; tv[c][4 * q + 3] = a.w;
            }
        } else {
#pragma unroll
            for (int k = 0; k < 16; ++k) tv[c][k] = 0.0f;
        }
    }
    const float su_ = in ? sU[unit] : 0.0f;
    const float gx = ((flags & LOPA_G_TILED) && in) ? Elem<uint16_t>::get1(x[unit % D]) : 0.0f;
    float inv = 1.0f;  // RMSNorm of t: every lane group sees all of t
    if (flags & LOPA_RMSNORM) {
        float ss = 0.0f;
#pragma unroll
        for (int c = 0; c < NR; ++c)
#pragma unroll
            for (int k = 0; k < 16; ++k) ss = fmaf(tv[c][k], tv[c][k], ss);
        inv = 1.0f / sqrtf(group16_sum(ss) / (float)r + RMS_EPS);
    }
    float sz = 0.0f;
#pragma unroll
    for (int c = 0; c < NR; ++c) sz = dot16_i8(u[c], tv[c], sz);
    const float z = group16_sum(sz) * su_ * inv + gx;
    const bool live = in && z > 0.0f;
    if (in && sub == 0) {
        if (live_out) live_out[unit] = live ? 1 : 0;
        if (!live) a_out[unit] = 0.0f;
    }
    uint64_t m = __ballot(live && sub == 0);
    // x only for waves with a live unit: its loads go out with the first W3 row's
    X32 xv[NC];
    if (m) {
#pragma unroll
        for (int c = 0; c < NC; ++c) xv[c] = load_x32(x, c * CW + lane * 32, D);
    }
    while (m) {
        const int g = __builtin_ctzll(m) >> 4;
        m &= m - 1;
        const int ul = base + g;
        const float zl = __shfl(z, 16 * g);
        u32x4 w3[NC];
        float sc3[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int col = c * CW + lane * 32;
            const bool ok = col < D;
            w3[c] = ok ? load_stream(W3 + (size_t)ul * rb + col / 2) : u32x4{0u, 0u, 0u, 0u};
            sc3[c] = ok ? s3[(size_t)ul * G + col / I4_GROUP] : 0.0f;
        }
        float s = 0.0f;
#pragma unroll
        for (int c = 0; c < NC; ++c) s = fmaf(sc3[c], dot32_i4(w3[c], xv[c]), s);
        const float uu = wave_sum_dpp(s);
        const float g3 = (flags & LOPA_DOUBLE_ACT) ? activation(act, uu) : uu;
        if (lane == 0) a_out[ul] = activation(act, zl) * g3;
    }
}

// Down projection, int4 W2T rows: y[slice] = sum_i a_i s2_ig q2[i, slice] with
// g the 128-column group of each lane's 16 columns. As k_down_t1_i8, with
// column slices of 16 lanes x 16 codes (8-byte loads) = 256 columns.
template <int PMAX>
__global__ __launch_bounds__(KD_THREADS) void k_down_t1_i4(const float* __restrict__ a,
                                                           const uint8_t* __restrict__ W2T,
                                                           const float* __restrict__ s2,
                                                           float* __restrict__ y, int D, int H,
                                                           int splits, int dense) {
    constexpr int LPR = 16;
    constexpr int CB = LPR * 16;
    constexpr int RPI = WAVE / LPR;
    constexpr int UF = 8;
    __shared__ float red[KD_WAVES][CB];

    const int slice = xcd_slice(blockIdx.x, (D + CB - 1) / CB);
    if (slice * CB >= D) return;
    const int col0 = slice * CB;
    const int hs = (H + splits - 1) / splits;
    const int h0 = blockIdx.y * hs;
    const int h1 = min(H, h0 + hs);
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int sub = lane % LPR, grp = lane / LPR;
    const int col = col0 + sub * 16;
    const bool col_ok = col < D;
    const int G = D / I4_GROUP;
    const size_t rb = (size_t)D / 2;

    float ar[PMAX];
#pragma unroll
    for (int p = 0; p < PMAX; ++p) {
        const int row = h0 + (wave * PMAX + p) * WAVE + lane;
        ar[p] = row < h1 ? a[row] : 0.0f;
    }
    float acc[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) acc[k] = 0.0f;
    uint64_t mk[PMAX];
#pragma unroll
    for (int p = 0; p < PMAX; ++p) {
        const int base = h0 + (wave * PMAX + p) * WAVE;
        mk[p] = __ballot(base + lane < h1 && (dense || ar[p] != 0.0f));
    }
    const int wbase = h0 + wave * PMAX * WAVE;
    while (any_bits(mk)) {
        int off[UF];
        float av[UF];
        next_live_round_multi<PMAX, RPI, UF>(mk, ar, grp, off, av);
        u32x2 wv[UF];
        float sg[UF];
#pragma unroll
        for (int u = 0; u < UF; ++u) {
            const bool ok = off[u] >= 0 && col_ok;
            const size_t row = (size_t)(wbase + (ok ? off[u] : 0));
            wv[u] = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(W2T + row * rb + col / 2))
                       : u32x2{0u, 0u};
            sg[u] = ok ? s2[row * G + col / I4_GROUP] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < UF; ++u) {
            const float aval = av[u] * sg[u];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const uint32_t wq = wv[u][q];
#pragma unroll
                for (int b = 0; b < 8; ++b)
                    acc[8 * q + b] = fmaf(aval, (float)((int)(wq << (28 - 4 * b)) >> 28), acc[8 * q + b]);
            }
        }
    }
    static_assert(LPR == 16, "two halving exchanges over 4 row groups");
    rowgroup4_reduce_scatter(acc, red[wave], lane);
    __syncthreads();
    for (int c = threadIdx.x; c < CB; c += KD_THREADS) {
        float s = 0.0f;
#pragma unroll
        for (int w2 = 0; w2 < KD_WAVES; ++w2) s += red[w2][c];
        if (col0 + c < D) {
            if (splits > 1)
                atomicAdd(y + col0 + c, s);
            else
                y[col0 + c] = s;
        }
    }
}

// Down projection of a quantised batch with per-token live lists: y_t[slice] =
// sum_{i in L_t} a'[i][t] q2[i, slice] (int8 rows; a' carries the row scale) or
// sum_{i in L_t} a[i][t] s2_ig q2[i, slice] (int4 rows, group scales). Grid =
// (column slices of 256 columns, unit-range splits, tokens); the blocks of token
// t walk the units of their split whose token mask has bit t (wave-local, as in
// k_down_pt) and gather only those W2T row slices, with the products from the
// unit-major batch buffer (row stride tp). y (T x D) is cleared by the gate pass.
template <int PMAX, int BITS>
__global__ __launch_bounds__(KD_THREADS) void k_down_pt_q(const float* __restrict__ a_rm,
                                                          const uint64_t* __restrict__ umask,
                                                          const uint8_t* __restrict__ W2T,
                                                          const float* __restrict__ s2,
                                                          float* __restrict__ y, int D, int H,
                                                          int tp, int splits) {
    static_assert(BITS == 8 || BITS == 4, "int8 or int4 rows");
    constexpr int LPR = 16;
    constexpr int CB = LPR * 16;
    constexpr int RPI = WAVE / LPR;
    constexpr int UF = 8;
    __shared__ float red[KD_WAVES][CB];

    const int slice = xcd_slice(blockIdx.x, (D + CB - 1) / CB);
    if (slice * CB >= D) return;
    const int t = blockIdx.z;
    const int col0 = slice * CB;
    const int hs = (H + splits - 1) / splits;
    const int h0 = blockIdx.y * hs;
    const int h1 = min(H, h0 + hs);
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int sub = lane % LPR, grp = lane / LPR;
    const int col = col0 + sub * 16;
    const bool col_ok = col < D;
    const int G = D / I4_GROUP;
    const size_t rb = BITS == 8 ? (size_t)D : (size_t)D / 2;

    uint64_t mk[PMAX];
#pragma unroll
    for (int p = 0; p < PMAX; ++p) {
        const int row = h0 + (wave * PMAX + p) * WAVE + lane;
        mk[p] = __ballot(row < h1 && ((umask[row] >> t) & 1ull));
    }
    float acc[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) acc[k] = 0.0f;
#pragma unroll
    for (int p = 0; p < PMAX; ++p) {
        const int base = h0 + (wave * PMAX + p) * WAVE;
        uint64_t m = mk[p];
        while (m) {
            int bit[UF];
            next_live_bits<RPI, UF>(m, grp, bit);
            u32x4 wv[UF];
            float av[UF];
#pragma unroll
            for (int u = 0; u < UF; ++u) {
                const bool ok = bit[u] >= 0;
                const size_t row = (size_t)(base + (ok ? bit[u] : 0));
                if (BITS == 8) {
                    wv[u] = (ok && col_ok) ? load_stream(W2T + row * rb + col) : u32x4{0u, 0u, 0u, 0u};
                    av[u] = ok ? a_rm[row * tp + t] : 0.0f;
                } else {
                    const u32x2 w2 = (ok && col_ok)
                        ? __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(W2T + row * rb + col / 2))
                        : u32x2{0u, 0u};
                    wv[u] = u32x4{w2[0], w2[1], 0u, 0u};
                    av[u] = (ok && col_ok) ? a_rm[row * tp + t] * s2[row * G + col / I4_GROUP] : 0.0f;
                }
            }
#pragma unroll
            for (int u = 0; u < UF; ++u) {
                if (BITS == 8) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t wq = wv[u][q];
#pragma unroll
                        for (int b = 0; b < 4; ++b)
                            acc[4 * q + b] = fmaf(av[u], (float)((int)(wq << (24 - 8 * b)) >> 24), acc[4 * q + b]);
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        const uint32_t wq = wv[u][q];
#pragma unroll
                        for (int b = 0; b < 8; ++b)
                            acc[8 * q + b] = fmaf(av[u], (float)((int)(wq << (28 - 4 * b)) >> 28), acc[8 * q + b]);
                    }
                }
            }
        }
    }
    static_assert(LPR == 16, "two halving exchanges over 4 row groups");
    rowgroup4_reduce_scatter(acc, red[wave], lane);
    __syncthreads();
    float* yt = y + (size_t)t * D;
    for (int c = threadIdx.x; c < CB; c += KD_THREADS) {
        float s = 0.0f;
#pragma unroll
        for (int w2 = 0; w2 < KD_WAVES; ++w2) s += red[w2][c];
        if (col0 + c < D) atomicAdd(yt + col0 + c, s);
    }
}

// ---------------------------------------------------------------------------
// Small batches (2 <= T <= TT <= 4), bf16, on the VALU.
//
// N partial sums per lane reduced over the wave at once: log2(N) halving
// exchanges (each lane keeps one half of its values and adds the partner's
// copy of that half), then a plain reduction of the one value left. Lane l ends
// with the total of value index rev(l mod N), rev = bit reversal over log2(N)
// bits (an involution).
template <int N>
__device__ inline float multi_reduce(float (&v)[N]) {
    const int lane = threadIdx.x & (WAVE - 1);
#pragma unroll
    for (int h = N / 2, m = 1; h >= 1; h /= 2, m *= 2) {
        const bool hi = (lane & m) != 0;
#pragma unroll
        for (int i = 0; i < h; ++i) {
            const float keep = hi ? v[i + h] : v[i];
            const float send = hi ? v[i] : v[i + h];
            v[i] = keep + __shfl_xor(send, m);
        }
    }
    float s = v[0];
#pragma unroll
    for (int m = N; m < WAVE; m *= 2) s += __shfl_xor(s, m);
    return s;
}

template <int N>
__device__ inline int bit_rev(int i) {
    int r = 0;
#pragma unroll
    for (int b = 1; b < N; b *= 2) r = (r << 1) | ((i & b) ? 1 : 0);
    return r;
}

// Gate and gathered up projection of a small batch, as k_gate_up_t1 for TT
// token slots: each wave owns RW consecutive units, keeps x of the T tokens
// for its columns in registers, streams each W1 row once against all of them,
// then reads the W3 row of each of its units that is live for some token
// (DENSE: every unit). Writes a_rm[unit][t] (row stride tp; 0 for dead pairs
// and for T <= t < TT) for units live for some token, umask[unit] (tokens for
// which the unit is live; DENSE: all T), live flags [T x H] when asked, and
// clears y (T x D) when y_zero is set.
template <int NC, int RW, int TT, bool DENSE>
__global__ __launch_bounds__(K1_THREADS) void k_gate_up_tb(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W1,
    const uint16_t* __restrict__ W3, float* __restrict__ a_rm, uint64_t* __restrict__ umask,
    uint8_t* __restrict__ live_out, float* __restrict__ y_zero, int D, int H, int T, int tp,
    int act) {
    constexpr int CW = WAVE * 8;
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int unit0 = (blockIdx.x * K1_WAVES + wave) * RW;
    u32x4 w[RW][NC];
#pragma unroll
    for (int q = 0; q < RW; ++q) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int col = c * CW + lane * 8;
            w[q][c] = (unit0 + q < H && col < D) ? load_stream(W1 + (size_t)(unit0 + q) * D + col)
                                                 : u32x4{0u, 0u, 0u, 0u};
        }
    }
    u32x4 xv[TT][NC];
#pragma unroll
    for (int t = 0; t < TT; ++t) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int col = c * CW + lane * 8;
            xv[t][c] = (t < T && col < D) ? load_cached(x + (size_t)t * D + col) : u32x4{0u, 0u, 0u, 0u};
        }
    }
    if (y_zero) {
        for (int j = blockIdx.x * K1_THREADS + threadIdx.x; j < T * D; j += gridDim.x * K1_THREADS)
            y_zero[j] = 0.0f;
    }
    const int tl = bit_rev<TT>(lane & (TT - 1));  // token whose sums this lane ends with
    float z[RW];
    bool any[RW];
#pragma unroll
    for (int q = 0; q < RW; ++q) {
        float v[TT];
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            float s = 0.0f;
#pragma unroll
            for (int c = 0; c < NC; ++c) s = dot2_chunk(w[q][c], xv[t][c], s);
            v[t] = s;
        }
        z[q] = multi_reduce<TT>(v);
        const int unit = unit0 + q;
        const bool lv = tl < T && z[q] > 0.0f;
        const uint64_t b = __ballot(lv && lane < TT);
        uint64_t m = 0;
#pragma unroll
        for (int t = 0; t < TT; ++t) m |= ((b >> bit_rev<TT>(t)) & 1ull) << t;
        any[q] = unit < H && (DENSE || m != 0);
        if (unit < H) {
            if (lane == 0) umask[unit] = DENSE ? ((T >= 64) ? ~0ull : ((1ull << T) - 1)) : m;
            if (live_out && lane < TT && tl < T) live_out[(size_t)tl * H + unit] = lv ? 1 : 0;
        }
    }
    // the wave's units live for some token: all W3 loads first (wave-uniform branches)
#pragma unroll
    for (int q = 0; q < RW; ++q) {
        if (!any[q]) continue;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int col = c * CW + lane * 8;
            w[q][c] = col < D ? load_stream(W3 + (size_t)(unit0 + q) * D + col) : u32x4{0u, 0u, 0u, 0u};
        }
    }
#pragma unroll
    for (int q = 0; q < RW; ++q) {
        if (!any[q]) continue;
        float v[TT];
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            float s = 0.0f;
#pragma unroll
            for (int c = 0; c < NC; ++c) s = dot2_chunk(w[q][c], xv[t][c], s);
            v[t] = s;
        }
        const float u = multi_reduce<TT>(v);
        if (lane < TT) a_rm[(size_t)(unit0 + q) * tp + tl] = tl < T ? activation(act, z[q]) * u : 0.0f;
    }
}

// ---------------------------------------------------------------------------
// Batched bf16 path on MFMA (v_mfma_f32_16x16x32_bf16). Lane l of a wave holds
// A[l%16][8(l/16) .. +8], B[8(l/16) .. +8][l%16] and C[4(l/16) .. +4][l%16].
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ inline f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ inline uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Unit product v of (unit row, token t) in a_rm, whose rows hold TP tokens in 4 TP
// bytes: fp32 a_rm[row][t] (split == 0), or the bf16 parts hi = rne(v) and
// lo = rne(v - hi) (about 16 significant bits together), the hi parts of the
// row's TP tokens first and then their lo parts (split != 0). The split form is
// what the MFMA down passes stage: splitting once here replaces a split of every
// product in each of the down pass's column tiles.
__device__ inline void store_product(float* __restrict__ a_rm, size_t row, int TP, int t, float v,
                                     int split) {
    if (split) {
        uint16_t* r = reinterpret_cast<uint16_t*>(a_rm + row * TP);
        const uint32_t hi = bf16_rne(v);
        r[t] = (uint16_t)hi;
        r[TP + t] = (uint16_t)bf16_rne(v - __uint_as_float(hi << 16));
    } else {
        a_rm[row * TP + t] = v;
    }
}

// Stage 1: gate and up projection of UB = 16*UT units for T <= 16*NT tokens,
// as [UB x D] x [D x TP] products on MFMA tiles (see mfma_gate_pass for the
// staging of the operands). The (unit tile, token tile) pairs are spread over the 4 waves;
// with fewer than 4 pairs the waves also split the chunks (K groups) and the
// partial tiles are summed in LDS. The gate reads every W1 row of the block;
// the up projection gathers only the W3 rows of units live for some token
// (DENSE: all units). Writes a_rm[unit][16*NT] (unit-major; 0 for dead (unit,
// token) pairs and padded tokens), umask[unit] (tokens for which the unit is
// live; DENSE: all tokens), live flags [T x H] when requested, and clears y
// (T x D) for a down pass that accumulates. `zeros`: at least 16 zero bytes.
constexpr int KM_THREADS = 256;

// Token mask of one unit in the batched gate epilogues, which walk the (unit,
// token) entries e = i TP + t of a block in strides of KM_THREADS: the TP
// entries of unit i are TP consecutive lanes of one wave (TP divides 64), so
// one ballot gives bit t = "live for token t" to every lane of the unit, with
// no LDS atomics (64 lanes or-ing one word serialise). Every lane of the wave
// must call it.
template <int TP>
__device__ inline uint64_t unit_token_mask(bool live) {
    static_assert(TP == 16 || TP == 32 || TP == 64, "token tile rows");
    const uint64_t b = __ballot(live);
    if constexpr (TP == 64) {
        return b;
    } else {
        const int lane = threadIdx.x & (WAVE - 1);
        return (b >> (lane & ~(TP - 1))) & ((1ull << TP) - 1);
    }
}
constexpr int KM_KC = 128;        // columns per chunk (4 MFMA steps of 32): 256 B per row

template <int NT, int UT>
struct GateTiles {
    static_assert(NT == 1 || NT == 2 || NT == 4, "token tiles: 1, 2 or 4");
    static_assert(UT == 1 || UT == 2 || UT == 4, "unit tiles: 1, 2 or 4");
    static constexpr int TP = 16 * NT;
    static constexpr int UB = 16 * UT;
    static constexpr int TILES = UT * NT;
    static constexpr int KG = TILES >= 4 ? 1 : 4 / TILES;  // K groups
    static constexpr int TPW = TILES >= 4 ? TILES / 4 : 1; // tiles per wave
    static constexpr int ROWS = UB + TP;                   // staged rows per chunk
    static constexpr int IPW = ROWS / 16;                  // 1 KB load instructions per wave per chunk
    static constexpr int STAGE = ROWS * 256;               // bytes per LDS stage
    // LDS stages (deeper rings measured slower); 3 from 24 KB on, so that at 33-64 tokens a
    // 32-unit block takes 74 KB and two share a CU
    static constexpr int NS = STAGE <= 16384 ? 4 : 3;
    static_assert((NS - 2) * IPW <= 24, "vmcnt wait table");
};

// s_waitcnt with only the vector-memory count limited (expcnt, lgkmcnt left
// free); n must be a constant after inlining, 0..31. The target builtins stay
// in plain (non-template) functions.
#define SFFN_VMCNT(N) __builtin_amdgcn_s_waitcnt(((N) & 15) | (7 << 4) | (15 << 8) | (((N) >> 4) << 14))
__device__ inline void wait_vmcnt(int n) {
    switch (n) {
        case 0: SFFN_VMCNT(0); break;   case 1: SFFN_VMCNT(1); break;
        case 2: SFFN_VMCNT(2); break;   case 3: SFFN_VMCNT(3); break;
        case 4: SFFN_VMCNT(4); break;   case 5: SFFN_VMCNT(5); break;
        case 6: SFFN_VMCNT(6); break;   case 7: SFFN_VMCNT(7); break;
        case 8: SFFN_VMCNT(8); break;   case 9: SFFN_VMCNT(9); break;
        case 10: SFFN_VMCNT(10); break; case 11: SFFN_VMCNT(11); break;
        case 12: SFFN_VMCNT(12); break; case 13: SFFN_VMCNT(13); break;
        case 14: SFFN_VMCNT(14); break; case 15: SFFN_VMCNT(15); break;
        case 16: SFFN_VMCNT(16); break; case 18: SFFN_VMCNT(18); break;
        case 20: SFFN_VMCNT(20); break; case 24: SFFN_VMCNT(24); break;
        default: SFFN_VMCNT(0); break;
    }
}
#undef SFFN_VMCNT

// One 16-byte piece per lane from global memory straight into LDS at
// lds + 16 * lane (the LDS address must be the same in every lane). Issued
// as inline assembly so that the compiler does not treat every later LDS read
// as waiting on it: the caller orders the pieces with wait_vmcnt. The
// compiler's own vmcnt waits stay correct (they can only wait longer), since
// vector-memory loads return in issue order.
// (m0 holds no compiler value across this code: it is written here and read
// only by the load that follows it in the same statement.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ inline void load_lds16(const void* g, void* lds) {
    typedef __attribute__((address_space(3))) void* lds_ptr;
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr)lds);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m0) : "memory", "m0");
}
#pragma clang diagnostic pop

// acc[i] (tiles of this wave) = rows[] of W x tokens of x, over all of D.
// Chunks of 128 columns of the UB weight rows and the TP token rows are
// loaded straight into an NS-stage LDS ring (global_load_lds, 16 B per lane:
// one wave instruction fills 4 rows of 256 B). In row r, LDS slot j holds the
// row's 16-byte piece j ^ (r % 16), so the fragment reads of 16 rows at one
// column hit 16 different slots (conflict-free without padding). Pieces
// outside the operands are read from `zeros`. Every chunk issues the same
// number of loads (also past the last chunk), so a fixed vmcnt wait marks a
// chunk as landed; one barrier per chunk.
template <int NT, int UT>
__device__ inline void mfma_gate_pass(f32x4* acc, const uint16_t* __restrict__ W,
                                      const int* rows, const uint16_t* __restrict__ x,
                                      const uint16_t* __restrict__ zeros, int D, int T,
                                      uint8_t* ring) {
    using G = GateTiles<NT, UT>;
    constexpr int NS = G::NS, IPW = G::IPW;
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int r16 = lane & 15, pq = lane >> 4;
    const int kgroup = G::TILES >= 4 ? 0 : wave / G::TILES;
    const int nchunks = (D + KM_KC - 1) / KM_KC;
#pragma unroll
    for (int i = 0; i < G::TPW; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    // the source row of each of this lane's pieces is the same for every chunk
    const uint16_t* src[IPW];
    bool rok[IPW];
    int pcol[IPW];
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
        const int r = 4 * (wave * IPW + i) + pq;  // staged row
        const int p = (lane & 15) ^ (r & 15);     // piece of the row this lane fetches
        pcol[i] = 8 * p;
        if (r < G::UB) {
            const int row = rows[r];
            rok[i] = row >= 0;
            src[i] = W + (rok[i] ? (size_t)row * D + 8 * p : 0);
        } else {
            rok[i] = r - G::UB < T;
            src[i] = x + (rok[i] ? (size_t)(r - G::UB) * D + 8 * p : 0);
        }
    }
    auto issue = [&](int stage, int c) {
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const bool ok = rok[i] && c * KM_KC + pcol[i] < D;
            const uint16_t* g = ok ? src[i] + (size_t)c * KM_KC : zeros;
            load_lds16(g, ring + stage * G::STAGE + 1024 * (wave * IPW + i));
        }
    };
    auto compute = [&](int stage) {
        const uint8_t* wt = ring + stage * G::STAGE;
        const uint8_t* xt = wt + G::UB * 256;
#pragma unroll
        for (int ks = 0; ks < KM_KC / 32; ++ks) {
            const int slot = (4 * ks + pq) ^ r16;
#pragma unroll
            for (int i = 0; i < G::TPW; ++i) {
                const int tile = G::TILES >= 4 ? wave * G::TPW + i : wave % G::TILES;
                const int ut = tile / NT, nt = tile % NT;
                const u32x4 af = *reinterpret_cast<const u32x4*>(wt + (ut * 16 + r16) * 256 + 16 * slot);
                const u32x4 bf = *reinterpret_cast<const u32x4*>(xt + (nt * 16 + r16) * 256 + 16 * slot);
                acc[i] = mfma_bf16(af, bf, acc[i]);
            }
        }
    };

#pragma unroll
    for (int d = 0; d < NS - 1; ++d) issue(d, d);
    const int niter = (nchunks + NS - 1) / NS * NS;
    for (int c0 = 0; c0 < niter; c0 += NS) {
#pragma unroll
        for (int d = 0; d < NS; ++d) {
            const int c = c0 + d;
            wait_vmcnt((NS - 2) * IPW);  // this wave's pieces of chunk c have landed
            __syncthreads();                // ... and every wave's; chunk c - 1 is consumed
            issue((d + NS - 1) % NS, c + NS - 1);
            if (c < nchunks && c % G::KG == kgroup) compute(d);
        }
    }
    wait_vmcnt(0);
    __syncthreads();
}

template <int NT, int UT, bool DENSE, bool LOPA>
__global__ __launch_bounds__(KM_THREADS) void k_gate_up_mfma(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W1,
    const uint16_t* __restrict__ W3, const uint16_t* __restrict__ zeros, float* __restrict__ a_rm,
    uint64_t* __restrict__ umask, uint8_t* __restrict__ live_out, float* __restrict__ y_zero, int D,
    int H, int T, int act, const uint16_t* __restrict__ t_hi, const uint16_t* __restrict__ t_lo,
    int r, unsigned flags, int split) {
    using G = GateTiles<NT, UT>;
    constexpr int TP = G::TP, UB = G::UB;
    constexpr int EPT = UB * TP / KM_THREADS;  // (unit, token) entries per thread
    static_assert(EPT * KM_THREADS == UB * TP, "entries per thread");
    static_assert(G::KG * UB * (TP + 1) * 4 <= G::NS * G::STAGE, "partial sums fit the ring");
    __shared__ __attribute__((aligned(16))) uint8_t ring[G::NS * G::STAGE];
    // the partial sums of a pass go through the ring once the pass has drained it; each
    // thread keeps the z of its (unit, token) entries in registers through the W3 pass
    float (*part)[UB][TP + 1] = reinterpret_cast<float (*)[UB][TP + 1]>(ring);
    __shared__ unsigned long long tmask[UB];
    __shared__ int rows_g[UB];
    __shared__ int rows_u[UB];
    __shared__ int upos[UB];
    __shared__ int nu_s;
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int r16 = lane & 15;
    const int u0 = blockIdx.x * UB;
    const int kgroup = G::TILES >= 4 ? 0 : wave / G::TILES;

    if (y_zero) {
        for (int j = blockIdx.x * KM_THREADS + threadIdx.x; j < T * D; j += gridDim.x * KM_THREADS)
            y_zero[j] = 0.0f;
    }
    if (threadIdx.x < UB) {
        tmask[threadIdx.x] = 0ull;
        rows_g[threadIdx.x] = (u0 + (int)threadIdx.x < H) ? u0 + (int)threadIdx.x : -1;
    }
    __syncthreads();

    auto store_tiles = [&](const f32x4 (&acc)[G::TPW]) {
#pragma unroll
        for (int i = 0; i < G::TPW; ++i) {
            const int tile = G::TILES >= 4 ? wave * G::TPW + i : wave % G::TILES;
            const int ut = tile / NT, nt = tile % NT;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                part[kgroup][ut * 16 + 4 * (lane >> 4) + j][nt * 16 + r16] = acc[i][j];
        }
    };

    // ---- gate: z[UB units][TP tokens]; LoPA: z = U t with t = t_hi + t_lo (two
    // bf16 parts of the fp32 rank vectors, K = r), plus (G x)_i when asked
    {
        f32x4 acc[G::TPW];
        if (LOPA) {
            f32x4 acc2[G::TPW];
            mfma_gate_pass<NT, UT>(acc, W1, rows_g, t_hi, zeros, r, T, ring);
            mfma_gate_pass<NT, UT>(acc2, W1, rows_g, t_lo, zeros, r, T, ring);
#pragma unroll
            for (int i = 0; i < G::TPW; ++i) acc[i] += acc2[i];
        } else {
            mfma_gate_pass<NT, UT>(acc, W1, rows_g, x, zeros, D, T, ring);
        }
        store_tiles(acc);
    }
    __syncthreads();
    float zr[EPT];
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
        const int e = threadIdx.x + k * KM_THREADS;
        const int i = e / TP, t = e % TP;
        float z = 0.0f;
#pragma unroll
        for (int g = 0; g < G::KG; ++g) z += part[g][i][t];
        if (LOPA && (flags & LOPA_G_TILED) && t < T && u0 + i < H)
            z += Elem<uint16_t>::get1(x[(size_t)t * D + (u0 + i) % D]);
        zr[k] = z;
        const bool ok = (u0 + i < H) && t < T;
        const bool live = ok && (DENSE || z > 0.0f);
        const uint64_t tm = unit_token_mask<TP>(live);
        if (t == 0) tmask[i] = tm;
        if (ok && live_out) live_out[(size_t)t * H + u0 + i] = (z > 0.0f) ? 1 : 0;
    }
    __syncthreads();
    if (wave == 0) {
        // compaction of the units live for some token (UB <= 64 = one wave)
        const bool any = lane < UB && tmask[lane] != 0ull;
        const uint64_t m = __ballot(any);
        const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
        if (lane < UB) {
            upos[lane] = any ? pos : -1;
            rows_u[lane] = -1;
            if (u0 + lane < H) umask[u0 + lane] = tmask[lane];
        }
        if (lane == 0) nu_s = __popcll(m);
    }
    __syncthreads();
    if (threadIdx.x < UB && upos[threadIdx.x] >= 0) rows_u[upos[threadIdx.x]] = u0 + threadIdx.x;
    const int nu = nu_s;
    __syncthreads();

    // ---- up projection over the gathered live units: u[p][token], p < nu
    if (nu > 0) {
        f32x4 acc[G::TPW];
        mfma_gate_pass<NT, UT>(acc, W3, rows_u, x, zeros, D, T, ring);
        store_tiles(acc);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
        const int e = threadIdx.x + k * KM_THREADS;
        const int i = e / TP, t = e % TP;
        if (u0 + i >= H) continue;
        const int p = upos[i];
        float av = 0.0f;
        if (p >= 0 && t < T && ((tmask[i] >> t) & 1ull)) {
            float u = 0.0f;
#pragma unroll
            for (int g = 0; g < G::KG; ++g) u += part[g][p][t];
            if (LOPA && (flags & LOPA_DOUBLE_ACT)) u = activation(act, u);
            av = activation(act, zr[k]) * u;
        }
        store_product(a_rm, (size_t)(u0 + i), TP, t, av, split);
    }
}

// Gate and up projection in one pass, for batches whose union covers most units
// (above 10 tokens: 1 - s^T > 0.68 at s = 0.9) and for the dense comparator:
// each chunk stages the block's W1 rows, its W3 rows and the token rows of x
// together, so x is staged once for both products. z and u of every (unit,
// token) pair come out of the same pass; the live test, the token masks and the
// products are those of k_gate_up_mfma (W3 rows of dead units are multiplied
// and dropped: up to a third of the W3 work at 11 tokens, 0.1 % at 64, no change
// to the result).
template <int NT, int UT>
struct FusedTiles {
    static_assert(NT == 1 || NT == 2 || NT == 4, "token tiles: 1, 2 or 4");
    static_assert(UT == 1 || UT == 2, "unit tiles: 1 or 2");
    static constexpr int TP = 16 * NT;
    static constexpr int UB = 16 * UT;
    static constexpr int TILES = UT * NT;
    static constexpr int KG = TILES >= 4 ? 1 : 4 / TILES;
    static constexpr int TPW = TILES >= 4 ? TILES / 4 : 1;
    static constexpr int ROWS = 2 * UB + TP;  // W1 rows, W3 rows, token rows
    static constexpr int IPW = ROWS / 16;
    static constexpr int STAGE = ROWS * 256;
    static constexpr int NS = STAGE <= 24576 ? 4 : 3;
    static_assert((NS - 2) * IPW <= 24, "vmcnt wait table");
};

template <int NT, int UT>
__device__ inline void mfma_fused_pass(f32x4* accz, f32x4* accu, const uint16_t* __restrict__ W1,
                                       const uint16_t* __restrict__ W3, const int* rows,
                                       const uint16_t* __restrict__ x,
                                       const uint16_t* __restrict__ zeros, int D, int T,
                                       uint8_t* ring) {
    using G = FusedTiles<NT, UT>;
    constexpr int NS = G::NS, IPW = G::IPW;
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int r16 = lane & 15, pq = lane >> 4;
    const int kgroup = G::TILES >= 4 ? 0 : wave / G::TILES;
    const int nchunks = (D + KM_KC - 1) / KM_KC;
#pragma unroll
    for (int i = 0; i < G::TPW; ++i) {
        accz[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        accu[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const uint16_t* src[IPW];
    bool rok[IPW];
    int pcol[IPW];
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
        const int r = 4 * (wave * IPW + i) + pq;  // staged row
        const int p = (lane & 15) ^ (r & 15);
        pcol[i] = 8 * p;
        if (r < 2 * G::UB) {
            const int row = rows[r % G::UB];
            rok[i] = row >= 0;
            src[i] = (r < G::UB ? W1 : W3) + (rok[i] ? (size_t)row * D + 8 * p : 0);
        } else {
            rok[i] = r - 2 * G::UB < T;
            src[i] = x + (rok[i] ? (size_t)(r - 2 * G::UB) * D + 8 * p : 0);
        }
    }
    auto issue = [&](int stage, int c) {
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const bool ok = rok[i] && c * KM_KC + pcol[i] < D;
            const uint16_t* g = ok ? src[i] + (size_t)c * KM_KC : zeros;
            load_lds16(g, ring + stage * G::STAGE + 1024 * (wave * IPW + i));
        }
    };
    auto compute = [&](int stage) {
        const uint8_t* w1t = ring + stage * G::STAGE;
        const uint8_t* w3t = w1t + G::UB * 256;
        const uint8_t* xt = w3t + G::UB * 256;
#pragma unroll
        for (int ks = 0; ks < KM_KC / 32; ++ks) {
            const int slot = (4 * ks + pq) ^ r16;
#pragma unroll
            for (int i = 0; i < G::TPW; ++i) {
                const int tile = G::TILES >= 4 ? wave * G::TPW + i : wave % G::TILES;
                const int ut = tile / NT, nt = tile % NT;
                const u32x4 a1 = *reinterpret_cast<const u32x4*>(w1t + (ut * 16 + r16) * 256 + 16 * slot);
                const u32x4 a3 = *reinterpret_cast<const u32x4*>(w3t + (ut * 16 + r16) * 256 + 16 * slot);
                const u32x4 bf = *reinterpret_cast<const u32x4*>(xt + (nt * 16 + r16) * 256 + 16 * slot);
                accz[i] = mfma_bf16(a1, bf, accz[i]);
                accu[i] = mfma_bf16(a3, bf, accu[i]);
            }
        }
    };
#pragma unroll
    for (int d = 0; d < NS - 1; ++d) issue(d, d);
    const int niter = (nchunks + NS - 1) / NS * NS;
    for (int c0 = 0; c0 < niter; c0 += NS) {
#pragma unroll
        for (int d = 0; d < NS; ++d) {
            const int c = c0 + d;
            wait_vmcnt((NS - 2) * IPW);
            __syncthreads();
            issue((d + NS - 1) % NS, c + NS - 1);
            if (c < nchunks && c % G::KG == kgroup) compute(d);
        }
    }
    wait_vmcnt(0);
    __syncthreads();
}

template <int NT, int UT, bool DENSE>
__global__ __launch_bounds__(KM_THREADS) void k_gate_up_mfma_fused(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W1,
    const uint16_t* __restrict__ W3, const uint16_t* __restrict__ zeros, float* __restrict__ a_rm,
    uint64_t* __restrict__ umask, uint8_t* __restrict__ live_out, float* __restrict__ y_zero, int D,
    int H, int T, int act, int split) {
    using G = FusedTiles<NT, UT>;
    constexpr int TP = G::TP, UB = G::UB;
    __shared__ __attribute__((aligned(16))) uint8_t ring[G::NS * G::STAGE];
    __shared__ float pz[G::KG][UB][TP + 1];
    __shared__ float pu[G::KG][UB][TP + 1];
    __shared__ unsigned long long tmask[UB];
    __shared__ int rows_g[UB];
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int r16 = lane & 15;
    const int u0 = blockIdx.x * UB;
    const int kgroup = G::TILES >= 4 ? 0 : wave / G::TILES;

    if (y_zero) {
        for (int j = blockIdx.x * KM_THREADS + threadIdx.x; j < T * D; j += gridDim.x * KM_THREADS)
            y_zero[j] = 0.0f;
    }
    if (threadIdx.x < UB) {
        tmask[threadIdx.x] = 0ull;
        rows_g[threadIdx.x] = (u0 + (int)threadIdx.x < H) ? u0 + (int)threadIdx.x : -1;
    }
    __syncthreads();
    {
        f32x4 accz[G::TPW], accu[G::TPW];
        mfma_fused_pass<NT, UT>(accz, accu, W1, W3, rows_g, x, zeros, D, T, ring);
#pragma unroll
        for (int i = 0; i < G::TPW; ++i) {
            const int tile = G::TILES >= 4 ? wave * G::TPW + i : wave % G::TILES;
            const int ut = tile / NT, nt = tile % NT;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                pz[kgroup][ut * 16 + 4 * (lane >> 4) + j][nt * 16 + r16] = accz[i][j];
                pu[kgroup][ut * 16 + 4 * (lane >> 4) + j][nt * 16 + r16] = accu[i][j];
            }
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < UB * TP; e += KM_THREADS) {
        const int i = e / TP, t = e % TP;
        float z = 0.0f, u = 0.0f;
#pragma unroll
        for (int g = 0; g < G::KG; ++g) {
            z += pz[g][i][t];
            u += pu[g][i][t];
        }
        const bool in = u0 + i < H;
        const bool ok = in && t < T;
        const bool live = ok && (DENSE || z > 0.0f);
        const uint64_t tm = unit_token_mask<TP>(live);  // before the wave's lanes part
        if (!in) continue;
        if (t == 0) tmask[i] = tm;
        if (ok && live_out) live_out[(size_t)t * H + u0 + i] = (z > 0.0f) ? 1 : 0;
        store_product(a_rm, (size_t)(u0 + i), TP, t, live ? activation(act, z) * u : 0.0f, split);
    }
    __syncthreads();
    if (threadIdx.x < UB && u0 + (int)threadIdx.x < H) umask[u0 + threadIdx.x] = tmask[threadIdx.x];
}

// The transposing LDS read ds_read_b64_tr_b16: in each group of 16 lanes, lane l
// receives element l%4 of the 4 consecutive bf16 that lane 4j + l/4 points at,
// as its element j (checked on the device), so two reads give a lane the 8
// consecutive K values of one column of a tile staged as K-rows.
typedef short i16x4 __attribute__((ext_vector_type(4)));

// Slot of 16-byte piece p in staged 256-byte K-row r (r < 32): a transposing
// read touches rows 8g + {0..3} (or + {4..7}) at two adjacent pieces, which
// land on 8 different slots; groups g and g + 1 use disjoint slot halves.
__device__ inline int swz256(int r, int p) { return p ^ (2 * (r & 3) + 8 * ((r >> 3) & 1)); }

__device__ inline u32x4 frag_tr(const uint8_t* part, int col0, int lane) {
    typedef __attribute__((address_space(3))) i16x4* lds_v4;
    const int g = lane >> 4, s = lane & 15;
    const int col = col0 + 4 * (s & 3);
    const int p = col >> 3, half = (col >> 2) & 1;
    const int r0 = 8 * g + (s >> 2), r1 = r0 + 4;
    const uint8_t* a0 = part + r0 * 256 + 16 * swz256(r0, p) + 8 * half;
    const uint8_t* a1 = part + r1 * 256 + 16 * swz256(r1, p) + 8 * half;
    const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4)(a0));
    const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4)(a1));
    const uint2 w0 = __builtin_bit_cast(uint2, v0), w1 = __builtin_bit_cast(uint2, v1);
    return u32x4{w0.x, w0.y, w1.x, w1.y};
}

// Slot of 16-byte piece p in a staged 128-byte K-row r (r < 32). A transposing
// read (frag_tr128) touches rows 8g + {0..3} (or + {4..7}) at two adjacent
// pieces; rows of the same parity share a half of the banks, and bits 1 and 3
// of the row put the four rows of each parity that one half-wave reads on four
// different 32-byte slot pairs.
__device__ inline int swz128(int r, int p) { return p ^ (2 * ((r >> 1) & 1) + 4 * ((r >> 3) & 1)); }

// Extra slot permutation of the lo parts of split products staged next to their
// hi parts: with 16 or 32 tokens a unit's hi and lo pieces of one token group are
// written by lanes of one 128-byte write group, and without it they would share banks
// (with 64 tokens the two parts fill separate write groups).
template <int TP>
constexpr int lo_slot_xor() { return TP == 16 ? 2 : (TP == 32 ? 4 : 0); }

// frag_tr over a part of 32 K-rows of 128 bytes (up to 64 bf16 columns); sx permutes
// the slots of the part as staged (0, or lo_slot_xor for the lo parts).
__device__ inline u32x4 frag_tr128(const uint8_t* part, int col0, int lane, int sx = 0) {
    typedef __attribute__((address_space(3))) i16x4* lds_v4;
    const int g = lane >> 4, s = lane & 15;
    const int col = col0 + 4 * (s & 3);
    const int p = col >> 3, half = (col >> 2) & 1;
    const int r0 = 8 * g + (s >> 2), r1 = r0 + 4;
    const uint8_t* a0 = part + r0 * 128 + 16 * (swz128(r0, p) ^ sx) + 8 * half;
    const uint8_t* a1 = part + r1 * 128 + 16 * (swz128(r1, p) ^ sx) + 8 * half;
    const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4)(a0));
    const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4)(a1));
    const uint2 w0 = __builtin_bit_cast(uint2, v0), w1 = __builtin_bit_cast(uint2, v1);
    return u32x4{w0.x, w0.y, w1.x, w1.y};
}

// LoPA rank projection for a batch: t[token][m] = V_m . x_token for 16 rank
// rows per block (the gate pass above with V for W1 and all D columns), stored
// token-major as two bf16 parts, t_hi = bf16(t) and t_lo = bf16(t - t_hi)
// (about 16 significant bits together), rows of r; tokens past T get zeros.
template <int NT>
__global__ __launch_bounds__(KM_THREADS) void k_rank_proj_mfma(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ zeros, uint16_t* __restrict__ t_hi, uint16_t* __restrict__ t_lo,
    int D, int r, int T) {
    using G = GateTiles<NT, 1>;
    constexpr int TP = G::TP;
    {
        // token tile of this block (grid y): its TP tokens of x and rows of t
        const int t0 = (int)blockIdx.y * TP;
        x += (size_t)t0 * D;
        t_hi += (size_t)t0 * r;
        t_lo += (size_t)t0 * r;
        T = min(TP, T - t0);
    }
    __shared__ __attribute__((aligned(16))) uint8_t ring[G::NS * G::STAGE];
    __shared__ float part[G::KG][16][TP + 1];
    __shared__ int rows[16];
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int m0 = blockIdx.x * 16;
    const int kgroup = G::TILES >= 4 ? 0 : wave / G::TILES;
    if (threadIdx.x < 16) rows[threadIdx.x] = m0 + (int)threadIdx.x < r ? m0 + (int)threadIdx.x : -1;
    __syncthreads();
    f32x4 acc[G::TPW];
    mfma_gate_pass<NT, 1>(acc, V, rows, x, zeros, D, T, ring);
#pragma unroll
    for (int i = 0; i < G::TPW; ++i) {
        const int tile = G::TILES >= 4 ? wave * G::TPW + i : wave % G::TILES;
        const int nt = tile % NT;
#pragma unroll
        for (int j = 0; j < 4; ++j) part[kgroup][4 * (lane >> 4) + j][nt * 16 + (lane & 15)] = acc[i][j];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 16 * TP; e += KM_THREADS) {
        const int m = e % 16, t = e / 16;
        if (m0 + m >= r) continue;
        float v = 0.0f;
#pragma unroll
        for (int g = 0; g < G::KG; ++g) v += part[g][m][t];
        if (t >= T) v = 0.0f;
        const uint32_t hi = bf16_rne(v);
        const uint32_t lo = bf16_rne(v - __uint_as_float(hi << 16));
        t_hi[(size_t)t * r + m0 + m] = (uint16_t)hi;
        t_lo[(size_t)t * r + m0 + m] = (uint16_t)lo;
    }
}

// Stage 2: y[T x D] (+)= sum over the units live for some token of
// a_rm[unit][t] W2T[unit][:] (y is cleared by stage 1 when splits > 1). Grid:
// (column tiles of 128, unit-range splits). The block loads the umask words of
// its split in one round and compacts the live units into an ascending list in
// LDS, then runs through them in chunks of 64 with the global loads of the next
// 4..6 chunks in flight in registers. A chunk is staged without reshaping: each
// W2T row slice goes to LDS as it is (256-byte K-rows), the unit products as the
// bf16 hi and lo parts the gate pass stored (store_product, split form) in
// 128-byte K-rows [unit][token]. Both MFMA operands are read with the
// transposing LDS read, which hands a lane the 8 consecutive units of one token
// or one column. Each wave owns 2*NT of the block's NT x 8 output tiles (one
// token tile) and adds them to y with fp32 atomics (one add per split per
// output), or stores them when there is one split.
constexpr int KDM_THREADS = 256;
constexpr int KDM_LCAP = 2048;
constexpr int KDM_KC = 64;         // units per chunk
constexpr int KDM_NB = 128;        // columns per block
template <int NT>
__global__ __launch_bounds__(KDM_THREADS) void k_down_mfma(
    const float* __restrict__ a_rm, const uint64_t* __restrict__ umask,
    const uint16_t* __restrict__ W2T, float* __restrict__ y, int D, int H, int T, int splits) {
    static_assert(NT == 1 || NT == 2 || NT == 4, "token tiles: 1, 2 or 4");
    constexpr int TP = 16 * NT;
    constexpr int APT = KDM_KC * TP / 4 / KDM_THREADS;            // float4 product pieces per thread
    constexpr int WPT = KDM_KC * KDM_NB * 2 / 16 / KDM_THREADS;   // 16-byte W2T pieces per thread
    constexpr int NCW = 2 * NT;                                   // column tiles per wave
    constexpr int DEPTH = NT == 1 ? 6 : (NT == 2 ? 5 : 4);        // chunks in flight
    constexpr int WPART = 32 * 256;                               // 32 W2T K-rows of 128 columns
    constexpr int APART = 32 * 128;                               // 32 product K-rows of <= 64 tokens
    constexpr int STAGE = 2 * WPART + 4 * APART;                  // W (ks 0, 1), hi (ks 0, 1), lo (ks 0, 1)
    constexpr int PM = KDM_LCAP / KDM_THREADS;                    // umask words per thread
    static_assert(WPT == 4 && KDM_KC == 64, "staging plan: 64 units x 128 columns");
    __shared__ int list[KDM_LCAP];
    __shared__ int wcnt[PM][KDM_THREADS / WAVE];
    __shared__ __attribute__((aligned(256))) uint8_t stg[2][STAGE];
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int col0 = blockIdx.x * KDM_NB;
    const int hs = (H + splits - 1) / splits;  // <= KDM_LCAP (host-checked)
    const int h0 = blockIdx.y * hs;
    const int h1 = min(H, h0 + hs);

    // compaction of the units live for some token, ascending: every umask word of
    // the split is requested before the first is used
    bool keep[PM];
#pragma unroll
    for (int p = 0; p < PM; ++p) {
        const int row = h0 + p * KDM_THREADS + threadIdx.x;
        keep[p] = row < h1 && umask[row] != 0ull;
    }
    uint64_t mk[PM];
#pragma unroll
    for (int p = 0; p < PM; ++p) {
        mk[p] = __ballot(keep[p]);
        if (lane == 0) wcnt[p][wave] = __popcll(mk[p]);
    }
    __syncthreads();
    int n = 0;
#pragma unroll
    for (int p = 0; p < PM; ++p) {
        int off = n;
        for (int w = 0; w < KDM_THREADS / WAVE; ++w) {
            const int c = wcnt[p][w];
            if (w < wave) off += c;
            n += c;
        }
        if (keep[p]) {
            const int pos = off + __builtin_amdgcn_mbcnt_hi((uint32_t)(mk[p] >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)mk[p], 0));
            list[pos] = h0 + p * KDM_THREADS + threadIdx.x;
        }
    }
    __syncthreads();
    const int nchunks = (n + KDM_KC - 1) / KDM_KC;

    // this wave's output tiles: token tile tt, column tiles cb .. cb + NCW - 1
    const int tt = wave / (4 / NT);
    const int cb = (wave % (4 / NT)) * NCW;
    f32x4 acc[NCW];
#pragma unroll
    for (int i = 0; i < NCW; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    // W2T piece g = tid + 256 k: unit row g / 16 of the chunk, 8 columns at 8 (g % 16)
    u32x4 wv[DEPTH][WPT];
    u32x4 av[DEPTH][APT];
    bool wok[DEPTH][WPT], aok[DEPTH][APT];
    auto fetch = [&](int slot, int c) {
#pragma unroll
        for (int k = 0; k < WPT; ++k) {
            const int g = threadIdx.x + k * KDM_THREADS;
            const int e = c * KDM_KC + (g >> 4), col = col0 + 8 * (g & 15);
            const bool ok = e < n && col < D;
            wv[slot][k] = load_stream(W2T + (ok ? (size_t)list[e] * D + col : 0));
            wok[slot][k] = ok;
        }
#pragma unroll
        for (int q = 0; q < APT; ++q) {
            const int idx = threadIdx.x + q * KDM_THREADS;
            const int e = c * KDM_KC + idx / (TP / 4);
            const bool ok = e < n;
            av[slot][q] = *reinterpret_cast<const u32x4*>(
                a_rm + (ok ? (size_t)list[e] * TP + 4 * (idx % (TP / 4)) : 0));
            aok[slot][q] = ok;
        }
    };
    auto stage_write = [&](int stage, int d) {
        uint8_t* st = stg[stage];
#pragma unroll
        for (int k = 0; k < WPT; ++k) {
            const int g = threadIdx.x + k * KDM_THREADS;
            const int row = g >> 4, r = row & 31;
            *reinterpret_cast<u32x4*>(st + (row >> 5) * WPART + r * 256 + 16 * swz256(r, g & 15)) =
                wok[d][k] ? wv[d][k] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int q = 0; q < APT; ++q) {
            // piece p of a unit's row: the hi parts of tokens 8p .. 8p + 7 for p < TP / 8,
            // else the lo parts of tokens 8 (p - TP / 8) .. + 7
            const int idx = threadIdx.x + q * KDM_THREADS;
            const int row = idx / (TP / 4), r = row & 31, p = idx % (TP / 4);
            const int part = p >= TP / 8 ? 1 : 0, tg = p - part * (TP / 8);
            const int off = 2 * WPART + (2 * part + (row >> 5)) * APART + r * 128 +
                            16 * (swz128(r, tg) ^ (part ? lo_slot_xor<TP>() : 0));
            *reinterpret_cast<u32x4*>(st + off) = aok[d][q] ? av[d][q] : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto compute = [&](int stage) {
        const uint8_t* st = stg[stage];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const uint8_t* ah = st + 2 * WPART + ks * APART;
            const u32x4 fh = frag_tr128(ah, tt * 16, lane);
            const u32x4 fl = frag_tr128(ah + 2 * APART, tt * 16, lane, lo_slot_xor<TP>());
#pragma unroll
            for (int i = 0; i < NCW; ++i) {
                const u32x4 b = frag_tr(st + ks * WPART, (cb + i) * 16, lane);
                acc[i] = mfma_bf16(fh, b, acc[i]);
                acc[i] = mfma_bf16(fl, b, acc[i]);
            }
        }
    };
    // chunk c + 1 is staged into the other buffer while chunk c is multiplied
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) fetch(d, d);
    stage_write(0, 0);
    __syncthreads();
    fetch(0, DEPTH);
    const int niter = (nchunks + DEPTH - 1) / DEPTH * DEPTH;
    for (int c0 = 0; c0 < niter; c0 += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const int c = c0 + d;
            const int nslot = (d + 1) % DEPTH;  // holds chunk c + 1
            stage_write((c + 1) & 1, nslot);
            if (c < nchunks) compute(c & 1);
            __syncthreads();
            fetch(nslot, c + 1 + DEPTH);
        }
    }
    if (n == 0 && splits > 1) return;  // nothing to add
    // C layout: row (token) 4*(lane/16) + j of the token tile, column lane%16 of the column tile
    const int r16 = lane & 15;
#pragma unroll
    for (int i = 0; i < NCW; ++i) {
        const int col = col0 + (cb + i) * 16 + r16;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = tt * 16 + 4 * (lane >> 4) + j;
            if (t < T && col < D) {
                if (splits > 1)
                    atomicAdd(y + (size_t)t * D + col, acc[i][j]);
                else
                    y[(size_t)t * D + col] = acc[i][j];
            }
        }
    }
}

// ---- weight-only int8 batches on MFMA (5..64 tokens)
// The plan of the bf16 batches with int8 codes: the codes are staged as they are
// (half the bytes of bf16 rows) and decoded exactly into bf16 where an MFMA operand
// is formed (an int8 value has at most 8 significant bits), and each row's scale
// multiplies its fp32 sums. Products and sums as in the bf16 batches.

// 8 int8 codes (two dwords, ascending columns) -> 8 bf16 values, exact: each code
// q goes through the offset byte q + 128 (byte ^ 0x80, read as unsigned), so the
// conversion never sees a sign-extended byte. (A signed bit-field extract feeding
// the int-to-float conversion was lowered to an unsigned byte conversion with a
// sign-extend modifier, which gave 2^32 + q for negative codes.)
__device__ inline u32x4 decode_i8x8(uint32_t w0, uint32_t w1) {
    u32x4 o;
    const uint32_t w[2] = {w0 ^ 0x80808080u, w1 ^ 0x80808080u};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const uint32_t f0 = __float_as_uint((float)((w[h] >> (16 * p)) & 0xffu) - 128.0f);
            const uint32_t f1 = __float_as_uint((float)((w[h] >> (16 * p + 8)) & 0xffu) - 128.0f);
            o[2 * h + p] = __builtin_amdgcn_perm(f1, f0, 0x07060302u);  // bf16 of f0, f1
        }
    }
    return o;
}

// Chunks of 256 columns: a weight row gives 256 bytes of codes (16 pieces of 16 B)
// and a token row of x 512 bytes, staged as two 256-byte rows (chunk columns
// 0..127 and 128..255). In a weight row r, LDS slot j holds piece j ^ (r % 16); in
// the two rows of token t, piece j ^ (t % 16): the 16-row fragment reads of one
// column hit 16 different slots.
constexpr int KQ_KC = 256;
// Wave w multiplies unit tile w % UT against all NT token tiles over the k-steps
// ks = w / UT (mod KG) of every chunk, so each weight operand is decoded once per
// block; the KG partial sums are added in LDS.
template <int NT, int UT>
struct GateTilesI8 {
    static_assert(NT == 1 || NT == 2 || NT == 4, "token tiles: 1, 2 or 4");
    static_assert(UT == 1 || UT == 2 || UT == 4, "unit tiles: 1, 2 or 4");
    static constexpr int TP = 16 * NT;
    static constexpr int UB = 16 * UT;
    static constexpr int KG = 4 / UT;                      // K groups
    static constexpr int TPW = NT;                         // tiles per wave (one unit tile)
    static constexpr int ROWS = UB + 2 * TP;               // staged 256-byte rows per chunk
    static constexpr int IPW = ROWS / 16;                  // 1 KB load instructions per wave per chunk
    static constexpr int STAGE = ROWS * 256;
    // 3 stages from 24 KB on: at 17-32 tokens (24 KB stages) two blocks then share a CU
    // (LDS within 80 KB), so the 306 blocks of a LoPA gate over H' = 9787 run in one
    // round (int8 LoPA union of 17 / 32 tokens 263k / 476k -> 361k / 642k tokens/s)
    static constexpr int NS = STAGE <= 16384 ? 4 : 3;
    static_assert((NS - 2) * IPW <= 24, "vmcnt wait table");
};

// 8 int8 codes (two dwords) -> the 8 bf16 values q + 128 (exact: 0..255 has at most 8
// significant bits): byte ^ 0x80 is q + 128 read as unsigned, one conversion each.
__device__ inline u32x4 decode_i8x8_offset(uint32_t w0, uint32_t w1) {
    u32x4 o;
    const uint32_t w[2] = {w0 ^ 0x80808080u, w1 ^ 0x80808080u};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const uint32_t f0 = __float_as_uint((float)((w[h] >> (16 * p)) & 0xffu));
            const uint32_t f1 = __float_as_uint((float)((w[h] >> (16 * p + 8)) & 0xffu));
            o[2 * h + p] = __builtin_amdgcn_perm(f1, f0, 0x07060302u);
        }
    }
    return o;
}

// acc[i] (tiles of this wave) = int8 rows[] of W x tokens of x, over K columns (K a
// multiple of 16). Each weight operand is decoded as q + 128 and a second MFMA with
// the constant operand -128 takes the offset off in the same accumulator, so the
// sum is that of q x. The k-steps of every chunk are spread over the K groups of
// waves (all four waves decode and multiply every chunk). The LDS ring and its waits
// as in mfma_gate_pass.
template <int NT, int UT>
__device__ inline void mfma_gate_pass_i8(f32x4* acc, const int8_t* __restrict__ W,
                                         const int* rows, const uint16_t* __restrict__ x,
                                         const uint16_t* __restrict__ zeros, int K, int T,
                                         uint8_t* ring) {
    using G = GateTilesI8<NT, UT>;
    constexpr int NS = G::NS, IPW = G::IPW;
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int r16 = lane & 15, pq = lane >> 4;
    const int ut = wave % UT, kgroup = wave / UT;
    const int nchunks = (K + KQ_KC - 1) / KQ_KC;
#pragma unroll
    for (int i = 0; i < G::TPW; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    // per load instruction: source of this lane's piece, its first column in the
    // chunk, and the bytes one chunk advances (a row of 4 staged rows is either a
    // weight row or half a token row in every lane)
    const uint8_t* src[IPW];
    bool rok[IPW];
    int pcol[IPW], cstep[IPW];
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
        const int r = 4 * (wave * IPW + i) + pq;  // staged row
        if (r < G::UB) {
            const int p = r16 ^ (r & 15);
            const int row = rows[r];
            rok[i] = row >= 0;
            pcol[i] = 16 * p;
            cstep[i] = KQ_KC;
            src[i] = reinterpret_cast<const uint8_t*>(W) + (rok[i] ? (size_t)row * K + 16 * p : 0);
        } else {
            const int xr = r - G::UB, tok = xr >> 1, half = xr & 1;
            const int p = r16 ^ (tok & 15);
            rok[i] = tok < T;
            pcol[i] = 128 * half + 8 * p;
            cstep[i] = 2 * KQ_KC;
            src[i] = reinterpret_cast<const uint8_t*>(x + (rok[i] ? (size_t)tok * K + pcol[i] : 0));
        }
    }
    auto issue = [&](int stage, int c) {
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const bool ok = rok[i] && c * KQ_KC + pcol[i] < K;
            const void* g = ok ? (const void*)(src[i] + (size_t)c * cstep[i]) : (const void*)zeros;
            load_lds16(g, ring + stage * G::STAGE + 1024 * (wave * IPW + i));
        }
    };
    const u32x4 neg128 = u32x4{0xC300C300u, 0xC300C300u, 0xC300C300u, 0xC300C300u};  // bf16 -128
    auto compute = [&](int stage) {
        const uint8_t* wt = ring + stage * G::STAGE;
        const uint8_t* xt = wt + G::UB * 256;
#pragma unroll
        for (int kk = 0; kk < KQ_KC / 32 / G::KG; ++kk) {
            const int ks = kk * G::KG + kgroup;
            // A: unit row 16 ut + r16, codes of columns 32 ks + 8 pq .. + 7
            const int pa = 2 * ks + (pq >> 1);
            const uint2 wv = *reinterpret_cast<const uint2*>(wt + (ut * 16 + r16) * 256 +
                                                             16 * (pa ^ r16) + 8 * (pq & 1));
            const u32x4 af = decode_i8x8_offset(wv.x, wv.y);
            // B: token 16 nt + r16, x of the same columns (half ks / 4 of the token row)
            const int pb = 4 * (ks & 3) + pq;
#pragma unroll
            for (int i = 0; i < G::TPW; ++i) {
                const int tok = i * 16 + r16;
                const u32x4 bf = *reinterpret_cast<const u32x4*>(xt + (2 * tok + (ks >> 2)) * 256 +
                                                                 16 * (pb ^ r16));
                acc[i] = mfma_bf16(af, bf, acc[i]);
                acc[i] = mfma_bf16(neg128, bf, acc[i]);
            }
        }
    };

#pragma unroll
    for (int d = 0; d < NS - 1; ++d) issue(d, d);
    const int niter = (nchunks + NS - 1) / NS * NS;
    for (int c0 = 0; c0 < niter; c0 += NS) {
#pragma unroll
        for (int d = 0; d < NS; ++d) {
            const int c = c0 + d;
            wait_vmcnt((NS - 2) * IPW);  // this wave's pieces of chunk c have landed
            __syncthreads();                // ... and every wave's; chunk c - 1 is consumed
            issue((d + NS - 1) % NS, c + NS - 1);
            if (c < nchunks) compute(d);
        }
    }
    wait_vmcnt(0);
    __syncthreads();
}

// Gate and gathered up projection of a batch, int8 weights (the plan of
// k_gate_up_mfma): z = s1_i (q1_i . x) (LoPA: W1 is U with K = r, z = sU_i (qU_i .
// t) over the two bf16 parts of t, plus (G x)_i when asked); for the units live for
// some token u = s3_i (q3_i . x) (through A under double activation), and the
// unit product is stored pre-multiplied by the W2T row scale, a_i s2_i, so the
// down pass reads only the codes of W2T.
template <int NT, int UT, bool DENSE, bool LOPA>
__global__ __launch_bounds__(KM_THREADS) void k_gate_up_mfma_i8(
    const uint16_t* __restrict__ x, const int8_t* __restrict__ W1, const float* __restrict__ s1,
    const int8_t* __restrict__ W3, const float* __restrict__ s3, const float* __restrict__ s2,
    const uint16_t* __restrict__ zeros, float* __restrict__ a_rm, uint64_t* __restrict__ umask,
    uint8_t* __restrict__ live_out, float* __restrict__ y_zero, int D, int H, int T, int act,
    const uint16_t* __restrict__ t_hi, const uint16_t* __restrict__ t_lo, int r, unsigned flags,
    int split) {
    using G = GateTilesI8<NT, UT>;
    constexpr int TP = G::TP, UB = G::UB;
    constexpr int EPT = UB * TP / KM_THREADS;  // (unit, token) entries per thread
    static_assert(EPT * KM_THREADS == UB * TP, "entries per thread");
    static_assert(G::KG * UB * (TP + 1) * 4 <= G::NS * G::STAGE, "partial sums fit the ring");
    __shared__ __attribute__((aligned(16))) uint8_t ring[G::NS * G::STAGE];
    // the partial sums of a pass go through the ring once the pass has drained it
    float (*part)[UB][TP + 1] = reinterpret_cast<float (*)[UB][TP + 1]>(ring);
    __shared__ unsigned long long tmask[UB];
    __shared__ int rows_g[UB];
    __shared__ int rows_u[UB];
    __shared__ int upos[UB];
    __shared__ int nu_s;
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int r16 = lane & 15;
    const int u0 = blockIdx.x * UB;
    const int ut = wave % UT, kgroup = wave / UT;

    if (y_zero) {
        for (int j = blockIdx.x * KM_THREADS + threadIdx.x; j < T * D; j += gridDim.x * KM_THREADS)
            y_zero[j] = 0.0f;
    }
    if (threadIdx.x < UB) {
        tmask[threadIdx.x] = 0ull;
        rows_g[threadIdx.x] = (u0 + (int)threadIdx.x < H) ? u0 + (int)threadIdx.x : -1;
    }
    __syncthreads();

    auto store_tiles = [&](const f32x4 (&acc)[G::TPW]) {
#pragma unroll
        for (int i = 0; i < G::TPW; ++i) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                part[kgroup][ut * 16 + 4 * (lane >> 4) + j][i * 16 + r16] = acc[i][j];
        }
    };

    {
        f32x4 acc[G::TPW];
        if (LOPA) {
            f32x4 acc2[G::TPW];
            mfma_gate_pass_i8<NT, UT>(acc, W1, rows_g, t_hi, zeros, r, T, ring);
            mfma_gate_pass_i8<NT, UT>(acc2, W1, rows_g, t_lo, zeros, r, T, ring);
#pragma unroll
            for (int i = 0; i < G::TPW; ++i) acc[i] += acc2[i];
        } else {
            mfma_gate_pass_i8<NT, UT>(acc, W1, rows_g, x, zeros, D, T, ring);
        }
        store_tiles(acc);
    }
    __syncthreads();
    // z of this thread's entries e = threadIdx.x + k KM_THREADS, kept in registers
    // through the W3 pass (the ring is reused by it)
    float zr[EPT];
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
        const int e = threadIdx.x + k * KM_THREADS;
        const int i = e / TP, t = e % TP;
        const bool ok = (u0 + i < H) && t < T;
        float z = 0.0f;
#pragma unroll
        for (int g = 0; g < G::KG; ++g) z += part[g][i][t];
        if (ok) {
            z *= s1[u0 + i];
            if (LOPA && (flags & LOPA_G_TILED)) z += Elem<uint16_t>::get1(x[(size_t)t * D + (u0 + i) % D]);
        }
        zr[k] = z;
        const bool live = ok && (DENSE || z > 0.0f);
        const uint64_t tm = unit_token_mask<TP>(live);
        if (t == 0) tmask[i] = tm;
        if (ok && live_out) live_out[(size_t)t * H + u0 + i] = (z > 0.0f) ? 1 : 0;
    }
    __syncthreads();
    if (wave == 0) {
        const bool any = lane < UB && tmask[lane] != 0ull;
        const uint64_t m = __ballot(any);
        const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
        if (lane < UB) {
            upos[lane] = any ? pos : -1;
            rows_u[lane] = -1;
            if (u0 + lane < H) umask[u0 + lane] = tmask[lane];
        }
        if (lane == 0) nu_s = __popcll(m);
    }
    __syncthreads();
    if (threadIdx.x < UB && upos[threadIdx.x] >= 0) rows_u[upos[threadIdx.x]] = u0 + threadIdx.x;
    const int nu = nu_s;
    __syncthreads();

    if (nu > 0) {
        f32x4 acc[G::TPW];
        mfma_gate_pass_i8<NT, UT>(acc, W3, rows_u, x, zeros, D, T, ring);
        store_tiles(acc);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
        const int e = threadIdx.x + k * KM_THREADS;
        const int i = e / TP, t = e % TP;
        if (u0 + i >= H) continue;
        const int p = upos[i];
        float av = 0.0f;
        if (p >= 0 && t < T && ((tmask[i] >> t) & 1ull)) {
            float u = 0.0f;
#pragma unroll
            for (int g = 0; g < G::KG; ++g) u += part[g][p][t];
            u *= s3[u0 + i];
            if (LOPA && (flags & LOPA_DOUBLE_ACT)) u = activation(act, u);
            av = activation(act, zr[k]) * u * s2[u0 + i];
        }
        store_product(a_rm, (size_t)(u0 + i), TP, t, av, split);
    }
}

// Gate and up projection of an int8 batch in one pass (standard gating, batches
// above 10 tokens and the dense comparator), as k_gate_up_mfma_fused does for bf16:
// each 256-column chunk stages the block's 32 W1 code rows, its 32 W3 code rows and
// the token rows of x (two 256-byte rows per token) together, so x is staged once
// for both products. Wave w owns unit tile w & 1 of matrix w >> 1 (W1, then W3)
// against every token tile and runs every k-step of the chunk, so no partial sums
// are combined across waves; the codes are decoded exactly as in mfma_gate_pass_i8
// (bf16 q + 128, the offset taken off by a second MFMA against a constant -128).
template <int NT>
struct FusedTilesI8 {
    static_assert(NT == 1 || NT == 2 || NT == 4, "token tiles: 1, 2 or 4");
    static constexpr int TP = 16 * NT;
    static constexpr int UB = 32;                          // units per block
    static constexpr int ROWS = 2 * UB + 2 * TP;           // W1 rows, W3 rows, token half rows
    static constexpr int IPW = ROWS / 16;                  // 1 KB load instructions per wave per chunk
    static constexpr int STAGE = ROWS * 256;
    static constexpr int NS = STAGE <= 32768 ? 4 : 3;
    static_assert((NS - 2) * IPW <= 24, "vmcnt wait table");
    static_assert(NS * STAGE <= 147456, "LDS ring");
    static_assert(2 * UB * (TP + 1) * 4 <= NS * STAGE, "z and u tiles fit the ring");
};

template <int NT>
__device__ inline void mfma_fused_pass_i8(f32x4 (&acc)[NT], const int8_t* __restrict__ W1,
                                          const int8_t* __restrict__ W3, int u0, int H,
                                          const uint16_t* __restrict__ x,
                                          const uint16_t* __restrict__ zeros, int K, int T,
                                          uint8_t* ring) {
    using G = FusedTilesI8<NT>;
    constexpr int NS = G::NS, IPW = G::IPW, UB = G::UB;
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int r16 = lane & 15, pq = lane >> 4;
    const int ut = wave & 1, mat = wave >> 1;
    const int nchunks = (K + KQ_KC - 1) / KQ_KC;
#pragma unroll
    for (int i = 0; i < NT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    const uint8_t* src[IPW];
    bool rok[IPW];
    int pcol[IPW], cstep[IPW];
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
        const int r = 4 * (wave * IPW + i) + pq;  // staged row
        if (r < 2 * UB) {
            const int row = u0 + (r & (UB - 1));
            const int8_t* W = r < UB ? W1 : W3;
            const int p = r16 ^ (r & 15);
            rok[i] = row < H;
            pcol[i] = 16 * p;
            cstep[i] = KQ_KC;
            src[i] = reinterpret_cast<const uint8_t*>(W) + (rok[i] ? (size_t)row * K + 16 * p : 0);
        } else {
            const int xr = r - 2 * UB, tok = xr >> 1, half = xr & 1;
            const int p = r16 ^ (tok & 15);
            rok[i] = tok < T;
            pcol[i] = 128 * half + 8 * p;
            cstep[i] = 2 * KQ_KC;
            src[i] = reinterpret_cast<const uint8_t*>(x + (rok[i] ? (size_t)tok * K + pcol[i] : 0));
        }
    }
    auto issue = [&](int stage, int c) {
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const bool ok = rok[i] && c * KQ_KC + pcol[i] < K;
            const void* g = ok ? (const void*)(src[i] + (size_t)c * cstep[i]) : (const void*)zeros;
            load_lds16(g, ring + stage * G::STAGE + 1024 * (wave * IPW + i));
        }
    };
    const u32x4 neg128 = u32x4{0xC300C300u, 0xC300C300u, 0xC300C300u, 0xC300C300u};  // bf16 -128
    auto compute = [&](int stage) {
        const uint8_t* wt = ring + stage * G::STAGE;
        const uint8_t* xt = wt + 2 * UB * 256;
        const int arow = mat * UB + ut * 16 + r16;  // arow & 15 == r16
#pragma unroll
        for (int ks = 0; ks < KQ_KC / 32; ++ks) {
            // A: codes of columns 32 ks + 8 pq .. + 7 of the wave's unit row
            const int pa = 2 * ks + (pq >> 1);
            const uint2 wv = *reinterpret_cast<const uint2*>(wt + arow * 256 + 16 * (pa ^ r16) +
                                                             8 * (pq & 1));
            const u32x4 af = decode_i8x8_offset(wv.x, wv.y);
            // B: token 16 i + r16, x of the same columns (half ks / 4 of the token row)
            const int pb = 4 * (ks & 3) + pq;
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                const int tok = i * 16 + r16;
                const u32x4 bf = *reinterpret_cast<const u32x4*>(xt + (2 * tok + (ks >> 2)) * 256 +
                                                                 16 * (pb ^ r16));
                acc[i] = mfma_bf16(af, bf, acc[i]);
                acc[i] = mfma_bf16(neg128, bf, acc[i]);
            }
        }
    };

#pragma unroll
    for (int d = 0; d < NS - 1; ++d) issue(d, d);
    const int niter = (nchunks + NS - 1) / NS * NS;
    for (int c0 = 0; c0 < niter; c0 += NS) {
#pragma unroll
        for (int d = 0; d < NS; ++d) {
            const int c = c0 + d;
            wait_vmcnt((NS - 2) * IPW);  // this wave's pieces of chunk c have landed
            __syncthreads();                // ... and every wave's; chunk c - 1 is consumed
            issue((d + NS - 1) % NS, c + NS - 1);
            if (c < nchunks) compute(d);
        }
    }
    wait_vmcnt(0);
    __syncthreads();
}

template <int NT, bool DENSE>
__global__ __launch_bounds__(KM_THREADS) void k_gate_up_mfma_fused_i8(
    const uint16_t* __restrict__ x, const int8_t* __restrict__ W1, const float* __restrict__ s1,
    const int8_t* __restrict__ W3, const float* __restrict__ s3, const float* __restrict__ s2,
    const uint16_t* __restrict__ zeros, float* __restrict__ a_rm, uint64_t* __restrict__ umask,
    uint8_t* __restrict__ live_out, float* __restrict__ y_zero, int D, int H, int T, int act,
    int split) {
    using G = FusedTilesI8<NT>;
    constexpr int TP = G::TP, UB = G::UB;
    __shared__ __attribute__((aligned(16))) uint8_t ring[G::NS * G::STAGE];
    __shared__ unsigned long long tmask[UB];
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int r16 = lane & 15;
    const int u0 = blockIdx.x * UB;
    const int ut = wave & 1, mat = wave >> 1;

    if (y_zero) {
        for (int j = blockIdx.x * KM_THREADS + threadIdx.x; j < T * D; j += gridDim.x * KM_THREADS)
            y_zero[j] = 0.0f;
    }
    if (threadIdx.x < UB) tmask[threadIdx.x] = 0ull;  // first read after the pass's barriers

    f32x4 acc[NT];
    mfma_fused_pass_i8<NT>(acc, W1, W3, u0, H, x, zeros, D, T, ring);
    // the ring is free after the pass (its loads have landed, every wave is past it):
    // z sums of the block's units in zu[0], u sums in zu[1]
    float (*zu)[UB][TP + 1] = reinterpret_cast<float (*)[UB][TP + 1]>(ring);
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) zu[mat][ut * 16 + 4 * (lane >> 4) + j][i * 16 + r16] = acc[i][j];
    __syncthreads();
    for (int e = threadIdx.x; e < UB * TP; e += KM_THREADS) {
        const int i = e / TP, t = e % TP;
        const bool in = u0 + i < H;
        const bool ok = in && t < T;
        const float z = in ? zu[0][i][t] * s1[u0 + i] : 0.0f;
        const bool live = ok && (DENSE || z > 0.0f);
        const uint64_t tm = unit_token_mask<TP>(live);  // before the wave's lanes part
        if (!in) continue;
        if (t == 0) tmask[i] = tm;
        if (ok && live_out) live_out[(size_t)t * H + u0 + i] = (z > 0.0f) ? 1 : 0;
        float av = 0.0f;
        if (live) {
            const float u = zu[1][i][t] * s3[u0 + i];
            av = activation(act, z) * u * s2[u0 + i];
        }
        store_product(a_rm, (size_t)(u0 + i), TP, t, av, split);
    }
    __syncthreads();
    if (threadIdx.x < UB && u0 + (int)threadIdx.x < H) umask[u0 + threadIdx.x] = tmask[threadIdx.x];
}

// LoPA rank projection for a batch, int8 V: t[token][m] = sV_m (qV_m . x_token),
// 16 rank rows per block, stored token-major as bf16 hi and lo parts (as
// k_rank_proj_mfma).
template <int NT>
__global__ __launch_bounds__(KM_THREADS) void k_rank_proj_mfma_i8(
    const uint16_t* __restrict__ x, const int8_t* __restrict__ V, const float* __restrict__ sV,
    const uint16_t* __restrict__ zeros, uint16_t* __restrict__ t_hi, uint16_t* __restrict__ t_lo,
    int D, int r, int T) {
    using G = GateTilesI8<NT, 1>;
    constexpr int TP = G::TP;
    {
        // token tile of this block (grid y): its TP tokens of x and rows of t
        const int t0 = (int)blockIdx.y * TP;
        x += (size_t)t0 * D;
        t_hi += (size_t)t0 * r;
        t_lo += (size_t)t0 * r;
        T = min(TP, T - t0);
    }
    __shared__ __attribute__((aligned(16))) uint8_t ring[G::NS * G::STAGE];
    __shared__ float part[G::KG][16][TP + 1];
    __shared__ int rows[16];
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int m0 = blockIdx.x * 16;
    const int kgroup = wave;  // one unit tile: the four waves split the k-steps
    if (threadIdx.x < 16) rows[threadIdx.x] = m0 + (int)threadIdx.x < r ? m0 + (int)threadIdx.x : -1;
    __syncthreads();
    f32x4 acc[G::TPW];
    mfma_gate_pass_i8<NT, 1>(acc, V, rows, x, zeros, D, T, ring);
#pragma unroll
    for (int i = 0; i < G::TPW; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) part[kgroup][4 * (lane >> 4) + j][i * 16 + (lane & 15)] = acc[i][j];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 16 * TP; e += KM_THREADS) {
        const int m = e % 16, t = e / 16;
        if (m0 + m >= r) continue;
        float v = 0.0f;
#pragma unroll
        for (int g = 0; g < G::KG; ++g) v += part[g][m][t];
        v = t < T ? v * sV[m0 + m] : 0.0f;
        const uint32_t hi = bf16_rne(v);
        const uint32_t lo = bf16_rne(v - __uint_as_float(hi << 16));
        t_hi[(size_t)t * r + m0 + m] = (uint16_t)hi;
        t_lo[(size_t)t * r + m0 + m] = (uint16_t)lo;
    }
}

// Down pass of an int8 batch: k_down_mfma with the codes of W2T (16 columns per
// 16-byte piece, two pieces per thread per chunk of 64 units x 128 columns)
// decoded exactly into the bf16 staging layout; the unit products already carry
// the W2T row scales. D a multiple of 16.
template <int NT>
__global__ __launch_bounds__(KDM_THREADS) void k_down_mfma_i8(
    const float* __restrict__ a_rm, const uint64_t* __restrict__ umask,
    const int8_t* __restrict__ W2T, float* __restrict__ y, int D, int H, int T, int splits) {
    static_assert(NT == 1 || NT == 2 || NT == 4, "token tiles: 1, 2 or 4");
    constexpr int TP = 16 * NT;
    constexpr int APT = KDM_KC * TP / 4 / KDM_THREADS;            // float4 product pieces per thread
    constexpr int WPT = KDM_KC * KDM_NB / 16 / KDM_THREADS;       // 16-byte code pieces per thread
    constexpr int NCW = 2 * NT;
    constexpr int DEPTH = NT == 1 ? 6 : (NT == 2 ? 5 : 4);
    constexpr int WPART = 32 * 256;
    constexpr int APART = 32 * 128;
    constexpr int STAGE = 2 * WPART + 4 * APART;
    constexpr int PM = KDM_LCAP / KDM_THREADS;
    static_assert(WPT == 2 && KDM_KC == 64, "staging plan: 64 units x 128 columns");
    __shared__ int list[KDM_LCAP];
    __shared__ int wcnt[PM][KDM_THREADS / WAVE];
    __shared__ __attribute__((aligned(256))) uint8_t stg[2][STAGE];
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int col0 = blockIdx.x * KDM_NB;
    const int hs = (H + splits - 1) / splits;  // <= KDM_LCAP (host-checked)
    const int h0 = blockIdx.y * hs;
    const int h1 = min(H, h0 + hs);

    bool keep[PM];
#pragma unroll
    for (int p = 0; p < PM; ++p) {
        const int row = h0 + p * KDM_THREADS + threadIdx.x;
        keep[p] = row < h1 && umask[row] != 0ull;
    }
    uint64_t mk[PM];
#pragma unroll
    for (int p = 0; p < PM; ++p) {
        mk[p] = __ballot(keep[p]);
        if (lane == 0) wcnt[p][wave] = __popcll(mk[p]);
    }
    __syncthreads();
    int n = 0;
#pragma unroll
    for (int p = 0; p < PM; ++p) {
        int off = n;
        for (int w = 0; w < KDM_THREADS / WAVE; ++w) {
            const int c = wcnt[p][w];
            if (w < wave) off += c;
            n += c;
        }
        if (keep[p]) {
            const int pos = off + __builtin_amdgcn_mbcnt_hi((uint32_t)(mk[p] >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)mk[p], 0));
            list[pos] = h0 + p * KDM_THREADS + threadIdx.x;
        }
    }
    __syncthreads();
    const int nchunks = (n + KDM_KC - 1) / KDM_KC;

    const int tt = wave / (4 / NT);
    const int cb = (wave % (4 / NT)) * NCW;
    f32x4 acc[NCW];
#pragma unroll
    for (int i = 0; i < NCW; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    // code piece g = tid + 256 k: unit row g / 8 of the chunk, 16 columns at 16 (g % 8)
    u32x4 wv[DEPTH][WPT];
    u32x4 av[DEPTH][APT];
    bool wok[DEPTH][WPT], aok[DEPTH][APT];
    auto fetch = [&](int slot, int c) {
#pragma unroll
        for (int k = 0; k < WPT; ++k) {
            const int g = threadIdx.x + k * KDM_THREADS;
            const int e = c * KDM_KC + (g >> 3), col = col0 + 16 * (g & 7);
            const bool ok = e < n && col < D;
            wv[slot][k] = load_stream(W2T + (ok ? (size_t)list[e] * D + col : 0));
            wok[slot][k] = ok;
        }
#pragma unroll
        for (int q = 0; q < APT; ++q) {
            const int idx = threadIdx.x + q * KDM_THREADS;
            const int e = c * KDM_KC + idx / (TP / 4);
            const bool ok = e < n;
            av[slot][q] = *reinterpret_cast<const u32x4*>(
                a_rm + (ok ? (size_t)list[e] * TP + 4 * (idx % (TP / 4)) : 0));
            aok[slot][q] = ok;
        }
    };
    auto stage_write = [&](int stage, int d) {
        uint8_t* st = stg[stage];
#pragma unroll
        for (int k = 0; k < WPT; ++k) {
            const int g = threadIdx.x + k * KDM_THREADS;
            const int row = g >> 3, r = row & 31, p0 = 2 * (g & 7);
            const u32x4 w = wok[d][k] ? wv[d][k] : u32x4{0u, 0u, 0u, 0u};
            uint8_t* base = st + (row >> 5) * WPART + r * 256;
            *reinterpret_cast<u32x4*>(base + 16 * swz256(r, p0)) = decode_i8x8(w[0], w[1]);
            *reinterpret_cast<u32x4*>(base + 16 * swz256(r, p0 + 1)) = decode_i8x8(w[2], w[3]);
        }
#pragma unroll
        for (int q = 0; q < APT; ++q) {
            // piece p of a unit's row: the hi parts of tokens 8p .. 8p + 7 for p < TP / 8,
            // else the lo parts of tokens 8 (p - TP / 8) .. + 7
            const int idx = threadIdx.x + q * KDM_THREADS;
            const int row = idx / (TP / 4), r = row & 31, p = idx % (TP / 4);
            const int part = p >= TP / 8 ? 1 : 0, tg = p - part * (TP / 8);
            const int off = 2 * WPART + (2 * part + (row >> 5)) * APART + r * 128 +
                            16 * (swz128(r, tg) ^ (part ? lo_slot_xor<TP>() : 0));
            *reinterpret_cast<u32x4*>(st + off) = aok[d][q] ? av[d][q] : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto compute = [&](int stage) {
        const uint8_t* st = stg[stage];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const uint8_t* ah = st + 2 * WPART + ks * APART;
            const u32x4 fh = frag_tr128(ah, tt * 16, lane);
            const u32x4 fl = frag_tr128(ah + 2 * APART, tt * 16, lane, lo_slot_xor<TP>());
#pragma unroll
            for (int i = 0; i < NCW; ++i) {
                const u32x4 b = frag_tr(st + ks * WPART, (cb + i) * 16, lane);
                acc[i] = mfma_bf16(fh, b, acc[i]);
                acc[i] = mfma_bf16(fl, b, acc[i]);
            }
        }
    };
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) fetch(d, d);
    stage_write(0, 0);
    __syncthreads();
    fetch(0, DEPTH);
    const int niter = (nchunks + DEPTH - 1) / DEPTH * DEPTH;
    for (int c0 = 0; c0 < niter; c0 += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const int c = c0 + d;
            const int nslot = (d + 1) % DEPTH;
            stage_write((c + 1) & 1, nslot);
            if (c < nchunks) compute(c & 1);
            __syncthreads();
            fetch(nslot, c + 1 + DEPTH);
        }
    }
    if (n == 0 && splits > 1) return;
    const int r16 = lane & 15;
#pragma unroll
    for (int i = 0; i < NCW; ++i) {
        const int col = col0 + (cb + i) * 16 + r16;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = tt * 16 + 4 * (lane >> 4) + j;
            if (t < T && col < D) {
                if (splits > 1)
                    atomicAdd(y + (size_t)t * D + col, acc[i][j]);
                else
                    y[(size_t)t * D + col] = acc[i][j];
            }
        }
    }
}

// ---- weight-only int4 batches on MFMA (5..64 tokens)
// As the int8 batches, with codes packed two per byte (column 2j in the low
// nibble) and one fp32 scale per 128 columns of a row. A 256-column chunk holds
// two scale groups, so each wave sums a group's k-steps in a separate tile and
// adds it into its accumulator times the group scale of each row.

// 8 int4 codes (one dword: columns 2b, 2b + 1 in byte b) -> the 8 bf16 values
// n + 136 in column order: the offset nibble n + 8 goes into the low mantissa bits
// of 128.0 (bf16 0x4300), one byte permute per pair of columns.
__device__ inline u32x4 decode_i4x8_offset(uint32_t w) {
    const uint32_t wq = w ^ 0x88888888u;
    const uint32_t lo = wq & 0x0F0F0F0Fu;         // byte b: column 2b
    const uint32_t hi = (wq >> 4) & 0x0F0F0F0Fu;  // byte b: column 2b + 1
    u32x4 o;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        // bytes: lo.b, 0, hi.b, 0 (selector 0x0c gives a zero byte)
        const uint32_t sel = (uint32_t)b | (0x0cu << 8) | ((4u + b) << 16) | (0x0cu << 24);
        o[b] = __builtin_amdgcn_perm(hi, lo, sel) | 0x43004300u;
    }
    return o;
}

// Staging of the int4 gate pass (32 units per block): per 256-column chunk a
// weight row gives 128 bytes of codes (8 pieces of 32 codes; in row r, LDS slot j
// holds piece j ^ ((r >> 1) % 8), so the 4-byte fragment reads of 16 rows at one
// k-step spread over the banks) and a token row of x 512 bytes, staged as in the
// int8 pass. Wave w multiplies unit tile w % 2 against all token tiles over the
// k-steps ks = w / 2 (mod 2) of each chunk.
constexpr int I4_GMAX = 64;  // scale groups per row (D <= 8192)
template <int NT>
struct GateTilesI4 {
    static_assert(NT == 1 || NT == 2 || NT == 4, "token tiles: 1, 2 or 4");
    static constexpr int TP = 16 * NT;
    static constexpr int UB = 32;
    static constexpr int KG = 2;
    static constexpr int TPW = NT;
    static constexpr int WI = UB / 8;                   // weight load instructions per chunk (1 KB each)
    static constexpr int IPW = (WI + TP / 2) / 4;       // load instructions per wave per chunk
    static constexpr int STAGE = UB * 128 + 2 * TP * 256;
    // 3 stages from 20 KB on: at 17-32 tokens the LoPA gate then fits two blocks per CU
    static constexpr int NS = STAGE <= 16384 ? 4 : 3;
    static constexpr int SPT = UB * I4_GMAX / KM_THREADS;  // scale entries per thread
    static_assert((WI + TP / 2) % 4 == 0, "whole load instructions per wave");
    static_assert((NS - 2) * IPW <= 24, "vmcnt wait table");
};

// acc[i] (tiles of this wave) = sum over the K columns (a multiple of 128) of
// scale(row, group) * (codes of rows[] x tokens of x). Each weight operand is
// decoded as n + 136 and a second MFMA with the constant -136 takes the offset
// off. `sc` (LDS, UB x I4_GMAX) receives the rows' group scales, loaded ahead of
// the ring and stored while chunk 0 lands.
template <int NT>
__device__ inline void mfma_gate_pass_i4(f32x4* acc, const uint8_t* __restrict__ W,
                                         const float* __restrict__ scales, const int* rows,
                                         const uint16_t* __restrict__ x,
                                         const uint16_t* __restrict__ zeros, int K, int T,
                                         uint8_t* ring, float (*sc)[I4_GMAX]) {
    using G = GateTilesI4<NT>;
    constexpr int NS = G::NS, IPW = G::IPW;
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int r16 = lane & 15, pq = lane >> 4;
    const int ut = wave % 2, kgroup = wave / 2;
    const int nchunks = (K + KQ_KC - 1) / KQ_KC;
    const int ng = K / I4_GROUP;
#pragma unroll
    for (int i = 0; i < G::TPW; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    // group scales of the block's rows (issued before the ring loads)
    float sv[G::SPT];
#pragma unroll
    for (int m = 0; m < G::SPT; ++m) {
        const int e = threadIdx.x + m * KM_THREADS;
        const int rl = e / I4_GMAX, g = e % I4_GMAX;
        const int row = rows[rl];
        sv[m] = (g < ng && row >= 0) ? scales[(size_t)row * ng + g] : 0.0f;
    }

    const uint8_t* src[IPW];
    bool rok[IPW];
    int pcol[IPW], cstep[IPW];
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
        const int q = wave * IPW + i;  // load instruction of the chunk
        if (q < G::WI) {
            const int rl = 8 * q + (lane >> 3);
            const int p = (lane & 7) ^ ((rl >> 1) & 7);
            const int row = rows[rl];
            rok[i] = row >= 0;
            pcol[i] = 32 * p;
            cstep[i] = KQ_KC / 2;
            src[i] = W + (rok[i] ? (size_t)row * (K / 2) + 16 * p : 0);
        } else {
            const int xr = 4 * (q - G::WI) + pq, tok = xr >> 1, half = xr & 1;
            const int p = r16 ^ (tok & 15);
            rok[i] = tok < T;
            pcol[i] = 128 * half + 8 * p;
            cstep[i] = 2 * KQ_KC;
            src[i] = reinterpret_cast<const uint8_t*>(x + (rok[i] ? (size_t)tok * K + pcol[i] : 0));
        }
    }
    auto issue = [&](int stage, int c) {
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const bool ok = rok[i] && c * KQ_KC + pcol[i] < K;
            const void* g = ok ? (const void*)(src[i] + (size_t)c * cstep[i]) : (const void*)zeros;
            load_lds16(g, ring + stage * G::STAGE + 1024 * (wave * IPW + i));
        }
    };
    const u32x4 neg136 = u32x4{0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u};  // bf16 -136
    const int arow = ut * 16 + r16;
    auto compute = [&](int stage, int c) {
        const uint8_t* wt = ring + stage * G::STAGE;
        const uint8_t* xt = wt + G::UB * 128;
#pragma unroll
        for (int gh = 0; gh < 2; ++gh) {  // the chunk's two scale groups
            f32x4 tmp[G::TPW];
#pragma unroll
            for (int i = 0; i < G::TPW; ++i) tmp[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int ks = 4 * gh + 2 * kk + kgroup;
                // A: codes of columns 32 ks + 8 pq .. + 7 (piece ks, bytes 4 pq .. + 3)
                const uint32_t wv = *reinterpret_cast<const uint32_t*>(
                    wt + arow * 128 + 16 * (ks ^ ((arow >> 1) & 7)) + 4 * pq);
                const u32x4 af = decode_i4x8_offset(wv);
                const int pb = 4 * (ks & 3) + pq;
#pragma unroll
                for (int i = 0; i < G::TPW; ++i) {
                    const int tok = i * 16 + r16;
                    const u32x4 bf = *reinterpret_cast<const u32x4*>(
                        xt + (2 * tok + (ks >> 2)) * 256 + 16 * (pb ^ r16));
                    tmp[i] = mfma_bf16(af, bf, tmp[i]);
                    tmp[i] = mfma_bf16(neg136, bf, tmp[i]);
                }
            }
            // C rows of this lane: 4 (lane / 16) + j of the unit tile
            const int g = 2 * c + gh;
            float s4[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) s4[j] = sc[ut * 16 + 4 * pq + j][g < I4_GMAX ? g : 0];
#pragma unroll
            for (int i = 0; i < G::TPW; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(s4[j], tmp[i][j], acc[i][j]);
        }
    };

#pragma unroll
    for (int d = 0; d < NS - 1; ++d) issue(d, d);
    const int niter = (nchunks + NS - 1) / NS * NS;
    for (int c0 = 0; c0 < niter; c0 += NS) {
#pragma unroll
        for (int d = 0; d < NS; ++d) {
            const int c = c0 + d;
            wait_vmcnt((NS - 2) * IPW);  // this wave's pieces of chunk c (and the scales) have landed
            if (c == 0) {
#pragma unroll
                for (int m = 0; m < G::SPT; ++m) {
                    const int e = threadIdx.x + m * KM_THREADS;
                    sc[e / I4_GMAX][e % I4_GMAX] = sv[m];
                }
            }
            __syncthreads();                // ... and every wave's; chunk c - 1 is consumed
            issue((d + NS - 1) % NS, c + NS - 1);
            if (c < nchunks) compute(d, c);
        }
    }
    wait_vmcnt(0);
    __syncthreads();
}

// Gate and gathered up projection of a batch, int4 up (and gate) weights:
// z = sum_g s1_ig (q1_i,g . x_g) over the int4 W1 (LoPA: z = sU_i (qU_i . t) over
// the int8 U and the two bf16 parts of t, plus (G x)_i when asked); for the units
// live for some token u = sum_g s3_ig (q3_i,g . x_g) (through A under double
// activation); a_i = A(z_i) u_i is stored unscaled (the W2T group scales vary
// along D, so the down pass applies them).
template <int NT, bool DENSE, bool LOPA>
__global__ __launch_bounds__(KM_THREADS) void k_gate_up_mfma_i4(
    const uint16_t* __restrict__ x, const void* __restrict__ W1, const float* __restrict__ s1,
    const uint8_t* __restrict__ W3, const float* __restrict__ s3,
    const uint16_t* __restrict__ zeros, float* __restrict__ a_rm, uint64_t* __restrict__ umask,
    uint8_t* __restrict__ live_out, float* __restrict__ y_zero, int D, int H, int T, int act,
    const uint16_t* __restrict__ t_hi, const uint16_t* __restrict__ t_lo, int r, unsigned flags) {
    using G4 = GateTilesI4<NT>;
    using G8 = GateTilesI8<NT, 2>;
    constexpr int TP = G4::TP, UB = G4::UB, KG = G4::KG;
    static_assert(G8::UB == UB && G8::KG == KG, "one tile plan for both passes");
    // LDS: the int4 ring with the group scales of its pass behind it (they are written
    // and read only while an int4 pass runs), or the int8 ring of the LoPA U pass if
    // larger; the partial sums of a pass go through the drained ring, and each thread
    // keeps the z of its (unit, token) entries in registers through the W3 pass
    constexpr int G4RING = G4::NS * G4::STAGE;
    constexpr int RING = (LOPA && G8::NS * G8::STAGE > G4RING + UB * I4_GMAX * 4)
                             ? G8::NS * G8::STAGE
                             : G4RING + UB * I4_GMAX * 4;
    constexpr int EPT = UB * TP / KM_THREADS;  // (unit, token) entries per thread
    static_assert(EPT * KM_THREADS == UB * TP, "entries per thread");
    static_assert(KG * UB * (TP + 1) * 4 <= G4RING, "partial sums fit the ring");
    __shared__ __attribute__((aligned(16))) uint8_t ring[RING];
    float (*part)[UB][TP + 1] = reinterpret_cast<float (*)[UB][TP + 1]>(ring);
    float (*sc)[I4_GMAX] = reinterpret_cast<float (*)[I4_GMAX]>(ring + G4RING);
    __shared__ unsigned long long tmask[UB];
    __shared__ int rows_g[UB];
    __shared__ int rows_u[UB];
    __shared__ int upos[UB];
    __shared__ int nu_s;
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int r16 = lane & 15;
    const int u0 = blockIdx.x * UB;
    const int ut = wave % 2, kgroup = wave / 2;

    if (y_zero) {
        for (int j = blockIdx.x * KM_THREADS + threadIdx.x; j < T * D; j += gridDim.x * KM_THREADS)
            y_zero[j] = 0.0f;
    }
    if (threadIdx.x < UB) {
        tmask[threadIdx.x] = 0ull;
        rows_g[threadIdx.x] = (u0 + (int)threadIdx.x < H) ? u0 + (int)threadIdx.x : -1;
    }
    __syncthreads();

    auto store_tiles = [&](const f32x4 (&acc)[NT]) {
#pragma unroll
        for (int i = 0; i < NT; ++i) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                part[kgroup][ut * 16 + 4 * (lane >> 4) + j][i * 16 + r16] = acc[i][j];
        }
    };

    {
        f32x4 acc[NT];
        if (LOPA) {
            f32x4 acc2[NT];
            mfma_gate_pass_i8<NT, 2>(acc, (const int8_t*)W1, rows_g, t_hi, zeros, r, T, ring);
            mfma_gate_pass_i8<NT, 2>(acc2, (const int8_t*)W1, rows_g, t_lo, zeros, r, T, ring);
#pragma unroll
            for (int i = 0; i < NT; ++i) acc[i] += acc2[i];
        } else {
            mfma_gate_pass_i4<NT>(acc, (const uint8_t*)W1, s1, rows_g, x, zeros, D, T, ring, sc);
        }
        store_tiles(acc);
    }
    __syncthreads();
    float zr[EPT];
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
        const int e = threadIdx.x + k * KM_THREADS;
        const int i = e / TP, t = e % TP;
        const bool ok = (u0 + i < H) && t < T;
        float z = 0.0f;
#pragma unroll
        for (int g = 0; g < KG; ++g) z += part[g][i][t];
        if (ok && LOPA) {
            z *= s1[u0 + i];
            if (flags & LOPA_G_TILED) z += Elem<uint16_t>::get1(x[(size_t)t * D + (u0 + i) % D]);
        }
        zr[k] = z;
        const bool live = ok && (DENSE || z > 0.0f);
        const uint64_t tm = unit_token_mask<TP>(live);
        if (t == 0) tmask[i] = tm;
        if (ok && live_out) live_out[(size_t)t * H + u0 + i] = (z > 0.0f) ? 1 : 0;
    }
    __syncthreads();
    if (wave == 0) {
        const bool any = lane < UB && tmask[lane] != 0ull;
        const uint64_t m = __ballot(any);
        const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
        if (lane < UB) {
            upos[lane] = any ? pos : -1;
            rows_u[lane] = -1;
            if (u0 + lane < H) umask[u0 + lane] = tmask[lane];
        }
        if (lane == 0) nu_s = __popcll(m);
    }
    __syncthreads();
    if (threadIdx.x < UB && upos[threadIdx.x] >= 0) rows_u[upos[threadIdx.x]] = u0 + threadIdx.x;
    const int nu = nu_s;
    __syncthreads();

    if (nu > 0) {
        f32x4 acc[NT];
        mfma_gate_pass_i4<NT>(acc, W3, s3, rows_u, x, zeros, D, T, ring, sc);
        store_tiles(acc);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
        const int e = threadIdx.x + k * KM_THREADS;
        const int i = e / TP, t = e % TP;
        if (u0 + i >= H) continue;
        const int p = upos[i];
        float av = 0.0f;
        if (p >= 0 && t < T && ((tmask[i] >> t) & 1ull)) {
            float u = 0.0f;
#pragma unroll
            for (int g = 0; g < KG; ++g) u += part[g][p][t];
            if (LOPA && (flags & LOPA_DOUBLE_ACT)) u = activation(act, u);
            av = activation(act, zr[k]) * u;
        }
        a_rm[(size_t)(u0 + i) * TP + t] = av;
    }
}

// Gate and up projection of an int4 batch in one pass (standard gating, batches
// above 10 tokens and the dense comparator), as k_gate_up_mfma_fused_i8 does for
// int8: each 256-column chunk stages the block's 32 W1 code rows and 32 W3 code rows
// (128 bytes each) and the token rows of x together. Wave w owns unit tile w & 1 of
// matrix w >> 1 over every k-step; each 128-column group is summed in its own
// accumulators and added with the row's group scale (both matrices' scales of the
// block in LDS), the same steps as mfma_gate_pass_i4.
template <int NT>
struct FusedTilesI4 {
    static_assert(NT == 1 || NT == 2 || NT == 4, "token tiles: 1, 2 or 4");
    static constexpr int TP = 16 * NT;
    static constexpr int UB = 32;
    static constexpr int WI = 2 * UB / 8;                  // weight load instructions per chunk (1 KB each)
    static constexpr int IPW = (WI + TP / 2) / 4;          // load instructions per wave per chunk
    static constexpr int STAGE = 2 * UB * 128 + 2 * TP * 256;
    static constexpr int NS = STAGE <= 24576 ? 4 : 3;
    static constexpr int SPT = 2 * UB * I4_GMAX / KM_THREADS;  // scale entries per thread
    static_assert((WI + TP / 2) % 4 == 0, "whole load instructions per wave");
    static_assert((NS - 2) * IPW <= 24, "vmcnt wait table");
    static_assert(2 * UB * (TP + 1) * 4 <= NS * STAGE, "z and u tiles fit the ring");
};

template <int NT>
__device__ inline void mfma_fused_pass_i4(f32x4 (&acc)[NT], const uint8_t* __restrict__ W1,
                                          const float* __restrict__ s1,
                                          const uint8_t* __restrict__ W3,
                                          const float* __restrict__ s3, int u0, int H,
                                          const uint16_t* __restrict__ x,
                                          const uint16_t* __restrict__ zeros, int K, int T,
                                          uint8_t* ring, float (*sc)[I4_GMAX]) {
    using G = FusedTilesI4<NT>;
    constexpr int NS = G::NS, IPW = G::IPW, UB = G::UB;
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int r16 = lane & 15, pq = lane >> 4;
    const int ut = wave & 1, mat = wave >> 1;
    const int nchunks = (K + KQ_KC - 1) / KQ_KC;
    const int ng = K / I4_GROUP;
#pragma unroll
    for (int i = 0; i < NT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    // group scales of the block's W1 rows (sc rows 0 .. UB - 1) and W3 rows (UB ..),
    // issued before the ring loads
    float sv[G::SPT];
#pragma unroll
    for (int m = 0; m < G::SPT; ++m) {
        const int e = threadIdx.x + m * KM_THREADS;
        const int rl = e / I4_GMAX, g = e % I4_GMAX;
        const int row = u0 + (rl & (UB - 1));
        const float* scales = rl < UB ? s1 : s3;
        sv[m] = (g < ng && row < H) ? scales[(size_t)row * ng + g] : 0.0f;
    }

    const uint8_t* src[IPW];
    bool rok[IPW];
    int pcol[IPW], cstep[IPW];
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
        const int q = wave * IPW + i;  // load instruction of the chunk
        if (q < G::WI) {
            const int rl = 8 * q + (lane >> 3);  // staged weight row: W1 rows, then W3 rows
            const int p = (lane & 7) ^ ((rl >> 1) & 7);
            const int row = u0 + (rl & (UB - 1));
            const uint8_t* W = rl < UB ? W1 : W3;
            rok[i] = row < H;
            pcol[i] = 32 * p;
            cstep[i] = KQ_KC / 2;
            src[i] = W + (rok[i] ? (size_t)row * (K / 2) + 16 * p : 0);
        } else {
            const int xr = 4 * (q - G::WI) + pq, tok = xr >> 1, half = xr & 1;
            const int p = r16 ^ (tok & 15);
            rok[i] = tok < T;
            pcol[i] = 128 * half + 8 * p;
            cstep[i] = 2 * KQ_KC;
            src[i] = reinterpret_cast<const uint8_t*>(x + (rok[i] ? (size_t)tok * K + pcol[i] : 0));
        }
    }
    auto issue = [&](int stage, int c) {
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const bool ok = rok[i] && c * KQ_KC + pcol[i] < K;
            const void* g = ok ? (const void*)(src[i] + (size_t)c * cstep[i]) : (const void*)zeros;
            load_lds16(g, ring + stage * G::STAGE + 1024 * (wave * IPW + i));
        }
    };
    const u32x4 neg136 = u32x4{0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u};  // bf16 -136
    const int arow = mat * UB + ut * 16 + r16;
    auto compute = [&](int stage, int c) {
        const uint8_t* wt = ring + stage * G::STAGE;
        const uint8_t* xt = wt + 2 * UB * 128;
#pragma unroll
        for (int gh = 0; gh < 2; ++gh) {  // the chunk's two scale groups
            f32x4 tmp[NT];
#pragma unroll
            for (int i = 0; i < NT; ++i) tmp[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int ks = 4 * gh + kk;
                // A: codes of columns 32 ks + 8 pq .. + 7 (piece ks, bytes 4 pq .. + 3)
                const uint32_t wv = *reinterpret_cast<const uint32_t*>(
                    wt + arow * 128 + 16 * (ks ^ ((arow >> 1) & 7)) + 4 * pq);
                const u32x4 af = decode_i4x8_offset(wv);
                const int pb = 4 * (ks & 3) + pq;
#pragma unroll
                for (int i = 0; i < NT; ++i) {
                    const int tok = i * 16 + r16;
                    const u32x4 bf = *reinterpret_cast<const u32x4*>(
                        xt + (2 * tok + (ks >> 2)) * 256 + 16 * (pb ^ r16));
                    tmp[i] = mfma_bf16(af, bf, tmp[i]);
                    tmp[i] = mfma_bf16(neg136, bf, tmp[i]);
                }
            }
            // C rows of this lane: 4 (lane / 16) + j of the unit tile
            const int g = 2 * c + gh;
            float s4[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) s4[j] = sc[mat * UB + ut * 16 + 4 * pq + j][g < I4_GMAX ? g : 0];
#pragma unroll
            for (int i = 0; i < NT; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(s4[j], tmp[i][j], acc[i][j]);
        }
    };

#pragma unroll
    for (int d = 0; d < NS - 1; ++d) issue(d, d);
    const int niter = (nchunks + NS - 1) / NS * NS;
    for (int c0 = 0; c0 < niter; c0 += NS) {
#pragma unroll
        for (int d = 0; d < NS; ++d) {
            const int c = c0 + d;
            wait_vmcnt((NS - 2) * IPW);  // this wave's pieces of chunk c (and the scales) have landed
            if (c == 0) {
#pragma unroll
                for (int m = 0; m < G::SPT; ++m) {
                    const int e = threadIdx.x + m * KM_THREADS;
                    sc[e / I4_GMAX][e % I4_GMAX] = sv[m];
                }
            }
            __syncthreads();                // ... and every wave's; chunk c - 1 is consumed
            issue((d + NS - 1) % NS, c + NS - 1);
            if (c < nchunks) compute(d, c);
        }
    }
    wait_vmcnt(0);
    __syncthreads();
}

template <int NT, bool DENSE>
__global__ __launch_bounds__(KM_THREADS) void k_gate_up_mfma_fused_i4(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ W1, const float* __restrict__ s1,
    const uint8_t* __restrict__ W3, const float* __restrict__ s3,
    const uint16_t* __restrict__ zeros, float* __restrict__ a_rm, uint64_t* __restrict__ umask,
    uint8_t* __restrict__ live_out, float* __restrict__ y_zero, int D, int H, int T, int act) {
    using G = FusedTilesI4<NT>;
    constexpr int TP = G::TP, UB = G::UB;
    __shared__ __attribute__((aligned(16))) uint8_t ring[G::NS * G::STAGE];
    __shared__ float sc[2 * UB][I4_GMAX];
    __shared__ unsigned long long tmask[UB];
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int r16 = lane & 15;
    const int u0 = blockIdx.x * UB;
    const int ut = wave & 1, mat = wave >> 1;

    if (y_zero) {
        for (int j = blockIdx.x * KM_THREADS + threadIdx.x; j < T * D; j += gridDim.x * KM_THREADS)
            y_zero[j] = 0.0f;
    }
    if (threadIdx.x < UB) tmask[threadIdx.x] = 0ull;  // first read after the pass's barriers

    f32x4 acc[NT];
    mfma_fused_pass_i4<NT>(acc, W1, s1, W3, s3, u0, H, x, zeros, D, T, ring, sc);
    // the ring is free after the pass: z sums in zu[0], u sums in zu[1]
    float (*zu)[UB][TP + 1] = reinterpret_cast<float (*)[UB][TP + 1]>(ring);
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) zu[mat][ut * 16 + 4 * (lane >> 4) + j][i * 16 + r16] = acc[i][j];
    __syncthreads();
    for (int e = threadIdx.x; e < UB * TP; e += KM_THREADS) {
        const int i = e / TP, t = e % TP;
        const bool in = u0 + i < H;
        const bool ok = in && t < T;
        const float z = zu[0][i][t];
        const bool live = ok && (DENSE || z > 0.0f);
        const uint64_t tm = unit_token_mask<TP>(live);  // before the wave's lanes part
        if (!in) continue;
        if (t == 0) tmask[i] = tm;
        if (ok && live_out) live_out[(size_t)t * H + u0 + i] = (z > 0.0f) ? 1 : 0;
        a_rm[(size_t)(u0 + i) * TP + t] = live ? activation(act, z) * zu[1][i][t] : 0.0f;
    }
    __syncthreads();
    if (threadIdx.x < UB && u0 + (int)threadIdx.x < H) umask[u0 + threadIdx.x] = tmask[threadIdx.x];
}

// Down pass of an int4 batch: k_down_mfma with the codes of W2T (32 columns per
// 16-byte piece, one piece per thread per chunk of 64 units x 128 columns)
// decoded exactly into the bf16 staging layout; the block's 128 columns are one
// scale group, so each unit's product is multiplied by its group scale as it is
// staged. D a multiple of 128.
template <int NT>
__global__ __launch_bounds__(KDM_THREADS) void k_down_mfma_i4(
    const float* __restrict__ a_rm, const uint64_t* __restrict__ umask,
    const uint8_t* __restrict__ W2T, const float* __restrict__ s2, float* __restrict__ y, int D,
    int H, int T, int splits) {
    static_assert(NT == 1 || NT == 2 || NT == 4, "token tiles: 1, 2 or 4");
    static_assert(KDM_NB == I4_GROUP, "one scale group per column tile");
    constexpr int TP = 16 * NT;
    constexpr int APT = KDM_KC * TP / 4 / KDM_THREADS;
    constexpr int NCW = 2 * NT;
    constexpr int DEPTH = NT == 1 ? 6 : (NT == 2 ? 5 : 4);
    constexpr int WPART = 32 * 256;
    constexpr int APART = 32 * 128;
    constexpr int STAGE = 2 * WPART + 4 * APART;
    constexpr int PM = KDM_LCAP / KDM_THREADS;
    static_assert(KDM_KC * KDM_NB / 32 == KDM_THREADS, "one code piece per thread per chunk");
    __shared__ int list[KDM_LCAP];
    __shared__ int wcnt[PM][KDM_THREADS / WAVE];
    __shared__ __attribute__((aligned(256))) uint8_t stg[2][STAGE];
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int col0 = blockIdx.x * KDM_NB;
    const int ng = D / I4_GROUP;
    const int grp = col0 / I4_GROUP;
    const int hs = (H + splits - 1) / splits;  // <= KDM_LCAP (host-checked)
    const int h0 = blockIdx.y * hs;
    const int h1 = min(H, h0 + hs);

    bool keep[PM];
#pragma unroll
    for (int p = 0; p < PM; ++p) {
        const int row = h0 + p * KDM_THREADS + threadIdx.x;
        keep[p] = row < h1 && umask[row] != 0ull;
    }
    uint64_t mk[PM];
#pragma unroll
    for (int p = 0; p < PM; ++p) {
        mk[p] = __ballot(keep[p]);
        if (lane == 0) wcnt[p][wave] = __popcll(mk[p]);
    }
    __syncthreads();
    int n = 0;
#pragma unroll
    for (int p = 0; p < PM; ++p) {
        int off = n;
        for (int w = 0; w < KDM_THREADS / WAVE; ++w) {
            const int c = wcnt[p][w];
            if (w < wave) off += c;
            n += c;
        }
        if (keep[p]) {
            const int pos = off + __builtin_amdgcn_mbcnt_hi((uint32_t)(mk[p] >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)mk[p], 0));
            list[pos] = h0 + p * KDM_THREADS + threadIdx.x;
        }
    }
    __syncthreads();
    const int nchunks = (n + KDM_KC - 1) / KDM_KC;

    const int tt = wave / (4 / NT);
    const int cb = (wave % (4 / NT)) * NCW;
    f32x4 acc[NCW];
#pragma unroll
    for (int i = 0; i < NCW; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    // code piece tid: unit row tid / 4 of the chunk, 32 columns at 32 (tid % 4)
    u32x4 wv[DEPTH];
    float4 av[DEPTH][APT];
    float sa[DEPTH][APT];
    bool wok[DEPTH], aok[DEPTH][APT];
    auto fetch = [&](int slot, int c) {
        {
            const int e = c * KDM_KC + (threadIdx.x >> 2), col = col0 + 32 * (threadIdx.x & 3);
            const bool ok = e < n && col < D;
            wv[slot] = load_stream(W2T + (ok ? (size_t)list[e] * (D / 2) + col / 2 : 0));
            wok[slot] = ok;
        }
#pragma unroll
        for (int q = 0; q < APT; ++q) {
            const int idx = threadIdx.x + q * KDM_THREADS;
            const int e = c * KDM_KC + idx / (TP / 4);
            const bool ok = e < n;
            const size_t unit = ok ? (size_t)list[e] : 0;
            av[slot][q] = *reinterpret_cast<const float4*>(a_rm + unit * TP + (ok ? 4 * (idx % (TP / 4)) : 0));
            sa[slot][q] = ok ? s2[unit * ng + grp] : 0.0f;
            aok[slot][q] = ok;
        }
    };
    auto stage_write = [&](int stage, int d) {
        uint8_t* st = stg[stage];
        {
            const int row = threadIdx.x >> 2, r = row & 31, p0 = 4 * (threadIdx.x & 3);
            const u32x4 w = wok[d] ? wv[d] : u32x4{0u, 0u, 0u, 0u};  // codes 0
            uint8_t* base = st + (row >> 5) * WPART + r * 256;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                // value n + 136 minus 136, exact in fp32; bf16 of the integer n
                const u32x4 o = decode_i4x8_offset(w[k]);
                u32x4 v;
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    const float f0 = __uint_as_float(o[h] << 16) - 136.0f;
                    const float f1 = __uint_as_float(o[h] & 0xffff0000u) - 136.0f;
                    v[h] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
                }
                *reinterpret_cast<u32x4*>(base + 16 * swz256(r, p0 + k)) = v;
            }
        }
#pragma unroll
        for (int q = 0; q < APT; ++q) {
            const int idx = threadIdx.x + q * KDM_THREADS;
            const int row = idx / (TP / 4), r = row & 31, t0 = 4 * (idx % (TP / 4));
            const float4 f = aok[d][q] ? av[d][q] : make_float4(0.f, 0.f, 0.f, 0.f);
            const float sg = sa[d][q];
            const float fv[4] = {f.x * sg, f.y * sg, f.z * sg, f.w * sg};
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                hi[j] = bf16_rne(fv[j]);
                lo[j] = bf16_rne(fv[j] - __uint_as_float(hi[j] << 16));
            }
            const int off = 2 * WPART + (row >> 5) * APART + r * 128 + 16 * swz128(r, t0 >> 3) + 8 * ((t0 >> 2) & 1);
            *reinterpret_cast<uint2*>(st + off) = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
            *reinterpret_cast<uint2*>(st + off + 2 * APART) = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
        }
    };
    auto compute = [&](int stage) {
        const uint8_t* st = stg[stage];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const uint8_t* ah = st + 2 * WPART + ks * APART;
            const u32x4 fh = frag_tr128(ah, tt * 16, lane);
            const u32x4 fl = frag_tr128(ah + 2 * APART, tt * 16, lane);
#pragma unroll
            for (int i = 0; i < NCW; ++i) {
                const u32x4 b = frag_tr(st + ks * WPART, (cb + i) * 16, lane);
                acc[i] = mfma_bf16(fh, b, acc[i]);
                acc[i] = mfma_bf16(fl, b, acc[i]);
            }
        }
    };
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) fetch(d, d);
    stage_write(0, 0);
    __syncthreads();
    fetch(0, DEPTH);
    const int niter = (nchunks + DEPTH - 1) / DEPTH * DEPTH;
    for (int c0 = 0; c0 < niter; c0 += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const int c = c0 + d;
            const int nslot = (d + 1) % DEPTH;
            stage_write((c + 1) & 1, nslot);
            if (c < nchunks) compute(c & 1);
            __syncthreads();
            fetch(nslot, c + 1 + DEPTH);
        }
    }
    if (n == 0 && splits > 1) return;
    const int r16 = lane & 15;
#pragma unroll
    for (int i = 0; i < NCW; ++i) {
        const int col = col0 + (cb + i) * 16 + r16;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = tt * 16 + 4 * (lane >> 4) + j;
            if (t < T && col < D) {
                if (splits > 1)
                    atomicAdd(y + (size_t)t * D + col, acc[i][j]);
                else
                    y[(size_t)t * D + col] = acc[i][j];
            }
        }
    }
}

// Epilogue of the small-batch down passes: each lane's TT x VEC column sums are
// reduced over the wave's lane groups (shuffles), the wave sums of up to TR
// tokens at a time are staged in LDS (red[TR][KD_WAVES][CB]), and after one
// barrier per round the block adds the sums over its waves into y (fp32 atomics
// when the unit range is split, else a plain store).
template <int TT, int TR, int VEC, int LPR, int CB>
__device__ inline void tb_down_epilogue(float (&acc)[TT][VEC], float (*red)[KD_WAVES][CB],
                                        float* __restrict__ y, int D, int T, int col0,
                                        int splits, int wave, int sub, int grp) {
#pragma unroll
    for (int t0 = 0; t0 < TT; t0 += TR) {
        if (t0 >= T) break;  // uniform
        if (t0 > 0) __syncthreads();  // the previous round has read red
#pragma unroll
        for (int j = 0; j < TR; ++j) {
            const int t = t0 + j;
            if (t >= T) continue;  // uniform; the loop stays unrolled so acc stays in registers
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                float v = acc[t][k];
                for (int o = LPR; o < WAVE; o <<= 1) v += __shfl_xor(v, o, WAVE);
                acc[t][k] = v;
            }
            if (grp == 0) {
#pragma unroll
                for (int k = 0; k < VEC; ++k) red[j][wave][sub * VEC + k] = acc[t][k];
            }
        }
        __syncthreads();
        const int nt = min(TR, T - t0);
        for (int i = threadIdx.x; i < nt * CB; i += KD_THREADS) {
            const int j = i / CB, c = i % CB;
            float s = 0.0f;
            for (int w2 = 0; w2 < KD_WAVES; ++w2) s += red[j][w2][c];
            if (col0 + c < D) {
                if (splits > 1)
                    atomicAdd(y + (size_t)(t0 + j) * D + col0 + c, s);
                else
                    y[(size_t)(t0 + j) * D + col0 + c] = s;
            }
        }
    }
}

// Down projection for small batches (T <= TT <= 8), bf16: like k_down_t1, but
// the units kept are those live for some token (umask != 0; DENSE: all), each
// lane keeps TT x 8 accumulators, and a unit's TT products come from the
// unit-major a_rm[unit][tp]. y is cleared by the gate pass when splits > 1.
template <int LPR, int PMAX, int TT>
__global__ __launch_bounds__(KD_THREADS) void k_down_tb(const float* __restrict__ a_rm,
                                                        const uint64_t* __restrict__ umask,
                                                        const uint16_t* __restrict__ W2T,
                                                        float* __restrict__ y, int D, int H,
                                                        int T, int tp, int splits) {
    constexpr int VEC = 8;
    constexpr int CB = LPR * VEC;
    constexpr int RPI = WAVE / LPR;
    constexpr int UF = 4;
    __shared__ float red[TT < 4 ? TT : 4][KD_WAVES][CB];

    const int nslices = (D + CB - 1) / CB;
    const int per_xcd = (nslices + 7) / 8;
    const int bx = blockIdx.x;
    const int slice = (bx & 7) * per_xcd + (bx >> 3);
    if (slice >= nslices) return;
    const int col0 = slice * CB;
    const int hs = (H + splits - 1) / splits;
    const int h0 = blockIdx.y * hs;
    const int h1 = min(H, h0 + hs);
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int sub = lane % LPR, grp = lane / LPR;
    const int col = col0 + sub * VEC;
    const bool col_ok = col < D;
    uint64_t mk[PMAX];
#pragma unroll
    for (int p = 0; p < PMAX; ++p) {
        const int row = h0 + (wave * PMAX + p) * WAVE + lane;
        mk[p] = __ballot(row < h1 && umask[row] != 0ull);
    }

    float acc[TT][VEC];
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int k = 0; k < VEC; ++k) acc[t][k] = 0.0f;

#pragma unroll
    for (int p = 0; p < PMAX; ++p) {
        const int base = h0 + (wave * PMAX + p) * WAVE;
        uint64_t m = mk[p];
        while (m) {
            int bit[UF];
            next_live_bits<RPI, UF>(m, grp, bit);
            u32x4 wv[UF];
            float av[UF][TT];
#pragma unroll
            for (int u = 0; u < UF; ++u) {
                const bool e_ok = bit[u] >= 0;
                const int row = e_ok ? (base + bit[u]) : 0;
                wv[u] = (e_ok && col_ok) ? load_stream(W2T + (size_t)row * D + col)
                                          : u32x4{0u, 0u, 0u, 0u};
                // TT <= 16 <= tp, and padded token slots of a_rm hold 0
                const float* ar = a_rm + (size_t)row * tp;
#pragma unroll
                for (int t = 0; t < TT; t += 2) {
                    const float2 v2 = e_ok ? *reinterpret_cast<const float2*>(ar + t)
                                            : make_float2(0.0f, 0.0f);
                    av[u][t] = v2.x;
                    av[u][t + 1] = v2.y;
                }
            }
#pragma unroll
            for (int u = 0; u < UF; ++u)
#pragma unroll
                for (int k = 0; k < VEC; ++k) {
                    const float w = Elem<uint16_t>::get(wv[u], k);
#pragma unroll
                    for (int t = 0; t < TT; ++t) acc[t][k] = fmaf(av[u][t], w, acc[t][k]);
                }
        }
    }
    tb_down_epilogue<TT, (TT < 4 ? TT : 4), VEC, LPR, CB>(acc, red, y, D, T, col0, splits, wave, sub, grp);
}

// Small batches (T <= TT <= 4) with weight-only int8 weights, union of the
// tokens' live sets. Gate/up: RW consecutive units per wave, their W1 rows
// issued first, x of the tokens and its sums taken once for all of them; every
// int8 weight of a W1 row (and of the W3 row when the unit is live for some
// token) is converted once and multiplied with the TT tokens' x (bf16, unpacked
// per use); the TT
// per-lane sums are reduced together (multi_reduce: lane l ends with token
// bitrev(l mod TT)). Writes a'[unit][tp] = A(z) u s2 (the W2T row scale folded
// in; 0 for dead pairs and padded slots), the token mask umask[unit] (DENSE:
// all tokens), live flags [T x H] when asked, and clears y for the down pass.
template <int NC, int TT, bool DENSE, int RW>
__global__ __launch_bounds__(K1_THREADS) void k_gate_up_tb_i8(
    const uint16_t* __restrict__ x, const int8_t* __restrict__ W1, const float* __restrict__ s1,
    const int8_t* __restrict__ W3, const float* __restrict__ s3, const float* __restrict__ s2,
    float* __restrict__ a_rm, uint64_t* __restrict__ umask, uint8_t* __restrict__ live_out,
    float* __restrict__ y_zero, int D, int H, int T, int tp, int act) {
    constexpr int CW = WAVE * 16;  // columns of one chunk: 16 int8 per lane
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int unit0 = (blockIdx.x * K1_WAVES + wave) * RW;  // RW consecutive units per wave
    u32x4 wr[RW][NC];  // every W1 row of the wave, issued first
#pragma unroll
    for (int q = 0; q < RW; ++q)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int col = c * CW + lane * 16;
            wr[q][c] = (unit0 + q < H && col < D) ? load_stream(W1 + (size_t)(unit0 + q) * D + col)
                                                  : u32x4{0u, 0u, 0u, 0u};
        }
    u32x4 xb[TT][NC][2];  // the lane's 16 columns of each token: two pieces of 8 bf16
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int col = c * CW + lane * 16;
            const bool ok = t < T && col < D;
            xb[t][c][0] = ok ? load_cached(x + (size_t)t * D + col) : u32x4{0u, 0u, 0u, 0u};
            xb[t][c][1] = ok ? load_cached(x + (size_t)t * D + col + 8) : u32x4{0u, 0u, 0u, 0u};
        }
    if (y_zero) {
        for (int j = blockIdx.x * K1_THREADS + threadIdx.x; j < T * D; j += gridDim.x * K1_THREADS)
            y_zero[j] = 0.0f;
    }
    // sum of each token's 16 x values of the lane per chunk (for the code offset)
    float xs[TT][NC];
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            float a = 0.0f;  // one bf16 dot2 against (1, 1) per pair
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint32_t xq = xb[t][c][k >> 2][k & 3];
                a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xq),
                                                    __builtin_bit_cast(bf16x2, 0x3F803F80u), a, false);
            }
            xs[t][c] = a;
        }
    // A weight q becomes q + 128 (byte ^ 0x80), converted exactly to fp32 and packed
    // two at a time as bf16 (8 significant bits hold 0..255); one bf16 dot2 per token
    // then takes two weights, and 128 * sum(x) comes off once per chunk.
    auto dot_tokens = [&](const u32x4 (&wr)[NC], float (&v)[TT]) {
#pragma unroll
        for (int t = 0; t < TT; ++t) v[t] = 0.0f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            float sp[TT];
#pragma unroll
            for (int t = 0; t < TT; ++t) sp[t] = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t wq = wr[c][q] ^ 0x80808080u;
                const uint32_t f0 = __float_as_uint((float)(wq & 0xffu));
                const uint32_t f1 = __float_as_uint((float)((wq >> 8) & 0xffu));
                const uint32_t f2 = __float_as_uint((float)((wq >> 16) & 0xffu));
                const uint32_t f3 = __float_as_uint((float)(wq >> 24));
                // high halves (the bf16 values): f0 | f1 << 16, f2 | f3 << 16
                const uint32_t p01 = __builtin_amdgcn_perm(f1, f0, 0x07060302u);
                const uint32_t p23 = __builtin_amdgcn_perm(f3, f2, 0x07060302u);
#pragma unroll
                for (int t = 0; t < TT; ++t) {
                    const u32x4 xq = xb[t][c][q >> 1];
                    const uint32_t x01 = xq[2 * (q & 1)], x23 = xq[2 * (q & 1) + 1];
                    sp[t] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p01),
                                                            __builtin_bit_cast(bf16x2, x01), sp[t], false);
                    sp[t] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p23),
                                                            __builtin_bit_cast(bf16x2, x23), sp[t], false);
                }
            }
#pragma unroll
            for (int t = 0; t < TT; ++t) v[t] += fmaf(-128.0f, xs[t][c], sp[t]);
        }
    };
    const int tl = bit_rev<TT>(lane & (TT - 1));  // token whose sums this lane ends with
#pragma unroll
    for (int q = 0; q < RW; ++q) {
        const int unit = unit0 + q;
        if (unit >= H) break;  // wave-uniform
        const float sc1 = s1[unit];
        float v[TT];
        dot_tokens(wr[q], v);
        const float z = multi_reduce<TT>(v) * sc1;
        const bool lv = tl < T && z > 0.0f;
        const uint64_t bl = __ballot(lv && lane < TT);
        uint64_t m = 0;
#pragma unroll
        for (int t = 0; t < TT; ++t) m |= ((bl >> bit_rev<TT>(t)) & 1ull) << t;
        if (lane == 0) umask[unit] = DENSE ? ((1ull << T) - 1) : m;
        if (live_out && lane < TT && tl < T) live_out[(size_t)tl * H + unit] = lv ? 1 : 0;
        if (!DENSE && m == 0) {
            if (lane < TT) a_rm[(size_t)unit * tp + tl] = 0.0f;
            continue;
        }
        u32x4 w[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int col = c * CW + lane * 16;
            w[c] = col < D ? load_stream(W3 + (size_t)unit * D + col) : u32x4{0u, 0u, 0u, 0u};
        }
        dot_tokens(w, v);
        const float u = multi_reduce<TT>(v) * s3[unit];
        if (lane < TT) a_rm[(size_t)unit * tp + tl] = tl < T ? activation(act, z) * u * s2[unit] : 0.0f;
    }
}

// Down pass of the int8 small batches: as k_down_t1_i8 (16 lanes x 16 int8
// columns per 256-column slice, 16 unit-range splits, fp32 atomics into y)
// over the units live for some token (umask != 0), with TT accumulators per
// column per lane; a unit's TT products a' come from a_rm[unit][tp].
template <int PMAX, int TT>
__global__ __launch_bounds__(KD_THREADS) void k_down_tb_i8(const float* __restrict__ a_rm,
                                                           const uint64_t* __restrict__ umask,
                                                           const int8_t* __restrict__ W2T,
                                                           float* __restrict__ y, int D, int H,
                                                           int T, int tp, int splits) {
    constexpr int LPR = 16;
    constexpr int VEC = 16;
    constexpr int CB = LPR * VEC;
    constexpr int RPI = WAVE / LPR;
    constexpr int UF = 4;
    __shared__ float red[TT < 4 ? TT : 4][KD_WAVES][CB];

    const int nslices = (D + CB - 1) / CB;
    const int per_xcd = (nslices + 7) / 8;
    const int bx = blockIdx.x;
    const int slice = (bx & 7) * per_xcd + (bx >> 3);
    if (slice >= nslices) return;
    const int col0 = slice * CB;
    const int hs = (H + splits - 1) / splits;
    const int h0 = blockIdx.y * hs;
    const int h1 = min(H, h0 + hs);
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int sub = lane % LPR, grp = lane / LPR;
    const int col = col0 + sub * VEC;
    const bool col_ok = col < D;
    uint64_t mk[PMAX];
#pragma unroll
    for (int p = 0; p < PMAX; ++p) {
        const int row = h0 + (wave * PMAX + p) * WAVE + lane;
        mk[p] = __ballot(row < h1 && umask[row] != 0ull);
    }

    float acc[TT][VEC];
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int k = 0; k < VEC; ++k) acc[t][k] = 0.0f;

#pragma unroll
    for (int p = 0; p < PMAX; ++p) {
        const int base = h0 + (wave * PMAX + p) * WAVE;
        uint64_t m = mk[p];
        while (m) {
            int bit[UF];
            next_live_bits<RPI, UF>(m, grp, bit);
            u32x4 wv[UF];
            float av[UF][TT];
#pragma unroll
            for (int u = 0; u < UF; ++u) {
                const bool e_ok = bit[u] >= 0;
                const int row = e_ok ? (base + bit[u]) : 0;
                wv[u] = (e_ok && col_ok) ? load_stream(W2T + (size_t)row * D + col)
                                          : u32x4{0u, 0u, 0u, 0u};
                // TT <= 16 <= tp, and padded token slots of a_rm hold 0
                const float* ar = a_rm + (size_t)row * tp;
#pragma unroll
                for (int t = 0; t < TT; t += 2) {
                    const float2 v2 = e_ok ? *reinterpret_cast<const float2*>(ar + t)
                                            : make_float2(0.0f, 0.0f);
                    av[u][t] = v2.x;
                    av[u][t + 1] = v2.y;
                }
            }
#pragma unroll
            for (int u = 0; u < UF; ++u)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t wq = wv[u][q];
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const float wf = (float)((int)(wq << (24 - 8 * b)) >> 24);
#pragma unroll
                        for (int t = 0; t < TT; ++t) acc[t][4 * q + b] = fmaf(av[u][t], wf, acc[t][4 * q + b]);
                    }
                }
        }
    }
    tb_down_epilogue<TT, (TT < 4 ? TT : 4), VEC, LPR, CB>(acc, red, y, D, T, col0, splits, wave, sub, grp);
}

// Small batches (T <= TT <= 4) with group-scaled int4 weights, union of the
// tokens' live sets: as k_gate_up_tb_i8 (RW units per wave), with each pair of codes turned into a
// bf16 pair once (the byte permute of dot32_i4) and met with every token's x
// pair by a bf16 dot2; 136 * sum(x) per token and 32 codes is taken off before
// the group scale. Stores a[unit][tp] = A(z) u (the down pass applies the W2T
// group scales).
template <int NC, int TT, bool DENSE, int RW>
__global__ __launch_bounds__(K1_THREADS) void k_gate_up_tb_i4(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ W1, const float* __restrict__ s1,
    const uint8_t* __restrict__ W3, const float* __restrict__ s3, float* __restrict__ a_rm,
    uint64_t* __restrict__ umask, uint8_t* __restrict__ live_out, float* __restrict__ y_zero,
    int D, int H, int T, int tp, int act) {
    constexpr int CW = WAVE * 32;  // columns of one chunk: 32 codes per lane
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int unit0 = (blockIdx.x * K1_WAVES + wave) * RW;  // RW consecutive units per wave
    const int G = D / I4_GROUP;
    const size_t rb = (size_t)D / 2;
    u32x4 wr[RW][NC];  // every W1 row of the wave, issued first
    float scr[RW][NC];
#pragma unroll
    for (int q = 0; q < RW; ++q)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int col = c * CW + lane * 32;
            const bool ok = unit0 + q < H && col < D;
            wr[q][c] = ok ? load_stream(W1 + (size_t)(unit0 + q) * rb + col / 2) : u32x4{0u, 0u, 0u, 0u};
            scr[q][c] = ok ? s1[(size_t)(unit0 + q) * G + col / I4_GROUP] : 0.0f;
        }
    X32 xv[TT][NC];
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int c = 0; c < NC; ++c)
            xv[t][c] = load_x32(x + (size_t)(t < T ? t : 0) * D, t < T ? c * CW + lane * 32 : D, D);
    if (y_zero) {
        for (int j = blockIdx.x * K1_THREADS + threadIdx.x; j < T * D; j += gridDim.x * K1_THREADS)
            y_zero[j] = 0.0f;
    }
    auto dot_tokens = [&](const u32x4 (&wr)[NC], const float (&scl)[NC], float (&v)[TT]) {
#pragma unroll
        for (int t = 0; t < TT; ++t) v[t] = 0.0f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            float sp[TT];
#pragma unroll
            for (int t = 0; t < TT; ++t) sp[t] = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t wq = wr[c][q] ^ 0x88888888u;
                const uint32_t lo = wq & 0x0F0F0F0Fu;
                const uint32_t hi = (wq >> 4) & 0x0F0F0F0Fu;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const uint32_t sel = (uint32_t)b | (0x0cu << 8) | ((4u + b) << 16) | (0x0cu << 24);
                    const uint32_t pair = __builtin_amdgcn_perm(hi, lo, sel) | 0x43004300u;
#pragma unroll
                    for (int t = 0; t < TT; ++t) {
                        const uint32_t xp = xv[t][c].v[q][b];
                        sp[t] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair),
                                                                __builtin_bit_cast(bf16x2, xp), sp[t], false);
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < TT; ++t) v[t] = fmaf(scl[c], fmaf(-136.0f, xv[t][c].sum, sp[t]), v[t]);
        }
    };
    const int tl = bit_rev<TT>(lane & (TT - 1));  // token whose sums this lane ends with
#pragma unroll
    for (int q = 0; q < RW; ++q) {
        const int unit = unit0 + q;
        if (unit >= H) break;  // wave-uniform
        float v[TT];
        dot_tokens(wr[q], scr[q], v);
        const float z = multi_reduce<TT>(v);
        const bool lv = tl < T && z > 0.0f;
        const uint64_t bl = __ballot(lv && lane < TT);
        uint64_t m = 0;
#pragma unroll
        for (int t = 0; t < TT; ++t) m |= ((bl >> bit_rev<TT>(t)) & 1ull) << t;
        if (lane == 0) umask[unit] = DENSE ? ((1ull << T) - 1) : m;
        if (live_out && lane < TT && tl < T) live_out[(size_t)tl * H + unit] = lv ? 1 : 0;
        if (!DENSE && m == 0) {
            if (lane < TT) a_rm[(size_t)unit * tp + tl] = 0.0f;
            continue;
        }
        u32x4 w[NC];
        float sc[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int col = c * CW + lane * 32;
            const bool ok = col < D;
            w[c] = ok ? load_stream(W3 + (size_t)unit * rb + col / 2) : u32x4{0u, 0u, 0u, 0u};
            sc[c] = ok ? s3[(size_t)unit * G + col / I4_GROUP] : 0.0f;
        }
        dot_tokens(w, sc, v);
        const float u = multi_reduce<TT>(v);
        if (lane < TT) a_rm[(size_t)unit * tp + tl] = tl < T ? activation(act, z) * u : 0.0f;
    }
}

// Down pass of the int4 small batches: 16 lanes x 16 codes (8 bytes) per
// 256-column slice, the group scale of each lane's 16 columns applied to the
// unit's products; otherwise as k_down_tb_i8.
template <int PMAX, int TT>
__global__ __launch_bounds__(KD_THREADS) void k_down_tb_i4(const float* __restrict__ a_rm,
                                                           const uint64_t* __restrict__ umask,
                                                           const uint8_t* __restrict__ W2T,
                                                           const float* __restrict__ s2,
                                                           float* __restrict__ y, int D, int H,
                                                           int T, int tp, int splits) {
    constexpr int LPR = 16;
    constexpr int VEC = 16;
    constexpr int CB = LPR * VEC;
    constexpr int RPI = WAVE / LPR;
    constexpr int UF = 4;
    __shared__ float red[TT < 4 ? TT : 4][KD_WAVES][CB];

    const int nslices = (D + CB - 1) / CB;
    const int per_xcd = (nslices + 7) / 8;
    const int bx = blockIdx.x;
    const int slice = (bx & 7) * per_xcd + (bx >> 3);
    if (slice >= nslices) return;
    const int col0 = slice * CB;
    const int hs = (H + splits - 1) / splits;
    const int h0 = blockIdx.y * hs;
    const int h1 = min(H, h0 + hs);
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int sub = lane % LPR, grp = lane / LPR;
    const int col = col0 + sub * VEC;
    const bool col_ok = col < D;
    const int G = D / I4_GROUP;
    const size_t rb = (size_t)D / 2;
    uint64_t mk[PMAX];
#pragma unroll
    for (int p = 0; p < PMAX; ++p) {
        const int row = h0 + (wave * PMAX + p) * WAVE + lane;
        mk[p] = __ballot(row < h1 && umask[row] != 0ull);
    }

    float acc[TT][VEC];
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int k = 0; k < VEC; ++k) acc[t][k] = 0.0f;

#pragma unroll
    for (int p = 0; p < PMAX; ++p) {
        const int base = h0 + (wave * PMAX + p) * WAVE;
        uint64_t m = mk[p];
        while (m) {
            int bit[UF];
            next_live_bits<RPI, UF>(m, grp, bit);
            u32x2 wv[UF];
            float av[UF][TT];
#pragma unroll
            for (int u = 0; u < UF; ++u) {
                const bool e_ok = bit[u] >= 0;
                const bool ok = e_ok && col_ok;
                const int row = e_ok ? (base + bit[u]) : 0;
                wv[u] = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(W2T + (size_t)row * rb + col / 2))
                           : u32x2{0u, 0u};
                const float sg = ok ? s2[(size_t)row * G + col / I4_GROUP] : 0.0f;
                // TT <= 16 <= tp, and padded token slots of a_rm hold 0
                const float* ar = a_rm + (size_t)row * tp;
#pragma unroll
                for (int t = 0; t < TT; t += 2) {
                    const float2 v2 = e_ok ? *reinterpret_cast<const float2*>(ar + t)
                                            : make_float2(0.0f, 0.0f);
                    av[u][t] = v2.x * sg;
                    av[u][t + 1] = v2.y * sg;
                }
            }
#pragma unroll
            for (int u = 0; u < UF; ++u)
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const uint32_t wq = wv[u][q];
#pragma unroll
                    for (int b = 0; b < 8; ++b) {
                        const float wf = (float)((int)(wq << (28 - 4 * b)) >> 28);  // nibble b, signed
#pragma unroll
                        for (int t = 0; t < TT; ++t) acc[t][8 * q + b] = fmaf(av[u][t], wf, acc[t][8 * q + b]);
                    }
                }
        }
    }
    tb_down_epilogue<TT, (TT < 4 ? TT : 4), VEC, LPR, CB>(acc, red, y, D, T, col0, splits, wave, sub, grp);
}

// Quantised LoPA, union of 2..4 tokens. Helpers: one decode of a weight piece
// against the TT tokens' x (as dot16_i8x and dot32_i4 for one token).
template <int TT>
__device__ inline void dot16_i8x_tt(const u32x4& w, const X16 (&xv)[TT], float (&v)[TT]) {
    float sp[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) sp[t] = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t wq = w[q] ^ 0x80808080u;
        const uint32_t f0 = __float_as_uint((float)(wq & 0xffu));
        const uint32_t f1 = __float_as_uint((float)((wq >> 8) & 0xffu));
        const uint32_t f2 = __float_as_uint((float)((wq >> 16) & 0xffu));
        const uint32_t f3 = __float_as_uint((float)(wq >> 24));
        const uint32_t p01 = __builtin_amdgcn_perm(f1, f0, 0x07060302u);
        const uint32_t p23 = __builtin_amdgcn_perm(f3, f2, 0x07060302u);
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            const u32x4 xq = xv[t].v[q >> 1];
            const uint32_t x01 = xq[2 * (q & 1)], x23 = xq[2 * (q & 1) + 1];
            sp[t] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p01),
                                                    __builtin_bit_cast(bf16x2, x01), sp[t], false);
            sp[t] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p23),
                                                    __builtin_bit_cast(bf16x2, x23), sp[t], false);
        }
    }
#pragma unroll
    for (int t = 0; t < TT; ++t) v[t] += fmaf(-128.0f, xv[t].sum, sp[t]);
}

template <int TT>
__device__ inline void dot32_i4_tt(const u32x4& w, const X32 (&xv)[TT], float scale, float (&v)[TT]) {
    float sp[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) sp[t] = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t wq = w[q] ^ 0x88888888u;
        const uint32_t lo = wq & 0x0F0F0F0Fu;
        const uint32_t hi = (wq >> 4) & 0x0F0F0F0Fu;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint32_t sel = (uint32_t)b | (0x0cu << 8) | ((4u + b) << 16) | (0x0cu << 24);
            const uint32_t pair = __builtin_amdgcn_perm(hi, lo, sel) | 0x43004300u;
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                const uint32_t xp = xv[t].v[q][b];
                sp[t] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair),
                                                        __builtin_bit_cast(bf16x2, xp), sp[t], false);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < TT; ++t) v[t] = fmaf(scale, fmaf(-136.0f, xv[t].sum, sp[t]), v[t]);
}

// Rank projection of the quantised LoPA batches: t[token][m] = sV_m (qV_m . x),
// one int8 V row per wave, each weight decoded once for the TT tokens; the
// block stages x of the batch in LDS (dynamic, T D bf16) once for its four
// waves. Writes t_out [T x r]; y_zero (nullable): T x D floats cleared for the
// down pass.
template <int NC, int TT>
__global__ __launch_bounds__(K1_THREADS) void k_rank_proj_tb_i8(
    const uint16_t* __restrict__ x, const int8_t* __restrict__ V, const float* __restrict__ sV,
    float* __restrict__ t_out, float* __restrict__ y_zero, int D, int r, int T) {
    constexpr int CW = WAVE * 16;
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int m = blockIdx.x * K1_WAVES + wave;
    const bool in = m < r;
    extern __shared__ uint16_t xrk[];  // [T][D]
    u32x4 w[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int col = c * CW + lane * 16;
        w[c] = (in && col < D) ? load_stream(V + (size_t)m * D + col) : u32x4{0u, 0u, 0u, 0u};
    }
    for (int j = threadIdx.x; j < T * D / 8; j += K1_THREADS)
        reinterpret_cast<u32x4*>(xrk)[j] = load_cached(x + 8 * (size_t)j);
    __syncthreads();
    X16 xv[NC][TT];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int col = c * CW + lane * 16;
#pragma unroll
        for (int t = 0; t < TT; ++t)
            xv[c][t] = load_x16(xrk + (t < T ? t : 0) * D, t < T ? col : D, D);
    }
    if (y_zero) {
        for (int j = blockIdx.x * K1_THREADS + threadIdx.x; j < T * D; j += gridDim.x * K1_THREADS)
            y_zero[j] = 0.0f;
    }
    float v[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) v[t] = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) dot16_i8x_tt<TT>(w[c], xv[c], v);
    const float tm = multi_reduce<TT>(v) * (in ? sV[m] : 0.0f);
    const int tl = bit_rev<TT>(lane & (TT - 1));
    if (in && lane < TT && tl < T) t_out[(size_t)tl * r + m] = tm;
}

// LoPA gate of the quantised batches and the up projection over the union:
// four units per wave, 16 lanes per int8 U row (pieces of 256 B: the first
// KLQ_NRU issued with the x loads at the start, any further ones in a loop);
// the T rank vectors t (fp32) and x of the batch (bf16) are staged in LDS by
// the block (dynamic LDS of T r floats, then T D bf16). z for each token against its t, through RMSNorm when asked, plus
// (G x)_i when asked. Then each unit of the wave live for some token takes the
// whole wave for its W3 row (int8 with a row scale, BITS = 8, or int4 with group
// scales, BITS = 4), every weight decoded once for the TT tokens; the next live
// unit's row is loaded while the current one is reduced. Stores
// a[unit][tp] = A(z_t) g(u_t) (times the W2T row scale for int8), 0 for dead
// pairs and padded slots, the token mask and live flags when asked.
constexpr int KLQ_NRU = 2;  // U pieces of 256 B loaded up front (r <= 512)
template <int NC, int TT, int BITS>
__global__ __launch_bounds__(K1_THREADS) void k_gate_up_lopa_tb_q(
    const uint16_t* __restrict__ x, const float* __restrict__ t_in, const int8_t* __restrict__ U,
    const float* __restrict__ sU, const uint8_t* __restrict__ W3, const float* __restrict__ s3,
    const float* __restrict__ s2, float* __restrict__ a_rm, uint64_t* __restrict__ umask,
    uint8_t* __restrict__ live_out, int D, int H, int r, int T, int tp, int act, unsigned flags) {
    static_assert(BITS == 8 || BITS == 4, "int8 or int4 W3 rows");
    constexpr int VPL = BITS == 8 ? 16 : 32;  // W3 columns per lane and chunk
    constexpr int CW = WAVE * VPL;
    extern __shared__ float ts[];  // [T][r]
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int sub = lane & 15, grp = lane >> 4;
    const int base = (blockIdx.x * K1_WAVES + wave) * KLQ_UPW;
    const int unit = base + grp;
    const bool in = unit < H;
    const int nr = (r + 255) / 256;
    u32x4 u[KLQ_NRU];
#pragma unroll
    for (int c = 0; c < KLQ_NRU; ++c) {
        const int col = c * 256 + sub * 16;
        u[c] = (in && col < r) ? load_stream(U + (size_t)unit * r + col) : u32x4{0u, 0u, 0u, 0u};
    }
    uint16_t* xq = reinterpret_cast<uint16_t*>(ts + T * r);  // [T][D]
    for (int j = threadIdx.x; j < T * r / 4; j += K1_THREADS)
        reinterpret_cast<float4*>(ts)[j] = reinterpret_cast<const float4*>(t_in)[j];
    for (int j = threadIdx.x; j < T * D / 8; j += K1_THREADS)
        reinterpret_cast<u32x4*>(xq)[j] = load_cached(x + 8 * (size_t)j);
    __syncthreads();
    using XT = typename std::conditional<BITS == 8, X16, X32>::type;
    XT xv[NC][TT];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int col = c * CW + lane * VPL;
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            const uint16_t* xr = xq + (t < T ? t : 0) * D;
            if constexpr (BITS == 8) xv[c][t] = load_x16(xr, t < T ? col : D, D);
            else xv[c][t] = load_x32(xr, t < T ? col : D, D);
        }
    }
    const float su_ = in ? sU[unit] : 0.0f;
    float sz[TT], ss[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) sz[t] = ss[t] = 0.0f;
    const bool rms = (flags & LOPA_RMSNORM) != 0;
    auto piece = [&](const u32x4& uw, int col) {  // one U piece, decoded once, against every token's t
        float uf[16];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int b = 0; b < 4; ++b) uf[4 * q + b] = (float)((int)(uw[q] << (24 - 8 * b)) >> 24);
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            if (t >= T) continue;
            float tv[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 a = *reinterpret_cast<const float4*>(ts + t * r + col + 4 * q);
                tv[4 * q] = a.x; tv[4 * q + 1] = a.y; tv[4 * q + 2] = a.z; tv[4 * q + 3] = a.w;
            }
            if (rms) {
#pragma unroll
                for (int k = 0; k < 16; ++k) ss[t] = fmaf(tv[k], tv[k], ss[t]);
            }
#pragma unroll
            for (int k = 0; k < 16; ++k) sz[t] = fmaf(uf[k], tv[k], sz[t]);
        }
    };
#pragma unroll
    for (int c = 0; c < KLQ_NRU; ++c) {
        const int col = c * 256 + sub * 16;
        if (col < r) piece(u[c], col);
    }
    for (int c = KLQ_NRU; c < nr; ++c) {
        const int col = c * 256 + sub * 16;
        if (col < r) piece(in ? load_stream(U + (size_t)unit * r + col) : u32x4{0u, 0u, 0u, 0u}, col);
    }
    float z[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        float inv = 1.0f;  // RMSNorm of the token's t: every lane group sees all of it
        if (rms) inv = 1.0f / sqrtf(group16_sum(ss[t]) / (float)r + RMS_EPS);
        const float gx = ((flags & LOPA_G_TILED) && in && t < T)
                             ? Elem<uint16_t>::get1(x[(size_t)t * D + unit % D]) : 0.0f;
        z[t] = group16_sum(sz[t]) * su_ * inv + gx;
    }
    uint32_t mb = 0;
#pragma unroll
    for (int t = 0; t < TT; ++t) mb |= (in && t < T && z[t] > 0.0f) ? (1u << t) : 0u;
    if (in && sub == 0) {
        umask[unit] = mb;
        if (live_out) {
#pragma unroll
            for (int t = 0; t < TT; ++t)
                if (t < T) live_out[(size_t)t * H + unit] = (mb >> t) & 1u;
        }
        if (mb == 0) {
#pragma unroll
            for (int t = 0; t < TT; ++t) a_rm[(size_t)unit * tp + t] = 0.0f;
        }
    }
    uint64_t m = __ballot(in && sub == 0 && mb != 0);
    if (m == 0) return;  // wave-uniform
    const int tl = bit_rev<TT>(lane & (TT - 1));
    const int G = D / I4_GROUP;
    const size_t rb = BITS == 8 ? (size_t)D : (size_t)D / 2;  // bytes per W3 row
    auto load_row = [&](int ul, u32x4 (&w3)[NC], float (&sc)[NC]) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int col = c * CW + lane * VPL;
            const bool ok = col < D;
            w3[c] = ok ? load_stream(W3 + (size_t)ul * rb + (BITS == 8 ? col : col / 2)) : u32x4{0u, 0u, 0u, 0u};
            sc[c] = (BITS == 4 && ok) ? s3[(size_t)ul * G + col / I4_GROUP] : 0.0f;
        }
    };
    int g = __builtin_ctzll(m) >> 4;
    m &= m - 1;
    u32x4 w3[NC];
    float sc[NC];
    load_row(base + g, w3, sc);
    while (true) {
        const bool more = m != 0;  // wave-uniform
        const int gn = more ? (__builtin_ctzll(m) >> 4) : g;
        u32x4 w3n[NC];
        float scn[NC];
        if (more) load_row(base + gn, w3n, scn);
        const int ul = base + g;
        float zt = 0.0f;  // z of unit ul for this lane's token tl
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            const float zv = __shfl(z[t], 16 * g);
            if (t == tl) zt = zv;
        }
        float v[TT];
#pragma unroll
        for (int t = 0; t < TT; ++t) v[t] = 0.0f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            if constexpr (BITS == 8) dot16_i8x_tt<TT>(w3[c], xv[c], v);
            else dot32_i4_tt<TT>(w3[c], xv[c], sc[c], v);
        }
        float uu = multi_reduce<TT>(v);
        if (BITS == 8) uu *= s3[ul];
        const float g3 = (flags & LOPA_DOUBLE_ACT) ? activation(act, uu) : uu;
        const float post = BITS == 8 ? s2[ul] : 1.0f;
        if (lane < TT) a_rm[(size_t)ul * tp + tl] = tl < T ? activation(act, zt) * g3 * post : 0.0f;
        if (!more) break;
        m &= m - 1;
        g = gn;
#pragma unroll
        for (int c = 0; c < NC; ++c) { w3[c] = w3n[c]; sc[c] = scn[c]; }
    }
}

// ---------------------------------------------------------------------------
// Sparse expert FFNs in a top-K mixture of experts (page "Model casting:
// compute the gate, then skip most of the FFN", section "Where it
// generalizes": the same gate-first skip applied to each expert's FFN). The
// tokens routed to one expert are gathered into a contiguous batch, the
// expert's FFN runs on it, and y_t = sum_k gate_{t,k} * y_slot(t,k) in k order.
// The routing tables travel by value in the kernel arguments.
constexpr int MOE_MAX_SLOTS = 128;  // T * K <= 64 * 2
struct MoeGather { int16_t src[MOE_MAX_SLOTS]; };                 // token of each slot
struct MoeCombine { int16_t slot[MOE_MAX_SLOTS]; float gate[MOE_MAX_SLOTS]; };  // [t * K + k]

// x_g[slot] = x[src[slot]]: one block per slot, 16-byte copies
__global__ __launch_bounds__(256) void k_moe_gather(const uint16_t* __restrict__ x,
                                                    uint16_t* __restrict__ x_g, int D,
                                                    MoeGather g) {
    const int slot = blockIdx.x;
    const u32x4* src = reinterpret_cast<const u32x4*>(x + (size_t)g.src[slot] * D);
    u32x4* dst = reinterpret_cast<u32x4*>(x_g + (size_t)slot * D);
    for (int i = threadIdx.x; i < D / 8; i += 256) dst[i] = src[i];
}

// y[t] = sum_k gate[t, k] * y_g[slot[t, k]], k ascending: one block per token
__global__ __launch_bounds__(256) void k_moe_combine(const float* __restrict__ y_g,
                                                     float* __restrict__ y, int D, int K,
                                                     MoeCombine c) {
    const int t = blockIdx.x;
    for (int j = threadIdx.x; j < D; j += 256) {
        float acc = 0.0f;
        for (int k = 0; k < K; ++k)
            acc = fmaf(c.gate[t * K + k], y_g[(size_t)c.slot[t * K + k] * D + j], acc);
        y[(size_t)t * D + j] = acc;
    }
}

// ---------------------------------------------------------------------------
// Large batches (prefill, T > 64): the FFN as three MFMA contractions. At this
// size the union of the tokens' live sets covers nearly every unit (1 - s^T),
// so the gate and the up projection run as one GEMM over all units, and the
// down projection is a GEMM whose reduction runs over the gathered list of
// units that are live for some token (the page on model casting notes in
// "Checking the three claims" that batching erodes the skip).
//
//   k_gate_up_gemm  z = X W1^T and u = X W3^T for a tile of 256 tokens x 128
//                   units (both weight rows of each unit in the tile), then
//                   a = A(z) * u rounded to bf16, stored unit-major
//                   a_um[unit][token], and a 64-bit mask of the tile's units
//                   that are live for some token of the tile.
//   k_union_list    ascending list of the units live for some token.
//   k_down_gemm     y = a W2 over the listed units: 128 tokens x 128 columns
//                   per block, split over unit ranges when the tiles alone do
//                   not fill the chip (fp32 atomics then; y cleared by the gate).
//
// Operands go from global memory straight into LDS rings (global_load_lds,
// 16 B per lane). The gate kernel's operands are K-contiguous rows (X, W1,
// W3), read as MFMA fragments with 16-byte LDS reads. The down kernel stages
// K-rows of both operands (a_um rows of 128 tokens and W2T rows of 128
// columns, one row per listed unit) and reads the fragments with the
// transposing LDS read (frag_tr, as the batched down kernel).

// Gate/up tile: TM tokens x UN units, one wave per 64 x 64 sub-tile (z and u).
template <int TM, int UN>
struct GemmTile {
    static_assert(TM % 64 == 0 && UN % 64 == 0, "64 x 64 wave tiles");
    static constexpr int WAVES = (TM / 64) * (UN / 64);
    static constexpr int THREADS = WAVES * WAVE;
    static constexpr int KC = 32;                 // columns per chunk: rows of 64 B
    static constexpr int ROWS = TM + 2 * UN;      // staged rows: X, then W1, then W3
    static constexpr int STAGE = ROWS * 64;
    static constexpr int NS = 4;                  // LDS stages
    static constexpr int IPW = STAGE / 1024 / WAVES;  // wave load instructions per wave per chunk
    static_assert(STAGE % (1024 * WAVES) == 0, "whole wave loads per wave");
    static_assert(NS * STAGE <= 131072, "LDS ring");
};
constexpr int KG_UN_MIN = 64;  // the smallest unit tile (masks of the union list are per 64 units)

// Slot of 16-byte piece p in staged 64-byte row r. A fragment read takes one
// piece of 16 consecutive rows; measured with the LDS bank-conflict counter on
// gfx950, p ^ ((r >> 1) & 3) reads them without conflicts, while p ^ ((r >> 2) & 3),
// p ^ (r & 3) and no swizzle cost 4 extra cycles per read.
__device__ inline int swz64(int r, int p) { return p ^ ((r >> 1) & 3); }

// Map a linear block id to a work item so that each XCD (block id mod 8)
// receives a contiguous range of work items.
__device__ inline int xcd_work_item(int b, int nblocks) {
    const int x = b & 7, j = b >> 3;
    const int per = nblocks >> 3, rem = nblocks & 7;
    return x * per + (x < rem ? x : rem) + j;
}

template <int TM, int UN, bool DENSE>
__global__ __launch_bounds__((TM / 64) * (UN / 64) * WAVE) void k_gate_up_gemm(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W1,
    const uint16_t* __restrict__ W3, const uint16_t* __restrict__ zeros,
    uint16_t* __restrict__ a_um, uint64_t* __restrict__ any_out, uint8_t* __restrict__ live_out,
    float* __restrict__ y_zero, int D, int H, int T, int TP, int act) {
    using G = GemmTile<TM, UN>;
    constexpr int KG_TM = TM, KG_UN = UN, KG_KC = G::KC, KG_NS = G::NS, KG_IPW = G::IPW;
    constexpr int KG_STAGE = G::STAGE, KG_THREADS = G::THREADS;
    __shared__ __attribute__((aligned(16))) uint8_t ring[KG_NS * KG_STAGE];
    __shared__ uint32_t umask[KG_UN / 16];
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int r16 = lane & 15, g = lane >> 4;
    const int tw = wave % (TM / 64), uw = wave / (TM / 64);  // wave tile: tokens 64 tw .., units 64 uw ..
    const int ntt = (T + KG_TM - 1) / KG_TM;
    const int nut = (H + KG_UN - 1) / KG_UN;
    const int wi = xcd_work_item(blockIdx.x, nut * ntt);
    const int ut0 = wi / ntt, tt0 = wi % ntt;
    const int u0 = ut0 * KG_UN, tok0 = tt0 * KG_TM;

    if (y_zero) {
        for (size_t j = (size_t)blockIdx.x * KG_THREADS + threadIdx.x; j < (size_t)T * D;
             j += (size_t)gridDim.x * KG_THREADS)
            y_zero[j] = 0.0f;
    }
    if (threadIdx.x < KG_UN / 16) umask[threadIdx.x] = 0u;

    // sources of this lane's pieces: row and piece are the same for every chunk
    const uint16_t* src[KG_IPW];
    bool rok[KG_IPW];
    int pcol[KG_IPW];
#pragma unroll
    for (int i = 0; i < KG_IPW; ++i) {
        const int r = 16 * (wave * KG_IPW + i) + (lane >> 2);
        const int p = swz64(r, lane & 3);
        pcol[i] = 8 * p;
        if (r < KG_TM) {
            const int t = tok0 + r;
            rok[i] = t < T;
            src[i] = x + (rok[i] ? (size_t)t * D + 8 * p : 0);
        } else {
            const int u = u0 + (r - KG_TM) % KG_UN;
            const uint16_t* W = (r < KG_TM + KG_UN) ? W1 : W3;
            rok[i] = u < H;
            src[i] = W + (rok[i] ? (size_t)u * D + 8 * p : 0);
        }
    }
    auto issue = [&](int stage, int c) {
#pragma unroll
        for (int i = 0; i < KG_IPW; ++i) {
            const bool ok = rok[i] && c * KG_KC + pcol[i] < D;
            const uint16_t* gp = ok ? src[i] + (size_t)c * KG_KC : zeros;
            load_lds16(gp, ring + stage * KG_STAGE + 1024 * (wave * KG_IPW + i));
        }
    };

    f32x4 accz[4][4], accu[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            accz[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
            accu[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    auto compute = [&](int stage) {
        const uint8_t* st = ring + stage * KG_STAGE;
        u32x4 xf[4], w1f[4], w3f[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rx = 64 * tw + 16 * i + r16;
            const int r1 = KG_TM + 64 * uw + 16 * i + r16;
            const int r3 = KG_TM + KG_UN + 64 * uw + 16 * i + r16;
            xf[i] = *reinterpret_cast<const u32x4*>(st + rx * 64 + 16 * swz64(rx, g));
            w1f[i] = *reinterpret_cast<const u32x4*>(st + r1 * 64 + 16 * swz64(r1, g));
            w3f[i] = *reinterpret_cast<const u32x4*>(st + r3 * 64 + 16 * swz64(r3, g));
        }
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                accz[a][b] = mfma_bf16(xf[a], w1f[b], accz[a][b]);
                accu[a][b] = mfma_bf16(xf[a], w3f[b], accu[a][b]);
            }
    };

    const int nchunks = (D + KG_KC - 1) / KG_KC;
#pragma unroll
    for (int d = 0; d < KG_NS - 1; ++d) issue(d, d);
    const int niter = (nchunks + KG_NS - 1) / KG_NS * KG_NS;
    for (int c0 = 0; c0 < niter; c0 += KG_NS) {
#pragma unroll
        for (int d = 0; d < KG_NS; ++d) {
            const int c = c0 + d;
            wait_vmcnt((KG_NS - 2) * KG_IPW);  // this wave's pieces of chunk c have landed
            __syncthreads();                     // ... and every wave's; chunk c - 1 is consumed
            issue((d + KG_NS - 1) % KG_NS, c + KG_NS - 1);
            if (c < nchunks) compute(d);
        }
    }
    wait_vmcnt(0);

    // epilogue: lane holds tokens 4g + j of each token tile, unit r16 of each unit tile
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int u = u0 + 64 * uw + 16 * b + r16;
        bool any = false;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int t0 = tok0 + 64 * tw + 16 * a + 4 * g;
            uint32_t packed[2];
#pragma unroll
            for (int j = 0; j < 4; j += 2) {
                const float z0 = accz[a][b][j], z1 = accz[a][b][j + 1];
                const float v0 = activation(act, z0) * accu[a][b][j];
                const float v1 = activation(act, z1) * accu[a][b][j + 1];
                packed[j / 2] = bf16_rne(v0) | (bf16_rne(v1) << 16);
                any |= (t0 + j < T && z0 > 0.0f) || (t0 + j + 1 < T && z1 > 0.0f);
            }
            if (u < H && t0 < TP)
                *reinterpret_cast<uint2*>(a_um + (size_t)u * TP + t0) = uint2{packed[0], packed[1]};
            if (live_out && u < H) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (t0 + j < T) live_out[(size_t)(t0 + j) * H + u] = accz[a][b][j] > 0.0f ? 1 : 0;
            }
        }
        if (!DENSE) {
            const uint64_t m = __ballot(any);
            const uint32_t m16 = (uint32_t)((m | (m >> 16) | (m >> 32) | (m >> 48)) & 0xFFFFull);
            if (lane == 0 && m16) atomicOr(&umask[4 * uw + b], m16);
        }
    }
    if (!DENSE) {
        // one 64-bit mask per 64 units: [token tile][64-unit tile]
        __syncthreads();
        constexpr int NM = KG_UN / 64;
        if (threadIdx.x < NM)
            any_out[((size_t)tt0 * nut + ut0) * NM + threadIdx.x] =
                (uint64_t)umask[4 * threadIdx.x] | ((uint64_t)umask[4 * threadIdx.x + 1] << 16) |
                ((uint64_t)umask[4 * threadIdx.x + 2] << 32) |
                ((uint64_t)umask[4 * threadIdx.x + 3] << 48);
    }
}

// Ascending list of the units live for some token, from the masks of every
// (token tile, unit tile): one block; each thread ORs one unit tile's masks over
// the token tiles, a block scan of the popcounts places its units.
__global__ __launch_bounds__(1024) void k_union_list(const uint64_t* __restrict__ any, int ntt,
                                                     int nut, int32_t* __restrict__ list,
                                                     int32_t* __restrict__ count) {
    __shared__ int wsum[16];
    __shared__ int base_s;
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    if (threadIdx.x == 0) base_s = 0;
    __syncthreads();
    for (int j0 = 0; j0 < nut; j0 += 1024) {
        const int j = j0 + threadIdx.x;
        uint64_t m = 0;
        if (j < nut) {
            int t = 0;
            for (; t + 4 <= ntt; t += 4) {
                const uint64_t a0 = any[(size_t)t * nut + j], a1 = any[(size_t)(t + 1) * nut + j];
                const uint64_t a2 = any[(size_t)(t + 2) * nut + j], a3 = any[(size_t)(t + 3) * nut + j];
                m |= a0 | a1 | a2 | a3;
            }
            for (; t < ntt; ++t) m |= any[(size_t)t * nut + j];
        }
        const int c = __popcll(m);
        // inclusive scan of c within the wave
        int incl = c;
#pragma unroll
        for (int d = 1; d < WAVE; d <<= 1) {
            const int v = __shfl_up(incl, d);
            if (lane >= d) incl += v;
        }
        if (lane == WAVE - 1) wsum[wave] = incl;
        __syncthreads();
        int off = base_s, tot = 0;
        for (int w = 0; w < 16; ++w) {
            if (w < wave) off += wsum[w];
            tot += wsum[w];
        }
        off += incl - c;
        while (m) {
            const int b = __builtin_ctzll(m);
            list[off++] = 64 * j + b;
            m &= m - 1;
        }
        __syncthreads();
        if (threadIdx.x == 0) base_s += tot;
        __syncthreads();
    }
    if (threadIdx.x == 0) *count = base_s;
}

constexpr int KDG_THREADS = 256;
constexpr int KDG_TM = 128;                 // tokens per down block
constexpr int KDG_NB = 128;                 // columns per down block
constexpr int KDG_KC = 32;                  // listed units per chunk
constexpr int KDG_STAGE = 2 * KDG_KC * 256; // a_um rows, then W2T rows: 16 KB
constexpr int KDG_NS = 4;
constexpr int KDG_SEG = 256;                  // list entries per staged segment (one wave load)
constexpr int KDG_SEG_CH = KDG_SEG / KDG_KC;  // chunks per segment
constexpr int KDG_IPW = KDG_STAGE / 1024 / 4;

// y[T x D] (+)= sum over listed units k of a_um[k][t] W2T[k][:]. list == nullptr:
// every unit 0..H-1. Grid: (token tiles x column tiles) x splits, XCD-contiguous.
__global__ __launch_bounds__(KDG_THREADS) void k_down_gemm(
    const uint16_t* __restrict__ a_um, const int32_t* __restrict__ list,
    const int32_t* __restrict__ count_ptr, const uint16_t* __restrict__ W2T,
    const uint16_t* __restrict__ zeros, float* __restrict__ y, int D, int H, int T, int TP,
    int splits) {
    __shared__ __attribute__((aligned(16))) uint8_t ring[KDG_NS * KDG_STAGE];
    __shared__ __attribute__((aligned(16))) int32_t lseg[2][KDG_SEG];
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int r16 = lane & 15, g = lane >> 4;
    const int nmt = (T + KDG_TM - 1) / KDG_TM;
    const int nnt = (D + KDG_NB - 1) / KDG_NB;
    const int wi = xcd_work_item(blockIdx.x, nmt * nnt * splits);
    const int mt = wi % nmt, rest = wi / nmt;
    const int nt = rest % nnt, split = rest / nnt;
    const int tok0 = mt * KDG_TM, col0 = nt * KDG_NB;
    const int count = list ? *count_ptr : H;
    const int nch_all = (count + KDG_KC - 1) / KDG_KC;
    const int per = (nch_all + splits - 1) / splits;
    const int cbeg = split * per;
    const int cend = min(nch_all, cbeg + per);
    const int nchunks = cend > cbeg ? cend - cbeg : 0;

    // Waves 0 and 1 stage the a_um rows of the chunk (rows 0-15 and 16-31),
    // waves 2 and 3 the W2T rows; instruction i of a wave covers rows 4i .. 4i + 3
    // of its 16, lane l row 4i + l / 16. The unit indices come from the list in
    // segments of 256 entries (8 chunks) that wave 0 stages into LDS through the
    // same ordered loads, one segment ahead: segment s is issued together with
    // the pieces of chunk 8 (s - 1), so the wait that marks chunk 8s - NS + 1 as
    // landed (before chunk 8s is issued) also covers it.
    static_assert(KDG_IPW == 4 && KDG_KC == 32, "staging plan: 4 waves x 4 instructions");
    static_assert(KDG_NS <= KDG_SEG_CH + 1, "list segments must land before they are read");
    const int wave_u = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool stage_a = wave_u < 2;
    const int rhalf = 16 * (wave_u & 1);
    int pof[KDG_IPW];
    bool cok[KDG_IPW];
#pragma unroll
    for (int i = 0; i < KDG_IPW; ++i) {
        const int r = rhalf + 4 * i + g;
        pof[i] = 8 * swz256(r, lane & 15);
        cok[i] = stage_a || col0 + pof[i] < D;
    }
    const uint16_t* base = stage_a ? a_um + tok0 : W2T + col0;
    const size_t rstride = stage_a ? (size_t)TP : (size_t)D;
    auto issue_seg = [&](int sg) {
        if (!list || wave_u != 0) return;
        const int pos = (cbeg + KDG_SEG_CH * sg) * KDG_KC + 4 * lane;
        const bool ok = KDG_SEG_CH * sg < nchunks && pos < count;
        load_lds16(ok ? (const void*)(list + pos) : (const void*)zeros, &lseg[sg & 1][0]);
    };
    auto issue = [&](int stage, int c) {
        if (c % KDG_SEG_CH == 0) issue_seg(c / KDG_SEG_CH + 1);
        const int k0 = (cbeg + c) * KDG_KC + rhalf;
        const int* seg = &lseg[(c / KDG_SEG_CH) & 1][(c % KDG_SEG_CH) * KDG_KC + rhalf];
#pragma unroll
        for (int i = 0; i < KDG_IPW; ++i) {
            const int k = k0 + 4 * i + g;
            const bool ok = c < nchunks && k < count && cok[i];
            const int unit = list ? seg[4 * i + g] : k;
            const uint16_t* gp = ok ? base + (size_t)unit * rstride + pof[i] : zeros;
            load_lds16(gp, ring + stage * KDG_STAGE + 1024 * (wave_u * KDG_IPW + i));
        }
    };

    // wave tile: tokens 64 (wave / 2) .. + 64, columns 64 (wave % 2) .. + 64
    const int wt0 = 64 * (wave >> 1), wc0 = 64 * (wave & 1);
    f32x4 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](int stage) {
        const uint8_t* pa = ring + stage * KDG_STAGE;
        const uint8_t* pb = pa + KDG_KC * 256;
        u32x4 af[4], bfr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            af[i] = frag_tr(pa, wt0 + 16 * i, lane);
            bfr[i] = frag_tr(pb, wc0 + 16 * i, lane);
        }
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[a][b] = mfma_bf16(af[a], bfr[b], acc[a][b]);
    };

    issue_seg(0);
    wait_vmcnt(0);
    __syncthreads();
#pragma unroll
    for (int d = 0; d < KDG_NS - 1; ++d) issue(d, d);
    const int niter = (nchunks + KDG_NS - 1) / KDG_NS * KDG_NS;
    for (int c0 = 0; c0 < niter; c0 += KDG_NS) {
#pragma unroll
        for (int d = 0; d < KDG_NS; ++d) {
            const int c = c0 + d;
            wait_vmcnt((KDG_NS - 2) * KDG_IPW);
            __syncthreads();
            issue((d + KDG_NS - 1) % KDG_NS, c + KDG_NS - 1);
            if (c < nchunks) compute(d);
        }
    }
    wait_vmcnt(0);
    if (nchunks == 0 && splits > 1) return;  // nothing to add
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int n = col0 + wc0 + 16 * b + r16;
            if (n >= D) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = tok0 + wt0 + 16 * a + 4 * g + j;
                if (t >= T) continue;
                if (splits > 1)
                    atomicAdd(y + (size_t)t * D + n, acc[a][b][j]);
                else
                    y[(size_t)t * D + n] = acc[a][b][j];
            }
        }
    }
}

// Ascending live lists from the live flags: one block per token.
__global__ __launch_bounds__(1024) void k_live_list(const uint8_t* __restrict__ live, int H,
                                                    int32_t* __restrict__ count,
                                                    int32_t* __restrict__ idx) {
    __shared__ int wc[16];
    __shared__ int base_s;
    const int t = blockIdx.x;
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    if (threadIdx.x == 0) base_s = 0;
    __syncthreads();
    for (int i0 = 0; i0 < H; i0 += 1024) {
        const int i = i0 + threadIdx.x;
        const bool l = i < H && live[(size_t)t * H + i] != 0;
        const uint64_t m = __ballot(l);
        if (lane == 0) wc[wave] = __popcll(m);
        __syncthreads();
        int off = base_s, tot = 0;
        for (int w = 0; w < 16; ++w) {
            if (w < wave) off += wc[w];
            tot += wc[w];
        }
        if (l)
            idx[(size_t)t * H + off +
                __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0))] = i;
        __syncthreads();
        if (threadIdx.x == 0) base_s += tot;
        __syncthreads();
    }
    if (threadIdx.x == 0) count[t] = base_s;
}

}  // namespace sffn
