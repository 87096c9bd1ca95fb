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
    static constexpr int VEC = 8;  // elements per 16-byte load
    __device__ static inline float get(const u32x4& v, int k) {
        uint32_t w = v[k >> 1];
        return (k & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
    }
};
template <> struct Elem<float> {
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
                               int row0, int nrows, int D, int H, int T, int act, int union_mode) {
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
            if (lane == 0) a_out[(size_t)t * H + row] = h * u;
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
                           H, T, act, union_mode);
}

// LoPA gate: z = U t with t = V x in fp32 (t_in [T x r]), then compact_and_up.
// NR = register chunks of a U row (r <= NR * 64 * VEC).
template <typename WT, int NC, int NR>
__global__ __launch_bounds__(K1_THREADS) void k_gate_up_lopa(
    const WT* __restrict__ x, const float* __restrict__ t_in, const WT* __restrict__ U,
    const WT* __restrict__ W3, float* __restrict__ a_out, uint8_t* __restrict__ live_out, int D,
    int H, int r, int T, int act, int union_mode, int rows_per_wave) {
    __shared__ float z_lds[MAXT * K1_MAX_ROWS];
    __shared__ uint32_t list[MAXT * K1_MAX_ROWS];
    __shared__ uint64_t masks[K1_MAX_ROWS];
    __shared__ int n_list;
    constexpr int VEC = Elem<WT>::VEC;
    constexpr int CW = WAVE * VEC;
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int rows_per_block = rows_per_wave * K1_WAVES;
    const int row0 = blockIdx.x * rows_per_block;
    const int nrows = min(rows_per_block, H - row0);

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
            sa = wave_sum(sa);
            sb = wave_sum(sb);
            if (lane == 0) {
                if (va) z_lds[t * K1_MAX_ROWS + ra] = sa;
                if (vb) z_lds[t * K1_MAX_ROWS + rb] = sb;
            }
        }
    }
    __syncthreads();
    compact_and_up<WT, NC>(z_lds, list, masks, &n_list, x, W3, a_out, live_out, row0, nrows, D,
                           H, T, act, union_mode);
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
