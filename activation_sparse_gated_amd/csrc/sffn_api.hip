// C ABI of the gate-first sparse FFN (declared in include/sffn.h): handle
// management, synchronous argument checks, and the launch plan of each
// forward call. All arithmetic runs in the kernels of sffn_kernels.hip.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "sffn.h"
#include "sffn_kernels.hip"

using namespace sffn;

namespace {

enum Kind { KIND_GATE_UP_SPARSE = 0, KIND_GATE_UP_LOPA, KIND_RANK_PROJ, KIND_GATE_UP_DENSE,
            KIND_DOWN, KIND_LIVE_LIST, KIND_GATE_UP_T1, KIND_DOWN_T1,
            KIND_FFN_DENSE_T1, KIND_REDUCE, KIND_RANK_PROJ_T1, KIND_GATE_UP_LOPA_T1,
            KIND_GATE_UP_MFMA, KIND_DOWN_MFMA, KIND_DOWN_TB, KIND_GATE_UP_T1_I8,
            KIND_GATE_UP_DENSE_T1_I8, KIND_DOWN_T1_I8, KIND_MOE_GATHER, KIND_MOE_COMBINE,
            KIND_GATE_UP_GEMM, KIND_UNION_LIST, KIND_DOWN_GEMM, KIND_RANK_PROJ_T1_I8,
            KIND_GATE_UP_LOPA_T1_I8, KIND_GATE_UP_TB, KIND_GATE_UP_T1_I4,
            KIND_GATE_UP_DENSE_T1_I4, KIND_DOWN_T1_I4, KIND_GATE_UP_LOPA_T1_I4,
            KIND_RANK_PROJ_MFMA, KIND_GATE_UP_TB_I8, KIND_DOWN_TB_I8, KIND_GATE_UP_TB_I4,
            KIND_DOWN_TB_I4, KIND_RANK_PROJ_TB_I8, KIND_GATE_UP_LOPA_TB_Q, KIND_DOWN_PT,
            KIND_GATE_UP_MFMA_I8, KIND_DOWN_MFMA_I8, KIND_RANK_PROJ_MFMA_I8,
            KIND_GATE_UP_MFMA_I4, KIND_DOWN_MFMA_I4, KIND_DOWN_PT_I8, KIND_DOWN_PT_I4,
            KIND_GATE_UP_MFMA_FUSED, KIND_GATE_UP_MFMA_FUSED_I8, KIND_GATE_UP_MFMA_FUSED_I4,
            KIND_DOWN_GEMM_BLT, KIND_COUNT };
const char* const kKindNames[KIND_COUNT] = {"k_gate_up_sparse", "k_gate_up_lopa", "k_rank_proj",
                                            "k_gate_up_dense", "k_down", "k_live_list",
                                            "k_gate_up_t1", "k_down_t1",
                                            "k_ffn_dense_t1", "k_reduce_partials",
                                            "k_rank_proj_t1", "k_gate_up_lopa_t1",
                                            "k_gate_up_mfma", "k_down_mfma", "k_down_tb",
                                            "k_gate_up_t1_i8", "k_gate_up_dense_t1_i8",
                                            "k_down_t1_i8", "k_moe_gather", "k_moe_combine",
                                            "k_gate_up_gemm", "k_union_list", "k_down_gemm",
                                            "k_rank_proj_t1_i8", "k_gate_up_lopa_t1_i8",
                                            "k_gate_up_tb", "k_gate_up_t1_i4",
                                            "k_gate_up_dense_t1_i4", "k_down_t1_i4",
                                            "k_gate_up_lopa_t1_i4", "k_rank_proj_mfma",
                                            "k_gate_up_tb_i8", "k_down_tb_i8", "k_gate_up_tb_i4",
                                            "k_down_tb_i4", "k_rank_proj_tb_i8", "k_gate_up_lopa_tb_q",
                                            "k_down_pt", "k_gate_up_mfma_i8", "k_down_mfma_i8",
                                            "k_rank_proj_mfma_i8", "k_gate_up_mfma_i4",
                                            "k_down_mfma_i4", "k_down_pt_i8", "k_down_pt_i4",
                                            "k_gate_up_mfma_fused", "k_gate_up_mfma_fused_i8",
                                            "k_gate_up_mfma_fused_i4", "down_gemm_hipblaslt"};

// Largest batch of a bf16 standard-gating handle (batches above MAXT run as GEMMs).
constexpr int MAXT_GEMM = 8192;
// From this many tokens the down pass runs as one library GEMM over every unit: against
// k_down_gemm (D=2560, H=7168, weights rotating through HBM) the union of 1280 / 1536 /
// 1792 / 2048 tokens 4.95M / 5.90M / 5.80M / 6.58M -> 5.17M / 6.49M / 6.85M / 7.62M
// tokens/s, level at 1024 (union +1 %, dense -3 %). Its workspace is allocated with the
// handle; plans are cached per handle.
constexpr int BLT_MIN_T = 1025;
constexpr size_t BLT_WS = size_t(64) << 20;
constexpr size_t BLT_MAX_PLANS = 16;

thread_local std::string g_thread_error = "no error";

}  // namespace

struct sffn_handle {
    int D = 0, H = 0, r = 0, max_tokens = 0, act = 0, dtype = 0;
    unsigned flags = 0;
    int device = 0;
    float* a_buf = nullptr;      // [max_tokens x H] unit products a_i
    uint8_t* live_buf = nullptr; // [max_tokens x H] live flags
    float* t_buf = nullptr;      // [max_tokens x r] LoPA rank vectors
    std::string err = "no error";
    // launch plan (fixed per shape at create; the constants come from measured sweeps)
    int gate_rows_per_wave = 4;    // units per wave of the general (fp32) gate kernels
    int t1_splits = 16;            // unit-range splits of the batch-1 down passes
    int f_rows_per_block = 0;      // units per block of that pass
    int f_rw = 0;                  // units per wave of that pass
    int f_blocks = 0;              // its blocks (= partial outputs)
    float* part_buf = nullptr;     // [f_blocks x D] partial outputs of the dense comparator
    // batched bf16 path on MFMA (union of live sets, dense)
    int m_tp = 0;                  // padded token count (16 * token tiles) the buffers hold
    int m_splits = 16;             // unit ranges of the MFMA down pass above 32 tokens
    int m_splits_s = 12;           // ... up to 32 tokens: column tiles x ranges <= CUs
    void* m_zero = nullptr;        // 4 KB of zeros (source of the staged pieces outside the operands)
    // mixture of experts: tokens gathered per expert, expert outputs per slot
    uint16_t* moe_x = nullptr;     // [2 * max_tokens x D] bf16
    float* moe_y = nullptr;        // [2 * max_tokens x D] fp32
    int tb_splits = 16;            // row splits of the small-batch down passes
    float* m_a = nullptr;          // [H x m_tp] unit products, unit-major
    uint64_t* m_mask = nullptr;    // [H] tokens for which each unit is live
    uint16_t* m_t = nullptr;       // LoPA: [2 x m_tp x r] bf16 rank vectors, hi then lo parts
    // large batches as GEMMs on MFMA (T > MAXT)
    int g_tp = 0;                  // padded token count of g_a (multiple of 256)
    uint16_t* g_a = nullptr;       // [H x g_tp] bf16 unit products, unit-major
    uint64_t* g_any = nullptr;     // [g_tp / 128 x 2 ceil(H / 128)] 64-unit live masks per token tile
    int32_t* g_list = nullptr;     // [H + 32] units live for some token, then the count
    // the down pass of batches of BLT_MIN_T tokens and more: y = a W2 over every unit as
    // one hipBLASLt GEMM (bf16 in, fp32 out), plans cached per token count
    struct BltPlan {
        int T = 0;
        hipblasLtMatmulDesc_t desc = nullptr;
        hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, ly = nullptr;
        hipblasLtMatmulAlgo_t algo{};
    };
    hipblasLtHandle_t blt = nullptr;
    void* blt_ws = nullptr;        // workspace of the library GEMM
    std::vector<BltPlan> blt_plans;

    // instrumentation
    int timing_every = 0;   // 0: off; N: the launches of every Nth forward call are timed
    int64_t call_seq = 0;   // forward calls checked since timing was enabled
    bool timed_call = false; // the launches of the current call are timed
    struct Rec { int kind; hipEvent_t start, stop; };
    std::vector<Rec> pending;
    std::vector<hipEvent_t> pool;
    double total_ms[KIND_COUNT] = {};
    int64_t launches[KIND_COUNT] = {};
};

namespace {

sffn_status fail(sffn_handle* h, sffn_status code, const std::string& msg) {
    if (h)
        h->err = msg;
    else
        g_thread_error = msg;
    return code;
}

sffn_status hip_fail(sffn_handle* h, hipError_t e, const char* what) {
    return fail(h, SFFN_HIP_ERROR, std::string(what) + ": " + hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

hipEvent_t take_event(sffn_handle* h) {
    if (!h->pool.empty()) {
        hipEvent_t e = h->pool.back();
        h->pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

template <typename... KArgs, typename... Args>
sffn_status launch_shm(sffn_handle* h, int kind, void (*kern)(KArgs...), dim3 grid, dim3 block,
                       size_t shm, hipStream_t s, Args... args) {
    if (grid.x == 0) return SFFN_OK;
    if (h->timed_call) {
        hipEvent_t e0 = take_event(h), e1 = take_event(h);
        if (!e0 || !e1) return fail(h, SFFN_HIP_ERROR, "hipEventCreate failed");
        hipExtLaunchKernelGGL(kern, grid, block, (uint32_t)shm, s, e0, e1, 0,
                              static_cast<KArgs>(args)...);
        h->pending.push_back({kind, e0, e1});
    } else {
        hipLaunchKernelGGL(kern, grid, block, shm, s, static_cast<KArgs>(args)...);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(h, e, kKindNames[kind]);
    return SFFN_OK;
}

template <typename... KArgs, typename... Args>
sffn_status launch(sffn_handle* h, int kind, void (*kern)(KArgs...), dim3 grid, dim3 block,
                   hipStream_t s, Args... args) {
    if (grid.x == 0) return SFFN_OK;
    if (h->timed_call) {
        hipEvent_t e0 = take_event(h), e1 = take_event(h);
        if (!e0 || !e1) return fail(h, SFFN_HIP_ERROR, "hipEventCreate failed");
        hipExtLaunchKernelGGL(kern, grid, block, 0, s, e0, e1, 0, static_cast<KArgs>(args)...);
        h->pending.push_back({kind, e0, e1});
    } else {
        hipLaunchKernelGGL(kern, grid, block, 0, s, static_cast<KArgs>(args)...);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(h, e, kKindNames[kind]);
    return SFFN_OK;
}

// ------------------------------------------------------------------ dispatch
// Register chunks per lane for a row of n elements (64 lanes x 16 bytes per chunk).
int chunks_needed(int n, int dtype) {
    const int cw = WAVE * (dtype == SFFN_BF16 ? 8 : 4);
    return (n + cw - 1) / cw;
}

// The instantiated chunk counts; the smallest one that covers the row is used.
constexpr int kNC[] = {1, 2, 3, 4, 5, 6, 8, 12, 16};
constexpr int kNR[] = {1, 2, 4, 8};

int pick(const int* set, int n, int need) {
    for (int i = 0; i < n; ++i)
        if (set[i] >= need) return set[i];
    return -1;
}

#define SFFN_NC_SWITCH(NCV, BODY)            \
    switch (NCV) {                           \
        case 1: { constexpr int NC = 1; BODY; } break;   \
        case 2: { constexpr int NC = 2; BODY; } break;   \
        case 3: { constexpr int NC = 3; BODY; } break;   \
        case 4: { constexpr int NC = 4; BODY; } break;   \
        case 5: { constexpr int NC = 5; BODY; } break;   \
        case 6: { constexpr int NC = 6; BODY; } break;   \
        case 8: { constexpr int NC = 8; BODY; } break;   \
        case 12: { constexpr int NC = 12; BODY; } break; \
        case 16: { constexpr int NC = 16; BODY; } break; \
        default: return fail(h, SFFN_INTERNAL, "no kernel for this width"); \
    }

#define SFFN_NR_SWITCH(NRV, BODY)            \
    switch (NRV) {                           \
        case 1: { constexpr int NR = 1; BODY; } break;   \
        case 2: { constexpr int NR = 2; BODY; } break;   \
        case 4: { constexpr int NR = 4; BODY; } break;   \
        case 8: { constexpr int NR = 8; BODY; } break;   \
        default: return fail(h, SFFN_INTERNAL, "no kernel for this rank"); \
    }

template <typename WT>
sffn_status run_down(sffn_handle* h, const void* W2T, float* y, int T, int union_mode, int dense,
                     hipStream_t s) {
    const int vec = Elem<WT>::VEC;
    const int cb = 8 * vec;
    const int nslices = (h->D + cb - 1) / cb;
    const int nb = ((nslices + 7) / 8) * 8;
    return launch(h, KIND_DOWN, k_down<WT, 8, 4>, dim3(nb), dim3(K2_THREADS), s, h->a_buf,
                  (const WT*)W2T, y, h->D, h->H, T, union_mode, dense);
}

sffn_status run_live_list(sffn_handle* h, int T, int32_t* live_count, int32_t* live_idx,
                          hipStream_t s) {
    if (!live_count) return SFFN_OK;
    return launch(h, KIND_LIVE_LIST, k_live_list, dim3(T), dim3(1024), s, h->live_buf, h->H,
                  live_count, live_idx);
}

constexpr int kNC_T1[] = {1, 2, 3, 4, 5, 6, 8};
constexpr int kPMAX[] = {1, 2, 4, 8, 16, 32};

// The batch-1 bf16 kernels hold a row of D in registers (at most 8 chunks of 512
// bf16); any H works, since the down pass splits the units into ranges of at most
// 32 x 512 (t1_splits is raised at create when H needs it).
bool t1_ok(const sffn_handle* h, int T) {
    return T == 1 && h->dtype == SFFN_BF16 && chunks_needed(h->D, h->dtype) <= 8;
}

#define SFFN_NCT1_SWITCH(NCV, BODY)                       \
    switch (NCV) {                                        \
        case 1: { constexpr int NC = 1; BODY; } break;    \
        case 2: { constexpr int NC = 2; BODY; } break;    \
        case 3: { constexpr int NC = 3; BODY; } break;    \
        case 4: { constexpr int NC = 4; BODY; } break;    \
        case 5: { constexpr int NC = 5; BODY; } break;    \
        case 6: { constexpr int NC = 6; BODY; } break;    \
        case 8: { constexpr int NC = 8; BODY; } break;    \
        default: return fail(h, SFFN_INTERNAL, "no batch-1 kernel for this width"); \
    }
#define SFFN_PMAX_SWITCH(PV, BODY)                        \
    switch (PV) {                                         \
        case 1: { constexpr int PMAX = 1; BODY; } break;  \
        case 2: { constexpr int PMAX = 2; BODY; } break;  \
        case 4: { constexpr int PMAX = 4; BODY; } break;  \
        case 8: { constexpr int PMAX = 8; BODY; } break;  \
        case 16: { constexpr int PMAX = 16; BODY; } break; \
        case 32: { constexpr int PMAX = 32; BODY; } break; \
        default: return fail(h, SFFN_INTERNAL, "hidden width too large for the down pass"); \
    }

// down pass, batch 1, bf16: 256-column slices (32 lanes x 16 B per W2T row
// slice), XCD-contiguous slice order, `splits` unit ranges
sffn_status run_down_t1(sffn_handle* h, const void* W2T, float* y, int splits, int dense,
                        hipStream_t s) {
    const int cb = 32 * 8;
    const int nslices = (h->D + cb - 1) / cb;
    const int nbx = ((nslices + 7) / 8) * 8;
    const int hs = (h->H + splits - 1) / splits;
    const int pmax = pick(kPMAX, 6, (hs + KD_THREADS - 1) / KD_THREADS);
    sffn_status st = SFFN_OK;
    SFFN_PMAX_SWITCH(pmax, st = launch(h, KIND_DOWN_T1, k_down_t1<PMAX>, dim3(nbx, splits),
                                       dim3(KD_THREADS), s, (const float*)h->a_buf,
                                       (const uint16_t*)W2T, y, h->D, h->H, splits, dense));
    return st;
}

#define SFFN_FRW_SWITCH(RWV, BODY)                        \
    switch (RWV) {                                        \
        case 1: { constexpr int RW = 1; BODY; } break;    \
        case 2: { constexpr int RW = 2; BODY; } break;    \
        case 4: { constexpr int RW = 4; BODY; } break;    \
        case 8: { constexpr int RW = 8; BODY; } break;    \
        default: return fail(h, SFFN_INTERNAL, "bad units per wave"); \
    }

// Batch-1 dense comparator as one fused pass (W1, W3 and W2T rows of every unit
// read together, one partial output per block) + the partial reduction.
sffn_status run_fused_dense_t1(sffn_handle* h, const void* x, const void* W1, const void* W3,
                               const void* W2T, float* y, hipStream_t s) {
    const int nc = pick(kNC_T1, 7, chunks_needed(h->D, h->dtype));
    const size_t shm = (size_t)KF_WAVES * h->D * sizeof(float);
    sffn_status st = SFFN_OK;
    SFFN_NCT1_SWITCH(nc, SFFN_FRW_SWITCH(h->f_rw,
        st = launch_shm(h, KIND_FFN_DENSE_T1, k_ffn_dense_t1<NC, RW>, dim3(h->f_blocks),
                        dim3(KF_THREADS), shm, s, (const uint16_t*)x, (const uint16_t*)W1,
                        (const uint16_t*)W3, (const uint16_t*)W2T, h->part_buf, h->D, h->H,
                        h->f_rows_per_block, h->act)));
    if (st != SFFN_OK) return st;
    return launch(h, KIND_REDUCE, k_reduce_partials, dim3((h->D + 63) / 64), dim3(KR_THREADS), s,
                  (const float*)h->part_buf, y, h->D, h->f_blocks);
}

// Allow the fused dense kernel its dynamic LDS (one y slice per wave).
sffn_status prepare_fused(sffn_handle* h) {
    const int nc = pick(kNC_T1, 7, chunks_needed(h->D, h->dtype));
    const int shm = KF_WAVES * h->D * (int)sizeof(float);
    hipError_t e = hipSuccess;
    SFFN_NCT1_SWITCH(nc, SFFN_FRW_SWITCH(h->f_rw,
        e = hipFuncSetAttribute((const void*)k_ffn_dense_t1<NC, RW>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, shm)));
    if (e != hipSuccess) return hip_fail(h, e, "hipFuncSetAttribute");
    return SFFN_OK;
}

// Batch-1 sparse pass: the gate kernel (one unit per wave, each wave reads the
// W3 row of its unit when it is live) and the down kernel.
sffn_status run_sparse_t1(sffn_handle* h, const void* x, const void* W1, const void* W3,
                          const void* W2T, float* y, int32_t* live_count, int32_t* live_idx,
                          hipStream_t s) {
    const int nc = pick(kNC_T1, 7, chunks_needed(h->D, h->dtype));
    const int nb = (h->H + K1_WAVES - 1) / K1_WAVES;
    const int splits = h->t1_splits;
    uint8_t* live = live_count ? h->live_buf : nullptr;
    float* yz = splits > 1 ? y : nullptr;
    sffn_status st = SFFN_OK;
    SFFN_NCT1_SWITCH(nc, st = launch(h, KIND_GATE_UP_T1, k_gate_up_t1<NC>, dim3(nb),
                                     dim3(K1_THREADS), s, (const uint16_t*)x, (const uint16_t*)W1,
                                     (const uint16_t*)W3, h->a_buf, live, yz, h->D, h->H,
                                     h->act));
    if (st != SFFN_OK) return st;
    st = run_down_t1(h, W2T, y, splits, 0, s);
    if (st != SFFN_OK) return st;
    return run_live_list(h, 1, live_count, live_idx, s);
}

// Batch-1 dense comparator: the fused pass (the batch-1 plan takes bf16 rows of
// at most 4096 = KF_DMAX columns, where its per-wave LDS slices always fit).
sffn_status run_dense_t1(sffn_handle* h, const void* x, const void* W1, const void* W3,
                         const void* W2T, float* y, hipStream_t s) {
    return run_fused_dense_t1(h, x, W1, W3, W2T, y, s);
}

// ---- batched bf16 path on MFMA
bool mfma_ok(const sffn_handle* h, int T) {
    return T >= 2 && h->dtype == SFFN_BF16 && h->m_a != nullptr && T <= h->max_tokens;
}

#define SFFN_NT_SWITCH(NTV, BODY)                         \
    switch (NTV) {                                        \
        case 1: { constexpr int NT = 1; BODY; } break;    \
        case 2: { constexpr int NT = 2; BODY; } break;    \
        case 4: { constexpr int NT = 4; BODY; } break;    \
        default: return fail(h, SFFN_INTERNAL, "bad token tile count"); \
    }

// token tiles of 16 for a batch of T tokens: 1, 2 or 4
inline int token_tiles(int T) { return T <= 16 ? 1 : (T <= 32 ? 2 : 4); }

// LOPA: W1 is U, V the rank factor; the batch's rank vectors go through m_t
// (bf16 hi and lo parts) into the MFMA gate, the rest is the standard plan.
// per_token: the down pass gathers each token's own live W2T rows (per-token
// lists) instead of the union's rows once for all tokens.
// unit ranges of the MFMA down pass for a batch of nt token tiles
inline int mfma_down_splits(const sffn_handle* h, int nt) {
    return nt <= 2 ? h->m_splits_s : h->m_splits;
}

template <bool DENSE, bool LOPA = false>
sffn_status run_mfma(sffn_handle* h, const void* x, const void* W1, const void* W3,
                     const void* W2T, float* y, int T, int32_t* live_count, int32_t* live_idx,
                     hipStream_t s, const void* V = nullptr, bool per_token = false) {
    const int nt = token_tiles(T);
    uint8_t* live = live_count ? h->live_buf : nullptr;
    sffn_status st = SFFN_OK;
    uint16_t* t_hi = h->m_t;
    uint16_t* t_lo = h->m_t ? h->m_t + (size_t)h->m_tp * h->r : nullptr;
    if (LOPA) {
        // 16 rank rows x 16 tokens per block (grid: rank tiles x token tiles): x is staged
        // once per token tile, V read once per token tile (from L2 after the first); at
        // 64 tokens 100 blocks instead of 25 (LoPA union of 40 / 64 tokens 490k / 755k ->
        // 508k / 788k tokens/s, int8 417k / 652k -> 441k / 691k)
        SFFN_NT_SWITCH(nt, st = launch(h, KIND_RANK_PROJ_MFMA, k_rank_proj_mfma<1>,
                                       dim3((h->r + 15) / 16, NT), dim3(KM_THREADS), s,
                                       (const uint16_t*)x, (const uint16_t*)V,
                                       (const uint16_t*)h->m_zero, t_hi, t_lo, h->D, h->r, T));
        if (st != SFFN_OK) return st;
    }
    // unit tiles per gate block: 32 units from 17 tokens on; at 33-64 tokens the 32-unit
    // block of the LoPA gate takes 74 KB of LDS, so its 306 blocks over H' = 9787 run two
    // per CU in one round (ahead of 153 blocks of 64 units: union of 40 / 64 tokens 573k /
    // 893k -> 596k / 898k tokens/s)
    const int ut = nt == 1 ? 1 : 2;
    const int nb = (h->H + 16 * ut - 1) / (16 * ut);
    // VALU kernels up to 4 tokens (the dense comparator up to 2: from 3 tokens its MFMA
    // passes are ahead, dense of 3 / 4 tokens 95.8k / 126k -> 101k / 134k tokens/s)
    const int valu_max = DENSE ? 2 : 4;
    const bool small_down = T <= valu_max;
    const int splits = per_token ? h->t1_splits : (small_down ? h->tb_splits : mfma_down_splits(h, nt));
    float* yz = splits > 1 ? y : nullptr;
    // the MFMA down pass takes the products split into bf16 hi and lo parts; the
    // per-token and small-batch down passes take them in fp32
    const int split = (!per_token && !small_down) ? 1 : 0;
    if (!LOPA && T <= valu_max && chunks_needed(h->D, h->dtype) <= 8) {
        // gate/up on the VALU: x of the batch in registers, W1 streamed once; units
        // per wave = token slots (2 or 4)
        const int nc = pick(kNC_T1, 7, chunks_needed(h->D, h->dtype));
        const int tt = T <= 2 ? 2 : 4;
        const int nbv = (h->H + K1_WAVES * tt - 1) / (K1_WAVES * tt);
#define SFFN_TBV(TTV)                                                                               \
        SFFN_NCT1_SWITCH(nc, st = launch(h, KIND_GATE_UP_TB,                                        \
            k_gate_up_tb<NC, TTV, TTV, DENSE>, dim3(nbv), dim3(K1_THREADS), s, (const uint16_t*)x,  \
            (const uint16_t*)W1, (const uint16_t*)W3, h->m_a, h->m_mask, live, yz, h->D, h->H, T,   \
            16 * nt, h->act))
        if (tt == 2) { SFFN_TBV(2); } else { SFFN_TBV(4); }
#undef SFFN_TBV
    } else if (!LOPA && (DENSE || T > 10)) {
        // above 10 tokens the union covers most units (1 - 0.9^11 = 69 %; dense: every
        // unit): W1 and W3 rows of the block in one pass, x staged once for both
        // (measured ahead of the gathered W3 pass from 12 tokens on, level at 10,
        // behind up to 8: union of 12 / 14 / 16 tokens 395k / 448k / 498k -> 400k /
        // 460k / 520k tokens/s, of 8 297k -> 295k)
#define SFFN_GATE_FUSED(NTV, UTV)                                                              \
    st = launch(h, KIND_GATE_UP_MFMA_FUSED, k_gate_up_mfma_fused<NTV, UTV, DENSE>, dim3(nb),   \
                dim3(KM_THREADS), s, (const uint16_t*)x, (const uint16_t*)W1,                  \
                (const uint16_t*)W3, (const uint16_t*)h->m_zero, h->m_a, h->m_mask, live, yz,   \
                h->D, h->H, T, h->act, split)
        if (nt == 1) {
            SFFN_GATE_FUSED(1, 1);
        } else if (nt == 2) {
            SFFN_GATE_FUSED(2, 2);
        } else {
            SFFN_GATE_FUSED(4, 2);
        }
#undef SFFN_GATE_FUSED
    } else {
#define SFFN_GATE_MFMA(NTV, UTV)                                                               \
    st = launch(h, KIND_GATE_UP_MFMA, k_gate_up_mfma<NTV, UTV, DENSE, LOPA>, dim3(nb),         \
                dim3(KM_THREADS), s, (const uint16_t*)x, (const uint16_t*)W1,                  \
                (const uint16_t*)W3, (const uint16_t*)h->m_zero, h->m_a, h->m_mask, live, yz,   \
                h->D, h->H, T, h->act, (const uint16_t*)t_hi, (const uint16_t*)t_lo, h->r,      \
                h->flags, split)
    if (nt == 1) {
        SFFN_GATE_MFMA(1, 1);
    } else if (nt == 2) {
        SFFN_GATE_MFMA(2, 2);
    } else {
        SFFN_GATE_MFMA(4, 2);
    }
    }
#undef SFFN_GATE_MFMA
    if (st != SFFN_OK) return st;
    if (per_token) {
        // per-token lists: one block row per token, 512-byte row slices
        const int cb = 32 * 8;
        const int nbx = (((h->D + cb - 1) / cb + 7) / 8) * 8;
        const int hs = (h->H + splits - 1) / splits;
        const int pmax = pick(kPMAX, 6, (hs + KD_THREADS - 1) / KD_THREADS);
        SFFN_PMAX_SWITCH(pmax, st = launch(h, KIND_DOWN_PT, k_down_pt<PMAX>, dim3(nbx, splits, T),
                                           dim3(KD_THREADS), s, (const float*)h->m_a,
                                           (const uint64_t*)h->m_mask, (const uint16_t*)W2T, y,
                                           h->D, h->H, 16 * nt, splits));
    } else if (small_down) {
        // 512-byte row slices (32 lanes x 16 B), XCD-contiguous slice order
        const int cb = 32 * 8;
        const int nslices = (h->D + cb - 1) / cb;
        const int nbx = ((nslices + 7) / 8) * 8;
        const int hs = (h->H + splits - 1) / splits;
        const int pmax = pick(kPMAX, 6, (hs + KD_THREADS - 1) / KD_THREADS);
        const int tt = T <= 2 ? 2 : 4;
#define SFFN_TB_LAUNCH(TTV)                                                                      \
        SFFN_PMAX_SWITCH(pmax, st = launch(h, KIND_DOWN_TB, k_down_tb<32, PMAX, TTV>,            \
                                           dim3(nbx, splits), dim3(KD_THREADS), s,               \
                                           (const float*)h->m_a, (const uint64_t*)h->m_mask,     \
                                           (const uint16_t*)W2T, y, h->D, h->H, T, 16 * nt,      \
                                           splits))
        if (tt == 2) { SFFN_TB_LAUNCH(2); } else { SFFN_TB_LAUNCH(4); }
#undef SFFN_TB_LAUNCH
    } else {
        const int ntile = (h->D + KDM_NB - 1) / KDM_NB;
        SFFN_NT_SWITCH(nt,
            st = launch(h, KIND_DOWN_MFMA, k_down_mfma<NT>, dim3(ntile, splits),
                        dim3(KDM_THREADS), s, (const float*)h->m_a, (const uint64_t*)h->m_mask,
                        (const uint16_t*)W2T, y, h->D, h->H, T, splits));
    }
    if (st != SFFN_OK) return st;
    if (!DENSE) return run_live_list(h, T, live_count, live_idx, s);
    return SFFN_OK;
}

// ---- large batches: gate/up GEMM, union list, gathered down GEMM
bool gemm_ok(const sffn_handle* h, int T) {
    return h->g_a != nullptr && T > MAXT && T <= h->max_tokens;
}

template <int TM, int UN, bool DENSE>
sffn_status run_gate_gemm(sffn_handle* h, const void* x, const void* W1, const void* W3,
                          uint8_t* live, float* yz, int T, hipStream_t s) {
    using G = GemmTile<TM, UN>;
    const int ntt = (T + TM - 1) / TM;
    const int nut = (h->H + UN - 1) / UN;
    sffn_status st = launch(h, KIND_GATE_UP_GEMM, k_gate_up_gemm<TM, UN, DENSE>,
                            dim3(nut * ntt), dim3(G::THREADS), s, (const uint16_t*)x,
                            (const uint16_t*)W1, (const uint16_t*)W3, (const uint16_t*)h->m_zero,
                            h->g_a, DENSE ? (uint64_t*)nullptr : h->g_any, live, yz, h->D, h->H,
                            T, h->g_tp, h->act);
    if (st != SFFN_OK || DENSE) return st;
    int32_t* count = h->g_list + h->H + 32;
    return launch(h, KIND_UNION_LIST, k_union_list, dim3(1), dim3(1024), s,
                  (const uint64_t*)h->g_any, ntt, nut * (UN / 64), h->g_list, count);
}

void blt_plan_free(sffn_handle::BltPlan& p) {
    if (p.la) (void)hipblasLtMatrixLayoutDestroy(p.la);
    if (p.lb) (void)hipblasLtMatrixLayoutDestroy(p.lb);
    if (p.ly) (void)hipblasLtMatrixLayoutDestroy(p.ly);
    if (p.desc) (void)hipblasLtMatmulDescDestroy(p.desc);
    p = sffn_handle::BltPlan{};
}

// Plan of y[T x D] = sum over units u of a[u][t] W2T[u][:], in the library's
// column-major terms Y (D x T) = A (W2T as D x H, ld D) . B^T (the unit-major products
// as T x H, ld g_tp), fp32 accumulation and output.
sffn_status blt_plan(sffn_handle* h, int T, const sffn_handle::BltPlan** out) {
    for (const auto& p : h->blt_plans)
        if (p.T == T) {
            *out = &p;
            return SFFN_OK;
        }
    sffn_handle::BltPlan p;
    p.T = T;
    hipblasStatus_t st = hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F);
    const hipblasOperation_t opn = HIPBLAS_OP_N, opt = HIPBLAS_OP_T;
    if (st == HIPBLAS_STATUS_SUCCESS)
        st = hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opn, sizeof(opn));
    if (st == HIPBLAS_STATUS_SUCCESS)
        st = hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opt, sizeof(opt));
    if (st == HIPBLAS_STATUS_SUCCESS) st = hipblasLtMatrixLayoutCreate(&p.la, HIP_R_16BF, h->D, h->H, h->D);
    if (st == HIPBLAS_STATUS_SUCCESS) st = hipblasLtMatrixLayoutCreate(&p.lb, HIP_R_16BF, T, h->H, h->g_tp);
    if (st == HIPBLAS_STATUS_SUCCESS) st = hipblasLtMatrixLayoutCreate(&p.ly, HIP_R_32F, h->D, T, h->D);
    int n = 0;
    if (st == HIPBLAS_STATUS_SUCCESS) {
        hipblasLtMatmulPreference_t pref = nullptr;
        st = hipblasLtMatmulPreferenceCreate(&pref);
        const uint64_t ws = BLT_WS;
        if (st == HIPBLAS_STATUS_SUCCESS)
            st = hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES,
                                                       &ws, sizeof(ws));
        hipblasLtMatmulHeuristicResult_t res[1];
        if (st == HIPBLAS_STATUS_SUCCESS)
            st = hipblasLtMatmulAlgoGetHeuristic(h->blt, p.desc, p.la, p.lb, p.ly, p.ly, pref, 1, res, &n);
        if (pref) (void)hipblasLtMatmulPreferenceDestroy(pref);
        if (st == HIPBLAS_STATUS_SUCCESS && n > 0) p.algo = res[0].algo;
    }
    if (st != HIPBLAS_STATUS_SUCCESS || n == 0) {
        blt_plan_free(p);
        return fail(h, SFFN_INTERNAL, "hipBLASLt has no plan for the down GEMM at T=" + std::to_string(T) +
                                          " (status " + std::to_string((int)st) + ")");
    }
    if (h->blt_plans.size() >= BLT_MAX_PLANS) {
        blt_plan_free(h->blt_plans.front());
        h->blt_plans.erase(h->blt_plans.begin());
    }
    h->blt_plans.push_back(p);
    *out = &h->blt_plans.back();
    return SFFN_OK;
}

sffn_status run_down_blt(sffn_handle* h, const void* W2T, float* y, int T, hipStream_t s) {
    const sffn_handle::BltPlan* p = nullptr;
    sffn_status st = blt_plan(h, T, &p);
    if (st != SFFN_OK) return st;
    const float alpha = 1.0f, beta = 0.0f;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (h->timed_call) {
        e0 = take_event(h);
        e1 = take_event(h);
        if (!e0 || !e1) return fail(h, SFFN_HIP_ERROR, "hipEventCreate failed");
        hipError_t e = hipEventRecord(e0, s);
        if (e != hipSuccess) return hip_fail(h, e, "hipEventRecord");
    }
    const hipblasStatus_t bs = hipblasLtMatmul(h->blt, p->desc, &alpha, W2T, p->la, h->g_a, p->lb, &beta,
                                               y, p->ly, y, p->ly, &p->algo, h->blt_ws, BLT_WS, s);
    if (h->timed_call) {
        hipError_t e = hipEventRecord(e1, s);
        if (e != hipSuccess) return hip_fail(h, e, "hipEventRecord");
        h->pending.push_back({KIND_DOWN_GEMM_BLT, e0, e1});
    }
    if (bs != HIPBLAS_STATUS_SUCCESS)
        return fail(h, SFFN_HIP_ERROR, "hipblasLtMatmul (down GEMM): status " + std::to_string((int)bs));
    return SFFN_OK;
}

template <bool DENSE>
sffn_status run_gemm(sffn_handle* h, const void* x, const void* W1, const void* W3,
                     const void* W2T, float* y, int T, int32_t* live_count, int32_t* live_idx,
                     hipStream_t s) {
    const int nmt = (T + KDG_TM - 1) / KDG_TM;
    const int nnt = (h->D + KDG_NB - 1) / KDG_NB;
    // unit-range splits only while the output tiles alone leave CUs idle, and
    // never below 8 chunks of units per split
    int splits = 1;
    const int nch = (h->H + KDG_KC - 1) / KDG_KC;
    while (nmt * nnt * splits < 256 && splits < 16 && nch / (2 * splits) >= 8) splits *= 2;
    uint8_t* live = live_count ? h->live_buf : nullptr;
    float* yz = splits > 1 ? y : nullptr;
    int32_t* count = h->g_list + h->H + 32;
    // 256 x 128 gate tiles once there are 200 of them, else 256 x 64 (more blocks); up to
    // 256 tokens 128 x 64 (twice the blocks at 64 KB of LDS, two per CU: union of 128 / 256
    // tokens 1.44M / 2.67M -> 1.46M / 2.73M tokens/s)
    const bool wide = (long)((T + 255) / 256) * ((h->H + 127) / 128) >= 200;
    const bool small = !wide && T <= 256;
    if (T >= BLT_MIN_T && h->blt) {
        // the down pass over every unit (the products of units dead for every token are
        // exact zeros: A(z) = 0 for z <= 0), so the gate writes no union masks, and y is
        // written by the GEMM (no clear)
        sffn_status st = wide ? run_gate_gemm<256, 128, true>(h, x, W1, W3, live, nullptr, T, s)
                              : run_gate_gemm<256, 64, true>(h, x, W1, W3, live, nullptr, T, s);
        if (st == SFFN_OK) st = run_down_blt(h, W2T, y, T, s);
        if (st != SFFN_OK || DENSE) return st;
        return run_live_list(h, T, live_count, live_idx, s);
    }
    sffn_status st = wide ? run_gate_gemm<256, 128, DENSE>(h, x, W1, W3, live, yz, T, s)
                          : (small ? run_gate_gemm<128, 64, DENSE>(h, x, W1, W3, live, yz, T, s)
                                   : run_gate_gemm<256, 64, DENSE>(h, x, W1, W3, live, yz, T, s));
    if (st != SFFN_OK) return st;
    st = launch(h, KIND_DOWN_GEMM, k_down_gemm, dim3(nmt * nnt * splits), dim3(KDG_THREADS), s,
                (const uint16_t*)h->g_a, DENSE ? (const int32_t*)nullptr : (const int32_t*)h->g_list,
                (const int32_t*)count, (const uint16_t*)W2T, (const uint16_t*)h->m_zero, y, h->D,
                h->H, T, h->g_tp, splits);
    if (st != SFFN_OK) return st;
    if (!DENSE) return run_live_list(h, T, live_count, live_idx, s);
    return SFFN_OK;
}

template <typename WT>
sffn_status run_sparse(sffn_handle* h, const void* x, const void* W1, const void* W3,
                       const void* W2T, float* y, int T, int mode, int32_t* live_count,
                       int32_t* live_idx, hipStream_t s) {
    const int nc = pick(kNC, sizeof(kNC) / sizeof(int), chunks_needed(h->D, h->dtype));
    const int rpw = h->gate_rows_per_wave;
    const int rows_per_block = rpw * K1_WAVES;
    const int nb = (h->H + rows_per_block - 1) / rows_per_block;
    uint8_t* live = live_count ? h->live_buf : nullptr;
    sffn_status st = SFFN_OK;
    SFFN_NC_SWITCH(nc, st = launch(h, KIND_GATE_UP_SPARSE, k_gate_up_sparse<WT, NC>, dim3(nb),
                                   dim3(K1_THREADS), s, (const WT*)x, (const WT*)W1,
                                   (const WT*)W3, h->a_buf, live, h->D, h->H, T, h->act,
                                   mode == SFFN_MODE_UNION ? 1 : 0, rpw));
    if (st != SFFN_OK) return st;
    st = run_down<WT>(h, W2T, y, T, mode == SFFN_MODE_UNION ? 1 : 0, 0, s);
    if (st != SFFN_OK) return st;
    return run_live_list(h, T, live_count, live_idx, s);
}

#define SFFN_NRT1_SWITCH(NRV, BODY)                       \
    switch (NRV) {                                        \
        case 1: { constexpr int NR = 1; BODY; } break;    \
        case 2: { constexpr int NR = 2; BODY; } break;    \
        case 4: { constexpr int NR = 4; BODY; } break;    \
        default: return fail(h, SFFN_INTERNAL, "no batch-1 kernel for this rank"); \
    }

sffn_status run_lopa_t1(sffn_handle* h, const void* x, const void* V, const void* U,
                        const void* W3, const void* W2T, float* y, int32_t* live_count,
                        int32_t* live_idx, hipStream_t s) {
    const int nc = pick(kNC_T1, 7, chunks_needed(h->D, h->dtype));
    const int nr = pick(kNR, 3, chunks_needed(h->r, h->dtype));
    const int splits = h->t1_splits;
    float* yz = splits > 1 ? y : nullptr;
    sffn_status st = SFFN_OK;
    const int nbr = (h->r + K1_WAVES - 1) / K1_WAVES;
    SFFN_NCT1_SWITCH(nc, st = launch(h, KIND_RANK_PROJ_T1, k_rank_proj_t1<NC>, dim3(nbr),
                                     dim3(K1_THREADS), s, (const uint16_t*)x, (const uint16_t*)V,
                                     h->t_buf, yz, h->D, h->r));
    if (st != SFFN_OK) return st;
    // one unit per wave (measured ahead of two once only live waves read x)
    const int nb = (h->H + K1_WAVES - 1) / K1_WAVES;
    uint8_t* live = live_count ? h->live_buf : nullptr;
    SFFN_NCT1_SWITCH(nc, SFFN_NRT1_SWITCH(nr,
        st = launch(h, KIND_GATE_UP_LOPA_T1, k_gate_up_lopa_t1<NC, NR, 1>, dim3(nb),
                    dim3(K1_THREADS), s, (const uint16_t*)x, (const float*)h->t_buf,
                    (const uint16_t*)U, (const uint16_t*)W3, h->a_buf, live, h->D, h->H, h->r,
                    h->act, h->flags)));
    if (st != SFFN_OK) return st;
    st = run_down_t1(h, W2T, y, splits, 0, s);
    if (st != SFFN_OK) return st;
    return run_live_list(h, 1, live_count, live_idx, s);
}

template <typename WT>
sffn_status run_lopa(sffn_handle* h, const void* x, const void* V, const void* U, const void* W3,
                     const void* W2T, float* y, int T, int mode, int32_t* live_count,
                     int32_t* live_idx, hipStream_t s) {
    const int nc = pick(kNC, sizeof(kNC) / sizeof(int), chunks_needed(h->D, h->dtype));
    const int nr = pick(kNR, sizeof(kNR) / sizeof(int), chunks_needed(h->r, h->dtype));
    sffn_status st = SFFN_OK;
    {
        const int rpw = 1;
        const int nb = (h->r + K1_WAVES * rpw - 1) / (K1_WAVES * rpw);
        SFFN_NC_SWITCH(nc, st = launch(h, KIND_RANK_PROJ, k_rank_proj<WT, NC>, dim3(nb),
                                       dim3(K1_THREADS), s, (const WT*)x, (const WT*)V, h->t_buf,
                                       h->D, h->r, T, rpw));
        if (st != SFFN_OK) return st;
    }
    const int rpw = h->gate_rows_per_wave;
    const int rows_per_block = rpw * K1_WAVES;
    const int nb = (h->H + rows_per_block - 1) / rows_per_block;
    uint8_t* live = live_count ? h->live_buf : nullptr;
    SFFN_NC_SWITCH(nc, SFFN_NR_SWITCH(nr, st = launch(h, KIND_GATE_UP_LOPA,
                                                      k_gate_up_lopa<WT, NC, NR>, dim3(nb),
                                                      dim3(K1_THREADS), s, (const WT*)x,
                                                      (const float*)h->t_buf, (const WT*)U,
                                                      (const WT*)W3, h->a_buf, live, h->D, h->H,
                                                      h->r, T, h->act,
                                                      mode == SFFN_MODE_UNION ? 1 : 0, rpw,
                                                      h->flags)));
    if (st != SFFN_OK) return st;
    st = run_down<WT>(h, W2T, y, T, mode == SFFN_MODE_UNION ? 1 : 0, 0, s);
    if (st != SFFN_OK) return st;
    return run_live_list(h, T, live_count, live_idx, s);
}

template <typename WT>
sffn_status run_dense(sffn_handle* h, const void* x, const void* W1, const void* W3,
                      const void* W2T, float* y, int T, hipStream_t s) {
    const int nc = pick(kNC, sizeof(kNC) / sizeof(int), chunks_needed(h->D, h->dtype));
    const int rpw = 2;
    const int nb = (h->H + K1_WAVES * rpw - 1) / (K1_WAVES * rpw);
    sffn_status st = SFFN_OK;
    SFFN_NC_SWITCH(nc, st = launch(h, KIND_GATE_UP_DENSE, k_gate_up_dense<WT, NC>, dim3(nb),
                                   dim3(K1_THREADS), s, (const WT*)x, (const WT*)W1,
                                   (const WT*)W3, h->a_buf, h->D, h->H, T, h->act, rpw));
    if (st != SFFN_OK) return st;
    return run_down<WT>(h, W2T, y, T, 1, 1, s);
}

// Weight-only int8, one token: gate (+ up) pass, then the int8 down pass over
// 256-column slices and 16 row splits (atomics into y, cleared by the gate pass).
// int8 down pass over the products the gate pass stored (pre-scaled by s2)
sffn_status run_down_t1_i8(sffn_handle* h, const void* W2T, float* y, int splits, bool dense,
                           hipStream_t s) {
    const int cb = 16 * 16;
    const int nslices = (h->D + cb - 1) / cb;
    const int nbx = ((nslices + 7) / 8) * 8;
    const int hs = (h->H + splits - 1) / splits;
    const int pmax = pick(kPMAX, 6, (hs + KD_THREADS - 1) / KD_THREADS);
    sffn_status st = SFFN_OK;
    SFFN_PMAX_SWITCH(pmax, st = launch(h, KIND_DOWN_T1_I8, k_down_t1_i8<PMAX>, dim3(nbx, splits),
                                       dim3(KD_THREADS), s, (const float*)h->a_buf,
                                       (const int8_t*)W2T, y, h->D, h->H, splits, dense ? 1 : 0));
    return st;
}

template <bool DENSE>
sffn_status run_i8_t1(sffn_handle* h, const void* x, const void* W1, const float* s1,
                      const void* W3, const float* s3, const void* W2T, const float* s2,
                      float* y, int32_t* live_count, int32_t* live_idx, hipStream_t s) {
    const int nc = pick(kNC_T1, 7, (h->D + 1023) / 1024);
    const int nb = (h->H + K1_WAVES - 1) / K1_WAVES;
    int splits = h->t1_splits;
    while ((h->H + splits - 1) / splits > 32 * KD_THREADS) ++splits;
    uint8_t* live = (!DENSE && live_count) ? h->live_buf : nullptr;
    float* yz = splits > 1 ? y : nullptr;
    sffn_status st = SFFN_OK;
    SFFN_NCT1_SWITCH(nc, st = launch(h, DENSE ? KIND_GATE_UP_DENSE_T1_I8 : KIND_GATE_UP_T1_I8,
                                     k_gate_up_t1_i8<NC, DENSE>, dim3(nb), dim3(K1_THREADS), s,
                                     (const uint16_t*)x, (const int8_t*)W1, s1, (const int8_t*)W3,
                                     s3, s2, h->a_buf, live, yz, h->D, h->H, h->act));
    if (st != SFFN_OK) return st;
    st = run_down_t1_i8(h, W2T, y, splits, DENSE, s);
    if (st != SFFN_OK) return st;
    if (DENSE) return SFFN_OK;
    return run_live_list(h, 1, live_count, live_idx, s);
}

// Per-token down pass of a quantised batch (int8 or int4 W2T rows): each token's
// own live W2T rows from the unit-major products and token masks the batch gate
// wrote (row stride tp); y is cleared by that gate.
sffn_status run_down_pt_q(sffn_handle* h, const void* W2T, const float* s2, float* y, int T,
                          int tp, int bits, hipStream_t s) {
    const int cb = 16 * 16;
    const int nbx = (((h->D + cb - 1) / cb + 7) / 8) * 8;
    const int splits = h->t1_splits;
    const int hs = (h->H + splits - 1) / splits;
    const int pmax = pick(kPMAX, 6, (hs + KD_THREADS - 1) / KD_THREADS);
    sffn_status st = SFFN_OK;
    if (bits == 8) {
        SFFN_PMAX_SWITCH(pmax, st = launch(h, KIND_DOWN_PT_I8, k_down_pt_q<PMAX, 8>,
                                           dim3(nbx, splits, T), dim3(KD_THREADS), s,
                                           (const float*)h->m_a, (const uint64_t*)h->m_mask,
                                           (const uint8_t*)W2T, s2, y, h->D, h->H, tp, splits));
    } else {
        SFFN_PMAX_SWITCH(pmax, st = launch(h, KIND_DOWN_PT_I4, k_down_pt_q<PMAX, 4>,
                                           dim3(nbx, splits, T), dim3(KD_THREADS), s,
                                           (const float*)h->m_a, (const uint64_t*)h->m_mask,
                                           (const uint8_t*)W2T, s2, y, h->D, h->H, tp, splits));
    }
    return st;
}

// int8 union (and dense) batches of 5..64 tokens on MFMA: every weight code read
// once for the batch (W1 or U, V, the W3 rows of the union, their W2T rows).
// LOPA: W1 is U (scales s1 = U's), V with its scales sV gives the rank vectors.
// min_t: the smallest batch taken on MFMA (5 unless the caller's plan says otherwise)
bool mfma_i8_ok(const sffn_handle* h, int T, int min_t = 5) {
    return T >= min_t && h->dtype == SFFN_I8 && h->m_a != nullptr && T <= h->max_tokens;
}

template <bool DENSE, bool LOPA = false>
sffn_status run_mfma_i8(sffn_handle* h, const void* x, const void* W1, const float* s1,
                        const void* W3, const float* s3, const void* W2T, const float* s2,
                        float* y, int T, int32_t* live_count, int32_t* live_idx, hipStream_t s,
                        const void* V = nullptr, const float* sV = nullptr, bool per_token = false) {
    const int nt = token_tiles(T);
    uint8_t* live = live_count ? h->live_buf : nullptr;
    sffn_status st = SFFN_OK;
    uint16_t* t_hi = h->m_t;
    uint16_t* t_lo = h->m_t ? h->m_t + (size_t)h->m_tp * h->r : nullptr;
    if (LOPA) {
        SFFN_NT_SWITCH(nt, st = launch(h, KIND_RANK_PROJ_MFMA_I8, k_rank_proj_mfma_i8<1>,
                                       dim3((h->r + 15) / 16, NT), dim3(KM_THREADS), s,
                                       (const uint16_t*)x, (const int8_t*)V, sV,
                                       (const uint16_t*)h->m_zero, t_hi, t_lo, h->D, h->r, T));
        if (st != SFFN_OK) return st;
    }
    // 32 units per gate block; LoPA above 32 tokens 64 (H' = 9787: 153 blocks in one
    // round against 306 in 1.2 rounds, x staged half as often)
    const int ut = (LOPA && nt == 4) ? 4 : 2;
    const int nb = (h->H + 16 * ut - 1) / (16 * ut);
    const int splits = mfma_down_splits(h, nt);
    float* yz = (per_token || splits > 1) ? y : nullptr;
    if (!LOPA) {
        // W1 and W3 codes of the block and x staged together, x once for both; ahead of
        // the gathered W3 pass at every batch size (union of 5 / 10 tokens, int8 196k /
        // 348k -> 211k / 372k tokens/s, int4 186k / 329k -> 220k / 382k)
        SFFN_NT_SWITCH(nt, st = launch(h, KIND_GATE_UP_MFMA_FUSED_I8,
                                       k_gate_up_mfma_fused_i8<NT, DENSE>, dim3(nb),
                                       dim3(KM_THREADS), s, (const uint16_t*)x, (const int8_t*)W1,
                                       s1, (const int8_t*)W3, s3, s2, (const uint16_t*)h->m_zero,
                                       h->m_a, h->m_mask, live, yz, h->D, h->H, T, h->act,
                                       per_token ? 0 : 1));
    } else {
#define SFFN_GATE_MFMA_I8(NTV, UTV)                                                            \
    st = launch(h, KIND_GATE_UP_MFMA_I8, k_gate_up_mfma_i8<NTV, UTV, DENSE, LOPA>, dim3(nb),   \
                dim3(KM_THREADS), s, (const uint16_t*)x, (const int8_t*)W1, s1,                \
                (const int8_t*)W3, s3, s2, (const uint16_t*)h->m_zero, h->m_a, h->m_mask, live, \
                yz, h->D, h->H, T, h->act, (const uint16_t*)t_hi, (const uint16_t*)t_lo, h->r,  \
                h->flags, per_token ? 0 : 1)
    if (nt == 1) {
        SFFN_GATE_MFMA_I8(1, 2);
    } else if (nt == 2) {
        SFFN_GATE_MFMA_I8(2, 2);
    } else {
        SFFN_GATE_MFMA_I8(4, LOPA ? 4 : 2);
    }
#undef SFFN_GATE_MFMA_I8
    }
    if (st != SFFN_OK) return st;
    const int ntile = (h->D + KDM_NB - 1) / KDM_NB;
    if (per_token)
        st = run_down_pt_q(h, W2T, s2, y, T, 16 * nt, 8, s);
    else
        SFFN_NT_SWITCH(nt, st = launch(h, KIND_DOWN_MFMA_I8, k_down_mfma_i8<NT>, dim3(ntile, splits),
                                       dim3(KDM_THREADS), s, (const float*)h->m_a,
                                       (const uint64_t*)h->m_mask, (const int8_t*)W2T, y, h->D,
                                       h->H, T, splits));
    if (st != SFFN_OK) return st;
    if (!DENSE) return run_live_list(h, T, live_count, live_idx, s);
    return SFFN_OK;
}

// int4 union (and dense) batches of 5..64 tokens on MFMA: every code read once for
// the batch. LOPA: W1 is U (int8 rows, scales s1 = U's), V int8 with sV.
bool mfma_i4_ok(const sffn_handle* h, int T, int min_t = 5) {
    return T >= min_t && h->dtype == SFFN_I4 && h->m_a != nullptr && T <= h->max_tokens;
}

template <bool DENSE, bool LOPA = false>
sffn_status run_mfma_i4(sffn_handle* h, const void* x, const void* W1, const float* s1,
                        const void* W3, const float* s3, const void* W2T, const float* s2,
                        float* y, int T, int32_t* live_count, int32_t* live_idx, hipStream_t s,
                        const void* V = nullptr, const float* sV = nullptr, bool per_token = false) {
    const int nt = token_tiles(T);
    uint8_t* live = live_count ? h->live_buf : nullptr;
    sffn_status st = SFFN_OK;
    uint16_t* t_hi = h->m_t;
    uint16_t* t_lo = h->m_t ? h->m_t + (size_t)h->m_tp * h->r : nullptr;
    if (LOPA) {
        SFFN_NT_SWITCH(nt, st = launch(h, KIND_RANK_PROJ_MFMA_I8, k_rank_proj_mfma_i8<1>,
                                       dim3((h->r + 15) / 16, NT), dim3(KM_THREADS), s,
                                       (const uint16_t*)x, (const int8_t*)V, sV,
                                       (const uint16_t*)h->m_zero, t_hi, t_lo, h->D, h->r, T));
        if (st != SFFN_OK) return st;
    }
    const int nb = (h->H + 31) / 32;
    const int splits = mfma_down_splits(h, nt);
    float* yz = (per_token || splits > 1) ? y : nullptr;
    if (!LOPA) {
        // W1 and W3 codes of the block and x staged together, x once for both; ahead of
        // the gathered W3 pass at every batch size (union of 5 / 10 tokens, int8 196k /
        // 348k -> 211k / 372k tokens/s, int4 186k / 329k -> 220k / 382k)
        SFFN_NT_SWITCH(nt, st = launch(h, KIND_GATE_UP_MFMA_FUSED_I4,
                                       k_gate_up_mfma_fused_i4<NT, DENSE>, dim3(nb),
                                       dim3(KM_THREADS), s, (const uint16_t*)x, (const uint8_t*)W1,
                                       s1, (const uint8_t*)W3, s3, (const uint16_t*)h->m_zero,
                                       h->m_a, h->m_mask, live, yz, h->D, h->H, T, h->act));
    } else {
        SFFN_NT_SWITCH(nt, st = launch(h, KIND_GATE_UP_MFMA_I4, k_gate_up_mfma_i4<NT, DENSE, LOPA>,
                                       dim3(nb), dim3(KM_THREADS), s, (const uint16_t*)x, W1, s1,
                                       (const uint8_t*)W3, s3, (const uint16_t*)h->m_zero, h->m_a,
                                       h->m_mask, live, yz, h->D, h->H, T, h->act,
                                       (const uint16_t*)t_hi, (const uint16_t*)t_lo, h->r,
                                       h->flags));
    }
    if (st != SFFN_OK) return st;
    const int ntile = (h->D + KDM_NB - 1) / KDM_NB;
    if (per_token)
        st = run_down_pt_q(h, W2T, s2, y, T, 16 * nt, 4, s);
    else
        SFFN_NT_SWITCH(nt, st = launch(h, KIND_DOWN_MFMA_I4, k_down_mfma_i4<NT>, dim3(ntile, splits),
                                       dim3(KDM_THREADS), s, (const float*)h->m_a,
                                       (const uint64_t*)h->m_mask, (const uint8_t*)W2T, s2, y,
                                       h->D, h->H, T, splits));
    if (st != SFFN_OK) return st;
    if (!DENSE) return run_live_list(h, T, live_count, live_idx, s);
    return SFFN_OK;
}

// int8 union of a batch of 2..4 tokens (and its dense comparator): W1 and the
// live W3 rows read once for the batch, the down pass over the union
template <bool DENSE>
sffn_status run_i8_tb(sffn_handle* h, const void* x, const void* W1, const float* s1,
                      const void* W3, const float* s3, const void* W2T, const float* s2,
                      float* y, int T, int32_t* live_count, int32_t* live_idx, hipStream_t s,
                      bool per_token = false) {
    const int nc = pick(kNC_T1, 7, (h->D + 1023) / 1024);
    const int rw = DENSE ? 1 : 2;  // units per wave: union calls 2, the dense comparator 1 (measured)
    const int nb = (h->H + K1_WAVES * rw - 1) / (K1_WAVES * rw);
    const int tp = 16 * token_tiles(T);
    const int tt = T <= 2 ? 2 : 4;
    int splits = h->tb_splits;
    while ((h->H + splits - 1) / splits > 32 * KD_THREADS) ++splits;
    uint8_t* live = (!DENSE && live_count) ? h->live_buf : nullptr;
    float* yz = (per_token || splits > 1) ? y : nullptr;
    sffn_status st = SFFN_OK;
#define SFFN_TBQ_GATE(TTV, RWV)                                                                   \
    SFFN_NCT1_SWITCH(nc, st = launch(h, KIND_GATE_UP_TB_I8, k_gate_up_tb_i8<NC, TTV, DENSE, RWV>,  \
                                     dim3(nb), dim3(K1_THREADS), s, (const uint16_t*)x,           \
                                     (const int8_t*)W1, s1, (const int8_t*)W3, s3, s2, h->m_a,     \
                                     h->m_mask, live, yz, h->D, h->H, T, tp, h->act))
#define SFFN_TBQ_RW(TTV)                                                                          \
    if (rw == 2) { SFFN_TBQ_GATE(TTV, 2); }                                                       \
    else { SFFN_TBQ_GATE(TTV, 1); }
    if (tt == 2) { SFFN_TBQ_RW(2); } else { SFFN_TBQ_RW(4); }
#undef SFFN_TBQ_RW
#undef SFFN_TBQ_GATE
    if (st != SFFN_OK) return st;
    if (per_token) {
        st = run_down_pt_q(h, W2T, s2, y, T, tp, 8, s);
        if (st != SFFN_OK) return st;
        return run_live_list(h, T, live_count, live_idx, s);
    }
    const int cb = 16 * 16;
    const int nslices = (h->D + cb - 1) / cb;
    const int nbx = ((nslices + 7) / 8) * 8;
    const int hs = (h->H + splits - 1) / splits;
    const int pmax = pick(kPMAX, 6, (hs + KD_THREADS - 1) / KD_THREADS);
#define SFFN_TBQ_DOWN(TTV)                                                                        \
    SFFN_PMAX_SWITCH(pmax, st = launch(h, KIND_DOWN_TB_I8, k_down_tb_i8<PMAX, TTV>,                \
                                       dim3(nbx, splits), dim3(KD_THREADS), s,                    \
                                       (const float*)h->m_a, (const uint64_t*)h->m_mask,          \
                                       (const int8_t*)W2T, y, h->D, h->H, T, tp, splits))
    if (tt == 2) { SFFN_TBQ_DOWN(2); } else { SFFN_TBQ_DOWN(4); }
#undef SFFN_TBQ_DOWN
    if (st != SFFN_OK) return st;
    if (DENSE) return SFFN_OK;
    return run_live_list(h, T, live_count, live_idx, s);
}

// int4 union of a batch of 2..4 tokens (and its dense comparator)
template <bool DENSE>
sffn_status run_i4_tb(sffn_handle* h, const void* x, const void* W1, const float* s1,
                      const void* W3, const float* s3, const void* W2T, const float* s2,
                      float* y, int T, int32_t* live_count, int32_t* live_idx, hipStream_t s,
                      bool per_token = false) {
    const int nc = (h->D + 2047) / 2048;
    const int rw = DENSE ? 1 : 2;  // as for int8
    const int nb = (h->H + K1_WAVES * rw - 1) / (K1_WAVES * rw);
    const int tp = 16 * token_tiles(T);
    const int tt = T <= 2 ? 2 : 4;
    int splits = h->tb_splits;
    while ((h->H + splits - 1) / splits > 32 * KD_THREADS) ++splits;
    uint8_t* live = (!DENSE && live_count) ? h->live_buf : nullptr;
    float* yz = (per_token || splits > 1) ? y : nullptr;
    sffn_status st = SFFN_OK;
#define SFFN_TB4_GATE(NCV, TTV)                                                                   \
    if (rw == 2)                                                                                  \
        st = launch(h, KIND_GATE_UP_TB_I4, k_gate_up_tb_i4<NCV, TTV, DENSE, 2>, dim3(nb),         \
                    dim3(K1_THREADS), s, (const uint16_t*)x, (const uint8_t*)W1, s1,             \
                    (const uint8_t*)W3, s3, h->m_a, h->m_mask, live, yz, h->D, h->H, T, tp, h->act);\
    else                                                                                          \
        st = launch(h, KIND_GATE_UP_TB_I4, k_gate_up_tb_i4<NCV, TTV, DENSE, 1>, dim3(nb),         \
                    dim3(K1_THREADS), s, (const uint16_t*)x, (const uint8_t*)W1, s1,             \
                    (const uint8_t*)W3, s3, h->m_a, h->m_mask, live, yz, h->D, h->H, T, tp, h->act)
#define SFFN_TB4_NC(TTV)                                                                          \
    switch (nc) {                                                                                 \
        case 1: SFFN_TB4_GATE(1, TTV); break;                                                     \
        case 2: SFFN_TB4_GATE(2, TTV); break;                                                     \
        case 3: SFFN_TB4_GATE(3, TTV); break;                                                     \
        case 4: SFFN_TB4_GATE(4, TTV); break;                                                     \
        default: return fail(h, SFFN_INTERNAL, "no int4 batch gate kernel for this width");      \
    }
    if (tt == 2) { SFFN_TB4_NC(2); } else { SFFN_TB4_NC(4); }
#undef SFFN_TB4_NC
#undef SFFN_TB4_GATE
    if (st != SFFN_OK) return st;
    if (per_token) {
        st = run_down_pt_q(h, W2T, s2, y, T, tp, 4, s);
        if (st != SFFN_OK) return st;
        return run_live_list(h, T, live_count, live_idx, s);
    }
    const int cb = 16 * 16;
    const int nslices = (h->D + cb - 1) / cb;
    const int nbx = ((nslices + 7) / 8) * 8;
    const int hs = (h->H + splits - 1) / splits;
    const int pmax = pick(kPMAX, 6, (hs + KD_THREADS - 1) / KD_THREADS);
#define SFFN_TB4_DOWN(TTV)                                                                        \
    SFFN_PMAX_SWITCH(pmax, st = launch(h, KIND_DOWN_TB_I4, k_down_tb_i4<PMAX, TTV>,                \
                                       dim3(nbx, splits), dim3(KD_THREADS), s,                    \
                                       (const float*)h->m_a, (const uint64_t*)h->m_mask,          \
                                       (const uint8_t*)W2T, s2, y, h->D, h->H, T, tp, splits))
    if (tt == 2) { SFFN_TB4_DOWN(2); } else { SFFN_TB4_DOWN(4); }
#undef SFFN_TB4_DOWN
    if (st != SFFN_OK) return st;
    if (DENSE) return SFFN_OK;
    return run_live_list(h, T, live_count, live_idx, s);
}

// int4 down pass over a_buf (group scales applied per 32-column piece)
sffn_status run_down_t1_i4(sffn_handle* h, const void* W2T, const float* s2, float* y, int splits,
                           bool dense, hipStream_t s) {
    const int cb = 8 * 32;
    const int nslices = (h->D + cb - 1) / cb;
    const int nbx = ((nslices + 7) / 8) * 8;
    const int hs = (h->H + splits - 1) / splits;
    const int pmax = pick(kPMAX, 6, (hs + KD_THREADS - 1) / KD_THREADS);
    sffn_status st = SFFN_OK;
    SFFN_PMAX_SWITCH(pmax, st = launch(h, KIND_DOWN_T1_I4, k_down_t1_i4<PMAX>, dim3(nbx, splits),
                                       dim3(KD_THREADS), s, (const float*)h->a_buf,
                                       (const uint8_t*)W2T, s2, y, h->D, h->H, splits,
                                       dense ? 1 : 0));
    return st;
}

// batch-1 int4 (group-scaled) standard gating
template <bool DENSE>
sffn_status run_i4_t1(sffn_handle* h, const void* x, const void* W1, const float* s1,
                      const void* W3, const float* s3, const void* W2T, const float* s2,
                      float* y, int32_t* live_count, int32_t* live_idx, hipStream_t s) {
    const int nc = (h->D + 2047) / 2048;
    const int nb = (h->H + K1_WAVES - 1) / K1_WAVES;
    int splits = h->t1_splits;
    while ((h->H + splits - 1) / splits > 32 * KD_THREADS) ++splits;
    uint8_t* live = (!DENSE && live_count) ? h->live_buf : nullptr;
    float* yz = splits > 1 ? y : nullptr;
    sffn_status st = SFFN_OK;
#define SFFN_I4_GATE(NCV)                                                                         \
    st = launch(h, DENSE ? KIND_GATE_UP_DENSE_T1_I4 : KIND_GATE_UP_T1_I4,                        \
                k_gate_up_t1_i4<NCV, DENSE>, dim3(nb), dim3(K1_THREADS), s, (const uint16_t*)x,   \
                (const uint8_t*)W1, s1, (const uint8_t*)W3, s3, h->a_buf, live, yz, h->D, h->H,   \
                h->act)
    switch (nc) {
        case 1: SFFN_I4_GATE(1); break;
        case 2: SFFN_I4_GATE(2); break;
        case 3: SFFN_I4_GATE(3); break;
        case 4: SFFN_I4_GATE(4); break;
        default: return fail(h, SFFN_INTERNAL, "no int4 gate kernel for this width");
    }
#undef SFFN_I4_GATE
    if (st != SFFN_OK) return st;
    st = run_down_t1_i4(h, W2T, s2, y, splits, DENSE, s);
    if (st != SFFN_OK) return st;
    if (DENSE) return SFFN_OK;
    return run_live_list(h, 1, live_count, live_idx, s);
}

// batch-1 LoPA with int8 V and U rows and group-scaled int4 W3 and W2T rows
sffn_status run_lopa_i4_t1(sffn_handle* h, const void* x, const void* V, const float* sV,
                           const void* U, const float* sU, const void* W3, const float* s3,
                           const void* W2T, const float* s2, float* y, int32_t* live_count,
                           int32_t* live_idx, hipStream_t s) {
    int splits = h->t1_splits;
    while ((h->H + splits - 1) / splits > 32 * KD_THREADS) ++splits;
    float* yz = splits > 1 ? y : nullptr;
    uint8_t* live = live_count ? h->live_buf : nullptr;
    sffn_status st = SFFN_OK;
    const int nc8 = pick(kNC_T1, 7, (h->D + 1023) / 1024);
    const int nbr = (h->r + K1_WAVES - 1) / K1_WAVES;
    SFFN_NCT1_SWITCH(nc8, st = launch(h, KIND_RANK_PROJ_T1_I8, k_rank_proj_t1_i8<NC>, dim3(nbr),
                                      dim3(K1_THREADS), s, (const uint16_t*)x, (const int8_t*)V,
                                      sV, h->t_buf, yz, h->D, h->r));
    if (st != SFFN_OK) return st;
    const int nb = (h->H + K1_WAVES * KLQ_UPW - 1) / (K1_WAVES * KLQ_UPW);
    const int nr = (h->r + 255) / 256;
    const int nc = (h->D + 2047) / 2048;
#define SFFN_LOPA_I4(NCV, NRV)                                                                    \
    st = launch(h, KIND_GATE_UP_LOPA_T1_I4, k_gate_up_lopa_t1_i4<NCV, NRV>, dim3(nb),             \
                dim3(K1_THREADS), s, (const uint16_t*)x, (const float*)h->t_buf, (const int8_t*)U, \
                sU, (const uint8_t*)W3, s3, h->a_buf, live, h->D, h->H, h->r, h->act, h->flags)
#define SFFN_LOPA_I4_NR(NCV)                                                                      \
    switch (nr) {                                                                                 \
        case 1: SFFN_LOPA_I4(NCV, 1); break;                                                      \
        case 2: SFFN_LOPA_I4(NCV, 2); break;                                                      \
        case 3: SFFN_LOPA_I4(NCV, 3); break;                                                      \
        case 4: SFFN_LOPA_I4(NCV, 4); break;                                                      \
        case 5: SFFN_LOPA_I4(NCV, 5); break;                                                      \
        case 6: SFFN_LOPA_I4(NCV, 6); break;                                                      \
        case 7: SFFN_LOPA_I4(NCV, 7); break;                                                      \
        case 8: SFFN_LOPA_I4(NCV, 8); break;                                                      \
        default: return fail(h, SFFN_INTERNAL, "rank too large for the int4 LoPA gate");          \
    }
    switch (nc) {
        case 1: SFFN_LOPA_I4_NR(1); break;
        case 2: SFFN_LOPA_I4_NR(2); break;
        case 3: SFFN_LOPA_I4_NR(3); break;
        case 4: SFFN_LOPA_I4_NR(4); break;
        default: return fail(h, SFFN_INTERNAL, "no int4 LoPA gate kernel for this width");
    }
#undef SFFN_LOPA_I4_NR
#undef SFFN_LOPA_I4
    if (st != SFFN_OK) return st;
    st = run_down_t1_i4(h, W2T, s2, y, splits, false, s);
    if (st != SFFN_OK) return st;
    return run_live_list(h, 1, live_count, live_idx, s);
}

// batch-1 LoPA with int8 V, U, W3, W2T rows
sffn_status run_lopa_i8_t1(sffn_handle* h, const void* x, const void* V, const float* sV,
                           const void* U, const float* sU, const void* W3, const float* s3,
                           const void* W2T, const float* s2, float* y, int32_t* live_count,
                           int32_t* live_idx, hipStream_t s) {
    const int nc = pick(kNC_T1, 7, (h->D + 1023) / 1024);
    int splits = h->t1_splits;
    while ((h->H + splits - 1) / splits > 32 * KD_THREADS) ++splits;
    float* yz = splits > 1 ? y : nullptr;
    uint8_t* live = live_count ? h->live_buf : nullptr;
    sffn_status st = SFFN_OK;
    const int nbr = (h->r + K1_WAVES - 1) / K1_WAVES;
    SFFN_NCT1_SWITCH(nc, st = launch(h, KIND_RANK_PROJ_T1_I8, k_rank_proj_t1_i8<NC>, dim3(nbr),
                                     dim3(K1_THREADS), s, (const uint16_t*)x, (const int8_t*)V,
                                     sV, h->t_buf, yz, h->D, h->r));
    if (st != SFFN_OK) return st;
    // two units per wave (32 lanes per U row) up to r = 1024, four (16 lanes) above
    const int upw = h->r <= 1024 ? 2 : 4;
    const int nb = (h->H + K1_WAVES * upw - 1) / (K1_WAVES * upw);
    const int nr = (h->r + 16 * (64 / upw) - 1) / (16 * (64 / upw));
#define SFFN_LOPA_I8(NRV, UPWV)                                                                    \
    SFFN_NCT1_SWITCH(nc, st = launch(h, KIND_GATE_UP_LOPA_T1_I8, k_gate_up_lopa_t1_i8<NC, NRV, UPWV>,\
                                     dim3(nb), dim3(K1_THREADS), s, (const uint16_t*)x,           \
                                     (const float*)h->t_buf, (const int8_t*)U, sU,                 \
                                     (const int8_t*)W3, s3, s2, h->a_buf, live, h->D, h->H, h->r,  \
                                     h->act, h->flags))
    if (upw == 2) {
        switch (nr) {
            case 1: SFFN_LOPA_I8(1, 2); break;
            case 2: SFFN_LOPA_I8(2, 2); break;
            default: return fail(h, SFFN_INTERNAL, "rank too large for the int8 LoPA gate");
        }
    } else {
        switch (nr) {
            case 1: SFFN_LOPA_I8(1, 4); break;
            case 2: SFFN_LOPA_I8(2, 4); break;
            case 3: SFFN_LOPA_I8(3, 4); break;
            case 4: SFFN_LOPA_I8(4, 4); break;
            case 5: SFFN_LOPA_I8(5, 4); break;
            case 6: SFFN_LOPA_I8(6, 4); break;
            case 7: SFFN_LOPA_I8(7, 4); break;
            case 8: SFFN_LOPA_I8(8, 4); break;
            default: return fail(h, SFFN_INTERNAL, "rank too large for the int8 LoPA gate");
        }
    }
#undef SFFN_LOPA_I8
    if (st != SFFN_OK) return st;
    st = run_down_t1_i8(h, W2T, y, splits, false, s);
    if (st != SFFN_OK) return st;
    return run_live_list(h, 1, live_count, live_idx, s);
}

// Launch plan of a checked sparse / dense call (no argument checks).
sffn_status dispatch_sparse(sffn_handle* h, const void* x, const void* W1, const void* W3,
                            const void* W2T, float* y, int T, int mode, int32_t* live_count,
                            int32_t* live_idx, hipStream_t s) {
    sffn_status st = SFFN_OK;
    if (T == 0) return SFFN_OK;
    if (t1_ok(h, T)) return run_sparse_t1(h, x, W1, W3, W2T, y, live_count, live_idx, s);
    if (mode == SFFN_MODE_PER_TOKEN && mfma_ok(h, T) && T <= MAXT && t1_ok(h, 1))
        // per-token lists: one batched gate and up pass (W1 read once for the batch),
        // then each token gathers the W2T rows of its own live list
        return run_mfma<false>(h, x, W1, W3, W2T, y, T, live_count, live_idx, s, nullptr, true);
    if (mode == SFFN_MODE_PER_TOKEN && gemm_ok(h, T))
        // above 64 tokens every unit is live for some token in practice (1 - s^T), so
        // per-token gathers would read nearly every row once per token: the batch takes
        // the union GEMMs (same result; the live lists are still per token)
        return run_gemm<false>(h, x, W1, W3, W2T, y, T, live_count, live_idx, s);
    if (mode == SFFN_MODE_PER_TOKEN && t1_ok(h, 1)) {
        // per-token lists above 64 tokens on handles without the GEMM path (standard
        // gating in fp32): every token runs the whole batch-1 pass on its own live set
        const size_t xb = (size_t)h->D * sizeof(uint16_t);
        for (int t = 0; t < T; ++t) {
            st = run_sparse_t1(h, (const char*)x + t * xb, W1, W3, W2T, y + (size_t)t * h->D,
                               live_count ? live_count + t : nullptr,
                               live_idx ? live_idx + (size_t)t * h->H : nullptr, s);
            if (st != SFFN_OK) return st;
        }
        return SFFN_OK;
    }
    if (mode == SFFN_MODE_UNION && gemm_ok(h, T))
        return run_gemm<false>(h, x, W1, W3, W2T, y, T, live_count, live_idx, s);
    if (mode == SFFN_MODE_UNION && mfma_ok(h, T) && T <= MAXT)
        return run_mfma<false>(h, x, W1, W3, W2T, y, T, live_count, live_idx, s);
    if (T > MAXT)
        return fail(h, SFFN_UNSUPPORTED, "no launch plan for this batch size and mode");
    return h->dtype == SFFN_BF16
               ? run_sparse<uint16_t>(h, x, W1, W3, W2T, y, T, mode, live_count, live_idx, s)
               : run_sparse<float>(h, x, W1, W3, W2T, y, T, mode, live_count, live_idx, s);
}

sffn_status dispatch_dense(sffn_handle* h, const void* x, const void* W1, const void* W3,
                           const void* W2T, float* y, int T, hipStream_t s) {
    if (T == 0) return SFFN_OK;
    if (t1_ok(h, T)) return run_dense_t1(h, x, W1, W3, W2T, y, s);
    if (gemm_ok(h, T)) return run_gemm<true>(h, x, W1, W3, W2T, y, T, nullptr, nullptr, s);
    if (mfma_ok(h, T) && T <= MAXT)
        return run_mfma<true>(h, x, W1, W3, W2T, y, T, nullptr, nullptr, s);
    if (T > MAXT) return fail(h, SFFN_UNSUPPORTED, "no launch plan for this batch size");
    return h->dtype == SFFN_BF16 ? run_dense<uint16_t>(h, x, W1, W3, W2T, y, T, s)
                                 : run_dense<float>(h, x, W1, W3, W2T, y, T, s);
}

sffn_status check_common(sffn_handle* h, const void* x, const void* W3, const void* W2T,
                         const float* y, int T, int32_t* live_count, int32_t* live_idx,
                         hipStream_t* stream_out, void* stream) {
    if (!h) return fail(nullptr, SFFN_INVALID_ARGUMENT, "null handle");
    if (T < 0 || T > h->max_tokens)
        return fail(h, SFFN_INVALID_ARGUMENT,
                    "T=" + std::to_string(T) + " outside [0, max_tokens=" +
                        std::to_string(h->max_tokens) + "]");
    if (!x || !W3 || !W2T || !y) return fail(h, SFFN_INVALID_ARGUMENT, "null tensor pointer");
    if (!aligned16(x) || !aligned16(W3) || !aligned16(W2T) || !aligned16(y))
        return fail(h, SFFN_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
    if ((live_count == nullptr) != (live_idx == nullptr))
        return fail(h, SFFN_INVALID_ARGUMENT, "live_count and live_idx must be both set or both NULL");
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(h, e, "hipGetDevice");
    if (dev != h->device)
        return fail(h, SFFN_INVALID_ARGUMENT, "current device differs from the handle's device");
    *stream_out = reinterpret_cast<hipStream_t>(stream);
    h->timed_call = h->timing_every > 0 && (h->call_seq++ % h->timing_every) == 0;
    return SFFN_OK;
}

}  // namespace

extern "C" {

int sffn_abi_version(void) { return 1; }

const char* sffn_status_string(sffn_status s) {
    switch (s) {
        case SFFN_OK: return "SFFN_OK";
        case SFFN_INVALID_ARGUMENT: return "SFFN_INVALID_ARGUMENT";
        case SFFN_UNSUPPORTED: return "SFFN_UNSUPPORTED";
        case SFFN_OUT_OF_MEMORY: return "SFFN_OUT_OF_MEMORY";
        case SFFN_HIP_ERROR: return "SFFN_HIP_ERROR";
        case SFFN_INTERNAL: return "SFFN_INTERNAL";
        default: return "unknown status";
    }
}

const char* sffn_last_error(const sffn_handle* h) {
    return h ? h->err.c_str() : g_thread_error.c_str();
}

sffn_status sffn_create(sffn_handle** out, int D, int H, int r, int max_tokens, int act,
                        int dtype, unsigned flags) {
    try {
        if (!out) return fail(nullptr, SFFN_INVALID_ARGUMENT, "out is NULL");
        *out = nullptr;
        if (act != SFFN_ACT_RELU && act != SFFN_ACT_RSPLUS)
            return fail(nullptr, SFFN_UNSUPPORTED, "unknown activation " + std::to_string(act));
        if (dtype != SFFN_BF16 && dtype != SFFN_F32 && dtype != SFFN_I8 && dtype != SFFN_I4)
            return fail(nullptr, SFFN_UNSUPPORTED, "unknown dtype " + std::to_string(dtype));
        if (dtype == SFFN_I4 && r != 0 && r % 16 != 0)
            return fail(nullptr, SFFN_INVALID_ARGUMENT, "int4 LoPA weights: r must be a multiple of 16");
        if (dtype == SFFN_I4 && D % 128 != 0)
            return fail(nullptr, SFFN_INVALID_ARGUMENT, "int4 weights: D must be a multiple of 128");
        if (dtype == SFFN_I4 && (H + KD_THREADS - 1) / KD_THREADS > 32 * 16)
            return fail(nullptr, SFFN_INVALID_ARGUMENT, "int4 weights: H too large");
        if (dtype == SFFN_I8 && r != 0 && r % 16 != 0)
            return fail(nullptr, SFFN_INVALID_ARGUMENT, "int8 weights: r must be a multiple of 16");
        if (dtype == SFFN_I8 && D % 16 != 0)
            return fail(nullptr, SFFN_INVALID_ARGUMENT, "int8 weights: D must be a multiple of 16");
        if (dtype == SFFN_I8 && (H + KD_THREADS - 1) / KD_THREADS > 32 * 16)
            return fail(nullptr, SFFN_INVALID_ARGUMENT, "int8 weights: H too large");
        const unsigned known = SFFN_FLAG_G_TILED | SFFN_FLAG_RMSNORM | SFFN_FLAG_DOUBLE_ACT;
        if (flags & ~known) return fail(nullptr, SFFN_UNSUPPORTED, "unknown flag bits");
        if (flags != 0 && r == 0)
            return fail(nullptr, SFFN_UNSUPPORTED, "the gate flags apply to LoPA handles (r > 0) only");
        const int dmax = dtype == SFFN_F32 ? 4096 : 8192;
        if (D <= 0 || D % 8 != 0 || D > dmax)
            return fail(nullptr, SFFN_INVALID_ARGUMENT,
                        "D must be a positive multiple of 8, at most " + std::to_string(dmax));
        if (H <= 0 || H > (1 << 20))
            return fail(nullptr, SFFN_INVALID_ARGUMENT, "H must be in [1, 2^20]");
        if (r != 0 && (r < 8 || r % 8 != 0 || r > 2048))
            return fail(nullptr, SFFN_INVALID_ARGUMENT,
                        "r must be 0 or a multiple of 8 in [8, 2048]");
        const bool big_ok = dtype == SFFN_BF16 && r == 0;
        if (max_tokens < 1 || max_tokens > (big_ok ? MAXT_GEMM : MAXT))
            return fail(nullptr, SFFN_INVALID_ARGUMENT,
                        big_ok ? "max_tokens must be in [1, 8192]"
                               : "max_tokens must be in [1, 64] for this dtype and gate");

        sffn_handle* h = new (std::nothrow) sffn_handle();
        if (!h) return fail(nullptr, SFFN_OUT_OF_MEMORY, "host allocation failed");
        h->D = D; h->H = H; h->r = r; h->max_tokens = max_tokens; h->act = act;
        h->dtype = dtype; h->flags = flags;
        hipError_t e = hipGetDevice(&h->device);
        if (e != hipSuccess) {
            delete h;
            return fail(nullptr, SFFN_HIP_ERROR, std::string("hipGetDevice: ") + hipGetErrorString(e));
        }
        const size_t th = (size_t)max_tokens * (size_t)H;
        const size_t th_small = (size_t)std::min(max_tokens, MAXT) * (size_t)H;
        e = hipMalloc(&h->a_buf, th_small * sizeof(float));
        if (e == hipSuccess) e = hipMalloc(&h->live_buf, th);
        if (e == hipSuccess && r > 0) e = hipMalloc(&h->t_buf, (size_t)max_tokens * r * sizeof(float));
        if (e != hipSuccess) {
            sffn_destroy(h);
            return fail(nullptr, e == hipErrorOutOfMemory ? SFFN_OUT_OF_MEMORY : SFFN_HIP_ERROR,
                        std::string("scratch allocation: ") + hipGetErrorString(e));
        }
        // launch plan: enough gate/up blocks of the general kernels to cover the 256
        // CUs several times over
        int rpw = 4;
        while (rpw > 1 && (H + rpw * K1_WAVES - 1) / (rpw * K1_WAVES) < 1024) rpw /= 2;
        h->gate_rows_per_wave = rpw;
        // batch-1 (and per-token) down passes: 16 unit ranges, more when a range would
        // exceed what one block's waves hold (32 x 512 units); bf16 ranges of at most
        // 512 units (one group of 64 per wave, one round of row loads) up to 64 ranges
        // (more ranges add same-address atomics to y)
        if (dtype == SFFN_BF16)
            while ((H + h->t1_splits - 1) / h->t1_splits > KD_THREADS && h->t1_splits < 64)
                ++h->t1_splits;
        while ((H + h->t1_splits - 1) / h->t1_splits > 32 * KD_THREADS) ++h->t1_splits;
        // fused batch-1 dense comparator: about one block per two CUs (128 blocks),
        // at most 8 units per wave
        if (dtype == SFFN_BF16 && D <= KF_DMAX) {
            int rpb = (H + 127) / 128;
            // keep the W1 tiles of a wave (units x register chunks) within 32 x 16 bytes per lane
            const int ncf = pick(kNC_T1, 7, chunks_needed(D, dtype));
            int rw_max = 1;
            while (rw_max * 2 <= 8 && rw_max * 2 * ncf <= 32) rw_max *= 2;
            if (rpb > KF_WAVES * rw_max) rpb = KF_WAVES * rw_max;
            int rw = 1;
            while (rw * KF_WAVES < rpb) rw *= 2;
            h->f_rows_per_block = rpb;
            h->f_rw = rw;
            h->f_blocks = (H + rpb - 1) / rpb;
            e = hipMalloc(&h->part_buf, (size_t)h->f_blocks * D * sizeof(float));
            if (e != hipSuccess) {
                sffn_destroy(h);
                return fail(nullptr, SFFN_OUT_OF_MEMORY, std::string("scratch allocation: ") + hipGetErrorString(e));
            }
            if (prepare_fused(h) != SFFN_OK) {
                std::string m = h->err;
                sffn_destroy(h);
                return fail(nullptr, SFFN_HIP_ERROR, m);
            }
        }
        // scratch that must start zeroed is cleared on a private stream of the
        // handle's own, which create waits for (no device-wide synchronisation)
        hipStream_t init = nullptr;
        e = hipStreamCreateWithFlags(&init, hipStreamNonBlocking);
        if (e != hipSuccess) {
            sffn_destroy(h);
            return fail(nullptr, SFFN_HIP_ERROR, std::string("hipStreamCreateWithFlags: ") + hipGetErrorString(e));
        }
        auto finish_init = [&](hipError_t err) {
            hipError_t e2 = hipStreamSynchronize(init);
            (void)hipStreamDestroy(init);
            return err != hipSuccess ? err : e2;
        };
        // batch plans: unit-major products for up to 16*ceil(max_tokens/16) tokens (bf16
        // MFMA and VALU batches, int8 and int4 VALU batches)
        if ((dtype == SFFN_BF16 || dtype == SFFN_I8 || dtype == SFFN_I4) && max_tokens >= 2) {
            h->m_tp = 16 * token_tiles(max_tokens);
            while ((H + h->m_splits - 1) / h->m_splits > KDM_LCAP) ++h->m_splits;
            // up to 32 tokens the down pass runs at one block per CU (measured ahead of
            // the 16 ranges that put two blocks on some CUs: union of 8 / 17 / 32 tokens
            // 272k / 455k / 814k -> 292k / 504k / 885k tokens/s at D=2560, H=7168); above
            // that the 16 ranges stay ahead
            int ncu = 256;
            if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, h->device) != hipSuccess || ncu < 1)
                ncu = 256;
            h->m_splits_s = std::max(1, ncu / ((D + KDM_NB - 1) / KDM_NB));
            while ((H + h->m_splits_s - 1) / h->m_splits_s > KDM_LCAP) ++h->m_splits_s;
            // bf16: ranges of at most 512 units, as for the batch-1 pass (up to 64)
            if (dtype == SFFN_BF16)
                while ((H + h->tb_splits - 1) / h->tb_splits > KD_THREADS && h->tb_splits < 64)
                    ++h->tb_splits;
            while ((H + h->tb_splits - 1) / h->tb_splits > 32 * KD_THREADS) ++h->tb_splits;
            e = hipMalloc(&h->m_a, (size_t)H * h->m_tp * sizeof(float));
            if (e == hipSuccess) e = hipMalloc(&h->m_mask, (size_t)H * sizeof(uint64_t));
            if (e == hipSuccess && r > 0)
                e = hipMalloc(&h->m_t, 2 * (size_t)h->m_tp * r * sizeof(uint16_t));
            if (e == hipSuccess) e = hipMalloc(&h->m_zero, 4096);
            if (e == hipSuccess) e = hipMemsetAsync(h->m_zero, 0, 4096, init);
            if (e != hipSuccess) {
                (void)finish_init(e);
                sffn_destroy(h);
                return fail(nullptr, SFFN_OUT_OF_MEMORY, std::string("scratch allocation: ") + hipGetErrorString(e));
            }
        }
        if (dtype == SFFN_BF16 && r == 0 && h->m_zero && max_tokens > MAXT) {
            // large batches as GEMMs: bf16 unit products for up to g_tp tokens
            h->g_tp = 256 * ((max_tokens + 255) / 256);
            const int ntt = h->g_tp / 128;  // token tiles of 128 (batches up to 256) or 256
            e = hipMalloc(&h->g_a, (size_t)H * h->g_tp * sizeof(uint16_t));
            // one 64-bit mask per 64 units of each gate tile (tiles of 64 or 128 units)
            const size_t nm = 2 * (((size_t)H + 127) / 128);
            if (e == hipSuccess) e = hipMalloc(&h->g_any, (size_t)ntt * nm * sizeof(uint64_t));
            if (e == hipSuccess) e = hipMalloc(&h->g_list, ((size_t)H + 33) * sizeof(int32_t));
            if (e == hipSuccess) e = hipMemsetAsync(h->g_list, 0, ((size_t)H + 33) * sizeof(int32_t), init);
            if (e == hipSuccess && max_tokens >= BLT_MIN_T) e = hipMalloc(&h->blt_ws, BLT_WS);
            if (e != hipSuccess) {
                (void)finish_init(e);
                sffn_destroy(h);
                return fail(nullptr, SFFN_OUT_OF_MEMORY, std::string("scratch allocation: ") + hipGetErrorString(e));
            }
            if (max_tokens >= BLT_MIN_T) {
                const hipblasStatus_t bs = hipblasLtCreate(&h->blt);
                if (bs != HIPBLAS_STATUS_SUCCESS) {
                    h->blt = nullptr;
                    (void)finish_init(hipSuccess);
                    sffn_destroy(h);
                    return fail(nullptr, SFFN_HIP_ERROR, "hipblasLtCreate: status " + std::to_string((int)bs));
                }
            }
        }
        e = finish_init(hipSuccess);
        if (e != hipSuccess) {
            sffn_destroy(h);
            return fail(nullptr, SFFN_HIP_ERROR, std::string("scratch initialisation: ") + hipGetErrorString(e));
        }
        if (dtype == SFFN_BF16 && r == 0) {
            const size_t rows = 2 * (size_t)std::min(max_tokens, MAXT);
            e = hipMalloc(&h->moe_x, rows * D * sizeof(uint16_t));
            if (e == hipSuccess) e = hipMalloc(&h->moe_y, rows * D * sizeof(float));
            if (e != hipSuccess) {
                sffn_destroy(h);
                return fail(nullptr, SFFN_OUT_OF_MEMORY, std::string("scratch allocation: ") + hipGetErrorString(e));
            }
        }
        *out = h;
        return SFFN_OK;
    } catch (...) {
        return fail(nullptr, SFFN_INTERNAL, "exception in sffn_create");
    }
}

void sffn_destroy(sffn_handle* h) {
    if (!h) return;
    for (auto& r : h->pending) {
        (void)hipEventDestroy(r.start);
        (void)hipEventDestroy(r.stop);
    }
    for (auto e : h->pool) (void)hipEventDestroy(e);
    if (h->a_buf) (void)hipFree(h->a_buf);
    if (h->live_buf) (void)hipFree(h->live_buf);
    if (h->t_buf) (void)hipFree(h->t_buf);
    if (h->part_buf) (void)hipFree(h->part_buf);
    if (h->m_a) (void)hipFree(h->m_a);
    if (h->m_mask) (void)hipFree(h->m_mask);
    if (h->m_zero) (void)hipFree(h->m_zero);
    if (h->m_t) (void)hipFree(h->m_t);
    if (h->moe_x) (void)hipFree(h->moe_x);
    if (h->moe_y) (void)hipFree(h->moe_y);
    if (h->g_a) (void)hipFree(h->g_a);
    if (h->g_any) (void)hipFree(h->g_any);
    if (h->g_list) (void)hipFree(h->g_list);
    for (auto& p : h->blt_plans) blt_plan_free(p);
    h->blt_plans.clear();
    if (h->blt) (void)hipblasLtDestroy(h->blt);
    if (h->blt_ws) (void)hipFree(h->blt_ws);

    delete h;
}

sffn_status sffn_forward_dense(sffn_handle* h, const void* x, const void* W1, const void* W3,
                               const void* W2T, float* y, int T, void* stream) {
    try {
        hipStream_t s;
        sffn_status st = check_common(h, x, W3, W2T, y, T, nullptr, nullptr, &s, stream);
        if (st != SFFN_OK) return st;
        if (h->dtype == SFFN_I8 || h->dtype == SFFN_I4)
            return fail(h, SFFN_INVALID_ARGUMENT, "int8 and int4 handles take the _i8 / _i4 forward calls");
        if (h->r != 0) return fail(h, SFFN_INVALID_ARGUMENT, "dense forward needs a standard-gating handle (r == 0)");
        if (!W1) return fail(h, SFFN_INVALID_ARGUMENT, "null W1");
        if (!aligned16(W1)) return fail(h, SFFN_INVALID_ARGUMENT, "W1 must be 16-byte aligned");
        return dispatch_dense(h, x, W1, W3, W2T, y, T, s);
    } catch (...) {
        return fail(h, SFFN_INTERNAL, "exception in sffn_forward_dense");
    }
}

sffn_status sffn_forward_moe(sffn_handle* h, const void* x, int E, const void* const* W1,
                             const void* const* W3, const void* const* W2T, int K,
                             const int32_t* route, const float* gate, float* y, int T, int dense,
                             void* stream) {
    try {
        if (!h) return fail(nullptr, SFFN_INVALID_ARGUMENT, "null handle");
        if (h->dtype != SFFN_BF16 || h->r != 0 || !h->moe_x)
            return fail(h, SFFN_INVALID_ARGUMENT, "mixture of experts needs a bf16 standard-gating handle");
        if (E < 1 || E > 1024) return fail(h, SFFN_INVALID_ARGUMENT, "E must be in [1, 1024]");
        if (K < 1 || K > 2) return fail(h, SFFN_INVALID_ARGUMENT, "K must be 1 or 2");
        if (!W1 || !W3 || !W2T || !route || !gate)
            return fail(h, SFFN_INVALID_ARGUMENT, "null expert table or routing array");
        hipStream_t s;
        // check_common validates x, y, T, the device; expert weights are checked below
        sffn_status st = check_common(h, x, h->moe_x, h->moe_y, y, T, nullptr, nullptr, &s, stream);
        if (st != SFFN_OK) return st;
        if (T == 0) return SFFN_OK;
        if (T * K > MOE_MAX_SLOTS)
            return fail(h, SFFN_INVALID_ARGUMENT, "T * K must be at most 128");
        for (int i = 0; i < T * K; ++i)
            if (route[i] < 0 || route[i] >= E)
                return fail(h, SFFN_INVALID_ARGUMENT, "route entry outside [0, E)");
        // slots in expert order; within an expert, tokens ascending
        MoeGather g{};
        MoeCombine c{};
        std::vector<int> first(E + 1, 0);
        for (int i = 0; i < T * K; ++i) ++first[route[i] + 1];
        for (int e = 0; e < E; ++e) first[e + 1] += first[e];
        std::vector<int> next(first.begin(), first.end() - 1);
        for (int t = 0; t < T; ++t)
            for (int k = 0; k < K; ++k) {
                const int e = route[t * K + k];
                const int slot = next[e]++;
                g.src[slot] = (int16_t)t;
                c.slot[t * K + k] = (int16_t)slot;
                c.gate[t * K + k] = gate[t * K + k];
            }
        for (int e = 0; e < E; ++e) {
            if (first[e + 1] == first[e]) continue;
            if (!W1[e] || !W3[e] || !W2T[e])
                return fail(h, SFFN_INVALID_ARGUMENT, "null weight pointer of a routed expert");
            if (!aligned16(W1[e]) || !aligned16(W3[e]) || !aligned16(W2T[e]))
                return fail(h, SFFN_INVALID_ARGUMENT, "expert weights must be 16-byte aligned");
        }
        st = launch(h, KIND_MOE_GATHER, k_moe_gather, dim3(T * K), dim3(256), s,
                    (const uint16_t*)x, h->moe_x, h->D, g);
        if (st != SFFN_OK) return st;
        for (int e = 0; e < E; ++e) {
            const int n = first[e + 1] - first[e];
            if (n == 0) continue;
            const uint16_t* xe = h->moe_x + (size_t)first[e] * h->D;
            float* ye = h->moe_y + (size_t)first[e] * h->D;
            st = dense ? dispatch_dense(h, xe, W1[e], W3[e], W2T[e], ye, n, s)
                       : dispatch_sparse(h, xe, W1[e], W3[e], W2T[e], ye, n, SFFN_MODE_UNION,
                                         nullptr, nullptr, s);
            if (st != SFFN_OK) return st;
        }
        return launch(h, KIND_MOE_COMBINE, k_moe_combine, dim3(T), dim3(256), s,
                      (const float*)h->moe_y, y, h->D, K, c);
    } catch (...) {
        return fail(h, SFFN_INTERNAL, "exception in sffn_forward_moe");
    }
}

sffn_status sffn_forward_sparse(sffn_handle* h, const void* x, const void* W1, const void* W3,
                                const void* W2T, float* y, int T, int mode, int32_t* live_count,
                                int32_t* live_idx, void* stream) {
    try {
        hipStream_t s;
        sffn_status st = check_common(h, x, W3, W2T, y, T, live_count, live_idx, &s, stream);
        if (st != SFFN_OK) return st;
        if (h->dtype == SFFN_I8 || h->dtype == SFFN_I4)
            return fail(h, SFFN_INVALID_ARGUMENT, "int8 and int4 handles take the _i8 / _i4 forward calls");
        if (h->r != 0) return fail(h, SFFN_INVALID_ARGUMENT, "sparse forward needs a standard-gating handle (r == 0)");
        if (mode != SFFN_MODE_PER_TOKEN && mode != SFFN_MODE_UNION)
            return fail(h, SFFN_UNSUPPORTED, "unknown mode " + std::to_string(mode));
        if (!W1) return fail(h, SFFN_INVALID_ARGUMENT, "null W1");
        if (!aligned16(W1)) return fail(h, SFFN_INVALID_ARGUMENT, "W1 must be 16-byte aligned");
        return dispatch_sparse(h, x, W1, W3, W2T, y, T, mode, live_count, live_idx, s);
    } catch (...) {
        return fail(h, SFFN_INTERNAL, "exception in sffn_forward_sparse");
    }
}

}  // extern "C"

// ------------------------------------------------------------ no-allocation variant
// Unit products of the batch-1 pass (the gate kernel's output, the down
// kernel's input) for sffn_forward_sparse_noalloc. Each GPU the library runs
// on holds one copy until the process ends; every call on that GPU uses it.
constexpr int NOALLOC_MAX_H = 16384;
static __device__ __align__(256) float scratch[NOALLOC_MAX_H];

namespace {

constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
float* g_scratch_dev[NOALLOC_MAX_DEVICES] = {};

// Device address of `scratch` on the current device, looked up once per device
// (the host-side name is only a stand-in for the symbol, not a device address).
sffn_status scratch_address(int dev, float** out) {
    if (dev < 0 || dev >= NOALLOC_MAX_DEVICES)
        return fail(nullptr, SFFN_UNSUPPORTED, "device index beyond the no-allocation table");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(nullptr, SFFN_HIP_ERROR,
                        std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
        g_scratch_dev[dev] = static_cast<float*>(p);
    }
    *out = g_scratch_dev[dev];
    return SFFN_OK;
}

}  // namespace

extern "C" {

sffn_status sffn_forward_sparse_noalloc(const void* x, const void* W1, const void* W3,
                                        const void* W2T, float* y, int D, int H, int T, int act,
                                        void* stream) {
    try {
        if (!x || !W1 || !W3 || !W2T || !y)
            return fail(nullptr, SFFN_INVALID_ARGUMENT, "null tensor pointer");
        if (!aligned16(x) || !aligned16(W1) || !aligned16(W3) || !aligned16(W2T) || !aligned16(y))
            return fail(nullptr, SFFN_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
        if (act != SFFN_ACT_RELU && act != SFFN_ACT_RSPLUS)
            return fail(nullptr, SFFN_UNSUPPORTED, "unknown activation " + std::to_string(act));
        if (D <= 0 || D % 8 != 0 || D > 64 * 8 * 8)
            return fail(nullptr, SFFN_INVALID_ARGUMENT, "D must be a positive multiple of 8, at most 4096");
        if (H <= 0 || H > NOALLOC_MAX_H)
            return fail(nullptr, SFFN_INVALID_ARGUMENT,
                        "H=" + std::to_string(H) + " outside [1, " + std::to_string(NOALLOC_MAX_H) +
                            "]: the static scratch holds the unit products of at most " +
                            std::to_string(NOALLOC_MAX_H) + " units");
        if (T < 0) return fail(nullptr, SFFN_INVALID_ARGUMENT, "T must be >= 0");
        if (T == 0) return SFFN_OK;
        int dev = -1;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return fail(nullptr, SFFN_HIP_ERROR, std::string("hipGetDevice: ") + hipGetErrorString(e));
        float* a = nullptr;
        sffn_status st = scratch_address(dev, &a);
        if (st != SFFN_OK) return st;
        hipStream_t s = reinterpret_cast<hipStream_t>(stream);
        const int nc = pick(kNC_T1, 7, chunks_needed(D, SFFN_BF16));
        const int nb = (H + K1_WAVES - 1) / K1_WAVES;
        // unit ranges of at most 512 units (one group of 64 per wave), at least 16 ranges;
        // H <= 16384 gives at most 32
        const int splits = std::max(16, (H + KD_THREADS - 1) / KD_THREADS);
        const int nbx = (((D + 255) / 256 + 7) / 8) * 8;
        const size_t xb = (size_t)D * sizeof(uint16_t);
        for (int t = 0; t < T; ++t) {
            const void* xt = (const char*)x + t * xb;
            float* yt = y + (size_t)t * D;
            switch (nc) {
                case 1: hipLaunchKernelGGL(k_gate_up_t1<1>, dim3(nb), dim3(K1_THREADS), 0, s, (const uint16_t*)xt, (const uint16_t*)W1, (const uint16_t*)W3, a, (uint8_t*)nullptr, yt, D, H, act); break;
                case 2: hipLaunchKernelGGL(k_gate_up_t1<2>, dim3(nb), dim3(K1_THREADS), 0, s, (const uint16_t*)xt, (const uint16_t*)W1, (const uint16_t*)W3, a, (uint8_t*)nullptr, yt, D, H, act); break;
                case 3: hipLaunchKernelGGL(k_gate_up_t1<3>, dim3(nb), dim3(K1_THREADS), 0, s, (const uint16_t*)xt, (const uint16_t*)W1, (const uint16_t*)W3, a, (uint8_t*)nullptr, yt, D, H, act); break;
                case 4: hipLaunchKernelGGL(k_gate_up_t1<4>, dim3(nb), dim3(K1_THREADS), 0, s, (const uint16_t*)xt, (const uint16_t*)W1, (const uint16_t*)W3, a, (uint8_t*)nullptr, yt, D, H, act); break;
                case 5: hipLaunchKernelGGL(k_gate_up_t1<5>, dim3(nb), dim3(K1_THREADS), 0, s, (const uint16_t*)xt, (const uint16_t*)W1, (const uint16_t*)W3, a, (uint8_t*)nullptr, yt, D, H, act); break;
                case 6: hipLaunchKernelGGL(k_gate_up_t1<6>, dim3(nb), dim3(K1_THREADS), 0, s, (const uint16_t*)xt, (const uint16_t*)W1, (const uint16_t*)W3, a, (uint8_t*)nullptr, yt, D, H, act); break;
                case 8: hipLaunchKernelGGL(k_gate_up_t1<8>, dim3(nb), dim3(K1_THREADS), 0, s, (const uint16_t*)xt, (const uint16_t*)W1, (const uint16_t*)W3, a, (uint8_t*)nullptr, yt, D, H, act); break;
                default: return fail(nullptr, SFFN_INTERNAL, "no batch-1 kernel for this width");
            }
            hipLaunchKernelGGL(k_down_t1<1>, dim3(nbx, splits), dim3(KD_THREADS), 0, s,
                               (const float*)a, (const uint16_t*)W2T, yt, D, H, splits, 0);
            e = hipGetLastError();
            if (e != hipSuccess)
                return fail(nullptr, SFFN_HIP_ERROR, std::string("launch: ") + hipGetErrorString(e));
        }
        return SFFN_OK;
    } catch (...) {
        return fail(nullptr, SFFN_INTERNAL, "exception in sffn_forward_sparse_noalloc");
    }
}

static sffn_status forward_i8(sffn_handle* h, const void* x, const void* W1, const float* s1,
                       const void* W3, const float* s3, const void* W2T, const float* s2,
                       float* y, int T, int mode, int32_t* live_count, int32_t* live_idx,
                       void* stream, bool dense, int bits = 8) {
    hipStream_t s;
    sffn_status st = check_common(h, x, W3, W2T, y, T, live_count, live_idx, &s, stream);
    if (st != SFFN_OK) return st;
    if (bits == 8 && h->dtype != SFFN_I8)
        return fail(h, SFFN_INVALID_ARGUMENT, "the int8 forward needs an SFFN_I8 handle");
    if (bits == 4 && h->dtype != SFFN_I4)
        return fail(h, SFFN_INVALID_ARGUMENT, "the int4 forward needs an SFFN_I4 handle");
    if (h->r != 0) return fail(h, SFFN_INVALID_ARGUMENT, "standard-gating forward needs a handle with r == 0");
    if (mode != SFFN_MODE_PER_TOKEN && mode != SFFN_MODE_UNION)
        return fail(h, SFFN_UNSUPPORTED, "unknown mode " + std::to_string(mode));
    if (!W1) return fail(h, SFFN_INVALID_ARGUMENT, "null W1");
    if (!aligned16(W1)) return fail(h, SFFN_INVALID_ARGUMENT, "W1 must be 16-byte aligned");
    if (!s1 || !s3 || !s2) return fail(h, SFFN_INVALID_ARGUMENT, "null scale pointer");
    auto al4 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; };
    if (!al4(s1) || !al4(s3) || !al4(s2)) return fail(h, SFFN_INVALID_ARGUMENT, "scales must be 4-byte aligned");
    // batches above 4 tokens: one MFMA gate pass over the weights for the batch, then
    // the union's W2T rows once (union, dense) or each token's own live rows (per-token
    // lists). From 3 tokens every mode is ahead on the fused MFMA pass (T = 4, against the
    // VALU kernels: int8 union 158k -> 172k, per-token 162k -> 175k, dense 133k -> 147k;
    // int4 union 139k -> 180k, per-token 140k -> 182k, dense 109k -> 148k tokens/s)
    const bool pt = !dense && mode == SFFN_MODE_PER_TOKEN;
    if (bits == 8 && mfma_i8_ok(h, T, 3))
        return dense ? run_mfma_i8<true>(h, x, W1, s1, W3, s3, W2T, s2, y, T, nullptr, nullptr, s)
                     : run_mfma_i8<false>(h, x, W1, s1, W3, s3, W2T, s2, y, T, live_count, live_idx,
                                          s, nullptr, nullptr, pt);
    if (bits == 4 && mfma_i4_ok(h, T, 3))
        return dense ? run_mfma_i4<true>(h, x, W1, s1, W3, s3, W2T, s2, y, T, nullptr, nullptr, s)
                     : run_mfma_i4<false>(h, x, W1, s1, W3, s3, W2T, s2, y, T, live_count, live_idx,
                                          s, nullptr, nullptr, pt);
    // batches of 2..4 tokens: one pass over the weights on the VALU, the same two ways
    if (T >= 2 && h->m_a) {
        const int ng = (T + 3) / 4;
        for (int g = 0, t0 = 0; g < ng; ++g) {
            const int tg = T / ng + (g < T % ng ? 1 : 0);
            const void* xg = (const char*)x + (size_t)t0 * h->D * sizeof(uint16_t);
            float* yg = y + (size_t)t0 * h->D;
            int32_t* lc = live_count ? live_count + t0 : nullptr;
            int32_t* li = live_idx ? live_idx + (size_t)t0 * h->H : nullptr;
            if (bits == 4)
                st = dense ? run_i4_tb<true>(h, xg, W1, s1, W3, s3, W2T, s2, yg, tg, nullptr, nullptr, s)
                           : run_i4_tb<false>(h, xg, W1, s1, W3, s3, W2T, s2, yg, tg, lc, li, s, pt);
            else
                st = dense ? run_i8_tb<true>(h, xg, W1, s1, W3, s3, W2T, s2, yg, tg, nullptr, nullptr, s)
                           : run_i8_tb<false>(h, xg, W1, s1, W3, s3, W2T, s2, yg, tg, lc, li, s, pt);
            if (st != SFFN_OK) return st;
            t0 += tg;
        }
        return SFFN_OK;
    }
    // other batches run token by token (both modes compute the same result)
    for (int t = 0; t < T; ++t) {
        const void* xt = (const char*)x + (size_t)t * h->D * sizeof(uint16_t);
        float* yt = y + (size_t)t * h->D;
        int32_t* lc = live_count ? live_count + t : nullptr;
        int32_t* li = live_idx ? live_idx + (size_t)t * h->H : nullptr;
        if (bits == 4)
            st = dense ? run_i4_t1<true>(h, xt, W1, s1, W3, s3, W2T, s2, yt, nullptr, nullptr, s)
                       : run_i4_t1<false>(h, xt, W1, s1, W3, s3, W2T, s2, yt, lc, li, s);
        else
            st = dense ? run_i8_t1<true>(h, xt, W1, s1, W3, s3, W2T, s2, yt, nullptr, nullptr, s)
                       : run_i8_t1<false>(h, xt, W1, s1, W3, s3, W2T, s2, yt, lc, li, s);
        if (st != SFFN_OK) return st;
    }
    return SFFN_OK;
}

sffn_status sffn_forward_sparse_i4(sffn_handle* h, const void* x, const void* W1,
                                   const float* W1_scale, const void* W3, const float* W3_scale,
                                   const void* W2T, const float* W2T_scale, float* y, int T,
                                   int mode, int32_t* live_count, int32_t* live_idx,
                                   void* stream) {
    try {
        return forward_i8(h, x, W1, W1_scale, W3, W3_scale, W2T, W2T_scale, y, T, mode, live_count,
                          live_idx, stream, false, 4);
    } catch (...) {
        return fail(h, SFFN_INTERNAL, "exception in sffn_forward_sparse_i4");
    }
}

sffn_status sffn_forward_dense_i4(sffn_handle* h, const void* x, const void* W1,
                                  const float* W1_scale, const void* W3, const float* W3_scale,
                                  const void* W2T, const float* W2T_scale, float* y, int T,
                                  void* stream) {
    try {
        return forward_i8(h, x, W1, W1_scale, W3, W3_scale, W2T, W2T_scale, y, T,
                          SFFN_MODE_PER_TOKEN, nullptr, nullptr, stream, true, 4);
    } catch (...) {
        return fail(h, SFFN_INTERNAL, "exception in sffn_forward_dense_i4");
    }
}

// quantised LoPA, union of 2..4 tokens: batched rank projection (int8 V), the
// LoPA gate and the W3 gather over the union (int8 or int4 W3), the down pass
// of the small batches. Widths up to 4 chunks of W3 (else false: token by token).
bool lopa_q_tb_ok(const sffn_handle* h, int T, int bits) {
    const int nc = bits == 8 ? (h->D + 1023) / 1024 : (h->D + 2047) / 2048;
    // the gate's dynamic LDS for a group of 4: t (4 r fp32) and x (4 D bf16), <= 64 KiB
    const bool lds_ok = 4 * ((size_t)h->r * sizeof(float) + (size_t)h->D * sizeof(uint16_t)) <= 65536;
    return T >= 2 && T <= 4 && h->m_a && nc <= 4 && (h->D + 1023) / 1024 <= 4 && lds_ok;
}

sffn_status run_lopa_q_tb(sffn_handle* h, const void* x, const void* V, const float* sV,
                          const void* U, const float* sU, const void* W3, const float* s3,
                          const void* W2T, const float* s2, float* y, int T, int32_t* live_count,
                          int32_t* live_idx, hipStream_t s, int bits, bool per_token = false) {
    const int tt = T <= 2 ? 2 : 4;
    const int tp = 16 * token_tiles(T);
    int splits = h->tb_splits;
    while ((h->H + splits - 1) / splits > 32 * KD_THREADS) ++splits;
    float* yz = (per_token || splits > 1) ? y : nullptr;
    uint8_t* live = live_count ? h->live_buf : nullptr;
    sffn_status st = SFFN_OK;
    const int nc8 = (h->D + 1023) / 1024;
    const int nbr = (h->r + K1_WAVES - 1) / K1_WAVES;
#define SFFN_RPTB(NCV, TTV)                                                                       \
    st = launch_shm(h, KIND_RANK_PROJ_TB_I8, k_rank_proj_tb_i8<NCV, TTV>, dim3(nbr),              \
                    dim3(K1_THREADS), (size_t)T * h->D * sizeof(uint16_t), s, (const uint16_t*)x,  \
                    (const int8_t*)V, sV, h->t_buf, yz, h->D, h->r, T)
#define SFFN_RPTB_NC(TTV)                                                                         \
    switch (nc8) {                                                                                \
        case 1: SFFN_RPTB(1, TTV); break;                                                         \
        case 2: SFFN_RPTB(2, TTV); break;                                                         \
        case 3: SFFN_RPTB(3, TTV); break;                                                         \
        case 4: SFFN_RPTB(4, TTV); break;                                                         \
        default: return fail(h, SFFN_INTERNAL, "no batched rank projection for this width");     \
    }
    if (tt == 2) { SFFN_RPTB_NC(2); } else { SFFN_RPTB_NC(4); }
#undef SFFN_RPTB_NC
#undef SFFN_RPTB
    if (st != SFFN_OK) return st;
    const int nb = (h->H + K1_WAVES * KLQ_UPW - 1) / (K1_WAVES * KLQ_UPW);
    const int nc = bits == 8 ? nc8 : (h->D + 2047) / 2048;
#define SFFN_LQTB(NCV, TTV, BV)                                                                   \
    st = launch_shm(h, KIND_GATE_UP_LOPA_TB_Q, k_gate_up_lopa_tb_q<NCV, TTV, BV>, dim3(nb),       \
                dim3(K1_THREADS), (size_t)T * (h->r * sizeof(float) + h->D * sizeof(uint16_t)), s, \
                (const uint16_t*)x,                                                               \
                (const float*)h->t_buf, (const int8_t*)U,                                         \
                sU, (const uint8_t*)W3, s3, s2, h->m_a, h->m_mask, live, h->D, h->H, h->r, T, tp, \
                h->act, h->flags)
#define SFFN_LQTB_NC(TTV, BV)                                                                     \
    switch (nc) {                                                                                 \
        case 1: SFFN_LQTB(1, TTV, BV); break;                                                     \
        case 2: SFFN_LQTB(2, TTV, BV); break;                                                     \
        case 3: SFFN_LQTB(3, TTV, BV); break;                                                     \
        case 4: SFFN_LQTB(4, TTV, BV); break;                                                     \
        default: return fail(h, SFFN_INTERNAL, "no batched LoPA gate for this width");           \
    }
    if (bits == 8) {
        if (tt == 2) { SFFN_LQTB_NC(2, 8); } else { SFFN_LQTB_NC(4, 8); }
    } else {
        if (tt == 2) { SFFN_LQTB_NC(2, 4); } else { SFFN_LQTB_NC(4, 4); }
    }
#undef SFFN_LQTB_NC
#undef SFFN_LQTB
    if (st != SFFN_OK) return st;
    if (per_token) {
        st = run_down_pt_q(h, W2T, s2, y, T, tp, bits, s);
        if (st != SFFN_OK) return st;
        return run_live_list(h, T, live_count, live_idx, s);
    }
    const int cb = 16 * 16;
    const int nslices = (h->D + cb - 1) / cb;
    const int nbx = ((nslices + 7) / 8) * 8;
    const int hs = (h->H + splits - 1) / splits;
    const int pmax = pick(kPMAX, 6, (hs + KD_THREADS - 1) / KD_THREADS);
#define SFFN_LQ_DOWN(TTV)                                                                         \
    if (bits == 8) {                                                                              \
        SFFN_PMAX_SWITCH(pmax, st = launch(h, KIND_DOWN_TB_I8, k_down_tb_i8<PMAX, TTV>,            \
                                           dim3(nbx, splits), dim3(KD_THREADS), s,                \
                                           (const float*)h->m_a, (const uint64_t*)h->m_mask,      \
                                           (const int8_t*)W2T, y, h->D, h->H, T, tp, splits));    \
    } else {                                                                                      \
        SFFN_PMAX_SWITCH(pmax, st = launch(h, KIND_DOWN_TB_I4, k_down_tb_i4<PMAX, TTV>,            \
                                           dim3(nbx, splits), dim3(KD_THREADS), s,                \
                                           (const float*)h->m_a, (const uint64_t*)h->m_mask,      \
                                           (const uint8_t*)W2T, s2, y, h->D, h->H, T, tp,         \
                                           splits));                                              \
    }
    if (tt == 2) { SFFN_LQ_DOWN(2); } else { SFFN_LQ_DOWN(4); }
#undef SFFN_LQ_DOWN
    if (st != SFFN_OK) return st;
    return run_live_list(h, T, live_count, live_idx, s);
}

// LoPA with quantised weights: int8 rows everywhere (bits 8), or int8 V and U
// rows with group-scaled int4 W3 and W2T rows (bits 4)
static sffn_status forward_lopa_q(sffn_handle* h, const void* x, const void* V, const float* sV,
                                  const void* U, const float* sU, const void* W3, const float* s3,
                                  const void* W2T, const float* s2, float* y, int T, int mode,
                                  int32_t* live_count, int32_t* live_idx, void* stream, int bits) {
    hipStream_t s;
    sffn_status st = check_common(h, x, W3, W2T, y, T, live_count, live_idx, &s, stream);
    if (st != SFFN_OK) return st;
    if (bits == 8 && h->dtype != SFFN_I8)
        return fail(h, SFFN_INVALID_ARGUMENT, "the int8 forward needs an SFFN_I8 handle");
    if (bits == 4 && h->dtype != SFFN_I4)
        return fail(h, SFFN_INVALID_ARGUMENT, "the int4 forward needs an SFFN_I4 handle");
    if (h->r == 0) return fail(h, SFFN_INVALID_ARGUMENT, "LoPA forward needs a handle with r > 0");
    if (mode != SFFN_MODE_PER_TOKEN && mode != SFFN_MODE_UNION)
        return fail(h, SFFN_UNSUPPORTED, "unknown mode " + std::to_string(mode));
    if (!V || !U) return fail(h, SFFN_INVALID_ARGUMENT, "null V or U");
    if (!aligned16(V) || !aligned16(U))
        return fail(h, SFFN_INVALID_ARGUMENT, "V and U must be 16-byte aligned");
    if (!sV || !sU || !s3 || !s2) return fail(h, SFFN_INVALID_ARGUMENT, "null scale pointer");
    auto al4 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; };
    if (!al4(sV) || !al4(sU) || !al4(s3) || !al4(s2))
        return fail(h, SFFN_INVALID_ARGUMENT, "scales must be 4-byte aligned");
    // batches above 2 tokens: one MFMA pass over V, U and the W3 rows of the union, then
    // the union's W2T rows once or each token's own (RMSNorm of t excepted: it needs
    // each token's whole t before the gate); at 3 / 4 tokens ahead of the VALU kernels
    // (union, int8: 82k / 96k -> 92k / 121k tokens/s; int4: 79k / 92k -> 91k / 119k)
    const bool pt = mode == SFFN_MODE_PER_TOKEN;
    if (bits == 8 && mfma_i8_ok(h, T, 3) && h->m_t && !(h->flags & SFFN_FLAG_RMSNORM))
        return run_mfma_i8<false, true>(h, x, U, sU, W3, s3, W2T, s2, y, T, live_count, live_idx,
                                        s, V, sV, pt);
    if (bits == 4 && mfma_i4_ok(h, T, 3) && h->m_t && !(h->flags & SFFN_FLAG_RMSNORM))
        return run_mfma_i4<false, true>(h, x, U, sU, W3, s3, W2T, s2, y, T, live_count, live_idx,
                                        s, V, sV, pt);
    // batches of 2..4 tokens read the weights once for the batch; larger ones (with
    // RMSNorm) go as groups of 2..4 consecutive tokens (sizes as equal as can be)
    if (T >= 2 && lopa_q_tb_ok(h, 2, bits)) {
        const int ng = (T + 3) / 4;
        for (int g = 0, t0 = 0; g < ng; ++g) {
            const int tg = T / ng + (g < T % ng ? 1 : 0);
            st = run_lopa_q_tb(h, (const char*)x + (size_t)t0 * h->D * sizeof(uint16_t), V, sV, U,
                               sU, W3, s3, W2T, s2, y + (size_t)t0 * h->D, tg,
                               live_count ? live_count + t0 : nullptr,
                               live_idx ? live_idx + (size_t)t0 * h->H : nullptr, s, bits, pt);
            if (st != SFFN_OK) return st;
            t0 += tg;
        }
        return SFFN_OK;
    }
    // other batches run token by token (both modes compute the same result)
    for (int t = 0; t < T; ++t) {
        const void* xt = (const char*)x + (size_t)t * h->D * sizeof(uint16_t);
        float* yt = y + (size_t)t * h->D;
        int32_t* lc = live_count ? live_count + t : nullptr;
        int32_t* li = live_idx ? live_idx + (size_t)t * h->H : nullptr;
        st = bits == 4 ? run_lopa_i4_t1(h, xt, V, sV, U, sU, W3, s3, W2T, s2, yt, lc, li, s)
                       : run_lopa_i8_t1(h, xt, V, sV, U, sU, W3, s3, W2T, s2, yt, lc, li, s);
        if (st != SFFN_OK) return st;
    }
    return SFFN_OK;
}

sffn_status sffn_forward_lopa_i8(sffn_handle* h, const void* x, const void* V,
                                 const float* V_scale, const void* U, const float* U_scale,
                                 const void* W3, const float* W3_scale, const void* W2T,
                                 const float* W2T_scale, float* y, int T, int mode,
                                 int32_t* live_count, int32_t* live_idx, void* stream) {
    try {
        return forward_lopa_q(h, x, V, V_scale, U, U_scale, W3, W3_scale, W2T, W2T_scale, y, T,
                              mode, live_count, live_idx, stream, 8);
    } catch (...) {
        return fail(h, SFFN_INTERNAL, "exception in sffn_forward_lopa_i8");
    }
}

sffn_status sffn_forward_lopa_i4(sffn_handle* h, const void* x, const void* V,
                                 const float* V_scale, const void* U, const float* U_scale,
                                 const void* W3, const float* W3_scale, const void* W2T,
                                 const float* W2T_scale, float* y, int T, int mode,
                                 int32_t* live_count, int32_t* live_idx, void* stream) {
    try {
        return forward_lopa_q(h, x, V, V_scale, U, U_scale, W3, W3_scale, W2T, W2T_scale, y, T,
                              mode, live_count, live_idx, stream, 4);
    } catch (...) {
        return fail(h, SFFN_INTERNAL, "exception in sffn_forward_lopa_i4");
    }
}

sffn_status sffn_forward_sparse_i8(sffn_handle* h, const void* x, const void* W1,
                                   const float* W1_scale, const void* W3, const float* W3_scale,
                                   const void* W2T, const float* W2T_scale, float* y, int T,
                                   int mode, int32_t* live_count, int32_t* live_idx,
                                   void* stream) {
    try {
        return forward_i8(h, x, W1, W1_scale, W3, W3_scale, W2T, W2T_scale, y, T, mode,
                          live_count, live_idx, stream, false);
    } catch (...) {
        return fail(h, SFFN_INTERNAL, "exception in sffn_forward_sparse_i8");
    }
}

sffn_status sffn_forward_dense_i8(sffn_handle* h, const void* x, const void* W1,
                                  const float* W1_scale, const void* W3, const float* W3_scale,
                                  const void* W2T, const float* W2T_scale, float* y, int T,
                                  void* stream) {
    try {
        return forward_i8(h, x, W1, W1_scale, W3, W3_scale, W2T, W2T_scale, y, T,
                          SFFN_MODE_PER_TOKEN, nullptr, nullptr, stream, true);
    } catch (...) {
        return fail(h, SFFN_INTERNAL, "exception in sffn_forward_dense_i8");
    }
}

sffn_status sffn_forward_lopa(sffn_handle* h, const void* x, const void* V, const void* U,
                              const void* W3, const void* W2T, float* y, int T, int mode,
                              int32_t* live_count, int32_t* live_idx, void* stream) {
    try {
        hipStream_t s;
        sffn_status st = check_common(h, x, W3, W2T, y, T, live_count, live_idx, &s, stream);
        if (st != SFFN_OK) return st;
        if (h->dtype == SFFN_I8 || h->dtype == SFFN_I4)
            return fail(h, SFFN_INVALID_ARGUMENT, "int8 and int4 handles take the _i8 / _i4 forward calls");
        if (h->r == 0) return fail(h, SFFN_INVALID_ARGUMENT, "LoPA forward needs a handle with r > 0");
        if (mode != SFFN_MODE_PER_TOKEN && mode != SFFN_MODE_UNION)
            return fail(h, SFFN_UNSUPPORTED, "unknown mode " + std::to_string(mode));
        if (!V || !U) return fail(h, SFFN_INVALID_ARGUMENT, "null V or U");
        if (!aligned16(V) || !aligned16(U))
            return fail(h, SFFN_INVALID_ARGUMENT, "V and U must be 16-byte aligned");
        if (T == 0) return SFFN_OK;
        if (t1_ok(h, T) && h->r <= 4 * WAVE * 8)
            return run_lopa_t1(h, x, V, U, W3, W2T, y, live_count, live_idx, s);
        // bf16 union batches: rank projection, U gate and W3 gather on MFMA (RMSNorm of
        // the rank vectors excepted: it needs each token's whole t before the gate)
        if (mfma_ok(h, T) && h->m_t && !(h->flags & SFFN_FLAG_RMSNORM) && t1_ok(h, 1))
            return run_mfma<false, true>(h, x, U, W3, W2T, y, T, live_count, live_idx, s, V,
                                         mode == SFFN_MODE_PER_TOKEN);
        if (mode == SFFN_MODE_UNION && mfma_ok(h, T) && h->m_t && !(h->flags & SFFN_FLAG_RMSNORM))
            return run_mfma<false, true>(h, x, U, W3, W2T, y, T, live_count, live_idx, s, V);
        // other bf16 batches: each token runs the batch-1 pass on its own live set (the
        // general kernels measured slower than this at every T)
        if (t1_ok(h, 1) && h->r <= 4 * WAVE * 8) {
            const size_t xb = (size_t)h->D * sizeof(uint16_t);
            for (int t = 0; t < T; ++t) {
                st = run_lopa_t1(h, (const char*)x + t * xb, V, U, W3, W2T, y + (size_t)t * h->D,
                                 live_count ? live_count + t : nullptr,
                                 live_idx ? live_idx + (size_t)t * h->H : nullptr, s);
                if (st != SFFN_OK) return st;
            }
            return SFFN_OK;
        }
        return h->dtype == SFFN_BF16
                   ? run_lopa<uint16_t>(h, x, V, U, W3, W2T, y, T, mode, live_count, live_idx, s)
                   : run_lopa<float>(h, x, V, U, W3, W2T, y, T, mode, live_count, live_idx, s);
    } catch (...) {
        return fail(h, SFFN_INTERNAL, "exception in sffn_forward_lopa");
    }
}

sffn_status sffn_timing_enable(sffn_handle* h, int enable) {
    if (!h) return fail(nullptr, SFFN_INVALID_ARGUMENT, "null handle");
    if (enable < 0) return fail(h, SFFN_INVALID_ARGUMENT, "enable must be >= 0");
    h->timing_every = enable;
    h->call_seq = 0;
    h->timed_call = false;
    return SFFN_OK;
}

sffn_status sffn_timing_read(sffn_handle* h, int kind, double* total_ms, int64_t* launches,
                             int reset) {
    if (!h) return fail(nullptr, SFFN_INVALID_ARGUMENT, "null handle");
    if (kind < 0 || kind >= KIND_COUNT) return fail(h, SFFN_INVALID_ARGUMENT, "unknown kernel kind");
    for (auto& rec : h->pending) {
        hipError_t e = hipEventSynchronize(rec.stop);
        if (e != hipSuccess) return hip_fail(h, e, "hipEventSynchronize");
        float ms = 0.0f;
        e = hipEventElapsedTime(&ms, rec.start, rec.stop);
        if (e != hipSuccess) return hip_fail(h, e, "hipEventElapsedTime");
        h->total_ms[rec.kind] += ms;
        h->launches[rec.kind] += 1;
        h->pool.push_back(rec.start);
        h->pool.push_back(rec.stop);
    }
    h->pending.clear();
    if (total_ms) *total_ms = h->total_ms[kind];
    if (launches) *launches = h->launches[kind];
    if (reset) {
        for (int k = 0; k < KIND_COUNT; ++k) {
            h->total_ms[k] = 0.0;
            h->launches[k] = 0;
        }
    }
    return SFFN_OK;
}

int sffn_kernel_kinds(void) { return KIND_COUNT; }

const char* sffn_kernel_name(int kind) {
    if (kind < 0 || kind >= KIND_COUNT) return "unknown";
    return kKindNames[kind];
}

}  // extern "C"
