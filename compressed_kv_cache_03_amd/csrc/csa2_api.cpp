// C-ABI entry points of libcsa2 (declared in include/csa2.h).
//
// Host side only: argument validation (before anything is launched), the
// workspace layout, the Full / Reindex / Reuse plumbing of a sharing group, and
// the kernel launches.  No entry point allocates or synchronises; the only
// global state is the per-device scratch of csa2_layer_step_noalloc.
#include "../../include/csa2.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "launch.h"

namespace {

using namespace csa2;

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// bytes per stored index-key element row of K elements (FP4: codes only)
size_t key_row_bytes(csa2_idx_dtype dt, int K) {
    return dt == CSA2_IDX_BF16 ? (size_t)K * 2 : dt == CSA2_IDX_FP8_E4M3 ? (size_t)K : (size_t)K / 2;
}
int query_elem_bytes(csa2_idx_dtype dt) { return dt == CSA2_IDX_FP8_E4M3 ? 1 : 2; }
int score_dtype(csa2_idx_dtype dt) { return dt == CSA2_IDX_BF16 ? 0 : dt == CSA2_IDX_FP8_E4M3 ? 1 : 2; }

// Workspace carve-up shared by all entry points.  Offsets are 256-byte aligned.
struct Layout {
    size_t hist = 0, hist_bytes = 0;     // [R][4096] u32 (zeroed per selection), then the
                                         // undecided-score counter (zeroed with it)
    size_t fix_list = 0;                 // [R][N] (row, entry) queue of the draft-row and FP4 scorers
    bool rows_scorer = false;
    size_t scores = 0;                   // [R][N] f32
    size_t cand_idx = 0, cand_key = 0;   // [R][N]
    size_t slice_cnt = 0;                // [R][slices]
    size_t bits = 0;                     // [R][ceil(N/32)] bitmap words of the split top-k
    int64_t bits_ld = 0;
    // prefill selection on MFMA (e4m3 index keys, Qs > 1)
    size_t samp = 0, theta = 0, cand = 0, cand_cnt = 0, flag = 0, flag_count = 0, knorm = 0;
    size_t kexp = 0, kseq_norm = 0, kseq_exp = 0;  // MFMA error-bound inputs
    size_t blk = 0, blkcnt = 0;
    int cap = 0, nblk = 0;
    size_t part = 0;                     // attention partials
    // hierarchical search
    size_t bmax = 0, blk_nv = 0, pool_nv = 0;
    int64_t ld_scores = 0, ld_blk = 0;
    size_t total = 0;
};

constexpr int64_t kSampleCols = 2048;  // threshold samples per prefill row

// Prefill chunks with e4m3 keys select through the MFMA candidate path, which
// never holds every score; a hierarchical group needs them for its block
// scores and takes the exact path.
bool mfma_prefill(const csa2_group* g, int Qs) {
    const int K = g->H_I * g->d_I;
    return Qs > 1 && g->idx_dtype == CSA2_IDX_FP8_E4M3 && (K == 128 || K == 256) &&
           g->k <= band_max_k() && g->pool_blocks == 0;
}

// Several bf16 query rows per sequence share each key load (score.hip), with a
// queue of undecided scores in the workspace.
bool rows_scorer(const csa2_group* g, int Qs) {
    const int K = g->H_I * g->d_I;
    return Qs >= 2 && g->idx_dtype == CSA2_IDX_BF16 && (K == 128 || K == 256);
}

int64_t pool_slots(const csa2_group* g) { return (int64_t)g->pool_blocks * CSA2_POOL_BLOCK; }
int64_t block_count(int64_t N) { return (N + CSA2_POOL_BLOCK - 1) / CSA2_POOL_BLOCK; }

struct TopkShape {
    int64_t R, N, slices;
};

void add_topk(Layout& L, size_t& off, const TopkShape& t) {
    L.hist = off;
    L.hist_bytes = (size_t)t.R * kHistBinsHost * 4;
    off = align_up(off + L.hist_bytes + 4);
    L.cand_idx = off;
    off = align_up(off + (size_t)t.R * t.N * 4);
    L.cand_key = off;
    off = align_up(off + (size_t)t.R * t.N * 4);
    L.slice_cnt = off;
    off = align_up(off + (size_t)t.R * t.slices * 4);
    L.bits_ld = (t.N + 31) / 32;
    L.bits = off;
    off = align_up(off + (size_t)t.R * L.bits_ld * 4);
}

size_t attend_part_bytes(int64_t R, int Hq, int D, int k, int W) {
    int splits, chunk;
    attend_splits(R, Hq, D, k, W, &splits, &chunk);
    return splits > 1 ? (size_t)R * splits * Hq * (D + 2) * 4 : 0;
}

Layout layer_layout(const csa2_group* g, int Qs, int Hq, int W) {
    Layout L;
    const int64_t R = (int64_t)g->B * Qs, N = g->N_cap;
    size_t off = 0;
    // a hierarchical group scores either every entry or the pool's slots
    L.ld_scores = std::max<int64_t>(N, pool_slots(g));
    L.scores = off;
    off = align_up(off + (size_t)R * L.ld_scores * 4);
    if (g->pool_blocks > 0) {
        L.ld_blk = block_count(N);
        L.bmax = off;
        off = align_up(off + (size_t)R * L.ld_blk * 4);
        L.blk_nv = off;
        off = align_up(off + (size_t)R * 4);
        L.pool_nv = off;
        off = align_up(off + (size_t)R * 4);
    }
    if (mfma_prefill(g, Qs)) {
        L.cap = (int)std::min<int64_t>(band_cap(g->k), N);
        L.nblk = (int)((N + 255) / 256);
        L.samp = off;
        off = align_up(off + (size_t)R * std::min<int64_t>(N, kSampleCols) * 4);
        L.theta = off;
        off = align_up(off + (size_t)R * 4);
        L.cand_cnt = off;
        off = align_up(off + (size_t)R * 4);
        L.flag = off;
        off = align_up(off + (size_t)R * 4);
        L.flag_count = off;
        off = align_up(off + 4);
        L.knorm = off;
        off = align_up(off + (size_t)g->B * L.nblk * 4);
        L.kexp = off;
        const size_t G = (size_t)(g->H_I * g->d_I / 8);  // groups of 8 index elements
        off = align_up(off + (size_t)g->B * L.nblk * G);
        L.kseq_norm = off;
        off = align_up(off + (size_t)g->B * 4);
        L.kseq_exp = off;
        off = align_up(off + (size_t)g->B * G);
        L.cand = off;
        off = align_up(off + (size_t)R * L.cap * 8);
        L.blkcnt = off;
        off = align_up(off + (size_t)R * filter_colblks(N) * 4);
        L.blk = off;
        off = align_up(off + (size_t)R * filter_colblks(N) * filter_blk_cap() * 8);
    } else {
        // one shape for every top-k of the layer: entries, blocks and pool slots
        int64_t slices = 0;
        for (int64_t n : {N, block_count(N), pool_slots(g)})
            if (n > 0) slices = std::max(slices, (n + topk_slice_len(n) - 1) / topk_slice_len(n));
        add_topk(L, off, TopkShape{R, L.ld_scores, slices});
        L.rows_scorer = rows_scorer(g, Qs);
        if (L.rows_scorer) {
            L.fix_list = off;
            off = align_up(off + (size_t)R * N * 8);
        }
    }
    L.part = off;
    off = align_up(off + attend_part_bytes(R, Hq, g->D, g->k, W));
    L.total = off;
    return L;
}

template <typename T>
T* at(void* ws, size_t off) {
    return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

csa2_status hip_status(hipError_t e) { return e == hipSuccess ? CSA2_OK : CSA2_ERR_HIP; }

// Records a caller's timing event on the stream (no event: nothing).
hipError_t mark(void* event, hipStream_t s) {
    return event ? hipEventRecord(static_cast<hipEvent_t>(event), s) : hipSuccess;
}

bool valid_dim(int32_t D) { return D >= 32 && D <= 256 && D % 32 == 0; }

// A C caller may pass any integer where the header declares an enum; reading
// such a value through the enum type is undefined in C++, so the bits are read
// as an integer and checked before the enum is used.
template <typename E>
int32_t enum_bits(const E& e) {
    static_assert(sizeof(E) == sizeof(int32_t), "enums of the ABI are int-sized");
    int32_t v;
    std::memcpy(&v, &e, sizeof v);
    return v;
}
bool valid_mode(const csa2_mode& m) {
    const int32_t v = enum_bits(m);
    return v == CSA2_MODE_FULL || v == CSA2_MODE_REINDEX || v == CSA2_MODE_REUSE;
}
bool valid_dtype(const csa2_idx_dtype& d) {
    const int32_t v = enum_bits(d);
    return v == CSA2_IDX_BF16 || v == CSA2_IDX_FP8_E4M3 || v == CSA2_IDX_FP4_E2M1;
}

bool valid_index_width(csa2_idx_dtype dt, int32_t H, int32_t d) {
    if (H < 1 || d < 1) return false;
    const int64_t K = (int64_t)H * d;
    if (dt == CSA2_IDX_FP4_E2M1) return K <= 4096 && K % 32 == 0;
    return K <= 4096 && K % 16 == 0 && (dt == CSA2_IDX_BF16 || dt == CSA2_IDX_FP8_E4M3);
}


// Host-tier image of a group: for entries 0 .. n_valid_max-1 of every
// sequence, codes, then scales, then index keys, then the selection when the
// group holds one (B * sel_qs rows of k).
struct ImageParts {
    int64_t n = 0;
    size_t code_row = 0, scale_row = 0, key_row = 0;  // bytes per entry
    size_t kscale_row = 0;                            // FP4 index keys only
    size_t pool = 0;                                  // hierarchical groups with a pool
    size_t codes = 0, scales = 0, keys = 0, kscales = 0, sel = 0, total = 0;
};

bool image_parts(const csa2_group* g, ImageParts* p) {
    if (!g || !valid_dtype(g->idx_dtype) || g->B < 1 || g->N_cap < 1 || !valid_dim(g->D) || g->k < 1 ||
        !valid_index_width(g->idx_dtype, g->H_I, g->d_I) || g->n_valid_max < 0 || g->n_valid_max > g->N_cap)
        return false;
    if (g->has_selection && (g->sel_qs < 1 || (int64_t)g->B * g->sel_qs > g->sel_rows)) return false;
    p->n = g->n_valid_max;
    p->code_row = (size_t)g->D / 2;
    p->scale_row = (size_t)g->D / 32 * 4;
    p->key_row = key_row_bytes(g->idx_dtype, g->H_I * g->d_I);
    p->kscale_row = g->idx_dtype == CSA2_IDX_FP4_E2M1 ? (size_t)g->H_I * g->d_I / 32 * 4 : 0;
    p->kscales = (size_t)g->B * p->n * p->kscale_row;
    p->codes = (size_t)g->B * p->n * p->code_row;
    p->scales = (size_t)g->B * p->n * p->scale_row;
    p->keys = (size_t)g->B * p->n * p->key_row;
    p->sel = g->has_selection ? (size_t)g->B * g->sel_qs * g->k * 4 : 0;
    if (g->has_pool && (g->pool_blocks < 1 || g->pool_qs < 1 || (int64_t)g->B * g->pool_qs > g->sel_rows))
        return false;
    p->pool = g->has_pool ? (size_t)g->B * g->pool_qs * g->pool_blocks * 4 : 0;
    p->total = p->codes + p->scales + p->keys + p->kscales + p->sel + p->pool;
    return true;
}

// One strided array between the group (row pitch N_cap entries) and the packed image.
hipError_t copy_rows(void* dst, size_t dpitch, const void* src, size_t spitch, size_t width, size_t rows,
                     hipMemcpyKind kind, hipStream_t s) {
    if (width == 0 || rows == 0) return hipSuccess;
    return hipMemcpy2DAsync(dst, dpitch, src, spitch, width, rows, kind, s);
}

// Every check of csa2_layer_step except the workspace: arguments, group
// geometry and state, and the launch sizes.  Touches no device.
csa2_status check_layer(const csa2_mode& mode, const csa2_layer_args* a, const csa2_group* g) {
    if (!a || !g) return CSA2_ERR_INVALID_ARG;
    if (!valid_mode(mode) || !valid_dtype(g->idx_dtype)) return CSA2_ERR_INVALID_ARG;
    // group geometry
    if (g->B < 1 || g->N_cap < 1 || !valid_dim(g->D) || g->k < 1 || g->k > g->N_cap ||
        !valid_index_width(g->idx_dtype, g->H_I, g->d_I))
        return CSA2_ERR_INVALID_ARG;
    if (g->N_cap >= (int64_t)1 << 31) return CSA2_ERR_UNSUPPORTED;
    if (!g->codes || !g->scales || !g->ikeys || !g->n_valid || !g->sel) return CSA2_ERR_INVALID_ARG;
    if (!aligned(g->codes, 16) || !aligned(g->scales, 16) || !aligned(g->ikeys, 16) ||
        !aligned(g->sel, 4) || !aligned(g->n_valid, 4))
        return CSA2_ERR_INVALID_ARG;
    if (g->idx_dtype == CSA2_IDX_FP4_E2M1 && (!g->ikey_scales || !aligned(g->ikey_scales, 16)))
        return CSA2_ERR_INVALID_ARG;
    if (g->pool_blocks < 0 ||
        (g->pool_blocks > 0 && (pool_slots(g) < g->k || g->pool_blocks > block_count(g->N_cap) || !g->pool ||
                                !aligned(g->pool, 4))))
        return CSA2_ERR_INVALID_ARG;
    // layer arguments
    const int Qs = a->Qs;
    if (Qs < 1 || a->Hq < 1 || a->Hq > 32 || a->W < 0 || a->W > 1024 || !std::isfinite(a->sm_scale))
        return CSA2_ERR_INVALID_ARG;
    if (g->n_valid_max < Qs || g->n_valid_max > g->N_cap) return CSA2_ERR_INVALID_ARG;
    if ((int64_t)g->B * Qs > 65535) return CSA2_ERR_UNSUPPORTED;
    if (g->sel_rows < (int64_t)g->B * Qs) return CSA2_ERR_INVALID_ARG;
    if (!a->q || !a->out || (a->W > 0 && (!a->wk || !a->wv))) return CSA2_ERR_INVALID_ARG;
    if (!aligned(a->q, 16) || !aligned(a->out, 16) || (a->wk && !aligned(a->wk, 16)) ||
        (a->wv && !aligned(a->wv, 16)))
        return CSA2_ERR_INVALID_ARG;
    const bool selects = mode != CSA2_MODE_REUSE;
    if (selects && (!a->iq || !aligned(a->iq, 16))) return CSA2_ERR_INVALID_ARG;
    if (mode == CSA2_MODE_FULL &&
        (!a->new_entry || !a->new_ikey || !aligned(a->new_entry, 16) ||
         !aligned(a->new_ikey, g->idx_dtype == CSA2_IDX_FP4_E2M1 ? 16 : 4)))
        return CSA2_ERR_INVALID_ARG;
    // group state
    if (mode == CSA2_MODE_REINDEX && !g->has_entries) return CSA2_ERR_STATE;
    if (mode == CSA2_MODE_REINDEX && g->pool_blocks > 0 && (!g->has_pool || g->pool_qs != Qs))
        return CSA2_ERR_STATE;
    if (mode == CSA2_MODE_REUSE && (!g->has_selection || g->sel_qs != Qs)) return CSA2_ERR_STATE;
    const int K = g->H_I * g->d_I;
    // launch sizes: HIP caps a grid at 2^32 - 1 work-items along x, which long
    // rows times many query rows can exceed; refuse before anything is enqueued
    if (selects && mfma_prefill(g, Qs)) {
        GemmArgs ga{};
        ga.K = K;
        ga.B = g->B;
        ga.Qs = Qs;
        ga.N = g->n_valid_max;
        ga.stride = (ga.N + kSampleCols - 1) / kSampleCols;
        ga.ncols = (ga.N + ga.stride - 1) / ga.stride;
        GemmArgs fa = ga;
        fa.stride = 1;
        fa.ncols = ga.N;
        if (gemm_grid_threads(ga, 0) > kMaxGridThreads || gemm_grid_threads(fa, 1) > kMaxGridThreads)
            return CSA2_ERR_UNSUPPORTED;
    } else if (selects) {
        const bool in_pool = mode == CSA2_MODE_REINDEX && g->pool_blocks > 0;
        ScoreArgs sa{};
        sa.dtype = score_dtype(g->idx_dtype);
        sa.K = K;
        sa.B = g->B;
        sa.Qs = Qs;
        sa.N = in_pool ? pool_slots(g) : g->n_valid_max;
        sa.pool = in_pool ? g->pool : nullptr;
        uint32_t queue_stand_in = 0;  // the plan only asks whether a queue exists
        sa.fix_cnt = rows_scorer(g, Qs) ? &queue_stand_in : nullptr;
        if (score_grid_threads(sa) > kMaxGridThreads) return CSA2_ERR_UNSUPPORTED;
    }
    return CSA2_OK;
}

}  // namespace

// Scratch of csa2_layer_step_noalloc: one copy per GPU, held until the process
// ends.  Host code never names it: its device address comes from
// hipGetSymbolAddress, resolved once per device (see static_scratch below).
static __device__ __align__(256) unsigned char scratch[CSA2_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of the current device's scratch array, looked up on the first
// call on that device (with it current) and kept for later calls.
hipError_t static_scratch(void** ptr) {
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(g_scratch_once[dev], [dev] {
        void* p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = p;
    });
    *ptr = g_scratch_ptr[dev];
    return g_scratch_err[dev];
}

}  // namespace

extern "C" {

const char* csa2_status_str(csa2_status s) {
    switch (s) {
        case CSA2_OK: return "CSA2_OK";
        case CSA2_ERR_INVALID_ARG: return "CSA2_ERR_INVALID_ARG";
        case CSA2_ERR_UNSUPPORTED: return "CSA2_ERR_UNSUPPORTED";
        case CSA2_ERR_WORKSPACE: return "CSA2_ERR_WORKSPACE";
        case CSA2_ERR_STATE: return "CSA2_ERR_STATE";
        case CSA2_ERR_HIP: return "CSA2_ERR_HIP";
    }
    return "CSA2_ERR_UNKNOWN";
}

const char* csa2_version(void) { return "csa2-gfx950 0.1"; }

int64_t csa2_cache_bytes(int64_t entries, int64_t numbers, int64_t copies, int64_t bits) {
    if (entries < 0 || numbers < 0 || copies < 0 || bits < 0) return -1;
    __int128 v = (__int128)entries * numbers;
    v *= copies;
    v *= bits;
    v /= 8;
    if (v > INT64_MAX) return -1;
    return (int64_t)v;
}

csa2_status csa2_fp4_pack(const float* x, int64_t rows, int32_t dim, uint8_t* codes, float* scales,
                          void* stream) {
    if (rows < 0 || dim <= 0 || dim % 32 != 0) return CSA2_ERR_INVALID_ARG;
    if (rows == 0) return CSA2_OK;
    if (rows > kMaxGridThreads / (dim / 8)) return CSA2_ERR_UNSUPPORTED;  // one lane per 8 elements
    if (!x || !codes || !scales) return CSA2_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(codes, 4) || !aligned(scales, 4)) return CSA2_ERR_INVALID_ARG;
    return hip_status(launch_fp4_pack(x, rows, dim, codes, scales, nullptr, 1, rows,
                                      static_cast<hipStream_t>(stream)));
}

csa2_status csa2_index_score(const void* iq, const void* ik, const float* ik_scales,
                             csa2_idx_dtype dtype, int32_t B, int32_t Qs, int64_t N, int32_t H,
                             int32_t d, int64_t causal_offset, int32_t exact, float* scores,
                             void* stream) {
    (void)exact;  // every score is exact (see the header)
    if (B < 0 || Qs < 1 || N < 0 || causal_offset < -1) return CSA2_ERR_INVALID_ARG;
    if (!valid_dtype(dtype) || !valid_index_width(dtype, H, d)) return CSA2_ERR_INVALID_ARG;
    if (N >= (int64_t)1 << 31) return CSA2_ERR_UNSUPPORTED;
    if (B == 0 || N == 0) return CSA2_OK;
    if (!iq || !ik || !scores || (dtype == CSA2_IDX_FP4_E2M1 && !ik_scales)) return CSA2_ERR_INVALID_ARG;
    if (!aligned(iq, 16) || !aligned(ik, 16) || !aligned(scores, 4) ||
        (dtype == CSA2_IDX_FP4_E2M1 && !aligned(ik_scales, 4)))
        return CSA2_ERR_INVALID_ARG;
    if ((int64_t)B * Qs > 65535) return CSA2_ERR_UNSUPPORTED;  // grid.y
    ScoreArgs a{};
    a.iq = iq;
    a.ik = ik;
    a.ik_scales = dtype == CSA2_IDX_FP4_E2M1 ? ik_scales : nullptr;
    a.dtype = score_dtype(dtype);
    a.K = H * d;
    a.B = B;
    a.Qs = Qs;
    a.N = N;
    a.N_cap = N;
    a.nvb = nullptr;
    a.causal = causal_offset;
    a.scores = scores;
    a.ld = N;
    a.hist = nullptr;
    if (score_grid_threads(a) > kMaxGridThreads) return CSA2_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = launch_score_exact(a, s);
    if (e == hipSuccess) e = launch_score_tail(a, s);
    return hip_status(e);
}

size_t csa2_topk_workspace_bytes(int64_t R, int64_t N, int32_t k) {
    (void)k;
    if (R <= 0 || N <= 0) return 0;
    Layout L;
    size_t off = 0;
    add_topk(L, off, TopkShape{R, N, (N + topk_slice_len(N) - 1) / topk_slice_len(N)});
    return off;
}

csa2_status csa2_topk(const float* scores, int64_t R, int64_t N, int64_t ld, const int32_t* n_valid,
                      int32_t k, int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
    if (R < 0 || N < 0 || k < 1 || ld < N) return CSA2_ERR_INVALID_ARG;
    if (N >= (int64_t)1 << 31 || R > 65535) return CSA2_ERR_UNSUPPORTED;
    if (R == 0) return CSA2_OK;
    if (!idx || (N > 0 && !scores)) return CSA2_ERR_INVALID_ARG;
    if (!aligned(idx, 4) || (scores && !aligned(scores, 4))) return CSA2_ERR_INVALID_ARG;
    const size_t need = csa2_topk_workspace_bytes(R, N > 0 ? N : 1, k);
    if (!ws || ws_bytes < need || !aligned(ws, 256)) return CSA2_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    Layout L;
    size_t off = 0;
    const int64_t Nn = N > 0 ? N : 1;
    const int64_t slices = (Nn + topk_slice_len(Nn) - 1) / topk_slice_len(Nn);
    add_topk(L, off, TopkShape{R, Nn, slices});
    TopkArgs t{};
    t.scores = scores;
    t.R = R;
    t.N = N;
    t.ld = ld;
    t.nvb = n_valid;
    t.Qs = 1;
    t.k = k;
    t.idx = idx;
    t.hist = at<uint32_t>(ws, L.hist);
    t.cand_idx = at<int32_t>(ws, L.cand_idx);
    t.cand_key = at<uint32_t>(ws, L.cand_key);
    t.slice_cnt = at<uint32_t>(ws, L.slice_cnt);
    t.slices = (int)slices;
    t.slice_len = topk_slice_len(Nn);
    t.bits = at<uint32_t>(ws, L.bits);
    t.bits_ld = L.bits_ld;
    hipError_t e = launch_zero(t.hist, (int64_t)R * kHistBinsHost, s);
    if (e == hipSuccess) e = launch_topk_hist(t, s);
    if (e == hipSuccess) e = launch_topk_select(t, s);
    return hip_status(e);
}

size_t csa2_attend_workspace_bytes(int32_t B, int32_t Qs, int32_t Hq, int32_t D, int32_t k,
                                   int32_t W) {
    if (B <= 0 || Qs <= 0 || Hq <= 0 || !valid_dim(D) || k < 0 || W < 0) return 0;
    return align_up(attend_part_bytes((int64_t)B * Qs, Hq, D, k, W));
}

csa2_status csa2_sparse_attend(const void* q, int32_t B, int32_t Qs, int32_t Hq, int32_t D,
                               const uint8_t* codes, const float* scales, int64_t N,
                               const int32_t* idx, int32_t k, const void* wk, const void* wv,
                               int32_t W, const int32_t* wlen, float sm_scale, float* out,
                               float* lse, void* ws, size_t ws_bytes, void* stream) {
    if (B < 0 || Qs < 1 || Hq < 1 || Hq > 32 || !valid_dim(D) || N < 0 || k < 0 || W < 0 ||
        W > 1024 || !std::isfinite(sm_scale))
        return CSA2_ERR_INVALID_ARG;
    if (k == 0 && W == 0) return CSA2_ERR_INVALID_ARG;
    if ((int64_t)B * Qs > 65535 || N >= (int64_t)1 << 31) return CSA2_ERR_UNSUPPORTED;
    if (B == 0) return CSA2_OK;
    if (!q || !out) return CSA2_ERR_INVALID_ARG;
    if (k > 0 && (!idx || !codes || !scales)) return CSA2_ERR_INVALID_ARG;
    if (W > 0 && (!wk || !wv)) return CSA2_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(out, 16) || (codes && !aligned(codes, 16)) ||
        (scales && !aligned(scales, 16)) || (wk && !aligned(wk, 16)) || (wv && !aligned(wv, 16)))
        return CSA2_ERR_INVALID_ARG;
    const size_t need = csa2_attend_workspace_bytes(B, Qs, Hq, D, k, W);
    if (!ws || ws_bytes < need) return CSA2_ERR_WORKSPACE;
    AttendArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.B = B;
    a.Qs = Qs;
    a.Hq = Hq;
    a.D = D;
    a.codes = codes;
    a.scales = scales;
    a.N = N;
    a.idx = idx;
    a.k = k;
    a.wk = static_cast<const uint16_t*>(wk);
    a.wv = static_cast<const uint16_t*>(wv);
    a.W = W;
    a.wlen = wlen;
    a.sm_scale = sm_scale;
    a.out = out;
    a.lse = lse;
    a.part = static_cast<float*>(ws);
    return hip_status(launch_attend(a, static_cast<hipStream_t>(stream)));
}

size_t csa2_layer_workspace_bytes(const csa2_group* g, int32_t Qs, int32_t Hq, int32_t W) {
    if (!g || !valid_dtype(g->idx_dtype) || g->B <= 0 || g->N_cap <= 0 || Qs <= 0 || Hq <= 0 || W < 0 || !valid_dim(g->D))
        return 0;
    return layer_layout(g, Qs, Hq, W).total;
}

csa2_status csa2_layer_step(csa2_mode mode, const csa2_layer_args* a, csa2_group* g, void* ws,
                            size_t ws_bytes, void* stream) {
    const csa2_status st = check_layer(mode, a, g);
    if (st != CSA2_OK) return st;
    const int Qs = a->Qs;
    const bool selects = mode != CSA2_MODE_REUSE;
    // workspace
    const Layout L = layer_layout(g, Qs, a->Hq, a->W);
    if (!ws || ws_bytes < L.total || !aligned(ws, 256)) return CSA2_ERR_WORKSPACE;

    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t R = (int64_t)g->B * Qs;
    const int K = g->H_I * g->d_I;
    hipError_t e = hipSuccess;

    const bool exact_select = selects && !mfma_prefill(g, Qs);
    if (mode == CSA2_MODE_FULL) {
        // S1: the step's new rows go to slots n_valid-Qs .. n_valid-1, with their
        // index keys; the same launch zeroes the digit histogram of the scoring
        FullPrepArgs fp{};
        fp.entry = a->new_entry;
        fp.rows = R;
        fp.D = g->D;
        fp.codes = g->codes;
        fp.scales = g->scales;
        fp.key = a->new_ikey;
        fp.key_fp4 = g->idx_dtype == CSA2_IDX_FP4_E2M1;
        fp.K = K;
        fp.key_words = (int)(key_row_bytes(g->idx_dtype, K) / 4);
        fp.ikeys = g->ikeys;
        fp.ikey_scales = g->ikey_scales;
        fp.nvb = g->n_valid;
        fp.Qs = Qs;
        fp.N_cap = g->N_cap;
        fp.zero = exact_select ? at<uint32_t>(ws, L.hist) : nullptr;
        fp.zero_words = exact_select ? R * kHistBinsHost + 1 : 0;  // histogram and queue counter
        e = launch_full_prep(fp, s);
    }
    if (e == hipSuccess && selects && mfma_prefill(g, Qs)) {
        // S2 + S3 for a prefill chunk: sampled thresholds, MFMA score GEMM with a
        // candidate filter, exact selection (index_gemm.hip)
        const int64_t N = g->n_valid_max;
        const int64_t stride = (N + kSampleCols - 1) / kSampleCols;
        GemmArgs ga{};
        ga.iq = static_cast<const uint8_t*>(a->iq);
        ga.ik = static_cast<const uint8_t*>(g->ikeys);
        ga.K = K;
        ga.B = g->B;
        ga.Qs = Qs;
        ga.N = N;
        ga.N_cap = g->N_cap;
        ga.nvb = g->n_valid;
        ga.stride = stride;
        ga.ncols = (N + stride - 1) / stride;
        ga.out = at<float>(ws, L.samp);
        BandArgs ba{};
        ba.B = g->B;
        ba.Qs = Qs;
        ba.K = K;
        ba.k = g->k;
        ba.N = N;
        ba.N_cap = g->N_cap;
        ba.nvb = g->n_valid;
        ba.iq = ga.iq;
        ba.ik = ga.ik;
        ba.stride = stride;
        ba.ncols = ga.ncols;
        ba.samp = ga.out;
        ba.theta = at<float>(ws, L.theta);
        ba.blk = at<uint2>(ws, L.blk);
        ba.blkcnt = at<uint32_t>(ws, L.blkcnt);
        ba.n_colblk = filter_colblks(N);
        ba.cand = at<uint2>(ws, L.cand);
        ba.cand_cnt = at<uint32_t>(ws, L.cand_cnt);
        ba.cap = L.cap;
        ba.knorm = at<float>(ws, L.knorm);
        ba.kexp = at<uint8_t>(ws, L.kexp);
        ba.kseq_norm = at<float>(ws, L.kseq_norm);
        ba.kseq_exp = at<uint8_t>(ws, L.kseq_exp);
        ba.nblk = (int)((N + 255) / 256);
        ba.idx = g->sel;
        ba.flag = at<int32_t>(ws, L.flag);
        ba.flag_count = at<uint32_t>(ws, L.flag_count);
        ba.scores = at<float>(ws, L.scores);
        ba.ld = g->N_cap;
        e = mark(a->index_events[0], s);
        if (e == hipSuccess) e = launch_gemm_fp8(ga, 0, s);
        if (e == hipSuccess) e = launch_key_norm(ga.ik, K, g->B, N, g->N_cap, ba.nblk, ba.knorm, ba.kexp, ba.kseq_norm,
                                                       ba.kseq_exp, s);
        if (e == hipSuccess) e = launch_sample_select(ba, s);
        if (e == hipSuccess) {
            GemmArgs fa = ga;
            fa.stride = 1;
            fa.ncols = N;
            fa.out = nullptr;
            fa.theta = ba.theta;
            fa.blk = at<uint2>(ws, L.blk);
            fa.blkcnt = at<uint32_t>(ws, L.blkcnt);
            fa.cand = at<uint2>(ws, L.cand);
            fa.cand_cnt = ba.cand_cnt;
            fa.cap = ba.cap;
            e = launch_gemm_fp8(fa, 1, s);
        }
        if (e == hipSuccess) e = mark(a->index_events[1], s);
        if (e == hipSuccess) e = launch_band_final(ba, s);
    } else if (e == hipSuccess && selects) {
        // S2 + S3: exact scores of the valid entries (or, for Reindex in a
        // hierarchical group, of the pool's entries), digit histogram, selection
        const bool in_pool = mode == CSA2_MODE_REINDEX && g->pool_blocks > 0;
        float* scores = at<float>(ws, L.scores);
        TopkArgs t{};
        t.scores = scores;
        t.R = R;
        t.ld = L.ld_scores;
        t.k = g->k;
        t.idx = g->sel;
        t.hist = at<uint32_t>(ws, L.hist);
        t.cand_idx = at<int32_t>(ws, L.cand_idx);
        t.cand_key = at<uint32_t>(ws, L.cand_key);
        t.slice_cnt = at<uint32_t>(ws, L.slice_cnt);
        t.bits = at<uint32_t>(ws, L.bits);
        t.bits_ld = L.bits_ld;
        ScoreArgs sa{};
        sa.iq = a->iq;
        sa.ik = g->ikeys;
        sa.dtype = score_dtype(g->idx_dtype);
        sa.ik_scales = g->ikey_scales;
        sa.K = K;
        sa.B = g->B;
        sa.Qs = Qs;
        sa.N_cap = g->N_cap;
        sa.nvb = g->n_valid;
        sa.scores = scores;
        sa.ld = L.ld_scores;
        sa.hist = t.hist;
        if (L.rows_scorer) {
            sa.fix_cnt = t.hist + R * kHistBinsHost;
            sa.fix_list = at<uint2>(ws, L.fix_list);
        }
        if (in_pool) {
            int32_t* pool_nv = at<int32_t>(ws, L.pool_nv);
            e = launch_pool_count(g->pool, R, g->pool_blocks, g->n_valid, Qs, pool_nv, s);
            sa.pool = g->pool;
            sa.pool_blocks = g->pool_blocks;
            sa.pool_nv = pool_nv;
            sa.N = pool_slots(g);
            t.N = pool_slots(g);
            t.nvb = pool_nv;
            t.Qs = 1;
            t.slice_len = topk_slice_len(pool_slots(g));
        } else {
            sa.N = g->n_valid_max;
            t.N = g->n_valid_max;
            t.nvb = g->n_valid;
            t.Qs = Qs;
            t.slice_len = topk_slice_len(g->N_cap);
        }
        t.slices = (int)((t.N + t.slice_len - 1) / t.slice_len);
        if (e == hipSuccess && mode != CSA2_MODE_FULL) e = launch_zero(t.hist, R * kHistBinsHost + 1, s);
        if (e == hipSuccess) e = mark(a->index_events[0], s);
        if (e == hipSuccess) e = launch_score_exact(sa, s);
        if (e == hipSuccess) e = mark(a->index_events[1], s);
        if (e == hipSuccess) e = launch_topk_select(t, s);
        // the selection holds pool slots: turn them into entries
        if (e == hipSuccess && in_pool) e = launch_pool_map(g->sel, R, g->k, g->pool, g->pool_blocks, s);
        if (e == hipSuccess && mode == CSA2_MODE_FULL && g->pool_blocks > 0) {
            // the pool: blocks of 8 entries ranked by their largest score
            float* bmax = at<float>(ws, L.bmax);
            int32_t* blk_nv = at<int32_t>(ws, L.blk_nv);
            TopkArgs tb = t;
            tb.scores = bmax;
            tb.N = block_count(g->n_valid_max);
            tb.ld = L.ld_blk;
            tb.nvb = blk_nv;
            tb.Qs = 1;
            tb.k = g->pool_blocks;
            tb.idx = g->pool;
            tb.slice_len = topk_slice_len(L.ld_blk);
            tb.slices = (int)((tb.N + tb.slice_len - 1) / tb.slice_len);
            e = launch_block_max(scores, R, g->n_valid_max, L.ld_scores, g->n_valid, Qs, bmax, L.ld_blk, blk_nv, s);
            if (e == hipSuccess) e = launch_zero(tb.hist, R * kHistBinsHost, s);
            if (e == hipSuccess) e = launch_topk_hist(tb, s);
            if (e == hipSuccess) e = launch_topk_select(tb, s);
        }
    }
    if (e == hipSuccess) {
        // S5 + S6: gather, dequantise, attend over the selection and the window
        AttendArgs at_{};
        at_.q = static_cast<const uint16_t*>(a->q);
        at_.B = g->B;
        at_.Qs = Qs;
        at_.Hq = a->Hq;
        at_.D = g->D;
        at_.codes = g->codes;
        at_.scales = g->scales;
        at_.N = g->N_cap;
        at_.idx = g->sel;
        at_.k = g->k;
        at_.wk = static_cast<const uint16_t*>(a->wk);
        at_.wv = static_cast<const uint16_t*>(a->wv);
        at_.W = a->W;
        at_.wlen = a->wlen;
        at_.sm_scale = a->sm_scale;
        at_.out = a->out;
        at_.lse = a->lse;
        at_.part = at<float>(ws, L.part);
        e = launch_attend(at_, s);
    }
    if (e != hipSuccess) return CSA2_ERR_HIP;
    if (mode == CSA2_MODE_FULL) g->has_entries = 1;
    if (selects) {
        g->has_selection = 1;
        g->sel_qs = Qs;
    }
    if (mode == CSA2_MODE_FULL && g->pool_blocks > 0) {
        g->has_pool = 1;
        g->pool_qs = Qs;
    }
    return CSA2_OK;
}

csa2_status csa2_layer_step_noalloc(csa2_mode mode, const csa2_layer_args* a, csa2_group* g,
                                    void* stream) {
    const csa2_status st = check_layer(mode, a, g);
    if (st != CSA2_OK) return st;
    if (layer_layout(g, a->Qs, a->Hq, a->W).total > CSA2_STATIC_SCRATCH_BYTES) return CSA2_ERR_WORKSPACE;
    void* ws = nullptr;
    if (static_scratch(&ws) != hipSuccess || !ws) return CSA2_ERR_HIP;
    return csa2_layer_step(mode, a, g, ws, CSA2_STATIC_SCRATCH_BYTES, stream);
}

size_t csa2_group_image_bytes(const csa2_group* g) {
    ImageParts p;
    return image_parts(g, &p) ? p.total : 0;
}

csa2_status csa2_group_save(const csa2_group* g, void* host, size_t bytes, void* stream) {
    ImageParts p;
    if (!image_parts(g, &p) || !host || !g->codes || !g->scales || !g->ikeys || (p.sel && !g->sel) ||
        (p.kscales && !g->ikey_scales) || (p.pool && !g->pool))
        return CSA2_ERR_INVALID_ARG;
    if (!g->has_entries) return CSA2_ERR_STATE;
    if (bytes < p.total) return CSA2_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* h = static_cast<char*>(host);
    const size_t B = (size_t)g->B, N = (size_t)g->N_cap, n = (size_t)p.n;
    hipError_t e = copy_rows(h, n * p.code_row, g->codes, N * p.code_row, n * p.code_row, B,
                             hipMemcpyDeviceToHost, s);
    if (e == hipSuccess)
        e = copy_rows(h + p.codes, n * p.scale_row, g->scales, N * p.scale_row, n * p.scale_row, B,
                      hipMemcpyDeviceToHost, s);
    if (e == hipSuccess)
        e = copy_rows(h + p.codes + p.scales, n * p.key_row, g->ikeys, N * p.key_row, n * p.key_row, B,
                      hipMemcpyDeviceToHost, s);
    if (e == hipSuccess && p.kscales)
        e = copy_rows(h + p.codes + p.scales + p.keys, n * p.kscale_row, g->ikey_scales, N * p.kscale_row,
                      n * p.kscale_row, B, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess && p.sel)
        e = hipMemcpyAsync(h + p.codes + p.scales + p.keys + p.kscales, g->sel, p.sel, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess && p.pool)
        e = hipMemcpyAsync(h + p.codes + p.scales + p.keys + p.kscales + p.sel, g->pool, p.pool,
                           hipMemcpyDeviceToHost, s);
    return hip_status(e);
}

csa2_status csa2_group_restore(csa2_group* g, const void* host, size_t bytes, void* stream) {
    ImageParts p;
    if (!image_parts(g, &p) || !host || !g->codes || !g->scales || !g->ikeys || (p.sel && !g->sel) ||
        (p.kscales && !g->ikey_scales) || (p.pool && !g->pool))
        return CSA2_ERR_INVALID_ARG;
    if (bytes < p.total) return CSA2_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const char* h = static_cast<const char*>(host);
    const size_t B = (size_t)g->B, N = (size_t)g->N_cap, n = (size_t)p.n;
    hipError_t e = copy_rows(g->codes, N * p.code_row, h, n * p.code_row, n * p.code_row, B,
                             hipMemcpyHostToDevice, s);
    if (e == hipSuccess)
        e = copy_rows(g->scales, N * p.scale_row, h + p.codes, n * p.scale_row, n * p.scale_row, B,
                      hipMemcpyHostToDevice, s);
    if (e == hipSuccess)
        e = copy_rows(g->ikeys, N * p.key_row, h + p.codes + p.scales, n * p.key_row, n * p.key_row, B,
                      hipMemcpyHostToDevice, s);
    if (e == hipSuccess && p.kscales)
        e = copy_rows(g->ikey_scales, N * p.kscale_row, h + p.codes + p.scales + p.keys, n * p.kscale_row,
                      n * p.kscale_row, B, hipMemcpyHostToDevice, s);
    if (e == hipSuccess && p.sel)
        e = hipMemcpyAsync(g->sel, h + p.codes + p.scales + p.keys + p.kscales, p.sel, hipMemcpyHostToDevice, s);
    if (e == hipSuccess && p.pool)
        e = hipMemcpyAsync(g->pool, h + p.codes + p.scales + p.keys + p.kscales + p.sel, p.pool,
                           hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return CSA2_ERR_HIP;
    g->has_entries = 1;
    return CSA2_OK;
}

}  // extern "C"
