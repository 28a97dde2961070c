/*
 * csa2.h - C ABI of the CSA2 layer-step library for AMD Instinct MI355X (gfx950).
 *
 * CSA2 (Compressed Sparse Attention 2, as described for DeepSeek-V4.1-Flash):
 * a lightweight indexer scores a compressed global KV cache, the top-k entries
 * are kept, and attention runs over those entries together with a local
 * sliding window ("Why Is DeepSeek V4.1 Flash So Fast?", sections 3 and 4).
 * Layers run in one of three modes that decide which of these steps they
 * repeat ("DeepSeek-V4.1-Flash", section "Sharing the cache across layers";
 * "Inference-Efficient LLMs: How Sparse Compute and Compressed Memory Work",
 * section 4).  The main cache is stored in FP4 with per-group scales (same
 * pages, "Fast memory, persistent storage and recomputation" and section 6).
 *
 * Parameters the pages leave open are fixed here:
 *   - FP4 element: OCP MX e2m1; one fp32 scale per 32 consecutive elements,
 *     scale = fl32(amax / 6); each element is rounded to the nearest multiple
 *     of the scale on the e2m1 grid, ties to the even code, magnitudes beyond
 *     6*scale saturate; element 2i sits in the low nibble of byte i.
 *   - Index score of entry j for query row r: the exact real value of
 *     sum_h sum_e iq[r,h,e] * ik[j,h,e], rounded once to fp32 (nearest, ties
 *     to even; an exact zero is +0).  Index elements are bf16 or fp8 e4m3fn.
 *   - Top-k: the k valid entries first in the order (score descending, index
 *     ascending), written in ascending index order, padded with -1.
 *   - Attention: one softmax over the selected entries and the query's window
 *     rows.  An entry (dequantised FP4 row of dim D) is both key and value and
 *     is shared by all Hq query heads; window keys and values are bf16 rows.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are device pointers owned by the caller, row-major
 *     and contiguous, 16-byte aligned.  bf16 and fp8 tensors are passed as raw
 *     bytes (const void*).
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *     asynchronously; no entry point synchronises or allocates device memory,
 *     and none but csa2_layer_step_noalloc keeps global mutable state, so calls
 *     on different streams with disjoint buffers may run concurrently.
 *   - Arguments are validated on the host before anything is launched; on an
 *     error nothing is enqueued and the status says why.  A launch failure
 *     returns CSA2_ERR_HIP.  No C++ exception crosses this interface.
 *   - Scratch memory is a caller-provided workspace of at least the size the
 *     matching *_workspace_bytes function returns; its contents on entry do
 *     not matter and are undefined on return.
 *   - Inputs must be finite; NaN or Inf inputs give unspecified results.
 */
#ifndef CSA2_H_
#define CSA2_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CSA2_OK = 0,
    CSA2_ERR_INVALID_ARG = 1, /* null pointer, bad size, misaligned pointer   */
    CSA2_ERR_UNSUPPORTED = 2, /* valid request outside the supported shapes   */
    CSA2_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required   */
    CSA2_ERR_STATE = 4,       /* mode not allowed in the group's current state */
    CSA2_ERR_HIP = 5          /* the HIP runtime reported an error             */
} csa2_status;

typedef enum {
    CSA2_MODE_FULL = 0,    /* writes its own entries, makes its own selection  */
    CSA2_MODE_REINDEX = 1, /* shares the group's entries, selects afresh        */
    CSA2_MODE_REUSE = 2    /* shares the group's entries and latest selection   */
} csa2_mode;

/* Index-key storage.  BF16 and FP8_E4M3: keys and index queries in that dtype.
 * FP4_E2M1 ("Why Is DeepSeek V4.1 Flash So Fast?", section 7: FP4 reaches the
 * indexer too): keys are stored with the cache's codec, e2m1 codes
 * [..][H*d/2] (element 2i in the low nibble) plus one fp32 scale per 32
 * consecutive elements [..][H*d/32], each key value code*scale exactly; index
 * queries are bf16 and H*d must be a multiple of 32. */
typedef enum { CSA2_IDX_BF16 = 0, CSA2_IDX_FP8_E4M3 = 1, CSA2_IDX_FP4_E2M1 = 2 } csa2_idx_dtype;

/* State of one sharing group ("DeepSeek-V4.1-Flash", "Sharing the cache
 * across layers": one stored copy of the entries per group, plus the
 * selection that Reuse layers share).  The struct lives in host memory and is
 * owned by the caller; the buffers it points to are device memory. */
typedef struct csa2_group {
    int32_t B;                /* sequences                                          */
    int64_t N_cap;            /* entry slots per sequence (row stride of the cache) */
    int32_t D;                /* entry dimension, multiple of 32, <= 256            */
    int32_t H_I, d_I;         /* index heads and index head dimension              */
    csa2_idx_dtype idx_dtype; /* dtype of index keys and index queries             */
    int32_t k;                /* entries kept per query row, 1 <= k <= N_cap        */
    uint8_t* codes;           /* [B][N_cap][D/2]   FP4 e2m1 codes                   */
    float* scales;            /* [B][N_cap][D/32]  fp32 block scales                */
    void* ikeys;              /* [B][N_cap][H_I][d_I] index keys                    */
    const int32_t* n_valid;   /* [B] valid entries per sequence, counting the step's
                                 own new rows; Qs <= n_valid[b] <= N_cap            */
    int64_t n_valid_max;      /* host copy of max_b n_valid[b], sizes the launches  */
    int32_t* sel;             /* [sel_rows][k] the group's current selection        */
    int32_t sel_rows;         /* rows sel can hold; must be >= B * Qs               */
    int32_t has_entries;      /* caller sets it after filling the cache; Full sets it */
    int32_t has_selection;    /* set by Full and Reindex, required by Reuse        */
    int32_t sel_qs;           /* Qs of the stored selection                         */
    float* ikey_scales;       /* FP4_E2M1 keys only: [B][N_cap][H_I*d_I/32] scales;
                                 ikeys then holds the codes [B][N_cap][H_I*d_I/2] */
    /* Hierarchical search ("Inference-Efficient LLMs", section 5): with
     * pool_blocks = P > 0 a Full layer also keeps, per query row, the P blocks of
     * CSA2_POOL_BLOCK consecutive entries whose largest index score ranks first
     * (ties to the lower block; blocks ascending, -1 padded), and Reindex layers
     * score and select only among the pool's valid entries.  P = 0: every
     * selecting layer searches all entries.  Requires k <= P * CSA2_POOL_BLOCK. */
    int32_t pool_blocks;
    int32_t* pool;            /* [sel_rows][pool_blocks] block indices (library-written) */
    int32_t has_pool;         /* set by Full when pool_blocks > 0                   */
    int32_t pool_qs;          /* Qs of the stored pool                              */
} csa2_group;

#define CSA2_POOL_BLOCK 8

/* Per-layer inputs.  Every mode uses its own queries and window ("every layer
 * keeps its own queries and its own local-window state"). */
typedef struct csa2_layer_args {
    int32_t Qs;            /* query rows per sequence: 1 for decode, >1 for a prefill
                              chunk (row i of the chunk sits at entry n_valid-Qs+i and
                              sees entries j <= n_valid-Qs+i)                       */
    int32_t Hq;            /* query heads, 1..32                                      */
    const void* q;         /* bf16 [B][Qs][Hq][D]                                     */
    const void* iq;        /* [B][Qs][H_I][d_I] in idx_dtype (bf16 for FP4_E2M1 keys);
                              Full and Reindex only                                   */
    const void* wk;        /* bf16 [B][Qs+W-1][D] window keys; row i..i+W-1 for row i */
    const void* wv;        /* bf16 [B][Qs+W-1][D] window values                       */
    int32_t W;             /* window rows per query (0..1024)                         */
    const int32_t* wlen;   /* [B] valid window rows, counted from the end of the
                              window buffer; NULL = all valid                         */
    const float* new_entry;/* fp32 [B][Qs][D]: Full writes these at slots
                              n_valid-Qs .. n_valid-1                                 */
    const void* new_ikey;  /* [B][Qs][H_I][d_I] index keys stored with them (Full); in
                              idx_dtype, or fp32 for FP4_E2M1 (packed on write)       */
    float sm_scale;        /* softmax scale, e.g. 1/sqrt(D)                           */
    float* out;            /* fp32 [B][Qs][Hq][D]                                     */
    float* lse;            /* fp32 [B][Qs][Hq] natural-log sum-exp, or NULL           */
    void* index_events[2]; /* optional hipEvent_t pair for timing (NULL = none): a Full
                              or Reindex layer records [0] on the stream right before its
                              first index-scoring kernel (S2; for a prefill chunk on the
                              MFMA path, the threshold-sample GEMM) and [1] right after
                              its last (the score stream, or the filter GEMM); Reuse
                              records neither                                         */
} csa2_layer_args;

/* Human-readable name of a status code (static storage). */
const char* csa2_status_str(csa2_status s);

/* Library version string (static storage). */
const char* csa2_version(void);

/* S1 - FP4 cache write ("Fast memory, persistent storage and recomputation";
 * "Inference-Efficient LLMs", section 6: FP4 main KV with per-group scaling).
 * x: fp32 [rows][dim]; codes: [rows][dim/2]; scales: [rows][dim/32].
 * dim must be a positive multiple of 32.  rows == 0 is a no-op. */
csa2_status csa2_fp4_pack(const float* x, int64_t rows, int32_t dim, uint8_t* codes,
                          float* scales, void* stream);

/* S2 - Index scores ("Why Is DeepSeek V4.1 Flash So Fast?", section 4: a
 * cheaper search scores positions before attention; "Inference-Efficient
 * LLMs", section 5).  iq: [B][Qs][H][d], ik: [B][N][H][d] in `dtype`
 * (FP4_E2M1: iq bf16, ik the codes [B][N][H*d/2] and ik_scales [B][N][H*d/32];
 * ik_scales is ignored for the other dtypes); scores: fp32 [B][Qs][N], each
 * the exact sum rounded once to fp32 (see the top of this file).
 * causal_offset: -1 scores every entry for every query row; c >= 0 makes row i
 * of each sequence a causal query at position c + i ("Why Is DeepSeek V4.1
 * Flash So Fast?", section 3: a query retrieves from the positions before it):
 * it scores entries j <= c + i, and scores[.., i, j] = -inf for the others.
 * exact: 1 asks for the exactly rounded scores; 0 allows a faster, inexact
 * variant.  Both give the exact scores: for bf16 and fp8 keys the exact stream
 * already runs at the memory bound, so no second, inexact kernel is kept.
 * H*d must be a multiple of 64 (bf16), 128 (fp8) or 256 (FP4) for the
 * streaming kernel, and at most 4096.  N == 0 is a no-op.  CSA2_ERR_UNSUPPORTED
 * when B*Qs > 65535, N >= 2^31 or the launch would exceed 2^32 - 1 work-items
 * (about B*Qs*N > 4.29e9), with nothing enqueued. */
csa2_status csa2_index_score(const void* iq, const void* ik, const float* ik_scales,
                             csa2_idx_dtype dtype, int32_t B, int32_t Qs, int64_t N, int32_t H,
                             int32_t d, int64_t causal_offset, int32_t exact, float* scores,
                             void* stream);

/* S3 - Top-k selection ("Why Is DeepSeek V4.1 Flash So Fast?", sections 3 and
 * 4: select the useful compressed positions).  scores: fp32 [R][ld], row r
 * considers entries j < n_valid[r] (n_valid: device int32 [R], or NULL = N).
 * idx: int32 [R][k] ascending, -1 padded.  Ties go to the lower index; -0 and
 * +0 are equal.  Scores must not be NaN. */
size_t csa2_topk_workspace_bytes(int64_t R, int64_t N, int32_t k);
csa2_status csa2_topk(const float* scores, int64_t R, int64_t N, int64_t ld,
                      const int32_t* n_valid, int32_t k, int32_t* idx, void* ws, size_t ws_bytes,
                      void* stream);

/* S5+S6 - Gather, dequantise and attend ("Why Is DeepSeek V4.1 Flash So
 * Fast?", sections 3 and 4: expensive attention only over the selected
 * positions plus the 128-token window).  q: bf16 [B][Qs][Hq][D]; codes/scales:
 * [B][N] records as in csa2_fp4_pack; idx: int32 [B*Qs][k] (-1 = empty slot,
 * other values must be < N); wk, wv: bf16 [B][Qs+W-1][D], query row i uses
 * window rows i..i+W-1 of which only the last wlen[b] rows of the buffer are
 * valid (wlen NULL = all); out fp32 [B][Qs][Hq][D]; lse fp32 [B][Qs][Hq] or
 * NULL.  A row with nothing to attend gets out = 0 and lse = -inf.  Window rows
 * outside the valid tail and records no slot selects never reach the result,
 * so they may hold any bits (NaN and Inf included). */
size_t csa2_attend_workspace_bytes(int32_t B, int32_t Qs, int32_t Hq, int32_t D, int32_t k,
                                   int32_t W);
csa2_status csa2_sparse_attend(const void* q, int32_t B, int32_t Qs, int32_t Hq, int32_t D,
                               const uint8_t* codes, const float* scales, int64_t N,
                               const int32_t* idx, int32_t k, const void* wk, const void* wv,
                               int32_t W, const int32_t* wlen, float sm_scale, float* out,
                               float* lse, void* ws, size_t ws_bytes, void* stream);

/* S4 - One CSA2 layer in the given mode ("DeepSeek-V4.1-Flash", "Sharing the
 * cache across layers"; "Why Is DeepSeek V4.1 Flash So Fast?", section 5):
 *   FULL    packs new_entry/new_ikey into slots n_valid-Qs .. n_valid-1,
 *           scores the group's keys with iq, selects into g->sel, attends;
 *           with pool_blocks > 0 it also writes the pool (g->pool);
 *   REINDEX scores the shared keys with its own iq, overwrites g->sel, attends;
 *           writes no entries (CSA2_ERR_STATE if g->has_entries == 0);
 *           with pool_blocks > 0 it scores only the entries of the pool the
 *           latest Full left and leaves the pool as it is (CSA2_ERR_STATE if
 *           g->has_pool == 0 or g->pool_qs != Qs);
 *   REUSE   attends with g->sel as left by the latest Full/Reindex of the
 *           group; writes neither entries nor the selection (CSA2_ERR_STATE if
 *           g->has_selection == 0 or g->sel_qs != Qs).
 * The library updates g->has_entries, g->has_selection and g->sel_qs on the
 * host when the work has been enqueued. */
size_t csa2_layer_workspace_bytes(const csa2_group* g, int32_t Qs, int32_t Hq, int32_t W);
csa2_status csa2_layer_step(csa2_mode mode, const csa2_layer_args* a, csa2_group* g, void* ws,
                            size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * layer step as csa2_layer_step, with the workspace taken from a scratch array
 * of CSA2_STATIC_SCRATCH_BYTES that the library keeps in device memory on each
 * GPU it runs on, from the first call there until the process ends.  It
 * allocates nothing.  Returns CSA2_ERR_WORKSPACE, with nothing enqueued, when
 * the layer needs more (csa2_layer_workspace_bytes > CSA2_STATIC_SCRATCH_BYTES;
 * a decode step needs about 12 bytes per (query row, entry slot) plus the
 * attention partials, so up to about 10 million slots fit, B = 64 at N =
 * 131,072 among them; prefill chunks do not); other errors as csa2_layer_step.  Every call on one GPU uses that GPU's one array,
 * which keeps the last call's contents (each call sets what it needs before
 * reading it): calls that overlap in time on one GPU (several streams or host
 * threads) race and give undefined results; calls ordered on one stream are
 * safe. */
#define CSA2_STATIC_SCRATCH_BYTES ((size_t)128 << 20)
csa2_status csa2_layer_step_noalloc(csa2_mode mode, const csa2_layer_args* a, csa2_group* g,
                                    void* stream);

/* S7 - Cache accounting ("DeepSeek-V4.1-Flash", "Several mechanisms in one
 * release": entries x numbers per entry x stored layer copies x bits per
 * number).  Returns bytes, or -1 if an argument is negative or the product
 * overflows int64. */
int64_t csa2_cache_bytes(int64_t entries, int64_t numbers, int64_t copies, int64_t bits);

/* Persistent tier ("DeepSeek-V4.1-Flash", "Fast memory, persistent storage
 * and recomputation": the FP4 main entries are what a slower storage tier keeps
 * and brings back; "Why Is DeepSeek V4.1 Flash So Fast?", section 7).
 *
 * A group image is a packed byte copy of what a group holds for entries
 * 0 .. n_valid_max-1 of every sequence, in this order:
 *   codes  [B][n_valid_max][D/2]     u8
 *   scales [B][n_valid_max][D/32]    f32
 *   ikeys  [B][n_valid_max][H_I][d_I] in idx_dtype (FP4: codes [..][H_I*d_I/2])
 *   ikey_scales [B][n_valid_max][H_I*d_I/32] f32, FP4 index keys only
 *   sel    [B*sel_qs][k]             i32, only when has_selection is set
 *   pool   [B*pool_qs][pool_blocks]  i32, only when has_pool is set.
 * csa2_group_image_bytes returns its size (0 for an invalid group).
 * csa2_group_save copies the group into `host` (bytes >= the image size;
 * CSA2_ERR_STATE if the group holds no entries).  csa2_group_restore copies an
 * image back into a group of the same geometry, n_valid_max, has_selection,
 * sel_qs, has_pool and pool_qs, and sets has_entries.  Both are asynchronous on `stream`: the host
 * buffer must stay alive until the stream reaches them, and it should be
 * pinned (page-locked) for the copies to run at full rate.  Copy failures
 * return CSA2_ERR_HIP; nothing is validated against the image's contents. */
size_t csa2_group_image_bytes(const csa2_group* group);
csa2_status csa2_group_save(const csa2_group* group, void* host, size_t bytes, void* stream);
csa2_status csa2_group_restore(csa2_group* group, const void* host, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_H_ */
