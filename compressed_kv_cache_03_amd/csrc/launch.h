// Internal launch interface between the C-ABI host code and the HIP kernels.
// Every function enqueues work on `stream` and returns hipGetLastError().
// Shapes are validated by the caller (csa2_api.cpp) before these are reached.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

constexpr int kHistBitsHost = 12;
constexpr int64_t kHistBinsHost = 1 << kHistBitsHost;  // first radix digit bins per row

// Zero `words` uint32 words (a plain fill kernel, safe inside graph capture).
// A Full layer's writes before scoring in one launch (pack.hip): entries,
// their index keys and the zeroed digit histogram.
struct FullPrepArgs {
    const float* entry;    // fp32 [rows][D]
    int64_t rows;
    int D;
    uint8_t* codes;
    float* scales;
    const void* key;       // [rows][K] stored as is (key_words u32 each) or fp32 to pack
    int key_fp4;
    int K, key_words;
    void* ikeys;
    float* ikey_scales;
    const int32_t* nvb;
    int Qs;
    int64_t N_cap;
    uint32_t* zero;
    int64_t zero_words;
    int64_t nb_pack = 0, nb_key = 0;  // filled by launch_full_prep
};
hipError_t launch_full_prep(const FullPrepArgs& a, hipStream_t stream);
hipError_t launch_zero(uint32_t* p, int64_t words, hipStream_t stream);

// S1: see pack.hip for the row -> slot mapping when nvb != nullptr.
hipError_t launch_fp4_pack(const float* x, int64_t rows, int dim, uint8_t* codes, float* scales,
                           const int32_t* nvb, int Qs, int64_t N_cap, hipStream_t stream);
// Copy rows of row_bytes (multiple of 4) to the same slots as launch_fp4_pack.
hipError_t launch_store_rows(const void* src, int64_t rows, int row_bytes, void* dst,
                             const int32_t* nvb, int Qs, int64_t N_cap, hipStream_t stream);

// Largest global size (work-items along one grid dimension) a launch may have.
constexpr int64_t kMaxGridThreads = 0xffffffffLL;

// S2: exact index scores.  Row r = b*Qs + i scores entries j < nv(r) of
// sequence b (ik row stride N_cap entries), where nv(r) = nvb[b] - Qs + i + 1
// when nvb is set, causal + i + 1 when causal >= 0, and N otherwise (clamped to
// [0, N]).  Writes scores[r*ld + j].
// When hist != nullptr, also accumulates the first radix digit histogram of
// every written score into hist[r*4096 + digit].
struct ScoreArgs {
    const void* iq;       // [R][K]
    const void* ik;       // [B][N_cap][K] (dtype 2: e2m1 codes [B][N_cap][K/2])
    const float* ik_scales;  // dtype 2: [B][N_cap][K/32]
    int dtype;            // 0 bf16, 1 e4m3, 2 FP4 e2m1 keys with bf16 queries
    int K;                // H*d
    int B, Qs;
    int64_t N;            // entries to consider per sequence (<= N_cap)
    int64_t N_cap;        // entry row stride of ik
    const int32_t* nvb;   // [B] or null
    int64_t causal = -1;  // with nvb null: row i sees j <= causal + i (-1: every entry)
    float* scores;        // [R][ld]
    int64_t ld;
    uint32_t* hist;       // [R][4096] or null
    // hierarchical search: score the positions of a candidate pool instead of
    // 0..N-1.  Slot s of row r is position 8 * pool[r][s / 8] + s % 8 (pool blocks
    // ascending, -1 padded); N is then 8 * pool_blocks and the row's valid slots
    // are the prefix 0 .. pool_nv[r] - 1.
    const int32_t* pool = nullptr;
    int pool_blocks = 0;
    const int32_t* pool_nv = nullptr;
    // several query rows per sequence (Qs >= 2, bf16 keys, K = 128 or 256):
    // with a queue for undecided scores (counter zeroed beforehand, room for
    // one (row, entry) per score) the rows share each key load
    uint32_t* fix_cnt = nullptr;
    uint2* fix_list = nullptr;
    // filled by launch_score_exact: with several query rows per sequence the
    // blocks of one entry block and all its rows run together on one XCD
    int64_t n_eblk = 0, blocks = 0, per_xcd = 0;
    int64_t persist = 0;  // single-row stream: resident workgroups per row (0: one per block)
};
hipError_t launch_score_exact(const ScoreArgs& a, hipStream_t stream);
// Work-items along x of the launches launch_score_exact would make for a.
int64_t score_grid_threads(const ScoreArgs& a);
// scores[r*ld + j] = -inf for nv(r) <= j < N (a causal cut-off's hidden entries).
hipError_t launch_score_tail(const ScoreArgs& a, hipStream_t stream);

// Hierarchical search helpers (pool.hip), positions grouped in blocks of 8.
constexpr int kPoolBlock = 8;
// bmax[r][j] = largest score among the valid positions 8j .. 8j+7 of row r
// (valid count as for TopkArgs: nvb and Qs, or N when nvb is null); blk_nv[r] =
// number of blocks holding a valid position.
hipError_t launch_block_max(const float* scores, int64_t R, int64_t N, int64_t ld, const int32_t* nvb,
                            int Qs, float* bmax, int64_t ld_blk, int32_t* blk_nv, hipStream_t stream);
// pool_nv[r] = number of leading slots of row r's pool whose position is valid.
hipError_t launch_pool_count(const int32_t* pool, int64_t R, int P, const int32_t* nvb, int Qs,
                             int32_t* pool_nv, hipStream_t stream);
// idx[r][j] (a slot of row r's pool, or -1) becomes the position it stands for.
hipError_t launch_pool_map(int32_t* idx, int64_t R, int k, const int32_t* pool, int P, hipStream_t stream);

// S3: top-k over scores [R][ld] with per-row valid counts nv(r) as above (Qs,
// nvb) and k.  hist must already hold the digit histogram of each row's valid
// scores (launch_topk_hist builds it when the scores come from elsewhere).
struct TopkArgs {
    const float* scores;
    int64_t R, N, ld;
    const int32_t* nvb;
    int Qs;
    int k;
    int32_t* idx;         // [R][k]
    uint32_t* hist;       // [R][4096]
    int32_t* cand_idx;    // [R][N]
    uint32_t* cand_key;   // [R][N]
    uint32_t* slice_cnt;  // [R][slices]
    int slices;           // slices per row
    int64_t slice_len;
    uint32_t* bits = nullptr;  // [R][bits_ld] bitmap words of the split path (null: no split path)
    int64_t bits_ld = 0;       // words per row, >= ceil(N / 32)
};
int64_t topk_slice_len(int64_t N);
hipError_t launch_topk_hist(const TopkArgs& a, hipStream_t stream);
hipError_t launch_topk_select(const TopkArgs& a, hipStream_t stream);

// S5+S6: sparse attention with split-k partials and a combine pass.
struct AttendArgs {
    const uint16_t* q;    // [R][Hq][D] bf16
    int B, Qs, Hq, D;
    const uint8_t* codes; // [B][N][D/2]
    const float* scales;  // [B][N][D/32]
    int64_t N;
    const int32_t* idx;   // [R][k]
    int k;
    const uint16_t* wk;   // [B][Qs+W-1][D]
    const uint16_t* wv;
    int W;
    const int32_t* wlen;  // [B] or null
    float sm_scale;
    float* out;           // [R][Hq][D]
    float* lse;           // [R][Hq] or null
    float* part;          // [R][splits][Hq][D+2] when a row is split, else unused
};
// Splits per query row (and keys per split) used by launch_attend for R rows.
void attend_splits(int64_t R, int Hq, int D, int k, int W, int* splits, int* chunk);
hipError_t launch_attend(const AttendArgs& a, hipStream_t stream);

// S2+S3 for prefill chunks with e4m3 index keys (index_gemm.hip).
struct GemmArgs {
    const uint8_t* iq;     // [B][Qs][K] e4m3
    const uint8_t* ik;     // [B][N_cap][K] e4m3
    int K;                 // 128 or 256
    int B, Qs;
    int64_t N;             // entries considered per sequence (<= N_cap)
    int64_t N_cap;
    const int32_t* nvb;    // [B]: row i sees j < nvb[b] - Qs + i + 1 (or null: j < N)
    int64_t stride;        // column c is entry c * stride
    int64_t ncols;         // columns per sequence
    // filled by launch_gemm_fp8
    int n_rowblk;
    int64_t n_colblk, tiles, per_xcd;
    float* out;            // mode 0: [B*Qs][ncols] scores (-inf where not visible)
    const float* theta;    // mode 1 (stride 1): [B*Qs] thresholds
    uint2* blk;            // mode 1: [filter_colblks(ncols)][B*Qs][filter_blk_cap()] (key, entry)
    uint32_t* blkcnt;      // mode 1: [filter_colblks(ncols)][B*Qs] candidates per region
    uint2* cand;           // mode 1: [B*Qs][cap] overflow beyond a region's capacity
    uint32_t* cand_cnt;    // mode 1: [B*Qs] overflow counts (zeroed beforehand)
    int cap;
};
hipError_t launch_gemm_fp8(GemmArgs a, int mode, hipStream_t stream);
int64_t gemm_grid_threads(const GemmArgs& a, int mode);  // work-items along x of that launch
int64_t filter_colblks(int64_t ncols);  // column-block regions per row of the filter
int filter_blk_cap();                   // candidates per region

struct BandArgs {
    int B, Qs, K, k;
    int64_t N, N_cap;
    const int32_t* nvb;
    const uint8_t* iq;
    const uint8_t* ik;
    int64_t stride, ncols;
    const float* samp;     // [B*Qs][ncols]
    float* theta;          // [B*Qs]
    const uint2* blk;      // filter regions and counts (see GemmArgs)
    const uint32_t* blkcnt;
    int64_t n_colblk;
    const uint2* cand;     // overflow lists
    uint32_t* cand_cnt;
    int cap;
    float* knorm;          // [B][nblk] bounds on max ||k||^2 per 256 entries
    uint8_t* kexp;         // [B][nblk][K/8] largest key exponent field per block and group of 8
    float* kseq_norm;      // [B] largest knorm of the sequence
    uint8_t* kseq_exp;     // [B][K/8] largest kexp of the sequence per group
    int nblk;
    int32_t* idx;          // [B*Qs][k] selection
    int32_t* flag;         // [B*Qs] rows recomputed exactly
    uint32_t* flag_count;
    float* scores;         // [B*Qs][ld] exact scores of flagged rows
    int64_t ld;
};
hipError_t launch_sample_select(const BandArgs& a, hipStream_t stream);
hipError_t launch_key_norm(const uint8_t* ik, int K, int B, int64_t N, int64_t N_cap, int nblk, float* knorm,
                           uint8_t* kexp, float* kseq_norm, uint8_t* kseq_exp, hipStream_t stream);
hipError_t launch_band_final(const BandArgs& a, hipStream_t stream);
int band_cap(int k);    // candidate list length per row
int band_max_k();       // largest k the candidate path handles

}  // namespace csa2
