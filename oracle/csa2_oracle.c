/*
 * CSA2 CPU ORACLE - TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, step-by-step CPU implementation of one CSA2 layer step
 * (Compressed Sparse Attention 2 as described for DeepSeek-V4.1-Flash), used
 * only to check the GPU library.  It is loaded solely by the tests, by the
 * smoke check and by the bench's CPU-baseline leg; the product path never
 * links or calls it, and it shares no source with the GPU library.
 *
 * Sources (page title, section):
 *   [P1] "Why Is DeepSeek V4.1 Flash So Fast?", sections 3 (CSA2: 128-token
 *        sliding window plus a small set of retrieved compressed positions),
 *        4 (the indexer: a cheap relevance search, then top-k, then the
 *        expensive attention only on what was selected) and 5 (Full, Reindex,
 *        Reuse layers).
 *   [P2] "DeepSeek-V4.1-Flash" (visual-learn), sections "Sharing the cache
 *        across layers" (the three modes; every layer keeps its own queries
 *        and window; the 16-layer x 4,096-entry worked cache figure),
 *        "Fast memory, persistent storage and recomputation" (main cache
 *        entries in FP4) and "Several mechanisms in one release" (the cache
 *        size formula).
 *   [P3] "Inference-Efficient LLMs: How Sparse Compute and Compressed Memory
 *        Work", sections 4 (CSA2 modes: all modes compute their own query and
 *        SWA state), 5 (scoring every compressed position is the expensive
 *        part of sparse attention) and 6 (FP4 main KV with per-group scaling;
 *        the window stays at higher precision).
 * The pages fix neither the score formula, the tie rule, the FP4 block layout
 * nor the merge of the global and window parts.  Each reading used below is
 * stated where it is used:
 *   - score of entry j: sum over heads h and dims e of iq[h,e]*ik[j,h,e],
 *     rounded once to fp32 (round-to-nearest-even) from the exact real sum;
 *   - top-k: order by (score descending, index ascending); emit the selected
 *     indices in ascending order, padded with -1 when fewer than k are valid;
 *   - FP4: OCP MX e2m1 element, fp32 scale per 32 consecutive elements equal
 *     to fl32(amax/6), element rounded to the nearest representable multiple
 *     of the scale with ties to the even code, element 2i in the low nibble;
 *   - attention: one joint softmax over the selected entries and the window
 *     rows; an entry is one 128-vector used as both key and value and shared
 *     by all query heads; window keys and values are separate bf16 rows.
 *
 * Pins: every function below is checked, in the CPU tests, against something
 * other than itself (the format's exhaustive code table, exact rational
 * arithmetic, brute-force sorts, textbook dense attention at k = N, the
 * pages' worked cache figure, mode invariants); none is parity unpinned.
 * What no test can pin is the real model behind the pages (its score
 * function, dimensions and scale rule, its bytes per token, the quality of
 * its selections): these are readings, stated above, not reproductions.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* FP4 e2m1 element: sign bit 3, exponent bits 2-1 (bias 1), mantissa bit 0. */
/* Exponent 0 encodes the subnormal 0.5*m.  Values +-{0,0.5,1,1.5,2,3,4,6}.  */
/* ------------------------------------------------------------------------ */
double orc_e2m1_value(int code) {
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* Magnitude code (0..7) nearest to a >= 0 on the grid {v_c * scale}; a tie
   between two neighbours goes to the even code.  The decision points are the
   midpoints t*scale with t = (v_c + v_{c+1})/2; t*scale and a are exact in
   fp64 (scale has 24 significant bits, t at most 3), so every comparison is
   exact. */
static int e2m1_nearest_mag(double a, double scale) {
    static const double t[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
    int c = 0;
    for (int i = 0; i < 7; ++i) {
        double thr = t[i] * scale;
        if (a > thr) {
            c = i + 1;
        } else {
            if (a == thr) c = (i % 2 == 0) ? i : i + 1;
            break;
        }
    }
    return c;
}

/* [P2 "Fast memory..."], [P3 s6]: quantise rows of x (fp32 [rows][dim],
   dim % 32 == 0) into e2m1 codes [rows][dim/2] and scales [rows][dim/32]. */
void orc_fp4_pack(const float* x, int64_t rows, int dim, uint8_t* codes, float* scales) {
    for (int64_t r = 0; r < rows; ++r) {
        const float* xr = x + r * dim;
        uint8_t* cr = codes + r * (dim / 2);
        memset(cr, 0, (size_t)(dim / 2));
        for (int b = 0; b < dim / 32; ++b) {
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                float v = fabsf(xr[32 * b + i]);
                if (v > amax) amax = v;
            }
            float scale = amax / 6.0f; /* one IEEE fp32 division */
            scales[r * (dim / 32) + b] = scale;
            for (int i = 0; i < 32; ++i) {
                int g = 32 * b + i;
                float v = xr[g];
                int code = e2m1_nearest_mag(fabs((double)v), (double)scale) | (signbit(v) ? 8 : 0);
                cr[g / 2] |= (uint8_t)((g & 1) ? (code << 4) : code);
            }
        }
    }
}

/* Exact dequantisation: value = e2m1(code) * scale, exact in fp64. */
void orc_fp4_dequant(const uint8_t* codes, const float* scales, int64_t rows, int dim, double* out) {
    for (int64_t r = 0; r < rows; ++r)
        for (int g = 0; g < dim; ++g) {
            uint8_t byte = codes[r * (dim / 2) + g / 2];
            int code = (g & 1) ? (byte >> 4) : (byte & 15);
            out[r * dim + g] = orc_e2m1_value(code) * (double)scales[r * (dim / 32) + g / 32];
        }
}

/* ------------------------------------------------------------------------ */
/* Stored index elements.  dtype 0: bf16 bits (uint16); dtype 1: OCP fp8     */
/* e4m3fn bits (uint8: bias 7, exponent 0 subnormal m*2^-9, S.1111.111 NaN).  */
/* ------------------------------------------------------------------------ */
static double bf16_value(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static double e4m3_value(uint8_t b) {
    int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
    double mag;
    if (e == 15 && m == 7) mag = NAN;
    else if (e == 0) mag = ldexp((double)m, -9);
    else mag = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

double orc_idx_value(int dtype, const void* base, int64_t i) {
    return dtype == 0 ? bf16_value(((const uint16_t*)base)[i]) : e4m3_value(((const uint8_t*)base)[i]);
}

/* ------------------------------------------------------------------------ */
/* Exact sum of exact fp64 terms, rounded once to fp32 (long accumulator).   */
/* The accumulator is a fixed-point integer with unit 2^KEMIN held in 32-bit */
/* digits (stored in int64 so that carries can be deferred).                 */
/* ------------------------------------------------------------------------ */
#define KL 72
#define KEMIN (-1140)

typedef struct {
    int64_t l[KL];
} kacc;

static void kacc_add(kacc* a, double p) {
    if (p == 0.0) return;
    int e;
    double f = frexp(p, &e);            /* p = f * 2^e with 0.5 <= |f| < 1 */
    int64_t m = (int64_t)ldexp(f, 53);  /* exact: p = m * 2^(e-53) */
    int pos = e - 53 - KEMIN;           /* digit position of m's unit bit */
    int li = pos >> 5, sh = pos & 31;
    __int128 v = (__int128)m * ((__int128)1 << sh);
    a->l[li] += (int64_t)(uint32_t)(unsigned __int128)v;
    a->l[li + 1] += (int64_t)(uint32_t)(unsigned __int128)(v >> 32);
    a->l[li + 2] += (int64_t)(v >> 64);
}

static void kacc_carry(kacc* a) {
    for (int i = 0; i < KL - 1; ++i) {
        int64_t c = a->l[i] >> 32; /* floor division by 2^32 */
        a->l[i] -= c * 4294967296LL;
        a->l[i + 1] += c;
    }
}

static int kacc_bit(const kacc* a, int i) {
    if (i < 0) return 0;
    return (int)((a->l[i >> 5] >> (i & 31)) & 1);
}

static int kacc_any_below(const kacc* a, int i) { /* any bit at position < i */
    if (i <= 0) return 0;
    int li = i >> 5;
    for (int j = 0; j < li; ++j)
        if (a->l[j]) return 1;
    int64_t mask = (((int64_t)1) << (i & 31)) - 1;
    return (a->l[li] & mask) != 0;
}

static float kacc_to_f32(kacc* a) {
    kacc_carry(a);
    int neg = a->l[KL - 1] < 0;
    if (neg) {
        for (int i = 0; i < KL; ++i) a->l[i] = -a->l[i];
        kacc_carry(a);
    }
    int top = -1;
    for (int i = KL - 1; i >= 0 && top < 0; --i)
        if (a->l[i]) top = 32 * i + 63 - __builtin_clzll((unsigned long long)a->l[i]);
    if (top < 0) return 0.0f; /* exact zero is +0 */
    int lsb = top - 23;                 /* 24 significant bits */
    const int lsb_min = -149 - KEMIN;   /* fp32 subnormal quantum 2^-149 */
    if (lsb < lsb_min) lsb = lsb_min;
    uint64_t mant = 0;
    for (int i = top; i >= lsb; --i) mant = (mant << 1) | (uint64_t)kacc_bit(a, i);
    int rbit = kacc_bit(a, lsb - 1);
    int sticky = kacc_any_below(a, lsb - 1);
    if (rbit && (sticky || (mant & 1))) mant += 1; /* round half to even */
    float r = (float)ldexp((double)mant, lsb + KEMIN); /* exact, or inf past the range */
    return neg ? -r : r;
}

/* fp32 RNE of the exact value of sum_i a[i]*b[i]; every product must be exact
   in fp64 (true for bf16*bf16 and e4m3*e4m3). */
float orc_exact_dot_f32(const double* a, const double* b, int n) {
    kacc acc;
    memset(&acc, 0, sizeof acc);
    for (int i = 0; i < n; ++i) kacc_add(&acc, a[i] * b[i]);
    return kacc_to_f32(&acc);
}

/* fp32 RNE of the exact sum of n exact fp64 terms. */
float orc_exact_sum_f32(const double* t, int n) {
    kacc acc;
    memset(&acc, 0, sizeof acc);
    for (int i = 0; i < n; ++i) kacc_add(&acc, t[i]);
    return kacc_to_f32(&acc);
}

/* [P1 s4], [P3 s5]: index scores.  iq [B][Qs][H][d], ik [B][N][H][d] in the
   stored dtype; scores [B][Qs][N] = fp32 RNE of the exact
   sum_h sum_e iq[b,i,h,e] * ik[b,j,h,e].  Rows r=(b,i) score entries
   j < n_valid_row[r] only (NULL: all N); the rest are set to -inf.
   dtype 2 ([P1 s7]: the indexer itself in FP4): keys are e2m1 codes
   [B][N][H*d/2] with fp32 scales [B][N][H*d/32] (the cache codec), each key
   value code*scale exactly; the index queries are bf16. */
void orc_index_score(int dtype, const void* iq, const void* ik, const float* ik_scales, int64_t B,
                     int64_t Qs, int64_t N, int H, int d, const int64_t* n_valid_row, float* scores) {
    const int K = H * d;
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t i = 0; i < Qs; ++i) {
            int64_t r = b * Qs + i;
            double* qv = (double*)malloc(sizeof(double) * K);
            double* kv = (double*)malloc(sizeof(double) * K);
            for (int e = 0; e < K; ++e) qv[e] = orc_idx_value(dtype == 2 ? 0 : dtype, iq, r * K + e);
            int64_t nv = n_valid_row ? n_valid_row[r] : N;
            for (int64_t j = 0; j < N; ++j) {
                if (j >= nv) {
                    scores[r * N + j] = -INFINITY;
                    continue;
                }
                if (dtype == 2)
                    orc_fp4_dequant((const uint8_t*)ik + (b * N + j) * (K / 2), ik_scales + (b * N + j) * (K / 32),
                                    1, K, kv);
                else
                    for (int e = 0; e < K; ++e) kv[e] = orc_idx_value(dtype, ik, (b * N + j) * K + e);
                scores[r * N + j] = orc_exact_dot_f32(qv, kv, K);
            }
            free(qv);
            free(kv);
        }
}

/* ------------------------------------------------------------------------ */
/* Top-k [P1 s3, s4]: the k valid entries that come first under the order    */
/* (score descending, index ascending); emitted in ascending index order and */
/* padded with -1 when fewer than k entries are valid.  Scores must not be   */
/* NaN; -0 and +0 compare equal.                                            */
/* ------------------------------------------------------------------------ */
typedef struct {
    float s;
    int32_t j;
} sj_t;

static int cmp_score_desc_index_asc(const void* A, const void* B) {
    const sj_t* a = (const sj_t*)A;
    const sj_t* b = (const sj_t*)B;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    return (a->j > b->j) - (a->j < b->j);
}

static int cmp_int_asc(const void* A, const void* B) {
    int32_t a = *(const int32_t*)A, b = *(const int32_t*)B;
    return (a > b) - (a < b);
}

void orc_topk(const float* scores, int64_t R, int64_t N, int64_t ld, const int64_t* n_valid, int k,
              int32_t* idx) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < R; ++r) {
        int64_t nv = n_valid ? n_valid[r] : N;
        if (nv > N) nv = N;
        if (nv < 0) nv = 0;
        sj_t* v = (sj_t*)malloc(sizeof(sj_t) * (size_t)(nv > 0 ? nv : 1));
        for (int64_t j = 0; j < nv; ++j) {
            v[j].s = scores[r * ld + j];
            v[j].j = (int32_t)j;
        }
        qsort(v, (size_t)nv, sizeof(sj_t), cmp_score_desc_index_asc);
        int64_t take = nv < k ? nv : k;
        int32_t* out = idx + r * k;
        for (int64_t t = 0; t < take; ++t) out[t] = v[t].j;
        qsort(out, (size_t)take, sizeof(int32_t), cmp_int_asc);
        for (int64_t t = take; t < k; ++t) out[t] = -1;
        free(v);
    }
}

/* ------------------------------------------------------------------------ */
/* Hierarchical search [P3 s5 "Hierarchical Sparse Indexing"]: a Full layer  */
/* searches every position and keeps a pool of P blocks of 8 consecutive     */
/* positions (the report's example: 2,048 blocks x 8 = 16,384 candidates);   */
/* Reindex layers then rank only the pool's positions.  The pages fix no     */
/* block-score rule; here a block's score is the largest index score among   */
/* its valid positions, blocks are ranked by (score descending, block index  */
/* ascending) with the same top-k as the positions, and the pool is the P    */
/* best blocks, ascending, -1 padded.                                        */
/* ------------------------------------------------------------------------ */
#define ORC_POOL_BLOCK 8

void orc_pool_blocks(const float* scores, int64_t R, int64_t ld, const int64_t* n_valid, int P,
                     int32_t* pool) {
    int64_t nb_max = 0;
    for (int64_t r = 0; r < R; ++r) {
        int64_t nb = (n_valid[r] + ORC_POOL_BLOCK - 1) / ORC_POOL_BLOCK;
        if (nb > nb_max) nb_max = nb;
    }
    if (nb_max < 1) nb_max = 1;
    float* bs = (float*)malloc(sizeof(float) * (size_t)(R * nb_max));
    int64_t* nb_row = (int64_t*)malloc(sizeof(int64_t) * (size_t)R);
    for (int64_t r = 0; r < R; ++r) {
        const int64_t nv = n_valid[r];
        nb_row[r] = (nv + ORC_POOL_BLOCK - 1) / ORC_POOL_BLOCK;
        for (int64_t j = 0; j < nb_row[r]; ++j) {
            float m = scores[r * ld + j * ORC_POOL_BLOCK];
            for (int64_t t = 1; t < ORC_POOL_BLOCK && j * ORC_POOL_BLOCK + t < nv; ++t) {
                const float x = scores[r * ld + j * ORC_POOL_BLOCK + t];
                if (x > m) m = x;
            }
            bs[r * nb_max + j] = m;
        }
    }
    orc_topk(bs, R, nb_max, nb_max, nb_row, P, pool);
    free(nb_row);
    free(bs);
}

void orc_pool_topk(const float* scores, int64_t R, int64_t ld, const int64_t* n_valid,
                   const int32_t* pool, int P, int k, int32_t* idx) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < R; ++r) {
        sj_t* v = (sj_t*)malloc(sizeof(sj_t) * (size_t)P * ORC_POOL_BLOCK);
        int64_t n = 0;
        for (int p = 0; p < P; ++p) {
            const int32_t blk = pool[r * P + p];
            if (blk < 0) continue;
            for (int t = 0; t < ORC_POOL_BLOCK; ++t) {
                const int64_t j = (int64_t)blk * ORC_POOL_BLOCK + t;
                if (j >= n_valid[r]) continue;
                v[n].s = scores[r * ld + j];
                v[n].j = (int32_t)j;
                ++n;
            }
        }
        qsort(v, (size_t)n, sizeof(sj_t), cmp_score_desc_index_asc);
        const int64_t take = n < k ? n : k;
        int32_t* out = idx + r * k;
        for (int64_t t = 0; t < take; ++t) out[t] = v[t].j;
        qsort(out, (size_t)take, sizeof(int32_t), cmp_int_asc);
        for (int64_t t = take; t < k; ++t) out[t] = -1;
        free(v);
    }
}

/* ------------------------------------------------------------------------ */
/* Attention [P1 s3, s4], [P2 "Sharing the cache across layers"]: for query  */
/* row r = (b, i) and head h, one softmax over                              */
/*   z_j = scale * q.c_j   for the selected entries j (c_j dequantised, used */
/*                         as key and as value),                            */
/*   z_t = scale * q.Kw_t  for the window rows t of this query (value Vw_t), */
/* all in fp64; o = sum e^(z-m) val / sum e^(z-m), lse = m + ln sum.  An    */
/* empty set gives o = 0 and lse = -inf.                                     */
/* Layouts: q bf16 [B][Qs][Hq][D]; codes [B][N][D/2], scales [B][N][D/32];   */
/* idx [B*Qs][k] (-1 = none); wk, wv bf16 [B][Qs+W-1][D]; query i uses       */
/* window rows i .. i+W-1, of which only the last wlen[b] rows of the        */
/* buffer are valid (NULL: all).  out fp32 [B][Qs][Hq][D], lse [B][Qs][Hq].  */
/* ------------------------------------------------------------------------ */
void orc_attend(const uint16_t* q, int64_t B, int64_t Qs, int Hq, int D, const uint8_t* codes,
                const float* scales, int64_t N, const int32_t* idx, int k, const uint16_t* wk,
                const uint16_t* wv, int W, const int32_t* wlen, float sm_scale, float* out,
                float* lse) {
    const int64_t wrows = Qs + W - 1;
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t i = 0; i < Qs; ++i) {
            int64_t r = b * Qs + i;
            int64_t wfirst = wlen ? wrows - wlen[b] : 0;
            if (wfirst < i) wfirst = i;
            int64_t wend = i + W; /* exclusive */
            int64_t nwin = wend > wfirst ? wend - wfirst : 0;
            int64_t nkeys = k + nwin;
            double* key = (double*)malloc(sizeof(double) * (size_t)(nkeys * D + 1));
            double* val = (double*)malloc(sizeof(double) * (size_t)(nkeys * D + 1));
            int64_t n = 0;
            for (int t = 0; t < k; ++t) {
                int32_t j = idx[r * k + t];
                if (j < 0) continue;
                orc_fp4_dequant(codes + (b * N + j) * (D / 2), scales + (b * N + j) * (D / 32), 1, D,
                                key + n * D);
                memcpy(val + n * D, key + n * D, sizeof(double) * D);
                ++n;
            }
            for (int64_t t = wfirst; t < wend; ++t) {
                for (int dd = 0; dd < D; ++dd) {
                    key[n * D + dd] = bf16_value(wk[(b * wrows + t) * D + dd]);
                    val[n * D + dd] = bf16_value(wv[(b * wrows + t) * D + dd]);
                }
                ++n;
            }
            double* z = (double*)malloc(sizeof(double) * (size_t)(n + 1));
            for (int h = 0; h < Hq; ++h) {
                const uint16_t* qh = q + (r * Hq + h) * D;
                double m = -INFINITY;
                for (int64_t t = 0; t < n; ++t) {
                    double dot = 0.0;
                    for (int dd = 0; dd < D; ++dd) dot += bf16_value(qh[dd]) * key[t * D + dd];
                    z[t] = (double)sm_scale * dot;
                    if (z[t] > m) m = z[t];
                }
                float* o = out + (r * Hq + h) * D;
                if (n == 0) {
                    for (int dd = 0; dd < D; ++dd) o[dd] = 0.0f;
                    if (lse) lse[r * Hq + h] = -INFINITY;
                    continue;
                }
                double sum = 0.0;
                for (int64_t t = 0; t < n; ++t) sum += exp(z[t] - m);
                for (int dd = 0; dd < D; ++dd) {
                    double acc = 0.0;
                    for (int64_t t = 0; t < n; ++t) acc += exp(z[t] - m) * val[t * D + dd];
                    o[dd] = (float)(acc / sum);
                }
                if (lse) lse[r * Hq + h] = (float)(m + log(sum));
            }
            free(z);
            free(key);
            free(val);
        }
}

/* ------------------------------------------------------------------------ */
/* Layer modes [P2 "Sharing the cache across layers"], [P1 s5], [P3 s4]:     */
/*   Full    writes its own entries (the step's new rows) and makes its own  */
/*           selection;                                                     */
/*   Reindex shares the group's entries and makes a fresh selection with its */
/*           own index query;                                               */
/*   Reuse   shares the entries and the most recent selection of the group.  */
/* Every mode attends with its own queries and its own window.              */
/* ------------------------------------------------------------------------ */
typedef struct {
    int32_t B;
    int64_t N_cap;
    int32_t D, H_I, d_I, idx_dtype, k;
    uint8_t* codes;        /* [B][N_cap][D/2] */
    float* scales;         /* [B][N_cap][D/32] */
    void* ikeys;           /* [B][N_cap][H_I][d_I]; dtype 2: e2m1 codes [B][N_cap][K/2] */
    const int64_t* n_valid;/* [B], counts the step's new rows */
    int32_t* sel;          /* [B*Qs][k] */
    int32_t has_entries, has_selection, sel_qs;
    float* ikey_scales;    /* dtype 2: [B][N_cap][K/32] */
    int32_t pool_blocks;   /* 0: flat search; P > 0: hierarchical with a pool of P blocks */
    int32_t* pool;         /* [B*Qs][P] block indices kept by the latest Full */
    int32_t has_pool, pool_qs;
} orc_group;

typedef struct {
    int32_t Qs, Hq;
    const uint16_t* q;
    const void* iq;
    const uint16_t* wk;
    const uint16_t* wv;
    int32_t W;
    const int32_t* wlen;
    const float* new_entry; /* fp32 [B][Qs][D] */
    const void* new_ikey;   /* [B][Qs][H_I][d_I]; dtype 2: fp32, packed on write */
    float sm_scale;
    float* out;
    float* lse;
} orc_layer;

enum { ORC_FULL = 0, ORC_REINDEX = 1, ORC_REUSE = 2 };

static void select_rows(int mode, const orc_layer* L, orc_group* G) {
    const int64_t B = G->B, Qs = L->Qs, N = G->N_cap;
    int64_t* nv_row = (int64_t*)malloc(sizeof(int64_t) * (size_t)(B * Qs));
    int64_t nmax = 0;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t i = 0; i < Qs; ++i) {
            /* causal: row i of the chunk sees entries up to its own position */
            nv_row[b * Qs + i] = G->n_valid[b] - Qs + i + 1;
            if (nv_row[b * Qs + i] > nmax) nmax = nv_row[b * Qs + i];
        }
    float* s = (float*)malloc(sizeof(float) * (size_t)(B * Qs * N));
    orc_index_score(G->idx_dtype, L->iq, G->ikeys, G->ikey_scales, B, Qs, N, G->H_I, G->d_I, nv_row, s);
    if (mode == ORC_REINDEX && G->pool_blocks > 0)
        orc_pool_topk(s, B * Qs, N, nv_row, G->pool, G->pool_blocks, G->k, G->sel);
    else
        orc_topk(s, B * Qs, N, N, nv_row, G->k, G->sel);
    if (mode == ORC_FULL && G->pool_blocks > 0) {
        orc_pool_blocks(s, B * Qs, N, nv_row, G->pool_blocks, G->pool);
        G->has_pool = 1;
        G->pool_qs = L->Qs;
    }
    free(s);
    free(nv_row);
    G->has_selection = 1;
    G->sel_qs = L->Qs;
}

/* Returns 0 on success, 1 for invalid arguments, 4 for a group-state error. */
int orc_layer_step(int mode, const orc_layer* L, orc_group* G) {
    if (!L || !G || L->Qs < 1) return 1;
    const int64_t B = G->B, Qs = L->Qs, K = (int64_t)G->H_I * G->d_I;
    const size_t kb = G->idx_dtype == 0 ? 2 : 1;
    for (int64_t b = 0; b < B; ++b)
        if (G->n_valid[b] < Qs || G->n_valid[b] > G->N_cap) return 1;
    if (mode == ORC_FULL) {
        if (!L->new_entry || !L->new_ikey || !L->iq) return 1;
        for (int64_t b = 0; b < B; ++b)
            for (int64_t i = 0; i < Qs; ++i) {
                int64_t slot = G->n_valid[b] - Qs + i;
                orc_fp4_pack(L->new_entry + (b * Qs + i) * G->D, 1, G->D,
                             G->codes + (b * G->N_cap + slot) * (G->D / 2),
                             G->scales + (b * G->N_cap + slot) * (G->D / 32));
                if (G->idx_dtype == 2)
                    orc_fp4_pack((const float*)L->new_ikey + (b * Qs + i) * K, 1, (int)K,
                                 (uint8_t*)G->ikeys + (b * G->N_cap + slot) * (K / 2),
                                 G->ikey_scales + (b * G->N_cap + slot) * (K / 32));
                else
                    memcpy((char*)G->ikeys + (size_t)((b * G->N_cap + slot) * K) * kb,
                           (const char*)L->new_ikey + (size_t)((b * Qs + i) * K) * kb, (size_t)K * kb);
            }
        G->has_entries = 1;
        select_rows(ORC_FULL, L, G);
    } else if (mode == ORC_REINDEX) {
        if (!G->has_entries) return 4;
        if (G->pool_blocks > 0 && (!G->has_pool || G->pool_qs != L->Qs)) return 4;
        if (!L->iq) return 1;
        select_rows(ORC_REINDEX, L, G);
    } else if (mode == ORC_REUSE) {
        if (!G->has_selection || G->sel_qs != L->Qs) return 4;
    } else {
        return 1;
    }
    orc_attend(L->q, B, Qs, L->Hq, G->D, G->codes, G->scales, G->N_cap, G->sel, G->k, L->wk, L->wv,
               L->W, L->wlen, L->sm_scale, L->out, L->lse);
    return 0;
}

/* [P2 "Several mechanisms in one release"]: cache bytes = entries x numbers
   per entry x stored layer copies x bits per number / 8. */
int64_t orc_cache_bytes(int64_t entries, int64_t numbers, int64_t copies, int64_t bits) {
    return entries * numbers * copies * bits / 8;
}
