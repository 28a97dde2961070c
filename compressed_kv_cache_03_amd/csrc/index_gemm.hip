// S2+S3 for prefill chunks with e4m3 index keys: the query-by-key index score
// matrix on MFMA, fused with a per-row threshold filter, then an exact top-k.
//
// "Why Is DeepSeek V4.1 Flash So Fast?", section 4 (a cheap relevance search
// over every compressed position, then selection) and "Inference-Efficient
// LLMs", section 5 (at long context scoring every position dominates).  In a
// prefill chunk every query row scores every visible entry, so the scores form
// a dense Qs x N matrix: a GEMM with K = H*d = 128 or 256 e4m3 values, run on
// v_mfma_scale_f32_16x16x128_f8f6f4 with unit scales.  The full matrix (2 GiB
// at 4,096 x 131,072) is never stored.
//
// MFMA sums in fp32, so its scores s^ differ from the exact ones s (the exact
// sum rounded once to fp32); the selection must still equal the exact top-k
// with the lower index winning ties.  The steps:
//   1. sample: s^ against every stride-th entry (same GEMM, scores stored),
//      and per row a threshold theta whose rank among the samples puts about
//      twice k entries above it, with a four-sigma margin;
//   2. filter: the full causal GEMM appends (key, index) of every s^ >= theta
//      to the row's candidate list; keys keep 24 of 32 bits (rounded down);
//   3. final: per row, T^ = k-th largest candidate key.  With delta a proven
//      bound on |approximation - s| (Cauchy-Schwarz on the MFMA summation
//      error, twice the textbook bound, plus the key truncation), entries
//      above T^ + 2 delta are surely selected, entries below T^ - 2 delta
//      surely not, and the band between is rescored exactly (fp64 sums of
//      e4m3 products are exact) and resolved by (score desc, index asc).
//      The argument needs theta <= T^ - 2 delta and at least k candidates;
//   4. any row where a check fails (too few or too many candidates, theta too
//      high) is flagged and recomputed by an exact row kernel.
#include "common.h"
#include "launch.h"

namespace csa2 {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGThreads = 512;     // 8 waves
constexpr int kGQG = 1;            // 16-row query groups per wave
constexpr int kGRows = kGThreads / 64 * 16 * kGQG;  // query rows per workgroup (128)
constexpr int kGCols = 128;        // entries per staged tile
constexpr int kGSlots = 16;        // candidates per (row, lane group) list between flushes
constexpr int kGFlushTiles = 2;    // tiles per flush: 256 columns, 8-bit offsets
constexpr int kBandThreads = 1024;
constexpr int kBandCap = 8192;     // candidates the final kernel holds in LDS
constexpr int kBandMaxValid = 1 << 18;  // rows up to this many entries (LDS bitmap)
constexpr int kBandList = 2048;    // band entries resolved in LDS

CSA2_DEV f32x4 mfma_fp8(i32x8 a, i32x8 b, f32x4 c) {
    // e4m3 x e4m3 with E8M0 scales 127 = 2^0
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

CSA2_DEV i32x8 join(u32x4 lo, u32x4 hi) {
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// Inverse of sort_key.
CSA2_DEV float key_to_float(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

CSA2_DEV int64_t gemm_row_valid(const GemmArgs& a, int b, int64_t qrow) {
    if (qrow >= a.Qs) return 0;
    const int64_t v = a.nvb ? (int64_t)a.nvb[b] - a.Qs + qrow + 1 : a.N;
    return v < 0 ? 0 : (v > a.N ? a.N : v);
}

// MODE 0 stores every score s^[row][col] (col = sample index, entry col*stride);
// MODE 1 appends candidates s^ >= theta[row].  Workgroups map to tiles so that
// the workgroups an XCD runs together share one column block (and its keys in
// that XCD's L2): tile t = (w % 8) * per_xcd + w / 8, row block fastest.
//
// The MFMA computes S^T = K Q^T (A = 16 staged entries, B = 16 query rows held
// in registers), so lane (n, g) owns query row qg*16 + n of each of its row
// groups and entries 4g + i of each 16-entry group.  In MODE 1 a passing score
// goes to the lane's own LDS list for (row, g), with the count in a register:
// the float bits with the low 8 mantissa bits replaced by the column offset in
// the 256-column flush window (|change| < 2^-15 |s^|).  The flush adds one
// global atomic per row per window.  A list that overflows (far rarer than one
// row per call) marks its row for the exact recomputation.
template <int KB, int MODE>
__global__ __launch_bounds__(kGThreads) void gemm_fp8_kernel(GemmArgs a) {
    constexpr int RB = KB * 128;    // bytes per row
    constexpr int PITCH = RB + 16;  // staged entry pitch, bytes
    constexpr int LIST = kGSlots + 1;  // the last slot of a list takes overflow writes
    __shared__ __attribute__((aligned(16))) uint8_t btile[kGCols * PITCH];
    __shared__ uint32_t stage[MODE ? kGRows * 4 * LIST : 1];  // [row][g][slot]
    __shared__ uint32_t scnt[MODE ? kGRows * 4 : 1];          // [row][g] at a flush

    const int64_t w = blockIdx.x;
    const int64_t t = (w & 7) * a.per_xcd + (w >> 3);
    if (t >= a.tiles) return;
    const int rb = (int)(t % a.n_rowblk);
    const int64_t rest = t / a.n_rowblk;
    const int64_t cb = rest % a.n_colblk;
    const int b = (int)(rest / a.n_colblk);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int64_t row0 = (int64_t)rb * kGRows;
    const int64_t col0 = cb * a.nsub * kGCols;
    // entries visible to the last and to the first row of the block
    const int64_t nv_blk = gemm_row_valid(a, b, min(row0 + kGRows, (int64_t)a.Qs) - 1);
    const int64_t nv_first = gemm_row_valid(a, b, row0);
    if (col0 >= a.ncols || col0 * a.stride >= nv_blk) return;

    // query fragments: row wave*(16*kGQG) + qg*16 + n, bytes kb*128 + 32g .. +32
    i32x8 qf[kGQG][KB];
    int32_t nvr[kGQG];
    float th[kGQG];
    uint32_t cnt[kGQG];
#pragma unroll
    for (int qg = 0; qg < kGQG; ++qg) {
        const int64_t qrow = row0 + wave * 16 * kGQG + qg * 16 + n;
        const bool ok = qrow < a.Qs;
        const uint8_t* src = a.iq + ((int64_t)b * a.Qs + (ok ? qrow : 0)) * RB + 32 * g;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const u32x4 lo = *reinterpret_cast<const u32x4*>(src + kb * 128);
            const u32x4 hi = *reinterpret_cast<const u32x4*>(src + kb * 128 + 16);
            qf[qg][kb] = ok ? join(lo, hi) : i32x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
        nvr[qg] = (int32_t)gemm_row_valid(a, b, qrow);
        th[qg] = (MODE && ok) ? a.theta[(int64_t)b * a.Qs + qrow] : INFINITY;
        cnt[qg] = 0;
    }

    const int ntiles = MODE ? a.nsub : 1;
    // key tiles are prefetched one tile ahead into registers: two threads per
    // entry, out-of-range entries load entry 0 (masked in the epilogue)
    constexpr int TPE = kGThreads / kGCols;  // threads per staged entry
    constexpr int BPT = RB / TPE;            // bytes per thread
    u32x4 pf[BPT / 16];
    auto load_tile = [&](int64_t tc) {
        const int64_t col = tc + tid / TPE;
        int64_t j = col * a.stride;
        if (col >= a.ncols || j >= a.N) j = 0;
        const uint8_t* src = a.ik + ((int64_t)b * a.N_cap + j) * RB + (tid % TPE) * BPT;
#pragma unroll
        for (int q = 0; q < BPT / 16; ++q) pf[q] = *reinterpret_cast<const u32x4*>(src + 16 * q);
    };
    load_tile(col0);
    for (int sub = 0; sub < ntiles; ++sub) {
        const int64_t tc0 = col0 + (int64_t)sub * kGCols;  // first column of the tile
        if (tc0 >= a.ncols || tc0 * a.stride >= nv_blk) break;  // workgroup-uniform
        __syncthreads();  // previous tile consumed (and staging flushed)
        {
            uint8_t* dst = btile + (tid / TPE) * PITCH + (tid % TPE) * BPT;
#pragma unroll
            for (int q = 0; q < BPT / 16; ++q) *reinterpret_cast<u32x4*>(dst + 16 * q) = pf[q];
        }
        if (sub + 1 < ntiles) load_tile(tc0 + kGCols);
        __syncthreads();
        // the window of the current flush starts at column fc0
        const int64_t fc0 = col0 + (int64_t)(sub - sub % kGFlushTiles) * kGCols;
        // every column of the tile visible to every row of the block: no per-score test
        const bool all_visible = (tc0 + kGCols) <= a.ncols && (tc0 + kGCols - 1) * a.stride < nv_first;
        if (MODE == 1 && all_visible) {
#pragma unroll 2
            for (int eg = 0; eg < kGCols / 16; ++eg) {
                i32x8 kf[KB];
                const uint8_t* ks = btile + (eg * 16 + n) * PITCH + 32 * g;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
                    kf[kb] = join(*reinterpret_cast<const u32x4*>(ks + kb * 128),
                                  *reinterpret_cast<const u32x4*>(ks + kb * 128 + 16));
                const uint32_t off = (uint32_t)(tc0 - fc0) + eg * 16 + 4 * g;  // column offset in the window
#pragma unroll
                for (int qg = 0; qg < kGQG; ++qg) {
                    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) acc = mfma_fp8(kf[kb], qf[qg][kb], acc);
                    uint32_t* list = stage + ((wave * 16 * kGQG + qg * 16 + n) * 4 + g) * LIST;
                    // branch-free: a score that does not pass is written to the trash slot
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const bool p = acc[i] >= th[qg];
                        list[p ? min(cnt[qg], (uint32_t)kGSlots) : (uint32_t)kGSlots] =
                            (__float_as_uint(acc[i]) & 0xffffff00u) | (off + i);
                        cnt[qg] += p ? 1u : 0u;
                    }
                }
            }
        } else {
#pragma unroll 1
            for (int eg = 0; eg < kGCols / 16; ++eg) {
                i32x8 kf[KB];
                const uint8_t* ks = btile + (eg * 16 + n) * PITCH + 32 * g;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
                    kf[kb] = join(*reinterpret_cast<const u32x4*>(ks + kb * 128),
                                  *reinterpret_cast<const u32x4*>(ks + kb * 128 + 16));
                const int64_t cbase = tc0 + eg * 16 + 4 * g;  // this lane's first column
#pragma unroll
                for (int qg = 0; qg < kGQG; ++qg) {
                    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) acc = mfma_fp8(kf[kb], qf[qg][kb], acc);
                    const int lr = wave * 16 * kGQG + qg * 16 + n;
                    uint32_t* list = stage + (lr * 4 + g) * LIST;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int64_t col = cbase + i;
                        const bool valid = col < a.ncols && col * a.stride < nvr[qg];
                        if (MODE == 0) {
                            const int64_t qr = row0 + lr;
                            if (col < a.ncols && qr < a.Qs)
                                a.out[((int64_t)b * a.Qs + qr) * a.ncols + col] = valid ? acc[i] : -INFINITY;
                        } else if (valid && acc[i] >= th[qg]) {
                            list[min(cnt[qg], (uint32_t)kGSlots)] =
                                (__float_as_uint(acc[i]) & 0xffffff00u) | (uint32_t)(col - fc0);
                            ++cnt[qg];
                        }
                    }
                }
            }
        }
        if (MODE) {
            const bool last = sub + 1 == ntiles || tc0 + kGCols >= a.ncols ||
                              (tc0 + kGCols) * a.stride >= nv_blk;
            if (last || sub % kGFlushTiles == kGFlushTiles - 1) {
#pragma unroll
                for (int qg = 0; qg < kGQG; ++qg) {
                    scnt[(wave * 16 * kGQG + qg * 16 + n) * 4 + g] = cnt[qg];
                    cnt[qg] = 0;
                }
                __syncthreads();
                if (tid < kGRows) {
                    const int64_t qr = row0 + tid;
                    uint32_t c4[4], tot = 0;
                    bool over = false;
#pragma unroll
                    for (int gg = 0; gg < 4; ++gg) {
                        c4[gg] = scnt[tid * 4 + gg];
                        over |= c4[gg] > (uint32_t)kGSlots;
                        tot += c4[gg];
                    }
                    if (qr < a.Qs && tot > 0) {
                        const int64_t r = (int64_t)b * a.Qs + qr;
                        if (over) {
                            // candidates were lost: push the count past the list length so
                            // that the final kernel recomputes the row exactly
                            atomicAdd(&a.cand_cnt[r], (uint32_t)a.cap + 1u);
                        } else {
                            uint32_t pos = atomicAdd(&a.cand_cnt[r], tot);
#pragma unroll
                            for (int gg = 0; gg < 4; ++gg)
                                for (uint32_t sl = 0; sl < c4[gg] && pos < (uint32_t)a.cap; ++sl, ++pos) {
                                    const uint32_t v = stage[(tid * 4 + gg) * LIST + sl];
                                    a.cand[r * a.cap + pos] = make_uint2(v, (uint32_t)(fc0 + (v & 0xffu)));
                                }
                        }
                    }
                }
            }
        }
    }
}

hipError_t launch_gemm_fp8(GemmArgs a, int mode, hipStream_t stream) {
    if (a.Qs == 0 || a.B == 0 || a.ncols == 0) return hipSuccess;
    a.n_rowblk = (int)((a.Qs + kGRows - 1) / kGRows);
    const int64_t cols_per_wg = (int64_t)a.nsub * kGCols;
    a.n_colblk = (a.ncols + cols_per_wg - 1) / cols_per_wg;
    a.tiles = (int64_t)a.B * a.n_colblk * a.n_rowblk;
    a.per_xcd = (a.tiles + 7) / 8;
    const dim3 grid((unsigned)(8 * a.per_xcd));
    if (a.K == 128) {
        if (mode == 0) hipLaunchKernelGGL((gemm_fp8_kernel<1, 0>), grid, dim3(kGThreads), 0, stream, a);
        else hipLaunchKernelGGL((gemm_fp8_kernel<1, 1>), grid, dim3(kGThreads), 0, stream, a);
    } else if (a.K == 256) {
        if (mode == 0) hipLaunchKernelGGL((gemm_fp8_kernel<2, 0>), grid, dim3(kGThreads), 0, stream, a);
        else hipLaunchKernelGGL((gemm_fp8_kernel<2, 1>), grid, dim3(kGThreads), 0, stream, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Radix select: the `need`-th largest key T among the positions p < C for
// which key_at(p, &k) returns true, and the count of such keys strictly above
// T.  Four 8-bit digits; block-wide; `hist` holds 256 words.  need >= 1 and at
// least `need` participating keys are required.
template <int THREADS, typename KeyAt>
CSA2_DEV void block_radix_select(uint32_t C, uint32_t need, KeyAt key_at, uint32_t* hist,
                                 uint32_t* scan_lds, uint32_t* dig, uint32_t* T_out,
                                 uint32_t* above_out) {
    uint32_t prefix = 0, fixed = 0, above = 0;
#pragma unroll
    for (int sh = 24; sh >= 0; sh -= 8) {
        for (int i = threadIdx.x; i < 256; i += THREADS) hist[i] = 0;
        __syncthreads();
        for (uint32_t p = threadIdx.x; p < C; p += THREADS) {
            uint32_t k;
            if (key_at(p, &k) && (k & fixed) == prefix) atomicAdd(&hist[(k >> sh) & 0xffu], 1u);
        }
        __syncthreads();
        find_digit<THREADS>(hist, 256, need, scan_lds, dig);
        prefix |= dig[0] << sh;
        fixed |= 0xffu << sh;
        need -= dig[1];
        above += dig[1];
        __syncthreads();
    }
    *T_out = prefix;
    *above_out = above;
}

// Per row: zero the candidate counter and pick theta (see the top of the file).
constexpr int kSampleMax = 2048;
__global__ __launch_bounds__(256) void sample_select_kernel(BandArgs a) {
    __shared__ uint32_t keys[kSampleMax];
    __shared__ uint32_t hist[256];
    __shared__ uint32_t scan_lds[256 / 64 + 1];
    __shared__ uint32_t dig[2];
    const int64_t r = blockIdx.x;
    const int b = (int)(r / a.Qs);
    const int64_t qrow = r % a.Qs;
    if (threadIdx.x == 0) {
        a.cand_cnt[r] = 0;
        a.flag[r] = 0;
        if (r == 0) *a.flag_count = 0;
    }
    int64_t nv = a.nvb ? (int64_t)a.nvb[b] - a.Qs + qrow + 1 : a.N;
    nv = nv < 0 ? 0 : (nv > a.N ? a.N : nv);
    const int64_t keff = nv < a.k ? nv : a.k;
    if (keff == 0) {
        if (threadIdx.x == 0) a.theta[r] = INFINITY;
        return;
    }
    const int64_t ns = min((nv + a.stride - 1) / a.stride, a.ncols);  // valid samples (<= 2048)
    const double kp = (double)keff * (double)ns / (double)nv;
    const int64_t rank = (int64_t)ceil(kp + 4.0 * sqrt(kp) + 8.0);
    if (rank > ns) {
        if (threadIdx.x == 0) a.theta[r] = -INFINITY;
        return;
    }
    const float* sv = a.samp + r * a.ncols;
    for (int p = threadIdx.x; p < ns; p += 256) keys[p] = sort_key(sv[p]);
    __syncthreads();
    uint32_t T, above;
    block_radix_select<256>((uint32_t)ns, (uint32_t)rank,
                            [&](uint32_t p, uint32_t* k) { *k = keys[p]; return true; }, hist, scan_lds,
                            dig, &T, &above);
    if (threadIdx.x == 0) a.theta[r] = key_to_float(T);
}

// Per block of 256 entries of a sequence: an upper bound on max_j sum_e ik[j][e]^2
// (e4m3 squares are exact in fp32; the fp32 sum is inflated by its rounding bound).
template <int KB>
__global__ __launch_bounds__(256) void key_norm_kernel(const uint8_t* __restrict__ ik, int64_t N,
                                                        int64_t N_cap, int nblk, float* out) {
    constexpr int RB = KB * 128;
    __shared__ float red[4];
    const int b = blockIdx.y;
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    float s = 0.0f;
    if (j < N) {
        const u32x4* src = reinterpret_cast<const u32x4*>(ik + ((int64_t)b * N_cap + j) * RB);
#pragma unroll
        for (int q = 0; q < RB / 16; ++q) {
            const u32x4 w = src[q];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const auto p0 = __builtin_amdgcn_cvt_pk_f32_fp8(w[u], false);
                const auto p1 = __builtin_amdgcn_cvt_pk_f32_fp8(w[u], true);
                s = fmaf(p0[0], p0[0], s);
                s = fmaf(p0[1], p0[1], s);
                s = fmaf(p1[0], p1[0], s);
                s = fmaf(p1[1], p1[1], s);
            }
        }
        s *= 1.0f + 0x1p-14f;  // >= the exact sum: K <= 256 additions, each within 2^-24
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) s = fmaxf(s, __shfl_xor(s, o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) out[(int64_t)b * nblk + blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Exact fp32 index score of (query row r, entry j): e4m3 products are exact in
// fp64 and so are all partial sums (multiples of 2^-18 below 2^30), so the fp64
// wave sum rounded once is the defined score.  Whole wave; result in every lane.
template <int KB>
CSA2_DEV float exact_score_fp8(const uint8_t* q, const uint8_t* k) {
    constexpr int RB = KB * 128;
    constexpr int PER = RB / 64;  // bytes per lane: 2 or 4
    const int lane = threadIdx.x & 63;
    uint32_t qw, kw;
    if constexpr (PER == 4) {
        qw = reinterpret_cast<const uint32_t*>(q)[lane];
        kw = reinterpret_cast<const uint32_t*>(k)[lane];
    } else {
        qw = reinterpret_cast<const uint16_t*>(q)[lane];
        kw = reinterpret_cast<const uint16_t*>(k)[lane];
    }
    double acc = 0.0;
#pragma unroll
    for (int e = 0; e < PER; ++e)
        acc = fma(e4m3_to_f64((qw >> (8 * e)) & 0xffu), e4m3_to_f64((kw >> (8 * e)) & 0xffu), acc);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
    const float f = (float)acc;
    return f == 0.0f ? 0.0f : f;
}

// Per row: exact selection from the candidate list, or a fallback flag.
// Candidates arrive as (float bits of s^ with the low 8 bits replaced, entry).
template <int KB>
__global__ __launch_bounds__(kBandThreads) void band_final_kernel(BandArgs a) {
    constexpr int RB = KB * 128;
    __shared__ uint32_t s_key[kBandCap];   // sort keys minus the smallest; later the output bitmap
    __shared__ int32_t s_idx[kBandCap];    // entry index; bit 31 = selected
    __shared__ uint32_t band[kBandList];   // positions of band entries
    __shared__ uint32_t bkey[kBandList];   // their exact sort keys
    __shared__ int32_t bidx[kBandList];    // and entries
    __shared__ uint32_t hist[kHistBins];
    __shared__ uint32_t scan_lds[kBandThreads / 64 + 1];
    __shared__ uint32_t dig[2];
    __shared__ uint32_t red_u[kBandThreads / 64];
    __shared__ double red_q[kBandThreads / 64];
    __shared__ float red_k[kBandThreads / 64];
    static_assert(kBandCap * 4 >= kBandMaxValid / 8, "the output bitmap overlays s_key");

    const int64_t r = blockIdx.x;
    const int b = (int)(r / a.Qs);
    const int64_t qrow = r % a.Qs;
    int64_t nv = a.nvb ? (int64_t)a.nvb[b] - a.Qs + qrow + 1 : a.N;
    nv = nv < 0 ? 0 : (nv > a.N ? a.N : nv);
    const int64_t keff = nv < a.k ? nv : a.k;
    int32_t* out = a.idx + r * a.k;
    for (int64_t t = keff + threadIdx.x; t < a.k; t += kBandThreads) out[t] = -1;
    if (keff == 0) return;

    const uint32_t C = a.cand_cnt[r];
    auto flag_row = [&]() {  // the exact row kernel recomputes this row
        if (threadIdx.x == 0) {
            a.flag[r] = 1;
            atomicAdd(a.flag_count, 1u);
        }
    };
    if (C < (uint32_t)keff || C > (uint32_t)a.cap || C > (uint32_t)kBandCap || nv > kBandMaxValid) {
        flag_row();
        return;
    }
    // keys relative to the smallest candidate key: they span few bits
    const uint2* cand = a.cand + r * a.cap;
    uint32_t kmin = 0xffffffffu, kmax = 0;
    for (uint32_t p = threadIdx.x; p < C; p += kBandThreads) {
        const uint2 c = cand[p];
        const uint32_t k = sort_key(__uint_as_float(c.x & 0xffffff00u));
        s_key[p] = k;
        s_idx[p] = (int32_t)c.y;
        kmin = min(kmin, k);
        kmax = max(kmax, k);
    }
    // ||q||^2 (exact in fp64) and the sequence's bound on max ||k||^2
    double q2 = 0.0;
    {
        const uint8_t* q = a.iq + r * RB;
        for (int e = threadIdx.x; e < RB; e += kBandThreads) {
            const double v = e4m3_to_f64(q[e]);
            q2 = fma(v, v, q2);
        }
    }
    float k2 = 0.0f;
    for (int i = threadIdx.x; i < a.nblk; i += kBandThreads) k2 = fmaxf(k2, a.knorm[(int64_t)b * a.nblk + i]);
    for (int o = 32; o >= 1; o >>= 1) {
        q2 += __shfl_xor(q2, o);
        k2 = fmaxf(k2, __shfl_xor(k2, o));
        kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
        kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
    }
    if ((threadIdx.x & 63) == 0) {
        red_q[threadIdx.x >> 6] = q2;
        red_k[threadIdx.x >> 6] = k2;
        red_u[threadIdx.x >> 6] = kmin;
        scan_lds[threadIdx.x >> 6] = kmax;
    }
    __syncthreads();
    double Q2 = 0.0;
    float K2 = 0.0f;
    uint32_t K0 = 0xffffffffu, K1 = 0;
    for (int wv = 0; wv < kBandThreads / 64; ++wv) {
        Q2 += red_q[wv];
        K2 = fmaxf(K2, red_k[wv]);
        K0 = min(K0, red_u[wv]);
        K1 = max(K1, scan_lds[wv]);
    }
    __syncthreads();
    for (uint32_t p = threadIdx.x; p < C; p += kBandThreads) s_key[p] -= K0;

    // T^: the keff-th largest key.  12-bit digits from the top of the used range;
    // once the digit's bin holds few keys, they are ranked directly.
    const int bits = 32 - __clz((int)(K1 - K0) | 1);
    uint32_t prefix = 0, fixed = 0, need = (uint32_t)keff;
    for (int sh = bits > 12 ? bits - 12 : 0;; sh = sh > 12 ? sh - 12 : 0) {
        for (int i = threadIdx.x; i < kHistBins; i += kBandThreads) hist[i] = 0;
        __syncthreads();
        for (uint32_t p = threadIdx.x; p < C; p += kBandThreads) {
            const uint32_t k = s_key[p];
            if ((k & fixed) == prefix) atomicAdd(&hist[(k >> sh) & 0xfffu], 1u);
        }
        __syncthreads();
        find_digit<kBandThreads>(hist, kHistBins, need, scan_lds, dig);
        const uint32_t inbin = hist[dig[0]];
        prefix |= dig[0] << sh;
        fixed |= 0xfffu << sh;
        need -= dig[1];
        if (sh == 0) break;
        if (inbin <= (uint32_t)kBandList) {
            // gather the bin's keys and find the need-th largest by counting
            if (threadIdx.x == 0) dig[0] = 0;
            __syncthreads();
            for (uint32_t p = threadIdx.x; p < C; p += kBandThreads) {
                const uint32_t k = s_key[p];
                if ((k & fixed) == prefix) bkey[atomicAdd(&dig[0], 1u)] = k;
            }
            __syncthreads();
            for (uint32_t t = threadIdx.x; t < inbin; t += kBandThreads) {
                const uint32_t kt = bkey[t];
                uint32_t gt = 0, ge = 0;
                for (uint32_t u = 0; u < inbin; ++u) {
                    gt += bkey[u] > kt ? 1u : 0u;
                    ge += bkey[u] >= kt ? 1u : 0u;
                }
                if (gt < need && need <= ge) dig[1] = kt;  // every writer writes the same key
            }
            __syncthreads();
            prefix = dig[1];
            break;
        }
    }
    const double That = key_to_float(prefix + K0);
    // |approximation - s| <= delta: MFMA fp32 summation of K exact products with
    // unit roundoff 2^-23 per addition (covers truncation), doubled, by
    // Cauchy-Schwarz sum|p| <= ||q|| ||k||; plus the 2^-15 relative key truncation
    // and the final rounding of s, plus an absolute term for subnormal flushing.
    const double Kd = (double)(RB - 1);
    const double gam = Kd * 0x1p-23 / (1.0 - Kd * 0x1p-23);
    const double E = 2.0 * gam * sqrt(Q2 * (double)K2) * (1.0 + 0x1p-20) + 0x1p-100;
    const double delta = E + 0x1p-14 * (fabs(That) + E);
    const double lo = That - 2.0 * delta, hi = That + 2.0 * delta;
    if (!(a.theta[r] <= lo)) {
        flag_row();
        return;
    }
    // classify: above the band -> selected (bit 31); inside -> band list (block-scan compaction)
    uint32_t nin_mine = 0;
    {
        uint32_t inb[kBandCap / kBandThreads];
        uint32_t nb_mine = 0;
#pragma unroll
        for (int u = 0; u < kBandCap / kBandThreads; ++u) {
            const uint32_t p = threadIdx.x * (kBandCap / kBandThreads) + u;  // contiguous per thread
            inb[u] = 0;
            if (p < C) {
                const double v = key_to_float(s_key[p] + K0);
                if (v > hi) {
                    ++nin_mine;
                    s_idx[p] |= (int32_t)0x80000000;
                } else if (v >= lo) {
                    inb[u] = 1;
                    ++nb_mine;
                }
            }
        }
        uint32_t nband_tot;
        uint32_t pos = block_exclusive_scan(nb_mine, scan_lds, &nband_tot);
#pragma unroll
        for (int u = 0; u < kBandCap / kBandThreads; ++u)
            if (inb[u]) {
                if (pos < (uint32_t)kBandList) band[pos] = threadIdx.x * (kBandCap / kBandThreads) + u;
                ++pos;
            }
        if (threadIdx.x == 0) dig[0] = nband_tot;
    }
    uint32_t nin;
    block_exclusive_scan(nin_mine, scan_lds, &nin);
    const uint32_t nband = dig[0];
    if (nband > (uint32_t)kBandList || nin > (uint32_t)keff || (uint32_t)keff - nin > nband) {
        flag_row();  // a very wide band, or the error bound did not hold
        return;
    }
    const uint32_t need_b = (uint32_t)keff - nin;
    if (need_b > 0) {
        // exact rescoring of the band, one wave per entry
        const uint8_t* q = a.iq + r * RB;
        for (uint32_t t = threadIdx.x >> 6; t < nband; t += kBandThreads / 64) {
            const int32_t j = s_idx[band[t]];
            const float sc = exact_score_fp8<KB>(q, a.ik + ((int64_t)b * a.N_cap + j) * RB);
            if ((threadIdx.x & 63) == 0) {
                bkey[t] = sort_key(sc);
                bidx[t] = j;
            }
        }
        __syncthreads();
        // rank in the band by (exact score desc, index asc); the first need_b are taken
        for (uint32_t t = threadIdx.x; t < nband; t += kBandThreads) {
            const uint32_t kt = bkey[t];
            const int32_t jt = bidx[t];
            uint32_t rank = 0;
            for (uint32_t v = 0; v < nband; ++v) {
                const uint32_t kv = bkey[v];
                rank += (kv > kt || (kv == kt && bidx[v] < jt)) ? 1u : 0u;
            }
            if (rank < need_b) s_idx[band[t]] = jt | (int32_t)0x80000000;
        }
    }
    __syncthreads();
    // ascending output from a bitmap of the selected entries (over s_key)
    uint32_t* bitmap = s_key;
    const int nwords = (int)((nv + 31) / 32);
    for (int i = threadIdx.x; i < nwords; i += kBandThreads) bitmap[i] = 0;
    __syncthreads();
    for (uint32_t p = threadIdx.x; p < C; p += kBandThreads) {
        const int32_t v = s_idx[p];
        if (v < 0) {
            const int32_t j = v & 0x7fffffff;
            atomicOr(&bitmap[j >> 5], 1u << (j & 31));
        }
    }
    __syncthreads();
    const int per = (nwords + kBandThreads - 1) / kBandThreads;
    uint32_t mine = 0;
    for (int wi = threadIdx.x * per; wi < min(nwords, (int)(threadIdx.x + 1) * per); ++wi) mine += __popc(bitmap[wi]);
    uint32_t total;
    uint32_t pos = block_exclusive_scan(mine, scan_lds, &total);
    if (total != (uint32_t)keff) {  // cannot happen when the bound holds
        flag_row();
        return;
    }
    for (int wi = threadIdx.x * per; wi < min(nwords, (int)(threadIdx.x + 1) * per); ++wi) {
        uint32_t word = bitmap[wi];
        while (word) {
            const int bit = __ffs(word) - 1;
            word &= word - 1;
            out[pos++] = wi * 32 + bit;
        }
    }
}

// Exact top-k of one flagged row, from scratch: exact scores of all visible
// entries into the workspace, then the radix select and an ordered pass.
template <int KB>
__global__ __launch_bounds__(kBandThreads) void band_fallback_kernel(BandArgs a) {
    constexpr int RB = KB * 128;
    __shared__ uint32_t hist[kHistBins];
    __shared__ uint32_t scan_lds[kBandThreads / 64 + 1];
    __shared__ uint32_t dig[2];
    const int64_t r = blockIdx.x;
    if (a.flag[r] == 0) return;
    const int b = (int)(r / a.Qs);
    const int64_t qrow = r % a.Qs;
    int64_t nv = a.nvb ? (int64_t)a.nvb[b] - a.Qs + qrow + 1 : a.N;
    nv = nv < 0 ? 0 : (nv > a.N ? a.N : nv);
    const int64_t keff = nv < a.k ? nv : a.k;
    float* sc = a.scores + r * a.ld;
    const uint8_t* q = a.iq + r * RB;
    for (int64_t j = threadIdx.x >> 6; j < nv; j += kBandThreads / 64) {
        const float s = exact_score_fp8<KB>(q, a.ik + ((int64_t)b * a.N_cap + j) * RB);
        if ((threadIdx.x & 63) == 0) sc[j] = s;
    }
    __syncthreads();
    __threadfence_block();
    uint32_t T, above;
    // the keys live in global memory; each pass reads them again
    block_radix_select<kBandThreads>((uint32_t)nv, (uint32_t)keff,
                                     [&](uint32_t p, uint32_t* k) { *k = sort_key(sc[p]); return true; },
                                     hist, scan_lds, dig, &T, &above);
    const uint32_t quota = (uint32_t)keff - above;
    int32_t* out = a.idx + r * a.k;
    uint32_t ties_before = 0, written = 0;
    for (int64_t p0 = 0; p0 < nv; p0 += kBandThreads) {
        const int64_t p = p0 + threadIdx.x;
        const uint32_t key = p < nv ? sort_key(sc[p]) : 0u;
        const uint32_t tie = (p < nv && key == T) ? 1u : 0u;
        uint32_t ntie;
        const uint32_t tie_rank = ties_before + block_exclusive_scan(tie, scan_lds, &ntie);
        const uint32_t sel = (p < nv && (key > T || (tie && tie_rank < quota))) ? 1u : 0u;
        uint32_t nsel;
        const uint32_t pos = written + block_exclusive_scan(sel, scan_lds, &nsel);
        if (sel && pos < (uint32_t)keff) out[pos] = (int32_t)p;
        ties_before += ntie;
        written += nsel;
    }
}

hipError_t launch_sample_select(const BandArgs& a, hipStream_t stream) {
    const int64_t R = (int64_t)a.B * a.Qs;
    if (R == 0) return hipSuccess;
    hipLaunchKernelGGL(sample_select_kernel, dim3((unsigned)R), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_key_norm(const uint8_t* ik, int K, int B, int64_t N, int64_t N_cap, int nblk, float* out,
                           hipStream_t stream) {
    if (B == 0 || N == 0) return hipSuccess;
    const dim3 grid((unsigned)nblk, (unsigned)B);
    if (K == 128) hipLaunchKernelGGL(key_norm_kernel<1>, grid, dim3(256), 0, stream, ik, N, N_cap, nblk, out);
    else if (K == 256) hipLaunchKernelGGL(key_norm_kernel<2>, grid, dim3(256), 0, stream, ik, N, N_cap, nblk, out);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_band_final(const BandArgs& a, hipStream_t stream) {
    const int64_t R = (int64_t)a.B * a.Qs;
    if (R == 0) return hipSuccess;
    if (a.K == 128) {
        hipLaunchKernelGGL(band_final_kernel<1>, dim3((unsigned)R), dim3(kBandThreads), 0, stream, a);
        hipLaunchKernelGGL(band_fallback_kernel<1>, dim3((unsigned)R), dim3(kBandThreads), 0, stream, a);
    } else if (a.K == 256) {
        hipLaunchKernelGGL(band_final_kernel<2>, dim3((unsigned)R), dim3(kBandThreads), 0, stream, a);
        hipLaunchKernelGGL(band_fallback_kernel<2>, dim3((unsigned)R), dim3(kBandThreads), 0, stream, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

int band_cap(int k) { return 3 * k + 2048 < kBandCap ? 3 * k + 2048 : kBandCap; }
int band_max_k() { return (kBandCap - 2048) / 3; }

}  // namespace csa2
