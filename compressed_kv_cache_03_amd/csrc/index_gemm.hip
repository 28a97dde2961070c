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
//      bound on |approximation - s| (the MFMA's truncation of each product in
//      its group of 8 to 13 bits below the group's largest exponent pair,
//      measured on gfx950; Cauchy-Schwarz on the fp32 summation of the group
//      sums, twice the textbook bound; plus the key truncation), entries
//      above T^ + 2 delta are surely selected, entries below T^ - 2 delta
//      surely not, and the band between is rescored exactly (fp64 sums of
//      e4m3 products are exact) and resolved by (score desc, index asc).
//      The argument needs theta <= T^ - 2 delta and at least k candidates;
//   4. any row where a check fails (too few or too many candidates, theta too
//      high) is flagged and recomputed by an exact row kernel.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace csa2 {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGCols = 128;         // entries per staged key tile
// sample GEMM: 8 waves of 16 query rows, one key tile per workgroup
constexpr int kSThreads = 512;
constexpr int kSRows = kSThreads / 64 * 16;
// filter GEMM: 4 waves of 64 query rows, 8 key tiles (a 1024-entry column block)
constexpr int kFWaves = 4;
constexpr int kFThreads = kFWaves * 64;
constexpr int kFQG = 4;                          // 16-row query groups per wave
constexpr int kFRows = kFWaves * 16 * kFQG;      // 256 query rows per workgroup
constexpr int kFSub = 8;
constexpr int kFBlkCols = kFSub * kGCols;        // 1024
constexpr int kFList = 640;                      // quads in a wave's staging list
constexpr int kFBlkCap = 64;                     // candidates per (row, column block) region
static_assert(kFThreads == kFRows, "one thread per query row of the workgroup");
static_assert(kFBlkCols / 16 <= 256 && kFQG * 64 <= 256, "tags fit 8 bits");
constexpr int kBandThreads = 1024;
constexpr int kBandCap = 8192;     // candidates the final kernel holds in LDS
constexpr int kBandOutChunk = 1 << 18;  // entries per pass of the output bitmap (over s_key)
constexpr int kBandRegBatch = 512;      // column-block regions gathered per batch
constexpr int kBandList = 1024;    // band entries resolved in LDS
constexpr int kBandBits = 11;      // radix digit of the final selection
constexpr int kBandHist = 1 << kBandBits;

CSA2_DEV f32x4 mfma_fp8(i32x8 a, i32x8 b, f32x4 c) {
    // e4m3 x e4m3 with E8M0 scales 127 = 2^0
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// The compiler treats the scaled MFMA as an ordinary operation and may sink it
// into a branch that uses its result, where it would run with part of the wave
// masked off: the masked lanes' operand fragments then drop out of every lane's
// product.  An empty asm that takes the accumulators keeps the MFMAs ahead of
// any such branch, at full EXEC.
CSA2_DEV void pin(f32x4& acc) { __asm__ volatile("" : "+v"(acc)); }

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

// Workgroup w takes tile t = (w % 8) * per_xcd + w / 8 (row block fastest), so
// the workgroups one XCD runs together share a column block and its keys in
// that XCD's L2.
struct GemmTile {
    int rb, b;
    int64_t cb;
    bool ok;
};
CSA2_DEV GemmTile gemm_tile(const GemmArgs& a) {
    const int64_t w = blockIdx.x;
    const int64_t t = (w & 7) * a.per_xcd + (w >> 3);
    GemmTile r;
    r.ok = t < a.tiles;
    r.rb = (int)(t % a.n_rowblk);
    const int64_t rest = t / a.n_rowblk;
    r.cb = rest % a.n_colblk;
    r.b = (int)(rest / a.n_colblk);
    return r;
}

// Sample scores: out[row][col] = s^(row, entry col*stride), -inf where the
// entry is not visible to the row.  The MFMA computes S^T = K Q^T (A = 16
// staged entries, B = 16 query rows in registers): lane (n, g) holds query
// row n of its wave and entries 4g + i of each 16-entry group.
template <int KB>
__global__ __launch_bounds__(kSThreads) void sample_gemm_kernel(GemmArgs a) {
    constexpr int RB = KB * 128;    // bytes per row
    constexpr int PITCH = RB + 16;  // staged entry pitch, bytes
    __shared__ __attribute__((aligned(16))) uint8_t btile[kGCols * PITCH];
    const GemmTile tl = gemm_tile(a);
    if (!tl.ok) return;
    const int b = tl.b;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int64_t row0 = (int64_t)tl.rb * kSRows;
    const int64_t col0 = tl.cb * kGCols;
    const int64_t nv_blk = gemm_row_valid(a, b, min(row0 + kSRows, (int64_t)a.Qs) - 1);
    if (col0 >= a.ncols || col0 * a.stride >= nv_blk) return;

    const int64_t qrow = row0 + wave * 16 + n;
    const bool qok = qrow < a.Qs;
    i32x8 qf[KB];
    {
        const uint8_t* src = a.iq + ((int64_t)b * a.Qs + (qok ? qrow : 0)) * RB + 32 * g;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const u32x4 lo = *reinterpret_cast<const u32x4*>(src + kb * 128);
            const u32x4 hi = *reinterpret_cast<const u32x4*>(src + kb * 128 + 16);
            qf[kb] = qok ? join(lo, hi) : i32x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
    }
    const int64_t nvr = gemm_row_valid(a, b, qrow);
    {
        constexpr int TPE = kSThreads / kGCols;  // threads per staged entry
        constexpr int BPT = RB / TPE;            // bytes per thread
        const int64_t col = col0 + tid / TPE;
        int64_t j = col * a.stride;
        if (col >= a.ncols || j >= a.N) j = 0;  // masked below
        const uint8_t* src = a.ik + ((int64_t)b * a.N_cap + j) * RB + (tid % TPE) * BPT;
        uint8_t* dst = btile + (tid / TPE) * PITCH + (tid % TPE) * BPT;
#pragma unroll
        for (int q = 0; q < BPT / 16; ++q)
            *reinterpret_cast<u32x4*>(dst + 16 * q) = *reinterpret_cast<const u32x4*>(src + 16 * q);
    }
    __syncthreads();
#pragma unroll 1
    for (int eg = 0; eg < kGCols / 16; ++eg) {
        const uint8_t* ks = btile + (eg * 16 + n) * PITCH + 32 * g;
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            acc = mfma_fp8(join(*reinterpret_cast<const u32x4*>(ks + kb * 128),
                                *reinterpret_cast<const u32x4*>(ks + kb * 128 + 16)),
                           qf[kb], acc);
        pin(acc);
        const int64_t cbase = col0 + eg * 16 + 4 * g;
        if (qok) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t col = cbase + i;
                if (col < a.ncols)
                    a.out[((int64_t)b * a.Qs + qrow) * a.ncols + col] = col * a.stride < nvr ? acc[i] : -INFINITY;
            }
        }
    }
}

// Candidate filter over every visible entry (stride 1): the (key, entry) of
// every score with s^ >= theta[row] goes to the row's region for this column
// block, blk[cb][row][0 .. kFBlkCap), with the count in blkcnt[cb][row];
// entries past a region's capacity go to the row's overflow list cand[row]
// (count cand_cnt[row], zeroed beforehand).  Keys are the float bits of s^
// with the low 8 bits cleared (|change| < 2^-15 |s^|).
//
// Each wave holds 64 query rows (four 16-row groups) in registers, so every
// key fragment it reads from LDS feeds 4 * KB MFMAs.  Lane (n, g) owns, per
// group, four consecutive entries of one query row (a quad).  A quad whose
// largest score reaches theta is appended to the wave's LDS list, compacted
// with a ballot; the score bits carry tags in their low 8 bits (lane and group
// in the first, the 16-entry group of the block in the second).  The wave
// alone drains its list at the start of every key tile, and before any 16-entry
// group whose quads might not fit: per quad it tests the four truncated keys,
// takes positions from a per-row LDS counter and writes the survivors.  No
// workgroup barrier, no global atomic unless a region overflows.
template <int KB>
__global__ __launch_bounds__(kFThreads, 2) void filter_gemm_kernel(GemmArgs a) {
    constexpr int RB = KB * 128;
    constexpr int PITCH = RB + 16;
    __shared__ __attribute__((aligned(16))) uint8_t btile[kGCols * PITCH];
    __shared__ u32x4 wlist[kFWaves][kFList];
    __shared__ uint2 s_row[kFRows];      // (theta bits, visible columns) per row
    __shared__ uint32_t s_cnt[kFRows];   // candidates per row in this column block
    const GemmTile tl = gemm_tile(a);
    if (!tl.ok) return;
    const int b = tl.b;
    const int64_t cb = tl.cb;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int64_t row0 = (int64_t)tl.rb * kFRows;
    const int64_t col0 = cb * kFBlkCols;
    const int64_t nv_blk = gemm_row_valid(a, b, min(row0 + kFRows, (int64_t)a.Qs) - 1);
    const int64_t nv_first = gemm_row_valid(a, b, row0);
    const int64_t cend = min(a.ncols, nv_blk);  // columns some row of the block sees
    if (col0 >= cend) return;
    {
        const int64_t qrow = row0 + tid;  // thread tid belongs to the wave that owns row tid
        const float thr = qrow < a.Qs ? a.theta[(int64_t)b * a.Qs + qrow] : INFINITY;
        s_row[tid] = make_uint2(__float_as_uint(thr), (uint32_t)min(a.ncols, gemm_row_valid(a, b, qrow)));
        s_cnt[tid] = 0;
    }

    i32x8 qf[kFQG][KB];
    uint32_t lim[kFQG];  // visible columns of the lane's row in each group
    float th[kFQG];
#pragma unroll
    for (int qg = 0; qg < kFQG; ++qg) {
        const int64_t qrow = row0 + wave * 64 + qg * 16 + n;
        const bool ok = qrow < a.Qs;
        const uint8_t* src = a.iq + ((int64_t)b * a.Qs + (ok ? qrow : 0)) * RB + 32 * g;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const u32x4 lo = *reinterpret_cast<const u32x4*>(src + kb * 128);
            const u32x4 hi = *reinterpret_cast<const u32x4*>(src + kb * 128 + 16);
            qf[qg][kb] = ok ? join(lo, hi) : i32x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
        lim[qg] = (uint32_t)min(a.ncols, gemm_row_valid(a, b, qrow));
        th[qg] = ok ? a.theta[(int64_t)b * a.Qs + qrow] : INFINITY;
    }

    u32x4* wl = wlist[wave];
    // thresholds all positive: the pretest may compare float bits as integers
    bool all_pos = true;
#pragma unroll
    for (int qg = 0; qg < kFQG; ++qg) all_pos = all_pos && th[qg] > 0.0f;
    const bool ipre = __ballot(!all_pos) == 0;
    // the tag mask and the lane tags live in VGPRs, so that each tag costs one v_and_or
    uint32_t vmask = 0xffffff00u, ltag[kFQG];
    asm volatile("" : "+v"(vmask));
#pragma unroll
    for (int qg = 0; qg < kFQG; ++qg) {
        ltag[qg] = (uint32_t)(lane | (qg << 6));
        asm volatile("" : "+v"(ltag[qg]));
    }
    // the block's regions, one per row, consecutive from wg_blk
    uint2* const wg_blk = a.blk + (cb * a.B * a.Qs + (int64_t)b * a.Qs + row0) * kFBlkCap;
    constexpr uint32_t row_pitch = kFBlkCap;  // the block's rows are consecutive regions
    // Drain: each lane takes U quads at a time, so that the LDS round trips
    // (quad, row data, row counter) of the U overlap (U = 4 at tile starts; 1
    // inside a tile, where few registers are free and drains are rare).
    auto drain = [&](uint32_t cq, auto u_c) __attribute__((always_inline)) {
        constexpr int U = decltype(u_c)::value;
        __builtin_amdgcn_wave_barrier();
        for (uint32_t j0 = 0; j0 < cq; j0 += 64 * U) {
            u32x4 v[U];
            uint32_t lr[U], c0[U], pm[U], pos[U];
            uint2 rw[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t j = j0 + u * 64 + lane;
                v[u] = wl[j < cq ? j : 0u];
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t lid = v[u][0] & 63u, qg = (v[u][0] >> 6) & 3u;
                lr[u] = (uint32_t)wave * 64u + qg * 16u + (lid & 15u);
                c0[u] = (uint32_t)col0 + (v[u][1] & 0xffu) * 16u + 4u * (lid >> 4);
                rw[u] = s_row[lr[u]];
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                // branch-free: bitwise and of the three tests
                const uint32_t lim_u = j0 + u * 64 + lane < cq ? rw[u].y : 0u;
                pm[u] = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    pm[u] |= (uint32_t)((c0[u] + i < lim_u) & (__uint_as_float(v[u][i] & vmask) >= __uint_as_float(rw[u].x))) << i;
                pos[u] = atomicAdd(&s_cnt[lr[u]], (uint32_t)__popc(pm[u]));  // adding 0 is harmless
            }
            bool over = false;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                uint2* dst = wg_blk + lr[u] * row_pitch;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t q = pos[u] + (uint32_t)__popc(pm[u] & ((1u << i) - 1u));
                    if (((pm[u] >> i) & 1u) && q < (uint32_t)kFBlkCap) dst[q] = make_uint2(v[u][i] & vmask, c0[u] + i);
                }
                over |= pos[u] + (uint32_t)__popc(pm[u]) > (uint32_t)kFBlkCap;
            }
            if (over) {  // a region is full: the row's overflow list
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int64_t r = (int64_t)b * a.Qs + row0 + lr[u];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t q = pos[u] + (uint32_t)__popc(pm[u] & ((1u << i) - 1u));
                        if (((pm[u] >> i) & 1u) && q >= (uint32_t)kFBlkCap) {
                            const uint32_t o = atomicAdd(&a.cand_cnt[r], 1u);
                            if (o < (uint32_t)a.cap) a.cand[r * a.cap + o] = make_uint2(v[u][i] & vmask, c0[u] + i);
                        }
                    }
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
    };

    // the key tile is kGCols consecutive entries, one contiguous run of bytes:
    // load c (16-byte chunk q * kFThreads + tid) lands at entry c / CPE, piece c % CPE
    constexpr int CPE = RB / 16;                   // chunks per entry
    constexpr int NLD = kGCols * CPE / kFThreads;  // chunks per thread
    u32x4 pf[NLD];
    auto load_tile = [&](int64_t tc) __attribute__((always_inline)) {  // the next key tile, into registers
#pragma unroll
        for (int q = 0; q < NLD; ++q) {
            const int c = q * kFThreads + tid;
            int64_t j = tc + c / CPE;
            if (j >= a.ncols) j = 0;  // masked in the epilogue
            pf[q] = *reinterpret_cast<const u32x4*>(a.ik + ((int64_t)b * a.N_cap + j) * RB + (c % CPE) * 16);
        }
    };
    const int ntiles = (int)min<int64_t>(kFSub, (cend - col0 + kGCols - 1) / kGCols);
    uint32_t wcnt = 0;  // quads in the wave's list (wave-uniform)
    load_tile(col0);
    for (int sub = 0; sub < ntiles; ++sub) {
        const int64_t tc0 = col0 + (int64_t)sub * kGCols;
        __syncthreads();  // previous tile consumed
#pragma unroll
        for (int q = 0; q < NLD; ++q) {
            const int c = q * kFThreads + tid;
            *reinterpret_cast<u32x4*>(btile + (c / CPE) * PITCH + (c % CPE) * 16) = pf[q];
        }
        __syncthreads();
        // drain here, before the next tile's loads are issued: the wait for those
        // loads (vmcnt counts stores too) then never waits for fresh stores
        if (wcnt) {
            drain(wcnt, std::integral_constant<int, 4>{});
            wcnt = 0;
        }
        if (sub + 1 < ntiles) load_tile(tc0 + kGCols);
        // every column of the tile visible to every row of the block: no per-score test
        const bool all_visible = tc0 + kGCols <= a.ncols && tc0 + kGCols <= nv_first;
        auto read_kf = [&](i32x8 (&kf)[KB], int eg) {
            const uint8_t* ks = btile + (eg * 16 + n) * PITCH + 32 * g;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
                kf[kb] = join(*reinterpret_cast<const u32x4*>(ks + kb * 128),
                              *reinterpret_cast<const u32x4*>(ks + kb * 128 + 16));
        };
        auto mma = [&](const i32x8 (&kf)[KB], f32x4 (&acc)[kFQG]) {
#pragma unroll
            for (int qg = 0; qg < kFQG; ++qg) acc[qg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int qg = 0; qg < kFQG; ++qg) acc[qg] = mfma_fp8(kf[kb], qf[qg][kb], acc[qg]);
#pragma unroll
            for (int qg = 0; qg < kFQG; ++qg) pin(acc[qg]);
        };
        // MASK: some column of the tile is hidden from some row.  IPRE: every
        // threshold of the wave is positive, so s >= theta is a signed integer
        // comparison of the float bits (no NaN handling, -0 below any theta).
        auto run_tile = [&](auto mask_c, auto ipre_c) __attribute__((always_inline)) {
            constexpr bool MASK = decltype(mask_c)::value, IPRE = decltype(ipre_c)::value;
            // The four query groups' tests are independent; their list positions
            // are wave-uniform prefix sums of the ballots plus the lane's rank, so
            // the four compactions do not wait on each other.  The list has room
            // for every quad of the group (checked before each group), so no
            // write needs a capacity test.
            auto epilogue = [&](f32x4 (&acc)[kFQG], int eg) {
                const uint32_t grp = __builtin_amdgcn_readfirstlane((uint32_t)(sub * (kGCols / 16) + eg));
                const uint32_t c0 = (uint32_t)tc0 + eg * 16 + 4 * g;
                bool p[kFQG];
                uint64_t bal[kFQG];
#pragma unroll
                for (int qg = 0; qg < kFQG; ++qg) {
                    if constexpr (MASK) {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (c0 + (uint32_t)i >= lim[qg]) acc[qg][i] = -INFINITY;
                    }
                    if constexpr (IPRE) {
                        const int32_t m = max(max(__float_as_int(acc[qg][0]), __float_as_int(acc[qg][1])),
                                              max(__float_as_int(acc[qg][2]), __float_as_int(acc[qg][3])));
                        p[qg] = m >= __float_as_int(th[qg]);
                    } else {
                        p[qg] = acc[qg][0] >= th[qg] || acc[qg][1] >= th[qg] || acc[qg][2] >= th[qg] ||
                                acc[qg][3] >= th[qg];
                    }
                    bal[qg] = __ballot(p[qg]);
                }
                uint32_t base[kFQG];
#pragma unroll
                for (int qg = 0; qg < kFQG; ++qg) {
                    base[qg] = wcnt;
                    wcnt += (uint32_t)__popcll(bal[qg]);
                }
#pragma unroll
                for (int qg = 0; qg < kFQG; ++qg) {
                    const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal[qg] >> 32),
                                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)bal[qg], 0u));
                    if (p[qg])
                        wl[base[qg] + below] = u32x4{(__float_as_uint(acc[qg][0]) & vmask) | ltag[qg],
                                                     (__float_as_uint(acc[qg][1]) & vmask) | grp,
                                                     __float_as_uint(acc[qg][2]), __float_as_uint(acc[qg][3])};
                }
            };
            // a group adds at most kFQG * 64 quads: drain first if they might not fit
            auto make_room = [&]() __attribute__((always_inline)) {
                if (wcnt > (uint32_t)(kFList - kFQG * 64)) {
                    drain(wcnt, std::integral_constant<int, 1>{});
                    wcnt = 0;
                }
            };
            // the key fragments of group e + 1 are read while group e computes
            // (VALU and MFMA issue do not overlap on this chip, so the MFMAs
            // themselves are not pipelined against the epilogue)
            i32x8 kfA[KB], kfB[KB];
            f32x4 acc[kFQG];
            read_kf(kfA, 0);
#pragma unroll 1
            for (int eg = 0; eg < kGCols / 16; eg += 2) {
                read_kf(kfB, eg + 1);
                mma(kfA, acc);
                make_room();
                epilogue(acc, eg);
                if (eg + 2 < kGCols / 16) read_kf(kfA, eg + 2);
                mma(kfB, acc);
                make_room();
                epilogue(acc, eg + 1);
            }
        };
        if (all_visible && ipre) run_tile(std::false_type{}, std::true_type{});
        else run_tile(std::true_type{}, std::false_type{});
    }
    if (wcnt) drain(wcnt, std::integral_constant<int, 4>{});
    {
        const int lr = wave * 64 + lane;  // the wave's own rows
        const int64_t qrow = row0 + lr;
        if (qrow < a.Qs) a.blkcnt[cb * a.B * a.Qs + (int64_t)b * a.Qs + qrow] = s_cnt[lr];
    }
}

hipError_t launch_gemm_fp8(GemmArgs a, int mode, hipStream_t stream) {
    if (a.Qs == 0 || a.B == 0 || a.ncols == 0) return hipSuccess;
    if (a.K != 128 && a.K != 256) return hipErrorInvalidValue;
    const int rows = mode == 0 ? kSRows : kFRows;
    const int64_t cols = mode == 0 ? kGCols : kFBlkCols;
    if (mode != 0 && a.stride != 1) return hipErrorInvalidValue;
    a.n_rowblk = (int)((a.Qs + rows - 1) / rows);
    a.n_colblk = (a.ncols + cols - 1) / cols;
    a.tiles = (int64_t)a.B * a.n_colblk * a.n_rowblk;
    a.per_xcd = (a.tiles + 7) / 8;
    const dim3 grid((unsigned)(8 * a.per_xcd));
    if (mode == 0) {
        if (a.K == 128) hipLaunchKernelGGL(sample_gemm_kernel<1>, grid, dim3(kSThreads), 0, stream, a);
        else hipLaunchKernelGGL(sample_gemm_kernel<2>, grid, dim3(kSThreads), 0, stream, a);
    } else {
        if (a.K == 128) hipLaunchKernelGGL(filter_gemm_kernel<1>, grid, dim3(kFThreads), 0, stream, a);
        else hipLaunchKernelGGL(filter_gemm_kernel<2>, grid, dim3(kFThreads), 0, stream, a);
    }
    return hipGetLastError();
}

int64_t gemm_grid_threads(const GemmArgs& a, int mode) {
    if (a.Qs == 0 || a.B == 0 || a.ncols == 0) return 0;
    const int rows = mode == 0 ? kSRows : kFRows;
    const int64_t cols = mode == 0 ? kGCols : kFBlkCols;
    const int64_t tiles = (int64_t)a.B * ((a.ncols + cols - 1) / cols) * ((a.Qs + rows - 1) / rows);
    return 8 * ((tiles + 7) / 8) * (mode == 0 ? kSThreads : kFThreads);
}

int64_t filter_colblks(int64_t ncols) { return (ncols + kFBlkCols - 1) / kFBlkCols; }
int filter_blk_cap() { return kFBlkCap; }

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

// Per-half maximum of two packed 16-bit fields.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
CSA2_DEV uint32_t pk_max_u16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}

// Largest e4m3 exponent field among the four bytes of w (0 for zero and
// subnormal bytes; the sign bit is ignored).
CSA2_DEV uint32_t max_e4m3_field(uint32_t w) {
    const uint32_t f = (w >> 3) & 0x0f0f0f0fu;
    return max(max(f & 0xffu, (f >> 8) & 0xffu), max((f >> 16) & 0xffu, f >> 24));
}

// Per block of 256 entries of a sequence: an upper bound on max_j sum_e ik[j][e]^2
// (e4m3 squares are exact in fp32; the fp32 sum is inflated by its rounding bound),
// and for every group of 8 consecutive elements the largest exponent field of
// the block's keys in that group (kexp[b][blk][g], one byte each).
template <int KB>
__global__ __launch_bounds__(256) void key_norm_kernel(const uint8_t* __restrict__ ik, int64_t N,
                                                        int64_t N_cap, int nblk, float* out, uint8_t* kexp) {
    constexpr int RB = KB * 128;
    constexpr int G = RB / 8;  // groups of 8 elements
    __shared__ float red[4];
    __shared__ uint32_t redx[4][G / 2];
    const int b = blockIdx.y;
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    float s = 0.0f;
    uint32_t gx[G / 2];  // two groups per word, one per 16-bit half
#pragma unroll
    for (int i = 0; i < G / 2; ++i) gx[i] = 0;
    if (j < N) {
        const u32x4* src = reinterpret_cast<const u32x4*>(ik + ((int64_t)b * N_cap + j) * RB);
#pragma unroll
        for (int q = 0; q < RB / 16; ++q) {
            const u32x4 w = src[q];
            // 16 bytes = groups 2q and 2q + 1
            gx[q] = max(max_e4m3_field(w[0]), max_e4m3_field(w[1])) |
                    (max(max_e4m3_field(w[2]), max_e4m3_field(w[3])) << 16);
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
    for (int o = 32; o >= 1; o >>= 1) {
        s = fmaxf(s, __shfl_xor(s, o));
#pragma unroll
        for (int i = 0; i < G / 2; ++i) gx[i] = pk_max_u16(gx[i], (uint32_t)__shfl_xor((int)gx[i], o));
    }
    if ((threadIdx.x & 63) == 0) {
        red[threadIdx.x >> 6] = s;
#pragma unroll
        for (int i = 0; i < G / 2; ++i) redx[threadIdx.x >> 6][i] = gx[i];
    }
    __syncthreads();
    if (threadIdx.x == 0) out[(int64_t)b * nblk + blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    if (threadIdx.x < G) {
        const int i = threadIdx.x >> 1, sh = 16 * (threadIdx.x & 1);
        uint32_t m = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) m = max(m, (redx[w][i] >> sh) & 0xffffu);
        kexp[((int64_t)b * nblk + blockIdx.x) * G + threadIdx.x] = (uint8_t)m;
    }
}

// Per sequence: the largest block bound on ||k||^2 (blockIdx.y == G) and, per group
// g = blockIdx.y < G of 8 elements, the largest key exponent field over all blocks.
__global__ __launch_bounds__(256) void key_bound_kernel(const float* __restrict__ knorm,
                                                         const uint8_t* __restrict__ kexp, int nblk, int G,
                                                         float* kseq_norm, uint8_t* kseq_exp) {
    __shared__ float red[4];
    const int b = blockIdx.x, g = blockIdx.y;
    float m = 0.0f;
    if (g == G) {
        for (int i = threadIdx.x; i < nblk; i += 256) m = fmaxf(m, knorm[(int64_t)b * nblk + i]);
    } else {
        for (int i = threadIdx.x; i < nblk; i += 256) m = fmaxf(m, (float)kexp[((int64_t)b * nblk + i) * G + g]);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        if (g == G) kseq_norm[b] = m;
        else kseq_exp[(int64_t)b * G + g] = (uint8_t)m;
    }
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
// Candidates arrive as (float bits of s^ with the low 8 bits cleared, entry) in
// the row's column-block regions and its overflow list.
template <int KB>
__global__ __launch_bounds__(kBandThreads, 8) void band_final_kernel(BandArgs a) {
    constexpr int RB = KB * 128;
    __shared__ uint32_t s_key[kBandCap];   // sort keys; later the output bitmap
    __shared__ int32_t s_idx[kBandCap];    // entry index; bit 31 = selected
    // the digit histogram is dead once T^ is known; the band list then reuses
    // its words (80 KB in all: two workgroups per CU)
    __shared__ uint32_t s_hist[kBandHist];
    static_assert(kBandHist >= kBandList, "the band list overlays the histogram");
    uint32_t* const hist = s_hist;
    uint32_t* const band = s_hist;                                        // positions of band entries
    __shared__ uint32_t bkey[kBandList];   // keys of the bin that holds T^ (the bin gather)
    __shared__ uint32_t scan_lds[kBandThreads / 64 + 1];
    __shared__ uint32_t dig[2];
    __shared__ uint32_t s_oc[kBandRegBatch];  // per region of a batch: first candidate | count << 16
    __shared__ uint32_t red_u[kBandThreads / 64];
    __shared__ double red_q[kBandThreads / 64];
    __shared__ double red_t[kBandThreads / 64];
    static_assert(kBandCap * 4 >= kBandOutChunk / 8, "the output bitmap overlays s_key");
    static_assert(kBandCap < (1 << 16) && kFBlkCap < (1 << 16), "offset and count share a word");

    const int64_t r = blockIdx.x;
    const int b = (int)(r / a.Qs);
    const int64_t qrow = r % a.Qs;
    int64_t nv = a.nvb ? (int64_t)a.nvb[b] - a.Qs + qrow + 1 : a.N;
    nv = nv < 0 ? 0 : (nv > a.N ? a.N : nv);
    const int64_t keff = nv < a.k ? nv : a.k;
    int32_t* out = a.idx + r * a.k;
    for (int64_t t = keff + threadIdx.x; t < a.k; t += kBandThreads) out[t] = -1;
    if (keff == 0) return;

    auto flag_row = [&]() {  // the exact row kernel recomputes this row
        if (threadIdx.x == 0) {
            a.flag[r] = 1;
            atomicAdd(a.flag_count, 1u);
        }
    };
    // every independent load first: overflow count, region counts, ||q||^2
    // (exact in fp64) and the sequence's bound on max ||k||^2
    const int64_t R = (int64_t)a.B * a.Qs;
    const int nreg = (int)((nv + kFBlkCols - 1) / kFBlkCols);
    const uint32_t novf = a.cand_cnt[r];
    uint32_t mine_c = 0;
    for (int i = threadIdx.x; i < nreg; i += kBandThreads) mine_c += min(a.blkcnt[(int64_t)i * R + r], (uint32_t)kFBlkCap);
    double q2 = 0.0;
    {
        const uint8_t* q = a.iq + r * RB;
        for (int e = threadIdx.x; e < RB; e += kBandThreads) {
            const double v = e4m3_to_f64(q[e]);
            q2 = fma(v, v, q2);
        }
    }
    const float k2 = a.kseq_norm[b];
    // MFMA truncation bound of this row, sum over groups g of 8 elements of
    // 2^(eq_g + ek_g - 10), eq_g / ek_g the largest exponent of the row's / any
    // key's elements in the group (zero and subnormal values count as 2^-6)
    double tr = 0.0;
    if (threadIdx.x < RB / 8) {
        const uint2 w = reinterpret_cast<const uint2*>(a.iq + r * RB)[threadIdx.x];
        const int fq = (int)max(max(max_e4m3_field(w.x), max_e4m3_field(w.y)), 1u);
        const int fk = max((int)a.kseq_exp[(int64_t)b * (RB / 8) + threadIdx.x], 1);
        tr = ldexp(1.0, fq + fk - 24);
    }
    if (novf > (uint32_t)a.cap) {
        flag_row();
        return;
    }
    // the candidates: the row's column-block regions in order, then its overflow list
    uint32_t nblkc;
    block_exclusive_scan(mine_c, scan_lds, &nblkc);
    const uint32_t C = nblkc + novf;
    if (C < (uint32_t)keff || C > (uint32_t)kBandCap) {
        flag_row();
        return;
    }
    // the radix select works on keys relative to the smallest candidate key,
    // which span few bits.  Regions are taken kBandRegBatch at a time (offsets
    // from a block scan of their counts); one wave per region (at most kFBlkCap =
    // 64 entries), so the loads are independent.
    static_assert(kFBlkCap <= 64, "one lane per region entry");
    uint32_t kmin = 0xffffffffu, kmax = 0;
    const int wv = threadIdx.x >> 6, ln = threadIdx.x & 63;
    auto put = [&](uint32_t p, uint2 c) {
        const uint32_t k = sort_key(__uint_as_float(c.x));
        s_key[p] = k;
        s_idx[p] = (int32_t)c.y;
        kmin = min(kmin, k);
        kmax = max(kmax, k);
    };
    uint32_t base = 0;
    for (int i0 = 0; i0 < nreg; i0 += kBandRegBatch) {
        const int nb = min(kBandRegBatch, nreg - i0);
        const uint32_t c = threadIdx.x < nb ? min(a.blkcnt[(int64_t)(i0 + threadIdx.x) * R + r], (uint32_t)kFBlkCap) : 0u;
        uint32_t tot;
        const uint32_t ex = base + block_exclusive_scan(c, scan_lds, &tot);
        if (threadIdx.x < nb) s_oc[threadIdx.x] = ex | (c << 16);
        __syncthreads();
        // a wave takes regions wv, wv + 16, ...: the loads of eight of them are
        // issued before any is stored, so they share one memory round trip
        constexpr int kGU = 8;
        for (int i = wv; i < nb; i += kGU * (kBandThreads / 64)) {
            uint32_t oc[kGU];
            uint2 cv[kGU];
#pragma unroll
            for (int u = 0; u < kGU; ++u) {
                const int iu = i + u * (kBandThreads / 64);
                oc[u] = iu < nb ? s_oc[iu] : 0u;
                // lanes past the region's count read its first slot (in bounds) and store nothing
                const int lu = (uint32_t)ln < (oc[u] >> 16) ? ln : 0;
                cv[u] = a.blk[((int64_t)(i0 + (iu < nb ? iu : i)) * R + r) * kFBlkCap + lu];
            }
#pragma unroll
            for (int u = 0; u < kGU; ++u)
                if ((uint32_t)ln < (oc[u] >> 16)) put((oc[u] & 0xffffu) + ln, cv[u]);
        }
        base += tot;
        __syncthreads();  // s_oc is rewritten by the next batch
    }
    for (uint32_t p = threadIdx.x; p < novf; p += kBandThreads) put(nblkc + p, a.cand[r * a.cap + p]);
    for (int o = 32; o >= 1; o >>= 1) {
        q2 += __shfl_xor(q2, o);
        tr += __shfl_xor(tr, o);
        kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
        kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
    }
    if ((threadIdx.x & 63) == 0) {
        red_q[threadIdx.x >> 6] = q2;
        red_t[threadIdx.x >> 6] = tr;
        red_u[threadIdx.x >> 6] = kmin;
        scan_lds[threadIdx.x >> 6] = kmax;
    }
    __syncthreads();
    double Q2 = 0.0, TR = 0.0;
    const float K2 = k2;
    uint32_t K0 = 0xffffffffu, K1 = 0;
#pragma unroll 2
    for (int wv = 0; wv < kBandThreads / 64; ++wv) {
        Q2 += red_q[wv];
        TR += red_t[wv];
        K0 = min(K0, red_u[wv]);
        K1 = max(K1, scan_lds[wv]);
    }
    __syncthreads();

    // T^: the keff-th largest key.  11-bit digits from the top of the used range;
    // once the digit's bin holds few keys, they are ranked directly.
    constexpr uint32_t DM = kBandHist - 1;
    const int bits = 32 - __clz((int)(K1 - K0) | 1);
    uint32_t prefix = 0, fixed = 0, need = (uint32_t)keff;
    for (int sh = bits > kBandBits ? bits - kBandBits : 0;; sh = sh > kBandBits ? sh - kBandBits : 0) {
        for (int i = threadIdx.x; i < kBandHist; i += kBandThreads) hist[i] = 0;
        __syncthreads();
        for (uint32_t p = threadIdx.x; p < C; p += kBandThreads) {
            const uint32_t k = s_key[p] - K0;
            if ((k & fixed) == prefix) atomicAdd(&hist[(k >> sh) & DM], 1u);
        }
        __syncthreads();
        find_digit<kBandThreads>(hist, kBandHist, need, scan_lds, dig);
        const uint32_t inbin = hist[dig[0]];
        prefix |= dig[0] << sh;
        fixed |= DM << sh;
        need -= dig[1];
        __syncthreads();  // every thread has read dig and hist
        if (sh == 0) break;
        if (inbin <= (uint32_t)kBandList) {
            // gather the bin's keys and find the need-th largest by counting
            if (threadIdx.x == 0) dig[0] = 0;
            __syncthreads();
            for (uint32_t p = threadIdx.x; p < C; p += kBandThreads) {
                const uint32_t k = s_key[p] - K0;
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
    // |approximation - s| <= delta.  The MFMA sums each group of 8 consecutive
    // products after cutting every product toward zero to a multiple of
    // 2^(ea + eb - 13), ea + eb the largest exponent pair of the group: an error
    // below 8 * 2^(eq_g + ek_g - 13) per group (TR).  The group sums, and the
    // accumulator between the KB products, are added in fp32: at most 2 * RB/8 + 1
    // roundings with unit roundoff 2^-23 (covers truncation), doubled, against
    // sum|p| <= ||q|| ||k|| (Cauchy-Schwarz).  Plus the 2^-15 relative key
    // truncation and the final rounding of s, and an absolute term for subnormal
    // flushing.
    const double Kd = (double)(2 * (RB / 8) + 1);
    const double gam = Kd * 0x1p-23 / (1.0 - Kd * 0x1p-23);
    const double E = 2.0 * gam * sqrt(Q2 * (double)K2) * (1.0 + 0x1p-20) + TR * (1.0 + 0x1p-40) + 0x1p-100;
    const double delta = E + 0x1p-14 * (fabs(That) + E);
    const double lo = That - 2.0 * delta, hi = That + 2.0 * delta;
    if (!(a.theta[r] <= lo)) {
        flag_row();
        return;
    }
    // classify: above the band -> selected (bit 31); inside -> band list (block-scan compaction)
    uint32_t nin_mine = 0;
    {
        uint32_t inb = 0;  // bit u: position threadIdx.x * PER + u is in the band
        uint32_t nb_mine = 0;
        constexpr int PER = kBandCap / kBandThreads;
        static_assert(PER <= 32, "one bit per position");
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const uint32_t p = threadIdx.x * PER + u;  // contiguous per thread
            if (p < C) {
                const double v = key_to_float(s_key[p]);
                if (v > hi) {
                    ++nin_mine;
                    s_idx[p] |= (int32_t)0x80000000;
                } else if (v >= lo) {
                    inb |= 1u << u;
                    ++nb_mine;
                }
            }
        }
        // both counts in one scan: band positions in the low 16 bits, selected
        // entries above (each total is at most kBandCap < 2^16)
        uint32_t tot2;
        uint32_t pos = block_exclusive_scan(nb_mine | (nin_mine << 16), scan_lds, &tot2) & 0xffffu;
        while (inb) {
            const int u = __ffs(inb) - 1;
            inb &= inb - 1;
            if (pos < (uint32_t)kBandList) band[pos] = threadIdx.x * PER + u;
            ++pos;
        }
        if (threadIdx.x == 0) {
            dig[0] = tot2 & 0xffffu;
            dig[1] = tot2 >> 16;
        }
    }
    __syncthreads();
    const uint32_t nband = dig[0], nin = dig[1];
    if (nband > (uint32_t)kBandList || nin > (uint32_t)keff || (uint32_t)keff - nin > nband) {
        flag_row();  // a very wide band, or the error bound did not hold
        return;
    }
    const uint32_t need_b = (uint32_t)keff - nin;
    if (need_b > 0) {
        uint64_t* const bcomp = reinterpret_cast<uint64_t*>(s_key);  // the band's exact keys
        static_assert(kBandCap >= 2 * kBandList, "bcomp fits s_key");
        // exact rescoring of the band, LPE lanes per entry: e4m3 products and all
        // their partial sums are exact in fp64 (multiples of 2^-18 below 2^30), so
        // the fp64 sum rounded once is the defined score
        constexpr int LPE = 8, BPL = RB / LPE;
        const int sub = threadIdx.x % LPE;
        const uint8_t* qrow = a.iq + r * RB + sub * BPL;
        for (uint32_t t0 = 0; t0 < nband; t0 += kBandThreads / LPE) {
            const uint32_t t = t0 + threadIdx.x / LPE;
            const bool live = t < nband;
            const int32_t j = live ? s_idx[band[t]] : s_idx[band[0]];
            const uint8_t* krow = a.ik + ((int64_t)b * a.N_cap + j) * RB + sub * BPL;
            double acc = 0.0;
            // the key chunks are requested together (the query chunks hit in cache)
            u32x4 kvs[BPL / 16];
#pragma unroll
            for (int c = 0; c < BPL / 16; ++c) kvs[c] = *reinterpret_cast<const u32x4*>(krow + 16 * c);
#pragma unroll 1
            for (int c = 0; c < BPL / 16; ++c) {
                const u32x4 qv = *reinterpret_cast<const u32x4*>(qrow + 16 * c);
                const u32x4 kv = kvs[c];
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const auto q0 = __builtin_amdgcn_cvt_pk_f32_fp8(qv[w], false), q1 = __builtin_amdgcn_cvt_pk_f32_fp8(qv[w], true);
                    const auto k0 = __builtin_amdgcn_cvt_pk_f32_fp8(kv[w], false), k1 = __builtin_amdgcn_cvt_pk_f32_fp8(kv[w], true);
                    acc = fma((double)q0[0], (double)k0[0], acc);
                    acc = fma((double)q0[1], (double)k0[1], acc);
                    acc = fma((double)q1[0], (double)k1[0], acc);
                    acc = fma((double)q1[1], (double)k1[1], acc);
                }
            }
#pragma unroll
            for (int o = LPE / 2; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
            if (live && sub == 0) {
                // (exact score desc, index asc) as one 64-bit key, larger first; the
                // candidate keys in s_key are no longer needed
                const float sc = (float)acc;
                bcomp[t] = ((uint64_t)sort_key(sc == 0.0f ? 0.0f : sc) << 32) | (uint32_t)~j;
            }
        }
        __syncthreads();
        // rank in the band: the entries ahead of t are those with a larger bcomp;
        // the first need_b are taken.  Four lanes share each t (every fourth v),
        // eight v per step so the LDS reads overlap.
        const uint32_t part = threadIdx.x & 3;
        for (uint32_t t0 = 0; t0 < nband; t0 += kBandThreads / 4) {
            const uint32_t t = t0 + (threadIdx.x >> 2);
            const uint64_t ct = t < nband ? bcomp[t] : ~0ull;
            uint32_t rank = 0;
            uint32_t v = part;
            for (; v + 28 < nband; v += 32) {
#pragma unroll
                for (int u = 0; u < 8; ++u) rank += bcomp[v + 4 * u] > ct ? 1u : 0u;
            }
            for (; v < nband; v += 4) rank += bcomp[v] > ct ? 1u : 0u;
            rank += __shfl_xor((int)rank, 1);
            rank += __shfl_xor((int)rank, 2);
            if (t < nband && part == 0 && rank < need_b) s_idx[band[t]] = (int32_t)~(uint32_t)ct | (int32_t)0x80000000;
        }
    }
    __syncthreads();
    // ascending output from a bitmap of the selected entries (over s_key), one
    // pass per kBandOutChunk entries of the row.  With one pass (rows of up to
    // kBandOutChunk entries) the count of selected entries is checked against
    // keff from the pass's own scan before anything is written; longer rows
    // count them first.
    uint32_t* bitmap = s_key;
    uint32_t written = 0;
    const bool one_pass = nv <= kBandOutChunk;
    if (!one_pass) {
        uint32_t nsel_mine = 0, nsel;
        for (uint32_t p = threadIdx.x; p < C; p += kBandThreads) nsel_mine += s_idx[p] < 0 ? 1u : 0u;
        block_exclusive_scan(nsel_mine, scan_lds, &nsel);
        if (nsel != (uint32_t)keff) {  // cannot happen when the bound holds
            flag_row();
            return;
        }
    }
    for (int64_t j0 = 0; j0 < nv; j0 += kBandOutChunk) {
        const int64_t jn = min(nv - j0, (int64_t)kBandOutChunk);
        const int nwords = (int)((jn + 31) / 32);
        for (int i = threadIdx.x; i < nwords; i += kBandThreads) bitmap[i] = 0;
        __syncthreads();
        for (uint32_t p = threadIdx.x; p < C; p += kBandThreads) {
            const int32_t v = s_idx[p];
            if (v < 0) {
                const int64_t j = (int64_t)(v & 0x7fffffff) - j0;
                if (j >= 0 && j < jn) atomicOr(&bitmap[j >> 5], 1u << (j & 31));
            }
        }
        __syncthreads();
        const int per = (nwords + kBandThreads - 1) / kBandThreads;
        uint32_t mine = 0;
        for (int wi = threadIdx.x * per; wi < min(nwords, (int)(threadIdx.x + 1) * per); ++wi) mine += __popc(bitmap[wi]);
        uint32_t total;
        uint32_t pos = written + block_exclusive_scan(mine, scan_lds, &total);
        if (one_pass && total != (uint32_t)keff) {  // cannot happen when the bound holds
            flag_row();
            return;
        }
        for (int wi = threadIdx.x * per; wi < min(nwords, (int)(threadIdx.x + 1) * per); ++wi) {
            uint32_t word = bitmap[wi];
            while (word) {
                const int bit = __ffs(word) - 1;
                word &= word - 1;
                if (pos < (uint32_t)keff) out[pos] = (int32_t)(j0 + wi * 32 + bit);
                ++pos;
            }
        }
        written += total;
        __syncthreads();  // the bitmap is cleared for the next pass
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

hipError_t launch_key_norm(const uint8_t* ik, int K, int B, int64_t N, int64_t N_cap, int nblk, float* knorm,
                           uint8_t* kexp, float* kseq_norm, uint8_t* kseq_exp, hipStream_t stream) {
    if (B == 0 || N == 0) return hipSuccess;
    const dim3 grid((unsigned)nblk, (unsigned)B);
    if (K == 128)
        hipLaunchKernelGGL(key_norm_kernel<1>, grid, dim3(256), 0, stream, ik, N, N_cap, nblk, knorm, kexp);
    else if (K == 256)
        hipLaunchKernelGGL(key_norm_kernel<2>, grid, dim3(256), 0, stream, ik, N, N_cap, nblk, knorm, kexp);
    else
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(key_bound_kernel, dim3((unsigned)B, (unsigned)(K / 8 + 1)), dim3(256), 0, stream, knorm, kexp,
                       nblk, K / 8, kseq_norm, kseq_exp);
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
