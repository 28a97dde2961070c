// S3 - Top-k selection: the k valid entries first in the order (score
// descending, index ascending), written in ascending index order, -1 padded.
//
// "Why Is DeepSeek V4.1 Flash So Fast?", sections 3-4: after the cheap
// relevance search only the useful compressed positions are kept (512 in the
// published configuration, k is a parameter here).
//
// Radix select on the order-preserving 32-bit key of each fp32 score:
//   1. digit 1 = key bits 31..20 (4096 bins).  Its per-row histogram is built
//      by the score kernel (or by topk_hist_kernel for caller-given scores);
//   2. topk_compact_kernel: every slice of a row (4096 entries, more for rows
//      beyond 2^24 entries) finds the bin b1 in which the k-th largest key
//      falls and writes, in index order, the entries whose digit is >= b1 to
//      its own segment of a candidate buffer;
//   3. topk_final_kernel: one workgroup per row scans the slice counts, copies
//      the candidates (slice order = index order) into LDS in one parallel
//      pass (or reads them in place when there are too many, e.g. under heavy
//      ties), resolves digit 2 (bits 19..8) and digit 3 (bits 7..0) among those
//      in bin b1 to the exact k-th key T and the number of entries equal to T
//      still to take, then writes the selection in index order: every key > T,
//      and the first `quota` keys == T (lowest indices).
// Every decision is an integer comparison of keys, so the result is identical
// to sorting with the stated order.
#include "common.h"
#include "launch.h"

namespace csa2 {

constexpr int kSliceThreads = 256;
constexpr int kSubLen = 4096;      // entries per compaction pass (16 per thread)
constexpr int kMaxSlices = 4096;   // slices per row (the final kernel scans their counts in LDS)
constexpr int kFinalThreads = 1024;
constexpr int kFinalCap = 5632;    // candidates the final kernel holds in LDS

// Slice length: a multiple of kSubLen with at most kMaxSlices slices per row.
int64_t topk_slice_len(int64_t N) {
    int64_t len = kSubLen;
    while ((N + len - 1) / len > kMaxSlices) len += kSubLen;
    return len;
}

CSA2_DEV int64_t topk_row_valid(const TopkArgs& a, int64_t r) {
    if (!a.nvb) return a.N;
    const int64_t b = r / a.Qs, i = r % a.Qs;
    int64_t nv = (int64_t)a.nvb[b] - a.Qs + i + 1;
    return nv < 0 ? 0 : (nv > a.N ? a.N : nv);
}

// Histogram of digit 1 over the valid scores of each row (caller-given scores).
__global__ __launch_bounds__(kSliceThreads) void topk_hist_kernel(TopkArgs a) {
    __shared__ uint32_t lh[kHistBins];
    const int64_t r = blockIdx.y;
    const int64_t nv = topk_row_valid(a, r);
    const int64_t j0 = (int64_t)blockIdx.x * a.slice_len;
    if (j0 >= nv) return;
    for (int i = threadIdx.x; i < kHistBins; i += kSliceThreads) lh[i] = 0;
    __syncthreads();
    const float* s = a.scores + r * a.ld;
    const int64_t j1 = j0 + a.slice_len < nv ? j0 + a.slice_len : nv;
    for (int64_t j = j0 + threadIdx.x; j < j1; j += kSliceThreads)
        atomicAdd(&lh[sort_key(s[j]) >> (32 - kHistBits)], 1u);
    __syncthreads();
    uint32_t* gh = a.hist + r * kHistBins;
    for (int i = threadIdx.x; i < kHistBins; i += kSliceThreads)
        if (lh[i]) atomicAdd(&gh[i], lh[i]);
}

// One workgroup per (slice, row): finds the digit-1 bin b1 of the row's k-th
// largest key and writes, in index order, the slice's entries whose digit is
// >= b1 to the slice's segment of the candidate buffer (segment = the slice's
// index range, so it cannot overflow), and their count to slice_cnt.
__global__ __launch_bounds__(kSliceThreads) void topk_compact_kernel(TopkArgs a) {
    __shared__ uint32_t scan_lds[kSliceThreads / 64 + 1];
    __shared__ uint32_t dig[2];
    const int64_t r = blockIdx.y;
    const int64_t nv = topk_row_valid(a, r);
    const int64_t keff = nv < a.k ? nv : a.k;
    const int64_t j0 = (int64_t)blockIdx.x * a.slice_len;
    uint32_t* cnt = a.slice_cnt + r * a.slices + blockIdx.x;
    if (j0 >= nv || keff == 0) {
        if (threadIdx.x == 0) *cnt = 0;
        return;
    }
    find_digit<kSliceThreads>(a.hist + r * kHistBins, kHistBins, (uint32_t)keff, scan_lds, dig);
    const uint32_t b1 = dig[0];
    const float* s = a.scores + r * a.ld;
    int32_t* ci = a.cand_idx + r * a.N + j0;
    uint32_t* ck = a.cand_key + r * a.N + j0;
    const int64_t j_end = j0 + a.slice_len < nv ? j0 + a.slice_len : nv;
    uint32_t written = 0;
    for (int64_t js = j0; js < j_end; js += kSubLen) {
        // thread t scans entries js + 16t .. js + 16t + 15 in order
        const int64_t jt = js + 16 * (int64_t)threadIdx.x;
        uint32_t keys[16];
        uint32_t mine = 0;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int64_t j = jt + u;
            keys[u] = j < j_end ? sort_key(s[j]) : 0u;
            const bool take = j < j_end && (keys[u] >> (32 - kHistBits)) >= b1;
            mine |= (uint32_t)take << u;
        }
        uint32_t total;
        uint32_t off = written + block_exclusive_scan(__popc(mine), scan_lds, &total);
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            if (mine >> u & 1u) {
                ci[off] = (int32_t)(jt + u);
                ck[off] = keys[u];
                ++off;
            }
        }
        written += total;
    }
    if (threadIdx.x == 0) *cnt = written;
}

// One workgroup per row.  The candidates of all slices form one list in index
// order; position p lies in the slice s with off[s] <= p < off[s+1].  When the
// list fits, it is first copied to LDS; every later pass reads it from there.
__global__ __launch_bounds__(kFinalThreads) void topk_final_kernel(TopkArgs a) {
    __shared__ uint32_t scan_lds[kFinalThreads / 64 + 1];
    __shared__ uint32_t h2[kHistBins];
    __shared__ uint32_t dig[2];
    __shared__ uint32_t s_off[kMaxSlices + 1];
    __shared__ uint32_t s_key[kFinalCap];
    __shared__ int32_t s_idx[kFinalCap];
    const int64_t r = blockIdx.x;
    const int64_t nv = topk_row_valid(a, r);
    const int64_t keff = nv < a.k ? nv : a.k;
    int32_t* out = a.idx + r * a.k;
    for (int64_t t = keff + threadIdx.x; t < a.k; t += kFinalThreads) out[t] = -1;
    if (keff == 0) return;

    find_digit<kFinalThreads>(a.hist + r * kHistBins, kHistBins, (uint32_t)keff, scan_lds, dig);
    const uint32_t b1 = dig[0];
    const uint32_t need1 = (uint32_t)keff - dig[1];  // still to take from bin b1

    // slice offsets: exclusive scan of the counts, four slices per thread
    const int nslices = (int)((nv + a.slice_len - 1) / a.slice_len);
    const uint32_t* cnts = a.slice_cnt + r * a.slices;
    {
        uint32_t c[4], sum = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int sl = 4 * threadIdx.x + u;
            c[u] = sl < nslices ? cnts[sl] : 0u;
            sum += c[u];
        }
        uint32_t total;
        uint32_t run = block_exclusive_scan(sum, scan_lds, &total);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int sl = 4 * threadIdx.x + u;
            if (sl < nslices) s_off[sl] = run;
            run += c[u];
        }
        if (threadIdx.x == 0) s_off[nslices] = total;
    }
    __syncthreads();
    const uint32_t C = s_off[nslices];
    const bool in_lds = C <= (uint32_t)kFinalCap;
    const int32_t* ci = a.cand_idx + r * a.N;
    const uint32_t* ck = a.cand_key + r * a.N;
    // global position of flat candidate p
    auto gpos = [&](uint32_t p) -> int64_t {
        int lo = 0, hi = nslices;  // s_off[lo] <= p < s_off[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_off[mid] <= p) lo = mid; else hi = mid;
        }
        return (int64_t)lo * a.slice_len + (p - s_off[lo]);
    };
    if (in_lds) {
        for (uint32_t p = threadIdx.x; p < C; p += kFinalThreads) {
            const int64_t gp = gpos(p);
            s_key[p] = ck[gp];
            s_idx[p] = ci[gp];
        }
    }
    auto key_at = [&](uint32_t p) -> uint32_t { return in_lds ? s_key[p] : ck[gpos(p)]; };
    auto idx_at = [&](uint32_t p) -> int32_t { return in_lds ? s_idx[p] : ci[gpos(p)]; };

    // digit 2 among candidates of bin b1
    for (int i = threadIdx.x; i < kHistBins; i += kFinalThreads) h2[i] = 0;
    __syncthreads();
    for (uint32_t p = threadIdx.x; p < C; p += kFinalThreads) {
        const uint32_t key = key_at(p);
        if ((key >> 20) == b1) atomicAdd(&h2[(key >> 8) & 0xfffu], 1u);
    }
    __syncthreads();
    find_digit<kFinalThreads>(h2, kHistBins, need1, scan_lds, dig);
    const uint32_t b2 = dig[0];
    const uint32_t need2 = need1 - dig[1];
    const uint32_t pre2 = (b1 << 12) | b2;  // key bits 31..8

    // digit 3 among candidates with bits 31..8 == pre2
    for (int i = threadIdx.x; i < 256; i += kFinalThreads) h2[i] = 0;
    __syncthreads();
    for (uint32_t p = threadIdx.x; p < C; p += kFinalThreads) {
        const uint32_t key = key_at(p);
        if ((key >> 8) == pre2) atomicAdd(&h2[key & 0xffu], 1u);
    }
    __syncthreads();
    find_digit<kFinalThreads>(h2, 256, need2, scan_lds, dig);
    const uint32_t T = (pre2 << 8) | dig[0];
    const uint32_t quota = need2 - dig[1];  // keys equal to T still to take

    // ordered output: keys > T, plus the first `quota` keys == T
    uint32_t ties_before = 0, written = 0;
    for (uint32_t p0 = 0; p0 < C; p0 += kFinalThreads) {
        const uint32_t p = p0 + threadIdx.x;
        uint32_t key = 0;
        int32_t j = -1;
        if (p < C) {
            key = key_at(p);
            j = idx_at(p);
        }
        const uint32_t tie = (p < C && key == T) ? 1u : 0u;
        uint32_t ntie;
        const uint32_t tie_rank = ties_before + block_exclusive_scan(tie, scan_lds, &ntie);
        const uint32_t sel = (p < C && (key > T || (tie && tie_rank < quota))) ? 1u : 0u;
        uint32_t nsel;
        const uint32_t pos = written + block_exclusive_scan(sel, scan_lds, &nsel);
        if (sel && pos < (uint32_t)keff) out[pos] = j;
        ties_before += ntie;
        written += nsel;
    }
}

// Rows of up to kRowMaxN entries: the whole selection in one workgroup per
// row and one pass over the scores (what the compact + final pair does in two
// launches).  Steps:
//   1. b1 = the digit-1 bin of the keff-th largest key, from the row histogram;
//   2. one coalesced pass: digit above b1 -> bit in an LDS bitmap of selected
//      entries; digit == b1 -> (key, index) into an LDS candidate list;
//   3. digits 2 and 3 over the candidates give the exact keff-th key T and the
//      number `quota` of entries equal to T to take;
//   4. candidates above T join the bitmap; entries equal to T join it too when
//      all of them are taken, otherwise the first `quota` in index order are
//      found with an ordered scan of the row;
//   5. the bitmap is written out in index order.
// A threshold bin with more than kRowCand entries (heavy ties) is resolved
// from the scores in global memory instead of the LDS list: slower, same result.
constexpr int kRowThreads = 1024;
constexpr int kRowCand = 4096;
constexpr int64_t kRowMaxN = 1 << 19;  // the bitmap (64 KiB) lives in LDS
constexpr int64_t kRowPassN = 1 << 17;  // longest row the row kernel takes when rows are few
constexpr int64_t kRowFill = 256;       // rows that keep every CU busy with the row kernel

__global__ __launch_bounds__(kRowThreads) void topk_row_kernel(TopkArgs a) {
    __shared__ __attribute__((aligned(16))) uint32_t s_hist[kHistBins];
    __shared__ uint32_t s_ckey[kRowCand];
    __shared__ int32_t s_cidx[kRowCand];
    __shared__ uint32_t s_bits[kRowMaxN / 32];
    __shared__ uint32_t scan_lds[kRowThreads / 64 + 1];
    __shared__ uint32_t dig[2];
    __shared__ uint32_t s_ncand;
    const int64_t r = blockIdx.x;
    const int64_t nv = topk_row_valid(a, r);
    const int64_t keff = nv < a.k ? nv : a.k;
    int32_t* out = a.idx + r * a.k;
    for (int64_t t = keff + threadIdx.x; t < a.k; t += kRowThreads) out[t] = -1;
    if (keff == 0) return;
    const float* s = a.scores + r * a.ld;
    const int nwords = (int)((nv + 31) / 32);
    // the first batch of the row's scores is requested before anything else,
    // so its latency overlaps the histogram's
    const int64_t nv4 = (reinterpret_cast<uintptr_t>(s) & 15) == 0 ? nv / 4 : 0;
    const float4* s4 = reinterpret_cast<const float4*>(s);
    constexpr int U = 8;  // 16-byte loads per thread per batch: 32K entries
    float4 v[U];
    auto load_batch = [&](int64_t q0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t q = q0 + u * kRowThreads + threadIdx.x;
            v[u] = s4[q < nv4 ? q : 0];
        }
    };
    if (nv4 > 0) load_batch(0);

    // 1. digit 1 (one uint4 of the histogram per thread: a single round trip,
    //    shared with the first batch of scores)
    static_assert(kHistBins / 4 == kRowThreads, "one uint4 of the histogram per thread");
    reinterpret_cast<uint4*>(s_hist)[threadIdx.x] = reinterpret_cast<const uint4*>(a.hist + r * kHistBins)[threadIdx.x];
    for (int i = threadIdx.x; i < nwords; i += kRowThreads) s_bits[i] = 0;
    if (threadIdx.x == 0) s_ncand = 0;
    __syncthreads();
    find_digit<kRowThreads>(s_hist, kHistBins, (uint32_t)keff, scan_lds, dig);
    const uint32_t b1 = dig[0];
    const uint32_t need2 = (uint32_t)keff - dig[1];  // still to take from bin b1
    const bool in_lds = s_hist[b1] <= (uint32_t)kRowCand;
    __syncthreads();

    // 2. one pass over the row
    auto visit = [&](uint32_t key, int64_t j) {
        const uint32_t d = key >> (32 - kHistBits);
        if (d > b1) {
            atomicOr(&s_bits[j >> 5], 1u << (j & 31));
        } else if (d == b1 && in_lds) {
            const uint32_t p = atomicAdd(&s_ncand, 1u);
            if (p < (uint32_t)kRowCand) {  // always, given the histogram of these scores
                s_ckey[p] = key;
                s_cidx[p] = (int32_t)j;
            }
        }
    };
    // The aligned part, one batch at a time, with no LDS atomics: a wave's 64
    // lanes hold 256 consecutive entries, so each bitmap word of entries above
    // bin b1 belongs to 8 lanes and is built with an OR across them and stored
    // once; the threshold bin's entries are counted per thread and placed in
    // the candidate list by a block scan.
    const int lane = threadIdx.x & 63;
    uint32_t cbase = 0;  // candidates placed by earlier batches
    for (int64_t q0 = 0; q0 < nv4; q0 += (int64_t)U * kRowThreads) {
        if (q0 > 0) load_batch(q0);
        uint32_t cm[U / 8] = {};  // bit 4u + c (mod 32): component c of load u lies in bin b1
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t q = q0 + u * kRowThreads + threadIdx.x;
            const bool ok = q < nv4;
            const float x4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
            uint32_t nib = 0;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t d = sort_key(x4[c]) >> (32 - kHistBits);
                nib |= (ok && d > b1) ? 1u << c : 0u;
                cm[u / 8] |= (ok && in_lds && d == b1) ? 1u << (4 * (u % 8) + c) : 0u;
            }
            uint32_t word = nib << (4 * (lane & 7));
            word |= (uint32_t)__builtin_amdgcn_ds_swizzle((int)word, (1 << 10) | 0x1f);
            word |= (uint32_t)__builtin_amdgcn_ds_swizzle((int)word, (2 << 10) | 0x1f);
            word |= (uint32_t)__builtin_amdgcn_ds_swizzle((int)word, (4 << 10) | 0x1f);
            if (ok && (lane & 7) == 0) s_bits[(4 * q) >> 5] = word;
        }
        uint32_t mine = 0;
#pragma unroll
        for (int i = 0; i < U / 8; ++i) mine += __popc(cm[i]);
        uint32_t batch_total;
        uint32_t pos = cbase + block_exclusive_scan(mine, scan_lds, &batch_total);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t m4 = (cm[u / 8] >> (4 * (u % 8))) & 15u;
            if (m4) {
                const int64_t q = q0 + u * kRowThreads + threadIdx.x;
                const float x4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    if ((m4 >> c) & 1u) {
                        if (pos < (uint32_t)kRowCand) {  // always, given the histogram of these scores
                            s_ckey[pos] = sort_key(x4[c]);
                            s_cidx[pos] = (int32_t)(4 * q + c);
                        }
                        ++pos;
                    }
                }
            }
        }
        cbase += batch_total;
    }
    if (threadIdx.x == 0) s_ncand = cbase;
    __syncthreads();  // words stored whole above; the tail below ORs into them
    for (int64_t j = 4 * nv4 + threadIdx.x; j < nv; j += kRowThreads) visit(sort_key(s[j]), j);
    __syncthreads();
    const uint32_t C = min(s_ncand, (uint32_t)kRowCand);

    // the threshold bin's keys: from LDS, or filtered from the row
    auto for_each_cand = [&](auto f) {
        if (in_lds) {
            for (uint32_t p = threadIdx.x; p < C; p += kRowThreads) f(s_ckey[p], (int64_t)s_cidx[p]);
        } else {
            for (int64_t j = threadIdx.x; j < nv; j += kRowThreads) {
                const uint32_t key = sort_key(s[j]);
                if ((key >> (32 - kHistBits)) == b1) f(key, j);
            }
        }
    };
    // 3. digits 2 (bits 19..8) and 3 (bits 7..0)
    uint32_t prefix = b1 << (32 - kHistBits), need = need2;
    {
        for (int i = threadIdx.x; i < kHistBins; i += kRowThreads) s_hist[i] = 0;
        __syncthreads();
        for_each_cand([&](uint32_t key, int64_t) { atomicAdd(&s_hist[(key >> 8) & 0xfffu], 1u); });
        __syncthreads();
        find_digit<kRowThreads>(s_hist, kHistBins, need, scan_lds, dig);
        prefix |= dig[0] << 8;
        need -= dig[1];
        __syncthreads();
        for (int i = threadIdx.x; i < 256; i += kRowThreads) s_hist[i] = 0;
        __syncthreads();
        for_each_cand([&](uint32_t key, int64_t) {
            if ((key & 0xffffff00u) == prefix) atomicAdd(&s_hist[key & 0xffu], 1u);
        });
        __syncthreads();
        find_digit<kRowThreads>(s_hist, 256, need, scan_lds, dig);
        prefix |= dig[0];
        need -= dig[1];
    }
    const uint32_t T = prefix, quota = need;  // take every key > T and `quota` keys == T
    const uint32_t ties = s_hist[T & 0xffu];
    __syncthreads();

    // 4. candidates above T; ties when all of them are taken
    for_each_cand([&](uint32_t key, int64_t j) {
        if (key > T || (key == T && quota == ties)) atomicOr(&s_bits[j >> 5], 1u << (j & 31));
    });
    if (quota != ties) {
        // the first `quota` entries equal to T in index order: ordered scan of the row
        uint32_t before = 0;
        for (int64_t j0 = 0; j0 < nv && before < quota; j0 += kRowThreads) {
            const int64_t j = j0 + threadIdx.x;
            const uint32_t tie = (j < nv && sort_key(s[j]) == T) ? 1u : 0u;
            uint32_t n;
            const uint32_t rank = before + block_exclusive_scan(tie, scan_lds, &n);
            if (tie && rank < quota) atomicOr(&s_bits[j >> 5], 1u << (j & 31));
            before += n;
        }
    }
    __syncthreads();

    // 5. ascending output
    const int per = (nwords + kRowThreads - 1) / kRowThreads;
    uint32_t mine = 0;
    for (int wi = threadIdx.x * per; wi < min(nwords, (int)(threadIdx.x + 1) * per); ++wi) mine += __popc(s_bits[wi]);
    uint32_t total;
    uint32_t pos = block_exclusive_scan(mine, scan_lds, &total);
    for (int wi = threadIdx.x * per; wi < min(nwords, (int)(threadIdx.x + 1) * per); ++wi) {
        uint32_t word = s_bits[wi];
        while (word) {
            const int bit = __ffs(word) - 1;
            word &= word - 1;
            if (pos < (uint32_t)keff) out[pos] = wi * 32 + bit;
            ++pos;
        }
    }
}

// Split path for rows of up to kRowMaxN entries when rows are too few to keep
// the chip busy with one workgroup each: the pass over the scores is spread
// over many workgroups per row, and one workgroup per row finishes.
//   topk_slice_kernel, one workgroup per (slice, row): b1 from the row
//     histogram, then for its slice the bitmap words of the entries whose
//     digit is above b1 (thread pairs own 32 consecutive entries, so each word
//     is stored once) and, in index order, the (index, key) of the entries in
//     bin b1, written to the slice's own segment of the candidate buffer;
//   topk_merge_kernel, one workgroup per row: the candidates of all slices
//     (one list in index order) to LDS, digits 2 and 3 to the exact keff-th
//     key T, the bitmap to LDS, candidates above T (and the first `quota`
//     equal to T, in index order) into it, then the ordered output.
constexpr int kSplitThreads = 256;
constexpr int kSplitSub = 16 * kSplitThreads;  // entries per pass: 16 per thread
constexpr int kSplitMaxSlices = kRowMaxN / kSplitSub;
constexpr int64_t kSplitMinN = 8192;          // shorter rows: the row kernel alone
constexpr int kSplitTargetBlocks = 512;

// Slice length of the split path: whole passes, about kSplitTargetBlocks
// workgroups in all.
int64_t split_len(int64_t R, int64_t N) {
    const int64_t subs = (N + kSplitSub - 1) / kSplitSub;
    int64_t per = R * subs / kSplitTargetBlocks;
    if (per < 1) per = 1;
    if (per > subs) per = subs;
    return per * kSplitSub;
}

__global__ __launch_bounds__(kSplitThreads) void topk_slice_kernel(TopkArgs a, int64_t len) {
    __shared__ __attribute__((aligned(16))) uint32_t s_hist[kHistBins];
    __shared__ uint32_t scan_lds[kSplitThreads / 64 + 1];
    __shared__ uint32_t dig[2];
    const int64_t r = blockIdx.y;
    const int tid = threadIdx.x;
    const int64_t nv = topk_row_valid(a, r);
    const int64_t keff = nv < a.k ? nv : a.k;
    const int64_t j0 = (int64_t)blockIdx.x * len;
    uint32_t* cnt = a.slice_cnt + r * a.slices + blockIdx.x;
    if (j0 >= nv || keff == 0) {
        if (tid == 0) *cnt = 0;
        return;
    }
    const float* s = a.scores + r * a.ld;
    const bool aligned16 = (reinterpret_cast<uintptr_t>(s) & 15) == 0;
    const int64_t j_end = j0 + len < nv ? j0 + len : nv;
    // thread t takes entries jt .. jt + 15 of each pass (jt a multiple of 16, of 32
    // for even t); the first pass's scores are requested before the histogram so
    // that the two latencies overlap, and each later pass's while the one before
    // it is processed
    float x[16], xn[16];
    auto load = [&](float(&dst)[16], int64_t jt) __attribute__((always_inline)) {
        if (aligned16 && jt + 16 <= j_end) {
            const float4* s4 = reinterpret_cast<const float4*>(s + jt);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float4 v = s4[c];
                dst[4 * c] = v.x;
                dst[4 * c + 1] = v.y;
                dst[4 * c + 2] = v.z;
                dst[4 * c + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int u = 0; u < 16; ++u) dst[u] = jt + u < j_end ? s[jt + u] : 0.0f;
        }
    };
    load(x, j0 + 16 * (int64_t)tid);
    {
        // all of a thread's histogram loads before any LDS store, so that one
        // memory round trip covers them
        constexpr int kPer = kHistBins / 4 / kSplitThreads;
        static_assert(kPer * 4 * kSplitThreads == kHistBins, "whole uint4 per thread");
        const uint4* h4 = reinterpret_cast<const uint4*>(a.hist + r * kHistBins);
        uint4 hv[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) hv[i] = h4[tid + i * kSplitThreads];
#pragma unroll
        for (int i = 0; i < kPer; ++i) reinterpret_cast<uint4*>(s_hist)[tid + i * kSplitThreads] = hv[i];
    }
    __syncthreads();
    find_digit<kSplitThreads>(s_hist, kHistBins, (uint32_t)keff, scan_lds, dig);
    const uint32_t b1 = dig[0];
    int32_t* ci = a.cand_idx + r * a.N + j0;
    uint32_t* ck = a.cand_key + r * a.N + j0;
    uint32_t* bits = a.bits + r * a.bits_ld;
    uint32_t written = 0;
    for (int64_t js = j0; js < j_end; js += kSplitSub) {
        const int64_t jt = js + 16 * (int64_t)tid;
        if (js > j0) {
#pragma unroll
            for (int u = 0; u < 16; ++u) x[u] = xn[u];
        }
        if (js + kSplitSub < j_end) load(xn, jt + kSplitSub);  // block-uniform
        uint32_t keys[16];
        uint32_t above = 0, eq = 0;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            keys[u] = sort_key(x[u]);
            const bool ok = jt + u < j_end;
            const uint32_t d = keys[u] >> (32 - kHistBits);
            above |= (uint32_t)(ok && d > b1) << u;
            eq |= (uint32_t)(ok && d == b1) << u;
        }
        uint32_t word = above << (16 * (tid & 1));
        word |= (uint32_t)__builtin_amdgcn_ds_swizzle((int)word, (1 << 10) | 0x1f);
        if ((tid & 1) == 0 && jt < j_end) bits[jt >> 5] = word;
        uint32_t total;
        uint32_t off = written + block_exclusive_scan((uint32_t)__popc(eq), scan_lds, &total);
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            if ((eq >> u) & 1u) {
                ci[off] = (int32_t)(jt + u);
                ck[off] = keys[u];
                ++off;
            }
        }
        written += total;
    }
    if (tid == 0) *cnt = written;
}

__global__ __launch_bounds__(kRowThreads) void topk_merge_kernel(TopkArgs a, int64_t len) {
    __shared__ __attribute__((aligned(16))) uint32_t s_hist[kHistBins];
    __shared__ uint32_t s_ckey[kRowCand];
    __shared__ int32_t s_cidx[kRowCand];
    __shared__ uint32_t s_bits[kRowMaxN / 32];
    __shared__ uint32_t s_off[kSplitMaxSlices + 1];
    __shared__ uint32_t scan_lds[kRowThreads / 64 + 1];
    __shared__ uint32_t dig[2];
    const int64_t r = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t nv = topk_row_valid(a, r);
    const int64_t keff = nv < a.k ? nv : a.k;
    int32_t* out = a.idx + r * a.k;
    for (int64_t t = keff + tid; t < a.k; t += kRowThreads) out[t] = -1;
    if (keff == 0) return;
    const int nwords = (int)((nv + 31) / 32);
    const int nslices = (int)((nv + len - 1) / len);

    // 1. the histogram, the slice counts and the bitmap are requested together;
    //    then b1, the count above it and the slices' candidate offsets
    //    (loads batched ahead of their LDS stores: the first 4 bitmap words per
    //    thread, the histogram and the count share one round trip, each further
    //    batch of 4 words takes one)
    static_assert(kHistBins / 4 == kRowThreads, "one uint4 of the histogram per thread");
    auto load_bits = [&](int w0, uint32_t(&bv)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int w = w0 + u * kRowThreads + tid;
            bv[u] = w < nwords ? a.bits[r * a.bits_ld + w] : 0u;
        }
    };
    auto store_bits = [&](int w0, const uint32_t(&bv)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int w = w0 + u * kRowThreads + tid;
            if (w < nwords) s_bits[w] = bv[u];
        }
    };
    uint32_t bv[4];
    load_bits(0, bv);
    const uint32_t c = tid < nslices ? a.slice_cnt[r * a.slices + tid] : 0u;
    const uint4 hv = reinterpret_cast<const uint4*>(a.hist + r * kHistBins)[tid];
    store_bits(0, bv);
    reinterpret_cast<uint4*>(s_hist)[tid] = hv;
    for (int w0 = 4 * kRowThreads; w0 < nwords; w0 += 4 * kRowThreads) {
        load_bits(w0, bv);
        store_bits(w0, bv);
    }
    __syncthreads();
    find_digit<kRowThreads>(s_hist, kHistBins, (uint32_t)keff, scan_lds, dig);
    const uint32_t b1 = dig[0];
    const uint32_t need2 = (uint32_t)keff - dig[1];
    {
        uint32_t total;
        const uint32_t run = block_exclusive_scan(c, scan_lds, &total);
        if (tid < nslices) s_off[tid] = run;
        if (tid == 0) s_off[nslices] = total;
    }
    __syncthreads();
    const uint32_t C = s_off[nslices];
    const bool in_lds = C <= (uint32_t)kRowCand;
    const int32_t* ci = a.cand_idx + r * a.N;
    const uint32_t* ck = a.cand_key + r * a.N;
    // global position of flat candidate p (slice order = index order)
    auto gpos = [&](uint32_t p) -> int64_t {
        int lo = 0, hi = nslices;  // s_off[lo] <= p < s_off[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_off[mid] <= p) lo = mid; else hi = mid;
        }
        return (int64_t)lo * len + (p - s_off[lo]);
    };
    if (in_lds) {
        for (uint32_t p = tid; p < C; p += kRowThreads) {
            const int64_t gp = gpos(p);
            s_ckey[p] = ck[gp];
            s_cidx[p] = ci[gp];
        }
    }
    auto key_at = [&](uint32_t p) -> uint32_t { return in_lds ? s_ckey[p] : ck[gpos(p)]; };
    auto idx_at = [&](uint32_t p) -> int32_t { return in_lds ? s_cidx[p] : ci[gpos(p)]; };
    __syncthreads();

    // 2. digits 2 (bits 19..8) and 3 (bits 7..0) among the candidates (all in bin b1)
    uint32_t prefix = b1 << (32 - kHistBits), need = need2;
    for (int i = tid; i < kHistBins; i += kRowThreads) s_hist[i] = 0;
    __syncthreads();
    for (uint32_t p = tid; p < C; p += kRowThreads) atomicAdd(&s_hist[(key_at(p) >> 8) & 0xfffu], 1u);
    __syncthreads();
    find_digit<kRowThreads>(s_hist, kHistBins, need, scan_lds, dig);
    prefix |= dig[0] << 8;
    need -= dig[1];
    __syncthreads();
    for (int i = tid; i < 256; i += kRowThreads) s_hist[i] = 0;
    __syncthreads();
    for (uint32_t p = tid; p < C; p += kRowThreads) {
        const uint32_t key = key_at(p);
        if ((key & 0xffffff00u) == prefix) atomicAdd(&s_hist[key & 0xffu], 1u);
    }
    __syncthreads();
    find_digit<kRowThreads>(s_hist, 256, need, scan_lds, dig);
    prefix |= dig[0];
    need -= dig[1];
    const uint32_t T = prefix, quota = need;  // take every key > T and `quota` keys == T
    const uint32_t ties = s_hist[T & 0xffu];
    __syncthreads();

    // 3. candidates above T, and the first `quota` equal to T in index order
    if (quota == ties) {
        for (uint32_t p = tid; p < C; p += kRowThreads) {
            const uint32_t key = key_at(p);
            if (key >= T) {
                const int32_t j = idx_at(p);
                atomicOr(&s_bits[j >> 5], 1u << (j & 31));
            }
        }
    } else {
        uint32_t before = 0;
        for (uint32_t p0 = 0; p0 < C; p0 += kRowThreads) {
            const uint32_t p = p0 + tid;
            const uint32_t key = p < C ? key_at(p) : 0u;
            const uint32_t tie = (p < C && key == T) ? 1u : 0u;
            uint32_t n;
            const uint32_t rank = before + block_exclusive_scan(tie, scan_lds, &n);
            if (p < C && (key > T || (tie && rank < quota))) {
                const int32_t j = idx_at(p);
                atomicOr(&s_bits[j >> 5], 1u << (j & 31));
            }
            before += n;
        }
    }
    __syncthreads();

    // 4. ascending output
    const int per = (nwords + kRowThreads - 1) / kRowThreads;
    uint32_t mine = 0;
    for (int wi = tid * per; wi < min(nwords, (tid + 1) * per); ++wi) mine += __popc(s_bits[wi]);
    uint32_t total;
    uint32_t pos = block_exclusive_scan(mine, scan_lds, &total);
    for (int wi = tid * per; wi < min(nwords, (tid + 1) * per); ++wi) {
        uint32_t word = s_bits[wi];
        while (word) {
            const int bit = __ffs(word) - 1;
            word &= word - 1;
            if (pos < (uint32_t)keff) out[pos] = wi * 32 + bit;
            ++pos;
        }
    }
}

hipError_t launch_topk_hist(const TopkArgs& a, hipStream_t stream) {
    if (a.R == 0 || a.N == 0) return hipSuccess;
    dim3 grid((unsigned)a.slices, (unsigned)a.R);
    hipLaunchKernelGGL(topk_hist_kernel, grid, dim3(kSliceThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_topk_select(const TopkArgs& a, hipStream_t stream) {
    if (a.R == 0) return hipSuccess;
    // One workgroup per row while a row is short or there are rows enough to
    // fill the chip: its single pass reads the row on one CU (about 23 GB/s,
    // 11 us at 2^16 entries).  Fewer, longer rows are compacted slice by slice
    // across the chip and then resolved per row.
    // Few rows of moderate length: the pass is spread over many workgroups per
    // row (split path), then one workgroup per row finishes.
    if (a.N <= kRowMaxN && a.N > kSplitMinN && a.R < kRowFill && a.bits) {
        const int64_t len = split_len(a.R, a.N);
        const dim3 grid((unsigned)((a.N + len - 1) / len), (unsigned)a.R);
        hipLaunchKernelGGL(topk_slice_kernel, grid, dim3(kSplitThreads), 0, stream, a, len);
        hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)a.R), dim3(kRowThreads), 0, stream, a, len);
        return hipGetLastError();
    }
    if (a.N <= kRowMaxN && (a.N <= kRowPassN || a.R >= kRowFill)) {
        hipLaunchKernelGGL(topk_row_kernel, dim3((unsigned)a.R), dim3(kRowThreads), 0, stream, a);
        return hipGetLastError();
    }
    if (a.N > 0) {
        dim3 grid((unsigned)a.slices, (unsigned)a.R);
        hipLaunchKernelGGL(topk_compact_kernel, grid, dim3(kSliceThreads), 0, stream, a);
    }
    hipLaunchKernelGGL(topk_final_kernel, dim3((unsigned)a.R), dim3(kFinalThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace csa2
