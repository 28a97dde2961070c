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

hipError_t launch_topk_hist(const TopkArgs& a, hipStream_t stream) {
    if (a.R == 0 || a.N == 0) return hipSuccess;
    dim3 grid((unsigned)a.slices, (unsigned)a.R);
    hipLaunchKernelGGL(topk_hist_kernel, grid, dim3(kSliceThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_topk_select(const TopkArgs& a, hipStream_t stream) {
    if (a.R == 0) return hipSuccess;
    if (a.N > 0) {
        dim3 grid((unsigned)a.slices, (unsigned)a.R);
        hipLaunchKernelGGL(topk_compact_kernel, grid, dim3(kSliceThreads), 0, stream, a);
    }
    hipLaunchKernelGGL(topk_final_kernel, dim3((unsigned)a.R), dim3(kFinalThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace csa2
