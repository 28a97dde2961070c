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
//   2. topk_compact_kernel: every 4096-entry slice of a row finds the bin b1 in
//      which the k-th largest key falls and writes, in index order, the
//      entries whose digit is >= b1 to its own segment of a candidate buffer;
//   3. topk_final_kernel: one workgroup per row walks the candidates (slice
//      order = index order), resolves digit 2 (bits 19..8) and digit 3 (bits
//      7..0) among those in bin b1 to the exact k-th key T and the number of
//      entries equal to T still to take, then writes the selection in index
//      order: every key > T, and the first `quota` keys == T (lowest indices).
// Every decision is an integer comparison of keys, so the result is identical
// to sorting with the stated order.
#include "common.h"
#include "launch.h"

namespace csa2 {

constexpr int kSliceThreads = 256;
constexpr int kSliceLen = 4096;  // entries per compaction workgroup (16 per thread)
constexpr int kFinalThreads = 1024;

int64_t topk_slice_len(int64_t) { return kSliceLen; }

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
    const int64_t j0 = (int64_t)blockIdx.x * kSliceLen;
    if (j0 >= nv) return;
    for (int i = threadIdx.x; i < kHistBins; i += kSliceThreads) lh[i] = 0;
    __syncthreads();
    const float* s = a.scores + r * a.ld;
    const int64_t j1 = j0 + kSliceLen < nv ? j0 + kSliceLen : nv;
    for (int64_t j = j0 + threadIdx.x; j < j1; j += kSliceThreads)
        atomicAdd(&lh[sort_key(s[j]) >> (32 - kHistBits)], 1u);
    __syncthreads();
    uint32_t* gh = a.hist + r * kHistBins;
    for (int i = threadIdx.x; i < kHistBins; i += kSliceThreads)
        if (lh[i]) atomicAdd(&gh[i], lh[i]);
}

// Find, within a histogram of `nbins` bins (highest bin = largest keys), the
// bin holding the `need`-th largest element: the largest b with
// sum_{b' >= b} h[b'] >= need.  Writes b and the count strictly above b to
// out[0], out[1].  need >= 1 and sum h >= need are required.  All threads of
// the block must call it; h may live in global or shared memory.
template <int THREADS>
CSA2_DEV void find_digit(const uint32_t* h, int nbins, uint32_t need, uint32_t* scan_lds,
                         uint32_t* out) {
    if (threadIdx.x == 0) {
        out[0] = 0;
        out[1] = 0;
    }
    const int per = (nbins + THREADS - 1) / THREADS;
    // thread t owns bins [nbins - per*(t+1), nbins - per*t), i.e. thread 0 the top
    const int hi = nbins - per * (int)threadIdx.x;
    const int lo = hi - per;
    uint32_t local = 0;
    for (int bin = hi - 1; bin >= lo && bin >= 0; --bin) local += h[bin];
    uint32_t total;
    const uint32_t before = block_exclusive_scan(local, scan_lds, &total);
    if (before < need && before + local >= need) {
        uint32_t run = before;
        for (int bin = hi - 1; bin >= lo && bin >= 0; --bin) {
            const uint32_t c = h[bin];
            if (run + c >= need) {
                out[0] = (uint32_t)bin;
                out[1] = run;
                break;
            }
            run += c;
        }
    }
    __syncthreads();
}

__global__ __launch_bounds__(kSliceThreads) void topk_compact_kernel(TopkArgs a) {
    __shared__ uint32_t scan_lds[kSliceThreads / 64 + 1];
    __shared__ uint32_t dig[2];
    const int64_t r = blockIdx.y;
    const int64_t nv = topk_row_valid(a, r);
    const int64_t keff = nv < a.k ? nv : a.k;
    const int64_t j0 = (int64_t)blockIdx.x * kSliceLen;
    uint32_t* cnt = a.slice_cnt + r * a.slices + blockIdx.x;
    if (j0 >= nv || keff == 0) {
        if (threadIdx.x == 0) *cnt = 0;
        return;
    }
    find_digit<kSliceThreads>(a.hist + r * kHistBins, kHistBins, (uint32_t)keff, scan_lds, dig);
    const uint32_t b1 = dig[0];

    // thread t scans entries j0 + 16t .. j0 + 16t + 15 in order
    const float* s = a.scores + r * a.ld;
    const int64_t jt = j0 + 16 * (int64_t)threadIdx.x;
    uint32_t keys[16];
    uint32_t mine = 0;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        const int64_t j = jt + u;
        keys[u] = j < nv ? sort_key(s[j]) : 0u;
        const bool take = j < nv && (keys[u] >> (32 - kHistBits)) >= b1;
        mine |= (uint32_t)take << u;
    }
    uint32_t total;
    uint32_t off = block_exclusive_scan(__popc(mine), scan_lds, &total);
    int32_t* ci = a.cand_idx + r * a.N + j0;
    uint32_t* ck = a.cand_key + r * a.N + j0;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        if (mine >> u & 1u) {
            ci[off] = (int32_t)(jt + u);
            ck[off] = keys[u];
            ++off;
        }
    }
    if (threadIdx.x == 0) *cnt = total;
}

__global__ __launch_bounds__(kFinalThreads) void topk_final_kernel(TopkArgs a) {
    __shared__ uint32_t scan_lds[kFinalThreads / 64 + 1];
    __shared__ uint32_t h2[kHistBins];
    __shared__ uint32_t dig[2];
    const int64_t r = blockIdx.x;
    const int64_t nv = topk_row_valid(a, r);
    const int64_t keff = nv < a.k ? nv : a.k;
    int32_t* out = a.idx + r * a.k;
    for (int64_t t = keff + threadIdx.x; t < a.k; t += kFinalThreads) out[t] = -1;
    if (keff == 0) return;

    find_digit<kFinalThreads>(a.hist + r * kHistBins, kHistBins, (uint32_t)keff, scan_lds, dig);
    const uint32_t b1 = dig[0];
    const uint32_t need1 = (uint32_t)keff - dig[1];  // still to take from bin b1
    const int nslices = (int)((nv + kSliceLen - 1) / kSliceLen);
    const uint32_t* cnts = a.slice_cnt + r * a.slices;
    const int32_t* ci = a.cand_idx + r * a.N;
    const uint32_t* ck = a.cand_key + r * a.N;

    // digit 2 among candidates of bin b1
    for (int i = threadIdx.x; i < kHistBins; i += kFinalThreads) h2[i] = 0;
    __syncthreads();
    for (int sl = 0; sl < nslices; ++sl) {
        const uint32_t c = cnts[sl];
        for (uint32_t t = threadIdx.x; t < c; t += kFinalThreads) {
            const uint32_t key = ck[(int64_t)sl * kSliceLen + t];
            if ((key >> 20) == b1) atomicAdd(&h2[(key >> 8) & 0xfffu], 1u);
        }
    }
    __syncthreads();
    find_digit<kFinalThreads>(h2, kHistBins, need1, scan_lds, dig);
    const uint32_t b2 = dig[0];
    const uint32_t need2 = need1 - dig[1];
    const uint32_t pre2 = (b1 << 12) | b2;  // key bits 31..8

    // digit 3 among candidates with bits 31..8 == pre2
    for (int i = threadIdx.x; i < 256; i += kFinalThreads) h2[i] = 0;
    __syncthreads();
    for (int sl = 0; sl < nslices; ++sl) {
        const uint32_t c = cnts[sl];
        for (uint32_t t = threadIdx.x; t < c; t += kFinalThreads) {
            const uint32_t key = ck[(int64_t)sl * kSliceLen + t];
            if ((key >> 8) == pre2) atomicAdd(&h2[key & 0xffu], 1u);
        }
    }
    __syncthreads();
    find_digit<kFinalThreads>(h2, 256, need2, scan_lds, dig);
    const uint32_t T = (pre2 << 8) | dig[0];
    const uint32_t quota = need2 - dig[1];  // keys equal to T still to take

    // ordered output: keys > T, plus the first `quota` keys == T
    uint32_t ties_before = 0, written = 0;
    for (int sl = 0; sl < nslices; ++sl) {
        const uint32_t c = cnts[sl];
        for (uint32_t t0 = 0; t0 < c; t0 += kFinalThreads) {
            const uint32_t t = t0 + threadIdx.x;
            uint32_t key = 0;
            int32_t j = -1;
            if (t < c) {
                key = ck[(int64_t)sl * kSliceLen + t];
                j = ci[(int64_t)sl * kSliceLen + t];
            }
            const uint32_t tie = (t < c && key == T) ? 1u : 0u;
            uint32_t ntie;
            const uint32_t tie_rank = ties_before + block_exclusive_scan(tie, scan_lds, &ntie);
            const uint32_t sel = (t < c && (key > T || (tie && tie_rank < quota))) ? 1u : 0u;
            uint32_t nsel;
            const uint32_t pos = written + block_exclusive_scan(sel, scan_lds, &nsel);
            if (sel && pos < (uint32_t)keff) out[pos] = j;
            ties_before += ntie;
            written += nsel;
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
    if (a.N > 0) {
        dim3 grid((unsigned)a.slices, (unsigned)a.R);
        hipLaunchKernelGGL(topk_compact_kernel, grid, dim3(kSliceThreads), 0, stream, a);
    }
    hipLaunchKernelGGL(topk_final_kernel, dim3((unsigned)a.R), dim3(kFinalThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace csa2
