// Hierarchical search helpers ("Inference-Efficient LLMs", section 5,
// Hierarchical Sparse Indexing): a Full layer keeps a pool of blocks of 8
// consecutive positions, ranked by their largest index score, and Reindex
// layers score and rank only the pool's positions.
//
//   * block_max_kernel: the block scores a Full layer ranks (one thread per
//     block, 32 bytes of scores each);
//   * pool_count_kernel: the number of leading pool slots whose position is
//     valid (one workgroup per row, a minimum over each block's first invalid
//     slot);
//   * pool_map_kernel: a selection of pool slots becomes a selection of
//     positions.
// The ranking itself is the ordinary top-k (topk.hip) on block scores or on the
// pool's scores; the pool's scores come from score_exact_kernel in pool mode.
#include "common.h"
#include "launch.h"

namespace csa2 {

namespace {

CSA2_DEV int64_t causal_valid(const int32_t* nvb, int Qs, int64_t N, int64_t r) {
    if (!nvb) return N;
    const int64_t b = r / Qs, i = r % Qs;
    const int64_t nv = (int64_t)nvb[b] - Qs + i + 1;
    return nv < 0 ? 0 : (nv > N ? N : nv);
}

__global__ __launch_bounds__(256) void block_max_kernel(const float* scores, int64_t N, int64_t ld,
                                                        const int32_t* nvb, int Qs, float* bmax,
                                                        int64_t ld_blk, int32_t* blk_nv) {
    const int64_t r = blockIdx.y;
    const int64_t nv = causal_valid(nvb, Qs, N, r);
    const int64_t nb = (nv + kPoolBlock - 1) / kPoolBlock;
    if (blockIdx.x == 0 && threadIdx.x == 0) blk_nv[r] = (int32_t)nb;
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (j >= nb) return;
    const float* s = scores + r * ld + j * kPoolBlock;
    const int64_t n = nv - j * kPoolBlock < kPoolBlock ? nv - j * kPoolBlock : kPoolBlock;
    float m = s[0];
#pragma unroll
    for (int t = 1; t < kPoolBlock; ++t) {
        if (t < n) {
            const float x = s[t];
            if (x > m) m = x;
        }
    }
    bmax[r * ld_blk + j] = m;
}

__global__ __launch_bounds__(256) void pool_count_kernel(const int32_t* pool, int P, const int32_t* nvb,
                                                         int Qs, int32_t* pool_nv) {
    const int64_t r = blockIdx.x;
    const int64_t nv = causal_valid(nvb, Qs, INT64_MAX, r);
    const int32_t* row = pool + r * P;
    int first = P * kPoolBlock;  // first slot whose position is not valid
#pragma unroll 8
    for (int j = threadIdx.x; j < P; j += 256) {
        // block j's slots 8j .. 8j+7 hold positions 8*blk .. 8*blk+7
        const int32_t blk = row[j];
        const int64_t room = blk < 0 ? 0 : nv - (int64_t)blk * kPoolBlock;
        if (room < kPoolBlock) first = min(first, j * kPoolBlock + (int)(room > 0 ? room : 0));
    }
    __shared__ int red[4];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) first = min(first, __shfl_xor(first, m));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = first;
    __syncthreads();
    if (threadIdx.x == 0) pool_nv[r] = min(min(red[0], red[1]), min(red[2], red[3]));
}

__global__ __launch_bounds__(256) void pool_map_kernel(int32_t* idx, int64_t total, int k, const int32_t* pool,
                                                       int P) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const int32_t s = idx[i];
    if (s < 0) return;
    const int64_t r = i / k;
    idx[i] = pool[r * P + s / kPoolBlock] * kPoolBlock + s % kPoolBlock;
}

}  // namespace

hipError_t launch_block_max(const float* scores, int64_t R, int64_t N, int64_t ld, const int32_t* nvb,
                            int Qs, float* bmax, int64_t ld_blk, int32_t* blk_nv, hipStream_t stream) {
    if (R == 0) return hipSuccess;
    const int64_t nb = (N + kPoolBlock - 1) / kPoolBlock;
    dim3 grid((unsigned)((nb + 255) / 256 > 0 ? (nb + 255) / 256 : 1), (unsigned)R);
    hipLaunchKernelGGL(block_max_kernel, grid, dim3(256), 0, stream, scores, N, ld, nvb, Qs, bmax, ld_blk,
                       blk_nv);
    return hipGetLastError();
}

hipError_t launch_pool_count(const int32_t* pool, int64_t R, int P, const int32_t* nvb, int Qs,
                             int32_t* pool_nv, hipStream_t stream) {
    if (R == 0) return hipSuccess;
    hipLaunchKernelGGL(pool_count_kernel, dim3((unsigned)R), dim3(256), 0, stream, pool, P, nvb, Qs, pool_nv);
    return hipGetLastError();
}

hipError_t launch_pool_map(int32_t* idx, int64_t R, int k, const int32_t* pool, int P, hipStream_t stream) {
    const int64_t total = R * k;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(pool_map_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, idx, total,
                       k, pool, P);
    return hipGetLastError();
}

}  // namespace csa2
