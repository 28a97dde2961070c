// S1 - FP4 cache write: fp32 rows -> e2m1 codes + one fp32 scale per 32 elements.
//
// Format ("DeepSeek-V4.1-Flash", "Fast memory, persistent storage and
// recomputation": main cache entries in 4-bit floating point; "Inference-
// Efficient LLMs", section 6: per-group scaling): OCP MX e2m1 elements, block of
// 32, scale = fl32(amax/6), nearest grid point with ties to the even code,
// saturation at 6*scale, element 2i in the low nibble of byte i.
//
// Layout of the work: each lane owns 8 consecutive elements (one uint32 of
// output codes); four lanes form one 32-element block and share its amax with
// two swizzle steps.  A wave therefore covers 16 blocks = 2 KiB of input in one
// coalesced sweep.
#include "common.h"
#include "launch.h"

namespace csa2 {

// Magnitude code on the e2m1 grid {0,.5,1,1.5,2,3,4,6}*s nearest to a >= 0.
// Decision points are the midpoints t*s; a and t*s are exact in fp64, so each
// comparison is exact.  c counts the midpoints strictly below a; a value lying
// exactly on midpoint c (between codes c and c+1) takes the even code.
CSA2_DEV uint32_t e2m1_mag_code(double a, double s) {
    const double t0 = 0.25 * s, t1 = 0.75 * s, t2 = 1.25 * s, t3 = 1.75 * s, t4 = 2.5 * s,
                 t5 = 3.5 * s, t6 = 5.0 * s;
    uint32_t c = (a > t0) + (a > t1) + (a > t2) + (a > t3) + (a > t4) + (a > t5) + (a > t6);
    double tc = c == 0 ? t0 : c == 1 ? t1 : c == 2 ? t2 : c == 3 ? t3 : c == 4 ? t4 : c == 5 ? t5 : t6;
    if (c < 7 && a == tc && (c & 1u)) c += 1;
    return c;
}

// rows: number of rows of x.  Destination row of source row r is
//   dst = r                                  when nvb == nullptr,
//   dst = b*N_cap + nvb[b] - Qs + i          with r = b*Qs + i otherwise
// (the Full-mode write of a step's new rows at slots n_valid-Qs .. n_valid-1).
CSA2_DEV void fp4_pack_lane(int64_t gid, const float* __restrict__ x, int64_t rows, int dim,
                             uint8_t* __restrict__ codes, float* __restrict__ scales,
                             const int32_t* __restrict__ nvb, int Qs, int64_t N_cap) {
    const int lanes_per_row = dim / 8;
    const int64_t total = rows * lanes_per_row;
    // every lane of a 4-lane block group must take part in the swizzles
    const bool active = gid < total;
    const int64_t r = active ? gid / lanes_per_row : 0;
    const int part = (int)(gid % lanes_per_row);  // which 8-element slice of the row
    float v[8];
    if (active) {
        const float4* src = reinterpret_cast<const float4*>(x + r * dim + part * 8);
        float4 a = src[0], b = src[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = fmaxf(amax, swz_xor<1>(amax));
    amax = fmaxf(amax, swz_xor<2>(amax));
    if (!active) return;
    const float scale = amax / 6.0f;  // IEEE division, round to nearest even
    const double s = (double)scale;
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t c = e2m1_mag_code(fabs((double)v[i]), s) | ((__float_as_uint(v[i]) >> 28) & 8u);
        word |= c << (4 * i);
    }
    int64_t dst = r;
    if (nvb) {
        const int64_t b = r / Qs, i = r % Qs;
        const int64_t slot = (int64_t)nvb[b] - Qs + i;
        if (slot < 0 || slot >= N_cap) return;  // n_valid out of range: nothing is written
        dst = b * N_cap + slot;
    }
    reinterpret_cast<uint32_t*>(codes + dst * (dim / 2))[part] = word;
    if ((part & 3) == 0) scales[dst * (dim / 32) + part / 4] = scale;
}

__global__ __launch_bounds__(256) void fp4_pack_kernel(const float* __restrict__ x, int64_t rows,
                                                       int dim, uint8_t* __restrict__ codes,
                                                       float* __restrict__ scales,
                                                       const int32_t* __restrict__ nvb, int Qs,
                                                       int64_t N_cap) {
    fp4_pack_lane((int64_t)blockIdx.x * blockDim.x + threadIdx.x, x, rows, dim, codes, scales, nvb, Qs, N_cap);
}

hipError_t launch_fp4_pack(const float* x, int64_t rows, int dim, uint8_t* codes, float* scales,
                           const int32_t* nvb, int Qs, int64_t N_cap, hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    const int64_t lanes = rows * (dim / 8);
    const int64_t blocks = (lanes + 255) / 256;
    hipLaunchKernelGGL(fp4_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, rows, dim,
                       codes, scales, nvb, Qs, N_cap);
    return hipGetLastError();
}

// Index keys of the new rows go next to their entries (same slot mapping).
CSA2_DEV void store_rows_lane(int64_t gid, const uint32_t* __restrict__ src, int64_t rows, int row_words,
                               uint32_t* __restrict__ dst, const int32_t* __restrict__ nvb, int Qs,
                               int64_t N_cap) {
    if (gid >= rows * row_words) return;
    const int64_t r = gid / row_words, w = gid % row_words;
    int64_t drow = r;
    if (nvb) {
        const int64_t b = r / Qs, i = r % Qs;
        const int64_t slot = (int64_t)nvb[b] - Qs + i;
        if (slot < 0 || slot >= N_cap) return;
        drow = b * N_cap + slot;
    }
    dst[drow * row_words + w] = src[gid];
}

__global__ __launch_bounds__(256) void store_rows_kernel(const uint32_t* __restrict__ src, int64_t rows,
                                                         int row_words, uint32_t* __restrict__ dst,
                                                         const int32_t* __restrict__ nvb, int Qs,
                                                         int64_t N_cap) {
    store_rows_lane((int64_t)blockIdx.x * blockDim.x + threadIdx.x, src, rows, row_words, dst, nvb, Qs, N_cap);
}

hipError_t launch_store_rows(const void* src, int64_t rows, int row_bytes, void* dst,
                             const int32_t* nvb, int Qs, int64_t N_cap, hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    const int words = row_bytes / 4;
    const int64_t blocks = (rows * words + 255) / 256;
    hipLaunchKernelGGL(store_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<const uint32_t*>(src), rows, words,
                       reinterpret_cast<uint32_t*>(dst), nvb, Qs, N_cap);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void zero_kernel(uint32_t* __restrict__ p, int64_t words) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

// A Full layer's writes before scoring, in one launch: the new entries' FP4
// records, their index keys (stored, or FP4-packed with their own scales) and
// the zeroed digit histogram.  Blocks [0, nb_pack) pack entries, the next
// nb_key blocks write keys, the rest zero the histogram.
__global__ __launch_bounds__(256) void full_prep_kernel(FullPrepArgs a) {
    const int64_t blk = blockIdx.x;
    if (blk < a.nb_pack) {
        fp4_pack_lane(blk * 256 + threadIdx.x, a.entry, a.rows, a.D, a.codes, a.scales, a.nvb, a.Qs, a.N_cap);
    } else if (blk < a.nb_pack + a.nb_key) {
        const int64_t gid = (blk - a.nb_pack) * 256 + threadIdx.x;
        if (a.key_fp4)
            fp4_pack_lane(gid, static_cast<const float*>(a.key), a.rows, a.K, static_cast<uint8_t*>(a.ikeys),
                          a.ikey_scales, a.nvb, a.Qs, a.N_cap);
        else
            store_rows_lane(gid, static_cast<const uint32_t*>(a.key), a.rows, a.key_words,
                            static_cast<uint32_t*>(a.ikeys), a.nvb, a.Qs, a.N_cap);
    } else {
        const int64_t first = blk - a.nb_pack - a.nb_key, nz = gridDim.x - a.nb_pack - a.nb_key;
        for (int64_t i = first * 256 + threadIdx.x; i < a.zero_words; i += nz * 256) a.zero[i] = 0u;
    }
}

hipError_t launch_full_prep(const FullPrepArgs& args, hipStream_t stream) {
    FullPrepArgs a = args;
    a.nb_pack = (a.rows * (a.D / 8) + 255) / 256;
    a.nb_key = a.key_fp4 ? (a.rows * (a.K / 8) + 255) / 256 : (a.rows * a.key_words + 255) / 256;
    int64_t nz = (a.zero_words + 255) / 256;
    if (nz > 1024) nz = 1024;
    if (nz < 1) nz = 1;
    const int64_t blocks = a.nb_pack + a.nb_key + nz;
    hipLaunchKernelGGL(full_prep_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_zero(uint32_t* p, int64_t words, hipStream_t stream) {
    if (words == 0) return hipSuccess;
    int64_t blocks = (words + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, words);
    return hipGetLastError();
}

}  // namespace csa2
