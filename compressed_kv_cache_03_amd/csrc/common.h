// Device helpers shared by the CSA2 HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define CSA2_DEV static __device__ __forceinline__
#define CSA2_DEV_HOST_INLINE static __host__ __device__ __forceinline__

namespace csa2 {

constexpr int kWave = 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kHistBits = 12;             // first radix digit: top 12 bits of the sort key
static_assert(kHistBits == 12, "host workspace sizing assumes 4096 bins");
constexpr int kHistBins = 1 << kHistBits;  // 4096

// bf16 bit pattern -> fp32 (exact).
CSA2_DEV float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
CSA2_DEV float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
CSA2_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// OCP fp8 e4m3fn byte -> fp64, exact, by field arithmetic (bias 7; exponent
// field 0 holds the subnormals m * 2^-9).  NaN (S.1111.111) is not produced
// for finite inputs and is not handled.
CSA2_DEV double e4m3_to_f64(uint32_t b) {
    uint32_t e = (b >> 3) & 15u, m = b & 7u;
    double mag = e ? __longlong_as_double((long long)(((uint64_t)(e + 1016u) << 52) | ((uint64_t)m << 49)))
                   : (double)m * 0x1p-9;
    return (b & 0x80u) ? -mag : mag;
}

// Order-preserving map fp32 -> uint32: a > b (as reals) <=> key(a) > key(b).
// -0 is mapped like +0 so the two compare equal.
CSA2_DEV uint32_t sort_key(float s) {
    uint32_t u = __float_as_uint(s);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Butterfly exchange inside groups of 32 lanes (ds_swizzle, bitmask mode).
template <int XOR>
CSA2_DEV float swz_xor(float v) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (XOR << 10) | 0x1f));
}
template <int XOR>
CSA2_DEV double swz_xor(double v) {
    int2 p = *reinterpret_cast<int2*>(&v);
    p.x = __builtin_amdgcn_ds_swizzle(p.x, (XOR << 10) | 0x1f);
    p.y = __builtin_amdgcn_ds_swizzle(p.y, (XOR << 10) | 0x1f);
    return *reinterpret_cast<double*>(&p);
}

// Inclusive prefix sum over the 64 lanes of a wave: DPP row shifts by 1, 2, 4
// and 8 (a lane with no source in its 16-lane row adds 0) give the sums inside
// each row, then every row adds the totals of the rows below it, read from
// lanes 15, 31 and 47.
CSA2_DEV uint32_t wave_inclusive_scan(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);  // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);  // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true);  // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true);  // row_shr:8
    const uint32_t t0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 15);
    const uint32_t t1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 31);
    const uint32_t t2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 47);
    const int row = (threadIdx.x & 63) >> 4;
    return x + (row >= 1 ? t0 : 0u) + (row >= 2 ? t1 : 0u) + (row >= 3 ? t2 : 0u);
}

// Block-wide exclusive prefix sum of one uint32 per thread (blockDim.x <= 1024,
// a multiple of 64).  `lds` must hold blockDim.x/64 + 1 words.  Returns the
// exclusive prefix; *total receives the block sum.  Every thread adds the wave
// totals itself (broadcast LDS reads), so there is no serial step.  Contains
// barriers.
CSA2_DEV uint32_t block_exclusive_scan(uint32_t v, uint32_t* lds, uint32_t* total) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const uint32_t x = wave_inclusive_scan(v);
    if (lane == 63) lds[wid] = x;
    __syncthreads();
    uint32_t before = 0, all = 0;
    for (int w = 0; w < nw; ++w) {
        const uint32_t t = lds[w];
        before += w < wid ? t : 0u;
        all += t;
    }
    *total = all;
    __syncthreads();  // the words are read before a later call overwrites them
    return before + x - v;
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

}  // namespace csa2
