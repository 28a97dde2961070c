// S2 - Index scores, exact: fp32 round-to-nearest-even of the exact value of
// sum_h sum_e iq[h,e] * ik[j,h,e].
//
// "Why Is DeepSeek V4.1 Flash So Fast?", section 4 (a lightweight indexer scores
// positions before the expensive attention) and "Inference-Efficient LLMs",
// section 5 (scoring every compressed position is the part that grows with the
// context).  In decode this is a pure stream over the index keys and the
// dominant HBM traffic of the step, so the kernel is shaped for bandwidth:
//
//   * 8 lanes share one entry; each lane loads 16-byte chunks at byte offset
//     c*128 + lane8*16, so one wave instruction reads eight 128-byte segments;
//   * every lane keeps its slice of the index query in registers as fp64;
//   * products of two bf16 (or two fp8) values are exact in fp64 and are summed
//     with fp64 FMAs; a 3-step swizzle butterfly finishes each entry.
//
// Exactness:
//   * e4m3: every product is a multiple of 2^-18 of magnitude < 2^17.6, so any
//     partial sum of up to 4096 of them is a multiple of 2^-18 below 2^30 and
//     is exact in fp64's 53 bits.  Rounding the fp64 result once gives the
//     exact answer.
//   * bf16: products of two bf16 values carry only 16 significant bits, so the
//     exact sum lands exactly on an fp32 rounding midpoint surprisingly often
//     (about 2% of N(0,1) scores); correctness therefore rests on proving the
//     fp64 sum exact rather than merely close.  Every product is a multiple of
//     2^L with L = lsb(min|q|) + lsb(min|k|) (bf16 value = M * 2^(E-134)), so if
//     sum|p| < 2^(L+53) every partial sum, in any order, is representable and
//     the fp64 result is the exact sum: rounding it once is the answer, ties
//     included.  The kernel tracks sum|p| (one extra fp64 FMA per element) and
//     the smallest exponent field of k (a packed 16-bit minimum per two
//     elements) per entry.  When that proof fails it falls back to an interval
//     certificate (error <= gamma_(K-1) sum|p| for any order; both ends of
//     [s - bound, s + bound] must round to the same fp32), and when both fail
//     (a tie together with a > 53-bit exponent spread) the entry is recomputed
//     with exact_bf16_dot, an integer long accumulator.
#include "common.h"
#include "launch.h"

namespace csa2 {

constexpr int kScoreThreads = 256;
constexpr int kScoreRounds = 8;                                   // rounds of 8 entries per wave
constexpr int kScoreEntriesPerWave = 8 * kScoreRounds;            // 64
constexpr int kScoreEntriesPerChunk = 4 * kScoreEntriesPerWave;   // 256 per pass of the workgroup
constexpr int kScoreChunks = 1;                                   // passes per workgroup
constexpr int kScoreEntriesPerBlock = kScoreChunks * kScoreEntriesPerChunk;  // 256

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Per-half minimum of two packed 16-bit fields.
CSA2_DEV uint32_t pk_min_u16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}

CSA2_DEV int64_t row_valid(const ScoreArgs& a, int64_t r) {
    if (!a.nvb) return a.N;
    const int64_t b = r / a.Qs, i = r % a.Qs;
    int64_t nv = (int64_t)a.nvb[b] - a.Qs + i + 1;
    return nv < 0 ? 0 : (nv > a.N ? a.N : nv);
}

// Exponent of the least significant bit of any bf16 value whose magnitude is at
// least x (x given as fp32): a bf16 value is M * 2^(E-134), M an integer, E the
// exponent field (taken as 1 for zero and subnormals).
CSA2_DEV int bf16_lsb_exp(float x) {
    const int e = (int)(__float_as_uint(x) >> 23) & 0xff;
    return (e > 0 ? e : 1) - 134;
}

// All products are multiples of 2^L and sum|p| < 2^(L+53): then every partial
// sum in any order is an integer multiple of 2^L below 2^(L+53), hence exact in
// fp64.  sumabs is an fp64 accumulation of sum|p| (relative error < 2^-40 for
// K <= 8192), inflated accordingly.
CSA2_DEV bool sum_is_exact(double sumabs, int L) {
    return sumabs * (1.0 + 0x1p-40) < ldexp(1.0, L + 53);
}

// Exact fp32 (round to nearest even) of sum_i q[i]*k[i] for bf16 q, k, with an
// integer long accumulator.  A bf16 value is (-1)^s * M * 2^(E-134) with
// M = 128+mant for exponent field E >= 1 and M = mant (E taken as 1) for
// subnormals, so a product is (-1)^(s1^s2) * M1*M2 * 2^(E1+E2-268) with
// M1*M2 < 2^16: an integer multiple of 2^-266 placed at bit E1+E2-2.  Digits are
// 32-bit, held in int64 so that carries are settled once at the end.  Every
// digit access uses a compile-time index (unrolled compare/select), so the
// routine lives in registers and the streaming kernel needs no scratch memory.
constexpr int kFixDigits = 20;  // 640 bits: products reach bit 522, sums add 12

CSA2_DEV float exact_bf16_dot(const uint16_t* q, const uint16_t* k, int K) {
    int64_t d[kFixDigits];
#pragma unroll
    for (int j = 0; j < kFixDigits; ++j) d[j] = 0;
    for (int i = 0; i < K; ++i) {
        const uint32_t x = q[i], y = k[i];
        const uint32_t ex = (x >> 7) & 0xff, ey = (y >> 7) & 0xff;
        const uint32_t mx = (x & 0x7f) | (ex ? 0x80u : 0u), my = (y & 0x7f) | (ey ? 0x80u : 0u);
        const int pos = (int)(ex ? ex : 1) + (int)(ey ? ey : 1) - 2;
        const uint64_t v = (uint64_t)(mx * my) << (pos & 31);
        const int li = pos >> 5;
        int64_t lo = (int64_t)(v & 0xffffffffu), hi = (int64_t)(v >> 32);
        if ((x ^ y) & 0x8000u) {
            lo = -lo;
            hi = -hi;
        }
#pragma unroll
        for (int j = 0; j < kFixDigits; ++j) d[j] += (j == li ? lo : 0) + (j == li + 1 ? hi : 0);
    }
    // settle carries (arithmetic shift = floor division by 2^32); the top digit
    // then carries the sign
#pragma unroll
    for (int j = 0; j < kFixDigits - 1; ++j) {
        const int64_t c = d[j] >> 32;
        d[j] -= c * 4294967296LL;
        d[j + 1] += c;
    }
    const bool neg = d[kFixDigits - 1] < 0;
    if (neg) {
#pragma unroll
        for (int j = 0; j < kFixDigits; ++j) d[j] = -d[j];
#pragma unroll
        for (int j = 0; j < kFixDigits - 1; ++j) {
            const int64_t c = d[j] >> 32;
            d[j] -= c * 4294967296LL;
            d[j + 1] += c;
        }
    }
    int ti = -1;  // highest nonzero digit
#pragma unroll
    for (int j = 0; j < kFixDigits; ++j)
        if (d[j] != 0) ti = j;
    if (ti < 0) return 0.0f;  // exact zero is +0
    uint64_t top = 0, mid = 0;
    bool below = false;
#pragma unroll
    for (int j = 0; j < kFixDigits; ++j) {
        top |= j == ti ? (uint64_t)d[j] : 0u;
        mid |= j == ti - 1 ? (uint64_t)d[j] : 0u;
        below |= (j < ti - 1) && d[j] != 0;
    }
    // X holds digits ti and ti-1; its bit 0 weighs 2^base
    const uint64_t X = (top << 32) | mid;
    const int base = 32 * (ti - 1) - 266;
    const int qbit = 63 - __builtin_clzll(X);  // >= 32: digit ti is nonzero
    int lsb_exp = qbit + base - 23;              // fp32 keeps 24 bits ...
    if (lsb_exp < -149) lsb_exp = -149;          // ... none below 2^-149
    const int b = lsb_exp - base;                // >= 9
    const uint64_t mant0 = b >= 64 ? 0 : X >> b;
    const uint32_t rbit = b - 1 >= 64 ? 0u : (uint32_t)((X >> (b - 1)) & 1u);
    const bool sticky = below || (b - 1 >= 64 ? X != 0 : (X & ((1ull << (b - 1)) - 1)) != 0);
    const uint64_t mant = mant0 + ((rbit && (sticky || (mant0 & 1))) ? 1u : 0u);
    const float res = (float)ldexp((double)mant, lsb_exp);  // exact, or inf beyond fp32
    return neg ? -res : res;
}

// DT: 0 = bf16, 1 = e4m3.  CPL: 16-byte chunks per lane per entry, so an entry
// is 128*CPL bytes (bf16: K = 64*CPL, e4m3: K = 128*CPL).
template <int DT, int CPL>
__global__ __launch_bounds__(kScoreThreads) void score_exact_kernel(ScoreArgs a) {
    constexpr int EPC = DT == 0 ? 8 : 16;  // elements per 16-byte chunk
    constexpr int EB = 128 * CPL;         // bytes per entry
    int64_t r, e_block;
    if (a.Qs == 1) {
        r = blockIdx.y;
        e_block = (int64_t)blockIdx.x * kScoreEntriesPerBlock;
    } else {
        // block w takes t = (w % 8) * per_xcd + w / 8: the Qs rows of a sequence
        // for one entry block are consecutive t on one XCD and share its L2
        const int64_t w = blockIdx.x;
        const int64_t t = (w & 7) * a.per_xcd + (w >> 3);
        if (t >= a.blocks) return;
        const int64_t rest = t / a.Qs;
        r = (rest / a.n_eblk) * a.Qs + t % a.Qs;
        e_block = (rest % a.n_eblk) * kScoreEntriesPerBlock;
    }
    const int64_t b = r / a.Qs;
    const int64_t nv = row_valid(a, r);
    if (e_block >= nv) return;

    __shared__ uint32_t lhist[kHistBins];
    const bool with_hist = a.hist != nullptr;
    if (with_hist) {
        for (int i = threadIdx.x; i < kHistBins; i += kScoreThreads) lhist[i] = 0;
    }

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 3, sub = lane & 7;

    // this lane's slice of the index query, as fp64
    double qd[CPL * EPC];
    {
        const uint8_t* qrow = reinterpret_cast<const uint8_t*>(a.iq) + r * (int64_t)EB;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(qrow + c * 128 + sub * 16);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if (DT == 0) {
                    qd[c * EPC + 2 * t] = bf16_lo(w[t]);
                    qd[c * EPC + 2 * t + 1] = bf16_hi(w[t]);
                } else {
                    const auto p0 = __builtin_amdgcn_cvt_pk_f32_fp8(w[t], false);
                    const auto p1 = __builtin_amdgcn_cvt_pk_f32_fp8(w[t], true);
                    qd[c * EPC + 4 * t + 0] = p0[0];
                    qd[c * EPC + 4 * t + 1] = p0[1];
                    qd[c * EPC + 4 * t + 2] = p1[0];
                    qd[c * EPC + 4 * t + 3] = p1[1];
                }
            }
        }
    }
    // |s_fp64 - s| <= gamma_(K-1) * sum|p| (any summation order), and the fp64
    // accumulation of sum|p| itself is low by at most a factor (1 - K*2^-53).
    const double bound_scale = (double)a.K * 0x1p-53 * 1.001 * (1.0 + (double)a.K * 0x1p-52);
    // least significant bit exponent of the smallest |q| of the row (bf16 values are
    // M * 2^(E-134) with integer M; a zero or subnormal gives the floor E = 1)
    int lq = 0;
    if (DT == 0) {
        float qmin = INFINITY;
#pragma unroll
        for (int i = 0; i < CPL * EPC; ++i) qmin = fminf(qmin, fabsf((float)qd[i]));
        qmin = fminf(qmin, swz_xor<1>(qmin));
        qmin = fminf(qmin, swz_xor<2>(qmin));
        qmin = fminf(qmin, swz_xor<4>(qmin));
        lq = bf16_lsb_exp(qmin);
    }

    const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.ik) + b * a.N_cap * (int64_t)EB;
    if (with_hist) __syncthreads();  // histogram zeroed before any chunk adds to it

    for (int chunk = 0; chunk < kScoreChunks; ++chunk) {
        const int64_t e_wave = e_block + chunk * kScoreEntriesPerChunk + wave * kScoreEntriesPerWave;
        if (e_wave >= nv) break;  // wave-uniform
        double keep = 0.0, keep_abs = 0.0;
        uint32_t keep_ex = 0;
#pragma unroll 2
        for (int t = 0; t < kScoreRounds; ++t) {
            const int64_t e = e_wave + t * 8 + g;
            u32x4 w[CPL];
            if (e < nv) {
                const uint8_t* src = kbase + e * EB + sub * 16;
#pragma unroll
                for (int c = 0; c < CPL; ++c)
                    w[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + c * 128));
            } else {
#pragma unroll
                for (int c = 0; c < CPL; ++c) w[c] = u32x4{0u, 0u, 0u, 0u};
            }
            double acc = 0.0, aacc = 0.0;
            uint32_t kex = 0x7fff7fffu;  // packed minimum of the two bf16 exponent fields
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if (DT == 0) {
                        const double lo = bf16_lo(w[c][u]), hi = bf16_hi(w[c][u]);
                        const double q0 = qd[c * EPC + 2 * u], q1 = qd[c * EPC + 2 * u + 1];
                        acc = fma(q0, lo, acc);
                        aacc = fma(fabs(q0), fabs(lo), aacc);
                        acc = fma(q1, hi, acc);
                        aacc = fma(fabs(q1), fabs(hi), aacc);
                        kex = pk_min_u16(kex, w[c][u] & 0x7f807f80u);
                    } else {
                        const auto p0 = __builtin_amdgcn_cvt_pk_f32_fp8(w[c][u], false);
                        const auto p1 = __builtin_amdgcn_cvt_pk_f32_fp8(w[c][u], true);
                        acc = fma(qd[c * EPC + 4 * u + 0], (double)p0[0], acc);
                        acc = fma(qd[c * EPC + 4 * u + 1], (double)p0[1], acc);
                        acc = fma(qd[c * EPC + 4 * u + 2], (double)p1[0], acc);
                        acc = fma(qd[c * EPC + 4 * u + 3], (double)p1[1], acc);
                    }
                }
            }
            acc += swz_xor<1>(acc);
            acc += swz_xor<2>(acc);
            acc += swz_xor<4>(acc);
            if (DT == 0) {
                aacc += swz_xor<1>(aacc);
                aacc += swz_xor<2>(aacc);
                aacc += swz_xor<4>(aacc);
                kex = pk_min_u16(kex, (uint32_t)__builtin_amdgcn_ds_swizzle((int)kex, (1 << 10) | 0x1f));
                kex = pk_min_u16(kex, (uint32_t)__builtin_amdgcn_ds_swizzle((int)kex, (2 << 10) | 0x1f));
                kex = pk_min_u16(kex, (uint32_t)__builtin_amdgcn_ds_swizzle((int)kex, (4 << 10) | 0x1f));
            }
            if (sub == t) {
                keep = acc;
                keep_abs = aacc;
                keep_ex = kex;
            }
        }

        // lane (g, sub) now owns entry e_wave + 8*sub + g
        const int64_t e = e_wave + 8 * sub + g;
        if (e < nv) {
            float res;
            bool ok = true;
            if (DT == 0) {
                res = (float)keep;
                // smallest exponent field among the entry's elements (0 = zero or subnormal)
                const uint32_t ex = min(keep_ex & 0xffffu, keep_ex >> 16) >> 7;
                const int lk = (int)(ex > 0 ? ex : 1u) - 134;
                if (!sum_is_exact(keep_abs, lq + lk)) {
                    const double eb = bound_scale * keep_abs + fabs(keep) * 0x1p-52;
                    const float lo = (float)(keep - eb), hi = (float)(keep + eb);
                    ok = __float_as_uint(lo) == __float_as_uint(hi);
                    res = lo;
                }
            } else {
                res = (float)keep;
            }
            if (!ok)
                res = exact_bf16_dot(reinterpret_cast<const uint16_t*>(a.iq) + r * a.K,
                                     reinterpret_cast<const uint16_t*>(a.ik) + (b * a.N_cap + e) * a.K, a.K);
            a.scores[r * a.ld + e] = res;
            if (with_hist) atomicAdd(&lhist[sort_key(res) >> (32 - kHistBits)], 1u);
        }
    }
    if (with_hist) {
        __syncthreads();
        uint32_t* ghist = a.hist + r * kHistBins;
        for (int i = threadIdx.x; i < kHistBins; i += kScoreThreads) {
            const uint32_t c = lhist[i];
            if (c) atomicAdd(&ghist[i], c);
        }
    }
}

// Fallback for index widths the streaming kernel does not tile: one thread per
// entry, same arithmetic and the same certification.
__global__ __launch_bounds__(256) void score_exact_generic_kernel(ScoreArgs a) {
    const int64_t r = blockIdx.y;
    const int64_t b = r / a.Qs;
    const int64_t nv = row_valid(a, r);
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= nv) return;
    const int K = a.K;
    double acc = 0.0, aacc = 0.0;
    float qmin = INFINITY, kmin = INFINITY;
    if (a.dtype == 0) {
        const uint16_t* q = reinterpret_cast<const uint16_t*>(a.iq) + r * K;
        const uint16_t* k = reinterpret_cast<const uint16_t*>(a.ik) + (b * a.N_cap + e) * K;
        for (int i = 0; i < K; ++i) {
            const float qf = bf16_to_f32(q[i]), kf = bf16_to_f32(k[i]);
            acc = fma((double)qf, (double)kf, acc);
            aacc = fma(fabs((double)qf), fabs((double)kf), aacc);
            qmin = fminf(qmin, fabsf(qf));
            kmin = fminf(kmin, fabsf(kf));
        }
    } else {
        const uint8_t* q = reinterpret_cast<const uint8_t*>(a.iq) + r * K;
        const uint8_t* k = reinterpret_cast<const uint8_t*>(a.ik) + (b * a.N_cap + e) * K;
        for (int i = 0; i < K; ++i) acc = fma(e4m3_to_f64(q[i]), e4m3_to_f64(k[i]), acc);
    }
    float res;
    bool ok = true;
    if (a.dtype == 0) {
        res = (float)acc;
        if (!sum_is_exact(aacc, bf16_lsb_exp(qmin) + bf16_lsb_exp(kmin))) {
            const double eb = (double)K * 0x1p-53 * 1.001 * aacc * (1.0 + K * 0x1p-52) +
                              fabs(acc) * 0x1p-52;
            const float lo = (float)(acc - eb), hi = (float)(acc + eb);
            ok = __float_as_uint(lo) == __float_as_uint(hi);
            res = lo;
        }
    } else {
        res = (float)acc;
    }
    if (!ok)
        res = exact_bf16_dot(reinterpret_cast<const uint16_t*>(a.iq) + r * K,
                             reinterpret_cast<const uint16_t*>(a.ik) + (b * a.N_cap + e) * K, K);
    a.scores[r * a.ld + e] = res;
    if (a.hist) atomicAdd(&a.hist[r * kHistBins + (sort_key(res) >> (32 - kHistBits))], 1u);
}

hipError_t launch_score_exact(const ScoreArgs& args, hipStream_t stream) {
    ScoreArgs a = args;
    const int64_t R = (int64_t)a.B * a.Qs;
    if (R == 0 || a.N == 0) return hipSuccess;
    const int eb = a.K * (a.dtype == 0 ? 2 : 1);
    const int cpl = eb / 128;
    const bool fast = eb % 128 == 0 && (cpl == 1 || cpl == 2 || cpl == 4 || cpl == 8);
    if (fast) {
        a.n_eblk = (a.N + kScoreEntriesPerBlock - 1) / kScoreEntriesPerBlock;
        a.blocks = a.n_eblk * R;
        a.per_xcd = (a.blocks + 7) / 8;
        const dim3 grid = a.Qs == 1 ? dim3((unsigned)a.n_eblk, (unsigned)R) : dim3((unsigned)(8 * a.per_xcd));
        if (a.dtype == 0) {
            if (cpl == 1) hipLaunchKernelGGL((score_exact_kernel<0, 1>), grid, dim3(kScoreThreads), 0, stream, a);
            if (cpl == 2) hipLaunchKernelGGL((score_exact_kernel<0, 2>), grid, dim3(kScoreThreads), 0, stream, a);
            if (cpl == 4) hipLaunchKernelGGL((score_exact_kernel<0, 4>), grid, dim3(kScoreThreads), 0, stream, a);
            if (cpl == 8) hipLaunchKernelGGL((score_exact_kernel<0, 8>), grid, dim3(kScoreThreads), 0, stream, a);
        } else {
            if (cpl == 1) hipLaunchKernelGGL((score_exact_kernel<1, 1>), grid, dim3(kScoreThreads), 0, stream, a);
            if (cpl == 2) hipLaunchKernelGGL((score_exact_kernel<1, 2>), grid, dim3(kScoreThreads), 0, stream, a);
            if (cpl == 4) hipLaunchKernelGGL((score_exact_kernel<1, 4>), grid, dim3(kScoreThreads), 0, stream, a);
            if (cpl == 8) hipLaunchKernelGGL((score_exact_kernel<1, 8>), grid, dim3(kScoreThreads), 0, stream, a);
        }
    } else {
        dim3 grid((unsigned)((a.N + 255) / 256), (unsigned)R);
        hipLaunchKernelGGL(score_exact_generic_kernel, grid, dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace csa2
