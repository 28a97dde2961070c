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
//   * every lane keeps its slice of the index query in registers (fp64; bf16
//     queries as fp32);
//   * products of two fp8 values are exact in fp64 and are summed with fp64
//     FMAs; products of two bf16 values (16 significant bits) are formed exactly
//     in fp32 and summed in fp64; a 3-step DPP butterfly finishes each entry;
//   * a workgroup of 8 waves takes one 512-entry block of one row; with e4m3
//     keys (K = 256) and one query row per sequence the workgroups instead stay
//     resident, one per CU, each streaming a run of its row's blocks with the
//     key loads running ahead across block boundaries.
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
//     2^L with L = lsb(min|q|) + lsb(min|k|) (bf16 value = M * 2^(E-134)); with
//     L >= -149 and every |p| below 2^128 each fp32 product is exact (with
//     L < -149 each is within 2^-150 of exact, which the interval below
//     absorbs).  If sum|p| < 2^(L+53) every partial sum, in any order, is
//     representable and the fp64 result is the exact sum: rounding it once is
//     the answer, ties included.  sum|p| is bounded by sum|q| * max|k|: the kernel tracks the
//     smallest and the largest exponent field of k (packed 16-bit minimum and
//     maximum per two elements) per entry.  When that proof fails it falls
//     back to an interval certificate (error <= gamma_(K-1) sum|p| for any
//     order; both ends of [s - bound, s + bound] must round to the same fp32),
//     and when both fail (a tie together with a > 53-bit exponent spread), or a
//     product may leave fp32's range, the entry is recomputed with an integer
//     long accumulator.
//   * FP4 keys (e2m1 code times an fp32 scale per 32-element block, bf16
//     queries): each lane sums its block's 32 products q * e2m1 in fp64, exact
//     whenever the query block's exponent spread allows (a per-row property
//     decided once per lane, else bounded by gamma_32 * 6 * sum|q|), then adds
//     block sum * scale with one fma.  The rounding of those fmas and of the
//     butterfly is bounded by (CPL + 3) * 2^-53 * sum |block sum * scale|, and
//     both ends of the resulting interval must round to the same fp32.
//   * The rare entries the certificate cannot decide are recomputed by the
//     whole wave at once: each lane accumulates K/64 exact products into its
//     own 640-bit integer accumulator, the accumulators are summed across the
//     wave, and the total is rounded once.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace csa2 {

constexpr int kScoreThreads = 256;  // workgroup of the multi-row scorer and the fixup
constexpr int kScoreRounds = 8;                                   // rounds of 8 entries per wave
constexpr int kScoreEntriesPerWave = 8 * kScoreRounds;            // 64
// The single-row stream runs 8 waves per workgroup: 512 entries share one LDS
// histogram, which halves the workgroups that flush one to global memory.
constexpr int kStreamThreads = 512;
constexpr int kScoreEntriesPerChunk = (kStreamThreads / 64) * kScoreEntriesPerWave;  // 512 per pass of the workgroup
constexpr int kScoreChunks = 1;                                   // passes per workgroup
constexpr int kScoreEntriesPerBlock = kScoreChunks * kScoreEntriesPerChunk;  // 512
// Persistent single-row stream (e4m3 keys, K = 256): one workgroup of 8 waves per
// CU (its 152 VGPRs leave room for no second one), each streaming a run of its
// row's 512-entry blocks with the key ring running on across them.
constexpr int64_t kPersistResident = 256;

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Cross-lane partner reads on DPP (VALU, no LDS round trip).  Applied in the
// order S = 1, 2, 4, 8 they all-reduce within groups of 8 (or 16) lanes: the two
// quad permutes pair xor 1 and xor 2, then the mirror of each 8-lane half pairs
// its two quads, and the mirror of the 16-lane row its two halves.
template <int S>
CSA2_DEV uint32_t dpp_u32(uint32_t v) {
    constexpr int kCtrl = S == 1 ? 0xB1 : S == 2 ? 0x4E : S == 4 ? 0x141 : 0x140;
    static_assert(S == 1 || S == 2 || S == 4 || S == 8, "a pairing of the reduction");
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kCtrl, 0xf, 0xf, false);
}
template <int S>
CSA2_DEV double dpp_f64(double v) {
    uint2 p = __builtin_bit_cast(uint2, v);
    p.x = dpp_u32<S>(p.x);
    p.y = dpp_u32<S>(p.y);
    return __builtin_bit_cast(double, p);
}

// Maximum over each 16-lane row, in every lane of the row.
CSA2_DEV uint32_t wave_row_max(uint32_t v) {
    v = max(v, dpp_u32<1>(v));
    v = max(v, dpp_u32<2>(v));
    v = max(v, dpp_u32<4>(v));
    return max(v, dpp_u32<8>(v));
}

CSA2_DEV uint32_t pk_max_u16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}

// Per-half minimum of two packed 16-bit fields.
CSA2_DEV uint32_t pk_min_u16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}

CSA2_DEV int64_t row_valid(const ScoreArgs& a, int64_t r) {
    if (a.pool) {
        const int64_t v = a.pool_nv[r];
        return v < 0 ? 0 : (v > a.N ? a.N : v);
    }
    if (!a.nvb) {
        if (a.causal < 0) return a.N;
        const int64_t nv = a.causal + r % a.Qs + 1;
        return nv > a.N ? a.N : nv;
    }
    const int64_t b = r / a.Qs, i = r % a.Qs;
    int64_t nv = (int64_t)a.nvb[b] - a.Qs + i + 1;
    return nv < 0 ? 0 : (nv > a.N ? a.N : nv);
}

// Position scored at slot s of row r: s itself, or in pool mode position
// 8 * pool[r][s / 8] + s % 8 (a round of 8 slots is one pool block).
CSA2_DEV int64_t slot_entry(const ScoreArgs& a, int64_t r, int64_t s) {
    return a.pool ? (int64_t)a.pool[r * a.pool_blocks + (s >> 3)] * kPoolBlock + (s & 7) : s;
}

// Exponent of the least significant bit of any bf16 value whose magnitude is at
// least x (x given as fp32): a bf16 value is M * 2^(E-134), M an integer, E the
// exponent field (taken as 1 for zero and subnormals).
typedef float f32x2 __attribute__((ext_vector_type(2)));

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

// Settle the carries of a digit accumulator whose bit 0 weighs 2^lsb0 and
// round its value to fp32 (nearest even; an exact zero is +0).
CSA2_DEV float fix_to_f32(int64_t (&d)[kFixDigits], int lsb0) {
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
    const int base = 32 * (ti - 1) + lsb0;
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

// Adds the exact product of bf16 values x and y to the digit accumulator.
CSA2_DEV void bf16_accum(int64_t (&d)[kFixDigits], uint32_t x, uint32_t y) {
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

// Sums every lane's digit accumulator into all lanes of the wave.  Each lane's
// digits stay below 2^32 * (K/64 + 3) in magnitude, so the sum of 64 of them
// fits an int64 digit.
CSA2_DEV void wave_sum_digits(int64_t (&d)[kFixDigits]) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
#pragma unroll
        for (int j = 0; j < kFixDigits; ++j) d[j] += __shfl_xor((long)d[j], m);
    }
}

CSA2_DEV float exact_bf16_dot(const uint16_t* q, const uint16_t* k, int K) {
    int64_t d[kFixDigits];
#pragma unroll
    for (int j = 0; j < kFixDigits; ++j) d[j] = 0;
    for (int i = 0; i < K; ++i) bf16_accum(d, q[i], k[i]);
    return fix_to_f32(d, -266);
}

// exact_bf16_dot computed by a whole wave (all 64 lanes active, same arguments
// in every lane): lane l takes elements l, l+64, ...; every lane returns the
// result.
CSA2_DEV float wave_exact_bf16_dot(const uint16_t* q, const uint16_t* k, int K, int lane) {
    int64_t d[kFixDigits];
#pragma unroll
    for (int j = 0; j < kFixDigits; ++j) d[j] = 0;
    for (int i = lane; i < K; i += 64) bf16_accum(d, q[i], k[i]);
    wave_sum_digits(d);
    return fix_to_f32(d, -266);
}

// Exact fp32 (RNE) of sum_i q[i] * v[i] for bf16 q and FP4 keys, v[i] = the e2m1
// value of code i times the fp32 scale of its 32-element block.  With
// q = Mq 2^(Eq-134), |e2m1| = Mc 2^Ec (Mc in {0, 1, 3}, Ec in -1..2) and
// scale = Ms 2^(Es-150), a product is Mq*Mc*Ms 2^(Eq+Ec+Es-284) with
// Mq*Mc*Ms < 2^34: an integer multiple of 2^-288 placed at bit Eq+Ec+Es+4.  Same
// 640-bit accumulator and final rounding as exact_bf16_dot.
// Adds the exact product of bf16 x, e2m1 code nib and fp32 scale bits sb.
CSA2_DEV void fp4_accum(int64_t (&d)[kFixDigits], uint32_t x, uint32_t nib, uint32_t sb) {
    const uint32_t ex = (x >> 7) & 0xff, es = (sb >> 23) & 0xff, cm = nib & 7u;
    const uint32_t mx = (x & 0x7f) | (ex ? 0x80u : 0u);
    const uint32_t ms = (sb & 0x7fffffu) | (es ? 0x800000u : 0u);
    // e2m1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 as Mc * 2^Ec (Ec + 1 stored)
    const uint32_t mc = cm == 0 ? 0u : ((cm & 1u) && cm > 1 ? 3u : 1u);
    const int ec1 = cm < 2 ? 0 : (int)(cm >> 1) - (int)(cm & 1u);  // Ec + 1
    const uint64_t M = (uint64_t)(mx * mc) * ms;
    if (M == 0) return;
    const int pos = (int)(ex ? ex : 1) + ec1 + (int)(es ? es : 1) + 3;
    const unsigned __int128 v = (unsigned __int128)M << (pos & 31);
    int64_t d0 = (int64_t)(uint64_t)(v & 0xffffffffu), d1 = (int64_t)(uint64_t)((v >> 32) & 0xffffffffu),
            d2 = (int64_t)(uint64_t)(v >> 64);
    if (((x >> 15) ^ (nib >> 3) ^ (sb >> 31)) & 1u) {
        d0 = -d0;
        d1 = -d1;
        d2 = -d2;
    }
    const int li = pos >> 5;
#pragma unroll
    for (int j = 0; j < kFixDigits; ++j)
        d[j] += (j == li ? d0 : 0) + (j == li + 1 ? d1 : 0) + (j == li + 2 ? d2 : 0);
}

CSA2_DEV float exact_fp4_dot(const uint16_t* q, const uint8_t* codes, const float* scales, int K) {
    int64_t d[kFixDigits];
#pragma unroll
    for (int j = 0; j < kFixDigits; ++j) d[j] = 0;
    for (int i = 0; i < K; ++i)
        fp4_accum(d, q[i], (codes[i >> 1] >> (4 * (i & 1))) & 15u, __float_as_uint(scales[i >> 5]));
    return fix_to_f32(d, -288);
}

// exact_fp4_dot computed by a whole wave, as wave_exact_bf16_dot.
CSA2_DEV float wave_exact_fp4_dot(const uint16_t* q, const uint8_t* codes, const float* scales, int K,
                                  int lane) {
    int64_t d[kFixDigits];
#pragma unroll
    for (int j = 0; j < kFixDigits; ++j) d[j] = 0;
    for (int i = lane; i < K; i += 64)
        fp4_accum(d, q[i], (codes[i >> 1] >> (4 * (i & 1))) & 15u, __float_as_uint(scales[i >> 5]));
    wave_sum_digits(d);
    return fix_to_f32(d, -288);
}

// wave_exact_fp4_dot for K = 256 with every lane's loads issued before the
// accumulation (lane l: elements l, l+64, l+128, l+192).
CSA2_DEV float wave_exact_fp4_256(const uint16_t* q, const uint8_t* codes, const float* scales, int lane) {
    uint32_t qx[4], nib[4], sb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int i = lane + 64 * u;
        qx[u] = q[i];
        nib[u] = codes[i >> 1];
        sb[u] = __float_as_uint(scales[i >> 5]);
    }
    int64_t d[kFixDigits];
#pragma unroll
    for (int j = 0; j < kFixDigits; ++j) d[j] = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) fp4_accum(d, qx[u], (nib[u] >> (4 * (lane & 1))) & 15u, sb[u]);
    wave_sum_digits(d);
    return fix_to_f32(d, -288);
}

// Bound on the error of a block sum of 32 products q * e2m1 accumulated with fp64
// FMAs: zero when the sum is provably exact, else gamma_32 * 6 * sum|q|.  Every
// product is a multiple of 2^(emin - 135) (bf16 lsb 2^(E-134), e2m1 lsb 2^-1), so
// if 6 * sum|q| < 2^(emin - 135 + 53) each partial sum is representable.  emin is
// the smallest exponent field (1 for subnormals) over the block's nonzero q;
// emin > 255 means every q is zero.
CSA2_DEV double fp4_block_err(double qn1, int emin) {
    if (emin > 255 || 6.0 * qn1 * (1.0 + 0x1p-40) < ldexp(1.0, emin - 135 + 53)) return 0.0;
    return 32.0 * 0x1p-53 * 1.001 * 6.0 * qn1;
}

// Smallest exponent field of the nonzero bf16 values packed in w (1 for
// subnormals, 1 << 20 when both are zero).
CSA2_DEV int bf16_pair_emin(uint32_t w) {
    const uint32_t lo = w & 0xffffu, hi = w >> 16;
    const int elo = (lo & 0x7fffu) ? max((int)((lo >> 7) & 0xff), 1) : (1 << 20);
    const int ehi = (hi & 0x7fffu) ? max((int)((hi >> 7) & 0xff), 1) : (1 << 20);
    return min(elo, ehi);
}


// DT: 0 = bf16, 1 = e4m3, 2 = FP4 e2m1 codes with fp32 block-32 scales (bf16
// queries).  CPL: 16-byte chunks per lane per entry, so an entry is 128*CPL
// bytes (bf16: K = 64*CPL, e4m3: K = 128*CPL, FP4: K = 256*CPL, one scale block
// per chunk).
// FP4 keys with K = 256 are held to 128 registers (4 waves per SIMD); only the
// rare exact-recompute path spills.
// POOL: the slots are a hierarchical pool's positions (a.pool set).
template <int DT, int CPL, bool POOL, bool PERSIST>
__global__ __launch_bounds__(kStreamThreads, DT == 2 && CPL == 1 ? 4 : 1) void score_exact_kernel(ScoreArgs a) {
    constexpr int EPC = DT == 0 ? 8 : DT == 1 ? 16 : 32;  // key elements per 16-byte chunk
    constexpr int EB = 128 * CPL;         // bytes per entry
    int64_t r, e_block, blk_end;
    if constexpr (PERSIST) {
        // a.persist workgroups per row, each a run of consecutive 512-entry blocks
        // of its row, resident for the whole launch
        const int64_t w = blockIdx.x, P = a.persist;
        r = w / P;
        const int64_t L = (a.n_eblk + P - 1) / P;
        const int64_t blk0 = (w % P) * L;
        const int64_t nblk_row = (row_valid(a, r) + kScoreEntriesPerBlock - 1) / kScoreEntriesPerBlock;
        blk_end = blk0 + L < nblk_row ? blk0 + L : nblk_row;
        if (blk0 >= blk_end) return;
        e_block = blk0 * kScoreEntriesPerBlock;
    } else {
        // block w takes t = (w % 8) * per_xcd + w / 8: each XCD gets a run of
        // consecutive t, so the Qs rows of a sequence for one entry block read
        // its keys through the same L2
        const int64_t w = blockIdx.x;
        const int64_t t = (w & 7) * a.per_xcd + (w >> 3);
        if (t >= a.blocks) return;
        const int64_t rest = t / a.Qs;
        r = (rest / a.n_eblk) * a.Qs + t % a.Qs;
        e_block = (rest % a.n_eblk) * kScoreEntriesPerBlock;
        blk_end = e_block / kScoreEntriesPerBlock + 1;
    }
    const int64_t b = r / a.Qs;
    const int64_t nv = row_valid(a, r);
    if (e_block >= nv) return;

    __shared__ uint32_t lhist[kHistBins];
    const bool with_hist = a.hist != nullptr;
    if (with_hist) {
        for (int i = threadIdx.x; i < kHistBins; i += kStreamThreads) lhist[i] = 0;
    }

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 3, sub = lane & 7;

    // this lane's slice of the index query, as fp64 (bf16: as fp32, exact)
    double qd[DT == 0 ? 1 : CPL * EPC];
    float qf[DT == 0 ? CPL * EPC : 1];
    double berr[DT == 2 ? CPL : 1];  // FP4 keys: error bound of each chunk's block sum
    constexpr double kBlkRound = (CPL + 3) * 0x1p-53 * 1.001;
    if constexpr (DT == 2) {
        // bf16 queries against 32-element key chunks: 64 query bytes per chunk
        const uint8_t* qrow = reinterpret_cast<const uint8_t*>(a.iq) + r * (int64_t)(4 * EB);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            double qn1 = 0.0;
            int emin = 1 << 20;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const u32x4 w = *reinterpret_cast<const u32x4*>(qrow + c * 512 + sub * 64 + v * 16);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    qd[c * EPC + 8 * v + 2 * t] = bf16_lo(w[t]);
                    qd[c * EPC + 8 * v + 2 * t + 1] = bf16_hi(w[t]);
                    qn1 += fabs(qd[c * EPC + 8 * v + 2 * t]) + fabs(qd[c * EPC + 8 * v + 2 * t + 1]);
                    emin = min(emin, bf16_pair_emin(w[t]));
                }
            }
            berr[c] = fp4_block_err(qn1, emin);
        }
    } else {
        const uint8_t* qrow = reinterpret_cast<const uint8_t*>(a.iq) + r * (int64_t)EB;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(qrow + c * 128 + sub * 16);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if constexpr (DT == 0) {
                    qf[c * EPC + 2 * t] = bf16_lo(w[t]);
                    qf[c * EPC + 2 * t + 1] = bf16_hi(w[t]);
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
    // accumulation of sum|p| itself is low by at most a factor (1 - K*2^-53)
    const double bound_scale = (double)a.K * 0x1p-53 * 1.001 * (1.0 + (double)a.K * 0x1p-52);
    // least significant bit exponent of the smallest |q| of the row (bf16 values are
    // M * 2^(E-134) with integer M; a zero or subnormal gives the floor E = 1)
    int lq = 0, eqmax = 0;
    double qabs = 0.0;  // sum |q| over the row, rounded up
    if constexpr (DT == 0) {
        float qmin = INFINITY, qmax = 0.0f;
#pragma unroll
        for (int i = 0; i < CPL * EPC; ++i) {
            qmin = fminf(qmin, fabsf(qf[i]));
            qmax = fmaxf(qmax, fabsf(qf[i]));
            qabs += (double)fabsf(qf[i]);
        }
        qmin = fminf(qmin, swz_xor<1>(qmin));
        qmin = fminf(qmin, swz_xor<2>(qmin));
        qmin = fminf(qmin, swz_xor<4>(qmin));
        qmax = fmaxf(qmax, swz_xor<1>(qmax));
        qmax = fmaxf(qmax, swz_xor<2>(qmax));
        qmax = fmaxf(qmax, swz_xor<4>(qmax));
        qabs += swz_xor<1>(qabs);
        qabs += swz_xor<2>(qabs);
        qabs += swz_xor<4>(qabs);
        qabs *= 1.0 + 0x1p-40;
        lq = bf16_lsb_exp(qmin);
        eqmax = (int)(__float_as_uint(qmax) >> 23);
    }

    const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.ik) + b * a.N_cap * (int64_t)EB;
    if (with_hist) __syncthreads();  // histogram zeroed before any chunk adds to it

    // keys are loaded kPD rounds ahead of their use from a ring of round buffers, so
    // enough bytes are in flight per wave (FP4 and e4m3 rows are short: 128 and
    // 256 bytes); a persistent workgroup's ring runs on across its blocks, so its
    // size divides the 8 rounds of a block and the slot of a round is static.
    // Entries past nv load entry nv - 1 (in bounds) and are never stored.
    static_assert(kScoreChunks == 1, "one pass of 512 entries per block");
    constexpr int kPD = DT == 1 ? 3 : (DT == 0 && CPL >= 8) ? 1 : 2;
    constexpr int kRing = kPD + 1;
    static_assert(!PERSIST || kScoreRounds % kRing == 0, "ring slots static across blocks");
    u32x4 wr[kRing][CPL];
    float kr[kRing][DT == 2 ? CPL : 1];
    auto load_round = [&](int64_t e_wave, int t, u32x4(&w)[CPL], float(&ks)[DT == 2 ? CPL : 1]) __attribute__((always_inline)) {
        int64_t e = e_wave + t * 8 + g;
        e = e < nv ? e : nv - 1;
        const int64_t pe = POOL ? slot_entry(a, r, e) : e;
        const uint8_t* src = kbase + pe * EB + sub * 16;
#pragma unroll
        for (int c = 0; c < CPL; ++c)
            w[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + c * 128));
        if constexpr (DT == 2) {
            const float* sp = a.ik_scales + (b * a.N_cap + pe) * (int64_t)(a.K / 32) + sub;
#pragma unroll
            for (int c = 0; c < CPL; ++c) ks[c] = __builtin_nontemporal_load(sp + 8 * c);
        } else {
            ks[0] = 0.0f;
        }
    };
    const int64_t nblk = PERSIST ? blk_end - e_block / kScoreEntriesPerBlock : 1;
    for (int64_t bi = 0; bi < nblk; ++bi) {
        const int64_t blk = e_block / kScoreEntriesPerBlock + bi;
        const int64_t e_wave = blk * kScoreEntriesPerBlock + wave * kScoreEntriesPerWave;
        if (e_wave >= nv) break;  // wave-uniform; only the row's last block is partial
        if (bi == 0) {
#pragma unroll
            for (int t = 0; t < kPD; ++t) load_round(e_wave, t, wr[t], kr[t]);
        }
        double keep = 0.0, keep_abs = 0.0;
        uint32_t keep_ex = 0, keep_mx = 0;
        // one round: 8 entries, 8 lanes each; lane sub == t keeps entry e_wave + 8t + g
        auto round_body = [&](int t, const u32x4(&w)[CPL], const float(&ksc)[DT == 2 ? CPL : 1])
                              __attribute__((always_inline)) {
            double acc = 0.0, aacc = 0.0;  // FP4 keys: aacc is the error bound of acc
            uint32_t kex = 0x7fff7fffu;  // packed minimum of the two bf16 exponent fields
            uint32_t kmx = 0u;           // and their packed maximum
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                if constexpr (DT == 2) {
                    // the chunk is one scale block: exact e2m1 values (scale 1) into an
                    // fp64 block sum, then one fma with the block scale
                    double blk = 0.0;
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const uint32_t cw = w[c][u];
                        const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 0);
                        const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 1);
                        const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 2);
                        const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 3);
                        const double* qq = qd + c * EPC + 8 * u;
                        blk = fma(qq[0], (double)v0[0], blk);
                        blk = fma(qq[1], (double)v0[1], blk);
                        blk = fma(qq[2], (double)v1[0], blk);
                        blk = fma(qq[3], (double)v1[1], blk);
                        blk = fma(qq[4], (double)v2[0], blk);
                        blk = fma(qq[5], (double)v2[1], blk);
                        blk = fma(qq[6], (double)v3[0], blk);
                        blk = fma(qq[7], (double)v3[1], blk);
                    }
                    // CPL fmas here and 3 butterfly adds each round once, relative to
                    // partial sums bounded by sum |blk * scale|
                    const double sd = (double)ksc[c];
                    acc = fma(blk, sd, acc);
                    aacc = fma(fma(kBlkRound, fabs(blk), berr[c]), fabs(sd), aacc);
                    continue;
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if constexpr (DT == 0) {
                        // bf16 x bf16 products are exact in fp32 when no product
                        // leaves fp32's range (checked per entry below)
                        const float p0 = qf[c * EPC + 2 * u] * bf16_lo(w[c][u]);
                        const float p1 = qf[c * EPC + 2 * u + 1] * bf16_hi(w[c][u]);
                        acc += (double)p0;
                        acc += (double)p1;
                        kex = pk_min_u16(kex, w[c][u] & 0x7f807f80u);
                        kmx = pk_max_u16(kmx, w[c][u] & 0x7f807f80u);
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
            acc += dpp_f64<1>(acc);
            acc += dpp_f64<2>(acc);
            acc += dpp_f64<4>(acc);
            if (DT == 2) {
                aacc += dpp_f64<1>(aacc);
                aacc += dpp_f64<2>(aacc);
                aacc += dpp_f64<4>(aacc);
            }
            if (DT == 0) {
                kex = pk_min_u16(kex, dpp_u32<1>(kex));
                kex = pk_min_u16(kex, dpp_u32<2>(kex));
                kex = pk_min_u16(kex, dpp_u32<4>(kex));
                kmx = pk_max_u16(kmx, dpp_u32<1>(kmx));
                kmx = pk_max_u16(kmx, dpp_u32<2>(kmx));
                kmx = pk_max_u16(kmx, dpp_u32<4>(kmx));
            }
            if (sub == t) {
                keep = acc;
                keep_abs = aacc;
                keep_ex = kex;
                keep_mx = kmx;
            }
        };
        {
            // the next block's first rounds are requested during this block's last
            const int64_t e_next = e_wave + kScoreEntriesPerBlock;
            const bool more = PERSIST && blk + 1 < blk_end && e_next < nv;  // wave-uniform
#pragma unroll
            for (int t = 0; t < kScoreRounds; ++t) {
                if (t + kPD < kScoreRounds)
                    load_round(e_wave, t + kPD, wr[(t + kPD) % kRing], kr[(t + kPD) % kRing]);
                else if (more)
                    load_round(e_next, t + kPD - kScoreRounds, wr[(t + kPD) % kRing], kr[(t + kPD) % kRing]);
                round_body(t, wr[t % kRing], kr[t % kRing]);
            }
        }

        // lane (g, sub) now owns entry e_wave + 8*sub + g
        const int64_t e = e_wave + 8 * sub + g;
        float res = 0.0f;
        bool ok = true;
        if (e < nv) {
            if (DT == 0) {
                res = (float)keep;
                // smallest and largest exponent field among the entry's elements
                // (0 = zero or subnormal)
                const uint32_t ex = min(keep_ex & 0xffffu, keep_ex >> 16) >> 7;
                const uint32_t emx = max(keep_mx & 0xffffu, keep_mx >> 16) >> 7;
                const int lk = (int)(ex > 0 ? ex : 1u) - 134;
                // every |p| below 2^(eqmax+emx-252) <= 2^127: no fp32 product
                // overflowed; every product a multiple of 2^(lq+lk) >= 2^-149 (zero
                // elements count as the smallest): none was rounded either,
                // otherwise each is within 2^-150 of its exact value
                const bool in_range = eqmax + (int)emx <= 379 && eqmax < 255 && emx < 255;
                const bool prod_exact = lq + lk >= -149;
                // sum |p| <= sum |q| * max |k| < qabs * 2^(emx - 126)
                const double sabs = qabs * ldexp(1.0, (int)(emx > 0 ? emx : 1u) - 126);
                if (!in_range) {
                    ok = false;
                } else if (!prod_exact || !sum_is_exact(sabs, lq + lk)) {
                    const double eb = bound_scale * sabs + fabs(keep) * 0x1p-52 +
                                      (prod_exact ? 0.0 : (double)a.K * 0x1p-149);
                    const float lo = (float)(keep - eb), hi = (float)(keep + eb);
                    ok = __float_as_uint(lo) == __float_as_uint(hi);
                    res = lo;
                }
            } else if (DT == 2) {
                // keep_abs bounds every rounding of the entry; |keep| * 2^-52 covers the
                // two interval ends' own rounding
                const double eb = (keep_abs + fabs(keep) * 0x1p-52) * (1.0 + 0x1p-40);
                const float lo = (float)(keep - eb), hi = (float)(keep + eb);
                ok = __float_as_uint(lo) == __float_as_uint(hi);
                res = lo;
            } else {
                res = (float)keep;
            }
        }
        if (DT != 1) {
            // entries the certificate could not decide: the whole wave computes
            // each one exactly with the integer accumulator
            uint64_t pend = __ballot(!ok);
            while (pend) {
                const int L = __builtin_ctzll(pend);
                pend &= pend - 1;
                const int64_t eS = __builtin_amdgcn_readlane((int)e, L);
                const int64_t eL = POOL ? slot_entry(a, r, eS) : eS;
                const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.iq) + r * a.K;
                float x;
                if (DT == 2)
                    x = wave_exact_fp4_dot(qp, reinterpret_cast<const uint8_t*>(a.ik) + (b * a.N_cap + eL) * (a.K / 2),
                                           a.ik_scales + (b * a.N_cap + eL) * (a.K / 32), a.K, lane);
                else
                    x = wave_exact_bf16_dot(qp, reinterpret_cast<const uint16_t*>(a.ik) + (b * a.N_cap + eL) * a.K,
                                            a.K, lane);
                if (lane == L) res = x;
            }
        }
        if (e < nv) {
            // streamed past the caches: plain stores of the scores among the key reads
            // made a launch over 64 rows x 131,072 bf16 entries about 2 % slower
            __builtin_nontemporal_store(res, a.scores + r * a.ld + e);
            if (with_hist) atomicAdd(&lhist[sort_key(res) >> (32 - kHistBits)], 1u);
        }
    }
    if (with_hist) {
        __syncthreads();
        uint32_t* ghist = a.hist + r * kHistBins;
        for (int i = threadIdx.x; i < kHistBins; i += kStreamThreads) {
            const uint32_t c = lhist[i];
            if (c) atomicAdd(&ghist[i], c);
        }
    }
}

// Several query rows of one sequence against bf16 keys (a draft block being
// verified, or a prefill chunk on the exact path): each key is loaded and
// widened to fp64 once and multiplied into QR row accumulators, instead of
// being streamed once per row.
//
//   * 16 lanes per entry, 4 entries per wave round; lane `sub` loads the
//     16-byte chunks at byte offset sub*16 + c*256 of the entry, so every
//     chunk round of a wave reads four 256-byte segments;
//   * rows are taken in groups of QR; workgroup tiles (sequence, row group,
//     256-entry block) are laid out XCD-contiguous like score_exact_kernel;
//   * exactness as for one row: Sum|p| is bounded by Sum|q| * max|k| (the
//     entry's largest exponent field), every product is a multiple of
//     2^(lsb(min|q|) + lsb(min|k|)); the rare undecided score is queued
//     (row, entry) for score_fixup_kernel, which recomputes it exactly with a
//     whole wave and adds it to the histogram, so the integer accumulator's
//     registers stay out of this kernel;
//   * the digit-1 histograms of the QR rows share the workgroup's LDS as
//     packed 16-bit counters (a workgroup adds at most 256 per bin).
constexpr int kRowsLanes = 16;                     // lanes per entry
constexpr int kRowsRounds = 16;                    // rounds of 4 entries per wave
constexpr int kRowsEntriesPerBlock = 4 * 4 * kRowsRounds;  // 256 per workgroup
constexpr int kRowsPD = 3;                         // rounds of loads in flight

template <int CPL, int QR>
__global__ __launch_bounds__(kScoreThreads) void score_rows_kernel(ScoreArgs a) {
    constexpr int CH = CPL / 2;   // 16-byte chunks per lane
    constexpr int EL = CH * 8;    // bf16 elements per lane
    constexpr int EB = 128 * CPL; // bytes per entry
    const int64_t w = blockIdx.x;
    const int64_t t = (w & 7) * a.per_xcd + (w >> 3);
    if (t >= a.blocks) return;
    const int64_t ngroups = (a.Qs + QR - 1) / QR;
    const int64_t eblk = t % a.n_eblk, bg = t / a.n_eblk;
    const int64_t b = bg / ngroups, i0 = (bg % ngroups) * QR;
    const int nrows = (int)(a.Qs - i0 < QR ? a.Qs - i0 : QR);
    const int64_t r0 = b * a.Qs + i0;
    // the group's last row sees the most entries
    const int64_t nv_last = row_valid(a, r0 + nrows - 1);
    const int64_t e_block = eblk * kRowsEntriesPerBlock;
    if (e_block >= nv_last) return;

    __shared__ uint32_t lhist[QR][kHistBins / 2];
    const bool with_hist = a.hist != nullptr;
    if (with_hist) {
        for (int i = threadIdx.x; i < QR * kHistBins / 2; i += kScoreThreads) (&lhist[0][0])[i] = 0;
    }

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, sub = lane & 15;

    // this lane's slice of every row's index query (bf16 values, exact in fp32,
    // widened to fp64 where they are used); per row Sum|q| and the least
    // significant bit exponent of the smallest |q|
    float qd[QR][EL];
    double qsum[QR];
    int lq[QR];
    int64_t nv[QR];
#pragma unroll
    for (int j = 0; j < QR; ++j) {
        const int jj = j < nrows ? j : nrows - 1;  // rows past the group repeat its last row
        nv[j] = j < nrows ? row_valid(a, r0 + j) : 0;
        const uint8_t* qrow = reinterpret_cast<const uint8_t*>(a.iq) + (r0 + jj) * (int64_t)EB;
        float qmin = INFINITY;
        double qs = 0.0;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const u32x4 qw = *reinterpret_cast<const u32x4*>(qrow + c * 256 + sub * 16);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                qd[j][c * 8 + 2 * u] = bf16_lo(qw[u]);
                qd[j][c * 8 + 2 * u + 1] = bf16_hi(qw[u]);
                qs += fabs((double)qd[j][c * 8 + 2 * u]) + fabs((double)qd[j][c * 8 + 2 * u + 1]);
                qmin = fminf(qmin, fminf(fabsf(bf16_lo(qw[u])), fabsf(bf16_hi(qw[u]))));
            }
        }
        qs += swz_xor<1>(qs);
        qs += swz_xor<2>(qs);
        qs += swz_xor<4>(qs);
        qs += swz_xor<8>(qs);
        qmin = fminf(qmin, swz_xor<1>(qmin));
        qmin = fminf(qmin, swz_xor<2>(qmin));
        qmin = fminf(qmin, swz_xor<4>(qmin));
        qmin = fminf(qmin, swz_xor<8>(qmin));
        qsum[j] = qs;
        lq[j] = bf16_lsb_exp(qmin);
    }
    const double bound_scale = (double)a.K * 0x1p-53 * 1.001 * (1.0 + (double)a.K * 0x1p-52);
    const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.ik) + b * a.N_cap * (int64_t)EB;
    if (with_hist) __syncthreads();

    const int64_t e_wave = e_block + wave * (4 * kRowsRounds);
    if (e_wave < nv_last) {
        // keys are loaded kRowsPD rounds ahead of their use (ring of kRowsPD + 1)
        u32x4 ring[kRowsPD + 1][CH];
        auto load = [&](int64_t e, u32x4(&dst)[CH]) __attribute__((always_inline)) {
            e = e < nv_last ? e : nv_last - 1;  // in bounds; results past nv are not stored
            const uint8_t* src = kbase + e * EB + sub * 16;
#pragma unroll
            for (int c = 0; c < CH; ++c) dst[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + c * 256));
        };
#pragma unroll
        for (int p = 0; p < kRowsPD; ++p) load(e_wave + 4 * p + g, ring[p]);
#pragma unroll
        for (int rd = 0; rd < kRowsRounds; ++rd) {
            const int64_t e = e_wave + 4 * rd + g;
            if (e_wave + 4 * rd >= nv_last) break;  // wave-uniform
            if (rd + kRowsPD < kRowsRounds) load(e + 4 * kRowsPD, ring[(rd + kRowsPD) % (kRowsPD + 1)]);
            const u32x4(&wk)[CH] = ring[rd % (kRowsPD + 1)];
            double acc[QR];
#pragma unroll
            for (int j = 0; j < QR; ++j) acc[j] = 0.0;
            uint32_t kex = 0x7fff7fffu, kmx = 0u;
#pragma unroll
            for (int c = 0; c < CH; ++c) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint32_t kw = wk[c][u];
                    const double lo = bf16_lo(kw), hi = bf16_hi(kw);
#pragma unroll
                    for (int j = 0; j < QR; ++j) {
                        acc[j] = fma((double)qd[j][c * 8 + 2 * u], lo, acc[j]);
                        acc[j] = fma((double)qd[j][c * 8 + 2 * u + 1], hi, acc[j]);
                    }
                    const uint32_t ef = kw & 0x7f807f80u;
                    kex = pk_min_u16(kex, ef);
                    kmx = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, kmx),
                                                                                 __builtin_bit_cast(u16x2, ef)));
                }
            }
            // 16-lane DPP butterfly (its pairings stay inside the entry's lanes)
            auto fold = [&](auto xr) __attribute__((always_inline)) {
                constexpr int X = decltype(xr)::value;
#pragma unroll
                for (int j = 0; j < QR; ++j) acc[j] += dpp_f64<X>(acc[j]);
                kex = pk_min_u16(kex, dpp_u32<X>(kex));
                kmx = pk_max_u16(kmx, dpp_u32<X>(kmx));
            };
            fold(std::integral_constant<int, 1>{});
            fold(std::integral_constant<int, 2>{});
            fold(std::integral_constant<int, 4>{});
            fold(std::integral_constant<int, 8>{});
            // lane sub (< QR) finishes row sub of entry e: pick that row's values
            // first, so the certificate below runs once per lane
            double sj = 0.0, qs = 0.0;
            int lqj = 0;
            int64_t nvj = 0;
#pragma unroll
            for (int j = 0; j < QR; ++j) {
                if (sub == j) {
                    sj = acc[j];
                    qs = qsum[j];
                    lqj = lq[j];
                    nvj = nv[j];
                }
            }
            const bool mine = e < nvj;  // nv is 0 for lanes and rows past the group
            const int64_t rr = r0 + sub;
            float res = (float)sj;
            bool ok = true;
            if (mine) {
                const uint32_t exmin = min(kex & 0xffffu, kex >> 16) >> 7;
                const uint32_t exmax = max(kmx & 0xffffu, kmx >> 16) >> 7;
                const double bound = ldexp(qs, (int)max(exmax, 1u) - 126);  // >= Sum|q||k|
                const int lk = (int)(exmin > 0 ? exmin : 1u) - 134;
                if (!sum_is_exact(bound, lqj + lk)) {
                    const double eb = bound_scale * bound + fabs(sj) * 0x1p-52;
                    const float lo = (float)(sj - eb), hi = (float)(sj + eb);
                    ok = __float_as_uint(lo) == __float_as_uint(hi);
                    res = lo;
                }
            }
            if (mine && !ok) {
                const uint32_t slot = atomicAdd(a.fix_cnt, 1u);
                a.fix_list[slot] = make_uint2((uint32_t)rr, (uint32_t)e);
            }
            if (mine && ok) {
                a.scores[rr * a.ld + e] = res;
                if (with_hist) {
                    const uint32_t bin = sort_key(res) >> (32 - kHistBits);
                    atomicAdd(&lhist[rr - r0][bin >> 1], 1u << (16 * (bin & 1u)));
                }
            }
        }
    }
    if (with_hist) {
        __syncthreads();
        for (int j = 0; j < nrows; ++j) {
            uint32_t* ghist = a.hist + (r0 + j) * kHistBins;
            for (int i = threadIdx.x; i < kHistBins / 2; i += kScoreThreads) {
                const uint32_t c = lhist[j][i];
                if (c & 0xffffu) atomicAdd(&ghist[2 * i], c & 0xffffu);
                if (c >> 16) atomicAdd(&ghist[2 * i + 1], c >> 16);
            }
        }
    }
}

// The scores score_rows_kernel could not decide: one wave per queued (row,
// entry) at a time, exact integer accumulation, result and histogram count.
// The queue holds at most one item per (row, entry), so the loop is bounded.
__global__ __launch_bounds__(kScoreThreads) void score_fixup_kernel(ScoreArgs a) {
    const uint32_t n = *a.fix_cnt;
    const int lane = threadIdx.x & 63;
    const uint32_t wid = blockIdx.x * (kScoreThreads / 64) + (threadIdx.x >> 6);
    const uint32_t nw = gridDim.x * (kScoreThreads / 64);
    for (uint32_t i = wid; i < n; i += nw) {
        const uint2 it = a.fix_list[i];
        const int64_t r = it.x, e = it.y, b = r / a.Qs;
        const float x = wave_exact_bf16_dot(reinterpret_cast<const uint16_t*>(a.iq) + r * a.K,
                                            reinterpret_cast<const uint16_t*>(a.ik) + (b * a.N_cap + e) * a.K,
                                            a.K, lane);
        if (lane == 0) {
            a.scores[r * a.ld + e] = x;
            if (a.hist) atomicAdd(&a.hist[r * kHistBins + (sort_key(x) >> (32 - kHistBits))], 1u);
        }
    }
}

// Score of (row r, position pe) computed by one thread with the arithmetic and
// certification of the streaming kernel: false when the certificate cannot
// decide (then *out is not the score).
// FP4 keys, one thread: per 32-element block an fp64 sum of q * e2m1 with its
// error bound, then one fma with the block scale; the bound covers every
// rounding.  false when it does not decide the fp32 rounding.
CSA2_DEV bool fp4_entry_certified(const uint16_t* q, const uint8_t* k, const float* sc, int K, float* out) {
    double acc = 0.0, aacc = 0.0;
    for (int blk0 = 0; blk0 < K; blk0 += 32) {
        double blk = 0.0, qn1 = 0.0;
        int emin = 1 << 20;
        for (int i = blk0; i < blk0 + 32; ++i) {
            const uint32_t nib = (k[i >> 1] >> (4 * (i & 1))) & 15u;
            const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(nib, 1.0f, 0);
            const double qv = (double)bf16_to_f32(q[i]);
            blk = fma(qv, (double)v[0], blk);
            qn1 += fabs(qv);
            emin = min(emin, bf16_pair_emin(q[i]));
        }
        const double sd = (double)sc[blk0 >> 5];
        acc = fma(blk, sd, acc);
        aacc = fma(fma((double)(K / 32) * 0x1p-53 * 1.001, fabs(blk), fp4_block_err(qn1, emin)), fabs(sd), aacc);
    }
    const double eb = (aacc + fabs(acc) * 0x1p-52) * (1.0 + 0x1p-40);
    const float lo = (float)(acc - eb), hi = (float)(acc + eb);
    *out = lo;
    return __float_as_uint(lo) == __float_as_uint(hi);
}

CSA2_DEV bool generic_entry_certified(const ScoreArgs& a, int64_t r, int64_t pe, float* out) {
    const int64_t b = r / a.Qs;
    const int K = a.K;
    if (a.dtype == 2)
        return fp4_entry_certified(reinterpret_cast<const uint16_t*>(a.iq) + r * K,
                                   reinterpret_cast<const uint8_t*>(a.ik) + (b * a.N_cap + pe) * (K / 2),
                                   a.ik_scales + (b * a.N_cap + pe) * (K / 32), K, out);
    double acc = 0.0, aacc = 0.0;
    float qmin = INFINITY, kmin = INFINITY;
    if (a.dtype == 0) {
        const uint16_t* q = reinterpret_cast<const uint16_t*>(a.iq) + r * K;
        const uint16_t* k = reinterpret_cast<const uint16_t*>(a.ik) + (b * a.N_cap + pe) * K;
        for (int i = 0; i < K; ++i) {
            const float qf = bf16_to_f32(q[i]), kf = bf16_to_f32(k[i]);
            acc = fma((double)qf, (double)kf, acc);
            aacc = fma(fabs((double)qf), fabs((double)kf), aacc);
            qmin = fminf(qmin, fabsf(qf));
            kmin = fminf(kmin, fabsf(kf));
        }
    } else {
        const uint8_t* q = reinterpret_cast<const uint8_t*>(a.iq) + r * K;
        const uint8_t* k = reinterpret_cast<const uint8_t*>(a.ik) + (b * a.N_cap + pe) * K;
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
    *out = res;
    return ok;
}

// Exact score of (row r, position pe) computed by one thread: the certified
// fp64 value, else the integer accumulator.
CSA2_DEV float generic_entry_score(const ScoreArgs& a, int64_t r, int64_t pe) {
    float res;
    if (generic_entry_certified(a, r, pe, &res)) return res;
    const int64_t b = r / a.Qs;
    const int K = a.K;
    return a.dtype == 2
               ? exact_fp4_dot(reinterpret_cast<const uint16_t*>(a.iq) + r * K,
                               reinterpret_cast<const uint8_t*>(a.ik) + (b * a.N_cap + pe) * (K / 2),
                               a.ik_scales + (b * a.N_cap + pe) * (K / 32), K)
               : exact_bf16_dot(reinterpret_cast<const uint16_t*>(a.iq) + r * K,
                                reinterpret_cast<const uint16_t*>(a.ik) + (b * a.N_cap + pe) * K, K);
}

// ---------------------------------------------------------------------------
// FP4 keys (K = 256) on the matrix cores.  The block sums T_c = sum_e q_e * c_e
// (bf16 query, e2m1 codes, one sum per 32-element key block c) come exactly out
// of v_mfma_scale_f32_16x16x128_f8f6f4 with e4m3 query parts against the raw FP4
// codes; fp64 then forms sum_c scale_c * T_c with an error bound, certified as
// in the streaming kernel.
//
// The MFMA is not an exact dot product: it cuts each product in a group of 8
// consecutive k toward zero to a multiple of 2^(ea + eb - 13), ea + eb the
// group's largest operand exponent pair (measured on gfx950; e2m1 0.5 counts as
// exponent 0), sums the group exactly and adds group sums in fp32.  The query
// side is therefore split so that nothing is ever cut:
//   * a block's query values fall into bands of 7 binades below its largest
//     exponent field emax: band b holds fe in (emax - 7(b+1), emax - 7b];
//   * each value is split into its top 4 significant bits (hi) and its low 4
//     mantissa bits (lo), both exact e4m3 numbers once scaled by 2^-S_b, S_b the
//     band's E8M0 scale (hi exponents 1..7, lo exponents -6..3);
//   * a group's products are then multiples of 2^-3 (hi) or 2^-7 (lo) of 2^S_b,
//     while its cut step is at most 2^(7+2-13) = 2^-4 or 2^(3+2-13) = 2^-8 of it;
//     32 products stay below 2^16 (hi) or 2^12 (lo), so every group sum, every
//     fp32 addition and hi + lo of one band are exact in fp32;
//   * bands 0-1 (14 binades) cover common rows with one MFMA per 128 codes,
//     bands 0-3 (28) with two; rows beyond that, with subnormal values, or
//     with exponents far from 1 take a per-thread fp64 path.
//
// MFMA layout (gfx950, probed): B = FP4 codes, lane (n, g) holds column n's
// codes k = 32g .. 32g+31 in nibble order; A = e4m3, lane (m, g2) holds row m's
// k = 16g2 .. 16g2+15 (bytes 0-15) and 64+16g2 .. 64+16g2+15 (bytes 16-31);
// C lane (n, g) holds rows 4g .. 4g+3 of column n.  A tile is 16 entries: lane
// (n, g) holds entry n's key blocks 2g and 2g+1 (32 contiguous bytes, one MFMA
// "slice" each) and their two scales, rearranged through LDS from loads of whole
// 128-byte lines; A row 4g + p carries part p (band 2j hi,
// band 2j lo, band 2j+1 hi, band 2j+1 lo) of key block 2g + slice, so C lane
// (n, g) receives exactly the parts of its own two blocks.  Four tiles (64
// entries) are reduced across g with permlane swaps so that lane l ends with
// entry l of the round.
constexpr int kF4Threads = 512;                                   // 8 waves
constexpr int kF4Rounds = 1;                                      // rounds of 64 entries per wave
constexpr int kF4Ahead = 1;                                       // rounds of keys loaded ahead
constexpr int kF4MinWaves = 4;                                    // waves per SIMD (launch bound)
constexpr int kF4EntriesPerBlock = (kF4Threads / 64) * 64 * kF4Rounds;  // 512
constexpr uint32_t kF4EmaxLo = 64, kF4EmaxHi = 220;  // block exponent fields kept on the MFMA path

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// The scaled MFMA with e4m3 A (query parts, E8M0 scale sa) and e2m1 B (codes,
// unit scale).  The empty asm keeps it at full EXEC: the compiler would
// otherwise sink it into the branch that stores a result.
CSA2_DEV f32x4 mfma_q8_k4(const i32x8& q, const u32x4& k, uint32_t sa) {
    const i32x8 kb = {(int)k[0], (int)k[1], (int)k[2], (int)k[3], 0, 0, 0, 0};
    f32x4 c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(q, kb, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 4, 0,
                                                              (int)sa, 0, 127);
    __asm__ volatile("" : "+v"(c));
    return c;
}

// permlane32 (D = 32) or permlane16 (D = 16) swap of an fp64 pair, then their
// sum: lanes with bit D clear get x(own) + x(lane + D), the others
// y(lane - D) + y(own).
template <int D>
CSA2_DEV double swap_add(double x, double y) {
    const uint2 xu = __builtin_bit_cast(uint2, x), yu = __builtin_bit_cast(uint2, y);
    uint2 a, c;
    if constexpr (D == 32) {
        const auto lo = __builtin_amdgcn_permlane32_swap(xu.x, yu.x, false, false);
        const auto hi = __builtin_amdgcn_permlane32_swap(xu.y, yu.y, false, false);
        a = uint2{lo[0], hi[0]};
        c = uint2{lo[1], hi[1]};
    } else {
        const auto lo = __builtin_amdgcn_permlane16_swap(xu.x, yu.x, false, false);
        const auto hi = __builtin_amdgcn_permlane16_swap(xu.y, yu.y, false, false);
        a = uint2{lo[0], hi[0]};
        c = uint2{lo[1], hi[1]};
    }
    return __builtin_bit_cast(double, a) + __builtin_bit_cast(double, c);
}
template <int D>
CSA2_DEV float swap_add(float x, float y) {
    const auto r = D == 32 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false)
                           : __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The two operands a permlane swap_add<D> would add, for checks on the sum.
template <int D>
CSA2_DEV void swap_pair(double x, double y, double& a, double& c) {
    const uint2 xu = __builtin_bit_cast(uint2, x), yu = __builtin_bit_cast(uint2, y);
    if constexpr (D == 32) {
        const auto lo = __builtin_amdgcn_permlane32_swap(xu.x, yu.x, false, false);
        const auto hi = __builtin_amdgcn_permlane32_swap(xu.y, yu.y, false, false);
        a = __builtin_bit_cast(double, uint2{lo[0], hi[0]});
        c = __builtin_bit_cast(double, uint2{lo[1], hi[1]});
    } else {
        const auto lo = __builtin_amdgcn_permlane16_swap(xu.x, yu.x, false, false);
        const auto hi = __builtin_amdgcn_permlane16_swap(xu.y, yu.y, false, false);
        a = __builtin_bit_cast(double, uint2{lo[0], hi[0]});
        c = __builtin_bit_cast(double, uint2{lo[1], hi[1]});
    }
}
template <int D>
CSA2_DEV uint32_t swap_and(uint32_t x, uint32_t y) {
    const auto r = D == 32 ? __builtin_amdgcn_permlane32_swap(x, y, false, false)
                           : __builtin_amdgcn_permlane16_swap(x, y, false, false);
    return r[0] & r[1];
}

// s = a + c and whether that addition was exact (the TwoSum error is zero).
CSA2_DEV double add_exact(double a, double c, uint32_t& exact) {
    const double s = a + c, bv = s - a;
    const double err = (a - (s - bv)) + (c - bv);
    exact &= err == 0.0 ? 1u : 0u;
    return s;
}

// One wave's rounds of 64 entries on the matrix cores, NB band pairs.
struct F4Round {
    u32x4 c[4][2];  // per tile: 16 bytes of each of two entries (as loaded)
    f32x2 sc[4];    // and two scales of one entry
};

// Loads one round (4 tiles of 16 entries from e_round) of a wave in whole 128-byte
// lines: per tile, lane L takes chunk L % 8 (16 bytes, one key block) of entries
// e_round + 16t + L / 8 and + 8, and scales 2(L % 4), 2(L % 4) + 1 of entry
// e_round + 16t + L / 4.  Entries past nv load entry nv - 1 (in bounds; never
// stored).  f4_tile rearranges a tile for the matrix cores.
CSA2_DEV void f4_load_round(const ScoreArgs& a, int64_t b, int64_t nv, int64_t e_round, F4Round& d) {
    const int lane = threadIdx.x & 63;
    const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.ik) + b * a.N_cap * 128 + 16 * (lane & 7);
    const float* sbase = a.ik_scales + b * a.N_cap * 8 + 2 * (lane & 3);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        int64_t e0 = e_round + 16 * t + (lane >> 3), e1 = e0 + 8, es = e_round + 16 * t + (lane >> 2);
        e0 = e0 < nv ? e0 : nv - 1;
        e1 = e1 < nv ? e1 : nv - 1;
        es = es < nv ? es : nv - 1;
        d.c[t][0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + e0 * 128));
        d.c[t][1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + e1 * 128));
        d.sc[t] = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(sbase + es * 8));
    }
}

constexpr int kF4TilePitch = 144;                   // bytes per entry row in LDS (128 + 16 against bank conflicts)
constexpr int kF4TileBytes = 16 * kF4TilePitch + 16 * 32;  // codes and scales of one tile

// Tile t of a loaded round in the matrix-core layout, through the wave's LDS
// buffer wb: lane (n, g) gets entry n's key blocks 2g and 2g + 1 (kc[0], kc[1])
// and their scales.
CSA2_DEV void f4_tile(const F4Round& d, int t, uint8_t* wb, u32x4 (&kc)[2], f32x2& ks) {
    const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
    *reinterpret_cast<u32x4*>(wb + (lane >> 3) * kF4TilePitch + 16 * (lane & 7)) = d.c[t][0];
    *reinterpret_cast<u32x4*>(wb + ((lane >> 3) + 8) * kF4TilePitch + 16 * (lane & 7)) = d.c[t][1];
    *reinterpret_cast<f32x2*>(wb + 16 * kF4TilePitch + 8 * lane) = d.sc[t];
    __builtin_amdgcn_wave_barrier();
    kc[0] = *reinterpret_cast<const u32x4*>(wb + n * kF4TilePitch + 32 * g);
    kc[1] = *reinterpret_cast<const u32x4*>(wb + n * kF4TilePitch + 32 * g + 16);
    ks = *reinterpret_cast<const f32x2*>(wb + 16 * kF4TilePitch + 32 * n + 8 * g);
    __builtin_amdgcn_wave_barrier();
}

// The rare paths of score_fp4_mfma_kernel, out of line so that the registers
// they need are not reserved in the streaming code; arguments are plain
// pointers (a struct passed by reference would be copied to scratch per lane).
// Exact score of an entry by the whole wave (q: the row's 256 bf16 values, k and
// sc: the entry's codes and scales).
static __device__ __attribute__((noinline)) float f4_wave_exact_ool(const uint16_t* q, const uint8_t* k, const float* sc,
                                                                int lane) {
    return wave_exact_fp4_256(q, k, sc, lane);
}
// fp4_entry_certified for K = 256, one thread.
static __device__ __attribute__((noinline)) bool f4_entry_certified_ool(const uint16_t* q, const uint8_t* k, const float* sc,
                                                                    float* out) {
    return fp4_entry_certified(q, k, sc, 256, out);
}
CSA2_DEV float f4_wave_exact(const ScoreArgs& a, int64_t r, int64_t e, int lane) {
    const int64_t b = r / a.Qs;
    return f4_wave_exact_ool(reinterpret_cast<const uint16_t*>(a.iq) + r * 256,
                             reinterpret_cast<const uint8_t*>(a.ik) + (b * a.N_cap + e) * 128,
                             a.ik_scales + (b * a.N_cap + e) * 8, lane);
}
CSA2_DEV bool f4_entry_certified(const ScoreArgs& a, int64_t r, int64_t e, float* out) {
    const int64_t b = r / a.Qs;
    return f4_entry_certified_ool(reinterpret_cast<const uint16_t*>(a.iq) + r * 256,
                                  reinterpret_cast<const uint8_t*>(a.ik) + (b * a.N_cap + e) * 128,
                                  a.ik_scales + (b * a.N_cap + e) * 8, out);
}

// The wave's rounds: e_block + (NW i + wave) * 64 for i < kF4Rounds.  Keys are
// loaded kF4Ahead rounds ahead into a ring of round buffers (the caller has
// issued the first ones); the loop is unrolled so the ring index is static.
// Entries the certificate cannot decide get a checked recompute, and what that
// leaves open the exact integer sum, both in place; every score is counted in
// the LDS histogram.
template <int NB>
CSA2_DEV void fp4_mfma_rows(const ScoreArgs& a, int64_t r, int64_t e_block, int64_t nv, const uint32_t (*s_afr)[2][64][8],
                            const uint32_t (*s_scl)[2][64], uint32_t* lhist, F4Round (&ring)[kF4Ahead + 1],
                            uint8_t* wb) {
    constexpr int NW = kF4Threads / 64;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t b = r / a.Qs;
    // the A fragments stay in LDS (read per MFMA) to leave registers for the key ring
    uint32_t scl[NB][2];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int s = 0; s < 2; ++s) scl[j][s] = s_scl[j][s][lane];
#pragma unroll
    for (int i = 0; i < kF4Rounds; ++i) {
        const int64_t e_round = e_block + (NW * i + wave) * 64;
        if (e_round >= nv) break;  // wave-uniform
        const int64_t e_ahead = e_round + kF4Ahead * NW * 64;
        if (i + kF4Ahead < kF4Rounds && e_ahead < nv)
            f4_load_round(a, b, nv, e_ahead, ring[(i + kF4Ahead) % (kF4Ahead + 1)]);
        const F4Round& cur = ring[i % (kF4Ahead + 1)];
        double P[4];
        float A[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            u32x4 kc[2];
            f32x2 ks;
            f4_tile(cur, t, wb, kc, ks);
            double T[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                double ts = 0.0;
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const f32x4 c = mfma_q8_k4(*reinterpret_cast<const i32x8*>(s_afr[j][s][lane]), kc[s], scl[j][s]);
                    // hi + lo of one band is exact in fp32; the bands sum exactly in fp64
                    ts += (double)(c[0] + c[1]) + (double)(c[2] + c[3]);
                }
                T[s] = ts;
            }
            const double p0 = T[0] * (double)ks[0], p1 = T[1] * (double)ks[1];
            P[t] = p0 + p1;
            A[t] = (float)(fabs(p0) + fabs(p1));
        }
        // lane l: entry e_round + l, summed over its 8 key blocks
        const double acc = swap_add<16>(swap_add<32>(P[0], P[2]), swap_add<32>(P[1], P[3])) + 0.0;
        const float sabs = swap_add<16>(swap_add<32>(A[0], A[2]), swap_add<32>(A[1], A[3]));
        // every term saw one product and at most three additions in fp64 (4u), and
        // sabs (fp32, three roundings) is within 2^-21 of its sum
        const double eb = (4.001 * 0x1p-53 * (double)sabs * (1.0 + 0x1p-20) + fabs(acc) * 0x1p-52) * (1.0 + 0x1p-40);
        const float lo = (float)(acc - eb), hi = (float)(acc + eb);
        const int64_t e = e_round + lane;
        bool decided = __float_as_uint(lo) == __float_as_uint(hi);
        float res = lo;
        if (__ballot(e < nv && !decided) != 0) {
            // rare (exact fp32 ties, mostly): the same sum again with every
            // product and addition checked; when none rounded, acc is the exact
            // value and its fp32 rounding is the score
            double Q[4];
            uint32_t X[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                uint32_t ex = 1u;
                double p[2];
                u32x4 kc[2];
                f32x2 ks;
                f4_tile(cur, t, wb, kc, ks);
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    double ts = 0.0;
#pragma unroll
                    for (int j = 0; j < NB; ++j) {
                        const f32x4 c = mfma_q8_k4(*reinterpret_cast<const i32x8*>(s_afr[j][s][lane]), kc[s], scl[j][s]);
                        ts += (double)(c[0] + c[1]) + (double)(c[2] + c[3]);
                    }
                    const double sd = (double)ks[s];
                    p[s] = ts * sd;
                    ex &= fma(ts, sd, -p[s]) == 0.0 ? 1u : 0u;
                }
                Q[t] = add_exact(p[0], p[1], ex);
                X[t] = ex;
            }
            double u0, u1, v0, v1, w0, w1;
            swap_pair<32>(Q[0], Q[2], u0, u1);
            swap_pair<32>(Q[1], Q[3], v0, v1);
            uint32_t xu = swap_and<32>(X[0], X[2]), xv = swap_and<32>(X[1], X[3]);
            const double su = add_exact(u0, u1, xu), sv = add_exact(v0, v1, xv);
            swap_pair<16>(su, sv, w0, w1);
            uint32_t xw = swap_and<16>(xu, xv);
            const double sw = add_exact(w0, w1, xw);
            if (!decided && xw != 0u) {
                decided = true;
                res = (float)sw;
            }
        }
        // rarer still: what the check leaves undecided is computed exactly by the
        // whole wave, one entry at a time (one round per wave: no keys in flight)
        uint64_t pend = __ballot(e < nv && !decided);
        while (pend) {
            const int L = __builtin_ctzll(pend);
            pend &= pend - 1;
            const float x = f4_wave_exact(a, r, e_round + L, lane);
            if (lane == L) res = x;
        }
        if (e < nv) {
            a.scores[r * a.ld + e] = res;
            if (lhist) atomicAdd(&lhist[sort_key(res) >> (32 - kHistBits)], 1u);
        }
    }
}

__global__ __launch_bounds__(kF4Threads, kF4MinWaves) void score_fp4_mfma_kernel(ScoreArgs a) {
    constexpr int NW = kF4Threads / 64;
    static_assert(kF4Threads >= 256, "one thread per query element");
    static_assert(kF4Rounds * kF4Threads == kF4EntriesPerBlock, "one entry per thread outside the bands");
    int64_t r, e_block;
    {
        // tiles are counted in 32 bits (fewer than 2^31 by the launch checks)
        const uint32_t w = blockIdx.x;
        const uint32_t t = (w & 7) * (uint32_t)a.per_xcd + (w >> 3);
        if (t >= (uint32_t)a.blocks) return;
        const uint32_t Qs = (uint32_t)a.Qs, neb = (uint32_t)a.n_eblk;
        const uint32_t rest = t / Qs;
        r = (int64_t)(rest / neb) * Qs + t % Qs;
        e_block = (int64_t)(rest % neb) * kF4EntriesPerBlock;
    }
    const int64_t nv = row_valid(a, r);
    if (e_block >= nv) return;

    __shared__ uint32_t lhist[kHistBins];
    __shared__ __attribute__((aligned(32))) uint32_t s_afr[2][2][64][8];  // [band pair][slice][lane][word]: A fragments
    __shared__ uint32_t s_scl[2][2][64];     // [band pair][slice][lane]: E8M0 scales
    __shared__ __attribute__((aligned(16))) uint8_t s_tile[NW][kF4TileBytes];  // per wave: a tile rearranged
    __shared__ uint32_t s_emax[8], s_band[NW], s_bad[NW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool with_hist = a.hist != nullptr;
    // query element tid & 255, loaded ahead of the keys: loads complete in the
    // order they are issued, so the query is prepared while the first round's
    // keys are in flight
    const int el = tid & 255;
    const uint32_t x = reinterpret_cast<const uint16_t*>(a.iq)[r * 256 + el];
    F4Round ring[kF4Ahead + 1];
    {
        const int64_t e0 = e_block + __builtin_amdgcn_readfirstlane(wave) * 64;
        // the first round unconditionally (past nv it loads entry nv - 1, in bounds),
        // so that the wait for the query is counted past the keys and never waits
        // for them
        f4_load_round(a, r / a.Qs, nv, e0, ring[0]);
#pragma unroll
        for (int i = 1; i < kF4Ahead; ++i)
            if (i < kF4Rounds && e0 + i * NW * 64 < nv) f4_load_round(a, r / a.Qs, nv, e0 + i * NW * 64, ring[i]);
    }
    if (with_hist)
        for (int i = tid; i < kHistBins; i += kF4Threads) lhist[i] = 0;
    for (int i = tid; i < 2 * 2 * 64 * 8 / 4; i += kF4Threads) reinterpret_cast<u32x4*>(s_afr)[i] = u32x4{0u, 0u, 0u, 0u};

    // query element el: its block's largest exponent field, its band and its two
    // e4m3 parts (threads 256.. repeat element tid % 256, which changes no maximum)
    const bool nz = (x & 0x7fffu) != 0;
    const uint32_t fe = (x >> 7) & 0xffu;
    // maxima across lanes on DPP and permlane swaps (VALU, no LDS round trips):
    // em over the element's 32-lane block, mb over the wave
    uint32_t em = wave_row_max(nz ? fe : 0u);
    {
        const auto p = __builtin_amdgcn_permlane16_swap(em, em, false, false);
        em = max(p[0], p[1]);
    }
    const uint32_t band = nz ? (em - fe) / 7 : 0u;
    uint32_t mb = wave_row_max(band);
    {
        const auto p = __builtin_amdgcn_permlane16_swap(mb, mb, false, false);
        mb = max(p[0], p[1]);
        const auto q = __builtin_amdgcn_permlane32_swap(mb, mb, false, false);
        mb = max(q[0], q[1]);
    }
    const bool bad = nz && (fe == 0 || em < kF4EmaxLo || em > kF4EmaxHi);
    const bool wbad = __ballot(bad) != 0;
    if ((tid & 31) == 0 && tid < 256) s_emax[tid >> 5] = em;
    if (lane == 0) {
        s_band[wave] = mb;
        s_bad[wave] = wbad ? 1u : 0u;
    }
    __syncthreads();  // also: the fragments are zeroed
    uint32_t maxband = 0, rowbad = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        maxband = max(maxband, s_band[w]);
        rowbad |= s_bad[w];
    }
    const int NB = rowbad || maxband >= 4 ? 0 : (maxband >= 2 ? 2 : 1);  // workgroup-uniform
    uint32_t* const lh = with_hist ? lhist : nullptr;

    if (NB == 0) {
        // outside the bands: one entry per thread in fp64 with its error bound
        // (generic_entry_certified), what that leaves undecided exactly by the
        // whole wave
        const int64_t e = e_block + tid;
        float res = 0.0f;
        const bool ok = e < nv && f4_entry_certified(a, r, e, &res);
        uint64_t pend = __ballot(e < nv && !ok);
        while (pend) {
            const int L = __builtin_ctzll(pend);
            pend &= pend - 1;
            const float x = f4_wave_exact(a, r, e_block + 64 * wave + L, lane);
            if (lane == L) res = x;
        }
        if (e < nv) {
            a.scores[r * a.ld + e] = res;
            if (lh) atomicAdd(&lh[sort_key(res) >> (32 - kHistBits)], 1u);
        }
    } else {
        if (tid < 256) {
            // element el's parts, as e4m3 bytes scaled by 2^-S (S + 127 = emax - 7 band
            // - 7): hi = sign, exponent field tt + 14, its top 3 mantissa bits; lo =
            // its low 4 mantissa bits l times 2^tt, normalised (exponent field tt +
            // msb(l) + 7).  They go to rows 4g + 2(band & 1) and + 1 of band pair
            // band / 2, slice blk & 1, at k = 32g + el % 32 (g = blk / 2)
            if (nz) {
                const uint32_t sign = (x >> 8) & 0x80u;
                const int tt = (int)fe - ((int)em - 7 * (int)band);  // -6 .. 0
                const uint32_t hib = sign | ((uint32_t)(tt + 14) << 3) | ((x >> 4) & 7u);
                const uint32_t l = x & 15u;
                const int msb = 31 - __builtin_clz(l | 1u);
                const uint32_t lob = l == 0 ? 0u : sign | ((uint32_t)(tt + msb + 7) << 3) | ((l << (3 - msb)) & 7u);
                const int blk = el >> 5, g = blk >> 1, sl = blk & 1;
                const int k = 32 * g + (el & 31);
                const int g2 = (k & 63) >> 4, jb = (k & 15) + (k >= 64 ? 16 : 0);
                const int m = 4 * g + 2 * (int)(band & 1);
                uint8_t* row = reinterpret_cast<uint8_t*>(&s_afr[band >> 1][sl][m + 16 * g2][0]);
                row[jb] = (uint8_t)hib;
                row[32 + jb] = (uint8_t)lob;  // lane m + 1 + 16 g2
            }
            // E8M0 scale of lane (j, slice, L): its row's band, of block 2g + slice
            const int j = tid >> 7, sl = (tid >> 6) & 1, L = tid & 63;
            if (j < NB) {
                const int m = L & 15, g = m >> 2, bnd = 2 * j + ((m & 3) >> 1);
                const uint32_t emx = s_emax[2 * g + sl];
                s_scl[j][sl][L] = emx == 0 ? 127u : emx - 7u * (uint32_t)bnd - 7u;
            }
        }
        __syncthreads();
        if (NB == 1)
            fp4_mfma_rows<1>(a, r, e_block, nv, s_afr, s_scl, lh, ring, s_tile[wave]);
        else
            fp4_mfma_rows<2>(a, r, e_block, nv, s_afr, s_scl, lh, ring, s_tile[wave]);
    }
    if (with_hist) {
        __syncthreads();
        uint32_t* ghist = a.hist + r * kHistBins;
        for (int i = tid; i < kHistBins; i += kF4Threads) {
            const uint32_t c = lhist[i];
            if (c) atomicAdd(&ghist[i], c);
        }
    }
}

// Fallback for index widths the streaming kernel does not tile: one thread per
// entry, same arithmetic and the same certification.
__global__ __launch_bounds__(256) void score_exact_generic_kernel(ScoreArgs a) {
    const int64_t r = blockIdx.y;
    const int64_t nv = row_valid(a, r);
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= nv) return;
    const float res = generic_entry_score(a, r, slot_entry(a, r, e));
    a.scores[r * a.ld + e] = res;
    if (a.hist) atomicAdd(&a.hist[r * kHistBins + (sort_key(res) >> (32 - kHistBits))], 1u);
}

// Which scoring kernel a call takes, with its tiling (n_eblk, blocks, per_xcd
// filled in a).  ROWS: several rows share key loads; FP4: FP4 keys with K = 256
// on the matrix cores; STREAM: one row per workgroup tile; GENERIC: one thread
// per entry.
enum class ScorePath { ROWS, FP4, STREAM, GENERIC };

static ScorePath plan_score(ScoreArgs& a, int* cpl_out, int* qr_out) {
    const int64_t R = (int64_t)a.B * a.Qs;
    const int eb = a.dtype == 0 ? a.K * 2 : a.dtype == 1 ? a.K : a.K / 2;  // key bytes per entry
    const int cpl = eb / 128;
    *cpl_out = cpl;
    *qr_out = 1;
    const bool fast = eb % 128 == 0 && (cpl == 1 || cpl == 2 || cpl == 4 || cpl == 8);
    if (a.dtype == 0 && a.Qs >= 2 && !a.pool && a.fix_cnt && eb % 128 == 0 && (cpl == 2 || cpl == 4)) {
        const int QR = a.Qs <= 5 ? a.Qs : 4;
        *qr_out = QR;
        a.n_eblk = (a.N + kRowsEntriesPerBlock - 1) / kRowsEntriesPerBlock;
        a.blocks = a.n_eblk * a.B * ((a.Qs + QR - 1) / QR);
        a.per_xcd = (a.blocks + 7) / 8;
        return ScorePath::ROWS;
    }
    if (a.dtype == 2 && a.K == 256 && !a.pool) {
        a.n_eblk = (a.N + kF4EntriesPerBlock - 1) / kF4EntriesPerBlock;
        a.blocks = a.n_eblk * R;
        a.per_xcd = (a.blocks + 7) / 8;
        return ScorePath::FP4;
    }
    if (fast) {
        a.n_eblk = (a.N + kScoreEntriesPerBlock - 1) / kScoreEntriesPerBlock;
        a.blocks = a.n_eblk * R;
        a.per_xcd = (a.blocks + 7) / 8;
        // e4m3 keys with K = 256, one query row per sequence, no pool: a.persist
        // resident workgroups per row, each streaming a run of the row's blocks (no
        // workgroup turnover; one histogram flush per workgroup)
        a.persist = 0;
        if (a.dtype == 1 && cpl == 2 && a.Qs == 1 && !a.pool && a.blocks > kPersistResident) {
            int64_t P = (kPersistResident + R / 2) / R;
            if (P < 1) P = 1;
            if (P > a.n_eblk) P = a.n_eblk;
            a.persist = P;
        }
        return ScorePath::STREAM;
    }
    return ScorePath::GENERIC;
}

int64_t score_grid_threads(const ScoreArgs& args) {
    ScoreArgs a = args;
    const int64_t R = (int64_t)a.B * a.Qs;
    if (R == 0 || a.N == 0) return 0;
    int cpl, qr;
    switch (plan_score(a, &cpl, &qr)) {
        case ScorePath::ROWS: return 8 * a.per_xcd * kScoreThreads;
        case ScorePath::FP4: return 8 * a.per_xcd * kF4Threads;
        case ScorePath::STREAM: return (a.persist > 0 ? R * a.persist : 8 * a.per_xcd) * kStreamThreads;
        default: return (a.N + 255) / 256 * 256;
    }
}

__global__ __launch_bounds__(256) void score_tail_kernel(ScoreArgs a, int64_t e0) {
    const int64_t r = blockIdx.y;
    const int64_t e = e0 + (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e < a.N && e >= row_valid(a, r)) a.scores[r * a.ld + e] = -INFINITY;
}

hipError_t launch_score_tail(const ScoreArgs& a, hipStream_t stream) {
    const int64_t R = (int64_t)a.B * a.Qs;
    if (R == 0 || a.N == 0 || a.pool || (!a.nvb && a.causal < 0)) return hipSuccess;
    // row 0 sees the fewest entries; nothing before its cut is hidden in any row
    int64_t first = a.nvb ? 0 : (a.causal + 1 < a.N ? a.causal + 1 : a.N);
    first = first / 256 * 256;
    if (first >= a.N) return hipSuccess;
    const dim3 grid((unsigned)((a.N - first + 255) / 256), (unsigned)R);
    hipLaunchKernelGGL(score_tail_kernel, grid, dim3(256), 0, stream, a, first);
    return hipGetLastError();
}

hipError_t launch_score_exact(const ScoreArgs& args, hipStream_t stream) {
    ScoreArgs a = args;
    const int64_t R = (int64_t)a.B * a.Qs;
    if (R == 0 || a.N == 0) return hipSuccess;
    int cpl, QR;
    const ScorePath path = plan_score(a, &cpl, &QR);
    if (path == ScorePath::ROWS) {
        // several rows of a sequence share every key load
        const dim3 grid((unsigned)(8 * a.per_xcd));
#define CSA2_ROWS_LAUNCH(CPLV, QRV)                                                                      \
    if (cpl == CPLV && QR == QRV)                                                                        \
        hipLaunchKernelGGL((score_rows_kernel<CPLV, QRV>), grid, dim3(kScoreThreads), 0, stream, a);
        CSA2_ROWS_LAUNCH(2, 2)
        CSA2_ROWS_LAUNCH(2, 3)
        CSA2_ROWS_LAUNCH(2, 4)
        CSA2_ROWS_LAUNCH(2, 5)
        CSA2_ROWS_LAUNCH(4, 2)
        CSA2_ROWS_LAUNCH(4, 3)
        CSA2_ROWS_LAUNCH(4, 4)
        CSA2_ROWS_LAUNCH(4, 5)
#undef CSA2_ROWS_LAUNCH
        hipLaunchKernelGGL(score_fixup_kernel, dim3(256), dim3(kScoreThreads), 0, stream, a);
    } else if (path == ScorePath::FP4) {
        hipLaunchKernelGGL(score_fp4_mfma_kernel, dim3((unsigned)(8 * a.per_xcd)), dim3(kF4Threads), 0, stream, a);

    } else if (path == ScorePath::STREAM) {
        const bool pool = a.pool != nullptr;
        const dim3 grid((unsigned)(8 * a.per_xcd));
        if (a.persist > 0)  // plan_score sets it for e4m3 keys with K = 256 only
            hipLaunchKernelGGL((score_exact_kernel<1, 2, false, true>), dim3((unsigned)(R * a.persist)),
                               dim3(kStreamThreads), 0, stream, a);
#define CSA2_SCORE_LAUNCH(DTV, CPLV)                                                                   \
    if (a.persist == 0 && a.dtype == DTV && cpl == CPLV) {                                           \
        if (pool)                                                                                    \
            hipLaunchKernelGGL((score_exact_kernel<DTV, CPLV, true, false>), grid, dim3(kStreamThreads), 0, stream, a); \
        else                                                                                         \
            hipLaunchKernelGGL((score_exact_kernel<DTV, CPLV, false, false>), grid, dim3(kStreamThreads), 0, stream, a); \
    }
        CSA2_SCORE_LAUNCH(0, 1)
        CSA2_SCORE_LAUNCH(0, 2)
        CSA2_SCORE_LAUNCH(0, 4)
        CSA2_SCORE_LAUNCH(0, 8)
        CSA2_SCORE_LAUNCH(1, 1)
        CSA2_SCORE_LAUNCH(1, 2)
        CSA2_SCORE_LAUNCH(1, 4)
        CSA2_SCORE_LAUNCH(1, 8)
        CSA2_SCORE_LAUNCH(2, 1)
        CSA2_SCORE_LAUNCH(2, 2)
        CSA2_SCORE_LAUNCH(2, 4)
        CSA2_SCORE_LAUNCH(2, 8)
#undef CSA2_SCORE_LAUNCH
    } else {
        dim3 grid((unsigned)((a.N + 255) / 256), (unsigned)R);
        hipLaunchKernelGGL(score_exact_generic_kernel, grid, dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace csa2
