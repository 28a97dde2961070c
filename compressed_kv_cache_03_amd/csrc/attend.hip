// S5+S6 - Gather the selected FP4 entries, dequantise them in registers and
// attend over them together with the query's window, one joint softmax.
//
// "Why Is DeepSeek V4.1 Flash So Fast?", sections 3-4 (attention over the
// retrieved compressed positions plus the recent 128-token window);
// "DeepSeek-V4.1-Flash", "Sharing the cache across layers" (each layer uses its
// own queries and window).  An entry is one D-vector used as key and value and
// shared by all query heads; window keys and values are bf16 rows.
//
// One wave works on one (query row, split of the key list, group of 16 heads)
// and walks its keys 32 at a time.  Both contractions run on bf16 MFMA
// (v_mfma_f32_16x16x32_bf16) in transposed form so that heads are the MFMA
// columns and every per-head quantity stays in one lane:
//   logits  S^T[key][h] = sum_d K[key][d] q[h][d]: one MFMA per 32-element scale
//           block (A = the block's e2m1 codes converted exactly to bf16, B = q),
//           then z = sum_blk S_blk^T * scale[key][blk] in fp32;
//   output  O^T[d][h] += sum_key V^T[d][key] (p[key][h] scale[key][blk(d)]):
//           A = exact codes of 16 d-rows of one block, B = p*scale split into a
//           bf16 high part and a bf16 remainder (two MFMAs, 16 significant bits).
// Products are exact (bf16 x e2m1, bf16 x bf16) and accumulate in fp32; the
// only rounding beyond fp32 is the 2^-16 relative split of p*scale.
//
// Register layouts (lane = m + 16 g, m = lane % 16, g = lane / 16):
//   MFMA A[row][kslot]: lane holds row m, kslots 8g .. 8g+7
//   MFMA B[kslot][col]: lane holds column m, kslots 8g .. 8g+7
//   MFMA C[row][col]  : lane holds column m, rows 4g .. 4g+3
// Logit tile kt (keys 16kt .. 16kt+15 of a step) leaves lane (h=m, g) with keys
// 16kt + 4g + i (i = 0..3); the output contraction uses kslot 8g+e <-> key
// 4g+e (e < 4) or 16+4g+(e-4) (e >= 4), which is exactly what the lane holds.
// Output tile (blk, half) has rows d = 32 blk + 2 row + half, so one code byte
// (16 blk + row) feeds both halves and every tile lies in one scale block.
//
// Splits: the key list is the selection padded to a multiple of 32 followed by
// the window padded to a multiple of 32; a split is a run of 32-key steps.
// With one split per row the wave writes the normalised output; otherwise it
// writes a partial (o, m, l) and attend_combine_kernel merges the partials of
// a row in split order, so results do not depend on scheduling.
#include "common.h"
#include "launch.h"

namespace csa2 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kStep = 32;          // keys per step
constexpr int kTargetWaves = 1024; // below this many waves a row's keys are split
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

CSA2_DEV bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Two e2m1 codes of byte `sel` of w -> bf16 pair (low nibble in the low half), exact.
template <int SEL>
CSA2_DEV uint32_t fp4x2_bf16(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL));
}

// Eight codes of one dword -> eight bf16 values in element order.
CSA2_DEV u32x4 fp4x8_bf16(uint32_t w) {
    return u32x4{fp4x2_bf16<0>(w), fp4x2_bf16<1>(w), fp4x2_bf16<2>(w), fp4x2_bf16<3>(w)};
}

// Low (SEL=0) or high (SEL=1) bf16 halves of a and b packed as (a, b).
CSA2_DEV uint32_t pack_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
CSA2_DEV uint32_t pack_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// x = hi + lo in bf16 pairs: hi = x with its low 16 bits cleared, lo = the
// exact remainder x - hi rounded to bf16, so |x - hi - lo| <= 2^-16 |x|.
CSA2_DEV void split_bf16(const float (&x)[8], u32x4& hi, u32x4& lo) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t u0 = __float_as_uint(x[2 * q]), u1 = __float_as_uint(x[2 * q + 1]);
        const float r0 = x[2 * q] - __uint_as_float(u0 & 0xffff0000u);
        const float r1 = x[2 * q + 1] - __uint_as_float(u1 & 0xffff0000u);
        hi[q] = __builtin_amdgcn_perm(u1, u0, 0x07060302u);
        lo[q] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{r0, r1}, bf16x2));
    }
}

CSA2_DEV f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

CSA2_DEV int kslot_key(int g, int e) { return e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4); }

void attend_splits(int64_t R, int Hq, int D, int k, int W, int* splits, int* chunk) {
    (void)D;
    const int kv = ((k + kStep - 1) / kStep + (W + kStep - 1) / kStep) * kStep;
    const int64_t groups = R * ((Hq + 15) / 16);
    const int steps = kv / kStep;
    int64_t want = (kTargetWaves + groups - 1) / groups;  // splits per row to reach the target
    if (want < 1) want = 1;
    if (want > (steps + 1) / 2) want = (steps + 1) / 2;   // at least two steps per split
    if (want < 1) want = 1;
    const int steps_per = (int)((steps + want - 1) / want);
    *chunk = steps_per * kStep;
    *splits = steps == 0 ? 1 : (steps + steps_per - 1) / steps_per;
}

// Online-softmax state of one wave: this lane's head h, its running maximum
// (log2 units), its share of the normaliser (the lane's own keys) and the
// unnormalised output tiles O^T[d][h], d = 32 blk + 2(4g+i) + half.
template <int NB>
struct SoftmaxState {
    f32x4 o[NB][2];
    float m_run, l_run;

    __device__ __forceinline__ void init() {
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) o[blk][0] = o[blk][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        m_run = -INFINITY;
        l_run = 0.0f;
    }

    // z: log2-scaled logits of the step's keys kslot_key(g, e) (-inf = masked),
    // at least one finite.  Returns p = 2^(z - m_run) in kslot order.  The
    // reference m_run moves (and o, l are rescaled) only when a logit exceeds
    // it by more than kLazy, so p <= 2^kLazy and the common step rescales
    // nothing; the result is the same softmax since o and l share the factor.
    __device__ __forceinline__ void update(const float (&z)[8], float (&p)[8]) {
        constexpr float kLazy = 8.0f;
        float tmax = -INFINITY;
#pragma unroll
        for (int e = 0; e < 8; ++e) tmax = fmaxf(tmax, z[e]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        if (__any(tmax > m_run + kLazy)) {  // wave-uniform
            const float m_new = fmaxf(m_run, tmax);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int blk = 0; blk < NB; ++blk)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) o[blk][hf] *= alpha;
            m_run = m_new;
        }
        float psum = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            p[e] = __builtin_amdgcn_exp2f(z[e] - m_run);
            psum += p[e];
        }
        l_run += psum;
    }

    // O^T[tile blk] += V^T (bhi + blo) for the two half tiles of block blk;
    // cv[e] holds the bf16 pair (d even, d odd) of key kslot_key(g, e).
    __device__ __forceinline__ void accumulate(int blk, const uint32_t (&cv)[8], u32x4 bhi, u32x4 blo) {
        const u32x4 a0{pack_lo(cv[0], cv[1]), pack_lo(cv[2], cv[3]), pack_lo(cv[4], cv[5]),
                       pack_lo(cv[6], cv[7])};
        const u32x4 a1{pack_hi(cv[0], cv[1]), pack_hi(cv[2], cv[3]), pack_hi(cv[4], cv[5]),
                       pack_hi(cv[6], cv[7])};
        o[blk][0] = mfma(a0, bhi, o[blk][0]);
        o[blk][1] = mfma(a1, bhi, o[blk][1]);
        o[blk][0] = mfma(a0, blo, o[blk][0]);
        o[blk][1] = mfma(a1, blo, o[blk][1]);
    }
};

template <int NB>
__global__ __launch_bounds__(64) void attend_kernel(AttendArgs a, int chunk, int splits) {
    constexpr int D = 32 * NB;
    constexpr int PITCH = 4 * NB + 4;  // staged code row, dwords (16-byte aligned rows)
    __shared__ __attribute__((aligned(16))) uint32_t lcode[kStep * PITCH];
    __shared__ __attribute__((aligned(16))) float lscale[kStep * NB];

    const int lane = threadIdx.x;
    const int m = lane & 15, g = lane >> 4;
    const int64_t r = blockIdx.y;
    const int split = blockIdx.x;
    const int h = blockIdx.z * 16 + m;  // head of this lane's MFMA column
    const bool hvalid = h < a.Hq;
    const int64_t b = r / a.Qs, qi = r % a.Qs;
    const int k32 = (a.k + kStep - 1) / kStep * kStep;
    const int kv = k32 + (a.W + kStep - 1) / kStep * kStep;
    const int v0 = split * chunk;
    const int v1 = min(v0 + chunk, kv);
    const float c2 = a.sm_scale * kLog2e;

    // q fragment: q[r][h][32 blk + 8g .. +7]
    u32x4 qf[NB];
    {
        const uint16_t* qh = a.q + (r * a.Hq + (hvalid ? h : 0)) * (int64_t)D + 8 * g;
#pragma unroll
        for (int blk = 0; blk < NB; ++blk)
            qf[blk] = hvalid ? *reinterpret_cast<const u32x4*>(qh + 32 * blk) : u32x4{0u, 0u, 0u, 0u};
    }
    SoftmaxState<NB> st;
    st.init();

    // ------------------------------------------------------------------
    // Selected entries, software-pipelined: the indices of step s+2 and the
    // records of step s+1 are in flight while step s computes.  Lanes 0..31
    // hold one index each; lane (x = lane/2, part = lane%2) carries half of
    // record x's codes, lane x < 32 its NB scales.  Loads are unconditional,
    // from clamped in-bounds addresses, so that they issue back to back and
    // nothing waits for them before it is used: an index slot beyond k reads
    // slot k-1 and an empty or out-of-range entry reads record 0; such keys get
    // logit -inf, so p = 0 multiplies finite data.  The last step prefetches a
    // step it does not use.  With no entries (N = 0) this part is skipped.
    const int vsel_end = a.N > 0 ? min(v1, k32) : v0;
    auto load_idx = [&](int v) -> int32_t {
        return a.idx[r * a.k + min(v + (lane & (kStep - 1)), a.k - 1)];
    };
    auto valid_j = [&](int v, int32_t j) -> bool {
        return lane < kStep && v + lane < a.k && j >= 0 && j < a.N;
    };
    uint32_t cw[2 * NB];  // prefetched codes
    float sw[NB];         // prefetched scales
    auto load_rec = [&](int v, int32_t jraw) {
        const int32_t j = valid_j(v, jraw) ? jraw : 0;
        const int jx = __shfl(j, lane >> 1);
        const uint32_t* src = reinterpret_cast<const uint32_t*>(
            a.codes + (b * a.N + jx) * (int64_t)(16 * NB)) + (lane & 1) * (2 * NB);
        // a half row is 2*NB dwords at an 8*NB-byte offset: 16-byte pieces
        // when NB is even, 8-byte pieces otherwise
        if constexpr (NB % 2 == 0) {
#pragma unroll
            for (int c = 0; c < NB / 2; ++c) {
                const u32x4 w = *reinterpret_cast<const u32x4*>(src + 4 * c);
                cw[4 * c] = w[0]; cw[4 * c + 1] = w[1]; cw[4 * c + 2] = w[2]; cw[4 * c + 3] = w[3];
            }
        } else {
#pragma unroll
            for (int c = 0; c < NB; ++c) {
                const uint2 w = *reinterpret_cast<const uint2*>(src + 2 * c);
                cw[2 * c] = w.x; cw[2 * c + 1] = w.y;
            }
        }
        const float* sp = a.scales + (b * a.N + j) * (int64_t)NB;
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) sw[blk] = sp[blk];
    };
    if (v0 < vsel_end) {
        int32_t j_cur = load_idx(v0);
        load_rec(v0, j_cur);
        int32_t j_nxt = load_idx(v0 + kStep);
        for (int v = v0; v < vsel_end; v += kStep) {
            // the prefetched records of this step go to LDS; the next step's loads start
            const uint64_t vmask = __ballot(valid_j(v, j_cur));
            {
                uint32_t* dst = lcode + (lane >> 1) * PITCH + (lane & 1) * (2 * NB);
                if constexpr (NB % 2 == 0) {
#pragma unroll
                    for (int c = 0; c < NB / 2; ++c)
                        *reinterpret_cast<u32x4*>(dst + 4 * c) = u32x4{cw[4 * c], cw[4 * c + 1], cw[4 * c + 2], cw[4 * c + 3]};
                } else {
#pragma unroll
                    for (int c = 0; c < NB; ++c)
                        *reinterpret_cast<uint2*>(dst + 2 * c) = uint2{cw[2 * c], cw[2 * c + 1]};
                }
                // an empty slot's scale is staged as 0, so its p = 0 meets finite data
                // even where the record it was clamped to holds a non-finite scale
                if (lane < kStep) {
                    const bool live = (vmask >> lane) & 1u;
#pragma unroll
                    for (int blk = 0; blk < NB; ++blk) lscale[lane * NB + blk] = live ? sw[blk] : 0.0f;
                }
            }
            load_rec(v + kStep, j_nxt);
            j_cur = j_nxt;
            j_nxt = load_idx(v + 2 * kStep);
            __syncthreads();
            if (vmask != 0) {  // wave-uniform
                float sc[8][NB];  // scale[kslot_key(g, e)][blk]
#pragma unroll
                for (int e = 0; e < 8; ++e)
#pragma unroll
                    for (int blk = 0; blk < NB; ++blk) sc[e][blk] = lscale[kslot_key(g, e) * NB + blk];
                // logits S^T = K q^T, block by block, scaled per (key, block)
                float z[8];
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    f32x4 acc[NB];
#pragma unroll
                    for (int blk = 0; blk < NB; ++blk) {
                        const uint32_t w = lcode[(16 * kt + m) * PITCH + 4 * blk + g];
                        acc[blk] = mfma(fp4x8_bf16(w), qf[blk], f32x4{0.f, 0.f, 0.f, 0.f});
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float sz = 0.0f;
#pragma unroll
                        for (int blk = 0; blk < NB; ++blk) sz = fmaf(acc[blk][i], sc[4 * kt + i][blk], sz);
                        const int x = 16 * kt + 4 * g + i;
                        z[4 * kt + i] = (vmask >> x) & 1u ? sz * c2 : -INFINITY;
                    }
                }
                float p[8];
                st.update(z, p);
                // output: O^T += V^T (P scale)^T, one scale block at a time
                const uint8_t* lbytes = reinterpret_cast<const uint8_t*>(lcode);
#pragma unroll
                for (int blk = 0; blk < NB; ++blk) {
                    float pv[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) pv[e] = p[e] * sc[e][blk];
                    u32x4 bhi, blo;
                    split_bf16(pv, bhi, blo);
                    uint32_t cv[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        cv[e] = fp4x2_bf16<0>(lbytes[kslot_key(g, e) * (PITCH * 4) + 16 * blk + m]);
                    st.accumulate(blk, cv, bhi, blo);
                }
            }
            __syncthreads();  // staged records consumed before the next step overwrites them
        }
    }

    // ------------------------------------------------------------------
    // Window rows: step keys x = 0..31 are window slots t = v - k32 + x, buffer
    // row qi + t, valid when t < W and the row is among the last wlen[b] rows.
    // Rows are clamped to the last window row for the loads.
    {
        const int64_t wrows = (int64_t)a.Qs + a.W - 1;
        const int64_t wfirst = a.wlen ? wrows - a.wlen[b] : 0;
        for (int v = max(v0, k32); v < v1; v += kStep) {
            const int t0 = v - k32;
            const int t = t0 + lane;
            const uint64_t vmask = __ballot(lane < kStep && t < a.W && qi + t >= wfirst);
            if (vmask == 0) continue;  // wave-uniform
            auto wrow = [&](int x) -> int64_t { return b * wrows + qi + min(t0 + x, a.W - 1); };
            u32x4 kw[2][NB];
            uint32_t wvv[8][NB];  // bf16 pair (32 blk + 2m, +1) of key kslot_key(g, e)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int blk = 0; blk < NB; ++blk)
                    kw[kt][blk] = *reinterpret_cast<const u32x4*>(a.wk + wrow(16 * kt + m) * D + 32 * blk + 8 * g);
#pragma unroll
            for (int e = 0; e < 8; ++e)
#pragma unroll
                for (int blk = 0; blk < NB; ++blk)
                    wvv[e][blk] = *reinterpret_cast<const uint32_t*>(a.wv + wrow(kslot_key(g, e)) * D + 32 * blk + 2 * m);
            // value rows outside the valid tail (or past W) are zeroed: the caller may
            // leave anything there, and p = 0 times a NaN or Inf would poison the sum
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (!((vmask >> kslot_key(g, e)) & 1u))
#pragma unroll
                    for (int blk = 0; blk < NB; ++blk) wvv[e][blk] = 0u;
            float z[8];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int blk = 0; blk < NB; ++blk) acc = mfma(kw[kt][blk], qf[blk], acc);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int x = 16 * kt + 4 * g + i;
                    z[4 * kt + i] = (vmask >> x) & 1u ? acc[i] * c2 : -INFINITY;
                }
            }
            float p[8];
            st.update(z, p);
            u32x4 bhi, blo;
            split_bf16(p, bhi, blo);
#pragma unroll
            for (int blk = 0; blk < NB; ++blk) {
                uint32_t cv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) cv[e] = wvv[e][blk];
                st.accumulate(blk, cv, bhi, blo);
            }
        }
    }

    // ---- finish: l over the four lanes of head h, then output or partial
    float l_tot = st.l_run + __shfl_xor(st.l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (!hvalid) return;
    // lane (h, g) owns d = 32 blk + 8g + e, e = 2i + half
    if (splits == 1) {
        const bool empty = st.m_run == -INFINITY;
        const float inv = empty ? 0.0f : 1.0f / l_tot;
        float* out = a.out + (r * a.Hq + h) * (int64_t)D + 8 * g;
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
            const f32x4 lo4{st.o[blk][0][0] * inv, st.o[blk][1][0] * inv, st.o[blk][0][1] * inv, st.o[blk][1][1] * inv};
            const f32x4 hi4{st.o[blk][0][2] * inv, st.o[blk][1][2] * inv, st.o[blk][0][3] * inv, st.o[blk][1][3] * inv};
            *reinterpret_cast<f32x4*>(out + 32 * blk) = lo4;
            *reinterpret_cast<f32x4*>(out + 32 * blk + 4) = hi4;
        }
        if (g == 0 && a.lse) a.lse[r * a.Hq + h] = empty ? -INFINITY : st.m_run * kLn2 + logf(l_tot);
    } else {
        float* part = a.part + ((r * splits + split) * (int64_t)a.Hq + h) * (D + 2);
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
            float* pd = part + 32 * blk + 8 * g;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pd[2 * i] = st.o[blk][0][i];
                pd[2 * i + 1] = st.o[blk][1][i];
            }
        }
        if (g == 0) {
            part[D] = st.m_run;
            part[D + 1] = l_tot;
        }
    }
}

// Merge of the split partials of one (row, head): thread (grp, d) folds the
// splits grp, grp + G, ... in that order with an online maximum (the loads of
// eight splits are issued together, so one memory round trip covers them),
// then group 0 folds groups 1 .. G-1 in order.  The order is fixed, so results
// do not depend on scheduling.  Partial maxima are in log2 units.
CSA2_DEV void fold(float& M, float& O, float& L, float m, float o, float l) {
    if (m == -INFINITY) return;  // a split that saw no key
    if (m > M) {
        const float c = exp2f(M - m);  // 0 while M is -inf
        O *= c;
        L *= c;
        M = m;
    }
    const float w = exp2f(m - M);
    O = fmaf(w, o, O);
    L = fmaf(w, l, L);
}

__global__ __launch_bounds__(256) void attend_combine_kernel(AttendArgs a, int splits) {
    __shared__ float sM[4], sO[256], sL[256];
    const int64_t r = blockIdx.x;
    const int h = blockIdx.y;
    const int Hq = a.Hq, D = a.D;
    const int Dp = (D + 63) / 64 * 64;
    const int G = 256 / Dp;
    const int t = threadIdx.x, d = t % Dp, grp = t / Dp;
    const int64_t stride = (int64_t)Hq * (D + 2);
    const float* part = a.part + (r * (int64_t)splits * Hq + h) * (D + 2);
    float M = -INFINITY, O = 0.0f, L = 0.0f;
    if (grp < G) {
        constexpr int U = 8;
        for (int s0 = grp; s0 < splits; s0 += U * G) {
            float ms[U], os[U], ls[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int s = s0 + u * G;
                const float* ps = part + (int64_t)(s < splits ? s : 0) * stride;
                ms[u] = s < splits ? ps[D] : -INFINITY;
                ls[u] = ps[D + 1];
                os[u] = d < D ? ps[d] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) fold(M, O, L, ms[u], os[u], ls[u]);
        }
    }
    sO[t] = O;
    sL[t] = L;
    if (d == 0 && grp < G) sM[grp] = M;
    __syncthreads();
    if (grp == 0 && d < D) {
        for (int q = 1; q < G; ++q) fold(M, O, L, sM[q], sO[q * Dp + d], sL[q * Dp + d]);
        a.out[(r * Hq + h) * D + d] = M == -INFINITY ? 0.0f : O / L;
        if (d == 0 && a.lse) a.lse[r * Hq + h] = M == -INFINITY ? -INFINITY : M * kLn2 + logf(L);
    }
}

hipError_t launch_attend(const AttendArgs& a, hipStream_t stream) {
    const int64_t R = (int64_t)a.B * a.Qs;
    if (R == 0) return hipSuccess;
    int splits, chunk;
    attend_splits(R, a.Hq, a.D, a.k, a.W, &splits, &chunk);
    const dim3 grid((unsigned)splits, (unsigned)R, (unsigned)((a.Hq + 15) / 16));
    switch (a.D / 32) {
        case 1: hipLaunchKernelGGL(attend_kernel<1>, grid, dim3(64), 0, stream, a, chunk, splits); break;
        case 2: hipLaunchKernelGGL(attend_kernel<2>, grid, dim3(64), 0, stream, a, chunk, splits); break;
        case 3: hipLaunchKernelGGL(attend_kernel<3>, grid, dim3(64), 0, stream, a, chunk, splits); break;
        case 4: hipLaunchKernelGGL(attend_kernel<4>, grid, dim3(64), 0, stream, a, chunk, splits); break;
        case 5: hipLaunchKernelGGL(attend_kernel<5>, grid, dim3(64), 0, stream, a, chunk, splits); break;
        case 6: hipLaunchKernelGGL(attend_kernel<6>, grid, dim3(64), 0, stream, a, chunk, splits); break;
        case 7: hipLaunchKernelGGL(attend_kernel<7>, grid, dim3(64), 0, stream, a, chunk, splits); break;
        case 8: hipLaunchKernelGGL(attend_kernel<8>, grid, dim3(64), 0, stream, a, chunk, splits); break;
        default: return hipErrorInvalidValue;
    }
    if (splits > 1)
        hipLaunchKernelGGL(attend_combine_kernel, dim3((unsigned)R, (unsigned)a.Hq), dim3(256), 0,
                           stream, a, splits);
    return hipGetLastError();
}

}  // namespace csa2
