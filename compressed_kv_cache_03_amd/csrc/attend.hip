// S5+S6 - Gather the selected FP4 entries, dequantise them in registers and
// attend over them together with the query's window, one joint softmax.
//
// "Why Is DeepSeek V4.1 Flash So Fast?", sections 3-4 (attention over the
// retrieved compressed positions plus the recent 128-token window);
// "DeepSeek-V4.1-Flash", "Sharing the cache across layers" (each layer uses its
// own queries and window).  An entry is one D-vector used as key and value and
// shared by all Hq heads; window keys and values are bf16 rows.
//
// Split-k with an online softmax: a workgroup takes up to 128 keys of one query
// row (a slice of the selection, or of the window), streams them through LDS in
// sub-chunks, keeps (m, l) per head and the unnormalised output in registers,
// and writes one partial (o, m, l).  attend_combine_kernel merges the partials
// of a row in split order (m = max m_s, o = sum e^(m_s-m) o_s / sum e^(m_s-m) l_s),
// so the result does not depend on scheduling.
#include "common.h"
#include "launch.h"

namespace csa2 {

constexpr int kAttThreads = 256;
constexpr int kKeysPerSplit = 128;
constexpr int kMaxOut = 32;  // outputs per thread: Hq*D/256 rounded up to 8-wide groups

// e2m1 magnitudes (OCP MX FP4)
__constant__ float kE2M1[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

CSA2_DEV float e2m1(uint32_t c) {
    const float m = kE2M1[c & 7u];
    return (c & 8u) ? -m : m;
}

// LDS of one workgroup for a sub-chunk of `sub` keys: q [Hq][D+1], K [sub][D+1]
// (padded: logits walk d with different keys per lane), V [sub][D] (PV reads
// contiguous d), p [Hq][sub], per-head m, l, alpha, and the key validity list.
// The q and K regions are rounded up to 4 floats so that V rows stay 16-byte aligned.
CSA2_DEV_HOST_INLINE int align4(int x) { return (x + 3) & ~3; }

static size_t attend_lds(int Hq, int D, int sub) {
    return 4u * ((size_t)align4(Hq * (D + 1)) + (size_t)align4(sub * (D + 1)) + (size_t)sub * D +
                 (size_t)Hq * sub + 3u * Hq + sub);
}

static int attend_sub(int Hq, int D) {
    for (int sub = 32; sub >= 4; sub >>= 1)
        if (attend_lds(Hq, D, sub) <= 65536) return sub;
    return 4;
}

void attend_splits(int Hq, int D, int k, int W, int* splits_g, int* splits_w) {
    (void)Hq;
    (void)D;
    *splits_g = (k + kKeysPerSplit - 1) / kKeysPerSplit;
    *splits_w = (W + kKeysPerSplit - 1) / kKeysPerSplit;
}

__global__ __launch_bounds__(kAttThreads) void attend_partial_kernel(AttendArgs a, int sub,
                                                                     int splits_g, int splits) {
    extern __shared__ float lds[];
    const int Hq = a.Hq, D = a.D, DP = D + 1;
    float* q_s = lds;                       // [Hq][DP]
    float* k_s = q_s + align4(Hq * DP);     // [sub][DP]
    float* v_s = k_s + align4(sub * DP);    // [sub][D], 16-byte aligned rows
    float* p_s = v_s + sub * D;             // [Hq][sub]
    float* m_s = p_s + Hq * sub;            // [Hq]
    float* l_s = m_s + Hq;                  // [Hq]
    float* al_s = l_s + Hq;                 // [Hq]
    int* valid_s = reinterpret_cast<int*>(al_s + Hq);  // [sub]

    const int64_t r = blockIdx.y;
    const int split = blockIdx.x;
    const int64_t b = r / a.Qs, i = r % a.Qs;
    const bool is_win = split >= splits_g;
    const int t0 = (is_win ? split - splits_g : split) * kKeysPerSplit;
    const int nkeys = is_win ? a.W : a.k;
    const int64_t wrows = (int64_t)a.Qs + a.W - 1;
    const int64_t wfirst = a.wlen ? wrows - a.wlen[b] : 0;

    // query row, bf16 -> fp32; per-head softmax state
    const uint16_t* qr = a.q + r * (int64_t)Hq * D;
    for (int e = threadIdx.x; e < Hq * D; e += kAttThreads) q_s[(e / D) * DP + (e % D)] = bf16_to_f32(qr[e]);
    for (int h = threadIdx.x; h < Hq; h += kAttThreads) {
        m_s[h] = -INFINITY;
        l_s[h] = 0.0f;
    }

    // output ownership: thread t holds 8 consecutive d of one head per pass
    const int tph = D / 8;                 // threads per head
    const int hpp = kAttThreads / tph;     // heads per pass
    const int passes = (Hq + hpp - 1) / hpp;
    const int my_h0 = threadIdx.x / tph, my_d0 = (threadIdx.x % tph) * 8;
    const bool owns = my_h0 < hpp;         // when tph does not divide 256, the last threads idle
    float o[kMaxOut];
#pragma unroll
    for (int u = 0; u < kMaxOut; ++u) o[u] = 0.0f;

    const int t_end = min(t0 + kKeysPerSplit, nkeys);
    for (int tb = t0; tb < t_end; tb += sub) {
        __syncthreads();  // previous sub-chunk fully consumed (and q_s, m_s ready)
        if (threadIdx.x < sub) {
            const int t = tb + threadIdx.x;
            int v = -1;
            if (t < t_end) {
                if (!is_win) {
                    const int32_t j = a.idx[r * a.k + t];
                    v = (j >= 0 && j < a.N) ? j : -1;
                } else {
                    const int64_t row = i + t;
                    v = (row >= wfirst && row < wrows) ? t : -1;
                }
            }
            valid_s[threadIdx.x] = v;
        }
        __syncthreads();
        if (!is_win) {
            const int per_row = D / 8;  // 8 elements (4 code bytes) per task
            for (int task = threadIdx.x; task < sub * per_row; task += kAttThreads) {
                const int t = task / per_row, part = task % per_row;
                const int32_t j = valid_s[t];
                float v8[8];
                if (j >= 0) {
                    const int64_t rec = b * a.N + j;
                    const uint32_t w = *reinterpret_cast<const uint32_t*>(a.codes + rec * (D / 2) + part * 4);
                    const float sc = a.scales[rec * (D / 32) + part / 4];
#pragma unroll
                    for (int u = 0; u < 8; ++u) v8[u] = e2m1((w >> (4 * u)) & 15u) * sc;
                } else {
#pragma unroll
                    for (int u = 0; u < 8; ++u) v8[u] = 0.0f;
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    k_s[t * DP + part * 8 + u] = v8[u];
                    v_s[t * D + part * 8 + u] = v8[u];
                }
            }
        } else {
            for (int e = threadIdx.x; e < sub * D; e += kAttThreads) {
                const int t = e / D, d = e % D;
                const bool ok = valid_s[t] >= 0;
                const int64_t row = b * wrows + i + tb + t;
                k_s[t * DP + d] = ok ? bf16_to_f32(a.wk[row * D + d]) : 0.0f;
                v_s[t * D + d] = ok ? bf16_to_f32(a.wv[row * D + d]) : 0.0f;
            }
        }
        __syncthreads();
        // logits of this sub-chunk
        for (int task = threadIdx.x; task < Hq * sub; task += kAttThreads) {
            const int h = task / sub, t = task % sub;
            float z = -INFINITY;
            if (valid_s[t] >= 0) {
                float acc = 0.0f;
                const float* qh = q_s + h * DP;
                const float* kt = k_s + t * DP;
                for (int d = 0; d < D; ++d) acc = fmaf(qh[d], kt[d], acc);
                z = a.sm_scale * acc;
            }
            p_s[h * sub + t] = z;
        }
        __syncthreads();
        // online softmax update per head
        for (int h = threadIdx.x; h < Hq; h += kAttThreads) {
            const float m_old = m_s[h];
            float m_new = m_old;
            for (int t = 0; t < sub; ++t) m_new = fmaxf(m_new, p_s[h * sub + t]);
            float lsum = 0.0f;
            for (int t = 0; t < sub; ++t) {
                const float z = p_s[h * sub + t];
                const float p = (z == -INFINITY) ? 0.0f : expf(z - m_new);
                p_s[h * sub + t] = p;
                lsum += p;
            }
            const float alpha = (m_old == -INFINITY) ? 0.0f : expf(m_old - m_new);
            al_s[h] = alpha;
            l_s[h] = l_s[h] * alpha + lsum;
            m_s[h] = m_new;
        }
        __syncthreads();
        // o = o * alpha + p V
        for (int ps = 0; ps < passes && owns; ++ps) {
            const int h = ps * hpp + my_h0;
            if (h >= Hq) break;
            const float alpha = al_s[h];
            float acc[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) acc[u] = o[ps * 8 + u] * alpha;
            for (int t = 0; t < sub; ++t) {
                const float p = p_s[h * sub + t];
                const float4 va = *reinterpret_cast<const float4*>(v_s + t * D + my_d0);
                const float4 vb = *reinterpret_cast<const float4*>(v_s + t * D + my_d0 + 4);
                acc[0] = fmaf(p, va.x, acc[0]);
                acc[1] = fmaf(p, va.y, acc[1]);
                acc[2] = fmaf(p, va.z, acc[2]);
                acc[3] = fmaf(p, va.w, acc[3]);
                acc[4] = fmaf(p, vb.x, acc[4]);
                acc[5] = fmaf(p, vb.y, acc[5]);
                acc[6] = fmaf(p, vb.z, acc[6]);
                acc[7] = fmaf(p, vb.w, acc[7]);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) o[ps * 8 + u] = acc[u];
        }
    }
    __syncthreads();
    float* part = a.part + ((r * splits + split) * (int64_t)Hq) * (D + 2);
    for (int ps = 0; ps < passes && owns; ++ps) {
        const int h = ps * hpp + my_h0;
        if (h >= Hq) break;
#pragma unroll
        for (int u = 0; u < 8; ++u) part[h * (D + 2) + my_d0 + u] = o[ps * 8 + u];
    }
    for (int h = threadIdx.x; h < Hq; h += kAttThreads) {
        part[h * (D + 2) + D] = m_s[h];
        part[h * (D + 2) + D + 1] = l_s[h];
    }
}

// One workgroup per (row, head); thread d owns output element d.
__global__ __launch_bounds__(256) void attend_combine_kernel(AttendArgs a, int splits) {
    __shared__ float red[256];
    __shared__ float M_s;
    const int64_t r = blockIdx.x;
    const int h = blockIdx.y;
    const int Hq = a.Hq, D = a.D;
    const float* part = a.part + r * (int64_t)splits * Hq * (D + 2);
    float m = -INFINITY;
    for (int s = threadIdx.x; s < splits; s += blockDim.x) m = fmaxf(m, part[((int64_t)s * Hq + h) * (D + 2) + D]);
    red[threadIdx.x] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        float M = -INFINITY;
        for (int t = 0; t < (int)blockDim.x; ++t) M = fmaxf(M, red[t]);
        M_s = M;
    }
    __syncthreads();
    const float M = M_s;
    float L = 0.0f, O = 0.0f;
    const int d = threadIdx.x;
    if (M != -INFINITY) {
        for (int s = 0; s < splits; ++s) {
            const float* ps = part + ((int64_t)s * Hq + h) * (D + 2);
            const float ms = ps[D];
            if (ms == -INFINITY) continue;
            const float w = expf(ms - M);
            L = fmaf(w, ps[D + 1], L);
            if (d < D) O = fmaf(w, ps[d], O);
        }
    }
    if (d < D) a.out[(r * Hq + h) * D + d] = M == -INFINITY ? 0.0f : O / L;
    if (d == 0 && a.lse) a.lse[r * Hq + h] = M == -INFINITY ? -INFINITY : M + logf(L);
}

hipError_t launch_attend(const AttendArgs& a, hipStream_t stream) {
    const int64_t R = (int64_t)a.B * a.Qs;
    if (R == 0) return hipSuccess;
    const int sub = attend_sub(a.Hq, a.D);
    int sg, sw;
    attend_splits(a.Hq, a.D, a.k, a.W, &sg, &sw);
    const int splits = sg + sw;
    if (splits > 0) {
        const size_t lds = attend_lds(a.Hq, a.D, sub);
        hipLaunchKernelGGL(attend_partial_kernel, dim3((unsigned)splits, (unsigned)R), dim3(kAttThreads),
                           lds, stream, a, sub, sg, splits);
    }
    const unsigned threads = a.D <= 64 ? 64u : (a.D <= 128 ? 128u : 256u);
    hipLaunchKernelGGL(attend_combine_kernel, dim3((unsigned)R, (unsigned)a.Hq), dim3(threads), 0, stream,
                       a, splits);
    return hipGetLastError();
}

}  // namespace csa2
