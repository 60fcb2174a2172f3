// Split-KV decode for gfx950: one query token per (batch, head) over a long
// key/value cache (the "Flash-decoding" exercise of the ML compiler page).
//
// Kernel 1 (partial): one workgroup per (head, key chunk). The chunk's keys are
// streamed once from HBM with fully coalesced 16-byte loads: D/8 lanes share a
// key row (each lane owns 8 of the D columns), so one wave instruction reads
// 1 KiB of consecutive rows. Each lane group keeps its own online-softmax state
// (m, l, o) over the keys it visits, updated a block of U keys at a time
// (iThome article, "three states"); at the end the group states are merged in
// LDS with the merge rule of section 11.6 and the chunk's partial (m, l, o) is
// written to the workspace. This work is bandwidth-bound (one FMA per byte), so
// it stays on the vector ALUs: there is no contraction worth an MFMA here.
//
// Kernel 2 (combine): one workgroup of D threads per (batch, head) merges the
// chunk partials with the same rule, M = max m_s, l = sum l_s 2^(m_s - M),
// o = sum o_s 2^(m_s - M), and writes O = o / l (bf16) and
// LSE = (M + log2 l) ln 2. Empty chunks carry (-inf, 0, 0) and weigh nothing.

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

constexpr int kDecThreads = 256;
constexpr int kDecUnroll = 4;

template <int D>
__global__ __launch_bounds__(kDecThreads)
void decode_partial_kernel(const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg,
                           const uint16_t* __restrict__ Vg, float* __restrict__ ws_o,
                           float* __restrict__ ws_ml, int Nk, int S, int chunk, float scale2) {
    constexpr int LPK = D / 8;                 // lanes per key row
    constexpr int G = kDecThreads / LPK;       // key groups per workgroup
    constexpr int U = kDecUnroll;

    __shared__ float sm_m[G];
    __shared__ float sm_l[G];
    __shared__ __attribute__((aligned(16))) float sm_o[G * D];

    const int tid = threadIdx.x;
    const int g = tid / LPK;
    const int sub = tid % LPK;
    const int split = blockIdx.x % S;
    const int bh = blockIdx.x / S;

    const long long jb = (long long)split * chunk;
    const int j0 = (int)(jb < Nk ? jb : Nk);
    const int j1 = (int)(jb + chunk < Nk ? jb + chunk : Nk);

    const uint16_t* K = Kg + (size_t)bh * Nk * D + sub * 8;
    const uint16_t* V = Vg + (size_t)bh * Nk * D + sub * 8;

    float q[8];
    {
        const u32x4_t w = *(const u32x4_t*)(Qg + (size_t)bh * D + sub * 8);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            q[2 * i] = bf16_lo(w[i]) * scale2;
            q[2 * i + 1] = bf16_hi(w[i]) * scale2;
        }
    }

    float m_run = -INFINITY, l_run = 0.f;
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = 0.f;

    for (int base = j0 + g; base < j1; base += G * U) {
        u32x4_t kr[U], vr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int key = base + u * G;
            if (key < j1) {
                kr[u] = *(const u32x4_t*)(K + (size_t)key * D);
                vr[u] = *(const u32x4_t*)(V + (size_t)key * D);
            } else {
                kr[u] = u32x4_t{0u, 0u, 0u, 0u};
                vr[u] = u32x4_t{0u, 0u, 0u, 0u};
            }
        }
        float sc[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc = __builtin_fmaf(q[2 * i], bf16_lo(kr[u][i]), acc);
                acc = __builtin_fmaf(q[2 * i + 1], bf16_hi(kr[u][i]), acc);
            }
            acc = group_sum<LPK>(acc);
            sc[u] = (base + u * G < j1) ? acc : -INFINITY;
        }
        float mx = sc[0];
#pragma unroll
        for (int u = 1; u < U; ++u) mx = fmaxf(mx, sc[u]);
        const float m_new = fmaxf(m_run, mx);      // finite: key `base` is always live
        const float alpha = exp2_hw(m_run - m_new);
        m_run = m_new;
        float p[U];
        float psum = 0.f;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            p[u] = exp2_hw(sc[u] - m_new);
            psum += p[u];
        }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float lo = o[2 * i] * alpha, hi = o[2 * i + 1] * alpha;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                lo = __builtin_fmaf(p[u], bf16_lo(vr[u][i]), lo);
                hi = __builtin_fmaf(p[u], bf16_hi(vr[u][i]), hi);
            }
            o[2 * i] = lo;
            o[2 * i + 1] = hi;
        }
    }

    if (sub == 0) {
        sm_m[g] = m_run;
        sm_l[g] = l_run;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) sm_o[g * D + sub * 8 + i] = o[i];
    __syncthreads();

    if (tid < D) {
        float M = -INFINITY;
#pragma unroll 8
        for (int gg = 0; gg < G; ++gg) M = fmaxf(M, sm_m[gg]);
        float L = 0.f, acc = 0.f;
        if (M != -INFINITY) {
#pragma unroll 8
            for (int gg = 0; gg < G; ++gg) {
                const float w = exp2_hw(sm_m[gg] - M);
                L = __builtin_fmaf(w, sm_l[gg], L);
                acc = __builtin_fmaf(w, sm_o[gg * D + tid], acc);
            }
        }
        const size_t slot = (size_t)bh * S + split;
        ws_o[slot * D + tid] = acc;
        if (tid == 0) {
            ws_ml[slot * 2 + 0] = M;
            ws_ml[slot * 2 + 1] = L;
        }
    }
}

template <int D>
__global__ __launch_bounds__(D)
void decode_combine_kernel(const float* __restrict__ ws_o, const float* __restrict__ ws_ml,
                           uint16_t* __restrict__ Og, float* __restrict__ LSEg, int S) {
    const int bh = blockIdx.x;
    const int d = threadIdx.x;
    const float* ml = ws_ml + (size_t)bh * S * 2;
    const float* po = ws_o + (size_t)bh * S * D + d;
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, ml[2 * s]);
    float L = 0.f, acc = 0.f;
    for (int s = 0; s < S; ++s) {
        const float ms = ml[2 * s];
        const float w = ms == -INFINITY ? 0.f : exp2_hw(ms - M);
        L = __builtin_fmaf(w, ml[2 * s + 1], L);
        acc = __builtin_fmaf(w, po[(size_t)s * D], acc);
    }
    const float out = acc / L;
    Og[(size_t)bh * D + d] = __builtin_bit_cast(uint16_t, (__bf16)out);
    if (d == 0 && LSEg) LSEg[bh] = (M + __log2f(L)) * kLn2;
}

template <int D>
static hipError_t launch_d(const DecodeArgs& a) {
    const int BH = a.B * a.H;
    hipLaunchKernelGGL((decode_partial_kernel<D>), dim3(BH * a.S), dim3(kDecThreads), 0, a.stream,
                       (const uint16_t*)a.Q, (const uint16_t*)a.K, (const uint16_t*)a.V, a.ws_o, a.ws_ml,
                       a.Nk, a.S, a.chunk, a.scale * kLog2e);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(BH), dim3(D), 0, a.stream, a.ws_o, a.ws_ml,
                       (uint16_t*)a.O, a.LSE, a.S);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a) {
    return a.D == 128 ? launch_d<128>(a) : launch_d<64>(a);
}

}  // namespace fa
