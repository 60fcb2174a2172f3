// Split-KV decode for gfx950: one query token per (batch, head) over a long
// key/value cache (the "Flash-decoding" exercise of the ML compiler page),
// bf16 or fp16 (Elem<T> widens the inputs and rounds O).
//
// Kernel 1 (partial): one workgroup per (head, key chunk). The chunk's keys are
// streamed once from HBM with fully coalesced 16-byte loads: D/8 lanes share a
// key row (each lane owns 8 of the D columns), so one wave instruction reads
// 1 KiB of consecutive rows. The loads are non-temporal: every byte of the
// cache is read exactly once, so it should not displace anything in L2/MALL. Each lane group keeps its own online-softmax state
// (m, l, o) over the keys it visits, updated a block of U keys at a time
// (iThome article, "three states"); at the end the group states are merged in
// LDS with the merge rule of section 11.6 and the chunk's partial (m, l, o) is
// written to the workspace. This work is bandwidth-bound (one FMA per byte), so
// it stays on the vector ALUs: there is no contraction worth an MFMA here.
//
// Kernel 2 (combine): one workgroup per (batch, head) merges the chunk
// partials with the same rule, M = max m_s, l = sum l_s 2^(m_s - M),
// o = sum o_s 2^(m_s - M), and writes O = o / l (bf16) and
// LSE = (M + log2 l) ln 2. Empty chunks carry (-inf, 0, 0) and weigh nothing.
//
// Key padding: batch entry b has Lk = kv_lens[b] real keys (all Nk without
// kv_lens), split into S chunks of ceil(Lk / S) keys. A cache with no real key
// has only empty chunks and gets O = 0, LSE = -inf.

#include <mutex>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

constexpr int kDecThreads = 1024;    // 16 waves: more loads in flight per chunk (measured +4% over 256)
constexpr int kDecUnroll = 4;

template <typename T, int D>
__global__ __launch_bounds__(kDecThreads)
void decode_partial_kernel(const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg,
                           const uint16_t* __restrict__ Vg, float* __restrict__ ws_o,
                           float* __restrict__ ws_ml, const int* __restrict__ kv_lens, int H, int Nk, int S,
                           float scale2) {
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

    const int Lk = real_keys(kv_lens, bh / H, Nk);
    const int chunk = (int)(((long long)Lk + S - 1) / S);
    const long long jb = (long long)split * chunk;
    const int j0 = (int)(jb < Lk ? jb : Lk);
    const int j1 = (int)(jb + chunk < Lk ? jb + chunk : Lk);

    const uint16_t* K = Kg + (size_t)bh * Nk * D + sub * 8;
    const uint16_t* V = Vg + (size_t)bh * Nk * D + sub * 8;

    float q[8];
    {
        const u32x4_t w = *(const u32x4_t*)(Qg + (size_t)bh * D + sub * 8);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            q[2 * i] = Elem<T>::lo(w[i]) * scale2;
            q[2 * i + 1] = Elem<T>::hi(w[i]) * scale2;
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
                kr[u] = __builtin_nontemporal_load((const u32x4_t*)(K + (size_t)key * D));
                vr[u] = __builtin_nontemporal_load((const u32x4_t*)(V + (size_t)key * D));
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
                acc = __builtin_fmaf(q[2 * i], Elem<T>::lo(kr[u][i]), acc);
                acc = __builtin_fmaf(q[2 * i + 1], Elem<T>::hi(kr[u][i]), acc);
            }
            acc = group_sum<LPK>(acc);
            sc[u] = (base + u * G < j1) ? acc : -INFINITY;
        }
        // NaN-propagating maxima: a NaN score must reach O and l even when a
        // whole group's scores are NaN (fmaxf would keep m = -inf, and the
        // group would then look empty to the merges below).
        float mx = sc[0];
#pragma unroll
        for (int u = 1; u < U; ++u) mx = fmax_nan(mx, sc[u]);
        const float m_new = fmax_nan(m_run, mx);   // not -inf: key `base` is always live
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
                lo = __builtin_fmaf(p[u], Elem<T>::lo(vr[u][i]), lo);
                hi = __builtin_fmaf(p[u], Elem<T>::hi(vr[u][i]), hi);
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
        for (int gg = 0; gg < G; ++gg) M = fmax_nan(M, sm_m[gg]);
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

constexpr int kCombThreads = 256;

// Combine: 256 threads per (batch, head); thread = (split group sg, column
// quad dq). Each thread folds splits sg, sg + SG, ... of its 4 columns (float4
// loads, several in flight), then the SG partial states are merged in LDS.
template <typename T, int D>
__global__ __launch_bounds__(kCombThreads)
void decode_combine_kernel(const float* __restrict__ ws_o, const float* __restrict__ ws_ml,
                           uint16_t* __restrict__ Og, float* __restrict__ LSEg, int S) {
    constexpr int DQ = D / 4;                       // column quads
    constexpr int SG = kCombThreads / DQ;           // split groups
    __shared__ float sm_max[kCombThreads];
    __shared__ float sm_l[SG];
    __shared__ __attribute__((aligned(16))) float sm_o[SG * D];

    const int bh = blockIdx.x;
    const int tid = threadIdx.x;
    const int dq = tid % DQ;
    const int sg = tid / DQ;
    const float* ml = ws_ml + (size_t)bh * S * 2;
    const float* po = ws_o + (size_t)bh * S * D + dq * 4;

    // Global maximum over all splits (every thread scans a strided share).
    float M = -INFINITY;
    for (int s = tid; s < S; s += kCombThreads) M = fmaxf(M, ml[2 * s]);
    sm_max[tid] = M;
    __syncthreads();
    for (int w = kCombThreads / 2; w > 0; w >>= 1) {
        if (tid < w) sm_max[tid] = fmaxf(sm_max[tid], sm_max[tid + w]);
        __syncthreads();
    }
    M = sm_max[0];

    // This thread's splits: l and o rescaled to M and summed (empty chunks,
    // m = -inf, weigh nothing).
    float L = 0.f;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int s = sg; s < S; s += SG) {
        const float ms = ml[2 * s];
        const float w = ms == -INFINITY ? 0.f : exp2_hw(ms - M);
        L = __builtin_fmaf(w, ml[2 * s + 1], L);
        const f32x4_t o = *(const f32x4_t*)(po + (size_t)s * D);
        acc[0] = __builtin_fmaf(w, o[0], acc[0]);
        acc[1] = __builtin_fmaf(w, o[1], acc[1]);
        acc[2] = __builtin_fmaf(w, o[2], acc[2]);
        acc[3] = __builtin_fmaf(w, o[3], acc[3]);
    }
    *(f32x4_t*)(sm_o + sg * D + dq * 4) = acc;
    if (dq == 0) sm_l[sg] = L;
    __syncthreads();

    if (tid < D) {
        float lt = 0.f, ot = 0.f;
#pragma unroll
        for (int g = 0; g < SG; ++g) {
            lt += sm_l[g];
            ot += sm_o[g * D + tid];
        }
        // No real key at all (every chunk empty): O = 0, LSE = -inf. A NaN
        // (l = NaN, carried by a split whose m is NaN: its weight below is
        // NaN) gives NaN in both.
        Og[(size_t)bh * D + tid] = (uint16_t)Elem<T>::pack2(lt != 0.f ? ot / lt : 0.f, 0.f);
        if (tid == 0 && LSEg) LSEg[bh] = lt != 0.f ? (M + __log2f(lt)) * kLn2 : -INFINITY;
    }
}

template <typename T, int D>
static hipError_t launch_d(const DecodeArgs& a) {
    const int BH = a.B * a.H;
    hipLaunchKernelGGL((decode_partial_kernel<T, D>), dim3(BH * a.S), dim3(kDecThreads), 0, a.stream,
                       (const uint16_t*)a.Q, (const uint16_t*)a.K, (const uint16_t*)a.V, a.ws_o, a.ws_ml,
                       a.kv_lens, a.H, a.Nk, a.S, a.scale * kLog2e);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(BH), dim3(kCombThreads), 0, a.stream, a.ws_o,
                       a.ws_ml, (uint16_t*)a.O, a.LSE, a.S);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a) {
    if (a.f16) return a.D == 128 ? launch_d<_Float16, 128>(a) : launch_d<_Float16, 64>(a);
    return a.D == 128 ? launch_d<__bf16, 128>(a) : launch_d<__bf16, 64>(a);
}

// Fixed scratch of the allocation-free decode entry point: the partial states
// (m, l, o) that launch_decode otherwise keeps in a caller's workspace. One
// copy per GPU, alive until the process ends. Host code must never pass the
// array's name to a kernel (on the host it is only a stand-in for the
// symbol): the device address comes from hipGetSymbolAddress, taken once per
// device with that device current, and is used everywhere instead.
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t decode_scratch(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace fa
