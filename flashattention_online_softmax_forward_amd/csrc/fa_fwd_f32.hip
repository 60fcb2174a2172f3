// fp32 FlashAttention forward for gfx950 (fp32 inputs, arithmetic and output).
//
// The same tiled online-softmax recurrence as the bf16 kernel (iThome article,
// "three states"; ML compiler page, section 11.9), in the precision of the FA2
// kernel sketch on "Kernel visualization: Flash Attention 2", on the vector
// ALUs: a workgroup of 256 threads owns 16 query rows and 16 threads share a
// row, so a single head of 256 rows already spreads over 16 workgroups (with
// 64 rows per workgroup it ran on 4 CUs, each wave issue-bound on its own
// share). Q, the K and V tiles and the P tile sit in LDS; each thread computes
// 4 scores of its row per 64-key tile, the row max / sum are reduced over the
// 16 threads with DPP, and each thread accumulates D/16 values of the row's
// output in VGPRs. Base-2 exponentials with log2(e) folded into the scale.
// Masks as in the bf16 kernel: key padding (kv_lens), top-left or
// bottom-right causal alignment (one diagonal offset), and rows with no
// visible key written as O = 0, LSE = -inf (the running maximum starts
// finite, kNoKeyMax).

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

constexpr int kF32Threads = 256;
constexpr int kF32TPR = 16;            // threads per query row
constexpr int kF32BN = 64;             // keys per tile
static_assert(BM_FWD_F32 * kF32TPR == kF32Threads, "one row per 16 threads");

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kF32Threads)
void fwd_f32_kernel(const float* __restrict__ Qg, const float* __restrict__ Kg,
                    const float* __restrict__ Vg, float* __restrict__ Og,
                    float* __restrict__ LSEg, const int* __restrict__ kv_lens, int H, int Nq, int Nk,
                    int nqb, float scale2, int bottom_right) {
    constexpr int BM = BM_FWD_F32;
    constexpr int BN = kF32BN;
    constexpr int TPR = kF32TPR;
    constexpr int P = D + 4;           // row pitch of Q/K/V tiles (floats)
    constexpr int PP = BN + 4;         // row pitch of the P tile
    constexpr int NS = BN / TPR;       // scores per thread and tile: keys sub + TPR*i
    constexpr int NE = D / (4 * TPR);  // float4 output chunks per thread: columns 4*sub + 4*TPR*e
    constexpr int C4 = D / 4;          // float4 chunks per row

    __shared__ __attribute__((aligned(16))) float Qs[BM * P];
    __shared__ __attribute__((aligned(16))) float Ks[BN * P];
    __shared__ __attribute__((aligned(16))) float Vs[BN * P];
    __shared__ __attribute__((aligned(16))) float Ps[BM * PP];

    const int tid = threadIdx.x;
    const int r = tid / TPR;           // query row within the block
    const int sub = tid % TPR;         // the thread's share of the row

    const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
    const int bh = logical / nqb;
    int qb = logical - bh * nqb;
    if (CAUSAL) qb = nqb - 1 - qb;
    const int q0 = qb * BM;
    const int qrow = q0 + r;

    const float* Q = Qg + (size_t)bh * Nq * D;
    const float* K = Kg + (size_t)bh * Nk * D;
    const float* V = Vg + (size_t)bh * Nk * D;
    const int Lk = real_keys(kv_lens, bh / H, Nk);
    const int off = bottom_right ? Lk - Nq : 0;    // key j visible from query i iff j <= i + off

    for (int c = tid; c < BM * C4; c += kF32Threads) {
        const int row = c / C4, col = c % C4;
        f32x4_t w = {0.f, 0.f, 0.f, 0.f};
        if (q0 + row < Nq) w = *(const f32x4_t*)(Q + (size_t)(q0 + row) * D + col * 4);
        *(f32x4_t*)(Qs + row * P + col * 4) = w;
    }

    int kend = Lk;
    if (CAUSAL) kend = max(0, min(Lk, min(q0 + BM, Nq) + off));
    const int ntiles = (kend + BN - 1) / BN;

    f32x4_t o[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) o[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = kNoKeyMax;
    float l_run = 0.f;                 // this thread's share of the row sum

    for (int t = 0; t < ntiles; ++t) {
        const int kv0 = t * BN;
        __syncthreads();
        for (int c = tid; c < BN * C4; c += kF32Threads) {
            const int row = c / C4, col = c % C4;
            const int key = kv0 + row;
            f32x4_t kw = {0.f, 0.f, 0.f, 0.f}, vw = {0.f, 0.f, 0.f, 0.f};
            if (key < Lk) {
                kw = *(const f32x4_t*)(K + (size_t)key * D + col * 4);
                vw = *(const f32x4_t*)(V + (size_t)key * D + col * 4);
            }
            *(f32x4_t*)(Ks + row * P + col * 4) = kw;
            *(f32x4_t*)(Vs + row * P + col * 4) = vw;
        }
        __syncthreads();

        float s[NS];
#pragma unroll
        for (int i = 0; i < NS; ++i) s[i] = 0.f;
#pragma unroll 4
        for (int k = 0; k < D; k += 4) {
            const f32x4_t qv = *(const f32x4_t*)(Qs + r * P + k);
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                const f32x4_t kv = *(const f32x4_t*)(Ks + (sub + TPR * i) * P + k);
                s[i] = __builtin_fmaf(qv[0], kv[0], s[i]);
                s[i] = __builtin_fmaf(qv[1], kv[1], s[i]);
                s[i] = __builtin_fmaf(qv[2], kv[2], s[i]);
                s[i] = __builtin_fmaf(qv[3], kv[3], s[i]);
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const int key = kv0 + sub + TPR * i;
            if (key >= Lk || (CAUSAL && key > qrow + off)) s[i] = -INFINITY;
            mx = fmaxf(mx, s[i]);
        }
        mx = group_max<TPR>(mx);
        const float m_new = fmaxf(m_run, mx * scale2);
        const float alpha = exp2_hw(m_run - m_new);
        m_run = m_new;
        float lsum = 0.f;
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const float p = exp2_hw(__builtin_fmaf(s[i], scale2, -m_new));
            lsum += p;
            Ps[r * PP + sub + TPR * i] = p;
        }
        l_run = l_run * alpha + lsum;
        __syncthreads();

#pragma unroll
        for (int e = 0; e < NE; ++e) o[e] *= alpha;
#pragma unroll 8
        for (int c = 0; c < BN; ++c) {
            const float p = Ps[r * PP + c];
#pragma unroll
            for (int e = 0; e < NE; ++e) {
                const f32x4_t vv = *(const f32x4_t*)(Vs + c * P + sub * 4 + e * 4 * TPR);
                o[e][0] = __builtin_fmaf(p, vv[0], o[e][0]);
                o[e][1] = __builtin_fmaf(p, vv[1], o[e][1]);
                o[e][2] = __builtin_fmaf(p, vv[2], o[e][2]);
                o[e][3] = __builtin_fmaf(p, vv[3], o[e][3]);
            }
        }
    }

    const float l_tot = group_sum<TPR>(l_run);
    if (qrow < Nq) {
        // l = 0: no key seen (O = 0, LSE = -inf); l = NaN: NaN in both.
        const float inv = l_tot != 0.f ? 1.0f / l_tot : 0.f;
        float* orow = Og + ((size_t)bh * Nq + qrow) * D;
#pragma unroll
        for (int e = 0; e < NE; ++e) *(f32x4_t*)(orow + sub * 4 + e * 4 * TPR) = o[e] * inv;
        if (sub == 0 && LSEg)
            LSEg[(size_t)bh * Nq + qrow] = l_tot != 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
}

template <int D, bool CAUSAL>
static hipError_t launch_one(const FwdArgs& a) {
    const int nqb = (a.Nq + BM_FWD_F32 - 1) / BM_FWD_F32;
    const int grid = a.B * a.H * nqb;
    hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3(grid), dim3(kF32Threads), 0, a.stream,
                       (const float*)a.Q, (const float*)a.K, (const float*)a.V, (float*)a.O, a.LSE,
                       a.kv_lens, a.H, a.Nq, a.Nk, nqb, a.scale * kLog2e,
                       (int)(a.causal == kCausalBottomRight));
    return hipGetLastError();
}

hipError_t launch_fwd_f32(const FwdArgs& a) {
    if (a.D == 128) return a.causal ? launch_one<128, true>(a) : launch_one<128, false>(a);
    return a.causal ? launch_one<64, true>(a) : launch_one<64, false>(a);
}

}  // namespace fa
