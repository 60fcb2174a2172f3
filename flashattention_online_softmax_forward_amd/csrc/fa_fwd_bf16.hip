// bf16 FlashAttention forward for gfx950: MFMA for both contractions.
//
// Method (iThome FlashAttention article, "three states"; ML compiler page,
// section 11.9): a workgroup owns BM = 128 query rows of one (batch, head) and
// streams key/value tiles of BN keys past them. Per row it carries the running
// maximum m, the running sum l and the unnormalised output O; for each tile
//     m_new = max(m, rowmax S),  alpha = exp(m - m_new),  P = exp(S - m_new),
//     l = alpha*l + rowsum P,    O = alpha*O + P V,       m = m_new
// and at the end O / l and LSE = m + ln l are written (FA2 visualization,
// "Write the data back to HBM"). Scores are kept in base 2: the scale is
// multiplied by log2(e) so every exponential is a bare exp2 (the ML compiler
// page, section 11.7), and LSE is converted back to natural log at the end.
//
// gfx950 mapping (own design):
//   * 4 waves x 32 query rows. Q stays in VGPRs for the whole key loop as the B
//     operand of v_mfma_f32_32x32x16_bf16.
//   * S is computed transposed, S^T = K Q^T (A = 32 keys of K from LDS), so that
//     every lane ends with 16 scores of ONE query row: the row max / row sum are
//     in-lane reductions plus one exchange with lane ^ 32.
//   * The rows of K fed to the A operand are permuted (bits 2 and 3 of the row
//     index swapped) so the accumulator registers of S^T, rounded to bf16, are
//     already the B operand of the second MFMA, O^T += V^T P^T, whose A operand
//     reads 8 consecutive keys of one V column from a transposed LDS copy of V.
//     P never leaves registers.
//   * O^T lives in 16*D/32 fp32 accumulators per lane, one query row per lane,
//     so the alpha rescale is a per-lane scalar multiply.
//   * K/V tiles are loaded with coalesced 16-byte global loads into registers
//     one tile ahead, then written to LDS (K row-major with a 16-byte pad, V
//     transposed with an XOR swizzle of its 16-byte chunks).
//   * Causal: key tiles past the block's last row are never visited, tiles a
//     whole wave cannot see are skipped by that wave, masks are applied only on
//     diagonal and ragged tiles, and the heaviest query blocks are issued first.

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

template <int D> struct Bf16Tile;
template <> struct Bf16Tile<128> { static constexpr int BN = 64; };
template <> struct Bf16Tile<64> { static constexpr int BN = 128; };

constexpr int kFwdWaves = 4;
constexpr int kFwdThreads = 64 * kFwdWaves;

// Key row (within a 32-key block) that lane-row i of the S^T A operand reads:
// bits 2 and 3 swapped. With it, accumulator register r of lane (j, h) holds
// key 16*(r/8) + 8*h + (r%8) of the block, i.e. 8 consecutive keys per half.
__device__ __forceinline__ int s_row_perm(int i) {
    return (i & ~0xC) | ((i & 4) << 1) | ((i & 8) >> 1);
}

// Physical 16-byte chunk of logical chunk c in row d of the transposed V tile.
__device__ __forceinline__ int vt_chunk(int d, int c) {
    return c ^ ((d ^ (d >> 3)) & 7);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kFwdThreads, 2)
void fwd_bf16_kernel(const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg,
                     const uint16_t* __restrict__ Vg, uint16_t* __restrict__ Og,
                     float* __restrict__ LSEg, int Nq, int Nk, int nqb, float scale2) {
    constexpr int BN = Bf16Tile<D>::BN;
    constexpr int KP = D + 8;                  // K tile row pitch (elements)
    constexpr int NCB = BN / 32;               // 32-key blocks of S^T
    constexpr int NKK = D / 16;                // 16-wide d steps of the S MFMA
    constexpr int NDB = D / 32;                // 32-wide d blocks of O^T
    constexpr int NPV = BN / 16;               // 16-key steps of the PV MFMA
    constexpr int CPR = D / 8;                 // 16-byte chunks per row
    constexpr int NKL = BN * CPR / kFwdThreads;
    constexpr int DG = D / 8;                  // V loader: 8-wide d groups
    constexpr int KG = kFwdThreads / DG;       // V loader: groups of 4 keys
    static_assert(KG * 4 == BN, "V loader covers the tile");
    static_assert(NKL * kFwdThreads == BN * CPR, "K loader covers the tile");

    __shared__ __attribute__((aligned(16))) uint16_t Ks[BN * KP];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[D * BN];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int j = lane & 31;
    const int h = lane >> 5;

    const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
    const int bh = logical / nqb;
    int qb = logical - bh * nqb;
    if (CAUSAL) qb = nqb - 1 - qb;             // longest rows first
    const int q0 = qb * BM_FWD;

    const uint16_t* Q = Qg + (size_t)bh * Nq * D;
    const uint16_t* K = Kg + (size_t)bh * Nk * D;
    const uint16_t* V = Vg + (size_t)bh * Nk * D;

    const int wrow0 = q0 + wave * 32;
    const int qrow = wrow0 + j;

    // Q as the B operand: lane (j, h) holds row qrow, d = 16*kk + 8*h .. +7.
    bf16x8_t qf[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        u32x4_t w = {0u, 0u, 0u, 0u};
        if (qrow < Nq) w = *(const u32x4_t*)(Q + (size_t)qrow * D + kk * 16 + h * 8);
        qf[kk] = __builtin_bit_cast(bf16x8_t, w);
    }

    int kend = Nk;
    if (CAUSAL) kend = min(Nk, min(q0 + BM_FWD, Nq));
    const int ntiles = (kend + BN - 1) / BN;

    u32x4_t kreg[NKL];
    u32x4_t vreg[4];
    const int vdg = tid % DG;
    const int vkg = tid / DG;

    auto load_tile = [&](int kv0) {
#pragma unroll
        for (int i = 0; i < NKL; ++i) {
            const int c = tid + i * kFwdThreads;
            const int row = c / CPR, col = c % CPR;
            const int key = kv0 + row;
            kreg[i] = key < Nk ? *(const u32x4_t*)(K + (size_t)key * D + col * 8) : u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int key = kv0 + vkg * 4 + r;
            vreg[r] = key < Nk ? *(const u32x4_t*)(V + (size_t)key * D + vdg * 8) : u32x4_t{0u, 0u, 0u, 0u};
        }
    };

    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < NKL; ++i) {
            const int c = tid + i * kFwdThreads;
            const int row = c / CPR, col = c % CPR;
            *(u32x4_t*)(Ks + row * KP + col * 8) = kreg[i];
        }
        // 4 keys x 8 d held as 4 rows of 8 -> 8 rows (one per d) of 4 keys.
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uint32_t w0, w1;
            if ((e & 1) == 0) {
                w0 = (vreg[0][e >> 1] & 0xffffu) | (vreg[1][e >> 1] << 16);
                w1 = (vreg[2][e >> 1] & 0xffffu) | (vreg[3][e >> 1] << 16);
            } else {
                w0 = (vreg[0][e >> 1] >> 16) | (vreg[1][e >> 1] & 0xffff0000u);
                w1 = (vreg[2][e >> 1] >> 16) | (vreg[3][e >> 1] & 0xffff0000u);
            }
            const int d = vdg * 8 + e;
            const int chunk = vt_chunk(d, vkg >> 1);
            *(u32x2_t*)(Vt + d * BN + chunk * 8 + (vkg & 1) * 4) = u32x2_t{w0, w1};
        }
    };

    f32x16_t acc_o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[db][r] = 0.f;

    float m_run = -INFINITY;   // running max of the base-2 scaled scores
    float l_run = 0.f;         // this lane's half of the running sum

    const int srow = s_row_perm(j);

    if (ntiles > 0) load_tile(0);
    for (int t = 0; t < ntiles; ++t) {
        const int kv0 = t * BN;
        __syncthreads();
        store_tile();
        __syncthreads();
        if (t + 1 < ntiles) load_tile(kv0 + BN);

        if (CAUSAL && kv0 > wrow0 + 31) continue;   // no row of this wave sees the tile

        // S^T = K Q^T for NCB blocks of 32 keys.
        f32x16_t s[NCB];
#pragma unroll
        for (int c = 0; c < NCB; ++c) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[c][r] = 0.f;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                const bf16x8_t a = *(const bf16x8_t*)(Ks + (c * 32 + srow) * KP + kk * 16 + h * 8);
                s[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s[c], 0, 0, 0);
            }
        }

        // Mask keys past Nk and, on diagonal tiles, keys after the row.
        const bool ragged = kv0 + BN > Nk;
        const bool diag = CAUSAL && (kv0 + BN - 1 > wrow0);
        if (ragged || diag) {
#pragma unroll
            for (int c = 0; c < NCB; ++c)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kv0 + c * 32 + (r >> 3) * 16 + h * 8 + (r & 7);
                    const bool dead = key >= Nk || (CAUSAL && key > qrow);
                    if (dead) s[c][r] = -INFINITY;
                }
        }

        // Row max (raw scores; scale2 > 0), then the new base-2 maximum.
        float mx = s[0][0];
#pragma unroll
        for (int c = 0; c < NCB; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[c][r]);
        mx = max_xor32(mx);
        const float m_new = fmaxf(m_run, mx * scale2);
        const float alpha = exp2_hw(m_run - m_new);
        m_run = m_new;

        // P = exp2(S*scale2 - m_new), row sum of this half, bf16 B operands.
        bf16x8_t pf[NPV];
        float lsum = 0.f;
#pragma unroll
        for (int c = 0; c < NCB; ++c)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                float p[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    p[e] = exp2_hw(__builtin_fmaf(s[c][u * 8 + e], scale2, -m_new));
                    lsum += p[e];
                }
                u32x4_t w;
                w[0] = pack_bf16x2(p[0], p[1]);
                w[1] = pack_bf16x2(p[2], p[3]);
                w[2] = pack_bf16x2(p[4], p[5]);
                w[3] = pack_bf16x2(p[6], p[7]);
                pf[c * 2 + u] = __builtin_bit_cast(bf16x8_t, w);
            }
        l_run = l_run * alpha + lsum;

#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc_o[db][r] *= alpha;

        // O^T += V^T P^T: A = V^T rows d = 32*db + j, keys 16*tt + 8*h .. +7.
#pragma unroll
        for (int tt = 0; tt < NPV; ++tt)
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const int d = db * 32 + j;
                const bf16x8_t a = *(const bf16x8_t*)(Vt + d * BN + vt_chunk(d, tt * 2 + h) * 8);
                acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[tt], acc_o[db], 0, 0, 0);
            }
    }

    // Epilogue: O / l to bf16, LSE = (m + log2 l) * ln 2.
    const float l_tot = sum_xor32(l_run);
    if (qrow < Nq) {
        const float inv = 1.0f / l_tot;
        uint16_t* orow = Og + ((size_t)bh * Nq + qrow) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const int d = db * 32 + a4 * 8 + h * 4;
                u32x2_t w;
                w[0] = pack_bf16x2(acc_o[db][a4 * 4 + 0] * inv, acc_o[db][a4 * 4 + 1] * inv);
                w[1] = pack_bf16x2(acc_o[db][a4 * 4 + 2] * inv, acc_o[db][a4 * 4 + 3] * inv);
                *(u32x2_t*)(orow + d) = w;
            }
        if (h == 0 && LSEg) LSEg[(size_t)bh * Nq + qrow] = (m_run + __log2f(l_tot)) * kLn2;
    }
}

template <int D, bool CAUSAL>
static hipError_t launch_one(const FwdArgs& a) {
    const int nqb = (a.Nq + BM_FWD - 1) / BM_FWD;
    const int grid = a.B * a.H * nqb;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3(grid), dim3(kFwdThreads), 0, a.stream,
                       (const uint16_t*)a.Q, (const uint16_t*)a.K, (const uint16_t*)a.V,
                       (uint16_t*)a.O, a.LSE, a.Nq, a.Nk, nqb, a.scale * kLog2e);
    return hipGetLastError();
}

hipError_t launch_fwd_bf16(const FwdArgs& a) {
    if (a.D == 128) return a.causal ? launch_one<128, true>(a) : launch_one<128, false>(a);
    return a.causal ? launch_one<64, true>(a) : launch_one<64, false>(a);
}

}  // namespace fa
