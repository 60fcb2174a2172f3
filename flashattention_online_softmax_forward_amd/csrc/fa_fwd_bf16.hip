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
//     already the B operand of the second MFMA, O^T += V^T P^T. P never leaves
//     registers.
//   * O^T lives in 16*D/32 fp32 accumulators per lane, one query row per lane,
//     so the alpha rescale is a per-lane scalar multiply.
//   * K and V tiles go from global memory straight into LDS
//     (global_load_lds_dwordx4: no VGPR staging), two tiles deep, one barrier
//     per tile. Both are row-major in LDS with an XOR swizzle of their 16-byte
//     chunks chosen so the MFMA operand reads are free of bank conflicts. The
//     V^T operand (8 consecutive keys of one column per lane) is read with
//     ds_read_b64_tr_b16, the LDS transpose read: within each 16-lane block,
//     source lane s points at 4 consecutive columns of key k0 + s/4, and lane
//     i receives column i of those 4 keys. Rows past Nk are clamped to the
//     last key instead of branching: they are masked out of S, and their
//     (finite) values are multiplied by P = 0.
//   * Conditional rescaling (the FA4 refinement the iThome article describes
//     after the alpha derivation): the running maximum of a wave's rows is
//     only moved, and O and l rescaled, when some row's tile maximum exceeds it
//     by more than 2^8 (base 2). Otherwise the tile is exponentiated against
//     the stale maximum (P <= 256, safe in fp32 and bf16), which is exact once
//     O is divided by the l accumulated on the same base.
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
// Growth of a row maximum (log2 units) that forces a rescale of O and l.
constexpr float kRescaleThreshold = 8.0f;

// Key row (within a 32-key block) that lane-row i of the S^T A operand reads:
// bits 2 and 3 swapped. With it, accumulator register r of lane (j, h) holds
// key 16*(r/8) + 8*h + (r%8) of the block, i.e. 8 consecutive keys per half.
__device__ __forceinline__ int s_row_perm(int i) {
    return (i & ~0xC) | ((i & 4) << 1) | ((i & 8) >> 1);
}

// 16-byte chunk swizzles (CPR = chunks per row; LDS banks span 256 bytes).
// K: the 16 rows read together by one MFMA operand hit 16 distinct bank groups.
template <int CPR>
__device__ __forceinline__ int k_swz(int row) {
    return CPR == 16 ? (row & 15) : ((row >> 1) & 7);
}
// V: the 4 keys x 4 column-quads of a transpose-read block, and the two blocks
// that share a key range, hit distinct bank groups.
template <int CPR>
__device__ __forceinline__ int v_swz(int key) {
    return CPR == 16 ? 4 * (key & 3) : 4 * ((key >> 1) & 1);
}

#define LDS_AS __attribute__((address_space(3)))
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kFwdThreads, 2)
void fwd_bf16_kernel(const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg,
                     const uint16_t* __restrict__ Vg, uint16_t* __restrict__ Og,
                     float* __restrict__ LSEg, int Nq, int Nk, int nqb, float scale2) {
    constexpr int BN = Bf16Tile<D>::BN;
    constexpr int TILE = BN * D;               // elements of one K (or V) tile
    constexpr int NCB = BN / 32;               // 32-key blocks of S^T
    constexpr int NKK = D / 16;                // 16-wide d steps of the S MFMA
    constexpr int NDB = D / 32;                // 32-wide d blocks of O^T
    constexpr int NPV = BN / 16;               // 16-key steps of the PV MFMA
    constexpr int CPR = D / 8;                 // 16-byte chunks per row
    constexpr int NLD = BN * CPR / kFwdThreads;   // DMA chunks per thread per tensor
    static_assert(NLD * kFwdThreads == BN * CPR, "loader covers the tile");

    // Two K/V tile buffers. Four distinct arrays, selected statically (the
    // loop below is unrolled by two), let the compiler see that a DMA into one
    // buffer never aliases reads of the other, so it adds no wait between them.
    __shared__ __attribute__((aligned(1024))) uint16_t k_lds0[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t v_lds0[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t k_lds1[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t v_lds1[TILE];

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

    // Per-thread DMA slots: chunk p = (i*4 + wave)*64 + lane of the tile lands
    // at byte 16*p of the LDS tile, and holds logical chunk (p % CPR) ^ swz(row).
    int ld_row[NLD], ld_kcol[NLD], ld_vcol[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
        const int p = (i * kFwdWaves + wave) * 64 + lane;
        ld_row[i] = p / CPR;
        ld_kcol[i] = ((p % CPR) ^ k_swz<CPR>(ld_row[i])) * 8;
        ld_vcol[i] = ((p % CPR) ^ v_swz<CPR>(ld_row[i])) * 8;
    }

    auto issue_tile = [&](int kv0, uint16_t* kb, uint16_t* vb) {
        const int last = Nk - 1 - kv0;
        const uint16_t* Kt = K + (size_t)kv0 * D;
        const uint16_t* Vt_g = V + (size_t)kv0 * D;
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int row = min(ld_row[i], last);
            const int slot = (i * kFwdWaves + wave) * 64 * 8;      // elements
            __builtin_amdgcn_global_load_lds((const void*)(Kt + (uint32_t)(row * D + ld_kcol[i])),
                                             (LDS_AS void*)(LDS_AS uint16_t*)(kb + slot), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((const void*)(Vt_g + (uint32_t)(row * D + ld_vcol[i])),
                                             (LDS_AS void*)(LDS_AS uint16_t*)(vb + slot), 16, 0, 0);
        }
    };

    f32x16_t acc_o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[db][r] = 0.f;

    float m_run = -INFINITY;   // base-2 scaled maximum the row is accumulated against
    float l_run = 0.f;         // this lane's half of the running sum

    // K operand address (element offset within a K tile) for block c, step kk.
    const int srow = s_row_perm(j);
    // V transpose-read addresses: lane s of 16-lane block b points at key
    // 16*tt + 8*h + 4*rd + s/4, columns 32*db + 16*(b%2) + 4*(s%4) .. +3.
    const int vb_blk = (lane >> 4) & 1;
    const int v_s = lane & 15;

    // One key tile: prefetch tile t+1 into the other buffer, compute tile t.
    auto step = [&](int t, const uint16_t* kb, const uint16_t* vb, uint16_t* kb_next, uint16_t* vb_next) {
        const int kv0 = t * BN;
        if (t + 1 < ntiles) issue_tile(kv0 + BN, kb_next, vb_next);

        // A wave skips a causal tile that lies entirely after all its rows.
        if (!CAUSAL || kv0 <= wrow0 + 31) {
            // S^T = K Q^T for NCB blocks of 32 keys.
            f32x16_t s[NCB];
#pragma unroll
            for (int c = 0; c < NCB; ++c) {
                const int row = c * 32 + srow;
                const int sw = k_swz<CPR>(row);
#pragma unroll
                for (int r = 0; r < 16; ++r) s[c][r] = 0.f;
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) {
                    const bf16x8_t a = *(const bf16x8_t*)(kb + row * D + (((kk * 2 + h) ^ sw) * 8));
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

            // Tile row max (raw scores; scale2 > 0) in base-2 units.
            float mx = s[0][0];
#pragma unroll
            for (int c = 0; c < NCB; ++c)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[c][r]);
            const float m_tile = max_xor32(mx) * scale2;

            // Move the maximum (and rescale O, l) only when some row of the
            // wave outgrew it by more than the threshold.
            if (__builtin_amdgcn_ballot_w64(m_tile > m_run + kRescaleThreshold)) {
                const float m_new = fmaxf(m_run, m_tile);
                const float alpha = exp2_hw(m_run - m_new);
                m_run = m_new;
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc_o[db][r] *= alpha;
            }

            // P = exp2(S*scale2 - m), row sum of this half, bf16 B operands.
            bf16x8_t pf[NPV];
            float lsum = 0.f;
#pragma unroll
            for (int c = 0; c < NCB; ++c)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    float p[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        p[e] = exp2_hw(__builtin_fmaf(s[c][u * 8 + e], scale2, -m_run));
                        lsum += p[e];
                    }
                    u32x4_t w;
                    w[0] = pack_bf16x2(p[0], p[1]);
                    w[1] = pack_bf16x2(p[2], p[3]);
                    w[2] = pack_bf16x2(p[4], p[5]);
                    w[3] = pack_bf16x2(p[6], p[7]);
                    pf[c * 2 + u] = __builtin_bit_cast(bf16x8_t, w);
                }
            l_run += lsum;

            // O^T += V^T P^T: A operand = 8 keys (16*tt + 8*h ..) of column
            // 32*db + j, gathered by two transpose reads of 4 keys each.
#pragma unroll
            for (int tt = 0; tt < NPV; ++tt)
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    bf16x4_t part[2];
#pragma unroll
                    for (int rd = 0; rd < 2; ++rd) {
                        const int key = tt * 16 + h * 8 + rd * 4 + (v_s >> 2);
                        const int col = db * 32 + vb_blk * 16 + (v_s & 3) * 4;
                        const int chunk = (col >> 3) ^ v_swz<CPR>(key);
                        const uint16_t* addr = vb + key * D + chunk * 8 + (col & 7);
                        part[rd] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                            (LDS_AS bf16x4_t*)(LDS_AS uint16_t*)addr);
                    }
                    const bf16x8_t a = {part[0][0], part[0][1], part[0][2], part[0][3],
                                        part[1][0], part[1][1], part[1][2], part[1][3]};
                    acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[tt], acc_o[db], 0, 0, 0);
                }
        }

        if (t + 1 < ntiles) {
            __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0): tile t+1 landed (this wave's part)
            __syncthreads();                    // ... every wave's part; all reads of tile t done
        }
    };

    issue_tile(0, k_lds0, v_lds0);
    __builtin_amdgcn_s_waitcnt(0xF70);          // vmcnt(0): this wave's DMA landed
    __syncthreads();
    for (int t = 0; t < ntiles; t += 2) {
        step(t, k_lds0, v_lds0, k_lds1, v_lds1);
        if (t + 1 < ntiles) step(t + 1, k_lds1, v_lds1, k_lds0, v_lds0);
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
