// FlashAttention forward for gfx950 with D = 64 and bf16 or fp16 inputs: MFMA
// for both contractions (v_mfma_f32_32x32x16_bf16 / _f16, fp32 accumulation).
// The two input types share every line below; Elem<T> supplies the MFMA, the
// LDS transpose read and the round-to-nearest-even packing of P and O. D = 128
// runs fa_fwd_mfma16.hip, the same schedule on the 16x16x32 MFMA; the launch
// helpers both use (the CU count, the persistent grid) are at the end of this
// file.
//
// Method (iThome FlashAttention article, "three states"; ML compiler page,
// section 11.9): a workgroup owns BM = 256 query rows of one (batch, head) and
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
//   * 8 waves x 32 query rows, one workgroup per CU (2 waves per SIMD). Q stays
//     in VGPRs for the whole key loop as the B operand of
//     v_mfma_f32_32x32x16_bf16. Q arrives, and O leaves, through an LDS row
//     staging area, so that both move whole rows between HBM and the CU. Both
//     carry the non-temporal cache policy (each is touched once), which leaves
//     L2 to the K/V tiles that every query block of a head re-reads.
//   * S is computed transposed, S^T = K Q^T (A = 32 keys of K from LDS), so that
//     every lane ends with 16 scores of ONE query row: the row max / row sum are
//     in-lane reductions plus one exchange with lane ^ 32.
//   * The rows of K fed to the A operand are permuted (bits 2 and 3 of the row
//     index swapped) so the accumulator registers of S^T, rounded to bf16, are
//     already the B operand of the second MFMA, O^T += V^T P^T. P never leaves
//     registers.
//   * O^T lives in 16*D/32 fp32 accumulators per lane, one query row per lane,
//     so the alpha rescale is a per-lane scalar multiply.
//   * Ping-pong: every wave alternates an MFMA step (PV of the previous tile
//     and QK of the current one) and a softmax step, separated by workgroup
//     barriers; the two wave groups (waves 0-3 and 4-7, one of each per SIMD)
//     run a step apart, so on every SIMD one wave feeds the matrix core while
//     the other runs the exponentials on the VALU.
//   * K and V tiles go from global memory straight into LDS (buffer_load_dwordx4
//     with the lds bit: no VGPR staging), two tiles deep. Both are
//     row-major in LDS with an XOR swizzle of their 16-byte chunks chosen so
//     the MFMA operand reads are free of bank conflicts. The V^T operand (8
//     consecutive keys of one column per lane) is read with ds_read_b64_tr_b16,
//     the LDS transpose read: within each 16-lane block, source lane s points
//     at 4 consecutive columns of key k0 + s/4, and lane i receives column i
//     of those 4 keys. The buffer resource of a tile spans only its real keys,
//     so rows past Lk are out of range and arrive in LDS as zeros: they are
//     masked out of S, and P = 0 meets a zero V row.
//   * Conditional rescaling (the FA4 refinement the iThome article describes
//     after the alpha derivation): the running maximum of a wave's rows is
//     only moved, and O and l rescaled, when a tile's P against it could
//     exceed 2^15. Otherwise the tile is exponentiated against the stale
//     maximum, which is exact once O is divided by the l accumulated on the
//     same base. The tile maximum, taken by the MFMA step, is compared with
//     the kept maximum plus the bound.
//   * Causal: key tiles past the block's last row are never visited, tiles a
//     whole wave cannot see are skipped by that wave, masks are applied only on
//     diagonal and ragged tiles, and the heaviest query blocks are issued first.
//     Causal self-attention with more query blocks than CUs runs a persistent
//     launch: one workgroup per CU works through a fixed list of blocks,
//     paired heavy with light.
//     Top-left alignment shows key j to query i iff j <= i; bottom-right iff
//     j <= i + (Lk - Nq), one diagonal offset in every bound and mask.
//   * Key padding: batch entry b has Lk = kv_lens[b] real keys (all Nk without
//     kv_lens); keys past Lk are never loaded or are masked like a ragged tail.
//   * Fully masked rows (bottom-right rows before the first key, or Lk = 0):
//     the running maximum starts at a large finite negative value instead of
//     -inf (the Pitfalls passage of the ML compiler page: exp2(-inf - -inf)
//     would be NaN), so a masked score gives exp2(-inf) = 0 and a row that
//     never sees a key ends with l = 0; it is written as O = 0, LSE = -inf.

#include <atomic>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {


constexpr int kFwdWaves = 8;
constexpr int kFwdThreads = 64 * kFwdWaves;
// Growth of a row maximum (log2 units) past which O and l are rescaled: a row
// that keeps a stale maximum has every P at most 2^15, within fp16's range
// (largest finite 65504) as well as bf16's (l and O are fp32 sums). bf16
// could take larger P, but accuracy sets the bound there: right after the
// maximum moves a row's largest P is exactly 1, under a stale maximum it is
// rounded like any other, and in a row that one key dominates that rounding
// reaches O almost unweighted. On causal 4x32x4096 inputs with Q and K scaled
// by 3, bounds of 2^24 and 2^32 put sampled O errors past 2e-2.
constexpr float kRescaleThreshold = 15.0f;

// Key row (within a 32-key block) that lane-row i of the S^T A operand reads:
// bits 2 and 3 swapped. With it, accumulator register r of lane (j, h) holds
// key 16*(r/8) + 8*h + (r%8) of the block, i.e. 8 consecutive keys per half.
__device__ __forceinline__ int s_row_perm(int i) {
    return (i & ~0xC) | ((i & 4) << 1) | ((i & 8) >> 1);
}

// 16-byte chunk swizzles of the 8-chunk (128-byte) rows; LDS banks span 256
// bytes, two rows.
// K: the 16 rows read together by one MFMA operand hit 16 distinct bank groups.
__device__ __forceinline__ int k_swz(int row) { return (row >> 1) & 7; }
// V: the 4 keys x 4 column-quads of a transpose-read block, and the two blocks
// that share a key range, hit distinct bank groups.
__device__ __forceinline__ int v_swz(int key) { return 4 * ((key >> 1) & 1); }

#define LDS_AS __attribute__((address_space(3)))

template <typename T, int D, bool PERSIST>
__global__ __launch_bounds__(kFwdThreads, 1)
void fwd_mfma_kernel(const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg,
                     const uint16_t* __restrict__ Vg, uint16_t* __restrict__ Og,
                     float* __restrict__ LSEg, const int* __restrict__ kv_lens, int H, int Nq, int Nk,
                     int nqb, float scale2, int causal, const float* __restrict__ rope_cos,
                     const float* __restrict__ rope_sin, int rope_style, int n_bh) {
    // The causal mode is a uniform run-time argument rather than a template
    // parameter: one code shape for all keeps register allocation stable.
    const bool CAUSAL = causal != kCausalNone;
    using E = Elem<T>;
    using V8 = typename E::v8;
    using V4 = typename E::v4;
    static_assert(D == 64, "D = 128 runs fa_fwd_mfma16.hip");
    constexpr int BN = 128;                    // keys per tile
    constexpr int TILE = BN * D;               // elements of one K (or V) tile
    constexpr int NCB = BN / 32;               // 32-key blocks of S^T
    constexpr int NKK = D / 16;                // 16-wide d steps of the S MFMA
    constexpr int NDB = D / 32;                // 32-wide d blocks of O^T
    constexpr int NPV = BN / 16;               // 16-key steps of the PV MFMA
    constexpr int CPR = D / 8;                 // 16-byte chunks per row
    constexpr int kLoadWaves = kFwdWaves / 2;     // one group's waves share a tile load
    constexpr int NLD = BN * CPR / (64 * kLoadWaves);   // DMA chunks per thread per tensor
    static_assert(NLD * 64 * kLoadWaves == BN * CPR, "loader covers the tile");
    // Group 0 loads the tiles, both K(t+1) and V(t) right after its MFMA step:
    // the softmax step, with its 64 exponentials per lane and tile, is the
    // longer one (splitting the loads between the groups measured 2% slower).
    // The MFMA step takes each tile's row maximum, one maximum3 per PV MFMA
    // after running QK(t) first, which takes VALU work off the softmax step
    // (+2-3%).

    // Two K and two V tile buffers. Four distinct arrays, selected statically
    // (the phase loop below is unrolled over two tiles), let the compiler see
    // that a DMA into one buffer never aliases reads of another, so it adds no
    // wait between them.
    __shared__ __attribute__((aligned(1024))) uint16_t k_lds0[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t k_lds1[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t v_lds0[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t v_lds1[TILE];
    // Row staging: Q rows on the way in, O rows on the way out (32 rows per
    // wave, 16-byte chunks swizzled by row), so that both move whole rows
    // between HBM and the CU.
    constexpr int RB = 32 * D;                 // elements of one wave's rows
    __shared__ __attribute__((aligned(1024))) uint16_t row_lds[kFwdWaves * RB];

    // Work of this workgroup: one query block or, in a persistent launch, a
    // fixed list of them. Persistent launches serve causal self-attention
    // with more query blocks than CUs: block qb of a head costs about qb + 1
    // key tiles, and handing such blocks to CUs one at a time in order leaves
    // CUs idle (the dispatcher assigns workgroups to shader engines in turn
    // and waits for a free CU in the next one's engine). Instead, the blocks of a
    // head are paired (nqb - 1 - r with r), every pair costing the same; each
    // XCD owns a contiguous range of pairs, so the heads in flight on it stay
    // few and their K/V stays in its L2, and its workgroups take the pairs in
    // turn, the heavy block of each first.
    const int npair = (nqb + 1) / 2;
    const int xcd = blockIdx.x & 7;            // workgroups go to the XCDs round-robin
    const int per_xcd = gridDim.x >> 3;        // a persistent grid is a multiple of 8
    const long long all_pairs = (long long)n_bh * npair;
    const int p_lo = (int)(all_pairs * xcd / 8), p_hi = (int)(all_pairs * (xcd + 1) / 8);
    for (int wi = 0;; ++wi) {
        int bh, qb;
        if constexpr (!PERSIST) {
            if (wi > 0) break;
            const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
            bh = logical / nqb;
            qb = logical - bh * nqb;
            if (CAUSAL) qb = nqb - 1 - qb;     // longest rows first
        } else {
            const int p = p_lo + (int)(blockIdx.x >> 3) + (wi >> 1) * per_xcd;
            if (p >= p_hi) break;
            bh = p / npair;
            const int r = p - bh * npair;
            qb = (wi & 1) ? r : nqb - 1 - r;
            if ((wi & 1) && qb == nqb - 1 - r) continue;   // odd nqb: the middle block is alone
        }
        // The thread index is made opaque per block, so that the per-lane
        // offsets and addresses derived from it are computed in each block
        // rather than hoisted out of this loop and held in registers across
        // every key loop.
        int tid = threadIdx.x;
        if constexpr (PERSIST) asm volatile("" : "+v"(tid));
        const int wave = tid >> 6;
        const int group = wave >> 2;           // ping-pong group (one wave of each per SIMD)
        const int lane = tid & 63;
        const int j = lane & 31;
        const int h = lane >> 5;

        const int q0 = qb * BM_FWD;

        const uint16_t* Q = Qg + (size_t)bh * Nq * D;
        const uint16_t* K = Kg + (size_t)bh * Nk * D;
        const uint16_t* V = Vg + (size_t)bh * Nk * D;
        const int Lk = real_keys(kv_lens, bh / H, Nk);
        // Causal diagonal offset: key j is visible from query i iff j <= i + off.
        const int off = causal == kCausalBottomRight ? Lk - Nq : 0;

        const int wrow0 = q0 + wave * 32;
        const int qrow = wrow0 + j;

        // The wave's Q rows go to LDS with buffer loads (whole rows, four per
        // load; rows past Nq are out of the resource's range and arrive as zeros);
        // issued in the prologue below and read into registers from there.
        const int qwave = __builtin_amdgcn_readfirstlane(wave);
        uint16_t* const qst = row_lds + qwave * RB;
        auto load_q = [&]() __attribute__((always_inline)) {
            constexpr int NQS = RB / 512;          // 1 KB slots per wave
            uint32_t qoff[NQS];
    #pragma unroll
            for (int i = 0; i < NQS; ++i) {
                const int p = i * 64 + lane;       // chunk of the wave's rows
                const int row = p / CPR;
                qoff[i] = (uint32_t)(row * D + ((p % CPR) ^ (row & (CPR - 1))) * 8) * 2 - (i % 4) * 1024;
            }
            // From the wave-uniform index, so the resource is scalar (a per-lane
            // resource would need a loop over its distinct values).
            const int qrow0 = q0 + qwave * 32;
            const int qrows = __builtin_amdgcn_readfirstlane(min(max(Nq - qrow0, 0), 32));
            const int qfirst = __builtin_amdgcn_readfirstlane(min(qrow0, Nq));
            const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(Q + (size_t)qfirst * D), (short)0, qrows * D * 2, kBufferRsrcWord3);
            static_assert(NQS % 4 == 0, "slots in groups of 4");
            // Each Q row is read by one workgroup only: streamed past L2.
    #pragma unroll
            for (int g = 0; g < NQS; g += 4)
                buffer_lds_slots<4, 0, kCachePolicyNT>(rsrc, (LDS_AS void*)(LDS_AS uint16_t*)(qst + g * 512), qoff + g);
        };
        // Q as the B operand: lane (j, h) holds row qrow, d = 16*kk + 8*h .. +7.
        u32x4_t qw[NKK];
        V8 qf[NKK];

        int kend = Lk;
        if (CAUSAL) kend = max(0, min(Lk, min(q0 + BM_FWD, Nq) + off));
        const int ntiles = (kend + BN - 1) / BN;
        // Tiles this wave computes: a causal tile entirely after all its rows is skipped.
        const int wlast = wrow0 + 31 + off;        // last key the wave's last row may see
        const int my_tiles = CAUSAL ? (wlast < 0 ? 0 : min(ntiles, wlast / BN + 1)) : ntiles;

        // Tile load slots: chunk p = (lwave*NLD + i)*64 + lane of a tile lands at
        // byte 16*p of the LDS tile and holds logical chunk (p % CPR) ^ swz(row)
        // of row p / CPR. The per-lane memory offsets are stored net of slot i's
        // immediate offset (i KB).
        const int lwave = __builtin_amdgcn_readfirstlane(wave & (kLoadWaves - 1));
        uint32_t ld_koff[NLD], ld_voff[NLD];
    #pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int p = (lwave * NLD + i) * 64 + lane;
            const int row = p / CPR;
            ld_koff[i] = (uint32_t)(row * D + ((p % CPR) ^ k_swz(row)) * 8) * 2 - i * 1024;
            ld_voff[i] = (uint32_t)(row * D + ((p % CPR) ^ v_swz(row)) * 8) * 2 - i * 1024;
        }
        // One tensor's tile at key kv0. The resource spans the tile's real keys
        // only, so every address is a per-lane constant and only the resource base
        // moves from tile to tile (scalar arithmetic).
        auto dma = [&](const uint16_t* src, const uint32_t* voff, int kv0, uint16_t* dst) __attribute__((always_inline)) {
            const int rows = min(Lk - kv0, BN);      // > 0: only tiles below kend <= Lk are loaded
            const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(src + (size_t)kv0 * D), (short)0, rows * D * 2, kBufferRsrcWord3);
            buffer_lds_slots<NLD>(rsrc, (LDS_AS void*)(LDS_AS uint16_t*)(dst + lwave * NLD * 512), voff);
        };

        f32x16_t acc_o[NDB];
    #pragma unroll
        for (int db = 0; db < NDB; ++db)
    #pragma unroll
            for (int r = 0; r < 16; ++r) acc_o[db][r] = 0.f;
        f32x16_t s[NCB];            // S^T of the tile between its MFMA step and its softmax step
        V8 pf[NPV];           // P of the tile between its softmax step and its PV step

        // Base-2 scaled maximum the row is accumulated against; kNoKeyMax until the
        // row's first visible key (finite, so masked scores give exp2(-inf) = 0).
        float m_run = kNoKeyMax;
        float l_run = 0.f;         // this lane's half of the running sum

        const int srow = s_row_perm(j);
        const int vb_blk = (lane >> 4) & 1;
        const int v_s = lane & 15;

        // MFMA step of tile t: O^T += V^T P^T for tile t-1, then S^T = K Q^T for tile t.
        // Only one wave per SIMD is in this step at a time, so it must keep the
        // matrix core busy on its own: LDS operands are read a few MFMAs ahead, and
        // sched_group_barrier pins that order (DS reads first, then one MFMA per
        // group of reads).
        constexpr int NPVM = NPV * NDB;            // PV MFMAs per tile
        constexpr int NSM = NKK * NCB;             // QK MFMAs per tile
        constexpr int LEAD = 4;                    // MFMAs of operand prefetch
        auto pv_operand = [&](const uint16_t* vb_prev, int i) __attribute__((always_inline)) {
            const int tt = i / NDB, db = i % NDB;
            V4 part[2];
    #pragma unroll
            for (int rd = 0; rd < 2; ++rd) {
                const int key = tt * 16 + h * 8 + rd * 4 + (v_s >> 2);
                const int col = db * 32 + vb_blk * 16 + (v_s & 3) * 4;
                const int chunk = (col >> 3) ^ v_swz(key);
                const uint16_t* addr = vb_prev + key * D + chunk * 8 + (col & 7);
                part[rd] = E::tr_read((LDS_AS V4*)(LDS_AS uint16_t*)addr);
            }
            return V8{part[0][0], part[0][1], part[0][2], part[0][3],
                            part[1][0], part[1][1], part[1][2], part[1][3]};
        };
        auto qk_operand = [&](const uint16_t* kb, int i) __attribute__((always_inline)) {
            const int kk = i / NCB, c = i % NCB;
            const int row = c * 32 + srow;
            return *(const V8*)(kb + row * D + (((kk * 2 + h) ^ k_swz(row)) * 8));
        };
        // Scaled row maximum of tile t's scores (NaN-propagating).
        auto tile_max = [&]() __attribute__((always_inline)) {
            constexpr int NCH = 4;
            float mxc[NCH];
    #pragma unroll
            for (int k = 0; k < NCH; ++k) mxc[k] = s[0][k];
    #pragma unroll
            for (int c = 0; c < NCB; ++c)
    #pragma unroll
                for (int r = 0; r < 16; ++r) mxc[r % NCH] = fmax_nan(mxc[r % NCH], s[c][r]);
            return max_xor32(fmax_nan(fmax_nan(mxc[0], mxc[1]), fmax_nan(mxc[2], mxc[3]))) * scale2;
        };
        float m_pre = kNoKeyMax;   // tile maximum taken by the MFMA step
        auto step_mfma = [&](int t, const uint16_t* kb, const uint16_t* vb_prev) __attribute__((always_inline)) {
            // lgkmcnt(0): nothing LDS-side is pending here (the barrier before
            // this step drained it), but a scalar load of a kernel argument used
            // only after the loop may be, on the first entry. Scalar loads return
            // out of order, so while one may be pending the compiler can only
            // wait for an operand with lgkmcnt(0), i.e. for every operand read
            // issued ahead. Waiting here once lets the first MFMA of the step
            // wait for its own operand alone.
            __builtin_amdgcn_s_waitcnt(0xC07F);
            __builtin_amdgcn_s_setprio(1);
            const bool do_pv = t >= 1 && t - 1 < my_tiles;
            const bool do_qk = t < my_tiles;
            if (do_pv && do_qk) {
                // QK(t) then PV(t-1); the row maximum of tile t runs on the VALU
                // beside the PV MFMAs. The last 4 scores start 4 chains, the
                // others join EPS per PV MFMA from the second one on (the QK
                // results are complete by then).
                constexpr int NM = NPVM + NSM;
                auto operand = [&](int i) __attribute__((always_inline)) {
                    return i < NSM ? qk_operand(kb, i) : pv_operand(vb_prev, i - NSM);
                };
                const f32x16_t zero = {};
                constexpr int NEL = NCB * 16;
                constexpr int EPS = (NEL - 4 + NPVM - 2) / (NPVM - 1);
                constexpr int NMX = (NEL - 4 + EPS - 1) / EPS;
                static_assert(NMX <= NPVM - 1, "the maximum fits beside the PV MFMAs");
                float mxc[4];
                V8 ring[LEAD];
    #pragma unroll
                for (int i = 0; i < LEAD; ++i) ring[i] = operand(i);
                __builtin_amdgcn_sched_group_barrier(0x100, LEAD, 0);
    #pragma unroll
                for (int i = 0; i < NM; ++i) {
                    const V8 a = ring[i % LEAD];
                    if (i + LEAD < NM) ring[i % LEAD] = operand(i + LEAD);
                    if (i < NSM)  // the first d step of each key block starts from zero
                        s[i % NCB] = E::mfma(a, qf[i / NCB], i < NCB ? zero : s[i % NCB]);
                    else
                        acc_o[(i - NSM) % NDB] = E::mfma(a, pf[(i - NSM) / NDB], acc_o[(i - NSM) % NDB]);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    const int nx = i + LEAD;
                    if (nx < NSM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    else if (nx < NM) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                    // Empty asm statements pin each chain step to its iteration
                    // (pure arithmetic would otherwise float up to the end of the
                    // QK MFMAs); every step depends on its chain's previous pin.
                    const int k = i - NSM - 1;
                    if (k == -1) {
    #pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            mxc[q] = s[(NEL - 4 + q) / 16][(NEL - 4 + q) % 16];
                            asm volatile("" : "+v"(mxc[q]));
                        }
                    }
                    if (k >= 0 && k < NMX) {
    #pragma unroll
                        for (int e = k * EPS; e < (k + 1) * EPS && e < NEL - 4; ++e)
                            mxc[k % 4] = fmax_nan(mxc[k % 4], s[e / 16][e % 16]);
                        asm volatile("" : "+v"(mxc[k % 4]));
                    }
                    if (i >= NSM) __builtin_amdgcn_sched_barrier(0);
                }
                m_pre = max_xor32(fmax_nan(fmax_nan(mxc[0], mxc[1]), fmax_nan(mxc[2], mxc[3]))) * scale2;
            } else if (do_pv) {
    #pragma unroll
                for (int i = 0; i < NPVM; ++i)
                    acc_o[i % NDB] = E::mfma(pv_operand(vb_prev, i), pf[i / NDB],
                                                                             acc_o[i % NDB]);
            } else if (do_qk) {
                const f32x16_t zero = {};
    #pragma unroll
                for (int i = 0; i < NSM; ++i)
                    s[i % NCB] = E::mfma(qk_operand(kb, i), qf[i / NCB],
                                                                         i < NCB ? zero : s[i % NCB]);
                m_pre = tile_max();
            }
            __builtin_amdgcn_s_setprio(0);
        };

        // Softmax step of tile t: mask, row max, conditional rescale, P and its row sum.
        auto step_softmax = [&](int t) __attribute__((always_inline)) {
            if (t < 0 || t >= my_tiles) return;
            const int kv0 = t * BN;
            const bool ragged = kv0 + BN > Lk;
            const bool diag = CAUSAL && (kv0 + BN - 1 > wrow0 + off);
            if (ragged || diag) {
    #pragma unroll
                for (int c = 0; c < NCB; ++c) {
                    // Keys from lim on are dead for this row: past Lk, or (causal)
                    // past qrow + off. Against the offset of key (c, r) within the
                    // lane's keys that is one compare with a small constant.
                    const int lim = CAUSAL ? min(Lk, qrow + off + 1) : Lk;
                    const int rel = lim - (kv0 + c * 32 + h * 8);
    #pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if ((r >> 3) * 16 + (r & 7) >= rel) s[c][r] = -INFINITY;
                }
            }
            // The row sum runs as several independent chains (one chain of
            // dependent adds would leave the VALU waiting on its own latency).
            constexpr int NCH = 4;
            // Row maximum: from the MFMA step unless this tile was
            // just masked.
            const float m_tile = (ragged || diag) ? tile_max() : m_pre;
            // Move the maximum (and rescale O, l) only when some row of the wave
            // outgrew it by more than the threshold.
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
            float lsc[NCH];            // chains start from the tile's first values (no 0 + p)
    #pragma unroll
            for (int c = 0; c < NCB; ++c)
    #pragma unroll
                for (int u = 0; u < 2; ++u) {
                    float p[8];
    #pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        p[e] = exp2_hw(__builtin_fmaf(s[c][u * 8 + e], scale2, -m_run));
                        lsc[e % NCH] = (c == 0 && u == 0 && e < NCH) ? p[e] : lsc[e % NCH] + p[e];
                    }
                    u32x4_t w;
                    w[0] = E::pack2(p[0], p[1]);
                    w[1] = E::pack2(p[2], p[3]);
                    w[2] = E::pack2(p[4], p[5]);
                    w[3] = E::pack2(p[6], p[7]);
                    pf[c * 2 + u] = __builtin_bit_cast(V8, w);
                }
            const float lsum = (lsc[0] + lsc[1]) + (lsc[2] + lsc[3]);
            l_run += lsum;
        };

        // Ping-pong schedule. Every wave runs the same sequence of steps
        //     M(0) | S(0) | M(1) | S(1) | ... | M(T)
        // separated by workgroup barriers, where M(t) = PV(t-1) + QK(t) on the
        // matrix core and S(t) = softmax of tile t on the VALU. Group 1 executes
        // one extra barrier first (and group 0 one at the end): barriers match by
        // count, so group 1 always runs one step behind group 0 and, on every SIMD,
        // one wave feeds the matrix core while the other does softmax.
        // Tile buffers: K(t) in k_lds[t%2], V(t) in v_lds[t%2]. Every load is
        // waited for at the end of the issuing wave's S step, and the barrier after
        // it publishes the tile.
        // Group 0 loads K(t+1) and V(t) right after its M(t); group 1's M(t-1),
        // the last reader of both buffers, is over, and group 0's M(t+1) is the
        // first reader. K(0) is loaded before the loop.
        // Wave-uniform by construction; readfirstlane makes that visible, so the
        // conditional barriers below are scalar branches.
        const bool loader = __builtin_amdgcn_readfirstlane(group) == 0;
        // One M step and one S step. The barrier between them protects no LDS data
        // (it only keeps the two groups a step apart), so it is a plain s_barrier
        // without the memory fence of __syncthreads, which would otherwise wait
        // for the tile DMA still in flight. The barrier after the S step publishes
        // the DMA that the loader waves have just waited for.
        auto tile_steps = [&](int t, const uint16_t* kb, uint16_t* vb_prev, uint16_t* kb_next,
                              uint16_t* vb_cur) __attribute__((always_inline)) {
            step_mfma(t, kb, vb_prev);
            if (loader && t < ntiles) {
                if (t + 1 < ntiles) dma(K, ld_koff, (t + 1) * BN, kb_next);
                dma(V, ld_voff, t * BN, vb_cur);
            }
            // sched_barrier(0): no instruction moves across the step boundary, so
            // the two steps keep their own (smaller) sets of live registers.
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            step_softmax(t);
            // vmcnt(0) on every wave (a no-op for waves with no DMA in flight), so
            // the compiler knows no tile DMA is pending past this point.
            __builtin_amdgcn_s_waitcnt(0xF70);
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
        };

        // Prologue. Group 0 needs its Q rows and K(0) for its first step, group 1
        // its own Q rows a step later (and V(0) is read first by group 0's second
        // step). With every workgroup of the launch reading its Q at once the
        // loads queue at HBM, so group 0 issues first and starts as soon as its
        // own loads have landed; group 1 issues after the first barrier and waits
        // for its loads only after the second, while group 0's first step runs.
        // Its extra barrier below (the one group 0 passes after that step) then
        // publishes V(0).
        if (loader) {
            load_q();
            if (ntiles > 0) dma(K, ld_koff, 0, k_lds0);
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (!loader) {
            load_q();
        }
        if (loader) __builtin_amdgcn_s_waitcnt(0xF70);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();              // K(0) complete
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0xF70);         // group 1: its Q rows and V(0)
        // The Q reads below must not move above the waits (the barrier and the
        // wait intrinsics do not order memory accesses for the compiler).
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        __builtin_amdgcn_sched_barrier(0);
        // Q rows from the staging area into the B operand registers.
    #pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
            qw[kk] = *(LDS_AS const u32x4_t*)(LDS_AS const uint16_t*)(qst + j * D + ((kk * 2 + h) ^ (j & (CPR - 1))) * 8);
        // Fused RoPE prologue on Q: the row is rotated in registers, once per
        // workgroup, at its position (qrow, shifted by the bottom-right offset so
        // the queries are the newest tokens). Both partners of every rotated pair
        // are in this lane: d and d + D/2 (rotate-half) are chunks kk and
        // kk + D/32 of the same half h; adjacent pairs share a chunk.
        if (rope_cos && qrow < Nq) {
            const int pos = max(0, qrow + off);
            const float* cr = rope_cos + (size_t)pos * (D / 2);
            const float* sr = rope_sin + (size_t)pos * (D / 2);
            if (rope_style == kRopeHalf) {
    #pragma unroll
                for (int kk = 0; kk < NKK / 2; ++kk) {
                    const int i0 = kk * 16 + h * 8;
                    const f32x4_t c0 = *(const f32x4_t*)(cr + i0), c1 = *(const f32x4_t*)(cr + i0 + 4);
                    const f32x4_t s0 = *(const f32x4_t*)(sr + i0), s1 = *(const f32x4_t*)(sr + i0 + 4);
                    const float c[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
                    const float sn[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
                    uint32_t a[4] = {qw[kk][0], qw[kk][1], qw[kk][2], qw[kk][3]};
                    uint32_t b[4] = {qw[kk + NKK / 2][0], qw[kk + NKK / 2][1], qw[kk + NKK / 2][2], qw[kk + NKK / 2][3]};
                    rope_half_chunks<T>(a, b, c, sn);
                    qw[kk] = u32x4_t{a[0], a[1], a[2], a[3]};
                    qw[kk + NKK / 2] = u32x4_t{b[0], b[1], b[2], b[3]};
                }
            } else {
    #pragma unroll
                for (int kk = 0; kk < NKK; ++kk) {
                    const int p0 = kk * 8 + h * 4;
                    const f32x4_t c4 = *(const f32x4_t*)(cr + p0), s4 = *(const f32x4_t*)(sr + p0);
                    const float c[4] = {c4[0], c4[1], c4[2], c4[3]};
                    const float sn[4] = {s4[0], s4[1], s4[2], s4[3]};
                    uint32_t x[4] = {qw[kk][0], qw[kk][1], qw[kk][2], qw[kk][3]};
                    rope_pair_chunk<T>(x, c, sn);
                    qw[kk] = u32x4_t{x[0], x[1], x[2], x[3]};
                }
            }
        }
    #pragma unroll
        for (int kk = 0; kk < NKK; ++kk) qf[kk] = __builtin_bit_cast(V8, qw[kk]);
        if (!loader) __builtin_amdgcn_s_barrier();
        // Steps M(t), S(t) for t = 0 .. ntiles (M(ntiles) is the last PV product,
        // S(ntiles) is empty); two tiles per iteration keep buffer choice static.
        for (int t = 0; t <= ntiles; t += 2) {
            tile_steps(t, k_lds0, v_lds1, k_lds1, v_lds0);
            if (t + 1 > ntiles) break;
            tile_steps(t + 1, k_lds1, v_lds0, k_lds0, v_lds1);
        }
        if (loader) __builtin_amdgcn_s_barrier();

        // Epilogue: O / l to bf16, LSE = (m + log2 l) * ln 2; a row that saw no
        // key (l = 0, O = 0) gets O = 0 and LSE = -inf, and a row that met a NaN
        // (l = NaN) gets NaN in both.
        const float l_tot = sum_xor32(l_run);
        const float inv = l_tot != 0.f ? 1.0f / l_tot : 0.f;
        // O goes out through the wave's row staging (its Q reads ended before
        // the key loop) so that every store writes whole rows. O and LSE are
        // stored non-temporal: nothing here reads them again, and they would
        // otherwise take L2 lines that hold other workgroups' K/V tiles.
        {
            uint16_t* ost = qst;
    #pragma unroll
            for (int db = 0; db < NDB; ++db)
    #pragma unroll
                for (int a4 = 0; a4 < 4; ++a4) {
                    const int c = db * 4 + a4;     // 16-byte chunk of the row: d = 8c .. 8c + 7
                    u32x2_t w;
                    w[0] = E::pack2(acc_o[db][a4 * 4 + 0] * inv, acc_o[db][a4 * 4 + 1] * inv);
                    w[1] = E::pack2(acc_o[db][a4 * 4 + 2] * inv, acc_o[db][a4 * 4 + 3] * inv);
                    *(LDS_AS u32x2_t*)(LDS_AS uint16_t*)(ost + j * D + (c ^ (j & (CPR - 1))) * 8 + h * 4) = w;
                }
            // The reads below take other lanes' writes: one wave's LDS
            // operations complete in order once issued, and the fence keeps the
            // compiler from moving the reads ahead.
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            constexpr int RPI = 64 / CPR;          // rows per read instruction
            constexpr int NIT = 32 / RPI;
            const int c = lane % CPR;
            u32x4_t w[NIT];
    #pragma unroll
            for (int it = 0; it < NIT; ++it) {
                const int r = it * RPI + lane / CPR;
                w[it] = *(LDS_AS const u32x4_t*)(LDS_AS const uint16_t*)(ost + r * D + (c ^ (r & (CPR - 1))) * 8);
            }
            uint16_t* orow = Og + ((size_t)bh * Nq + wrow0 + lane / CPR) * D + c * 8;
    #pragma unroll
            for (int it = 0; it < NIT; ++it)
                if (wrow0 + it * RPI + lane / CPR < Nq) __builtin_nontemporal_store(w[it], (u32x4_t*)(orow + it * RPI * D));
        }
        if (qrow < Nq && h == 0 && LSEg)
            __builtin_nontemporal_store(l_tot != 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY, &LSEg[(size_t)bh * Nq + qrow]);

        // The next block's loads reuse the tile buffers and the row staging.
        if constexpr (PERSIST) __syncthreads();
    }
}

namespace {
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];     // 0 until the device is first asked
}  // namespace

int paired_schedule_grid(int slots, int n_bh, int blocks_per_head) {
    const int g = slots & ~7;
    const long long blocks = (long long)n_bh * blocks_per_head;
    const long long pairs = (long long)n_bh * ((blocks_per_head + 1) / 2);
    if (g <= 0 || blocks <= g || pairs < g) return 0;
    // The busiest workgroup runs ceil(pairs / g) pairs against pairs / g on
    // average: keep that loss within 5% (a grid with 1.3 pairs per
    // workgroup would run 2 on some and idle the rest half the time).
    const long long rounds = (pairs + g - 1) / g;
    return (rounds * g - pairs) * 20 <= pairs ? g : 0;
}

hipError_t device_cu_count(int* n) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    int c = g_cu_count[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        g_cu_count[dev].store(c, std::memory_order_relaxed);
    }
    *n = c;
    return hipSuccess;
}

template <typename T, int D>
static hipError_t launch_one(const FwdArgs& a) {
    const int nqb = (a.Nq + BM_FWD - 1) / BM_FWD;
    const int n_bh = a.B * a.H;
    int grid = n_bh * nqb;
    bool persist = false;
    // Causal blocks of unequal cost and more of them than one per CU: a
    // persistent grid of one workgroup per CU (the kernel fits one per CU)
    // with the paired schedule above, when every workgroup gets a pair. Only
    // for self-attention shapes (Nq = Nk, no key padding), where a block's
    // cost is linear in its index and paired blocks cost the same; clamped
    // costs (Nq != Nk) or padding that differs between batch entries keep the
    // one-block-per-workgroup launch.
    if (a.causal != kCausalNone && !a.kv_lens && a.Nq == a.Nk && grid > 0) {
        int cus = 0;
        const hipError_t e = device_cu_count(&cus);
        if (e != hipSuccess) return e;
        const int g = paired_schedule_grid(cus, n_bh, nqb);
        if (g > 0) {
            grid = g;
            persist = true;
        }
    }
    auto kern = persist ? fwd_mfma_kernel<T, D, true> : fwd_mfma_kernel<T, D, false>;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kFwdThreads), 0, a.stream,
                       (const uint16_t*)a.Q, (const uint16_t*)a.K, (const uint16_t*)a.V,
                       (uint16_t*)a.O, a.LSE, a.kv_lens, a.H, a.Nq, a.Nk, nqb, a.scale * kLog2e, a.causal,
                       a.rope_cos, a.rope_sin, a.rope_style, n_bh);
    return hipGetLastError();
}

hipError_t launch_fwd_bf16(const FwdArgs& a) {
    return a.D == 128 ? launch_fwd16(a, false) : launch_one<__bf16, 64>(a);
}

hipError_t launch_fwd_f16(const FwdArgs& a) {
    return a.D == 128 ? launch_fwd16(a, true) : launch_one<_Float16, 64>(a);
}

}  // namespace fa
