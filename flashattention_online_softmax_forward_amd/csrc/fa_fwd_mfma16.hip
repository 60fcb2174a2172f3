// FlashAttention forward for gfx950 with D = 128 and bf16 or fp16 inputs, on
// the 16x16x32 MFMA (v_mfma_f32_16x16x32_bf16 / _f16, fp32 accumulation).
//
// Method (iThome FlashAttention article, "three states"; ML compiler page,
// section 11.9): a workgroup owns BM = 256 query rows of one (batch, head) and
// streams key/value tiles of 64 keys past them, carrying per row the running
// maximum m, the running sum l and the unnormalised output O; each tile moves
// m (conditionally, see below), rescales O and l by alpha = exp(m_old - m_new),
// adds P = exp(S - m) to l and P V to O, and the block ends with O / l and
// LSE = m + ln l (FA2 visualization, "Write the data back to HBM"). Scores are
// kept in base 2 (scale times log2(e); ML compiler page, section 11.7).
//
// The schedule is the one of fa_fwd_mfma.hip (8 waves x 32 query rows, one
// workgroup per CU, the two wave groups a step apart in a ping-pong of MFMA
// and softmax steps, K/V tiles DMA'd into swizzled LDS, persistent launches
// for causal self-attention); what differs is the MFMA shape. On random
// operands the 32x32x16 MFMA holds the chip at its power limit at a much
// lower engine clock than the 16x16x32 one doing the same work (a bare MFMA
// loop: 1.33-1.47 PFLOP/s at 1.67-1.71 GHz against 1.97 PFLOP/s at
// 1.96 GHz), and this kernel is bound by that power limit.
//
// 16x16x32 layouts (lane l, n = l % 16, g = l / 16): A lane holds row n,
// k = 8g..8g+7; B lane holds k = 8g..8g+7 of column n; the accumulator lane
// holds rows 4g..4g+3 of column n. A wave's 32 query rows are two row blocks
// rb of 16, so each lane carries two query rows, rb*16 + n.
//   * S^T = K Q^T per 16-key block kb: A = 16 K rows (d = 32kc + 8g.., from
//     LDS), B = Q (registers for the whole key loop); the lane ends with keys
//     4g..4g+3 of the block for its row. The K rows are permuted: row m of
//     block kb reads key 32(kb/2) + 8(m/4) + 4(kb%2) + m%4, so that blocks
//     2c and 2c+1 give the lane keys 32c + 8g .. 32c + 8g + 7 of its row, in
//     order, which rounded to 16 bits is exactly its B operand of the PV MFMA
//     over that 32-key step. P never leaves registers.
//   * O^T += V^T P^T per 16-wide d block: A = V^T (8 consecutive keys of one
//     column per lane: two ds_read_b64_tr_b16), B = P^T from the S
//     accumulators. One A operand serves both row blocks, as does one K
//     operand above.
//   * Row maximum: in-lane over the lane's 16 keys, then across the four lane
//     groups with v_permlane16_swap and v_permlane32_swap. Row sums stay
//     per lane until the end.

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kW16 = 8;                          // waves per workgroup
constexpr int kT16 = 64 * kW16;
constexpr int kD16 = 128;
constexpr int kBN16 = 64;                        // keys per tile
constexpr int kTile16 = kBN16 * kD16;            // elements of one K (or V) tile
constexpr int kCpr16 = kD16 / 8;                 // 16-byte chunks per row
constexpr int kNkb16 = kBN16 / 16;               // 16-key blocks of S^T per tile
constexpr int kNkc16 = kD16 / 32;                // 32-wide d steps of the S MFMA
constexpr int kNdb16 = kD16 / 16;                // 16-wide d blocks of O^T
constexpr int kNpc16 = kBN16 / 32;               // 32-key steps of the PV MFMA
constexpr int kRb16 = 32 * kD16;                 // elements of one wave's 32 rows
constexpr int kNld16 = kBN16 * kCpr16 / (64 * (kW16 / 2));   // DMA chunks per thread and tensor
// Conditional rescaling bounds (as in fa_fwd_mfma.hip): the maximum moves only
// when a tile's P against it could exceed 2^15, tested on the tile maximum or
// on a lane's share of the row sum.
constexpr float kThr16 = 15.0f;
constexpr float kSum16 = 32768.0f;

// 16-byte chunk swizzles of the row-major K and V tiles (16 chunks per row,
// a row spans the 64 LDS banks once).
// K: the 16 lanes of a lane group read one chunk of keys 8(m/4) + m%4 (+ 4
// for odd blocks), m = 0..15: (key & 3) | ((key >> 3) & 3) << 2 is then m,
// a distinct chunk per lane.
__device__ __forceinline__ int k16_swz(int key) { return (key & 3) | (((key >> 3) & 3) << 2); }
// V: a transpose read of lanes 0-31 covers keys k0 + 8g + 0..3 (g = 0, 1)
// and the two chunks of a 16-column block, each lane 8 bytes: the even
// swizzle 2((key & 3) | ((key >> 3) & 1) << 2) keeps all 16 chunks apart.
__device__ __forceinline__ int v16_swz(int key) { return 2 * ((key & 3) | (((key >> 3) & 1) << 2)); }

}  // namespace

#define LDS16 __attribute__((address_space(3)))

template <typename T, bool PERSIST>
__global__ __launch_bounds__(kT16, 1)
void fwd_mfma16_kernel(const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg,
                       const uint16_t* __restrict__ Vg, uint16_t* __restrict__ Og,
                       float* __restrict__ LSEg, const int* __restrict__ kv_lens, int H, int Nq, int Nk,
                       int nqb, float scale2, int causal, const float* __restrict__ rope_cos,
                       const float* __restrict__ rope_sin, int rope_style, int n_bh) {
    const bool CAUSAL = causal != kCausalNone;
    using E = Elem<T>;
    using V8 = typename E::v8;
    using V4 = typename E::v4;
    constexpr int D = kD16, BN = kBN16, TILE = kTile16, CPR = kCpr16, RB = kRb16, NLD = kNld16;

    // Two K and two V tile buffers, distinct arrays selected statically (the
    // phase loop is unrolled over two tiles), so a DMA into one is known not
    // to alias reads of another; row staging for Q in and O out.
    __shared__ __attribute__((aligned(1024))) uint16_t k_lds0[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t k_lds1[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t v_lds0[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t v_lds1[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t row_lds[kW16 * RB];

    // Work of this workgroup: one query block or, in a persistent launch
    // (causal self-attention with more query blocks than CUs), the paired
    // list of fa_fwd_mfma.hip: blocks nqb - 1 - r and r of a head at equal
    // cost, contiguous pair ranges per XCD, taken in turn.
    const int npair = (nqb + 1) / 2;
    const int xcd = blockIdx.x & 7;
    const int per_xcd = gridDim.x >> 3;
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
        // Opaque per block (persistent launches): offsets derived from the
        // thread index are recomputed in each block, not held across the loop.
        int tid = threadIdx.x;
        if constexpr (PERSIST) asm volatile("" : "+v"(tid));
        const int wave = tid >> 6;
        const int group = wave >> 2;
        const int lane = tid & 63;
        const int n = lane & 15;
        const int g = lane >> 4;

        const int q0 = qb * BM_FWD;
        const uint16_t* Q = Qg + (size_t)bh * Nq * D;
        const uint16_t* K = Kg + (size_t)bh * Nk * D;
        const uint16_t* V = Vg + (size_t)bh * Nk * D;
        const int Lk = real_keys(kv_lens, bh / H, Nk);
        const int off = causal == kCausalBottomRight ? Lk - Nq : 0;   // key j visible from row i iff j <= i + off
        const int wrow0 = q0 + wave * 32;

        // The wave's 32 Q rows go to its row staging with buffer loads (whole
        // rows, four per load; rows past Nq are out of the resource and arrive
        // as zeros), streamed past L2 (each is read by one workgroup).
        const int qwave = __builtin_amdgcn_readfirstlane(wave);
        uint16_t* const qst = row_lds + qwave * RB;
        auto load_q = [&]() __attribute__((always_inline)) {
            constexpr int NQS = RB / 512;
            uint32_t qoff[NQS];
#pragma unroll
            for (int i = 0; i < NQS; ++i) {
                const int p = i * 64 + lane;
                const int row = p / CPR;
                qoff[i] = (uint32_t)(row * D + ((p % CPR) ^ (row & (CPR - 1))) * 8) * 2 - (i % 4) * 1024;
            }
            const int qrow0 = q0 + qwave * 32;
            const int qrows = __builtin_amdgcn_readfirstlane(min(max(Nq - qrow0, 0), 32));
            const int qfirst = __builtin_amdgcn_readfirstlane(min(qrow0, Nq));
            const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(Q + (size_t)qfirst * D), (short)0, qrows * D * 2, kBufferRsrcWord3);
            static_assert(NQS % 4 == 0, "slots in groups of 4");
#pragma unroll
            for (int gq = 0; gq < NQS; gq += 4)
                buffer_lds_slots<4, 0, kCachePolicyNT>(rsrc, (LDS16 void*)(LDS16 uint16_t*)(qst + gq * 512), qoff + gq);
        };
        // Q as the B operand of S^T: row block rb, d = 32kc + 8g .. +7 of row rb*16 + n.
        u32x4_t qw[2][kNkc16];
        V8 qf[2][kNkc16];

        int kend = Lk;
        if (CAUSAL) kend = max(0, min(Lk, min(q0 + BM_FWD, Nq) + off));
        const int ntiles = (kend + BN - 1) / BN;
        const int wlast = wrow0 + 31 + off;    // last key the wave's last row may see
        const int my_tiles = CAUSAL ? (wlast < 0 ? 0 : min(ntiles, wlast / BN + 1)) : ntiles;

        // Tile loads: chunk p = (lwave*NLD + i)*64 + lane of a tile lands at
        // byte 16p of the LDS tile and holds logical chunk (p % CPR) ^ swz(row)
        // of row p / CPR; offsets stored net of slot i's immediate (i KB).
        const int lwave = __builtin_amdgcn_readfirstlane(wave & 3);
        uint32_t ld_koff[NLD], ld_voff[NLD];
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int p = (lwave * NLD + i) * 64 + lane;
            const int row = p / CPR;
            ld_koff[i] = (uint32_t)(row * D + ((p % CPR) ^ k16_swz(row)) * 8) * 2 - i * 1024;
            ld_voff[i] = (uint32_t)(row * D + ((p % CPR) ^ v16_swz(row)) * 8) * 2 - i * 1024;
        }
        auto dma = [&](const uint16_t* src, const uint32_t* voff, int kv0, uint16_t* dst) __attribute__((always_inline)) {
            const int rows = min(Lk - kv0, BN);
            const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(src + (size_t)kv0 * D), (short)0, rows * D * 2, kBufferRsrcWord3);
            buffer_lds_slots<NLD>(rsrc, (LDS16 void*)(LDS16 uint16_t*)(dst + lwave * NLD * 512), voff);
        };

        // O^T per d block and row block: rows 4g..4g+3 of the block's d, column
        // (row) n.
        f32x4_t acc_o[kNdb16][2];
#pragma unroll
        for (int db = 0; db < kNdb16; ++db)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) acc_o[db][rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        f32x4_t s[kNkb16][2];      // S^T of the tile between its MFMA step and its softmax step
        V8 pf[kNpc16][2];          // P of the tile between its softmax step and its PV step

        float m_run[2] = {kNoKeyMax, kNoKeyMax};   // base-2 scaled maximum per row
        float l_run[2] = {0.f, 0.f};               // this lane's share of each row's sum
        bool spec = false;                          // exponentials before the maximum (wave-uniform)

        // Operands. K block kb, d step kc: lane (n, g) reads 16 bytes of key
        // 32(kb/2) + 8(n/4) + 4(kb%2) + n%4 at d = 32kc + 8g.
        const int kperm = 8 * (n >> 2) + (n & 3);
        auto k_operand = [&](const uint16_t* kb_lds, int i) __attribute__((always_inline)) {
            const int kc = i / kNkb16, kb = i % kNkb16;
            const int key = 32 * (kb >> 1) + 4 * (kb & 1) + kperm;
            return *(LDS16 const V8*)(LDS16 const uint16_t*)(kb_lds + key * D + (((4 * kc + g) ^ k16_swz(key)) * 8));
        };
        // V^T, 32-key step c, d block db: lane (n, g) gets column 16db + n of keys
        // 32c + 8g .. +7, as two transpose reads of 4 keys (source lane s of a
        // 16-lane group points at 4 columns of key k0 + s/4).
        auto v_operand = [&](const uint16_t* vb, int i) __attribute__((always_inline)) {
            const int c = i / kNdb16, db = i % kNdb16;
            V4 part[2];
#pragma unroll
            for (int rd = 0; rd < 2; ++rd) {
                const int key = 32 * c + 8 * g + 4 * rd + (n >> 2);
                const int col = 16 * db + 4 * (n & 3);
                const int chunk = (col >> 3) ^ v16_swz(key);
                part[rd] = E::tr_read((LDS16 V4*)(LDS16 uint16_t*)(vb + key * D + chunk * 8 + (col & 7)));
            }
            return V8{part[0][0], part[0][1], part[0][2], part[0][3], part[1][0], part[1][1], part[1][2], part[1][3]};
        };
        // Scaled maximum of each row over the tile (NaN-propagating).
        auto tile_max = [&](float* mx) __attribute__((always_inline)) {
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                float a = fmax_nan(fmax_nan(s[0][rb][0], s[0][rb][1]), fmax_nan(s[0][rb][2], s[0][rb][3]));
                float b = fmax_nan(fmax_nan(s[1][rb][0], s[1][rb][1]), fmax_nan(s[1][rb][2], s[1][rb][3]));
#pragma unroll
                for (int kb = 2; kb < kNkb16; ++kb) {
                    float& acc = (kb & 1) ? b : a;
                    acc = fmax_nan(acc, fmax_nan(fmax_nan(s[kb][rb][0], s[kb][rb][1]), fmax_nan(s[kb][rb][2], s[kb][rb][3])));
                }
                mx[rb] = max_xor32(max_xor16(fmax_nan(a, b))) * scale2;
            }
        };

        // MFMA step of tile t: O^T += V^T P^T for tile t-1, then S^T = K Q^T for
        // tile t, one stream of operands (each feeding both row blocks) read
        // LEAD operands ahead.
        constexpr int NPVO = kNpc16 * kNdb16;      // PV operands per tile
        constexpr int NQKO = kNkc16 * kNkb16;      // QK operands per tile
        constexpr int LEAD = 4;
        auto step_mfma = [&](int t, const uint16_t* kb_lds, const uint16_t* vb_prev) __attribute__((always_inline)) {
            // Nothing LDS-side is pending here, but a kernel-argument scalar load
            // may be on the first entry; waiting once lets the first MFMA wait
            // for its own operand only (scalar loads return out of order).
            // Unlike the 32x32x16 kernel, this step keeps the default wave
            // priority: with twice the MFMA instructions per step it would
            // otherwise win the SIMD's issue slots from the other wave's
            // softmax step too often (measured: priority 1 is 1-2% slower on
            // causal 4x32x4096 and level elsewhere).
            __builtin_amdgcn_s_waitcnt(0xC07F);
            const bool do_pv = t >= 1 && t - 1 < my_tiles;
            const bool do_qk = t < my_tiles;
            const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
            auto pv_mfmas = [&](int i, V8 a) __attribute__((always_inline)) {
                const int c = i / kNdb16, db = i % kNdb16;
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) acc_o[db][rb] = E::mfma16(a, pf[c][rb], acc_o[db][rb]);
            };
            auto qk_mfmas = [&](int i, V8 a) __attribute__((always_inline)) {
                const int kc = i / kNkb16, kb = i % kNkb16;
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) s[kb][rb] = E::mfma16(a, qf[rb][kc], kc == 0 ? zero : s[kb][rb]);
            };
            if (do_pv && do_qk) {
                constexpr int NO = NPVO + NQKO;
                auto operand = [&](int i) __attribute__((always_inline)) {
                    return i < NPVO ? v_operand(vb_prev, i) : k_operand(kb_lds, i - NPVO);
                };
                V8 ring[LEAD];
#pragma unroll
                for (int i = 0; i < LEAD; ++i) ring[i] = operand(i);
                __builtin_amdgcn_sched_group_barrier(0x100, 2 * LEAD, 0);
#pragma unroll
                for (int i = 0; i < NO; ++i) {
                    const V8 a = ring[i % LEAD];
                    if (i + LEAD < NO) ring[i % LEAD] = operand(i + LEAD);
                    if (i < NPVO) pv_mfmas(i, a);
                    else qk_mfmas(i - NPVO, a);
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                    const int nx = i + LEAD;
                    if (nx < NPVO) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                    else if (nx < NO) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
            } else if (do_pv) {
#pragma unroll
                for (int i = 0; i < NPVO; ++i) pv_mfmas(i, v_operand(vb_prev, i));
            } else if (do_qk) {
#pragma unroll
                for (int i = 0; i < NQKO; ++i) qk_mfmas(i, k_operand(kb_lds, i));
            }
        };

        // Softmax step of tile t: mask, conditional rescale, P and its row sums.
        auto step_softmax = [&](int t) __attribute__((always_inline)) {
            if (t < 0 || t >= my_tiles) return;
            const int kv0 = t * BN;
            const bool ragged = kv0 + BN > Lk;
            const bool diag = CAUSAL && (kv0 + BN - 1 > wrow0 + off);
            if (ragged || diag) {
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) {
                    // Keys from lim on are dead for the row: past Lk, or (causal)
                    // past row + off. Key (kb, i) of this lane is kv0 + 32(kb/2)
                    // + 8g + 4(kb%2) + i.
                    const int row = wrow0 + rb * 16 + n;
                    const int lim = CAUSAL ? min(Lk, row + off + 1) : Lk;
                    const int rel = lim - (kv0 + 8 * g);
#pragma unroll
                    for (int kb = 0; kb < kNkb16; ++kb)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (32 * (kb >> 1) + 4 * (kb & 1) + i >= rel) s[kb][rb][i] = -INFINITY;
                }
            }
            // P against m_run, packed into the PV operands; the lane's share of
            // each row's sum of the tile.
            auto exp_tile = [&](float* lsum) __attribute__((always_inline)) {
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) {
                    float acc[2];
#pragma unroll
                    for (int c = 0; c < kNpc16; ++c) {
                        float p[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float sv = s[2 * c + (e >> 2)][rb][e & 3];
                            p[e] = exp2_hw(__builtin_fmaf(sv, scale2, -m_run[rb]));
                        }
                        const float part = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
                        acc[c & 1] = c < 2 ? part : acc[c & 1] + part;
                        u32x4_t w;
                        w[0] = E::pack2(p[0], p[1]);
                        w[1] = E::pack2(p[2], p[3]);
                        w[2] = E::pack2(p[4], p[5]);
                        w[3] = E::pack2(p[6], p[7]);
                        pf[c][rb] = __builtin_bit_cast(V8, w);
                    }
                    lsum[rb] = kNpc16 > 1 ? acc[0] + acc[1] : acc[0];
                }
            };
            auto move_max = [&](const float* m_tile) __attribute__((always_inline)) {
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) {
                    const float m_new = fmaxf(m_run[rb], m_tile[rb]);
                    const float alpha = exp2_hw(m_run[rb] - m_new);
                    m_run[rb] = m_new;
                    l_run[rb] *= alpha;
#pragma unroll
                    for (int db = 0; db < kNdb16; ++db) acc_o[db][rb] *= alpha;
                }
            };
            float lsum[2];
            if (spec) {
                // Exponentials against the kept maxima first: a lane whose share
                // of a row's sum is at most 2^15 has every P of it at most 2^15,
                // so the tile stands unless some lane went past that (or met a
                // NaN, or overflowed); then the maxima move and the tile is
                // exponentiated again.
                exp_tile(lsum);
                if (__builtin_amdgcn_ballot_w64(!(lsum[0] <= kSum16 && lsum[1] <= kSum16))) {
                    float m_tile[2];
                    tile_max(m_tile);
                    move_max(m_tile);
                    exp_tile(lsum);
                }
            } else {
                // The maxima first, moved only past the bound (always on the
                // first tile, against kNoKeyMax; O and l are 0 there).
                float m_tile[2];
                tile_max(m_tile);
                if (__builtin_amdgcn_ballot_w64(m_tile[0] > m_run[0] + kThr16 || m_tile[1] > m_run[1] + kThr16))
                    move_max(m_tile);
                exp_tile(lsum);
                // The first tile's row sums against their own maxima pick the
                // wave's way for later tiles: near 1 when one score stands far
                // above the rest (maxima that keep moving), near 10 for
                // unit-variance Q and K. Each row counted once (lane group 0).
                if (t == 0) {
                    const float r0 = sum_xor32(sum_xor16(lsum[0]));
                    const float r1 = sum_xor32(sum_xor16(lsum[1]));
                    const int small = __builtin_popcountll(__builtin_amdgcn_ballot_w64(g == 0 && r0 < 3.0f)) +
                                      __builtin_popcountll(__builtin_amdgcn_ballot_w64(g == 0 && r1 < 3.0f));
                    spec = small <= 2;
                }
            }
            l_run[0] += lsum[0];
            l_run[1] += lsum[1];
        };

        // Ping-pong schedule (see fa_fwd_mfma.hip): every wave runs
        //     M(0) | S(0) | M(1) | S(1) | ... | M(T)
        // separated by workgroup barriers; group 1 runs one barrier behind group
        // 0. Group 0 loads K(t+1) and group 1 V(t+1), each at the start of its
        // S(t), into the buffers whose last readers have finished.
        const bool loader = __builtin_amdgcn_readfirstlane(group) == 0;
        auto tile_steps = [&](int t, const uint16_t* kb_lds, uint16_t* vb_prev, uint16_t* kb_next) __attribute__((always_inline)) {
            step_mfma(t, kb_lds, vb_prev);
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            if (t + 1 < ntiles) {
                if (loader) dma(K, ld_koff, (t + 1) * BN, kb_next);
                else dma(V, ld_voff, (t + 1) * BN, vb_prev);
            }
            step_softmax(t);
            __builtin_amdgcn_s_waitcnt(0xF70);
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
        };

        // Prologue: group 0 issues its Q rows and K(0) first and starts as soon
        // as they have landed; group 1 issues its Q rows and V(0) after the
        // first barrier and waits for them after the second, while group 0's
        // first step runs.
        if (loader) {
            load_q();
            if (ntiles > 0) dma(K, ld_koff, 0, k_lds0);
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (!loader) {
            load_q();
            if (ntiles > 0) dma(V, ld_voff, 0, v_lds0);
        }
        if (loader) __builtin_amdgcn_s_waitcnt(0xF70);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();              // K(0) complete
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0xF70);         // group 1: its Q rows and V(0)
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int kc = 0; kc < kNkc16; ++kc) {
                const int row = rb * 16 + n;
                qw[rb][kc] = *(LDS16 const u32x4_t*)(LDS16 const uint16_t*)(qst + row * D + (((4 * kc + g) ^ (row & (CPR - 1))) * 8));
            }
        // Fused RoPE on Q, in registers: d and d + D/2 (rotate-half) are d steps
        // kc and kc + D/64 of the same lane group; adjacent pairs share a chunk.
        if (rope_cos) {
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const int qrow = wrow0 + rb * 16 + n;
                if (qrow >= Nq) continue;
                const int pos = max(0, qrow + off);
                const float* cr = rope_cos + (size_t)pos * (D / 2);
                const float* sr = rope_sin + (size_t)pos * (D / 2);
                if (rope_style == kRopeHalf) {
#pragma unroll
                    for (int kc = 0; kc < kNkc16 / 2; ++kc) {
                        const int i0 = 32 * kc + 8 * g;
                        const f32x4_t c0 = *(const f32x4_t*)(cr + i0), c1 = *(const f32x4_t*)(cr + i0 + 4);
                        const f32x4_t s0 = *(const f32x4_t*)(sr + i0), s1 = *(const f32x4_t*)(sr + i0 + 4);
                        const float cv[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
                        const float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
                        uint32_t a[4] = {qw[rb][kc][0], qw[rb][kc][1], qw[rb][kc][2], qw[rb][kc][3]};
                        const int kc2 = kc + kNkc16 / 2;
                        uint32_t b[4] = {qw[rb][kc2][0], qw[rb][kc2][1], qw[rb][kc2][2], qw[rb][kc2][3]};
                        rope_half_chunks<T>(a, b, cv, sv);
                        qw[rb][kc] = u32x4_t{a[0], a[1], a[2], a[3]};
                        qw[rb][kc2] = u32x4_t{b[0], b[1], b[2], b[3]};
                    }
                } else {
#pragma unroll
                    for (int kc = 0; kc < kNkc16; ++kc) {
                        const int p0 = 16 * kc + 4 * g;
                        const f32x4_t c4 = *(const f32x4_t*)(cr + p0), s4 = *(const f32x4_t*)(sr + p0);
                        const float cv[4] = {c4[0], c4[1], c4[2], c4[3]};
                        const float sv[4] = {s4[0], s4[1], s4[2], s4[3]};
                        uint32_t x[4] = {qw[rb][kc][0], qw[rb][kc][1], qw[rb][kc][2], qw[rb][kc][3]};
                        rope_pair_chunk<T>(x, cv, sv);
                        qw[rb][kc] = u32x4_t{x[0], x[1], x[2], x[3]};
                    }
                }
            }
        }
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int kc = 0; kc < kNkc16; ++kc) qf[rb][kc] = __builtin_bit_cast(V8, qw[rb][kc]);
        if (!loader) __builtin_amdgcn_s_barrier();
        for (int t = 0; t <= ntiles; t += 2) {
            tile_steps(t, k_lds0, v_lds1, k_lds1);
            if (t + 1 > ntiles) break;
            tile_steps(t + 1, k_lds1, v_lds0, k_lds0);
        }
        if (loader) __builtin_amdgcn_s_barrier();

        // Epilogue: O / l rounded to T, LSE = (m + log2 l) ln 2; a row that saw
        // no key (l = 0) gets O = 0 and LSE = -inf, a row that met a NaN NaN in
        // both. O goes out through the row staging as whole rows.
        float l_tot[2], inv[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            l_tot[rb] = sum_xor32(sum_xor16(l_run[rb]));
            inv[rb] = l_tot[rb] != 0.f ? 1.0f / l_tot[rb] : 0.f;
        }
        {
            uint16_t* ost = qst;
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const int row = rb * 16 + n;
#pragma unroll
                for (int db = 0; db < kNdb16; ++db) {
                    const int c = 2 * db + (g >> 1);       // chunk of d = 16db + 4g .. +3
                    u32x2_t w;
                    w[0] = E::pack2(acc_o[db][rb][0] * inv[rb], acc_o[db][rb][1] * inv[rb]);
                    w[1] = E::pack2(acc_o[db][rb][2] * inv[rb], acc_o[db][rb][3] * inv[rb]);
                    *(LDS16 u32x2_t*)(LDS16 uint16_t*)(ost + row * D + (c ^ (row & (CPR - 1))) * 8 + (g & 1) * 4) = w;
                }
            }
            // The reads below take other lanes' writes: one wave's LDS operations
            // complete in order, and the fence keeps the compiler from moving the
            // reads ahead.
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            constexpr int RPI = 64 / CPR;
            constexpr int NIT = 32 / RPI;
            const int c = lane % CPR;
            u32x4_t w[NIT];
#pragma unroll
            for (int it = 0; it < NIT; ++it) {
                const int r = it * RPI + lane / CPR;
                w[it] = *(LDS16 const u32x4_t*)(LDS16 const uint16_t*)(ost + r * D + (c ^ (r & (CPR - 1))) * 8);
            }
            uint16_t* orow = Og + ((size_t)bh * Nq + wrow0 + lane / CPR) * D + c * 8;
#pragma unroll
            for (int it = 0; it < NIT; ++it)
                if (wrow0 + it * RPI + lane / CPR < Nq) __builtin_nontemporal_store(w[it], (u32x4_t*)(orow + it * RPI * D));
        }
        if (g == 0 && LSEg) {
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const int qrow = wrow0 + rb * 16 + n;
                if (qrow < Nq)
                    __builtin_nontemporal_store(l_tot[rb] != 0.f ? (m_run[rb] + __log2f(l_tot[rb])) * kLn2 : -INFINITY,
                                                &LSEg[(size_t)bh * Nq + qrow]);
            }
        }
        // The next block's loads reuse the tile buffers and the row staging.
        if constexpr (PERSIST) __syncthreads();
    }
}

template <typename T>
hipError_t launch_fwd16_t(const FwdArgs& a) {
    const int nqb = (a.Nq + BM_FWD - 1) / BM_FWD;
    const int n_bh = a.B * a.H;
    int grid = n_bh * nqb;
    bool persist = false;
    if (a.causal != kCausalNone && !a.kv_lens && a.Nq == a.Nk && grid > 0) {
        int cus = 0;
        const hipError_t e = device_cu_count(&cus);
        if (e != hipSuccess) return e;
        const int gp = paired_schedule_grid(cus, n_bh, nqb);
        if (gp > 0) {
            grid = gp;
            persist = true;
        }
    }
    auto kern = persist ? fwd_mfma16_kernel<T, true> : fwd_mfma16_kernel<T, false>;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kT16), 0, a.stream,
                       (const uint16_t*)a.Q, (const uint16_t*)a.K, (const uint16_t*)a.V,
                       (uint16_t*)a.O, a.LSE, a.kv_lens, a.H, a.Nq, a.Nk, nqb, a.scale * kLog2e, a.causal,
                       a.rope_cos, a.rope_sin, a.rope_style, n_bh);
    return hipGetLastError();
}

hipError_t launch_fwd16(const FwdArgs& a, bool f16) {
    return f16 ? launch_fwd16_t<_Float16>(a) : launch_fwd16_t<__bf16>(a);
}

}  // namespace fa
