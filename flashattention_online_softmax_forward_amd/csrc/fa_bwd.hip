// Backward pass with recompute for gfx950 on the 16x16x32 MFMA
// (v_mfma_f32_16x16x32_bf16 / _f16), D = 64 or 128: the products of the
// "Backward with recompute" exercise and section 11.9 of the ML compiler page
// (only O and the per-row log-sum-exp L are kept from the forward pass; P is
// recomputed tile by tile as exp(S - L)). For one (batch, head):
//     D_i = sum_d dO[i,d] O[i,d]                      (bwd_dq16_kernel, stored)
//     P = exp(scale Q K^T - L),  dP = dO V^T,  dS = P * (dP - D)
//     dQ = scale dS K                                 (bwd_dq16_kernel)
//     dV = P^T dO,  dK = scale dS^T Q                 (bwd_dkdv16_kernel)
// with base-2 exponentials (L and scale multiplied by log2 e).
//
// gfx950 mapping (own design): two product kernels of 4 waves x 32 own rows
// (queries for dQ, keys for dK/dV), two or more workgroups per CU, the other
// side streamed through LDS in 32-row tiles (buffer_load_dwordx4 straight to
// LDS, double-buffered, one barrier per tile), no atomics: every output is
// written once. The 16x16x32 shape keeps the chip's power limit at a higher
// engine clock than the 32x32x16 one for the same work on random operands.
//
// 16x16x32 layouts (lane l, n = l % 16, g = l / 16): A lane holds row n,
// k = 8g..8g+7; B lane holds k = 8g..8g+7 of column n; the accumulator lane
// holds rows 4g..4g+3 of column n. A wave's 32 own rows are two column blocks
// of 16, and a 32-row tile of the streamed side is two row blocks of 16:
//   * The first products (S and dP, or their transposes) take the tile's rows
//     as A, with row m of block b reading tile row 8(m/4) + 4b + m%4, so the
//     lane ends with tile rows 8g + 4b + 0..3 of its own row: over both
//     blocks, the eight rows 8g..8g+7 in order, which rounded to 16 bits is
//     the B operand of the 32-row step of the products that follow (dV, dK or
//     dQ). P and dS never leave registers.
//   * The A operands of those products (the tile transposed: row d = 16db + n,
//     tile rows 8g..8g+7) are two ds_read_b64_tr_b16 of 4 rows each.
//   * Tiles are staged once and read both ways, with a 16-byte chunk swizzle
//     free of bank conflicts for the row reads (16 lanes, 16 rows, one chunk)
//     and the transpose reads (32 lanes, 8 rows of 2 chunks) that ignores row
//     bit 2, so the second row block and the second transpose read are
//     constant offsets.
//   * Masking: causal (key j visible from query i iff j <= i + off, off = 0
//     top-left or Lk - Nq bottom-right), padding keys (past the batch entry's
//     real key count Lk) and queries past Nq get P = 0 (so dS = 0 too); rows
//     past the end are staged as zeros and never stored.
//   * dQ, dK, dV are accumulated in fp32 and rounded to 16 bits once.

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kKvWaves = 4;
constexpr int kKvThreads = 64 * kKvWaves;
constexpr int kQT = 32;                          // rows per streamed tile
static_assert(BM_BWD == 32 * kKvWaves, "32 own rows per wave");
// Per head dimension D: 16-byte chunks per row, 32-wide d steps of the first
// products, 16-wide d blocks of the second ones, elements of one tile.
template <int D> struct Dims {
    static constexpr int CPR = D / 8, NKC = D / 32, NDB = D / 16, TILE = kQT * D, ROW4 = 4 * D * 2;
};

#define LDS16B __attribute__((address_space(3)))

// Chunk swizzle of the streamed tiles (see the header). With D = 64 a row is
// 8 chunks and two rows share the 64 banks: 2(row bit 1) | 4(row bit 3) |
// (row bit 4) does for each row parity what the D = 128 swizzle does (checked
// bank by bank on the host for both read patterns).
template <int D>
__device__ __forceinline__ int tile_swz(int row) {
    if constexpr (D == 128) return ((row & 3) << 1) | (((row >> 3) & 1) << 3) | ((row >> 4) & 1);
    else return (((row >> 1) & 1) << 1) | (((row >> 3) & 1) << 2) | ((row >> 4) & 1);
}
// Chunk swizzle of the dK/dV kernel's V block, read by 16 consecutive rows at a time.
template <int D>
__device__ __forceinline__ int vblk_swz(int row) {
    if constexpr (D == 128) return row & 15;
    else return (row >> 1) & 7;
}

// Staging of ROWS rows of a row-major [*, 128] array into LDS with chunk
// swizzle SWZ: chunk p of the tile lands at byte 16p and holds logical chunk
// (p % 16) ^ SWZ(row) of row p / 16. Wave w moves chunks (w*PER + i)*64 +
// lane with buffer loads straight to LDS; rows past `valid` are outside the
// resource and arrive as zeros.
template <int D, int ROWS, bool VBLK>
struct Stage16 {
    static constexpr int kCpr = D / 8;
    static constexpr int PER = ROWS * kCpr / kKvThreads;
    static_assert(PER * kKvThreads == ROWS * kCpr, "whole chunks per lane");
    static_assert(PER <= 4 || PER % 4 == 0, "slots in groups of up to 4");
    uint32_t voff[PER];
    __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int p = (wave * PER + i) * 64 + lane;
            const int row = p / kCpr;
            const int sw = VBLK ? vblk_swz<D>(row) : tile_swz<D>(row);
            voff[i] = (uint32_t)(row * D + ((p % kCpr) ^ sw) * 8) * 2u - (i % 4) * 1024u;
        }
    }
    __device__ __forceinline__ void stage(const uint16_t* src, int valid, uint16_t* dst, int wave) const {
        const __amdgpu_buffer_rsrc_t rsrc =
            __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, valid * D * 2, kBufferRsrcWord3);
        if constexpr (PER <= 4) {
            buffer_lds_slots<PER>(rsrc, (LDS16B void*)(LDS16B uint16_t*)(dst + wave * PER * 512), voff);
        } else {
#pragma unroll
            for (int q = 0; q < PER; q += 4)
                buffer_lds_slots<4>(rsrc, (LDS16B void*)(LDS16B uint16_t*)(dst + (wave * PER + q) * 512), voff + q);
        }
    }
};

// Store 32 rows x 128 of fp32 accumulators in the 16x16 layout (acc[db][kb2]:
// lane (n, g) holds columns 16db + 4g .. +3 of row 16kb2 + n) as 16-bit
// values times `mul` to rows dst[0 .. valid), through `stage` (32 x 128
// elements of LDS private to the wave), so that every store writes whole
// rows, 16 bytes per lane.
template <typename T, int D>
__device__ __forceinline__ void store_rows16(uint16_t* dst, int valid, const f32x4_t (*acc)[2], float mul,
                                             uint16_t* stage, int lane) {
    constexpr int kD = D, kCpr = D / 8, kNdb = D / 16;
    const int n = lane & 15, g = lane >> 4;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
        const int row = kb2 * 16 + n;
#pragma unroll
        for (int db = 0; db < kNdb; ++db) {
            const int c = 2 * db + (g >> 1);   // chunk of columns 16db + 4g .. +3
            u32x2_t w;
            w[0] = Elem<T>::pack2(acc[db][kb2][0] * mul, acc[db][kb2][1] * mul);
            w[1] = Elem<T>::pack2(acc[db][kb2][2] * mul, acc[db][kb2][3] * mul);
            *(LDS16B u32x2_t*)(LDS16B uint16_t*)(stage + row * kD + (c ^ (row & (kCpr - 1))) * 8 + (g & 1) * 4) = w;
        }
    }
    // The reads take other lanes' writes: one wave's LDS operations complete
    // in order once issued, and the fence keeps the compiler from moving the
    // reads ahead.
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    constexpr int RPI = 64 / kCpr;             // rows per store instruction
    constexpr int NIT = 32 / RPI;
    const int c = lane % kCpr;
    u32x4_t w[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int r = it * RPI + lane / kCpr;
        w[it] = *(LDS16B const u32x4_t*)(LDS16B const uint16_t*)(stage + r * kD + (c ^ (r & (kCpr - 1))) * 8);
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int r = it * RPI + lane / kCpr;
        if (r < valid) *(u32x4_t*)(dst + (size_t)r * kD + c * 8) = w[it];
    }
}

// N steps step(i, op(i)), each operand read LEAD steps ahead and no further
// (sched_barrier after every step), which bounds the registers a phase holds.
template <int N, int LEAD, typename Op, typename Step>
__device__ __forceinline__ void op_stream(Op op, Step step) {
    decltype(op(0)) ring[LEAD];
#pragma unroll
    for (int i = 0; i < LEAD && i < N; ++i) ring[i] = op(i);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const auto a = ring[i % LEAD];
        if (i + LEAD < N) ring[i % LEAD] = op(i + LEAD);
        step(i, a);
        __builtin_amdgcn_sched_barrier(0);
    }
}

}  // namespace

// dK and dV for 128 keys of one (batch, head): 4 waves x 32 keys, K in
// registers (B operand of S = Q K^T) and the block's V rows in LDS (B operand
// of dP = dO V^T), Q and dO streamed in 32-row tiles with their L and D
// values. A tile's phases (S, P, dV, dP, dS, dK) are separated by
// sched_barrier and read their LDS operands a bounded number of steps ahead,
// which keeps the D = 128 kernel within 256 VGPRs.
template <typename T, int D, bool PERSIST>
__global__ __launch_bounds__(kKvThreads, 2)
void bwd_dkdv16_kernel(const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg,
                       const uint16_t* __restrict__ Vg, const uint16_t* __restrict__ dOg,
                       const float* __restrict__ LSEg, const float* __restrict__ Dg,
                       uint16_t* __restrict__ dKg, uint16_t* __restrict__ dVg, const int* __restrict__ kv_lens,
                       int H, int Nq, int Nk, int nkb, float scale, float scale2, int causal, int n_bh) {
    using E = Elem<T>;
    using V8 = typename E::v8;
    using V4 = typename E::v4;
    constexpr int kD = D, kNkc = Dims<D>::NKC, kNdb = Dims<D>::NDB, kQTile = Dims<D>::TILE, kRow4 = Dims<D>::ROW4;
    const bool CAUSAL = causal != kCausalNone;

    // Small arrays first: every buffer's base then fits the 16-bit offset
    // field of the LDS instructions.
    __shared__ __attribute__((aligned(16))) float ld_lds[2][2 * kQT];  // per tile: L (base 2), then D
    __shared__ __attribute__((aligned(1024))) uint16_t q_lds0[kQTile];
    __shared__ __attribute__((aligned(1024))) uint16_t q_lds1[kQTile];
    __shared__ __attribute__((aligned(1024))) uint16_t o_lds0[kQTile];   // dO tiles
    __shared__ __attribute__((aligned(1024))) uint16_t o_lds1[kQTile];
    __shared__ __attribute__((aligned(1024))) uint16_t v_blk[BM_BWD * kD];

    // One key block per workgroup or, in a persistent launch (causal
    // self-attention with more blocks than resident workgroups), the forward
    // kernel's paired static schedule: low key blocks carry the most queries,
    // so block r pairs with nkb - 1 - r at equal cost; each XCD owns a
    // contiguous range of pairs and its workgroups take them in turn.
    const int npair = (nkb + 1) / 2;
    const int xcd = blockIdx.x & 7;
    const int per_xcd = gridDim.x >> 3;
    const long long all_pairs = (long long)n_bh * npair;
    const int p_lo = (int)(all_pairs * xcd / 8), p_hi = (int)(all_pairs * (xcd + 1) / 8);
    for (int wi = 0;; ++wi) {
        int bh, kb;
        if constexpr (!PERSIST) {
            if (wi > 0) break;
            const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
            bh = logical / nkb;
            kb = logical - bh * nkb;           // causal: low key blocks carry the most queries
        } else {
            const int p = p_lo + (int)(blockIdx.x >> 3) + (wi >> 1) * per_xcd;
            if (p >= p_hi) break;
            bh = p / npair;
            const int r = p - bh * npair;
            kb = (wi & 1) ? nkb - 1 - r : r;
            if ((wi & 1) && nkb - 1 - r == r) continue;   // odd count: the middle block is alone
        }
        int tid = threadIdx.x;
        if constexpr (PERSIST) asm volatile("" : "+v"(tid));
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int lane = tid & 63;
        const int n = lane & 15;
        const int g = lane >> 4;
        const int k0 = kb * BM_BWD;
        const int kw0 = k0 + wave * 32;
        const int Lk = real_keys(kv_lens, bh / H, Nk);
        const int doff = causal == kCausalBottomRight ? Lk - Nq : 0;   // key j visible from query i iff j <= i + doff

        const uint16_t* Q = Qg + (size_t)bh * Nq * kD;
        const uint16_t* dO = dOg + (size_t)bh * Nq * kD;
        const float* L = LSEg + (size_t)bh * Nq;
        const float* Dv = Dg + (size_t)bh * Nq;

        // K of the wave's keys as B operands of S = Q K^T: key kw0 + 16kb2 + n,
        // d = 32kc + 8g .. +7. Keys past Lk (padding) are zeros, so S = dP = 0
        // there and, with P = 0, dS = 0 whatever the padded cache holds.
        V8 kf[2][kNkc];
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
            const int key = kw0 + kb2 * 16 + n;
#pragma unroll
            for (int kc = 0; kc < kNkc; ++kc) {
                u32x4_t w = {0u, 0u, 0u, 0u};
                if (key < Lk) w = *(const u32x4_t*)(Kg + ((size_t)bh * Nk + key) * kD + kc * 32 + g * 8);
                kf[kb2][kc] = __builtin_bit_cast(V8, w);
            }
        }
        // Lane byte offsets of the LDS operand reads, the same for every tile
        // buffer (whose base folds into the instruction's offset field):
        //   rowoff[kc]: tile row 8(n/4) + n%4, chunk 4kc + g (row block 1: +4 rows);
        //   troff[db]: tile row 8g + n/4, columns 16db + 4(n%4) .. +3 (second
        //              transpose read: +4 rows);
        //   voff[kc]: V block row 32 wave + n, chunk 4kc + g (kb2 = 1: +16 rows).
        uint32_t rowoff[kNkc], troff[kNdb], voff[kNkc];
        {
            const int r = 8 * (n >> 2) + (n & 3);
            const int q = 8 * g + (n >> 2);
            const int vr = wave * 32 + n;
#pragma unroll
            for (int kc = 0; kc < kNkc; ++kc) {
                rowoff[kc] = (uint32_t)(r * kD + ((4 * kc + g) ^ tile_swz<D>(r)) * 8) * 2u;
                voff[kc] = (uint32_t)(vr * kD + ((4 * kc + g) ^ vblk_swz<D>(vr)) * 8) * 2u;
                asm volatile("" : "+v"(rowoff[kc]));
                asm volatile("" : "+v"(voff[kc]));
            }
#pragma unroll
            for (int db = 0; db < kNdb; ++db) {
                const int col = 16 * db + 4 * (n & 3);
                troff[db] = (uint32_t)(q * kD + ((col >> 3) ^ tile_swz<D>(q)) * 8 + (col & 7)) * 2u;
                asm volatile("" : "+v"(troff[db]));
            }
        }
        auto a_row = [&](const uint16_t* tile, int qb, int kc) __attribute__((always_inline)) {
            return *(LDS16B const V8*)((LDS16B const char*)(LDS16B const uint16_t*)tile + rowoff[kc] + qb * kRow4);
        };
        auto a_tr = [&](const uint16_t* tile, int db) __attribute__((always_inline)) {
            const V4 p0 = E::tr_read((LDS16B V4*)((LDS16B char*)(LDS16B uint16_t*)tile + troff[db]));
            const V4 p1 = E::tr_read((LDS16B V4*)((LDS16B char*)(LDS16B uint16_t*)tile + troff[db] + kRow4));
            return V8{p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
        };
        auto b_v = [&](int kb2, int kc) __attribute__((always_inline)) {
            return *(LDS16B const V8*)((LDS16B const char*)(LDS16B const uint16_t*)v_blk + voff[kc] + kb2 * 16 * kD * 2);
        };

        // dK^T and dV^T: acc[db][kb2], lane (n, g) holds d = 16db + 4g .. +3 of key 16kb2 + n.
        f32x4_t adk[kNdb][2], adv[kNdb][2];
#pragma unroll
        for (int db = 0; db < kNdb; ++db)
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2) {
                adk[db][kb2] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                adv[db][kb2] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }

        const int nqt = (Nq + kQT - 1) / kQT;
        // Causal: key j is seen by queries i >= j - off only, so tiles start at
        // the block's (the wave's) first such query. Keys at or past Lk are
        // padding: a block (a wave) made of them runs no tile and stores zeros.
        auto first_tile = [&](int key0) __attribute__((always_inline)) {
            if (key0 >= Lk) return nqt;
            return CAUSAL ? min(nqt, max(0, key0 - doff) / kQT) : 0;
        };
        const int first = first_tile(k0);
        const int my_first = first_tile(kw0);

        // L and D of tile u through registers of wave 0 (lanes 0-31: L, 32-63:
        // D), loaded with the tile's DMA and written to LDS (L scaled to base 2)
        // after the next tile's compute.
        float ld_reg = 0.f;
        auto fetch_ld = [&](int u) __attribute__((always_inline)) {
            if (wave == 0) {
                const int q = min(u * kQT + (lane & 31), Nq - 1);
                ld_reg = lane < 32 ? L[q] : Dv[q];
            }
        };
        auto put_ld = [&](int buf) __attribute__((always_inline)) {
            if (wave == 0) ld_lds[buf][lane] = lane < 32 ? ld_reg * kLog2e : ld_reg;
        };
        Stage16<D, kQT, false> slots;                 // Q and dO tiles share the offsets
        slots.init(wave, lane);
        auto stage = [&](int u, uint16_t* qd, uint16_t* od) __attribute__((always_inline)) {
            const int q0 = u * kQT;                // < Nq
            const int valid = min(Nq - q0, kQT);
            slots.stage(Q + (size_t)q0 * kD, valid, qd, wave);
            slots.stage(dO + (size_t)q0 * kD, valid, od, wave);
        };

        // One tile in phases with their own live registers (sched_barrier
        // between them): S = Q K^T, P, dV^T += dO^T P, dP = dO V^T, dS,
        // dK^T += Q^T dS.
        auto compute = [&](int u, const uint16_t* qt, const uint16_t* ot, int buf) __attribute__((always_inline)) {
            constexpr int LEAD = 2;                // operand prefetch depth (register budget: 256 VGPRs)
            const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
            // S: s[qb][kb2], lane (n, g): queries 8g + 4qb + e (e = 0..3) of the tile, key 16kb2 + n.
            f32x4_t s[2][2];
            op_stream<2 * kNkc, LEAD>([&](int i) { return a_row(qt, i & 1, i >> 1); },
                                        [&](int i, V8 a) {
                                            const int qb = i & 1, kc = i >> 1;
#pragma unroll
                                            for (int kb2 = 0; kb2 < 2; ++kb2)
                                                s[qb][kb2] = E::mfma16(a, kf[kb2][kc], kc == 0 ? zero : s[qb][kb2]);
                                        });
            const int q0 = u * kQT;
            const bool edge = q0 + kQT > Nq || kw0 + 32 > Lk || (CAUSAL && q0 + doff < kw0 + 31);
            // P in place (fp32, kept for dS), then the mask of an edge tile in one branch.
            const f32x4_t la = *(const f32x4_t*)&ld_lds[buf][8 * g];
            const f32x4_t lb = *(const f32x4_t*)&ld_lds[buf][8 * g + 4];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        s[qb][kb2][e] = exp2_hw(__builtin_fmaf(s[qb][kb2][e], scale2, -(qb ? lb[e] : la[e])));
            if (edge) {
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int q = q0 + 8 * g + 4 * qb + e;
                            const int key = kw0 + 16 * kb2 + n;
                            if (q >= Nq || key >= Lk || (CAUSAL && q + doff < key)) s[qb][kb2][e] = 0.f;
                        }
            }
            // P^T of the 32-query step, B operand of dV^T += dO^T P: queries 8g .. 8g+7 of key 16kb2 + n.
            V8 pf[2];
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2) {
                u32x4_t w;
                w[0] = E::pack2(s[0][kb2][0], s[0][kb2][1]);
                w[1] = E::pack2(s[0][kb2][2], s[0][kb2][3]);
                w[2] = E::pack2(s[1][kb2][0], s[1][kb2][1]);
                w[3] = E::pack2(s[1][kb2][2], s[1][kb2][3]);
                pf[kb2] = __builtin_bit_cast(V8, w);
            }
            __builtin_amdgcn_sched_barrier(0);
            op_stream<kNdb, LEAD>([&](int db) { return a_tr(ot, db); },
                                    [&](int db, V8 a) {
#pragma unroll
                                        for (int kb2 = 0; kb2 < 2; ++kb2)
                                            adv[db][kb2] = E::mfma16(a, pf[kb2], adv[db][kb2]);
                                    });
            // dP: both operands from LDS (the dO tile and the block's V rows),
            // the two A and the two B operands of a d step read one step ahead.
            f32x4_t dp[2][2];
            struct Ops { V8 a[2], b[2]; };
            op_stream<kNkc, 1>([&](int kc) {
                                     Ops o;
                                     o.a[0] = a_row(ot, 0, kc);
                                     o.a[1] = a_row(ot, 1, kc);
                                     o.b[0] = b_v(0, kc);
                                     o.b[1] = b_v(1, kc);
                                     return o;
                                 },
                                 [&](int kc, const Ops& o) {
#pragma unroll
                                     for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                                         for (int kb2 = 0; kb2 < 2; ++kb2)
                                             dp[qb][kb2] = E::mfma16(o.a[qb], o.b[kb2], kc == 0 ? zero : dp[qb][kb2]);
                                 });
            // dS = P (dP - D), packed like P.
            const f32x4_t da = *(const f32x4_t*)&ld_lds[buf][kQT + 8 * g];
            const f32x4_t dbv = *(const f32x4_t*)&ld_lds[buf][kQT + 8 * g + 4];
            V8 dsf[2];
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2) {
                float ds[2][4];
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) ds[qb][e] = s[qb][kb2][e] * (dp[qb][kb2][e] - (qb ? dbv[e] : da[e]));
                u32x4_t x;
                x[0] = E::pack2(ds[0][0], ds[0][1]);
                x[1] = E::pack2(ds[0][2], ds[0][3]);
                x[2] = E::pack2(ds[1][0], ds[1][1]);
                x[3] = E::pack2(ds[1][2], ds[1][3]);
                dsf[kb2] = __builtin_bit_cast(V8, x);
            }
            __builtin_amdgcn_sched_barrier(0);
            op_stream<kNdb, LEAD>([&](int db) { return a_tr(qt, db); },
                                    [&](int db, V8 a) {
#pragma unroll
                                        for (int kb2 = 0; kb2 < 2; ++kb2)
                                            adk[db][kb2] = E::mfma16(a, dsf[kb2], adk[db][kb2]);
                                    });
        };

        // Prologue: the block's V rows (zeros past Lk) and the first tile.
        {
            Stage16<D, BM_BWD, true> vslots;
            vslots.init(wave, lane);
            vslots.stage(Vg + ((size_t)bh * Nk + k0) * kD, max(0, min(Lk - k0, BM_BWD)), v_blk, wave);
        }
        if (first < nqt) {
            stage(first, q_lds0, o_lds0);
            fetch_ld(first);
            put_ld(0);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        // Tile first + 2i in buffer 0, first + 2i + 1 in buffer 1.
        for (int u = first; u < nqt; u += 2) {
            // Alternating priorities by tile pair and block parity (workgroups share a CU).
            if ((((u - first) >> 1) + blockIdx.x) & 1) __builtin_amdgcn_s_setprio(1);
            else __builtin_amdgcn_s_setprio(0);
            if (u + 1 < nqt) {
                stage(u + 1, q_lds1, o_lds1);
                fetch_ld(u + 1);
            }
            if (u >= my_first) compute(u, q_lds0, o_lds0, 0);
            if (u + 1 < nqt) put_ld(1);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (u + 1 >= nqt) break;
            if (u + 2 < nqt) {
                stage(u + 2, q_lds0, o_lds0);
                fetch_ld(u + 2);
            }
            if (u + 1 >= my_first) compute(u + 1, q_lds1, o_lds1, 1);
            if (u + 2 < nqt) put_ld(0);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        }

        // The last barrier above ended every read of the Q / dO tiles and of the
        // V block: each wave stages its dK rows in one tile buffer and its dV rows
        // in its own quarter of the V block. Rows past Nk are not stored.
        uint16_t* const kst = wave == 0 ? q_lds0 : wave == 1 ? q_lds1 : wave == 2 ? o_lds0 : o_lds1;
        store_rows16<T, D>(dKg + ((size_t)bh * Nk + kw0) * kD, Nk - kw0, adk, scale, kst, lane);
        store_rows16<T, D>(dVg + ((size_t)bh * Nk + kw0) * kD, Nk - kw0, adv, 1.0f, v_blk + wave * 32 * kD, lane);

        // The next block's loads reuse the LDS buffers.
        if constexpr (PERSIST) __syncthreads();
    }
}

// dQ (and D) for 128 query rows of one (batch, head): 4 waves x 32 queries,
// two or more workgroups per CU, K and V streamed through LDS in 32-key tiles
// (double-buffered, one barrier per tile), with the dK/dV kernel's 16x16x32
// layouts on the query side. A wave's 32 queries are two column blocks qb of
// 16 (Q and dO in registers as B operands); a tile is two row blocks kb of 16
// keys whose A rows are permuted (row m of block kb reads key 8(m/4) + 4kb +
// m%4), so the lane ends with keys 8g + 4kb + 0..3 of its query and dS^T packs
// straight into the B operand of dQ^T += K^T dS^T, whose K^T operand is two
// transpose reads of the same tile.
template <typename T, int D, bool PERSIST>
__global__ __launch_bounds__(kKvThreads, 2)
void bwd_dq16_kernel(const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg,
                     const uint16_t* __restrict__ Vg, const uint16_t* __restrict__ Og,
                     const uint16_t* __restrict__ dOg, const float* __restrict__ LSEg, float* __restrict__ Dg,
                     uint16_t* __restrict__ dQg, const int* __restrict__ kv_lens, int H, int Nq, int Nk,
                     int nqb, float scale, float scale2, int causal, int n_bh) {
    using E = Elem<T>;
    using V8 = typename E::v8;
    using V4 = typename E::v4;
    constexpr int kD = D, kNkc = Dims<D>::NKC, kNdb = Dims<D>::NDB, kQTile = Dims<D>::TILE, kRow4 = Dims<D>::ROW4;
    constexpr int LEAD = 4;                    // operand prefetch depth of the product streams
    const bool CAUSAL = causal != kCausalNone;

    __shared__ __attribute__((aligned(1024))) uint16_t k_lds0[kQTile];
    __shared__ __attribute__((aligned(1024))) uint16_t k_lds1[kQTile];
    __shared__ __attribute__((aligned(1024))) uint16_t v_lds0[kQTile];
    __shared__ __attribute__((aligned(1024))) uint16_t v_lds1[kQTile];

    // One query block per workgroup or, in a persistent launch, the paired
    // static schedule (blocks nqb - 1 - r and r of a head at equal cost,
    // contiguous pair ranges per XCD, taken in turn).
    const int npair = (nqb + 1) / 2;
    const int xcd = blockIdx.x & 7;
    const int per_xcd = gridDim.x >> 3;
    const long long all_pairs = (long long)n_bh * npair;
    const int p_lo = (int)(all_pairs * xcd / 8), p_hi = (int)(all_pairs * (xcd + 1) / 8);
    for (int wi = 0;; ++wi) {
        int bh, qb0;
        if constexpr (!PERSIST) {
            if (wi > 0) break;
            const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
            bh = logical / nqb;
            qb0 = logical - bh * nqb;
            if (CAUSAL) qb0 = nqb - 1 - qb0;   // longest rows first
        } else {
            const int p = p_lo + (int)(blockIdx.x >> 3) + (wi >> 1) * per_xcd;
            if (p >= p_hi) break;
            bh = p / npair;
            const int r = p - bh * npair;
            qb0 = (wi & 1) ? r : nqb - 1 - r;
            if ((wi & 1) && r == nqb - 1 - r) continue;   // odd count: the middle block is alone
        }
        int tid = threadIdx.x;
        if constexpr (PERSIST) asm volatile("" : "+v"(tid));
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int lane = tid & 63;
        const int n = lane & 15;
        const int g = lane >> 4;
        const int q0 = qb0 * BM_BWD;
        const int wrow0 = q0 + wave * 32;

        const uint16_t* K = Kg + (size_t)bh * Nk * kD;
        const uint16_t* V = Vg + (size_t)bh * Nk * kD;
        const int Lk = real_keys(kv_lens, bh / H, Nk);
        const int doff = causal == kCausalBottomRight ? Lk - Nq : 0;   // key j visible from query i iff j <= i + doff

        // Q and dO of the wave's queries as B operands: query wrow0 + 16qb + n,
        // d = 32kc + 8g .. +7 (zero past Nq); D = rowsum(dO * O) of those
        // queries from the O rows read the same way, over the four lane groups,
        // written for the dK/dV kernel.
        V8 qf[2][kNkc], dof[2][kNkc];
        float l2[2], dr[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int q = wrow0 + 16 * qb + n;
            const bool qv = q < Nq;
            const size_t rowb = ((size_t)bh * Nq + min(q, Nq - 1)) * kD;
            float a2[2] = {0.f, 0.f};
#pragma unroll
            for (int kc = 0; kc < kNkc; ++kc) {
                u32x4_t wq = *(const u32x4_t*)(Qg + rowb + kc * 32 + g * 8);
                u32x4_t wd = *(const u32x4_t*)(dOg + rowb + kc * 32 + g * 8);
                const u32x4_t wo = *(const u32x4_t*)(Og + rowb + kc * 32 + g * 8);
                if (!qv) wq = wd = u32x4_t{0u, 0u, 0u, 0u};
                qf[qb][kc] = __builtin_bit_cast(V8, wq);
                dof[qb][kc] = __builtin_bit_cast(V8, wd);
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    a2[w & 1] = __builtin_fmaf(E::lo(wo[w]), E::lo(wd[w]), a2[w & 1]);
                    a2[w & 1] = __builtin_fmaf(E::hi(wo[w]), E::hi(wd[w]), a2[w & 1]);
                }
            }
            dr[qb] = sum_xor32(sum_xor16(a2[0] + a2[1]));
            if (qv && g == 0) Dg[(size_t)bh * Nq + q] = dr[qb];
            l2[qb] = qv ? LSEg[(size_t)bh * Nq + q] * kLog2e : 0.f;
        }

        // Lane byte offsets of the LDS operand reads (tile bases fold into the
        // instruction's offset field): rowoff[kc], tile row 8(n/4) + n%4, chunk
        // 4kc + g (row block 1: +4 rows); troff[db], tile row 8g + n/4, columns
        // 16db + 4(n%4) .. +3 (second transpose read: +4 rows).
        uint32_t rowoff[kNkc], troff[kNdb];
        {
            const int r = 8 * (n >> 2) + (n & 3);
            const int q = 8 * g + (n >> 2);
#pragma unroll
            for (int kc = 0; kc < kNkc; ++kc) {
                rowoff[kc] = (uint32_t)(r * kD + ((4 * kc + g) ^ tile_swz<D>(r)) * 8) * 2u;
                asm volatile("" : "+v"(rowoff[kc]));
            }
#pragma unroll
            for (int db = 0; db < kNdb; ++db) {
                const int col = 16 * db + 4 * (n & 3);
                troff[db] = (uint32_t)(q * kD + ((col >> 3) ^ tile_swz<D>(q)) * 8 + (col & 7)) * 2u;
                asm volatile("" : "+v"(troff[db]));
            }
        }
        auto a_row = [&](const uint16_t* tile, int kb, int kc) __attribute__((always_inline)) {
            return *(LDS16B const V8*)((LDS16B const char*)(LDS16B const uint16_t*)tile + rowoff[kc] + kb * kRow4);
        };
        auto a_tr = [&](const uint16_t* tile, int db) __attribute__((always_inline)) {
            const V4 p0 = E::tr_read((LDS16B V4*)((LDS16B char*)(LDS16B uint16_t*)tile + troff[db]));
            const V4 p1 = E::tr_read((LDS16B V4*)((LDS16B char*)(LDS16B uint16_t*)tile + troff[db] + kRow4));
            return V8{p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
        };

        // dQ^T: acc[db][qb], lane (n, g) holds d = 16db + 4g .. +3 of query 16qb + n.
        f32x4_t acc[kNdb][2];
#pragma unroll
        for (int db = 0; db < kNdb; ++db)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) acc[db][qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        int kend = Lk;
        if (CAUSAL) kend = max(0, min(Lk, min(q0 + BM_BWD, Nq) + doff));
        const int ntiles = (kend + kQT - 1) / kQT;
        const int wlast = wrow0 + 31 + doff;        // last key the wave's last row may see
        const int my_tiles = CAUSAL ? (wlast < 0 ? 0 : min(ntiles, wlast / kQT + 1)) : ntiles;

        Stage16<D, kQT, false> slots;                 // K and V tiles share the offsets
        slots.init(wave, lane);
        auto stage = [&](int t, uint16_t* kd, uint16_t* vd) __attribute__((always_inline)) {
            const int kv0 = t * kQT;               // < kend <= Lk
            const int valid = min(Lk - kv0, kQT);
            slots.stage(K + (size_t)kv0 * kD, valid, kd, wave);
            slots.stage(V + (size_t)kv0 * kD, valid, vd, wave);
        };
        auto compute = [&](int t, const uint16_t* kt, const uint16_t* vt) __attribute__((always_inline)) {
            const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
            // S^T = K Q^T and dP^T = V dO^T: s[kb][qb], lane (n, g) holds keys
            // 8g + 4kb + 0..3 of the tile for query 16qb + n; the operands K kb 0,
            // K kb 1, V kb 0, V kb 1 of each d step in one stream.
            f32x4_t s[2][2], dp[2][2];
            op_stream<4 * kNkc, LEAD>([&](int k) { return a_row((k & 2) ? vt : kt, k & 1, k >> 2); },
                                      [&](int k, V8 a) {
                                          const int kb = k & 1, kc = k >> 2;
                                          if (k & 2) {
#pragma unroll
                                              for (int qb = 0; qb < 2; ++qb)
                                                  dp[kb][qb] = E::mfma16(a, dof[qb][kc], kc == 0 ? zero : dp[kb][qb]);
                                          } else {
#pragma unroll
                                              for (int qb = 0; qb < 2; ++qb)
                                                  s[kb][qb] = E::mfma16(a, qf[qb][kc], kc == 0 ? zero : s[kb][qb]);
                                          }
                                      });
            const int kv0 = t * kQT;
            const bool edge = kv0 + kQT > Lk || (CAUSAL && kv0 + kQT - 1 > wrow0 + doff);
            // P in place, then the mask of an edge tile in one branch.
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        s[kb][qb][e] = exp2_hw(__builtin_fmaf(s[kb][qb][e], scale2, -l2[qb]));
            if (edge) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int key = kv0 + 8 * g + 4 * kb + e;
                            const int q = wrow0 + 16 * qb + n;
                            if (key >= Lk || (CAUSAL && key > q + doff)) s[kb][qb][e] = 0.f;
                        }
            }
            // dS^T as B operands: keys 8g .. 8g+7 of query 16qb + n.
            V8 dsf[2];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                float ds[2][4];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) ds[kb][e] = s[kb][qb][e] * (dp[kb][qb][e] - dr[qb]);
                u32x4_t w;
                w[0] = E::pack2(ds[0][0], ds[0][1]);
                w[1] = E::pack2(ds[0][2], ds[0][3]);
                w[2] = E::pack2(ds[1][0], ds[1][1]);
                w[3] = E::pack2(ds[1][2], ds[1][3]);
                dsf[qb] = __builtin_bit_cast(V8, w);
            }
            __builtin_amdgcn_sched_barrier(0);
            // dQ^T += K^T dS^T.
            op_stream<kNdb, LEAD>([&](int db) { return a_tr(kt, db); },
                                  [&](int db, V8 a) {
#pragma unroll
                                      for (int qb = 0; qb < 2; ++qb) acc[db][qb] = E::mfma16(a, dsf[qb], acc[db][qb]);
                                  });
        };

        if (ntiles > 0) stage(0, k_lds0, v_lds0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        // Tile t in buffer t % 2; the next tile is loaded while t is computed and
        // published by the barrier that ends the iteration.
        for (int t = 0; t < ntiles; t += 2) {
            // Workgroups share a CU. Left alone, one of them takes most of the
            // issue slots; priorities that alternate by tile pair and block
            // parity even them out.
            if (((t >> 1) + blockIdx.x) & 1) __builtin_amdgcn_s_setprio(1);
            else __builtin_amdgcn_s_setprio(0);
            if (t + 1 < ntiles) stage(t + 1, k_lds1, v_lds1);
            if (t < my_tiles) compute(t, k_lds0, v_lds0);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (t + 1 >= ntiles) break;
            if (t + 2 < ntiles) stage(t + 2, k_lds0, v_lds0);
            if (t + 1 < my_tiles) compute(t + 1, k_lds1, v_lds1);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        }

        // The last barrier above ended every read of the tile buffers: each wave
        // stages its dQ rows in one of them.
        uint16_t* const qst = wave == 0 ? k_lds0 : wave == 1 ? k_lds1 : wave == 2 ? v_lds0 : v_lds1;
        store_rows16<T, D>(dQg + ((size_t)bh * Nq + wrow0) * kD, Nq - wrow0, acc, scale, qst, lane);

        // The next block's loads reuse the LDS buffers.
        if constexpr (PERSIST) __syncthreads();
    }
}

template <typename T, int D>
static hipError_t launch_dkdv16_t(const BwdArgs& a, float scale2, bool paired) {
    const int n_bh = a.B * a.H;
    const int nkb = (a.Nk + BM_BWD - 1) / BM_BWD;
    int grid = 0;
    if (paired) {
        int cus = 0, per_cu = 0;
        hipError_t e = device_cu_count(&cus);
        if (e != hipSuccess) return e;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(bwd_dkdv16_kernel<T, D, true>), kKvThreads, 0);
        if (e != hipSuccess) return e;
        grid = paired_schedule_grid(cus * per_cu, n_bh, nkb);
    }
    const bool persist = grid > 0;
    if (!persist) grid = n_bh * nkb;
    auto kern = persist ? bwd_dkdv16_kernel<T, D, true> : bwd_dkdv16_kernel<T, D, false>;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kKvThreads), 0, a.stream,
                       (const uint16_t*)a.Q, (const uint16_t*)a.K, (const uint16_t*)a.V,
                       (const uint16_t*)a.dO, a.LSE, a.Dvec, (uint16_t*)a.dK, (uint16_t*)a.dV, a.kv_lens,
                       a.H, a.Nq, a.Nk, nkb, a.scale, scale2, a.causal, n_bh);
    return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_dq16_t(const BwdArgs& a, float scale2, bool paired) {
    const int n_bh = a.B * a.H;
    const int nqb = (a.Nq + BM_BWD - 1) / BM_BWD;
    int grid = 0;
    if (paired) {
        int cus = 0, per_cu = 0;
        hipError_t e = device_cu_count(&cus);
        if (e != hipSuccess) return e;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(bwd_dq16_kernel<T, D, true>), kKvThreads, 0);
        if (e != hipSuccess) return e;
        grid = paired_schedule_grid(cus * per_cu, n_bh, nqb);
    }
    const bool persist = grid > 0;
    if (!persist) grid = n_bh * nqb;
    auto kern = persist ? bwd_dq16_kernel<T, D, true> : bwd_dq16_kernel<T, D, false>;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kKvThreads), 0, a.stream,
                       (const uint16_t*)a.Q, (const uint16_t*)a.K, (const uint16_t*)a.V, (const uint16_t*)a.O,
                       (const uint16_t*)a.dO, a.LSE, a.Dvec, (uint16_t*)a.dQ, a.kv_lens, a.H, a.Nq, a.Nk, nqb,
                       a.scale, scale2, a.causal, n_bh);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_bwd_d(const BwdArgs& a, float scale2, bool paired) {
    if (a.Nq > 0) {
        const hipError_t e = a.f16 ? launch_dq16_t<_Float16, D>(a, scale2, paired) : launch_dq16_t<__bf16, D>(a, scale2, paired);
        if (e != hipSuccess) return e;
    }
    // With Nq = 0 the dK/dV kernel stages only V, runs no query tile and
    // stores zeros.
    return a.f16 ? launch_dkdv16_t<_Float16, D>(a, scale2, paired) : launch_dkdv16_t<__bf16, D>(a, scale2, paired);
}

hipError_t launch_bwd(const BwdArgs& a) {
    const float scale2 = a.scale * kLog2e;
    // Persistent launches for causal self-attention (Nq = Nk, no key padding),
    // where a block's cost is linear in its index, so that paired blocks cost
    // the same.
    const bool paired = a.causal != kCausalNone && !a.kv_lens && a.Nq == a.Nk;
    return a.D == 64 ? launch_bwd_d<64>(a, scale2, paired) : launch_bwd_d<128>(a, scale2, paired);
}

}  // namespace fa
