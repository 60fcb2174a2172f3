// Backward pass with recompute for gfx950 ("Backward with recompute" exercise
// and section 11.9 of the ML compiler page: only O and the per-row
// log-sum-exp L are kept from the forward pass; P is recomputed block by block
// as exp(S - L)). For one (batch, head):
//     D_i = sum_d dO[i,d] O[i,d]                       (bwd_dq_kernel, stored)
//     P = exp(scale Q K^T - L),  dP = dO V^T,  dS = P * (dP - D)
//     dQ = scale dS K                                  (bwd_dq_kernel)
//     dV = P^T dO,  dK = scale dS^T Q                  (bwd_dkdv_kernel)
// Exponentials are base 2 (scale and L multiplied by log2 e).
//
// This file holds the D = 64 kernels; D = 128 runs on the 16x16x32 MFMA in
// fa_bwd16.hip, with the same structure and its own operand layouts.
//
// gfx950 mapping (own design, on the forward kernel's MFMA layouts):
//   * bf16 or fp16 inputs (Elem<T>: MFMA, transpose read, packing).
//   * Both product kernels use v_mfma_f32_32x32x16_bf16 (_f16) with 4 waves x 32
//     rows per workgroup and stream the other operand through LDS in tiles of
//     32 rows (buffer_load_dwordx4 straight to LDS, double-buffered, one
//     barrier per tile).
//   * dQ: a wave owns 32 query rows; Q and dO stay in VGPRs as B operands.
//     S^T = K Q^T and dP^T = V dO^T put one query per lane, so L and D are
//     per-lane scalars. The rows of K and V fed to the A operand are permuted
//     (bits 2 and 3 of the row swapped) so the accumulator of dS^T, rounded to
//     bf16, is directly the B operand of dQ^T += K^T dS^T; K^T is read from
//     the same LDS tile with ds_read_b64_tr_b16.
//   * dK, dV: a wave owns 32 keys; K stays in VGPRs and the workgroup's 128
//     V rows in LDS (both as B operands). S = Q K^T and dP = dO V^T put one
//     key per lane (L and D, per query, come from LDS); P and dS, rounded to
//     bf16, are the B operands of dV^T += dO^T P and dK^T += Q^T dS, whose A
//     operands are transpose reads of the Q and dO tiles.
//   * Every tile is read both row-wise (16-byte MFMA operand rows) and
//     transposed (8-byte transpose reads of 4 consecutive rows). One XOR
//     swizzle of the 16-byte chunks makes both patterns free of LDS bank
//     conflicts, so each tile is staged once.
//   * Masking: causal (key j visible from query i iff j <= i + off, off = 0
//     top-left or Lk - Nq bottom-right), padding keys (past the batch entry's
//     real key count Lk) and queries past Nq get P = 0 (so dS = 0 too); rows
//     past the end are staged as zeros and never stored. A
//     query row with no visible key (LSE = -inf) only ever meets masked pairs,
//     so its P is forced to 0 before exp2(+inf) can be used; its dQ is 0.
//   * dQ, dK, dV are accumulated in fp32 and rounded to bf16 once.

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kBwdWaves = 4;
constexpr int kBwdThreads = 64 * kBwdWaves;
constexpr int kBT = 32;                    // rows per streamed tile
static_assert(BM_BWD == 32 * kBwdWaves, "32 rows per wave");

#define LDS_AS __attribute__((address_space(3)))


// Lane-row i of an MFMA A operand reads tile row perm(i) (bits 2 and 3
// swapped): accumulator register r of lane (j, h) then holds row
// 16*(r/8) + 8*h + (r%8), 8 consecutive rows per lane half.
__device__ __forceinline__ int row_perm(int i) {
    return (i & ~0xC) | ((i & 4) << 1) | ((i & 8) >> 1);
}

// 16-byte chunk swizzle of a row of CPR chunks, conflict-free both for 16
// lanes reading 16 different rows at one chunk and for transpose reads of 4
// consecutive rows x 4 chunks (checked bank by bank on the host).
template <int CPR>
__device__ __forceinline__ int swz(int row) {
    return CPR == 16 ? (((row & 3) << 2) | ((row >> 2) & 3))
                     : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}

__device__ __forceinline__ void lds_dma_wait_all() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Staging of ROWS rows of a row-major [*, D] 16-bit array into LDS with the
// chunk swizzle: chunk p of the tile lands at byte 16*p and holds logical
// chunk (p % CPR) ^ swz(row) of row p / CPR. Wave w moves chunks
// (w*PER + i)*64 + lane, i < PER, with buffer loads straight to LDS; the
// per-lane offsets are computed once, and a tile's resource spans only its
// valid rows, so rows past them arrive as zeros (always masked).
template <int D, int ROWS>
struct StageSlots {
    static constexpr int CPR = D / 8;
    static constexpr int PER = ROWS * CPR / kBwdThreads;   // chunks per lane
    static_assert(PER * kBwdThreads == ROWS * CPR, "whole chunks per lane");
    uint32_t voff[PER];        // memory byte offsets, net of the slot's immediate offset
    __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int p = (wave * PER + i) * 64 + lane;
            const int row = p / CPR;
            voff[i] = (uint32_t)(row * D + ((p % CPR) ^ swz<CPR>(row)) * 8) * 2u - (i % 4) * 1024u;
        }
    }
    // Rows [valid, ROWS) of src (0 <= valid <= ROWS) are not read.
    __device__ __forceinline__ void stage(const uint16_t* src, int valid, uint16_t* dst, int wave) const {
        const __amdgpu_buffer_rsrc_t rsrc =
            __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, valid * D * 2, kBufferRsrcWord3);
        static_assert(PER <= 4 || PER % 4 == 0, "slots go in groups of up to 4");
        if constexpr (PER <= 4) {
            buffer_lds_slots<PER>(rsrc, (LDS_AS void*)(LDS_AS uint16_t*)(dst + wave * PER * 512), voff);
        } else {
#pragma unroll
            for (int g = 0; g < PER; g += 4)
                buffer_lds_slots<4>(rsrc, (LDS_AS void*)(LDS_AS uint16_t*)(dst + (wave * PER + g) * 512), voff + g);
        }
    }
};

// Lane-dependent LDS byte offsets of the MFMA operand reads of a staged
// 32-row tile. They are the same for every tile buffer (the buffer's base is
// a compile-time constant that folds into the instruction's offset field),
// computed once and pinned in VGPRs.
//   row[kk]: A operand rows, lane (j, h) reads row row_perm(j), elements
//            16*kk + 8*h .. +7.
//   tr[2*db + rd]: A operand transposed, element (i, k) = tile[16*tt + k]
//            [32*db + i], two transpose reads rd = 0, 1 (rows 16*tt + 8*h +
//            4*rd + s/4 for source lane s of each 16-lane block, 4 columns
//            from 32*db + 16*(lane/16 % 2) + 4*(s%4)); add 16*tt rows.
template <int D>
struct TileOffsets {
    uint32_t row[D / 16];
    uint32_t tr[2 * (D / 32)];
    __device__ __forceinline__ void init(int lane) {
        constexpr int CPR = D / 8;
        const int j = lane & 31, h = lane >> 5, blk = (lane >> 4) & 1, v_s = lane & 15;
        const int r = row_perm(j);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            row[kk] = (uint32_t)(r * D + ((kk * 2 + h) ^ swz<CPR>(r)) * 8) * 2u;
            asm volatile("" : "+v"(row[kk]));
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int rd = 0; rd < 2; ++rd) {
                const int rr = h * 8 + rd * 4 + (v_s >> 2);
                const int col = db * 32 + blk * 16 + (v_s & 3) * 4;
                tr[db * 2 + rd] = (uint32_t)(rr * D + ((col >> 3) ^ swz<CPR>(rr)) * 8 + (col & 7)) * 2u;
                asm volatile("" : "+v"(tr[db * 2 + rd]));
            }
    }
};

template <typename T, int D>
__device__ __forceinline__ typename Elem<T>::v8 row_operand(const uint16_t* tile, const TileOffsets<D>& o, int kk) {
    using V8 = typename Elem<T>::v8;
    return *(LDS_AS const V8*)((LDS_AS const char*)(LDS_AS const uint16_t*)tile + o.row[kk]);
}

template <typename T, int D>
__device__ __forceinline__ typename Elem<T>::v8 tr_operand(const uint16_t* tile, const TileOffsets<D>& o, int tt, int db) {
    using V4 = typename Elem<T>::v4;
    using V8 = typename Elem<T>::v8;
    V4 part[2];
#pragma unroll
    for (int rd = 0; rd < 2; ++rd)
        part[rd] = Elem<T>::tr_read(
            (LDS_AS V4*)((LDS_AS char*)(LDS_AS uint16_t*)tile + o.tr[db * 2 + rd] + (uint32_t)(tt * 16 * D * 2)));
    return V8{part[0][0], part[0][1], part[0][2], part[0][3],
                    part[1][0], part[1][1], part[1][2], part[1][3]};
}

// Row `row` of a [*, D] array as MFMA B operands: lane (j, h) holds elements
// 16*kk + 8*h .. +7 (zero when the row is past the end).
template <typename T, int D>
__device__ __forceinline__ void load_b_rows(const uint16_t* base, int row, bool valid, int h,
                                            typename Elem<T>::v8* out) {
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
        u32x4_t w = {0u, 0u, 0u, 0u};
        if (valid) w = *(const u32x4_t*)(base + (size_t)row * D + kk * 16 + h * 8);
        out[kk] = __builtin_bit_cast(typename Elem<T>::v8, w);
    }
}

// Store an fp32 accumulator of 32 rows x D held transposed (lane j = row,
// register r of block db = column 32*db + 8*(r/4) + 4*h + r%4) as 16-bit
// values multiplied by `mul`, to rows dst[0 .. valid) (row-major [*, D]).
// The rows go through `stage`, 32*D elements of LDS private to the wave, with
// their 16-byte chunks swizzled by row, so that every store instruction
// writes whole rows, 16 bytes per lane.
template <typename T, int D>
__device__ __forceinline__ void store_rows_staged(uint16_t* dst, int valid, const f32x16_t* acc, float mul,
                                                  uint16_t* stage, int lane) {
    constexpr int CPR = D / 8;
    const int j = lane & 31, h = lane >> 5;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
            const int c = db * 4 + a4;         // 16-byte chunk: columns 8c .. 8c + 7
            u32x2_t w;
            w[0] = Elem<T>::pack2(acc[db][a4 * 4 + 0] * mul, acc[db][a4 * 4 + 1] * mul);
            w[1] = Elem<T>::pack2(acc[db][a4 * 4 + 2] * mul, acc[db][a4 * 4 + 3] * mul);
            *(LDS_AS u32x2_t*)(LDS_AS uint16_t*)(stage + j * D + (c ^ (j & (CPR - 1))) * 8 + h * 4) = w;
        }
    // The reads take other lanes' writes: one wave's LDS operations complete
    // in order once issued, and the fence keeps the compiler from moving the
    // reads ahead.
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    constexpr int RPI = 64 / CPR;              // rows per store instruction
    constexpr int NIT = 32 / RPI;
    const int c = lane % CPR;
    u32x4_t w[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int r = it * RPI + lane / CPR;
        w[it] = *(LDS_AS const u32x4_t*)(LDS_AS const uint16_t*)(stage + r * D + (c ^ (r & (CPR - 1))) * 8);
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int r = it * RPI + lane / CPR;
        if (r < valid) *(u32x4_t*)(dst + (size_t)r * D + c * 8) = w[it];
    }
}

// The two LDS operands of one MFMA, prefetched together.
template <typename V>
struct OperandPair {
    V a, b;
};

// N MFMAs acc[dst(i)] += op(i) x b(i), each A operand read LEAD MFMAs ahead
// and no further (sched_barrier after every step), which bounds the operand
// registers a phase holds.
template <int N, int LEAD, typename Op, typename Step>
__device__ __forceinline__ void mfma_stream(Op op, Step step) {
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

// dQ for 128 query rows of one (batch, head), streaming K and V tiles; also
// D of those rows, which the dK/dV kernel reads.
template <typename T, int D, bool PERSIST>
__global__ __launch_bounds__(kBwdThreads, 2)
void bwd_dq_kernel(const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg,
                   const uint16_t* __restrict__ Vg, const uint16_t* __restrict__ Og,
                   const uint16_t* __restrict__ dOg, const float* __restrict__ LSEg, float* __restrict__ Dg,
                   uint16_t* __restrict__ dQg, const int* __restrict__ kv_lens, int H, int Nq, int Nk,
                   int nqb, float scale, float scale2, int causal, int n_bh) {
    using V8 = typename Elem<T>::v8;
    constexpr int NKK = D / 16, NDB = D / 32;
    constexpr int TILE = kBT * D;
    const bool CAUSAL = causal != kCausalNone;

    __shared__ __attribute__((aligned(1024))) uint16_t k_lds0[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t k_lds1[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t v_lds0[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t v_lds1[TILE];

    // One block per workgroup or, in a persistent launch (causal masks,
    // blocks of unequal cost, more of them than the resident workgroups),
    // the paired static schedule of the forward kernel: the blocks of a head
    // are paired heavy with light at equal cost, each XCD owns a contiguous
    // range of pairs and its workgroups take them in turn.
    const int npair = (nqb + 1) / 2;
    const int xcd = blockIdx.x & 7;
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
            if ((wi & 1) && r == nqb - 1 - r) continue;   // odd count: the middle block is alone
        }
        // Opaque per block: offsets derived from the thread index are
        // recomputed in each block, not held in registers across the loop.
        int tid = threadIdx.x;
        if constexpr (PERSIST) asm volatile("" : "+v"(tid));
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int lane = tid & 63;
        const int j = lane & 31;
        const int h = lane >> 5;
        const int q0 = qb * BM_BWD;
        const int wrow0 = q0 + wave * 32;
        const int qrow = wrow0 + j;
        const bool qvalid = qrow < Nq;

        const uint16_t* K = Kg + (size_t)bh * Nk * D;
        const uint16_t* V = Vg + (size_t)bh * Nk * D;
        const int Lk = real_keys(kv_lens, bh / H, Nk);
        const int doff = causal == kCausalBottomRight ? Lk - Nq : 0;   // key j visible from query i iff j <= i + doff

        V8 qf[NKK], dof[NKK];
        load_b_rows<T, D>(Qg + (size_t)bh * Nq * D, qrow, qvalid, h, qf);
        load_b_rows<T, D>(dOg + (size_t)bh * Nq * D, qrow, qvalid, h, dof);
        const float l2 = qvalid ? LSEg[(size_t)bh * Nq + qrow] * kLog2e : 0.f;
        // D of this row, sum_d dO O in fp32 from the same B-operand layout (lane
        // (j, h) holds half of row j), written for the dK/dV kernel.
        float dr;
        {
            V8 of[NKK];
            load_b_rows<T, D>(Og + (size_t)bh * Nq * D, qrow, qvalid, h, of);
            float acc[2] = {0.f, 0.f};
    #pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                const u32x4_t a = __builtin_bit_cast(u32x4_t, of[kk]);
                const u32x4_t b = __builtin_bit_cast(u32x4_t, dof[kk]);
    #pragma unroll
                for (int w = 0; w < 4; ++w) {
                    acc[w & 1] = __builtin_fmaf(Elem<T>::lo(a[w]), Elem<T>::lo(b[w]), acc[w & 1]);
                    acc[w & 1] = __builtin_fmaf(Elem<T>::hi(a[w]), Elem<T>::hi(b[w]), acc[w & 1]);
                }
            }
            dr = sum_xor32(acc[0] + acc[1]);
            if (qvalid && h == 0) Dg[(size_t)bh * Nq + qrow] = dr;
        }

        TileOffsets<D> off;
        off.init(lane);

        f32x16_t acc[NDB];
    #pragma unroll
        for (int db = 0; db < NDB; ++db)
    #pragma unroll
            for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

        int kend = Lk;
        if (CAUSAL) kend = max(0, min(Lk, min(q0 + BM_BWD, Nq) + doff));
        const int ntiles = (kend + kBT - 1) / kBT;
        const int wlast = wrow0 + 31 + doff;        // last key the wave's last row may see
        const int my_tiles = CAUSAL ? (wlast < 0 ? 0 : min(ntiles, wlast / kBT + 1)) : ntiles;

        StageSlots<D, kBT> slots;                  // K and V tiles share the offsets
        slots.init(wave, lane);
        auto stage = [&](int t, uint16_t* kd, uint16_t* vd) __attribute__((always_inline)) {
            const int kv0 = t * kBT;               // < kend <= Lk
            const int valid = min(Lk - kv0, kBT);
            slots.stage(K + (size_t)kv0 * D, valid, kd, wave);
            slots.stage(V + (size_t)kv0 * D, valid, vd, wave);
        };
        auto compute = [&](int t, const uint16_t* kt, const uint16_t* vt) __attribute__((always_inline)) {
            // S^T = K Q^T and dP^T = V dO^T for 32 keys x this wave's 32 queries
            // (the compiler's order: a bounded operand ring measured 1.4% slower).
            f32x16_t s = {}, dp = {};
    #pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                s = Elem<T>::mfma(row_operand<T, D>(kt, off, kk), qf[kk], s);
                dp = Elem<T>::mfma(row_operand<T, D>(vt, off, kk), dof[kk], dp);
            }
            const int kv0 = t * kBT;
            const bool edge = kv0 + kBT > Lk || (CAUSAL && kv0 + kBT - 1 > wrow0 + doff);
            // P in place (register r is key 16*(r/8) + 8*h + r%8 of the tile),
            // then the mask of an edge tile in one branch: a per-score branch
            // would cut the exponentials into one basic block each, so no two of
            // them could overlap (measured 670 cycles per tile for this phase).
    #pragma unroll
            for (int r = 0; r < 16; ++r) s[r] = exp2_hw(__builtin_fmaf(s[r], scale2, -l2));
            if (edge) {
    #pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kv0 + (r / 8) * 16 + h * 8 + r % 8;
                    if (key >= Lk || (CAUSAL && key > qrow + doff)) s[r] = 0.f;
                }
            }
            V8 dsf[2];
    #pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                float ds[8];
    #pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int r = tt * 8 + e;
                    ds[e] = s[r] * (dp[r] - dr);
                }
                u32x4_t w;
                w[0] = Elem<T>::pack2(ds[0], ds[1]);
                w[1] = Elem<T>::pack2(ds[2], ds[3]);
                w[2] = Elem<T>::pack2(ds[4], ds[5]);
                w[3] = Elem<T>::pack2(ds[6], ds[7]);
                dsf[tt] = __builtin_bit_cast(V8, w);
            }
            // dQ^T += K^T dS^T.
    #pragma unroll
            for (int tt = 0; tt < 2; ++tt)
    #pragma unroll
                for (int db = 0; db < NDB; ++db)
                    acc[db] = Elem<T>::mfma(tr_operand<T, D>(kt, off, tt, db), dsf[tt], acc[db]);
        };

        if (ntiles > 0) stage(0, k_lds0, v_lds0);
        lds_dma_wait_all();
        __syncthreads();
        // Tile t in buffer t % 2; the next tile is loaded while t is computed and
        // published by the barrier that ends the iteration.
        for (int t = 0; t < ntiles; t += 2) {
            // Two workgroups share a CU. Left alone, one of them takes most of
            // the issue slots (measured per workgroup: two clusters of key-loop
            // times, ~72 and ~85 us, at 2048 keys); priorities that alternate by
            // tile pair and block parity even them out (one cluster, ~83 us).
            if (((t >> 1) + blockIdx.x) & 1) __builtin_amdgcn_s_setprio(1);
            else __builtin_amdgcn_s_setprio(0);
            if (t + 1 < ntiles) stage(t + 1, k_lds1, v_lds1);
            if (t < my_tiles) compute(t, k_lds0, v_lds0);
            lds_dma_wait_all();
            __syncthreads();
            if (t + 1 >= ntiles) break;
            if (t + 2 < ntiles) stage(t + 2, k_lds0, v_lds0);
            if (t + 1 < my_tiles) compute(t + 1, k_lds1, v_lds1);
            lds_dma_wait_all();
            __syncthreads();
        }

        // The last barrier above ended every read of the tile buffers: each wave
        // stages its dQ rows in one of them.
        uint16_t* const qst = wave == 0 ? k_lds0 : wave == 1 ? k_lds1 : wave == 2 ? v_lds0 : v_lds1;
        store_rows_staged<T, D>(dQg + ((size_t)bh * Nq + wrow0) * D, Nq - wrow0, acc, scale, qst, lane);

        // The next block's loads reuse the LDS buffers.
        if constexpr (PERSIST) __syncthreads();
    }
}

// dK and dV for 128 keys of one (batch, head), streaming Q, dO, L and D tiles.
template <typename T, int D, bool PERSIST>
__global__ __launch_bounds__(kBwdThreads, 2)
void bwd_dkdv_kernel(const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg,
                     const uint16_t* __restrict__ Vg, const uint16_t* __restrict__ dOg,
                     const float* __restrict__ LSEg, const float* __restrict__ Dg,
                     uint16_t* __restrict__ dKg, uint16_t* __restrict__ dVg, const int* __restrict__ kv_lens,
                     int H, int Nq, int Nk, int nkb, float scale, float scale2, int causal, int n_bh) {
    using V8 = typename Elem<T>::v8;
    constexpr int NKK = D / 16, NDB = D / 32, CPR = D / 8;
    constexpr int TILE = kBT * D;
    const bool CAUSAL = causal != kCausalNone;

    // Small arrays first: every buffer's base then fits the 16-bit offset
    // field of the LDS instructions.
    __shared__ __attribute__((aligned(16))) float ld_lds[2][2 * kBT];  // per tile: L (base 2), then D
    __shared__ __attribute__((aligned(1024))) uint16_t q_lds0[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t q_lds1[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t o_lds0[TILE];    // dO tiles
    __shared__ __attribute__((aligned(1024))) uint16_t o_lds1[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t v_blk[BM_BWD * D];

    // One block per workgroup or, in a persistent launch (causal masks,
    // blocks of unequal cost, more of them than the resident workgroups),
    // the paired static schedule of the forward kernel: the blocks of a head
    // are paired heavy with light at equal cost, each XCD owns a contiguous
    // range of pairs and its workgroups take them in turn.
    const int npair = (nkb + 1) / 2;
    const int xcd = blockIdx.x & 7;
    const int per_xcd = gridDim.x >> 3;        // a persistent grid is a multiple of 8
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
        // Opaque per block: offsets derived from the thread index are
        // recomputed in each block, not held in registers across the loop.
        int tid = threadIdx.x;
        if constexpr (PERSIST) asm volatile("" : "+v"(tid));
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int lane = tid & 63;
        const int j = lane & 31;
        const int h = lane >> 5;
        const int k0 = kb * BM_BWD;
        const int kw0 = k0 + wave * 32;
        const int krow = kw0 + j;
        const int Lk = real_keys(kv_lens, bh / H, Nk);
        // Keys past Lk (padding) are never read: their K rows and V rows are
        // zeros here, so S = dP = 0 and, with P = 0, dS = 0 exactly whatever the
        // padded cache holds (a NaN there would otherwise survive 0 * NaN).
        const bool kvalid = krow < Lk;
        const int doff = causal == kCausalBottomRight ? Lk - Nq : 0;   // key j visible from query i iff j <= i + doff

        const uint16_t* Q = Qg + (size_t)bh * Nq * D;
        const uint16_t* dO = dOg + (size_t)bh * Nq * D;
        const float* L = LSEg + (size_t)bh * Nq;
        const float* Dv = Dg + (size_t)bh * Nq;

        V8 kf[NKK];
        load_b_rows<T, D>(Kg + (size_t)bh * Nk * D, krow, kvalid, h, kf);
        TileOffsets<D> off;
        off.init(lane);
        // V rows of this wave as MFMA B operands of dP = dO V^T: lane (j, h)
        // reads row 32*wave + j of the block, elements 16*kk + 8*h .. +7.
        uint32_t voff[NKK];
    #pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            const int row = wave * 32 + j;
            voff[kk] = (uint32_t)(row * D + ((kk * 2 + h) ^ swz<CPR>(row)) * 8) * 2u;
            asm volatile("" : "+v"(voff[kk]));
        }

        f32x16_t adk[NDB], adv[NDB];
    #pragma unroll
        for (int db = 0; db < NDB; ++db)
    #pragma unroll
            for (int r = 0; r < 16; ++r) {
                adk[db][r] = 0.f;
                adv[db][r] = 0.f;
            }

        const int nqt = (Nq + kBT - 1) / kBT;
        // Causal: key j is seen by queries i >= j - off only, so tiles start at the
        // block's (the wave's) first such query. Keys at or past Lk are padding:
        // a block (a wave) made of them runs no tile and stores zeros.
        auto first_tile = [&](int key0) __attribute__((always_inline)) {
            if (key0 >= Lk) return nqt;
            return CAUSAL ? min(nqt, max(0, key0 - doff) / kBT) : 0;
        };
        const int first = first_tile(k0);
        const int my_first = first_tile(kw0);

        // L and D of tile u through registers of wave 0 (lanes 0-31: L, 32-63: D).
        // The load is issued with the tile's DMA and its value first used after
        // the next tile's compute, when it is scaled and written to LDS, so the
        // global-load latency stays off the critical path.
        float ld_reg = 0.f;
        auto fetch_ld = [&](int u) __attribute__((always_inline)) {
            if (wave == 0) {
                const int q = min(u * kBT + j, Nq - 1);
                ld_reg = h == 0 ? L[q] : Dv[q];
            }
        };
        auto put_ld = [&](int buf) __attribute__((always_inline)) {
            if (wave == 0) ld_lds[buf][lane] = h == 0 ? ld_reg * kLog2e : ld_reg;
        };
        StageSlots<D, kBT> slots;                  // Q and dO tiles share the offsets
        slots.init(wave, lane);
        auto stage = [&](int u, uint16_t* qd, uint16_t* od) __attribute__((always_inline)) {
            const int q0 = u * kBT;                // < Nq
            const int valid = min(Nq - q0, kBT);
            slots.stage(Q + (size_t)q0 * D, valid, qd, wave);
            slots.stage(dO + (size_t)q0 * D, valid, od, wave);
        };
        auto v_operand = [&](int kk) __attribute__((always_inline)) {
            return *(LDS_AS const V8*)((LDS_AS const char*)(LDS_AS const uint16_t*)v_blk + voff[kk]);
        };
        // One tile in phases with their own live registers (sched_barrier between
        // them): S = Q K^T, P, dV^T += dO^T P, dP = dO V^T, dS, dK^T += Q^T dS.
        auto compute = [&](int u, const uint16_t* qt, const uint16_t* ot, int buf) __attribute__((always_inline)) {
            constexpr int LEAD = 2;                // operand prefetch depth (register budget: 256 VGPRs)
            f32x16_t s = {};
            mfma_stream<NKK, LEAD>([&](int kk) { return row_operand<T, D>(qt, off, kk); },
                                   [&](int kk, V8 a) { s = Elem<T>::mfma(a, kf[kk], s); });
            const int q0 = u * kBT;
            const bool edge = q0 + kBT > Nq || kw0 + 32 > Lk || (CAUSAL && q0 + doff < kw0 + 31);
            // P (fp32, kept for dS) and its bf16 copy. Register r of lane (j, h)
            // is query 16*(r/8) + 8*h + r%8 of the tile.
            // P in place, then the mask of an edge tile in one branch (a
            // per-score branch would cut the exponentials into one basic block
            // each, so no two of them could overlap: measured 818 cycles per tile
            // for this phase).
    #pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const f32x4_t la = *(const f32x4_t*)&ld_lds[buf][tt * 16 + h * 8];
                const f32x4_t lb = *(const f32x4_t*)&ld_lds[buf][tt * 16 + h * 8 + 4];
    #pragma unroll
                for (int e = 0; e < 8; ++e)
                    s[tt * 8 + e] = exp2_hw(__builtin_fmaf(s[tt * 8 + e], scale2, -(e < 4 ? la[e] : lb[e - 4])));
            }
            if (edge) {
    #pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int q = q0 + (r / 8) * 16 + h * 8 + r % 8;
                    if (q >= Nq || krow >= Lk || (CAUSAL && q + doff < krow)) s[r] = 0.f;
                }
            }
            V8 pf[2];
    #pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                u32x4_t w;
                w[0] = Elem<T>::pack2(s[tt * 8 + 0], s[tt * 8 + 1]);
                w[1] = Elem<T>::pack2(s[tt * 8 + 2], s[tt * 8 + 3]);
                w[2] = Elem<T>::pack2(s[tt * 8 + 4], s[tt * 8 + 5]);
                w[3] = Elem<T>::pack2(s[tt * 8 + 6], s[tt * 8 + 7]);
                pf[tt] = __builtin_bit_cast(V8, w);
            }
            __builtin_amdgcn_sched_barrier(0);
            mfma_stream<2 * NDB, LEAD>([&](int i) { return tr_operand<T, D>(ot, off, i / NDB, i % NDB); },
                                       [&](int i, V8 a) {
                                           adv[i % NDB] = Elem<T>::mfma(a, pf[i / NDB], adv[i % NDB]);
                                       });
            f32x16_t dp = {};
            // Both operands of dP come from LDS (the dO tile and the block's V
            // rows), and both go through the prefetch ring.
            mfma_stream<NKK, LEAD>([&](int kk) { return OperandPair<V8>{row_operand<T, D>(ot, off, kk), v_operand(kk)}; },
                                   [&](int kk, OperandPair<V8> ab) {
                                       dp = Elem<T>::mfma(ab.a, ab.b, dp);
                                   });
            V8 dsf[2];
    #pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const f32x4_t da = *(const f32x4_t*)&ld_lds[buf][kBT + tt * 16 + h * 8];
                const f32x4_t dbv = *(const f32x4_t*)&ld_lds[buf][kBT + tt * 16 + h * 8 + 4];
                float ds[8];
    #pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int r = tt * 8 + e;
                    ds[e] = s[r] * (dp[r] - (e < 4 ? da[e] : dbv[e - 4]));
                }
                u32x4_t x;
                x[0] = Elem<T>::pack2(ds[0], ds[1]);
                x[1] = Elem<T>::pack2(ds[2], ds[3]);
                x[2] = Elem<T>::pack2(ds[4], ds[5]);
                x[3] = Elem<T>::pack2(ds[6], ds[7]);
                dsf[tt] = __builtin_bit_cast(V8, x);
            }
            __builtin_amdgcn_sched_barrier(0);
            mfma_stream<2 * NDB, LEAD>([&](int i) { return tr_operand<T, D>(qt, off, i / NDB, i % NDB); },
                                       [&](int i, V8 a) {
                                           adk[i % NDB] = Elem<T>::mfma(a, dsf[i / NDB], adk[i % NDB]);
                                       });
        };

        // Prologue: the block's V rows (zeros past Lk) and the first tile.
        {
            StageSlots<D, BM_BWD> vslots;
            vslots.init(wave, lane);
            vslots.stage(Vg + ((size_t)bh * Nk + k0) * D, max(0, min(Lk - k0, BM_BWD)), v_blk, wave);
        }
        if (first < nqt) {
            stage(first, q_lds0, o_lds0);
            fetch_ld(first);
            put_ld(0);
        }
        lds_dma_wait_all();
        __syncthreads();
        // Tile first + 2i in buffer 0, first + 2i + 1 in buffer 1.
        for (int u = first; u < nqt; u += 2) {
            // Alternating priorities, as in the dQ kernel (two workgroups per CU).
            if ((((u - first) >> 1) + blockIdx.x) & 1) __builtin_amdgcn_s_setprio(1);
            else __builtin_amdgcn_s_setprio(0);
            if (u + 1 < nqt) {
                stage(u + 1, q_lds1, o_lds1);
                fetch_ld(u + 1);
            }
            if (u >= my_first) compute(u, q_lds0, o_lds0, 0);
            if (u + 1 < nqt) put_ld(1);
            lds_dma_wait_all();
            __syncthreads();
            if (u + 1 >= nqt) break;
            if (u + 2 < nqt) {
                stage(u + 2, q_lds0, o_lds0);
                fetch_ld(u + 2);
            }
            if (u + 1 >= my_first) compute(u + 1, q_lds1, o_lds1, 1);
            if (u + 2 < nqt) put_ld(0);
            lds_dma_wait_all();
            __syncthreads();
        }

        // The last barrier above ended every read of the Q / dO tiles and of the
        // V block: each wave stages its dK rows in one tile buffer and its dV rows
        // in its own quarter of the V block. Rows past Nk are not stored.
        uint16_t* const kst = wave == 0 ? q_lds0 : wave == 1 ? q_lds1 : wave == 2 ? o_lds0 : o_lds1;
        store_rows_staged<T, D>(dKg + ((size_t)bh * Nk + kw0) * D, Nk - kw0, adk, scale, kst, lane);
        store_rows_staged<T, D>(dVg + ((size_t)bh * Nk + kw0) * D, Nk - kw0, adv, 1.0f, v_blk + wave * 32 * D, lane);

        // The next block's loads reuse the LDS buffers.
        if constexpr (PERSIST) __syncthreads();
    }
}

// Grid of a persistent launch for kernel f over n_bh heads of
// blocks_per_head blocks (the kernels' paired schedule): every resident
// workgroup slot of the device, or 0 for one block per workgroup.
template <typename Kern>
static hipError_t persistent_grid(Kern f, int n_bh, int blocks_per_head, int* grid) {
    *grid = 0;
    int cus = 0, per_cu = 0;
    hipError_t e = device_cu_count(&cus);
    if (e != hipSuccess) return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(f), kBwdThreads, 0);
    if (e != hipSuccess) return e;
    *grid = paired_schedule_grid(cus * per_cu, n_bh, blocks_per_head);
    return hipSuccess;
}

template <typename T, int D>
static hipError_t launch_bwd_d(const BwdArgs& a) {
    const float scale2 = a.scale * kLog2e;
    const int n_bh = a.B * a.H;
    // Persistent launches for causal self-attention (Nq = Nk, no key
    // padding), where a block's cost is linear in its index, so that the
    // paired blocks cost the same.
    const bool paired = a.causal != kCausalNone && !a.kv_lens && a.Nq == a.Nk;
    if (a.Nq > 0) {
        const int nqb = (a.Nq + BM_BWD - 1) / BM_BWD;
        int grid = 0;
        if (paired) {
            const hipError_t e = persistent_grid(bwd_dq_kernel<T, D, true>, n_bh, nqb, &grid);
            if (e != hipSuccess) return e;
        }
        const bool persist = grid > 0;
        if (!persist) grid = n_bh * nqb;
        auto kern = persist ? bwd_dq_kernel<T, D, true> : bwd_dq_kernel<T, D, false>;
        hipLaunchKernelGGL(kern, dim3(grid), dim3(kBwdThreads), 0, a.stream,
                           (const uint16_t*)a.Q, (const uint16_t*)a.K, (const uint16_t*)a.V,
                           (const uint16_t*)a.O, (const uint16_t*)a.dO, a.LSE, a.Dvec, (uint16_t*)a.dQ,
                           a.kv_lens, a.H, a.Nq, a.Nk, nqb, a.scale, scale2, a.causal, n_bh);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // With Nq = 0 the dK/dV kernel stages only V, runs no query tile and
    // stores zeros.
    const int nkb = (a.Nk + BM_BWD - 1) / BM_BWD;
    int grid = 0;
    if (paired) {
        const hipError_t e = persistent_grid(bwd_dkdv_kernel<T, D, true>, n_bh, nkb, &grid);
        if (e != hipSuccess) return e;
    }
    const bool persist = grid > 0;
    if (!persist) grid = n_bh * nkb;
    auto kern = persist ? bwd_dkdv_kernel<T, D, true> : bwd_dkdv_kernel<T, D, false>;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kBwdThreads), 0, a.stream,
                       (const uint16_t*)a.Q, (const uint16_t*)a.K, (const uint16_t*)a.V,
                       (const uint16_t*)a.dO, a.LSE, a.Dvec, (uint16_t*)a.dK, (uint16_t*)a.dV, a.kv_lens,
                       a.H, a.Nq, a.Nk, nkb, a.scale, scale2, a.causal, n_bh);
    return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a) {
    // D = 128 runs on the 16x16x32 MFMA (fa_bwd16.hip).
    if (a.D == 128) return launch_bwd16(a);
    return a.f16 ? launch_bwd_d<_Float16, 64>(a) : launch_bwd_d<__bf16, 64>(a);
}

}  // namespace fa
