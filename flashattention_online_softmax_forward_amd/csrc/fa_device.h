// Device-side helpers shared by the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Running maximum of a row that has not seen a visible key yet (base 2). Finite,
// so exp2(masked score - it) = exp2(-inf) = 0 and exp2(it - real maximum) = 0,
// where -inf would give exp2(-inf - -inf) = NaN.
constexpr float kNoKeyMax = -1e30f;

// Two fp32 values to a packed pair of bf16 (round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Low / high bf16 of a packed word widened to fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
// The fp16 MFMA and transpose-read builtins take __fp16 vectors.
typedef __fp16 fp16x8_t __attribute__((ext_vector_type(8)));
typedef __fp16 fp16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

// Low / high fp16 of a packed word widened to fp32 (exact).
__device__ __forceinline__ float f16_lo(uint32_t w) {
    return (float)__builtin_bit_cast(f16x2_t, w)[0];
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
    return (float)__builtin_bit_cast(f16x2_t, w)[1];
}

// The 16-bit input types the MFMA kernels are instantiated for (bf16 and
// fp16): operand vectors, the 32x32x16 and 16x16x32 MFMAs with fp32 accumulation, the LDS
// transpose read, round-to-nearest-even packing of two fp32 values, and
// widening of the halves of a packed word.
template <typename T> struct Elem;
template <> struct Elem<__bf16> {
    using v8 = bf16x8_t;
    using v4 = bf16x4_t;
    __device__ static __forceinline__ f32x16_t mfma(v8 a, v8 b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static __forceinline__ f32x4_t mfma16(v8 a, v8 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static __forceinline__ v4 tr_read(__attribute__((address_space(3))) v4* p) {
        return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(p);
    }
    __device__ static __forceinline__ uint32_t pack2(float lo, float hi) { return pack_bf16x2(lo, hi); }
    __device__ static __forceinline__ float lo(uint32_t w) { return bf16_lo(w); }
    __device__ static __forceinline__ float hi(uint32_t w) { return bf16_hi(w); }
};
template <> struct Elem<_Float16> {
    using v8 = fp16x8_t;
    using v4 = fp16x4_t;
    __device__ static __forceinline__ f32x16_t mfma(v8 a, v8 b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    __device__ static __forceinline__ f32x4_t mfma16(v8 a, v8 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    __device__ static __forceinline__ v4 tr_read(__attribute__((address_space(3))) v4* p) {
        return __builtin_amdgcn_ds_read_tr16_b64_v4f16(p);
    }
    __device__ static __forceinline__ uint32_t pack2(float lo, float hi) {
        f16x2_t v = {(_Float16)lo, (_Float16)hi};
        return __builtin_bit_cast(uint32_t, v);
    }
    __device__ static __forceinline__ float lo(uint32_t w) { return f16_lo(w); }
    __device__ static __forceinline__ float hi(uint32_t w) { return f16_hi(w); }
};

// Rotary position embedding of 16-byte chunks (8 elements of type T), in
// fp32 and rounded back to T (phobos page, "Rotary position embeddings").
//   rotate-half: chunk `a` holds elements i..i+7 of the first half of a row
//   and `b` the same elements of the second half; with c = cos[i..i+7] and
//   s = sin[i..i+7], a <- a c - b s and b <- b c + a s.
//   adjacent pairs: chunk `w` holds elements 2p..2p+7, i.e. pairs p..p+3;
//   with c = cos[p..p+3], s = sin[p..p+3], (x0, x1) <- (x0 c - x1 s, x1 c + x0 s).
template <typename T>
__device__ __forceinline__ void rope_half_chunks(uint32_t* a, uint32_t* b, const float* c, const float* s) {
    using E = Elem<T>;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const float a0 = E::lo(a[w]), a1 = E::hi(a[w]), b0 = E::lo(b[w]), b1 = E::hi(b[w]);
        const float c0 = c[2 * w], c1 = c[2 * w + 1], s0 = s[2 * w], s1 = s[2 * w + 1];
        a[w] = E::pack2(__builtin_fmaf(a0, c0, -b0 * s0), __builtin_fmaf(a1, c1, -b1 * s1));
        b[w] = E::pack2(__builtin_fmaf(b0, c0, a0 * s0), __builtin_fmaf(b1, c1, a1 * s1));
    }
}

template <typename T>
__device__ __forceinline__ void rope_pair_chunk(uint32_t* x, const float* c, const float* s) {
    using E = Elem<T>;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const float x0 = E::lo(x[w]), x1 = E::hi(x[w]);
        x[w] = E::pack2(__builtin_fmaf(x0, c[w], -x1 * s[w]), __builtin_fmaf(x1, c[w], x0 * s[w]));
    }
}

// Hardware base-2 exponential (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Word 3 of a raw buffer resource on gfx9-family parts: 32-bit data format,
// no swizzle, no index stride.
constexpr int kBufferRsrcWord3 = 0x00020000;

// Cache-policy operand of a buffer access on gfx950 (the gfx940 encoding:
// bit 0 SC0, bit 1 NT, bit 4 SC1). NT marks the line non-temporal, so L2
// streams it instead of keeping it for reuse. Used for data one workgroup touches once, which would
// otherwise push out K/V lines that other workgroups of the head re-read.
constexpr int kCachePolicyNT = 2;

// Slots I .. N-1 (N <= 4) of a wave's share of a tile load into LDS
// (buffer_load_dwordx4 with the lds bit): slot I moves 16 bytes per lane from
// the resource at voff[I] + 1 KB * I to base + 1 KB * I + 16 * lane. The
// immediate offset supplies the 1 KB step (it moves the LDS destination and
// the memory address alike), so voff[I] is stored net of it. A lane whose
// offset is past the resource's size writes zeros. POLICY holds the cache
// policy bits (0 or kCachePolicyNT).
template <int N, int I = 0, int POLICY = 0>
__device__ __forceinline__ void buffer_lds_slots(__amdgpu_buffer_rsrc_t rsrc, __attribute__((address_space(3))) void* base,
                                                 const uint32_t* voff) {
    static_assert(N <= 4, "the immediate offset field holds at most 3 KB");
    if constexpr (I < N) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, base, 16, voff[I], 0, I * 1024, POLICY);
        buffer_lds_slots<N, I + 1, POLICY>(rsrc, base, voff);
    }
}

// NaN-propagating maximum (IEEE 754-2019 maximum). gfx950 has it as
// v_maximum3_f32, which needs no quieting of its operands, where fmaxf's
// number-preferring maxnum costs a canonicalising v_max per raw MFMA result.
__device__ __forceinline__ float fmax_nan(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Combine a value with the one held by lane (lane ^ 32): v_permlane32_swap
// returns both halves, so a symmetric op of the two results is the same in
// every lane.
__device__ __forceinline__ float max_xor32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmax_nan(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The same with lane (lane ^ 16), through v_permlane16_swap.
__device__ __forceinline__ float max_xor16(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmax_nan(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// DPP lane moves inside a row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

// Sum over aligned groups of N lanes (N = 4, 8 or 16); every lane of the
// group ends with the group total.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(N == 4 || N == 8 || N == 16, "group of 4, 8 or 16 lanes");
    x += dpp_mov<kDppQuadXor1>(x);
    x += dpp_mov<kDppQuadXor2>(x);
    if (N >= 8) x += dpp_mov<kDppRowHalfMirror>(x);
    if (N >= 16) x += dpp_mov<kDppRowMirror>(x);
    return x;
}
template <int N>
__device__ __forceinline__ float group_max(float x) {
    static_assert(N == 4 || N == 8 || N == 16, "group of 4, 8 or 16 lanes");
    x = fmaxf(x, dpp_mov<kDppQuadXor1>(x));
    x = fmaxf(x, dpp_mov<kDppQuadXor2>(x));
    if (N >= 8) x = fmaxf(x, dpp_mov<kDppRowHalfMirror>(x));
    if (N >= 16) x = fmaxf(x, dpp_mov<kDppRowMirror>(x));
    return x;
}

// Workgroups are handed to the 8 XCDs round-robin (id % 8). Renumber them so
// that each XCD runs a contiguous range of logical tiles: consecutive logical
// tiles share K/V of one (batch, head), which then stays in that XCD's L2.
__device__ __forceinline__ int xcd_logical_block(int id, int total) {
    const int per = total / 8;
    const int full = per * 8;
    return id < full ? (id % 8) * per + id / 8 : id;
}

}  // namespace fa
