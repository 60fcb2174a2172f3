// Rotary position embedding of [B, H, N, D] rows, bf16 or fp16 (phobos page,
// "Rotary position embeddings": rope, rotate-half form, and rope_pairs,
// adjacent pairs). Row n of every (batch, head) is rotated by the angles of
// position n: cos and sin are [n_pos, D/2] fp32 tables. The arithmetic is
// fp32 and the result is rounded to the input type (nearest even).
//
// This is the K half of the forward pass's fused RoPE prologue (Q is rotated
// in registers inside the attention kernel): every K tile is read by all the
// query blocks of its head, so K is rotated once here, streaming, rather than
// once per query block inside the key loop. The kernel is HBM-bound: D/16
// threads share a row, each rotating two 16-byte chunks (the partners d and
// d + D/2, or two chunks of adjacent pairs) with their cos/sin values, which
// are shared by every head and stay in the caches.

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

constexpr int kRopeThreads = 256;

template <typename T, int D>
__global__ __launch_bounds__(kRopeThreads)
void rope_kernel(const uint16_t* X, uint16_t* Y, const float* __restrict__ cos_t,
                 const float* __restrict__ sin_t, long long rows, int N, int style) {
    constexpr int TPR = D / 16;                    // threads per row
    constexpr int RPB = kRopeThreads / TPR;        // rows per block
    const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
    const int c = threadIdx.x % TPR;
    if (row >= rows) return;
    const int pos = (int)(row % N);
    const uint16_t* x = X + row * D;
    uint16_t* y = Y + row * D;
    const float* cr = cos_t + (size_t)pos * (D / 2);
    const float* sr = sin_t + (size_t)pos * (D / 2);
    // Chunks (16 bytes, 8 elements) handled by this thread.
    const int ca = style == kRopeHalf ? c : 2 * c;
    const int cb = style == kRopeHalf ? c + D / 16 : 2 * c + 1;
    u32x4_t wa = *(const u32x4_t*)(x + ca * 8);
    u32x4_t wb = *(const u32x4_t*)(x + cb * 8);
    const f32x4_t c0 = *(const f32x4_t*)(cr + 8 * c), c1 = *(const f32x4_t*)(cr + 8 * c + 4);
    const f32x4_t s0 = *(const f32x4_t*)(sr + 8 * c), s1 = *(const f32x4_t*)(sr + 8 * c + 4);
    uint32_t a[4] = {wa[0], wa[1], wa[2], wa[3]};
    uint32_t b[4] = {wb[0], wb[1], wb[2], wb[3]};
    if (style == kRopeHalf) {
        // Elements 8c..8c+7 of both halves, angles 8c..8c+7.
        const float cc[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
        const float ss[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
        rope_half_chunks<T>(a, b, cc, ss);
    } else {
        // Elements 16c..16c+15: pairs 8c..8c+3 in chunk a, 8c+4..8c+7 in chunk b.
        const float ca4[4] = {c0[0], c0[1], c0[2], c0[3]}, sa4[4] = {s0[0], s0[1], s0[2], s0[3]};
        const float cb4[4] = {c1[0], c1[1], c1[2], c1[3]}, sb4[4] = {s1[0], s1[1], s1[2], s1[3]};
        rope_pair_chunk<T>(a, ca4, sa4);
        rope_pair_chunk<T>(b, cb4, sb4);
    }
    *(u32x4_t*)(y + ca * 8) = u32x4_t{a[0], a[1], a[2], a[3]};
    *(u32x4_t*)(y + cb * 8) = u32x4_t{b[0], b[1], b[2], b[3]};
}

template <typename T, int D>
static hipError_t launch_rope_t(const RopeArgs& a) {
    constexpr int RPB = kRopeThreads / (D / 16);
    const long long rows = (long long)a.B * a.H * a.N;
    hipLaunchKernelGGL((rope_kernel<T, D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(kRopeThreads), 0,
                       a.stream, (const uint16_t*)a.X, (uint16_t*)a.Y, a.cos, a.sin, rows, a.N, a.style);
    return hipGetLastError();
}

hipError_t launch_rope(const RopeArgs& a) {
    if (a.f16) return a.D == 128 ? launch_rope_t<_Float16, 128>(a) : launch_rope_t<_Float16, 64>(a);
    return a.D == 128 ? launch_rope_t<__bf16, 128>(a) : launch_rope_t<__bf16, 64>(a);
}

}  // namespace fa
