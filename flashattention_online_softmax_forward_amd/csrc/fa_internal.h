// Host-side launch interface between the C ABI (fa_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

constexpr int BM_FWD = 256;      // query rows per workgroup, bf16 forward (8 waves x 32)
constexpr int BM_FWD_F32 = 16;   // query rows per workgroup, fp32 forward (16 threads per row)
constexpr int BM_BWD = 128;      // rows (queries for dQ, keys for dK/dV) per workgroup, backward (4 waves x 32)

// Causal alignment: none, top-left (key j visible from query i iff j <= i),
// bottom-right (iff j <= i + Lk - Nq, Lk the batch entry's real key count).
constexpr int kCausalNone = 0;
constexpr int kCausalTopLeft = 1;
constexpr int kCausalBottomRight = 2;

// RoPE forms: rotate-half (halves a, b of a row) and adjacent pairs.
constexpr int kRopeHalf = 0;
constexpr int kRopePairs = 1;

// Real key count of batch entry b: kv_lens[b] clamped to [0, Nk], or Nk.
__device__ __forceinline__ int real_keys(const int* kv_lens, int b, int Nk) {
    return kv_lens ? min(max(kv_lens[b], 0), Nk) : Nk;
}

struct FwdArgs {
    const void* Q;
    const void* K;
    const void* V;
    void* O;
    float* LSE;
    const int* kv_lens;   // [B] real key counts, or NULL (all Nk)
    int B, H, Nq, Nk, D;
    float scale;
    int causal;           // kCausalNone / kCausalTopLeft / kCausalBottomRight
    hipStream_t stream;
    // Fused RoPE on Q (bf16/fp16 MFMA forward only): cos/sin [n_pos, D/2] fp32,
    // or NULL for none; K is expected already rotated.
    const float* rope_cos = nullptr;
    const float* rope_sin = nullptr;
    int rope_style = 0;   // kRopeHalf / kRopePairs
};

struct RopeArgs {
    const void* X;
    void* Y;
    const float* cos;
    const float* sin;
    int B, H, N, D;
    int style;            // kRopeHalf / kRopePairs
    bool f16;             // element type: fp16 (else bf16)
    hipStream_t stream;
};

struct DecodeArgs {
    const void* Q;
    const void* K;
    const void* V;
    void* O;
    float* LSE;
    float* ws_o;     // [B*H, S, D] partial unnormalised outputs
    float* ws_ml;    // [B*H, S, 2] partial (m in base 2, l)
    const int* kv_lens;   // [B] real key counts, or NULL (all Nk)
    int B, H, Nk, D, S;
    float scale;
    hipStream_t stream;
    bool f16 = false;     // element type: fp16 (else bf16)
};

struct BwdArgs {
    const void* Q;
    const void* K;
    const void* V;
    const void* O;
    const void* dO;
    const float* LSE;
    void* dQ;
    void* dK;
    void* dV;
    float* Dvec;     // [B*H, Nq] row dot products sum_d dO * O
    const int* kv_lens;   // [B] real key counts, or NULL (all Nk)
    int B, H, Nq, Nk, D;
    float scale;
    int causal;           // kCausalNone / kCausalTopLeft / kCausalBottomRight
    hipStream_t stream;
    bool f16 = false;     // element type: fp16 (else bf16)
};

hipError_t launch_fwd_bf16(const FwdArgs& a);
hipError_t launch_fwd_f16(const FwdArgs& a);
// The D = 128 forward on the 16x16x32 MFMA (fa_fwd_mfma16.hip), bf16 or fp16.
hipError_t launch_fwd16(const FwdArgs& a, bool f16);
hipError_t launch_rope(const RopeArgs& a);
hipError_t launch_fwd_f32(const FwdArgs& a);
hipError_t launch_decode(const DecodeArgs& a);

// Size of the fixed per-GPU scratch of fa_decode_splitkv_noalloc.
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;
// Device address of that scratch on the current device (looked up once per
// device, then cached).
hipError_t decode_scratch(void** ptr);
hipError_t launch_bwd(const BwdArgs& a);
// Compute units of the current device (asked once per device), for the
// persistent causal launches.
hipError_t device_cu_count(int* n);
// Grid of a persistent launch with the paired causal schedule, given the
// device's resident workgroup slots, or 0 when one block per workgroup is
// the better launch (too few pairs, or pairs that do not share out evenly).
int paired_schedule_grid(int slots, int n_bh, int blocks_per_head);

}  // namespace fa
