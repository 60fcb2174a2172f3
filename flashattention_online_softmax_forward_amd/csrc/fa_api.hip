// C ABI of the library (declared in include/fa.h): argument checks, then one
// launch (two for decode) on the caller's stream. No allocation, no
// synchronisation, no state.

#include <climits>
#include <cmath>
#include <cstdint>

#include "fa.h"
#include "fa_internal.h"

static_assert(FA_DECODE_NOALLOC_SCRATCH_BYTES == fa::kDecodeScratchBytes,
              "the header states the size of the decode scratch");
static_assert(FA_ROPE_HALF == fa::kRopeHalf && FA_ROPE_PAIRS == fa::kRopePairs,
              "RoPE styles of the C ABI and the kernels agree");
static_assert(FA_CAUSAL_NONE == fa::kCausalNone && FA_CAUSAL_TOP_LEFT == fa::kCausalTopLeft &&
                  FA_CAUSAL_BOTTOM_RIGHT == fa::kCausalBottomRight,
              "causal modes of the C ABI and the kernels agree");

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

bool good_scale(float s) { return std::isfinite(s) && s > 0.0f; }

bool good_causal(int c) { return c == FA_CAUSAL_NONE || c == FA_CAUSAL_TOP_LEFT || c == FA_CAUSAL_BOTTOM_RIGHT; }

// kv_lens (NULL or B ints, 4-byte aligned) must not overlap the call's two
// largest outputs (it is read while they are written).
bool good_kv_lens(const int* kv_lens, int B, const void* out1, size_t n1, const void* out2, size_t n2) {
    if (!kv_lens) return true;
    if (!aligned4(kv_lens)) return false;
    const size_t nb = (size_t)B * sizeof(int);
    return !overlaps(kv_lens, nb, out1, n1) && !overlaps(kv_lens, nb, out2, n2);
}

// Shared checks of the two forward entry points; `elem` is the element size.
fa_status check_forward(const void* Q, const void* K, const void* V, const void* O, const float* LSE,
                        int B, int H, int Nq, int Nk, int D, float scale, size_t elem, int bm,
                        bool* nothing_to_do) {
    *nothing_to_do = false;
    if (B < 0 || H < 0 || Nq < 0 || Nk < 0) return FA_ERR_INVALID_ARG;
    if (!good_scale(scale)) return FA_ERR_INVALID_ARG;
    if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
    if ((long long)B * H * Nq == 0) {
        *nothing_to_do = true;
        return FA_OK;
    }
    if (Nk < 1) return FA_ERR_INVALID_ARG;
    if (!Q || !K || !V || !O) return FA_ERR_INVALID_ARG;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return FA_ERR_INVALID_ARG;
    if (LSE && !aligned4(LSE)) return FA_ERR_INVALID_ARG;
    const long long nqb = ((long long)Nq + bm - 1) / bm;
    if ((long long)B * H * nqb > INT_MAX) return FA_ERR_UNSUPPORTED;
    const size_t bytes_q = (size_t)B * H * Nq * D * elem;
    const size_t bytes_kv = (size_t)B * H * Nk * D * elem;
    const size_t bytes_l = (size_t)B * H * Nq * sizeof(float);
    if (overlaps(O, bytes_q, Q, bytes_q) || overlaps(O, bytes_q, K, bytes_kv) ||
        overlaps(O, bytes_q, V, bytes_kv) || overlaps(O, bytes_q, LSE, bytes_l))
        return FA_ERR_INVALID_ARG;
    return FA_OK;
}

}  // namespace

extern "C" {

const char* fa_status_string(fa_status s) {
    switch (s) {
        case FA_OK: return "FA_OK";
        case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG: invalid argument (pointer, size, alignment, scale or workspace)";
        case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: unsupported head dimension or problem size";
        case FA_ERR_LAUNCH: return "FA_ERR_LAUNCH: kernel launch failed";
    }
    return "FA_ERR_UNKNOWN: unknown status code";
}

fa_status fa_forward_masked(const void* Q, const void* K, const void* V, void* O, float* LSE,
                            const int* kv_lens, int B, int H, int Nq, int Nk, int D, float scale, int causal,
                            hipStream_t stream) {
    if (!good_causal(causal)) return FA_ERR_INVALID_ARG;
    bool nothing = false;
    const fa_status st = check_forward(Q, K, V, O, LSE, B, H, Nq, Nk, D, scale, 2, fa::BM_FWD, &nothing);
    if (st != FA_OK || nothing) return st;
    if (!good_kv_lens(kv_lens, B, O, (size_t)B * H * Nq * D * 2, LSE, (size_t)B * H * Nq * 4))
        return FA_ERR_INVALID_ARG;
    const fa::FwdArgs a{Q, K, V, O, LSE, kv_lens, B, H, Nq, Nk, D, scale, causal, stream};
    return fa::launch_fwd_bf16(a) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

fa_status fa_forward(const void* Q, const void* K, const void* V, void* O, float* LSE,
                     int B, int H, int Nq, int Nk, int D, float scale, int causal, hipStream_t stream) {
    return fa_forward_masked(Q, K, V, O, LSE, nullptr, B, H, Nq, Nk, D, scale, causal, stream);
}

fa_status fa_forward_f16_masked(const void* Q, const void* K, const void* V, void* O, float* LSE,
                                const int* kv_lens, int B, int H, int Nq, int Nk, int D, float scale, int causal,
                                hipStream_t stream) {
    if (!good_causal(causal)) return FA_ERR_INVALID_ARG;
    bool nothing = false;
    const fa_status st = check_forward(Q, K, V, O, LSE, B, H, Nq, Nk, D, scale, 2, fa::BM_FWD, &nothing);
    if (st != FA_OK || nothing) return st;
    if (!good_kv_lens(kv_lens, B, O, (size_t)B * H * Nq * D * 2, LSE, (size_t)B * H * Nq * 4))
        return FA_ERR_INVALID_ARG;
    const fa::FwdArgs a{Q, K, V, O, LSE, kv_lens, B, H, Nq, Nk, D, scale, causal, stream};
    return fa::launch_fwd_f16(a) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

fa_status fa_forward_f16(const void* Q, const void* K, const void* V, void* O, float* LSE,
                         int B, int H, int Nq, int Nk, int D, float scale, int causal, hipStream_t stream) {
    return fa_forward_f16_masked(Q, K, V, O, LSE, nullptr, B, H, Nq, Nk, D, scale, causal, stream);
}

size_t fa_rope_workspace_bytes(int B, int H, int Nk, int D) {
    if (B < 0 || H < 0 || Nk < 0 || (D != 64 && D != 128)) return 0;
    return (size_t)B * H * Nk * D * 2;
}

fa_status fa_rope(const void* X, void* Y, const float* cos_t, const float* sin_t, int n_pos, int style,
                  int dtype, int B, int H, int N, int D, hipStream_t stream) {
    if (B < 0 || H < 0 || N < 0 || n_pos < 0) return FA_ERR_INVALID_ARG;
    if (style != FA_ROPE_HALF && style != FA_ROPE_PAIRS) return FA_ERR_INVALID_ARG;
    if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16) return FA_ERR_INVALID_ARG;
    if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
    if ((long long)B * H * N == 0) return FA_OK;
    if (n_pos < N) return FA_ERR_INVALID_ARG;
    if (!X || !Y || !cos_t || !sin_t) return FA_ERR_INVALID_ARG;
    if (!aligned16(X) || !aligned16(Y) || !aligned16(cos_t) || !aligned16(sin_t)) return FA_ERR_INVALID_ARG;
    const size_t bytes = (size_t)B * H * N * D * 2, tab = (size_t)n_pos * (D / 2) * sizeof(float);
    // In place (Y == X) is allowed; a partial overlap is not.
    if (Y != X && overlaps(X, bytes, Y, bytes)) return FA_ERR_INVALID_ARG;
    if (overlaps(Y, bytes, cos_t, tab) || overlaps(Y, bytes, sin_t, tab)) return FA_ERR_INVALID_ARG;
    if ((long long)B * H * N / (256 / (D / 16)) + 1 > INT_MAX) return FA_ERR_UNSUPPORTED;
    const fa::RopeArgs a{X, Y, cos_t, sin_t, B, H, N, D, style, dtype == FA_DTYPE_F16, stream};
    return fa::launch_rope(a) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

fa_status fa_forward_rope(const void* Q, const void* K, const void* V, void* O, float* LSE, const int* kv_lens,
                          const float* cos_t, const float* sin_t, int n_pos, int style, int dtype,
                          void* workspace, size_t workspace_bytes, int B, int H, int Nq, int Nk, int D,
                          float scale, int causal, hipStream_t stream) {
    if (!good_causal(causal)) return FA_ERR_INVALID_ARG;
    if (style != FA_ROPE_HALF && style != FA_ROPE_PAIRS) return FA_ERR_INVALID_ARG;
    if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16) return FA_ERR_INVALID_ARG;
    bool nothing = false;
    const fa_status st = check_forward(Q, K, V, O, LSE, B, H, Nq, Nk, D, scale, 2, fa::BM_FWD, &nothing);
    if (st != FA_OK || nothing) return st;
    const size_t bq = (size_t)B * H * Nq * D * 2, bkv = (size_t)B * H * Nk * D * 2;
    const size_t bl = (size_t)B * H * Nq * 4, tab = (size_t)n_pos * (D / 2) * sizeof(float);
    if (!good_kv_lens(kv_lens, B, O, bq, LSE, bl)) return FA_ERR_INVALID_ARG;
    if (n_pos < Nq || n_pos < Nk || !cos_t || !sin_t || !aligned16(cos_t) || !aligned16(sin_t))
        return FA_ERR_INVALID_ARG;
    const size_t need = fa_rope_workspace_bytes(B, H, Nk, D);
    if (!workspace || !aligned16(workspace) || workspace_bytes < need) return FA_ERR_INVALID_ARG;
    const void* ins[5] = {Q, K, V, cos_t, sin_t};
    const size_t in_bytes[5] = {bq, bkv, bkv, tab, tab};
    for (int j = 0; j < 5; ++j)
        if (overlaps(workspace, need, ins[j], in_bytes[j]) || overlaps(O, bq, ins[j], in_bytes[j]))
            return FA_ERR_INVALID_ARG;
    if (overlaps(workspace, need, O, bq) || overlaps(workspace, need, LSE, bl) ||
        overlaps(workspace, need, kv_lens, (size_t)B * 4))
        return FA_ERR_INVALID_ARG;
    if ((long long)B * H * Nk / (256 / (D / 16)) + 1 > INT_MAX) return FA_ERR_UNSUPPORTED;
    // K rotated once into the workspace (positions 0..Nk-1), then the
    // attention kernel rotates Q in registers and reads the rotated K.
    const fa::RopeArgs r{K, workspace, cos_t, sin_t, B, H, Nk, D, style, dtype == FA_DTYPE_F16, stream};
    if (fa::launch_rope(r) != hipSuccess) return FA_ERR_LAUNCH;
    fa::FwdArgs a{Q, workspace, V, O, LSE, kv_lens, B, H, Nq, Nk, D, scale, causal, stream};
    a.rope_cos = cos_t;
    a.rope_sin = sin_t;
    a.rope_style = style;
    const hipError_t e = dtype == FA_DTYPE_F16 ? fa::launch_fwd_f16(a) : fa::launch_fwd_bf16(a);
    return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

fa_status fa_forward_f32_masked(const float* Q, const float* K, const float* V, float* O, float* LSE,
                                const int* kv_lens, int B, int H, int Nq, int Nk, int D, float scale,
                                int causal, hipStream_t stream) {
    if (!good_causal(causal)) return FA_ERR_INVALID_ARG;
    bool nothing = false;
    const fa_status st = check_forward(Q, K, V, O, LSE, B, H, Nq, Nk, D, scale, 4, fa::BM_FWD_F32, &nothing);
    if (st != FA_OK || nothing) return st;
    if (!good_kv_lens(kv_lens, B, O, (size_t)B * H * Nq * D * 4, LSE, (size_t)B * H * Nq * 4))
        return FA_ERR_INVALID_ARG;
    const fa::FwdArgs a{Q, K, V, O, LSE, kv_lens, B, H, Nq, Nk, D, scale, causal, stream};
    return fa::launch_fwd_f32(a) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

fa_status fa_forward_f32(const float* Q, const float* K, const float* V, float* O, float* LSE,
                         int B, int H, int Nq, int Nk, int D, float scale, int causal, hipStream_t stream) {
    return fa_forward_f32_masked(Q, K, V, O, LSE, nullptr, B, H, Nq, Nk, D, scale, causal, stream);
}

size_t fa_decode_workspace_bytes(int B, int H, int D, int num_splits) {
    if (B < 0 || H < 0 || num_splits < 1 || (D != 64 && D != 128)) return 0;
    return (size_t)B * H * num_splits * (D + 2) * sizeof(float);
}

}  // extern "C"

namespace {

fa_status decode_impl(const void* Q, const void* K, const void* V, void* O, float* LSE, const int* kv_lens,
                      void* workspace, size_t workspace_bytes, int B, int H, int Nk, int D, float scale,
                      int num_splits, hipStream_t stream, bool f16) {
    if (B < 0 || H < 0 || Nk < 0 || num_splits < 1) return FA_ERR_INVALID_ARG;
    if (!good_scale(scale)) return FA_ERR_INVALID_ARG;
    if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
    if ((long long)B * H == 0) return FA_OK;
    if (Nk < 1) return FA_ERR_INVALID_ARG;
    if (!Q || !K || !V || !O || !workspace) return FA_ERR_INVALID_ARG;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(workspace))
        return FA_ERR_INVALID_ARG;
    if (LSE && !aligned4(LSE)) return FA_ERR_INVALID_ARG;
    if ((long long)B * H * num_splits > INT_MAX) return FA_ERR_UNSUPPORTED;
    const size_t need = fa_decode_workspace_bytes(B, H, D, num_splits);
    if (workspace_bytes < need) return FA_ERR_INVALID_ARG;
    const size_t bytes_q = (size_t)B * H * D * 2;
    const size_t bytes_kv = (size_t)B * H * Nk * D * 2;
    if (overlaps(O, bytes_q, Q, bytes_q) || overlaps(O, bytes_q, K, bytes_kv) ||
        overlaps(O, bytes_q, V, bytes_kv) || overlaps(O, bytes_q, LSE, (size_t)B * H * 4) ||
        overlaps(workspace, need, Q, bytes_q) || overlaps(workspace, need, K, bytes_kv) ||
        overlaps(workspace, need, V, bytes_kv) || overlaps(workspace, need, O, bytes_q) ||
        overlaps(workspace, need, LSE, (size_t)B * H * 4))
        return FA_ERR_INVALID_ARG;
    if (!good_kv_lens(kv_lens, B, O, bytes_q, LSE, (size_t)B * H * 4) ||
        overlaps(kv_lens, (size_t)B * 4, workspace, need))
        return FA_ERR_INVALID_ARG;
    float* ws_o = static_cast<float*>(workspace);
    float* ws_ml = ws_o + (size_t)B * H * num_splits * D;
    fa::DecodeArgs a{Q, K, V, O, LSE, ws_o, ws_ml, kv_lens, B, H, Nk, D, num_splits, scale, stream};
    a.f16 = f16;
    return fa::launch_decode(a) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

fa_status fa_decode_splitkv_masked(const void* Q, const void* K, const void* V, void* O, float* LSE,
                                   const int* kv_lens, void* workspace, size_t workspace_bytes, int B, int H,
                                   int Nk, int D, float scale, int num_splits, hipStream_t stream) {
    return decode_impl(Q, K, V, O, LSE, kv_lens, workspace, workspace_bytes, B, H, Nk, D, scale, num_splits,
                       stream, false);
}

fa_status fa_decode_splitkv_f16_masked(const void* Q, const void* K, const void* V, void* O, float* LSE,
                                       const int* kv_lens, void* workspace, size_t workspace_bytes, int B, int H,
                                       int Nk, int D, float scale, int num_splits, hipStream_t stream) {
    return decode_impl(Q, K, V, O, LSE, kv_lens, workspace, workspace_bytes, B, H, Nk, D, scale, num_splits,
                       stream, true);
}

fa_status fa_decode_splitkv_f16(const void* Q, const void* K, const void* V, void* O, float* LSE,
                                void* workspace, size_t workspace_bytes, int B, int H, int Nk, int D,
                                float scale, int num_splits, hipStream_t stream) {
    return decode_impl(Q, K, V, O, LSE, nullptr, workspace, workspace_bytes, B, H, Nk, D, scale, num_splits,
                       stream, true);
}

fa_status fa_decode_splitkv(const void* Q, const void* K, const void* V, void* O, float* LSE,
                            void* workspace, size_t workspace_bytes, int B, int H, int Nk, int D,
                            float scale, int num_splits, hipStream_t stream) {
    return fa_decode_splitkv_masked(Q, K, V, O, LSE, nullptr, workspace, workspace_bytes, B, H, Nk, D, scale,
                                    num_splits, stream);
}

fa_status fa_decode_splitkv_noalloc(const void* Q, const void* K, const void* V, void* O, float* LSE, int B,
                                    int H, int Nk, int D, float scale, int num_splits, hipStream_t stream) {
    if (B < 0 || H < 0 || Nk < 0 || num_splits < 1) return FA_ERR_INVALID_ARG;
    if (!good_scale(scale)) return FA_ERR_INVALID_ARG;
    if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
    if ((long long)B * H == 0) return FA_OK;
    // The partial states must fit the fixed scratch; checked before any HIP call.
    if (fa_decode_workspace_bytes(B, H, D, num_splits) > FA_DECODE_NOALLOC_SCRATCH_BYTES) return FA_ERR_UNSUPPORTED;
    if (!Q || !K || !V || !O || Nk < 1) return FA_ERR_INVALID_ARG;
    void* scratch = nullptr;
    if (fa::decode_scratch(&scratch) != hipSuccess) return FA_ERR_LAUNCH;
    return decode_impl(Q, K, V, O, LSE, nullptr, scratch, FA_DECODE_NOALLOC_SCRATCH_BYTES, B, H, Nk, D, scale,
                       num_splits, stream, false);
}

size_t fa_backward_workspace_bytes(int B, int H, int Nq) {
    if (B < 0 || H < 0 || Nq < 0) return 0;
    return (size_t)B * H * Nq * sizeof(float);
}

}  // extern "C"

namespace {

fa_status backward_impl(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                        const float* LSE, const int* kv_lens, void* dQ, void* dK, void* dV, void* workspace,
                        size_t workspace_bytes, int B, int H, int Nq, int Nk, int D, float scale, int causal,
                        hipStream_t stream, bool f16) {
    if (B < 0 || H < 0 || Nq < 0 || Nk < 0) return FA_ERR_INVALID_ARG;
    if (!good_scale(scale) || !good_causal(causal)) return FA_ERR_INVALID_ARG;
    if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
    if ((long long)B * H == 0 || ((long long)Nq == 0 && Nk == 0)) return FA_OK;
    if (Nk < 1) return FA_ERR_INVALID_ARG;
    const long long nkb = ((long long)Nk + fa::BM_BWD - 1) / fa::BM_BWD;
    if ((long long)B * H * nkb > INT_MAX) return FA_ERR_UNSUPPORTED;
    const size_t bkv = (size_t)B * H * Nk * D * 2;
    if (Nq == 0) {
        // No query reads any key: dK = dV = 0 (only K, V, dK, dV are used).
        if (!dK || !dV || !aligned16(dK) || !aligned16(dV)) return FA_ERR_INVALID_ARG;
        if (overlaps(dK, bkv, dV, bkv) || overlaps(dK, bkv, K, bkv) || overlaps(dK, bkv, V, bkv) ||
            overlaps(dV, bkv, K, bkv) || overlaps(dV, bkv, V, bkv))
            return FA_ERR_INVALID_ARG;
        if (!good_kv_lens(kv_lens, B, dK, bkv, dV, bkv)) return FA_ERR_INVALID_ARG;
    } else {
        if (!Q || !K || !V || !O || !dO || !LSE || !dQ || !dK || !dV || !workspace) return FA_ERR_INVALID_ARG;
        if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(dO) ||
            !aligned16(dQ) || !aligned16(dK) || !aligned16(dV) || !aligned16(workspace) || !aligned4(LSE))
            return FA_ERR_INVALID_ARG;
        const long long nqb = ((long long)Nq + fa::BM_BWD - 1) / fa::BM_BWD;
        if ((long long)B * H * nqb > INT_MAX || (long long)B * H * Nq > INT_MAX) return FA_ERR_UNSUPPORTED;
        const size_t need = fa_backward_workspace_bytes(B, H, Nq);
        if (workspace_bytes < need) return FA_ERR_INVALID_ARG;
        const size_t bq = (size_t)B * H * Nq * D * 2;
        const size_t bl = (size_t)B * H * Nq * sizeof(float);
        const void* ins[6] = {Q, K, V, O, dO, LSE};
        const size_t in_bytes[6] = {bq, bkv, bkv, bq, bq, bl};
        const void* outs[4] = {dQ, dK, dV, workspace};
        const size_t out_bytes[4] = {bq, bkv, bkv, need};
        for (int i = 0; i < 4; ++i) {
            for (int j = 0; j < 6; ++j)
                if (overlaps(outs[i], out_bytes[i], ins[j], in_bytes[j])) return FA_ERR_INVALID_ARG;
            for (int j = i + 1; j < 4; ++j)
                if (overlaps(outs[i], out_bytes[i], outs[j], out_bytes[j])) return FA_ERR_INVALID_ARG;
        }
        if (!good_kv_lens(kv_lens, B, dQ, bq, dK, bkv) || overlaps(kv_lens, (size_t)B * 4, dV, bkv) ||
            overlaps(kv_lens, (size_t)B * 4, workspace, need))
            return FA_ERR_INVALID_ARG;
    }
    fa::BwdArgs a{Q, K, V, O, dO, LSE, dQ, dK, dV, static_cast<float*>(workspace), kv_lens,
                  B, H, Nq, Nk, D, scale, causal, stream};
    a.f16 = f16;
    return fa::launch_bwd(a) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

fa_status fa_backward_masked(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                             const float* LSE, const int* kv_lens, void* dQ, void* dK, void* dV, void* workspace,
                             size_t workspace_bytes, int B, int H, int Nq, int Nk, int D, float scale,
                             int causal, hipStream_t stream) {
    return backward_impl(Q, K, V, O, dO, LSE, kv_lens, dQ, dK, dV, workspace, workspace_bytes, B, H, Nq, Nk, D,
                         scale, causal, stream, false);
}

fa_status fa_backward_f16_masked(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                                 const float* LSE, const int* kv_lens, void* dQ, void* dK, void* dV,
                                 void* workspace, size_t workspace_bytes, int B, int H, int Nq, int Nk, int D,
                                 float scale, int causal, hipStream_t stream) {
    return backward_impl(Q, K, V, O, dO, LSE, kv_lens, dQ, dK, dV, workspace, workspace_bytes, B, H, Nq, Nk, D,
                         scale, causal, stream, true);
}

fa_status fa_backward_f16(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                          const float* LSE, void* dQ, void* dK, void* dV, void* workspace,
                          size_t workspace_bytes, int B, int H, int Nq, int Nk, int D, float scale,
                          int causal, hipStream_t stream) {
    return backward_impl(Q, K, V, O, dO, LSE, nullptr, dQ, dK, dV, workspace, workspace_bytes, B, H, Nq, Nk, D,
                         scale, causal, stream, true);
}

fa_status fa_backward(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                      const float* LSE, void* dQ, void* dK, void* dV, void* workspace,
                      size_t workspace_bytes, int B, int H, int Nq, int Nk, int D, float scale,
                      int causal, hipStream_t stream) {
    return fa_backward_masked(Q, K, V, O, dO, LSE, nullptr, dQ, dK, dV, workspace, workspace_bytes, B, H, Nq,
                              Nk, D, scale, causal, stream);
}

}  // extern "C"
