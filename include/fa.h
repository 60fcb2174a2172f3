/*
 * fa.h — C ABI of the MI355X (gfx950) FlashAttention library: forward pass,
 * split-KV decode and backward pass.
 *
 * The operation (the same for every entry point) is exact softmax attention
 *     O[b,h,i,:] = sum_j softmax_j(scale * Q[b,h,i,:] . K[b,h,j,:]) * V[b,h,j,:]
 * computed without materialising the score matrix: a tile of queries stays on
 * chip while tiles of keys/values stream past it, and each query row carries a
 * running maximum m, a running denominator l and an unnormalised accumulator
 * O that is rescaled by exp(m_old - m_new) whenever the maximum grows; O is
 * divided by l once at the end. Sources: "11. Fusion, recompute, and flash
 * attention" (ML compiler from scratch), sections 11.2, 11.6 and 11.9; the
 * iThome FlashAttention article, section on the three running states; "Kernel
 * visualization: Flash Attention 2", sections "Set up pointers and shared
 * memory" and "Write the data back to HBM".
 *
 * Conventions shared by every call:
 *   - All tensor pointers are DEVICE pointers owned by the caller. The library
 *     never allocates, frees, synchronises or prints. Every call only enqueues
 *     kernels on `stream` (0 = the null stream) and returns.
 *   - Layout is contiguous row-major [B, H, N, D] (head dimension fastest);
 *     LSE is contiguous [B, H, Nq] fp32. Pointers must be 16-byte aligned.
 *   - bf16 means IEEE bfloat16 stored as 16-bit words; outputs are rounded to
 *     nearest-even. Accumulation, m and l are fp32.
 *   - LSE (may be NULL to skip it) is the natural-log log-sum-exp of the
 *     scaled scores of the row, m + ln(l), the per-row value the FA2 write-back
 *     step stores beside O for a backward pass.
 *   - scale must be finite and > 0 (the pages use 1/sqrt(D)).
 *   - D (head dimension) must be 64 or 128.
 *   - O must not overlap Q, K, V or LSE; inputs are never written.
 *   - Sizes: B, H, Nq >= 0 (a zero size is a no-op returning FA_OK); Nk >= 1.
 *   - Errors are reported before anything is enqueued, except FA_ERR_LAUNCH,
 *     which reports hipGetLastError() after the launch. Calls are stateless and
 *     thread-safe.
 *   - causal is one of fa_causal below; any other value is FA_ERR_INVALID_ARG.
 *   - The *_masked variants add kv_lens: NULL, or a DEVICE array of B int32
 *     giving the number of real keys of each batch entry; keys j >= kv_lens[b]
 *     are padding and never attended (the padding masks of the Pitfalls
 *     passage of the ML compiler page). Values are clamped to [0, Nk] on the
 *     device (the library cannot read device memory before enqueueing).
 *     kv_lens must be 4-byte aligned and must not overlap any output. Without
 *     kv_lens every batch entry has Nk real keys.
 *   - A query row that may attend no key at all (kv_lens[b] = 0, or the first
 *     Nq - Lk rows under bottom-right alignment) has no softmax; it is written
 *     as the empty sums the definition reduces to: O = 0 and LSE = -inf, and
 *     its backward contributions are zero (the Pitfalls passage: such rows
 *     must not produce NaN).
 *   - NaN inputs: a NaN in a query row, or in a key row that row attends,
 *     makes the row's softmax NaN, so its O and LSE are NaN; no other row
 *     changes. A NaN in column c of a value row makes column c of O NaN in
 *     every row that attends it, and may also reach column c of a row that
 *     masks that key causally but reads its key tile (the masked weight is
 *     an exact zero, and 0 * NaN is NaN); the LSE and the other columns never
 *     change. Padding keys (past kv_lens[b]) are never read.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Causal alignment. With Lk real keys (kv_lens[b], else Nk):
 *   FA_CAUSAL_NONE:         every real key;
 *   FA_CAUSAL_TOP_LEFT:     key j <= i (absolute indices from the first key,
 *                           the rule of the exercise "Causal mask" on the ML
 *                           compiler page and of phobos' causal_attention);
 *   FA_CAUSAL_BOTTOM_RIGHT: key j <= i + (Lk - Nq), the last query aligned
 *                           with the last real key (the queries are the newest
 *                           Nq tokens); equal to top-left when Nq == Lk. */
typedef enum fa_causal {
    FA_CAUSAL_NONE = 0,
    FA_CAUSAL_TOP_LEFT = 1,
    FA_CAUSAL_BOTTOM_RIGHT = 2
} fa_causal;

/* Element type of the 16-bit entry points that take one (fa_rope, fa_forward_rope). */
typedef enum fa_dtype {
    FA_DTYPE_BF16 = 0,
    FA_DTYPE_F16 = 1
} fa_dtype;

/* RoPE forms of the phobos page ("Rotary position embeddings"): rope, the
 * rotate-half form of GPT-NeoX / LLaMA (halves a, b of a row become
 * a cos - b sin, b cos + a sin), and rope_pairs, GPT-J's adjacent pairs
 * (x[2i], x[2i+1]) rotated the same way by angle i. */
typedef enum fa_rope_style {
    FA_ROPE_HALF = 0,
    FA_ROPE_PAIRS = 1
} fa_rope_style;

typedef enum fa_status {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, bad size, bad scale, workspace too small */
    FA_ERR_UNSUPPORTED = 2,   /* D not in {64, 128}, or a problem too large for the launch grid */
    FA_ERR_LAUNCH = 3         /* the HIP runtime rejected a kernel launch */
} fa_status;

/*
 * Prefill / full forward pass, bf16 in and out.
 *   Q: bf16 [B,H,Nq,D]; K, V: bf16 [B,H,Nk,D]; O: bf16 [B,H,Nq,D] (written);
 *   LSE: fp32 [B,H,Nq] (written) or NULL.
 *   causal: an fa_causal value; keys past Nk are never attended (the masked
 *   last block of phobos' attention).
 * Score and PV products use bf16 MFMA with fp32 accumulation; P is rounded to
 * bf16 before the PV product.
 */
fa_status fa_forward(const void* Q, const void* K, const void* V,
                     void* O, float* LSE,
                     int B, int H, int Nq, int Nk, int D,
                     float scale, int causal, hipStream_t stream);

/* fa_forward with key padding: kv_lens as in the conventions above. */
fa_status fa_forward_masked(const void* Q, const void* K, const void* V,
                            void* O, float* LSE, const int* kv_lens,
                            int B, int H, int Nq, int Nk, int D,
                            float scale, int causal, hipStream_t stream);

/*
 * The same operation with IEEE fp16 inputs and output (the f16 tensors of
 * phobos' flash_attention kernel): fp16 MFMA with fp32 accumulation, P rounded
 * to fp16 (round to nearest even) before the PV product, O rounded to fp16.
 * Arguments as fa_forward / fa_forward_masked.
 */
fa_status fa_forward_f16(const void* Q, const void* K, const void* V,
                         void* O, float* LSE,
                         int B, int H, int Nq, int Nk, int D,
                         float scale, int causal, hipStream_t stream);
fa_status fa_forward_f16_masked(const void* Q, const void* K, const void* V,
                                void* O, float* LSE, const int* kv_lens,
                                int B, int H, int Nq, int Nk, int D,
                                float scale, int causal, hipStream_t stream);

/*
 * Rotary position embedding of every row of X [B,H,N,D] (bf16 or fp16 per
 * dtype) into Y: row n of each (b, h) is rotated by the angles of position n,
 * cos[n, :] and sin[n, :] (fp32 [n_pos, D/2] tables, n_pos >= N, 16-byte
 * aligned), in the given style. fp32 arithmetic, result rounded to the
 * element type (nearest even). Y == X (in place) is allowed; any other
 * overlap is not.
 */
fa_status fa_rope(const void* X, void* Y, const float* cos, const float* sin,
                  int n_pos, int style, int dtype,
                  int B, int H, int N, int D, hipStream_t stream);

/* Bytes of workspace fa_forward_rope needs: B*H*Nk*D*2 (the rotated K). */
size_t fa_rope_workspace_bytes(int B, int H, int Nk, int D);

/*
 * Forward pass with a fused RoPE prologue: O = softmax(rope(Q) rope(K)^T *
 * scale) V (phobos page, "Rotary position embeddings", applied to the Q and K
 * of its flash_attention). Key j has position j; query row i has position i,
 * or i + (Lk - Nq) with FA_CAUSAL_BOTTOM_RIGHT (the queries are the newest
 * tokens), clamped at 0 for rows that see no key. Q is rotated in registers
 * inside the attention kernel; K is rotated once into `workspace` by the RoPE
 * kernel (every K tile is read by every query block of its head, so rotating
 * it in the key loop would repeat the work) and read from there. The rotated
 * Q and K are rounded to the element type before the score product, as a
 * separate RoPE pass writing that type would.
 *   Q, K, V, O: dtype [B,H,N,D] as fa_forward / fa_forward_f16; LSE, kv_lens,
 *   causal as fa_forward_masked; cos, sin: fp32 [n_pos, D/2], n_pos >= Nq and
 *   >= Nk; workspace: >= fa_rope_workspace_bytes(B,H,Nk,D) bytes of device
 *   memory, contents undefined on return, not shared by calls that overlap in
 *   time. Two kernels run on `stream`.
 */
fa_status fa_forward_rope(const void* Q, const void* K, const void* V,
                          void* O, float* LSE, const int* kv_lens,
                          const float* cos, const float* sin, int n_pos, int style, int dtype,
                          void* workspace, size_t workspace_bytes,
                          int B, int H, int Nq, int Nk, int D,
                          float scale, int causal, hipStream_t stream);

/*
 * The same operation in fp32 end to end (fp32 inputs, fp32 arithmetic, fp32
 * O), as the FA2 kernel sketch on "Kernel visualization: Flash Attention 2"
 * computes it. Arguments as fa_forward.
 */
fa_status fa_forward_f32(const float* Q, const float* K, const float* V,
                         float* O, float* LSE,
                         int B, int H, int Nq, int Nk, int D,
                         float scale, int causal, hipStream_t stream);

/* fa_forward_f32 with key padding: kv_lens as in the conventions above. */
fa_status fa_forward_f32_masked(const float* Q, const float* K, const float* V,
                                float* O, float* LSE, const int* kv_lens,
                                int B, int H, int Nq, int Nk, int D,
                                float scale, int causal, hipStream_t stream);

/*
 * Bytes of device workspace fa_decode_splitkv needs: B*H*num_splits*(D+2)*4
 * (one fp32 partial state (m, l, o[D]) per head and key chunk). Returns 0 for
 * invalid arguments.
 */
size_t fa_decode_workspace_bytes(int B, int H, int D, int num_splits);

/*
 * Flash-decoding: one query token per (b, h) over a whole key/value cache,
 * no mask ("Flash-decoding" exercise on the ML compiler page). The Nk keys are
 * split into num_splits chunks of c = ceil(Nk / num_splits) keys (chunk s is
 * [s*c, min(Nk, (s+1)*c)); trailing chunks may be empty). A first kernel
 * reduces each chunk to a partial (m, l, o) in `workspace`; a second kernel on
 * the same stream merges the partials of each (b, h) with the rule of section
 * 11.6 and writes O and LSE.
 *   Q: bf16 [B,H,1,D]; K, V: bf16 [B,H,Nk,D]; O: bf16 [B,H,1,D];
 *   LSE: fp32 [B,H] or NULL;
 *   workspace: caller-owned device memory of at least
 *   fa_decode_workspace_bytes(B,H,D,num_splits) bytes (workspace_bytes says
 *   how much was passed); its contents on entry are ignored and are left
 *   undefined. Calls that overlap in time must not share a workspace.
 *   num_splits >= 1.
 */
fa_status fa_decode_splitkv(const void* Q, const void* K, const void* V,
                            void* O, float* LSE,
                            void* workspace, size_t workspace_bytes,
                            int B, int H, int Nk, int D,
                            float scale, int num_splits, hipStream_t stream);

/*
 * fa_decode_splitkv over caches of different lengths: batch entry b attends
 * its first Lk = kv_lens[b] keys (kv_lens as in the conventions above), split
 * into num_splits chunks of ceil(Lk / num_splits) keys. Lk = 0 gives O = 0,
 * LSE = -inf. kv_lens must not overlap the workspace either.
 */
fa_status fa_decode_splitkv_masked(const void* Q, const void* K, const void* V,
                                   void* O, float* LSE, const int* kv_lens,
                                   void* workspace, size_t workspace_bytes,
                                   int B, int H, int Nk, int D,
                                   float scale, int num_splits, hipStream_t stream);

/* fa_decode_splitkv and fa_decode_splitkv_masked for fp16 Q, K, V and O. */
fa_status fa_decode_splitkv_f16(const void* Q, const void* K, const void* V,
                                void* O, float* LSE,
                                void* workspace, size_t workspace_bytes,
                                int B, int H, int Nk, int D,
                                float scale, int num_splits, hipStream_t stream);
fa_status fa_decode_splitkv_f16_masked(const void* Q, const void* K, const void* V,
                                       void* O, float* LSE, const int* kv_lens,
                                       void* workspace, size_t workspace_bytes,
                                       int B, int H, int Nk, int D,
                                       float scale, int num_splits, hipStream_t stream);

/*
 * fa_decode_splitkv without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). The partial states live in a fixed scratch
 * array inside the library, FA_DECODE_NOALLOC_SCRATCH_BYTES bytes per GPU,
 * held from the first call on a device until the process ends; the call
 * itself allocates nothing. Arguments, results and errors as
 * fa_decode_splitkv (bf16), plus:
 *   - FA_ERR_UNSUPPORTED when fa_decode_workspace_bytes(B,H,D,num_splits)
 *     exceeds FA_DECODE_NOALLOC_SCRATCH_BYTES (checked before any HIP call);
 *   - FA_ERR_LAUNCH when the scratch's device address cannot be looked up.
 *   - `stream` must belong to the calling thread's current device, whose copy
 *     of the scratch is used.
 * Every call on one GPU shares that GPU's scratch: calls that may overlap in
 * time on one GPU (on different streams, or from different threads) race and
 * must be serialised by the caller. Nothing in the scratch needs clearing:
 * every call overwrites all the partial states it reads.
 */
#define FA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
fa_status fa_decode_splitkv_noalloc(const void* Q, const void* K, const void* V,
                                    void* O, float* LSE,
                                    int B, int H, int Nk, int D,
                                    float scale, int num_splits, hipStream_t stream);

/*
 * Bytes of device workspace fa_backward needs: B*H*Nq*4 (one fp32 value per
 * query row, D_i = sum_d dO[i,d] * O[i,d]). Returns 0 for invalid arguments.
 */
size_t fa_backward_workspace_bytes(int B, int H, int Nq);

/*
 * Backward pass with recompute: the gradients dQ, dK, dV of a loss whose
 * gradient with respect to O is dO, for the forward pass fa_forward computed
 * ("Backward with recompute" exercise and section 11.9 of the ML compiler
 * page: only O and the per-row log-sum-exp are kept from the forward pass;
 * the probabilities are recomputed block by block as P = exp(S - LSE)).
 *     dV = P^T dO,   dP = dO V^T,   D_i = sum_d dO[i,d] O[i,d],
 *     dS = P * (dP - D),   dQ = scale * dS K,   dK = scale * dS^T Q.
 *   Q, O, dO: bf16 [B,H,Nq,D]; K, V: bf16 [B,H,Nk,D]; LSE: fp32 [B,H,Nq], the
 *   natural-log values fa_forward wrote for the same Q, K, V, scale and causal
 *   (required, not NULL); dQ: bf16 [B,H,Nq,D]; dK, dV: bf16 [B,H,Nk,D]
 *   (written; fully overwritten).
 *   workspace: caller-owned device memory of at least
 *   fa_backward_workspace_bytes(B,H,Nq) bytes (holds D); contents on entry
 *   ignored, left undefined. Calls that overlap in time must not share it.
 *   scale, causal, D, sizes and alignment as fa_forward. dQ, dK, dV must not
 *   overlap each other, any input or the workspace.
 *   B*H == 0, or Nq == Nk == 0: nothing to do, FA_OK. Nq == 0 < Nk: no query
 *   reads a key, so dK and dV are set to zero and only K, V, dK, dV are
 *   looked at. Nk == 0 < Nq: FA_ERR_INVALID_ARG (the forward pass is
 *   undefined there).
 * Products use bf16 MFMA with fp32 accumulation; P and dS are rounded to bf16
 * before the products that consume them. Two kernels run on `stream`: dQ
 * (which also forms D and stores it in the workspace), then dK and dV.
 */
fa_status fa_backward(const void* Q, const void* K, const void* V,
                      const void* O, const void* dO, const float* LSE,
                      void* dQ, void* dK, void* dV,
                      void* workspace, size_t workspace_bytes,
                      int B, int H, int Nq, int Nk, int D,
                      float scale, int causal, hipStream_t stream);

/*
 * fa_backward with key padding (kv_lens as in the conventions above; pass the
 * kv_lens and causal of the forward call). Padding keys get dK = dV = 0; rows
 * with no visible key (LSE = -inf) get dQ = 0 and contribute nothing.
 * kv_lens must not overlap dQ, dK, dV or the workspace.
 */
fa_status fa_backward_masked(const void* Q, const void* K, const void* V,
                             const void* O, const void* dO, const float* LSE,
                             const int* kv_lens,
                             void* dQ, void* dK, void* dV,
                             void* workspace, size_t workspace_bytes,
                             int B, int H, int Nq, int Nk, int D,
                             float scale, int causal, hipStream_t stream);

/* fa_backward and fa_backward_masked for fp16 inputs and gradients (the O and
 * LSE of fa_forward_f16 / fa_forward_f16_masked); fp16 MFMA, P and dS rounded
 * to fp16. */
fa_status fa_backward_f16(const void* Q, const void* K, const void* V,
                          const void* O, const void* dO, const float* LSE,
                          void* dQ, void* dK, void* dV,
                          void* workspace, size_t workspace_bytes,
                          int B, int H, int Nq, int Nk, int D,
                          float scale, int causal, hipStream_t stream);
fa_status fa_backward_f16_masked(const void* Q, const void* K, const void* V,
                                 const void* O, const void* dO, const float* LSE,
                                 const int* kv_lens,
                                 void* dQ, void* dK, void* dV,
                                 void* workspace, size_t workspace_bytes,
                                 int B, int H, int Nq, int Nk, int D,
                                 float scale, int causal, hipStream_t stream);

/* Static, human-readable name of a status code (never NULL). */
const char* fa_status_string(fa_status s);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
