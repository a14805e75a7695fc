/*
 * vc_model.h -- C ABI of the decoder-layer kernels that the end-to-end
 * draft-and-verify round runs around the attention calls of vc.h.
 *
 * The VeriCache pages ("VeriCache: Turning Lossy KV Cache into Lossless LLM
 * Inference", neuraltrendhub.com summary, "What the paper found") run the target
 * model itself twice -- on the compressed cache to draft and on the full cache to
 * verify -- and require the verified output to equal greedy full-KV decoding.  The
 * model here is a random-initialised Llama-style pre-norm decoder (RMSNorm, rotary
 * embeddings, SwiGLU feed-forward, untied vocabulary head); the pages name no model
 * for this, so its shape is a stand-in.
 *
 * Batch invariance: every kernel below computes each output row from its own input
 * row with an arithmetic order that does not depend on the number of rows M (no
 * split reductions across rows, fixed reduction trees within a row).  Together with
 * vc_verify_attn_full's fixed split size this makes a k-row verify pass reproduce,
 * bit for bit, k one-row greedy steps.
 *
 * Conventions are those of vc.h: device pointers, caller-owned memory, row-major
 * layouts, `stream` a hipStream_t as void*, host-side validation before any launch,
 * errors reported through vc_last_error().
 */
#ifndef VC_MODEL_H_
#define VC_MODEL_H_

#include "vc.h"

#ifdef __cplusplus
extern "C" {
#endif

/* C[m][n] = sum_k A[m][k] * W[n][k] (+ R[m][n] if R is not NULL).
 * A bf16 [M, K] with row stride lda; W bf16 [N, K] (one row per output feature)
 * with row stride ldw; C (c_dtype VC_BF16 or VC_F32) [M, N] with row stride ldc;
 * R bf16 with the layout of C (bf16 C only; C may be R itself).  A and W 16-byte
 * aligned, lda and ldw multiples of 8, K % 32 == 0.
 *
 * Batch invariant: k is cut into 8 slices fixed by K alone; each slice is summed in
 * float32 in ascending 32-wide steps on bf16 matrix cores and the 8 partial sums
 * are added in a fixed tree, then the residual (float32) and one rounding to the
 * output type -- so row m's result is the same for any M and any position of the
 * row in A.  Built for few rows (decode and verify steps stream W once). */
vc_status vc_gemm_bf16(const void* A, int64_t lda, const void* W, int64_t ldw, int64_t M, int32_t N, int32_t K,
                       void* C, int64_t ldc, int32_t c_dtype, const void* R, void* stream);

/* The gate/up projection of a SwiGLU block fused with the activation:
 * act[m][j] = vc_swiglu of the bf16-rounded products (gate j, up j) of A[m], equal bit
 * for bit to vc_gemm_bf16 into a [M, 2F] buffer followed by vc_swiglu, with one launch
 * and no intermediate.  W bf16 [2F, K] holds the gate and up rows interleaved in
 * blocks of 8: rows 16j .. 16j + 7 are gate rows 8j .. 8j + 7 and rows 16j + 8 ..
 * 16j + 15 the up rows 8j .. 8j + 7.  act bf16 [M, F] with row stride ld_act;
 * F % 8 == 0; other arguments and errors as vc_gemm_bf16. */
vc_status vc_gemm_bf16_swiglu(const void* A, int64_t lda, const void* W, int64_t ldw, int64_t M, int32_t F, int32_t K,
                              void* act, int64_t ld_act, void* stream);

/* The QKV projection fused with vc_rope_qkv: the rows A [B*k, K] are projected by W
 * and the result is rotated and scattered exactly as vc_rope_qkv does it with the
 * bf16-rounded product (same outputs, same arguments, bit for bit), with one launch
 * and no intermediate.  W bf16 [(Hq + 2 Hkv) hd, K] is the projection with the rows
 * of each q and k head permuted in tiles of 16: rows (16 t .. 16 t + 7) of a head
 * are its elements 8 t .. 8 t + 7 and rows 16 t + 8 .. 16 t + 15 the elements
 * hd/2 + 8 t .. hd/2 + 8 t + 7 (the rotation partners); the v rows keep their order.
 * hd % 16 == 0, K % 32 == 0; A and W 16-byte aligned, lda, ldw multiples of 8. */
vc_status vc_gemm_bf16_rope(const void* A, int64_t lda, const void* W, int64_t ldw, int32_t B, int32_t k, int32_t K,
                            int32_t Hq, int32_t Hkv, int32_t hd, float theta, const int32_t* pos, void* q_out,
                            void* k_dst, void* v_dst, int64_t dst_rows, const int32_t* row0, void* stream);

/* The same product for many rows (prompt processing): k summed in one ascending
 * pass per output, so its rounding differs from vc_gemm_bf16's.  Same arguments
 * and requirements. */
vc_status vc_gemm_bf16_wide(const void* A, int64_t lda, const void* W, int64_t ldw, int64_t M, int32_t N, int32_t K,
                            void* C, int64_t ldc, int32_t c_dtype, const void* R, void* stream);

/* y[m] = x[m] / sqrt(mean_j x[m][j]^2 + eps) * w, x and y bf16 [M, d], w bf16 [d];
 * d % 8 == 0, x, w, y 16-byte aligned (VC_ERR_INVALID_ARG otherwise).  float32
 * arithmetic, fixed per-row reduction order. */
vc_status vc_rmsnorm(const void* x, const void* w, int64_t M, int32_t d, float eps, void* y, void* stream);

/* Rotary embedding of the q and k parts of a fused projection and scatter into the
 * attention layouts.  qkv bf16 [B*k, (Hq + 2 Hkv) * hd], row b*k + i holding token i
 * of sequence b at position pos[b*k + i] (int32, device).  Pairs (j, j + hd/2) of each
 * head are rotated by pos * theta^(-2j/hd) (float32 angle, float64-accurate sin/cos
 * not required).  Outputs: q_out bf16 [B, Hq, k, hd]; the (rotated) k and the v parts
 * are written to rows row0[b] + i of k_dst, v_dst bf16 [B, Hkv, dst_rows, hd]
 * (row0 int32 [B], device).  Every row0[b] + k must be <= dst_rows; the kernel
 * skips key/value rows that fall outside [0, dst_rows) rather than write them. */
vc_status vc_rope_qkv(const void* qkv, int32_t B, int32_t k, int32_t Hq, int32_t Hkv, int32_t hd, float theta,
                      const int32_t* pos, void* q_out, void* k_dst, void* v_dst, int64_t dst_rows,
                      const int32_t* row0, void* stream);

/* out[m][j] = silu(gu[m][j]) * gu[m][F + j], gu bf16 [M, 2F], out bf16 [M, F]. */
vc_status vc_swiglu(const void* gu, int64_t M, int32_t F, void* out, void* stream);

/* x[m] = E[tokens[m]], E bf16 [V, d], tokens int32 [M] (each in [0, V); a row whose
 * token is outside that range is written as zeros), x bf16 [M, d]. */
vc_status vc_embed(const void* E, int32_t V, int32_t d, const int32_t* tokens, int64_t M, void* x, void* stream);

/* [B, H, k, hd] -> [B*k, H*hd] (bf16): attention output rows for the next projection. */
vc_status vc_heads_to_rows(const void* o, int32_t B, int32_t H, int32_t k, int32_t hd, void* out, void* stream);

/* tokens[r] = argmax_v logits[r][v] (float32 [R, V]); equal maxima go to the lowest v. */
vc_status vc_argmax_rows(const float* logits, int64_t R, int32_t V, int32_t* tokens, void* stream);

/* Per-sequence row copies between two caches of layout [B, Hkv, rows, d] (elem_bytes
 * per element, 16-byte multiple rows): for each sequence b, rows
 * [src_row0[b], src_row0[b] + count[b]) of src_k/src_v go to rows
 * [dst_row0[b], dst_row0[b] + count[b]) of dst_k/dst_v.  src_row0, dst_row0, count
 * int32 [B] (device); count[b] <= max_count (rows past max_count are not copied);
 * all rows must lie in their caches (the kernel skips rows that do not).  Source
 * and destination ranges must not overlap. */
vc_status vc_copy_kv_rows(const void* src_k, const void* src_v, int64_t src_rows, const int32_t* src_row0,
                          void* dst_k, void* dst_v, int64_t dst_rows, const int32_t* dst_row0,
                          const int32_t* count, int32_t max_count, int32_t B, int32_t Hkv, int32_t d,
                          int32_t elem_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VC_MODEL_H_ */
