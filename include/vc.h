/*
 * vc.h -- C ABI of the VeriCache draft-and-verify hot path for AMD Instinct
 * MI355X (gfx950).
 *
 * The operations follow "VeriCache: Turning Lossy KV Cache into Lossless LLM
 * Inference" (neuraltrendhub.com summary, "What the paper found" and "Original
 * abstract"; the same abstract on the pith.science record of arXiv 2605.17613):
 * the target model drafts tokens with a compressed KV cache (quantization or token
 * dropping behind one compressor interface), the full KV cache is kept off the GPU
 * and swapped in, the drafted window is verified against the full KV cache, and
 * only the prefix that greedy full-KV decoding would also produce is committed.
 *
 * Conventions shared by every call
 * ---------------------------------
 * - Pointers named host_* are host memory (pinned, from hipHostMalloc or a
 *   pinned torch tensor); every other data pointer is device memory on the
 *   current HIP device.  The caller owns all memory; the library never allocates
 *   or frees and keeps no per-call state beyond the thread-local error message,
 *   except inside a vc_file_stager, which owns its threads and pinned buffers.
 * - Tensors are dense, row-major, with the shapes given in each comment (last
 *   index fastest).  Element types: VC_F32 = IEEE float32, VC_BF16 = bfloat16,
 *   int32/uint32 where stated.
 * - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Every
 *   call only enqueues work on it and returns; nothing synchronizes the host.
 * - Workspace (`ws`, `ws_bytes`): device scratch sized by the matching
 *   *_workspace_bytes call.  It must be zero-filled once before its first use;
 *   every call leaves it zero-filled again, so the same workspace can be reused by
 *   calls that do not overlap in time.  Calls that run concurrently need separate
 *   workspaces.
 * - Errors: arguments are validated on the host before anything is enqueued.  A
 *   bad argument returns VC_ERR_INVALID_ARG (or VC_ERR_UNSUPPORTED for a legal but
 *   unimplemented combination, VC_ERR_WORKSPACE for a short workspace) with no
 *   side effect.  A HIP launch or copy failure returns VC_ERR_HIP, a failed file
 *   read VC_ERR_IO.  The message of
 *   the last failure on the calling thread is returned by vc_last_error().  No
 *   C++ exception crosses this interface.
 */
#ifndef VC_H_
#define VC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VC_OK = 0,
  VC_ERR_INVALID_ARG = 1,
  VC_ERR_UNSUPPORTED = 2,
  VC_ERR_WORKSPACE = 3,
  VC_ERR_HIP = 4,
  VC_ERR_IO = 5
} vc_status;

typedef enum { VC_F32 = 0, VC_BF16 = 1 } vc_dtype;

/* Compressor families behind the uniform interface (summary page, "What the paper
 * found": one interface over token-dropping and quantization methods). */
typedef enum { VC_QUANT_KIVI = 1, VC_DROP_TOPK = 2 } vc_method;

/*
 * Compressed KV cache of one attention layer, for B sequences x Hkv KV heads of
 * head dimension d.  A descriptor of caller-owned device arrays.
 *
 * VC_QUANT_KIVI -- KIVI-style asymmetric group quantization (episode page, source
 * 4): K per channel (a group is `group` consecutive tokens of one channel), V per
 * token (a group is `group` consecutive channels of one token); per group
 * s = fl32(max - min) / (2^bits - 1) and z = min, both stored as param_dtype;
 * code = clamp(rint_half_even((x - z) / s), 0, 2^bits - 1) in float32, all codes
 * 0 when s == 0; dequantized value z + code * s.
 *   k_codes  uint32 [B, Hkv, capacity, d*k_bits/32]   packed rows (see below)
 *   v_codes  uint32 [B, Hkv, capacity, d*v_bits/32]
 *   k_scale, k_zero  param_dtype [B, Hkv, capacity/group, d]
 *   v_scale, v_zero  param_dtype [B, Hkv, capacity, d/group]
 *   Packing: each token row of d codes is one little-endian bitstream, code c at
 *   bits bits*c .. bits*c+bits-1, uint32 word w holding bits 32w .. 32w+31 (3-bit
 *   codes straddle words).  bits in {2, 3, 4, 8, 16}; d*bits % 32 == 0.
 *
 * VC_DROP_TOPK -- token dropping by accumulated attention (episode page, source 3,
 * H2O): rows kept unchanged, addressed by their source positions.
 *   k_kept, v_kept  kv_dtype [B, Hkv, capacity, d]
 *   kept_idx        int32 [B, Hkv, capacity], ascending source token positions
 *
 * Both: a full-precision tail appended after the compressed rows (recent tokens
 * that do not yet fill a quantization group, and the current draft tokens):
 *   tail_k, tail_v  kv_dtype [B, Hkv, tail_cap, d]
 *
 * Live lengths: n_main compressed rows and tail_len tail rows for every sequence,
 * unless per-sequence device arrays are passed to the call that reads them.
 */
typedef struct {
  int32_t method;       /* vc_method */
  int32_t k_bits;       /* quantization: bits per K code */
  int32_t v_bits;       /* quantization: bits per V code */
  int32_t group;        /* quantization: group size (tokens for K, channels for V) */
  int32_t param_dtype;  /* vc_dtype of scales and zero-points */
  int32_t kv_dtype;     /* vc_dtype of keys, values, queries, outputs, tail, kept rows */
  float keep_ratio;     /* token dropping: fraction of tokens kept, in (0, 1] */
  int32_t B, Hkv, d;
  int64_t capacity;     /* compressed rows allocated per (sequence, kv-head) */
  int64_t n_main;       /* live compressed rows (or their maximum, see above) */
  uint32_t* k_codes;
  uint32_t* v_codes;
  void* k_scale;
  void* k_zero;
  void* v_scale;
  void* v_zero;
  void* k_kept;
  void* v_kept;
  int32_t* kept_idx;
  void* tail_k;
  void* tail_v;
  int64_t tail_cap;
  int64_t tail_len;     /* live tail rows (or their maximum) */
  int32_t flags;        /* VC_CKV_* bits below, 0 for the defaults */
} vc_ckv;

/* vc_ckv.flags.
 * VC_CKV_DECODE_F32: vc_decode_attn_compressed keeps every operand in float32 (the
 *   generic kernel) instead of the f16 matrix-core operands of the fast path.  Set
 *   it for a quantized cache outside the f16 domain stated at that call. */
enum { VC_CKV_DECODE_F32 = 1 };

/* Arrays of a vc_ckv, in the order vc_ckv_sizes reports them. */
typedef enum {
  VC_CKV_K_CODES = 0,
  VC_CKV_V_CODES,
  VC_CKV_K_SCALE,
  VC_CKV_K_ZERO,
  VC_CKV_V_SCALE,
  VC_CKV_V_ZERO,
  VC_CKV_K_KEPT,
  VC_CKV_V_KEPT,
  VC_CKV_KEPT_IDX,
  VC_CKV_TAIL_K,
  VC_CKV_TAIL_V,
  VC_CKV_NARRAYS
} vc_ckv_array;

/* Byte size of every device array a vc_ckv descriptor points to, from its method,
 * bits, group, param_dtype, kv_dtype, B, Hkv, d, capacity and tail_cap (the layouts
 * above; the pointers and live lengths are not read).  out_bytes[VC_CKV_NARRAYS]
 * receives the sizes indexed by vc_ckv_array; arrays the method does not use are
 * 0 (the codes and parameters for VC_DROP_TOPK, the kept rows and positions for
 * VC_QUANT_KIVI), and so are the tail arrays when tail_cap is 0.  A caller
 * allocates each array with exactly this many bytes.  The uniform compressor
 * interface of the summary page ("What the paper found"): one call sizes the
 * storage of either family.  VC_ERR_INVALID_ARG for an invalid descriptor (bits
 * outside {2, 3, 4, 8, 16}, a group that does not divide d, d * bits not a
 * multiple of 32, a capacity that is not a multiple of the group, negative sizes);
 * out_bytes is then left unchanged. */
vc_status vc_ckv_sizes(const vc_ckv* ckv, size_t* out_bytes);

/* ---------------------------------------------------------------------------
 * Compression (summary page, "What the paper found": one compressor interface
 * over quantization and token dropping).
 *
 * VC_QUANT_KIVI: quantizes source rows [src_begin, src_begin + n_tokens) of every
 * (sequence, kv-head) of k_src, v_src (kv_dtype [B, Hkv, src_rows, d]) and writes
 * them as compressed rows [dst_begin, dst_begin + n_tokens).  n_tokens, src_begin
 * and dst_begin must be multiples of `group` and the rows must fit in capacity.
 * Does not change ckv->n_main (the caller tracks lengths).  probes must be NULL.
 *
 * VC_DROP_TOPK: src_begin = dst_begin = 0 and n_tokens = N source tokens.  Scores
 * every token by accumulated attention of n_probes probe queries (probes: bf16
 * [Hkv, n_probes, d], shared by the batch): score_n = sum_p softmax_n(P_p . K_n *
 * sm_scale); keeps the n_keep = ceil(keep_ratio * N) highest scores (equal scores:
 * lower position first), writes their positions ascending to kept_idx and copies
 * their K and V rows unchanged to k_kept, v_kept rows [0, n_keep).  Scores are
 * float32.  n_keep must fit in capacity.
 * ------------------------------------------------------------------------- */
vc_status vc_compress(const vc_ckv* ckv, const void* k_src, const void* v_src, int64_t src_rows,
                      int64_t src_begin, int64_t n_tokens, int64_t dst_begin,
                      const void* probes, int32_t n_probes, float sm_scale,
                      void* ws, size_t ws_bytes, void* stream);
size_t vc_compress_workspace_bytes(const vc_ckv* ckv, int64_t n_tokens, int32_t n_probes);

/* Number of rows kept by VC_DROP_TOPK for N source tokens: ceil(keep_ratio * N),
 * at least 1 and at most N. */
int64_t vc_drop_keep_count(float keep_ratio, int64_t N);

/* Token-drop pieces, exposed on their own so each can be checked separately.
 * vc_drop_scores: k bf16/f32 (kv_dtype) [B, Hkv, N, d], probes bf16 [Hkv, P, d]
 *   -> scores float32 [B, Hkv, N].
 * vc_drop_select: scores float32 [B, Hkv, N] -> kept_idx int32 [B, Hkv, n_keep]
 *   (top n_keep, ties to the lower position, ascending).  n_keep <= N.  Scores
 *   are ranked as numbers: negative scores are allowed, -0.0 equals +0.0, and a NaN
 *   ranks below every other score (NaNs among themselves by position).  ws: device
 *   memory of vc_drop_select_workspace_bytes(B, Hkv, N) bytes, any contents (the call
 *   clears what it needs; calls sharing one workspace must not overlap);
 *   VC_ERR_WORKSPACE if ws is NULL or smaller.
 * vc_gather_rows: src kv_dtype [B, Hkv, src_rows, d], idx int32 [B, Hkv, n]
 *   -> dst [B, Hkv, dst_rows, d] rows [0, n).  Every idx must be < src_rows. */
vc_status vc_drop_scores(const void* k, int32_t kv_dtype, const void* probes, int32_t B, int32_t Hkv,
                         int64_t N, int32_t d, int32_t n_probes, float sm_scale, float* scores,
                         void* ws, size_t ws_bytes, void* stream);
size_t vc_drop_scores_workspace_bytes(int32_t B, int32_t Hkv, int64_t N, int32_t n_probes);
vc_status vc_drop_select(const float* scores, int32_t B, int32_t Hkv, int64_t N, int64_t n_keep,
                         int32_t* kept_idx, void* ws, size_t ws_bytes, void* stream);
size_t vc_drop_select_workspace_bytes(int32_t B, int32_t Hkv, int64_t N);
vc_status vc_gather_rows(const void* src, int32_t kv_dtype, int32_t B, int32_t Hkv, int64_t src_rows,
                         int32_t d, const int32_t* idx, int64_t n, void* dst, int64_t dst_rows,
                         void* stream);

/* ---------------------------------------------------------------------------
 * Drafting: single-token decode attention over the compressed cache (summary
 * page, "What the paper found": drafting with the compressed KV cache is
 * HBM-bandwidth-bound).
 *
 * q kv_dtype [B, Hq, d]; q-head h reads kv-head h / (Hq / Hkv).  Each query
 * attends to the sequence's compressed rows [0, main_len) -- dequantized, or the
 * kept rows -- followed by tail rows [0, tail_len):
 *   s_n = (q . k_n) * sm_scale, o = sum_n softmax(s)_n v_n, lse = ln sum_n exp(s_n).
 * main_lens / tail_lens: device int32 [B] per-sequence lengths, or NULL to use
 * ckv->n_main / ckv->tail_len for every sequence (when given, ckv->n_main and
 * ckv->tail_len are the largest lengths of the call, and every entry is clamped
 * to [0, ckv->n_main] / [0, ckv->tail_len] on the device; for quantization main
 * lengths are multiples of the group).  A sequence with no rows at all gets o = 0 and
 * lse = -inf.  out kv_dtype [B, Hq, d]; lse float32 [B, Hq] or NULL.
 * Accumulation is float32.
 *
 * Precision.  A quantized bf16 cache with d = 128, Hq/Hkv <= 16, 2/3/4-bit K and V
 * codes, group 16, 32, 64 or 128 and a capacity that is a multiple of 32 runs on
 * matrix cores unless ckv->flags has VC_CKV_DECODE_F32: the operands q_c * sm_scale *
 * log2(e) (and its products with the K scales), the zero-points, the V scales times
 * the codes and the probabilities are rounded to f16 (11 significant bits) and the
 * products accumulate in float32; with 2- or 4-bit V codes in 64- or 128-channel
 * groups the V scale is applied to the probabilities instead, each product p * s_V
 * rounded to bf16 (8 significant bits).  Range: every |z| and 64 * s_V must be at
 * most 65504.  Accuracy: each score carries an error of about 2^-10 * sm_scale *
 * sum_c |q_c k_c| (the f16 rounding of its terms) and the output that error times
 * the spread of the values, plus about 2^-11 |v| (2^-9 |v| with the bf16 products).
 * For keys, values and queries of unit scale (N(0,1) entries, x10 on a few outlier
 * channels) that is 1e-4 to 2e-3, inside the 2e-2 bar; it grows with the square of
 * the scale and leaves the bar near twice it.  For larger activations set
 * VC_CKV_DECODE_F32 (float32 operands throughout, the generic kernel); every other
 * cache runs in float32 as well.
 * ------------------------------------------------------------------------- */
vc_status vc_decode_attn_compressed(const vc_ckv* ckv, const void* q, int32_t Hq, float sm_scale,
                                    const int32_t* main_lens, const int32_t* tail_lens,
                                    void* out, float* lse, void* ws, size_t ws_bytes, void* stream);
size_t vc_decode_workspace_bytes(const vc_ckv* ckv, int32_t Hq);

/* vc_decode_attn_compressed without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, serving loops and harnesses that forbid
 * hipMalloc.  The same kernels and splits as vc_decode_attn_compressed, so the same
 * results bit for bit; the split partials go to a device array of
 * VC_DECODE_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on,
 * from the first call on that GPU until the process ends.  The call allocates
 * nothing.  A call whose partials exceed the array -- B*Hkv*S*(Hq/Hkv)*(d + 2)*4
 * bytes plus alignment, S the call's split count (at most 64; e.g. B 8, Hkv 8, d 128,
 * 4 q-heads per kv-head and 12 splits need 1.6 MB) -- returns VC_ERR_WORKSPACE with
 * nothing enqueued.  Every call on a GPU uses the same array and nothing in it has to
 * start at zero: calls that overlap in time on one GPU (other streams, other host
 * threads) race on it and must not be issued; calls in one stream's order are fine. */
#define VC_DECODE_NOALLOC_SCRATCH_BYTES (8u << 20)
vc_status vc_decode_attn_compressed_noalloc(const vc_ckv* ckv, const void* q, int32_t Hq, float sm_scale,
                                            const int32_t* main_lens, const int32_t* tail_lens, void* out,
                                            float* lse, void* stream);

/* ---------------------------------------------------------------------------
 * Verification: causal attention of the k-row draft window over the full KV
 * (summary page, "What the paper found": verification against the full KV cache;
 * abstract: outputs identical to full-KV decoding).
 *
 * k_cache, v_cache kv_dtype [B, Hkv, cache_rows, d] hold the full cache with the
 * window's own keys/values already written at rows [L, L + k), L = the sequence's
 * context length (ctx_lens[b], or ctx_len for all when ctx_lens is NULL).  With
 * ctx_lens, ctx_len is the longest context of the call: it sizes the splits and the
 * workspace, and every entry is clamped to [0, ctx_len] on the device (an entry
 * above ctx_len is read as ctx_len).  q
 * kv_dtype [B, Hq, k, d]; row i of sequence b attends to cache rows [0, L + i].
 * out kv_dtype [B, Hq, k, d]; lse float32 [B, Hq, k] or NULL.  L + k <= cache_rows.
 * bf16 inputs run on bf16 matrix cores with float32 accumulation; f32 inputs run
 * in float32.
 *
 * Batch invariance: the cache is cut into splits of split_tokens rows at absolute
 * positions (0 = the library default for this B, Hkv and cache_rows, see
 * vc_verify_split_tokens) and every row is reduced in the same order whatever k,
 * its position in the window or the other sequences' lengths are; so row i equals,
 * bit for bit, the 1-row call made with ctx length L + i and the same split_tokens.
 * split_tokens must be a multiple of 64.
 *
 * vc_verify_workspace_bytes: workspace for calls with contexts up to max_len and
 * this k and split_tokens (0: the default for a cache of max_len + k rows, which
 * also covers the default of any larger cache).  ws must be 16-byte aligned
 * (VC_ERR_INVALID_ARG otherwise).
 * vc_verify_split_tokens: the default split, a multiple of 64 chosen so that a
 * cache of cache_rows rows is cut into at most as many splits per (sequence,
 * kv-head) as workgroups of the verification kernel fit on the current device
 * for all B*Hkv of them at once (512 are assumed when no device is present).
 * ------------------------------------------------------------------------- */
vc_status vc_verify_attn_full(const void* q, const void* k_cache, const void* v_cache, int32_t kv_dtype,
                              int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int32_t k,
                              int64_t cache_rows, int64_t ctx_len, const int32_t* ctx_lens,
                              int32_t split_tokens, float sm_scale, void* out, float* lse,
                              void* ws, size_t ws_bytes, void* stream);
size_t vc_verify_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int32_t k,
                                 int64_t max_len, int32_t split_tokens);
int32_t vc_verify_split_tokens(int32_t B, int32_t Hkv, int64_t cache_rows);

/* ---------------------------------------------------------------------------
 * Greedy tokens (summary page: greedy-decoding output identical to full-KV
 * inference).
 *
 * vc_head_mean: o kv_dtype, rows r = (b, i) of an attention output laid out with
 *   element strides (stride_b, stride_h, stride_i) and unit stride over d ->
 *   u float32 [B*k, d], u[b*k + i] = mean over the Hq heads.
 * vc_logits_argmax: u float32/bf16 (u_dtype) [R, Kdim], W w_dtype [V, Kdim] (one
 *   row per vocabulary entry) -> tokens int32 [R] = argmax_v (u_r . W_v), equal
 *   logits going to the lowest v.  Logits accumulate in float32.  With bf16 W and
 *   Kdim 64 or 128 (the matrix-core path) u and W must be 16-byte aligned
 *   (VC_ERR_INVALID_ARG otherwise).
 * ------------------------------------------------------------------------- */
vc_status vc_head_mean(const void* o, int32_t kv_dtype, int32_t B, int32_t Hq, int32_t k, int32_t d,
                       int64_t stride_b, int64_t stride_h, int64_t stride_i, float* u, void* stream);
vc_status vc_logits_argmax(const void* u, int32_t u_dtype, int64_t R, int32_t Kdim, const void* W,
                           int32_t w_dtype, int32_t V, int32_t* tokens, void* ws, size_t ws_bytes,
                           void* stream);
size_t vc_logits_workspace_bytes(int64_t R, int32_t V);

/* ---------------------------------------------------------------------------
 * Channel rotation before quantization (summary page, "What the paper found":
 * rotation-based low-bit quantizers such as RotateKV and TurboQuant behind the uniform
 * compressor interface).
 *
 * vc_hadamard_rows: out[r] = x[r] H / sqrt(d) for rows r < rows, H the Sylvester
 *   Hadamard matrix of order d (d = 64, 128 or 256).  x, out dtype (VC_BF16 or
 *   VC_F32) [rows, d], contiguous and 16-byte aligned (VC_ERR_INVALID_ARG
 *   otherwise); out may be x (in place), but no other overlap.  float32
 *   arithmetic, one rounding to dtype.  The map is its own inverse and keeps dot products, so keys
 *   and queries rotated alike give the same scores, and an attention output over
 *   rotated values is rotated back by a second call.  A compressor with the
 *   pre-pass rotates K and V rows before vc_compress; the drafter rotates q before
 *   vc_decode_attn_compressed and its output after.
 * ------------------------------------------------------------------------- */
vc_status vc_hadamard_rows(const void* x, int32_t dtype, int64_t rows, int32_t d, void* out, void* stream);

/* ---------------------------------------------------------------------------
 * Acceptance: longest prefix where draft equals target (episode page, source 2,
 * speculative decoding; summary page, greedy identity).
 *
 * draft, target int32 [B, k] -> accept_len int32 [B] (first i with
 * draft[i] != target[i], or k), n_commit int32 [B] (accept_len + (accept_len < k)),
 * commit int32 [B, k] (draft[0:accept_len], then target[accept_len] when
 * accept_len < k, then -1).  1 <= k <= 1024.
 * ------------------------------------------------------------------------- */
vc_status vc_accept(const int32_t* draft, const int32_t* target, int32_t B, int32_t k,
                    int32_t* accept_len, int32_t* n_commit, int32_t* commit, void* stream);

/* ---------------------------------------------------------------------------
 * Full-KV swap-in (abstract: the full KV cache is kept out of GPU memory and
 * swapped in for verification, overlapped with drafting).
 *
 * Copies token rows [tok_begin, tok_end) of every (sequence, kv-head) of the
 * pinned host arrays host_k, host_v (elem_bytes-sized elements, [B, Hkv,
 * host_rows, d]) to the same rows of dev_k, dev_v ([B, Hkv, dev_rows, d]) with
 * asynchronous DMA copies on copy_stream, then records `done` (a hipEvent_t
 * passed as void*, or NULL) on copy_stream.  A consumer waits for the event on its
 * own stream.  vc_stage_full_kv_d2h copies the same rows back (device to host),
 * e.g. to append accepted rows to the host copy.
 * ------------------------------------------------------------------------- */
vc_status vc_stage_full_kv(const void* host_k, const void* host_v, void* dev_k, void* dev_v,
                           int32_t B, int32_t Hkv, int32_t d, int32_t elem_bytes, int64_t host_rows,
                           int64_t dev_rows, int64_t tok_begin, int64_t tok_end, void* copy_stream,
                           void* done);
vc_status vc_stage_full_kv_d2h(const void* dev_k, const void* dev_v, void* host_k, void* host_v,
                               int32_t B, int32_t Hkv, int32_t d, int32_t elem_bytes, int64_t host_rows,
                               int64_t dev_rows, int64_t tok_begin, int64_t tok_end, void* copy_stream,
                               void* done);

/* ---------------------------------------------------------------------------
 * Split-stream form of a quantized cache (thelatestinai.com listing page for
 * 2604.15409, the Lynx abstract: an anchor stream of the most significant bits, a
 * residual stream of the rest; decoding may start on the anchor).  The anchor is an
 * ordinary VC_QUANT_KIVI cache that vc_decode_attn_compressed reads as it is.
 *
 * full, anchor: VC_QUANT_KIVI descriptors with equal B, Hkv, d (a multiple of 32),
 *   capacity, group and param_dtype; full K/V bits b in {2, 3, 4, 8}, anchor bits a
 *   in {2, 3, 4} with a <= b (per tensor), r = b - a.
 * k_resid, v_resid: uint32 [B, Hkv, capacity, d * r / 32], codes packed like every
 *   other code row (NULL allowed where r = 0).
 * vc_split_planes: for rows [0, n_tokens) (a multiple of group) of every (sequence,
 *   kv-head): anchor code = c >> r, residual code = c & (2^r - 1); anchor scale =
 *   s * 2^r, anchor zero = z + s * (2^r - 1) / 2 (float32 product, then sum, then
 *   rounding to param_dtype), i.e. each anchor level is the midpoint of the full
 *   levels it covers.  The anchor must not share arrays with the full cache.  The
 *   full cache's own parameters are the residual stream's.
 * vc_join_planes: full code = (anchor code << r) | residual code for the same rows
 *   (codes only; the full cache keeps its parameters).  Restores the split codes
 *   exactly.
 * ------------------------------------------------------------------------- */
vc_status vc_split_planes(const vc_ckv* full, const vc_ckv* anchor, uint32_t* k_resid, uint32_t* v_resid,
                          int64_t n_tokens, void* stream);
vc_status vc_join_planes(const vc_ckv* anchor, const uint32_t* k_resid, const uint32_t* v_resid,
                         const vc_ckv* full, int64_t n_tokens, void* stream);

/* ---------------------------------------------------------------------------
 * Full-KV staging from a file: the remote-prefix-cache setting (summary page, "What
 * the paper found" and "Original abstract": the same method serves remote prefix
 * caching, where the full KV's swap-in is network-bound rather than PCIe-bound).
 * A file descriptor that supports pread stands in for the remote store.
 *
 * vc_file_stager_create: n_threads reader threads (1..64), n_buffers pinned
 *   bounce buffers of chunk_bytes each (n_threads <= n_buffers <= 1024,
 *   4 KiB <= chunk_bytes <= 1 GiB), reads capped at max_bytes_per_s (0 =
 *   uncapped: the link being modelled).  Uses the current HIP device.  *out is
 *   the stager, owned by the caller until vc_file_stager_destroy, which first
 *   finishes every queued read and copy.
 * vc_stage_full_kv_file: copies token rows [tok_begin, tok_end) of every
 *   (sequence, kv-head) from the file -- K at byte k_offset and V at v_offset,
 *   each laid out [B, Hkv, file_rows, d] of elem_bytes-sized elements -- to the
 *   same rows of dev_k, dev_v ([B, Hkv, dev_rows, d]).  Returns at once with
 *   *ticket; the reads and the host-to-device copies (on copy_stream) run on the
 *   stager's threads, and `done` (a hipEvent_t as void*, or NULL) is recorded on
 *   copy_stream once every copy of the call has been issued.  The file must not
 *   change while the call is in flight; the device rows must not be read before
 *   `done`.
 * vc_file_stager_wait: blocks until every copy of the ticket's call has been
 *   issued and `done` recorded, then returns the call's status (VC_ERR_IO with
 *   the reason when a read failed, e.g. past the end of the file; the remaining
 *   chunks of that call are skipped).  Every ticket is waited for exactly once;
 *   a consumer waits for the ticket before it makes its stream wait for `done`.
 * ------------------------------------------------------------------------- */
typedef struct vc_file_stager vc_file_stager;
vc_status vc_file_stager_create(int32_t n_threads, size_t chunk_bytes, int32_t n_buffers, double max_bytes_per_s,
                                vc_file_stager** out);
vc_status vc_file_stager_destroy(vc_file_stager* st);
vc_status vc_stage_full_kv_file(vc_file_stager* st, int32_t fd, int64_t k_offset, int64_t v_offset, void* dev_k,
                                void* dev_v, int32_t B, int32_t Hkv, int32_t d, int32_t elem_bytes, int64_t file_rows,
                                int64_t dev_rows, int64_t tok_begin, int64_t tok_end, void* copy_stream, void* done,
                                int64_t* ticket);
vc_status vc_file_stager_wait(vc_file_stager* st, int64_t ticket);

/* ---------------------------------------------------------------------------
 * One workspace query for the calls that take a workspace (the boundary's single
 * size query; the per-call *_workspace_bytes functions return the same numbers).
 * VC_OP_COMPRESS reads ckv, n_tokens, n_probes; VC_OP_DECODE reads ckv, Hq;
 * VC_OP_VERIFY reads B, Hq, Hkv, d, k, max_len, split_tokens; VC_OP_LOGITS reads
 * rows, vocab.  Returns 0 for an unknown op, a NULL query or shapes the matching
 * call would reject.
 * ------------------------------------------------------------------------- */
typedef enum { VC_OP_COMPRESS = 1, VC_OP_DECODE = 2, VC_OP_VERIFY = 3, VC_OP_LOGITS = 4 } vc_op;
typedef struct {
  const vc_ckv* ckv;
  int64_t n_tokens;
  int32_t n_probes;
  int32_t Hq;
  int32_t B, Hkv, d, k;
  int64_t max_len;
  int32_t split_tokens;
  int64_t rows;
  int32_t vocab;
} vc_ws_query;
size_t vc_workspace_size(int32_t op, const vc_ws_query* query);

/* Message of the last failed call on this thread ("" if none).  Valid until the
 * next vc_* call on the same thread. */
const char* vc_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* VC_H_ */
