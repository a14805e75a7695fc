// Entry points that only dispatch (compression) or drive the copy engines (full-KV
// staging), and the thread-local error message.
//
// Staging follows the abstract of "VeriCache: Turning Lossy KV Cache into Lossless
// LLM Inference" (neuraltrendhub.com summary, "Original abstract"): the full KV
// cache stays out of GPU memory and is swapped in for verification, overlapped with
// compressed-KV drafting because one is bound by HBM and the other by PCIe.  The
// rows of every (sequence, kv-head) are one strided 2-D copy per tensor, issued as
// hipMemcpy2DAsync on the caller's copy stream so the DMA engines move them while
// the compute queues draft.

#include "common.h"

namespace vc {

static thread_local char g_err[512];

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

void clear_error() { g_err[0] = '\0'; }

vc_status compress_quant(const vc_ckv* c, const void* k_src, const void* v_src, int64_t src_rows, int64_t src_begin,
                         int64_t n_tokens, int64_t dst_begin, hipStream_t stream);
vc_status drop_scores_impl(const void* k, int32_t kv_dtype, const void* probes, int32_t B, int32_t Hkv, int64_t N,
                           int32_t d, int32_t P, float sm_scale, float* scores, void* ws, size_t ws_bytes,
                           hipStream_t s);
vc_status drop_select_impl(const float* scores, int32_t B, int32_t Hkv, int64_t N, int64_t n_keep, int32_t* kept,
                           int64_t kept_pitch, void* ws, size_t ws_bytes, hipStream_t s);
size_t drop_select_ws_bytes(int32_t B, int32_t Hkv, int64_t N);
vc_status gather_impl(const void* src, int32_t kv_dtype, int32_t B, int32_t Hkv, int64_t src_rows, int32_t d,
                      const int32_t* idx, int64_t n, int64_t idx_pitch, void* dst, int64_t dst_rows, hipStream_t s);

static vc_status stage_rows(const void* src_k, const void* src_v, void* dst_k, void* dst_v, int32_t B, int32_t Hkv,
                            int32_t d, int32_t elem_bytes, int64_t src_rows, int64_t dst_rows, int64_t tok_begin,
                            int64_t tok_end, hipMemcpyKind kind, void* copy_stream, void* done) {
  VC_REQUIRE(src_k && src_v && dst_k && dst_v, "NULL pointer argument");
  VC_REQUIRE(B > 0 && Hkv > 0 && d > 0, "bad B/Hkv/d");
  VC_REQUIRE(elem_bytes == 1 || elem_bytes == 2 || elem_bytes == 4 || elem_bytes == 8, "bad elem_bytes %d",
             elem_bytes);
  VC_REQUIRE(tok_begin >= 0 && tok_begin <= tok_end && tok_end <= src_rows && tok_end <= dst_rows,
             "rows [%lld, %lld) do not fit host_rows %lld / dev_rows %lld", (long long)tok_begin, (long long)tok_end,
             (long long)(kind == hipMemcpyHostToDevice ? src_rows : dst_rows),
             (long long)(kind == hipMemcpyHostToDevice ? dst_rows : src_rows));
  hipStream_t s = as_stream(copy_stream);
  const size_t row = static_cast<size_t>(d) * elem_bytes;
  const size_t width = static_cast<size_t>(tok_end - tok_begin) * row;
  if (width > 0) {
    const size_t spitch = static_cast<size_t>(src_rows) * row, dpitch = static_cast<size_t>(dst_rows) * row;
    const size_t off_s = static_cast<size_t>(tok_begin) * row, off_d = off_s;
    const size_t height = static_cast<size_t>(B) * Hkv;
    VC_HIP(hipMemcpy2DAsync(static_cast<char*>(dst_k) + off_d, dpitch, static_cast<const char*>(src_k) + off_s, spitch,
                            width, height, kind, s));
    VC_HIP(hipMemcpy2DAsync(static_cast<char*>(dst_v) + off_d, dpitch, static_cast<const char*>(src_v) + off_s, spitch,
                            width, height, kind, s));
  }
  if (done) VC_HIP(hipEventRecord(reinterpret_cast<hipEvent_t>(done), s));
  return VC_OK;
}

}  // namespace vc

using namespace vc;

extern "C" const char* vc_last_error(void) { return g_err; }

extern "C" vc_status vc_ckv_sizes(const vc_ckv* c, size_t* out_bytes) {
  clear_error();
  VC_REQUIRE(c && out_bytes, "ckv / out_bytes is NULL");
  VC_REQUIRE(c->B > 0 && c->Hkv > 0 && c->d > 0, "bad B/Hkv/d (%d, %d, %d)", c->B, c->Hkv, c->d);
  VC_REQUIRE(c->capacity >= 0 && c->tail_cap >= 0, "capacity / tail_cap must be non-negative");
  VC_REQUIRE(valid_dtype(c->kv_dtype), "bad kv_dtype %d", c->kv_dtype);
  size_t sz[VC_CKV_NARRAYS] = {};
  const size_t bh = static_cast<size_t>(c->B) * c->Hkv, d = static_cast<size_t>(c->d);
  const size_t cap = static_cast<size_t>(c->capacity), eb = dtype_bytes(c->kv_dtype);
  if (c->method == VC_QUANT_KIVI) {
    auto ok_bits = [](int b) { return b == 2 || b == 3 || b == 4 || b == 8 || b == 16; };
    VC_REQUIRE(ok_bits(c->k_bits) && ok_bits(c->v_bits), "bits must be one of 2,3,4,8,16 (got K %d, V %d)",
               c->k_bits, c->v_bits);
    VC_REQUIRE(c->group > 0 && c->d % c->group == 0, "group %d must divide d %d", c->group, c->d);
    VC_REQUIRE((c->d * c->k_bits) % 32 == 0 && (c->d * c->v_bits) % 32 == 0, "d*bits must be a multiple of 32");
    VC_REQUIRE(c->capacity % c->group == 0, "capacity %lld must be a multiple of group %d", (long long)c->capacity,
               c->group);
    VC_REQUIRE(valid_dtype(c->param_dtype), "bad param_dtype %d", c->param_dtype);
    const size_t pb = dtype_bytes(c->param_dtype), G = static_cast<size_t>(c->group);
    sz[VC_CKV_K_CODES] = bh * cap * (d * c->k_bits / 32) * 4;
    sz[VC_CKV_V_CODES] = bh * cap * (d * c->v_bits / 32) * 4;
    sz[VC_CKV_K_SCALE] = sz[VC_CKV_K_ZERO] = bh * (cap / G) * d * pb;
    sz[VC_CKV_V_SCALE] = sz[VC_CKV_V_ZERO] = bh * cap * (d / G) * pb;
  } else {
    VC_REQUIRE(c->method == VC_DROP_TOPK, "unknown ckv.method %d", c->method);
    sz[VC_CKV_K_KEPT] = sz[VC_CKV_V_KEPT] = bh * cap * d * eb;
    sz[VC_CKV_KEPT_IDX] = bh * cap * sizeof(int32_t);
  }
  sz[VC_CKV_TAIL_K] = sz[VC_CKV_TAIL_V] = bh * static_cast<size_t>(c->tail_cap) * d * eb;
  memcpy(out_bytes, sz, sizeof(sz));
  return VC_OK;
}

extern "C" size_t vc_workspace_size(int32_t op, const vc_ws_query* q) {
  if (!q) return 0;
  switch (op) {
    case VC_OP_COMPRESS: return q->ckv ? vc_compress_workspace_bytes(q->ckv, q->n_tokens, q->n_probes) : 0;
    case VC_OP_DECODE: return q->ckv ? vc_decode_workspace_bytes(q->ckv, q->Hq) : 0;
    case VC_OP_VERIFY:
      return vc_verify_workspace_bytes(q->B, q->Hq, q->Hkv, q->d, q->k, q->max_len, q->split_tokens);
    case VC_OP_LOGITS: return q->rows > 0 && q->vocab > 0 ? vc_logits_workspace_bytes(q->rows, q->vocab) : 0;
    default: return 0;
  }
}

extern "C" size_t vc_compress_workspace_bytes(const vc_ckv* c, int64_t n_tokens, int32_t n_probes) {
  if (!c || c->method != VC_DROP_TOPK || n_tokens <= 0 || n_probes <= 0 || c->B <= 0 || c->Hkv <= 0) return 0;
  size_t scores = align_up(static_cast<size_t>(c->B) * c->Hkv * n_tokens * sizeof(float), 256);
  // after the scores array: the scoring statistics, then (reusing the same bytes) the selection's histograms
  const size_t stats = vc_drop_scores_workspace_bytes(c->B, c->Hkv, n_tokens, n_probes);
  const size_t sel = drop_select_ws_bytes(c->B, c->Hkv, n_tokens);
  return scores + (stats > sel ? stats : sel);
}

extern "C" vc_status vc_compress(const vc_ckv* c, const void* k_src, const void* v_src, int64_t src_rows,
                                 int64_t src_begin, int64_t n_tokens, int64_t dst_begin, const void* probes,
                                 int32_t n_probes, float sm_scale, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  VC_REQUIRE(c != nullptr, "ckv is NULL");
  hipStream_t s = as_stream(stream);
  if (c->method == VC_QUANT_KIVI) {
    VC_REQUIRE(probes == nullptr && n_probes == 0, "probes must be NULL for quantization");
    return compress_quant(c, k_src, v_src, src_rows, src_begin, n_tokens, dst_begin, s);
  }
  VC_REQUIRE(c->method == VC_DROP_TOPK, "unknown ckv.method %d", c->method);
  VC_REQUIRE(src_begin == 0 && dst_begin == 0, "token dropping compresses whole sequences (src_begin = dst_begin = 0)");
  VC_REQUIRE(k_src && v_src && probes, "k_src / v_src / probes is NULL");
  VC_REQUIRE(c->B > 0 && c->Hkv > 0 && c->d > 0, "bad B/Hkv/d");
  VC_REQUIRE(valid_dtype(c->kv_dtype), "bad kv_dtype");
  VC_REQUIRE(n_tokens > 0 && n_tokens <= src_rows, "n_tokens must be in [1, src_rows]");
  VC_REQUIRE(src_rows == n_tokens, "token dropping needs src_rows == n_tokens");
  VC_REQUIRE(c->keep_ratio > 0.f && c->keep_ratio <= 1.f, "keep_ratio must be in (0, 1]");
  const int64_t keep = vc_drop_keep_count(c->keep_ratio, n_tokens);
  VC_REQUIRE(keep <= c->capacity, "n_keep %lld exceeds capacity %lld", (long long)keep, (long long)c->capacity);
  VC_REQUIRE(c->k_kept && c->v_kept && c->kept_idx, "kept arrays are NULL");
  size_t need = vc_compress_workspace_bytes(c, n_tokens, n_probes);
  if (!ws || ws_bytes < need) {
    set_error("compress workspace needs %zu bytes (got %zu)", need, ws_bytes);
    return VC_ERR_WORKSPACE;
  }
  float* scores = static_cast<float*>(ws);
  size_t sb = align_up(static_cast<size_t>(c->B) * c->Hkv * n_tokens * sizeof(float), 256);
  vc_status st = drop_scores_impl(k_src, c->kv_dtype, probes, c->B, c->Hkv, n_tokens, c->d, n_probes, sm_scale,
                                  scores, static_cast<char*>(ws) + sb, ws_bytes - sb, s);
  if (st != VC_OK) return st;
  st = drop_select_impl(scores, c->B, c->Hkv, n_tokens, keep, c->kept_idx, c->capacity, static_cast<char*>(ws) + sb,
                        ws_bytes - sb, s);
  if (st != VC_OK) return st;
  st = gather_impl(k_src, c->kv_dtype, c->B, c->Hkv, src_rows, c->d, c->kept_idx, keep, c->capacity, c->k_kept,
                   c->capacity, s);
  if (st != VC_OK) return st;
  return gather_impl(v_src, c->kv_dtype, c->B, c->Hkv, src_rows, c->d, c->kept_idx, keep, c->capacity, c->v_kept,
                     c->capacity, s);
}

extern "C" vc_status vc_stage_full_kv(const void* host_k, const void* host_v, void* dev_k, void* dev_v, int32_t B,
                                      int32_t Hkv, int32_t d, int32_t elem_bytes, int64_t host_rows, int64_t dev_rows,
                                      int64_t tok_begin, int64_t tok_end, void* copy_stream, void* done) {
  clear_error();
  return stage_rows(host_k, host_v, dev_k, dev_v, B, Hkv, d, elem_bytes, host_rows, dev_rows, tok_begin, tok_end,
                    hipMemcpyHostToDevice, copy_stream, done);
}

extern "C" vc_status vc_stage_full_kv_d2h(const void* dev_k, const void* dev_v, void* host_k, void* host_v, int32_t B,
                                          int32_t Hkv, int32_t d, int32_t elem_bytes, int64_t host_rows,
                                          int64_t dev_rows, int64_t tok_begin, int64_t tok_end, void* copy_stream,
                                          void* done) {
  clear_error();
  return stage_rows(dev_k, dev_v, host_k, host_v, B, Hkv, d, elem_bytes, dev_rows, host_rows, tok_begin, tok_end,
                    hipMemcpyDeviceToHost, copy_stream, done);
}
