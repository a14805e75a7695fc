// Split-stream form of a KIVI-quantized cache: an anchor stream of each code's most
// significant bits, itself a quantized cache the drafter can decode, and a residual
// stream of the remaining bits that restores the full codes.
//
// thelatestinai.com listing page for 2604.15409, the Lynx abstract: the quantized
// cache is cut into a high-priority anchor stream (most significant bits) and a
// low-priority residual stream (the rest of the precision); decoding may start on
// the anchor and is verified afterwards.  In VeriCache's terms (neuraltrendhub.com
// summary, "What the paper found": compressors behind one interface) the anchor is
// one more compressed cache to draft from.  A b-bit code c with scale s and zero z
// becomes, for an a-bit anchor and r = b - a, the anchor code c >> r with scale
// s 2^r and zero z + s (2^r - 1) / 2 (the midpoint of the 2^r levels it covers: two
// float32 operations, then one rounding to the parameter type) and the residual
// code c & (2^r - 1).  The residual keeps the full cache's parameters.
//
// Packed rows are little-endian bitstreams, so 32 consecutive codes of any width b
// fill exactly b words: one thread handles one 32-code chunk, reading b words and
// writing a anchor words and r residual words (all indices compile-time constants).
// Built without floating-point contraction: the zero is a product, then a sum.

#include <algorithm>

#include "common.h"

namespace vc {

// code i of a chunk of B-bit codes held in w[0..B)
template <int B>
__device__ __forceinline__ uint32_t chunk_code(const uint32_t (&w)[B], int i) {
  const int pos = B * i, wi = pos >> 5, off = pos & 31;
  uint32_t c = w[wi] >> off;
  if (off + B > 32) c |= w[wi + 1] << (32 - off);
  return c & ((1u << B) - 1u);
}

template <int B>
__device__ __forceinline__ void chunk_put(uint32_t (&w)[B], int i, uint32_t c) {
  const int pos = B * i, wi = pos >> 5, off = pos & 31;
  w[wi] |= c << off;
  if (off + B > 32) w[wi + 1] |= c >> (32 - off);
}

template <int N>
__device__ __forceinline__ void load_words(const uint32_t* p, uint32_t (&w)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) w[i] = p[i];
}
template <int N>
__device__ __forceinline__ void store_words(uint32_t* p, const uint32_t (&w)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) p[i] = w[i];
}

// One thread per 32-code chunk of rows [0, n) of every (sequence, kv-head).
// JOIN = false: full (B bits) -> anchor (A bits) + residual (B - A bits);
// JOIN = true:  anchor + residual -> full.
template <int B, int A, bool JOIN>
__global__ void __launch_bounds__(256) split_codes_kernel(uint32_t* full, uint32_t* anchor, uint32_t* resid,
                                                          int64_t bh_count, int64_t capacity, int64_t n,
                                                          int chunks_per_row) {
  constexpr int R = B - A;
  const int64_t per_bh = n * chunks_per_row;
  const int64_t total = bh_count * per_bh;
  for (int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; g < total;
       g += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t bh = g / per_bh, rest = g % per_bh;
    const int64_t row = bh * capacity + rest / chunks_per_row;
    const int ch = static_cast<int>(rest % chunks_per_row);
    uint32_t* pf = full + (row * chunks_per_row + ch) * B;
    uint32_t* pa = anchor + (row * chunks_per_row + ch) * A;
    uint32_t* pr = resid + (row * chunks_per_row + ch) * (R > 0 ? R : 1);
    uint32_t wf[B] = {}, wa[A] = {};
    uint32_t wr[R > 0 ? R : 1] = {};
    if constexpr (!JOIN) {
      load_words(pf, wf);
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const uint32_t c = chunk_code<B>(wf, i);
        chunk_put<A>(wa, i, c >> R);
        if constexpr (R > 0) chunk_put<R>(wr, i, c & ((1u << R) - 1u));
      }
      store_words(pa, wa);
      if constexpr (R > 0) store_words(pr, wr);
    } else {
      load_words(pa, wa);
      if constexpr (R > 0) load_words(pr, wr);
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        uint32_t c = chunk_code<A>(wa, i) << R;
        if constexpr (R > 0) c |= chunk_code<R>(wr, i);
        chunk_put<B>(wf, i, c);
      }
      store_words(pf, wf);
    }
  }
}

// Anchor parameters: s_a = s * 2^r, z_a = z + s * (2^r - 1) / 2 for `count` rows of
// `per_row` live parameters out of a row pitch of `pitch` (the rest untouched).
template <typename P>
__global__ void __launch_bounds__(256) anchor_params_kernel(const P* s, const P* z, P* sa, P* za, int64_t rows,
                                                            int64_t rows_per_bh, int64_t bh_pitch, int per_row,
                                                            float mul_s, float mul_h) {
  const int64_t total = rows * per_row;
  for (int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; g < total;
       g += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t r = g / per_row;
    const int64_t i = (r / rows_per_bh) * bh_pitch + (r % rows_per_bh) * per_row + g % per_row;
    const float sv = Elem<P>::load(s, i), zv = Elem<P>::load(z, i);
    const float h = sv * mul_h;
    Elem<P>::store(sa, i, sv * mul_s);
    Elem<P>::store(za, i, zv + h);
  }
}

template <int B, int A>
struct BitsTag {
  static constexpr int b = B, a = A;
};

// Calls f(BitsTag<b, a>{}) for a supported (b, a); false otherwise.
template <class F>
bool with_bits(int b, int a, F&& f) {
  switch (b * 16 + a) {
    case 2 * 16 + 2: f(BitsTag<2, 2>{}); return true;
    case 3 * 16 + 2: f(BitsTag<3, 2>{}); return true;
    case 3 * 16 + 3: f(BitsTag<3, 3>{}); return true;
    case 4 * 16 + 2: f(BitsTag<4, 2>{}); return true;
    case 4 * 16 + 3: f(BitsTag<4, 3>{}); return true;
    case 4 * 16 + 4: f(BitsTag<4, 4>{}); return true;
    case 8 * 16 + 2: f(BitsTag<8, 2>{}); return true;
    case 8 * 16 + 3: f(BitsTag<8, 3>{}); return true;
    case 8 * 16 + 4: f(BitsTag<8, 4>{}); return true;
    default: return false;
  }
}

vc_status validate_quant_ckv(const vc_ckv* c);

static vc_status check_pair(const vc_ckv* full, const vc_ckv* anchor, const uint32_t* k_resid,
                            const uint32_t* v_resid, int64_t n) {
  vc_status st = validate_quant_ckv(full);
  if (st != VC_OK) return st;
  st = validate_quant_ckv(anchor);
  if (st != VC_OK) return st;
  VC_REQUIRE(full->B == anchor->B && full->Hkv == anchor->Hkv && full->d == anchor->d &&
                 full->capacity == anchor->capacity && full->group == anchor->group &&
                 full->param_dtype == anchor->param_dtype,
             "full and anchor caches differ in B, Hkv, d, capacity, group or parameter type");
  VC_REQUIRE(full->d % 32 == 0, "d %d must be a multiple of 32", full->d);
  VC_REQUIRE(n >= 0 && n <= full->capacity && n % full->group == 0,
             "n_tokens %lld must be a multiple of group %d within capacity %lld", (long long)n, full->group,
             (long long)full->capacity);
  VC_REQUIRE(anchor->k_bits <= full->k_bits && anchor->v_bits <= full->v_bits,
             "anchor bits (K %d, V %d) exceed the full cache's (K %d, V %d)", anchor->k_bits, anchor->v_bits,
             full->k_bits, full->v_bits);
  auto nop = [](auto) {};
  VC_UNSUPPORTED(with_bits(full->k_bits, anchor->k_bits, nop) && with_bits(full->v_bits, anchor->v_bits, nop),
                 "split (K %d -> %d, V %d -> %d) bits: full 2, 3, 4 or 8, anchor 2, 3 or 4", full->k_bits,
                 anchor->k_bits, full->v_bits, anchor->v_bits);
  VC_REQUIRE((full->k_bits == anchor->k_bits || k_resid) && (full->v_bits == anchor->v_bits || v_resid),
             "residual array is NULL");
  return VC_OK;
}

static int64_t grid_for(int64_t work) { return std::max<int64_t>(1, std::min<int64_t>(cdiv(work, 256), 8192)); }

static vc_status launch_codes(bool join, int b, int a, uint32_t* full, uint32_t* anchor, uint32_t* resid,
                              const vc_ckv* c, int64_t n, hipStream_t s) {
  const int64_t bh = static_cast<int64_t>(c->B) * c->Hkv;
  const int cpr = c->d / 32;
  const unsigned blocks = static_cast<unsigned>(grid_for(bh * n * cpr));
  with_bits(b, a, [&](auto tag) {
    constexpr int B = decltype(tag)::b, A = decltype(tag)::a;
    if (join)
      hipLaunchKernelGGL((split_codes_kernel<B, A, true>), dim3(blocks), dim3(256), 0, s, full, anchor, resid, bh,
                         c->capacity, n, cpr);
    else
      hipLaunchKernelGGL((split_codes_kernel<B, A, false>), dim3(blocks), dim3(256), 0, s, full, anchor, resid, bh,
                         c->capacity, n, cpr);
  });
  VC_LAUNCHED("split_codes_kernel");
  return VC_OK;
}

template <typename P>
static vc_status launch_params(const vc_ckv* f, const vc_ckv* an, int64_t n, hipStream_t s) {
  const int64_t bh = static_cast<int64_t>(f->B) * f->Hkv;
  const int G = f->group, d = f->d, ngv = d / G;
  auto go = [&](const void* sp, const void* zp, void* sap, void* zap, int64_t rows_per_bh, int64_t pitch, int per_row,
                int r) {
    const int64_t rows = bh * rows_per_bh;
    if (rows == 0) return;
    const float mul_s = static_cast<float>(1 << r), mul_h = static_cast<float>((1 << r) - 1) * 0.5f;
    hipLaunchKernelGGL(anchor_params_kernel<P>, dim3(static_cast<unsigned>(grid_for(rows * per_row))), dim3(256), 0,
                       s, static_cast<const P*>(sp), static_cast<const P*>(zp), static_cast<P*>(sap),
                       static_cast<P*>(zap), rows, rows_per_bh, pitch, per_row, mul_s, mul_h);
  };
  // K: [bh][capacity / G][d], groups [0, n / G);  V: [bh][capacity][d / G], tokens [0, n)
  go(f->k_scale, f->k_zero, an->k_scale, an->k_zero, n / G, (f->capacity / G) * d, d, f->k_bits - an->k_bits);
  go(f->v_scale, f->v_zero, an->v_scale, an->v_zero, n, f->capacity * ngv, ngv, f->v_bits - an->v_bits);
  VC_LAUNCHED("anchor_params_kernel");
  return VC_OK;
}

}  // namespace vc

using namespace vc;

extern "C" vc_status vc_split_planes(const vc_ckv* full, const vc_ckv* anchor, uint32_t* k_resid, uint32_t* v_resid,
                                     int64_t n_tokens, void* stream) {
  clear_error();
  vc_status st = check_pair(full, anchor, k_resid, v_resid, n_tokens);
  if (st != VC_OK) return st;
  VC_REQUIRE(full->k_codes != anchor->k_codes && full->v_codes != anchor->v_codes &&
                 full->k_scale != anchor->k_scale && full->k_zero != anchor->k_zero &&
                 full->v_scale != anchor->v_scale && full->v_zero != anchor->v_zero,
             "the anchor must not share arrays with the full cache");
  if (n_tokens == 0) return VC_OK;
  hipStream_t s = as_stream(stream);
  st = launch_codes(false, full->k_bits, anchor->k_bits, full->k_codes, anchor->k_codes, k_resid, full, n_tokens, s);
  if (st != VC_OK) return st;
  st = launch_codes(false, full->v_bits, anchor->v_bits, full->v_codes, anchor->v_codes, v_resid, full, n_tokens, s);
  if (st != VC_OK) return st;
  return full->param_dtype == VC_F32 ? launch_params<float>(full, anchor, n_tokens, s)
                                     : launch_params<bf16_t>(full, anchor, n_tokens, s);
}

extern "C" vc_status vc_join_planes(const vc_ckv* anchor, const uint32_t* k_resid, const uint32_t* v_resid,
                                    const vc_ckv* full, int64_t n_tokens, void* stream) {
  clear_error();
  vc_status st = check_pair(full, anchor, k_resid, v_resid, n_tokens);
  if (st != VC_OK) return st;
  VC_REQUIRE(full->k_codes != anchor->k_codes && full->v_codes != anchor->v_codes,
             "the full cache's code arrays must not be the anchor's");
  if (n_tokens == 0) return VC_OK;
  hipStream_t s = as_stream(stream);
  st = launch_codes(true, full->k_bits, anchor->k_bits, full->k_codes, anchor->k_codes, const_cast<uint32_t*>(k_resid),
                    full, n_tokens, s);
  if (st != VC_OK) return st;
  return launch_codes(true, full->v_bits, anchor->v_bits, full->v_codes, anchor->v_codes,
                      const_cast<uint32_t*>(v_resid), full, n_tokens, s);
}
