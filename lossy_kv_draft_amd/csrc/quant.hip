// KIVI-style group quantization and bit packing (compression of the draft cache).
//
// Method: episode page "VeriCache: Lossless LLM Inference from Lossy KV Caches",
// source 4 (KIVI, tuning-free asymmetric low-bit KV quantization); summary page
// "VeriCache: Turning Lossy KV Cache into Lossless LLM Inference", "What the paper
// found" (KIVI is one of the compressors behind the uniform interface).
//
// K is quantized per channel (a group = G tokens of one channel), V per token (a
// group = G channels of one token).  Per group: s = fl32(fl32(max - min) /
// (2^b - 1)) and z = min, both rounded to the parameter dtype; then
// code = clamp(rint((x - z) / s), 0, 2^b - 1) with IEEE float32 subtract and
// divide and round-half-even, or 0 for every element when s == 0.  Every step is
// an explicitly rounded float32 operation so that codes match a float32 reference
// bit for bit.
//
// One workgroup quantizes one tile of G tokens x d channels of one (sequence,
// kv-head): the tile is staged in LDS in the source type (bf16 values convert to
// float32 exactly when read), parameters are computed by one
// thread per K channel / per (token, V group), then each thread builds whole
// 32-bit words of packed codes (a word may hold a code that straddles into the
// next word; both words compute that code).  HBM-bound: each input element is
// read once and each output word written once.

#include "common.h"

namespace vc {

constexpr int kQuantThreads = 256;
constexpr int kQuantMaxTileBytes = 32768;  // G * d source elements per tile (32 KiB of LDS)

template <typename T>
__device__ __forceinline__ void group_params(float mn, float mx, int bits, int param_f32,
                                             float& s, float& z) {
  float levels = static_cast<float>((1 << bits) - 1);
  float s32 = __fdiv_rn(__fsub_rn(mx, mn), levels);
  if (param_f32) {
    s = s32;
    z = mn;
  } else {
    s = bf16_to_f32(f32_to_bf16(s32));
    z = bf16_to_f32(f32_to_bf16(mn));
  }
}

__device__ __forceinline__ uint32_t quant_code(float x, float s, float z, int bits) {
  if (s == 0.0f) return 0u;
  float t = rintf(__fdiv_rn(__fsub_rn(x, z), s));
  float hi = static_cast<float>((1 << bits) - 1);
  t = fminf(fmaxf(t, 0.0f), hi);
  return static_cast<uint32_t>(t);
}

__device__ __forceinline__ void store_param(void* base, int param_f32, int64_t i, float v) {
  if (param_f32)
    static_cast<float*>(base)[i] = v;
  else
    static_cast<bf16_t*>(base)[i] = f32_to_bf16(v);  // exact: v is already a bf16 value
}

// Builds packed word w of a token row whose codes are code(c) for c in [0, d).
template <typename CodeFn>
__device__ __forceinline__ uint32_t pack_word(int w, int bits, CodeFn code) {
  int bit0 = 32 * w;
  int c_first = bit0 / bits;
  int c_last = (bit0 + 31) / bits;
  uint32_t word = 0;
  for (int c = c_first; c <= c_last; ++c) {
    uint32_t q = code(c);
    int pos = c * bits - bit0;  // may be negative for a code straddling in from the previous word
    if (pos >= 0)
      word |= q << pos;
    else
      word |= q >> (-pos);
  }
  return word;
}

template <typename T>
__global__ void __launch_bounds__(kQuantThreads)
quant_pack_kernel(const T* __restrict__ k_src, const T* __restrict__ v_src, int64_t src_rows,
                  int64_t src_begin, int Hkv, int d, int G, int k_bits, int v_bits, int param_f32,
                  int64_t capacity, int64_t dst_begin, uint32_t* __restrict__ k_codes,
                  uint32_t* __restrict__ v_codes, void* k_scale, void* k_zero, void* v_scale,
                  void* v_zero) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  T* tile = reinterpret_cast<T*>(smem_raw);                                  // [G][d]
  float* ks = reinterpret_cast<float*>(smem_raw + static_cast<size_t>(G) * d * sizeof(T));  // [d]
  float* kz = ks + d;                 // [d]
  float* vs = kz + d;                 // [G][d/G]
  float* vz = vs + d;                 // [G][d/G]  (G * d/G == d)

  const int grp = blockIdx.x;
  const int bh = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t src_base = (static_cast<int64_t>(bh) * src_rows + src_begin + static_cast<int64_t>(grp) * G) * d;
  const int64_t dst_tok0 = dst_begin + static_cast<int64_t>(grp) * G;
  const int n = G * d;
  const int vgroups = d / G;

  for (int pass = 0; pass < 2; ++pass) {
    const T* src = pass == 0 ? k_src : v_src;
    for (int i = tid; i < n; i += kQuantThreads) tile[i] = src[src_base + i];
    __syncthreads();
    if (pass == 0) {
      // K: one group per channel over the tile's G tokens.
      for (int c = tid; c < d; c += kQuantThreads) {
        float mn = Elem<T>::load(tile, c), mx = mn;
        for (int t = 1; t < G; ++t) {
          float x = Elem<T>::load(tile, t * d + c);
          mn = fminf(mn, x);
          mx = fmaxf(mx, x);
        }
        float s, z;
        group_params<T>(mn, mx, k_bits, param_f32, s, z);
        ks[c] = s;
        kz[c] = z;
        int64_t pi = (static_cast<int64_t>(bh) * (capacity / G) + dst_tok0 / G) * d + c;
        store_param(k_scale, param_f32, pi, s);
        store_param(k_zero, param_f32, pi, z);
      }
    } else {
      // V: one group per (token, G consecutive channels).
      for (int j = tid; j < G * vgroups; j += kQuantThreads) {
        int t = j / vgroups, g = j % vgroups;
        const T* row = tile + t * d + g * G;
        float mn = Elem<T>::load(row, 0), mx = mn;
        for (int c = 1; c < G; ++c) {
          const float x = Elem<T>::load(row, c);
          mn = fminf(mn, x);
          mx = fmaxf(mx, x);
        }
        float s, z;
        group_params<T>(mn, mx, v_bits, param_f32, s, z);
        vs[j] = s;
        vz[j] = z;
        int64_t pi = (static_cast<int64_t>(bh) * capacity + dst_tok0 + t) * vgroups + g;
        store_param(v_scale, param_f32, pi, s);
        store_param(v_zero, param_f32, pi, z);
      }
    }
    __syncthreads();
    const int bits = pass == 0 ? k_bits : v_bits;
    const int wpr = d * bits / 32;  // words per token row
    uint32_t* codes = pass == 0 ? k_codes : v_codes;
    for (int j = tid; j < G * wpr; j += kQuantThreads) {
      int t = j / wpr, w = j % wpr;
      const T* row = tile + t * d;
      uint32_t word;
      if (pass == 0)
        word = pack_word(w, bits, [&](int c) { return quant_code(Elem<T>::load(row, c), ks[c], kz[c], bits); });
      else
        word = pack_word(w, bits, [&](int c) {
          int g = c / G;
          return quant_code(Elem<T>::load(row, c), vs[t * vgroups + g], vz[t * vgroups + g], bits);
        });
      codes[(static_cast<int64_t>(bh) * capacity + dst_tok0 + t) * wpr + w] = word;
    }
    __syncthreads();
  }
}

static bool valid_bits(int b) { return b == 2 || b == 3 || b == 4 || b == 8 || b == 16; }

vc_status validate_quant_ckv(const vc_ckv* c) {
  VC_REQUIRE(c != nullptr, "ckv is NULL");
  VC_REQUIRE(c->method == VC_QUANT_KIVI, "ckv.method is not VC_QUANT_KIVI");
  VC_REQUIRE(c->B > 0 && c->Hkv > 0 && c->d > 0, "bad B/Hkv/d (%d, %d, %d)", c->B, c->Hkv, c->d);
  VC_REQUIRE(valid_bits(c->k_bits) && valid_bits(c->v_bits), "bits must be one of 2,3,4,8,16 (got K %d, V %d)",
             c->k_bits, c->v_bits);
  VC_REQUIRE(c->group > 0 && c->d % c->group == 0, "group %d must divide d %d", c->group, c->d);
  VC_REQUIRE((c->d * c->k_bits) % 32 == 0 && (c->d * c->v_bits) % 32 == 0, "d*bits must be a multiple of 32");
  VC_REQUIRE(valid_dtype(c->param_dtype) && valid_dtype(c->kv_dtype), "bad dtype");
  VC_REQUIRE(c->capacity >= 0 && c->capacity % c->group == 0, "capacity %lld must be a multiple of group %d",
             (long long)c->capacity, c->group);
  VC_REQUIRE(c->n_main >= 0 && c->n_main <= c->capacity && c->n_main % c->group == 0,
             "n_main %lld must be in [0, capacity] and a multiple of group", (long long)c->n_main);
  VC_REQUIRE(c->tail_len >= 0 && c->tail_len <= c->tail_cap, "tail_len must be in [0, tail_cap]");
  VC_REQUIRE(c->tail_len == 0 || (c->tail_k && c->tail_v), "tail arrays are NULL");
  VC_REQUIRE(c->capacity == 0 || (c->k_codes && c->v_codes && c->k_scale && c->k_zero && c->v_scale && c->v_zero),
             "quantized arrays are NULL");
  return VC_OK;
}

vc_status compress_quant(const vc_ckv* c, const void* k_src, const void* v_src, int64_t src_rows,
                         int64_t src_begin, int64_t n_tokens, int64_t dst_begin, hipStream_t stream) {
  vc_status st = validate_quant_ckv(c);
  if (st != VC_OK) return st;
  const int G = c->group;
  VC_REQUIRE(k_src && v_src, "k_src / v_src is NULL");
  VC_REQUIRE(n_tokens >= 0 && n_tokens % G == 0, "n_tokens %lld must be a multiple of group %d", (long long)n_tokens, G);
  VC_REQUIRE(src_begin >= 0 && src_begin % G == 0 && src_begin + n_tokens <= src_rows,
             "source rows [%lld, %lld) do not fit src_rows %lld or are not group-aligned", (long long)src_begin,
             (long long)(src_begin + n_tokens), (long long)src_rows);
  VC_REQUIRE(dst_begin >= 0 && dst_begin % G == 0 && dst_begin + n_tokens <= c->capacity,
             "destination rows [%lld, %lld) exceed capacity %lld or are not group-aligned", (long long)dst_begin,
             (long long)(dst_begin + n_tokens), (long long)c->capacity);
  const size_t tile_bytes = static_cast<size_t>(G) * c->d * dtype_bytes(c->kv_dtype);
  VC_UNSUPPORTED(tile_bytes <= kQuantMaxTileBytes, "group*d*element size = %zu bytes exceeds %d", tile_bytes,
                 kQuantMaxTileBytes);
  if (n_tokens == 0) return VC_OK;
  dim3 grid(static_cast<unsigned>(n_tokens / G), static_cast<unsigned>(c->B * c->Hkv));
  size_t lds = tile_bytes + 4 * static_cast<size_t>(c->d) * sizeof(float);
  int pf32 = c->param_dtype == VC_F32;
  if (c->kv_dtype == VC_F32)
    hipLaunchKernelGGL(quant_pack_kernel<float>, grid, dim3(kQuantThreads), lds, stream,
                       static_cast<const float*>(k_src), static_cast<const float*>(v_src), src_rows, src_begin,
                       c->Hkv, c->d, G, c->k_bits, c->v_bits, pf32, c->capacity, dst_begin, c->k_codes,
                       c->v_codes, c->k_scale, c->k_zero, c->v_scale, c->v_zero);
  else
    hipLaunchKernelGGL(quant_pack_kernel<bf16_t>, grid, dim3(kQuantThreads), lds, stream,
                       static_cast<const bf16_t*>(k_src), static_cast<const bf16_t*>(v_src), src_rows, src_begin,
                       c->Hkv, c->d, G, c->k_bits, c->v_bits, pf32, c->capacity, dst_begin, c->k_codes,
                       c->v_codes, c->k_scale, c->k_zero, c->v_scale, c->v_zero);
  VC_LAUNCHED("quant_pack_kernel");
  return VC_OK;
}

}  // namespace vc
