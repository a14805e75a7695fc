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
// float32 exactly when read), the group parameters are computed, then threads build
// whole 32-bit words of packed codes.  Each input element is read from HBM once and
// each output word written once; at the measured shapes the vector instructions per
// element, not HBM, set the time.  quant_pack_kernel is the direct form (one thread
// per K channel / per (token, V group) for the parameters, a code that straddles two
// words computed by both); quant_pack_fast_kernel, further down, the restructured one
// used wherever its shape limits allow.

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

// The code of x from the reciprocal r of the scale, when the product certifies it.  r
// comes from v_rcp_f32 (within 1 ulp), so qa = fl(fl(x - z) r) differs from the correctly
// rounded quotient fl(fl(x - z) / s) by at most 2^-22 of it.  Where |qa| <= 2^(BITS+1)
// and qa lies further than 2^(BITS-20) from every half-integer, both round to the same
// integer; where |qa| is larger, both clamp to the same end of [0, 2^BITS - 1].  ok is
// cleared otherwise, and for NaN (scale_reciprocal returns NaN for a scale whose
// reciprocal would not be accurate), and the caller then forms the code with quant_code.
// The code is returned in biased form: the bits of fl(clamp(qa, 0, 2^BITS - 1) + 1.5 2^23),
// which are kCodeBias plus the code (the addition rounds half to even to an integer, and
// rounding after the clamp equals clamping after it).
constexpr uint32_t kCodeBias = 0x4B400000u;  // bits of 1.5 2^23
template <int BITS>
__device__ __forceinline__ uint32_t quant_biased_certified(float x, float z, float r, bool& ok) {
  static_assert(BITS <= 8, "the margin grows with the code width");
  const float qa = __fmul_rn(__fsub_rn(x, z), r);
  ok = ok & (fabsf(__builtin_amdgcn_fractf(qa) - 0.5f) > static_cast<float>(1 << BITS) * 0x1p-20f);
  return __float_as_uint(
      __fadd_rn(__builtin_amdgcn_fmed3f(qa, 0.0f, static_cast<float>((1 << BITS) - 1)), 0x1.8p23f));
}

// sum over the N codes of a word of kCodeBias << (i BITS), modulo 2^32
template <int BITS, int N>
constexpr uint32_t word_bias() {
  uint32_t b = 0;
  for (int i = 0; i < N; ++i) b += kCodeBias << (i * BITS);
  return b;
}

// 1/s for a normal finite scale, else NaN (zero, subnormal and non-finite scales go to
// quant_code).
__device__ __forceinline__ float scale_reciprocal(float s) {
  return (s >= 0x1p-126f && s <= 0x1.fffffep127f) ? __builtin_amdgcn_rcpf(s) : __builtin_nanf("");
}

// One word of N = 32 / BITS codes from elements x with per-code parameters (s, z) and
// reciprocals r: each code from the certified product, and a code that some lane of the
// wave could not certify from the division (quant_code) in those lanes.  The branch per
// code is wave-uniform: with bf16 data and parameters about 0.2% of the quotients are
// exact half-integers (never certified), so a code position needs the division in
// about one wave in eight, a whole word in most.  16-bit codes always divide.
template <int BITS, int N, typename SZ>
__device__ __forceinline__ uint32_t pack_word_fast(const float (&x)[N], SZ sz) {
  if constexpr (BITS <= 8) {
    uint32_t b[N];
    bool ok[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
      ok[i] = true;
      b[i] = quant_biased_certified<BITS>(x[i], sz.z(i), sz.r(i), ok[i]);
    }
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (__builtin_amdgcn_ballot_w64(!ok[i]))
        if (!ok[i]) b[i] = kCodeBias + quant_code(x[i], sz.s(i), sz.z(i), BITS);
    uint32_t acc = 0;  // the biased codes, each shifted to its field: the biases sum to word_bias
#pragma unroll
    for (int i = 0; i < N; ++i) acc += b[i] << (i * BITS);
    return acc - word_bias<BITS, N>();
  } else {
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) word |= quant_code(x[i], sz.s(i), sz.z(i), BITS) << (i * BITS);
    return word;
  }
}

// N consecutive tile elements as float32 from an LDS run that starts at a multiple of
// N elements (so a run of 8 bf16 or 4 float32 is one 16-byte read)
template <int N, typename T>
__device__ __forceinline__ void load_run(const T* p, float (&x)[N]) {
  if constexpr (sizeof(T) == 2 && N >= 2) {
    constexpr int W = N / 2;  // 32-bit words, two bf16 each (element 2k in the low half)
    uint32_t u[W];
    if constexpr (W % 4 == 0) {
#pragma unroll
      for (int k = 0; k < W / 4; ++k) {
        const uint4 v = reinterpret_cast<const uint4*>(p)[k];
        u[4 * k] = v.x; u[4 * k + 1] = v.y; u[4 * k + 2] = v.z; u[4 * k + 3] = v.w;
      }
    } else if constexpr (W == 2) {
      const uint2 v = *reinterpret_cast<const uint2*>(p);
      u[0] = v.x; u[1] = v.y;
    } else {
      u[0] = *reinterpret_cast<const uint32_t*>(p);
    }
#pragma unroll
    for (int k = 0; k < W; ++k) {
      x[2 * k] = __uint_as_float(u[k] << 16);
      x[2 * k + 1] = __uint_as_float(u[k] & 0xFFFF0000u);
    }
  } else if constexpr (sizeof(T) == 4 && N % 4 == 0) {
#pragma unroll
    for (int k = 0; k < N / 4; ++k) {
      const float4 v = reinterpret_cast<const float4*>(p)[k];
      x[4 * k] = v.x; x[4 * k + 1] = v.y; x[4 * k + 2] = v.z; x[4 * k + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = Elem<T>::load(p, i);
  }
}

template <int BITS, typename T>
__device__ __forceinline__ void pack_k_columns(const T* tile, const float* ks, const float* kz, int d, int G, int ld,
                                               uint32_t* codes, int64_t row0, int tid) {
  constexpr int CPW = 32 / BITS, LCPW = BITS == 2 ? 4 : BITS == 4 ? 3 : BITS == 8 ? 2 : 1;
  const int lw = ld - LCPW, wpr = 1 << lw;  // words per row (d and CPW are powers of two)
  const int w = tid & (wpr - 1), rstep = kQuantThreads >> lw;
  const int c0 = w * CPW;
  float z[CPW], r[CPW];  // the scales themselves are read from LDS on the division path only
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    z[i] = kz[c0 + i];
    r[i] = scale_reciprocal(ks[c0 + i]);
  }
  for (int t = tid >> lw; t < G; t += rstep) {
    float x[CPW];
    load_run<CPW>(tile + (t << ld) + c0, x);
    struct {
      const float *s_, *z_, *r_;
      __device__ float s(int i) const { return s_[i]; }
      __device__ float z(int i) const { return z_[i]; }
      __device__ float r(int i) const { return r_[i]; }
    } sz{ks + c0, z, r};
    codes[((row0 + t) << lw) + w] = pack_word_fast<BITS>(x, sz);
  }
}

template <int BITS, typename T>
__device__ __forceinline__ void pack_v_words(const T* tile, const float* vs, const float* vz, int d, int G, int ld,
                                             int lg, uint32_t* codes, int64_t row0, int tid) {
  constexpr int CPW = 32 / BITS, LCPW = BITS == 2 ? 4 : BITS == 4 ? 3 : BITS == 8 ? 2 : 1;
  const int lw = ld - LCPW, wpr = 1 << lw;
  for (int j = tid; j < (G << lw); j += kQuantThreads) {
    const int t = j >> lw, c0 = (j & (wpr - 1)) * CPW;
    const int gi = (t << (ld - lg)) + (c0 >> lg);  // CPW <= 16 <= G: one group per word
    const float s = vs[gi], z = vz[gi];
    const float r = scale_reciprocal(s);
    float x[CPW];
    load_run<CPW>(tile + (t << ld) + c0, x);
    struct {
      float s_, z_, r_;
      __device__ float s(int) const { return s_; }
      __device__ float z(int) const { return z_; }
      __device__ float r(int) const { return r_; }
    } sz{s, z, r};
    codes[((row0 + t) << lw) + (j & (wpr - 1))] = pack_word_fast<BITS>(x, sz);
  }
}

// 16 3-bit codes q (channels 16 h .. 16 h + 15 of a row) into the row's words: the 32
// codes of channels [32 u, 32 u + 32) fill exactly words 3 u .. 3 u + 2.  The threads of a
// pair (adjacent lanes, h even in the first) swap the low half of the odd one's 48 bits,
// then the even thread stores words 3 u and 3 u + 1 and the odd thread word 3 u + 2.
// Both lanes of every pair must execute this together.
__device__ __forceinline__ void store_3bit_half(const uint32_t (&q)[16], int h, uint32_t* row_words) {
  uint32_t lo = 0, hi = 0;  // bits [0, 32) and [32, 48) of this half
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (3 * i + 3 <= 32) lo |= q[i] << (3 * i);
    else if (3 * i >= 32) hi |= q[i] << (3 * i - 32);
    else {
      lo |= q[i] << (3 * i);
      hi |= q[i] >> (32 - 3 * i);
    }
  }
  const uint32_t other = static_cast<uint32_t>(
      __builtin_amdgcn_mov_dpp(static_cast<int>(lo), 0xB1, 0xF, 0xF, false));  // quad_perm [1, 0, 3, 2]
  uint32_t* w = row_words + 3 * (h >> 1);
  if ((h & 1) == 0) {
    w[0] = lo;
    w[1] = (hi & 0xFFFFu) | (other << 16);
  } else {
    w[2] = (lo >> 16) | (hi << 16);
  }
}

// 3-bit K codes: a thread keeps the column of 16 channels 16 h .. (its zeros and
// reciprocals in registers) over rows t = tid / (d / 16), + 256 / (d / 16), ...
template <typename T>
__device__ __forceinline__ void pack_k_3bit(const T* tile, const float* ks, const float* kz, int d, int G, int ld,
                                            uint32_t* codes, int64_t row0, int tid) {
  const int lh = ld - 4, wpr = d * 3 / 32;  // 16-code halves per row (a power of two), words per row
  const int h = tid & ((1 << lh) - 1), c0 = 16 * h, rstep = kQuantThreads >> lh;
  float z[16], r[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    z[i] = kz[c0 + i];
    r[i] = scale_reciprocal(ks[c0 + i]);
  }
  for (int t = tid >> lh; t < G; t += rstep) {  // the lanes of a pair share t
    float x[16];
    load_run<16>(tile + (t << ld) + c0, x);
    uint32_t q[16];
    bool ok[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      ok[i] = true;
      q[i] = quant_biased_certified<3>(x[i], z[i], r[i], ok[i]) & 7u;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)  // the division where a lane could not certify (wave-uniform test)
      if (__builtin_amdgcn_ballot_w64(!ok[i]))
        if (!ok[i]) q[i] = quant_code(x[i], ks[c0 + i], z[i], 3);
    store_3bit_half(q, h, codes + (row0 + t) * wpr);
  }
}

// 3-bit V codes: a thread forms the 16 codes of channels 16 h .. 16 h + 15 of one token
// (one group's parameters, since G >= 16) and stores them with store_3bit_half.
template <typename T>
__device__ __forceinline__ void pack_v_3bit(const T* tile, const float* vs, const float* vz, int d, int G, int ld,
                                            int lg, uint32_t* codes, int64_t row0, int tid) {
  const int lh = ld - 4, wpr = d * 3 / 32;               // 16-code halves (a power of two) and words per row
  for (int j = tid; j < (G << lh); j += kQuantThreads) {  // G d / 16 is even: pairs stay together
    const int t = j >> lh, h = j & ((1 << lh) - 1), c0 = 16 * h;
    const int gi = (t << (ld - lg)) + (c0 >> lg);
    const float s = vs[gi], z = vz[gi], r = scale_reciprocal(s);
    float x[16];
    load_run<16>(tile + (t << ld) + c0, x);
    uint32_t q[16];
    bool ok[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      ok[i] = true;
      q[i] = quant_biased_certified<3>(x[i], z, r, ok[i]) & 7u;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)  // the division where a lane could not certify (wave-uniform test)
      if (__builtin_amdgcn_ballot_w64(!ok[i]))
        if (!ok[i]) q[i] = quant_code(x[i], s, z, 3);
    store_3bit_half(q, h, codes + (row0 + t) * wpr);
  }
}

// Two consecutive tile elements as float32 (one 4-byte LDS read for bf16, 8 for float32)
template <typename T>
__device__ __forceinline__ void load_pair(const T* p, float& a, float& b) {
  if constexpr (sizeof(T) == 2) {
    const uint32_t u = *reinterpret_cast<const uint32_t*>(p);
    a = __uint_as_float(u << 16);
    b = __uint_as_float(u & 0xFFFF0000u);
  } else {
    const float2 v = *reinterpret_cast<const float2*>(p);
    a = v.x;
    b = v.y;
  }
}

// Minimum and maximum of the elements of a 16-byte chunk (8 bf16 or 4 float32)
template <typename T>
__device__ __forceinline__ void chunk_minmax(uint4 u, float& mn, float& mx) {
  constexpr int N = 16 / static_cast<int>(sizeof(T));
  float x[N];
  if constexpr (sizeof(T) == 2) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = __uint_as_float(w[k] << 16);
      x[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
  } else {
    x[0] = __uint_as_float(u.x); x[1] = __uint_as_float(u.y); x[2] = __uint_as_float(u.z); x[3] = __uint_as_float(u.w);
  }
  mn = x[0];
  mx = x[0];
#pragma unroll
  for (int i = 1; i < N; ++i) {
    mn = fminf(mn, x[i]);
    mx = fmaxf(mx, x[i]);
  }
}

// Extrema of a run of M 16-byte chunks, visited from chunk (lane M / 16) mod M on
template <typename T, int M>
__device__ __forceinline__ void run_minmax(const uint4* run, int lane, float& mn, float& mx) {
  const int rot = (lane * M / 16) & (M - 1);
  chunk_minmax<T>(run[rot], mn, mx);
#pragma unroll
  for (int k = 1; k < M; ++k) {
    float a, b;
    chunk_minmax<T>(run[(rot + k) & (M - 1)], a, b);
    mn = fminf(mn, a);
    mx = fmaxf(mx, b);
  }
}

// Lane l receives lane l - N of its row of 16 (bound_ctrl: lanes with no such source read
// 0, and only lanes whose sources are all in the row use the result)
template <int N>
__device__ __forceinline__ float row_shr(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x110 + N, 0xF, 0xF, true));
}

// The same computation restructured for throughput; its output is identical to
// quant_pack_kernel's.  The min and max instructions order -0 below +0 and skip quiet
// NaNs, so a group's extrema do not depend on the order its elements are visited in, and
// the restructured kernel visits them in whichever order suits the hardware:
//  - V groups: each thread takes a contiguous run of the tile (a group is 256 / d runs in
//    adjacent lanes, joined by row shifts), reading its 16-byte chunks from a rotated
//    start so that the lanes of a row hit different LDS banks;
//  - K channels: two channels per thread (one 4- or 8-byte read per token) over a slice
//    of the group's tokens, the P = 512 / d slices then combined per channel.
// Codes: with 2-, 4- or 8-bit codes a word holds whole codes of consecutive channels, so a
// thread keeps one K word column (its channels' parameters in registers for all its
// rows), a V word reads one group's parameters, a word's elements come from one vector
// LDS read and its codes from the certified reciprocal product (quant_biased_certified);
// 16-bit codes divide; 3-bit codes (whose words straddle) are formed 16 per thread, the
// lanes of a pair completing each other's words (pack_k_3bit, pack_v_3bit).  Requires d
// and G powers of two with 32 <= d <= 256 and G >= 16, a tile of 4 to 32 KB, no more LDS
// than a workgroup may allocate (160 KB on gfx950) and 16-byte aligned sources (the
// launch checks; other shapes take quant_pack_kernel).
template <typename T, int M, bool K3>
__global__ void __launch_bounds__(kQuantThreads)
quant_pack_fast_kernel(const T* __restrict__ k_src, const T* __restrict__ v_src, int64_t src_rows,
                       int64_t src_begin, int d, int G, int k_bits, int v_bits, int param_f32, int64_t capacity,
                       int64_t dst_begin, uint32_t* __restrict__ k_codes, uint32_t* __restrict__ v_codes,
                       void* k_scale, void* k_zero, void* v_scale, void* v_zero) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  constexpr int n = M * kQuantThreads * 16 / static_cast<int>(sizeof(T));  // G d elements
  T* kt = reinterpret_cast<T*>(smem_raw);             // [G][d]
  T* vt = kt + n;                                     // [G][d]
  float* ks = reinterpret_cast<float*>(vt + n);       // [d]
  float* kz = ks + d;                                 // [d]
  float* vs = kz + d;                                 // [G][d/G]
  float* vz = vs + d;                                 // [G][d/G]
  float* vmn = vz + d;                                // [G][d/G] V group extrema
  float* vmx = vmn + d;                               // [G][d/G]
  float* kmn = vmx + d;                               // [512/d][d] K slice extrema
  float* kmx = kmn + 2 * kQuantThreads;               // [512/d][d]
  const int tid = threadIdx.x;
  const int grp = blockIdx.x, bh = blockIdx.y;
  const int ld = __builtin_ctz(d), lg = __builtin_ctz(G);  // d and G are powers of two
  const int64_t src_base = (static_cast<int64_t>(bh) * src_rows + src_begin + static_cast<int64_t>(grp) * G) * d;
  const int64_t dst_tok0 = dst_begin + static_cast<int64_t>(grp) * G;
  const int64_t row0 = static_cast<int64_t>(bh) * capacity + dst_tok0;  // first destination token row

  {  // both tiles, 16 bytes per load
    const uint4* k4 = reinterpret_cast<const uint4*>(k_src + src_base);
    const uint4* v4 = reinterpret_cast<const uint4*>(v_src + src_base);
    uint4* kt4 = reinterpret_cast<uint4*>(kt);
    uint4* vt4 = reinterpret_cast<uint4*>(vt);
    uint4 a[M], b[M];
#pragma unroll
    for (int i = 0; i < M; ++i) {
      a[i] = k4[i * kQuantThreads + tid];
      b[i] = v4[i * kQuantThreads + tid];
    }
#pragma unroll
    for (int i = 0; i < M; ++i) {
      kt4[i * kQuantThreads + tid] = a[i];
      vt4[i * kQuantThreads + tid] = b[i];
    }
  }
  __syncthreads();

  // V: thread tid takes the run of G d / 256 elements (M = 1, 2, 4 or 8 chunks of 16
  // bytes) that starts at element tid G d / 256; a group is 256 / d such runs, in
  // adjacent lanes of one 16-lane row.  Each lane starts at chunk tid M / 16 of its run
  // (mod M), so the 16 lanes of a row read 16 different 16-byte bank columns at every step.
  {
    float mn, mx;
    run_minmax<T, M>(reinterpret_cast<const uint4*>(vt) + tid * M, tid, mn, mx);
    const int pv = kQuantThreads >> ld;  // runs per group: 1, 2, 4 or 8
    if (pv > 1) {
      mn = fminf(mn, row_shr<1>(mn));
      mx = fmaxf(mx, row_shr<1>(mx));
    }
    if (pv > 2) {
      mn = fminf(mn, row_shr<2>(mn));
      mx = fmaxf(mx, row_shr<2>(mx));
    }
    if (pv > 4) {
      mn = fminf(mn, row_shr<4>(mn));
      mx = fmaxf(mx, row_shr<4>(mx));
    }
    if ((tid & (pv - 1)) == pv - 1) {
      vmn[tid >> (8 - ld)] = mn;
      vmx[tid >> (8 - ld)] = mx;
    }
  }

  // K: thread (pair cp, slice p) takes channels 2 cp, 2 cp + 1 over tokens [p span, (p + 1) span)
  const int P = 2 * kQuantThreads >> ld, span = G >> (9 - ld);
  {
    const int cp = tid & ((d >> 1) - 1), p = tid >> (ld - 1);
    const T* col = kt + 2 * cp + ((p * span) << ld);
    float mn0, mn1;
    load_pair(col, mn0, mn1);
    float mx0 = mn0, mx1 = mn1;
#pragma unroll 4
    for (int t = 1; t < span; ++t) {
      float a, b;
      load_pair(col + (t << ld), a, b);
      mn0 = fminf(mn0, a);
      mx0 = fmaxf(mx0, a);
      mn1 = fminf(mn1, b);
      mx1 = fmaxf(mx1, b);
    }
    reinterpret_cast<float2*>(kmn)[tid] = make_float2(mn0, mn1);  // kmn[p d + 2 cp + {0, 1}]
    reinterpret_cast<float2*>(kmx)[tid] = make_float2(mx0, mx1);
  }
  __syncthreads();
  for (int q = tid; q < 2 * d; q += kQuantThreads) {  // K channel q, or V group q - d: the parameters
    float s, z;
    if (q < d) {
      float mn = kmn[q], mx = kmx[q];
      for (int p = 1; p < P; ++p) {
        mn = fminf(mn, kmn[(p << ld) + q]);
        mx = fmaxf(mx, kmx[(p << ld) + q]);
      }
      group_params<T>(mn, mx, k_bits, param_f32, s, z);
      ks[q] = s;
      kz[q] = z;
      const int64_t pi = ((static_cast<int64_t>(bh) * (capacity >> lg) + (dst_tok0 >> lg)) << ld) + q;
      store_param(k_scale, param_f32, pi, s);
      store_param(k_zero, param_f32, pi, z);
    } else {
      const int j = q - d;
      group_params<T>(vmn[j], vmx[j], v_bits, param_f32, s, z);
      vs[j] = s;
      vz[j] = z;
      const int64_t pi = (row0 << (ld - lg)) + j;  // (row0 + j / vg) vg + j mod vg, vg = d / G
      store_param(v_scale, param_f32, pi, s);
      store_param(v_zero, param_f32, pi, z);
    }
  }
  __syncthreads();

  // 3-bit K codes (K3, an instance of its own: its 16-channel columns need more
  // registers than every other width) or the word columns of the other widths
  if constexpr (K3) pack_k_3bit(kt, ks, kz, d, G, ld, k_codes, row0, tid);
  else switch (k_bits) {  // wave-uniform; the bit widths are validated
    case 2: pack_k_columns<2>(kt, ks, kz, d, G, ld, k_codes, row0, tid); break;
    case 4: pack_k_columns<4>(kt, ks, kz, d, G, ld, k_codes, row0, tid); break;
    case 8: pack_k_columns<8>(kt, ks, kz, d, G, ld, k_codes, row0, tid); break;
    default: pack_k_columns<16>(kt, ks, kz, d, G, ld, k_codes, row0, tid); break;
  }
  switch (v_bits) {
    case 2: pack_v_words<2>(vt, vs, vz, d, G, ld, lg, v_codes, row0, tid); break;
    case 3: pack_v_3bit(vt, vs, vz, d, G, ld, lg, v_codes, row0, tid); break;
    case 4: pack_v_words<4>(vt, vs, vz, d, G, ld, lg, v_codes, row0, tid); break;
    case 8: pack_v_words<8>(vt, vs, vz, d, G, ld, lg, v_codes, row0, tid); break;
    default: pack_v_words<16>(vt, vs, vz, d, G, ld, lg, v_codes, row0, tid); break;
  }
}

// quant_pack_fast_kernel<T, M, K3> for M = chunks: one workgroup per tile
template <typename T, int M>
static vc_status launch_quant_fast_m(const T* k_src, const T* v_src, int64_t src_rows, int64_t src_begin, int d,
                                     int G, const vc_ckv* c, int pf32, int64_t dst_begin, dim3 grid, size_t flds,
                                     hipStream_t stream) {
  if (c->k_bits == 3)
    hipLaunchKernelGGL((quant_pack_fast_kernel<T, M, true>), grid, dim3(kQuantThreads), flds, stream, k_src, v_src,
                       src_rows, src_begin, d, G, c->k_bits, c->v_bits, pf32, c->capacity, dst_begin, c->k_codes,
                       c->v_codes, c->k_scale, c->k_zero, c->v_scale, c->v_zero);
  else
    hipLaunchKernelGGL((quant_pack_fast_kernel<T, M, false>), grid, dim3(kQuantThreads), flds, stream, k_src, v_src,
                       src_rows, src_begin, d, G, c->k_bits, c->v_bits, pf32, c->capacity, dst_begin, c->k_codes,
                       c->v_codes, c->k_scale, c->k_zero, c->v_scale, c->v_zero);
  return VC_OK;
}

template <typename T>
static vc_status launch_quant_fast(int chunks, const T* k_src, const T* v_src, int64_t src_rows, int64_t src_begin,
                                   int d, int G, const vc_ckv* c, int pf32, int64_t dst_begin, dim3 grid, size_t flds,
                                   hipStream_t stream) {
  switch (chunks) {
    case 1: return launch_quant_fast_m<T, 1>(k_src, v_src, src_rows, src_begin, d, G, c, pf32, dst_begin, grid, flds, stream);
    case 2: return launch_quant_fast_m<T, 2>(k_src, v_src, src_rows, src_begin, d, G, c, pf32, dst_begin, grid, flds, stream);
    case 4: return launch_quant_fast_m<T, 4>(k_src, v_src, src_rows, src_begin, d, G, c, pf32, dst_begin, grid, flds, stream);
    default: return launch_quant_fast_m<T, 8>(k_src, v_src, src_rows, src_begin, d, G, c, pf32, dst_begin, grid, flds, stream);
  }
}

// LDS a workgroup may allocate on the current device (queried once per device)
static size_t max_lds_per_block() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 65536;
  if (cached[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || v <= 0) v = 65536;
    cached[dev] = v;
  }
  return static_cast<size_t>(cached[dev]);
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
  const int d = c->d;
  const size_t flds = 2 * tile_bytes + 6 * static_cast<size_t>(d) * sizeof(float) + 4 * kQuantThreads * sizeof(float);
  const bool pow2_d = d >= 32 && d <= kQuantThreads && (d & (d - 1)) == 0;
  const bool pow2_g = G >= 16 && (G & (G - 1)) == 0;
  const bool fast = pow2_d && pow2_g && tile_bytes >= 16 * kQuantThreads && flds <= max_lds_per_block() &&
                    reinterpret_cast<uintptr_t>(k_src) % 16 == 0 &&
                    reinterpret_cast<uintptr_t>(v_src) % 16 == 0;
  if (fast) {
    const int chunks = static_cast<int>(tile_bytes / (16 * kQuantThreads));  // 1, 2, 4 or 8
    st = c->kv_dtype == VC_F32
             ? launch_quant_fast<float>(chunks, static_cast<const float*>(k_src), static_cast<const float*>(v_src),
                                        src_rows, src_begin, d, G, c, pf32, dst_begin, grid, flds, stream)
             : launch_quant_fast<bf16_t>(chunks, static_cast<const bf16_t*>(k_src),
                                         static_cast<const bf16_t*>(v_src), src_rows, src_begin, d, G, c, pf32,
                                         dst_begin, grid, flds, stream);
    if (st != VC_OK) return st;
    VC_LAUNCHED("quant_pack_fast_kernel");
    return VC_OK;
  }
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
