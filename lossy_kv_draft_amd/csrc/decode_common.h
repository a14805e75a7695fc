// Pieces shared by the decode kernels: arguments, the dense tail pass and the
// fixed-order merge of per-split softmax partials.
#pragma once

#include "common.h"

namespace vc {

constexpr int kDecThreads = 256;
constexpr int kDecMaxSplits = 64;     // partials per (sequence, kv-head), tail included

struct DecodeArgs {
  // compressed cache
  const uint32_t* k_codes;
  const uint32_t* v_codes;
  const void* k_scale;
  const void* k_zero;
  const void* v_scale;
  const void* v_zero;
  const void* k_kept;
  const void* v_kept;
  const void* tail_k;
  const void* tail_v;
  int64_t capacity, tail_cap, n_main, tail_len;
  const int32_t* main_lens;
  const int32_t* tail_lens;
  int k_bits, v_bits, G;
  // problem
  const void* q;
  void* out;
  float* lse;
  int Hkv, H, d;
  float qscale;  // sm_scale * log2(e): scores are kept in base-2 units
  int splits;    // partials per (sequence, kv-head)
  int64_t chunk; // compressed rows per split
  // workspace
  float* part_o;   // [B*Hkv][splits][H][d]   unnormalized outputs
  float* part_ml;  // [B*Hkv][splits][H][2]   running max (base 2) and sum
  int* counters;   // [B*Hkv]                 splits finished (reset to 0 by the merger)
};

__device__ __forceinline__ int64_t dec_main_len(const DecodeArgs& a, int b) {
  return a.main_lens ? a.main_lens[b] : a.n_main;
}
__device__ __forceinline__ int64_t dec_tail_len(const DecodeArgs& a, int b) {
  return a.tail_lens ? a.tail_lens[b] : a.tail_len;
}

// Tail rows (full precision) of one (sequence, kv-head): each wave owns heads
// wave, wave + 4, ...; lanes own channel pairs.  Writes the partial of `split`.
template <typename T>
__device__ void decode_tail_partial(const DecodeArgs& a, int bh, int split) {
  const int b = bh / a.Hkv, hk = bh % a.Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int d = a.d, H = a.H;
  const int64_t tl = dec_tail_len(a, b);
  const T* q = static_cast<const T*>(a.q);
  const T* tk = static_cast<const T*>(a.tail_k) + static_cast<int64_t>(bh) * a.tail_cap * d;
  const T* tv = static_cast<const T*>(a.tail_v) + static_cast<int64_t>(bh) * a.tail_cap * d;
  const int64_t pbase = static_cast<int64_t>(bh) * a.splits + split;
  for (int h = wave; h < H; h += kDecThreads / 64) {
    float qv[4], ov[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int c = lane + 64 * j;
      qv[j] = c < d ? Elem<T>::load(q, (static_cast<int64_t>(b) * a.Hkv * H + hk * H + h) * d + c) * a.qscale : 0.f;
      ov[j] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    for (int64_t t = 0; t < tl; ++t) {
      float x = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int c = lane + 64 * j;
        if (c < d) x = fmaf(qv[j], Elem<T>::load(tk, t * d + c), x);
      }
      x = warp_sum(x);
      float mn = fmaxf(m, x);
      float al = exp2f(m - mn);
      float p = exp2f(x - mn);
      l = l * al + p;
      m = mn;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int c = lane + 64 * j;
        if (c < d) ov[j] = fmaf(p, Elem<T>::load(tv, t * d + c), ov[j] * al);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int c = lane + 64 * j;
      if (c < d) a.part_o[(pbase * H + h) * d + c] = ov[j];
    }
    if (lane == 0) {
      a.part_ml[(pbase * H + h) * 2] = m;
      a.part_ml[(pbase * H + h) * 2 + 1] = l;
    }
  }
}

// Called by every block after writing its partial.  The last block of a
// (sequence, kv-head) to arrive merges all partials in split order (so the result
// does not depend on arrival order), writes out/lse and resets the counter.
template <typename T>
__device__ void decode_finish(const DecodeArgs& a, int bh) {
  __shared__ int s_last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) s_last = (atomicAdd(a.counters + bh, 1) == a.splits - 1);
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const int b = bh / a.Hkv, hk = bh % a.Hkv;
  const int H = a.H, d = a.d;
  T* out = static_cast<T*>(a.out);
  for (int i = threadIdx.x; i < H * d; i += blockDim.x) {
    const int h = i / d;
    float M = -INFINITY;
    for (int s = 0; s < a.splits; ++s)
      M = fmaxf(M, a.part_ml[((static_cast<int64_t>(bh) * a.splits + s) * H + h) * 2]);
    float L = 0.f, O = 0.f;
    for (int s = 0; s < a.splits; ++s) {
      const int64_t ps = static_cast<int64_t>(bh) * a.splits + s;
      const float m = a.part_ml[(ps * H + h) * 2];
      const float w = (m == -INFINITY) ? 0.f : exp2f(m - M);
      L = fmaf(a.part_ml[(ps * H + h) * 2 + 1], w, L);
      O = fmaf(a.part_o[ps * H * d + i], w, O);
    }
    const int64_t oi = (static_cast<int64_t>(b) * a.Hkv * H + hk * H) * d + i;
    Elem<T>::store(out, oi, L > 0.f ? O / L : 0.f);
    if (a.lse && (i % d) == 0)
      a.lse[static_cast<int64_t>(b) * a.Hkv * H + hk * H + h] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
  }
  if (threadIdx.x == 0) a.counters[bh] = 0;
}

}  // namespace vc
