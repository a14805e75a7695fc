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
};

// per-sequence lengths, clamped to [0, n_main] and [0, tail_len]
__device__ __forceinline__ int64_t dec_main_len(const DecodeArgs& a, int b) {
  return a.main_lens ? min(max(static_cast<int64_t>(a.main_lens[b]), static_cast<int64_t>(0)), a.n_main) : a.n_main;
}
__device__ __forceinline__ int64_t dec_tail_len(const DecodeArgs& a, int b) {
  return a.tail_lens ? min(max(static_cast<int64_t>(a.tail_lens[b]), static_cast<int64_t>(0)), a.tail_len)
                     : a.tail_len;
}

// Tail rows (full precision, bf16, d = 128) of one (sequence, kv-head), H <= 16
// q-heads; writes the partial of `split`.  Rows go in chunks of 64, all in
// parallel: one thread per (head, row) score, one wave per head for the chunk's
// softmax (online across chunks), and for the outputs 16 lanes per head covering
// 8 channels each, the chunk's rows strided over the remaining threads and summed
// in a fixed order through LDS.  lds: >= 5 * 1024 floats of scratch.
__device__ void decode_tail_partial_d128(const DecodeArgs& a, int bh, int split, float* lds) {
  constexpr int D = 128, TC = 64;
  const int b = bh / a.Hkv, hk = bh % a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = a.H;
  const int tl = static_cast<int>(min(dec_tail_len(a, b), a.tail_cap));
  float* s_q = lds;                    // [16][128] scaled queries
  float* s_p = lds + 16 * D;           // [16][64] scores, then probabilities
  float* s_red = lds + 16 * D + 16 * TC;  // [16 * RS][128] per-row-set output sums
  float* s_st = s_red + 16 * D;        // [3][16] running max, running sum, rescale
  const bf16_t* q = static_cast<const bf16_t*>(a.q) + (static_cast<int64_t>(b) * a.Hkv * H + hk * H) * D;
  const bf16_t* tk = static_cast<const bf16_t*>(a.tail_k) + static_cast<int64_t>(bh) * a.tail_cap * D;
  const bf16_t* tv = static_cast<const bf16_t*>(a.tail_v) + static_cast<int64_t>(bh) * a.tail_cap * D;
  for (int e = tid; e < H * D; e += kDecThreads) s_q[e] = bf16_to_f32(q[e]) * a.qscale;
  if (tid < H) {
    s_st[tid] = -INFINITY;
    s_st[16 + tid] = 0.f;
  }
  const int RS = 16 / H;  // row sets per head in the output pass
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  for (int r0 = 0; r0 < tl; r0 += TC) {
    const int nr = min(TC, tl - r0);
    __syncthreads();
    // scores
    for (int e = tid; e < H * TC; e += kDecThreads) {
      const int hh = e / TC, r = e % TC;
      float sc = -INFINITY;
      if (r < nr) {
        const uint4* kr = reinterpret_cast<const uint4*>(tk + static_cast<int64_t>(r0 + r) * D);
        const float* qh = s_q + hh * D;
        float x = 0.f;
#pragma unroll
        for (int v = 0; v < D / 8; ++v) {
          const uint4 w = kr[v];
          const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const float kv = __uint_as_float((c & 1) ? (ws[c >> 1] & 0xFFFF0000u) : (ws[c >> 1] << 16));
            x = fmaf(qh[8 * v + c], kv, x);
          }
        }
        sc = x;
      }
      s_p[hh * TC + r] = sc;
    }
    __syncthreads();
    // softmax of the chunk, one wave per head
    for (int hh = wave; hh < H; hh += kDecThreads / 64) {
      const float v = s_p[hh * TC + lane];
      const float mo = s_st[hh];
      const float mn = fmaxf(mo, warp_max(v));
      const float p = v == -INFINITY ? 0.f : exp2f(v - mn);
      s_p[hh * TC + lane] = p;
      const float sum = warp_sum(p);
      if (lane == 0) {
        const float sc = mo == -INFINITY ? 0.f : exp2f(mo - mn);
        s_st[32 + hh] = sc;
        s_st[16 + hh] = s_st[16 + hh] * sc + sum;
        s_st[hh] = mn;
      }
    }
    __syncthreads();
    // weighted rows: thread (head, row set, 8-channel group)
    if (tid < 16 * H * RS) {
      const int c8 = tid & 15, g = tid >> 4, hh = g / RS, rs = g % RS;
      float part[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) part[c] = 0.f;
      for (int r = rs; r < nr; r += RS) {
        const float p = s_p[hh * TC + r];
        const uint4 w = *reinterpret_cast<const uint4*>(tv + static_cast<int64_t>(r0 + r) * D + 8 * c8);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int c = 0; c < 8; ++c)
          part[c] = fmaf(p, __uint_as_float((c & 1) ? (ws[c >> 1] & 0xFFFF0000u) : (ws[c >> 1] << 16)), part[c]);
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) s_red[g * D + 8 * c8 + c] = part[c];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = tid + kDecThreads * j;
      if (e < H * D) {
        const int hh = e / D, c = e % D;
        float v = 0.f;
        for (int rs = 0; rs < RS; ++rs) v += s_red[(hh * RS + rs) * D + c];
        acc[j] = fmaf(acc[j], s_st[32 + hh], v);
      }
    }
  }
  __syncthreads();
  const int64_t pbase = static_cast<int64_t>(bh) * a.splits + split;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int e = tid + kDecThreads * j;
    if (e < H * D) a.part_o[pbase * H * D + e] = acc[j];
  }
  if (tid < H) {
    a.part_ml[(pbase * H + tid) * 2] = s_st[tid];
    a.part_ml[(pbase * H + tid) * 2 + 1] = s_st[16 + tid];
  }
}

// Merge of the split partials of one (sequence, kv-head) per workgroup, in split
// order (the result does not depend on which split finished first).  A kernel of
// its own: handing the partials from one workgroup to another inside the decode
// kernel would need a device-scope release by every workgroup, which on a part
// with several L2 caches costs a write-back of its L2 each time.
template <typename T>
__global__ void __launch_bounds__(kDecThreads) decode_merge_kernel(DecodeArgs a) {
  // one workgroup per (sequence, kv-head) and q-head of it; splits <= 64
  __shared__ float s_w[kDecMaxSplits];
  __shared__ float s_fin[2];
  __shared__ float s_part[kDecThreads];
  const int bh = blockIdx.x, h = blockIdx.y;
  const int b = bh / a.Hkv, hk = bh % a.Hkv;
  const int H = a.H, d = a.d, S = a.splits;
  const int tid = threadIdx.x;
  // tpo threads per output channel, each summing a contiguous share of the splits;
  // the first 16 of its partials are loaded before the weights are known, so the
  // two rounds of global loads overlap
  const int tpo = kDecThreads / d;
  const int c = tid % d, part = tid / d;
  const int per = (S + tpo - 1) / tpo;
  const int s_lo = part < tpo ? part * per : S, s_hi = min(S, s_lo + per);
  const float* p = a.part_o + (static_cast<int64_t>(bh) * S * H + h) * d + c;
  const int64_t stride = static_cast<int64_t>(H) * d;
  float v[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = s_lo + j < s_hi ? p[(s_lo + j) * stride] : 0.f;
  if (tid < 64) {  // split weights: a wave holds one split per lane
    float m = -INFINITY, l = 0.f;
    if (tid < S) {
      const float2 mv = reinterpret_cast<const float2*>(a.part_ml)[(static_cast<int64_t>(bh) * S + tid) * H + h];
      m = mv.x;
      l = mv.y;
    }
    const float M = warp_max(m);
    const float w = m == -INFINITY ? 0.f : exp2f(m - M);
    const float L = warp_sum(l * w);
    if (tid < S) s_w[tid] = w;
    if (tid == 0) {
      s_fin[0] = M;
      s_fin[1] = L;
    }
  }
  __syncthreads();
  float O = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (s_lo + j < s_hi) O = fmaf(v[j], s_w[s_lo + j], O);
  for (int s0 = s_lo + 16; s0 < s_hi; s0 += 16) {
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = p[min(s0 + j, s_hi - 1) * stride];
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (s0 + j < s_hi) O = fmaf(v[j], s_w[s0 + j], O);
  }
  s_part[tid] = O;
  __syncthreads();
  if (tid < d) {
    float sum = 0.f;
    for (int q = 0; q < tpo; ++q) sum += s_part[q * d + tid];
    const float L = s_fin[1];
    const int64_t oi = (static_cast<int64_t>(b) * a.Hkv * H + hk * H + h) * d + tid;
    Elem<T>::store(static_cast<T*>(a.out), oi, L > 0.f ? sum / L : 0.f);
    if (a.lse && tid == 0)
      a.lse[static_cast<int64_t>(b) * a.Hkv * H + hk * H + h] = L > 0.f ? (s_fin[0] + log2f(L)) * kLn2 : -INFINITY;
  }
}

}  // namespace vc
