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

// Partial of the full-precision tail rows (bf16, d = 128) for q-head h of one
// (sequence, kv-head), by the 256 threads of a merge workgroup, float32 throughout.
// Rows go in chunks of 64 with an online softmax across chunks.  The partial is on
// the path of every decode call after the decode kernel, so the work is spread to
// keep the chain of dependent steps short: the query slice, a chunk's K rows and
// its V values are loaded at once (tail_load, issued before the merge's own loads),
// then (tail_chunk)
// * scores: four threads per row, 32 channels each, summed over the quad;
// * every wave takes the chunk's maximum and the sum of its probabilities itself
//   (one row per lane), so all threads know them;
// * outputs: thread (c, part) sums channel c over the rows of parity `part`.
// The running maximum and sum end in every thread, the output share of channel c
// in thread (c, part).
// Max and sum over the 64 lanes of a wave without LDS round trips: DPP exchanges within
// each row of 16 lanes (xor 1, xor 2, the mirrors of 8 and of 16), then the lane-swap
// instructions across rows.  Every step combines two equal-ranked values (a op b in one
// lane, b op a in its partner), so all 64 lanes end with the same result.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <typename Op>
__device__ __forceinline__ float wave_reduce_dpp(float v, Op op) {
  v = op(v, dpp_mov<0xB1>(v));   // quad_perm [1, 0, 3, 2]
  v = op(v, dpp_mov<0x4E>(v));   // quad_perm [2, 3, 0, 1]
  v = op(v, dpp_mov<0x141>(v));  // row_half_mirror
  v = op(v, dpp_mov<0x140>(v));  // row_mirror
  const unsigned u = __float_as_uint(v);
  const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = op(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const unsigned w = __float_as_uint(v);
  const auto r32 = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return op(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}
__device__ __forceinline__ float wave_max_dpp(float v) {
  return wave_reduce_dpp(v, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  return wave_reduce_dpp(v, [](float a, float b) { return a + b; });
}

struct TailPartial {
  float m, l, o;
};
constexpr int kTailChunk = 64;
struct TailRegs {
  uint4 qw[4], kw[4];             // the query's and a K row's channels 32 quarter .. + 31
  uint32_t vr[kTailChunk / 2];    // V channel c of the rows of parity part (bf16 bits)
};
// Loads of rows [r0, r0 + nr) (0 <= nr <= 64); rows past the end read the last row,
// or with no rows at all the first 256 bytes of the partials (no branch around a
// load, so they issue back to back and ahead of the merge's own loads): their
// scores are dropped and their probabilities are 0.
__device__ __forceinline__ void tail_load(TailRegs& x, const DecodeArgs& a, int bh, int h, int r0, int nr) {
  constexpr int D = 128;
  const int b = bh / a.Hkv, hk = bh % a.Hkv;
  const int tid = threadIdx.x, c = tid % D, part = tid / D, rr = tid >> 2, quarter = tid & 3;
  const bf16_t* q = static_cast<const bf16_t*>(a.q) + (static_cast<int64_t>(b) * a.Hkv * a.H + hk * a.H + h) * D;
  const bool rows = nr > 0;
  const bf16_t* tk = rows ? static_cast<const bf16_t*>(a.tail_k) + static_cast<int64_t>(bh) * a.tail_cap * D
                          : reinterpret_cast<const bf16_t*>(a.part_o);
  const uint16_t* tv = rows ? reinterpret_cast<const uint16_t*>(a.tail_v) + static_cast<int64_t>(bh) * a.tail_cap * D
                            : reinterpret_cast<const uint16_t*>(a.part_o);
  if (!rows) r0 = 0, nr = 1;
  const int kr = min(rr, nr - 1);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    x.qw[u] = reinterpret_cast<const uint4*>(q + 32 * quarter)[u];
    x.kw[u] = reinterpret_cast<const uint4*>(tk + static_cast<int64_t>(r0 + kr) * D + 32 * quarter)[u];
  }
#pragma unroll
  for (int j = 0; j < kTailChunk / 2; ++j) x.vr[j] = tv[static_cast<int64_t>(r0 + min(part + 2 * j, nr - 1)) * D + c];
}
// s_s holds the chunk's scores and s_p its probabilities (two arrays, so that no barrier
// has to separate the reads of the one from the writes of the other); a caller running a
// further chunk places a barrier before it (both arrays are rewritten).
__device__ __forceinline__ void tail_chunk(TailPartial& t, const TailRegs& x, float qscale, int nr, float* s_s,
                                           float* s_p) {
  const int tid = threadIdx.x, lane = tid & 63, part = tid / 128, rr = tid >> 2, quarter = tid & 3;
  auto f32_lo = [](uint32_t w) { return __uint_as_float(w << 16); };
  auto f32_hi = [](uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); };
  float y = 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint32_t qs[4] = {x.qw[u].x, x.qw[u].y, x.qw[u].z, x.qw[u].w};
    const uint32_t ks[4] = {x.kw[u].x, x.kw[u].y, x.kw[u].z, x.kw[u].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      y = fmaf(f32_lo(qs[e]), f32_lo(ks[e]), y);
      y = fmaf(f32_hi(qs[e]), f32_hi(ks[e]), y);
    }
  }
  y += dpp_mov<0xB1>(y);  // the quad's four quarters: xor 1, then xor 2
  y += dpp_mov<0x4E>(y);
  if (quarter == 0) s_s[rr] = y * qscale;
  __syncthreads();
  const float sr = lane < nr ? s_s[lane] : -INFINITY;
  const float mn = fmaxf(t.m, wave_max_dpp(sr));
  const float pr = lane < nr ? exp2f(sr - mn) : 0.f;
  const float lc = wave_sum_dpp(pr);
  if (tid < 64) s_p[lane] = pr;
  __syncthreads();
  const float sc = t.m == -INFINITY ? 0.f : exp2f(t.m - mn);
  float o = t.o * sc;
#pragma unroll
  for (int j = 0; j < kTailChunk / 2; ++j)
    o = fmaf(s_p[part + 2 * j], __uint_as_float(x.vr[j] << 16), o);
  t.o = o;
  t.l = t.l * sc + lc;
  t.m = mn;
}

// Merge of the split partials of one (sequence, kv-head) per workgroup, in split
// order (the result does not depend on which split finished first).  A kernel of
// its own: handing the partials from one workgroup to another inside the decode
// kernel would need a device-scope release by every workgroup, which on a part
// with several L2 caches costs a write-back of its L2 each time.  TAIL: the
// full-precision tail rows (bf16, d = 128) are not in the splits; the workgroup
// computes their partial itself (while its loads of the split partials are in
// flight) and merges it after the splits.
template <typename T, bool TAIL>
__global__ void __launch_bounds__(kDecThreads) decode_merge_kernel(DecodeArgs a) {
  // one workgroup per (sequence, kv-head) and q-head of it; splits (and the tail)
  // <= 64
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
  TailPartial t{-INFINITY, 0.f, 0.f};
  TailRegs tr;
  const int tl = TAIL ? static_cast<int>(min(dec_tail_len(a, b), a.tail_cap)) : 0;
  if (TAIL) tail_load(tr, a, bh, h, 0, min(tl, kTailChunk));
  // the splits' (maximum, sum), one split per lane of the first wave, loaded with the
  // partials so that no later round of global loads waits on them
  float2 mv = make_float2(-INFINITY, 0.f);
  if (tid < S) mv = reinterpret_cast<const float2*>(a.part_ml)[(static_cast<int64_t>(bh) * S + tid) * H + h];
  float v[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = s_lo + j < s_hi ? p[(s_lo + j) * stride] : 0.f;
  if constexpr (TAIL) {
    __shared__ float s_s[kTailChunk], s_p[kTailChunk];
    if (tl > 0) {
      tail_chunk(t, tr, a.qscale, min(tl, kTailChunk), s_s, s_p);
      for (int r0 = kTailChunk; r0 < tl; r0 += kTailChunk) {
        tail_load(tr, a, bh, h, r0, min(tl - r0, kTailChunk));
        __syncthreads();  // every wave is done with the previous chunk's scores and probabilities
        tail_chunk(t, tr, a.qscale, min(tl - r0, kTailChunk), s_s, s_p);
      }
    }
  }
  if (tid < 64) {  // split weights: a wave holds one split per lane (the tail after them)
    float m = -INFINITY, l = 0.f;
    if (tid < S) {
      m = mv.x;
      l = mv.y;
    } else if (TAIL && tid == S) {
      m = t.m;
      l = t.l;
    }
    const float M = wave_max_dpp(m);
    const float w = m == -INFINITY ? 0.f : exp2f(m - M);
    const float L = wave_sum_dpp(l * w);
    if (tid < S + (TAIL ? 1 : 0)) s_w[tid] = w;
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
  if (TAIL && part < 2) O = fmaf(t.o, s_w[S], O);
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
