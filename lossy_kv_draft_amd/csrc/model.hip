// Decoder-layer kernels of the end-to-end draft-and-verify round (vc_model.h).
//
// The VeriCache pages ("VeriCache: Turning Lossy KV Cache into Lossless LLM
// Inference", neuraltrendhub.com summary, "What the paper found") draft with the
// target model on the compressed cache and verify with the same model on the full
// cache; verified output must equal greedy full-KV decoding.  Exactness across the
// two passes needs every kernel here to be batch invariant: an output row is a
// function of its own input row only, computed in an order that does not depend on
// how many rows are processed together.  This file is built without floating-point
// contraction so that every template instantiation rounds identically.
//
// GEMMs C = A W^T on v_mfma_f32_16x16x32_bf16 (W rows are the MFMA A operand, read
// with 16-byte loads; rows of A are the B operand).
//
// gemm_bf16_kernel -- the decode and verify passes, where M is a few rows per
// sequence and the call streams W from HBM once: a workgroup of 8 waves owns 16
// output features and up to 64 rows; wave w reduces its own slice of k (chunks
// [w P, w P + P) of 32, P = ceil(K / 256), fixed by K alone) with W loads issued 8
// chunks ahead, and the 8 partial sums are combined through LDS in a fixed tree.
// Every row's result therefore depends on K only, never on M or the row's place in
// the tile: the k-row verify pass reproduces k one-row greedy steps bit for bit.
//
// gemm_wide_kernel -- prompt processing (thousands of rows): one wave per 16
// features x 128 rows, k ascending; its rounding differs from gemm_bf16_kernel's.

#include "common.h"

namespace vc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

union MP16 {
  uint4 u;
  bf16x8_t v;
};

template <int MT, bool CF32, bool RES>
__global__ void __launch_bounds__(64) gemm_wide_kernel(const bf16_t* __restrict__ A, int64_t lda,
                                                       const bf16_t* __restrict__ W, int64_t ldw, int64_t M, int N,
                                                       int K, void* C, int64_t ldc,
                                                       const bf16_t* R) {  // C may alias R
  const int lane = threadIdx.x, nl = lane & 15, kb = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int64_t m_base = static_cast<int64_t>(blockIdx.y) * 16 * MT;
  const int n = n0 + nl;
  const bool n_ok = n < N;
  const bf16_t* wrow = W + static_cast<int64_t>(n_ok ? n : N - 1) * ldw + 8 * kb;
  const bf16_t* arow[MT];
  bool m_ok[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int64_t m = m_base + 16 * t + nl;
    m_ok[t] = m < M;
    arow[t] = A + (m_ok[t] ? m : M - 1) * lda + 8 * kb;
  }
  f32x4_t acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int k0 = 0; k0 < K; k0 += 32) {
    MP16 a;
    a.u = *reinterpret_cast<const uint4*>(wrow + k0);
    if (!n_ok) a.u = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      MP16 b;
      b.u = *reinterpret_cast<const uint4*>(arow[t] + k0);
      if (!m_ok[t]) b.u = make_uint4(0, 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc[t], 0, 0, 0);
    }
  }
  // acc[t][i] = C[m_base + 16 t + nl][n0 + 4 kb + i]
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    if (!m_ok[t]) continue;
    const int64_t m = m_base + 16 * t + nl;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int nn = n0 + 4 * kb + i;
      if (nn >= N) continue;
      float v = acc[t][i];
      if constexpr (RES) v = v + bf16_to_f32(R[m * ldc + nn]);
      if constexpr (CF32)
        static_cast<float*>(C)[m * ldc + nn] = v;
      else
        static_cast<bf16_t*>(C)[m * ldc + nn] = f32_to_bf16(v);
    }
  }
}

constexpr int kGemmWaves = 8;  // k slices per workgroup
constexpr int kGemmAhead = 8;  // W chunks in flight per wave

// Epilogue of gemm_bf16_kernel: the rounded output (plus residual), or SwiGLU of the
// gate and up halves of an interleaved gate/up projection (each 16-row tile of W
// holds gate rows 8j .. 8j + 7, then up rows 8j .. 8j + 7): C is then the
// activation [M, N / 2], computed from the bf16-rounded gate and up values exactly
// as swiglu_kernel computes it from the stored product.
// kEpiRope: the QKV projection with the rotary embedding and the scatter of
// rope_qkv_kernel in its epilogue; W's q and k rows are permuted so that each 16-row
// tile holds the rotation pairs (j0 .. j0 + 7, j0 + hd/2 .. j0 + hd/2 + 7) of one
// head, the v rows are in their order.
constexpr int kEpiStore = 0, kEpiSwiglu = 1, kEpiRope = 2;

struct RopeArgs {
  int k, Hq, Hkv, hd;
  float log2_theta;
  const int32_t* pos;
  bf16_t* q_out;
  bf16_t* k_dst;
  bf16_t* v_dst;
  int64_t dst_rows;
  const int32_t* row0;
};

// rotation of the pair (x0, x1) of element j at position p, as rope_qkv_kernel does it
__device__ __forceinline__ void rope_pair(float x0, float x1, int j, int hd, float log2_theta, float p, float& y0,
                                          float& y1) {
  const float inv_freq = exp2f(-static_cast<float>(2 * j) / static_cast<float>(hd) * log2_theta);
  float sn, cs;
  sincosf(p * inv_freq, &sn, &cs);
  y0 = x0 * cs - x1 * sn;
  y1 = x1 * cs + x0 * sn;
}

template <int MT, bool CF32, bool RES, int EPI = kEpiStore>
__global__ void __launch_bounds__(512) gemm_bf16_kernel(const bf16_t* __restrict__ A, int64_t lda,
                                                        const bf16_t* __restrict__ W, int64_t ldw, int64_t M, int N,
                                                        int K, void* C, int64_t ldc,
                                                        const bf16_t* R,  // C may alias R
                                                        RopeArgs ra = RopeArgs{}) {
  __shared__ f32x4_t red[kGemmWaves][MT][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nl = lane & 15, kb = lane >> 4;
  const int n0 = blockIdx.y * 16;
  const int64_t m_base = static_cast<int64_t>(blockIdx.x) * 16 * MT;
  const int nk = K >> 5;
  const int P = (nk + kGemmWaves - 1) / kGemmWaves;
  const int c_first = wave * P;
  const int c_end = min(c_first + P, nk);
  const int nblk = (P + kGemmAhead - 1) / kGemmAhead;
  const int n = n0 + nl;
  const bool n_ok = n < N;
  const bf16_t* wrow = W + static_cast<int64_t>(n_ok ? n : N - 1) * ldw + 8 * kb;
  const bf16_t* arow[MT];
  bool m_ok[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int64_t m = m_base + 16 * t + nl;
    m_ok[t] = m < M;
    arow[t] = A + (m_ok[t] ? m : M - 1) * lda + 8 * kb;
  }
  auto chunk_off = [&](int c) { return static_cast<int64_t>(min(c, nk - 1)) * 32; };
  f32x4_t acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  uint4 wv[kGemmAhead];
#pragma unroll
  for (int u = 0; u < kGemmAhead; ++u) wv[u] = *reinterpret_cast<const uint4*>(wrow + chunk_off(c_first + u));
  const uint4 zero = make_uint4(0, 0, 0, 0);
  for (int blk = 0; blk < nblk; ++blk) {
    const int cb = c_first + blk * kGemmAhead;
    uint4 av[kGemmAhead][MT];
#pragma unroll
    for (int u = 0; u < kGemmAhead; ++u)
#pragma unroll
      for (int t = 0; t < MT; ++t) av[u][t] = *reinterpret_cast<const uint4*>(arow[t] + chunk_off(cb + u));
#pragma unroll
    for (int u = 0; u < kGemmAhead; ++u) {
      const bool live = cb + u < c_end;  // wave-uniform: chunks past the slice add exact zeros
      MP16 a;
      a.u = (live && n_ok) ? wv[u] : zero;
      wv[u] = *reinterpret_cast<const uint4*>(wrow + chunk_off(cb + u + kGemmAhead));
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        MP16 b;
        b.u = (live && m_ok[t]) ? av[u][t] : zero;
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc[t], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < MT; ++t) red[wave][t][lane] = acc[t];
  __syncthreads();
  // acc[t][i] of lane ln = C[m_base + 16 t + (ln & 15)][n0 + 4 (ln >> 4) + i]
  auto total = [&](int t, int ln) {
    return ((red[0][t][ln] + red[1][t][ln]) + (red[2][t][ln] + red[3][t][ln])) +
           ((red[4][t][ln] + red[5][t][ln]) + (red[6][t][ln] + red[7][t][ln]));
  };
  if constexpr (EPI == kEpiSwiglu) {
    // lanes 0 .. 31 hold the gate features of the tile, lanes 32 .. 63 the up ones
    for (int e = tid; e < MT * 32; e += 64 * kGemmWaves) {
      const int t = e >> 5, ln = e & 31;
      const int64_t m = m_base + 16 * t + (ln & 15);
      if (m >= M) continue;
      const f32x4_t g = total(t, ln), u = total(t, ln + 32);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = (n0 >> 1) + 4 * (ln >> 4) + i;
        if (2 * j >= N) continue;
        const float gb = bf16_to_f32(f32_to_bf16(g[i])), ub = bf16_to_f32(f32_to_bf16(u[i]));
        static_cast<bf16_t*>(C)[m * ldc + j] = f32_to_bf16(gb / (1.0f + expf(-gb)) * ub);
      }
    }
    return;
  }
  if constexpr (EPI == kEpiRope) {
    const int half = ra.hd / 2;
    const int qk_width = (ra.Hq + ra.Hkv) * ra.hd;
    if (n0 < qk_width) {  // a tile of rotation pairs: lanes 0 .. 31 first halves, 32 .. 63 second
      const int tpb = half / 8;  // tiles per head
      const int h = (n0 / 16) / tpb, j0 = 8 * ((n0 / 16) % tpb);
      for (int e = tid; e < MT * 32; e += 64 * kGemmWaves) {
        const int t = e >> 5, ln = e & 31;
        const int64_t m = m_base + 16 * t + (ln & 15);
        if (m >= M) continue;
        const int b = static_cast<int>(m / ra.k), i = static_cast<int>(m % ra.k);
        const float p = static_cast<float>(ra.pos[m]);
        const int64_t krow = static_cast<int64_t>(ra.row0[b]) + i;
        const bool kv_in = krow >= 0 && krow < ra.dst_rows;
        const f32x4_t x0v = total(t, ln), x1v = total(t, ln + 32);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j = j0 + 4 * (ln >> 4) + q;
          float y0, y1;
          rope_pair(bf16_to_f32(f32_to_bf16(x0v[q])), bf16_to_f32(f32_to_bf16(x1v[q])), j, ra.hd, ra.log2_theta, p,
                    y0, y1);
          bf16_t* dst;
          if (h < ra.Hq) dst = ra.q_out + ((static_cast<int64_t>(b) * ra.Hq + h) * ra.k + i) * ra.hd;
          else if (kv_in) dst = ra.k_dst + ((static_cast<int64_t>(b) * ra.Hkv + (h - ra.Hq)) * ra.dst_rows + krow) * ra.hd;
          else continue;
          dst[j] = f32_to_bf16(y0);
          dst[j + half] = f32_to_bf16(y1);
        }
      }
    } else {  // value rows: scattered as they are
      for (int e = tid; e < MT * 64; e += 64 * kGemmWaves) {
        const int t = e >> 6, ln = e & 63;
        const int64_t m = m_base + 16 * t + (ln & 15);
        if (m >= M) continue;
        const int b = static_cast<int>(m / ra.k), i = static_cast<int>(m % ra.k);
        const int64_t krow = static_cast<int64_t>(ra.row0[b]) + i;
        if (krow < 0 || krow >= ra.dst_rows) continue;
        const f32x4_t v = total(t, ln);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int nn = n0 + 4 * (ln >> 4) + q;
          if (nn >= N) continue;
          const int hv = (nn - qk_width) / ra.hd, c = (nn - qk_width) % ra.hd;
          ra.v_dst[((static_cast<int64_t>(b) * ra.Hkv + hv) * ra.dst_rows + krow) * ra.hd + c] = f32_to_bf16(v[q]);
        }
      }
    }
    return;
  }
  for (int e = tid; e < MT * 64; e += 64 * kGemmWaves) {
    const int t = e >> 6, ln = e & 63;
    const int64_t m = m_base + 16 * t + (ln & 15);
    if (m >= M) continue;
    const f32x4_t v = total(t, ln);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int nn = n0 + 4 * (ln >> 4) + i;
      if (nn >= N) continue;
      float x = v[i];
      if constexpr (RES) x = x + bf16_to_f32(R[m * ldc + nn]);
      if constexpr (CF32)
        static_cast<float*>(C)[m * ldc + nn] = x;
      else
        static_cast<bf16_t*>(C)[m * ldc + nn] = f32_to_bf16(x);
    }
  }
}

// Sum of squares of a row of d bf16 values (d % 8 == 0, 16-byte aligned) by one
// wave: lane l takes the 8-value chunks l, l + 64, ... in order, then the wave's
// fixed butterfly.  Every lane returns the total.
__device__ __forceinline__ float row_sumsq(const bf16_t* xr, int d, int lane) {
  float s = 0.f;
  for (int c = lane; c < d / 8; c += 64) {
    const uint4 v = *reinterpret_cast<const uint4*>(xr + 8 * c);
    const uint32_t ws[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = bf16_to_f32(static_cast<bf16_t>(ws[i] & 0xFFFFu));
      const float hi = bf16_to_f32(static_cast<bf16_t>(ws[i] >> 16));
      s = fmaf(lo, lo, s);
      s = fmaf(hi, hi, s);
    }
  }
  return warp_sum(s);
}

// 8 values x (bf16) times inv times the weights w (bf16), each rounded to bf16
__device__ __forceinline__ uint4 scale_rms8(uint4 x, uint4 w, float inv) {
  const uint32_t xs[4] = {x.x, x.y, x.z, x.w}, ws[4] = {w.x, w.y, w.z, w.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16_t lo = f32_to_bf16(bf16_to_f32(static_cast<bf16_t>(xs[i] & 0xFFFFu)) * inv *
                                  bf16_to_f32(static_cast<bf16_t>(ws[i] & 0xFFFFu)));
    const bf16_t hi = f32_to_bf16(bf16_to_f32(static_cast<bf16_t>(xs[i] >> 16)) * inv *
                                  bf16_to_f32(static_cast<bf16_t>(ws[i] >> 16)));
    o[i] = static_cast<uint32_t>(lo) | (static_cast<uint32_t>(hi) << 16);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// one wave per row (four rows per workgroup), 16-byte loads and stores
__global__ void __launch_bounds__(256) rmsnorm_kernel(const bf16_t* x, const bf16_t* w, int64_t M, int d, float eps,
                                                      bf16_t* y) {
  const int lane = threadIdx.x & 63;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= M) return;
  const bf16_t* xr = x + r * d;
  const float inv = 1.0f / sqrtf(row_sumsq(xr, d, lane) / static_cast<float>(d) + eps);
  for (int c = lane; c < d / 8; c += 64)
    *reinterpret_cast<uint4*>(y + r * d + 8 * c) =
        scale_rms8(*reinterpret_cast<const uint4*>(xr + 8 * c), *reinterpret_cast<const uint4*>(w + 8 * c), inv);
}

// one block per token row: rotary embedding of q and k, scatter of q, k, v
__global__ void __launch_bounds__(256) rope_qkv_kernel(const bf16_t* qkv, int k, int Hq, int Hkv, int hd, float log2_theta,
                                                       const int32_t* pos, bf16_t* q_out, bf16_t* k_dst, bf16_t* v_dst,
                                                       int64_t dst_rows, const int32_t* row0) {
  const int64_t r = blockIdx.x;
  const int b = static_cast<int>(r / k), i = static_cast<int>(r % k);
  const int half = hd / 2;
  const int width = (Hq + 2 * Hkv) * hd;
  const bf16_t* src = qkv + r * width;
  const float p = static_cast<float>(pos[r]);
  const int64_t krow = static_cast<int64_t>(row0[b]) + i;
  const bool kv_in = krow >= 0 && krow < dst_rows;  // rows outside the cache are not written
  const int rot_tasks = (Hq + Hkv) * half;
  for (int t = threadIdx.x; t < rot_tasks + Hkv * hd; t += 256) {
    if (t < rot_tasks) {
      const int h = t / half, j = t % half;  // h < Hq: q head, else k head h - Hq
      float y0, y1;
      rope_pair(bf16_to_f32(src[h * hd + j]), bf16_to_f32(src[h * hd + j + half]), j, hd, log2_theta, p, y0, y1);
      if (h < Hq) {
        bf16_t* dst = q_out + ((static_cast<int64_t>(b) * Hq + h) * k + i) * hd;
        dst[j] = f32_to_bf16(y0);
        dst[j + half] = f32_to_bf16(y1);
      } else if (kv_in) {
        bf16_t* dst = k_dst + ((static_cast<int64_t>(b) * Hkv + (h - Hq)) * dst_rows + krow) * hd;
        dst[j] = f32_to_bf16(y0);
        dst[j + half] = f32_to_bf16(y1);
      }
    } else if (kv_in) {
      const int e = t - rot_tasks, h = e / hd, c = e % hd;
      v_dst[((static_cast<int64_t>(b) * Hkv + h) * dst_rows + krow) * hd + c] = src[(Hq + Hkv + h) * hd + c];
    }
  }
}

__global__ void swiglu_kernel(const bf16_t* gu, int64_t M, int F, bf16_t* out) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= M * F) return;
  const int64_t m = e / F;
  const int j = static_cast<int>(e % F);
  const float g = bf16_to_f32(gu[m * 2 * F + j]);
  const float u = bf16_to_f32(gu[m * 2 * F + F + j]);
  out[e] = f32_to_bf16(g / (1.0f + expf(-g)) * u);
}

__global__ void embed_kernel(const uint4* E, int V, int row_vecs, const int32_t* tokens, int64_t M, uint4* x) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= M * row_vecs) return;
  const int64_t m = e / row_vecs;
  const int c = static_cast<int>(e % row_vecs);
  const int t = tokens[m];
  x[e] = (t >= 0 && t < V) ? E[static_cast<int64_t>(t) * row_vecs + c] : make_uint4(0, 0, 0, 0);
}

__global__ void heads_to_rows_kernel(const bf16_t* o, int H, int k, int hd, int64_t total, bf16_t* out) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= total) return;
  const int c = static_cast<int>(e % hd);
  int64_t t = e / hd;
  const int h = static_cast<int>(t % H);
  t /= H;  // t = b * k + i
  const int64_t b = t / k, i = t % k;
  out[e] = o[((b * H + h) * k + i) * hd + c];
}

__device__ __forceinline__ bool better_idx(float v, int i, float bv, int bi) { return v > bv || (v == bv && i < bi); }

// One workgroup of 16 waves per row: each thread keeps 8 loads (16 bytes each when
// the rows allow it) in flight and its own (max, lowest index); a fixed-order
// reduction over lanes, then waves.  The result is the row's largest logit with the
// lowest index among equal ones, whatever the order of the comparisons.
constexpr int kArgThreads = 1024;
__global__ void __launch_bounds__(kArgThreads) argmax_rows_kernel(const float* logits, int V, int32_t* tok) {
  __shared__ float sv[kArgThreads / 64];
  __shared__ int si[kArgThreads / 64];
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x;
  const float* row = logits + r * V;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  if (V % 4 == 0 && (reinterpret_cast<uintptr_t>(logits) & 15) == 0) {
    const float4* r4 = reinterpret_cast<const float4*>(row);
    const int n4 = V / 4;
    for (int base = 0; base < n4; base += 8 * kArgThreads) {
      float4 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = base + u * kArgThreads + tid;
        x[u] = i < n4 ? r4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = base + u * kArgThreads + tid;
        if (i < n4) {
          if (better_idx(x[u].x, 4 * i, bv, bi)) { bv = x[u].x; bi = 4 * i; }
          if (better_idx(x[u].y, 4 * i + 1, bv, bi)) { bv = x[u].y; bi = 4 * i + 1; }
          if (better_idx(x[u].z, 4 * i + 2, bv, bi)) { bv = x[u].z; bi = 4 * i + 2; }
          if (better_idx(x[u].w, 4 * i + 3, bv, bi)) { bv = x[u].w; bi = 4 * i + 3; }
        }
      }
    }
  } else {
    for (int base = 0; base < V; base += 8 * kArgThreads) {
      float x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int v = base + u * kArgThreads + tid;
        x[u] = v < V ? row[v] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int v = base + u * kArgThreads + tid;
        if (v < V && better_idx(x[u], v, bv, bi)) { bv = x[u]; bi = v; }
      }
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o);
    const int oi = __shfl_xor(bi, o);
    if (better_idx(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
  if ((tid & 63) == 0) { sv[tid >> 6] = bv; si[tid >> 6] = bi; }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kArgThreads / 64; ++w)
      if (better_idx(sv[w], si[w], bv, bi)) { bv = sv[w]; bi = si[w]; }
    tok[r] = bi == 0x7fffffff ? 0 : bi;
  }
}

__global__ void copy_kv_rows_kernel(const uint4* sk, const uint4* sv, int64_t src_rows, const int32_t* src_row0,
                                    uint4* dk, uint4* dv, int64_t dst_rows, const int32_t* dst_row0,
                                    const int32_t* count, int Hkv, int row_vecs, int max_count) {
  const int bh = blockIdx.y;
  const int b = bh / Hkv;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= static_cast<int64_t>(max_count) * row_vecs) return;
  const int j = static_cast<int>(e / row_vecs), c = static_cast<int>(e % row_vecs);
  if (j >= count[b]) return;
  const int64_t sr = static_cast<int64_t>(src_row0[b]) + j, dr = static_cast<int64_t>(dst_row0[b]) + j;
  if (sr < 0 || sr >= src_rows || dr < 0 || dr >= dst_rows) return;  // rows outside a cache are skipped
  const int64_t s = (static_cast<int64_t>(bh) * src_rows + sr) * row_vecs + c;
  const int64_t t = (static_cast<int64_t>(bh) * dst_rows + dr) * row_vecs + c;
  dk[t] = sk[s];
  dv[t] = sv[s];
}

}  // namespace vc

using namespace vc;

static bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

template <int MT>
static void launch_wide(bool cf32, bool res, dim3 grid, hipStream_t s, const bf16_t* A, int64_t lda, const bf16_t* W,
                        int64_t ldw, int64_t M, int N, int K, void* C, int64_t ldc, const bf16_t* R) {
  if (cf32)
    hipLaunchKernelGGL((gemm_wide_kernel<MT, true, false>), grid, dim3(64), 0, s, A, lda, W, ldw, M, N, K, C, ldc, R);
  else if (res)
    hipLaunchKernelGGL((gemm_wide_kernel<MT, false, true>), grid, dim3(64), 0, s, A, lda, W, ldw, M, N, K, C, ldc, R);
  else
    hipLaunchKernelGGL((gemm_wide_kernel<MT, false, false>), grid, dim3(64), 0, s, A, lda, W, ldw, M, N, K, C, ldc, R);
}

template <int MT>
static void launch_inv(bool cf32, bool res, dim3 grid, hipStream_t s, const bf16_t* A, int64_t lda, const bf16_t* W,
                       int64_t ldw, int64_t M, int N, int K, void* C, int64_t ldc, const bf16_t* R) {
  const dim3 blk(64 * kGemmWaves);
  if (cf32)
    hipLaunchKernelGGL((gemm_bf16_kernel<MT, true, false>), grid, blk, 0, s, A, lda, W, ldw, M, N, K, C, ldc, R);
  else if (res)
    hipLaunchKernelGGL((gemm_bf16_kernel<MT, false, true>), grid, blk, 0, s, A, lda, W, ldw, M, N, K, C, ldc, R);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<MT, false, false>), grid, blk, 0, s, A, lda, W, ldw, M, N, K, C, ldc, R);
}

static vc_status gemm_common(bool wide, const void* A, int64_t lda, const void* W, int64_t ldw, int64_t M, int32_t N,
                             int32_t K, void* C, int64_t ldc, int32_t c_dtype, const void* R, void* stream) {
  clear_error();
  VC_REQUIRE(A && W && C, "A / W / C is NULL");
  VC_REQUIRE(M > 0 && N > 0 && K > 0, "bad shape (M %lld, N %d, K %d)", (long long)M, N, K);
  VC_REQUIRE(K % 32 == 0, "K must be a multiple of 32 (got %d)", K);
  VC_REQUIRE(lda >= K && ldw >= K && ldc >= N, "leading dimensions too small");
  VC_REQUIRE(lda % 8 == 0 && ldw % 8 == 0, "lda and ldw must be multiples of 8 elements");
  VC_REQUIRE(aligned16(A) && aligned16(W), "A and W must be 16-byte aligned");
  VC_REQUIRE(valid_dtype(c_dtype), "bad c_dtype");
  VC_REQUIRE(R == nullptr || c_dtype == VC_BF16, "a residual needs a bf16 output");
  const int64_t cap = wide ? 128 : 64;  // rows per workgroup
  const int64_t mt_rows = M >= cap ? cap : ((M + 15) / 16) * 16;
  const int MT = static_cast<int>(mt_rows / 16);
  VC_REQUIRE(cdiv(M, mt_rows) <= (wide ? 65535 : 0x7fffffff) && cdiv(N, 16) <= (wide ? 0x7fffffff : 65535),
             "grid too large");
  const unsigned mtiles = static_cast<unsigned>(cdiv(M, mt_rows)), ntiles = static_cast<unsigned>(cdiv(N, 16));
  // wide: feature tiles along x; batch-invariant: row tiles along x (the workgroups
  // sharing a feature tile run together and read its W rows from L2)
  const dim3 grid = wide ? dim3(ntiles, mtiles) : dim3(mtiles, ntiles);
  hipStream_t s = as_stream(stream);
  const bf16_t* a = static_cast<const bf16_t*>(A);
  const bf16_t* w = static_cast<const bf16_t*>(W);
  const bf16_t* r = static_cast<const bf16_t*>(R);
  const bool cf = c_dtype == VC_F32, res = R != nullptr;
  if (wide) {
    switch (MT) {
      case 1: launch_wide<1>(cf, res, grid, s, a, lda, w, ldw, M, N, K, C, ldc, r); break;
      case 2: launch_wide<2>(cf, res, grid, s, a, lda, w, ldw, M, N, K, C, ldc, r); break;
      case 3: launch_wide<3>(cf, res, grid, s, a, lda, w, ldw, M, N, K, C, ldc, r); break;
      case 4: launch_wide<4>(cf, res, grid, s, a, lda, w, ldw, M, N, K, C, ldc, r); break;
      case 5: launch_wide<5>(cf, res, grid, s, a, lda, w, ldw, M, N, K, C, ldc, r); break;
      case 6: launch_wide<6>(cf, res, grid, s, a, lda, w, ldw, M, N, K, C, ldc, r); break;
      case 7: launch_wide<7>(cf, res, grid, s, a, lda, w, ldw, M, N, K, C, ldc, r); break;
      default: launch_wide<8>(cf, res, grid, s, a, lda, w, ldw, M, N, K, C, ldc, r); break;
    }
  } else {
    switch (MT) {
      case 1: launch_inv<1>(cf, res, grid, s, a, lda, w, ldw, M, N, K, C, ldc, r); break;
      case 2: launch_inv<2>(cf, res, grid, s, a, lda, w, ldw, M, N, K, C, ldc, r); break;
      case 3: launch_inv<3>(cf, res, grid, s, a, lda, w, ldw, M, N, K, C, ldc, r); break;
      default: launch_inv<4>(cf, res, grid, s, a, lda, w, ldw, M, N, K, C, ldc, r); break;
    }
  }
  VC_LAUNCHED(wide ? "gemm_wide_kernel" : "gemm_bf16_kernel");
  return VC_OK;
}

extern "C" vc_status vc_gemm_bf16(const void* A, int64_t lda, const void* W, int64_t ldw, int64_t M, int32_t N,
                                  int32_t K, void* C, int64_t ldc, int32_t c_dtype, const void* R, void* stream) {
  return gemm_common(false, A, lda, W, ldw, M, N, K, C, ldc, c_dtype, R, stream);
}

extern "C" vc_status vc_gemm_bf16_swiglu(const void* A, int64_t lda, const void* W, int64_t ldw, int64_t M,
                                         int32_t F, int32_t K, void* act, int64_t ld_act, void* stream) {
  clear_error();
  VC_REQUIRE(A && W && act, "A / W / act is NULL");
  VC_REQUIRE(M > 0 && F > 0 && K > 0, "bad shape (M %lld, F %d, K %d)", (long long)M, F, K);
  VC_REQUIRE(F % 8 == 0, "F must be a multiple of 8 (got %d)", F);
  VC_REQUIRE(K % 32 == 0, "K must be a multiple of 32 (got %d)", K);
  VC_REQUIRE(lda >= K && ldw >= K && ld_act >= F, "leading dimensions too small");
  VC_REQUIRE(lda % 8 == 0 && ldw % 8 == 0, "lda and ldw must be multiples of 8 elements");
  VC_REQUIRE(aligned16(A) && aligned16(W), "A and W must be 16-byte aligned");
  const int64_t mt_rows = M >= 64 ? 64 : ((M + 15) / 16) * 16;
  const int MT = static_cast<int>(mt_rows / 16);
  const int N = 2 * F;
  VC_REQUIRE(cdiv(N, 16) <= 65535, "grid too large");
  const dim3 grid(static_cast<unsigned>(cdiv(M, mt_rows)), static_cast<unsigned>(cdiv(N, 16)));
  const dim3 blk(64 * kGemmWaves);
  hipStream_t s = as_stream(stream);
  const bf16_t* a = static_cast<const bf16_t*>(A);
  const bf16_t* w = static_cast<const bf16_t*>(W);
#define VC_SWIGLU_LAUNCH(MT_)                                                                                   \
  hipLaunchKernelGGL((gemm_bf16_kernel<MT_, false, false, kEpiSwiglu>), grid, blk, 0, s, a, lda, w, ldw, M, N, K, \
                     act, ld_act, nullptr)
  switch (MT) {
    case 1: VC_SWIGLU_LAUNCH(1); break;
    case 2: VC_SWIGLU_LAUNCH(2); break;
    case 3: VC_SWIGLU_LAUNCH(3); break;
    default: VC_SWIGLU_LAUNCH(4); break;
  }
#undef VC_SWIGLU_LAUNCH
  VC_LAUNCHED("gemm_bf16_kernel");
  return VC_OK;
}

extern "C" vc_status vc_gemm_bf16_rope(const void* A, int64_t lda, const void* W, int64_t ldw, int32_t B, int32_t k,
                                       int32_t K, int32_t Hq, int32_t Hkv, int32_t hd, float theta, const int32_t* pos,
                                       void* q_out, void* k_dst, void* v_dst, int64_t dst_rows, const int32_t* row0,
                                       void* stream) {
  clear_error();
  VC_REQUIRE(A && W && pos && q_out && k_dst && v_dst && row0, "NULL pointer argument");
  VC_REQUIRE(B > 0 && k > 0 && K > 0 && Hq > 0 && Hkv > 0 && hd > 0, "bad shape");
  VC_REQUIRE(hd % 16 == 0, "hd must be a multiple of 16 (got %d)", hd);
  VC_REQUIRE(K % 32 == 0, "K must be a multiple of 32 (got %d)", K);
  VC_REQUIRE(theta > 1.f, "theta must exceed 1");
  VC_REQUIRE(dst_rows >= k, "dst_rows must hold at least k rows");
  VC_REQUIRE(lda >= K && ldw >= K && lda % 8 == 0 && ldw % 8 == 0, "bad leading dimensions");
  VC_REQUIRE(aligned16(A) && aligned16(W), "A and W must be 16-byte aligned");
  const int64_t M = static_cast<int64_t>(B) * k;
  const int N = (Hq + 2 * Hkv) * hd;
  const int64_t mt_rows = M >= 64 ? 64 : ((M + 15) / 16) * 16;
  const int MT = static_cast<int>(mt_rows / 16);
  VC_REQUIRE(cdiv(N, 16) <= 65535, "grid too large");
  const dim3 grid(static_cast<unsigned>(cdiv(M, mt_rows)), static_cast<unsigned>(cdiv(N, 16)));
  const dim3 blk(64 * kGemmWaves);
  const RopeArgs ra{k, Hq, Hkv, hd, log2f(theta), pos, static_cast<bf16_t*>(q_out), static_cast<bf16_t*>(k_dst),
                    static_cast<bf16_t*>(v_dst), dst_rows, row0};
  hipStream_t s = as_stream(stream);
  const bf16_t* a = static_cast<const bf16_t*>(A);
  const bf16_t* w = static_cast<const bf16_t*>(W);
#define VC_ROPE_LAUNCH(MT_)                                                                                           \
  hipLaunchKernelGGL((gemm_bf16_kernel<MT_, false, false, kEpiRope>), grid, blk, 0, s, a, lda, w, ldw, M, N, K, nullptr, \
                     0, nullptr, ra)
  switch (MT) {
    case 1: VC_ROPE_LAUNCH(1); break;
    case 2: VC_ROPE_LAUNCH(2); break;
    case 3: VC_ROPE_LAUNCH(3); break;
    default: VC_ROPE_LAUNCH(4); break;
  }
#undef VC_ROPE_LAUNCH
  VC_LAUNCHED("gemm_bf16_kernel");
  return VC_OK;
}

extern "C" vc_status vc_gemm_bf16_wide(const void* A, int64_t lda, const void* W, int64_t ldw, int64_t M, int32_t N,
                                       int32_t K, void* C, int64_t ldc, int32_t c_dtype, const void* R, void* stream) {
  return gemm_common(true, A, lda, W, ldw, M, N, K, C, ldc, c_dtype, R, stream);
}

extern "C" vc_status vc_rmsnorm(const void* x, const void* w, int64_t M, int32_t d, float eps, void* y, void* stream) {
  clear_error();
  VC_REQUIRE(x && w && y, "x / w / y is NULL");
  VC_REQUIRE(M > 0 && d > 0, "bad shape");
  VC_REQUIRE(eps > 0.f, "eps must be positive");
  VC_REQUIRE(d % 8 == 0, "d must be a multiple of 8 (got %d)", d);
  VC_REQUIRE(aligned16(x) && aligned16(w) && aligned16(y), "x, w and y must be 16-byte aligned");
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(static_cast<unsigned>(cdiv(M, 4))), dim3(256), 0, as_stream(stream),
                     static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(w), M, d, eps, static_cast<bf16_t*>(y));
  VC_LAUNCHED("rmsnorm_kernel");
  return VC_OK;
}

extern "C" vc_status vc_rope_qkv(const void* qkv, int32_t B, int32_t k, int32_t Hq, int32_t Hkv, int32_t hd,
                                 float theta, const int32_t* pos, void* q_out, void* k_dst, void* v_dst,
                                 int64_t dst_rows, const int32_t* row0, void* stream) {
  clear_error();
  VC_REQUIRE(qkv && pos && q_out && k_dst && v_dst && row0, "NULL pointer argument");
  VC_REQUIRE(B > 0 && k > 0 && Hq > 0 && Hkv > 0 && hd > 0 && hd % 2 == 0, "bad shape");
  VC_REQUIRE(theta > 1.f, "theta must exceed 1");
  VC_REQUIRE(dst_rows >= k, "dst_rows must hold at least k rows");
  hipLaunchKernelGGL(rope_qkv_kernel, dim3(static_cast<unsigned>(B * k)), dim3(256), 0, as_stream(stream),
                     static_cast<const bf16_t*>(qkv), k, Hq, Hkv, hd, log2f(theta), pos, static_cast<bf16_t*>(q_out),
                     static_cast<bf16_t*>(k_dst), static_cast<bf16_t*>(v_dst), dst_rows, row0);
  VC_LAUNCHED("rope_qkv_kernel");
  return VC_OK;
}

extern "C" vc_status vc_swiglu(const void* gu, int64_t M, int32_t F, void* out, void* stream) {
  clear_error();
  VC_REQUIRE(gu && out, "NULL pointer argument");
  VC_REQUIRE(M > 0 && F > 0, "bad shape");
  hipLaunchKernelGGL(swiglu_kernel, dim3(static_cast<unsigned>(cdiv(M * F, 256))), dim3(256), 0, as_stream(stream),
                     static_cast<const bf16_t*>(gu), M, F, static_cast<bf16_t*>(out));
  VC_LAUNCHED("swiglu_kernel");
  return VC_OK;
}

extern "C" vc_status vc_embed(const void* E, int32_t V, int32_t d, const int32_t* tokens, int64_t M, void* x,
                              void* stream) {
  clear_error();
  VC_REQUIRE(E && tokens && x, "NULL pointer argument");
  VC_REQUIRE(V > 0 && d > 0 && M > 0, "bad shape");
  VC_UNSUPPORTED(d % 8 == 0, "d must be a multiple of 8");
  VC_REQUIRE(aligned16(E) && aligned16(x), "E and x must be 16-byte aligned");
  const int rv = d / 8;
  hipLaunchKernelGGL(embed_kernel, dim3(static_cast<unsigned>(cdiv(M * rv, 256))), dim3(256), 0, as_stream(stream),
                     static_cast<const uint4*>(E), V, rv, tokens, M, static_cast<uint4*>(x));
  VC_LAUNCHED("embed_kernel");
  return VC_OK;
}

extern "C" vc_status vc_heads_to_rows(const void* o, int32_t B, int32_t H, int32_t k, int32_t hd, void* out,
                                      void* stream) {
  clear_error();
  VC_REQUIRE(o && out, "NULL pointer argument");
  VC_REQUIRE(B > 0 && H > 0 && k > 0 && hd > 0, "bad shape");
  const int64_t total = static_cast<int64_t>(B) * H * k * hd;
  hipLaunchKernelGGL(heads_to_rows_kernel, dim3(static_cast<unsigned>(cdiv(total, 256))), dim3(256), 0,
                     as_stream(stream), static_cast<const bf16_t*>(o), H, k, hd, total, static_cast<bf16_t*>(out));
  VC_LAUNCHED("heads_to_rows_kernel");
  return VC_OK;
}

extern "C" vc_status vc_argmax_rows(const float* logits, int64_t R, int32_t V, int32_t* tokens, void* stream) {
  clear_error();
  VC_REQUIRE(logits && tokens, "NULL pointer argument");
  VC_REQUIRE(R > 0 && V > 0, "bad shape");
  hipLaunchKernelGGL(argmax_rows_kernel, dim3(static_cast<unsigned>(R)), dim3(kArgThreads), 0, as_stream(stream), logits,
                     V, tokens);
  VC_LAUNCHED("argmax_rows_kernel");
  return VC_OK;
}

extern "C" vc_status vc_copy_kv_rows(const void* src_k, const void* src_v, int64_t src_rows, const int32_t* src_row0,
                                     void* dst_k, void* dst_v, int64_t dst_rows, const int32_t* dst_row0,
                                     const int32_t* count, int32_t max_count, int32_t B, int32_t Hkv, int32_t d,
                                     int32_t elem_bytes, void* stream) {
  clear_error();
  VC_REQUIRE(src_k && src_v && dst_k && dst_v && src_row0 && dst_row0 && count, "NULL pointer argument");
  VC_REQUIRE(B > 0 && Hkv > 0 && d > 0 && max_count >= 0, "bad shape");
  VC_REQUIRE(elem_bytes == 2 || elem_bytes == 4, "elem_bytes must be 2 or 4");
  VC_UNSUPPORTED((static_cast<int64_t>(d) * elem_bytes) % 16 == 0, "rows must be a multiple of 16 bytes");
  VC_REQUIRE(aligned16(src_k) && aligned16(src_v) && aligned16(dst_k) && aligned16(dst_v),
             "caches must be 16-byte aligned");
  if (max_count == 0) return VC_OK;
  const int rv = static_cast<int>(static_cast<int64_t>(d) * elem_bytes / 16);
  dim3 grid(static_cast<unsigned>(cdiv(static_cast<int64_t>(max_count) * rv, 256)), static_cast<unsigned>(B * Hkv));
  hipLaunchKernelGGL(copy_kv_rows_kernel, grid, dim3(256), 0, as_stream(stream), static_cast<const uint4*>(src_k),
                     static_cast<const uint4*>(src_v), src_rows, src_row0, static_cast<uint4*>(dst_k),
                     static_cast<uint4*>(dst_v), dst_rows, dst_row0, count, Hkv, rv, max_count);
  VC_LAUNCHED("copy_kv_rows_kernel");
  return VC_OK;
}
