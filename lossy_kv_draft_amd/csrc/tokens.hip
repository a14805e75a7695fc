// Greedy tokens and prefix acceptance.
//
// Summary page "VeriCache: Turning Lossy KV Cache into Lossless LLM Inference",
// "What the paper found": greedy-decoding output identical to full-KV inference;
// episode page "VeriCache: Lossless LLM Inference from Lossy KV Caches", source 2
// (speculative decoding): the longest prefix on which draft and target agree is
// accepted and the target's token at the first disagreement is committed.
//
// vc_head_mean: mean over q-heads of an attention output row (float32).
// vc_logits_argmax: tokens = argmax_v (u . W_v), ties to the lowest v.
//   bf16 W (matrix cores): u is float32, split exactly into u_hi + u_lo with both
//   parts bf16, and W (u_hi + u_lo) is accumulated in float32 on
//   v_mfma_f32_16x16x32_bf16 (each product is exact; u keeps ~16 significant bits).
//   A workgroup owns 128 vocabulary rows (32 per wave, held as A operands in
//   registers) and sweeps every input row in 16-row tiles, so W is read from HBM
//   once; per tile it reduces (max, lowest index) over its 128 rows and writes one
//   partial per (row, block); a second kernel reduces the blocks in order.
//   float32 W or other shapes: one workgroup per row, float32 dot products.
// vc_accept: one thread per sequence.

#include <type_traits>

#include "common.h"

namespace vc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <typename T>
__global__ void head_mean_kernel(const T* o, int B, int Hq, int k, int d, int64_t sb, int64_t sh, int64_t si,
                                 float* u) {
  int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= static_cast<int64_t>(B) * k * d) return;
  int c = static_cast<int>(e % d);
  int64_t r = e / d;
  int b = static_cast<int>(r / k), i = static_cast<int>(r % k);
  const int64_t base = b * sb + i * si + c;
  // eight loads in flight, summed in head order
  float s = 0.f;
  int h = 0;
  for (; h + 8 <= Hq; h += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = Elem<T>::load(o, base + (h + j) * sh);
#pragma unroll
    for (int j = 0; j < 8; ++j) s += v[j];
  }
  for (; h < Hq; ++h) s += Elem<T>::load(o, base + h * sh);
  u[e] = s / static_cast<float>(Hq);
}

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// ---- float32 / generic path: one block per row
template <typename TU, typename TW>
__global__ void __launch_bounds__(256) argmax_rowwise_kernel(const TU* u, const TW* W, int K, int V, int32_t* tok) {
  __shared__ float su[1024];
  __shared__ float bv_s[4];
  __shared__ int bi_s[4];
  const int64_t r = blockIdx.x;
  for (int c = threadIdx.x; c < K; c += 256) su[c] = Elem<TU>::load(u, r * K + c);
  __syncthreads();
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int v = threadIdx.x; v < V; v += 256) {
    float x = 0.f;
    for (int c = 0; c < K; ++c) x = fmaf(su[c], Elem<TW>::load(W, static_cast<int64_t>(v) * K + c), x);
    if (better(x, v, bv, bi)) { bv = x; bi = v; }
  }
  for (int o = 32; o > 0; o >>= 1) {
    float ov = __shfl_xor(bv, o);
    int oi = __shfl_xor(bi, o);
    if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
  if ((threadIdx.x & 63) == 0) { bv_s[threadIdx.x >> 6] = bv; bi_s[threadIdx.x >> 6] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w)
      if (better(bv_s[w], bi_s[w], bv, bi)) { bv = bv_s[w]; bi = bi_s[w]; }
    // NaN-free inputs always find an index; keep 0 otherwise
    tok[r] = bi == 0x7fffffff ? 0 : bi;
  }
}

// ---- bf16 W on matrix cores
// Each wave owns kLgWave consecutive vocabulary rows of W, held in registers as the A
// operand (16 rows per tile); the workgroup sweeps all R rows of u in chunks of
// kLgChunk rows (the B operand).  A chunk is loaded from global memory once per
// workgroup, split exactly into bf16 hi + lo (float32 u; bf16 u is its own hi) and
// staged in LDS, double-buffered; the loads of the next kLgAhead chunks are in
// flight while the current one is multiplied, two products per step for float32 u,
// one for bf16.  Per (row, wave slice) the largest logit and its lowest index go to
// the partials; argmax_reduce_kernel combines the slices of a row.  At most 128
// registers a wave, so two workgroups share a compute unit.
constexpr int kLgWave = 64;                     // vocabulary rows per wave
constexpr int kLgWaves = 8;                     // waves per workgroup
constexpr int kLgVBlock = kLgWaves * kLgWave;   // vocabulary rows per workgroup
constexpr int kLgChunk = 16;                    // rows of u staged at a time
constexpr int kLgAhead = 1;                     // chunks of u loaded ahead of the one staged

template <int KD, typename TU>
__global__ void __launch_bounds__(64 * kLgWaves) __attribute__((amdgpu_waves_per_eu(4))) argmax_mfma_kernel(const TU* u, const bf16_t* W, int64_t R, int V,
                                                                   float* part_v, int* part_i, int nsl) {
  constexpr int KS = KD / 32, VT = kLgWave / 16;
  constexpr bool kF32 = std::is_same<TU, float>::value;
  constexpr int NP = kF32 ? 2 : 1;               // staged parts of u: hi (and lo)
  constexpr int PITCH = KD + 8;                  // bf16 elements per staged row
  constexpr int EPT = kLgChunk * KD / (64 * kLgWaves);  // chunk elements staged per thread
  static_assert(EPT >= 1 && KD % EPT == 0, "staging shape");
  __shared__ __attribute__((aligned(16))) bf16_t su[2][NP][kLgChunk * PITCH];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, kb = lane >> 4;
  const int slice = blockIdx.x * kLgWaves + wave;
  const int v0 = slice * kLgWave;
  const bool active = v0 < V;  // wave-uniform; idle waves still stage u and meet the barriers
  union P16 { uint4 u; bf16x8_t v; };
  bf16x8_t wa[VT][KS];
#pragma unroll
  for (int vt = 0; vt < VT; ++vt) {
    const int v = v0 + vt * 16 + l16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      P16 p;
      p.u = make_uint4(0, 0, 0, 0);
      if (v < V) p.u = *reinterpret_cast<const uint4*>(W + static_cast<int64_t>(v) * KD + 32 * ks + 8 * kb);
      wa[vt][ks] = p.v;
    }
  }
  // staging: this thread's EPT consecutive elements of a chunk
  const int srow = (tid * EPT) / KD, scol = (tid * EPT) % KD;
  float xq[kLgAhead][EPT];  // chunks c + 1 .. c + kLgAhead, oldest first
  auto load = [&](int64_t r0, float (&xs)[EPT]) {
    const int64_t r = r0 + srow;
#pragma unroll
    for (int j = 0; j < EPT; ++j) xs[j] = r < R ? Elem<TU>::load(u, r * KD + scol + j) : 0.f;
  };
  auto stage = [&](int buf, const float (&xs)[EPT]) {
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const __bf16 h = static_cast<__bf16>(xs[j]);
      su[buf][0][srow * PITCH + scol + j] = __builtin_bit_cast(bf16_t, h);
      if constexpr (kF32)
        su[buf][NP - 1][srow * PITCH + scol + j] = __builtin_bit_cast(bf16_t, static_cast<__bf16>(xs[j] - static_cast<float>(h)));
    }
  };
  {
    float x0[EPT];
    load(0, x0);
#pragma unroll
    for (int q = 0; q < kLgAhead; ++q) load(static_cast<int64_t>(q + 1) * kLgChunk, xq[q]);
    stage(0, x0);
  }
  __syncthreads();
  int buf = 0;
  for (int64_t c0 = 0; c0 < R; c0 += kLgChunk) {
    const bool more = c0 + kLgChunk < R;
    for (int rt = 0; rt < kLgChunk / 16 && active; ++rt) {
      const int64_t r0 = c0 + 16 * rt;
      if (r0 >= R) break;
      f32x4_t acc[VT];
#pragma unroll
      for (int vt = 0; vt < VT; ++vt) acc[vt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int pt = 0; pt < NP; ++pt) {
          P16 b;
          b.u = *reinterpret_cast<const uint4*>(&su[buf][pt][(16 * rt + l16) * PITCH + 32 * ks + 8 * kb]);
#pragma unroll
          for (int vt = 0; vt < VT; ++vt)
            acc[vt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[vt][ks], b.v, acc[vt], 0, 0, 0);
        }
      }
      // acc[vt][i] = logit(vocabulary v0 + 16 vt + 4 kb + i, row r0 + l16)
      float bv = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int vt = 0; vt < VT; ++vt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int v = v0 + vt * 16 + 4 * kb + i;
          if (v < V && better(acc[vt][i], v, bv, bi)) { bv = acc[vt][i]; bi = v; }
        }
#pragma unroll
      for (int o = 16; o <= 32; o <<= 1) {
        const float ov = __shfl_xor(bv, o);
        const int oi = __shfl_xor(bi, o);
        if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
      }
      if (kb == 0 && r0 + l16 < R) {
        part_v[(r0 + l16) * nsl + slice] = bv;
        part_i[(r0 + l16) * nsl + slice] = bi;
      }
    }
    if (more) {
      stage(buf ^ 1, xq[0]);  // into the buffer read one chunk ago; the barrier below orders it
#pragma unroll
      for (int q = 0; q + 1 < kLgAhead; ++q)
#pragma unroll
        for (int j = 0; j < EPT; ++j) xq[q][j] = xq[q + 1][j];
      load(c0 + static_cast<int64_t>(kLgAhead + 1) * kLgChunk, xq[kLgAhead - 1]);
    }
    __syncthreads();
    buf ^= 1;
  }
}

__global__ void __launch_bounds__(256) argmax_reduce_kernel(const float* part_v, const int* part_i, int nvb,
                                                            int32_t* tok) {
  const int64_t r = blockIdx.x;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int j = threadIdx.x; j < nvb; j += 256) {
    float v = part_v[r * nvb + j];
    int i = part_i[r * nvb + j];
    if (better(v, i, bv, bi)) { bv = v; bi = i; }
  }
  __shared__ float sv[4];
  __shared__ int si[4];
  for (int o = 32; o > 0; o >>= 1) {
    float ov = __shfl_xor(bv, o);
    int oi = __shfl_xor(bi, o);
    if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
  if ((threadIdx.x & 63) == 0) { sv[threadIdx.x >> 6] = bv; si[threadIdx.x >> 6] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w)
      if (better(sv[w], si[w], bv, bi)) { bv = sv[w]; bi = si[w]; }
    tok[r] = bi == 0x7fffffff ? 0 : bi;
  }
}

__global__ void accept_kernel(const int32_t* draft, const int32_t* target, int B, int k, int32_t* acc,
                              int32_t* nc, int32_t* commit) {
  int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int32_t* d = draft + static_cast<int64_t>(b) * k;
  const int32_t* t = target + static_cast<int64_t>(b) * k;
  int32_t* c = commit + static_cast<int64_t>(b) * k;
  int a = 0;
  while (a < k && d[a] == t[a]) {
    c[a] = d[a];
    ++a;
  }
  int n = a;
  if (a < k) c[n++] = t[a];
  for (int j = n; j < k; ++j) c[j] = -1;
  acc[b] = a;
  nc[b] = n;
}

static bool use_mfma_argmax(int32_t w_dtype, int32_t K) { return w_dtype == VC_BF16 && (K == 64 || K == 128); }

}  // namespace vc

using namespace vc;

extern "C" vc_status vc_head_mean(const void* o, int32_t kv_dtype, int32_t B, int32_t Hq, int32_t k, int32_t d,
                                  int64_t stride_b, int64_t stride_h, int64_t stride_i, float* u, void* stream) {
  clear_error();
  VC_REQUIRE(o && u, "o / u is NULL");
  VC_REQUIRE(valid_dtype(kv_dtype), "bad kv_dtype");
  VC_REQUIRE(B > 0 && Hq > 0 && k > 0 && d > 0, "bad shape");
  int64_t n = static_cast<int64_t>(B) * k * d;
  dim3 grid(static_cast<unsigned>(cdiv(n, 256)));
  if (kv_dtype == VC_F32)
    hipLaunchKernelGGL(head_mean_kernel<float>, grid, dim3(256), 0, as_stream(stream), static_cast<const float*>(o),
                       B, Hq, k, d, stride_b, stride_h, stride_i, u);
  else
    hipLaunchKernelGGL(head_mean_kernel<bf16_t>, grid, dim3(256), 0, as_stream(stream),
                       static_cast<const bf16_t*>(o), B, Hq, k, d, stride_b, stride_h, stride_i, u);
  VC_LAUNCHED("head_mean_kernel");
  return VC_OK;
}

extern "C" size_t vc_logits_workspace_bytes(int64_t R, int32_t V) {
  if (R <= 0 || V <= 0) return 0;
  size_t nsl = static_cast<size_t>(cdiv(V, kLgWave));
  return align_up(R * nsl * sizeof(float), 256) + align_up(R * nsl * sizeof(int), 256);
}

extern "C" vc_status vc_logits_argmax(const void* u, int32_t u_dtype, int64_t R, int32_t K, const void* W,
                                      int32_t w_dtype, int32_t V, int32_t* tokens, void* ws, size_t ws_bytes,
                                      void* stream) {
  clear_error();
  VC_REQUIRE(u && W && tokens, "u / W / tokens is NULL");
  VC_REQUIRE(valid_dtype(u_dtype) && valid_dtype(w_dtype), "bad dtype");
  VC_REQUIRE(R > 0 && K > 0 && V > 0, "bad shape (R %lld, K %d, V %d)", (long long)R, K, V);
  hipStream_t s = as_stream(stream);
  if (use_mfma_argmax(w_dtype, K)) {
    VC_REQUIRE(reinterpret_cast<uintptr_t>(u) % 16 == 0 && reinterpret_cast<uintptr_t>(W) % 16 == 0,
               "u and W must be 16-byte aligned");
    size_t need = vc_logits_workspace_bytes(R, V);
    if (!ws || ws_bytes < need) {
      set_error("logits workspace needs %zu bytes (got %zu)", need, ws_bytes);
      return VC_ERR_WORKSPACE;
    }
    const int nsl = static_cast<int>(cdiv(V, kLgWave));
    const unsigned nwg = static_cast<unsigned>(cdiv(V, kLgVBlock));
    float* pv = static_cast<float*>(ws);
    int* pi = reinterpret_cast<int*>(static_cast<char*>(ws) + align_up(R * nsl * sizeof(float), 256));
    const bf16_t* w = static_cast<const bf16_t*>(W);
    if (K == 128) {
      if (u_dtype == VC_F32)
        hipLaunchKernelGGL((argmax_mfma_kernel<128, float>), dim3(nwg), dim3(64 * kLgWaves), 0, s, static_cast<const float*>(u), w, R, V, pv, pi, nsl);
      else
        hipLaunchKernelGGL((argmax_mfma_kernel<128, bf16_t>), dim3(nwg), dim3(64 * kLgWaves), 0, s, static_cast<const bf16_t*>(u), w, R, V, pv, pi, nsl);
    } else {
      if (u_dtype == VC_F32)
        hipLaunchKernelGGL((argmax_mfma_kernel<64, float>), dim3(nwg), dim3(64 * kLgWaves), 0, s, static_cast<const float*>(u), w, R, V, pv, pi, nsl);
      else
        hipLaunchKernelGGL((argmax_mfma_kernel<64, bf16_t>), dim3(nwg), dim3(64 * kLgWaves), 0, s, static_cast<const bf16_t*>(u), w, R, V, pv, pi, nsl);
    }
    VC_LAUNCHED("argmax_mfma_kernel");
    hipLaunchKernelGGL(argmax_reduce_kernel, dim3(static_cast<unsigned>(R)), dim3(256), 0, s, pv, pi, nsl, tokens);
    VC_LAUNCHED("argmax_reduce_kernel");
    return VC_OK;
  }
  VC_UNSUPPORTED(K <= 1024, "K must be at most 1024 on the float32 path (got %d)", K);
  dim3 grid(static_cast<unsigned>(R));
#define VC_AM(TU, TW) \
  hipLaunchKernelGGL((argmax_rowwise_kernel<TU, TW>), grid, dim3(256), 0, s, static_cast<const TU*>(u), static_cast<const TW*>(W), K, V, tokens)
  if (u_dtype == VC_F32 && w_dtype == VC_F32) VC_AM(float, float);
  else if (u_dtype == VC_F32) VC_AM(float, bf16_t);
  else if (w_dtype == VC_F32) VC_AM(bf16_t, float);
  else VC_AM(bf16_t, bf16_t);
#undef VC_AM
  VC_LAUNCHED("argmax_rowwise_kernel");
  return VC_OK;
}

extern "C" vc_status vc_accept(const int32_t* draft, const int32_t* target, int32_t B, int32_t k, int32_t* accept_len,
                               int32_t* n_commit, int32_t* commit, void* stream) {
  clear_error();
  VC_REQUIRE(draft && target && accept_len && n_commit && commit, "NULL pointer argument");
  VC_REQUIRE(B > 0, "B must be positive");
  VC_REQUIRE(k >= 1 && k <= 1024, "k must be in [1, 1024] (got %d)", k);
  hipLaunchKernelGGL(accept_kernel, dim3(static_cast<unsigned>(cdiv(B, 64))), dim3(64), 0, as_stream(stream), draft,
                     target, B, k, accept_len, n_commit, commit);
  VC_LAUNCHED("accept_kernel");
  return VC_OK;
}
