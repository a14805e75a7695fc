// Token dropping by accumulated attention (compression of the draft cache).
//
// Episode page "VeriCache: Lossless LLM Inference from Lossy KV Caches", source 3
// (H2O, heavy-hitter tokens collect most of the attention); summary page
// "VeriCache: Turning Lossy KV Cache into Lossless LLM Inference", "Original
// abstract" (token dropping is one of the compressor families).
//
// score_n = sum_p softmax_n(P_p . K_n * sm_scale) over n_probes probe queries,
// per (sequence, kv-head); the n_keep highest scores are kept (equal scores: lower
// position first), their positions stored ascending and their K/V rows copied.
//
// Scoring runs on matrix cores (v_mfma_f32_16x16x32_bf16: K and probes are bf16,
// products exact, float32 accumulation) in two passes over K:
//   pass 1 (grid = chunks x B*Hkv): per chunk and probe the running max and sum of
//           exp2 of the scaled scores;
//   pass 2: every block merges the per-chunk statistics of its (sequence, head)
//           in chunk order, recomputes the scores of its chunk and sums the
//           probabilities over the probes (fixed butterfly order).
// Selection: a 4 x 8-bit radix select over order-preserving keys of the scores finds
// the n_keep-th largest, workgroups over slices of every (sequence, kv-head) adding
// into global digit histograms; then the positions with a larger score plus the
// lowest-positioned equal ones are written in position order (sel_* below).

#include "common.h"

namespace vc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kDropChunk = 2048;
constexpr int kDropMaxProbes = 64;

union DP16 {
  uint4 u;
  bf16x8_t v;
};

template <int D>
__device__ __forceinline__ void load_probes(const bf16_t* probes, int hk, int P, int l16, int kb,
                                            bf16x8_t (&pf)[4][D / 32]) {
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    int p = ct * 16 + l16;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      DP16 x;
      x.u = make_uint4(0, 0, 0, 0);
      if (p < P)
        x.u = *reinterpret_cast<const uint4*>(probes + (static_cast<int64_t>(hk) * P + p) * D + 32 * ks + 8 * kb);
      pf[ct][ks] = x.v;
    }
  }
}

// The 16 x D tile of K rows tok0 .. tok0 + 15 as matrix-core operands: lane (l16, kb)
// holds row tok0 + l16, channels 32 ks + 8 kb .. + 7 for each k-step ks (float32 rows
// are rounded to bf16 when the operand is formed).  A row at or past N reads row N - 1:
// the scores it yields are masked by the callers (no zeroing after the loads, which
// would have to wait for them).
template <int D, typename T>
struct KTile {
  static constexpr int kVecs = (sizeof(T) == 2 ? 1 : 2) * (D / 32);
  uint4 v[kVecs];
};

template <int D, typename T>
__device__ __forceinline__ void ktile_load(const T* krows, int64_t tok, int64_t N, int kb, KTile<D, T>& t) {
  const int64_t row = tok < N ? tok : N - 1;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    const uint4* p = reinterpret_cast<const uint4*>(krows + row * D + 32 * ks + 8 * kb);
    if constexpr (sizeof(T) == 2) {
      t.v[ks] = p[0];
    } else {
      t.v[2 * ks] = p[0];
      t.v[2 * ks + 1] = p[1];
    }
  }
}

template <int D, typename T>
__device__ __forceinline__ bf16x8_t ktile_op(const KTile<D, T>& t, int ks) {
  if constexpr (sizeof(T) == 2) {
    DP16 a;
    a.u = t.v[ks];
    return a.v;
  } else {
    const uint4 u0 = t.v[2 * ks], u1 = t.v[2 * ks + 1];
    const float f[8] = {__uint_as_float(u0.x), __uint_as_float(u0.y), __uint_as_float(u0.z), __uint_as_float(u0.w),
                        __uint_as_float(u1.x), __uint_as_float(u1.y), __uint_as_float(u1.z), __uint_as_float(u1.w)};
    bf16x8_t a;
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = static_cast<__bf16>(f[j]);
    return a;
  }
}

// Sum over the four 16-lane groups of a wave (lanes l, l ^ 16, l ^ 32, l ^ 48), left in
// every lane of the four: the lane-swap instructions pair each lane with its partner,
// and each step adds the pair (two operands: the same sum in both lanes).
__device__ __forceinline__ float group4_sum(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
  const unsigned w = __float_as_uint(x);
  const auto r32 = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

// Pass 1: per chunk and probe, a reference m and the sum of exp2 of the scaled scores
// minus m.  Lane (l16, kb) of a wave keeps probes 16 ct + l16 over tokens 4 kb .. + 3 of
// each 16-token step (S = K P^T: K rows are the A operand); the reference moves only when
// a score exceeds it by more than 8 (so every term is below 2^8), and the rows of the
// next two steps are loaded while the current one is multiplied.
template <int D, typename T>
__global__ void __launch_bounds__(256) drop_stats_kernel(const T* k, const bf16_t* probes, int Hkv, int64_t N, int P,
                                                         float qscale, int nchunks, float* stat_m, float* stat_l) {
  __shared__ float sm[4][kDropMaxProbes], sl[4][kDropMaxProbes];
  const int chunk = blockIdx.x, bh = blockIdx.y, hk = bh % Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15, kb = lane >> 4;
  bf16x8_t pf[4][D / 32];
  load_probes<D>(probes, hk, P, l16, kb, pf);
  const T* krows = k + static_cast<int64_t>(bh) * N * D;
  float m[4], l[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) { m[ct] = -1e30f; l[ct] = 0.f; }  // finite: a masked -inf term adds exp2(-inf) = 0
  const int64_t c0 = static_cast<int64_t>(chunk) * kDropChunk;
  const int64_t c1 = min(N, c0 + kDropChunk);
  auto step = [&](const KTile<D, T>& cur, int64_t t0) {
    f32x4_t s[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) s[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const bf16x8_t a = ktile_op<D, T>(cur, ks);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) s[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[ct][ks], s[ct], 0, 0, 0);
    }
    if (t0 + 64 > c1) {  // the chunk's last steps (wave-uniform): tokens at or past c1 drop out
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (t0 + 4 * kb + r >= c1) s[ct][r] = -INFINITY;
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      // the maximum of the raw scores (the scale is positive), scaled once
      const float mt = fmaxf(fmaxf(s[ct][0], s[ct][1]), fmaxf(s[ct][2], s[ct][3])) * qscale;
      if (mt > m[ct] + 8.f) {
        l[ct] *= exp2f(m[ct] - mt);
        m[ct] = mt;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)  // results below 2^-126 read as 0
        l[ct] += __builtin_amdgcn_exp2f(__builtin_fmaf(s[ct][r], qscale, -m[ct]));
    }
  };
  KTile<D, T> tl[3];  // a ring of three tiles: loads two steps ahead of the products
  int64_t t0 = c0 + wave * 16;
  ktile_load<D, T>(krows, t0 + l16, N, kb, tl[0]);
  ktile_load<D, T>(krows, t0 + 64 + l16, N, kb, tl[1]);
  while (t0 < c1) {
    ktile_load<D, T>(krows, t0 + 128 + l16, N, kb, tl[2]);  // unconditional (rows clamped): exact waits
    __builtin_amdgcn_sched_barrier(0);                      // and issued here, not next to their first use
    step(tl[0], t0);
    t0 += 64;
    if (t0 >= c1) break;
    ktile_load<D, T>(krows, t0 + 128 + l16, N, kb, tl[0]);
    __builtin_amdgcn_sched_barrier(0);
    step(tl[1], t0);
    t0 += 64;
    if (t0 >= c1) break;
    ktile_load<D, T>(krows, t0 + 128 + l16, N, kb, tl[1]);
    __builtin_amdgcn_sched_barrier(0);
    step(tl[2], t0);
    t0 += 64;
  }
  // combine the 4 lane groups (same probe), then the 4 waves
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      const float om = __shfl_xor(m[ct], o), ol = __shfl_xor(l[ct], o);
      const float mn = fmaxf(m[ct], om);
      l[ct] = l[ct] * exp2f(m[ct] - mn) + ol * exp2f(om - mn);
      m[ct] = mn;
    }
    if (kb == 0) { sm[wave][ct * 16 + l16] = m[ct]; sl[wave][ct * 16 + l16] = l[ct]; }
  }
  __syncthreads();
  if (tid < P) {
    float mm = sm[0][tid], ll = sl[0][tid];
    for (int w = 1; w < 4; ++w) {
      const float om = sm[w][tid], ol = sl[w][tid];
      const float mn = fmaxf(mm, om);
      ll = ll * exp2f(mm - mn) + ol * exp2f(om - mn);
      mm = mn;
    }
    stat_m[(static_cast<int64_t>(bh) * nchunks + chunk) * P + tid] = mm;
    stat_l[(static_cast<int64_t>(bh) * nchunks + chunk) * P + tid] = ll;
  }
}

// The chunks' statistics of each (sequence, kv-head) merged once: off[bh][p] = M + log2 L
// for the probe's softmax over all N tokens (M its reference, L the sum of exp2(s - M)),
// so that a token's probability under probe p is exp2(s - off).  Thread (p, g) merges
// chunks g, g + 4, ... in order; the four partial results are then merged in order of g.
__global__ void __launch_bounds__(256) drop_stats_merge_kernel(const float* stat_m, const float* stat_l, int nchunks,
                                                               int P, float* off) {
  __shared__ float pm[4][kDropMaxProbes], pl[4][kDropMaxProbes];
  const int bh = blockIdx.x, p = threadIdx.x & 63, g = threadIdx.x >> 6;
  float mm = -1e30f, ll = 0.f;
  if (p < P) {
    for (int c = g; c < nchunks; c += 4) {
      const float om = stat_m[(static_cast<int64_t>(bh) * nchunks + c) * P + p];
      const float ol = stat_l[(static_cast<int64_t>(bh) * nchunks + c) * P + p];
      const float mn = fmaxf(mm, om);
      ll = ll * exp2f(mm - mn) + ol * exp2f(om - mn);
      mm = mn;
    }
  }
  pm[g][p] = mm;
  pl[g][p] = ll;
  __syncthreads();
  if (g == 0) {
    for (int h = 1; h < 4; ++h) {
      const float om = pm[h][p], ol = pl[h][p];
      const float mn = fmaxf(mm, om);
      ll = ll * exp2f(mm - mn) + ol * exp2f(om - mn);
      mm = mn;
    }
    off[bh * kDropMaxProbes + p] = p < P ? mm + log2f(ll) : INFINITY;  // no probe: probability 0
  }
}

// Pass 2: every token's probabilities summed over the probes.  Here the probes are the A
// operand (P K^T), so lane (l16, kb) holds token l16 of the step under probes
// 16 ct + 4 kb + r: its 16 probabilities are summed in the lane, then over the four lane
// groups; the rows of the next two steps are loaded while the current one is multiplied.
template <int D, typename T>
__global__ void __launch_bounds__(256) drop_scores_kernel(const T* k, const bf16_t* probes, int Hkv, int64_t N, int P,
                                                          float qscale, const float* off, float* scores) {
  const int chunk = blockIdx.x, bh = blockIdx.y, hk = bh % Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15, kb = lane >> 4;
  bf16x8_t pf[4][D / 32];
  load_probes<D>(probes, hk, P, l16, kb, pf);
  float po[4][4];  // off of probe 16 ct + 4 kb + r (+inf for p >= P)
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) po[ct][r] = off[bh * kDropMaxProbes + 16 * ct + 4 * kb + r];
  const T* krows = k + static_cast<int64_t>(bh) * N * D;
  const int64_t c0 = static_cast<int64_t>(chunk) * kDropChunk;
  const int64_t c1 = min(N, c0 + kDropChunk);
  auto step = [&](const KTile<D, T>& cur, int64_t t0) {
    f32x4_t s[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) s[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const bf16x8_t a = ktile_op<D, T>(cur, ks);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) s[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf[ct][ks], a, s[ct], 0, 0, 0);
    }
    float acc = 0.f;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc += __builtin_amdgcn_exp2f(__builtin_fmaf(s[ct][r], qscale, -po[ct][r]));
    acc = group4_sum(acc);
    if (kb == 0 && t0 + l16 < c1) scores[static_cast<int64_t>(bh) * N + t0 + l16] = acc;
  };
  KTile<D, T> tl[3];  // a ring of three tiles: loads two steps ahead of the products
  int64_t t0 = c0 + wave * 16;
  ktile_load<D, T>(krows, t0 + l16, N, kb, tl[0]);
  ktile_load<D, T>(krows, t0 + 64 + l16, N, kb, tl[1]);
  while (t0 < c1) {
    ktile_load<D, T>(krows, t0 + 128 + l16, N, kb, tl[2]);  // unconditional (rows clamped): exact waits
    __builtin_amdgcn_sched_barrier(0);                      // and issued here, not next to their first use
    step(tl[0], t0);
    t0 += 64;
    if (t0 >= c1) break;
    ktile_load<D, T>(krows, t0 + 128 + l16, N, kb, tl[0]);
    __builtin_amdgcn_sched_barrier(0);
    step(tl[1], t0);
    t0 += 64;
    if (t0 >= c1) break;
    ktile_load<D, T>(krows, t0 + 128 + l16, N, kb, tl[1]);
    __builtin_amdgcn_sched_barrier(0);
    step(tl[2], t0);
    t0 += 64;
  }
}

// ---- top-k selection
// The n_keep-th largest key is found by a radix select on 8-bit digits, most significant
// first, over the whole grid: N / kSelSlice workgroups per (sequence, kv-head) each add the
// digit histogram of their slice (keys that share the digits fixed so far) into a global
// one, and every workgroup of the next launch re-derives the digits fixed so far from
// those histograms (a one-wave scan each, identical in every workgroup).  Then each slice
// counts its keys above and equal to the threshold, and the last launch writes the kept
// positions in ascending order: a position's slot is the number of kept positions below
// it, from the counts of the earlier slices and a scan inside the slice.  The kept set is
// fixed by the order (key descending, position ascending), so it does not depend on the
// split; the histogram sums are integer atomics, so nothing depends on their order.
constexpr int kSelSlice = 8192;  // scores per workgroup
constexpr int kSelT = 256;       // threads per workgroup
constexpr int kSelRun = kSelSlice / kSelT;  // consecutive positions per thread in the write

// Unsigned key whose order is the numeric order of the score: a negative float's
// bits are flipped, a non-negative one gets its sign bit set; -0.0 is read as +0.0
// (equal scores) and every NaN as key 0, below -inf.
__device__ __forceinline__ uint32_t select_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

static int sel_slices(int64_t N) { return static_cast<int>(cdiv(N, kSelSlice)); }
static size_t sel_hist_bytes(int32_t B, int32_t Hkv) {
  return align_up(4 * static_cast<size_t>(B) * Hkv * 256 * sizeof(uint32_t), 256);
}
static size_t sel_ws_bytes(int32_t B, int32_t Hkv, int64_t N) {
  return sel_hist_bytes(B, Hkv) + align_up(static_cast<size_t>(B) * Hkv * sel_slices(N) * 2 * sizeof(uint32_t), 256);
}

// One digit of the select, by one whole wave: h[256] counts the keys that share the digits
// fixed so far, remain (>= 1) is the rank from the top of the wanted key among them.
// Returns the wanted key's digit; remain becomes its rank among the keys with that digit.
__device__ __forceinline__ uint32_t sel_digit(const uint32_t* h, int64_t& remain, int lane) {
  uint32_t c[4], sum = 0;  // lane l: bins 255 - 4 l down to 252 - 4 l
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    c[j] = h[255 - 4 * lane - j];
    sum += c[j];
  }
  int64_t incl = sum;  // inclusive sum over the lanes up to this one (descending bins)
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  const int64_t excl = incl - sum;
  const int L = __ffsll(static_cast<unsigned long long>(__ballot(excl < remain && remain <= incl))) - 1;
  uint32_t digit = 0;
  int64_t r = remain - excl;
  if (lane == L) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (r <= c[j]) {
        digit = 255u - 4u * lane - j;
        break;
      }
      r -= c[j];
    }
  }
  remain = __shfl(r, L);
  return static_cast<uint32_t>(__shfl(static_cast<int>(digit), L));
}

// The digits fixed by passes [0, npass) as a key prefix, and the rank that goes with it
__device__ __forceinline__ uint32_t sel_prefix(const uint32_t* hist, int BH, int bh, int npass, int64_t n_keep,
                                               int64_t& remain, int lane) {
  uint32_t prefix = 0;
  remain = n_keep;
  for (int q = 0; q < npass; ++q)
    prefix |= sel_digit(hist + (static_cast<size_t>(q) * BH + bh) * 256, remain, lane) << (24 - 8 * q);
  return prefix;
}

__global__ void __launch_bounds__(256) sel_zero_kernel(uint32_t* p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

__global__ void __launch_bounds__(kSelT) sel_hist_kernel(const float* scores, int64_t N, int64_t n_keep,
                                                         uint32_t* hist, int BH, int pass) {
  __shared__ uint32_t lh[kSelT / 64][256];
  __shared__ uint32_t s_prefix;
  const int slice = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (wave == 0) {
    int64_t remain;
    const uint32_t prefix = sel_prefix(hist, BH, bh, pass, n_keep, remain, lane);
    if (lane == 0) s_prefix = prefix;
  }
  for (int i = tid; i < (kSelT / 64) * 256; i += kSelT) (&lh[0][0])[i] = 0u;
  __syncthreads();
  const uint32_t prefix = s_prefix;
  const int shift = 24 - 8 * pass;
  const uint32_t pmask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
  const float* sc = scores + static_cast<int64_t>(bh) * N;
  const int64_t n0 = static_cast<int64_t>(slice) * kSelSlice, n1 = min(N, n0 + kSelSlice);
  for (int64_t n = n0 + tid; n < n1; n += kSelT) {
    const uint32_t key = select_key(sc[n]);
    if ((key & pmask) == (prefix & pmask)) atomicAdd(&lh[wave][(key >> shift) & 255u], 1u);
  }
  __syncthreads();
  uint32_t v = 0;  // kSelT == 256: one bin per thread
#pragma unroll
  for (int w = 0; w < kSelT / 64; ++w) v += lh[w][tid];
  if (v) atomicAdd(&hist[(static_cast<size_t>(pass) * BH + bh) * 256 + tid], v);
}

// Block-wide exclusive sum of x (kSelT threads); total in *tot
__device__ __forceinline__ int64_t sel_block_scan(int64_t x, int64_t* wsum, int lane, int wave, int64_t* tot) {
  int64_t incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int64_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kSelT / 64; ++w) {
    before += w < wave ? wsum[w] : 0;
    all += wsum[w];
  }
  __syncthreads();
  *tot = all;
  return before + incl - x;
}

// Keys above the threshold and equal to it in each slice: cnt[bh][slice] = {gt, eq}
__global__ void __launch_bounds__(kSelT) sel_count_kernel(const float* scores, int64_t N, int64_t n_keep,
                                                          const uint32_t* hist, int BH, uint32_t* cnt, int S) {
  __shared__ uint32_t s_thr;
  __shared__ int64_t wsum[kSelT / 64];
  const int slice = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (wave == 0) {
    int64_t remain;
    const uint32_t thr = sel_prefix(hist, BH, bh, 4, n_keep, remain, lane);
    if (lane == 0) s_thr = thr;
  }
  __syncthreads();
  const uint32_t thr = s_thr;
  const float* sc = scores + static_cast<int64_t>(bh) * N;
  const int64_t n0 = static_cast<int64_t>(slice) * kSelSlice, n1 = min(N, n0 + kSelSlice);
  int64_t gt = 0, eq = 0;
  for (int64_t n = n0 + tid; n < n1; n += kSelT) {
    const uint32_t key = select_key(sc[n]);
    gt += key > thr;
    eq += key == thr;
  }
  int64_t tg, te;
  sel_block_scan(gt, wsum, lane, wave, &tg);
  sel_block_scan(eq, wsum, lane, wave, &te);
  if (tid == 0) {
    cnt[(static_cast<size_t>(bh) * S + slice) * 2] = static_cast<uint32_t>(tg);
    cnt[(static_cast<size_t>(bh) * S + slice) * 2 + 1] = static_cast<uint32_t>(te);
  }
}

// The kept positions of each slice, in ascending order: thread t takes the kSelRun
// consecutive positions from n0 + kSelRun t
__global__ void __launch_bounds__(kSelT) sel_write_kernel(const float* scores, int64_t N, int64_t n_keep,
                                                          const uint32_t* hist, int BH, const uint32_t* cnt, int S,
                                                          int32_t* kept, int64_t kept_pitch) {
  __shared__ uint32_t s_thr;
  __shared__ int64_t s_need, s_g0, s_e0;
  __shared__ int64_t wsum[kSelT / 64];
  const int slice = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (wave == 0) {
    int64_t remain;  // after all four digits: how many keys equal to the threshold are kept
    const uint32_t thr = sel_prefix(hist, BH, bh, 4, n_keep, remain, lane);
    int64_t g = 0, e = 0;  // kept-above and equal keys in the earlier slices
    for (int q = lane; q < slice; q += 64) {
      g += cnt[(static_cast<size_t>(bh) * S + q) * 2];
      e += cnt[(static_cast<size_t>(bh) * S + q) * 2 + 1];
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      g += __shfl_xor(g, o);
      e += __shfl_xor(e, o);
    }
    if (lane == 0) {
      s_thr = thr;
      s_need = remain;
      s_g0 = g;
      s_e0 = e;
    }
  }
  __syncthreads();
  const uint32_t thr = s_thr;
  const int64_t need = s_need;
  const float* sc = scores + static_cast<int64_t>(bh) * N;
  const int64_t p0 = static_cast<int64_t>(slice) * kSelSlice + static_cast<int64_t>(tid) * kSelRun;
  uint32_t key[kSelRun];
  int64_t gt = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < kSelRun; ++i) {
    key[i] = p0 + i < N ? select_key(sc[p0 + i]) : 0u;
    const bool in = p0 + i < N;
    gt += in && key[i] > thr;
    eq += in && key[i] == thr;
  }
  int64_t tg, te;
  int64_t g = s_g0 + sel_block_scan(gt, wsum, lane, wave, &tg);  // above the threshold, before this run
  int64_t e = s_e0 + sel_block_scan(eq, wsum, lane, wave, &te);  // equal to it, before this run
  int32_t* out = kept + static_cast<int64_t>(bh) * kept_pitch;
#pragma unroll
  for (int i = 0; i < kSelRun; ++i) {
    if (p0 + i >= N) break;
    if (key[i] > thr) {
      const int64_t slot = g + min(e, need);
      if (slot < n_keep) out[slot] = static_cast<int32_t>(p0 + i);
      ++g;
    } else if (key[i] == thr) {
      if (e < need && g + e < n_keep) out[g + e] = static_cast<int32_t>(p0 + i);
      ++e;
    }
  }
}

template <int VEC>
__global__ void __launch_bounds__(256) gather_rows_kernel(const uint4* src, int64_t src_rows, int row_vecs,
                                                          const int32_t* idx, int64_t n, int64_t idx_pitch,
                                                          uint4* dst, int64_t dst_rows) {
  const int bh = blockIdx.y;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= n * row_vecs) return;
  const int64_t j = e / row_vecs;
  const int c = static_cast<int>(e % row_vecs);
  const int64_t s = idx[static_cast<int64_t>(bh) * idx_pitch + j];
  if (s < 0 || s >= src_rows) return;  // out-of-range index: row left untouched
  dst[(static_cast<int64_t>(bh) * dst_rows + j) * row_vecs + c] = src[(static_cast<int64_t>(bh) * src_rows + s) * row_vecs + c];
}

// The same copy for rows of 2^lrv 16-byte pieces: indices by shifts instead of a 64-bit
// division per piece (which has no instruction and costs on the order of a hundred)
__global__ void __launch_bounds__(256) gather_rows_pow2_kernel(const uint4* src, int64_t src_rows, int lrv,
                                                               const int32_t* idx, int64_t n, int64_t idx_pitch,
                                                               uint4* dst, int64_t dst_rows) {
  const int bh = blockIdx.y;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= (n << lrv)) return;
  const int64_t j = e >> lrv;
  const int64_t c = e & ((int64_t{1} << lrv) - 1);
  const int64_t s = idx[static_cast<int64_t>(bh) * idx_pitch + j];
  if (s < 0 || s >= src_rows) return;  // out-of-range index: row left untouched
  dst[((static_cast<int64_t>(bh) * dst_rows + j) << lrv) + c] = src[((static_cast<int64_t>(bh) * src_rows + s) << lrv) + c];
}

static int drop_chunks(int64_t N) { return static_cast<int>(cdiv(N, kDropChunk)); }

static size_t scores_ws_bytes(int32_t B, int32_t Hkv, int64_t N, int32_t P) {
  size_t n = static_cast<size_t>(B) * Hkv * drop_chunks(N) * P;
  return 2 * align_up(n * sizeof(float), 256) + align_up(static_cast<size_t>(B) * Hkv * kDropMaxProbes * sizeof(float), 256);
}

vc_status drop_scores_impl(const void* k, int32_t kv_dtype, const void* probes, int32_t B, int32_t Hkv, int64_t N,
                           int32_t d, int32_t P, float sm_scale, float* scores, void* ws, size_t ws_bytes,
                           hipStream_t s) {
  VC_REQUIRE(k && probes && scores, "k / probes / scores is NULL");
  VC_REQUIRE(valid_dtype(kv_dtype), "bad kv_dtype");
  VC_REQUIRE(B > 0 && Hkv > 0 && N > 0, "bad shape");
  VC_REQUIRE(P >= 1 && P <= kDropMaxProbes, "n_probes must be in [1, %d] (got %d)", kDropMaxProbes, P);
  VC_REQUIRE(sm_scale > 0.f && sm_scale < INFINITY, "sm_scale must be positive and finite");
  VC_UNSUPPORTED(d == 64 || d == 128, "token-drop scoring supports d = 64 or 128 (got %d)", d);
  size_t need = scores_ws_bytes(B, Hkv, N, P);
  if (!ws || ws_bytes < need) {
    set_error("drop-score workspace needs %zu bytes (got %zu)", need, ws_bytes);
    return VC_ERR_WORKSPACE;
  }
  int nch = drop_chunks(N);
  size_t n = static_cast<size_t>(B) * Hkv * nch * P;
  float* sm = static_cast<float*>(ws);
  float* sl = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up(n * sizeof(float), 256));
  float* off = reinterpret_cast<float*>(static_cast<char*>(ws) + 2 * align_up(n * sizeof(float), 256));
  dim3 grid(nch, static_cast<unsigned>(B * Hkv));
  float qs = sm_scale * kLog2e;
  const bf16_t* pr = static_cast<const bf16_t*>(probes);
#define VC_DS(D_, T_)                                                                                               \
  do {                                                                                                              \
    hipLaunchKernelGGL((drop_stats_kernel<D_, T_>), grid, dim3(256), 0, s, static_cast<const T_*>(k), pr, Hkv, N, P, \
                       qs, nch, sm, sl);                                                                            \
    hipLaunchKernelGGL(drop_stats_merge_kernel, dim3(static_cast<unsigned>(B * Hkv)), dim3(256), 0, s, sm, sl, nch, P, \
                       off);                                                                                        \
    hipLaunchKernelGGL((drop_scores_kernel<D_, T_>), grid, dim3(256), 0, s, static_cast<const T_*>(k), pr, Hkv, N,  \
                       P, qs, off, scores);                                                                         \
  } while (0)
  if (kv_dtype == VC_BF16) {
    if (d == 128) VC_DS(128, bf16_t); else VC_DS(64, bf16_t);
  } else {
    if (d == 128) VC_DS(128, float); else VC_DS(64, float);
  }
#undef VC_DS
  VC_LAUNCHED("drop_scores_kernel");
  return VC_OK;
}

size_t drop_select_ws_bytes(int32_t B, int32_t Hkv, int64_t N) { return sel_ws_bytes(B, Hkv, N); }

vc_status drop_select_impl(const float* scores, int32_t B, int32_t Hkv, int64_t N, int64_t n_keep, int32_t* kept,
                           int64_t kept_pitch, void* ws, size_t ws_bytes, hipStream_t s) {
  VC_REQUIRE(scores && kept, "scores / kept_idx is NULL");
  VC_REQUIRE(B > 0 && Hkv > 0 && N > 0, "bad shape");
  VC_REQUIRE(n_keep >= 1 && n_keep <= N, "n_keep must be in [1, N] (got %lld, N %lld)", (long long)n_keep,
             (long long)N);
  VC_REQUIRE(N <= 0x7fffffffLL, "N too large for int32 indices");
  const size_t need = sel_ws_bytes(B, Hkv, N);
  if (!ws || ws_bytes < need) {
    set_error("drop-select workspace needs %zu bytes (got %zu)", need, ws_bytes);
    return VC_ERR_WORKSPACE;
  }
  const int BH = B * Hkv, S = sel_slices(N);
  uint32_t* hist = static_cast<uint32_t*>(ws);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + sel_hist_bytes(B, Hkv));
  const int64_t nh = 4 * static_cast<int64_t>(BH) * 256;
  hipLaunchKernelGGL(sel_zero_kernel, dim3(static_cast<unsigned>(cdiv(nh, 256))), dim3(256), 0, s, hist, nh);
  const dim3 grid(static_cast<unsigned>(S), static_cast<unsigned>(BH));
  for (int pass = 0; pass < 4; ++pass)
    hipLaunchKernelGGL(sel_hist_kernel, grid, dim3(kSelT), 0, s, scores, N, n_keep, hist, BH, pass);
  hipLaunchKernelGGL(sel_count_kernel, grid, dim3(kSelT), 0, s, scores, N, n_keep, hist, BH, cnt, S);
  hipLaunchKernelGGL(sel_write_kernel, grid, dim3(kSelT), 0, s, scores, N, n_keep, hist, BH, cnt, S, kept,
                     kept_pitch);
  VC_LAUNCHED("sel_write_kernel");
  return VC_OK;
}

vc_status gather_impl(const void* src, int32_t kv_dtype, int32_t B, int32_t Hkv, int64_t src_rows, int32_t d,
                      const int32_t* idx, int64_t n, int64_t idx_pitch, void* dst, int64_t dst_rows, hipStream_t s) {
  VC_REQUIRE(src && idx && dst, "NULL pointer argument");
  VC_REQUIRE(valid_dtype(kv_dtype), "bad kv_dtype");
  VC_REQUIRE(B > 0 && Hkv > 0 && d > 0 && n >= 0 && n <= dst_rows, "bad shape");
  size_t row_bytes = static_cast<size_t>(d) * dtype_bytes(kv_dtype);
  VC_UNSUPPORTED(row_bytes % 16 == 0, "row size must be a multiple of 16 bytes");
  if (n == 0) return VC_OK;
  int rv = static_cast<int>(row_bytes / 16);
  dim3 grid(static_cast<unsigned>(cdiv(n * rv, 256)), static_cast<unsigned>(B * Hkv));
  if ((rv & (rv - 1)) == 0) {
    hipLaunchKernelGGL(gather_rows_pow2_kernel, grid, dim3(256), 0, s, static_cast<const uint4*>(src), src_rows,
                       __builtin_ctz(static_cast<unsigned>(rv)), idx, n, idx_pitch, static_cast<uint4*>(dst),
                       dst_rows);
    VC_LAUNCHED("gather_rows_pow2_kernel");
    return VC_OK;
  }
  hipLaunchKernelGGL(gather_rows_kernel<1>, grid, dim3(256), 0, s, static_cast<const uint4*>(src), src_rows, rv, idx, n,
                     idx_pitch, static_cast<uint4*>(dst), dst_rows);
  VC_LAUNCHED("gather_rows_kernel");
  return VC_OK;
}

}  // namespace vc

using namespace vc;

extern "C" int64_t vc_drop_keep_count(float keep_ratio, int64_t N) {
  if (N <= 0 || !(keep_ratio > 0.f)) return 0;
  double x = static_cast<double>(keep_ratio) * static_cast<double>(N);
  int64_t n = static_cast<int64_t>(ceil(x - 1e-9));
  if (n < 1) n = 1;
  if (n > N) n = N;
  return n;
}

extern "C" size_t vc_drop_scores_workspace_bytes(int32_t B, int32_t Hkv, int64_t N, int32_t n_probes) {
  if (B <= 0 || Hkv <= 0 || N <= 0 || n_probes <= 0) return 0;
  return scores_ws_bytes(B, Hkv, N, n_probes);
}

extern "C" vc_status vc_drop_scores(const void* k, int32_t kv_dtype, const void* probes, int32_t B, int32_t Hkv,
                                    int64_t N, int32_t d, int32_t n_probes, float sm_scale, float* scores, void* ws,
                                    size_t ws_bytes, void* stream) {
  clear_error();
  return drop_scores_impl(k, kv_dtype, probes, B, Hkv, N, d, n_probes, sm_scale, scores, ws, ws_bytes,
                          as_stream(stream));
}

extern "C" size_t vc_drop_select_workspace_bytes(int32_t B, int32_t Hkv, int64_t N) {
  if (B <= 0 || Hkv <= 0 || N <= 0) return 0;
  return sel_ws_bytes(B, Hkv, N);
}

extern "C" vc_status vc_drop_select(const float* scores, int32_t B, int32_t Hkv, int64_t N, int64_t n_keep,
                                    int32_t* kept_idx, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  return drop_select_impl(scores, B, Hkv, N, n_keep, kept_idx, n_keep, ws, ws_bytes, as_stream(stream));
}

extern "C" vc_status vc_gather_rows(const void* src, int32_t kv_dtype, int32_t B, int32_t Hkv, int64_t src_rows,
                                    int32_t d, const int32_t* idx, int64_t n, void* dst, int64_t dst_rows,
                                    void* stream) {
  clear_error();
  return gather_impl(src, kv_dtype, B, Hkv, src_rows, d, idx, n, n, dst, dst_rows, as_stream(stream));
}
