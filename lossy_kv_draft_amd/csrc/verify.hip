// Verification: causal attention of the k-row draft window over the full KV cache.
//
// Summary page "VeriCache: Turning Lossy KV Cache into Lossless LLM Inference",
// "What the paper found" and "Original abstract": drafted tokens are verified
// against the full KV cache so that the output equals full-KV greedy decoding.
// Row i of a sequence with context length L attends to cache rows [0, L + i] (the
// window's own keys/values are already written at rows [L, L + k)).
//
// bf16 paths (matrix cores, v_mfma_f32_16x16x32_bf16, float32 accumulation).  The
// rows of all Hq/Hkv q-heads that read one kv-head are stacked (M = (Hq/Hkv) * k
// rows) so every K/V tile is read from HBM once per row block; each of the 4 waves
// of a workgroup owns 16*RT rows.  Per tile the wave computes S^T = K Q^T (tokens x
// rows), masks positions beyond each row's limit, runs an online softmax per row
// (base 2), rounds P to bf16 and accumulates O^T += V^T P^T.  The probabilities stay
// in the lanes that produced them: the S^T output layout of a pair of 16-token tiles
// is exactly the B-operand layout of the P.V product once the 32 token indices of
// that product are enumerated in the same (permuted) order on both operands.
//   d = 128 (verify_tile_kernel): K and V tiles go global -> LDS through the direct
//   LDS load, V is read transposed by the LDS transpose load; see the notes above
//   verify_tiles.
//   d = 64 (verify_mfma_kernel): grid = (splits, row blocks, B*Hkv); K staged in LDS
//   as [token][d] and V transposed as [d][token] by the waves themselves, the global
//   loads of the next tile issued before the current tile is computed (register
//   prefetch).
//
// float32 path: one wave per (row, split), lanes over d, float32 throughout.
//
// Splits are cut at absolute cache positions (multiples of split_tokens); every row
// is reduced over the same tiles in the same order whatever k, its window position
// or the neighbouring rows are (tiles and splits past a row's limit contribute
// exact zeros), and the merge kernel combines splits in split order.  So row i of a
// k-row call equals bit for bit the 1-row call with context L + i.  All sources in
// this file are compiled without floating-point contraction so that every
// instantiation performs the same roundings.

#include <algorithm>

#include "common.h"
#include "decode_common.h"
#include "verify_common.h"

namespace vc {

template <int D, int RT>
__global__ void __launch_bounds__(kVerThreads) verify_mfma_kernel(VerifyArgs a) {
  constexpr int KP = D + 8;          // K tile row pitch (bf16 elements)
  constexpr int VP = kVerTile + 8;   // V^T row pitch
  constexpr int KS = D / 32;         // k-steps of the score product
  constexpr int DT = D / 16;         // 16-channel tiles of the output
  constexpr int KCH = kVerTile * D / 8 / kVerThreads;   // 16-byte K chunks per thread
  constexpr int VCH = kVerTile * D / 16 / kVerThreads;  // (2 tokens x 8 channels) V items per thread
  __shared__ __attribute__((aligned(16))) bf16_t k_lds[kVerTile * KP];
  __shared__ __attribute__((aligned(16))) bf16_t vt_lds[D * VP];

  const int split = blockIdx.x, rblk = blockIdx.y, bh = blockIdx.z;
  const int b = bh / a.Hkv, hk = bh % a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, kb = lane >> 4;
  const int M = a.H * a.k;
  const int row0 = rblk * a.rows_per_block + wave * 16 * RT;
  const int64_t L = ver_ctx_len(a, b);
  const int64_t limit = L + a.k;  // readable positions [0, limit)
  const int64_t s_begin = static_cast<int64_t>(split) * a.C;
  const int64_t s_end = min(s_begin + a.C, limit);

  const bf16_t* q = static_cast<const bf16_t*>(a.q) + (static_cast<int64_t>(b) * a.Hq + hk * a.H) * a.k * D;
  const bf16_t* kc = static_cast<const bf16_t*>(a.kc) + static_cast<int64_t>(bh) * a.cache_rows * D;
  const bf16_t* vc = static_cast<const bf16_t*>(a.vc) + static_cast<int64_t>(bh) * a.cache_rows * D;

  bf16x8_t qf[RT][KS];
  int64_t rlim[RT];  // last position row may see (inclusive); -1 for padding rows
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    int row = row0 + rt * 16 + l16;
    rlim[rt] = row < M ? L + (row % a.k) : -1;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      Pack16 p;
      p.u = make_uint4(0, 0, 0, 0);
      if (row < M) p.u = *reinterpret_cast<const uint4*>(q + static_cast<int64_t>(row) * D + 32 * ks + 8 * kb);
      qf[rt][ks] = p.v;
    }
  }

  f32x4_t o[DT][RT];
  float m[RT], lsum[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m[rt] = -INFINITY;
    lsum[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  uint4 kreg[KCH];
  uint4 vreg[VCH][2];
  auto gload = [&](int64_t t0) {
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      int id = tid + j * kVerThreads;
      int t = id / (D / 8), c8 = id % (D / 8);
      int64_t pos = t0 + t;
      kreg[j] = pos < limit ? *reinterpret_cast<const uint4*>(kc + pos * D + c8 * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < VCH; ++j) {
      int id = tid + j * kVerThreads;
      int tp = id / (D / 8), c8 = id % (D / 8);
      int64_t pos = t0 + 2 * tp;
      vreg[j][0] = pos < limit ? *reinterpret_cast<const uint4*>(vc + pos * D + c8 * 8) : make_uint4(0, 0, 0, 0);
      vreg[j][1] = pos + 1 < limit ? *reinterpret_cast<const uint4*>(vc + (pos + 1) * D + c8 * 8) : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      int id = tid + j * kVerThreads;
      int t = id / (D / 8), c8 = id % (D / 8);
      *reinterpret_cast<uint4*>(k_lds + t * KP + c8 * 8) = kreg[j];
    }
#pragma unroll
    for (int j = 0; j < VCH; ++j) {
      int id = tid + j * kVerThreads;
      int tp = id / (D / 8), c8 = id % (D / 8);
      Pack16 x0, x1;
      x0.u = vreg[j][0];
      x1.u = vreg[j][1];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t w = static_cast<uint32_t>(x0.h[e]) | (static_cast<uint32_t>(x1.h[e]) << 16);
        *reinterpret_cast<uint32_t*>(vt_lds + (c8 * 8 + e) * VP + 2 * tp) = w;
      }
    }
  };

  if (s_begin < s_end) gload(s_begin);
  for (int64_t t0 = s_begin; t0 < s_end; t0 += kVerTile) {
    __syncthreads();
    lstore();
    __syncthreads();
    if (t0 + kVerTile < s_end) gload(t0 + kVerTile);
    if (row0 >= M) continue;  // padding wave: only helps staging

    // ---- S^T = K Q^T : s[tt][rt][r] = score(token t0 + 16 tt + 4 kb + r, row row0 + 16 rt + l16)
    f32x4_t s[4][RT];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) s[tt][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        Pack16 ka;
        ka.u = *reinterpret_cast<const uint4*>(k_lds + (tt * 16 + l16) * KP + 32 * ks + 8 * kb);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          s[tt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka.v, qf[rt][ks], s[tt][rt], 0, 0, 0);
      }
    }

    // ---- online softmax per row; P^T operand built in place
    bf16x8_t pb[RT][2];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float mt = -INFINITY;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          int64_t pos = t0 + tt * 16 + 4 * kb + r;
          float v = pos <= rlim[rt] ? s[tt][rt][r] * a.qscale : -INFINITY;
          s[tt][rt][r] = v;
          mt = fmaxf(mt, v);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      float mnew = fmaxf(m[rt], mt);
      float alpha = mnew == -INFINITY ? 1.f : exp2f(m[rt] - mnew);
      m[rt] = mnew;
      lsum[rt] *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt][rt] *= alpha;
      Pack16 p0, p1;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float p = mnew == -INFINITY ? 0.f : exp2f(s[tt][rt][r] - mnew);
          __bf16 pbv = static_cast<__bf16>(p);
          lsum[rt] += static_cast<float>(pbv);
          Pack16& dst = (tt < 2) ? p0 : p1;
          dst.v[(tt & 1) * 4 + r] = pbv;
        }
      pb[rt][0] = p0.v;
      pb[rt][1] = p1.v;
    }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16_t* vr = vt_lds + (dt * 16 + l16) * VP + 32 * ks2 + 4 * kb;
        uint2 lo = *reinterpret_cast<const uint2*>(vr);
        uint2 hi = *reinterpret_cast<const uint2*>(vr + 16);
        Pack16 va;
        va.u = make_uint4(lo.x, lo.y, hi.x, hi.y);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          o[dt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va.v, pb[rt][ks2], o[dt][rt], 0, 0, 0);
      }
    }
  }

  if (row0 >= M) return;
  // ---- partials: o[dt][rt][r] = O^T[d = 16 dt + 4 kb + r][row = row0 + 16 rt + l16]
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float l = lsum[rt];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    int row = row0 + rt * 16 + l16;
    if (row >= M) continue;
    int64_t pr = (static_cast<int64_t>(bh) * a.splits + split) * M + row;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<f32x4_t*>(a.part_o + pr * D + dt * 16 + 4 * kb) = o[dt][rt];
    if (kb == 0) {
      a.part_ml[pr * 2] = m[rt];
      a.part_ml[pr * 2 + 1] = l;
    }
  }
}

// RT 16-row tiles per wave, W waves per workgroup (16 RT W rows per workgroup), a
// ring of S tiles.
template <int RT, int W, int S, int PF = kVtPrefetch>
__device__ __forceinline__ void verify_tiles(const VerifyArgs& a, int split, int row0, int bh, VtStage* ring) {
  constexpr int D = 128, KS = D / 32, DT = D / 16;
  static_assert(S >= 2 && kVtTile % W == 0, "ring shape");
  constexpr int kWaveRows = kVtTile / W;   // rows each wave copies per tile
  constexpr int kCopies = kWaveRows / 4;   // instructions per wave per tile, K and V each
  static_assert(kWaveRows % 4 == 0, "copy shape");
  constexpr int NT = kVtTile / 16;  // 16-position score tiles per tile
  constexpr int KP = kVtTile / 32;  // 32-position k-steps of the P V product per tile
  const int b = bh / a.Hkv, hk = bh % a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, kb = lane >> 4;
  const int M = a.H * a.k;
  const int64_t L = ver_ctx_len(a, b);
  const int64_t limit = L + a.k;  // readable positions [0, limit)
  const int64_t s_begin = static_cast<int64_t>(split) * a.C;
  const int64_t s_end = min(s_begin + a.C, limit);
  const int ntile = s_end > s_begin ? static_cast<int>((s_end - s_begin + kVtTile - 1) / kVtTile) : 0;

  const bf16_t* q = static_cast<const bf16_t*>(a.q) + (static_cast<int64_t>(b) * a.Hq + hk * a.H) * a.k * D;
  bf16x8_t qf[RT][KS];
  int64_t rlim[RT];  // last position the row may see (inclusive); -1 for padding rows
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = row0 + rt * 16 + l16;
    rlim[rt] = row < M ? L + (row % a.k) : -1;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      Pack16 p;
      p.u = make_uint4(0, 0, 0, 0);
      if (row < M) p.u = *reinterpret_cast<const uint4*>(q + static_cast<int64_t>(row) * D + 32 * ks + 8 * kb);
      qf[rt][ks] = p.v;
    }
  }
  f32x4_t o[DT][RT], lacc[RT];
  float m[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m[rt] = -INFINITY;
    lacc[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  Pack16 ones;
  ones.u = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);  // bf16 1.0

  // copies: wave w moves rows kWaveRows w .. kWaveRows (w + 1) - 1 of the K and V
  // tiles, 4 rows per instruction (lane l: row base + l / 16, LDS chunk l % 16)
  const unsigned char* kbase = static_cast<const unsigned char*>(a.kc) + static_cast<size_t>(bh) * a.cache_rows * kVtRow;
  const unsigned char* vbase = static_cast<const unsigned char*>(a.vc) + static_cast<size_t>(bh) * a.cache_rows * kVtRow;
  uint32_t voff[kCopies];  // byte offset within a tile of this lane's chunk (the global chunk at LDS chunk lane % 16)
#pragma unroll
  for (int i = 0; i < kCopies; ++i) {
    const int r = kWaveRows * wave + 4 * i + (lane >> 4);
    voff[i] = r * kVtRow + vt_chunk(r, lane & 15) * 16;
  }
  auto issue = [&](int j) {
    const int64_t t0 = s_begin + static_cast<int64_t>(j) * kVtTile;
    // descriptors over the tile's readable rows: rows at or past the end read as zeros
    const uint32_t nb = static_cast<uint32_t>(min(limit - t0, static_cast<int64_t>(kVtTile))) * kVtRow;
    const vt_rsrc_t kr = vt_rsrc(kbase + t0 * kVtRow, nb);
    const vt_rsrc_t vr = vt_rsrc(vbase + t0 * kVtRow, nb);
    unsigned char* st = ring[j % S];
#pragma unroll
    for (int i = 0; i < kCopies; ++i) {
      const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(st + (kWaveRows * wave + 4 * i) * kVtRow));
      lds_copy16_buf(kr, voff[i], dst);
      lds_copy16_buf(vr, voff[i], dst + kVtTileBytes);
    }
  };
  // per-lane LDS byte offsets of the operand reads within a stage: K fragment (k-step
  // ks) of position tile 0, V fragment (channel tile dt) of position 4 kb + e; the other
  // tiles and halves are constant offsets from these (16-position tiles 4096 bytes
  // apart, halves 8192), which the LDS reads take as immediates
  uint32_t kofs[KS], vofs[DT];
  {
    const int e = l16 >> 2, qd = l16 & 3, ra = 4 * kb + e;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kofs[ks] = l16 * kVtRow + ((4 * ks + kb) ^ l16) * 16;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vofs[dt] = ra * kVtRow + vt_chunk(ra, 2 * dt + (qd >> 1)) * 16 + 8 * (qd & 1);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the query loads complete before the copies start
  for (int t = 0; t < S - 1 && t < ntile; ++t) issue(t);
  for (int j = 0; j < ntile; ++j) {
    vt_wait<2 * kCopies, S - 2>(ntile - 1 - j);  // this wave's copies of tile j have landed
    __syncthreads();  // ... and every wave's; every wave is done with tile j - 1
    if (j + S - 1 < ntile) issue(j + S - 1);  // into the stage of tile j - 1
    const unsigned char* kt = ring[j % S];
    const unsigned char* vt = kt + kVtTileBytes;
    const int64_t t0 = s_begin + static_cast<int64_t>(j) * kVtTile;
    if (row0 < M) {  // wave-uniform; padding waves only copy
      // the offsets as values of this iteration, so that their sums with the constant
      // tile and half offsets are not hoisted out of the loop as registers of their own
      uint32_t ko[KS], vo[DT];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        ko[ks] = kofs[ks];
        asm volatile("" : "+v"(ko[ks]));
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        vo[dt] = vofs[dt];
        asm volatile("" : "+v"(vo[dt]));
      }
      // The tile in 32-position halves (scores, softmax and both products of one half
      // before the next), so that a wave holds the scores of half a tile
#pragma unroll
      for (int hh = 0; hh < KP; ++hh) {
        const int64_t h0 = t0 + 32 * hh;
        // ---- S^T = K Q^T: s[tt][rt][r] = score(position h0 + 16 tt + 4 kb + r, row row0 + 16 rt + l16);
        //      K fragments are read ahead of the products that take them
        f32x4_t s[2][RT];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) s[tt][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        // fragment i = (step i / 2, position tile 2 hh + i % 2); PF of them in flight
        auto kload = [&](Pack16& dst, int i) {
          const int ks = i / 2, tt = 2 * hh + i % 2;
          dst.u = *reinterpret_cast<const uint4*>(kt + ko[ks] + 16 * tt * kVtRow);
        };
        Pack16 kf[PF];
#pragma unroll
        for (int i = 0; i < PF; ++i) kload(kf[i], i);
#pragma unroll
        for (int i = 0; i < KS * 2; ++i) {
          const Pack16 ka = kf[i % PF];
          if (i + PF < KS * 2) kload(kf[i % PF], i + PF);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
            s[i % 2][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka.v, qf[rt][i / 2], s[i % 2][rt], 0, 0, 0);
        }
        // ---- V^T fragments (A operand of the P V product), PF of them in flight:
        //      fragment dt = channel tile; k-slot j of lane group kb is position
        //      32 hh + 4 kb + j (j < 4), 32 hh + 16 + 4 kb + (j - 4) otherwise, as in P^T
        auto vload = [&](Pack16& dst, int dt) {  // rows 32 hh + 4 kb + e and 16 further: same swizzle
          const uint2 lo = lds_read_tr16(vt + vo[dt] + 32 * hh * kVtRow);
          const uint2 hi = lds_read_tr16(vt + vo[dt] + (32 * hh + 16) * kVtRow);
          dst.u = make_uint4(lo.x, lo.y, hi.x, hi.y);
        };
        Pack16 vf[PF];
#pragma unroll
        for (int i = 0; i < PF; ++i) vload(vf[i], i);  // in flight during the softmax
        // ---- softmax per row over the half
        const bool full = h0 + 31 <= L;  // every row sees every position of the half
        bf16x8_t pb[RT];
        float mt[RT];
        bool up = false;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          mt[rt] = -INFINITY;
          if (full) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
              for (int r = 0; r < 4; ++r) mt[rt] = fmaxf(mt[rt], s[tt][rt][r]);
          } else {
            const int lr = static_cast<int>(max(min(rlim[rt] - h0, static_cast<int64_t>(32)), static_cast<int64_t>(-1)));
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const float v = 16 * tt + 4 * kb + r <= lr ? s[tt][rt][r] : -INFINITY;
                s[tt][rt][r] = v;
                mt[rt] = fmaxf(mt[rt], v);
              }
          }
          up = up | (mt[rt] * a.qscale > m[rt] + 8.f);
        }
        // The running maximum moves only when a score exceeds it by more than 8: a lane
        // tests its own scores (rounding is monotone, so fl(max x * q) > m + 8 exactly
        // when some fl(x * q) > m + 8), one wave vote over all of the wave's rows gates
        // the row maxima, and each row still decides alone
        if (__any(up)) {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            const float mts = group4_max(mt[rt]) * a.qscale;
            if (mts > m[rt] + 8.f) {  // the row's own decision (all lanes of a row agree)
              const float al = __builtin_amdgcn_exp2f(m[rt] - mts);  // 0 on the row's first scores
#pragma unroll
              for (int dt = 0; dt < DT; ++dt) o[dt][rt] *= al;
              lacc[rt] *= al;
              m[rt] = mts;
            }
          }
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const float nm = m[rt] == -INFINITY ? 0.f : -m[rt];
          Pack16 pp;
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int r = 0; r < 4; r += 2) {
              const f2_t ex = {__builtin_amdgcn_exp2f(fmaf(s[tt][rt][r], a.qscale, nm)),
                               __builtin_amdgcn_exp2f(fmaf(s[tt][rt][r + 1], a.qscale, nm))};
              const bf16x2_t h = __builtin_convertvector(ex, bf16x2_t);
              pp.v[tt * 4 + r] = h[0];
              pp.v[tt * 4 + r + 1] = h[1];
            }
          pb[rt] = pp.v;
          lacc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones.v, pb[rt], lacc[rt], 0, 0, 0);
        }
        // ---- O^T += V^T P^T over the half
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const Pack16 va = vf[dt % PF];
          if (dt + PF < DT) vload(vf[dt % PF], dt + PF);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
            o[dt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va.v, pb[rt], o[dt][rt], 0, 0, 0);
        }
      }
    }
  }

  if (row0 >= M) return;
  // ---- partials: o[dt][rt][r] = O^T[d = 16 dt + 4 kb + r][row = row0 + 16 rt + l16]
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = row0 + rt * 16 + l16;
    if (row >= M) continue;
    const int64_t pr = (static_cast<int64_t>(bh) * a.splits + split) * M + row;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<f32x4_t*>(a.part_o + pr * D + dt * 16 + 4 * kb) = o[dt][rt];
    if (kb == 0) {
      a.part_ml[pr * 2] = m[rt];
      a.part_ml[pr * 2 + 1] = lacc[rt][0];
    }
  }
}

// One workgroup per (split, bh, row block), from a one-dimensional grid: the row
// blocks of one (split, bh) share their K and V tiles, so their workgroup ids are
// congruent mod 8 (workgroups go to the eight XCDs, each with its own L2, in id
// order) and lie within 8 * nblk of each other.  Ids past the last (split, bh) exit.
template <int RT, int W, int S>
__global__ void __launch_bounds__(64 * W) verify_tile_kernel(VerifyArgs a, int nblk, int units) {
  __shared__ __attribute__((aligned(16))) VtStage ring[S];
  const int id = blockIdx.x;
  const int u = (id / (8 * nblk)) * 8 + (id & 7);
  if (u >= units) return;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  verify_tiles<RT, W, S>(a, u % a.splits, ((id >> 3) % nblk) * a.rows_per_block + wave * 16 * RT, u / a.splits, ring);
}

// Rows of one kv-head in 8 waves with unequal row tiles: waves 0-3 hold RTA 16-row
// tiles each, waves 4-7 RTB, so every SIMD (waves w and w + 4) carries RTA + RTB
// tiles: 64 (RTA + RTB) rows in one workgroup that reads each K/V tile once (320 rows,
// i.e. 8 q-heads x 40 window rows, as 3 + 2).  One workgroup per (split, sequence,
// kv-head).
template <int RTA, int RTB, int S>
__global__ void __launch_bounds__(512) verify_mixed_kernel(VerifyArgs a) {
  __shared__ __attribute__((aligned(16))) VtStage ring[S];
  const int u = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  if (wave < 4)
    verify_tiles<RTA, 8, S, 2>(a, u % a.splits, wave * 16 * RTA, u / a.splits, ring);
  else
    verify_tiles<RTB, 8, S, 2>(a, u % a.splits, 64 * RTA + (wave - 4) * 16 * RTB, u / a.splits, ring);
}

// Draft-side decode over kept (token-dropped) bf16 rows, d = 128, at most 16 q-heads
// per kv-head: the same tile loop with one query row per q-head, a window of one and
// the context length set to the kept rows minus one, so that row 0 attends to every
// kept row; the S splits cover the kept rows and write the decode partials, and
// decode_merge_kernel adds the full-precision tail rows and combines them.
constexpr int kDdStages = 2;  // LDS ring of decode_dense_kernel (4 waves)
__global__ void __launch_bounds__(kVerThreads) decode_dense_kernel(VerifyArgs a) {
  __shared__ __attribute__((aligned(16))) VtStage ring[kDdStages];
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  verify_tiles<1, 4, kDdStages>(a, blockIdx.x, 16 * wave, blockIdx.z, ring);
}

// float32 path: one 64-lane wave per (row, split); lanes cover d (d <= 256).
template <typename T>
__global__ void __launch_bounds__(256) verify_f32_kernel(VerifyArgs a) {
  const int split = blockIdx.x, bh = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.y * 4 + wave;
  const int b = bh / a.Hkv, hk = bh % a.Hkv;
  const int M = a.H * a.k, d = a.d;
  if (row >= M) return;
  const int64_t L = ver_ctx_len(a, b);
  const int64_t last = L + (row % a.k);
  const int64_t s_begin = static_cast<int64_t>(split) * a.C;
  const int64_t s_end = min(s_begin + a.C, last + 1);
  const T* q = static_cast<const T*>(a.q) + ((static_cast<int64_t>(b) * a.Hq + hk * a.H) * a.k + row) * d;
  const T* kc = static_cast<const T*>(a.kc) + static_cast<int64_t>(bh) * a.cache_rows * d;
  const T* vc = static_cast<const T*>(a.vc) + static_cast<int64_t>(bh) * a.cache_rows * d;
  float qv[4], ov[4];
  for (int j = 0; j < 4; ++j) {
    int c = lane + 64 * j;
    qv[j] = c < d ? Elem<T>::load(q, c) : 0.f;
    ov[j] = 0.f;
  }
  float mrun = -INFINITY, lrun = 0.f;
  for (int64_t pos = s_begin; pos < s_end; ++pos) {
    float x = 0.f;
    for (int j = 0; j < 4; ++j) {
      int c = lane + 64 * j;
      if (c < d) x = fmaf(qv[j], Elem<T>::load(kc, pos * d + c), x);
    }
    x = warp_sum(x) * a.qscale;
    float mnew = fmaxf(mrun, x);
    float al = exp2f(mrun - mnew);
    float p = exp2f(x - mnew);
    lrun = lrun * al + p;
    mrun = mnew;
    for (int j = 0; j < 4; ++j) {
      int c = lane + 64 * j;
      if (c < d) ov[j] = fmaf(p, Elem<T>::load(vc, pos * d + c), ov[j] * al);
    }
  }
  int64_t pr = (static_cast<int64_t>(bh) * a.splits + split) * M + row;
  for (int j = 0; j < 4; ++j) {
    int c = lane + 64 * j;
    if (c < d) a.part_o[pr * d + c] = ov[j];
  }
  if (lane == 0) {
    a.part_ml[pr * 2] = mrun;
    a.part_ml[pr * 2 + 1] = lrun;
  }
}

// Merge of the split partials in split order; one thread per (row, V consecutive
// channels).
template <typename T, int V>
__global__ void __launch_bounds__(256) verify_merge_kernel(VerifyArgs a, void* out, float* lse) {
  typedef float fv_t __attribute__((ext_vector_type(V)));
  const int bh = blockIdx.y;
  const int M = a.H * a.k, d = a.d, dv = d / V;
  const int e = static_cast<int>(blockIdx.x) * 256 + static_cast<int>(threadIdx.x);  // M * dv < 2^31 (host check)
  if (e >= M * dv) return;
  const int row = e / dv, c = (e - row * dv) * V;
  const int b = bh / a.Hkv, hk = bh % a.Hkv;
  const int S = a.splits;
  const float2* ml = reinterpret_cast<const float2*>(a.part_ml) + static_cast<int64_t>(bh) * S * M + row;
  const float* po = a.part_o + (static_cast<int64_t>(bh) * S * M + row) * d + c;
  // the partials of 8 splits are loaded at once (V channels per thread); the sums
  // still run in split order
  float Mx = -INFINITY;
  float Lsum = 0.f;
  fv_t O = {};
  float2 p[8];
  fv_t ov[8];
  auto load8 = [&](int s0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t sp = min(s0 + j, S - 1);
      p[j] = ml[sp * M];
      ov[j] = *reinterpret_cast<const fv_t*>(po + sp * M * d);
    }
  };
  auto add8 = [&](int s0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (s0 + j >= S) break;
      const float w = p[j].x == -INFINITY ? 0.f : exp2f(p[j].x - Mx);
      Lsum = fmaf(p[j].y, w, Lsum);
#pragma unroll
      for (int v = 0; v < V; ++v) O[v] = fmaf(ov[j][v], w, O[v]);
    }
  };
  if (S <= 8) {  // one round of loads: the maximum from the same (maximum, sum) pairs
    load8(0);
#pragma unroll
    for (int j = 0; j < 8; ++j) Mx = fmaxf(Mx, p[j].x);
    add8(0);
  } else {
    for (int s0 = 0; s0 < S; s0 += 8) {
      float mv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) mv[j] = ml[static_cast<int64_t>(min(s0 + j, S - 1)) * M].x;
#pragma unroll
      for (int j = 0; j < 8; ++j) Mx = fmaxf(Mx, mv[j]);
    }
    for (int s0 = 0; s0 < S; s0 += 8) {
      load8(s0);
      add8(s0);
    }
  }
  int64_t orow = (static_cast<int64_t>(b) * a.Hq + hk * a.H) * a.k + row;
#pragma unroll
  for (int v = 0; v < V; ++v) Elem<T>::store(static_cast<T*>(out), orow * d + c + v, Lsum > 0.f ? O[v] / Lsum : 0.f);
  if (lse && c == 0) lse[orow] = Lsum > 0.f ? (Mx + log2f(Lsum)) * kLn2 : -INFINITY;
}

// Row tiling of the bf16 kernel: RT 16-row tiles per wave, 4 waves per block.
static void verify_tiling(int M, int& RT, int& nblk) {
  nblk = static_cast<int>(cdiv(M, 256));
  int per = static_cast<int>(cdiv(M, nblk));
  RT = static_cast<int>(cdiv(per, 64));
  if (RT < 1) RT = 1;
  if (RT > 4) RT = 4;
  nblk = static_cast<int>(cdiv(M, 64 * RT));
}

// Dense decode over kept rows (see decode_dense_kernel): S row splits of `chunk`
// positions (a multiple of the 64-position tile).
vc_status launch_decode_dense(const vc_ckv* c, const DecodeArgs& d, hipStream_t s) {
  VerifyArgs a{};
  a.q = d.q;
  a.kc = c->k_kept;
  a.vc = c->v_kept;
  a.Hq = c->Hkv * d.H;
  a.Hkv = c->Hkv;
  a.H = d.H;
  a.d = 128;
  a.k = 1;
  a.cache_rows = c->capacity;
  a.ctx_len = c->n_main - 1;
  a.ctx_lens = d.main_lens;
  a.ctx_off = -1;
  a.C = d.chunk;
  a.splits = d.splits;
  a.rows_per_block = 64;
  a.qscale = d.qscale;
  a.part_o = d.part_o;
  a.part_ml = d.part_ml;
  const dim3 grid(static_cast<unsigned>(d.splits), 1, static_cast<unsigned>(c->B * c->Hkv));
  hipLaunchKernelGGL(decode_dense_kernel, grid, dim3(kVerThreads), 0, s, a);
  VC_LAUNCHED("decode_dense_kernel");
  return VC_OK;
}

}  // namespace vc

using namespace vc;

// Workgroups of the bf16 tile kernel that fit on the device at once (queried once;
// 512 without a device).
static int verify_resident() {
  static const int r = [] {
    int dev = 0, cus = 0, per = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 512;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 512;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, verify_tile_kernel<2, 4, 2>, 256, 0) != hipSuccess)
      return 512;
    return (per > 0 ? per : 1) * (cus > 0 ? cus : 1);
  }();
  return r;
}

// The default split: a full cache of cache_rows rows is cut into as many splits per
// (sequence, kv-head) as workgroups fit on the device for all of them at once, so a
// pass over a nearly full cache is one round of workgroups with no short trailing
// split.  It depends on the cache, not on the context length or the window, so the
// calls that must agree bit for bit (a k-row pass and its 1-row steps) share it.
extern "C" int32_t vc_verify_split_tokens(int32_t B, int32_t Hkv, int64_t cache_rows) {
  const int64_t bh = static_cast<int64_t>(B > 0 ? B : 1) * (Hkv > 0 ? Hkv : 1);
  const int64_t S = std::max<int64_t>(1, verify_resident() / bh);
  const int64_t c = cdiv(std::max<int64_t>(cache_rows, 1), S);
  return static_cast<int32_t>(std::min<int64_t>(cdiv(c, kVerTile) * kVerTile, 1ll << 30));
}

extern "C" size_t vc_verify_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int32_t k,
                                            int64_t max_len, int32_t split_tokens) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || k <= 0 || max_len < 0) return 0;
  // the default for the smallest cache that holds max_len + k rows: a larger cache
  // gets a larger default split, so fewer splits and less workspace
  int64_t C = split_tokens > 0 ? split_tokens : vc_verify_split_tokens(B, Hkv, max_len + k);
  int64_t S = cdiv(max_len + k, C);
  if (S < 1) S = 1;
  size_t M = static_cast<size_t>(Hq / Hkv) * k;
  size_t bh = static_cast<size_t>(B) * Hkv;
  return align_up(bh * S * M * d * sizeof(float), 256) + align_up(bh * S * M * 2 * sizeof(float), 256);
}

extern "C" vc_status vc_verify_attn_full(const void* q, const void* k_cache, const void* v_cache, int32_t kv_dtype,
                                         int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int32_t k,
                                         int64_t cache_rows, int64_t ctx_len, const int32_t* ctx_lens,
                                         int32_t split_tokens, float sm_scale, void* out, float* lse, void* ws,
                                         size_t ws_bytes, void* stream) {
  clear_error();
  VC_REQUIRE(q && k_cache && v_cache && out, "q / k_cache / v_cache / out is NULL");
  VC_REQUIRE(valid_dtype(kv_dtype), "bad kv_dtype %d", kv_dtype);
  VC_REQUIRE(B > 0 && Hkv > 0 && Hq > 0 && Hq % Hkv == 0, "bad B/Hq/Hkv (%d, %d, %d)", B, Hq, Hkv);
  VC_REQUIRE(k >= 1 && k <= 1024, "k must be in [1, 1024] (got %d)", k);
  VC_REQUIRE(d > 0, "bad d");
  VC_REQUIRE(ctx_len >= 0 && ctx_len + k <= cache_rows, "ctx_len + k (%lld) exceeds cache_rows %lld",
             (long long)(ctx_len + k), (long long)cache_rows);
  VC_REQUIRE(sm_scale > 0.f && sm_scale < INFINITY, "sm_scale must be positive and finite");
  VC_REQUIRE(split_tokens >= 0 && split_tokens % kVerTile == 0, "split_tokens must be a multiple of %d", kVerTile);
  if (kv_dtype == VC_BF16)
    VC_UNSUPPORTED(d == 64 || d == 128, "bf16 verify supports d = 64 or 128 (got %d)", d);
  else
    VC_UNSUPPORTED(d <= 256, "f32 verify supports d <= 256 (got %d)", d);
  VC_REQUIRE(static_cast<int64_t>(Hq / Hkv) * k * d <= 0x7fffffffLL, "q-heads per kv-head * k * d must be below 2^31");
  const int64_t C = split_tokens > 0 ? split_tokens : vc_verify_split_tokens(B, Hkv, cache_rows);
  size_t need = vc_verify_workspace_bytes(B, Hq, Hkv, d, k, ctx_len, static_cast<int32_t>(C));
  if (!ws || ws_bytes < need) {
    set_error("verify workspace needs %zu bytes (got %zu)", need, ws_bytes);
    return VC_ERR_WORKSPACE;
  }
  VC_REQUIRE(reinterpret_cast<uintptr_t>(ws) % 16 == 0, "verify workspace must be 16-byte aligned");
  VerifyArgs a{};
  a.q = q;
  a.kc = k_cache;
  a.vc = v_cache;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.H = Hq / Hkv;
  a.d = d;
  a.k = k;
  a.cache_rows = cache_rows;
  a.ctx_len = ctx_len;
  a.ctx_lens = ctx_lens;
  a.ctx_off = 0;
  a.C = C;
  a.splits = static_cast<int>(cdiv(ctx_len + k, C));
  a.qscale = sm_scale * kLog2e;
  const int M = a.H * k;
  size_t bh = static_cast<size_t>(B) * Hkv;
  a.part_o = static_cast<float*>(ws);
  a.part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up(bh * a.splits * M * d * sizeof(float), 256));
  hipStream_t s = as_stream(stream);
  if (kv_dtype == VC_BF16 && d == 128) {
    // Row blocks: 4 waves of one 16-row tile (up to 64 rows) or two (128 rows per
    // workgroup), two workgroups per CU with a 2-tile ring; for 128 < M <= 256 one
    // block of 8 waves of two tiles each and a 4-tile ring (one workgroup per CU), so
    // K and V are read once instead of twice.  Larger M: as many 128-row blocks as
    // needed (64-row blocks for M = 320, or 256-row ones, were slower).  The arithmetic
    // of a row does not depend on the block shape.
    const int W = M > 128 && M <= 256 ? 8 : 4;
    const int RT = M <= 16 * W ? 1 : 2;
    const int nblk = static_cast<int>(cdiv(M, 16 * W * RT));
    a.rows_per_block = 16 * W * RT;
    const int units = a.splits * static_cast<int>(bh);
    const dim3 grid(static_cast<unsigned>(cdiv(units, 8) * 8 * nblk));
    if (M > 256 && M <= 320) {
      // one 8-wave block per (split, kv-head): 3 row tiles in waves 0-3, 2 in waves 4-7
      a.rows_per_block = 320;
      hipLaunchKernelGGL((verify_mixed_kernel<3, 2, 4>), dim3(static_cast<unsigned>(units)), dim3(512), 0, s, a);
    } else if (W == 8)
      hipLaunchKernelGGL((verify_tile_kernel<2, 8, 4>), grid, dim3(512), 0, s, a, nblk, units);
    else if (RT == 1)
      hipLaunchKernelGGL((verify_tile_kernel<1, 4, 2>), grid, dim3(256), 0, s, a, nblk, units);
    else
      hipLaunchKernelGGL((verify_tile_kernel<2, 4, 2>), grid, dim3(256), 0, s, a, nblk, units);
    VC_LAUNCHED("verify_tile_kernel");
    dim3 mgrid(static_cast<unsigned>(cdiv(static_cast<int64_t>(M) * d / 4, 256)), static_cast<unsigned>(bh));
    hipLaunchKernelGGL((verify_merge_kernel<bf16_t, 4>), mgrid, dim3(256), 0, s, a, out, lse);
  } else if (kv_dtype == VC_BF16) {
    int RT, nblk;
    verify_tiling(M, RT, nblk);
    a.rows_per_block = 64 * RT;
    dim3 grid(a.splits, nblk, static_cast<unsigned>(bh));
    // d = 64 (d = 128 took the tile kernels above)
#define VC_VER_LAUNCH(RT_) \
  hipLaunchKernelGGL((verify_mfma_kernel<64, RT_>), grid, dim3(kVerThreads), 0, s, a)
    if (RT == 1) VC_VER_LAUNCH(1);
    else if (RT == 2) VC_VER_LAUNCH(2);
    else if (RT == 3) VC_VER_LAUNCH(3);
    else VC_VER_LAUNCH(4);
#undef VC_VER_LAUNCH
    VC_LAUNCHED("verify_mfma_kernel");
    dim3 mgrid(static_cast<unsigned>(cdiv(static_cast<int64_t>(M) * d / 4, 256)), static_cast<unsigned>(bh));
    hipLaunchKernelGGL((verify_merge_kernel<bf16_t, 4>), mgrid, dim3(256), 0, s, a, out, lse);
  } else {
    dim3 grid(a.splits, static_cast<unsigned>(cdiv(M, 4)), static_cast<unsigned>(bh));
    hipLaunchKernelGGL(verify_f32_kernel<float>, grid, dim3(256), 0, s, a);
    VC_LAUNCHED("verify_f32_kernel");
    if (d % 4 == 0) {
      dim3 mgrid(static_cast<unsigned>(cdiv(static_cast<int64_t>(M) * d / 4, 256)), static_cast<unsigned>(bh));
      hipLaunchKernelGGL((verify_merge_kernel<float, 4>), mgrid, dim3(256), 0, s, a, out, lse);
    } else {
      dim3 mgrid(static_cast<unsigned>(cdiv(static_cast<int64_t>(M) * d, 256)), static_cast<unsigned>(bh));
      hipLaunchKernelGGL((verify_merge_kernel<float, 1>), mgrid, dim3(256), 0, s, a, out, lse);
    }
  }
  VC_LAUNCHED("verify_merge_kernel");
  return VC_OK;
}
