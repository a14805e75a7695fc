// Draft-side single-token decode attention over the compressed KV cache.
//
// Summary page "VeriCache: Turning Lossy KV Cache into Lossless LLM Inference",
// "What the paper found": drafting runs the target model on the compressed KV
// cache and is HBM-bandwidth-bound.  Keys/values are either KIVI-quantized packed
// codes (dequantized in registers as z + code * s) or token-dropped rows kept in
// full precision, followed by a short full-precision tail.
//
// Generic kernel (any bit width, float32 or bf16 storage, d <= 256):
//   grid = (splits, B*Hkv); one workgroup streams one contiguous range of token
//   positions of one (sequence, kv-head) and serves all Hq/Hkv q-heads that read
//   that kv-head, so each packed row is fetched from HBM once.  Per 32-token tile:
//   dequantize K and V into LDS (float32), scores per (head, token), online
//   softmax per head (base-2, scale folded into q), then P.V accumulated in
//   registers per (head, channel).  Each split writes (m, l, o) partials to the
//   workspace; decode_merge_kernel, launched next, merges the splits of each
//   (sequence, kv-head) in split order (deterministic) and writes the normalized
//   output and the log-sum-exp.  The matrix-core and kept-row kernels cover only
//   the compressed rows; their merge adds the full-precision tail rows itself.

#include <mutex>

#include "decode_common.h"

namespace vc {

constexpr int kDecTile = 32;
constexpr int kDecMaxAcc = 16;     // (H * d) / kDecThreads accumulators per thread
constexpr int kDecTargetBlocks = 2048;

bool decode_mfma_supported(const vc_ckv* c, int H);
int decode_mfma_splits(const vc_ckv* c);
void launch_decode_mfma(const vc_ckv* c, const DecodeArgs& a, dim3 grid, hipStream_t s);
vc_status launch_decode_dense(const vc_ckv* c, const DecodeArgs& a, hipStream_t s);



template <typename P>
__device__ __forceinline__ float load_param(const void* p, int64_t i) {
  return Elem<P>::load(static_cast<const P*>(p), i);
}

__device__ __forceinline__ uint32_t extract_code(const uint32_t* row, int c, int bits) {
  int pos = c * bits;
  int w = pos >> 5, off = pos & 31;
  uint32_t x = row[w] >> off;
  if (off + bits > 32) x |= row[w + 1] << (32 - off);
  return x & ((1u << bits) - 1u);
}

// QUANT = true: packed codes; false: kept (dense) rows.
template <typename T, typename P, bool QUANT>
__global__ void __launch_bounds__(kDecThreads) decode_generic_kernel(DecodeArgs a) {
  extern __shared__ float smem[];
  const int d = a.d, H = a.H;
  const int kpitch = d + 1;
  float* qs = smem;                          // [H][d]
  float* kt = qs + H * d;                    // [kDecTile][d+1]
  float* vt = kt + kDecTile * kpitch;        // [kDecTile][d]
  float* sc = vt + kDecTile * d;             // [H][kDecTile]
  float* alpha = sc + H * kDecTile;          // [H]
  float* mrun = alpha + H;                   // [H]
  float* lrun = mrun + H;                    // [H]

  const int split = blockIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / a.Hkv;
  const int hk = bh % a.Hkv;
  const int tid = threadIdx.x;

  const int64_t main_len = dec_main_len(a, b);
  const int64_t tail_len = dec_tail_len(a, b);
  const int64_t total = main_len + tail_len;
  const int64_t start = static_cast<int64_t>(split) * a.chunk;
  const int64_t end = min(total, start + a.chunk);

  const T* q = static_cast<const T*>(a.q);
  for (int i = tid; i < H * d; i += kDecThreads) {
    int h = i / d, c = i % d;
    qs[i] = Elem<T>::load(q, (static_cast<int64_t>(b) * a.Hkv * H + hk * H + h) * d + c) * a.qscale;
  }
  for (int h = tid; h < H; h += kDecThreads) {
    mrun[h] = -INFINITY;
    lrun[h] = 0.f;
  }
  float acc[kDecMaxAcc];
#pragma unroll
  for (int j = 0; j < kDecMaxAcc; ++j) acc[j] = 0.f;
  __syncthreads();

  const int kw = d * a.k_bits / 32, vw = d * a.v_bits / 32;
  const int vgroups = d / a.G;
  for (int64_t t0 = start; t0 < end; t0 += kDecTile) {
    // ---- stage dequantized K and V of the tile
    for (int i = tid; i < kDecTile * d; i += kDecThreads) {
      int t = i / d, c = i % d;
      int64_t pos = t0 + t;
      float kv = 0.f, vv = 0.f;
      if (pos < end) {
        if (pos < main_len) {
          if constexpr (QUANT) {
            const uint32_t* krow = a.k_codes + (static_cast<int64_t>(bh) * a.capacity + pos) * kw;
            const uint32_t* vrow = a.v_codes + (static_cast<int64_t>(bh) * a.capacity + pos) * vw;
            int64_t kp = (static_cast<int64_t>(bh) * (a.capacity / a.G) + pos / a.G) * d + c;
            int64_t vp = (static_cast<int64_t>(bh) * a.capacity + pos) * vgroups + c / a.G;
            kv = load_param<P>(a.k_zero, kp) + static_cast<float>(extract_code(krow, c, a.k_bits)) * load_param<P>(a.k_scale, kp);
            vv = load_param<P>(a.v_zero, vp) + static_cast<float>(extract_code(vrow, c, a.v_bits)) * load_param<P>(a.v_scale, vp);
          } else {
            int64_t e = (static_cast<int64_t>(bh) * a.capacity + pos) * d + c;
            kv = Elem<T>::load(static_cast<const T*>(a.k_kept), e);
            vv = Elem<T>::load(static_cast<const T*>(a.v_kept), e);
          }
        } else {
          int64_t e = (static_cast<int64_t>(bh) * a.tail_cap + (pos - main_len)) * d + c;
          kv = Elem<T>::load(static_cast<const T*>(a.tail_k), e);
          vv = Elem<T>::load(static_cast<const T*>(a.tail_v), e);
        }
      }
      kt[t * kpitch + c] = kv;
      vt[t * d + c] = vv;
    }
    __syncthreads();
    // ---- scores
    for (int j = tid; j < H * kDecTile; j += kDecThreads) {
      int h = j / kDecTile, t = j % kDecTile;
      float s = -INFINITY;
      if (t0 + t < end) {
        const float* kr = kt + t * kpitch;
        const float* qr = qs + h * d;
        float x = 0.f;
        for (int c = 0; c < d; ++c) x = fmaf(qr[c], kr[c], x);
        s = x;
      }
      sc[j] = s;
    }
    __syncthreads();
    // ---- online softmax, one thread per head
    for (int h = tid; h < H; h += kDecThreads) {
      float mt = -INFINITY;
      for (int t = 0; t < kDecTile; ++t) mt = fmaxf(mt, sc[h * kDecTile + t]);
      float mn = fmaxf(mrun[h], mt);
      float l = 0.f;
      for (int t = 0; t < kDecTile; ++t) {
        float p = exp2f(sc[h * kDecTile + t] - mn);
        sc[h * kDecTile + t] = p;
        l += p;
      }
      float al = exp2f(mrun[h] - mn);
      alpha[h] = al;
      lrun[h] = lrun[h] * al + l;
      mrun[h] = mn;
    }
    __syncthreads();
    // ---- P.V
#pragma unroll
    for (int j = 0; j < kDecMaxAcc; ++j) {
      int i = tid + j * kDecThreads;
      if (i < H * d) {
        int h = i / d, c = i % d;
        float x = acc[j] * alpha[h];
        const float* pr = sc + h * kDecTile;
        for (int t = 0; t < kDecTile; ++t) x = fmaf(pr[t], vt[t * d + c], x);
        acc[j] = x;
      }
    }
    __syncthreads();
  }

  // ---- partials
  const int64_t pbase = static_cast<int64_t>(bh) * a.splits + split;
#pragma unroll
  for (int j = 0; j < kDecMaxAcc; ++j) {
    int i = tid + j * kDecThreads;
    if (i < H * d) a.part_o[pbase * H * d + i] = acc[j];
  }
  for (int h = tid; h < H; h += kDecThreads) {
    a.part_ml[(pbase * H + h) * 2 + 0] = mrun[h];
    a.part_ml[(pbase * H + h) * 2 + 1] = lrun[h];
  }
}

// ------------------------------------------------------------------ host side

vc_status validate_quant_ckv(const vc_ckv* c);

static int decode_splits(const vc_ckv* c) {
  int bh = c->B * c->Hkv;
  int s = static_cast<int>(cdiv(kDecTargetBlocks, bh));
  return s < 1 ? 1 : (s > kDecMaxSplits ? kDecMaxSplits : s);
}

static vc_status validate_decode_ckv(const vc_ckv* c) {
  VC_REQUIRE(c != nullptr, "ckv is NULL");
  if (c->method == VC_QUANT_KIVI) return validate_quant_ckv(c);
  VC_REQUIRE(c->method == VC_DROP_TOPK, "unknown ckv.method %d", c->method);
  VC_REQUIRE(c->B > 0 && c->Hkv > 0 && c->d > 0, "bad B/Hkv/d");
  VC_REQUIRE(valid_dtype(c->kv_dtype), "bad kv_dtype");
  VC_REQUIRE(c->n_main >= 0 && c->n_main <= c->capacity, "n_main must be in [0, capacity]");
  VC_REQUIRE(c->n_main == 0 || (c->k_kept && c->v_kept), "kept arrays are NULL");
  VC_REQUIRE(c->tail_len >= 0 && c->tail_len <= c->tail_cap, "tail_len must be in [0, tail_cap]");
  VC_REQUIRE(c->tail_len == 0 || (c->tail_k && c->tail_v), "tail arrays are NULL");
  return VC_OK;
}

}  // namespace vc

using namespace vc;

extern "C" size_t vc_decode_workspace_bytes(const vc_ckv* c, int32_t Hq) {
  if (!c || c->B <= 0 || c->Hkv <= 0 || c->d <= 0 || Hq <= 0) return 0;
  size_t bh = static_cast<size_t>(c->B) * c->Hkv;
  size_t S = kDecMaxSplits;
  size_t H = Hq / c->Hkv;
  size_t bytes = align_up(bh * S * H * c->d * sizeof(float), 256);
  bytes += align_up(bh * S * H * 2 * sizeof(float), 256);
  return bytes;
}

namespace vc {

// Splits of one decode call and the compressed rows each covers: the kernel is chosen
// by the cache (matrix-core quantized, kept bf16 rows, generic), and so is the split.
struct DecodePlan {
  bool mfma, dense;
  int S;
  int64_t chunk;
};

static DecodePlan plan_decode(const vc_ckv* c, int H) {
  DecodePlan p{};
  p.mfma = decode_mfma_supported(c, H);
  // kept bf16 rows, d = 128: the verification tile loop with one query row per head
  p.dense = !p.mfma && c->method == VC_DROP_TOPK && c->kv_dtype == VC_BF16 && c->d == 128 && H <= 16;
  if (p.mfma) {
    // compressed-row splits (the kernel deals the rows out itself); the tail rows are
    // merged by decode_merge_kernel
    p.S = decode_mfma_splits(c);
    p.chunk = 0;
  } else if (p.dense) {
    // two 4-wave workgroups per compute unit (64 KB of LDS each): the row splits
    // fill the device once; the tail rows are merged by decode_merge_kernel
    const int bh = c->B * c->Hkv;
    p.S = 512 / bh;
    if (p.S < 1) p.S = 1;
    if (p.S > kDecMaxSplits - 1) p.S = kDecMaxSplits - 1;
    p.chunk = cdiv(cdiv(c->n_main > 0 ? c->n_main : 1, p.S), 64) * 64;
  } else {
    p.S = decode_splits(c);
    const int64_t total = c->n_main + c->tail_len;
    p.chunk = cdiv(cdiv(total > 0 ? total : 1, p.S), kDecTile) * kDecTile;
  }
  return p;
}

// Bytes of the split partials a call with S splits writes: outputs, then (max, sum).
static size_t decode_partials_bytes(const vc_ckv* c, int H, int S) {
  const size_t bh = static_cast<size_t>(c->B) * c->Hkv;
  return align_up(bh * S * H * c->d * sizeof(float), 256) + align_up(bh * S * H * 2 * sizeof(float), 256);
}

static vc_status validate_decode_call(const vc_ckv* c, const void* q, int32_t Hq, float sm_scale, const void* out) {
  vc_status st = validate_decode_ckv(c);
  if (st != VC_OK) return st;
  VC_REQUIRE(q && out, "q / out is NULL");
  VC_REQUIRE(Hq > 0 && Hq % c->Hkv == 0, "Hq %d must be a positive multiple of Hkv %d", Hq, c->Hkv);
  VC_REQUIRE(sm_scale > 0.f && sm_scale < INFINITY, "sm_scale must be positive and finite");
  const int H = Hq / c->Hkv;
  VC_UNSUPPORTED(c->d % 32 == 0 && c->d <= 256, "d must be a multiple of 32 and at most 256 (got %d)", c->d);
  VC_UNSUPPORTED(H * c->d <= kDecMaxAcc * kDecThreads, "Hq/Hkv * d = %d exceeds %d", H * c->d,
                 kDecMaxAcc * kDecThreads);
  return VC_OK;
}

// The decode kernel and the merge of its partials, with the partials at ws.
static vc_status decode_launch(const vc_ckv* c, const void* q, int H, float sm_scale, const int32_t* main_lens,
                               const int32_t* tail_lens, void* out, float* lse, const DecodePlan& p, void* ws,
                               hipStream_t s) {
  DecodeArgs a{};
  a.k_codes = c->k_codes;
  a.v_codes = c->v_codes;
  a.k_scale = c->k_scale;
  a.k_zero = c->k_zero;
  a.v_scale = c->v_scale;
  a.v_zero = c->v_zero;
  a.k_kept = c->k_kept;
  a.v_kept = c->v_kept;
  a.tail_k = c->tail_k;
  a.tail_v = c->tail_v;
  a.capacity = c->capacity;
  a.tail_cap = c->tail_cap;
  a.n_main = c->n_main;
  a.tail_len = c->tail_len;
  a.main_lens = main_lens;
  a.tail_lens = tail_lens;
  a.k_bits = c->k_bits;
  a.v_bits = c->v_bits;
  a.G = c->method == VC_QUANT_KIVI ? c->group : 1;
  a.q = q;
  a.out = out;
  a.lse = lse;
  a.Hkv = c->Hkv;
  a.H = H;
  a.d = c->d;
  a.qscale = sm_scale * kLog2e;
  a.splits = p.S;
  a.chunk = p.chunk;
  const size_t bh = static_cast<size_t>(c->B) * c->Hkv;
  char* w = static_cast<char*>(ws);
  a.part_o = reinterpret_cast<float*>(w);
  w += align_up(bh * p.S * H * c->d * sizeof(float), 256);
  a.part_ml = reinterpret_cast<float*>(w);

  const dim3 grid(p.S, static_cast<unsigned>(bh));
  // the matrix-core and kept-row kernels leave the tail rows (bf16, d = 128) to the
  // merge; the generic kernel's splits cover them
  auto merge = [&]() -> vc_status {
    const dim3 mgrid(static_cast<unsigned>(bh), static_cast<unsigned>(H));
    if (p.mfma || p.dense)
      hipLaunchKernelGGL((decode_merge_kernel<bf16_t, true>), mgrid, dim3(kDecThreads), 0, s, a);
    else if (c->kv_dtype == VC_BF16)
      hipLaunchKernelGGL((decode_merge_kernel<bf16_t, false>), mgrid, dim3(kDecThreads), 0, s, a);
    else
      hipLaunchKernelGGL((decode_merge_kernel<float, false>), mgrid, dim3(kDecThreads), 0, s, a);
    VC_LAUNCHED("decode_merge_kernel");
    return VC_OK;
  };
  if (p.mfma) {
    launch_decode_mfma(c, a, grid, s);
    VC_LAUNCHED("decode_mfma_kernel");
    return merge();
  }
  if (p.dense) {
    const vc_status st = launch_decode_dense(c, a, s);
    if (st != VC_OK) return st;
    return merge();
  }
  size_t lds = (static_cast<size_t>(H) * c->d + kDecTile * (c->d + 1) + kDecTile * c->d + H * kDecTile + 3 * H) *
               sizeof(float);
  const bool quant = c->method == VC_QUANT_KIVI;
  const bool bf = c->kv_dtype == VC_BF16;
  const bool pbf = c->param_dtype == VC_BF16;
  if (quant) {
    if (bf && pbf)
      hipLaunchKernelGGL((decode_generic_kernel<bf16_t, bf16_t, true>), grid, dim3(kDecThreads), lds, s, a);
    else if (bf)
      hipLaunchKernelGGL((decode_generic_kernel<bf16_t, float, true>), grid, dim3(kDecThreads), lds, s, a);
    else if (pbf)
      hipLaunchKernelGGL((decode_generic_kernel<float, bf16_t, true>), grid, dim3(kDecThreads), lds, s, a);
    else
      hipLaunchKernelGGL((decode_generic_kernel<float, float, true>), grid, dim3(kDecThreads), lds, s, a);
  } else {
    if (bf)
      hipLaunchKernelGGL((decode_generic_kernel<bf16_t, float, false>), grid, dim3(kDecThreads), lds, s, a);
    else
      hipLaunchKernelGGL((decode_generic_kernel<float, float, false>), grid, dim3(kDecThreads), lds, s, a);
  }
  VC_LAUNCHED("decode_generic_kernel");
  return merge();
}

// ---- the entry point that allocates nothing: its split partials live in `scratch`,
// a file-scope device array (one copy per GPU, held until the process ends).  In host
// code the array's name is only a host-side stand-in: the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
constexpr int kScratchMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[VC_DECODE_NOALLOC_SCRATCH_BYTES];

static vc_status scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[kScratchMaxDevices] = {};
  int dev = -1;
  VC_HIP(hipGetDevice(&dev));
  VC_REQUIRE(dev >= 0 && dev < kScratchMaxDevices, "device %d beyond the %d the library tracks", dev,
             kScratchMaxDevices);
  std::lock_guard<std::mutex> g(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    VC_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    VC_REQUIRE(p != nullptr, "no device address for the decode scratch array");
    addr[dev] = p;
  }
  *out = addr[dev];
  return VC_OK;
}

}  // namespace vc

extern "C" vc_status vc_decode_attn_compressed(const vc_ckv* c, const void* q, int32_t Hq, float sm_scale,
                                               const int32_t* main_lens, const int32_t* tail_lens, void* out,
                                               float* lse, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  vc_status st = validate_decode_call(c, q, Hq, sm_scale, out);
  if (st != VC_OK) return st;
  const size_t need = vc_decode_workspace_bytes(c, Hq);
  if (!ws || ws_bytes < need) {
    set_error("decode workspace needs %zu bytes (got %zu)", need, ws_bytes);
    return VC_ERR_WORKSPACE;
  }
  const int H = Hq / c->Hkv;
  return decode_launch(c, q, H, sm_scale, main_lens, tail_lens, out, lse, plan_decode(c, H), ws, as_stream(stream));
}

extern "C" vc_status vc_decode_attn_compressed_noalloc(const vc_ckv* c, const void* q, int32_t Hq, float sm_scale,
                                                       const int32_t* main_lens, const int32_t* tail_lens, void* out,
                                                       float* lse, void* stream) {
  clear_error();
  vc_status st = validate_decode_call(c, q, Hq, sm_scale, out);
  if (st != VC_OK) return st;
  const int H = Hq / c->Hkv;
  const DecodePlan p = plan_decode(c, H);
  const size_t need = decode_partials_bytes(c, H, p.S);
  if (need > VC_DECODE_NOALLOC_SCRATCH_BYTES) {
    set_error("decode partials need %zu bytes, beyond the %zu of the library's scratch array", need,
              static_cast<size_t>(VC_DECODE_NOALLOC_SCRATCH_BYTES));
    return VC_ERR_WORKSPACE;
  }
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != VC_OK) return st;
  return decode_launch(c, q, H, sm_scale, main_lens, tail_lens, out, lse, p, ws, as_stream(stream));
}
