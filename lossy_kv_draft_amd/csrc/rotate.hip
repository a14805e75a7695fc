// Walsh-Hadamard rotation of rows: the channel rotation applied to keys, values and
// queries before a rotation-based quantizer compresses them.
//
// Summary page "VeriCache: Turning Lossy KV Cache into Lossless LLM Inference", "What
// the paper found": rotation-based low-bit quantizers (RotateKV, TurboQuant) sit behind
// the uniform compressor interface.  The rotation here is the fixed orthonormal one,
// x -> x H / sqrt(d) with H the Sylvester Hadamard matrix; it is symmetric and
// orthogonal, hence its own inverse, and keeps every dot product.
//
// Each lane holds E = 16 / sizeof(T) contiguous channels (one 16-byte load and
// store), so a row spans L = d / E lanes and a wave holds 64 / L rows side by side;
// every lane keeps U such loads in flight.  The log2(d) butterfly stages
// (x_i, x_j) -> (x_i + x_j, x_i - x_j) over channel-index bit s run inside a lane for
// s < E and across the row's lanes (lane ^ s / E) otherwise; float32 throughout, one
// rounding to the storage type at the end.  A row is read whole before anything of it
// is written, so out may be x.

#include <algorithm>
#include <cmath>
#include <type_traits>

#include "common.h"

namespace vc {

template <typename T>
struct rot_tag {
  using type = T;
};

template <typename T>
__device__ __forceinline__ void unpack16(const uint4& w, float* v) {
  if constexpr (sizeof(T) == 4) {
    v[0] = __uint_as_float(w.x), v[1] = __uint_as_float(w.y), v[2] = __uint_as_float(w.z), v[3] = __uint_as_float(w.w);
  } else {
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) v[2 * i] = __uint_as_float(u[i] << 16), v[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
  }
}

template <typename T>
__device__ __forceinline__ uint4 pack16(const float* v, float scale) {
  if constexpr (sizeof(T) == 4) {
    return uint4{__float_as_uint(v[0] * scale), __float_as_uint(v[1] * scale), __float_as_uint(v[2] * scale),
                 __float_as_uint(v[3] * scale)};
  } else {
    uint32_t u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      u[i] = static_cast<uint32_t>(f32_to_bf16(v[2 * i] * scale)) |
             (static_cast<uint32_t>(f32_to_bf16(v[2 * i + 1] * scale)) << 16);
    return uint4{u[0], u[1], u[2], u[3]};
  }
}

template <typename T, int D>
struct RotShape {
  static constexpr int E = 16 / sizeof(T);  // channels per lane
  static constexpr int L = D / E;           // lanes per row
  static constexpr int RPW = 64 / L;        // rows per wave and load
  static constexpr int U = 4;               // loads in flight per lane
  static constexpr int ROWS_PER_BLOCK = 4 * RPW * U;
};

template <typename T, int D>
__global__ void __launch_bounds__(256) hadamard_rows_kernel(const T* x, int64_t rows, T* out, float scale) {
  using S = RotShape<T, D>;
  constexpr int E = S::E, L = S::L, RPW = S::RPW, U = S::U;
  const int lane = threadIdx.x & 63;
  const int sub = lane % L;  // position inside the row
  const int64_t first = (static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6)) * (RPW * U) + lane / L;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * S::ROWS_PER_BLOCK;
  for (int64_t r0 = first; r0 - lane / L < rows; r0 += stride) {
    uint4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t r = r0 + u * RPW;
      w[u] = r < rows ? *reinterpret_cast<const uint4*>(x + r * D + sub * E) : uint4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float v[E];
      unpack16<T>(w[u], v);
#pragma unroll
      for (int s = 1; s < E; s <<= 1)
#pragma unroll
        for (int e = 0; e < E; ++e)
          if (!(e & s)) {
            const float a = v[e], b = v[e + s];
            v[e] = a + b;
            v[e + s] = a - b;
          }
#pragma unroll
      for (int ls = 1; ls < L; ls <<= 1) {
        const bool upper = sub & ls;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float o = __shfl_xor(v[e], ls);
          v[e] = upper ? o - v[e] : v[e] + o;
        }
      }
      w[u] = pack16<T>(v, scale);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t r = r0 + u * RPW;
      if (r < rows) *reinterpret_cast<uint4*>(out + r * D + sub * E) = w[u];
    }
  }
}

}  // namespace vc

using namespace vc;

extern "C" vc_status vc_hadamard_rows(const void* x, int32_t dtype, int64_t rows, int32_t d, void* out, void* stream) {
  clear_error();
  VC_REQUIRE(valid_dtype(dtype), "bad dtype %d", dtype);
  VC_REQUIRE(rows >= 0, "rows must be >= 0");
  VC_UNSUPPORTED(d == 64 || d == 128 || d == 256, "the rotation supports d = 64, 128 or 256 (got %d)", d);
  VC_REQUIRE(rows == 0 || (x && out), "x / out is NULL");
  VC_REQUIRE(rows == 0 || ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(out)) & 15) == 0,
             "x and out must be 16-byte aligned");
  if (rows == 0) return VC_OK;
  const float scale = static_cast<float>(1.0 / std::sqrt(static_cast<double>(d)));
  hipStream_t s = as_stream(stream);
  auto go = [&](auto tag, auto d_tag) {
    using T = typename decltype(tag)::type;
    constexpr int D = decltype(d_tag)::value;
    // at most 8 workgroups of 4 waves per compute unit; the rest loop
    const int64_t blocks = std::min<int64_t>(cdiv(rows, RotShape<T, D>::ROWS_PER_BLOCK), 2048);
    hipLaunchKernelGGL((hadamard_rows_kernel<T, D>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                       static_cast<const T*>(x), rows, static_cast<T*>(out), scale);
  };
  auto by_e = [&](auto tag) {
    if (d == 64) go(tag, std::integral_constant<int, 64>{});
    else if (d == 128) go(tag, std::integral_constant<int, 128>{});
    else go(tag, std::integral_constant<int, 256>{});
  };
  if (dtype == VC_BF16) by_e(rot_tag<bf16_t>{});
  else by_e(rot_tag<float>{});
  VC_LAUNCHED("hadamard_rows_kernel");
  return VC_OK;
}
