// Walsh-Hadamard rotation of rows: the channel rotation applied to keys, values and
// queries before a rotation-based quantizer compresses them.
//
// Summary page "VeriCache: Turning Lossy KV Cache into Lossless LLM Inference", "What
// the paper found": rotation-based low-bit quantizers (RotateKV, TurboQuant) sit behind
// the uniform compressor interface.  The rotation here is the fixed orthonormal one,
// x -> x H / sqrt(d) with H the Sylvester Hadamard matrix; it is symmetric and
// orthogonal, hence its own inverse, and keeps every dot product.
//
// One wave per row, lane l holding channels [E l, E l + E) (E = d / 64): the log2(d)
// butterfly stages (x_i, x_j) -> (x_i + x_j, x_i - x_j) over index bit s run inside a
// lane for s < E and across lanes (lane ^ s / E) otherwise; float32 throughout, one
// rounding to the storage type at the end.  The row is read whole before anything is
// written, so out may be x.

#include <algorithm>
#include <cmath>
#include <type_traits>

#include "common.h"

namespace vc {

template <typename T>
struct rot_tag {
  using type = T;
};

template <typename T, int E>
__global__ void __launch_bounds__(256) hadamard_rows_kernel(const T* x, int64_t rows, T* out, float scale) {
  constexpr int D = 64 * E;
  const int lane = threadIdx.x & 63;
  const int64_t waves = static_cast<int64_t>(gridDim.x) * 4;
  for (int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6); r < rows; r += waves) {
    const T* src = x + r * D + E * lane;
    float v[E];
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = Elem<T>::load(src, e);
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
    for (int ls = 1; ls < 64; ls <<= 1) {
      const bool upper = lane & ls;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float o = __shfl_xor(v[e], ls);
        v[e] = upper ? o - v[e] : v[e] + o;
      }
    }
    T* dst = out + r * D + E * lane;
#pragma unroll
    for (int e = 0; e < E; ++e) Elem<T>::store(dst, e, v[e] * scale);
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
  if (rows == 0) return VC_OK;
  const float scale = static_cast<float>(1.0 / std::sqrt(static_cast<double>(d)));
  const int64_t blocks = std::min<int64_t>(cdiv(rows, 4), 4096);
  hipStream_t s = as_stream(stream);
  auto go = [&](auto tag, auto e_tag) {
    using T = typename decltype(tag)::type;
    constexpr int E = decltype(e_tag)::value;
    hipLaunchKernelGGL((hadamard_rows_kernel<T, E>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                       static_cast<const T*>(x), rows, static_cast<T*>(out), scale);
  };
  auto by_e = [&](auto tag) {
    if (d == 64) go(tag, std::integral_constant<int, 1>{});
    else if (d == 128) go(tag, std::integral_constant<int, 2>{});
    else go(tag, std::integral_constant<int, 4>{});
  };
  if (dtype == VC_BF16) by_e(rot_tag<bf16_t>{});
  else by_e(rot_tag<float>{});
  VC_LAUNCHED("hadamard_rows_kernel");
  return VC_OK;
}
