// Internal helpers shared by the library's HIP sources (not part of the ABI): the
// host-side helpers plus the device types and primitives of the kernels.
#pragma once

#include "host_common.h"

namespace vc {

// ---------------------------------------------------------------- device types
typedef uint16_t bf16_t;  // raw bfloat16 storage

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest, ties to even (inputs are finite in this library).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void store(bf16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};

__device__ __forceinline__ float warp_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float warp_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Global -> LDS copy of 16 bytes per active lane, written at (lds + 16 * lane).  It
// is issued from inline assembly so that the compiler does not treat every later
// LDS read as depending on every copy in flight (it would wait for all of them
// before each read); kernels that use it place the vmcnt waits themselves.  Loads
// the compiler issues are still waited for correctly: copies it does not know of
// can only make its own waits stricter.
__device__ __forceinline__ void lds_copy16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds) : "memory", "m0");
}
// Buffer descriptor over `bytes` bytes from `base` (raw, stride 0): 16-byte loads at
// offsets at or past `bytes` return zeros.  Every field is made wave-uniform.
typedef int32_t buf_rsrc_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ buf_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  buf_rsrc_t r;
  r.x = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(p));
  r.y = __builtin_amdgcn_readfirstlane(static_cast<int32_t>((p >> 32) & 0xFFFFu));
  r.z = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(bytes));
  r.w = 0x00020000;
  return r;
}
// Buffer -> LDS copy of 16 bytes per active lane at (lds + 16 * lane), from byte
// offset soff + voff of the descriptor's range: the per-lane part voff stays in a
// register, the wave-uniform part soff is a scalar, so that moving the copy along
// the buffer costs no vector instruction (inline assembly for the reason given at
// lds_copy16).
__device__ __forceinline__ void lds_copy16_buf_so(buf_rsrc_t r, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(r), "s"(soff), "s"(lds)
               : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace vc
