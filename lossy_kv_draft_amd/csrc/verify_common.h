// Pieces shared by the verification kernels and the kept-row decode: arguments, operand
// types, the tile ring's layout and its copy and read primitives.
#pragma once

#include "common.h"
#include "decode_common.h"

namespace vc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kVerThreads = 256;
constexpr int kVerTile = 64;

struct VerifyArgs {
  const void* q;
  const void* kc;
  const void* vc;
  int Hq, Hkv, H, d, k;
  int64_t cache_rows, ctx_len;
  const int32_t* ctx_lens;
  int ctx_off;    // added to ctx_lens[b] (decode over kept rows: lengths minus one)
  int64_t C;      // split size in positions
  int splits;
  int rows_per_block;
  float qscale;   // sm_scale * log2(e)
  float* part_o;  // [B*Hkv][splits][M][d]
  float* part_ml; // [B*Hkv][splits][M][2]
};

// Context length of sequence b: ctx_lens[b] clamped to [0, ctx_len - ctx_off], plus
// ctx_off (decode over kept rows passes row counts and ctx_off = -1); else ctx_len.
__device__ __forceinline__ int64_t ver_ctx_len(const VerifyArgs& a, int b) {
  if (!a.ctx_lens) return a.ctx_len;
  const int64_t x = a.ctx_lens[b];
  return min(max(x, static_cast<int64_t>(0)), a.ctx_len - a.ctx_off) + a.ctx_off;
}

union Pack16 {
  uint4 u;
  bf16x8_t v;
  bf16_t h[8];
};

// ---------------------------------------------------------------- bf16, d = 128
// Tiles of kVtTile positions of K and V are copied global -> LDS by all W waves of
// the workgroup (16 bytes per lane per instruction, buffer loads through descriptors
// that end at the last readable row, so rows past it arrive as zeros and every wave's
// offsets are loop invariant) into a ring of S tiles: while tile j is computed, the
// copies of the next S - 1 tiles are in flight.  One barrier per tile: after it,
// tile j has landed for every wave and every wave is done with tile j - 1, whose
// stage then receives tile j + S - 1.  16-byte chunks of a row are XOR-swizzled by
// the row so that the matrix-core operand reads spread over the banks.  K feeds
// S^T = K Q^T as the A operand (16-byte reads).  V stays position-major: the A
// operand of O^T += V^T P^T (channels x positions) is read with the transposing LDS
// load ds_read_b64_tr_b16, which within each 16-lane group returns to lane j the
// element j & 3 of the four values addressed by lane 4e + (j >> 2) as element e; so
// lane (4e + i) addresses position e and channels 4i .. 4i + 3.
// Softmax per row: masking only on tiles that reach past a row's limit; the running
// maximum moves, and the row's accumulators are rescaled, only when a tile's maximum
// exceeds it by more than 8 (base 2), so probabilities stay below 2^8 and the rescale
// is rare (a decision of the row alone, so batch invariance holds); exp2 of an fma;
// bf16 P; the row sums come from one more product with an all-ones A operand.
constexpr int kVtTile = 64;                       // positions per tile
constexpr int kVtRow = 256;                       // bytes per position row
constexpr int kVtPrefetch = 4;                    // K or V fragments read ahead of their product
constexpr int kVtTileBytes = kVtTile * kVtRow;    // one K or V tile
static_assert(kVtTile % 32 == 0, "tile shape");
typedef unsigned char VtStage[2 * kVtTileBytes];  // K tile, then V tile
typedef short s4_t __attribute__((ext_vector_type(4)));
typedef float f2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int vt_chunk(int r, int c) { return c ^ (r & 15); }

// Buffer descriptors of the K/V tiles (common.h)
typedef buf_rsrc_t vt_rsrc_t;
__device__ __forceinline__ vt_rsrc_t vt_rsrc(const void* base, uint32_t bytes) { return buf_rsrc(base, bytes); }
// Buffer -> LDS copy of 16 bytes per active lane at (lds + 16 * lane), from byte
// offset voff of the descriptor's range (inline assembly for the reason given at
// lds_copy16).
__device__ __forceinline__ void lds_copy16_buf(vt_rsrc_t r, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(r), "s"(lds) : "memory", "m0");
}

__device__ __forceinline__ uint2 lds_read_tr16(const unsigned char* p) {
  typedef __attribute__((address_space(3))) s4_t lds_s4;
  const s4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s4*)(__attribute__((address_space(3))) unsigned char*)(p));
  return __builtin_bit_cast(uint2, v);
}

// Maximum over the four 16-lane groups of a wave (lanes l, l ^ 16, l ^ 32, l ^ 48)
// with the lane-swap instructions: given the same register twice, the 16-lane swap
// returns the pair {x[l], x[l ^ 16]} and the 32-lane swap {x[l], x[l ^ 32]} (one in
// each result, in an order that does not matter for the maximum).
__device__ __forceinline__ float group4_max(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const unsigned w = __float_as_uint(x);
  const auto r32 = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

// Wait until at most `ahead` tiles of this wave's copies (I instructions per tile)
// are still in flight.
template <int I, int A>
__device__ __forceinline__ void vt_wait(int ahead) {
  if constexpr (A == 0) {
    wait_vmcnt<0>();
  } else {
    if (ahead >= A) wait_vmcnt<I * A>();
    else vt_wait<I, A - 1>(ahead);
  }
}

}  // namespace vc
