// Draft-side decode attention over KIVI-quantized packed K/V on matrix cores.
//
// Summary page "VeriCache: Turning Lossy KV Cache into Lossless LLM Inference",
// "What the paper found": drafting on the compressed cache is HBM-bandwidth-bound.
// A scalar implementation of grouped-query decode is not: every code costs an
// extract, a convert and an FMA per q-head, which on CDNA4 exceeds the vector ALU
// budget long before HBM is saturated.  This kernel moves both contractions onto
// v_mfma_f32_16x16x32_f16 and keeps the vector ALU work to turning codes into f16:
//
// * one wave processes 32-token blocks of one (sequence, kv-head); the q-heads that
//   read the kv-head are the 16 columns of the B operand (zero beyond Hq/Hkv), so
//   every packed row is read from HBM once for all of them;
// * a code c becomes an f16 value of a fixed binade, off + w c, by placing it under
//   the exponent bits of off: 4-bit K codes as 1024 + c or 1024 + 16 c (one AND-OR
//   per pair of codes), other codes as 64 + c (one v_perm_b32 per pair);
// * K needs no dequantization: with per-channel scale s and zero z, q . k_hat =
//   sum_c (q s / w)_c (off + w c) + [sum_c q_c z_c - off sum_c (q s / w)_c]; the
//   query operand becomes q * s / w (packed f16 multiplies) and the bracket, a bias
//   per q-head and K group, is formed on the matrix cores when the group changes;
//   minus the running maximum it seeds the score accumulator, so the scores come
//   out relative to the maximum;
// * V (per-token scale and zero), 64- and 128-channel groups with 2- or 4-bit codes:
//   lane n holds channels 64 hf + 4 n .. + 3 of each half hf, so a channel tile lies
//   in one V group and the scale moves to the probabilities: A = the codes as the
//   exact bf16 values 128 + c (one AND-OR per pair), B = p * s of the tile's group
//   (bf16); the offset (-128 sum of B, exact) and the zero-point term sum_t p_t z_t
//   are products of their own into one correction accumulator.  The block's scales
//   and zeros are converted once by the wave (one token and group per lane) into LDS;
// * V otherwise: each pair becomes c * s with one packed fused multiply-add of
//   (64 + c) by s with addend -64 s (exact, rounded once); the zero-point term is one
//   extra product per block (its A operand the tokens' zeros);
// * S^T = K_hat Q^T for two 16-token tiles, online softmax per q-head in base 2 with
//   a lazy rescale (only when the block maximum exceeds the running one by more than
//   8, i.e. probabilities stay below 2^8), probabilities rounded to f16, then
//   O^T += V_hat^T P^T; the denominators are the sums of the same rounded
//   probabilities, formed on the matrix cores.  The probabilities stay in the lanes that produced them: the
//   S^T layout of two 16-token tiles is the B-operand layout of the 32-token P.V
//   product once both operands enumerate the block's tokens in the same order;
// * within an operand the order of the contraction index is free as long as both
//   operands agree, so K channels and V tokens are enumerated in whatever order the
//   byte permutes produce them (korder / vorder below);
// * each wave copies its blocks global -> LDS itself, kDepth blocks ahead into a ring
//   of its own (buffer loads at scalar offsets); a slot is refilled as soon as its
//   block is in registers, so two blocks are in flight while one is computed.  The
//   V and K parameters of two blocks are copied as one entry of a parameter ring;
// * K's code row is read from LDS as 32-channel chunks (one 64/96/128-bit read per
//   lane), V's as the lane's fields of 8 tokens; they are decoded only when used;
// * a merge by the last workgroup to finish would need a device-scope release by
//   every workgroup (an L2 write-back each, on a part with one L2 per XCD): measured,
//   that costs more than the separate merge kernel;
// * a sequence's 32-token blocks are dealt out evenly over the waves of its
//   workgroups (in order: wave loads differ by at most one block); the 4 waves of a
//   workgroup are merged in LDS and the workgroup writes one partial per split;
//   decode_merge_kernel, launched next, adds the full-precision tail rows and merges
//   the splits in split order;
// * the number of splits is chosen so that all workgroups are resident at once
//   (occupancy times compute units, queried from the runtime).
//
// Precision: q * s, c * s, the zero-points and p are f16 (11-bit significands), p * s
// bf16 (8-bit) on the scaled-probability path, with float32 accumulation; against
// float64 attention on the outlier workloads the error is 1e-4 to 2e-3 at unit scale,
// below the bf16 output resolution of those outputs.  Values and 64 * s must lie
// within the f16 range (65504).

#include <type_traits>

#include "decode_common.h"

namespace vc {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr uint32_t kMagic = 0x64646464u;  // exponent byte of 1024.0 in f16, in every byte

__device__ __forceinline__ h2_t as_h2(uint32_t u) { return __builtin_bit_cast(h2_t, u); }
__device__ __forceinline__ uint32_t as_u32(h2_t h) { return __builtin_bit_cast(uint32_t, h); }

// pair of f16 values (64 + c0, 64 + c1) -> (c0 * s0, c1 * s1): one fused multiply-add
// with the addend -64 s (exact: a power-of-two multiple), rounded once
__device__ __forceinline__ uint32_t scale_pair(uint32_t magic, uint32_t s2, uint32_t ns2) {
  return as_u32(__builtin_elementwise_fma(as_h2(magic), as_h2(s2), as_h2(ns2)));
}

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  h2_t h = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
  return as_u32(h);
}

// bytes [x.b_i, 0x64, x.b_j, 0x64]: the f16 pair (1024 + x.b_i, 1024 + x.b_j)
__device__ __forceinline__ uint32_t magic_bytes(uint32_t x, uint32_t sel) { return __builtin_amdgcn_perm(kMagic, x, sel); }
constexpr uint32_t kSel01 = 0x04010400u;  // bytes 0, 1
constexpr uint32_t kSel23 = 0x04030402u;  // bytes 2, 3
constexpr uint32_t kSel02 = 0x04020400u;  // bytes 0, 2
constexpr uint32_t kSel13 = 0x04030401u;  // bytes 1, 3

// Channel (within a lane's 8-channel k-step chunk) of contraction index j.
template <int KB>
__device__ __forceinline__ constexpr int korder(int j) {
  return (j & 1) ? (j >> 1) + 4 : (j >> 1);  // 0,4,1,5,2,6,3,7
}

// K codes enter the score product as f16 values of one binade, so that the scale
// can be folded into the query and the zero-point and the offset into a per-group
// bias (see use_kp) and K needs no dequantization arithmetic:
// * 4-bit codes: 1024 + c for the even channels of a word (code in bits 0..3 of a
//   16-bit half under the exponent bits of 1024) and 1024 + 16 c for the odd ones
//   (code in bits 4..7), each pair made by one AND-OR of the word or of the word
//   shifted by a byte; the factor 16 of the odd channels is taken out of their
//   query operand (q s / 16).  The cancellation of the offset in the float32
//   accumulation, about 2^-14 of sum |q s|, stays well below the f16 rounding of
//   q s itself (2^-11 of sum |q s c|);
// * 2- and 3-bit codes: 64 + c (code in bits 4.. of a byte under the exponent byte
//   0x54) by one byte permute per pair.
constexpr uint32_t kMagicK = 0x54545454u;
__device__ __forceinline__ uint32_t kmagic(uint32_t x, uint32_t sel) { return __builtin_amdgcn_perm(kMagicK, x, sel); }
constexpr uint32_t kMagic1024 = 0x64006400u;  // (1024, 1024) in f16
constexpr uint32_t kMagicV = 0x43004300u;     // (128, 128) in bf16
// the offset of the K code values (negated, an f16 pair) and the factor of channel c
template <int KB>
__device__ __forceinline__ constexpr uint32_t kneg_offset() { return KB == 4 ? 0xE400E400u : 0xD400D400u; }
template <int KB>
__device__ __forceinline__ constexpr float kweight(int c) { return (KB == 4 && (c & 1)) ? 0.0625f : 1.f; }

// The constants of the 4-bit K pairs, held in registers the compiler cannot see
// through: with two literal operands it would split each AND-OR into two
// instructions (a VOP3 instruction takes no literal here); with the masks in scalar
// registers and the exponent pattern in a vector register it is one v_and_or_b32.
struct KConst {
  uint32_t lo, hi, lo2, magic, vmagic;
  __device__ __forceinline__ KConst()
      : lo(0x000F000Fu), hi(0x00F000F0u), lo2(0x00030003u), magic(kMagic1024), vmagic(kMagicV) {
    asm("" : "+s"(lo));
    asm("" : "+s"(hi));
    asm("" : "+s"(lo2));
    asm("" : "+v"(magic));
    asm("" : "+v"(vmagic));
  }
};

// K: the four f16 pairs of code values of k-step s from a lane's 32-channel chunk
// (KB words); pair jj holds channels korder(2jj), korder(2jj+1).
template <int KB>
__device__ __forceinline__ void kpairs(const uint32_t* w, int s, uint32_t (&out)[4], const KConst& kc) {
  if constexpr (KB == 4) {
    const uint32_t x = w[s], y = x >> 8;
    out[0] = (x & kc.lo) | kc.magic;  // channels 0, 4: 1024 + c
    out[1] = (x & kc.hi) | kc.magic;  // channels 1, 5: 1024 + 16 c
    out[2] = (y & kc.lo) | kc.magic;  // channels 2, 6
    out[3] = (y & kc.hi) | kc.magic;  // channels 3, 7
  } else if constexpr (KB == 2) {
    const uint32_t x = w[s >> 1];
    const uint32_t sel = (s & 1) ? kSel23 : kSel01;
    // bytes: codes r, 4+r, 8+r, 12+r of the word, each moved to bits 4..5
    out[0] = kmagic((x << 4) & 0x30303030u, sel);
    out[1] = kmagic((x << 2) & 0x30303030u, sel);
    out[2] = kmagic(x & 0x30303030u, sel);
    out[3] = kmagic((x >> 2) & 0x30303030u, sel);
  } else {  // 3 bits: 24-bit fields at bit 24 s of a 96-bit chunk
    uint32_t f;
    if (s == 0) f = w[0] & 0xFFFFFFu;
    else if (s == 1) f = __builtin_amdgcn_alignbit(w[1], w[0], 24) & 0xFFFFFFu;
    else if (s == 2) f = __builtin_amdgcn_alignbit(w[2], w[1], 16) & 0xFFFFFFu;
    else f = w[2] >> 8;
    const uint32_t u = (f & 0xFFFu) | ((f >> 12) << 16);  // codes 0..3 low half, 4..7 high half
    out[0] = ((u << 4) & 0x00700070u) | 0x54005400u;       // code j of each half to bits 4..6
    out[1] = ((u << 1) & 0x00700070u) | 0x54005400u;
    out[2] = ((u >> 2) & 0x00700070u) | 0x54005400u;
    out[3] = ((u >> 5) & 0x00700070u) | 0x54005400u;
  }
}

// Channel of V tile t for a field of VB-bit codes.
template <int VB>
__device__ __forceinline__ constexpr int vorder(int t) {
  if constexpr (VB == 4) return (t & 3) * 2 + (t >> 2);  // 0,2,4,6,1,3,5,7
  else if constexpr (VB == 2) return (t & 1) ? (t >> 1) + 4 : (t >> 1);
  else return t;
}

// V: for two tokens' 8-code fields fa, fb, the f16 pair (64 + a_c, 64 + b_c) of each
// of the 8 channels, tile t holding channel vorder(t) (codes moved to bits 4.. of a
// byte under the exponent byte 0x54, as for K).
template <int VB>
__device__ __forceinline__ void vpairs(uint32_t fa, uint32_t fb, uint32_t (&out)[8]) {
  if constexpr (VB == 4) {
    const uint32_t w0 = __builtin_amdgcn_perm(fb, fa, 0x05010400u);  // bytes a.0 b.0 a.1 b.1
    const uint32_t w1 = __builtin_amdgcn_perm(fb, fa, 0x07030602u);  // bytes a.2 b.2 a.3 b.3
    const uint32_t x0 = (w0 << 4) & 0xF0F0F0F0u;  // a0 b0 a2 b2
    const uint32_t x1 = (w1 << 4) & 0xF0F0F0F0u;  // a4 b4 a6 b6
    const uint32_t y0 = w0 & 0xF0F0F0F0u;         // a1 b1 a3 b3
    const uint32_t y1 = w1 & 0xF0F0F0F0u;         // a5 b5 a7 b7
    out[0] = kmagic(x0, kSel01);
    out[1] = kmagic(x0, kSel23);
    out[2] = kmagic(x1, kSel01);
    out[3] = kmagic(x1, kSel23);
    out[4] = kmagic(y0, kSel01);
    out[5] = kmagic(y0, kSel23);
    out[6] = kmagic(y1, kSel01);
    out[7] = kmagic(y1, kSel23);
  } else if constexpr (VB == 2) {
    const uint32_t comb = (fa & 0xFFFFu) | (fb << 16);
    // bytes: a_r, a_{4+r}, b_r, b_{4+r}, each moved to bits 4..5
    const uint32_t m[4] = {(comb << 4) & 0x30303030u, (comb << 2) & 0x30303030u, comb & 0x30303030u,
                           (comb >> 2) & 0x30303030u};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      out[2 * r] = kmagic(m[r], kSel02);
      out[2 * r + 1] = kmagic(m[r], kSel13);
    }
  } else {
    const uint32_t lo = (fa & 0xFFFu) | ((fb & 0xFFFu) << 16);
    const uint32_t hi = ((fa >> 12) & 0xFFFu) | (((fb >> 12) & 0xFFFu) << 16);
    out[0] = ((lo << 4) & 0x00700070u) | 0x54005400u;
    out[1] = ((lo << 1) & 0x00700070u) | 0x54005400u;
    out[2] = ((lo >> 2) & 0x00700070u) | 0x54005400u;
    out[3] = ((lo >> 5) & 0x00700070u) | 0x54005400u;
    out[4] = ((hi << 4) & 0x00700070u) | 0x54005400u;
    out[5] = ((hi << 1) & 0x00700070u) | 0x54005400u;
    out[6] = ((hi >> 2) & 0x00700070u) | 0x54005400u;
    out[7] = ((hi >> 5) & 0x00700070u) | 0x54005400u;
  }
}

// V with the scale on the probabilities (64- and 128-channel V groups, 2- and 4-bit
// codes): lane n holds channels 64 hf + 4 n + i of half hf (i = 0..3); comb holds the
// lane's 4 codes of token a in its low and of token b in its high 16 bits (one byte
// permute of the two tokens' words), and pair i becomes the bf16 values
// (128 + a_i, 128 + b_i): code i shifted to bits 0.. of each half under the exponent
// bits of 128, one AND-OR (after a shift for i > 0).
template <int VB>
__device__ __forceinline__ void vpairs_bf16(uint32_t comb, uint32_t (&out)[4], uint32_t mask, uint32_t magic) {
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = ((comb >> (VB * i)) & mask) | magic;
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, bf16x2_t{static_cast<__bf16>(a), static_cast<__bf16>(b)});
}

// token of slot j (0..7) of lane group kb in a 32-token block
__device__ __forceinline__ int slot_token(int kb, int j) { return j < 4 ? 4 * kb + j : 16 + 4 * kb + (j - 4); }

template <typename P>
__device__ __forceinline__ float param_f32(const P* p, int i) { return Elem<P>::load(p, i); }

// The ring is filled with lds_copy16_buf_so (common.h): 16 bytes per lane, global ->
// LDS, with the vmcnt waits placed by the kernel itself.

// Slot layout of one 32-token block and the ring depth for one kernel instance.
template <int KB, int VB, int NGV, typename P>
struct DecRing {
  static constexpr int kD = 128;
  static constexpr int kG = kD / NGV;
  static constexpr int kNKG = kG >= 32 ? 1 : 2;                        // K groups per block
  static constexpr int kKC = 32 * kD * KB / 8;                         // K code bytes
  static constexpr int kVC = 32 * kD * VB / 8;                         // V code bytes
  static constexpr int kVP = 32 * NGV * static_cast<int>(sizeof(P));  // V scale (and zero) bytes
  static constexpr int kKPG = kD * static_cast<int>(sizeof(P));        // one K parameter row
  // The parameters go to a ring of their own, one entry per kPB = 2 blocks: the V
  // scales of its 64 rows, their zeros, and with whole K groups per block the
  // [scale row, zero row] of the (at most two) K groups those rows touch.  An entry
  // is copied with its first block, by two instructions of up to 1 KB (the V
  // parameters of a block are 128-256 bytes, too small a read to use the memory
  // well); with two K groups per block the K parameters sit in the block's slot.
  static constexpr bool kGroupKP = kNKG == 1;
  static constexpr int kPB = 2;
  static constexpr int kOffK = 0;
  static constexpr int kOffV = kOffK + kKC;
  static constexpr int kOffKP = kOffV + kVC;
  static constexpr int kSlot = kOffKP + (kGroupKP ? 0 : kNKG * 2 * kKPG);
  static constexpr int kVPE = kPB * kVP;  // V scale (and zero) bytes of an entry
  static constexpr int kOffEK = 2 * kVPE;
  static constexpr int kEntry = kOffEK + (kGroupKP ? 2 * 2 * kKPG : 0);
  static constexpr int pieces(int bytes) { return (bytes + 1023) / 1024; }
  // copy instructions per block and per entry
  static constexpr int kInstr = pieces(kKC) + pieces(kVC) + (kGroupKP ? 0 : kNKG * 2 * pieces(kKPG));
  static constexpr int kEInstr = pieces(2 * kVPE) + (kGroupKP ? pieces(4 * kKPG) : 0);
  // entries in the ring for a block ring of depth d: an entry is refilled when the
  // block kPB * ring entries later is issued, i.e. while the block d before that one
  // is processed, so every block of the entry must be at or before it
  static constexpr int entries(int d) { return (kPB - 1 + d + kPB - 1) / kPB; }
  // kWgPerCu workgroups of 4 waves per compute unit share its 160 KB of LDS (~3.5 KB
  // of each outside the rings): 4 * (depth * slot + entries * entry) <= 160 KB /
  // kWgPerCu - 3.5 KB.  Three (three waves per SIMD, at most 168 registers a wave: a
  // shallower ring, but more waves to hide the latency of the code conversion) where
  // that measured faster and needs no register spills: bf16 parameters with
  // 64-channel V groups; else two.
  static constexpr int kWgPerCu = (sizeof(P) == 2 && NGV == 2) ? 3 : 2;
  static constexpr int depth_fit() {
    int d = 8;
    while (d > 2 && 4 * (d * kSlot + entries(d) * kEntry) > 163840 / kWgPerCu - 3584) --d;
    return d;
  }
  static constexpr int kDepth = depth_fit();
  static constexpr int kNE = entries(kDepth);
  static_assert(kSlot % 16 == 0 && kVP % 16 == 0 && kKPG % 16 == 0 && kEntry % 16 == 0, "16-byte pieces");
  static_assert((kDepth - 1) * kInstr + ((kDepth + kPB - 2) / kPB) * kEInstr <= 63, "vmcnt range");

  // `bytes` contiguous bytes at byte soff of buffer r into LDS at `lds`, 16 bytes per
  // lane and instruction (voff = 16 * lane)
  static __device__ __forceinline__ void copy_buf(buf_rsrc_t r, uint32_t soff, int bytes, uint32_t lds, uint32_t voff,
                                                  int lane) {
#pragma unroll
    for (int c = 0; c < pieces(bytes); ++c)
      if (1024 * c + 16 * lane < bytes) lds_copy16_buf_so(r, voff, soff + 1024 * c, lds + 1024 * c);
  }
  // `bytes` into LDS at `lds` from the per-lane sources src[c] of pieces c
  static __device__ __forceinline__ void copy_lanes(const unsigned char* const* src, int bytes, uint32_t lds, int lane) {
#pragma unroll
    for (int c = 0; c < pieces(bytes); ++c)
      if (1024 * c + 16 * lane < bytes) lds_copy16(src[c], lds + 1024 * c);
  }
  template <int N>
  static __device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
  }
  // wait for a block while the next kDepth - 1 blocks, ne of which start an entry,
  // may still be in flight (ne wave-uniform)
  template <int K = 0>
  static __device__ __forceinline__ void wait_ahead(int ne) {
    if constexpr (K < (kDepth + kPB - 2) / kPB) {
      if (ne > K) {
        wait_ahead<K + 1>(ne);
        return;
      }
    }
    wait_vm<(kDepth - 1) * kInstr + K * kEInstr>();
  }
  static __device__ __forceinline__ void wait_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
  static __device__ __forceinline__ void lds_reads_done() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
};

template <typename T>
struct type_tag {
  using type = T;
};

template <int KB, int VB, int NGV, typename P>
__global__ void __launch_bounds__(kDecThreads)
__attribute__((amdgpu_waves_per_eu(DecRing<KB, VB, NGV, P>::kWgPerCu)))
decode_mfma_kernel(DecodeArgs a) {
  constexpr int D = 128;
  constexpr int G = D / NGV;                          // K: tokens per group; V: channels per group
  constexpr int KW = D * KB / 32;                     // words per packed K row
  constexpr int VW = D * VB / 32;
  constexpr int VWR = VB == 3 ? 2 : 1;                // raw words per V field
  constexpr int HW = D * static_cast<int>(sizeof(P)) / 4;  // words per K parameter row
  constexpr int KPW = 2 * HW / 64;                    // K-parameter words per lane
  constexpr int NKG = G >= 32 ? 1 : 2;                // K groups per 32-token block
  using Ring = DecRing<KB, VB, NGV, P>;
  // per-wave rings of block slots; after the main loop the same memory holds the
  // waves' outputs for the merge
  constexpr int kRingBytes = 4 * Ring::kDepth * Ring::kSlot > 4 * 16 * D * 4 ? 4 * Ring::kDepth * Ring::kSlot : 4 * 16 * D * 4;
  __shared__ __attribute__((aligned(16))) unsigned char ring[kRingBytes];
  __shared__ __attribute__((aligned(16))) unsigned char pring[4 * Ring::kNE * Ring::kEntry];
  float (*sh_o)[16][D] = reinterpret_cast<float (*)[16][D]>(ring);
  __shared__ float sh_m[4][16], sh_l[4][16];
  __shared__ __attribute__((aligned(16))) uint32_t sh_kq[4][2][4][16];  // per wave: K scale / zero f16 pairs
  // V scales on the probabilities: per wave the block's V scales (float) and zeros
  // (f16) by group, lane group and slot, converted once per block by the wave
  constexpr bool kBS = NGV <= 2 && VB != 3;
  __shared__ __attribute__((aligned(16))) float sh_vs[kBS ? 4 : 1][2][4][8];
  __shared__ __attribute__((aligned(16))) _Float16 sh_vz[kBS ? 4 : 1][2][4][8];

  const int split = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.Hkv, hk = bh % a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar loop control
  const int n = lane & 15, kb = lane >> 4;
  const int H = a.H;
  const int main_len = static_cast<int>(dec_main_len(a, b));
  // the sequence's 32-row blocks dealt out evenly over the 4 * splits waves of its
  // workgroups, in order (so the wave loads differ by at most one block)
  const int nb_all = (main_len + 31) / 32, nwaves = 4 * a.splits, wv = 4 * split + wave;
  const int t_begin = 32 * static_cast<int>(static_cast<int64_t>(wv) * nb_all / nwaves);
  const int t_end = min(main_len, 32 * static_cast<int>(static_cast<int64_t>(wv + 1) * nb_all / nwaves));

  // queries as the B operand: column n = q-head n of this kv-head (0 beyond H),
  // lane group kb holds channels 32 kb + 8 s + korder(j) for k-step s
  h8_t bq[4];
  {
    const bf16_t* q = static_cast<const bf16_t*>(a.q) +
                      (static_cast<int64_t>(b) * a.Hkv * H + hk * H + (n < H ? n : 0)) * D + 32 * kb;
    const float qs = n < H ? a.qscale : 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 x = *reinterpret_cast<const uint4*>(q + 8 * s);
      const uint32_t w[4] = {x.x, x.y, x.z, x.w};  // channels (0,1) (2,3) (4,5) (6,7)
      float v[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) v[c] = __uint_as_float((c & 1) ? (w[c >> 1] & 0xFFFF0000u) : (w[c >> 1] << 16));
      uint32_t pr[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) pr[jj] = pack_h2(v[korder<KB>(2 * jj)] * qs, v[korder<KB>(2 * jj + 1)] * qs);
      bq[s] = __builtin_bit_cast(h8_t, pr);
    }
  }

  // uniform bases of this (sequence, kv-head); per-lane 32-bit word offsets
  const uint32_t* kcodes = a.k_codes + static_cast<int64_t>(bh) * a.capacity * KW;
  const uint32_t* vcodes = a.v_codes + static_cast<int64_t>(bh) * a.capacity * VW;
  const uint32_t* kscale = reinterpret_cast<const uint32_t*>(static_cast<const P*>(a.k_scale) +
                                                             static_cast<int64_t>(bh) * (a.capacity / G) * D);
  const uint32_t* kzero = reinterpret_cast<const uint32_t*>(static_cast<const P*>(a.k_zero) +
                                                            static_cast<int64_t>(bh) * (a.capacity / G) * D);
  const P* vscale = static_cast<const P*>(a.v_scale) + static_cast<int64_t>(bh) * a.capacity * NGV;
  const P* vzero = static_cast<const P*>(a.v_zero) + static_cast<int64_t>(bh) * a.capacity * NGV;
  const int gv = (8 * n) / G;  // V group of this lane's 8-channel field
  const uint32_t vfw = VB == 4 ? n : (VB == 2 ? (n >> 1) : ((24 * n) >> 5));  // first word of field n
  const uint32_t vfo = VB == 4 ? 0 : (VB == 2 ? 16 * (n & 1) : ((24 * n) & 31));  // its bit offset
  const uint32_t vfw2 = (VB == 3 && vfw + 1 < VW) ? vfw + 1 : vfw;
  const uint32_t k_lane = n * KW + kb * KB;

  f4_t acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f4_t{0.f, 0.f, 0.f, 0.f};
  // V zero-points: sum over tokens of p * z, the same for every channel of a field's
  // group, so one product per block; added to every channel tile at the end
  f4_t accz = f4_t{0.f, 0.f, 0.f, 0.f};
  // softmax denominators: the column sums of the f16 probabilities that enter the
  // P.V product (one more product with an all-ones A operand, so every row of a
  // column holds the column's sum)
  f4_t accl = f4_t{0.f, 0.f, 0.f, 0.f};
  // The running column maximum m is a reference that the scores are taken relative
  // to: the score accumulators are seeded with (bias - m), so the exponent needs no
  // subtraction.  Until the first block sets it, m is 0 and every block rescales
  // (thr = -inf); afterwards a block rescales when a score exceeds m by more than 8.
  float m = 0.f;
  float thr = -INFINITY;
  f4_t seed = f4_t{0.f, 0.f, 0.f, 0.f};  // the current K group's bias minus m
  // the score operands of one K group: the queries times the group's scales (the B
  // operand of the scores) and sum_c q_c z_c - 64 sum_c qt_c per q-head column
  struct KQ {
    h8_t qt[4];
    f4_t kbias;
  };

  // The block's bytes (K codes, V codes, and with two K groups per block their K
  // parameters) are copied global -> LDS by the wave itself (16 bytes per lane per
  // instruction, Ring::kInstr instructions per block) kDepth blocks ahead, into a
  // ring of slots private to the wave; the first block of each parameter entry also
  // copies the entry (Ring::kEInstr instructions) into the wave's parameter ring.  A
  // block is read from its slot into registers only when it is processed.  Rows of a
  // block that starts before the end are inside the allocation (capacity is a
  // multiple of 32); rows past the end are masked (scores -inf, V scale and zero 0).
  unsigned char* const wring = ring + wave * Ring::kDepth * Ring::kSlot;
  unsigned char* const wpr = pring + wave * Ring::kNE * Ring::kEntry;
  const int nblk = t_end > t_begin ? (t_end - t_begin + 31) / 32 : 0;
  const unsigned char* kbytes = reinterpret_cast<const unsigned char*>(kcodes);
  const unsigned char* vbytes = reinterpret_cast<const unsigned char*>(vcodes);
  const unsigned char* ksb = reinterpret_cast<const unsigned char*>(kscale);
  const unsigned char* kzb = reinterpret_cast<const unsigned char*>(kzero);
  const unsigned char* vsb = reinterpret_cast<const unsigned char*>(vscale);
  const unsigned char* vzb = reinterpret_cast<const unsigned char*>(vzero);
  // buffer descriptors over this wave's rows of the code arrays (whole 32-row
  // blocks): the copies move along them by scalar offsets
  const uint32_t wrows = 32u * static_cast<uint32_t>(nblk);
  const int g_first = t_begin / G;
  const int g_last = nblk > 0 ? (t_begin + static_cast<int>(wrows) - 1) / G : g_first;  // inside the allocation
  const uint32_t g_count = nblk > 0 ? static_cast<uint32_t>(g_last - g_first + 1) : 0u;
  const buf_rsrc_t rk = buf_rsrc(kbytes + static_cast<size_t>(t_begin) * KW * 4, wrows * KW * 4);
  const buf_rsrc_t rv = buf_rsrc(vbytes + static_cast<size_t>(t_begin) * VW * 4, wrows * VW * 4);
  const buf_rsrc_t rks = buf_rsrc(ksb + static_cast<size_t>(g_first) * Ring::kKPG, g_count * Ring::kKPG);
  const buf_rsrc_t rkz = buf_rsrc(kzb + static_cast<size_t>(g_first) * Ring::kKPG, g_count * Ring::kKPG);
  const uint32_t voff = 16u * static_cast<uint32_t>(lane);
  // Parameter entry e (blocks kPB e, kPB e + 1): each lane's 16-byte pieces.  V: piece
  // c of the lane is byte off = 1024 c + 16 lane of [scales of the 64 rows][zeros],
  // i.e. row off / (NGV sizeof(P)) of either; K: byte off of [scale row, zero row of
  // the entry's first group][the same of its last group].
  constexpr int kVPieces = Ring::pieces(2 * Ring::kVPE), kKPieces = Ring::kGroupKP ? Ring::pieces(4 * Ring::kKPG) : 1;
  constexpr int kRowBytes = NGV * static_cast<int>(sizeof(P));  // V parameter bytes of one row
  const unsigned char* vp_src[kVPieces];
  int vp_row[kVPieces];  // the piece's row within the entry
#pragma unroll
  for (int c = 0; c < kVPieces; ++c) {
    const int off = 1024 * c + 16 * lane;
    const int w = off < Ring::kVPE ? off : off - Ring::kVPE;
    vp_src[c] = (off < Ring::kVPE ? vsb : vzb) + static_cast<size_t>(t_begin) * kRowBytes + w;
    vp_row[c] = w / kRowBytes;
  }
  const unsigned char* kp_src[kKPieces];
  bool kp_last[kKPieces];  // the piece belongs to the entry's last group
#pragma unroll
  for (int c = 0; c < kKPieces; ++c) {
    const int off = 1024 * c + 16 * lane, r = off / Ring::kKPG;
    kp_src[c] = ((r & 1) ? kzb : ksb) + off % Ring::kKPG;
    kp_last[c] = (r >> 1) != 0;
  }
  auto entry = [&](int i) { return wpr + ((i / Ring::kPB) % Ring::kNE) * Ring::kEntry; };  // block i's entry
  // first group of block i's entry (absolute group index)
  auto entry_g0 = [&](int i) { return (t_begin + 32 * Ring::kPB * (i / Ring::kPB)) / G; };
  auto issue = [&](int i) {  // block i of this wave's range into slot i % kDepth
    const uint32_t r0 = 32u * static_cast<uint32_t>(i);  // its first row within the range
    if (i % Ring::kPB == 0) {  // the entry: V parameters of its rows, K parameters of its groups
      const uint32_t el = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(entry(i))));
      // rows past the range's end copy the range's first row instead (every
      // instruction keeps its lanes, so the count the waits rely on holds); they
      // are never read
      const int rows = min(32 * Ring::kPB, static_cast<int>(wrows - r0));
      const unsigned char* vs[kVPieces];
#pragma unroll
      for (int c = 0; c < kVPieces; ++c)
        vs[c] = vp_row[c] < rows ? vp_src[c] + static_cast<size_t>(r0) * kRowBytes : vp_src[c] - vp_row[c] * kRowBytes;
      Ring::copy_lanes(vs, 2 * Ring::kVPE, el, lane);
      if constexpr (Ring::kGroupKP) {
        const int ga = entry_g0(i), gb = min((t_begin + static_cast<int>(r0) + rows - 1) / G, g_last);
        const unsigned char* ks[kKPieces];
#pragma unroll
        for (int c = 0; c < kKPieces; ++c) ks[c] = kp_src[c] + static_cast<size_t>(kp_last[c] ? gb : ga) * Ring::kKPG;
        Ring::copy_lanes(ks, 4 * Ring::kKPG, el + Ring::kOffEK, lane);
      }
    }
    const uint32_t lds = __builtin_amdgcn_readfirstlane(
        static_cast<uint32_t>(reinterpret_cast<uintptr_t>(wring + (i % Ring::kDepth) * Ring::kSlot)));
    // codes: 32 consecutive rows of each
    Ring::copy_buf(rk, r0 * KW * 4, Ring::kKC, lds + Ring::kOffK, voff, lane);
    Ring::copy_buf(rv, r0 * VW * 4, Ring::kVC, lds + Ring::kOffV, voff, lane);
    if constexpr (!Ring::kGroupKP) {
      // K parameters of the block's two groups: [scale row, zero row] per group
      const uint32_t g0 = static_cast<uint32_t>((t_begin + static_cast<int>(r0)) / G - g_first);
#pragma unroll
      for (int gi = 0; gi < NKG; ++gi) {
        const uint32_t kp = lds + Ring::kOffKP + gi * 2 * Ring::kKPG;
        Ring::copy_buf(rks, (g0 + gi) * Ring::kKPG, Ring::kKPG, kp, voff, lane);
        Ring::copy_buf(rkz, (g0 + gi) * Ring::kKPG, Ring::kKPG, kp + Ring::kKPG, voff, lane);
      }
    }
  };
  // block i's V scales (zeros kVPE bytes further) and, with whole K groups per block,
  // the K parameters of the group that starts at block i
  auto vparams_of = [&](int i) { return entry(i) + (i % Ring::kPB) * 32 * kRowBytes; };
  auto kparams_of = [&](int i) {
    return entry(i) + Ring::kOffEK + ((t_begin + 32 * i) / G == entry_g0(i) ? 0 : 2 * Ring::kKPG);
  };

  struct BlkA {  // V scaled in the A operand
    uint32_t kw[2][KB];
    uint32_t vw[8][VWR];
    uint32_t vs[8], vz[8];  // word holding the slot token's group-gv parameter
  };
  struct BlkB {  // V scale on the probabilities
    uint32_t kw[2][KB];
    uint32_t vh[2][8];  // the word holding the lane's 4 codes of half hf, per slot token
  };
  using Blk = std::conditional_t<kBS, BlkB, BlkA>;
  // word of a V row holding the lane's 4 channels of half hf, and the byte permute
  // that puts those codes of two tokens into the two 16-bit halves
  const uint32_t vbw0 = VB == 4 ? (n >> 1) : (n >> 2), vbw1 = vbw0 + (VB == 4 ? 8 : 4);
  const uint32_t vbsel = VB == 4 ? ((n & 1) ? 0x07060302u : 0x05040100u)
                                 : (0x0C000C00u | ((4u + (n & 3)) << 16) | static_cast<uint32_t>(n & 3));
  // the block's V parameters, one (token, group) per lane, as float scales and f16
  // zeros in the order of the lanes' k-slots; rows at or past t_end get 0
  auto conv_vparams = [&](int i) {
    const int g = lane >> 5, tok = lane & 31;
    if (g < NGV) {
      const P* vsp = reinterpret_cast<const P*>(vparams_of(i));
      const bool ok = t_begin + 32 * i + tok < t_end;
      const float sv = ok ? param_f32<P>(vsp, tok * NGV + g) : 0.f;
      const float zv = ok ? param_f32<P>(vsp + Ring::kVPE / sizeof(P), tok * NGV + g) : 0.f;
      const int kbt = (tok & 15) >> 2, j = (tok & 3) + 4 * (tok >> 4);
      sh_vs[wave][g][kbt][j] = sv;
      sh_vz[wave][g][kbt][j] = static_cast<_Float16>(zv);
    }
  };
  auto read_blk = [&](const unsigned char* slot, Blk& x, int i) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const uint32_t* src = reinterpret_cast<const uint32_t*>(slot + Ring::kOffK) + (16 * tt + n) * KW + kb * KB;
      if constexpr (KB == 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(src);
        x.kw[tt][0] = v.x; x.kw[tt][1] = v.y; x.kw[tt][2] = v.z; x.kw[tt][3] = v.w;
      } else if constexpr (KB == 2) {
        const uint2 v = *reinterpret_cast<const uint2*>(src);
        x.kw[tt][0] = v.x; x.kw[tt][1] = v.y;
      } else {
#pragma unroll
        for (int i = 0; i < KB; ++i) x.kw[tt][i] = src[i];
      }
    }
    const uint32_t* vw = reinterpret_cast<const uint32_t*>(slot + Ring::kOffV);
    if constexpr (kBS) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t tok = static_cast<uint32_t>(slot_token(kb, j));
        x.vh[0][j] = vw[tok * VW + vbw0];
        x.vh[1][j] = vw[tok * VW + vbw1];
      }
      conv_vparams(i);
    } else {
      const uint32_t* vp = reinterpret_cast<const uint32_t*>(vparams_of(i));
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t tok = static_cast<uint32_t>(slot_token(kb, j));
        x.vw[j][0] = vw[tok * VW + vfw];
        if constexpr (VB == 3) x.vw[j][1] = vw[tok * VW + vfw2];
        const uint32_t e = sizeof(P) == 2 ? (tok * NGV + gv) >> 1 : tok * NGV + gv;
        x.vs[j] = vp[e];
        x.vz[j] = vp[Ring::kVPE / 4 + e];
      }
    }
  };
  // A new K group: the lane's 32 channels of its (scale, zero) rows are read from the
  // block's slot and packed as f16 pairs in contraction order; the query operand
  // becomes q * s (times the channel's factor) and the bias sum_c q_c z_c minus the
  // code offset times sum_c (q s)_c is formed on the
  // matrix cores (every row of its A operands is the same, so every score row of a
  // column receives its column's bias).
  auto use_kp = [&](const unsigned char* kp) -> KQ {
    // the scale and zero pairs do not depend on the q-head column: each lane converts
    // one pair of each (step n / 4, pair n % 4 of its channel chunk) and the wave
    // shares them through LDS; only q * s is per lane
    {
      const int st = n >> 2, jj = n & 3;
      const int c0 = 32 * kb + 8 * st + korder<KB>(2 * jj), c1 = 32 * kb + 8 * st + korder<KB>(2 * jj + 1);
      const P* sp = reinterpret_cast<const P*>(kp);
      const P* zp = sp + D;
      sh_kq[wave][0][kb][n] = pack_h2(param_f32<P>(sp, c0) * kweight<KB>(c0), param_f32<P>(sp, c1) * kweight<KB>(c1));
      sh_kq[wave][1][kb][n] = pack_h2(param_f32<P>(zp, c0), param_f32<P>(zp, c1));
    }
    __builtin_amdgcn_wave_barrier();
    constexpr uint32_t kNegOff = kneg_offset<KB>();
    const uint32_t negoff[4] = {kNegOff, kNegOff, kNegOff, kNegOff};
    KQ r;
    r.kbias = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 sw = *reinterpret_cast<const uint4*>(&sh_kq[wave][0][kb][4 * s]);
      const uint4 zw = *reinterpret_cast<const uint4*>(&sh_kq[wave][1][kb][4 * s]);
      const uint32_t s2[4] = {sw.x, sw.y, sw.z, sw.w};
      const uint32_t z2[4] = {zw.x, zw.y, zw.z, zw.w};
      const h8_t qs = bq[s];
      const uint32_t* qw = reinterpret_cast<const uint32_t*>(&qs);
      uint32_t q2[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) q2[jj] = as_u32(as_h2(qw[jj]) * as_h2(s2[jj]));
      r.qt[s] = __builtin_bit_cast(h8_t, q2);
      r.kbias = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, z2), bq[s], r.kbias, 0, 0, 0);
      r.kbias = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, negoff), r.qt[s], r.kbias, 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
    return r;
  };
  // V parameter (as float) of a slot token from its raw word
  // (with one group per token the element parity is the slot's parity; otherwise the
  // token index is even times NGV and the parity is the group's)
  // (bf16 parameters: one byte permute moves the lane's half of the word to the top)
  const uint32_t vsel = (gv & 1) ? 0x03020C0Cu : 0x01000C0Cu;
  auto vparam = [&](uint32_t w, int j) -> float {
    if constexpr (sizeof(P) == 2) {
      if constexpr (NGV == 1) return __uint_as_float((j & 1) ? (w & 0xFFFF0000u) : (w << 16));
      else return __uint_as_float(__builtin_amdgcn_perm(0u, w, vsel));
    } else {
      return __uint_as_float(w);
    }
  };

  // kq: the score operands of the block's K group when a group spans whole blocks
  // (G >= 32); with 16-token groups each 16-token tile forms its own from the slot
  const KConst kc;
  auto process = [&](int t0, const Blk& cur, const unsigned char* slot, const KQ& kq, auto full_tag) {
    constexpr bool full = decltype(full_tag)::value;  // every row of the block is live
    // ---- S^T = K_hat Q^T for the two 16-token tiles
    f4_t sc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      KQ kt;
      if constexpr (NKG == 2) kt = use_kp(slot + Ring::kOffKP + tt * 2 * D * sizeof(P));
      const KQ& k = NKG == 2 ? kt : kq;
      if constexpr (NKG == 2) sc[tt] = k.kbias - m;
      else sc[tt] = seed;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        uint32_t mp[4];
        kpairs<KB>(cur.kw[tt], s, mp, kc);
        sc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, mp), k.qt[s], sc[tt], 0, 0, 0);
      }
    }

    // ---- online softmax of column n over tokens 16 tt + 4 kb + i
    float s8[8];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) s8[4 * tt + i] = (full || t0 + 16 * tt + 4 * kb + i < t_end) ? sc[tt][i] : -INFINITY;
    // the column maximum is only needed when some score exceeds the running maximum
    // by more than 8 (probabilities up to 2^8 are fine in f16): a wave vote on the
    // lanes' own maxima, then the cross-lane maximum inside the (rare) rescale
    auto vmax = [](float a, float b) { return __builtin_elementwise_maximum(a, b); };
    float mb = vmax(vmax(vmax(s8[0], s8[1]), vmax(s8[2], s8[3])), vmax(vmax(s8[4], s8[5]), vmax(s8[6], s8[7])));
    if (__any(mb > thr)) {
      mb = fmaxf(mb, __shfl_xor(mb, 16));
      mb = fmaxf(mb, __shfl_xor(mb, 32));
      // the shift of the reference: the column maximum on the first block, else only
      // upwards (thr - 8 is -inf, then 0)
      const float dm = fmaxf(mb, thr - 8.f);
      // accumulators are zero before the first block, so any finite factor will do
      const float al = __builtin_amdgcn_exp2f(fminf(-dm, 0.f));
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] *= al;
      accz *= al;
      accl *= al;
#pragma unroll
      for (int j = 0; j < 8; ++j) s8[j] -= dm;
      seed -= dm;
      m += dm;
      thr = 8.f;
    }
    float p[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      p[j] = __builtin_amdgcn_exp2f(s8[j]);  // v_exp_f32: results below 2^-126 flush to 0
    }
    uint32_t pw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) pw[j] = pack_h2(p[2 * j], p[2 * j + 1]);
    const h8_t bp = __builtin_bit_cast(h8_t, pw);
    {
      const uint32_t one2[4] = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};  // f16 1.0
      accl = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, one2), bp, accl, 0, 0, 0);
    }

    if constexpr (kBS) {
      // ---- O^T[64 hf + 4 (4 kb' + i) + t % 4][n] += C^T (P s_hf)^T, hf = t / 4, over
      // the block's 32 tokens: A the code values 128 + c (bf16, exact), B the
      // probabilities times the tokens' scales of the half's group (bf16); the offset
      // (-128 sum of B) and the zero-points (sum p z, f16) go to accz: rows 0-7 for
      // half 0, rows 8-15 for half 1
      __builtin_amdgcn_wave_barrier();  // the wave's parameter writes of this block
      uint32_t bs[2][4];
#pragma unroll
      for (int hf = 0; hf < (NGV == 2 ? 2 : 1); ++hf) {
        const float4 s0 = *reinterpret_cast<const float4*>(&sh_vs[wave][hf][kb][0]);
        const float4 s1 = *reinterpret_cast<const float4*>(&sh_vs[wave][hf][kb][4]);
        const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) bs[hf][q2] = pack_bf16(p[2 * q2] * sv[2 * q2], p[2 * q2 + 1] * sv[2 * q2 + 1]);
      }
      if constexpr (NGV == 1) {
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) bs[1][q2] = bs[0][q2];
      }
      {
        const uint4 zw = *reinterpret_cast<const uint4*>(&sh_vz[wave][NGV == 2 ? (n >> 3) : 0][kb][0]);
        accz = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, zw), bp, accz, 0, 0, 0);
        const uint32_t o0 = (NGV == 1 || n < 8) ? 0xC300C300u : 0u, o1 = (NGV == 1 || n >= 8) ? 0xC300C300u : 0u;
        const uint32_t a0[4] = {o0, o0, o0, o0}, a1[4] = {o1, o1, o1, o1};
        accz = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a0), __builtin_bit_cast(bf16x8_t, bs[0]),
                                                       accz, 0, 0, 0);
        if constexpr (NGV == 2)
          accz = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a1), __builtin_bit_cast(bf16x8_t, bs[1]),
                                                         accz, 0, 0, 0);
      }
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        uint32_t cv[4][4];  // [pair][channel i]
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
          const uint32_t comb = __builtin_amdgcn_perm(cur.vh[hf][2 * q2 + 1], cur.vh[hf][2 * q2], vbsel);
          vpairs_bf16<VB>(comb, cv[q2], VB == 4 ? kc.lo : kc.lo2, kc.vmagic);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t av[4] = {cv[0][i], cv[1][i], cv[2][i], cv[3][i]};
          acc[4 * hf + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, bs[hf]), acc[4 * hf + i], 0, 0, 0);
        }
      }
    } else {
      // ---- O^T[8 (4 kb' + i) + vorder(t)][n] += V_hat^T P^T over the block's 32 tokens
      uint32_t sv2[4], nsv2[4], zv2[4], vp[4][8];
  #pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) {
        const uint32_t ta = t0 + slot_token(kb, 2 * q2), tb = t0 + slot_token(kb, 2 * q2 + 1);
        float sa = vparam(cur.vs[2 * q2], 2 * q2), sb = vparam(cur.vs[2 * q2 + 1], 2 * q2 + 1);
        float za = vparam(cur.vz[2 * q2], 2 * q2), zb = vparam(cur.vz[2 * q2 + 1], 2 * q2 + 1);
        if constexpr (!full) {  // rows past the end dequantize to exactly 0
          const bool oka = static_cast<int>(ta) < t_end, okb = static_cast<int>(tb) < t_end;
          sa = oka ? sa : 0.f; za = oka ? za : 0.f;
          sb = okb ? sb : 0.f; zb = okb ? zb : 0.f;
        }
        sv2[q2] = pack_h2(sa, sb);
        zv2[q2] = pack_h2(za, zb);
        uint32_t fa, fb;
        if constexpr (VB == 3) {
          fa = __builtin_amdgcn_alignbit(cur.vw[2 * q2][VWR - 1], cur.vw[2 * q2][0], vfo) & 0xFFFFFFu;
          fb = __builtin_amdgcn_alignbit(cur.vw[2 * q2 + 1][VWR - 1], cur.vw[2 * q2 + 1][0], vfo) & 0xFFFFFFu;
        } else if constexpr (VB == 2) {
          fa = cur.vw[2 * q2][0] >> vfo;
          fb = cur.vw[2 * q2 + 1][0] >> vfo;
        } else {
          fa = cur.vw[2 * q2][0];
          fb = cur.vw[2 * q2 + 1][0];
        }
        vpairs<VB>(fa, fb, vp[q2]);
        nsv2[q2] = as_u32(as_h2(sv2[q2]) * as_h2(0xD400D400u));  // -64 s, exact
      }
      accz = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, zv2), bp, accz, 0, 0, 0);
  #pragma unroll
      for (int t = 0; t < 8; ++t) {
        uint32_t av[4];
  #pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) av[q2] = scale_pair(vp[q2][t], sv2[q2], nsv2[q2]);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, av), bp, acc[t], 0, 0, 0);
      }
    }
  };

  // Main loop over the wave's blocks.  Before block i is read, its copies must have
  // landed: kInstr copies are issued per block, so while blocks i+1 .. i+kDepth-1 are
  // still in flight the wait is vmcnt((kDepth-1) kInstr); near the end, where fewer
  // blocks follow, everything is drained.  The slot is refilled (block i + kDepth)
  // only after block i has been processed, so its reads are complete by then.
  using Full = std::integral_constant<bool, true>;
  using Part = std::integral_constant<bool, false>;
  const int nfull = t_end > t_begin ? (t_end - t_begin) / 32 : 0;  // blocks with every row live
  // the query loads complete before the first copies are issued (a wait the compiler
  // tracks, so it adds none behind the copies, which would drain the ring)
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  for (int i = 0; i < nblk && i < Ring::kDepth; ++i) issue(i);
  auto wait_blk = [&](int i) {
    if (i + Ring::kDepth <= nblk) {
      // entries started by the next kDepth - 1 blocks
      const int ne = (i + Ring::kDepth - 1) / Ring::kPB - i / Ring::kPB;
      Ring::wait_ahead(ne);
    } else {
      Ring::wait_all();
    }
  };
  // one pass of the outer loop per K group (its blocks in the inner loop), so that the
  // group's score operands are formed once and are not loop-carried
  for (int i = 0; i < nfull;) {
    KQ kq;
    int nb = nfull - i;
    if constexpr (NKG == 1) {
      const int t0 = t_begin + 32 * i;
      nb = min(nb, (G - t0 % G) / 32);  // blocks left in this group
      wait_blk(i);
      kq = use_kp(kparams_of(i));
      seed = kq.kbias - m;
    }
    for (int e = i + nb; i < e; ++i) {
      wait_blk(i);
      const unsigned char* slot = wring + (i % Ring::kDepth) * Ring::kSlot;
      Blk cur;
      read_blk(slot, cur, i);
      // with one K group per block every read of the slot is in cur: the slot is
      // refilled before the block is computed, so that two blocks are in flight
      // during the computation
      if (NKG == 1 && i + Ring::kDepth < nblk) {
        Ring::lds_reads_done();
        issue(i + Ring::kDepth);
      }
      process(t_begin + 32 * i, cur, slot, kq, Full{});
      if (NKG == 2 && i + Ring::kDepth < nblk) {
        Ring::lds_reads_done();
        issue(i + Ring::kDepth);
      }
    }
  }
  Ring::wait_all();
  if (nfull < nblk) {  // the partial last block (its copies were issued above)
    const unsigned char* slot = wring + (nfull % Ring::kDepth) * Ring::kSlot;
    KQ kq;
    if constexpr (NKG == 1) {
      kq = use_kp(kparams_of(nfull));
      seed = kq.kbias - m;
    }
    Blk cur;
    read_blk(slot, cur, nfull);
    process(t_begin + 32 * nfull, cur, slot, kq, Part{});
  }
  if (thr == -INFINITY) m = -INFINITY;  // no rows: the merge gives this wave no weight
  __syncthreads();  // every wave's copies have landed before the ring is reused

  // ---- merge the 4 waves in LDS, write this split's partial
  const float l = accl[0];
  if (kb == 0) {
    sh_m[wave][n] = m;
    sh_l[wave][n] = l;
  }
  if constexpr (kBS) {
    // the rows of accz are alike within a half: this lane's is half kb / 2, the other
    // half's is in lane ^ 32
    const float cmine = accz[0], cother = __shfl_xor(cmine, 32);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float corr = (kb >> 1) == (t >> 2) ? cmine : cother;
#pragma unroll
      for (int i = 0; i < 4; ++i) sh_o[wave][n][64 * (t >> 2) + 4 * (4 * kb + i) + (t & 3)] = acc[t][i] + corr;
    }
  } else {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) sh_o[wave][n][8 * (4 * kb + i) + vorder<VB>(t)] = acc[t][i] + accz[i];
  }
  __syncthreads();
  const int64_t pbase = static_cast<int64_t>(bh) * a.splits + split;
  for (int idx = tid; idx < H * D; idx += kDecThreads) {
    const int h = idx / D, c = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sh_m[w][h]);
    float O = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float wt = sh_m[w][h] == -INFINITY ? 0.f : exp2f(sh_m[w][h] - M);
      O = fmaf(sh_o[w][h][c], wt, O);
      L = fmaf(sh_l[w][h], wt, L);
    }
    a.part_o[(pbase * H + h) * D + c] = O;
    if (c == 0) {
      a.part_ml[(pbase * H + h) * 2] = M;
      a.part_ml[(pbase * H + h) * 2 + 1] = L;
    }
  }
}

// ------------------------------------------------------------------ dispatch

bool decode_mfma_supported(const vc_ckv* c, int H) {
  if (c->flags & VC_CKV_DECODE_F32) return false;  // the caller asked for float32 operands
  if (c->method != VC_QUANT_KIVI || c->kv_dtype != VC_BF16 || c->d != 128 || H < 1 || H > 16) return false;
  auto ok_bits = [](int b) { return b == 2 || b == 3 || b == 4; };
  if (!ok_bits(c->k_bits) || !ok_bits(c->v_bits)) return false;
  if (c->capacity % 32 != 0 || c->capacity > (1ll << 26)) return false;
  return c->group == 16 || c->group == 32 || c->group == 64 || c->group == 128;
}

// Every instance of the kernel, chosen by (k bits, v bits, groups per V row,
// parameter type): op.run<...>() is called for the one matching the cache.
template <class Op>
static void dispatch_decode_mfma(const vc_ckv* c, const Op& op) {
  const int ngv = 128 / c->group;
  auto by_ngv = [&](auto kb, auto vb, auto p) {
    constexpr int KB = decltype(kb)::value, VB = decltype(vb)::value;
    using P = typename decltype(p)::type;
    switch (ngv) {
      case 1: op.template run<KB, VB, 1, P>(); break;
      case 2: op.template run<KB, VB, 2, P>(); break;
      case 4: op.template run<KB, VB, 4, P>(); break;
      default: op.template run<KB, VB, 8, P>(); break;
    }
  };
  auto by_vb = [&](auto kb, auto p) {
    if (c->v_bits == 2) by_ngv(kb, std::integral_constant<int, 2>{}, p);
    else if (c->v_bits == 3) by_ngv(kb, std::integral_constant<int, 3>{}, p);
    else by_ngv(kb, std::integral_constant<int, 4>{}, p);
  };
  auto by_kb = [&](auto p) {
    if (c->k_bits == 2) by_vb(std::integral_constant<int, 2>{}, p);
    else if (c->k_bits == 3) by_vb(std::integral_constant<int, 3>{}, p);
    else by_vb(std::integral_constant<int, 4>{}, p);
  };
  if (c->param_dtype == VC_BF16) by_kb(type_tag<bf16_t>{});
  else by_kb(type_tag<float>{});
}

// Workgroups of an instance that fit on the device at once (queried once).
template <int KB, int VB, int NGV, typename P>
static int decode_mfma_resident() {
  static const int r = [] {
    int dev = 0, cus = 0, per = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 512;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 512;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, decode_mfma_kernel<KB, VB, NGV, P>, kDecThreads, 0) !=
        hipSuccess)
      return 512;
    return (per > 0 ? per : 1) * (cus > 0 ? cus : 1);
  }();
  return r;
}

struct ResidentOp {
  int* out;
  template <int KB, int VB, int NGV, typename P>
  void run() const { *out = decode_mfma_resident<KB, VB, NGV, P>(); }
};

struct LaunchOp {
  dim3 grid;
  hipStream_t s;
  const DecodeArgs* a;
  template <int KB, int VB, int NGV, typename P>
  void run() const {
    hipLaunchKernelGGL((decode_mfma_kernel<KB, VB, NGV, P>), grid, dim3(kDecThreads), 0, s, *a);
  }
};

// Compressed-row splits sized so that they run in one pass over the device:
// splits * B * Hkv workgroups <= the resident count (the tail rows are merged by
// decode_merge_kernel, which takes one more partial).
int decode_mfma_splits(const vc_ckv* c) {
  const int bh = c->B * c->Hkv;
  int resident = 512;
  dispatch_decode_mfma(c, ResidentOp{&resident});
  int s = resident / bh;
  if (s < 1) s = 1;
  if (s > kDecMaxSplits - 1) s = kDecMaxSplits - 1;
  return s;
}

void launch_decode_mfma(const vc_ckv* c, const DecodeArgs& a, dim3 grid, hipStream_t s) {
  dispatch_decode_mfma(c, LaunchOp{grid, s, &a});
}

}  // namespace vc
