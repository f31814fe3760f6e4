// In-register dequantization of 4-bit expert weights to fp16 matrix-core
// operands, shared by the expert GEMM kernels (the symmetric and asymmetric
// 4-bit expert formats of the hipfire 0.4.3 benchmarks page, "Known
// limits": w = (n - 8) * scale, or w = n * scale + min, one fp16 scale and
// min per group of G weights along K).
#pragma once

#include "common.h"

namespace qmoe {

// Eight consecutive 4-bit weights (one 32-bit word) of one row -> eight fp16
// weights in the kperm chunk order: output word i holds the pair of elements
// (i, i + 4), i.e. nibble i of the word's low and high halves. A nibble ORed
// into the low four mantissa bits of the fp16 pattern 0x6400 gives exactly
// 1024 + n; ORed into mantissa bits 4-7 of 0x5400 (exponent 6, so those bits
// count in units of one) it gives exactly 64 + n. So nibbles 0 and 1 of each
// half need no shift and nibbles 2 and 3 one shift of the word by 8:
// thirteen instructions per word instead of fifteen. Subtracting 1032 or 72
// (symmetric) or 1024 or 64 (asymmetric) is exact, and the final multiply
// (or fused multiply-add with the min) rounds once. ONE_SHIFT = false gives
// the form with a shift per nibble (the same values, one fewer live
// register), for kernels that are at their register limit.
template <bool ASYM, bool ONE_SHIFT = true>
__device__ __forceinline__ f16x8 dequant8_f16(uint32_t w, f16x2 s2, f16x2 m2) {
  if constexpr (!ONE_SHIFT) {
    const f16x2 off = ASYM ? f16x2{(_Float16)1024.0f, (_Float16)1024.0f}
                           : f16x2{(_Float16)1032.0f, (_Float16)1032.0f};
    const uint32_t mask = __builtin_amdgcn_readfirstlane(0x000f000fu);
    uint32_t magic = 0x64006400u;
    asm("" : "+v"(magic));
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t t = ((w >> (4 * i)) & mask) | magic;  // (1024 + n_i, 1024 + n_{i+4})
      const f16x2 n = __builtin_bit_cast(f16x2, t) - off;
      const f16x2 v = ASYM ? __builtin_elementwise_fma(n, s2, m2) : n * s2;
      o[i] = __builtin_bit_cast(uint32_t, v);
    }
    return __builtin_bit_cast(f16x8, o);
  }
  const f16x2 off_lo = ASYM ? f16x2{(_Float16)1024.0f, (_Float16)1024.0f}
                            : f16x2{(_Float16)1032.0f, (_Float16)1032.0f};
  const f16x2 off_hi = ASYM ? f16x2{(_Float16)64.0f, (_Float16)64.0f}
                            : f16x2{(_Float16)72.0f, (_Float16)72.0f};
  // the masks live in scalar registers and the fp16 patterns in vector ones,
  // so that each mask-and-or is a single v_and_or_b32 (VOP3 takes no literal
  // and at most one scalar operand on gfx9)
  const uint32_t mask_lo = __builtin_amdgcn_readfirstlane(0x000f000fu);
  const uint32_t mask_hi = __builtin_amdgcn_readfirstlane(0x00f000f0u);
  uint32_t magic_lo = 0x64006400u, magic_hi = 0x54005400u;
  asm("" : "+v"(magic_lo), "+v"(magic_hi));
  const uint32_t w8 = w >> 8;
  const uint32_t t[4] = {(w & mask_lo) | magic_lo, (w & mask_hi) | magic_hi,
                         (w8 & mask_lo) | magic_lo, (w8 & mask_hi) | magic_hi};
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 n = __builtin_bit_cast(f16x2, t[i]) - ((i & 1) ? off_hi : off_lo);
    const f16x2 v = ASYM ? __builtin_elementwise_fma(n, s2, m2) : n * s2;
    o[i] = __builtin_bit_cast(uint32_t, v);
  }
  return __builtin_bit_cast(f16x8, o);
}

// Lower-bit symmetric codes (w = (q - 2^(b-1)) * scale) in the library's
// 2- and 3-bit row layouts. A 32-bit word of 2-bit codes holds 16 elements:
// bytes 0..3 = elements 0-3, 8-11, 4-7, 12-15, two bits each, so that
// (w >> (8 h + 2 i)) & 0x00030003 is the pair (i, i + 4) of the word's
// 8-element chunk h, already in the kperm order of the fp16 operands (and
// one mask-and-or with the fp16 pattern 0x6400 gives 1024 + q).

// Chunk `h` (0 or 1) of a word of 2-bit codes -> eight fp16 weights.
__device__ __forceinline__ f16x8 dequant8_f16_b2(uint32_t w, int h, f16x2 s2) {
  const f16x2 off = {(_Float16)1026.0f, (_Float16)1026.0f};
  const uint32_t mask = __builtin_amdgcn_readfirstlane(0x00030003u);
  uint32_t magic = 0x64006400u;
  asm("" : "+v"(magic));
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t t = ((w >> (8 * h + 2 * i)) & mask) | magic;
    o[i] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, t) - off) * s2);
  }
  return __builtin_bit_cast(f16x8, o);
}

// 3-bit codes: the low two bits as above; the word `hb` holds the third bit
// of the 32-element block, bit 4c + i for element 8c + i and bit 16 + 4c + i
// for element 8c + i + 4. Chunk c (0..3) of the block -> eight fp16 weights
// (its low bits are chunk c % 2 of 2-bit word c / 2, passed as w).
__device__ __forceinline__ f16x8 dequant8_f16_b3(uint32_t w, uint32_t hb, int c, f16x2 s2) {
  // (an opaque copy per call: otherwise the compiler computes the shifted
  // high-bit words of every chunk up front and holds them in registers)
  asm("" : "+v"(hb));
  const f16x2 off = {(_Float16)1028.0f, (_Float16)1028.0f};
  const uint32_t mask = __builtin_amdgcn_readfirstlane(0x00030003u);
  uint32_t magic = 0x64006400u;
  asm("" : "+v"(magic));
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = 4 * c + i;
    const uint32_t hi = p >= 2 ? (hb >> (p - 2)) : (hb << (2 - p));  // bits p, 16+p -> 2, 18
    uint32_t t = ((w >> (8 * (c & 1) + 2 * i)) & mask) | magic;
    t |= hi & 0x00040004u;
    o[i] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, t) - off) * s2);
  }
  return __builtin_bit_cast(f16x8, o);
}

// The same codes without a shift per pair: the fp16 pattern ORed around pair
// i (bits 2i, 2i + 1 of each half) has exponent 25 - 2i, which makes mantissa
// bit 2i count in units of one, so the pair reads as 2^(10 - 2i) + q from the
// unshifted word (one shift by 8 for the upper byte of each half). The
// subtraction of 2^(10 - 2i) + 2^(b-1) is exact and the multiply rounds once:
// the same fp16 weights as the per-pair shift form.
struct LowBitMagic {
  uint32_t magic[4];  // 2^(10 - 2i) in both halves, in vector registers
  uint32_t m2[4];     // 0x00030003 << 2i, in scalar registers
  uint32_t m4[4];     // 0x00040004 << 2i (the 3-bit high bit of pair i)
};
__device__ __forceinline__ LowBitMagic low_bit_magic() {
  LowBitMagic k;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    k.magic[i] = (uint32_t)(0x6400 - 0x0800 * i) * 0x10001u;
    asm("" : "+v"(k.magic[i]));
    k.m2[i] = __builtin_amdgcn_readfirstlane(0x00030003u << (2 * i));
    k.m4[i] = __builtin_amdgcn_readfirstlane(0x00040004u << (2 * i));
  }
  return k;
}

// Chunk `h` (0 or 1) of a word of 2-bit codes -> eight fp16 weights.
__device__ __forceinline__ f16x8 dequant8_f16_b2x(uint32_t w, int h, f16x2 s2) {
  const LowBitMagic k = low_bit_magic();
  const uint32_t wl = h ? w >> 8 : w;
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const _Float16 base = (_Float16)(float)((1024 >> (2 * i)) + 2);
    const uint32_t t = (wl & k.m2[i]) | k.magic[i];
    o[i] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, t) - f16x2{base, base}) * s2);
  }
  return __builtin_bit_cast(f16x8, o);
}

// 3-bit codes in the tiled layout (moe_pack_tier), whose third-bit word holds
// the high bit of element 8c + i + 4h at bit (2 + 2i + 16h + (0, 1, 8, 9)[c])
// mod 32: rotated right by (0, 1, 8, 9)[c], chunk c's high bits sit just
// above the low bits of their pair (bit 2i + 2 of each half), so one rotate
// per chunk replaces a shift per pair.
__device__ __forceinline__ f16x8 dequant8_f16_b3t(uint32_t w, uint32_t hb, int c, f16x2 s2) {
  asm("" : "+v"(hb));
  const LowBitMagic k = low_bit_magic();
  const uint32_t wl = (c & 1) ? w >> 8 : w;
  constexpr int rot[4] = {0, 1, 8, 9};
  const uint32_t hc = c == 0 ? hb : __builtin_amdgcn_alignbit(hb, hb, rot[c & 3]);
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const _Float16 base = (_Float16)(float)((1024 >> (2 * i)) + 4);
    uint32_t t = (wl & k.m2[i]) | k.magic[i];
    t |= hc & k.m4[i];
    o[i] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, t) - f16x2{base, base}) * s2);
  }
  return __builtin_bit_cast(f16x8, o);
}

// The third-bit word of a 3-bit block rearranged for dequant8_f16_b3t: bit
// 4c + i + 16h moves to bit (2 + 2i + 16h + (0, 1, 8, 9)[c]) mod 32.
__host__ __device__ inline uint32_t b3_high_tiled(uint32_t hb) {
  const int rot[4] = {0, 1, 8, 9};
  uint32_t o = 0;
  for (int c = 0; c < 4; ++c)
    for (int i = 0; i < 4; ++i)
      for (int h = 0; h < 2; ++h)
        o |= ((hb >> (4 * c + i + 16 * h)) & 1u) << ((2 + 2 * i + 16 * h + rot[c]) & 31);
  return o;
}

}  // namespace qmoe
