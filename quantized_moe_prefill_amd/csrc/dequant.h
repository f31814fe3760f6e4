// In-register dequantization of 4-bit expert weights to fp16 matrix-core
// operands, shared by the expert GEMM kernels (the symmetric and asymmetric
// 4-bit expert formats of the hipfire 0.4.3 benchmarks page, "Known
// limits": w = (n - 8) * scale, or w = n * scale + min, one fp16 scale and
// min per group of G weights along K).
#pragma once

#include "common.h"

namespace qmoe {

// Eight consecutive 4-bit weights (one 32-bit word) of one row -> eight fp16
// weights in the kperm chunk order. OR-ing a nibble n into the fp16 pattern
// 0x6400 gives exactly 1024 + n; subtracting 1032 (symmetric) or 1024
// (asymmetric) is exact, and the final multiply (or fused multiply-add with
// the min) rounds once.
template <bool ASYM>
__device__ __forceinline__ f16x8 dequant8_f16(uint32_t w, f16x2 s2, f16x2 m2) {
  const f16x2 off = ASYM ? f16x2{(_Float16)1024.0f, (_Float16)1024.0f}
                         : f16x2{(_Float16)1032.0f, (_Float16)1032.0f};
  // the two constants live in registers so that mask-and-or is a single
  // v_and_or_b32 (VOP3 takes no literal and at most one scalar operand on
  // gfx9): the mask in a scalar register, the fp16 pattern in a vector one
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

}  // namespace qmoe
