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

}  // namespace qmoe
