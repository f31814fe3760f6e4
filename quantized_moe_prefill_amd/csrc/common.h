// Shared device helpers for the gfx950 (CDNA4) kernels of the MoE prefill
// library: vector types for the bf16 matrix-core instructions, bit-pattern
// conversions, and wave-level reductions for 64-wide wavefronts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmoe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
// Low / high bf16 of a packed pair.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}
// Low / high fp16 of a packed pair.
__device__ __forceinline__ float f16lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
// Largest finite fp16 value.
constexpr float kF16Max = 65504.0f;

// Two fp32 -> packed fp16 pair (round to nearest even), saturating: values
// beyond the fp16 range become +-65504 instead of infinity (one v_med3_f32
// each; the identity on every value that rounds to a finite fp16, so results
// in range are unchanged). Every fp16 intermediate of the layer (the fp16
// copy of x, h, y_perm, y_shared) is stored through this.
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  a = __builtin_amdgcn_fmed3f(a, -kF16Max, kF16Max);
  b = __builtin_amdgcn_fmed3f(b, -kF16Max, kF16Max);
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

// silu(z) = z / (1 + e^-z), with the hardware reciprocal (about one fp32
// ulp) in place of an IEEE division, which compiles to a ten-instruction
// sequence; every caller rounds the result to fp16. Large |z| behaves:
// e^-z overflows to infinity and the reciprocal to zero for very negative z.
__device__ __forceinline__ float silu_f32(float z) {
  return z * __builtin_amdgcn_rcpf(1.f + __expf(-z));
}

// Eight bf16 values (x0..x7, two per word) -> fp16 in kperm chunk order
// (positions 0..7 hold x0, x4, x1, x5, x2, x6, x3, x7); exact for
// 2^-14 <= |x| <= 65504 (and zero), saturating beyond.
__device__ __forceinline__ u32x4 bf16x8_to_f16_kperm(u32x4 d) {
  u32x4 o;
  o[0] = pack_f16x2(bf16lo(d[0]), bf16lo(d[2]));  // x0, x4
  o[1] = pack_f16x2(bf16hi(d[0]), bf16hi(d[2]));  // x1, x5
  o[2] = pack_f16x2(bf16lo(d[1]), bf16lo(d[3]));  // x2, x6
  o[3] = pack_f16x2(bf16hi(d[1]), bf16hi(d[3]));  // x3, x7
  return o;
}

// D = A(16x32) * B(32x16) + C on the bf16 matrix cores, fp32 accumulation.
// Operand layout per lane l: A row l%16 / B column l%16, eight consecutive K
// values starting at 8*(l/16). Result: lane l holds rows 4*(l/16)+0..3 of
// column l%16. (The K order inside an operand only has to agree between A
// and B, which it does by construction.)
__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// Same shape and operand layout on fp16 operands.
__device__ __forceinline__ f32x4 mfma_16x16x32_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// K order of the fp16 expert operands. Unpacking a 32-bit word of eight
// nibbles as (w >> 4i) & 0x000F000F yields element pairs (i, i+4), so every
// 8-element chunk of an fp16 operand holds its elements in the order
// 0,4,1,5,2,6,3,7. Activations (and h) are stored in that order too, so both
// matrix-core operands agree; position p of a chunk holds element kperm(p),
// and element i sits at position kpos(i).
__host__ __device__ constexpr inline int kperm(int p) { return (p >> 1) + 4 * (p & 1); }
__host__ __device__ constexpr inline int kpos(int i) { return 2 * (i & 3) + (i >> 2); }

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// a[i] += w * (element i of eight bf16 / fp16 values)
__device__ __forceinline__ void acc8_bf16(float* a, u32x4 v, float w) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[2 * i] = fmaf(w, bf16lo(v[i]), a[2 * i]);
    a[2 * i + 1] = fmaf(w, bf16hi(v[i]), a[2 * i + 1]);
  }
}
__device__ __forceinline__ void acc8_f16(float* a, u32x4 v, float w) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[2 * i] = fmaf(w, f16lo(v[i]), a[2 * i]);
    a[2 * i + 1] = fmaf(w, f16hi(v[i]), a[2 * i + 1]);
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Word 3 of a raw buffer resource on gfx950 (32-bit data format, offset
// mode).
constexpr int kRsrcWord3 = 0x00020000;

// s_waitcnt immediates (gfx9 encoding): wait until at most n vector memory
// operations are outstanding, leaving the LDS and export counters alone.
// The builtin form keeps the compiler's own wait bookkeeping exact.
__host__ __device__ constexpr inline int waitcnt_vm(int n) {
  return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00;
}

// Address-space pointer types of the direct global->LDS loads.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

__host__ __device__ constexpr inline int cdiv(int a, int b) { return (a + b - 1) / b; }

// Workgroup barrier for LDS hand-offs only. __syncthreads() also orders
// global memory, which on this target means waiting for every outstanding
// vector memory operation (loads included) first and would drain the load
// pipeline; the callers wait for exactly the loads
// they need (s_waitcnt vmcnt) before this barrier. It completes this wave's
// own LDS operations, and the empty asm statements keep the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The LDS writes of this wave are complete and visible to its own later
// reads (a wave's LDS operations complete in order; the wait also keeps the
// compiler from reordering across it).
__device__ __forceinline__ void lds_wave_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
}

}  // namespace qmoe
