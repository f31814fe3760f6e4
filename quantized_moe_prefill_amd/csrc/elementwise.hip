// Combine (weighted unpermute) and RMSNorm for the MoE prefill layer on
// gfx950. Both are HBM-bound row operations: each thread owns 8 consecutive
// bf16 channels (one 16-byte load/store), consecutive threads cover
// consecutive channels of a row, so every row is read and written with
// fully coalesced 16-byte accesses.
#include "common.h"
#include "dequant.h"
#include "kernels.h"

namespace qmoe {

namespace {

// out[t] = sum_j w[t,j] y_perm[inv[t*k+j]] (+ sw[t] y_sh[t]) (+ res[t]);
// y_perm and y_sh are fp16, res and out bf16.
template <int K>
__global__ __launch_bounds__(256) void combine_kernel(
    const uint16_t* __restrict__ yperm, const int32_t* __restrict__ inv,
    const float* __restrict__ tw, const uint16_t* __restrict__ ysh,
    const float* __restrict__ sw, const uint16_t* res, uint16_t* out, int T, int H) {
  const int cpr = H / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)T * cpr) return;
  const int t = (int)(idx / cpr);
  const int c = (int)(idx - (int64_t)t * cpr) * 8;
  // every load of the token is issued before the first sum: the row
  // indices and weights, then the K rows, the shared row and the residual;
  // the sums then run in the fixed order j = 0 .. K-1, shared, residual
  int r[K];
  float w[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    r[j] = inv[(int64_t)t * K + j];
    w[j] = tw[(int64_t)t * K + j];
  }
  u32x4 v[K];
#pragma unroll
  for (int j = 0; j < K; ++j) v[j] = ld16(yperm + (int64_t)r[j] * H + c);
  u32x4 vs = {0u, 0u, 0u, 0u}, vr = {0u, 0u, 0u, 0u};
  if (ysh != nullptr) vs = ld16(ysh + (int64_t)t * H + c);
  if (res != nullptr) vr = ld16(res + (int64_t)t * H + c);
  float a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = 0.f;
#pragma unroll
  for (int j = 0; j < K; ++j) acc8_f16(a, v[j], w[j]);
  if (ysh != nullptr) acc8_f16(a, vs, sw[t]);
  if (res != nullptr) acc8_bf16(a, vr, 1.f);
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(a[2 * i], a[2 * i + 1]);
  st16(out + (int64_t)t * H + c, o);
}

// One wave per row.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const uint16_t* __restrict__ x,
                                                     const float* __restrict__ w, float eps,
                                                     uint16_t* __restrict__ out, int T, int H) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= T) return;
  const uint16_t* xr = x + (int64_t)row * H;
  float ss = 0.f;
  for (int c = lane * 8; c < H; c += 64 * 8) {
    const u32x4 v = ld16(xr + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float l = bf16lo(v[i]), h = bf16hi(v[i]);
      ss = fmaf(l, l, ss);
      ss = fmaf(h, h, ss);
    }
  }
  ss = wave_sum(ss);
  const float r = 1.f / sqrtf(ss / (float)H + eps);
  for (int c = lane * 8; c < H; c += 64 * 8) {
    const u32x4 v = ld16(xr + c);
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float l = bf16lo(v[i]) * r * w[c + 2 * i];
      const float h = bf16hi(v[i]) * r * w[c + 2 * i + 1];
      o[i] = pack_bf16x2(l, h);
    }
    st16(out + (int64_t)row * H + c, o);
  }
}

}  // namespace

hipError_t launch_combine(const uint16_t* y_perm, const int32_t* inv, const float* topk_w,
                          const uint16_t* y_shared, const float* shared_w,
                          const uint16_t* residual, uint16_t* out, int T, int H, int k,
                          hipStream_t s) {
  const int64_t n = (int64_t)T * (H / 8);
  const dim3 grid((unsigned)((n + 255) / 256)), block(256);
  LaunchScope ls("combine", s);
#define QMOE_COMBINE(KK)                                                                       \
  case KK:                                                                                     \
    hipLaunchKernelGGL(combine_kernel<KK>, grid, block, 0, s, y_perm, inv, topk_w, y_shared,  \
                       shared_w, residual, out, T, H);                                         \
    break;
  switch (k) {
    QMOE_COMBINE(1)
    QMOE_COMBINE(2)
    QMOE_COMBINE(3)
    QMOE_COMBINE(4)
    QMOE_COMBINE(5)
    QMOE_COMBINE(6)
    QMOE_COMBINE(7)
    default: QMOE_COMBINE(8)
  }
#undef QMOE_COMBINE
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void write_maps_kernel(ExpertMaps m, int E, int32_t* group,
                                                         int32_t* slot) {
  const int e = threadIdx.x;
  if (e < E) {
    group[e] = m.group[e];
    slot[e] = m.slot[e];
  }
}

hipError_t launch_write_maps(const ExpertMaps& m, int E, int32_t* group, int32_t* slot,
                             hipStream_t s) {
  if (E <= 0 || E > 256) return hipErrorInvalidValue;
  LaunchScope ls("write_maps", s);
  hipLaunchKernelGGL(write_maps_kernel, dim3(1), dim3(256), 0, s, m, E, group, slot);
  return hipGetLastError();
}

// The tiled 4-bit layout: 16-byte chunk c of the destination is lane
// l = c % 64 of block b = c / 64, i.e. row group b / nk, K stage b % nk;
// lane l = 16 lg + r holds row 16 (b / nk) + r, bytes [64 stage + 16 lg, +16)
// of the row-major matrix (the 32 elements the lane feeds the matrix cores
// in that stage).
__global__ __launch_bounds__(256) void pack_w4_kernel(const uint8_t* __restrict__ src,
                                                      uint8_t* __restrict__ dst, int64_t chunks,
                                                      int nk, int row_bytes) {
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < chunks;
       c += (int64_t)gridDim.x * 256) {
    const int64_t b = c >> 6;
    const int l = (int)(c & 63);
    const int64_t grp = b / nk;
    const int st = (int)(b - grp * nk);
    const int64_t so = (grp * 16 + (l & 15)) * row_bytes + st * 64 + (l >> 4) * 16;
    st16(dst + c * 16, ld16(src + so));
  }
}

hipError_t launch_pack_w4(const uint8_t* src, uint8_t* dst, int64_t rows, int64_t K,
                          hipStream_t s) {
  const int64_t chunks = rows * K / 32;
  int64_t blocks = (chunks + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  if (blocks < 1) return hipSuccess;
  LaunchScope ls("pack_w4", s);
  hipLaunchKernelGGL(pack_w4_kernel, dim3((unsigned)blocks), dim3(256), 0, s, src, dst, chunks,
                     (int)(K / 128), (int)(K / 2));
  return hipGetLastError();
}

// Any width b (4, 3 or 2 bits): the 4b-byte 32-element blocks of a matrix
// [rows][K b / 8] regrouped into blocks of 16 rows x 128 K (256 b bytes;
// lane l = ((k % 128) / 32) * 16 + r % 16 at 4 b l), one 32-bit word per
// thread. With `interleave` (the 3- and 2-bit gate/up matrices, whose kernel
// gives fragment f of a 32-row group the rows 2 (f % 2) + prow(r)), block
// row 16 p + r of each 32-row group takes source row 2 p + prow(r),
// prow(r) = 8 (r / 4) + kperm(r % 4). With 3 bits the third word of each
// lane's 12 bytes (the block's high bits) is rearranged by b3_high_tiled.
__global__ __launch_bounds__(256) void pack_tier_kernel(const uint32_t* __restrict__ src,
                                                        uint32_t* __restrict__ dst,
                                                        int64_t words, int nk, int bits,
                                                        int row_words, int interleave) {
  const int blk_words = 64 * bits;  // words of one 16-row x 128-K block
  for (int64_t w = (int64_t)blockIdx.x * 256 + threadIdx.x; w < words;
       w += (int64_t)gridDim.x * 256) {
    const int64_t b = w / blk_words;
    const int in = (int)(w - b * blk_words);
    const int l = in / bits, j = in - l * bits;
    const int64_t stripe = b / nk;
    const int st = (int)(b - stripe * nk);
    const int r = l & 15;
    int64_t row = stripe * 16 + r;
    if (interleave) {
      const int p = (int)(stripe & 1);
      row = (stripe >> 1) * 32 + 2 * p + 8 * (r >> 2) + kperm(r & 3);
    }
    const uint32_t v = src[row * row_words + st * 4 * bits + (l >> 4) * bits + j];
    // (3 bits: the third-bit word of each 32-element block in the order the
    // tiled kernels decode it)
    dst[w] = bits == 3 && j == 2 ? b3_high_tiled(v) : v;
  }
}

hipError_t launch_pack_tier(const uint8_t* src, uint8_t* dst, int64_t rows, int64_t K, int bits,
                            bool interleave, hipStream_t s) {
  const int64_t words = rows * K / 32 * bits;
  int64_t blocks = (words + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  if (blocks < 1) return hipSuccess;
  LaunchScope ls("pack_tier", s);
  hipLaunchKernelGGL(pack_tier_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<const uint32_t*>(src), reinterpret_cast<uint32_t*>(dst), words,
                     (int)(K / 128), bits, (int)(K / 32 * bits), interleave ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const uint16_t* x, const float* w, float eps, uint16_t* out, int T,
                          int H, hipStream_t s) {
  const dim3 grid(cdiv(T, 4)), block(256);
  LaunchScope ls("rmsnorm", s);
  hipLaunchKernelGGL(rmsnorm_kernel, grid, block, 0, s, x, w, eps, out, T, H);
  return hipGetLastError();
}

}  // namespace qmoe
