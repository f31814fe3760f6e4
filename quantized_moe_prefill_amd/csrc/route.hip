// Router for the MoE prefill layer on gfx950: fp32 router logits on the bf16
// matrix cores, then a wavefront-level top-k and softmax per token.
//
// The logits are an fp32 GEMM L = x * Wr^T over bf16 activations. Each fp32
// router weight is split exactly into three bf16 terms (w = w1 + w2 + w3,
// truncating the significand 8 bits at a time), so every bf16 x bf16 product
// on the matrix cores is exact and only the fp32 accumulation rounds - the
// same error class as an fp32 GEMM, at bf16 matrix-core speed. The split is a
// tiny pre-pass over E*H weights.
#include "common.h"
#include "kernels.h"

namespace qmoe {

namespace {

constexpr int kRouteRows = 32;  // tokens per workgroup

__global__ __launch_bounds__(256) void router_split_kernel(const float* __restrict__ wr,
                                                          const float* __restrict__ sg, int E,
                                                          int H, int Epad,
                                                          uint16_t* __restrict__ out) {
  const int64_t n = (int64_t)Epad * H;
  const int64_t plane = n;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int e = (int)(i / H);
    const int h = (int)(i - (int64_t)e * H);
    float w = 0.f;
    if (e < E)
      w = wr[(int64_t)e * H + h];
    else if (e == E && sg != nullptr)
      w = sg[h];
    const uint32_t u1 = __float_as_uint(w) & 0xffff0000u;  // top 8 significant bits
    const float r1 = w - __uint_as_float(u1);                // exact
    const uint32_t u2 = __float_as_uint(r1) & 0xffff0000u;  // next 8
    const float r2 = r1 - __uint_as_float(u2);               // exact, <= 8 bits left
    const uint32_t u3 = __float_as_uint(r2) >> 16;           // r2 fits bf16 exactly
    out[i] = (uint16_t)(u1 >> 16);
    out[plane + i] = (uint16_t)(u2 >> 16);
    out[2 * plane + i] = (uint16_t)u3;
  }
}

// (value, index) order used by the selection: larger value first, then the
// lower index. idx < 0 marks "nothing".
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  if (ia < 0) return false;
  if (ib < 0) return true;
  return va > vb || (va == vb && ia < ib);
}

template <int MAXN>
__global__ __launch_bounds__(256) void router_topk_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ split,
    const float* __restrict__ bias, int T, int H, int E, int Epad, int k, int has_shared,
    float* __restrict__ logits_out, int32_t* __restrict__ ids_out, float* __restrict__ w_out,
    float* __restrict__ sw_out) {
  constexpr int MSUB = kRouteRows / 16;
  __shared__ float s_log[kRouteRows][272 + 1];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int NT = Epad / 16;
  const int t0 = blockIdx.x * kRouteRows;
  const int64_t plane = (int64_t)Epad * H;

  f32x4 acc[MSUB][MAXN];
#pragma unroll
  for (int m = 0; m < MSUB; ++m)
#pragma unroll
    for (int i = 0; i < MAXN; ++i) acc[m][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int kq = 8 * (lane >> 4);  // this lane's 8-wide K slot within a 32-step
  const int r16 = lane & 15;

  for (int kb = 0; kb < H; kb += 32) {
    bf16x8 a[MSUB];
#pragma unroll
    for (int m = 0; m < MSUB; ++m) {
      const int row = t0 + m * 16 + r16;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row < T) v = ld16(x + (int64_t)row * H + kb + kq);
      a[m] = __builtin_bit_cast(bf16x8, v);
    }
#pragma unroll
    for (int i = 0; i < MAXN; ++i) {
      const int n = wave + 4 * i;
      if (n < NT) {
        const uint16_t* bp = split + (int64_t)(n * 16 + r16) * H + kb + kq;
#pragma unroll
        for (int s = 0; s < 3; ++s) {
          const bf16x8 b = __builtin_bit_cast(bf16x8, ld16(bp + s * plane));
#pragma unroll
          for (int m = 0; m < MSUB; ++m) acc[m][i] = mfma_16x16x32(a[m], b, acc[m][i]);
        }
      }
    }
  }

  // logits tile -> LDS (biased)
#pragma unroll
  for (int i = 0; i < MAXN; ++i) {
    const int n = wave + 4 * i;
    if (n < NT) {
      const int col = n * 16 + r16;
      const float b = (bias != nullptr && col < E) ? bias[col] : 0.f;
#pragma unroll
      for (int m = 0; m < MSUB; ++m)
#pragma unroll
        for (int v = 0; v < 4; ++v) s_log[m * 16 + 4 * (lane >> 4) + v][col] = acc[m][i][v] + b;
    }
  }
  __syncthreads();

  if (logits_out != nullptr) {
    for (int i = tid; i < kRouteRows * E; i += 256) {
      const int r = i / E, c = i - (i / E) * E;
      if (t0 + r < T) logits_out[(int64_t)(t0 + r) * E + c] = s_log[r][c];
    }
  }

  // top-k + softmax: one wave per token, E/64 candidates per lane
  for (int r = wave; r < kRouteRows; r += 4) {
    const int t = t0 + r;
    if (t >= T) break;
    float v[4];
    int id[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      id[q] = e < E ? e : -1;
      v[q] = e < E ? s_log[r][e] : 0.f;
    }
    float sel_v[8];
    int sel_i[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j >= k) break;
      float bv = 0.f;
      int bi = -1;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (better(v[q], id[q], bv, bi)) { bv = v[q]; bi = id[q]; }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
      }
      sel_v[j] = bv;
      sel_i[j] = bi;
      // retire the winner from its owner lane
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (id[q] == bi) id[q] = -1;
    }
    if (lane == 0) {
      const float m = sel_v[0];
      float ex[8];
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j >= k) break;
        ex[j] = expf(sel_v[j] - m);
        sum += ex[j];
      }
      const float inv = 1.f / sum;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j >= k) break;
        ids_out[(int64_t)t * k + j] = sel_i[j];
        w_out[(int64_t)t * k + j] = ex[j] * inv;
      }
      if (has_shared) sw_out[t] = 1.f / (1.f + expf(-s_log[r][E]));
    }
  }
}

}  // namespace

int router_padded_rows(int E, bool has_shared) { return cdiv(E + (has_shared ? 1 : 0), 16) * 16; }

size_t router_split_bytes(int E, bool has_shared, int H) {
  return (size_t)3 * router_padded_rows(E, has_shared) * H * sizeof(uint16_t);
}

hipError_t launch_router_split(const float* w_router, const float* shared_gate, int E, int H,
                               uint16_t* split, hipStream_t s) {
  const int Epad = router_padded_rows(E, shared_gate != nullptr);
  const int64_t n = (int64_t)Epad * H;
  int blocks = (int)((n + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  LaunchScope ls("router_split", s);
  hipLaunchKernelGGL(router_split_kernel, dim3(blocks), dim3(256), 0, s, w_router, shared_gate, E,
                     H, Epad, split);
  return hipGetLastError();
}

hipError_t launch_router_topk(const uint16_t* x, const uint16_t* split, const float* bias, int T,
                              int H, int E, int k, bool has_shared, float* logits, int32_t* ids,
                              float* topk_w, float* shared_w, hipStream_t s) {
  const int Epad = router_padded_rows(E, has_shared);
  const int NT = Epad / 16;
  const int maxn = cdiv(NT, 4);
  const dim3 grid(cdiv(T, kRouteRows)), block(256);
  LaunchScope ls("router_topk", s);
#define QMOE_ROUTE_CASE(NN)                                                                    \
  case NN:                                                                                     \
    hipLaunchKernelGGL(router_topk_kernel<NN>, grid, block, 0, s, x, split, bias, T, H, E, Epad, \
                       k, has_shared ? 1 : 0, logits, ids, topk_w, shared_w);                  \
    break;
  switch (maxn) {
    QMOE_ROUTE_CASE(1)
    QMOE_ROUTE_CASE(2)
    QMOE_ROUTE_CASE(3)
    QMOE_ROUTE_CASE(4)
    QMOE_ROUTE_CASE(5)
    default:
      return hipErrorInvalidValue;
  }
#undef QMOE_ROUTE_CASE
  return hipGetLastError();
}

}  // namespace qmoe
