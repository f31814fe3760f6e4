// Device code of the router shared by the router kernels and the fused
// small-batch layer kernel: the top-k and softmax of one token's logits
// (16 lanes per token) and one router row's fp32 products with a few tokens.
#pragma once

#include "common.h"
#include "kernels.h"

namespace qmoe {

// DPP row patterns: after xor-1, xor-2 (quad_perm), half-mirror and mirror
// exchanges every lane of a 16-lane row has combined all 16 lanes.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
  const int lo = dpp<CTRL>((int)(uint32_t)v);
  const int hi = dpp<CTRL>((int)(uint32_t)(v >> 32));
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

template <int CTRL>
__device__ __forceinline__ float sum_step(float x) {
  return x + __int_as_float(dpp<CTRL>(__float_as_int(x)));
}

// 16 lanes per token (16 tokens per 256-thread workgroup). Lane r holds the
// logits of experts 64*i + 4*r + c (i < Q/4, c < 4). The selection order is
// the larger logit first, then the lower expert index; each of the k rounds
// takes the lane-local best, reduces it over the row with DPP exchanges and
// retires the winner; lane j keeps round j's winner for the softmax.
// Logits, top-k and softmax of token t (16 lanes per token: lane r of the
// group); the selected ids also go to lds_ids[t * k + j] if it is given.
// P holds ksplit (at most kRouterMaxKsplit) planes [T][Epad] of partial sums
// over slices of K, added in plane order.
template <int Q>
__device__ __forceinline__ void select_token(
    const float* __restrict__ P, int ksplit, int T, int E, int Epad, int k,
    const float* __restrict__ bias, int has_shared, float* __restrict__ logits_out,
    int32_t* __restrict__ ids_out, float* __restrict__ w_out, float* __restrict__ sw_out, int t,
    int32_t* lds_ids, float* lds_w = nullptr, float* lds_sw = nullptr) {
  // (any of the global outputs may be null; the LDS copies go where given)
  auto put_sw = [&](float v) {
    if (sw_out != nullptr) sw_out[t] = v;
    if (lds_sw != nullptr) lds_sw[t] = v;
  };
  const int r = threadIdx.x & 15;
  const bool live = t < T;
  const int tt = live ? t : T - 1;
  const int64_t plane = (int64_t)T * Epad;

  float v[Q];
#pragma unroll
  for (int i = 0; i < Q / 4; ++i) {
    const int e0 = 64 * i + 4 * r;
    f32x4 l = {0.f, 0.f, 0.f, 0.f};
    if (e0 < Epad) {
      // every plane's load in flight at once, then the sum in plane order
      const float* p = P + (int64_t)tt * Epad + e0;
      f32x4 pl[kRouterMaxKsplit];
#pragma unroll
      for (int s = 0; s < kRouterMaxKsplit; ++s)
        if (s < ksplit) pl[s] = *reinterpret_cast<const f32x4*>(p + s * plane);
      l = pl[0];
#pragma unroll
      for (int s = 1; s < kRouterMaxKsplit; ++s)
        if (s < ksplit) l += pl[s];
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = e0 + c;
      float x = l[c];
      if (e < E) {
        if (bias != nullptr) x += bias[e];
        if (logits_out != nullptr && live) logits_out[(int64_t)t * E + e] = x;
      } else if (e == E && has_shared && live) {
        put_sw(1.f / (1.f + expf(-x)));
      }
      v[4 * i + c] = x;
    }
  }
  // the shared-gate column past the last lane's range (E a multiple of 64)
  if (has_shared && E >= 16 * Q && r == 0 && live) {
    const float* p = P + (int64_t)tt * Epad + E;
    float pl[kRouterMaxKsplit];
#pragma unroll
    for (int s = 0; s < kRouterMaxKsplit; ++s)
      if (s < ksplit) pl[s] = p[s * plane];
    float x = pl[0];
#pragma unroll
    for (int s = 1; s < kRouterMaxKsplit; ++s)
      if (s < ksplit) x += pl[s];
    put_sw(1.f / (1.f + expf(-x)));
  }

  // Each candidate as one 64-bit key whose unsigned order is the selection
  // order: the logit's bits mapped to an order-preserving integer (-0.0
  // made +0.0 first, so the two compare equal), then 0xffff - e, so that of
  // equal logits the lower expert index wins. 0 marks "nothing" (every
  // finite logit maps above it). Each round takes the largest key of the
  // lane, reduces it over the row with DPP exchanges (unique keys: every lane
  // ends with the same winner) and clears it where it came from.
  uint64_t kq[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int e = 64 * (q >> 2) + 4 * r + (q & 3);
    uint32_t b = __float_as_uint(v[q] + 0.0f);
    b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    kq[q] = e < E ? ((uint64_t)b << 32) | (uint32_t)(0xffff - e) : 0ull;
  }
  auto kmax = [](uint64_t a, uint64_t b) { return a > b ? a : b; };
  uint64_t best0 = 0, selk = 0;
  for (int j = 0; j < k; ++j) {
    uint64_t bk = kq[0];
#pragma unroll
    for (int q = 1; q < Q; ++q) bk = kmax(bk, kq[q]);
    bk = kmax(bk, dpp64<kDppXor1>(bk));
    bk = kmax(bk, dpp64<kDppXor2>(bk));
    bk = kmax(bk, dpp64<kDppHalfMirror>(bk));
    bk = kmax(bk, dpp64<kDppMirror>(bk));
    if (j == 0) best0 = bk;
    if (r == j) selk = bk;
#pragma unroll
    for (int q = 0; q < Q; ++q) kq[q] = kq[q] == bk ? 0ull : kq[q];
  }
  // back to the logit and the expert index
  auto key_value = [](uint64_t kk) {
    const uint32_t b = (uint32_t)(kk >> 32);
    return __uint_as_float((b & 0x80000000u) ? (b & 0x7fffffffu) : ~b);
  };
  const float m0 = key_value(best0), selv = key_value(selk);
  const int seli = 0xffff - (int)(uint32_t)(selk & 0xffffu);
  // softmax over the k winners (the largest is round 0's)
  const float ex = r < k ? expf(selv - m0) : 0.f;
  float sum = sum_step<kDppXor1>(ex);
  sum = sum_step<kDppXor2>(sum);
  sum = sum_step<kDppHalfMirror>(sum);
  sum = sum_step<kDppMirror>(sum);
  if (live && r < k) {
    const float wt = ex * (1.f / sum);
    if (ids_out != nullptr) ids_out[(int64_t)t * k + r] = seli;
    if (w_out != nullptr) w_out[(int64_t)t * k + r] = wt;
    if (lds_ids != nullptr) lds_ids[t * k + r] = seli;
    if (lds_w != nullptr) lds_w[t * k + r] = wt;
  }
}

// L[t][n] = sum_h f32(x[t][h]) * w[n][h] for the E router rows and the
// shared-gate row (n = E), T <= kRouterGemvT tokens. One workgroup per row
// n; wave w takes the K quarter [w H/4, (w + 1) H/4), lane l the values 8 l
// .. 8 l + 7 of every 512-wide piece of it, reading the fp32 row and every
// token's bf16 values straight from memory. The per-lane sums are reduced
// across the wave, then across the four waves, in a fixed order.
// (256 threads; part: LDS scratch of the four waves' sums)
__device__ __forceinline__ void router_row(const uint16_t* __restrict__ x,
                                           const float* __restrict__ wr,
                                           const float* __restrict__ sg, int T, int H, int E,
                                           int Epad, int n, float* __restrict__ out,
                                           float (*part)[kRouterGemvT]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rows = E + (sg != nullptr ? 1 : 0);
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc((void*)x, 0, T * H * 2, kRsrcWord3);
  float acc[kRouterGemvT];
#pragma unroll
  for (int t = 0; t < kRouterGemvT; ++t) acc[t] = 0.f;
  if (n < rows) {
    const float* wrow = n < E ? wr + (int64_t)n * H : sg;  // n == E: the shared gate
    const int kq = H / 4;
    for (int c = 0; c < kq; c += 512) {
      const int k = wave * kq + c + 8 * lane;
      if (c + 8 * lane < kq) {
        const f32x4 w0 = *reinterpret_cast<const f32x4*>(wrow + k);
        const f32x4 w1 = *reinterpret_cast<const f32x4*>(wrow + k + 4);
        u32x4 xv[kRouterGemvT];
#pragma unroll
        for (int t = 0; t < kRouterGemvT; ++t) {
          // past the last token: past the end of x, which reads zero
          const uint32_t off = t < T ? (uint32_t)(t * H + k) * 2u : 0x7ffffff0u;
          xv[t] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
        }
#pragma unroll
        for (int t = 0; t < kRouterGemvT; ++t) {
          float a = acc[t];
          a = fmaf(bf16lo(xv[t][0]), w0[0], a);
          a = fmaf(bf16hi(xv[t][0]), w0[1], a);
          a = fmaf(bf16lo(xv[t][1]), w0[2], a);
          a = fmaf(bf16hi(xv[t][1]), w0[3], a);
          a = fmaf(bf16lo(xv[t][2]), w1[0], a);
          a = fmaf(bf16hi(xv[t][2]), w1[1], a);
          a = fmaf(bf16lo(xv[t][3]), w1[2], a);
          a = fmaf(bf16hi(xv[t][3]), w1[3], a);
          acc[t] = a;
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kRouterGemvT; ++t) acc[t] = wave_sum(acc[t]);
  if (lane == 0) {
#pragma unroll
    for (int t = 0; t < kRouterGemvT; ++t) part[wave][t] = acc[t];
  }
  __syncthreads();
  if (tid < T) out[(int64_t)tid * Epad + n] = ((part[0][tid] + part[1][tid]) + part[2][tid]) + part[3][tid];
}

}  // namespace qmoe
