// Expert grouping of (token, slot) pairs for the MoE prefill route on gfx950:
// histogram, prefix scan and a stable scatter into expert-sorted row blocks
// (the "per-expert buffers" arrangement of the MoE prefill route).
//
// One workgroup per expert scans the whole id list, so the result is
// deterministic and stable (ascending pair index inside each expert) without
// atomics: pass 1 counts, pass 2 derives the expert's offset from all counts
// and compacts its pairs with a block-wide scan of match flags.
#include "common.h"
#include "kernels.h"

namespace qmoe {

namespace {

constexpr int kThreads = 256;
constexpr int kPer = 4;  // ids per thread per sweep (one 16-byte load)

__device__ __forceinline__ void load4(const int32_t* ids, int p, int P, int v[4]) {
  if (p + 3 < P) {
    const u32x4 q = ld16(ids + p);
    v[0] = (int)q[0]; v[1] = (int)q[1]; v[2] = (int)q[2]; v[3] = (int)q[3];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (p + i < P) ? ids[p + i] : -1;
  }
}

__device__ __forceinline__ int block_sum(int v, int* s_red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum_i(v);
  if (lane == 0) s_red[wave] = v;
  __syncthreads();
  const int tot = s_red[0] + s_red[1] + s_red[2] + s_red[3];
  __syncthreads();
  return tot;
}

__global__ __launch_bounds__(kThreads) void permute_count_kernel(const int32_t* __restrict__ ids,
                                                                  int P,
                                                                  int32_t* __restrict__ counts) {
  __shared__ int s_red[4];
  const int e = blockIdx.x;
  int c = 0;
  for (int p = threadIdx.x * kPer; p < P; p += kThreads * kPer) {
    int v[4];
    load4(ids, p, P, v);
    c += (v[0] == e) + (v[1] == e) + (v[2] == e) + (v[3] == e);
  }
  const int tot = block_sum(c, s_red);
  if (threadIdx.x == 0) counts[e] = tot;
}

__global__ __launch_bounds__(kThreads) void permute_scatter_kernel(
    const int32_t* __restrict__ ids, int P, int E, const int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pairs,
    int32_t* __restrict__ inv) {
  __shared__ int s_red[4];
  __shared__ int s_wave[4];
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  int part = 0;
  for (int i = tid; i < e; i += kThreads) part += counts[i];
  const int base = block_sum(part, s_red);
  if (tid == 0) {
    offsets[e] = base;
    if (e == E - 1) offsets[E] = base + counts[e];
  }

  int running = 0;
  for (int p0 = 0; p0 < P; p0 += kThreads * kPer) {
    const int p = p0 + tid * kPer;
    int v[4];
    load4(ids, p, P, v);
    const int f0 = v[0] == e, f1 = v[1] == e, f2 = v[2] == e, f3 = v[3] == e;
    const int n = f0 + f1 + f2 + f3;
    // inclusive scan of n across the wave
    int incl = n;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    int wbase = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int c = s_wave[w];
      if (w < wave) wbase += c;
      tot += c;
    }
    __syncthreads();
    int pos = base + running + wbase + incl - n;
    if (f0) { sorted_pairs[pos] = p;     inv[p] = pos;     ++pos; }
    if (f1) { sorted_pairs[pos] = p + 1; inv[p + 1] = pos; ++pos; }
    if (f2) { sorted_pairs[pos] = p + 2; inv[p + 2] = pos; ++pos; }
    if (f3) { sorted_pairs[pos] = p + 3; inv[p + 3] = pos; ++pos; }
    running += tot;
  }
}

}  // namespace

hipError_t launch_permute(const int32_t* ids, int P, int E, int32_t* counts, int32_t* offsets,
                          int32_t* sorted_pairs, int32_t* inv, hipStream_t s) {
  {
    LaunchScope ls("permute_count", s);
    hipLaunchKernelGGL(permute_count_kernel, dim3(E), dim3(kThreads), 0, s, ids, P, counts);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  LaunchScope ls("permute_scatter", s);
  hipLaunchKernelGGL(permute_scatter_kernel, dim3(E), dim3(kThreads), 0, s, ids, P, E, counts,
                     offsets, sorted_pairs, inv);
  return hipGetLastError();
}

}  // namespace qmoe
