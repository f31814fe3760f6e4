// Expert grouping of (token, slot) pairs for the MoE prefill route on gfx950:
// histogram, prefix scan and a stable scatter into expert-sorted row blocks
// (the "per-expert buffers" arrangement of the MoE prefill route).
//
// Deterministic and stable (ascending pair index inside each expert), with
// no global atomics, in two passes over the id list:
//  permute_rank   : each workgroup takes a chunk of PCH consecutive pairs and
//                   gives every pair its rank among the chunk's pairs of the
//                   same expert (wavefront match with one ballot per id bit,
//                   then a prefix over the waves); writes the rank to inv[p]
//                   and the chunk's per-expert histogram
//  permute_scatter: each workgroup sums the histograms (all chunks: counts
//                   and offsets; earlier chunks: its own base per expert) and
//                   writes sorted_pairs[base + rank] = p, inv[p] = that position
//  permute_small  : at most one chunk of pairs: both passes in one workgroup
//                   (the ranks stay in registers, the scan over the experts in
//                   LDS), one launch
#include "common.h"
#include "kernels.h"
#include "permute_impl.h"

namespace qmoe {

namespace {

__global__ __launch_bounds__(PT) void permute_rank_kernel(const int32_t* __restrict__ ids, int P,
                                                          int E, int nbits,
                                                          int32_t* __restrict__ hist,
                                                          int32_t* __restrict__ rank_out) {
  __shared__ int cnt[4][PMAXE];
  const int tid = threadIdx.x, wave = tid >> 6;
  int ev[PSEG], rk[PSEG];
  const int total = chunk_ranks(ids, P, E, nbits, blockIdx.x, cnt, ev, rk);
  if (tid < E) hist[(int64_t)blockIdx.x * E + tid] = total;
  const int p0 = blockIdx.x * PCH + wave * PSEG * 64 + (tid & 63);
#pragma unroll
  for (int s = 0; s < PSEG; ++s) {
    const int p = p0 + s * 64;
    if (p < P) rank_out[p] = ev[s] >= 0 ? rk[s] + cnt[wave][ev[s]] : 0;
  }
}

__global__ __launch_bounds__(PT) void permute_small_kernel(
    const int32_t* __restrict__ ids, int P, int E, int nbits, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pairs, int32_t* __restrict__ inv) {
  __shared__ int cnt[4][PMAXE];
  __shared__ int s_off[PMAXE];
  __shared__ int s_wave[4];
  const int tid = threadIdx.x, wave = tid >> 6;
  int ev[PSEG], rk[PSEG];
  const int total = chunk_ranks(ids, P, E, nbits, 0, cnt, ev, rk);
  const int off = expert_scan(total, s_wave);
  if (tid < E) {
    counts[tid] = total;
    offsets[tid] = off;
    s_off[tid] = off;
    if (tid == E - 1) offsets[E] = off + total;
  }
  __syncthreads();
  const int p0 = wave * PSEG * 64 + (tid & 63);
#pragma unroll
  for (int s = 0; s < PSEG; ++s) {
    const int p = p0 + s * 64;
    if (p < P) {
      const int e = ev[s];
      if (e >= 0) {
        const int pos = s_off[e] + cnt[wave][e] + rk[s];
        sorted_pairs[pos] = p;
        inv[p] = pos;
      } else {
        inv[p] = 0;
      }
    }
  }
}

__global__ __launch_bounds__(PT) void permute_scatter_kernel(
    const int32_t* __restrict__ ids, int P, int E, const int32_t* __restrict__ hist,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_pairs, int32_t* __restrict__ inv) {
  __shared__ int s_base[PMAXE];
  __shared__ int s_wave[4];
  const int tid = threadIdx.x;
  const int nb = gridDim.x, b = blockIdx.x;

  // one thread per expert (E <= 256 = PT)
  int total = 0, before = 0;
  if (tid < E) {
#pragma unroll 8
    for (int j = 0; j < nb; ++j) {
      const int h = hist[(int64_t)j * E + tid];
      total += h;
      before += j < b ? h : 0;
    }
  }
  const int off = expert_scan(total, s_wave);
  if (tid < E) {
    s_base[tid] = off + before;
    if (b == 0) {
      counts[tid] = total;
      offsets[tid] = off;
      if (tid == E - 1) offsets[E] = off + total;
    }
  }
  __syncthreads();

  // the chunk's ids and ranks are loaded before any is used
  constexpr int PER = PCH / PT;
  int ev[PER], rk[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int p = b * PCH + tid + q * PT;
    ev[q] = p < P ? ids[p] : -1;
    rk[q] = p < P ? inv[p] : 0;
  }
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int p = b * PCH + tid + q * PT;
    if (p < P) {
      const int e = ev[q];
      if ((unsigned)e < (unsigned)E) {
        const int pos = s_base[e] + rk[q];
        sorted_pairs[pos] = p;
        inv[p] = pos;
      } else {
        inv[p] = 0;
      }
    }
  }
}

}  // namespace

int permute_chunks(int P) { return P > 0 ? cdiv(P, PCH) : 1; }

size_t permute_ws_bytes(int P, int E) { return (size_t)permute_chunks(P) * E * sizeof(int32_t); }

hipError_t launch_permute(const int32_t* ids, int P, int E, int32_t* counts, int32_t* offsets,
                          int32_t* sorted_pairs, int32_t* inv, int32_t* hist, hipStream_t s) {
  const int nb = permute_chunks(P);
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  if (nb == 1) {
    LaunchScope ls("permute_rank", s);
    hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(PT), 0, s, ids, P, E, nbits, counts,
                       offsets, sorted_pairs, inv);
    return hipGetLastError();
  }
  {
    LaunchScope ls("permute_rank", s);
    hipLaunchKernelGGL(permute_rank_kernel, dim3(nb), dim3(PT), 0, s, ids, P, E, nbits, hist, inv);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  LaunchScope ls("permute_scatter", s);
  hipLaunchKernelGGL(permute_scatter_kernel, dim3(nb), dim3(PT), 0, s, ids, P, E, hist, counts,
                     offsets, sorted_pairs, inv);
  return hipGetLastError();
}

}  // namespace qmoe
