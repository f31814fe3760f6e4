// Device helpers of the expert grouping (histogram, prefix scan, stable
// ranks), shared by the permutation kernels and the fused small-batch
// routing kernel.
#pragma once

#include "common.h"

namespace qmoe {

constexpr int PT = 256;              // threads per workgroup (4 waves)
constexpr int PSEG = 8;              // 64-pair segments per wave
constexpr int PCH = 4 * PSEG * 64;   // pairs per workgroup (2048)
constexpr int PMAXE = 256;

// number of lanes below this one whose bit is set in m
__device__ __forceinline__ int count_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Ranks of this workgroup's chunk of PCH pairs (chunk c): ev[s] = expert of
// pair p0 + 64 s (-1 if none or out of range), rk[s] = its rank among the
// chunk's pairs of that expert; afterwards cnt[w][e] holds the number of
// pairs of e in the waves before w and the return value, for thread e < E,
// the chunk's total of e. Ends with the workgroup synchronized.
__device__ __forceinline__ int chunk_ranks(const int32_t* __restrict__ ids, int P, int E, int nbits,
                                           int chunk, int (*cnt)[PMAXE], int* ev, int* rk) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < 4 * PMAXE; i += PT) (&cnt[0][0])[i] = 0;
  __syncthreads();

  const int p0 = chunk * PCH + wave * PSEG * 64 + lane;
#pragma unroll
  for (int s = 0; s < PSEG; ++s) {
    const int p = p0 + s * 64;
    int e = p < P ? ids[p] : -1;
    if ((unsigned)e >= (unsigned)E) e = -1;
    ev[s] = e;
  }
  // Segments in pair order. The lanes holding the same expert are found by
  // one ballot per id bit: a lane keeps the lanes that agree with it on
  // every bit. Its rank is the running count of its expert in this wave plus
  // the number of matching lanes below it.
#pragma unroll
  for (int s = 0; s < PSEG; ++s) {
    const int e = ev[s];
    const bool valid = e >= 0;
    uint64_t m = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool set = (e >> bit) & 1;
      const uint64_t bb = __ballot(set);
      m &= set ? bb : ~bb;
    }
    const int below = count_below(m);
    int c = 0;
    if (valid) c = cnt[wave][e];
    // every lane has read before the group's lowest lane writes (LDS
    // operations of one wave complete in order)
    if (valid && below == 0) cnt[wave][e] = c + __popcll(m);
    rk[s] = c + below;
  }
  __syncthreads();
  // exclusive prefix over the waves per expert (E <= PT: one expert per thread)
  int run = 0;
  if (tid < E) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int c = cnt[w][tid];
      cnt[w][tid] = run;
      run += c;
    }
  }
  __syncthreads();
  return run;
}

// Exclusive scan over the experts of `total` (thread e holds expert e's
// total, E <= PT); returns thread e's offset.
__device__ __forceinline__ int expert_scan(int total, int* s_wave) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int incl = total;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  int wbase = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    if (w < wave) wbase += s_wave[w];
  return wbase + incl - total;
}

}  // namespace qmoe
