// The MoE layer for a few tokens (at most 16) on gfx950 in four launches.
//
// With so few tokens every step is short and the layer is bound by reading
// the active experts' packed weights once, plus one launch and ramp-up per
// step. The steps:
//
//   router_gemv       fp32 router logits, one workgroup per router row
//                     (route.hip)
//   small_gateup      every workgroup first computes top-k, softmax and the
//                     grouping of all tokens in LDS itself (a few
//                     microseconds repeated by every workgroup instead of a
//                     launch of its own), then its share of the gate/up items
//                     of the routed and the shared expert; workgroup 0 also
//                     writes the grouping for the launches after it
//   small_down        the down items of the routed and the shared expert
//   combine           (elementwise.hip)
//
// The work items are those of the weight-streaming kernels (stream_impl.h):
// the same products, grouping order and combine order as the separate
// small-batch kernels, so the output is the same, bit for bit.
//
// (One persistent launch for the whole layer, with the steps handed out as
// tickets and release/acquire counters between them, was built and measured:
// on MI355X every agent-scope release writes back and every acquire
// invalidates an XCD's whole L2, and with one per work item the layer took
// 4-7x longer than separate launches, whose boundaries do that once.)
#include "permute_impl.h"  // PMAXE, expert_scan
#include "select_impl.h"
#include "stream_impl.h"

namespace qmoe {

namespace {

// Top-k, softmax and grouping of all T tokens into LDS, as the routing and
// permutation kernels compute them: s_ids / s_tw / s_sw the selection,
// s_inv[p] the sorted row of pair p, s_tok[r] the token of sorted row r, and
// the list of experts with rows (s_grp / s_rows / s_row0, n_act of them),
// then the shared expert (rows 0..T-1 of its own buffers) if any.
template <int Q>
__device__ __forceinline__ int small_list(const SmallLayer& a, int32_t* s_ids, float* s_tw,
                                          float* s_sw, int* s_inv, int* s_tok, int* s_tok_sh,
                                          int* s_grp, int* s_rows, int* s_row0, int* s_off,
                                          int* s_cnt, int* s_cnt_e, int* s_cnt_w0, int* s_wave,
                                          int32_t* g_counts, int32_t* g_offsets) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = a.T, k = a.k, E = a.E, P = T * k;
  if (tid < PMAXE) {
    s_cnt_e[tid] = 0;
    s_cnt_w0[tid] = 0;
  }
  select_token<Q>(a.logits, 1, T, E, a.Epad, k, a.bias, a.has_shared, nullptr, nullptr,
                  nullptr, nullptr, tid >> 4, s_ids, s_tw, s_sw);
  __syncthreads();
  // The grouping of the pairs by expert, stable (pair order within an
  // expert), as the permutation kernels compute it. At most 128 pairs, in
  // waves 0 and 1: per-expert counts by LDS atomic adds (the totals do not
  // depend on their order), offsets by a scan over the experts, and each
  // pair's rank among the earlier pairs of its expert from one ballot per
  // id bit (the lanes of its wave with the same id) plus, in wave 1, wave
  // 0's count of that id.
  int e = -1;
  if (tid < P) {
    e = s_ids[tid];
    atomicAdd(&s_cnt_e[e], 1);
    if (wave == 0) atomicAdd(&s_cnt_w0[e], 1);
  }
  uint64_t same = __ballot(tid < P);
  for (int bit = 0; bit < a.nbits; ++bit) {
    const bool on = tid < P && ((e >> bit) & 1);
    const uint64_t bb = __ballot(on);
    same &= on ? bb : ~bb;
  }
  const int rank = lanes_below(same);
  __syncthreads();
  const int total = tid < E ? s_cnt_e[tid] : 0;
  const int off = expert_scan(total, s_wave);
  if (tid < E) {
    s_off[tid] = off;
    if (g_counts != nullptr) {
      g_counts[tid] = total;
      g_offsets[tid] = off;
      if (tid == E - 1) g_offsets[E] = off + total;
    }
  }
  __syncthreads();
  if (tid < P) {
    const int pos = s_off[e] + (wave == 1 ? s_cnt_w0[e] : 0) + rank;
    s_inv[tid] = pos;
    s_tok[pos] = tid / k;
  }
  // the experts with rows, in expert order (as the streaming kernel lists
  // them), then the shared expert
  const int c = tid < E ? total : 0;
  const uint64_t m = __ballot(c > 0);
  if (lane == 0) s_cnt[wave] = __popcll(m);
  __syncthreads();
  int base = 0, n_act = 0;
#pragma unroll
  for (int w = 0; w < SWAVES; ++w) {
    const int cw = s_cnt[w];
    base += w < wave ? cw : 0;
    n_act += cw;
  }
  if (c > 0) {
    const int i = base + lanes_below(m);
    s_grp[i] = tid;
    s_rows[i] = c;
    s_row0[i] = off;
  }
  if (tid == 0 && a.has_shared) {
    s_grp[n_act] = 0;
    s_rows[n_act] = T;
    s_row0[n_act] = 0;
  }
  if (tid < kRouterGemvT) s_tok_sh[tid] = tid;
  __syncthreads();
  return n_act;
}

// Q: logits per lane of the selection (16 lanes per token), E <= 16 Q
template <bool ASYM, int G, int NSG, int Q>
__global__ __launch_bounds__(STHREADS, 2) void small_gateup_kernel(SmallLayer a) {
  constexpr int NFG = NSG == 1 ? 4 : 2;  // fragments per item (as the streaming tiling)
  __shared__ __attribute__((aligned(16))) float red[SWAVES][NFG][4][64];
  __shared__ int s_grp[SMAXG + 1], s_rows[SMAXG + 1], s_row0[SMAXG + 1];
  __shared__ int s_tok[STHREADS];         // token of every sorted pair row
  __shared__ int s_tok_sh[kRouterGemvT];  // shared expert: row t is token t
  __shared__ __attribute__((aligned(16))) int32_t s_ids[kRouterGemvT * 8];
  __shared__ float s_tw[kRouterGemvT * 8], s_sw[kRouterGemvT];
  __shared__ int s_inv[kRouterGemvT * 8];
  __shared__ int s_off[PMAXE], s_cnt_e[PMAXE], s_cnt_w0[PMAXE];
  __shared__ int s_cnt[SWAVES], s_wave[SWAVES];

  const int tid = threadIdx.x;
  const bool first = blockIdx.x == 0;
  const int n_act = small_list<Q>(a, s_ids, s_tw, s_sw, s_inv, s_tok, s_tok_sh, s_grp, s_rows,
                                  s_row0, s_off, s_cnt, s_cnt_e, s_cnt_w0, s_wave,
                                  first ? a.counts : nullptr, a.offsets);
  const int T = a.T, k = a.k, P = T * k;
  if (first) {
    // the selection and grouping for the down and combine launches
    if (tid < P) {
      a.ids[tid] = s_ids[tid];
      a.tw[tid] = s_tw[tid];
      a.inv[tid] = s_inv[tid];
      a.sorted[s_inv[tid]] = tid;
    }
    if (a.has_shared && tid < T) a.sw[tid] = s_sw[tid];
  }
  const int n_cb = a.I / (8 * NFG);  // gate/up items per expert (8 NF h columns each)
  const int nR = n_act * n_cb;
  const int nG = (n_act + a.has_shared) * n_cb;
  const int i0 = (int)((int64_t)nG * blockIdx.x / gridDim.x);
  const int i1 = (int)((int64_t)nG * (blockIdx.x + 1) / gridDim.x);
  GroupedGemm g{};
  g.A = a.x;
  g.a_bf16 = true;
  g.a_rows = T;
  g.W = a.w13;
  g.Wscale = a.w13_scale;
  g.Wmin = a.w13_min;
  g.N = 2 * a.I;
  g.K = a.H;
  g.C = a.h;
  g.ldc = a.I;
  g.w_tiled = a.w_tiled;
  stream_items<true, ASYM, NSG, NFG, G>(g, a.E, n_cb, i0, min(i1, nR), s_grp, s_rows, s_row0,
                                        s_tok, red);
  if (a.has_shared) {
    g.W = a.s13;
    g.Wscale = a.s13_scale;
    g.Wmin = a.s13_min;
    g.C = a.hs;
    stream_items<true, ASYM, NSG, NFG, G>(g, 1, n_cb, max(i0, nR), i1, s_grp, s_rows, s_row0,
                                          s_tok_sh, red);
  }
}

// The down items of the routed experts (grouping from the gate/up launch)
// and of the shared expert.
template <bool ASYM, int G, int NSD>
__global__ __launch_bounds__(STHREADS, 2) void small_down_kernel(SmallLayer a) {
  constexpr int NFD = NSD == 1 ? 4 : 2;
  __shared__ __attribute__((aligned(16))) float red[SWAVES][NFD][4][64];
  __shared__ int s_grp[SMAXG + 1], s_rows[SMAXG + 1], s_row0[SMAXG + 1];
  __shared__ int s_cnt[SWAVES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int E = a.E, T = a.T;
  const int c = tid < E ? a.counts[tid] : 0;
  const int o = tid < E ? a.offsets[tid] : 0;
  const uint64_t m = __ballot(c > 0);
  if (lane == 0) s_cnt[wave] = __popcll(m);
  __syncthreads();
  int base = 0, n_act = 0;
#pragma unroll
  for (int w = 0; w < SWAVES; ++w) {
    const int cw = s_cnt[w];
    base += w < wave ? cw : 0;
    n_act += cw;
  }
  if (c > 0) {
    const int i = base + lanes_below(m);
    s_grp[i] = tid;
    s_rows[i] = c;
    s_row0[i] = o;
  }
  if (tid == 0 && a.has_shared) {
    s_grp[n_act] = 0;
    s_rows[n_act] = T;
    s_row0[n_act] = 0;
  }
  __syncthreads();
  const int n_cb = a.H / (16 * NFD);  // down items per expert (16 NF y columns each)
  const int nR = n_act * n_cb;
  const int nD = (n_act + a.has_shared) * n_cb;
  const int i0 = (int)((int64_t)nD * blockIdx.x / gridDim.x);
  const int i1 = (int)((int64_t)nD * (blockIdx.x + 1) / gridDim.x);
  GroupedGemm d{};
  d.A = a.h;
  d.a_bf16 = false;
  d.a_rows = T * a.k;
  d.W = a.w2;
  d.Wscale = a.w2_scale;
  d.Wmin = a.w2_min;
  d.N = a.H;
  d.K = a.I;
  d.C = a.yperm;
  d.ldc = a.H;
  d.w_tiled = a.w_tiled;
  stream_items<false, ASYM, NSD, NFD, G>(d, E, n_cb, i0, min(i1, nR), s_grp, s_rows, s_row0,
                                         nullptr, red);
  if (a.has_shared) {
    d.A = a.hs;
    d.a_rows = T;
    d.W = a.s2;
    d.Wscale = a.s2_scale;
    d.Wmin = a.s2_min;
    d.C = a.ysh;
    stream_items<false, ASYM, NSD, NFD, G>(d, 1, n_cb, max(i0, nR), i1, s_grp, s_rows, s_row0,
                                           nullptr, red);
  }
}

// resident workgroups per CU of one instance (cached; at least one)
template <typename Kern>
int small_resident(Kern kern) {
  static int cached = 0;
  if (cached == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, STHREADS, 0) != hipSuccess || n < 1)
      n = 1;
    cached = n;
  }
  return cached;
}

int g_small_cus = 0;

hipError_t small_cus() {
  if (g_small_cus != 0) return hipSuccess;
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  return hipDeviceGetAttribute(&g_small_cus, hipDeviceAttributeMultiprocessorCount, dev);
}

// a persistent grid of at most as many workgroups as the CUs hold at once,
// and no more than there can be items
template <typename Kern>
int small_grid(Kern kern, int64_t bound) {
  const int64_t cap = (int64_t)small_resident(kern) * g_small_cus;
  return (int)(bound < cap ? bound : cap);
}

template <bool ASYM, int G, int NSG, int NSD>
hipError_t launch_small_inst(const SmallLayer& a, hipStream_t s) {
  hipError_t e = small_cus();
  if (e != hipSuccess) return e;
  const int slots = (a.E < a.T * a.k ? a.E : a.T * a.k) + a.has_shared;
  {
    constexpr int NFG = NSG == 1 ? 4 : 2;
    LaunchScope ls("gateup_gemm", s);
    // (8 logits per selection lane cover E <= 128, 16 E <= 256: each round
    // of the top-k costs in proportion)
    if (a.E <= 128) {
      auto kern = small_gateup_kernel<ASYM, G, NSG, 8>;
      hipLaunchKernelGGL(kern, dim3(small_grid(kern, (int64_t)slots * (a.I / (8 * NFG)))),
                         dim3(STHREADS), 0, s, a);
    } else {
      auto kern = small_gateup_kernel<ASYM, G, NSG, 16>;
      hipLaunchKernelGGL(kern, dim3(small_grid(kern, (int64_t)slots * (a.I / (8 * NFG)))),
                         dim3(STHREADS), 0, s, a);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  constexpr int NFD = NSD == 1 ? 4 : 2;
  LaunchScope ls("down_gemm", s);
  auto kern = small_down_kernel<ASYM, G, NSD>;
  hipLaunchKernelGGL(kern, dim3(small_grid(kern, (int64_t)slots * (a.H / (16 * NFD)))),
                     dim3(STHREADS), 0, s, a);
  return hipGetLastError();
}

// 128-wide K blocks per wave of the streaming tiling for a K (as
// stream_tiling in ffn_stream.hip)
int small_ns(int K) {
  const int nk = K / SBK;
  return nk <= 4 ? 1 : nk <= 8 ? 2 : 4;
}

template <bool ASYM, int G>
hipError_t launch_small_g(const SmallLayer& a, int nsg, int nsd, hipStream_t s) {
  if (nsg == 4 && nsd == 2) return launch_small_inst<ASYM, G, 4, 2>(a, s);
  if (nsg == 4 && nsd == 1) return launch_small_inst<ASYM, G, 4, 1>(a, s);
  return launch_small_inst<ASYM, G, 1, 1>(a, s);
}

}  // namespace

bool small_layer_supported(int T, int H, int I, int Is, int E, int k, int G) {
  if (T < 1 || T > kRouterGemvT || k < 1 || k > 8 || E < 1 || E > SMAXG) return false;
  if (G != 32 && G != 128) return false;
  if (Is != 0 && Is != I) return false;
  if (H % SBK != 0 || I % SBK != 0 || H / SBK > 16 || I / SBK > 16) return false;
  const int nsg = small_ns(H), nsd = small_ns(I);
  if (!((nsg == 4 && nsd == 2) || (nsg == 4 && nsd == 1) || (nsg == 1 && nsd == 1))) return false;
  const int nfg = nsg == 1 ? 4 : 2, nfd = nsd == 1 ? 4 : 2;
  return I % (8 * nfg) == 0 && H % (16 * nfd) == 0;
}

hipError_t launch_small_experts(const SmallLayer& a, hipStream_t s) {
  if (!small_layer_supported(a.T, a.H, a.I, a.has_shared ? a.I : 0, a.E, a.k, a.G))
    return hipErrorInvalidValue;
  const int nsg = small_ns(a.H), nsd = small_ns(a.I);
  const bool asym = a.w13_min != nullptr;
  if (a.G == 32)
    return asym ? launch_small_g<true, 32>(a, nsg, nsd, s) : launch_small_g<false, 32>(a, nsg, nsd, s);
  return asym ? launch_small_g<true, 128>(a, nsg, nsd, s) : launch_small_g<false, 128>(a, nsg, nsd, s);
}

}  // namespace qmoe
