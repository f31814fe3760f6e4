// Weight-streaming expert GEMMs for the MoE layer when each expert gets only
// a handful of rows (prefill of a few tokens: the weight-streaming end of the
// MoE prefill route, where the layer is bound by reading the active experts'
// packed weights once). Same operation, formats and operand layout as the
// tiled expert GEMM (ffn.hip); different work split:
//
//  - work items are (group with rows, block of output columns), listed group
//    by group; a persistent grid (two workgroups per CU) gives each
//    workgroup a contiguous range of items, so the items of one workgroup
//    mostly share their group's activation rows;
//  - the four waves split K four ways (wave w takes the 128-wide K stages
//    w, w + 4, ...); each wave holds its share of an item's packed weights
//    in registers and loads those of the item after next while it
//    computes, so a workgroup always has two whole items in flight;
//  - every lane dequantizes its weights in registers as in the tiled kernel
//    and feeds v_mfma_f32_16x16x32_f16. Gate/up (at most 16 tokens): the
//    16 activation rows are simply the tokens, loaded once per workgroup, so
//    no gathered row has to be fetched before the products; each output row
//    of a group then takes the products of its own token. Down: the group's
//    rows of h, 16 at a time (more are walked block by block with the same
//    weights);
//  - the four partial sums meet in LDS in a fixed order (deterministic) and
//    the result leaves as 16-byte row pieces: h = silu(g) * u in kperm chunk
//    order for gate/up, y in natural order for down.
#include <type_traits>

#include "stream_impl.h"

namespace qmoe {

namespace {

int g_stream_cus = 0;

template <bool GATEUP, bool ASYM, int NS, int NF, int G>
__global__ __launch_bounds__(STHREADS, SWG_PER_CU) void expert_stream_kernel(GroupedGemm g,
                                                                             int n_cb) {
  // per-wave partial sums, [wave][fragment][v][lane]: the lanes of one
  // accumulator element are contiguous, so eight consecutive output columns
  // of a row are eight consecutive floats
  __shared__ __attribute__((aligned(16))) float red[SWAVES][NF][4][64];
  __shared__ int s_grp[SMAXG], s_rows[SMAXG], s_row0[SMAXG];
  __shared__ int s_tok[STHREADS];  // gate/up: token of every row (at most 256 rows)
  __shared__ int s_cnt[SWAVES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // ---- the groups with rows, in order, with their rows and first row ----
  int n_act = 1;
  if (g.counts != nullptr) {
    const int c = tid < g.E ? g.counts[tid] : 0;
    const int o = tid < g.E ? g.offsets[tid] : 0;
    const uint64_t m = __ballot(c > 0);
    if (lane == 0) s_cnt[wave] = __popcll(m);
    __syncthreads();
    int base = 0;
    n_act = 0;
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
  } else if (tid == 0) {
    s_grp[0] = 0;
    s_rows[0] = g.rows_single;
    s_row0[0] = 0;
  }
  if (GATEUP) {
    const int n_rows = g.counts != nullptr ? g.max_rows : g.rows_single;
    if (tid < n_rows) s_tok[tid] = g.gather != nullptr ? g.gather[tid] / g.gather_div : tid;
  }
  __syncthreads();
  const int items = n_act * n_cb;
  const int i0 = (int)((int64_t)items * blockIdx.x / gridDim.x);
  const int i1 = (int)((int64_t)items * (blockIdx.x + 1) / gridDim.x);
  if (i0 >= i1) return;

  stream_items<GATEUP, ASYM, NS, NF, G>(g, g.counts != nullptr ? g.E : 1, n_cb, i0, i1, s_grp,
                                        s_rows, s_row0, s_tok, red);
}

// Resident workgroups per CU of one kernel instance (cached; at least one).
template <typename Kern>
int resident_per_cu(Kern kern) {
  static int cached = 0;
  if (cached == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, STHREADS, 0) != hipSuccess || n < 1)
      n = 1;
    cached = n;
  }
  return cached;
}

template <bool GATEUP, bool ASYM, int NS, int NF, int G>
hipError_t launch_stream_inst(const GroupedGemm& g, int n_cb, hipStream_t s) {
  auto kern = expert_stream_kernel<GATEUP, ASYM, NS, NF, G>;
  // items: at most one per (group that could have rows, column block); a
  // persistent grid of as many workgroups as the CUs hold at once
  const int slots = g.counts != nullptr ? min(g.E, g.max_rows) : 1;
  const int64_t bound = (int64_t)slots * n_cb;
  const int64_t cap = (int64_t)resident_per_cu(kern) * g_stream_cus;
  const int wgs = (int)(bound < cap ? bound : cap);
  if (wgs <= 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(wgs), dim3(STHREADS), 0, s, g, n_cb);
  return hipGetLastError();
}

template <bool GATEUP, bool ASYM, int NS, int NF>
hipError_t launch_stream_g(const GroupedGemm& g, int n_cb, hipStream_t s) {
  if (g.G == 32) return launch_stream_inst<GATEUP, ASYM, NS, NF, 32>(g, n_cb, s);
  if (g.G == 64) return launch_stream_inst<GATEUP, ASYM, NS, NF, 64>(g, n_cb, s);
  return launch_stream_inst<GATEUP, ASYM, NS, NF, 128>(g, n_cb, s);
}

template <bool GATEUP, bool ASYM>
hipError_t launch_stream_ns(const GroupedGemm& g, int ns, int n_cb, hipStream_t s) {
  if (g_stream_cus == 0) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    err = hipDeviceGetAttribute(&g_stream_cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
  }
  if (ns == 1) return launch_stream_g<GATEUP, ASYM, 1, 4>(g, n_cb, s);
  if (ns == 2) return launch_stream_g<GATEUP, ASYM, 2, 2>(g, n_cb, s);
  return launch_stream_g<GATEUP, ASYM, 4, 2>(g, n_cb, s);
}

// 128-wide K blocks per wave and 16-column fragments per item for a K
void stream_tiling(int K, int* ns, int* nf) {
  const int nk = K / SBK;
  *ns = nk <= 4 ? 1 : nk <= 8 ? 2 : 4;
  *nf = *ns == 1 ? 4 : 2;
}

}  // namespace

bool stream_supported(const GroupedGemm& g, bool gateup) {
  // K in whole stages, at most 16 of them (four per wave); whole items of
  // columns; at most 256 groups; gate/up: at most 16 tokens and 256 rows
  if (g.K % SBK != 0 || g.K / SBK > 16 || g.E > SMAXG) return false;
  if (g.tier != nullptr || g.slot != nullptr || (g.bits != 0 && g.bits != 4)) return false;
  int ns, nf;
  stream_tiling(g.K, &ns, &nf);
  if (gateup) {
    const int rows = g.counts != nullptr ? g.max_rows : g.rows_single;
    return (g.N / 2) % (8 * nf) == 0 && g.a_rows <= 16 && rows <= STHREADS;
  }
  return g.N % (16 * nf) == 0;
}

hipError_t launch_stream(const GroupedGemm& g, bool gateup, hipStream_t s, const char* name) {
  int ns, nf;
  stream_tiling(g.K, &ns, &nf);
  const int n_cb = gateup ? (g.N / 2) / (8 * nf) : g.N / (16 * nf);
  LaunchScope ls(name, s);
  const bool asym = g.Wmin != nullptr;
  if (gateup)
    return asym ? launch_stream_ns<true, true>(g, ns, n_cb, s)
                : launch_stream_ns<true, false>(g, ns, n_cb, s);
  return asym ? launch_stream_ns<false, true>(g, ns, n_cb, s)
              : launch_stream_ns<false, false>(g, ns, n_cb, s);
}

}  // namespace qmoe
