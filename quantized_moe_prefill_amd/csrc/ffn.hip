// Grouped expert GEMMs for the MoE prefill layer on gfx950.
//
// Rows are processed in expert-sorted blocks ("per-expert buffers" in the
// MoE prefill route of the hipfire 0.4.3 benchmarks page, section "Read this
// before comparing columns"); each expert's weights are 4-bit integers with
// an fp16 scale (and min) per group of G elements along K, as in that page's
// symmetric and asymmetric expert files ("Known limits").
//
// Tile: BM = 128 rows of one expert x BN = 512 weight rows, K in stages of
// 128, one 512-thread workgroup per CU (eight waves, two per SIMD). The
// gathered activation rows go through a three-stage LDS ring (direct
// global->LDS loads, two stages ahead) and are read by all eight waves; each
// wave owns 64 weight rows (four 16-column fragments) across all 128 rows,
// loads its packed weights straight from global memory into registers (16
// bytes = 32 K values per lane per fragment and stage, one stage ahead) and
// dequantizes them in registers, so no weight is dequantized twice and no
// weight touches LDS. v_mfma_f32_16x16x32_f16 with fp32 accumulators; the
// results leave through a per-wave LDS sub-tile as 16-byte row pieces
// (gate/up with 3- or 2-bit weights: straight from the accumulators).
//
// The gate/up kernel pairs gate and up rows of the same intermediate columns
// in one wave, so h = silu(g) * u is formed in registers and written once.
//
// Operands are fp16 rather than bf16: the matrix cores run both at the same
// rate, and fp16's three extra significand bits on the dequantized weights,
// on h and on the expert outputs are what keeps the layer output within its
// error budget. Activations arrive as bf16 and are converted exactly (for
// |x| < 65504) by x_to_f16 before the gate/up GEMM.
//
// Scheduling: persistent workgroups. Each one derives the tile list from the
// per-expert row counts, takes the contiguous range of tiles that belongs to
// its XCD (workgroups are dealt to the 8 XCDs round-robin), and walks it, so
// the N tiles of one row block and the row blocks of one expert run on the
// same XCD and share its L2.
#include <type_traits>

#include "common.h"
#include "dequant.h"
#include "kernels.h"

namespace qmoe {

namespace {

constexpr int BM = 128;          // rows per tile
constexpr int NWAVES = 8;        // waves per workgroup, 64 weight rows each
constexpr int NTHREADS = 64 * NWAVES;
constexpr int BN = 64 * NWAVES;  // weight rows per tile
constexpr int BK = 128;          // K per pipeline stage
constexpr int NXCD = 8;
constexpr int NFRAG = 4;         // 16-column fragments per wave
constexpr int WGS_PER_CU = 1;    // persistent workgroups per CU (two waves per SIMD)
constexpr int ASTAGES = 3;       // activation stages in the LDS ring
constexpr int ALD = 32 / NWAVES; // direct activation loads per wave and stage (4 rows each)
constexpr int A_STAGE_BYTES = BM * BK * 2;
constexpr int SUB_BYTES = BM * 128;  // one wave's epilogue sub-tile (128 rows x 64 fp16)
// (128-row tiles: two sub-tiles fit in each activation stage, an extra
// region holds the rest)
static_assert(A_STAGE_BYTES == 2 * SUB_BYTES && NWAVES > 2 * ASTAGES, "epilogue LDS layout");

// bf16 activations -> fp16 in kperm chunk order (exact for |x| < 65504).
__global__ __launch_bounds__(256) void x_to_f16_kernel(const uint16_t* __restrict__ x,
                                                       uint16_t* __restrict__ out,
                                                       int64_t n_chunks) {
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < n_chunks;
       c += (int64_t)gridDim.x * 256) {
    st16(out + c * 8, bf16x8_to_f16_kperm(ld16(x + c * 8)));
  }
}


// Slot swizzle of the activation tiles: chunk c of row r sits in slot
// c ^ rowswz(r), the row's low four bits with their two halves swapped. A
// fragment read has 16 lanes on 16 consecutive rows and, per group of 16
// lanes, chunk 4*group + step; a plain c ^ (r & 15) leaves it two-way bank
// conflicted on gfx950 (measured with the LDS conflict counter), the swapped
// form is conflict-free.
__device__ __forceinline__ int rowswz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Source rows of n activation rows starting at local row r_first (stride
// r_step) of a tile: rows past the expert's end read the tile's first row
// (finite data whose outputs are never stored). All gathers are issued
// before any is used, so their latencies overlap.
template <int NL>
__device__ __forceinline__ void gather_rows(const GroupedGemm& g, int row0, int rows, int r_first,
                                            int r_step, int* src, bool direct = false) {
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int r = r_first + i * r_step;
    src[i] = row0 + (r < rows ? r : 0);
  }
  if (g.gather != nullptr && !direct) {
#pragma unroll
    for (int i = 0; i < NL; ++i) src[i] = g.gather[src[i]];
    const int div = g.gather_div;
#pragma unroll
    for (int i = 0; i < NL; ++i) src[i] /= div;
  }
}

// The uniform description of one tile: a block of BM sorted rows of one
// expert (or of the extra group) times one N tile. (At namespace scope: a
// class local to a kernel template keeps the compiler from emitting the
// kernel's host-side launch stub.)
struct TileU {
  int row0, rows;  // first sorted row of the block and its valid rows
  int e;           // the expert's index in the weight tensors (0: extra group)
  int shared;      // the tile belongs to the extra group
  int c0;          // this wave's first weight row (gate/up: h column) in it
};

// Scales (and mins) of a tile in LDS: each wave's rows take two 1 KB slots,
// filled by two direct loads per tile instead of one 2-byte load per
// fragment and K stage. Gate/up: slot 0 = the 32 gate rows' scales, slot 1 =
// the 32 up rows' (symmetric only, at most 16 groups per row); down: the 64
// rows' scales over both slots (at most 16 groups per row), or, asymmetric,
// scales in slot 0 and mins in slot 1 (at most 8 groups per row).
constexpr int SC_SLOT = 1024;
constexpr int SC_WAVE = 2 * SC_SLOT;

// How a kernel variant reads the group scales (and mins):
//  - SC_STAGE: one 2-byte load per fragment and K stage;
//  - SC_TILE: the tile's scales through the per-wave LDS tile above;
//  - SC_WINDOW (G = 32): a row's 8 groups of two consecutive K stages are 16
//    contiguous bytes, so one direct 16-byte-per-lane load per wave (lane l
//    = the wave's weight row l) fills a window of two stages for its 64
//    rows: 1 KB of scales in slot 0, 1 KB of mins in slot 1, refilled every
//    other stage, in place of eight 2-byte loads per stage.
constexpr int SC_STAGE = 0, SC_TILE = 1, SC_WINDOW = 2;

// BITS: the weights' width (4; or 3 or 2, symmetric, see dequant.h). A
// lane's 32-element K block of a row is 4 * BITS bytes: one 16-, 12- or
// 8-byte load per fragment and stage. MIX: one group of experts of a
// mixed layer (the expert filter and slot map of GroupedGemm are read).
// TBM: rows per tile, 128, or 64 for layers whose experts get about 64
// rows or fewer (a 128-row tile would be mostly padding there). WT: a mixed
// layer's weights are tiled (a compile-time choice there: the runtime one
// makes the 3-bit gate/up instance spill; the plain instances read
// g.w_tiled).
template <bool GATEUP, bool ASYM, int SCM, bool FOLD, int BITS = 4, bool MIX = false,
          int TBM = 128, bool WT = false>
__global__ __launch_bounds__(NTHREADS, 1) void expert_gemm_kernel(GroupedGemm g, int n_ntiles) {
  static_assert(TBM == 128 || TBM == 64, "tile rows");
  static_assert(TBM / 4 / NWAVES <= 4, "activation loads per wave");
  // this instance's tile height and what follows from it (the names hide
  // the 128-row constants above)
  constexpr int BM = TBM;
  constexpr int MSUB = BM / 16;
  constexpr int ALD = BM / 4 / NWAVES;  // direct activation loads per wave and stage
  constexpr int A_STAGE_BYTES = BM * BK * 2;
  // epilogue: a 4 KB sub-tile per wave, filled and emptied in passes of 64
  // rows x 64 B (h) or 32 rows x 128 B (y)
  constexpr int SUBW = 4096;
  // LDS, two uses:
  //  - K loop: a ring of three activation tiles (As0..As2), BM rows x 128
  //    fp16 each, no padding; the 16-byte chunk c of row r sits in slot
  //    c ^ rowswz(r) (see rowswz), which keeps the fragment reads free of
  //    bank conflicts and lets a direct global->LDS load fill four whole rows.
  //    Separate arrays (and a K loop unrolled by three) let the compiler see
  //    that a stage's LDS reads never touch the tiles still being loaded, so
  //    it does not wait for those loads before reading. The ring runs on
  //    across tiles: a tile's first stage sits in the slot after its
  //    predecessor's last;
  //  - epilogue: each wave's output sub-tile in Ex, which no direct load
  //    ever targets, so that the results leave as 16-byte row pieces while
  //    the next tile's first stages are already landing in the ring.
  __shared__ __attribute__((aligned(16))) uint8_t As0[A_STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t As1[A_STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t As2[A_STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t Ex[NWAVES * SUBW];
  constexpr bool SCL = SCM == SC_TILE;
  constexpr bool WIN = SCM == SC_WINDOW;
  // each stage dequantizes the next stage's first K step (symmetric experts:
  // with a min per group the extra live registers spill)
  constexpr bool XDQ = !ASYM;
  // Gate/up with 3- or 2-bit weights writes h straight from the accumulators
  // (the LDS-staged epilogue below needs registers that the wider dequant of
  // those widths already takes: the 3-bit instance spilled 45 of them and ran
  // 1.4x slower); 4-bit gate/up and every down GEMM stage their results
  // through the LDS, which leaves as whole row spans and measured faster.
  constexpr bool DIRECT = GATEUP && BITS != 4;
  // a lane's packed weights of one fragment and stage: 4 * BITS bytes
  typedef uint32_t WV __attribute__((ext_vector_type(BITS)));
  __shared__ __attribute__((aligned(16))) uint8_t Sc[SCM != SC_STAGE ? NWAVES * SC_WAVE : 16];
  __shared__ int s_scan[258];
  // per group: first sorted row and row count (tile decoding without global
  // loads), and a mixed layer's weight slot
  __shared__ int s_offs[257];
  __shared__ int s_cnts[257];
  __shared__ int s_slot[MIX ? 256 : 1];
  // the gathered activation rows of the next tile, 64 per wave (a direct
  // 4-byte-per-lane load of the gather map; each wave reads its own)
  __shared__ __attribute__((aligned(16))) int s_gidx[NWAVES][64];
  __shared__ int s_wave[NWAVES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = g.K, N = g.N;
  const int KG = K / g.G;
  const int nk = K / BK;
  const int Nc = GATEUP ? N / 2 : N;  // columns of the output

  // ---- tile list: per-expert tile prefix (tiles of BM rows) ----
  int n_mtiles;
  const bool has2 = FOLD && g.counts != nullptr && g.rows2 > 0;
  const int ngrp = g.E + (has2 ? 1 : 0);
  if (g.counts != nullptr) {
    // (a launch for one width of a mixed layer takes only that width's experts)
    const int cnt = tid < g.E ? g.counts[tid] : 0;
    const int c = tid < g.E ? ((!MIX || g.tier[tid] == g.tier_id) ? cnt : 0)
                            : (has2 && tid == g.E ? g.rows2 : 0);
    if (tid < g.E) {
      s_offs[tid] = g.offsets[tid];
      s_cnts[tid] = cnt;
      if (MIX) s_slot[tid] = g.slot[tid];
    }
    int incl = (c + BM - 1) / BM;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    for (int w = 0; w < wave; ++w) incl += s_wave[w];
    if (tid < 257) s_scan[tid + 1] = incl;
    if (tid == 0) s_scan[0] = 0;
    __syncthreads();
    n_mtiles = s_scan[ngrp];
  } else {
    n_mtiles = cdiv(g.rows_single, BM);
  }
  const int total = n_mtiles * n_ntiles;
  // this XCD's contiguous share of the tiles, dealt to its workgroups
  const int xcd = blockIdx.x % NXCD;
  const int wg_in_xcd = blockIdx.x / NXCD;
  const int wgs_per_xcd = gridDim.x / NXCD;
  const int t_begin = (int)((int64_t)total * xcd / NXCD);
  const int t_end = (int)((int64_t)total * (xcd + 1) / NXCD);

  // buffer resources: 32-bit offsets instead of 64-bit addresses (the host
  // guarantees every byte size below fits in 31 bits); a read past the end
  // of a buffer returns zero
  const int n_groups = g.counts != nullptr ? (MIX ? g.w_experts : g.E) : 1;
  const int wrow_bytes = K / 8 * BITS;  // bytes of one packed weight row
  const __amdgpu_buffer_rsrc_t rA =
      __builtin_amdgcn_make_buffer_rsrc((void*)g.A, 0, g.a_rows * K * 2, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rW =
      __builtin_amdgcn_make_buffer_rsrc((void*)g.W, 0, n_groups * N * wrow_bytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rS =
      __builtin_amdgcn_make_buffer_rsrc((void*)g.Wscale, 0, n_groups * N * KG * 2, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rM = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(ASYM ? g.Wmin : g.Wscale), 0, n_groups * N * KG * 2, kRsrcWord3);
  // the gather map: max_rows entries
  const __amdgpu_buffer_rsrc_t rG = __builtin_amdgcn_make_buffer_rsrc(
      (void*)g.gather, 0, g.gather != nullptr ? g.max_rows * 4 : 0, kRsrcWord3);
  const int s_step = (BK / g.G) * 2;  // scale bytes per stage along a row
  // the extra group's operands (one expert)
  const __amdgpu_buffer_rsrc_t rA2 =
      has2 ? __builtin_amdgcn_make_buffer_rsrc((void*)g.A2, 0, g.rows2 * K * 2, kRsrcWord3) : rA;
  const __amdgpu_buffer_rsrc_t rW2 =
      has2 ? __builtin_amdgcn_make_buffer_rsrc((void*)g.W2, 0, N * (K / 2), kRsrcWord3) : rW;
  const __amdgpu_buffer_rsrc_t rS2 =
      has2 ? __builtin_amdgcn_make_buffer_rsrc((void*)g.Wscale2, 0, N * KG * 2, kRsrcWord3) : rS;
  const __amdgpu_buffer_rsrc_t rM2 =
      has2 ? __builtin_amdgcn_make_buffer_rsrc((void*)(ASYM ? g.Wmin2 : g.Wscale2), 0, N * KG * 2,
                                               kRsrcWord3)
           : rM;

  // Per-lane constants are derived from an opaque copy of the lane index, so
  // the compiler cannot compute them once up front and hold them in
  // registers across the whole persistent loop.
  int lane_o = lane, r16, lg;
  auto refresh_lane = [&]() {
    asm volatile("" : "+v"(lane_o));
    r16 = lane_o & 15;
    lg = lane_o >> 4;
  };
  refresh_lane();
  // Matrix-core row r of fragment f is weight row c0 + frow(f) + prow(r).
  // With DIRECT the gate and up fragments interleave their rows in pairs:
  // lane (r16, lg) ends with rows 4 lg .. 4 lg + 3 of each fragment, and
  // fragments 0, 1 (gate; 2, 3 up) then give it positions
  // 8 lg + 4 (f % 2) + 0..3 of the wave's 32 h columns in kperm chunk order,
  // i.e. natural columns 8 lg + kperm(4 (f % 2) + 0..3) (kperm(4 + p) =
  // kperm(p) + 2): eight consecutive h values, one 16-byte piece.
  auto frow = [&](int f) {
    return GATEUP ? (DIRECT ? 2 : 16) * (f & 1) + (f < 2 ? 0 : N / 2) : 16 * f;
  };
  auto prow = [&](int r) { return DIRECT ? 8 * (r >> 2) + kperm(r & 3) : r; };

  // ---- a tile: decoding, and this lane's load offsets ----
  auto decode = [&](int tile) {
    const int mtile = tile / n_ntiles;
    const int ntile = tile - mtile * n_ntiles;
    int e = 0, shared = 0, row0, rows;
    if (g.counts != nullptr) {
      // largest e with s_scan[e] <= mtile (binary search over the prefixes)
      int lo = 0, hi = ngrp;  // s_scan[lo] <= mtile < s_scan[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_scan[mid] <= mtile) lo = mid; else hi = mid;
      }
      e = lo;
      const int local = mtile - s_scan[e];
      shared = FOLD && e == g.E ? 1 : 0;
      if (shared) {
        e = 0;
        row0 = local * BM;
        rows = min(BM, g.rows2 - row0);
      } else {
        row0 = s_offs[e] + local * BM;
        rows = min(BM, s_cnts[e] - local * BM);
        // (the expert's index in the weight tensors: a mixed layer's width
        // tensors hold only that width's experts)
        if (MIX) e = s_slot[e];
      }
    } else {
      row0 = mtile * BM;
      rows = min(BM, g.rows_single - row0);
    }
    TileU t;
    t.row0 = __builtin_amdgcn_readfirstlane(row0);
    t.rows = __builtin_amdgcn_readfirstlane(rows);
    t.e = __builtin_amdgcn_readfirstlane(e);
    t.shared = __builtin_amdgcn_readfirstlane(shared);
    t.c0 = __builtin_amdgcn_readfirstlane(GATEUP ? ntile * (BN / 2) + wave * 32
                                                 : ntile * BN + wave * 64);
    return t;
  };
  // the first weight row of the wave's rows of tile t (uniform)
  auto wrow_first = [&](const TileU& t) { return t.e * N + (t.c0 < Nc ? t.c0 : 0); };
  // Load i of wave w fills rows 4 (ALD w + i) .. +3; lane l covers row
  // 4 (ALD w + i) + l/16, LDS slot l%16, i.e. source chunk (l%16) ^ rowswz(row).
  auto a_offset = [&](int src, int i) {
    const int r = 4 * (ALD * wave + i) + lg;
    return (uint32_t)(src * (K / 8) + (r16 ^ rowswz(r))) * 16u;
  };
  // the activation offsets of tile t from gathers straight from memory
  // (rows past the expert's end read the tile's first row: finite data
  // whose outputs are never stored)
  auto aoff_mem = [&](const TileU& t, uint32_t* ao) {
    int src[ALD];
    gather_rows<ALD>(g, t.row0, t.rows, 4 * ALD * wave + lg, 4, src, t.shared != 0);
#pragma unroll
    for (int i = 0; i < ALD; ++i) ao[i] = a_offset(src[i], i);
  };
  // the gather map entries of tile t's rows of this wave into s_gidx[wave]
  auto load_gidx = [&](const TileU& t) {
    if (g.gather != nullptr && !t.shared)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rG, (lds_void_t*)&s_gidx[wave][0], 4,
                                               (uint32_t)lane_o * 4u,
                                               (t.row0 + 4 * ALD * wave) * 4, 0, 0);
  };
  // the activation offsets of tile t from s_gidx (rows past the expert's
  // end read activation row 0 when gathered, the tile's first row if not)
  auto aoff_lds = [&](const TileU& t, uint32_t* ao) {
    const bool gath = g.gather != nullptr && !t.shared;
#pragma unroll
    for (int i = 0; i < ALD; ++i) {
      const int r = 4 * (ALD * wave + i) + lg;
      int src;
      if (gath) src = r < t.rows ? s_gidx[wave][4 * i + lg] / g.gather_div : 0;
      else src = t.row0 + (r < t.rows ? r : 0);
      ao[i] = a_offset(src, i);
    }
  };
  // ---- loads. The load state names the tile whose activations (ash, aoff)
  // and weights (wsh, bl, sl, wl) are loaded next: the current tile's until
  // its last stages switch them to the next tile's. ----
  // byte offsets of this lane's activation loads (the first ALD; a
  // fixed-size array: one sized by the template's ALD, captured by the
  // lambdas below, keeps the compiler from emitting the host-side launch
  // stub)
  uint32_t aoff[4];
  uint32_t bl = 0;     // this lane's packed weights
  uint32_t sl = 0;     // SC_STAGE: this lane's scales
  uint32_t wl = 0;     // SC_WINDOW: this lane's row's scale groups
  int ash = 0, wsh = 0;
  // tiled weights (moe_pack_w4, moe_pack_tier): fragment f's 16 rows x 128
  // K of a stage are one block of 256 BITS bytes, lane l's 4 BITS bytes at
  // 4 BITS l. The block of fragment f is the 16-row stripe at frow_t(f);
  // with DIRECT the pack has already put the rows frow(f) + prow(r) of each
  // 32-row group into that stripe's row r.
  const bool wt = MIX ? WT : BITS == 4 && g.w_tiled;
  const int w_kstep = wt ? 256 * BITS : BK / 8 * BITS;  // bytes from one K stage to the next
  auto frow_t = [&](int f) { return GATEUP ? 16 * (f & 1) + (f < 2 ? 0 : N / 2) : 16 * f; };
  auto set_w = [&](const TileU& t) {
    const int wr0 = wrow_first(t);
    bl = wt ? (uint32_t)wr0 * wrow_bytes + (uint32_t)lane_o * (4u * BITS)
            : (uint32_t)(wr0 + prow(r16)) * wrow_bytes + lg * 4 * BITS;
    if (SCM == SC_STAGE) sl = ((uint32_t)(wr0 + prow(r16)) * KG + (lg * 32) / g.G) * 2;
    if (WIN) {
      // lane l loads the window of the wave's weight row l: gate/up lanes
      // 0-31 the gate rows c0 + l, 32-63 the up rows of the same columns
      const int l = lane_o;
      const int wr = GATEUP ? (l < 32 ? l : N / 2 + l - 32) : l;
      wl = (uint32_t)(wr0 + wr) * KG * 2;
    }
    wsh = t.shared;
  };
  auto load_a = [&](int kt, uint8_t* __restrict__ dst) {
#pragma unroll
    for (int i = 0; i < ALD; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ash ? rA2 : rA, (lds_void_t*)(dst + 4 * (ALD * wave + i) * BK * 2), 16, aoff[i],
          kt * BK * 2, 0, 0);
  };
  // weights and the group's scale (and min) of stage kt into registers
  auto load_b = [&](int kt, WV* cb, uint32_t* rs, uint32_t* rm) {
#pragma unroll
    for (int f = 0; f < NFRAG; ++f) {
      const int so = (wt ? frow_t(f) : frow(f)) * wrow_bytes + kt * w_kstep;
      if constexpr (BITS == 4) {
        cb[f] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                              wsh ? rW2 : rW, bl, so, 0));
      } else if constexpr (BITS == 3) {
        cb[f] = __builtin_bit_cast(WV, __builtin_amdgcn_raw_buffer_load_b96(rW, bl, so, 0));
      } else {
        cb[f] = __builtin_bit_cast(WV, __builtin_amdgcn_raw_buffer_load_b64(rW, bl, so, 0));
      }
    }
    if (SCM == SC_STAGE) {
#pragma unroll
      for (int f = 0; f < NFRAG; ++f) {
        const int so = frow(f) * KG * 2 + kt * s_step;
        rs[f] = __builtin_amdgcn_raw_buffer_load_b16(wsh ? rS2 : rS, sl, so, 0);
        rm[f] = ASYM ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(wsh ? rM2 : rM, sl, so, 0)
                     : 0u;
      }
    }
  };
  // this wave's scale tile: two direct 1 KB loads (past a block's end they
  // read other rows' scales or zeros, never used)
  uint8_t* const sc_wave = Sc + wave * SC_WAVE;
  // the scale (and min) window w (K stages 2w, 2w+1) of the wave's rows
  auto load_win = [&](int w) {
    if (WIN) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wsh ? rS2 : rS, (lds_void_t*)sc_wave, 16, wl,
                                               w * 16, 0, 0);
      if (ASYM)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wsh ? rM2 : rM, (lds_void_t*)(sc_wave + SC_SLOT),
                                                 16, wl, w * 16, 0, 0);
    }
  };
  // the scales (and mins) of stage kt from the current window: fragment f's
  // rows are the wave's rows 16 f + r16, and lane group lg's K block is group
  // 4 (kt % 2) + lg of the window
  auto read_win = [&](int kt, uint32_t* rs, uint32_t* rm) {
#pragma unroll
    for (int f = 0; f < NFRAG; ++f) {
      const int wr = GATEUP ? (f >= 2 ? 32 : 0) + (DIRECT ? 2 : 16) * (f & 1) : 16 * f;
      const int off = (wr + prow(r16)) * 16 + (4 * (kt & 1) + lg) * 2;
      rs[f] = *reinterpret_cast<const uint16_t*>(sc_wave + off);
      rm[f] = ASYM ? *reinterpret_cast<const uint16_t*>(sc_wave + SC_SLOT + off) : 0u;
    }
  };
  // tile t's scale tile (SC_TILE) into the wave's slots
  auto load_sc_tile = [&](const TileU& t) {
    if (SCL) {
      const uint32_t r0 = (uint32_t)wrow_first(t);  // e = 0 for the extra group
      const uint32_t s0 = __builtin_amdgcn_readfirstlane(r0 * KG * 2);
      const uint32_t s1 = GATEUP ? __builtin_amdgcn_readfirstlane((r0 + N / 2) * KG * 2)
                                 : (ASYM ? s0 : s0 + SC_SLOT);
      const uint32_t lo = (uint32_t)lane_o * 16u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(t.shared ? rS2 : rS, (lds_void_t*)sc_wave, 16, lo,
                                               s0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ASYM && !GATEUP ? (t.shared ? rM2 : rM)
                                                               : (t.shared ? rS2 : rS),
                                               (lds_void_t*)(sc_wave + SC_SLOT), 16, lo, s1, 0, 0);
    }
  };
  // the scales (and mins) of stage kt from the wave's scale tile
  auto read_sc = [&](const uint8_t* __restrict__ scw, int kt, uint32_t* rs, uint32_t* rm) {
    const int grp = (lg * 32 + kt * BK) / g.G;
#pragma unroll
    for (int f = 0; f < NFRAG; ++f) {
      const int row = (GATEUP ? (DIRECT ? 2 : 16) * (f & 1) : 16 * f) + prow(r16);
      const int off = (GATEUP && f >= 2 ? SC_SLOT : 0) + (row * KG + grp) * 2;
      rs[f] = *reinterpret_cast<const uint16_t*>(scw + off);
      rm[f] = ASYM ? *reinterpret_cast<const uint16_t*>(scw + SC_SLOT + off) : 0u;
    }
  };

  f32x4 acc[MSUB][NFRAG];


  // chunk c (elements 8c .. 8c+7 of the lane's 32-element K block) of one
  // fragment's packed weights -> eight fp16 weights
  auto dequant_chunk = [&](const WV& w, int c, f16x2 s2, f16x2 m2) {
    // (the down GEMM keeps the shift-per-nibble form: with the one-shift
    // form its 128-row instance spills)
    // (3 bits, tiled: the third-bit word rearranged by the pack, one rotate
    // per chunk instead of a shift per pair)
    if constexpr (BITS == 4) return dequant8_f16<ASYM, GATEUP>(w[c], s2, m2);
    else if constexpr (BITS == 2) return dequant8_f16_b2x(w[c >> 1], c & 1, s2);
    else if constexpr (MIX && WT) return dequant8_f16_b3t(w[c >> 1], w[2], c, s2);
    else return dequant8_f16_b3(w[c >> 1], w[2], c, s2);
  };

  // One K stage from ring slot `as_base`: four 32-wide K steps x eight
  // 16-row sub-tiles. Two waves share each SIMD, so the hardware interleaves
  // one wave's dequant and LDS reads with the other's MFMAs. Every sub-tile
  // is computed; rows past the end of an expert hold finite data whose
  // results are never stored. The down GEMM (and DIRECT gate/up) swaps the
  // operands (C^T = W A^T), so each lane ends up with four output columns of
  // one row.
  auto compute_stage = [&](const uint8_t* __restrict__ as_base, const WV* cb, const uint32_t* rs,
                           const uint32_t* rm, f16x8* b, const WV* cbn, uint32_t* rsn,
                           uint32_t* rmn, int nkt) {
    f16x2 cs[NFRAG], cm[NFRAG];
#pragma unroll
    for (int f = 0; f < NFRAG; ++f) {
      cs[f] = __builtin_bit_cast(f16x2, rs[f] * 0x10001u);
      cm[f] = __builtin_bit_cast(f16x2, rm[f] * 0x10001u);
    }
    const uint8_t* ap[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) ap[j] = as_base + r16 * (BK * 2) + (((lg * 4 + j) ^ rowswz(r16)) * 16);
    auto read_a = [&](int j, int mi) {
      return __builtin_bit_cast(f16x8, ld16(ap[j] + mi * 16 * BK * 2));
    };
    // The weights of step j+1 are dequantized while step j's MFMAs run (one
    // fragment behind each of the first sub-tiles). With XDQ, step 0's come
    // in dequantized (by the previous stage, or before a tile's first stage)
    // and step 3 dequantizes the next stage's step 0, so that no stage
    // starts with a run of dequant work that no MFMA overlaps (the two waves
    // of a SIMD leave the stage barrier together).
    if (!XDQ) {
#pragma unroll
      for (int f = 0; f < NFRAG; ++f) b[f] = dequant_chunk(cb[f], 0, cs[f], cm[f]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f16x8 bn[NFRAG];
      f16x2 csn[NFRAG], cmn[NFRAG];
      if (XDQ && j == 3) {
        if (WIN) {
          // the window refilled in this stage has landed
          __builtin_amdgcn_s_waitcnt(waitcnt_vm(ALD));
          read_win(nkt, rsn, rmn);
        }
#pragma unroll
        for (int f = 0; f < NFRAG; ++f) {
          csn[f] = __builtin_bit_cast(f16x2, rsn[f] * 0x10001u);
          cmn[f] = __builtin_bit_cast(f16x2, rmn[f] * 0x10001u);
        }
      }
      f16x8 a = read_a(j, 0);
#pragma unroll
      for (int mi = 0; mi < MSUB; ++mi) {
        f16x8 an;
        if (mi + 1 < MSUB) an = read_a(j, mi + 1);
#pragma unroll
        for (int f = 0; f < NFRAG; ++f)
          acc[mi][f] = GATEUP && !DIRECT ? mfma_16x16x32_f16(a, b[f], acc[mi][f])
                                         : mfma_16x16x32_f16(b[f], a, acc[mi][f]);
        if (mi < NFRAG) {
          if (j < 3) bn[mi] = dequant_chunk(cb[mi], j + 1, cs[mi], cm[mi]);
          else if (XDQ) bn[mi] = dequant_chunk(cbn[mi], 0, csn[mi], cmn[mi]);
        }
        if (mi + 1 < MSUB) a = an;
      }
      if (j < 3 || XDQ) {
#pragma unroll
        for (int f = 0; f < NFRAG; ++f) b[f] = bn[f];
      }
    }
  };

  // Epilogue, from the wave's 4 KB sub-tile in Ex. Gate/up: h = silu(g) * u,
  // stored as fp16 in kperm chunk order, in passes of 64 rows x 64 B so that
  // it leaves as 16-byte row pieces (3- and 2-bit: straight from the
  // accumulators). Down: y in passes of 32 rows x 128 B. No barrier: the
  // sub-tile is the wave's own, and the stores drain while the next tile's
  // first stage runs.
  auto epilogue = [&](const TileU& t) {
    int rq = 4 * lg, rr = r16, row0 = t.row0, rows = t.rows;
    uint16_t* const C = t.shared ? g.C2 : g.C;
    const int ldc = t.shared ? g.ldc2 : g.ldc;
    const bool cvalid = t.c0 < Nc;
    asm volatile("" : "+v"(rq), "+v"(rr), "+v"(row0), "+v"(rows));
    if (DIRECT) {
      // eight consecutive h values of row 16 mi + r16 per lane (see frow):
      // one 16-byte piece, 64 contiguous bytes of each of 16 rows per store
      uint16_t* const crow = C + (int64_t)(row0 + rr) * ldc + t.c0 + 2 * rq;
#pragma unroll
      for (int mi = 0; mi < MSUB; ++mi) {
        float h[8];
#pragma unroll
        for (int v = 0; v < 8; ++v)
          h[v] = silu_f32(acc[mi][v >> 2][v & 3]) * acc[mi][2 + (v >> 2)][v & 3];
        const u32x4 d = {pack_f16x2(h[0], h[1]), pack_f16x2(h[2], h[3]), pack_f16x2(h[4], h[5]),
                         pack_f16x2(h[6], h[7])};
        if (cvalid && mi * 16 + rr < rows) st16(crow + (int64_t)(mi * 16) * ldc, d);
      }
    } else if (GATEUP) {
      uint8_t* const sub = Ex + wave * SUBW;
      // the 16-byte piece p of row r sits at p ^ ((r >> 2) & 3), so the four
      // row groups of one write land in different banks
#pragma unroll
      for (int ps = 0; ps < BM / 64; ++ps) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int pc = 8 * (r16 >> 3) + kpos(r16 & 7);  // column in its pair of pieces
#pragma unroll
          for (int mh = 0; mh < 4; ++mh)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int mi = 4 * ps + mh;
              const int rl = mh * 16 + rq + v;
              const float h = silu_f32(acc[mi][j][v]) * acc[mi][j + 2][v];
              const int piece = (2 * j + (pc >> 3)) ^ ((rl >> 2) & 3);
              *reinterpret_cast<uint16_t*>(sub + rl * 64 + piece * 16 + (pc & 7) * 2) =
                  (uint16_t)(pack_f16x2(h, 0.f) & 0xffffu);
            }
        }
        lds_wave_sync();
        // 16 rows x 64 bytes per wave-wide read: lane -> row lane/4, piece lane%4
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int rl = q * 16 + (lane_o >> 2);
          const int p = lane_o & 3;
          const u32x4 d = ld16(sub + rl * 64 + (p ^ ((rl >> 2) & 3)) * 16);
          const int row = ps * 64 + rl;
          if (cvalid && row < rows) st16(C + (int64_t)(row0 + row) * ldc + t.c0 + p * 8, d);
        }
      }
    } else {
      // lane (r16, lg) holds columns 16 f + 4 lg .. +3 of row 16 mi + r16;
      // the 16-byte piece p of row r of a pass sits at p ^ (r & 7)
      uint8_t* const sub = Ex + wave * SUBW;
#pragma unroll
      for (int ps = 0; ps < BM / 32; ++ps) {
#pragma unroll
        for (int mh = 0; mh < 2; ++mh) {
          const int mi = ps * 2 + mh;
          const int rl = mh * 16 + rr;  // row within the pass
#pragma unroll
          for (int f = 0; f < NFRAG; ++f) {
            uint2 d;
            d.x = pack_f16x2(acc[mi][f][0], acc[mi][f][1]);
            d.y = pack_f16x2(acc[mi][f][2], acc[mi][f][3]);
            const int piece = (2 * f + (lg >> 1)) ^ (rl & 7);
            *reinterpret_cast<uint2*>(sub + rl * 128 + piece * 16 + (lg & 1) * 8) = d;
          }
        }
        lds_wave_sync();
        // 8 rows x 128 bytes per wave-wide read: lane -> row lane/8, piece lane%8
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int rl = q * 8 + (lane_o >> 3);
          const int p = lane_o & 7;
          const u32x4 d = ld16(sub + rl * 128 + (p ^ (rl & 7)) * 16);
          const int row = ps * 32 + rl;
          if (cvalid && row < rows) st16(C + (int64_t)(row0 + row) * ldc + t.c0 + p * 8, d);
        }
      }
    }
  };

  // ---- persistent loop. K loop: weights one stage ahead in registers
  // (issued at the top of each stage), activations into the ring slot two
  // stages ahead (issued at the end of each stage), so "at most ALD loads
  // outstanding" at the end of stage s means: stage s+1's activations and
  // weights have landed (loads complete in issue order). With at least three
  // stages per tile the pipeline runs on across tiles: the last two stages
  // of a tile load the next tile's first two (its activations into the next
  // ring slots, its weights and scales into registers and the wave's scale
  // slots), so a tile starts with its first stage in place and its
  // predecessor's stores still draining. Past the workgroup's last tile, and
  // for shorter K, the last stages repeat their own loads instead (into ring
  // slots nobody reads), so the waits are the same at every stage and the
  // compiler's own wait bookkeeping stays exact; with shorter K each tile
  // then starts from scratch.
  int tile = t_begin + wg_in_xcd;
  if (tile >= t_end) return;
  const int klast = nk - 1;
  // (not with 3-bit weights, whose wider dequant leaves no registers for the
  // next tile's load state, nor for the 2-bit gate/up kernel, which it did
  // not make faster: their tiles keep the plain loop)
  constexpr bool XT = BITS == 4 || (!GATEUP && BITS == 2);
  const bool xt = XT && nk >= 3;
  TileU cu = decode(tile);
  int ntile_id = tile + wgs_per_xcd;
  bool has_next = ntile_id < t_end;
  TileU nx = cu;  // the next tile (cross-tile pipeline only)
  if (xt && has_next) nx = decode(ntile_id);
  WV cb[NFRAG];
  uint32_t rs[NFRAG], rm[NFRAG];
  f16x8 b0[NFRAG];  // dequantized weights of a stage's first K step
  // a tile's first two stages from scratch (the first tile; every tile if
  // nk < 3), into ring slots 0 and 1
  auto start_plain = [&](const TileU& t, uint8_t* __restrict__ s0, uint8_t* __restrict__ s1) {
    aoff_mem(t, aoff);
    ash = t.shared;
    set_w(t);
    load_sc_tile(t);
    load_win(0);
    load_b(0, cb, rs, rm);
    load_a(0, s0);
    load_a(min(1, klast), s1);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(ALD));
    lds_barrier();  // stage 0 in every wave
  };
  // (the next tile's gather entries first: the start's wait covers them)
  if (xt && has_next) load_gidx(nx);
  int ph = 0;         // ring slot of the current tile's first stage
  bool plain = true;  // the tile starts from scratch
  while (true) {
    if (plain) {
      start_plain(cu, As0, As1);
      ph = 0;
    }
    refresh_lane();
    if (SCL) read_sc(sc_wave, 0, rs, rm);
    if (WIN) read_win(0, rs, rm);
    if (XDQ) {
      // the tile's first step
#pragma unroll
      for (int f = 0; f < NFRAG; ++f)
        b0[f] = dequant_chunk(cb[f], 0, __builtin_bit_cast(f16x2, rs[f] * 0x10001u),
                              __builtin_bit_cast(f16x2, rm[f] * 0x10001u));
    }
#pragma unroll
    for (int i = 0; i < MSUB; ++i)
#pragma unroll
      for (int j = 0; j < NFRAG; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const bool go_next = xt && has_next;
    // stage kt reads ring slot `curs` and loads stage kt + 2 (of this tile
    // or, past its end, of the next) into `nxt2`
    auto stage = [&](int kt, const uint8_t* __restrict__ curs, uint8_t* __restrict__ nxt2) {
      WV cbn[NFRAG];
      uint32_t rsn[NFRAG], rmn[NFRAG];
      const bool wlast = kt + 1 == nk;     // the weights loaded here are the next tile's
      const int nkt = wlast ? 0 : kt + 1;  // local index of the stage after this one
      if (wlast && go_next) {
        set_w(nx);
        load_sc_tile(nx);  // the wave read its scale tile for the last time a stage ago
      }
      load_b(wlast ? (go_next ? 0 : klast) : kt + 1, cbn, rsn, rmn);
      if (WIN) {
        // windows refill at odd stages (stages kt + 1, kt + 2); the last
        // stage fetches the next tile's first window
        if (wlast) {
          if (go_next) load_win(0);
        } else if (kt & 1) {
          load_win((kt + 1) >> 1);
        }
      }
      // issue the weight loads here, a whole stage before they are needed:
      // left to itself the scheduler sinks them to the end of the stage (to
      // shorten register lifetimes), right before the wait for them
      __builtin_amdgcn_sched_barrier(0);
      // (the last stage's scales are already in registers; past it the
      // wave's slots are being refilled with the next tile's, which the
      // tile start reads)
      auto next_sc = [&]() {
        if (wlast && go_next) {
#pragma unroll
          for (int f = 0; f < NFRAG; ++f) {
            rsn[f] = rs[f];
            rmn[f] = rm[f];
          }
        } else {
          read_sc(sc_wave, min(kt + 1, klast), rsn, rmn);
        }
      };
      if (XDQ && SCL) next_sc();
      // a wave in its MFMA and dequant stream outranks its SIMD partner while
      // that one issues loads, waits or crosses the barrier (gate/up 1.4-2.4 %
      // faster over six A/B runs on two boxes; down unchanged)
      __builtin_amdgcn_s_setprio(1);
      compute_stage(curs, cb, rs, rm, b0, cbn, rsn, rmn, nkt);
      __builtin_amdgcn_s_setprio(0);
      if (!XDQ && SCL) next_sc();
      // The activation loads go last: their direct writes into the LDS then
      // land while the stage ends and the next one starts, not in the middle
      // of this stage's fragment reads (issued at the top of the stage they
      // cost gate/up 1-3 % and down 2-4 %). They still have a whole stage to
      // land, and being the last loads issued, "at most ALD outstanding"
      // below still means this stage's weights have arrived.
      __builtin_amdgcn_sched_barrier(0);
      if (kt + 2 == nk && go_next) {
        aoff_lds(nx, aoff);
        ash = nx.shared;
      }
      load_a(kt + 2 < nk ? kt + 2 : (go_next ? kt + 2 - nk : klast), nxt2);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(ALD));
      // (after the wait: a window refilled in this stage has landed)
      if (!XDQ && WIN) read_win(nkt, rsn, rmn);
      lds_barrier();
      // the hand-over of the next stage's registers stays here: moved up into
      // the stage it would wait for loads that were just issued
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int f = 0; f < NFRAG; ++f) {
        cb[f] = cbn[f];
        rs[f] = rsn[f];
        rm[f] = rmn[f];
      }
    };
    if constexpr (XT) {
      // the three ring slots in turn, entered at the tile's first slot
      int kt = 0;
      for (;;) {
        if (ph == 0) {
          stage(kt, As0, As2);
          ph = 1;
          if (++kt == nk) break;
        }
        if (ph == 1) {
          stage(kt, As1, As0);
          ph = 2;
          if (++kt == nk) break;
        }
        if (ph == 2) {
          stage(kt, As2, As1);
          ph = 0;
          if (++kt == nk) break;
        }
      }
    } else {
      // every tile starts in slot 0
      for (int kt = 0; kt < nk; kt += 3) {
        stage(kt, As0, As2);
        if (kt + 1 < nk) stage(kt + 1, As1, As0);
        if (kt + 2 < nk) stage(kt + 2, As2, As1);
      }
    }
    epilogue(cu);
    if (!has_next) break;
    refresh_lane();
    tile = ntile_id;
    ntile_id = tile + wgs_per_xcd;
    has_next = ntile_id < t_end;
    plain = !xt;
    if (xt) {
      cu = nx;
      if (has_next) {
        nx = decode(ntile_id);
        // (read at the new tile's second-to-last stage, after several waits)
        load_gidx(nx);
      }
    } else {
      cu = decode(tile);
      // the repeated loads of the last stages have landed everywhere
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      lds_barrier();
    }
  }
  // the repeated loads of the last stages land before the workgroup ends
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
}

int g_num_cus = 0;

template <bool GATEUP>
hipError_t launch_grouped(const GroupedGemm& g, hipStream_t s, const char* name) {
  const int n_ntiles = GATEUP ? cdiv(g.N / 2, BN / 2) : cdiv(g.N, BN);
  // 64-row tiles when the experts get few rows each on average (grouped
  // launches of one width, without an extra group): up to 128 for gate/up,
  // 64 for down (measured at T = 512 .. 4096 on the A3B shape)
  const bool fold = g.counts != nullptr && g.rows2 > 0;
  const bool rows64 = g.counts != nullptr && !fold && g.tier == nullptr &&
                      (int64_t)g.max_rows <= (GATEUP ? 128LL : 64LL) * g.E;
  const int tbm = rows64 ? 64 : BM;
  const int m_bound =
      g.counts != nullptr
          ? cdiv(g.max_rows, tbm) + g.E + (g.rows2 > 0 ? cdiv(g.rows2, tbm) + 1 : 0)
          : cdiv(g.rows_single, tbm);
  if (m_bound <= 0) return hipSuccess;
  if (g_num_cus == 0) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    err = hipDeviceGetAttribute(&g_num_cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
  }
  // persistent grid: WGS_PER_CU workgroups per CU, a multiple of the XCD
  // count, never more than the tile bound
  int wgs = WGS_PER_CU * g_num_cus;
  const int bound = cdiv(m_bound * n_ntiles, NXCD) * NXCD;
  if (wgs > bound) wgs = bound;
  wgs = cdiv(wgs, NXCD) * NXCD;
  const dim3 grid(wgs), block(NTHREADS);
  LaunchScope ls(name, s);
  // scales through LDS when a wave's rows fit its two 1 KB slots; an extra
  // (shared-expert) group is a variant of its own, without the LDS scales,
  // so that the common kernels keep their registers
  const int KG = g.K / g.G;
  const bool asym = g.Wmin != nullptr;
  const bool scl = !fold && (GATEUP ? (!asym && KG <= 16) : (asym ? KG <= 8 : KG <= 16));
  // scale windows: asymmetric experts with G = 32 whose scales do not fit
  // the tile (the shared-expert variant included)
  const bool win = asym && !scl && g.G == 32;
  auto go = [&](auto a, auto m, auto f) {
    constexpr bool A = decltype(a)::value, F = decltype(f)::value;
    constexpr int M = decltype(m)::value;
    if constexpr (!F) {
      if (rows64) {
        hipLaunchKernelGGL((expert_gemm_kernel<GATEUP, A, M, F, 4, false, 64>), grid, block, 0, s,
                           g, n_ntiles);
        return;
      }
    }
    hipLaunchKernelGGL((expert_gemm_kernel<GATEUP, A, M, F>), grid, block, 0, s, g, n_ntiles);
  };
  const std::true_type yes{};
  const std::false_type no{};
  const std::integral_constant<int, SC_STAGE> stage_sc{};
  const std::integral_constant<int, SC_TILE> tile_sc{};
  const std::integral_constant<int, SC_WINDOW> win_sc{};
  if (g.tier != nullptr) {
    // one width of a mixed-width layer (symmetric, no extra group)
    auto go_b = [&](auto m, auto b) {
      constexpr int M = decltype(m)::value, B = decltype(b)::value;
      if (g.w_tiled)
        hipLaunchKernelGGL((expert_gemm_kernel<GATEUP, false, M, false, B, true, 128, true>), grid,
                           block, 0, s, g, n_ntiles);
      else
        hipLaunchKernelGGL((expert_gemm_kernel<GATEUP, false, M, false, B, true>), grid, block, 0,
                           s, g, n_ntiles);
    };
    const std::integral_constant<int, 4> b4{};
    const std::integral_constant<int, 3> b3{};
    const std::integral_constant<int, 2> b2{};
    if (g.bits == 3) {
      if (scl) go_b(tile_sc, b3);
      else go_b(stage_sc, b3);
    } else if (g.bits == 2) {
      if (scl) go_b(tile_sc, b2);
      else go_b(stage_sc, b2);
    } else {
      if (scl) go_b(tile_sc, b4);
      else go_b(stage_sc, b4);
    }
  } else if (asym) {
    if (fold) {
      if (win) go(yes, win_sc, yes);
      else go(yes, stage_sc, yes);
    } else if (scl) {
      go(yes, tile_sc, no);
    } else if (win) {
      go(yes, win_sc, no);
    } else {
      go(yes, stage_sc, no);
    }
  } else {
    if (fold) go(no, stage_sc, yes);
    else if (scl) go(no, tile_sc, no);
    else go(no, stage_sc, no);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_x_to_f16(const uint16_t* x, uint16_t* x16, int64_t n, hipStream_t s) {
  const int64_t chunks = n / 8;
  int64_t blocks = (chunks + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) return hipSuccess;
  LaunchScope ls("x_to_f16", s);
  hipLaunchKernelGGL(x_to_f16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, x16, chunks);
  return hipGetLastError();
}

// A few rows per group: the layer is bound by reading the weights once, and
// the weight-streaming kernel spreads them over the whole chip.
static bool use_stream(const GroupedGemm& g, bool gateup) {
  return g.expect_rows > 0 && g.expect_rows <= kStreamMaxRows && stream_supported(g, gateup);
}

bool gemm_streams(const GroupedGemm& g, bool gateup) { return use_stream(g, gateup); }

hipError_t launch_gateup(const GroupedGemm& g, hipStream_t s, const char* name) {
  if (use_stream(g, true)) return launch_stream(g, true, s, name);
  return launch_grouped<true>(g, s, name);
}
hipError_t launch_down(const GroupedGemm& g, hipStream_t s, const char* name) {
  if (use_stream(g, false)) return launch_stream(g, false, s, name);
  return launch_grouped<false>(g, s, name);
}

}  // namespace qmoe
