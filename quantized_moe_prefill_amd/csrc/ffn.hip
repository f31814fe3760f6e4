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
// results leave through a per-wave LDS sub-tile as 16-byte row pieces.
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

__device__ __forceinline__ float silu(float z) { return z / (1.f + __expf(-z)); }

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

// What one tile of the expert GEMM needs besides the shared setup: its
// rows, this lane's activation sources and weight offsets. (At namespace
// scope: a class local to a kernel template keeps the compiler from emitting
// the kernel's host-side launch stub.)
struct GemmTile {
  int row0, rows, c0;
  bool cvalid;
  int shared;  // the tile belongs to the extra group (uniform)
  uint32_t a_off[ALD];  // byte offsets of this lane's activation loads
  uint32_t b_lane, s_lane;
  uint32_t sc_src[2];  // scale tiles in LDS: byte offsets of the two 1 KB sources
  uint32_t win_lane;   // scale windows: byte offset of this lane's row's groups
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
// rows or fewer (a 128-row tile would be mostly padding there).
template <bool GATEUP, bool ASYM, int SCM, bool FOLD, int BITS = 4, bool MIX = false,
          int TBM = 128>
__global__ __launch_bounds__(NTHREADS, 1) void expert_gemm_kernel(GroupedGemm g, int n_ntiles) {
  static_assert(TBM == 128 || TBM == 64, "tile rows");
  // this instance's tile height and what follows from it (the names hide
  // the 128-row constants above)
  constexpr int BM = TBM;
  constexpr int MSUB = BM / 16;
  constexpr int ALD = BM / 4 / NWAVES;  // direct activation loads per wave and stage
  constexpr int A_STAGE_BYTES = BM * BK * 2;
  // epilogue sub-tiles: gate/up BM rows x 64 B per wave; down 64-row halves
  // x 128 B per wave. 128-row tiles put waves 0-3 in As2, 4-7 in Ex; 64-row
  // tiles put all eight in Ex.
  constexpr int SUBW = GATEUP ? BM * 64 : 64 * 128;
  constexpr int EX_BYTES = BM == 128 ? (NWAVES - 2 * ASTAGES) * SUB_BYTES : NWAVES * SUBW;
  // LDS, two uses:
  //  - K loop: a ring of three activation tiles (As0..As2), BM rows x 128
  //    fp16 each, no padding; the 16-byte chunk c of row r sits in slot
  //    c ^ rowswz(r) (see rowswz), which keeps the fragment reads free of
  //    bank conflicts and lets a direct global->LDS load fill four whole rows.
  //    Separate arrays (and a K loop unrolled by three) let the compiler see
  //    that a stage's LDS reads never touch the tiles still being loaded, so
  //    it does not wait for those loads before reading;
  //  - epilogue: each wave's output sub-tile (BM rows x 64 B for h, 64-row
  //    halves x 128 B for y) in As2 and Ex, so the results leave in whole
  //    16-byte row pieces.
  __shared__ __attribute__((aligned(16))) uint8_t As0[A_STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t As1[A_STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t As2[A_STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t Ex[EX_BYTES];
  constexpr bool SCL = SCM == SC_TILE;
  constexpr bool WIN = SCM == SC_WINDOW;
  // each stage dequantizes the next stage's first K step (symmetric experts:
  // with a min per group the extra live registers spill)
  constexpr bool XDQ = !ASYM;
  // a lane's packed weights of one fragment and stage: 4 * BITS bytes
  typedef uint32_t WV __attribute__((ext_vector_type(BITS)));
  __shared__ __attribute__((aligned(16))) uint8_t Sc[SCM != SC_STAGE ? NWAVES * SC_WAVE : 16];
  __shared__ int s_scan[258];
  __shared__ int s_wave[NWAVES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = g.K, N = g.N;
  const int KG = K / g.G;
  const int nk = K / BK;

  // ---- tile list: per-expert tile prefix (tiles of BM rows) ----
  int n_mtiles;
  const bool has2 = FOLD && g.counts != nullptr && g.rows2 > 0;
  const int ngrp = g.E + (has2 ? 1 : 0);
  if (g.counts != nullptr) {
    // (a launch for one width of a mixed layer takes only that width's experts)
    const int c = tid < g.E ? ((!MIX || g.tier[tid] == g.tier_id) ? g.counts[tid] : 0)
                            : (has2 && tid == g.E ? g.rows2 : 0);
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
  auto frow = [&](int f) { return GATEUP ? 16 * (f & 1) + (f < 2 ? 0 : N / 2) : 16 * f; };

  // Fragment f of a wave covers weight rows c0 + frow(f) + 0..15 of
  // the expert (gate/up: fragments 0, 1 are gate columns c0 + 16 f, 2, 3 the
  // up rows of the same columns). Lane (r16, lg) reads row r16 of each
  // fragment, K values [32 lg, 32 lg + 32) of every stage (16 bytes), which
  // is also the K range its A fragments cover, so the two operands agree
  // without any reordering: one per-lane offset plus a uniform offset per
  // fragment and stage.
  auto setup = [&](int tile, GemmTile& ts) {
    const int mtile = tile / n_ntiles;
    const int ntile = tile - mtile * n_ntiles;
    int e;
    if (g.counts != nullptr) {
      // largest e with s_scan[e] <= mtile (binary search over the prefixes)
      int lo = 0, hi = ngrp;  // s_scan[lo] <= mtile < s_scan[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_scan[mid] <= mtile) lo = mid; else hi = mid;
      }
      e = lo;
      const int local = mtile - s_scan[e];
      ts.shared = FOLD ? __builtin_amdgcn_readfirstlane(e == g.E ? 1 : 0) : 0;
      if (ts.shared) {
        e = 0;
        ts.row0 = local * BM;
        ts.rows = min(BM, g.rows2 - ts.row0);
      } else {
        ts.row0 = g.offsets[e] + local * BM;
        ts.rows = min(BM, g.counts[e] - local * BM);
      }
    } else {
      e = 0;
      ts.shared = 0;
      ts.row0 = mtile * BM;
      ts.rows = min(BM, g.rows_single - ts.row0);
    }
    // load i of wave w fills rows 4 (ALD w + i) .. +3; lane l covers row
    // 4 (ALD w + i) + l/16, LDS slot l%16, i.e. source chunk (l%16) ^ rowswz(row)
    int src[ALD];
    gather_rows<ALD>(g, ts.row0, ts.rows, 4 * ALD * wave + lg, 4, src, ts.shared != 0);
#pragma unroll
    for (int i = 0; i < ALD; ++i) {
      const int r = 4 * (ALD * wave + i) + lg;
      ts.a_off[i] = (uint32_t)(src[i] * (K / 8) + (r16 ^ rowswz(r))) * 16u;
    }
    ts.c0 = GATEUP ? ntile * (BN / 2) + wave * 32 : ntile * BN + wave * 64;
    ts.cvalid = ts.c0 < (GATEUP ? N / 2 : N);
    // the expert's index in the weight tensors (a mixed layer's width
    // tensors hold only that width's experts)
    if (MIX) e = g.slot[e];
    const int wrow0 = e * N + (ts.cvalid ? ts.c0 : 0) + r16;
    ts.b_lane = (uint32_t)wrow0 * wrow_bytes + lg * 4 * BITS;
    ts.s_lane = ((uint32_t)wrow0 * KG + (lg * 32) / g.G) * 2;
    if (WIN) {
      // lane l loads the window of the wave's weight row l: gate/up lanes
      // 0-31 the gate rows c0 + l, 32-63 the up rows of the same columns
      const int l = lane_o;
      const int wr = GATEUP ? (l < 32 ? l : N / 2 + l - 32) : l;
      ts.win_lane = (uint32_t)(e * N + (ts.cvalid ? ts.c0 : 0) + wr) * KG * 2;
    }
    if (SCL) {
      const uint32_t r0 = (uint32_t)(e * N + (ts.cvalid ? ts.c0 : 0));  // e = 0 for the extra group
      const uint32_t s0 = __builtin_amdgcn_readfirstlane(r0 * KG * 2);
      ts.sc_src[0] = s0;
      ts.sc_src[1] = GATEUP ? __builtin_amdgcn_readfirstlane((r0 + N / 2) * KG * 2)
                            : (ASYM ? s0 : s0 + SC_SLOT);
    }
  };
  auto load_a = [&](const GemmTile& ts, int kt, uint8_t* __restrict__ dst) {
#pragma unroll
    for (int i = 0; i < ALD; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ts.shared ? rA2 : rA, (lds_void_t*)(dst + 4 * (ALD * wave + i) * BK * 2), 16, ts.a_off[i],
          kt * BK * 2, 0, 0);
  };
  // weights and the group's scale (and min) of stage kt into registers
  auto load_b = [&](const GemmTile& ts, int kt, WV* cb, uint32_t* rs, uint32_t* rm) {
#pragma unroll
    for (int f = 0; f < NFRAG; ++f) {
      const int so = frow(f) * wrow_bytes + kt * (BK / 8 * BITS);
      if constexpr (BITS == 4) {
        cb[f] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                              ts.shared ? rW2 : rW, ts.b_lane, so, 0));
      } else if constexpr (BITS == 3) {
        cb[f] = __builtin_bit_cast(WV, __builtin_amdgcn_raw_buffer_load_b96(rW, ts.b_lane, so, 0));
      } else {
        cb[f] = __builtin_bit_cast(WV, __builtin_amdgcn_raw_buffer_load_b64(rW, ts.b_lane, so, 0));
      }
    }
    if (SCM == SC_STAGE) {
#pragma unroll
      for (int f = 0; f < NFRAG; ++f) {
        const int so = frow(f) * KG * 2 + kt * s_step;
        rs[f] = __builtin_amdgcn_raw_buffer_load_b16(ts.shared ? rS2 : rS, ts.s_lane, so, 0);
        rm[f] = ASYM ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(ts.shared ? rM2 : rM,
                                                                     ts.s_lane, so, 0)
                     : 0u;
      }
    }
  };
  // this wave's scale tile: two direct 1 KB loads (past a block's end they
  // read other rows' scales or zeros, never used)
  uint8_t* const sc_wave = Sc + wave * SC_WAVE;
  // the scale (and min) window w (K stages 2w, 2w+1) of the wave's rows
  auto load_win = [&](const GemmTile& ts, int w) {
    if (WIN) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ts.shared ? rS2 : rS, (lds_void_t*)sc_wave, 16,
                                               ts.win_lane, w * 16, 0, 0);
      if (ASYM)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ts.shared ? rM2 : rM,
                                                 (lds_void_t*)(sc_wave + SC_SLOT), 16,
                                                 ts.win_lane, w * 16, 0, 0);
    }
  };
  // the scales (and mins) of stage kt from the current window: fragment f's
  // rows are the wave's rows 16 f + r16, and lane group lg's K block is group
  // 4 (kt % 2) + lg of the window
  auto read_win = [&](int kt, uint32_t* rs, uint32_t* rm) {
#pragma unroll
    for (int f = 0; f < NFRAG; ++f) {
      const int off = (16 * f + r16) * 16 + (4 * (kt & 1) + lg) * 2;
      rs[f] = *reinterpret_cast<const uint16_t*>(sc_wave + off);
      rm[f] = ASYM ? *reinterpret_cast<const uint16_t*>(sc_wave + SC_SLOT + off) : 0u;
    }
  };
  auto load_sc = [&](const GemmTile& ts) {
    if (WIN) load_win(ts, 0);
    if (SCL) {
      const uint32_t lo = (uint32_t)lane_o * 16u;
      const __amdgpu_buffer_rsrc_t s_r = ts.shared ? rS2 : rS;
      const __amdgpu_buffer_rsrc_t m_r = ts.shared ? rM2 : rM;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(s_r, (lds_void_t*)sc_wave, 16, lo, ts.sc_src[0], 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ASYM && !GATEUP ? m_r : s_r,
                                               (lds_void_t*)(sc_wave + SC_SLOT), 16, lo,
                                               ts.sc_src[1], 0, 0);
    }
  };
  // the scales (and mins) of stage kt from the wave's scale tile
  auto read_sc = [&](const uint8_t* __restrict__ scw, int kt, uint32_t* rs, uint32_t* rm) {
    const int grp = (lg * 32 + kt * BK) / g.G;
#pragma unroll
    for (int f = 0; f < NFRAG; ++f) {
      const int row = GATEUP ? 16 * (f & 1) + r16 : 16 * f + r16;
      const int off = (GATEUP && f >= 2 ? SC_SLOT : 0) + (row * KG + grp) * 2;
      rs[f] = *reinterpret_cast<const uint16_t*>(scw + off);
      rm[f] = ASYM ? *reinterpret_cast<const uint16_t*>(scw + SC_SLOT + off) : 0u;
    }
  };

  f32x4 acc[MSUB][NFRAG];

  // chunk c (elements 8c .. 8c+7 of the lane's 32-element K block) of one
  // fragment's packed weights -> eight fp16 weights
  auto dequant_chunk = [&](const WV& w, int c, f16x2 s2, f16x2 m2) {
    if constexpr (BITS == 4) return dequant8_f16<ASYM>(w[c], s2, m2);
    else if constexpr (BITS == 2) return dequant8_f16_b2(w[c >> 1], c & 1, s2);
    else return dequant8_f16_b3(w[c >> 1], w[2], c, s2);
  };

  // One K stage from ring slot `as_base`: four 32-wide K steps x eight
  // 16-row sub-tiles. Two waves share each SIMD, so the hardware interleaves
  // one wave's dequant and LDS reads with the other's MFMAs. Every sub-tile
  // is computed; rows past the end of an expert hold finite data whose
  // results are never stored. The down GEMM swaps the operands
  // (C^T = W A^T), so each lane ends up with four consecutive output
  // columns of one row.
  auto compute_stage = [&](const uint8_t* __restrict__ as_base, const WV* cb, const uint32_t* rs,
                           const uint32_t* rm, f16x8* b, const WV* cbn, uint32_t* rsn,
                           uint32_t* rmn, int kt) {
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
          read_win(kt + 1, rsn, rmn);
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
          acc[mi][f] = GATEUP ? mfma_16x16x32_f16(a, b[f], acc[mi][f])
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

  // Epilogue. Gate/up: h = silu(g) * u, stored as fp16 in kperm chunk order
  // through this wave's LDS sub-tile (128 rows x 64 B, in As2 or Ex, which
  // the next tile's first two stages leave alone) so that it leaves as
  // 16-byte row pieces. Down: the same, in two halves of 64 rows.
  auto epilogue = [&](const GemmTile& ts) {
    int rq = 4 * lg, rr = r16, row0 = ts.row0, rows = ts.rows;
    uint16_t* const C = ts.shared ? g.C2 : g.C;
    const int ldc = ts.shared ? g.ldc2 : g.ldc;
    asm volatile("" : "+v"(rq), "+v"(rr), "+v"(row0), "+v"(rows));
    if (GATEUP) {
      uint8_t* sub = BM == 128 ? (wave < 4 ? As2 : Ex) + (wave & 3) * SUBW : Ex + wave * SUBW;
      // the 16-byte piece p of row r sits at p ^ ((r >> 2) & 3), so the four
      // row groups of one write land in different banks
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int pc = 8 * (r16 >> 3) + kpos(r16 & 7);  // column in its pair of pieces
#pragma unroll
        for (int mi = 0; mi < MSUB; ++mi)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int rl = mi * 16 + rq + v;
            const float h = silu(acc[mi][j][v]) * acc[mi][j + 2][v];
            const int piece = (2 * j + (pc >> 3)) ^ ((rl >> 2) & 3);
            *reinterpret_cast<uint16_t*>(sub + rl * 64 + piece * 16 + (pc & 7) * 2) =
                (uint16_t)(pack_f16x2(h, 0.f) & 0xffffu);
          }
      }
      lds_wave_sync();
      // 16 rows x 64 bytes per wave-wide read: lane -> row lane/4, piece lane%4
#pragma unroll
      for (int q = 0; q < BM / 16; ++q) {
        const int rl = q * 16 + (lane_o >> 2);
        const int p = lane_o & 3;
        const u32x4 d = ld16(sub + rl * 64 + (p ^ ((rl >> 2) & 3)) * 16);
        if (ts.cvalid && rl < rows) st16(C + (int64_t)(row0 + rl) * ldc + ts.c0 + p * 8, d);
      }
    } else {
      // y in two halves of 64 rows: this wave's half sub-tile is 64 rows x
      // 128 B (its 64 columns) in As2 or Ex; lane (r16, lg) holds columns
      // 16 f + 4 lg .. +3 of row 16 mi + r16, and the 16-byte piece p of row
      // r sits at p ^ (r & 7)
      uint8_t* sub = BM == 128 ? (wave < 4 ? As2 : Ex) + (wave & 3) * SUBW : Ex + wave * SUBW;
#pragma unroll
      for (int half = 0; half < BM / 64; ++half) {
#pragma unroll
        for (int mh = 0; mh < 4; ++mh) {
          const int mi = half * 4 + mh;
          const int rl = mh * 16 + rr;  // row within the half
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
        for (int q = 0; q < 8; ++q) {
          const int rl = q * 8 + (lane_o >> 3);
          const int p = lane_o & 7;
          const u32x4 d = ld16(sub + rl * 128 + (p ^ (rl & 7)) * 16);
          const int row = half * 64 + rl;
          if (ts.cvalid && row < rows) st16(C + (int64_t)(row0 + row) * ldc + ts.c0 + p * 8, d);
        }
      }
    }
  };

  // ---- persistent loop. K loop: activations two stages ahead in the LDS
  // ring, weights one stage ahead in registers. Within a stage the weight
  // loads are issued before the activation loads, so "at most ALD loads
  // outstanding" at the end of stage s means: stage s+1's activations and
  // weights have landed (loads complete in issue order). Every stage issues
  // the same loads (past the last stage they repeat it, into a slot nobody
  // reads), so the waits are the same at every stage and the compiler's own
  // wait bookkeeping stays exact. The next tile's first two stages are loaded
  // while this tile's epilogue runs: weights and stage 0 before it, stage 1
  // after its stores, so that "at most ALD outstanding" again means stage 0
  // has landed.
  int tile = t_begin + wg_in_xcd;
  if (tile >= t_end) return;
  const int klast = nk - 1;
  GemmTile cur;
  setup(tile, cur);
  WV cb[NFRAG];
  uint32_t rs[NFRAG], rm[NFRAG];
  f16x8 b0[NFRAG];  // dequantized weights of a stage's first K step
  load_sc(cur);
  load_b(cur, 0, cb, rs, rm);
  load_a(cur, 0, As0);
  load_a(cur, min(1, klast), As1);
  while (true) {
    refresh_lane();
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(ALD));
    lds_barrier();  // stage 0 in every wave; the previous epilogue is done with the LDS
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
    // stage kt reads ring slot kt % 3 and loads stage kt + 2 into slot (kt + 2) % 3
    // `odd`: kt is odd (a constant at every call), the stage that refills the
    // scale window with that of stages kt + 1, kt + 2
    auto stage = [&](int kt, const uint8_t* __restrict__ curs, uint8_t* __restrict__ nxt2,
                     bool odd) {
      WV cbn[NFRAG];
      uint32_t rsn[NFRAG], rmn[NFRAG];
      load_b(cur, min(kt + 1, klast), cbn, rsn, rmn);
      if (WIN && odd) load_win(cur, (kt + 1) >> 1);
      load_a(cur, min(kt + 2, klast), nxt2);
      // issue the loads here, a whole stage before they are needed: left to
      // itself the scheduler sinks them to the end of the stage (to shorten
      // register lifetimes), right before the wait for them
      __builtin_amdgcn_sched_barrier(0);
      if (XDQ && SCL) read_sc(sc_wave, min(kt + 1, klast), rsn, rmn);
      compute_stage(curs, cb, rs, rm, b0, cbn, rsn, rmn, kt);
      if (!XDQ && SCL) read_sc(sc_wave, min(kt + 1, klast), rsn, rmn);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(ALD));
      // (after the wait: a window refilled in this stage has landed)
      if (!XDQ && WIN) read_win(kt + 1, rsn, rmn);
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
    if (WIN) {
      // unrolled by six, so that the window refills sit at fixed stages
      for (int kt = 0; kt < nk; kt += 6) {
        stage(kt, As0, As2, false);
        if (kt + 1 < nk) stage(kt + 1, As1, As0, true);
        if (kt + 2 < nk) stage(kt + 2, As2, As1, false);
        if (kt + 3 < nk) stage(kt + 3, As0, As2, true);
        if (kt + 4 < nk) stage(kt + 4, As1, As0, false);
        if (kt + 5 < nk) stage(kt + 5, As2, As1, true);
      }
    } else {
      for (int kt = 0; kt < nk; kt += 3) {
        stage(kt, As0, As2, false);
        if (kt + 1 < nk) stage(kt + 1, As1, As0, false);
        if (kt + 2 < nk) stage(kt + 2, As2, As1, false);
      }
    }
    // the repeated loads of the last stages land before the ring is reused
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));

    const int next = tile + wgs_per_xcd;
    const bool has_next = next < t_end;
    GemmTile nts;
    refresh_lane();
    if (has_next) {
      setup(next, nts);
      load_sc(nts);
      load_b(nts, 0, cb, rs, rm);
      load_a(nts, 0, As0);
    }
    epilogue(cur);
    if (!has_next) break;
    load_a(nts, min(1, klast), As1);
    cur = nts;
    tile = next;
  }
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
