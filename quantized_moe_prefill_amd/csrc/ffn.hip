// Grouped expert GEMMs for the MoE prefill layer on gfx950.
//
// Rows are processed in expert-sorted blocks ("per-expert buffers" in the
// MoE prefill route of the hipfire 0.4.3 benchmarks page, section "Read this
// before comparing columns"); each expert's weights are 4-bit integers with
// an fp16 scale (and min) per group of G elements along K, as in that page's
// symmetric and asymmetric expert files ("Known limits").
//
// Tile: BM = 128 rows of one expert x BN = 256 weight rows, K in stages of
// 128. The gathered activation rows go through LDS (double buffered) and are
// read by all four waves; each wave owns 64 weight rows (four 16-column
// fragments) across all 128 rows, loads its packed weights straight from
// global memory (16 bytes = 32 K values per lane per fragment and stage) and
// dequantizes them in registers, so no weight is dequantized twice and no
// dequantized weight touches LDS. v_mfma_f32_16x16x32_f16 with fp32
// accumulators.
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
#include "common.h"
#include "kernels.h"

namespace qmoe {

namespace {

constexpr int BM = 128;          // rows per tile
#ifndef QMOE_NWAVES
#define QMOE_NWAVES 8
#endif
constexpr int NWAVES = QMOE_NWAVES;  // waves per workgroup, 64 weight rows each
constexpr int NTHREADS = 64 * NWAVES;
constexpr int BN = 64 * NWAVES;  // weight rows per tile
constexpr int BK = 128;          // K per pipeline stage
constexpr int NXCD = 8;
constexpr int MSUB = BM / 16;    // 16-row sub-tiles
constexpr int NFRAG = 4;         // 16-column fragments per wave
constexpr int WGS_PER_CU = 1;    // persistent workgroups per CU (one wave per SIMD)

// Eight consecutive 4-bit weights (one 32-bit word) of one row -> eight fp16
// weights in the kperm chunk order. OR-ing a nibble n into the fp16 pattern
// 0x6400 gives exactly 1024 + n; subtracting 1032 (symmetric) or 1024
// (asymmetric) is exact, and the final multiply (or fused multiply-add with
// the min) rounds once.
template <bool ASYM>
__device__ __forceinline__ f16x8 dequant8_f16(uint32_t w, f16x2 s2, f16x2 m2) {
  const f16x2 off = ASYM ? f16x2{(_Float16)1024.0f, (_Float16)1024.0f}
                         : f16x2{(_Float16)1032.0f, (_Float16)1032.0f};
  // the two constants live in registers so that mask-and-or is a single
  // v_and_or_b32 (VOP3 takes no literal and at most one scalar operand on gfx9)
  const uint32_t mask = __builtin_amdgcn_readfirstlane(0x000f000fu);
  const uint32_t magic = 0x64006400u;
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t t;  // (1024 + n_i, 1024 + n_{i+4}) as an fp16 pair
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(t) : "v"(w >> (4 * i)), "s"(mask), "v"(magic));
    const f16x2 n = __builtin_bit_cast(f16x2, t) - off;
    const f16x2 v = ASYM ? __builtin_elementwise_fma(n, s2, m2) : n * s2;
    o[i] = __builtin_bit_cast(uint32_t, v);
  }
  return __builtin_bit_cast(f16x8, o);
}

// bf16 activations -> fp16 in kperm chunk order (exact for |x| < 65504).
__global__ __launch_bounds__(256) void x_to_f16_kernel(const uint16_t* __restrict__ x,
                                                       uint16_t* __restrict__ out,
                                                       int64_t n_chunks) {
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < n_chunks;
       c += (int64_t)gridDim.x * 256) {
    const u32x4 d = ld16(x + c * 8);  // (x0,x1) (x2,x3) (x4,x5) (x6,x7)
    u32x4 o;
    o[0] = pack_f16x2(bf16lo(d[0]), bf16lo(d[2]));  // x0, x4
    o[1] = pack_f16x2(bf16hi(d[0]), bf16hi(d[2]));  // x1, x5
    o[2] = pack_f16x2(bf16lo(d[1]), bf16lo(d[3]));  // x2, x6
    o[3] = pack_f16x2(bf16hi(d[1]), bf16hi(d[3]));  // x3, x7
    st16(out + c * 8, o);
  }
}

__device__ __forceinline__ float silu(float z) { return z / (1.f + __expf(-z)); }

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

template <bool GATEUP, bool ASYM>
__global__ __launch_bounds__(NTHREADS, 1) void expert_gemm_kernel(GroupedGemm g, int n_ntiles) {
  // A tile, two stages, 128 rows x 128 fp16 each, no padding: the 16-byte
  // chunk c of row r sits in slot c ^ (r & 15) of its row, which keeps the
  // 16-row fragment reads free of bank conflicts and lets every wave fill
  // four whole rows per direct global->LDS load.
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM][BK];
  // packed weights of the stage, per wave: 64 rows x 64 bytes (128 K
  // nibbles); the 16-byte chunk c of row r sits at position c ^ ((r >> 1) & 3),
  // so the 16-row fragment reads are free of bank conflicts
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][NWAVES][64][64];
  __shared__ int s_scan[257];
  __shared__ int s_wave[NWAVES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = g.K, N = g.N;
  const int KG = K / g.G;
  const int nk = K / BK;

  // ---- tile list: per-expert tile prefix (tiles of BM rows) ----
  int n_mtiles;
  if (g.counts != nullptr) {
    const int c = tid < g.E ? g.counts[tid] : 0;
    int incl = (c + BM - 1) / BM;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    for (int w = 0; w < wave; ++w) incl += s_wave[w];
    if (tid < 256) s_scan[tid + 1] = incl;
    if (tid == 0) s_scan[0] = 0;
    __syncthreads();
    n_mtiles = s_scan[g.E];
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

  for (int tile = t_begin + wg_in_xcd; tile < t_end; tile += wgs_per_xcd) {
    // per-lane constants are derived from an opaque copy of the lane index in
    // every tile, so the compiler cannot compute them once up front and hold
    // them in registers across the whole persistent loop
    int lane_o = lane;
    asm volatile("" : "+v"(lane_o));
    const int r16 = lane_o & 15, lg = lane_o >> 4;
    const int mtile = tile / n_ntiles;
    const int ntile = tile - mtile * n_ntiles;

    // ---- which expert / rows ----
    int e, row0, rows;
    if (g.counts != nullptr) {
      // largest e with s_scan[e] <= mtile (binary search over the E+1 prefixes)
      int lo = 0, hi = g.E;  // s_scan[lo] <= mtile < s_scan[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_scan[mid] <= mtile) lo = mid; else hi = mid;
      }
      e = lo;
      const int local = mtile - s_scan[e];
      row0 = g.offsets[e] + local * BM;
      rows = min(BM, g.counts[e] - local * BM);
    } else {
      e = 0;
      row0 = mtile * BM;
      rows = min(BM, g.rows_single - row0);
    }

    // ---- A: this lane's source offsets for its direct loads per stage.
    // Load i of wave w fills rows 4*(ALD*w+i) .. +3; lane l covers row
    // 4*(ALD*w+i) + l/16, LDS slot l%16, i.e. source chunk (l%16) ^ (row & 15).
    // Rows past the expert's end read row 0 of the tile's source (finite
    // data whose outputs are never stored).
    // offsets are in 16-byte chunks (the host guarantees rows * K / 8 < 2^31)
    constexpr int ALD = 32 / NWAVES;
    int a_off[ALD];
#pragma unroll
    for (int i = 0; i < ALD; ++i) {
      const int r = 4 * (ALD * wave + i) + lg;
      const int ar = row0 + (r < rows ? r : 0);
      const int src = g.gather != nullptr ? g.gather[ar] / g.gather_div : ar;
      a_off[i] = src * (K / 8) + (r16 ^ (r & 15));
    }

    // ---- this wave's weight rows ----
    int wrow[NFRAG];
    bool fvalid[NFRAG];
#pragma unroll
    for (int f = 0; f < NFRAG; ++f) {
      if (GATEUP) {
        // fragments 0,1: gate columns c0 + 0..31 ; 2,3: up rows of the same columns
        const int I = N / 2;
        const int c = ntile * (BN / 2) + wave * 32 + (f & 1) * 16;
        fvalid[f] = c < I;
        wrow[f] = (f < 2 ? c : I + c) + r16;
      } else {
        const int c = ntile * BN + wave * 64 + f * 16;
        fvalid[f] = c < N;
        wrow[f] = c + r16;
      }
    }
    int wr_base[NFRAG];  // global weight row index (E * N < 2^24)
#pragma unroll
    for (int f = 0; f < NFRAG; ++f) wr_base[f] = e * N + (fvalid[f] ? wrow[f] : 0);

    // B staging: load f of this wave fills fragment f's 16 rows; lane l
    // covers row l/4 and LDS position l%4, i.e. source chunk (l%4) ^ ((row>>1)&3)
    const int b_row = lane >> 2;
    const int b_chunk = (lane & 3) ^ ((b_row >> 1) & 3);
    int b_src[NFRAG];  // this lane's source row (global weight row index)
#pragma unroll
    for (int f = 0; f < NFRAG; ++f) {
      int wr;
      if (GATEUP) {
        const int I = N / 2;
        const int c = ntile * (BN / 2) + wave * 32 + (f & 1) * 16;
        wr = (c < I) ? (f < 2 ? c : I + c) + b_row : 0;
      } else {
        const int c = ntile * BN + wave * 64 + f * 16;
        wr = (c < N) ? c + b_row : 0;
      }
      b_src[f] = e * N + wr;
    }

    uint32_t rs[NFRAG], rm[NFRAG];
    auto load_stage = [&](int kt, int buf) {
      const int k0 = kt * BK;
#pragma unroll
      for (int i = 0; i < ALD; ++i)
        __builtin_amdgcn_global_load_lds((glb_void_t*)(g.A + (int64_t)a_off[i] * 8 + k0),
                                         (lds_void_t*)&As[buf][4 * (ALD * wave + i)][0], 16, 0, 0);
#pragma unroll
      for (int f = 0; f < NFRAG; ++f)
        __builtin_amdgcn_global_load_lds(
            (glb_void_t*)(g.W + (int64_t)b_src[f] * (K / 2) + k0 / 2 + b_chunk * 16),
            (lds_void_t*)&Bs[buf][wave][f * 16][0], 16, 0, 0);
      const int grp = (k0 + lg * 32) / g.G;
#pragma unroll
      for (int f = 0; f < NFRAG; ++f) {
        rs[f] = (uint32_t)g.Wscale[(int64_t)wr_base[f] * KG + grp] * 0x10001u;
        rm[f] = ASYM ? (uint32_t)g.Wmin[(int64_t)wr_base[f] * KG + grp] * 0x10001u : 0u;
      }
    };

    f32x4 acc[MSUB][NFRAG];
#pragma unroll
    for (int i = 0; i < MSUB; ++i)
#pragma unroll
      for (int j = 0; j < NFRAG; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // One K stage on LDS buffer `buf`: four 32-wide K steps x eight 16-row
    // sub-tiles, flattened into 32 (step, sub-tile) slots of four MFMAs each.
    // A fragments are read two slots ahead through a three-deep rotation; the
    // next step's weights are dequantized while the current step's MFMAs run.
    // The scheduling groups pin one LDS read and four MFMAs per slot with two
    // VALU ops between MFMAs, so neither LDS latency nor dequant work sits on
    // the matrix core's critical path. Every sub-tile is computed; rows past
    // the end of an expert hold finite data whose results are never stored.
    auto compute_stage = [&](int buf, const f16x2* cs, const f16x2* cm) {
      // Per-lane LDS byte addresses; every other term of an address is a
      // compile-time offset (sub-tile, stage buffer, fragment), which keeps
      // the address state to five registers.
      const uint8_t* as_base = reinterpret_cast<const uint8_t*>(&As[buf][0][0]);
      const uint8_t* bs_base = reinterpret_cast<const uint8_t*>(&Bs[buf][wave][0][0]);
      u32x4 cb[NFRAG];  // this lane's packed weights of the stage (32 K values per fragment)
      {
        const uint8_t* bp = bs_base + r16 * 64 + ((lg ^ ((r16 >> 1) & 3)) * 16);
#pragma unroll
        for (int f = 0; f < NFRAG; ++f) cb[f] = ld16(bp + f * 16 * 64);
      }
      const uint8_t* ap[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) ap[j] = as_base + r16 * (BK * 2) + ((((lg * 4) ^ r16) ^ j) * 16);
      auto read_a = [&](int p) {
        const int j = p >> 3, mi = p & 7;
        return __builtin_bit_cast(f16x8, ld16(ap[j] + mi * 16 * BK * 2));
      };
      if constexpr (NWAVES >= 8) {
        // Two waves share each SIMD, so the hardware interleaves one wave's
        // dequant and LDS reads with the other's MFMAs: keep the live set
        // small (weights dequantized just in time, A read one sub-tile ahead).
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f16x8 b[NFRAG];
#pragma unroll
          for (int f = 0; f < NFRAG; ++f) b[f] = dequant8_f16<ASYM>(cb[f][j], cs[f], cm[f]);
          f16x8 a = read_a(j * 8);
#pragma unroll
          for (int mi = 0; mi < MSUB; ++mi) {
            f16x8 an;
            if (mi + 1 < MSUB) an = read_a(j * 8 + mi + 1);
#pragma unroll
            for (int f = 0; f < NFRAG; ++f) acc[mi][f] = mfma_16x16x32_f16(a, b[f], acc[mi][f]);
            if (mi + 1 < MSUB) a = an;
          }
        }
        return;
      }
      f16x8 abuf[3], b_cur[NFRAG], b_nxt[NFRAG];
      abuf[0] = read_a(0);
      abuf[1] = read_a(1);
#pragma unroll
      for (int f = 0; f < NFRAG; ++f) b_cur[f] = dequant8_f16<ASYM>(cb[f][0], cs[f], cm[f]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int p = 0; p < 32; ++p) {
        const int j = p >> 3, mi = p & 7;
        if (p + 2 < 32) abuf[(p + 2) % 3] = read_a(p + 2);
        if (mi == 0 && j + 1 < 4) {
#pragma unroll
          for (int f = 0; f < NFRAG; ++f) b_nxt[f] = dequant8_f16<ASYM>(cb[f][j + 1], cs[f], cm[f]);
        }
#pragma unroll
        for (int f = 0; f < NFRAG; ++f)
          acc[mi][f] = mfma_16x16x32_f16(abuf[p % 3], b_cur[f], acc[mi][f]);
        if (p + 2 < 32) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // 2 VALU
        }
        if (mi == 7 && j + 1 < 4) {
#pragma unroll
          for (int f = 0; f < NFRAG; ++f) b_cur[f] = b_nxt[f];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    auto k_loop = [&]() {
      load_stage(0, 0);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        // this stage's scales move to registers; the next stage's loads fly
        f16x2 cs[NFRAG], cm[NFRAG];
#pragma unroll
        for (int f = 0; f < NFRAG; ++f) {
          cs[f] = __builtin_bit_cast(f16x2, rs[f]);
          cm[f] = __builtin_bit_cast(f16x2, rm[f]);
        }
        if (kt + 1 < nk) load_stage(kt + 1, buf ^ 1);
        compute_stage(buf, cs, cm);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
      }
    };
    k_loop();

    // ---- epilogue ----
    // Opaque redefinitions of the per-lane row offsets: they are constants
    // per lane, and without this the compiler computes all 32 row indices
    // once at kernel start and holds them in registers through the K loop.
    int rq = 4 * lg;
    asm volatile("" : "+v"(rq), "+v"(row0), "+v"(rows));
    if (GATEUP) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (!fvalid[j]) continue;
        // h is the A operand of the down GEMM: stored in kperm chunk order
        const int col = wrow[j];
        const int pcol = (col & ~7) | kpos(col & 7);
#pragma unroll
        for (int mi = 0; mi < MSUB; ++mi)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int rl = mi * 16 + rq + v;
            if (rl < rows) {
              const float h = silu(acc[mi][j][v]) * acc[mi][j + 2][v];
              g.C[(int64_t)(row0 + rl) * g.ldc + pcol] = (uint16_t)(pack_f16x2(h, 0.f) & 0xffffu);
            }
          }
      }
    } else {
#pragma unroll
      for (int f = 0; f < NFRAG; ++f) {
        if (!fvalid[f]) continue;
        const int col = wrow[f];
#pragma unroll
        for (int mi = 0; mi < MSUB; ++mi)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int rl = mi * 16 + rq + v;
            if (rl < rows)
              g.C[(int64_t)(row0 + rl) * g.ldc + col] =
                  (uint16_t)(pack_f16x2(acc[mi][f][v], 0.f) & 0xffffu);
          }
      }
    }
  }
}

int g_num_cus = 0;

template <bool GATEUP>
hipError_t launch_grouped(const GroupedGemm& g, hipStream_t s, const char* name) {
  const int n_ntiles = GATEUP ? cdiv(g.N / 2, BN / 2) : cdiv(g.N, BN);
  const int m_bound =
      g.counts != nullptr ? cdiv(g.max_rows, BM) + g.E : cdiv(g.rows_single, BM);
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
  if (g.Wmin != nullptr)
    hipLaunchKernelGGL((expert_gemm_kernel<GATEUP, true>), grid, block, 0, s, g, n_ntiles);
  else
    hipLaunchKernelGGL((expert_gemm_kernel<GATEUP, false>), grid, block, 0, s, g, n_ntiles);
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

hipError_t launch_gateup(const GroupedGemm& g, hipStream_t s, const char* name) {
  return launch_grouped<true>(g, s, name);
}
hipError_t launch_down(const GroupedGemm& g, hipStream_t s, const char* name) {
  return launch_grouped<false>(g, s, name);
}

}  // namespace qmoe
