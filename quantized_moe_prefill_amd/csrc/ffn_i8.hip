// Integer route of the grouped expert GEMMs on gfx950: 8-bit activations x
// symmetric 4-bit weights on the int8 matrix cores.
//
// The pages admit an integer MoE prefill route for the symmetric expert
// file only (hipfire 0.4.3 benchmarks page, "Read this before comparing
// columns": the "symmetric IU4 MoE" route) and report an INT8 prefill route
// that replaced an F16 one (same page, "Qwen3.8-Flash (Flash-Next)" table).
// They fix no activation format. Here every activation row (x per token, h
// per (token, expert) row) is quantized to int8 with one fp32 scale per row.
// A weight code n (w = (n - 8) * scale) becomes the int8 value 16 (n - 8):
// xor 8 turns the nibble into a 4-bit two's complement number and a shift
// puts it in the high half of a byte, four instructions per eight weights.
// One quantization group (G = 128 along K) is then an exact int32 sum of two
// v_mfma_i32_16x16x64_i8; its fp16 scale / 16 is applied in fp32, and the
// row scale of the activations once at the end.
//
// The group sums reach fp32 without a conversion instruction: the first
// product of a group accumulates onto the integer bit pattern of
// M = 1.5 * 2^23, and since |sum| < 128 * 127 * 128 < 2^22 the result's bits
// read as the float M + sum exactly. The fp32 accumulator takes
// scale * (M + sum) in one fma and drops the offsets scale * M every three
// groups (one fma per result), which keeps its magnitude within a few group
// offsets: the rounding error stays near 2^-24 * 3M * scale per group, about
// 1e-4 of a typical group sum's contribution.
//
// Tile and schedule as in the fp16 grouped GEMM (ffn.hip): BM = 128 rows x
// BN = 512 weight rows per persistent 512-thread workgroup, eight waves of
// 64 weight rows each, the gathered int8 activation rows in a three-stage
// LDS ring filled by direct global->LDS loads two stages ahead, each wave's
// packed weights straight from global memory into registers one stage
// ahead, the tile list walked XCD by XCD. A stage is one group (K = 128):
// 16 KB of activations per stage instead of 32 KB for fp16. The group
// scales of a wave's 64 weight rows (up to 16 groups per row) come in once
// per tile, by two direct 1 KB loads into a per-wave LDS tile, instead of
// one 2-byte load per fragment and stage.
#include "common.h"
#include "kernels.h"

namespace qmoe {

namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128;           // rows per tile
constexpr int NWAVES = 8;
constexpr int NTHREADS = 64 * NWAVES;
constexpr int BN = 64 * NWAVES;   // weight rows per tile
constexpr int BK = 128;           // K per stage = the quantization group
constexpr int NXCD = 8;
constexpr int MSUB = BM / 16;
constexpr int NFRAG = 4;
constexpr int ALD = 2;            // direct activation loads per wave and stage (8 rows each)
constexpr int A_STAGE_BYTES = BM * BK;
constexpr int SUB_BYTES = BM * 64;  // one wave's epilogue sub-tile
// Per-wave scale tile: two 1 KB slots. Gate/up: slot 0 = the 32 gate rows'
// scales, slot 1 = the 32 up rows'; down: the 64 rows' scales over both.
constexpr int SC_SLOT = 1024;
constexpr int SC_WAVE = 2 * SC_SLOT;
constexpr int SC_MAX_GROUPS = 16;  // groups per row that fit
constexpr int kMagicBits = 0x4B400000;  // 1.5 * 2^23
constexpr float kMagic = 12582912.0f;
static_assert(ALD * NWAVES * 8 == BM, "the direct loads of a stage cover its rows");

// ---------------------------------------------------------------------------
// per-row quantization
// ---------------------------------------------------------------------------

// One wave per row: the row's max |v|, then q = rint(v * r) with r = 127 / a
// (both divisions correctly rounded: this file is built without fast-math),
// the product rounded to fp32 first. |v * r| <= 127 (1 + 2^-24) < 127.5, so
// no clamp is needed.
template <bool SRC_F16, bool GEMM_ORDER>
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ src,
                                                         int rows, int cols,
                                                         int8_t* __restrict__ q,
                                                         float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int nchunks = cols / 8;
  auto lo = [](uint32_t w) { return SRC_F16 ? f16lo(w) : bf16lo(w); };
  auto hi = [](uint32_t w) { return SRC_F16 ? f16hi(w) : bf16hi(w); };
  for (int row = blockIdx.x * 4 + (threadIdx.x >> 6); row < rows; row += gridDim.x * 4) {
    const uint16_t* s = src + (int64_t)row * cols;
    float a = 0.f;
    for (int c = lane; c < nchunks; c += 64) {
      const u32x4 d = ld16(s + c * 8);
#pragma unroll
      for (int i = 0; i < 4; ++i) a = fmaxf(a, fmaxf(fabsf(lo(d[i])), fabsf(hi(d[i]))));
    }
    a = wave_max(a);
    const bool ok = a >= 0x1p-100f;
    const float r = ok ? 127.f / a : 0.f;
    int8_t* qr = q + (int64_t)row * cols;
    for (int c = lane; c < nchunks; c += 64) {
      const u32x4 d = ld16(s + c * 8);
      uint32_t b[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        b[2 * i] = (uint32_t)(int)rintf(lo(d[i]) * r) & 0xffu;
        b[2 * i + 1] = (uint32_t)(int)rintf(hi(d[i]) * r) & 0xffu;
      }
      uint2 o;
      if (GEMM_ORDER) {  // elements 0,2,4,6 | 1,3,5,7
        o.x = b[0] | (b[2] << 8) | (b[4] << 16) | (b[6] << 24);
        o.y = b[1] | (b[3] << 8) | (b[5] << 16) | (b[7] << 24);
      } else {
        o.x = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
        o.y = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
      }
      *reinterpret_cast<uint2*>(qr + c * 8) = o;
    }
    if (lane == 0) scale[row] = ok ? a / 127.f : 0.f;
  }
}

// ---------------------------------------------------------------------------
// grouped int8 GEMM
// ---------------------------------------------------------------------------

// One tile's rows, this lane's activation sources and weight offsets (at
// namespace scope: a class local to a kernel template keeps the compiler
// from emitting the kernel's host-side launch stub).
struct TileI8 {
  int row0, rows, c0, par;
  bool cvalid;
  uint32_t a_off[ALD];
  uint32_t b_lane, s_lane;
  uint32_t sc_src[2];  // byte offsets of the two scale slots' sources
};


// Eight packed codes (one word, byte j = elements 2j | 2j+1 << 4) -> two
// words of int8 values 16 (n - 8): elements 0,2,4,6 and 1,3,5,7.
__device__ __forceinline__ void unpack8_i8(uint32_t w, uint32_t& even, uint32_t& odd) {
  const uint32_t t = w ^ 0x88888888u;
  even = (t << 4) & 0xF0F0F0F0u;
  odd = t & 0xF0F0F0F0u;
}

template <bool GATEUP, bool SCL>
__global__ __launch_bounds__(NTHREADS, 1) void expert_gemm_i8_kernel(GemmI8 g, int n_ntiles) {
  // LDS: the activation ring (128 rows x 128 bytes per stage; the 16-byte
  // chunk c of row r sits in slot c ^ (r & 7), so that the eight lanes of a
  // fragment read phase hit eight different bank groups), one epilogue
  // sub-tile per wave, the per-row activation scales of two tiles in flight.
  __shared__ __attribute__((aligned(16))) uint8_t As0[A_STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t As1[A_STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t As2[A_STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t Ep[NWAVES * SUB_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t Sc[SCL ? NWAVES * SC_WAVE : 16];
  __shared__ float s_rs[2][BM];
  __shared__ int s_scan[258];
  __shared__ int s_wave[NWAVES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = g.K, N = g.N;
  const int KG = K / BK;
  const int nk = K / BK;

  // ---- tile list: per-expert tile prefix ----
  {
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
    if (tid < 257) s_scan[tid + 1] = incl;
    if (tid == 0) s_scan[0] = 0;
    __syncthreads();
  }
  const int n_mtiles = s_scan[g.E];
  const int total = n_mtiles * n_ntiles;
  const int xcd = blockIdx.x % NXCD;
  const int wg_in_xcd = blockIdx.x / NXCD;
  const int wgs_per_xcd = gridDim.x / NXCD;
  const int t_begin = (int)((int64_t)total * xcd / NXCD);
  const int t_end = (int)((int64_t)total * (xcd + 1) / NXCD);

  // buffer resources (the host guarantees every size fits in 31 bits); a
  // read past the end returns zero
  const __amdgpu_buffer_rsrc_t rA =
      __builtin_amdgcn_make_buffer_rsrc((void*)g.A, 0, g.a_rows * K, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rW =
      __builtin_amdgcn_make_buffer_rsrc((void*)g.W, 0, g.E * N * (K / 2), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rS =
      __builtin_amdgcn_make_buffer_rsrc((void*)g.Wscale, 0, g.E * N * KG * 2, kRsrcWord3);

  // per-lane constants from an opaque copy of the lane index (so they are
  // recomputed per tile instead of held in registers across the loop)
  int lane_o = lane, r16, lg;
  auto refresh_lane = [&]() {
    asm volatile("" : "+v"(lane_o));
    r16 = lane_o & 15;
    lg = lane_o >> 4;
  };
  refresh_lane();
  // fragment f: weight rows c0 + frow(f) + 0..15 (gate/up: f = 0, 1 gate
  // columns c0 + 16 f, f = 2, 3 the up rows of the same columns)
  auto frow = [&](int f) { return GATEUP ? 16 * (f & 1) + (f < 2 ? 0 : N / 2) : 16 * f; };

  // Lane (r16, lg) covers K [32 lg, 32 lg + 32) of every stage: 16 bytes of
  // packed weights of row r16 of each fragment, and chunks 2 lg and 2 lg + 1
  // of its activation rows; chunk j feeds the j-th of the stage's two
  // 64-deep products.
  auto setup = [&](int tile, TileI8& ts, int par) {
    const int mtile = tile / n_ntiles;
    const int ntile = tile - mtile * n_ntiles;
    int lo = 0, hi = g.E;  // s_scan[lo] <= mtile < s_scan[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_scan[mid] <= mtile) lo = mid; else hi = mid;
    }
    const int e = lo;
    const int local = mtile - s_scan[e];
    ts.row0 = g.offsets[e] + local * BM;
    ts.rows = min(BM, g.counts[e] - local * BM);
    ts.par = par;
    // load i of wave w fills rows 8 (ALD w + i) .. +7; lane l writes row
    // 8 (ALD w + i) + l/8, slot l%8, i.e. source chunk (l%8) ^ (l/8)
    int src[ALD];
#pragma unroll
    for (int i = 0; i < ALD; ++i) {
      const int r = 8 * (ALD * wave + i) + (lane_o >> 3);
      src[i] = ts.row0 + (r < ts.rows ? r : 0);
    }
    if (g.gather != nullptr) {
#pragma unroll
      for (int i = 0; i < ALD; ++i) src[i] = g.gather[src[i]] / g.gather_div;
    }
#pragma unroll
    for (int i = 0; i < ALD; ++i)
      ts.a_off[i] = (uint32_t)src[i] * K + (uint32_t)(((lane_o & 7) ^ (lane_o >> 3)) * 16);
    ts.c0 = GATEUP ? ntile * (BN / 2) + wave * 32 : ntile * BN + wave * 64;
    ts.cvalid = ts.c0 < (GATEUP ? N / 2 : N);
    const int wrow0 = e * N + (ts.cvalid ? ts.c0 : 0) + r16;
    ts.b_lane = (uint32_t)wrow0 * (K / 2) + lg * 16;
    ts.s_lane = (uint32_t)wrow0 * KG * 2;
    if (SCL) {
      const uint32_t r0 = (uint32_t)(e * N + (ts.cvalid ? ts.c0 : 0));
      const uint32_t s0 = __builtin_amdgcn_readfirstlane(r0 * KG * 2);
      ts.sc_src[0] = s0;
      ts.sc_src[1] = GATEUP ? __builtin_amdgcn_readfirstlane((r0 + N / 2) * KG * 2) : s0 + SC_SLOT;
    }
    // the rows' activation scales (read by the epilogue, after at least one
    // workgroup barrier)
    if (tid < BM) {
      float sv = 0.f;
      if (tid < ts.rows) {
        int a = ts.row0 + tid;
        if (g.gather != nullptr) a = g.gather[a] / g.gather_div;
        sv = g.a_scale[a];
      }
      s_rs[par][tid] = sv;
    }
  };
  auto load_a = [&](const TileI8& ts, int kt, uint8_t* __restrict__ dst) {
#pragma unroll
    for (int i = 0; i < ALD; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_void_t*)(dst + 8 * (ALD * wave + i) * BK),
                                               16, ts.a_off[i], kt * BK, 0, 0);
  };
  auto load_b = [&](const TileI8& ts, int kt, u32x4* cb, uint32_t* rs) {
#pragma unroll
    for (int f = 0; f < NFRAG; ++f)
      cb[f] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            rW, ts.b_lane, frow(f) * (K / 2) + kt * (BK / 2), 0));
    if (!SCL) {
#pragma unroll
      for (int f = 0; f < NFRAG; ++f)
        rs[f] = __builtin_amdgcn_raw_buffer_load_b16(rS, ts.s_lane, frow(f) * KG * 2 + kt * 2, 0);
    }
  };
  // this wave's scale tile (past a block's end the loads read other rows'
  // scales or zeros, never used)
  uint8_t* const sc_wave = Sc + wave * (SCL ? SC_WAVE : 0);
  auto load_sc = [&](const TileI8& ts) {
    if (SCL) {
      const uint32_t lo = (uint32_t)lane_o * 16u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rS, (lds_void_t*)sc_wave, 16, lo, ts.sc_src[0], 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rS, (lds_void_t*)(sc_wave + SC_SLOT), 16, lo,
                                               ts.sc_src[1], 0, 0);
    }
  };
  // the scales of stage kt from the wave's scale tile
  auto read_sc = [&](const uint8_t* __restrict__ scw, int kt, uint32_t* rs) {
#pragma unroll
    for (int f = 0; f < NFRAG; ++f) {
      const int row = GATEUP ? 16 * (f & 1) + r16 : 16 * f + r16;
      const int off = (GATEUP && f >= 2 ? SC_SLOT : 0) + (row * KG + kt) * 2;
      rs[f] = *reinterpret_cast<const uint16_t*>(scw + off);
    }
  };

  f32x4 acc[MSUB][NFRAG];

  // One stage: the weights unpacked once, then per 16-row sub-tile two
  // int8 products per fragment (an exact group sum, offset by M) and one
  // fp32 fma per result with the group's scale; off[f] collects the scales
  // whose offsets are still in the accumulators.
  auto compute_stage = [&](const uint8_t* __restrict__ as_base, const u32x4* cb,
                           const uint32_t* rs, float* off) {
    i32x4 b0[NFRAG], b1[NFRAG];
    float sc[NFRAG];
#pragma unroll
    for (int f = 0; f < NFRAG; ++f) {
      sc[f] = f16_to_f32((uint16_t)rs[f]) * 0.0625f;
      off[f] += sc[f];
      uint32_t e0, o0, e1, o1, e2, o2, e3, o3;
      unpack8_i8(cb[f][0], e0, o0);
      unpack8_i8(cb[f][1], e1, o1);
      unpack8_i8(cb[f][2], e2, o2);
      unpack8_i8(cb[f][3], e3, o3);
      b0[f] = i32x4{(int)e0, (int)o0, (int)e1, (int)o1};
      b1[f] = i32x4{(int)e2, (int)o2, (int)e3, (int)o3};
    }
    const int sw = r16 & 7;
    const uint8_t* ap0 = as_base + r16 * BK + (((2 * lg) ^ sw) * 16);
    const uint8_t* ap1 = as_base + r16 * BK + (((2 * lg + 1) ^ sw) * 16);
    const i32x4 magic = {kMagicBits, kMagicBits, kMagicBits, kMagicBits};
#pragma unroll
    for (int mi = 0; mi < MSUB; ++mi) {
      const i32x4 a0 = __builtin_bit_cast(i32x4, ld16(ap0 + mi * 16 * BK));
      const i32x4 a1 = __builtin_bit_cast(i32x4, ld16(ap1 + mi * 16 * BK));
      i32x4 t[NFRAG];
#pragma unroll
      for (int f = 0; f < NFRAG; ++f) t[f] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0[f], magic, 0, 0, 0);
#pragma unroll
      for (int f = 0; f < NFRAG; ++f) t[f] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1[f], t[f], 0, 0, 0);
#pragma unroll
      for (int f = 0; f < NFRAG; ++f) {
        // (the whole vector is reinterpreted: a bit cast of one element of
        // an ext_vector_type value is compiled as a cast of element 0)
        const f32x4 tf = __builtin_bit_cast(f32x4, t[f]);
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[mi][f][v] = fmaf(sc[f], tf[v], acc[mi][f][v]);
      }
    }
  };

  // Epilogue: lane (r16, lg) holds rows 16 mi + 4 lg + v of weight column
  // c0 + frow(f) + r16. The results go through this wave's LDS sub-tile so
  // that they leave as 16-byte row pieces. Gate/up: h = silu(s g) * (s u)
  // with the row scale s, 128 rows x 32 columns of fp16; down: y = s acc,
  // 64 columns, in two halves of 64 rows.
  auto epilogue = [&](const TileI8& ts) {
    int rq = 4 * lg, row0 = ts.row0, rows = ts.rows;
    asm volatile("" : "+v"(rq), "+v"(row0), "+v"(rows));
    uint8_t* sub = Ep + wave * SUB_BYTES;
    const float* rsc = s_rs[ts.par];
    if (GATEUP) {
      // the 16-byte piece p of row r sits at p ^ ((r >> 2) & 3)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = 16 * j + r16;
#pragma unroll
        for (int mi = 0; mi < MSUB; ++mi)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int rl = mi * 16 + rq + v;
            const float s = rsc[rl];
            const float h = silu_f32(s * acc[mi][j][v]) * (s * acc[mi][j + 2][v]);
            const int piece = (col >> 3) ^ ((rl >> 2) & 3);
            *reinterpret_cast<uint16_t*>(sub + rl * 64 + piece * 16 + (col & 7) * 2) =
                (uint16_t)(pack_f16x2(h, 0.f) & 0xffffu);
          }
      }
      lds_wave_sync();
#pragma unroll
      for (int q = 0; q < BM / 16; ++q) {
        const int rl = q * 16 + (lane_o >> 2);
        const int p = lane_o & 3;
        const u32x4 d = ld16(sub + rl * 64 + (p ^ ((rl >> 2) & 3)) * 16);
        if (ts.cvalid && rl < rows) st16(g.C + (int64_t)(row0 + rl) * g.ldc + ts.c0 + p * 8, d);
      }
    } else {
      // half sub-tile: 64 rows x 128 B; the 16-byte piece p of row r sits
      // at p ^ (r & 7)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int mh = 0; mh < MSUB / 2; ++mh) {
          const int mi = half * (MSUB / 2) + mh;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int rl = mh * 16 + rq + v;  // row within the half
            const float s = rsc[half * 64 + rl];
#pragma unroll
            for (int f = 0; f < NFRAG; ++f) {
              const int col = 16 * f + r16;
              const int piece = (col >> 3) ^ (rl & 7);
              *reinterpret_cast<uint16_t*>(sub + rl * 128 + piece * 16 + (col & 7) * 2) =
                  (uint16_t)(pack_f16x2(s * acc[mi][f][v], 0.f) & 0xffffu);
            }
          }
        }
        lds_wave_sync();
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int rl = q * 8 + (lane_o >> 3);
          const int p = lane_o & 7;
          const u32x4 d = ld16(sub + rl * 128 + (p ^ (rl & 7)) * 16);
          const int row = half * 64 + rl;
          if (ts.cvalid && row < rows) st16(g.C + (int64_t)(row0 + row) * g.ldc + ts.c0 + p * 8, d);
        }
      }
    }
  };

  // ---- persistent loop; waits as in the fp16 kernel: within a stage the
  // weight (and scale) loads are issued before the activation loads, so "at
  // most ALD outstanding" at the end of stage s means stage s+1 has landed;
  // a tile's scale tile is loaded before its first weights.
  int tile = t_begin + wg_in_xcd;
  if (tile >= t_end) return;
  const int klast = nk - 1;
  TileI8 cur;
  int par = 0;
  setup(tile, cur, par);
  u32x4 cb[NFRAG];
  uint32_t rs[NFRAG];
  load_sc(cur);
  load_b(cur, 0, cb, rs);
  load_a(cur, 0, As0);
  load_a(cur, min(1, klast), As1);
  while (true) {
    refresh_lane();
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(ALD));
    lds_barrier();  // stage 0 in every wave; the previous epilogue is done with the LDS
    if (SCL) read_sc(sc_wave, 0, rs);
#pragma unroll
    for (int i = 0; i < MSUB; ++i)
#pragma unroll
      for (int j = 0; j < NFRAG; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    float off[NFRAG] = {0.f, 0.f, 0.f, 0.f};
    auto recenter = [&]() {
#pragma unroll
      for (int f = 0; f < NFRAG; ++f) {
#pragma unroll
        for (int i = 0; i < MSUB; ++i)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[i][f][v] = fmaf(-kMagic, off[f], acc[i][f][v]);
        off[f] = 0.f;
      }
    };
    auto stage = [&](int kt, const uint8_t* __restrict__ curs, uint8_t* __restrict__ nxt2) {
      u32x4 cbn[NFRAG];
      uint32_t rsn[NFRAG];
      load_b(cur, min(kt + 1, klast), cbn, rsn);
      load_a(cur, min(kt + 2, klast), nxt2);
      __builtin_amdgcn_sched_barrier(0);
      compute_stage(curs, cb, rs, off);
      if (SCL) read_sc(sc_wave, min(kt + 1, klast), rsn);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(ALD));
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int f = 0; f < NFRAG; ++f) {
        cb[f] = cbn[f];
        rs[f] = rsn[f];
      }
    };
    for (int kt = 0; kt < nk; kt += 3) {
      stage(kt, As0, As2);
      if (kt + 1 < nk) stage(kt + 1, As1, As0);
      if (kt + 2 < nk) stage(kt + 2, As2, As1);
      recenter();
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));

    const int next = tile + wgs_per_xcd;
    const bool has_next = next < t_end;
    TileI8 nts;
    refresh_lane();
    if (has_next) {
      setup(next, nts, par ^ 1);
      load_sc(nts);
      load_b(nts, 0, cb, rs);
      load_a(nts, 0, As0);
    }
    epilogue(cur);
    if (!has_next) break;
    load_a(nts, min(1, klast), As1);
    cur = nts;
    par ^= 1;
    tile = next;
  }
}

int g_i8_cus = 0;

template <bool GATEUP>
hipError_t launch_i8(const GemmI8& g, hipStream_t s, const char* name) {
  const bool scl = g.K / BK <= SC_MAX_GROUPS;
  const int n_ntiles = GATEUP ? cdiv(g.N / 2, BN / 2) : cdiv(g.N, BN);
  const int m_bound = cdiv(g.max_rows, BM) + g.E;
  if (g.max_rows <= 0) return hipSuccess;
  if (g_i8_cus == 0) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    err = hipDeviceGetAttribute(&g_i8_cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
  }
  int wgs = g_i8_cus;
  const int bound = cdiv(m_bound * n_ntiles, NXCD) * NXCD;
  if (wgs > bound) wgs = bound;
  wgs = cdiv(wgs, NXCD) * NXCD;
  LaunchScope ls(name, s);
  if (scl)
    hipLaunchKernelGGL((expert_gemm_i8_kernel<GATEUP, true>), dim3(wgs), dim3(NTHREADS), 0, s, g,
                       n_ntiles);
  else
    hipLaunchKernelGGL((expert_gemm_i8_kernel<GATEUP, false>), dim3(wgs), dim3(NTHREADS), 0, s, g,
                       n_ntiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_rows_i8(const uint16_t* src, bool src_f16, int rows, int cols,
                                bool gemm_order, int8_t* q, float* scale, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  int blocks = cdiv(rows, 4);
  if (blocks > 16384) blocks = 16384;
  LaunchScope ls(src_f16 ? "quant_h_i8" : "quant_x_i8", s);
  if (src_f16) {
    if (gemm_order)
      hipLaunchKernelGGL((quant_rows_kernel<true, true>), dim3(blocks), dim3(256), 0, s, src, rows, cols, q, scale);
    else
      hipLaunchKernelGGL((quant_rows_kernel<true, false>), dim3(blocks), dim3(256), 0, s, src, rows, cols, q, scale);
  } else {
    if (gemm_order)
      hipLaunchKernelGGL((quant_rows_kernel<false, true>), dim3(blocks), dim3(256), 0, s, src, rows, cols, q, scale);
    else
      hipLaunchKernelGGL((quant_rows_kernel<false, false>), dim3(blocks), dim3(256), 0, s, src, rows, cols, q, scale);
  }
  return hipGetLastError();
}

hipError_t launch_gateup_i8(const GemmI8& g, hipStream_t s) {
  return launch_i8<true>(g, s, "gateup_gemm_i8");
}
hipError_t launch_down_i8(const GemmI8& g, hipStream_t s) {
  return launch_i8<false>(g, s, "down_gemm_i8");
}

}  // namespace qmoe
