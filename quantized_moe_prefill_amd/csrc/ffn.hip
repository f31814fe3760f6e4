// Grouped expert GEMMs for the MoE prefill layer on gfx950.
//
// Rows are processed in expert-sorted blocks ("per-expert buffers" in the
// MoE prefill route of the hipfire 0.4.3 benchmarks page, section "Read this
// before comparing columns"); each expert's weights are 4-bit integers with
// an fp16 scale (and min) per group of G elements along K, as in that page's
// symmetric and asymmetric expert files ("Known limits").
//
// One workgroup computes a BM x BN tile of one expert: activation rows are
// gathered (gate/up: token = sorted_pairs[r] / k) into LDS, the packed weight
// tile is read once per workgroup and dequantized to fp16 into LDS with
// packed fp16 arithmetic (w = q*s rounded once), and four waves (2 x 2) run
// v_mfma_f32_16x16x32_f16 on 64 x 64 sub-tiles with fp32 accumulators. The
// gate/up kernel pairs gate and up rows of the same intermediate columns in
// one tile so that h = silu(g) * u is formed in registers and written once.
//
// Operands are fp16 rather than bf16: the matrix cores run both at the same
// rate, and fp16's three extra significand bits on the dequantized weights,
// on h and on the expert outputs are what keeps the layer output within its
// error budget. Activations arrive as bf16 and are converted exactly (for
// |x| < 65504) by x_to_f16 before the gate/up GEMM.
#include "common.h"
#include "kernels.h"

namespace qmoe {

namespace {

constexpr int BM = 128;       // rows per tile
constexpr int BNW = 128;      // weight rows per tile
constexpr int BK = 64;        // K per pipeline stage
constexpr int PITCH = BK + 8; // LDS row pitch in bf16 elements (144 B: conflict-free b128 reads)

// 32 consecutive 4-bit weights of one row (one group-aligned block, scale s
// and min m as fp16 pairs) -> 32 fp16 weights in the kperm chunk order.
// OR-ing a nibble n into the fp16 pattern 0x6400 gives exactly 1024 + n;
// subtracting 1032 (symmetric) or 1024 (asymmetric) is exact, and the final
// multiply (or fused multiply-add with the min) rounds once.
template <bool ASYM>
__device__ __forceinline__ void dequant32_f16(u32x4 q, uint32_t s2bits, uint32_t m2bits,
                                              uint16_t* dst) {
  const f16x2 s2 = __builtin_bit_cast(f16x2, s2bits);
  const f16x2 m2 = __builtin_bit_cast(f16x2, m2bits);
  const f16x2 off = ASYM ? f16x2{(_Float16)1024.0f, (_Float16)1024.0f}
                         : f16x2{(_Float16)1032.0f, (_Float16)1032.0f};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t w = q[j];
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t t = ((w >> (4 * i)) & 0x000f000fu) | 0x64006400u;  // (1024+n_i, 1024+n_{i+4})
      const f16x2 n = __builtin_bit_cast(f16x2, t) - off;
      const f16x2 v = ASYM ? __builtin_elementwise_fma(n, s2, m2) : n * s2;
      o[i] = __builtin_bit_cast(uint32_t, v);
    }
    st16(dst + 8 * j, o);
  }
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

template <bool GATEUP, bool ASYM>
__global__ __launch_bounds__(256, 2) void grouped_gemm_kernel(GroupedGemm g, int n_ntiles) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM][PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BNW][PITCH];
  __shared__ int s_scan[257];
  __shared__ int s_wave[4];
  __shared__ int s_e;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int mtile = blockIdx.x / n_ntiles;
  const int ntile = blockIdx.x - mtile * n_ntiles;
  const int K = g.K, N = g.N;

  // ---- which expert / rows does this tile cover ----
  int e, row0, rows;
  if (g.counts != nullptr) {
    const int c = tid < g.E ? g.counts[tid] : 0;
    const int tl = (c + BM - 1) / BM;
    int incl = tl;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    if (lane == 63) s_wave[wave] = incl;
    if (tid == 0) s_e = -1;
    __syncthreads();
    int wb = 0;
    for (int w = 0; w < wave; ++w) wb += s_wave[w];
    incl += wb;
    s_scan[tid + 1] = incl;
    if (tid == 0) s_scan[0] = 0;
    __syncthreads();
    if (tid < g.E && mtile >= s_scan[tid] && mtile < s_scan[tid + 1]) s_e = tid;
    __syncthreads();
    e = s_e;
    if (e < 0) return;  // beyond the last tile: uniform exit
    const int local = mtile - s_scan[e];
    const int ce = g.counts[e];
    row0 = g.offsets[e] + local * BM;
    rows = min(BM, ce - local * BM);
  } else {
    e = 0;
    row0 = mtile * BM;
    rows = min(BM, g.rows_single - row0);
    if (rows <= 0) return;
  }

  // ---- staging assignments ----
  const int a_kc = tid & 7;  // 16-byte chunk of a BK-wide row
  const uint16_t* a_src[4];
  bool a_ok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 3) + 32 * i;
    a_ok[i] = r < rows;
    int src = 0;
    if (a_ok[i]) {
      const int ar = row0 + r;
      src = g.gather != nullptr ? g.gather[ar] / g.gather_div : ar;
    }
    a_src[i] = g.A + (int64_t)src * K + a_kc * 8;
  }
  const int b_wrow = tid >> 1, b_half = tid & 1;
  int gw;
  if (GATEUP) {
    const int I = N / 2;
    const int n0 = ntile * (BNW / 2);
    gw = b_wrow < BNW / 2 ? n0 + b_wrow : I + n0 + (b_wrow - BNW / 2);
  } else {
    gw = ntile * BNW + b_wrow;
  }
  const int KG = K / g.G;
  const int64_t wrow_index = (int64_t)e * N + gw;
  const uint8_t* b_src = g.W + wrow_index * (K / 2) + b_half * 16;
  const uint16_t* sc_src = g.Wscale + wrow_index * KG;
  const uint16_t* mn_src = ASYM ? g.Wmin + wrow_index * KG : nullptr;

  u32x4 ra[4];
  u32x4 rb;
  uint32_t rs, rm = 0;
  auto load_stage = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) ra[i] = a_ok[i] ? ld16(a_src[i] + k0) : u32x4{0u, 0u, 0u, 0u};
    rb = ld16(b_src + k0 / 2);
    const int grp = (k0 + b_half * 32) / g.G;
    rs = (uint32_t)sc_src[grp] * 0x10001u;
    if (ASYM) rm = (uint32_t)mn_src[grp] * 0x10001u;
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) st16(&As[buf][(tid >> 3) + 32 * i][a_kc * 8], ra[i]);
    dequant32_f16<ASYM>(rb, rs, rm, &Bs[buf][b_wrow][b_half * 32]);
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = K / BK;
  load_stage(0);
  store_stage(0);
  __syncthreads();

  const int r16 = lane & 15, kq = 8 * (lane >> 4);
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_stage(kt + 1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      f16x8 a[4], b[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        a[mi] = __builtin_bit_cast(f16x8, ld16(&As[buf][wm * 64 + mi * 16 + r16][ks * 32 + kq]));
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        int brow;
        if (GATEUP)
          brow = (ni < 2) ? wn * 32 + ni * 16 : BNW / 2 + wn * 32 + (ni - 2) * 16;
        else
          brow = wn * 64 + ni * 16;
        b[ni] = __builtin_bit_cast(f16x8, ld16(&Bs[buf][brow + r16][ks * 32 + kq]));
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = mfma_16x16x32_f16(a[mi], b[ni], acc[mi][ni]);
    }
    if (kt + 1 < nk) store_stage(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue ----
  const int rq = 4 * (lane >> 4);
  if (GATEUP) {
    const int n0 = ntile * (BNW / 2);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        // h is the A operand of the down GEMM: store it in kperm chunk order
        const int col = n0 + wn * 32 + j * 16 + r16;
        const int pcol = (col & ~7) | kpos(col & 7);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int rl = wm * 64 + mi * 16 + rq + v;
          if (rl < rows) {
            const float h = silu(acc[mi][j][v]) * acc[mi][j + 2][v];
            g.C[(int64_t)(row0 + rl) * g.ldc + pcol] = (uint16_t)(pack_f16x2(h, 0.f) & 0xffffu);
          }
        }
      }
  } else {
    const int n0 = ntile * BNW;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int col = n0 + wn * 64 + ni * 16 + r16;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int rl = wm * 64 + mi * 16 + rq + v;
          if (rl < rows)
            g.C[(int64_t)(row0 + rl) * g.ldc + col] =
                (uint16_t)(pack_f16x2(acc[mi][ni][v], 0.f) & 0xffffu);
        }
      }
  }
}

template <bool GATEUP>
hipError_t launch_grouped(const GroupedGemm& g, hipStream_t s, const char* name) {
  const int n_ntiles = GATEUP ? (g.N / 2) / (BNW / 2) : g.N / BNW;
  const int m_tiles =
      g.counts != nullptr ? cdiv(g.max_rows, BM) + g.E : cdiv(g.rows_single, BM);
  if (m_tiles <= 0) return hipSuccess;
  const dim3 grid(m_tiles * n_ntiles), block(256);
  LaunchScope ls(name, s);
  if (g.Wmin != nullptr)
    hipLaunchKernelGGL((grouped_gemm_kernel<GATEUP, true>), grid, block, 0, s, g, n_ntiles);
  else
    hipLaunchKernelGGL((grouped_gemm_kernel<GATEUP, false>), grid, block, 0, s, g, n_ntiles);
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
