// Router for the MoE prefill layer on gfx950: fp32 router logits on the bf16
// matrix cores, then a wavefront-level top-k and softmax per token.
//
// The logits are an fp32 GEMM L = x * Wr^T over bf16 activations. Each fp32
// router weight is split exactly into three bf16 terms (w = w1 + w2 + w3,
// truncating the significand 8 bits at a time), so every bf16 x bf16 product
// on the matrix cores is exact and only the fp32 accumulation rounds - the
// same error class as an fp32 GEMM, at bf16 matrix-core speed.
//
//  router_split : Wr (+ shared gate row) -> Wsplit [3*Epad][H] bf16 (the three
//                 terms are separate rows, so the product is one dense GEMM)
//  router_gemm  : P[ks][t][n] = sum over the ks-th K slice of x[t] . Wsplit[n],
//                 fp32; 128 x 256 tiles, 8 waves, a three-stage ring of
//                 direct global->LDS loads; the K dimension is split across
//                 workgroups when there are too few token tiles to fill the GPU
//  router_select: L[t,e] = sum_ks ((P[e] + P[Epad+e]) + P[2Epad+e]) + b[e] in a
//                 fixed order, then top-k and softmax (16 lanes per token)
//
// For a few tokens (at most kRouterGemvT) the product is a plain fp32
// matrix-vector product instead, router_gemv: one workgroup per router row
// reads the fp32 row once and takes its dot product with every token (fp32
// multiply-add, same error class), writing the finished logits as the single
// plane router_select then reads; the split and the K slices are skipped.
#include "common.h"
#include "kernels.h"
#include "permute_impl.h"

namespace qmoe {

namespace {

constexpr int RBM = 128;   // tokens per GEMM tile
constexpr int RBN = 192;   // output columns (split rows) per tile: 3 x 128 experts = 2 tiles
constexpr int RBK = 64;    // K per stage
constexpr int RTHREADS = 512;

__global__ __launch_bounds__(256) void router_split_kernel(const float* __restrict__ wr,
                                                          const float* __restrict__ sg, int E,
                                                          int H, int Epad,
                                                          uint16_t* __restrict__ out) {
  const int64_t n = (int64_t)Epad * H;
  const int64_t plane = n;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int e = (int)(i / H);
    const int h = (int)(i - (int64_t)e * H);
    float w = 0.f;
    if (e < E)
      w = wr[(int64_t)e * H + h];
    else if (e == E && sg != nullptr)
      w = sg[h];
    const uint32_t u1 = __float_as_uint(w) & 0xffff0000u;  // top 8 significant bits
    const float r1 = w - __uint_as_float(u1);                // exact
    const uint32_t u2 = __float_as_uint(r1) & 0xffff0000u;  // next 8
    const float r2 = r1 - __uint_as_float(u2);               // exact, <= 8 bits left
    const uint32_t u3 = __float_as_uint(r2) >> 16;           // r2 fits bf16 exactly
    out[i] = (uint16_t)(u1 >> 16);
    out[plane + i] = (uint16_t)(u2 >> 16);
    out[2 * plane + i] = (uint16_t)u3;
  }
}

// Dense bf16 GEMM P = x * Wsplit^T over one K slice. LDS rows are 64 bf16
// (128 B, eight 16-byte chunks); chunk c of row r sits in slot c ^ (r & 7),
// which keeps the 16-row fragment reads conflict-free and lets one direct
// load fill eight whole rows. With x16 set, the workgroups of column tile 0
// also write their rows' fp16 copy in kperm chunk order (the expert GEMMs'
// operand, what x_to_f16 computes) from the tiles they stage anyway.
__global__ __launch_bounds__(RTHREADS, 1) void router_gemm_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, float* __restrict__ P,
    uint16_t* __restrict__ x16, int T, int H, int N, int n_mt, int n_nt, int ksplit) {
  // a three-slot ring in separate arrays, with the stage loop unrolled by
  // three: the compiler then sees that a stage's LDS reads never touch the
  // slot being filled, and does not wait for those loads before reading
  __shared__ __attribute__((aligned(16))) uint16_t As0[RBM][RBK];
  __shared__ __attribute__((aligned(16))) uint16_t As1[RBM][RBK];
  __shared__ __attribute__((aligned(16))) uint16_t As2[RBM][RBK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs0[RBN][RBK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs1[RBN][RBK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs2[RBN][RBK];
  typedef uint16_t ARow[RBK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;  // 2 x 4 waves, 64 x 48 each
  const int r16 = lane & 15, lg = lane >> 4;

  int b = blockIdx.x;
  const int ks = b % ksplit;
  b /= ksplit;
  const int nt = b % n_nt;
  const int mt = b / n_nt;
  const int row0 = mt * RBM, col0 = nt * RBN;
  const int klen = H / ksplit;
  const int kbeg = ks * klen;
  const int nst = klen / RBK;

  // direct loads: A 128 rows = 16 loads of 8 rows, B 192 rows = 24 loads;
  // wave w issues A loads 2w, 2w+1 and B loads 3w .. 3w+2 each stage
  // (buffer loads with 32-bit offsets: the host keeps x and the split
  // matrix below 2^31 bytes)
  const __amdgpu_buffer_rsrc_t rX =
      __builtin_amdgcn_make_buffer_rsrc((void*)x, 0, T * H * 2, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rB =
      __builtin_amdgcn_make_buffer_rsrc((void*)w, 0, N * H * 2, kRsrcWord3);
  const int lrow = lane >> 3, lslot = lane & 7;
  uint32_t a_off[2], b_off[3];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = (2 * wave + i) * 8 + lrow;
    const int t = min(row0 + r, T - 1);
    a_off[i] = (uint32_t)(t * H + kbeg + 8 * (lslot ^ (r & 7))) * 2u;
  }
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int r = (3 * wave + i) * 8 + lrow;
    const int n = min(col0 + r, N - 1);
    b_off[i] = (uint32_t)(n * H + kbeg + 8 * (lslot ^ (r & 7))) * 2u;
  }
  auto load_stage = [&](int s, ARow* __restrict__ A, ARow* __restrict__ B) {
    const int k0 = s * RBK * 2;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rX, (lds_void_t*)&A[(2 * wave + i) * 8][0], 16,
                                               a_off[i], k0, 0, 0);
#pragma unroll
    for (int i = 0; i < 3; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_void_t*)&B[(3 * wave + i) * 8][0], 16,
                                               b_off[i], k0, 0, 0);
  };

  // the fp16 copy: thread t converts chunks 2 (t % 4), +1 of tile row t / 4
  const bool write_x16 = x16 != nullptr && nt == 0;
  const int xr = tid >> 2, xc = 2 * (tid & 3);
  const bool xrow_ok = row0 + xr < T;
  uint16_t* const x16_row = write_x16 ? x16 + (int64_t)(row0 + xr) * H + kbeg : nullptr;

  f32x4 acc[4][3];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 3; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // stage s: slot (A, B) holds it; stage s + 2 is loaded into (A2, B2) (the
  // slot of stage s - 1, which every wave finished before the last barrier).
  // Each stage is five direct loads per wave, so "at most 5 outstanding"
  // after the loads of stage s + 2 means stage s + 1 has landed. Every stage
  // issues its loads (past the last stage they load it again, into a slot
  // no later stage reads), so the waits are the same at every stage and the
  // compiler's own wait bookkeeping stays exact.
  auto stage = [&](int s, const ARow* __restrict__ A, const ARow* __restrict__ B,
                   ARow* __restrict__ A2, ARow* __restrict__ B2) {
    load_stage(min(s + 2, nst - 1), A2, B2);
    if (write_x16 && xrow_ok) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int c = xc + q;
        st16(x16_row + s * RBK + 8 * c, bf16x8_to_f16_kperm(ld16(&A[xr][(c ^ (xr & 7)) * 8])));
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      bf16x8 a[4], bb[3];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ra = wm * 64 + i * 16 + r16;
        a[i] = __builtin_bit_cast(bf16x8, ld16(&A[ra][((j * 4 + lg) ^ (ra & 7)) * 8]));
      }
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const int rb = wn * 48 + i * 16 + r16;
        bb[i] = __builtin_bit_cast(bf16x8, ld16(&B[rb][((j * 4 + lg) ^ (rb & 7)) * 8]));
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 3; ++ni) acc[mi][ni] = mfma_16x16x32(a[mi], bb[ni], acc[mi][ni]);
    }
    // (stores of the fp16 copy count in vmcnt as well; the loads still land
    // in issue order, so the wait below still covers stage s + 1)
    // (the builtin, not inline asm: the compiler counts it in its own wait
    // bookkeeping and adds no conservative waits of its own)
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(5));
    lds_barrier();
  };

  load_stage(0, As0, Bs0);
  load_stage(min(1, nst - 1), As1, Bs1);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(5));
  lds_barrier();
  for (int s = 0; s < nst; s += 3) {
    stage(s, As0, Bs0, As2, Bs2);
    if (s + 1 < nst) stage(s + 1, As1, Bs1, As0, Bs0);
    if (s + 2 < nst) stage(s + 2, As2, Bs2, As1, Bs1);
  }
  // the repeated loads of the last stages land before the workgroup ends
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));

  float* Pk = P + (int64_t)ks * T * N;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 3; ++ni) {
      const int col = col0 + wn * 48 + ni * 16 + r16;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = row0 + wm * 64 + mi * 16 + 4 * lg + v;
        if (row < T && col < N) Pk[(int64_t)row * N + col] = acc[mi][ni][v];
      }
    }
}

// (value, index) order used by the selection: larger value first, then the
// lower index. idx < 0 marks "nothing".
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  if (ia < 0) return false;
  if (ib < 0) return true;
  return va > vb || (va == vb && ia < ib);
}

// DPP row patterns: after xor-1, xor-2 (quad_perm), half-mirror and mirror
// exchanges every lane of a 16-lane row has combined all 16 lanes.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ void best_step(float& bv, int& bi) {
  const float ov = __int_as_float(dpp<CTRL>(__float_as_int(bv)));
  const int oi = dpp<CTRL>(bi);
  if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
}

template <int CTRL>
__device__ __forceinline__ float sum_step(float x) {
  return x + __int_as_float(dpp<CTRL>(__float_as_int(x)));
}

// 16 lanes per token (16 tokens per 256-thread workgroup). Lane r holds the
// logits of experts 64*i + 4*r + c (i < Q/4, c < 4). Each of the k rounds
// takes the lane-local best, reduces it over the row with DPP exchanges and
// retires the winner; lane j keeps round j's winner for the softmax.
// Logits, top-k and softmax of token t (16 lanes per token: lane r of the
// group); the selected ids also go to lds_ids[t * k + j] if it is given.
template <int Q>
__device__ __forceinline__ void select_token(
    const float* __restrict__ P, int ksplit, int planes, int T, int E, int Epad, int k,
    const float* __restrict__ bias, int has_shared, float* __restrict__ logits_out,
    int32_t* __restrict__ ids_out, float* __restrict__ w_out, float* __restrict__ sw_out, int t,
    int32_t* lds_ids) {
  const int r = threadIdx.x & 15;
  const bool live = t < T;
  const int tt = live ? t : T - 1;
  const int N = planes * Epad;

  float v[Q];
#pragma unroll
  for (int i = 0; i < Q / 4; ++i) {
    const int e0 = 64 * i + 4 * r;
    f32x4 l = {0.f, 0.f, 0.f, 0.f};
    if (e0 < Epad) {
      if (planes == 1) {
        l = *reinterpret_cast<const f32x4*>(P + (int64_t)tt * N + e0);
      } else {
        for (int s = 0; s < ksplit; ++s) {
          const float* p = P + ((int64_t)s * T + tt) * N + e0;
          const f32x4 a = *reinterpret_cast<const f32x4*>(p);
          const f32x4 b = *reinterpret_cast<const f32x4*>(p + Epad);
          const f32x4 c = *reinterpret_cast<const f32x4*>(p + 2 * Epad);
          l += (a + b) + c;
        }
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = e0 + c;
      float x = l[c];
      if (e < E) {
        if (bias != nullptr) x += bias[e];
        if (logits_out != nullptr && live) logits_out[(int64_t)t * E + e] = x;
      } else if (e == E && has_shared && live) {
        sw_out[t] = 1.f / (1.f + expf(-x));
      }
      v[4 * i + c] = x;
    }
  }
  // the shared-gate column past the last lane's range (E a multiple of 64)
  if (has_shared && E >= 16 * Q && r == 0 && live) {
    float x = 0.f;
    if (planes == 1) {
      x = P[(int64_t)tt * N + E];
    } else {
      for (int s = 0; s < ksplit; ++s) {
        const float* p = P + ((int64_t)s * T + tt) * N + E;
        x += (p[0] + p[Epad]) + p[2 * Epad];
      }
    }
    sw_out[t] = 1.f / (1.f + expf(-x));
  }

  uint32_t avail = 0;  // bit q: v[q] is a candidate
#pragma unroll
  for (int q = 0; q < Q; ++q)
    if (64 * (q >> 2) + 4 * r + (q & 3) < E) avail |= 1u << q;

  float m0 = 0.f, selv = 0.f;
  int seli = 0;
  for (int j = 0; j < k; ++j) {
    float bv = 0.f;
    int bi = -1;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int e = 64 * (q >> 2) + 4 * r + (q & 3);
      if (((avail >> q) & 1) && better(v[q], e, bv, bi)) { bv = v[q]; bi = e; }
    }
    best_step<kDppXor1>(bv, bi);
    best_step<kDppXor2>(bv, bi);
    best_step<kDppHalfMirror>(bv, bi);
    best_step<kDppMirror>(bv, bi);
    if (j == 0) m0 = bv;
    if (r == j) { selv = bv; seli = bi; }
    if (((bi & 63) >> 2) == r) avail &= ~(1u << (4 * (bi >> 6) + (bi & 3)));
  }
  // softmax over the k winners (the largest is round 0's)
  const float ex = r < k ? expf(selv - m0) : 0.f;
  float sum = sum_step<kDppXor1>(ex);
  sum = sum_step<kDppXor2>(sum);
  sum = sum_step<kDppHalfMirror>(sum);
  sum = sum_step<kDppMirror>(sum);
  if (live && r < k) {
    ids_out[(int64_t)t * k + r] = seli;
    w_out[(int64_t)t * k + r] = ex * (1.f / sum);
    if (lds_ids != nullptr) lds_ids[t * k + r] = seli;
  }
}

template <int Q>
__global__ __launch_bounds__(256) void router_select_kernel(
    const float* __restrict__ P, int ksplit, int planes, int T, int E, int Epad, int k,
    const float* __restrict__ bias, int has_shared, float* __restrict__ logits_out,
    int32_t* __restrict__ ids_out, float* __restrict__ w_out, float* __restrict__ sw_out) {
  select_token<Q>(P, ksplit, planes, T, E, Epad, k, bias, has_shared, logits_out, ids_out, w_out,
                  sw_out, blockIdx.x * 16 + (threadIdx.x >> 4), nullptr);
}

// At most 16 tokens: top-k and softmax of every token (one workgroup, 16
// lanes per token) and then, in the same workgroup, the grouping of the
// (token, slot) pairs by expert (counts, offsets, sorted_pairs, inv, as
// permute computes them), the ids handed over in LDS.
template <int Q>
__global__ __launch_bounds__(PT) void router_select_permute_kernel(
    const float* __restrict__ P, int T, int E, int Epad, int k, int nbits,
    const float* __restrict__ bias, int has_shared, int32_t* __restrict__ ids_out,
    float* __restrict__ w_out, float* __restrict__ sw_out, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pairs,
    int32_t* __restrict__ inv) {
  __shared__ int32_t s_ids[16 * 8];
  __shared__ int cnt[4][PMAXE];
  __shared__ int s_off[PMAXE];
  __shared__ int s_wave[4];
  select_token<Q>(P, 1, 1, T, E, Epad, k, bias, has_shared, nullptr, ids_out, w_out, sw_out,
                  threadIdx.x >> 4, s_ids);
  __syncthreads();
  const int Pn = T * k;
  const int tid = threadIdx.x, wave = tid >> 6;
  int ev[PSEG], rk[PSEG];
  const int total = chunk_ranks(s_ids, Pn, E, nbits, 0, cnt, ev, rk);
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
    if (p < Pn) {
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

// L[t][n] = sum_h f32(x[t][h]) * w[n][h] for the E router rows and the
// shared-gate row (n = E), T <= kRouterGemvT tokens. One workgroup per row
// n; wave w takes the K quarter [w H/4, (w + 1) H/4), lane l the values 8 l
// .. 8 l + 7 of every 512-wide piece of it, reading the fp32 row and every
// token's bf16 values straight from memory. The per-lane sums are reduced
// across the wave, then across the four waves, in a fixed order.
__global__ __launch_bounds__(256) void router_gemv_kernel(const uint16_t* __restrict__ x,
                                                          const float* __restrict__ wr,
                                                          const float* __restrict__ sg, int T,
                                                          int H, int E, int Epad,
                                                          float* __restrict__ out) {
  __shared__ float part[4][kRouterGemvT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = blockIdx.x;
  const int rows = E + (sg != nullptr ? 1 : 0);
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc((void*)x, 0, T * H * 2, kRsrcWord3);
  float acc[kRouterGemvT];
#pragma unroll
  for (int t = 0; t < kRouterGemvT; ++t) acc[t] = 0.f;
  if (n < rows) {
    const float* wrow = n < E ? wr + (int64_t)n * H : sg;  // n == E: the shared gate
    const int kq = H / 4;
    for (int c = 0; c < kq; c += 512) {
      const int k = wave * kq + c + 8 * lane;
      if (c + 8 * lane < kq) {
        const f32x4 w0 = *reinterpret_cast<const f32x4*>(wrow + k);
        const f32x4 w1 = *reinterpret_cast<const f32x4*>(wrow + k + 4);
        u32x4 xv[kRouterGemvT];
#pragma unroll
        for (int t = 0; t < kRouterGemvT; ++t) {
          // past the last token: past the end of x, which reads zero
          const uint32_t off = t < T ? (uint32_t)(t * H + k) * 2u : 0x7ffffff0u;
          xv[t] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
        }
#pragma unroll
        for (int t = 0; t < kRouterGemvT; ++t) {
          float a = acc[t];
          a = fmaf(bf16lo(xv[t][0]), w0[0], a);
          a = fmaf(bf16hi(xv[t][0]), w0[1], a);
          a = fmaf(bf16lo(xv[t][1]), w0[2], a);
          a = fmaf(bf16hi(xv[t][1]), w0[3], a);
          a = fmaf(bf16lo(xv[t][2]), w1[0], a);
          a = fmaf(bf16hi(xv[t][2]), w1[1], a);
          a = fmaf(bf16lo(xv[t][3]), w1[2], a);
          a = fmaf(bf16hi(xv[t][3]), w1[3], a);
          acc[t] = a;
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kRouterGemvT; ++t) acc[t] = wave_sum(acc[t]);
  if (lane == 0) {
#pragma unroll
    for (int t = 0; t < kRouterGemvT; ++t) part[wave][t] = acc[t];
  }
  __syncthreads();
  if (tid < T) out[(int64_t)tid * Epad + n] = ((part[0][tid] + part[1][tid]) + part[2][tid]) + part[3][tid];
}

int router_ksplit(int T, int E, bool has_shared, int H) {
  const int N = 3 * router_padded_rows(E, has_shared);
  const int tiles = cdiv(T, RBM) * cdiv(N, RBN);
  int ks = 1;
  while (ks < 16 && tiles * ks * 2 <= 256 && (H / RBK) % (ks * 2) == 0) ks *= 2;
  return ks;
}

}  // namespace

bool router_uses_gemv(int T) { return T <= kRouterGemvT; }

hipError_t launch_route_permute_small(const uint16_t* x, const float* w_router,
                                      const float* shared_gate, float* partial, const float* bias,
                                      int T, int H, int E, int k, int32_t* ids, float* topk_w,
                                      float* shared_w, int32_t* counts, int32_t* offsets,
                                      int32_t* sorted_pairs, int32_t* inv, hipStream_t s) {
  const bool has_shared = shared_gate != nullptr;
  const int Epad = router_padded_rows(E, has_shared);
  {
    LaunchScope ls("router_gemm", s);
    hipLaunchKernelGGL(router_gemv_kernel, dim3(Epad), dim3(256), 0, s, x, w_router, shared_gate,
                       T, H, E, Epad, partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const int hs = has_shared ? 1 : 0;
  LaunchScope ls("router_select", s);
  if (E <= 64)
    hipLaunchKernelGGL(router_select_permute_kernel<4>, dim3(1), dim3(PT), 0, s, partial, T, E, Epad,
                       k, nbits, bias, hs, ids, topk_w, shared_w, counts, offsets, sorted_pairs, inv);
  else if (E <= 128)
    hipLaunchKernelGGL(router_select_permute_kernel<8>, dim3(1), dim3(PT), 0, s, partial, T, E, Epad,
                       k, nbits, bias, hs, ids, topk_w, shared_w, counts, offsets, sorted_pairs, inv);
  else
    hipLaunchKernelGGL(router_select_permute_kernel<16>, dim3(1), dim3(PT), 0, s, partial, T, E,
                       Epad, k, nbits, bias, hs, ids, topk_w, shared_w, counts, offsets,
                       sorted_pairs, inv);
  return hipGetLastError();
}

int router_padded_rows(int E, bool has_shared) { return cdiv(E + (has_shared ? 1 : 0), 16) * 16; }

size_t router_split_bytes(int E, bool has_shared, int H) {
  return (size_t)3 * router_padded_rows(E, has_shared) * H * sizeof(uint16_t);
}

size_t router_partial_bytes(int T, int E, bool has_shared, int H) {
  const int N = 3 * router_padded_rows(E, has_shared);
  return (size_t)router_ksplit(T, E, has_shared, H) * T * N * sizeof(float);
}

hipError_t launch_router_split(const float* w_router, const float* shared_gate, int E, int H,
                               uint16_t* split, hipStream_t s) {
  const int Epad = router_padded_rows(E, shared_gate != nullptr);
  const int64_t n = (int64_t)Epad * H;
  int blocks = (int)((n + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  LaunchScope ls("router_split", s);
  hipLaunchKernelGGL(router_split_kernel, dim3(blocks), dim3(256), 0, s, w_router, shared_gate, E,
                     H, Epad, split);
  return hipGetLastError();
}

hipError_t launch_router_topk(const uint16_t* x, const float* w_router, const float* shared_gate,
                              const uint16_t* split, float* partial, const float* bias, int T,
                              int H, int E, int k, float* logits, int32_t* ids, float* topk_w,
                              float* shared_w, uint16_t* x16, hipStream_t s) {
  const bool has_shared = shared_gate != nullptr;
  const int Epad = router_padded_rows(E, has_shared);
  int ks = 1, planes = 1;
  if (router_uses_gemv(T)) {
    // the finished fp32 logits, one plane [T][Epad]
    LaunchScope ls("router_gemm", s);
    hipLaunchKernelGGL(router_gemv_kernel, dim3(Epad), dim3(256), 0, s, x, w_router, shared_gate,
                       T, H, E, Epad, partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else {
    const int N = 3 * Epad;
    const int n_mt = cdiv(T, RBM), n_nt = cdiv(N, RBN);
    ks = router_ksplit(T, E, has_shared, H);
    planes = 3;
    LaunchScope ls("router_gemm", s);
    hipLaunchKernelGGL(router_gemm_kernel, dim3(n_mt * n_nt * ks), dim3(RTHREADS), 0, s, x,
                       split, partial, x16, T, H, N, n_mt, n_nt, ks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  LaunchScope ls("router_select", s);
  const dim3 grid(cdiv(T, 16)), block(256);
  const int hs = has_shared ? 1 : 0;
  if (E <= 64)
    hipLaunchKernelGGL(router_select_kernel<4>, grid, block, 0, s, partial, ks, planes, T, E, Epad,
                       k, bias, hs, logits, ids, topk_w, shared_w);
  else if (E <= 128)
    hipLaunchKernelGGL(router_select_kernel<8>, grid, block, 0, s, partial, ks, planes, T, E, Epad,
                       k, bias, hs, logits, ids, topk_w, shared_w);
  else
    hipLaunchKernelGGL(router_select_kernel<16>, grid, block, 0, s, partial, ks, planes, T, E,
                       Epad, k, bias, hs, logits, ids, topk_w, shared_w);
  return hipGetLastError();
}

}  // namespace qmoe
