// Router for the MoE prefill layer on gfx950: fp32 router logits on the bf16
// matrix cores, then a wavefront-level top-k and softmax per token.
//
// The logits are an fp32 GEMM L = x * Wr^T over bf16 activations. Each fp32
// router weight is split exactly into three bf16 terms (w = w1 + w2 + w3,
// truncating the significand 8 bits at a time), so every bf16 x bf16 product
// on the matrix cores is exact and only the fp32 accumulation rounds - the
// same error class as an fp32 GEMM, at bf16 matrix-core speed.
//
//  router_split : Wr (+ shared gate row) -> Wsplit [3][Epad][H] bf16 (one
//                 plane per term)
//  router_gemm  : P[ks][t][e] = sum over the ks-th K slice of x[t] . (the three
//                 terms of row e), fp32, the three terms accumulated into the
//                 same accumulator (they are three more K steps of the same
//                 dot product); tiles of 128 tokens x 64 router rows (192 split
//                 rows), 8 waves, a three-stage ring of direct global->LDS
//                 loads; the K dimension is split across workgroups when there
//                 are too few token tiles to fill the GPU
//  router_select: L[t,e] = sum_ks P[ks][t][e] + b[e] in plane order, then top-k
//                 and softmax (16 lanes per token)
//
// For a few tokens (at most kRouterGemvT) the product is a plain fp32
// matrix-vector product instead, router_gemv: one workgroup per router row
// reads the fp32 row once and takes its dot product with every token (fp32
// multiply-add, same error class), writing the finished logits as the single
// plane router_select then reads; the split and the K slices are skipped.
#include "common.h"
#include "kernels.h"
#include "permute_impl.h"
#include "select_impl.h"

namespace qmoe {

namespace {

constexpr int RBM = 128;   // tokens per GEMM tile
constexpr int RBE = 64;    // router rows per tile
constexpr int RBN = 3 * RBE;  // split rows per tile (the three terms of each row)
constexpr int RBK = 64;    // K per stage
constexpr int RTHREADS = 512;

// Three bf16 terms per fp32 router weight whose sum is the weight exactly.
// Thread (x, row) takes eight consecutive weights of router row blockIdx.y
// (the shared gate after the E experts, zeros up to Epad): two 16-byte
// loads, one 16-byte store per term.
__global__ __launch_bounds__(256) void router_split_kernel(const float* __restrict__ wr,
                                                          const float* __restrict__ sg, int E,
                                                          int H, int Epad,
                                                          uint16_t* __restrict__ out) {
  const int e = blockIdx.y;
  const int h = 8 * (blockIdx.x * blockDim.x + threadIdx.x);
  if (h >= H) return;
  const float* src = e < E ? wr + (int64_t)e * H : (e == E ? sg : nullptr);
  float w[8];
  if (src != nullptr) {
    const u32x4 a = ld16(src + h), b = ld16(src + h + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w[i] = __uint_as_float(a[i]);
      w[4 + i] = __uint_as_float(b[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = 0.f;
  }
  u32x4 t1, t2, t3;
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    uint32_t hi[3][2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float x = w[i + j];
      const uint32_t u1 = __float_as_uint(x) & 0xffff0000u;  // top 8 significant bits
      const float r1 = x - __uint_as_float(u1);                // exact
      const uint32_t u2 = __float_as_uint(r1) & 0xffff0000u;  // next 8
      const float r2 = r1 - __uint_as_float(u2);               // exact, <= 8 bits left
      hi[0][j] = u1 >> 16;
      hi[1][j] = u2 >> 16;
      hi[2][j] = __float_as_uint(r2) >> 16;                    // r2 fits bf16 exactly
    }
    t1[i / 2] = hi[0][0] | (hi[0][1] << 16);
    t2[i / 2] = hi[1][0] | (hi[1][1] << 16);
    t3[i / 2] = hi[2][0] | (hi[2][1] << 16);
  }
  const int64_t plane = (int64_t)Epad * H, o = (int64_t)e * H + h;
  st16(out + o, t1);
  st16(out + plane + o, t2);
  st16(out + 2 * plane + o, t3);
}

// bf16 GEMM P = x * (sum of the three split terms)^T over one K slice. LDS
// rows are 64 bf16 (128 B, eight 16-byte chunks); chunk c of row r sits in
// slot c ^ (r & 7), which keeps the 16-row fragment reads conflict-free and
// lets one direct load fill eight whole rows. The B tile holds the three
// terms of RBE router rows (tile row 64 term + j). With x16 set, the
// workgroups of column tile 0 also write their rows' fp16 copy in kperm chunk
// order (the expert GEMMs' operand, what x_to_f16 computes) from the tiles
// they stage anyway.
__global__ __launch_bounds__(RTHREADS, 1) void router_gemm_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, float* __restrict__ P,
    uint16_t* __restrict__ x16, int T, int H, int Epad, int n_mt, int n_nt, int ksplit) {
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
  const int wm = wave >> 2, wn = wave & 3;  // 2 x 4 waves, 64 tokens x 16 rows each
  const int r16 = lane & 15, lg = lane >> 4;

  int b = blockIdx.x;
  const int ks = b % ksplit;
  b /= ksplit;
  const int nt = b % n_nt;
  const int mt = b / n_nt;
  const int row0 = mt * RBM, col0 = nt * RBE;
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
      __builtin_amdgcn_make_buffer_rsrc((void*)w, 0, 3 * Epad * H * 2, kRsrcWord3);
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
    // tile row r: term r / 64 of router row col0 + r % 64 (rows past Epad
    // read the last one; their sums are never stored)
    const int r = (3 * wave + i) * 8 + lrow;
    const int n = min(col0 + (r & (RBE - 1)), Epad - 1);
    b_off[i] = (uint32_t)(((r / RBE) * Epad + n) * H + kbeg + 8 * (lslot ^ (r & 7))) * 2u;
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

  f32x4 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

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
        const int rb = i * RBE + wn * 16 + r16;  // term i of the wave's rows
        bb[i] = __builtin_bit_cast(bf16x8, ld16(&B[rb][((j * 4 + lg) ^ (rb & 7)) * 8]));
      }
      // (term-major, so consecutive products go to different accumulators)
#pragma unroll
      for (int ti = 0; ti < 3; ++ti)
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) acc[mi] = mfma_16x16x32(a[mi], bb[ti], acc[mi]);
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

  float* Pk = P + (int64_t)ks * T * Epad;
  const int col = col0 + wn * 16 + r16;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = row0 + wm * 64 + mi * 16 + 4 * lg + v;
      if (row < T && col < Epad) Pk[(int64_t)row * Epad + col] = acc[mi][v];
    }
}

template <int Q>
__global__ __launch_bounds__(256) void router_select_kernel(
    const float* __restrict__ P, int ksplit, int T, int E, int Epad, int k,
    const float* __restrict__ bias, int has_shared, float* __restrict__ logits_out,
    int32_t* __restrict__ ids_out, float* __restrict__ w_out, float* __restrict__ sw_out) {
  select_token<Q>(P, ksplit, T, E, Epad, k, bias, has_shared, logits_out, ids_out, w_out,
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
  select_token<Q>(P, 1, T, E, Epad, k, bias, has_shared, nullptr, ids_out, w_out, sw_out,
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

// One workgroup per router row (router_row, select_impl.h).
__global__ __launch_bounds__(256) void router_gemv_kernel(const uint16_t* __restrict__ x,
                                                          const float* __restrict__ wr,
                                                          const float* __restrict__ sg, int T,
                                                          int H, int E, int Epad,
                                                          float* __restrict__ out) {
  __shared__ float part[4][kRouterGemvT];
  router_row(x, wr, sg, T, H, E, Epad, blockIdx.x, out, part);
}

// The K split that finishes the tiles in the fewest stage times on one
// workgroup per CU: rounds of 256 workgroups times the stages per tile (the
// smallest split on ties). Beyond one round it stops at 4 planes, since the
// top-k reads every plane: 320 tiles (E = 256 with the shared gate at T =
// 8192) take 5 rounds of 8 stages at 4 planes instead of 2 rounds of 32 at
// one; within one round it is the largest split that fits, as before.
int router_ksplit(int T, int E, bool has_shared, int H) {
  const int tiles = cdiv(T, RBM) * cdiv(router_padded_rows(E, has_shared), RBE);
  const int S = H / RBK;
  int best = 1;
  int64_t best_cost = (int64_t)cdiv(tiles, 256) * S;
  for (int ks = 2; ks <= kRouterMaxKsplit && S % ks == 0; ks *= 2) {
    if (ks > 4 && tiles * ks > 256) break;
    const int64_t cost = (int64_t)cdiv(tiles * ks, 256) * (S / ks);
    if (cost < best_cost) {
      best = ks;
      best_cost = cost;
    }
  }
  return best;
}

}  // namespace

bool router_uses_gemv(int T) { return T <= kRouterGemvT; }

hipError_t launch_router_gemv(const uint16_t* x, const float* w_router, const float* shared_gate,
                              int T, int H, int E, float* partial, hipStream_t s) {
  const int Epad = router_padded_rows(E, shared_gate != nullptr);
  LaunchScope ls("router_gemm", s);
  hipLaunchKernelGGL(router_gemv_kernel, dim3(Epad), dim3(256), 0, s, x, w_router, shared_gate, T,
                     H, E, Epad, partial);
  return hipGetLastError();
}

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
  return (size_t)router_ksplit(T, E, has_shared, H) * T * router_padded_rows(E, has_shared) *
         sizeof(float);
}

hipError_t launch_router_split(const float* w_router, const float* shared_gate, int E, int H,
                               uint16_t* split, hipStream_t s) {
  const int Epad = router_padded_rows(E, shared_gate != nullptr);
  LaunchScope ls("router_split", s);
  hipLaunchKernelGGL(router_split_kernel, dim3(cdiv(H / 8, 256), Epad), dim3(256), 0, s, w_router,
                     shared_gate, E, H, Epad, split);
  return hipGetLastError();
}

hipError_t launch_router_topk(const uint16_t* x, const float* w_router, const float* shared_gate,
                              const uint16_t* split, float* partial, const float* bias, int T,
                              int H, int E, int k, float* logits, int32_t* ids, float* topk_w,
                              float* shared_w, uint16_t* x16, hipStream_t s) {
  const bool has_shared = shared_gate != nullptr;
  const int Epad = router_padded_rows(E, has_shared);
  int ks = 1;
  if (router_uses_gemv(T)) {
    // the finished fp32 logits, one plane [T][Epad]
    LaunchScope ls("router_gemm", s);
    hipLaunchKernelGGL(router_gemv_kernel, dim3(Epad), dim3(256), 0, s, x, w_router, shared_gate,
                       T, H, E, Epad, partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else {
    const int n_mt = cdiv(T, RBM), n_nt = cdiv(Epad, RBE);
    ks = router_ksplit(T, E, has_shared, H);
    LaunchScope ls("router_gemm", s);
    hipLaunchKernelGGL(router_gemm_kernel, dim3(n_mt * n_nt * ks), dim3(RTHREADS), 0, s, x,
                       split, partial, x16, T, H, Epad, n_mt, n_nt, ks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  LaunchScope ls("router_select", s);
  const dim3 grid(cdiv(T, 16)), block(256);
  const int hs = has_shared ? 1 : 0;
  if (E <= 64)
    hipLaunchKernelGGL(router_select_kernel<4>, grid, block, 0, s, partial, ks, T, E, Epad,
                       k, bias, hs, logits, ids, topk_w, shared_w);
  else if (E <= 128)
    hipLaunchKernelGGL(router_select_kernel<8>, grid, block, 0, s, partial, ks, T, E, Epad,
                       k, bias, hs, logits, ids, topk_w, shared_w);
  else
    hipLaunchKernelGGL(router_select_kernel<16>, grid, block, 0, s, partial, ks, T, E,
                       Epad, k, bias, hs, logits, ids, topk_w, shared_w);
  return hipGetLastError();
}

}  // namespace qmoe
