// Device code of the weight-streaming expert GEMMs (a few rows per expert),
// shared by the streaming kernels and the fused small-batch layer kernel.
#pragma once

#include "common.h"
#include "dequant.h"
#include "kernels.h"

namespace qmoe {

constexpr int SWAVES = 4;              // waves per workgroup (K split four ways)
constexpr int STHREADS = 64 * SWAVES;
constexpr int SBK = 128;               // K per stage
constexpr int SWG_PER_CU = 2;          // resident workgroups per CU (at least)
constexpr int SMAXG = 256;             // groups per launch

// number of lanes below this one whose bit is set in m
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// One wave's share of an item's weights: per fragment, this lane's 16 NS
// bytes of packed nibbles and the fp16 scales (and mins) of the groups they
// fall in (at most four, packed two per word).
template <int NS, int NF>
struct StreamW {
  u32x4 w[NS][NF];
  uint32_t s[NF][2], m[NF][2];
};

// NS = 128-wide K blocks per wave (K <= 4 * NS * 128); NF = 16-column
// fragments per item (gate/up: NF / 2 gate and NF / 2 up fragments); G =
// quantization group size.
//
// Items i0 .. i1-1 of one workgroup (STHREADS threads, all of them call):
// item i is column block i % n_cb of list slot i / n_cb, whose group (expert
// index into g's n_groups experts), rows and first row are s_grp, s_rows,
// s_row0 of that slot; gate/up output row r takes the products of token
// s_tok[r]. red: the LDS of the partial sums.
template <bool GATEUP, bool ASYM, int NS, int NF, int G>
__device__ __forceinline__ void stream_items(const GroupedGemm& g, int n_groups, int n_cb, int i0,
                                             int i1, const int* s_grp, const int* s_rows,
                                             const int* s_row0, const int* s_tok,
                                             float (*red)[NF][4][64]) {
  if (i0 >= i1) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, lg = lane >> 4;
  const int K = g.K, N = g.N, KG = K / G;

  // K split: wave w takes [128 NS w, 128 NS (w + 1)), and within it lane
  // group lg the contiguous block [kb, kb + 32 NS). Matrix-core step s of a
  // fragment (s < 4 NS) takes K values kb + 8 s .. kb + 8 s + 7 from every
  // lane, from the weights and the activations alike, so the two operands
  // agree. A block at or past K (K is a multiple of 128, so blocks are whole)
  // loads block 0 again and has its scales (and mins) zeroed: it adds zeros.
  const int kb = SBK * NS * wave + 32 * NS * lg;
  const bool kvalid = kb < K;
  const int kbc = kvalid ? kb : 0;
  const bool wave_has_k = SBK * NS * wave < K;
  // scales per lane and fragment: the groups its block falls in
  constexpr int NSC = 32 * NS > G ? 32 * NS / G : 1;

  const __amdgpu_buffer_rsrc_t rA =
      __builtin_amdgcn_make_buffer_rsrc((void*)g.A, 0, g.a_rows * K * 2, kRsrcWord3);
  // activation operand: lane (r16, lg) supplies row r16, its K block
  u32x4 av[NS][4];
  auto load_a_row = [&](int src) {
    const uint32_t a_lane = ((uint32_t)src * (uint32_t)K + kbc) * 2;
#pragma unroll
    for (int i = 0; i < NS; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        av[i][j] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rA, a_lane, 64 * i + 16 * j, 0));
  };

  const __amdgpu_buffer_rsrc_t rW =
      __builtin_amdgcn_make_buffer_rsrc((void*)g.W, 0, n_groups * N * (K / 2), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rS =
      __builtin_amdgcn_make_buffer_rsrc((void*)g.Wscale, 0, n_groups * N * KG * 2, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rM = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(ASYM ? g.Wmin : g.Wscale), 0, n_groups * N * KG * 2, kRsrcWord3);

  // Fragment f of an item covers weight rows c0 + frow(f) + 0..15 of its
  // group. Gate/up: fragments 0 .. NF/2 - 1 are gate rows (h columns c0 ..
  // c0 + 8 NF - 1), the others the up rows of the same columns. Lane (r16,
  // lg) holds row r16 of a fragment, its K block: 16 NS bytes of nibbles and
  // NSC consecutive scales (one load of 2, 4 or 8 bytes, naturally aligned
  // since K is a multiple of 128).
  const int cstep = GATEUP ? 8 * NF : 16 * NF;  // output columns per item
  auto frow = [&](int f) {
    return GATEUP ? (f < NF / 2 ? 16 * f : N / 2 + 16 * (f - NF / 2)) : 16 * f;
  };
  auto load_w = [&](int it, StreamW<NS, NF>& W) {
    const int slot = it / n_cb;
    const int e = s_grp[slot];
    const int c0 = (it - slot * n_cb) * cstep;
    const uint32_t wrow0 = (uint32_t)(e * N + c0 + r16);
    // row-major: row wrow0, bytes from kbc / 2 on, 16 per load; tiled
    // (moe_pack_w4): the 1 KB block of the fragment's 16 rows and kbc's K
    // stage, 16-byte slot 16 ((kbc % 128) / 32 + i) + r16 for load i
    // (a lane's 32 NS elements never cross a stage)
    const uint32_t b_lane =
        g.w_tiled ? (wrow0 - r16) * (uint32_t)(K / 2) + (uint32_t)(kbc >> 7) * 1024u +
                        (uint32_t)((kbc >> 5) & 3) * 256u + (uint32_t)r16 * 16u
                  : wrow0 * (uint32_t)(K / 2) + kbc / 2;
    const int i_step = g.w_tiled ? 256 : 16;
    const uint32_t s_lane = (wrow0 * (uint32_t)KG + kbc / G) * 2;
#pragma unroll
    for (int i = 0; i < NS; ++i)
#pragma unroll
      for (int f = 0; f < NF; ++f)
        W.w[i][f] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rW, b_lane, frow(f) * (K / 2) + i_step * i, 0));
    auto load_sc = [&](__amdgpu_buffer_rsrc_t r, int so, uint32_t* d) {
      if (NSC == 4) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, s_lane, so, 0);
        d[0] = v[0];
        d[1] = v[1];
      } else if (NSC == 2) {
        d[0] = __builtin_amdgcn_raw_buffer_load_b32(r, s_lane, so, 0);
        d[1] = 0u;
      } else {
        d[0] = __builtin_amdgcn_raw_buffer_load_b16(r, s_lane, so, 0);
        d[1] = 0u;
      }
    };
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int so = frow(f) * KG * 2;
      load_sc(rS, so, W.s[f]);
      if (ASYM) load_sc(rM, so, W.m[f]);
      else W.m[f][0] = W.m[f][1] = 0u;
    }
  };

  // down: rows rb + r16 of a group's h (past its end: its last row, whose
  // products are never stored)
  auto load_a_group = [&](int row0, int rows, int rb) {
    int r = rb + r16;
    if (r >= rows) r = rows - 1;
    load_a_row(row0 + r);
  };

  // products of one 16-row block, the four partial sums in wave order, and
  // the block's output rows
  auto block = [&](StreamW<NS, NF>& W, int row0, int rb, int nrows, int c0) {
    // Opaque here: a group with several row blocks reuses the same weights,
    // and the compiler would otherwise unpack their nibbles once ahead of
    // the blocks and hold four times the registers.
#pragma unroll
    for (int i = 0; i < NS; ++i)
#pragma unroll
      for (int f = 0; f < NF; ++f) asm volatile("" : "+v"(W.w[i][f]));
#pragma unroll
    for (int f = 0; f < NF; ++f)
      asm volatile("" : "+v"(W.s[f][0]), "+v"(W.s[f][1]), "+v"(W.m[f][0]), "+v"(W.m[f][1]));
    f32x4 acc[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
    // (the dequant and matrix-core run outranks the other workgroups' waves
    // on the SIMD while they issue loads or wait: T=16 layer 78.5 -> 77.5 us
    // over three A/B runs, T=1 unchanged)
    __builtin_amdgcn_s_setprio(1);
    if (wave_has_k) {
      // this lane's scales (and mins); zero for a block past K
      uint32_t sw[NF][2], mw[NF][2];
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          sw[f][q] = kvalid ? W.s[f][q] : 0u;
          mw[f][q] = kvalid ? W.m[f][q] : 0u;
        }
#pragma unroll
      for (int i = 0; i < NS; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // K values kb + 8 (4 i + j) ..: scale number (32 i + 8 j) / G of the block
          const int si = NSC > 1 ? (32 * i + 8 * j) / G : 0;
#pragma unroll
          for (int f = 0; f < NF; ++f) {
            const uint32_t sh = (sw[f][si >> 1] >> (16 * (si & 1))) & 0xffffu;
            const uint32_t mh = (mw[f][si >> 1] >> (16 * (si & 1))) & 0xffffu;
            const f16x8 b = dequant8_f16<ASYM>(W.w[i][f][j], __builtin_bit_cast(f16x2, sh * 0x10001u),
                                               __builtin_bit_cast(f16x2, mh * 0x10001u));
            acc[f] = mfma_16x16x32_f16(__builtin_bit_cast(f16x8, av[i][j]), b, acc[f]);
          }
        }
    }

    __builtin_amdgcn_s_setprio(0);
    // LDS-only barriers here: __syncthreads() would also wait for every
    // outstanding load, the weights of the next two items included
    lds_barrier();  // the previous block's output rows have been read from red
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[wave][f][v][lane] = acc[f][v];
    lds_barrier();
    // lane (r16, lg) of fragment f holds rows 4 lg + v, column r16: output
    // row rr, columns 8 h .. 8 h + 7 of fragment f are red[.][f][rr & 3]
    // [16 (rr >> 2) + 8 h + 0..7]
    auto sum8 = [&](int f, int rr, int half, float* o) {
      const int l0 = 16 * (rr >> 2) + 8 * half;
#pragma unroll
      for (int c = 0; c < 8; ++c) o[c] = 0.f;
#pragma unroll
      for (int w = 0; w < SWAVES; ++w) {
        const f32x4 p0 = *reinterpret_cast<const f32x4*>(&red[w][f][rr & 3][l0]);
        const f32x4 p1 = *reinterpret_cast<const f32x4*>(&red[w][f][rr & 3][l0 + 4]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          o[c] += p0[c];
          o[c + 4] += p1[c];
        }
      }
    };
    if (GATEUP) {
      // every row of the group x NF chunks of 8 h columns: row r takes the
      // product row of its token. A fixed number of passes (at most 256 rows
      // of at most 4 chunks), so that the compiler can count the stores when
      // it waits for the next item's weights.
#pragma unroll
      for (int pass = 0; pass < NF; ++pass) {
        const int i = tid + pass * STHREADS;
        if (i >= nrows * NF) break;
        const int r = i / NF, q = i - r * NF;
        const int t = s_tok[row0 + r];
        float gv[8], uv[8];
        sum8(q >> 1, t, q & 1, gv);
        sum8(NF / 2 + (q >> 1), t, q & 1, uv);
        float hv[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) hv[c] = silu_f32(gv[c]) * uv[c];
        // kperm order inside the chunk: positions 0..7 hold columns 0,4,1,5,2,6,3,7
        u32x4 o;
#pragma unroll
        for (int p = 0; p < 4; ++p) o[p] = pack_f16x2(hv[kperm(2 * p)], hv[kperm(2 * p + 1)]);
        st16(g.C + (int64_t)(row0 + r) * g.ldc + c0 + 8 * q, o);
      }
    } else {
      // 16 rows x 2 NF chunks of 8 output columns
      const int rr = tid / (2 * NF), q = tid % (2 * NF);
      if (tid < 32 * NF && rr < nrows) {
        float yv[8];
        sum8(q >> 1, rr, q & 1, yv);
        u32x4 o;
#pragma unroll
        for (int p = 0; p < 4; ++p) o[p] = pack_f16x2(yv[2 * p], yv[2 * p + 1]);
        st16(g.C + (int64_t)(row0 + rb + rr) * g.ldc + c0 + 8 * q, o);
      }
    }
  };

  // ---- the items: weights two items ahead, in three register sets used in
  // turn (a copy from one set to another would wait for its loads) ----
  int a_slot = -1;  // down: group whose first row block av holds
  if (!GATEUP) {
    const int slot0 = i0 / n_cb;
    load_a_group(s_row0[slot0], s_rows[slot0], 0);
    a_slot = slot0;
  }
  auto item = [&](int it, StreamW<NS, NF>& Wc, StreamW<NS, NF>& Wp) {
    const int slot = it / n_cb;
    const int c0 = (it - slot * n_cb) * cstep;
    const int rows = s_rows[slot], row0 = s_row0[slot];
    if (!GATEUP && slot != a_slot) {
      // before the later items' weights, so that waiting for these rows
      // does not wait for those
      load_a_group(row0, rows, 0);
      a_slot = slot;
    }
    load_w(min(it + 2, i1 - 1), Wp);  // the last items load themselves again
    __builtin_amdgcn_sched_barrier(0);
    if (GATEUP) {
      block(Wc, row0, 0, rows, c0);
    } else {
      block(Wc, row0, 0, min(16, rows), c0);
      if (rows > 16) {
        // more than 16 rows (only when a token sends several rows to one
        // group): further blocks with the same weights
        for (int rb = 16; rb < rows; rb += 16) {
          load_a_group(row0, rows, rb);
          block(Wc, row0, rb, min(16, rows - rb), c0);
        }
        a_slot = -1;
      }
    }
  };
  // Start-up order, for vector loads complete in issue order: the first
  // item's weights, then (gate/up) the token rows, which every product
  // needs, then the second item's weights, so that the first products wait
  // for neither the second item nor anything issued later.
  StreamW<NS, NF> W0, W1, W2;
  load_w(i0, W0);
  // gate/up: rows 0..15 are the tokens themselves (past the last token: the
  // last one again, whose products are never used)
  if (GATEUP) load_a_row(min(r16, g.a_rows - 1));
  load_w(min(i0 + 1, i1 - 1), W1);
  if (GATEUP && g.a_bf16) {
    // bf16 activations -> fp16 in kperm chunk order (exact for |x| < 65504),
    // once: the token rows are the same for every item
#pragma unroll
    for (int i = 0; i < NS; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 d = av[i][j];  // (x0,x1) (x2,x3) (x4,x5) (x6,x7)
        av[i][j] = u32x4{pack_f16x2(bf16lo(d[0]), bf16lo(d[2])), pack_f16x2(bf16hi(d[0]), bf16hi(d[2])),
                         pack_f16x2(bf16lo(d[1]), bf16lo(d[3])), pack_f16x2(bf16hi(d[1]), bf16hi(d[3]))};
      }
  }
  for (int it = i0; it < i1; it += 3) {
    item(it, W0, W2);
    if (it + 1 < i1) item(it + 1, W1, W0);
    if (it + 2 < i1) item(it + 2, W2, W1);
  }
}

}  // namespace qmoe
