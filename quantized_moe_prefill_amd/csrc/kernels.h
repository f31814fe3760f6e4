// Host-side launchers of the gfx950 kernels. Each returns the HIP error of
// its launch(es); argument validation happens in the C ABI layer (api.cpp)
// before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmoe {

// Hook used by the launchers to bracket each kernel with profiling events.
struct LaunchScope {
  LaunchScope(const char* name, hipStream_t s);
  ~LaunchScope();
  const char* name;
  hipStream_t stream;
  int slot;
};

// ---- router -----------------------------------------------------------
// Rows of the router matrix padded to a multiple of 16: E routed rows, then
// the shared-gate row (if any), then zeros.
int router_padded_rows(int E, bool has_shared);
size_t router_split_bytes(int E, bool has_shared, int H);
// fp32 partial logits of the router GEMM (one plane per K slice, at most
// kRouterMaxKsplit planes)
constexpr int kRouterMaxKsplit = 16;
size_t router_partial_bytes(int T, int E, bool has_shared, int H);
hipError_t launch_router_split(const float* w_router, const float* shared_gate, int E, int H,
                               uint16_t* split, hipStream_t s);
// At most this many tokens: the router logits are an fp32 matrix-vector
// product straight from the fp32 router rows (no split matrix needed).
constexpr int kRouterGemvT = 16;
bool router_uses_gemv(int T);
// router GEMM (or matrix-vector product) into `partial`, then per-token
// logits, top-k and softmax; `split` is only read when !router_uses_gemv(T).
// x16 (optional, GEMM path only): also written with x in fp16 kperm chunk
// order, as launch_x_to_f16 would.
hipError_t launch_router_topk(const uint16_t* x, const float* w_router, const float* shared_gate,
                              const uint16_t* split, float* partial, const float* bias, int T,
                              int H, int E, int k, float* logits, int32_t* ids, float* topk_w,
                              float* shared_w, uint16_t* x16, hipStream_t s);

// At most kRouterGemvT tokens: router logits, top-k and softmax, and the
// grouping by expert (as launch_permute), in two launches.
hipError_t launch_route_permute_small(const uint16_t* x, const float* w_router,
                                      const float* shared_gate, float* partial, const float* bias,
                                      int T, int H, int E, int k, int32_t* ids, float* topk_w,
                                      float* shared_w, int32_t* counts, int32_t* offsets,
                                      int32_t* sorted_pairs, int32_t* inv, hipStream_t s);

// ---- permutation ------------------------------------------------------
// scratch: per-chunk expert histograms, permute_ws_bytes(P, E) bytes
size_t permute_ws_bytes(int P, int E);
hipError_t launch_permute(const int32_t* ids, int P, int E, int32_t* counts, int32_t* offsets,
                          int32_t* sorted_pairs, int32_t* inv, int32_t* hist, hipStream_t s);

// ---- grouped expert GEMMs --------------------------------------------
// bf16 [n] (n % 8 == 0) -> fp16 in the kperm chunk order of the expert GEMMs.
hipError_t launch_x_to_f16(const uint16_t* x, uint16_t* x16, int64_t n, hipStream_t s);

struct GroupedGemm {
  const uint16_t* A;       // fp16 activation rows, kperm chunk order
  const int32_t* gather;   // row r -> A row gather[r] / gather_div ; NULL: A row r
  int gather_div;
  const int32_t* counts;   // [E] rows per group; NULL: one group of rows_single rows
  const int32_t* offsets;  // [E+1] first row of each group
  int rows_single;
  int E;
  int max_rows;            // upper bound of all rows (sizes the grid)
  int a_rows;              // rows of A (bounds the activation reads)
  const uint8_t* W;        // [E][N][K/2] packed nibbles
  const uint16_t* Wscale;  // fp16 [E][N][K/G]
  const uint16_t* Wmin;    // fp16 [E][N][K/G] or NULL (symmetric)
  int N, K, G;
  uint16_t* C;             // output rows, fp16, leading dimension ldc
  int ldc;
  // Rows per group the caller expects at most (the token count for routed
  // groups and for the shared expert). At most kStreamMaxRows selects the
  // weight-streaming kernel; any actual count is still computed correctly.
  int expect_rows;
  // A holds bf16 rows in natural order (the weight-streaming gate/up kernel
  // converts them itself); otherwise fp16 in kperm chunk order
  bool a_bf16;
  // Tiled kernel only: one more group after the E routed ones (a shared
  // expert with the same N and K), rows2 rows of A2 in order (no gather),
  // one expert's weights W2 / Wscale2 / Wmin2, output C2 with leading
  // dimension ldc2. rows2 == 0: none.
  int rows2;
  const uint16_t* A2;
  const uint8_t* W2;
  const uint16_t* Wscale2;
  const uint16_t* Wmin2;
  uint16_t* C2;
  int ldc2;
  // One group of experts of a mixed layer (tier != NULL; symmetric, no
  // extra group): the launch computes only the experts e with
  // tier[e] == tier_id (tier and slot are device arrays), whose weights and
  // scales are expert slot[e] of W / Wscale, which hold w_experts experts.
  // bits is the group's width: 4, or 3 / 2 for the lower-bit codes of
  // dequant.h (rows of K * bits / 8 bytes).
  const int32_t* tier;
  const int32_t* slot;
  int tier_id;
  int w_experts;
  int bits;
  // W and W2 in the tiled 4-bit layout (moe_pack_w4: 1024-byte blocks of 16
  // rows x 128 K) instead of row-major; 4-bit only
  bool w_tiled;
};

// Per-expert group and slot maps of a mixed layer (at most 256 experts),
// passed by value and written to device arrays by one small kernel.
struct ExpertMaps {
  int32_t group[256];
  int32_t slot[256];
};
hipError_t launch_write_maps(const ExpertMaps& m, int E, int32_t* group, int32_t* slot,
                             hipStream_t s);
constexpr int kStreamMaxRows = 16;
// gate/up with fused SwiGLU: N = 2I weight rows, writes h = silu(g)*u
// (fp16, kperm chunk order), ldc = I.
hipError_t launch_gateup(const GroupedGemm& g, hipStream_t s, const char* name = "gateup_gemm");
// down projection: N = H weight rows, writes y (fp16, natural order), ldc = H.
hipError_t launch_down(const GroupedGemm& g, hipStream_t s, const char* name = "down_gemm");
// Weight-streaming form of the two GEMMs above for a few rows per group.
bool stream_supported(const GroupedGemm& g, bool gateup);
// launch_gateup(g) / launch_down(g) would run the weight-streaming kernel
// (which reads bf16 activations directly, a_bf16, and ignores rows2)
bool gemm_streams(const GroupedGemm& g, bool gateup);
hipError_t launch_stream(const GroupedGemm& g, bool gateup, hipStream_t s, const char* name);

// ---- the layer's experts for a few tokens (small.hip) -----------------
struct SmallLayer {
  const uint16_t* x;         // bf16 [T][H]
  const float* bias;         // fp32 [E] router bias or NULL
  // experts as in moe_experts_t (mins NULL: symmetric)
  const uint8_t *w13, *w2, *s13, *s2;
  const uint16_t *w13_scale, *w13_min, *w2_scale, *w2_min;
  const uint16_t *s13_scale, *s13_min, *s2_scale, *s2_min;
  int T, H, E, k, I, G, has_shared, Epad, nbits;
  const float* logits;       // [T][Epad] fp32 (router_gemv; column E: the shared gate)
  // outputs: h [T k][I], hs [T][I], yperm [T k][H], ysh [T][H] (fp16), and
  // the selection and grouping (ids, tw, inv, sorted [T k], sw [T],
  // counts [E], offsets [E + 1]) as route / permute write them
  uint16_t *h, *hs, *yperm, *ysh;
  int32_t *ids, *inv, *sorted, *counts, *offsets;
  float *tw, *sw;
  bool w_tiled;  // the packed weights in the tiled layout
};
// shapes these kernels cover (T <= kRouterGemvT, k <= 8, E <= 256, G 32 or
// 128, a shared expert of the routed experts' width, H and I whose
// weight-streaming tilings they instantiate); the rest take the separate
// routing and streaming kernels
bool small_layer_supported(int T, int H, int I, int Is, int E, int k, int G);
// Two launches, after the router logits: top-k, grouping and gate/up (with
// the shared expert), then down (with the shared expert).
hipError_t launch_small_experts(const SmallLayer& a, hipStream_t s);
// One 4-bit matrix [rows][K/2] regrouped into the tiled layout (rows % 16 == 0,
// K % 128 == 0).
hipError_t launch_pack_w4(const uint8_t* src, uint8_t* dst, int64_t rows, int64_t K,
                          hipStream_t s);
// Any width, into the tiled layout (interleave: the 3- and 2-bit gate/up row
// order within 32-row groups); rows % 16 == 0 (32 with interleave), K % 128 == 0.
hipError_t launch_pack_tier(const uint8_t* src, uint8_t* dst, int64_t rows, int64_t K, int bits,
                            bool interleave, hipStream_t s);
// The router logits alone for at most kRouterGemvT tokens (one plane, [T][Epad]).
hipError_t launch_router_gemv(const uint16_t* x, const float* w_router, const float* shared_gate,
                              int T, int H, int E, float* partial, hipStream_t s);

// ---- integer route: 8-bit activations x symmetric 4-bit weights --------
// Per-row 8-bit quantization of bf16 (or fp16) rows [rows][cols], cols % 8
// == 0: q = rint(v * (127 / a)), s = a / 127, a = max |v| of the row (rows
// with a < 2^-100 give zeros). gemm_order stores each 8-element chunk as
// elements 0,2,4,6,1,3,5,7 (the int8 GEMMs' operand order), else natural.
hipError_t launch_quant_rows_i8(const uint16_t* src, bool src_f16, int rows, int cols,
                                bool gemm_order, int8_t* q, float* scale, hipStream_t s);

struct GemmI8 {
  const int8_t* A;         // int8 activation rows [a_rows][K], int8 GEMM chunk order
  const float* a_scale;    // [a_rows] row scales
  const int32_t* gather;   // row r -> A row gather[r] / gather_div ; NULL: A row r
  int gather_div;
  const int32_t* counts;   // [E] rows per group
  const int32_t* offsets;  // [E+1]
  int E;
  int max_rows;            // upper bound of all rows (sizes the grid)
  int a_rows;
  const uint8_t* W;        // [E][N][K/2] symmetric 4-bit codes
  const uint16_t* Wscale;  // fp16 [E][N][K/128]
  int N, K;                // K % 128 == 0; the group size is 128
  uint16_t* C;             // fp16 output rows, leading dimension ldc
  int ldc;
};
// gate/up (N = 2I) with SwiGLU: C = h [rows][I] fp16, natural order
hipError_t launch_gateup_i8(const GemmI8& g, hipStream_t s);
// down (N = H): C = y [rows][H] fp16
hipError_t launch_down_i8(const GemmI8& g, hipStream_t s);

// ---- combine / norm ---------------------------------------------------
hipError_t launch_combine(const uint16_t* y_perm, const int32_t* inv, const float* topk_w,
                          const uint16_t* y_shared, const float* shared_w,
                          const uint16_t* residual, uint16_t* out, int T, int H, int k,
                          hipStream_t s);
hipError_t launch_rmsnorm(const uint16_t* x, const float* w, float eps, uint16_t* out, int T,
                          int H, hipStream_t s);

}  // namespace qmoe
