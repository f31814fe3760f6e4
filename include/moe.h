/*
 * moe.h - C ABI of the 4-bit block-quantized MoE prefill library (gfx950).
 *
 * One MoE FFN layer over a prefill chunk of T tokens:
 *   route   : fp32 router logits, top-k selection, softmax over the k chosen
 *   permute : group the T*k (token, slot) pairs by expert
 *   experts : per expert, SwiGLU FFN with 4-bit block-quantized weights
 *   combine : weighted sum of each token's k expert outputs (+ shared expert,
 *             + residual)
 *
 * The pages this follows describe the route, not an interface: the hipfire
 * 0.4.3 benchmarks page, "Read this before comparing columns" (the MoE
 * prefill route is "per-expert buffers" or "symmetric IU4 MoE", prompts are
 * processed in row chunks of 8192) and "Known limits" (symmetric vs
 * asymmetric 4-bit expert files). Everything below the method level (the
 * router form, the nibble layout, the group size) is this library's
 * definition, stated per argument.
 *
 * Conventions for every call:
 *  - Tensors are row-major, little-endian, densely packed. bf16 and fp16
 *    values travel as uint16_t bit patterns.
 *  - Every tensor pointer is a DEVICE pointer (hipMalloc'd or equivalent),
 *    owned by the caller, 16-byte aligned, and must stay valid until the
 *    enqueued work has finished. The library never allocates or frees device
 *    memory on the call path and keeps no state between calls (except the
 *    optional profiling pool, see moe_profile_*).
 *  - Calls only enqueue work on `stream` (NULL = the default stream) and
 *    return; faults inside kernels surface at the caller's next
 *    synchronization.
 *  - Validation happens on the host before anything is launched. On a non-OK
 *    status nothing was launched and no output was touched; moe_last_error()
 *    describes the problem. T == 0 is a valid no-op that returns MOE_OK.
 *  - No output may alias an input, except that moe_combine's and
 *    moe_layer_forward's `out` may alias `residual`.
 *  - No C++ exception crosses this interface. Calls on different streams
 *    with disjoint buffers may run concurrently.
 *
 * Supported shapes (MOE_ERR_UNSUPPORTED otherwise):
 *    hidden H % 128 == 0, 128 <= H <= 16384;  1 <= E <= 256;  1 <= k <= min(E, 8);
 *    group_size G in {32, 64, 128};  inter I % 128 == 0;
 *    shared_inter == 0 or shared_inter % 128 == 0;
 *    T * k < 2^31;  the kernels address tensors through 32-bit buffer
 *    descriptors, so each of these must be below 2^31 bytes:
 *      activations  x, x16: T*H*2;  h: T*k*I*2;  h_shared: T*Is*2
 *                   (174,762 tokens per call at H = 2048, k = 8, I = 768:
 *                   longer prompts go through in chunks);
 *      experts      w13: E*2I*H/2;  w2: E*H*I/2;  their scales (and mins):
 *                   E*2I*(H/G)*2 and E*H*(I/G)*2.
 */
#ifndef QMOE_MOE_H
#define QMOE_MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,   /* null/negative/mismatched argument */
  MOE_ERR_UNSUPPORTED = 2,        /* legal but not implemented (shape, G, alignment) */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,
  MOE_ERR_HIP = 4                 /* a HIP runtime call or launch failed */
} moe_status_t;

/* 4-bit formats. Two weights per byte: byte j of a row holds element 2j in
 * bits 0-3 and element 2j+1 in bits 4-7. A group of G consecutive elements
 * along K (the input dimension) of one row shares one fp16 scale (and min).
 *   MOE_Q4_SYM : w = (nibble - 8) * scale          (all 16 codes decode)
 *   MOE_Q4_ASYM: w = nibble * scale + min                                     */
typedef enum { MOE_Q4_SYM = 0, MOE_Q4_ASYM = 1 } moe_quant_t;

/* Byte order of the packed 4-bit weight matrices (w13, w2, s13, s2; the
 * scales and mins are always row-major [rows][K/G]):
 *   MOE_W_ROWS : row-major [rows][K/2], the bytes as described above.
 *   MOE_W_TILED: the same bytes regrouped by moe_pack_w4 into 1024-byte
 *                blocks, one per 16 rows x 128 elements of K, in the order the
 *                matrix cores consume them, so that every load of the
 *                library's GEMM kernels reads whole cache lines. Accepted by
 *                moe_expert_ffn, moe_layer_forward and moe_layer_forward_static
 *                (the same results, bit for bit), and by the mixed-width calls
 *                with every tier regrouped by moe_pack_tier; the integer and
 *                host-streamed calls return MOE_ERR_UNSUPPORTED for it. */
typedef enum { MOE_W_ROWS = 0, MOE_W_TILED = 1 } moe_w_layout_t;

typedef struct {
  int64_t hidden;        /* H */
  int64_t num_experts;   /* E routed experts */
  int64_t top_k;         /* k experts per token */
  int64_t inter;         /* I, routed expert intermediate size */
  int64_t group_size;    /* G, quantization group along K */
  int32_t quant;         /* moe_quant_t */
  int32_t w_layout;      /* moe_w_layout_t of the expert weights */
  int64_t shared_inter;  /* I_s of the always-on shared expert; 0 = none */
} moe_shape_t;

/* Expert weights (device pointers, read only). For MOE_Q4_SYM every *_min
 * must be NULL; for MOE_Q4_ASYM every *_min of a present matrix is required.
 * The shared-expert pointers are NULL iff shape.shared_inter == 0. */
typedef struct {
  const uint8_t  *w13;        /* [E][2I][H/2]: rows 0..I-1 gate, I..2I-1 up  */
  const uint16_t *w13_scale;  /* fp16 [E][2I][H/G]                           */
  const uint16_t *w13_min;    /* fp16 [E][2I][H/G] or NULL                   */
  const uint8_t  *w2;         /* [E][H][I/2]: down projection                */
  const uint16_t *w2_scale;   /* fp16 [E][H][I/G]                            */
  const uint16_t *w2_min;     /* fp16 [E][H][I/G] or NULL                    */
  const uint8_t  *s13;        /* shared expert [2I_s][H/2]                   */
  const uint16_t *s13_scale;  /* fp16 [2I_s][H/G]                            */
  const uint16_t *s13_min;
  const uint8_t  *s2;         /* shared expert [H][I_s/2]                    */
  const uint16_t *s2_scale;   /* fp16 [H][I_s/G]                             */
  const uint16_t *s2_min;
} moe_experts_t;

/* Which call a workspace is sized for. Any call accepts a workspace of the
 * MOE_WS_LAYER size for the same shape and T. */
typedef enum {
  MOE_WS_LAYER = 0,       /* moe_layer_forward */
  MOE_WS_ROUTE = 1,       /* moe_route */
  MOE_WS_PERMUTE = 2,     /* moe_permute */
  MOE_WS_EXPERT_FFN = 3,  /* moe_expert_ffn */
  MOE_WS_LAYER_I8 = 4,    /* moe_layer_forward_i8 */
  MOE_WS_EXPERT_FFN_I8 = 5 /* moe_expert_ffn_i8 */
} moe_ws_kind_t;

int moe_abi_version(void);

/* Message for the last non-OK status returned on the calling thread. */
const char *moe_last_error(void);

/* Bytes of device workspace a call needs for this shape and T (host only,
 * launches nothing). */
moe_status_t moe_workspace_size(const moe_shape_t *shape, int64_t T, int32_t kind,
                                size_t *bytes);

/* Router: L[t,e] = sum_h x[t,h] * w_router[e,h] (+ router_bias[e]), fp32;
 * ids[t] = the k experts with the largest L (largest first; equal logits
 * ordered by ascending expert index; -0.0 == +0.0; inputs must be finite);
 * topk_w[t,j] = exp(L_j - L_max) / sum over the k chosen of exp(L_i - L_max).
 * If shared_gate is given, shared_w[t] = 1 / (1 + exp(-(x[t] . shared_gate))).
 * The dot products are formed from exact products of the bf16 activations
 * with an exact three-term bf16 split of each fp32 router weight, summed in
 * fp32 on the matrix cores (an fp32 GEMM to within its usual error bound).
 *   x           [T][H] bf16          w_router [E][H] fp32
 *   router_bias [E] fp32 or NULL     shared_gate [H] fp32 or NULL; only with
 *                                    shape.shared_inter > 0 (else INVALID_ARGUMENT)
 *   logits      [T][E] fp32 or NULL: receives the (biased) logits used for selection
 *   topk_ids    [T][k] int32         topk_w [T][k] fp32
 *   shared_w    [T] fp32, required iff shared_gate != NULL
 *   ws          >= moe_workspace_size(MOE_WS_ROUTE, T) bytes of scratch (the
 *               split router matrix and fp32 partial logits; grows with T)   */
moe_status_t moe_route(const moe_shape_t *shape, int64_t T, const uint16_t *x,
                       const float *w_router, const float *router_bias,
                       const float *shared_gate, float *logits, int32_t *topk_ids,
                       float *topk_w, float *shared_w, void *ws, size_t ws_bytes,
                       hipStream_t stream);

/* Expert grouping of the P = T*k pairs, pair p = t*k + j:
 *   counts[e]      number of pairs routed to expert e            [E] int32
 *   offsets[e]     exclusive prefix sum of counts                [E+1] int32
 *   sorted_pairs   expert by expert, that expert's pairs in ascending p  [P] int32
 *   inv[p]         position of pair p in sorted_pairs            [P] int32
 * topk_ids entries must lie in [0, E); a pair with an id outside that range
 * is a caller error: it is left out of counts and sorted_pairs and its inv
 * entry is 0. Deterministic (no atomics). T == 0 writes zero counts/offsets
 * (topk_ids, sorted_pairs and inv may then be NULL).
 *   ws  >= moe_workspace_size(MOE_WS_PERMUTE, T) bytes (per-chunk expert
 *          histograms, 4 * E * ceil(T*k / 2048) bytes)                     */
moe_status_t moe_permute(const moe_shape_t *shape, int64_t T, const int32_t *topk_ids,
                         int32_t *counts, int32_t *offsets, int32_t *sorted_pairs,
                         int32_t *inv, void *ws, size_t ws_bytes, hipStream_t stream);

/* Expert FFNs. Row r of expert e (offsets[e] <= r < offsets[e+1]) is token
 * sorted_pairs[r] / k; it is multiplied by the dequantized expert weights:
 *   h = silu(x W_gate^T) * (x W_up^T),  silu(z) = z / (1 + exp(-z))
 *   y_perm[r] = h W_down^T                       (unweighted, fp16 [P][H])
 * The shared expert (if present) runs the same FFN on every token into
 * y_shared [T][H] fp16 (required iff shape.shared_inter > 0).
 * Numerics: activations are converted exactly to fp16 (for |x| <= 65504;
 * magnitudes under 2^-14 keep fewer bits), weights are dequantized in
 * registers to fp16 (q * scale, or q * scale + min, rounded once; every
 * dequantized weight must be finite in fp16), both products run on the fp16
 * matrix cores with fp32 accumulation, and h is rounded to fp16 between
 * them. fp16 range: every fp16 value the layer stores (the copy of x, h,
 * y_perm, y_shared) saturates to +-65504 instead of becoming infinite, so
 * the result stays finite; for a token whose x, h or y leaves the fp16
 * range the result is then not the layer's value (other tokens are
 * unaffected: tokens do not interact). counts/offsets/sorted_pairs are
 * moe_permute's outputs. */
moe_status_t moe_expert_ffn(const moe_shape_t *shape, int64_t T, const uint16_t *x,
                            const moe_experts_t *experts, const int32_t *counts,
                            const int32_t *offsets, const int32_t *sorted_pairs,
                            uint16_t *y_perm, uint16_t *y_shared, void *ws,
                            size_t ws_bytes, hipStream_t stream);

/* out[t] = bf16( sum_j topk_w[t,j] * y_perm[inv[t*k+j]]
 *                (+ shared_w[t] * y_shared[t]) (+ residual[t]) ), fp32 sums.
 * y_perm [P][H] and y_shared [T][H] are fp16 (moe_expert_ffn's outputs);
 * y_shared and shared_w go together (both NULL or both set); residual
 * [T][H] bf16 may be NULL and may alias out; out [T][H] bf16. */
moe_status_t moe_combine(const moe_shape_t *shape, int64_t T, const uint16_t *y_perm,
                         const int32_t *inv, const float *topk_w, const uint16_t *y_shared,
                         const float *shared_w, const uint16_t *residual, uint16_t *out,
                         hipStream_t stream);

/* The whole layer: route -> permute -> experts -> combine, all on `stream`,
 * with every intermediate in ws (>= moe_workspace_size(MOE_WS_LAYER)).
 * x [T][H] bf16 (fp16 range: see moe_expert_ffn), out [T][H] bf16.
 * shared_gate is required iff shape.shared_inter > 0. residual may be NULL
 * and may alias out. No device-to-host transfer happens. */
moe_status_t moe_layer_forward(const moe_shape_t *shape, int64_t T, const uint16_t *x,
                               const float *w_router, const float *router_bias,
                               const float *shared_gate, const moe_experts_t *experts,
                               const uint16_t *residual, uint16_t *out, void *ws,
                               size_t ws_bytes, hipStream_t stream);

/* Size of the library's static workspace (bytes, per GPU). */
#define MOE_STATIC_WS_BYTES (128u << 20)

/* moe_layer_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc). Same arguments, results and
 * kernels as moe_layer_forward (the same bits), with every intermediate in
 * a fixed array inside the library: MOE_STATIC_WS_BYTES of device memory,
 * one copy per GPU the library runs on, held until the process ends. The
 * call allocates nothing. Limit: calls whose moe_workspace_size(MOE_WS_LAYER)
 * exceeds MOE_STATIC_WS_BYTES return MOE_ERR_UNSUPPORTED before anything is
 * launched (2,583 tokens at H = 2048, E = 128, k = 8, I = 768; 2,493 at
 * H = 2048, E = 256, k = 8, I = 512 with a shared expert of 512; split
 * longer batches). Every call on one GPU uses that GPU's one array, and
 * nothing in it has to start at zero: calls that overlap on one GPU
 * (concurrent streams, other threads) race on it and must be serialized by
 * the caller. The first call on a GPU looks up that GPU's copy of the array
 * (MOE_ERR_HIP if the lookup fails). */
moe_status_t moe_layer_forward_static(const moe_shape_t *shape, int64_t T, const uint16_t *x,
                                      const float *w_router, const float *router_bias,
                                      const float *shared_gate, const moe_experts_t *experts,
                                      const uint16_t *residual, uint16_t *out,
                                      hipStream_t stream);

/* ---- integer route: 8-bit activations x symmetric 4-bit experts ----------
 * The pages admit an integer MoE prefill route for the symmetric expert file
 * only (hipfire 0.4.3 benchmarks page, "Read this before comparing columns":
 * the "symmetric IU4 MoE" route) and report an INT8 prefill route replacing
 * an F16 one within a quality budget (same page, "Qwen3.8-Flash
 * (Flash-Next)" table). This library's definition of that route:
 *   - every activation row is quantized to int8 with one scale per row
 *     (moe_quantize_rows_i8): x per token; h per (token, expert) row, after
 *     rounding h to fp16;
 *   - the expert products are then exact: y = s_row * sum over groups of
 *     scale_g * sum_k q[k] * (nibble[k] - 8), int32 per group of 128,
 *     scales applied in fp32.
 * So the result is the exact layer evaluated on the 8-bit-rounded
 * activations; it differs from moe_expert_ffn by that rounding (about 1 % of
 * x's RMS per element for Gaussian rows, more for heavy-tailed h rows).
 * Supported: quant == MOE_Q4_SYM, group_size == 128, shared_inter == 0
 * (MOE_ERR_UNSUPPORTED otherwise), and T * H, T * k * I and the packed
 * weight bytes E * 2I * H / 2 below 2^31. */

/* Per-row int8 quantization of bf16 rows x [rows][cols] (cols % 8 == 0):
 *   a = max_c |x[r,c]|;  scale[r] = a / 127;
 *   q[r,c] = rint(x[r,c] * (127 / a))   (ties to even, in [-127, 127]),
 * with both divisions correctly rounded and the product rounded to fp32
 * before rint; a row with a < 2^-100 gives q = 0 and scale = 0.
 *   q [rows][cols] int8 (natural order), scale [rows] fp32.              */
moe_status_t moe_quantize_rows_i8(int64_t rows, int64_t cols, const uint16_t *x, int8_t *q,
                                  float *scale, hipStream_t stream);

/* moe_expert_ffn on the integer route (see above); same arguments, no shared
 * expert. y_perm [P][H] fp16, unweighted.
 *   h_perm  [P][I] fp16 or NULL: if given, receives the fp16 h rows (row r
 *           of expert-sorted order) from which the int8 h is quantized
 *   ws  >= moe_workspace_size(MOE_WS_EXPERT_FFN_I8, T) bytes (int8 x and its
 *          scales, fp16 h, int8 h and its scales)                          */
moe_status_t moe_expert_ffn_i8(const moe_shape_t *shape, int64_t T, const uint16_t *x,
                               const moe_experts_t *experts, const int32_t *counts,
                               const int32_t *offsets, const int32_t *sorted_pairs,
                               uint16_t *y_perm, uint16_t *h_perm, void *ws, size_t ws_bytes,
                               hipStream_t stream);

/* moe_layer_forward with the experts on the integer route: routing, grouping
 * and combine exactly as moe_layer_forward (fp32 router on the bf16 x).
 *   ws  >= moe_workspace_size(MOE_WS_LAYER_I8, T) bytes                   */
moe_status_t moe_layer_forward_i8(const moe_shape_t *shape, int64_t T, const uint16_t *x,
                                  const float *w_router, const float *router_bias,
                                  const moe_experts_t *experts, const uint16_t *residual,
                                  uint16_t *out, void *ws, size_t ws_bytes,
                                  hipStream_t stream);

/* ---- mixed-width experts: lower-bit tiers beside 4-bit experts ------------
 * The pages ship expert files where most routed experts are stored below
 * 4 bits and the rest stay at 4 bits (hipfire 0.4.3 benchmarks page, "New
 * Flash-Next tiers": 3-bit experts, and 2-bit experts, there with an E8P
 * codebook). They define neither format; this library's lower-bit codes are
 * plain symmetric scalar codes, w = (q - 2^(bits-1)) * scale, one fp16 scale
 * per group of G along K, with these row layouts (K * bits / 8 bytes a row):
 *   bits 4: byte j = element 2j (bits 0-3) | element 2j+1 (bits 4-7);
 *   bits 2: little-endian 32-bit word m holds elements 16m .. 16m+15, its
 *           bytes 0, 1, 2, 3 the word's elements 0-3, 8-11, 4-7, 12-15,
 *           element i of a byte's four in bits 2i, 2i+1;
 *   bits 3: 12 bytes per 32-element block: the low two bits of its elements
 *           in the 2-bit layout (8 bytes), then a 32-bit word whose bit 4c+i
 *           is the third bit of element 8c+i and bit 16+4c+i that of element
 *           8c+i+4 (c, i in 0..3).
 * (E8P's lattice codebook is not implemented.) Each width's experts are
 * stored in their own tensors; expert e of the layer is expert
 * expert_slot[e] of the tier whose bits equal expert_bits[e]. */
typedef struct {
  int32_t bits;                /* 4, 3 or 2 */
  int32_t num_experts;         /* E_b: experts stored at this width */
  const uint8_t  *w13;         /* [E_b][2I][H * bits / 8] */
  const uint16_t *w13_scale;   /* fp16 [E_b][2I][H/G] */
  const uint8_t  *w2;          /* [E_b][H][I * bits / 8] */
  const uint16_t *w2_scale;    /* fp16 [E_b][H][I/G] */
} moe_tier_t;

/* moe_expert_ffn over mixed-width experts (same numerics: fp16 weights
 * dequantized in registers, fp16 matrix cores, fp32 accumulation).
 *   tiers        host array of n_tiers (1..3) descriptors of distinct widths
 *   expert_bits  [E] int32 device array: each expert's width (one of the tiers')
 *   expert_slot  [E] int32 device array: its index within that tier's tensors
 *                (a slot outside [0, E_b) reads zeros, no fault)
 * Needs quant == MOE_Q4_SYM and shared_inter == 0; the tiers' w13 and w2 in
 * shape.w_layout (MOE_W_TILED: each one regrouped by moe_pack_tier); ws as
 * moe_expert_ffn (MOE_WS_EXPERT_FFN). One launch per tier and GEMM. */
moe_status_t moe_expert_ffn_mixed(const moe_shape_t *shape, int64_t T, const uint16_t *x,
                                  const moe_tier_t *tiers, int32_t n_tiers,
                                  const int32_t *expert_bits, const int32_t *expert_slot,
                                  const int32_t *counts, const int32_t *offsets,
                                  const int32_t *sorted_pairs, uint16_t *y_perm, void *ws,
                                  size_t ws_bytes, hipStream_t stream);

/* moe_layer_forward over mixed-width experts: routing, grouping and combine
 * as moe_layer_forward; ws as moe_layer_forward (MOE_WS_LAYER). */
moe_status_t moe_layer_forward_mixed(const moe_shape_t *shape, int64_t T, const uint16_t *x,
                                     const float *w_router, const float *router_bias,
                                     const moe_tier_t *tiers, int32_t n_tiers,
                                     const int32_t *expert_bits, const int32_t *expert_slot,
                                     const uint16_t *residual, uint16_t *out, void *ws,
                                     size_t ws_bytes, hipStream_t stream);

/* ---- host-resident experts streamed over PCIe, hot set in HBM --------------
 * The pages run models whose experts do not all fit the GPU: experts stay in
 * host memory and are streamed over PCIe during prefill, with a set of hot
 * experts kept resident, and long prompts become limited by that stream
 * (hipfire 0.4.3 benchmarks page, the Flash-Next rows: 2-bit experts held
 * in host memory behind a narrow PCIe link, and the note that a 4096-row
 * prefill chunk is bound by the expert transfers over PCIe). Here: the hot
 * experts are device tensors, the others (cold) sit in
 * host memory (pinned, hipHostMalloc, for asynchronous copies); every call
 * copies the cold experts, as many at a time as half of `stage` holds, into
 * the device staging buffer and runs them through the same grouped GEMMs
 * (symmetric 4-bit experts, no shared expert). With copy_stream NULL the
 * copies are ordered on `stream` with the kernels (time = copies +
 * compute); with another stream they run there, ordered by events (the
 * library creates and releases them in the call): they start once the work
 * `stream` held at entry is done, run at most two chunks ahead of the
 * kernels, and every kernel that reads a chunk waits for its copies, so they
 * overlap the routing, the hot experts and the previous chunk's compute.
 * When the call returns, work queued later on `stream` is ordered after
 * every copy. The result is bit-identical to moe_layer_forward with
 * every expert on the device.
 * Ownership: the caller keeps the cold host memory, `stage`, `ws` and `out`
 * alive and unchanged until the work the call queued (on both streams) has
 * completed; two calls in flight at once that share `stage` or `ws` race.
 *   hot        device experts, hot_count of them (hot may be NULL iff hot_count == 0)
 *   cold       host experts: the cold ones in ascending expert index, same
 *              layouts as moe_experts_t ([E_cold][...]); min and shared-expert
 *              pointers NULL
 *   hot_slot   HOST array [E]: expert e's index in `hot`, or -1 if it is cold
 *   stage      device buffer of stage_bytes; must hold at least two experts'
 *              packed weights and scales (moe_stream_stage_bytes(shape, 2))
 *   ws         >= moe_workspace_size(MOE_WS_LAYER, T) + 2 * 4 * E + 512 bytes */
moe_status_t moe_stream_stage_bytes(const moe_shape_t *shape, int32_t experts, size_t *bytes);
moe_status_t moe_layer_forward_streamed(const moe_shape_t *shape, int64_t T, const uint16_t *x,
                                        const float *w_router, const float *router_bias,
                                        const moe_experts_t *hot, int32_t hot_count,
                                        const moe_experts_t *cold, const int32_t *hot_slot,
                                        void *stage, size_t stage_bytes,
                                        const uint16_t *residual, uint16_t *out, void *ws,
                                        size_t ws_bytes, hipStream_t stream,
                                        hipStream_t copy_stream);

/* RMSNorm over rows of [T][H] bf16:
 *   out[t,h] = bf16( x[t,h] * (mean_h x[t,h]^2 + eps)^(-1/2) * weight[h] )
 * computed in fp32; weight [H] fp32. out must not alias x. */
/* Regroups one packed 4-bit matrix from MOE_W_ROWS into MOE_W_TILED, once,
 * when the weights are loaded (the layout a forward call then reads with
 * shape.w_layout = MOE_W_TILED):
 *   dst[((r / 16) * (K / 128) + k / 128) * 1024
 *       + (((k % 128) / 32) * 16 + r % 16) * 16 + (k % 32) / 2] = src[r * (K / 2) + k / 2]
 * for every row r < rows and even k < K (each byte holds elements k, k + 1).
 *   src [rows][K/2] bytes, dst the same size (device; must not overlap);
 *   rows % 16 == 0, K % 128 == 0, rows * K / 2 < 2^31 (else INVALID_ARGUMENT /
 *   UNSUPPORTED). Pack w13 with (E * 2I, H), w2 with (E * H, I), s13 with
 *   (2 I_s, H), s2 with (H, I_s). Enqueued on `stream`. */
moe_status_t moe_pack_w4(const uint8_t *src, uint8_t *dst, int64_t rows, int64_t K,
                         hipStream_t stream);

/* Regroups one packed matrix of a mixed-width tier (bits 4, 3 or 2, the row
 * layouts of moe_tier_t) into MOE_W_TILED, once, when the weights are
 * loaded; a mixed-width call with shape.w_layout = MOE_W_TILED reads every
 * tier this way. Each row's 32-element blocks (4 * bits bytes) move whole:
 *   block k / 32 of source row sigma(r) goes to byte offset
 *   ((r / 16) * (K / 128) + k / 128) * 256 * bits
 *       + (((k % 128) / 32) * 16 + r % 16) * 4 * bits
 * of dst, for every destination row r < rows. sigma(r) = r, except for the
 * 3- and 2-bit gate/up matrices (gate_up != 0, bits < 4), whose kernel reads
 * the rows of each 32-row group in pairs: for r = 32 g + 16 p + i (i < 16),
 *   sigma(r) = 32 g + 2 p + 8 (i / 4) + (0, 4, 1, 5)[i % 4].
 * With bits = 3 the block's third 32-bit word (the third bits) is also
 * re-ordered: its bit 4c + i + 16h (c, i < 4, h < 2) moves to bit
 *   (2 + 2i + 16h + (0, 1, 8, 9)[c]) mod 32.
 * With bits = 4 the result is that of moe_pack_w4.
 *   src [rows][K * bits / 8] bytes, dst the same size (device; 4-byte
 *   aligned; must not overlap); rows % 16 == 0 (% 32 for a 3- or 2-bit
 *   gate/up matrix), K % 128 == 0, rows * K * bits / 8 < 2^31 (else
 *   INVALID_ARGUMENT / UNSUPPORTED). Pack a tier's w13 with (E_b * 2I, H,
 *   bits, 1) and its w2 with (E_b * H, I, bits, 0). Enqueued on `stream`. */
moe_status_t moe_pack_tier(const uint8_t *src, uint8_t *dst, int64_t rows, int64_t K,
                           int32_t bits, int32_t gate_up, hipStream_t stream);

moe_status_t moe_rmsnorm(int64_t T, int64_t H, const uint16_t *x, const float *weight,
                         float eps, uint16_t *out, hipStream_t stream);

/* Optional kernel timing. While enabled, the library brackets each of its
 * kernel launches with HIP events recorded on the launch stream (a pool of
 * `max_launches` event pairs is created by moe_profile_enable; this is the
 * only allocation the library ever makes, and it happens outside the call
 * path). moe_profile_read synchronizes on the recorded events and returns,
 * for the kernel named `kernel`, the number of recorded launches and their
 * summed duration in milliseconds. moe_profile_enable(0) frees the pool. */
moe_status_t moe_profile_enable(int32_t max_launches);
moe_status_t moe_profile_reset(void);
moe_status_t moe_profile_read(const char *kernel, int64_t *launches, double *total_ms);

#ifdef __cplusplus
}
#endif
#endif /* QMOE_MOE_H */
