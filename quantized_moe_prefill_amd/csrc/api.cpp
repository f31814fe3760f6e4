// C ABI of the MoE prefill library: host-side validation, workspace layout,
// kernel sequencing on the caller's stream, error reporting and optional
// per-kernel event timing. See include/moe.h for the contract.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/moe.h"
#include "kernels.h"

namespace qmoe {

// ---------------------------------------------------------------------------
// errors
// ---------------------------------------------------------------------------

static thread_local char g_err[512] = "";

static moe_status_t fail(moe_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

static moe_status_t hip_fail(const char* what, hipError_t e) {
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ---------------------------------------------------------------------------
// profiling pool (events around each launch, only while enabled)
// ---------------------------------------------------------------------------

struct ProfRecord {
  const char* name;
  int slot;
};

static std::mutex g_prof_mu;
static std::vector<hipEvent_t> g_prof_events;  // 2 per slot
static std::vector<ProfRecord> g_prof_records;
static int g_prof_slots = 0;
static int g_prof_next = 0;

LaunchScope::LaunchScope(const char* n, hipStream_t s) : name(n), stream(s), slot(-1) {
  if (g_prof_slots == 0) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (g_prof_slots == 0 || g_prof_next >= g_prof_slots) return;
  slot = g_prof_next++;
  (void)hipEventRecord(g_prof_events[2 * slot], stream);
}

LaunchScope::~LaunchScope() {
  if (slot < 0) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  (void)hipEventRecord(g_prof_events[2 * slot + 1], stream);
  g_prof_records.push_back({name, slot});
}

// ---------------------------------------------------------------------------
// shapes and workspace
// ---------------------------------------------------------------------------

struct Shape {
  int H, E, k, I, G, Is;
  bool asym;
  bool tiled;  // expert weights in MOE_W_TILED
};

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

static moe_status_t check_shape(const moe_shape_t* s, int64_t T, Shape* out) {
  if (s == nullptr) return fail(MOE_ERR_INVALID_ARGUMENT, "shape is NULL");
  if (T < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "T must be >= 0 (got %lld)", (long long)T);
  if (s->hidden <= 0 || s->num_experts <= 0 || s->top_k <= 0 || s->inter <= 0 ||
      s->group_size <= 0 || s->shared_inter < 0)
    return fail(MOE_ERR_INVALID_ARGUMENT, "shape fields must be positive");
  if (s->w_layout != MOE_W_ROWS && s->w_layout != MOE_W_TILED)
    return fail(MOE_ERR_INVALID_ARGUMENT, "w_layout must be MOE_W_ROWS or MOE_W_TILED");
  if (s->quant != MOE_Q4_SYM && s->quant != MOE_Q4_ASYM)
    return fail(MOE_ERR_INVALID_ARGUMENT, "quant must be MOE_Q4_SYM or MOE_Q4_ASYM");
  if (s->top_k > s->num_experts)
    return fail(MOE_ERR_INVALID_ARGUMENT, "top_k (%lld) > num_experts (%lld)",
                (long long)s->top_k, (long long)s->num_experts);
  const int64_t G = s->group_size;
  if (G != 32 && G != 64 && G != 128)
    return fail(MOE_ERR_UNSUPPORTED, "group_size must be 32, 64 or 128 (got %lld)", (long long)G);
  if (s->hidden % 128 != 0 || s->hidden > 16384)
    return fail(MOE_ERR_UNSUPPORTED, "hidden must be a multiple of 128 and <= 16384");
  if (s->hidden % G != 0) return fail(MOE_ERR_UNSUPPORTED, "hidden must be a multiple of G");
  if (s->inter % 128 != 0 || s->inter > 65536)
    return fail(MOE_ERR_UNSUPPORTED, "inter must be a multiple of 128");
  if (s->shared_inter != 0 && (s->shared_inter % 128 != 0 || s->shared_inter > 65536))
    return fail(MOE_ERR_UNSUPPORTED, "shared_inter must be 0 or a multiple of 128");
  if (s->num_experts > 256) return fail(MOE_ERR_UNSUPPORTED, "num_experts must be <= 256");
  if (s->top_k > 8) return fail(MOE_ERR_UNSUPPORTED, "top_k must be <= 8");
  // The GEMM kernels address each activation, weight, scale and min tensor
  // through a 32-bit buffer descriptor with offsets computed in int: every
  // such tensor must stay below 2^31 bytes.
  const int64_t lim = int64_t(1) << 31;
  const int64_t E = s->num_experts, H = s->hidden, I = s->inter, Is = s->shared_inter;
  if (T * s->top_k >= lim) return fail(MOE_ERR_UNSUPPORTED, "T * top_k must be < 2^31");
  if (T * H * 2 >= lim || T * s->top_k * I * 2 >= lim || T * Is * 2 >= lim)
    return fail(MOE_ERR_UNSUPPORTED,
                "activation tensors (x, h, h_shared) must be below 2^31 bytes; "
                "split the tokens into chunks");
  if (E * 2 * I * (H / 2) >= lim || E * H * (I / 2) >= lim || E * 2 * I * (H / G) * 2 >= lim ||
      E * H * (I / G) * 2 >= lim)
    return fail(MOE_ERR_UNSUPPORTED, "expert weight tensors must be below 2^31 bytes");
  out->H = (int)s->hidden;
  out->E = (int)s->num_experts;
  out->k = (int)s->top_k;
  out->I = (int)s->inter;
  out->G = (int)G;
  out->Is = (int)s->shared_inter;
  out->asym = s->quant == MOE_Q4_ASYM;
  out->tiled = s->w_layout == MOE_W_TILED;
  return MOE_OK;
}

// calls whose kernels read only row-major weights
static moe_status_t rows_only(const Shape& s, const char* call) {
  if (s.tiled) return fail(MOE_ERR_UNSUPPORTED, "%s reads MOE_W_ROWS weights only", call);
  return MOE_OK;
}

static size_t al(size_t x) { return (x + 255) & ~size_t(255); }

struct Layout {
  size_t split, partial, hist, ids, tw, sw, counts, offsets, sorted, inv, x16, h, hs, yperm, ysh, total;
};

// Carve-up of the layer workspace. Each region is 256-byte aligned.
static Layout layer_layout(const Shape& s, int64_t T) {
  Layout L{};
  const size_t P = (size_t)T * s.k;
  size_t o = 0;
  L.split = o;   o = al(o + router_split_bytes(s.E, s.Is > 0, s.H));
  L.partial = o; o = al(o + router_partial_bytes((int)T, s.E, s.Is > 0, s.H));
  L.hist = o;    o = al(o + permute_ws_bytes((int)P, s.E));
  L.ids = o;     o = al(o + P * 4);
  L.tw = o;      o = al(o + P * 4);
  L.sw = o;      o = al(o + (size_t)T * 4);
  L.counts = o;  o = al(o + (size_t)s.E * 4);
  L.offsets = o; o = al(o + (size_t)(s.E + 1) * 4);
  L.sorted = o;  o = al(o + P * 4);
  L.inv = o;     o = al(o + P * 4);
  L.x16 = o;     o = al(o + (size_t)T * s.H * 2);
  L.h = o;       o = al(o + P * s.I * 2);
  L.hs = o;      o = al(o + (size_t)T * s.Is * 2);
  L.yperm = o;   o = al(o + P * s.H * 2);
  L.ysh = o;     o = al(o + (size_t)T * (s.Is > 0 ? s.H : 0) * 2);
  L.total = o;
  return L;
}

// moe_route scratch: the split router matrix, then the fp32 partial logits.
static size_t route_ws(const Shape& s, int64_t T) {
  return al(router_split_bytes(s.E, s.Is > 0, s.H)) +
         al(router_partial_bytes((int)T, s.E, s.Is > 0, s.H));
}
// moe_expert_ffn scratch: fp16 activations, h, shared h.
static size_t ffn_ws(const Shape& s, int64_t T) {
  const size_t P = (size_t)T * s.k;
  return al((size_t)T * s.H * 2) + al(P * s.I * 2) + al((size_t)T * s.Is * 2);
}

// ---- integer route ----
static moe_status_t check_i8(const Shape& s, int64_t T) {
  if (rows_only(s, "the integer route") != MOE_OK) return MOE_ERR_UNSUPPORTED;
  if (s.asym) return fail(MOE_ERR_UNSUPPORTED, "the integer route needs MOE_Q4_SYM experts");
  if (s.G != 128) return fail(MOE_ERR_UNSUPPORTED, "the integer route needs group_size 128");
  if (s.Is != 0) return fail(MOE_ERR_UNSUPPORTED, "the integer route has no shared expert");
  const int64_t lim = int64_t(1) << 31;
  if (T * s.H >= lim || T * s.k * s.I >= lim || (int64_t)s.E * s.I * s.H >= lim)
    return fail(MOE_ERR_UNSUPPORTED,
                "the integer route needs T*H, T*k*I and E*2I*H/2 below 2^31");
  return MOE_OK;
}

struct LayoutI8 {
  size_t xq, sx, h16, hq, sh, total;
};
// moe_expert_ffn_i8 scratch: int8 x and scales, fp16 h, int8 h and scales
static LayoutI8 ffn_i8_layout(const Shape& s, int64_t T, size_t base) {
  LayoutI8 L{};
  const size_t P = (size_t)T * s.k;
  size_t o = base;
  L.xq = o;  o = al(o + (size_t)T * s.H);
  L.sx = o;  o = al(o + (size_t)T * 4);
  L.h16 = o; o = al(o + P * s.I * 2);
  L.hq = o;  o = al(o + P * s.I);
  L.sh = o;  o = al(o + P * 4);
  L.total = o;
  return L;
}
// moe_layer_forward_i8: routing and grouping regions of the layer layout,
// then the integer FFN scratch, then y_perm
struct LayerI8 {
  Layout r;
  LayoutI8 f;
  size_t yperm, total;
};
static LayerI8 layer_i8_layout(const Shape& s, int64_t T) {
  LayerI8 L{};
  L.r = layer_layout(s, T);
  L.f = ffn_i8_layout(s, T, L.r.x16);  // replaces x16 .. ysh of the fp16 layer
  L.yperm = L.f.total;
  L.total = al(L.yperm + (size_t)T * s.k * s.H * 2);
  return L;
}

static moe_status_t check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return MOE_OK;
  if (ws == nullptr) return fail(MOE_ERR_INVALID_ARGUMENT, "workspace is NULL (need %zu bytes)", need);
  if (!aligned16(ws)) return fail(MOE_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
  if (have < need)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", have, need);
  return MOE_OK;
}

#define QMOE_REQUIRE(p, what)                                                   \
  do {                                                                          \
    if ((p) == nullptr) return fail(MOE_ERR_INVALID_ARGUMENT, "%s is NULL", what); \
    if (!aligned16(p)) return fail(MOE_ERR_UNSUPPORTED, "%s must be 16-byte aligned", what); \
  } while (0)
#define QMOE_OPTIONAL(p, what)                                                  \
  do {                                                                          \
    if ((p) != nullptr && !aligned16(p))                                        \
      return fail(MOE_ERR_UNSUPPORTED, "%s must be 16-byte aligned", what);     \
  } while (0)
#define QMOE_HIP(call, what)                                                    \
  do {                                                                          \
    hipError_t e_ = (call);                                                     \
    if (e_ != hipSuccess) return hip_fail(what, e_);                            \
  } while (0)

static moe_status_t check_experts(const Shape& s, const moe_experts_t* w) {
  if (w == nullptr) return fail(MOE_ERR_INVALID_ARGUMENT, "experts is NULL");
  QMOE_REQUIRE(w->w13, "experts->w13");
  QMOE_REQUIRE(w->w13_scale, "experts->w13_scale");
  QMOE_REQUIRE(w->w2, "experts->w2");
  QMOE_REQUIRE(w->w2_scale, "experts->w2_scale");
  if (s.asym) {
    QMOE_REQUIRE(w->w13_min, "experts->w13_min");
    QMOE_REQUIRE(w->w2_min, "experts->w2_min");
  } else if (w->w13_min != nullptr || w->w2_min != nullptr || w->s13_min != nullptr ||
             w->s2_min != nullptr) {
    return fail(MOE_ERR_INVALID_ARGUMENT, "min tensors must be NULL for MOE_Q4_SYM");
  }
  if (s.Is > 0) {
    QMOE_REQUIRE(w->s13, "experts->s13");
    QMOE_REQUIRE(w->s13_scale, "experts->s13_scale");
    QMOE_REQUIRE(w->s2, "experts->s2");
    QMOE_REQUIRE(w->s2_scale, "experts->s2_scale");
    if (s.asym) {
      QMOE_REQUIRE(w->s13_min, "experts->s13_min");
      QMOE_REQUIRE(w->s2_min, "experts->s2_min");
    }
  } else if (w->s13 != nullptr || w->s2 != nullptr) {
    return fail(MOE_ERR_INVALID_ARGUMENT, "shared-expert weights given but shared_inter == 0");
  }
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// implementations (arguments already validated)
// ---------------------------------------------------------------------------

static moe_status_t route_impl(const Shape& s, int64_t T, const uint16_t* x, const float* wr,
                               const float* bias, const float* sg, float* logits,
                               int32_t* ids, float* tw, float* sw, uint16_t* split,
                               float* partial, uint16_t* x16, hipStream_t st) {
  if (!router_uses_gemv((int)T))
    QMOE_HIP(launch_router_split(wr, sg, s.E, s.H, split, st), "router_split launch");
  QMOE_HIP(launch_router_topk(x, wr, sg, split, partial, bias, (int)T, s.H, s.E, s.k, logits, ids,
                              tw, sw, x16, st),
           "router launch");
  return MOE_OK;
}

static moe_status_t ffn_impl(const Shape& s, int64_t T, const uint16_t* x,
                             const moe_experts_t* w, const int32_t* counts,
                             const int32_t* offsets, const int32_t* sorted, uint16_t* yperm,
                             uint16_t* ysh, uint16_t* x16, uint16_t* h, uint16_t* hs,
                             bool x16_ready, hipStream_t st) {
  // x16_ready: x16 already holds x in fp16 kperm order (written by the router GEMM)
  const int P = (int)(T * s.k);
  GroupedGemm g{};
  g.A = x16;
  g.gather = sorted;
  g.gather_div = s.k;
  g.counts = counts;
  g.offsets = offsets;
  g.E = s.E;
  g.max_rows = P;
  g.a_rows = (int)T;
  g.W = w->w13;
  g.Wscale = w->w13_scale;
  g.Wmin = s.asym ? w->w13_min : nullptr;
  g.N = 2 * s.I;
  g.K = s.H;
  g.G = s.G;
  g.C = h;
  g.ldc = s.I;
  g.expect_rows = (int)T;
  g.w_tiled = s.tiled;
  // the weight-streaming gate/up reads the bf16 activations itself; the tiled
  // one wants them as fp16 in kperm order
  const bool x_direct = gemm_streams(g, true);
  if (x_direct) {
    g.A = x;
    g.a_bf16 = true;
  } else if (!x16_ready) {
    QMOE_HIP(launch_x_to_f16(x, x16, T * s.H, st), "x_to_f16 launch");
  }
  // A shared expert of the routed experts' shape runs as one more group of
  // the tiled launches (its T rows join the routed tiles instead of two
  // launches of their own that fill a fraction of the GPU).
  const bool fold_gu = s.Is > 0 && s.Is == s.I && !x_direct;
  if (fold_gu) {
    g.rows2 = (int)T;
    g.A2 = x16;
    g.W2 = w->s13;
    g.Wscale2 = w->s13_scale;
    g.Wmin2 = s.asym ? w->s13_min : nullptr;
    g.C2 = hs;
    g.ldc2 = s.Is;
  }
  QMOE_HIP(launch_gateup(g, st), "gateup launch");

  GroupedGemm d = g;
  d.A = h;
  d.a_bf16 = false;
  d.a_rows = P;
  d.gather = nullptr;
  d.W = w->w2;
  d.Wscale = w->w2_scale;
  d.Wmin = s.asym ? w->w2_min : nullptr;
  d.N = s.H;
  d.K = s.I;
  d.C = yperm;
  d.ldc = s.H;
  d.rows2 = 0;
  const bool fold_dn = fold_gu && !gemm_streams(d, false);
  if (fold_dn) {
    d.rows2 = (int)T;
    d.A2 = hs;
    d.W2 = w->s2;
    d.Wscale2 = w->s2_scale;
    d.Wmin2 = s.asym ? w->s2_min : nullptr;
    d.C2 = ysh;
    d.ldc2 = s.H;
  }
  QMOE_HIP(launch_down(d, st), "down launch");

  if (s.Is > 0 && !(fold_gu && fold_dn)) {
    GroupedGemm gs{};
    gs.A = x_direct ? x : x16;
    gs.a_bf16 = x_direct;
    gs.gather = nullptr;
    gs.gather_div = 1;
    gs.counts = nullptr;
    gs.offsets = nullptr;
    gs.rows_single = (int)T;
    gs.E = 1;
    gs.max_rows = (int)T;
    gs.a_rows = (int)T;
    gs.W = w->s13;
    gs.Wscale = w->s13_scale;
    gs.Wmin = s.asym ? w->s13_min : nullptr;
    gs.N = 2 * s.Is;
    gs.K = s.H;
    gs.G = s.G;
    gs.C = hs;
    gs.ldc = s.Is;
    gs.expect_rows = (int)T;
    gs.w_tiled = s.tiled;
    if (!fold_gu) {
      if (gs.a_bf16 && !gemm_streams(gs, true)) {
        if (!x16_ready) QMOE_HIP(launch_x_to_f16(x, x16, T * s.H, st), "x_to_f16 launch");
        gs.A = x16;
        gs.a_bf16 = false;
      }
      QMOE_HIP(launch_gateup(gs, st, "shared_gateup_gemm"), "shared gateup launch");
    }
    GroupedGemm ds = gs;
    ds.A = hs;
    ds.a_bf16 = false;
    ds.W = w->s2;
    ds.Wscale = w->s2_scale;
    ds.Wmin = s.asym ? w->s2_min : nullptr;
    ds.N = s.H;
    ds.K = s.Is;
    ds.C = ysh;
    ds.ldc = s.H;
    QMOE_HIP(launch_down(ds, st, "shared_down_gemm"), "shared down launch");
  }
  return MOE_OK;
}

static moe_status_t ffn_i8_impl(const Shape& s, int64_t T, const uint16_t* x,
                                const moe_experts_t* w, const int32_t* counts,
                                const int32_t* offsets, const int32_t* sorted, uint16_t* yperm,
                                uint16_t* h_out, uint8_t* base, const LayoutI8& L,
                                hipStream_t st) {
  const int P = (int)(T * s.k);
  auto* xq = reinterpret_cast<int8_t*>(base + L.xq);
  auto* sx = reinterpret_cast<float*>(base + L.sx);
  auto* h16 = h_out != nullptr ? h_out : reinterpret_cast<uint16_t*>(base + L.h16);
  auto* hq = reinterpret_cast<int8_t*>(base + L.hq);
  auto* sh = reinterpret_cast<float*>(base + L.sh);
  QMOE_HIP(launch_quant_rows_i8(x, false, (int)T, s.H, true, xq, sx, st), "quantize x launch");
  GemmI8 g{};
  g.A = xq;
  g.a_scale = sx;
  g.gather = sorted;
  g.gather_div = s.k;
  g.counts = counts;
  g.offsets = offsets;
  g.E = s.E;
  g.max_rows = P;
  g.a_rows = (int)T;
  g.W = w->w13;
  g.Wscale = w->w13_scale;
  g.N = 2 * s.I;
  g.K = s.H;
  g.C = h16;
  g.ldc = s.I;
  QMOE_HIP(launch_gateup_i8(g, st), "gateup (int8) launch");
  QMOE_HIP(launch_quant_rows_i8(h16, true, P, s.I, true, hq, sh, st), "quantize h launch");
  GemmI8 d = g;
  d.A = hq;
  d.a_scale = sh;
  d.gather = nullptr;
  d.gather_div = 1;
  d.a_rows = P;
  d.W = w->w2;
  d.Wscale = w->w2_scale;
  d.N = s.H;
  d.K = s.I;
  d.C = yperm;
  d.ldc = s.H;
  QMOE_HIP(launch_down_i8(d, st), "down (int8) launch");
  return MOE_OK;
}

// ---- mixed-width experts ----
static moe_status_t check_tiers(const Shape& s, const moe_tier_t* tiers, int32_t n) {
  if (s.asym) return fail(MOE_ERR_UNSUPPORTED, "mixed-width experts need MOE_Q4_SYM");
  if (s.Is != 0) return fail(MOE_ERR_UNSUPPORTED, "mixed-width layers have no shared expert");
  if (tiers == nullptr) return fail(MOE_ERR_INVALID_ARGUMENT, "tiers is NULL");
  if (n < 1 || n > 3) return fail(MOE_ERR_INVALID_ARGUMENT, "n_tiers must be 1..3 (got %d)", n);
  unsigned seen = 0;
  for (int i = 0; i < n; ++i) {
    const moe_tier_t& t = tiers[i];
    if (t.bits != 4 && t.bits != 3 && t.bits != 2)
      return fail(MOE_ERR_UNSUPPORTED, "tier bits must be 4, 3 or 2 (got %d)", t.bits);
    if (seen & (1u << t.bits)) return fail(MOE_ERR_INVALID_ARGUMENT, "two tiers of %d bits", t.bits);
    seen |= 1u << t.bits;
    if (t.num_experts < 1) return fail(MOE_ERR_INVALID_ARGUMENT, "tier num_experts must be >= 1");
    QMOE_REQUIRE(t.w13, "tier w13");
    QMOE_REQUIRE(t.w13_scale, "tier w13_scale");
    QMOE_REQUIRE(t.w2, "tier w2");
    QMOE_REQUIRE(t.w2_scale, "tier w2_scale");
    if ((int64_t)t.num_experts * 2 * s.I * s.H / 8 * t.bits >= (int64_t(1) << 31))
      return fail(MOE_ERR_UNSUPPORTED, "a tier's packed weights must be below 2^31 bytes");
  }
  return MOE_OK;
}

static moe_status_t ffn_mixed_impl(const Shape& s, int64_t T, const uint16_t* x,
                                   const moe_tier_t* tiers, int32_t n_tiers,
                                   const int32_t* ebits, const int32_t* eslot,
                                   const int32_t* counts, const int32_t* offsets,
                                   const int32_t* sorted, uint16_t* yperm, uint16_t* x16,
                                   uint16_t* h, bool x16_ready, hipStream_t st) {
  const int P = (int)(T * s.k);
  if (!x16_ready) QMOE_HIP(launch_x_to_f16(x, x16, T * s.H, st), "x_to_f16 launch");
  GroupedGemm g{};
  g.A = x16;
  g.gather = sorted;
  g.gather_div = s.k;
  g.counts = counts;
  g.offsets = offsets;
  g.E = s.E;
  g.max_rows = P;
  g.a_rows = (int)T;
  g.N = 2 * s.I;
  g.K = s.H;
  g.G = s.G;
  g.C = h;
  g.ldc = s.I;
  g.tier = ebits;
  g.slot = eslot;
  g.w_tiled = s.tiled;  // every tier packed by moe_pack_tier
  for (int i = 0; i < n_tiers; ++i) {
    g.W = tiers[i].w13;
    g.Wscale = tiers[i].w13_scale;
    g.w_experts = tiers[i].num_experts;
    g.bits = tiers[i].bits;
    g.tier_id = tiers[i].bits;  // expert_bits holds the widths
    QMOE_HIP(launch_gateup(g, st), "gateup launch");
  }
  GroupedGemm d = g;
  d.A = h;
  d.a_rows = P;
  d.gather = nullptr;
  d.N = s.H;
  d.K = s.I;
  d.C = yperm;
  d.ldc = s.H;
  for (int i = 0; i < n_tiers; ++i) {
    d.W = tiers[i].w2;
    d.Wscale = tiers[i].w2_scale;
    d.w_experts = tiers[i].num_experts;
    d.bits = tiers[i].bits;
    d.tier_id = tiers[i].bits;
    QMOE_HIP(launch_down(d, st), "down launch");
  }
  return MOE_OK;
}

// ---- host-streamed experts ----
// One expert's packed bytes (symmetric 4-bit, no mins), each array padded
// to 256 bytes inside a staging slot.
struct StageLayout {
  size_t w13, s13, w2, s2;  // bytes per expert of each array
};
static StageLayout stage_layout(const Shape& s) {
  StageLayout L;
  L.w13 = (size_t)2 * s.I * s.H / 2;
  L.s13 = (size_t)2 * s.I * (s.H / s.G) * 2;
  L.w2 = (size_t)s.H * s.I / 2;
  L.s2 = (size_t)s.H * (s.I / s.G) * 2;
  return L;
}
static size_t stage_slot_bytes(const StageLayout& L, int n) {
  return al(L.w13 * n) + al(L.s13 * n) + al(L.w2 * n) + al(L.s2 * n);
}


// Arguments of moe_layer_forward and moe_layer_forward_static (everything
// but the workspace).
static moe_status_t check_layer_args(const moe_shape_t* shape, int64_t T, const uint16_t* x,
                                     const float* w_router, const float* router_bias,
                                     const float* shared_gate, const moe_experts_t* experts,
                                     const uint16_t* residual, uint16_t* out, Shape* sp) {
  Shape& s = *sp;
  moe_status_t st = check_shape(shape, T, &s);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  QMOE_REQUIRE(x, "x");
  QMOE_REQUIRE(w_router, "w_router");
  QMOE_REQUIRE(out, "out");
  QMOE_OPTIONAL(router_bias, "router_bias");
  QMOE_OPTIONAL(residual, "residual");
  st = check_experts(s, experts);
  if (st != MOE_OK) return st;
  if (s.Is > 0) {
    QMOE_REQUIRE(shared_gate, "shared_gate");
  } else if (shared_gate != nullptr) {
    return fail(MOE_ERR_INVALID_ARGUMENT, "shared_gate given but shared_inter == 0");
  }
  return MOE_OK;
}

// The layer on a validated call, with scratch carved from `b` (at least
// layer_layout(s, T).total bytes).
static moe_status_t layer_run(const Shape& s, int64_t T, const uint16_t* x,
                              const float* w_router, const float* router_bias,
                              const float* shared_gate, const moe_experts_t* experts,
                              const uint16_t* residual, uint16_t* out, uint8_t* b,
                              hipStream_t stream) {
  moe_status_t st;
  const Layout L = layer_layout(s, T);
  auto* split = reinterpret_cast<uint16_t*>(b + L.split);
  auto* partial = reinterpret_cast<float*>(b + L.partial);
  auto* hist = reinterpret_cast<int32_t*>(b + L.hist);
  auto* ids = reinterpret_cast<int32_t*>(b + L.ids);
  auto* tw = reinterpret_cast<float*>(b + L.tw);
  auto* sw = s.Is > 0 ? reinterpret_cast<float*>(b + L.sw) : nullptr;
  auto* counts = reinterpret_cast<int32_t*>(b + L.counts);
  auto* offsets = reinterpret_cast<int32_t*>(b + L.offsets);
  auto* sorted = reinterpret_cast<int32_t*>(b + L.sorted);
  auto* inv = reinterpret_cast<int32_t*>(b + L.inv);
  auto* x16 = reinterpret_cast<uint16_t*>(b + L.x16);
  auto* h = reinterpret_cast<uint16_t*>(b + L.h);
  auto* hs = reinterpret_cast<uint16_t*>(b + L.hs);
  auto* yperm = reinterpret_cast<uint16_t*>(b + L.yperm);
  auto* ysh = s.Is > 0 ? reinterpret_cast<uint16_t*>(b + L.ysh) : nullptr;

  if (router_uses_gemv((int)T) && (s.Is == 0 || shared_gate != nullptr) &&
      small_layer_supported((int)T, s.H, s.I, s.Is, s.E, s.k, s.G)) {
    // a few tokens: router logits, then top-k, grouping and gate/up in one
    // launch, down in another (both with the shared expert), then combine
    QMOE_HIP(launch_router_gemv(x, w_router, s.Is > 0 ? shared_gate : nullptr, (int)T, s.H, s.E,
                                partial, stream),
             "router launch");
    SmallLayer a{};
    a.x = x;
    a.bias = router_bias;
    a.w13 = experts->w13;
    a.w13_scale = experts->w13_scale;
    a.w13_min = s.asym ? experts->w13_min : nullptr;
    a.w2 = experts->w2;
    a.w2_scale = experts->w2_scale;
    a.w2_min = s.asym ? experts->w2_min : nullptr;
    a.s13 = experts->s13;
    a.s13_scale = experts->s13_scale;
    a.s13_min = s.asym ? experts->s13_min : nullptr;
    a.s2 = experts->s2;
    a.s2_scale = experts->s2_scale;
    a.s2_min = s.asym ? experts->s2_min : nullptr;
    a.T = (int)T;
    a.H = s.H;
    a.E = s.E;
    a.k = s.k;
    a.I = s.I;
    a.G = s.G;
    a.has_shared = s.Is > 0 ? 1 : 0;
    a.w_tiled = s.tiled;
    a.Epad = router_padded_rows(s.E, s.Is > 0);
    a.nbits = 0;
    while ((1 << a.nbits) < s.E) ++a.nbits;
    a.logits = partial;
    a.h = h;
    a.hs = hs;
    a.yperm = yperm;
    a.ysh = ysh;
    a.ids = ids;
    a.inv = inv;
    a.sorted = sorted;
    a.counts = counts;
    a.offsets = offsets;
    a.tw = tw;
    a.sw = sw;
    QMOE_HIP(launch_small_experts(a, stream), "expert launches");
    QMOE_HIP(launch_combine(yperm, inv, tw, ysh, sw, residual, out, (int)T, s.H, s.k, stream),
             "combine launch");
    return MOE_OK;
  }
  if (router_uses_gemv((int)T)) {
    // a few tokens: the router product, then top-k and grouping in one workgroup
    QMOE_HIP(launch_route_permute_small(x, w_router, shared_gate, partial, router_bias, (int)T,
                                        s.H, s.E, s.k, ids, tw, sw, counts, offsets, sorted, inv,
                                        stream),
             "router launch");
  } else {
    st = route_impl(s, T, x, w_router, router_bias, shared_gate, nullptr, ids, tw, sw, split,
                    partial, x16, stream);
    if (st != MOE_OK) return st;
    QMOE_HIP(launch_permute(ids, (int)(T * s.k), s.E, counts, offsets, sorted, inv, hist, stream),
             "permute launch");
  }
  st = ffn_impl(s, T, x, experts, counts, offsets, sorted, yperm, ysh, x16, h, hs,
                !router_uses_gemv((int)T), stream);
  if (st != MOE_OK) return st;
  QMOE_HIP(launch_combine(yperm, inv, tw, ysh, sw, residual, out, (int)T, s.H, s.k, stream),
           "combine launch");
  return MOE_OK;
}


// ---------------------------------------------------------------------------
// static workspace of moe_layer_forward_static
// ---------------------------------------------------------------------------

// One array per GPU the library runs on, held until the process ends. In
// host code `scratch` is only a stand-in for the symbol: the device address
// of each GPU's copy comes from hipGetSymbolAddress with that GPU current.
static __device__ __align__(256) uint8_t scratch[MOE_STATIC_WS_BYTES];

static std::mutex g_scratch_mu;
static std::vector<uint8_t*> g_scratch_dev;  // device address per device index

// The current device's copy of `scratch`, looked up once per device.
static moe_status_t static_workspace(uint8_t** out) {
  int dev = 0;
  QMOE_HIP(hipGetDevice(&dev), "hipGetDevice");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if ((size_t)dev >= g_scratch_dev.size()) g_scratch_dev.resize(dev + 1, nullptr);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    QMOE_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255u) != 0)
      return fail(MOE_ERR_HIP, "static workspace: unexpected device address %p", p);
    g_scratch_dev[dev] = static_cast<uint8_t*>(p);
  }
  *out = g_scratch_dev[dev];
  return MOE_OK;
}

}  // namespace qmoe

using namespace qmoe;

// ---------------------------------------------------------------------------
// exported C ABI
// ---------------------------------------------------------------------------

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_last_error(void) { return g_err; }

moe_status_t moe_workspace_size(const moe_shape_t* shape, int64_t T, int32_t kind,
                                size_t* bytes) {
  Shape s;
  moe_status_t st = check_shape(shape, T, &s);
  if (st != MOE_OK) return st;
  if (bytes == nullptr) return fail(MOE_ERR_INVALID_ARGUMENT, "bytes is NULL");
  switch (kind) {
    case MOE_WS_LAYER: *bytes = layer_layout(s, T).total; break;
    case MOE_WS_ROUTE: *bytes = route_ws(s, T); break;
    case MOE_WS_PERMUTE: *bytes = al(permute_ws_bytes((int)(T * s.k), s.E)); break;
    case MOE_WS_EXPERT_FFN: *bytes = ffn_ws(s, T); break;
    case MOE_WS_LAYER_I8:
    case MOE_WS_EXPERT_FFN_I8:
      st = check_i8(s, T);
      if (st != MOE_OK) return st;
      *bytes = kind == MOE_WS_LAYER_I8 ? layer_i8_layout(s, T).total : ffn_i8_layout(s, T, 0).total;
      break;
    default: return fail(MOE_ERR_INVALID_ARGUMENT, "unknown workspace kind %d", kind);
  }
  return MOE_OK;
}

moe_status_t moe_route(const moe_shape_t* shape, int64_t T, const uint16_t* x,
                       const float* w_router, const float* router_bias,
                       const float* shared_gate, float* logits, int32_t* topk_ids,
                       float* topk_w, float* shared_w, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  Shape s;
  moe_status_t st = check_shape(shape, T, &s);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  QMOE_REQUIRE(x, "x");
  QMOE_REQUIRE(w_router, "w_router");
  QMOE_REQUIRE(topk_ids, "topk_ids");
  QMOE_REQUIRE(topk_w, "topk_w");
  QMOE_OPTIONAL(router_bias, "router_bias");
  QMOE_OPTIONAL(shared_gate, "shared_gate");
  QMOE_OPTIONAL(logits, "logits");
  if ((shared_gate == nullptr) != (shared_w == nullptr))
    return fail(MOE_ERR_INVALID_ARGUMENT, "shared_gate and shared_w go together");
  QMOE_OPTIONAL(shared_w, "shared_w");
  // the shared gate belongs to a shape with a shared expert (as in
  // moe_layer_forward), so the MOE_WS_ROUTE size, which pads the split router
  // matrix for the gate row exactly when shared_inter > 0, always suffices
  if (shared_gate != nullptr && s.Is == 0)
    return fail(MOE_ERR_INVALID_ARGUMENT, "shared_gate given but shared_inter == 0");
  st = check_ws(ws, ws_bytes, route_ws(s, T));
  if (st != MOE_OK) return st;
  auto* wsb = static_cast<uint8_t*>(ws);
  return route_impl(s, T, x, w_router, router_bias, shared_gate, logits, topk_ids, topk_w,
                    shared_w, reinterpret_cast<uint16_t*>(wsb),
                    reinterpret_cast<float*>(wsb + al(router_split_bytes(s.E, s.Is > 0, s.H))),
                    nullptr, stream);
}

moe_status_t moe_permute(const moe_shape_t* shape, int64_t T, const int32_t* topk_ids,
                         int32_t* counts, int32_t* offsets, int32_t* sorted_pairs,
                         int32_t* inv, void* ws, size_t ws_bytes, hipStream_t stream) {
  Shape s;
  moe_status_t st = check_shape(shape, T, &s);
  if (st != MOE_OK) return st;
  QMOE_REQUIRE(counts, "counts");
  QMOE_REQUIRE(offsets, "offsets");
  const int P = (int)(T * s.k);
  st = check_ws(ws, ws_bytes, al(permute_ws_bytes(P, s.E)));
  if (st != MOE_OK) return st;
  if (P > 0) {
    QMOE_REQUIRE(topk_ids, "topk_ids");
    QMOE_REQUIRE(sorted_pairs, "sorted_pairs");
    QMOE_REQUIRE(inv, "inv");
  }
  // an empty batch still launches, so that zero counts/offsets are written
  // asynchronously like every other result
  QMOE_HIP(launch_permute(topk_ids, P, s.E, counts, offsets, sorted_pairs, inv,
                          static_cast<int32_t*>(ws), stream),
           "permute launch");
  return MOE_OK;
}

moe_status_t moe_expert_ffn(const moe_shape_t* shape, int64_t T, const uint16_t* x,
                            const moe_experts_t* experts, const int32_t* counts,
                            const int32_t* offsets, const int32_t* sorted_pairs,
                            uint16_t* y_perm, uint16_t* y_shared, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  Shape s;
  moe_status_t st = check_shape(shape, T, &s);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  QMOE_REQUIRE(x, "x");
  st = check_experts(s, experts);
  if (st != MOE_OK) return st;
  QMOE_REQUIRE(counts, "counts");
  QMOE_REQUIRE(offsets, "offsets");
  QMOE_REQUIRE(sorted_pairs, "sorted_pairs");
  QMOE_REQUIRE(y_perm, "y_perm");
  if (s.Is > 0) {
    QMOE_REQUIRE(y_shared, "y_shared");
  } else if (y_shared != nullptr) {
    return fail(MOE_ERR_INVALID_ARGUMENT, "y_shared given but shared_inter == 0");
  }
  st = check_ws(ws, ws_bytes, ffn_ws(s, T));
  if (st != MOE_OK) return st;
  uint8_t* base = static_cast<uint8_t*>(ws);
  const size_t P = (size_t)T * s.k;
  uint16_t* x16 = reinterpret_cast<uint16_t*>(base);
  uint16_t* h = reinterpret_cast<uint16_t*>(base + al((size_t)T * s.H * 2));
  uint16_t* hs = reinterpret_cast<uint16_t*>(base + al((size_t)T * s.H * 2) + al(P * s.I * 2));
  return ffn_impl(s, T, x, experts, counts, offsets, sorted_pairs, y_perm, y_shared, x16, h,
                  hs, false, stream);
}

moe_status_t moe_combine(const moe_shape_t* shape, int64_t T, const uint16_t* y_perm,
                         const int32_t* inv, const float* topk_w, const uint16_t* y_shared,
                         const float* shared_w, const uint16_t* residual, uint16_t* out,
                         hipStream_t stream) {
  Shape s;
  moe_status_t st = check_shape(shape, T, &s);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  QMOE_REQUIRE(y_perm, "y_perm");
  QMOE_REQUIRE(inv, "inv");
  QMOE_REQUIRE(topk_w, "topk_w");
  QMOE_REQUIRE(out, "out");
  QMOE_OPTIONAL(y_shared, "y_shared");
  QMOE_OPTIONAL(residual, "residual");
  if ((y_shared == nullptr) != (shared_w == nullptr))
    return fail(MOE_ERR_INVALID_ARGUMENT, "y_shared and shared_w go together");
  QMOE_HIP(launch_combine(y_perm, inv, topk_w, y_shared, shared_w, residual, out, (int)T, s.H,
                          s.k, stream),
           "combine launch");
  return MOE_OK;
}

moe_status_t moe_layer_forward(const moe_shape_t* shape, int64_t T, const uint16_t* x,
                               const float* w_router, const float* router_bias,
                               const float* shared_gate, const moe_experts_t* experts,
                               const uint16_t* residual, uint16_t* out, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
  Shape s;
  moe_status_t st = check_layer_args(shape, T, x, w_router, router_bias, shared_gate, experts,
                                     residual, out, &s);
  if (st != MOE_OK || T == 0) return st;
  st = check_ws(ws, ws_bytes, layer_layout(s, T).total);
  if (st != MOE_OK) return st;
  return layer_run(s, T, x, w_router, router_bias, shared_gate, experts, residual, out,
                   static_cast<uint8_t*>(ws), stream);
}

moe_status_t moe_layer_forward_static(const moe_shape_t* shape, int64_t T, const uint16_t* x,
                                      const float* w_router, const float* router_bias,
                                      const float* shared_gate, const moe_experts_t* experts,
                                      const uint16_t* residual, uint16_t* out,
                                      hipStream_t stream) {
  Shape s;
  moe_status_t st = check_layer_args(shape, T, x, w_router, router_bias, shared_gate, experts,
                                     residual, out, &s);
  if (st != MOE_OK || T == 0) return st;
  const size_t need = layer_layout(s, T).total;
  if (need > (size_t)MOE_STATIC_WS_BYTES)
    return fail(MOE_ERR_UNSUPPORTED,
                "this call needs %zu bytes of workspace; the static workspace holds %zu "
                "(use moe_layer_forward with a caller workspace, or fewer tokens per call)",
                need, (size_t)MOE_STATIC_WS_BYTES);
  uint8_t* ws = nullptr;
  st = static_workspace(&ws);
  if (st != MOE_OK) return st;
  return layer_run(s, T, x, w_router, router_bias, shared_gate, experts, residual, out, ws,
                   stream);
}

moe_status_t moe_quantize_rows_i8(int64_t rows, int64_t cols, const uint16_t* x, int8_t* q,
                                  float* scale, hipStream_t stream) {
  if (rows < 0 || cols <= 0) return fail(MOE_ERR_INVALID_ARGUMENT, "rows must be >= 0 and cols > 0");
  if (cols % 8 != 0) return fail(MOE_ERR_UNSUPPORTED, "cols must be a multiple of 8");
  if (rows >= (int64_t(1) << 31) || cols >= (int64_t(1) << 31))
    return fail(MOE_ERR_UNSUPPORTED, "rows and cols must be below 2^31");
  if (rows == 0) return MOE_OK;
  QMOE_REQUIRE(x, "x");
  QMOE_REQUIRE(q, "q");
  QMOE_REQUIRE(scale, "scale");
  QMOE_HIP(launch_quant_rows_i8(x, false, (int)rows, (int)cols, false, q, scale, stream),
           "quantize launch");
  return MOE_OK;
}

moe_status_t moe_expert_ffn_i8(const moe_shape_t* shape, int64_t T, const uint16_t* x,
                               const moe_experts_t* experts, const int32_t* counts,
                               const int32_t* offsets, const int32_t* sorted_pairs,
                               uint16_t* y_perm, uint16_t* h_perm, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
  Shape s;
  moe_status_t st = check_shape(shape, T, &s);
  if (st != MOE_OK) return st;
  st = check_i8(s, T);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  QMOE_REQUIRE(x, "x");
  st = check_experts(s, experts);
  if (st != MOE_OK) return st;
  QMOE_REQUIRE(counts, "counts");
  QMOE_REQUIRE(offsets, "offsets");
  QMOE_REQUIRE(sorted_pairs, "sorted_pairs");
  QMOE_REQUIRE(y_perm, "y_perm");
  QMOE_OPTIONAL(h_perm, "h_perm");
  const LayoutI8 L = ffn_i8_layout(s, T, 0);
  st = check_ws(ws, ws_bytes, L.total);
  if (st != MOE_OK) return st;
  return ffn_i8_impl(s, T, x, experts, counts, offsets, sorted_pairs, y_perm, h_perm,
                     static_cast<uint8_t*>(ws), L, stream);
}

moe_status_t moe_layer_forward_i8(const moe_shape_t* shape, int64_t T, const uint16_t* x,
                                  const float* w_router, const float* router_bias,
                                  const moe_experts_t* experts, const uint16_t* residual,
                                  uint16_t* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  Shape s;
  moe_status_t st = check_shape(shape, T, &s);
  if (st != MOE_OK) return st;
  st = check_i8(s, T);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  QMOE_REQUIRE(x, "x");
  QMOE_REQUIRE(w_router, "w_router");
  QMOE_REQUIRE(out, "out");
  QMOE_OPTIONAL(router_bias, "router_bias");
  QMOE_OPTIONAL(residual, "residual");
  st = check_experts(s, experts);
  if (st != MOE_OK) return st;
  const LayerI8 L = layer_i8_layout(s, T);
  st = check_ws(ws, ws_bytes, L.total);
  if (st != MOE_OK) return st;
  uint8_t* b = static_cast<uint8_t*>(ws);
  auto* split = reinterpret_cast<uint16_t*>(b + L.r.split);
  auto* partial = reinterpret_cast<float*>(b + L.r.partial);
  auto* hist = reinterpret_cast<int32_t*>(b + L.r.hist);
  auto* ids = reinterpret_cast<int32_t*>(b + L.r.ids);
  auto* tw = reinterpret_cast<float*>(b + L.r.tw);
  auto* counts = reinterpret_cast<int32_t*>(b + L.r.counts);
  auto* offsets = reinterpret_cast<int32_t*>(b + L.r.offsets);
  auto* sorted = reinterpret_cast<int32_t*>(b + L.r.sorted);
  auto* inv = reinterpret_cast<int32_t*>(b + L.r.inv);
  auto* yperm = reinterpret_cast<uint16_t*>(b + L.yperm);
  if (router_uses_gemv((int)T)) {
    QMOE_HIP(launch_route_permute_small(x, w_router, nullptr, partial, router_bias, (int)T, s.H,
                                        s.E, s.k, ids, tw, nullptr, counts, offsets, sorted, inv,
                                        stream),
             "router launch");
  } else {
    st = route_impl(s, T, x, w_router, router_bias, nullptr, nullptr, ids, tw, nullptr, split,
                    partial, nullptr, stream);
    if (st != MOE_OK) return st;
    QMOE_HIP(launch_permute(ids, (int)(T * s.k), s.E, counts, offsets, sorted, inv, hist, stream),
             "permute launch");
  }
  st = ffn_i8_impl(s, T, x, experts, counts, offsets, sorted, yperm, nullptr, b, L.f, stream);
  if (st != MOE_OK) return st;
  QMOE_HIP(launch_combine(yperm, inv, tw, nullptr, nullptr, residual, out, (int)T, s.H, s.k, stream),
           "combine launch");
  return MOE_OK;
}

moe_status_t moe_expert_ffn_mixed(const moe_shape_t* shape, int64_t T, const uint16_t* x,
                                  const moe_tier_t* tiers, int32_t n_tiers,
                                  const int32_t* expert_bits, const int32_t* expert_slot,
                                  const int32_t* counts, const int32_t* offsets,
                                  const int32_t* sorted_pairs, uint16_t* y_perm, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
  Shape s;
  moe_status_t st = check_shape(shape, T, &s);
  if (st != MOE_OK) return st;
  st = check_tiers(s, tiers, n_tiers);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  QMOE_REQUIRE(x, "x");
  QMOE_REQUIRE(expert_bits, "expert_bits");
  QMOE_REQUIRE(expert_slot, "expert_slot");
  QMOE_REQUIRE(counts, "counts");
  QMOE_REQUIRE(offsets, "offsets");
  QMOE_REQUIRE(sorted_pairs, "sorted_pairs");
  QMOE_REQUIRE(y_perm, "y_perm");
  st = check_ws(ws, ws_bytes, ffn_ws(s, T));
  if (st != MOE_OK) return st;
  uint8_t* base = static_cast<uint8_t*>(ws);
  uint16_t* x16 = reinterpret_cast<uint16_t*>(base);
  uint16_t* h = reinterpret_cast<uint16_t*>(base + al((size_t)T * s.H * 2));
  return ffn_mixed_impl(s, T, x, tiers, n_tiers, expert_bits, expert_slot, counts, offsets,
                        sorted_pairs, y_perm, x16, h, false, stream);
}

moe_status_t moe_layer_forward_mixed(const moe_shape_t* shape, int64_t T, const uint16_t* x,
                                     const float* w_router, const float* router_bias,
                                     const moe_tier_t* tiers, int32_t n_tiers,
                                     const int32_t* expert_bits, const int32_t* expert_slot,
                                     const uint16_t* residual, uint16_t* out, void* ws,
                                     size_t ws_bytes, hipStream_t stream) {
  Shape s;
  moe_status_t st = check_shape(shape, T, &s);
  if (st != MOE_OK) return st;
  st = check_tiers(s, tiers, n_tiers);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  QMOE_REQUIRE(x, "x");
  QMOE_REQUIRE(w_router, "w_router");
  QMOE_REQUIRE(out, "out");
  QMOE_REQUIRE(expert_bits, "expert_bits");
  QMOE_REQUIRE(expert_slot, "expert_slot");
  QMOE_OPTIONAL(router_bias, "router_bias");
  QMOE_OPTIONAL(residual, "residual");
  const Layout L = layer_layout(s, T);
  st = check_ws(ws, ws_bytes, L.total);
  if (st != MOE_OK) return st;
  uint8_t* b = static_cast<uint8_t*>(ws);
  auto* split = reinterpret_cast<uint16_t*>(b + L.split);
  auto* partial = reinterpret_cast<float*>(b + L.partial);
  auto* hist = reinterpret_cast<int32_t*>(b + L.hist);
  auto* ids = reinterpret_cast<int32_t*>(b + L.ids);
  auto* tw = reinterpret_cast<float*>(b + L.tw);
  auto* counts = reinterpret_cast<int32_t*>(b + L.counts);
  auto* offsets = reinterpret_cast<int32_t*>(b + L.offsets);
  auto* sorted = reinterpret_cast<int32_t*>(b + L.sorted);
  auto* inv = reinterpret_cast<int32_t*>(b + L.inv);
  auto* x16 = reinterpret_cast<uint16_t*>(b + L.x16);
  auto* h = reinterpret_cast<uint16_t*>(b + L.h);
  auto* yperm = reinterpret_cast<uint16_t*>(b + L.yperm);
  if (router_uses_gemv((int)T)) {
    QMOE_HIP(launch_route_permute_small(x, w_router, nullptr, partial, router_bias, (int)T, s.H,
                                        s.E, s.k, ids, tw, nullptr, counts, offsets, sorted, inv,
                                        stream),
             "router launch");
  } else {
    st = route_impl(s, T, x, w_router, router_bias, nullptr, nullptr, ids, tw, nullptr, split,
                    partial, x16, stream);
    if (st != MOE_OK) return st;
    QMOE_HIP(launch_permute(ids, (int)(T * s.k), s.E, counts, offsets, sorted, inv, hist, stream),
             "permute launch");
  }
  st = ffn_mixed_impl(s, T, x, tiers, n_tiers, expert_bits, expert_slot, counts, offsets, sorted,
                      yperm, x16, h, !router_uses_gemv((int)T), stream);
  if (st != MOE_OK) return st;
  QMOE_HIP(launch_combine(yperm, inv, tw, nullptr, nullptr, residual, out, (int)T, s.H, s.k, stream),
           "combine launch");
  return MOE_OK;
}

moe_status_t moe_stream_stage_bytes(const moe_shape_t* shape, int32_t experts, size_t* bytes) {
  Shape s;
  moe_status_t st = check_shape(shape, 0, &s);
  if (st != MOE_OK) return st;
  st = rows_only(s, "moe_stream_stage_bytes");
  if (st != MOE_OK) return st;
  if (bytes == nullptr || experts < 1) return fail(MOE_ERR_INVALID_ARGUMENT, "bad argument");
  // two slots of experts / 2 (at least one) experts each
  const int per = experts > 1 ? (experts + 1) / 2 : 1;
  *bytes = 2 * stage_slot_bytes(stage_layout(s), per);
  return MOE_OK;
}

moe_status_t moe_layer_forward_streamed(const moe_shape_t* shape, int64_t T, const uint16_t* x,
                                        const float* w_router, const float* router_bias,
                                        const moe_experts_t* hot, int32_t hot_count,
                                        const moe_experts_t* cold, const int32_t* hot_slot,
                                        void* stage, size_t stage_bytes,
                                        const uint16_t* residual, uint16_t* out, void* ws,
                                        size_t ws_bytes, hipStream_t stream,
                                        hipStream_t copy_stream) {
  Shape s;
  moe_status_t st = check_shape(shape, T, &s);
  if (st != MOE_OK) return st;
  if (s.asym) return fail(MOE_ERR_UNSUPPORTED, "streamed experts need MOE_Q4_SYM");
  st = rows_only(s, "moe_layer_forward_streamed");
  if (st != MOE_OK) return st;
  if (s.Is != 0) return fail(MOE_ERR_UNSUPPORTED, "streamed layers have no shared expert");
  if (hot_slot == nullptr) return fail(MOE_ERR_INVALID_ARGUMENT, "hot_slot is NULL");
  if (hot_count < 0 || hot_count > s.E) return fail(MOE_ERR_INVALID_ARGUMENT, "bad hot_count");
  // the host-side maps: hot experts keep their slot in `hot` (group 0), the
  // cold ones are numbered in expert order and dealt to chunks of `cap`
  ExpertMaps maps;
  std::vector<int> cold_ids;
  for (int e = 0; e < s.E; ++e) {
    const int h = hot_slot[e];
    if (h >= 0) {
      if (h >= hot_count) return fail(MOE_ERR_INVALID_ARGUMENT, "hot_slot[%d] = %d >= hot_count", e, h);
      maps.group[e] = 0;
      maps.slot[e] = h;
    } else {
      cold_ids.push_back(e);
    }
  }
  const int n_cold = (int)cold_ids.size();
  if (hot_count > 0) {
    if (hot == nullptr) return fail(MOE_ERR_INVALID_ARGUMENT, "hot is NULL");
    QMOE_REQUIRE(hot->w13, "hot->w13");
    QMOE_REQUIRE(hot->w13_scale, "hot->w13_scale");
    QMOE_REQUIRE(hot->w2, "hot->w2");
    QMOE_REQUIRE(hot->w2_scale, "hot->w2_scale");
  }
  const StageLayout SL = stage_layout(s);
  int cap = 0;
  if (n_cold > 0) {
    if (cold == nullptr || cold->w13 == nullptr || cold->w13_scale == nullptr ||
        cold->w2 == nullptr || cold->w2_scale == nullptr)
      return fail(MOE_ERR_INVALID_ARGUMENT, "cold experts missing");
    QMOE_REQUIRE(stage, "stage");
    while (cap < n_cold && 2 * stage_slot_bytes(SL, cap + 1) <= stage_bytes) ++cap;
    if (cap == 0)
      return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "stage holds no two experts (%zu bytes)", stage_bytes);
    for (int c = 0; c < n_cold; ++c) {
      maps.group[cold_ids[c]] = 1 + c / cap;
      maps.slot[cold_ids[c]] = c % cap;
    }
  }
  if (T == 0) return MOE_OK;
  QMOE_REQUIRE(x, "x");
  QMOE_REQUIRE(w_router, "w_router");
  QMOE_REQUIRE(out, "out");
  QMOE_OPTIONAL(router_bias, "router_bias");
  QMOE_OPTIONAL(residual, "residual");
  const Layout L = layer_layout(s, T);
  const size_t maps_off = L.total;
  st = check_ws(ws, ws_bytes, maps_off + al((size_t)2 * 4 * s.E));
  if (st != MOE_OK) return st;
  uint8_t* b = static_cast<uint8_t*>(ws);
  auto* split = reinterpret_cast<uint16_t*>(b + L.split);
  auto* partial = reinterpret_cast<float*>(b + L.partial);
  auto* hist = reinterpret_cast<int32_t*>(b + L.hist);
  auto* ids = reinterpret_cast<int32_t*>(b + L.ids);
  auto* tw = reinterpret_cast<float*>(b + L.tw);
  auto* counts = reinterpret_cast<int32_t*>(b + L.counts);
  auto* offsets = reinterpret_cast<int32_t*>(b + L.offsets);
  auto* sorted = reinterpret_cast<int32_t*>(b + L.sorted);
  auto* inv = reinterpret_cast<int32_t*>(b + L.inv);
  auto* x16 = reinterpret_cast<uint16_t*>(b + L.x16);
  auto* h = reinterpret_cast<uint16_t*>(b + L.h);
  auto* yperm = reinterpret_cast<uint16_t*>(b + L.yperm);
  auto* dgroup = reinterpret_cast<int32_t*>(b + maps_off);
  auto* dslot = dgroup + s.E;
  // Copies on a stream of their own: the first two chunks' copies wait for
  // what `stream` held at entry (a previous call's kernels may still read the
  // staging slots), chunk j's copies for the kernels of chunk j-2 (the last
  // user of the same slot), and chunk j's kernels for chunk j's copies.
  const bool overlap = copy_stream != nullptr && copy_stream != stream && n_cold > 0;
  const int n_chunks = cap > 0 ? (n_cold + cap - 1) / cap : 0;
  std::vector<hipEvent_t> ready, freed;
  hipEvent_t entry = nullptr;
  struct EventGuard {
    std::vector<hipEvent_t>* v[2];
    hipEvent_t* one;
    ~EventGuard() {
      for (auto* vec : v)
        for (hipEvent_t e : *vec) (void)hipEventDestroy(e);
      if (*one != nullptr) (void)hipEventDestroy(*one);
    }
  } guard{{&ready, &freed}, &entry};
  if (overlap) {
    QMOE_HIP(hipEventCreateWithFlags(&entry, hipEventDisableTiming), "event create");
    for (int j = 0; j < n_chunks + 2; ++j) {
      hipEvent_t e;
      QMOE_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming), "event create");
      (j < n_chunks ? ready : freed).push_back(e);
    }
    QMOE_HIP(hipEventRecord(entry, stream), "event record");
  }
  QMOE_HIP(launch_write_maps(maps, s.E, dgroup, dslot, stream), "maps launch");
  if (router_uses_gemv((int)T)) {
    QMOE_HIP(launch_route_permute_small(x, w_router, nullptr, partial, router_bias, (int)T, s.H,
                                        s.E, s.k, ids, tw, nullptr, counts, offsets, sorted, inv,
                                        stream),
             "router launch");
  } else {
    st = route_impl(s, T, x, w_router, router_bias, nullptr, nullptr, ids, tw, nullptr, split,
                    partial, x16, stream);
    if (st != MOE_OK) return st;
    QMOE_HIP(launch_permute(ids, (int)(T * s.k), s.E, counts, offsets, sorted, inv, hist, stream),
             "permute launch");
  }
  // (the router GEMM wrote x16 already; the matrix-vector router does not)
  if (router_uses_gemv((int)T))
    QMOE_HIP(launch_x_to_f16(x, x16, T * s.H, stream), "x_to_f16 launch");
  const int P = (int)(T * s.k);
  GroupedGemm g{};
  g.A = x16;
  g.gather = sorted;
  g.gather_div = s.k;
  g.counts = counts;
  g.offsets = offsets;
  g.E = s.E;
  g.max_rows = P;
  g.a_rows = (int)T;
  g.N = 2 * s.I;
  g.K = s.H;
  g.G = s.G;
  g.C = h;
  g.ldc = s.I;
  g.tier = dgroup;
  g.slot = dslot;
  g.bits = 4;
  GroupedGemm d = g;
  d.A = h;
  d.a_rows = P;
  d.gather = nullptr;
  d.N = s.H;
  d.K = s.I;
  d.C = yperm;
  d.ldc = s.H;
  auto run_group = [&](int id, int nexp, const uint8_t* w13, const uint16_t* s13,
                       const uint8_t* w2, const uint16_t* s2) -> moe_status_t {
    g.tier_id = d.tier_id = id;
    g.w_experts = d.w_experts = nexp;
    g.W = w13;
    g.Wscale = s13;
    d.W = w2;
    d.Wscale = s2;
    QMOE_HIP(launch_gateup(g, stream), "gateup launch");
    QMOE_HIP(launch_down(d, stream), "down launch");
    return MOE_OK;
  };
  if (hot_count > 0) {
    st = run_group(0, hot_count, hot->w13, hot->w13_scale, hot->w2, hot->w2_scale);
    if (st != MOE_OK) return st;
  }
  const size_t slot_bytes = stage_slot_bytes(SL, cap);
  hipStream_t cs = overlap ? copy_stream : stream;
  for (int c0 = 0, j = 0; c0 < n_cold; c0 += cap, ++j) {
    const int n = std::min(cap, n_cold - c0);
    uint8_t* base = static_cast<uint8_t*>(stage) + (size_t)(j & 1) * slot_bytes;
    uint8_t* w13 = base;
    uint8_t* s13 = w13 + al(SL.w13 * cap);
    uint8_t* w2 = s13 + al(SL.s13 * cap);
    uint8_t* s2 = w2 + al(SL.w2 * cap);
    if (overlap) QMOE_HIP(hipStreamWaitEvent(cs, j < 2 ? entry : freed[j & 1], 0), "stream wait");
    // the chunk's experts are consecutive in the cold tensors
    QMOE_HIP(hipMemcpyAsync(w13, cold->w13 + SL.w13 * c0, SL.w13 * n, hipMemcpyHostToDevice, cs),
             "expert copy");
    QMOE_HIP(hipMemcpyAsync(s13, reinterpret_cast<const uint8_t*>(cold->w13_scale) + SL.s13 * c0,
                            SL.s13 * n, hipMemcpyHostToDevice, cs),
             "expert copy");
    QMOE_HIP(hipMemcpyAsync(w2, cold->w2 + SL.w2 * c0, SL.w2 * n, hipMemcpyHostToDevice, cs),
             "expert copy");
    QMOE_HIP(hipMemcpyAsync(s2, reinterpret_cast<const uint8_t*>(cold->w2_scale) + SL.s2 * c0,
                            SL.s2 * n, hipMemcpyHostToDevice, cs),
             "expert copy");
    if (overlap) {
      QMOE_HIP(hipEventRecord(ready[j], cs), "event record");
      QMOE_HIP(hipStreamWaitEvent(stream, ready[j], 0), "stream wait");
    }
    st = run_group(1 + j, cap, w13, reinterpret_cast<const uint16_t*>(s13), w2,
                   reinterpret_cast<const uint16_t*>(s2));
    if (st != MOE_OK) return st;
    if (overlap) QMOE_HIP(hipEventRecord(freed[j & 1], stream), "event record");
  }
  QMOE_HIP(launch_combine(yperm, inv, tw, nullptr, nullptr, residual, out, (int)T, s.H, s.k, stream),
           "combine launch");
  return MOE_OK;
}

moe_status_t moe_pack_w4(const uint8_t* src, uint8_t* dst, int64_t rows, int64_t K,
                         hipStream_t stream) {
  if (src == nullptr || dst == nullptr || rows <= 0 || K <= 0)
    return fail(MOE_ERR_INVALID_ARGUMENT, "moe_pack_w4: null pointer or non-positive size");
  if (rows % 16 != 0 || K % 128 != 0)
    return fail(MOE_ERR_INVALID_ARGUMENT, "moe_pack_w4: rows must be a multiple of 16, K of 128");
  if (rows * (K / 2) >= (int64_t(1) << 31))
    return fail(MOE_ERR_UNSUPPORTED, "moe_pack_w4: matrix must be below 2^31 bytes");
  if (!aligned16(src) || !aligned16(dst))
    return fail(MOE_ERR_INVALID_ARGUMENT, "moe_pack_w4: pointers must be 16-byte aligned");
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(src), b0 = reinterpret_cast<uintptr_t>(dst);
  const uintptr_t n = (uintptr_t)(rows * (K / 2));
  if (a0 < b0 + n && b0 < a0 + n)
    return fail(MOE_ERR_INVALID_ARGUMENT, "moe_pack_w4: src and dst overlap");
  QMOE_HIP(launch_pack_w4(src, dst, rows, K, stream), "pack_w4 launch");
  return MOE_OK;
}

moe_status_t moe_pack_tier(const uint8_t* src, uint8_t* dst, int64_t rows, int64_t K, int32_t bits,
                           int32_t gate_up, hipStream_t stream) {
  if (src == nullptr || dst == nullptr || rows <= 0 || K <= 0)
    return fail(MOE_ERR_INVALID_ARGUMENT, "moe_pack_tier: null pointer or non-positive size");
  if (bits != 4 && bits != 3 && bits != 2)
    return fail(MOE_ERR_UNSUPPORTED, "moe_pack_tier: bits must be 4, 3 or 2 (got %d)", bits);
  const bool inter = gate_up != 0 && bits != 4;
  if (rows % (inter ? 32 : 16) != 0 || K % 128 != 0)
    return fail(MOE_ERR_INVALID_ARGUMENT,
                "moe_pack_tier: rows must be a multiple of %d, K of 128", inter ? 32 : 16);
  const int64_t bytes = rows * (K / 8) * bits;
  if (bytes >= (int64_t(1) << 31))
    return fail(MOE_ERR_UNSUPPORTED, "moe_pack_tier: matrix must be below 2^31 bytes");
  if ((reinterpret_cast<uintptr_t>(src) & 3) != 0 || (reinterpret_cast<uintptr_t>(dst) & 3) != 0)
    return fail(MOE_ERR_INVALID_ARGUMENT, "moe_pack_tier: pointers must be 4-byte aligned");
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(src), b0 = reinterpret_cast<uintptr_t>(dst);
  if (a0 < b0 + (uintptr_t)bytes && b0 < a0 + (uintptr_t)bytes)
    return fail(MOE_ERR_INVALID_ARGUMENT, "moe_pack_tier: src and dst overlap");
  QMOE_HIP(launch_pack_tier(src, dst, rows, K, bits, inter, stream), "pack_tier launch");
  return MOE_OK;
}

moe_status_t moe_rmsnorm(int64_t T, int64_t H, const uint16_t* x, const float* weight, float eps,
                         uint16_t* out, hipStream_t stream) {
  if (T < 0 || H <= 0) return fail(MOE_ERR_INVALID_ARGUMENT, "T must be >= 0 and H > 0");
  if (H % 8 != 0 || H > 65536) return fail(MOE_ERR_UNSUPPORTED, "H must be a multiple of 8");
  if (!(eps >= 0.f)) return fail(MOE_ERR_INVALID_ARGUMENT, "eps must be >= 0");
  if (T == 0) return MOE_OK;
  QMOE_REQUIRE(x, "x");
  QMOE_REQUIRE(weight, "weight");
  QMOE_REQUIRE(out, "out");
  if (x == out) return fail(MOE_ERR_INVALID_ARGUMENT, "out must not alias x");
  QMOE_HIP(launch_rmsnorm(x, weight, eps, out, (int)T, (int)H, stream), "rmsnorm launch");
  return MOE_OK;
}

moe_status_t moe_profile_enable(int32_t max_launches) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (hipEvent_t ev : g_prof_events) (void)hipEventDestroy(ev);
  g_prof_events.clear();
  g_prof_records.clear();
  g_prof_slots = 0;
  g_prof_next = 0;
  if (max_launches < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "max_launches must be >= 0");
  if (max_launches == 0) return MOE_OK;
  g_prof_events.resize(2 * (size_t)max_launches, nullptr);
  for (auto& ev : g_prof_events) {
    hipError_t e = hipEventCreate(&ev);
    if (e != hipSuccess) {
      for (hipEvent_t x : g_prof_events)
        if (x) (void)hipEventDestroy(x);
      g_prof_events.clear();
      return hip_fail("hipEventCreate", e);
    }
  }
  g_prof_records.reserve(max_launches);
  g_prof_slots = max_launches;
  return MOE_OK;
}

moe_status_t moe_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_records.clear();
  g_prof_next = 0;
  return MOE_OK;
}

moe_status_t moe_profile_read(const char* kernel, int64_t* launches, double* total_ms) {
  if (kernel == nullptr || launches == nullptr || total_ms == nullptr)
    return fail(MOE_ERR_INVALID_ARGUMENT, "NULL argument");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  int64_t n = 0;
  double ms = 0.0;
  for (const ProfRecord& r : g_prof_records) {
    if (std::strcmp(r.name, kernel) != 0) continue;
    hipEvent_t a = g_prof_events[2 * r.slot], b = g_prof_events[2 * r.slot + 1];
    hipError_t e = hipEventSynchronize(b);
    if (e != hipSuccess) return hip_fail("hipEventSynchronize", e);
    float t = 0.f;
    e = hipEventElapsedTime(&t, a, b);
    if (e != hipSuccess) return hip_fail("hipEventElapsedTime", e);
    ms += t;
    ++n;
  }
  *launches = n;
  *total_ms = ms;
  return MOE_OK;
}

}  // extern "C"
