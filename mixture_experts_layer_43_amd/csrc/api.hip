// C ABI of libmoe (declared in include/moe.h): argument checks, workspace
// carving and the launch sequence of each entry point.  Every check runs on
// the host before anything is enqueued.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "../../include/moe.h"
#include "kernels.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Layout {
  size_t cap_counts, cap_offsets, cap_row_token, cap_slot_row, cap_start, cap_base;
  size_t router_part, stats_part, block_counts, block_base, local_rank, topk_idx, topk_w, counts, offsets, row_token,
      slot_row, h, y_perm, h_shared, y_shared, total;
};

size_t elt_bytes(const moe_layer* L) { return L->dtype == MOE_BF16 ? 2 : 4; }

// moe_forward folds the shared experts into the routed grouped launches
// (K_s extra groups of T rows each) when they have the routed width.
bool fold_shared(const moe_layer* L) { return L->n_shared > 0 && L->d_ff_shared == L->d_ff; }

// Rows of the H / y_perm matrices in moe_forward: the P routed rows, then
// K_s blocks of T rows when the shared experts are folded in.
int64_t forward_rows(const moe_layer* L, int64_t T) {
  return T * L->top_k + (fold_shared(L) ? T * L->n_shared : 0);
}

// Expert capacity: tokens per group (S) and number of groups (G).
int64_t cap_group_len(const moe_layer* L, int64_t T) {
  return (L->group_size > 0 && L->group_size < T) ? L->group_size : std::max<int64_t>(T, 1);
}
int64_t cap_groups(const moe_layer* L, int64_t T) {
  const int64_t S = cap_group_len(L, T);
  return std::max<int64_t>(1, (T + S - 1) / S);
}

Layout layout_of(const moe_layer* L, int64_t T) {
  Layout o{};
  const size_t P = static_cast<size_t>(T) * L->top_k;
  const size_t R = static_cast<size_t>(forward_rows(L, T));
  const size_t NB = static_cast<size_t>((T + moe::kCountBlock - 1) / moe::kCountBlock);
  const size_t Nr = L->n_routed, e = elt_bytes(L), d = L->d_model;
  size_t cur = 0;
  auto take = [&](size_t bytes) {
    const size_t at = cur;
    cur += align_up(bytes);
    return at;
  };
  o.router_part = take(moe::router_partial_bytes(T));
  o.block_counts = take(NB * Nr * 4);
  o.block_base = take(NB * Nr * 4);
  o.local_rank = take(P * 4);
  o.topk_idx = take(P * 4);
  o.topk_w = take(P * 4);
  o.counts = take(Nr * 4);
  o.offsets = take((Nr + 1) * 4);
  o.row_token = take(P * 4);
  o.slot_row = take(P * 4);
  // H holds either the forward rows or, for moe_shared_ffn and the unfolded
  // forward (after the routed GEMMs are done with it), the T x K_s*I_s
  // shared intermediate.
  const size_t wsh = static_cast<size_t>(L->n_shared) * (L->n_shared > 0 ? L->d_ff_shared : 0);
  o.h = take(std::max(R * L->d_ff, static_cast<size_t>(T) * wsh) * e);
  o.h_shared = o.h;
  o.y_perm = take(R * d * e);
  o.y_shared = take(L->n_shared > 0 && !fold_shared(L) ? static_cast<size_t>(T) * d * e : 0);
  o.stats_part = take(moe::route_stats_bytes(T));   // moe_route_stats only
  // Expert capacity: the dropless dispatch and the per-group tables.
  const bool cap = L->capacity > 0;
  const size_t G = static_cast<size_t>(cap_groups(L, T));
  o.cap_counts = take(cap ? Nr * 4 : 0);
  o.cap_offsets = take(cap ? (Nr + 1) * 4 : 0);
  o.cap_row_token = take(cap ? P * 4 : 0);
  o.cap_slot_row = take(cap ? P * 4 : 0);
  o.cap_start = take(cap ? (G + 1) * Nr * 4 : 0);
  o.cap_base = take(cap ? G * Nr * 4 : 0);
  o.total = cur;
  return o;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The packed router order is read only by the bf16 matrix-core router.
bool router_packable(const moe_layer* L) {
  return L->dtype == MOE_BF16 && L->d_model % 64 == 0 && L->n_routed <= 128;
}

int check_layer(const moe_layer* L, int64_t T) {
  if (L == nullptr || T < 0) return MOE_ERR_INVALID_ARG;
  if (L->dtype != MOE_F32 && L->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (L->gate != MOE_GATE_SOFTMAX_TOPK && L->gate != MOE_GATE_TOPK_SOFTMAX) return MOE_ERR_INVALID_ARG;
  if (L->d_model <= 0 || L->n_routed <= 0 || L->n_shared < 0 || L->d_ff <= 0)
    return MOE_ERR_INVALID_ARG;
  if (L->n_shared > 0 && L->d_ff_shared <= 0) return MOE_ERR_INVALID_ARG;
  if (L->capacity < 0 || L->group_size < 0) return MOE_ERR_INVALID_ARG;
  if (L->ffn != MOE_FFN_SILU_GATED && L->ffn != MOE_FFN_RELU) return MOE_ERR_INVALID_ARG;
  if (L->bias_mode != MOE_BIAS_LOGITS && L->bias_mode != MOE_BIAS_SELECTION) return MOE_ERR_INVALID_ARG;
  if (L->weight_layout != MOE_WEIGHTS_ROW_MAJOR && L->weight_layout != MOE_WEIGHTS_PACKED)
    return MOE_ERR_INVALID_ARG;
  if (L->router_layout != MOE_ROUTER_ROW_MAJOR && L->router_layout != MOE_ROUTER_PACKED)
    return MOE_ERR_INVALID_ARG;
  if (L->top_k < 1 || L->top_k > L->n_routed || L->top_k > 16) return MOE_ERR_INVALID_ARG;
  if (L->n_routed > 256) return MOE_ERR_UNSUPPORTED;
  if (T >= (int64_t{1} << 31) / 16) return MOE_ERR_UNSUPPORTED;
  // Every activation and weight matrix must stay below 4 GB (32-bit byte
  // offsets inside the GEMM kernels).
  const int64_t e = static_cast<int64_t>(elt_bytes(L));
  const int64_t R = forward_rows(L, T);
  const int64_t wsh = static_cast<int64_t>(L->n_shared) * (L->n_shared > 0 ? L->d_ff_shared : 0);
  const int64_t lim = int64_t{1} << 32;
  if (R >= (int64_t{1} << 31)) return MOE_ERR_UNSUPPORTED;
  if (R * std::max(L->d_model, L->d_ff) * e >= lim || T * wsh * e >= lim ||
      wsh * L->d_model * e >= lim || static_cast<int64_t>(L->d_ff) * L->d_model * e >= lim)
    return MOE_ERR_UNSUPPORTED;
  // bf16: rows move in 16-byte chunks of 8 values (d % 8) and expert widths
  // are multiples of 16 (I, I_s); neither has to fill whole 64-wide K steps
  // of the GEMMs.  f32: 16-byte chunks of 4 values.
  const int qd = (L->dtype == MOE_BF16) ? 8 : 4;
  const int qi = (L->dtype == MOE_BF16) ? 16 : 4;
  if (L->d_model % qd != 0 || L->d_ff % qi != 0) return MOE_ERR_UNSUPPORTED;
  if (L->n_shared > 0 && L->d_ff_shared % qi != 0) return MOE_ERR_UNSUPPORTED;
  if (L->weight_layout == MOE_WEIGHTS_PACKED) {
    // Packed tiles are kPackRows rows of every expert matrix (I rows of W1/W3,
    // d rows of W2) and bf16 only.
    const int r = moe::kPackRows;
    if (L->dtype != MOE_BF16 || L->d_model % r != 0 || L->d_ff % r != 0) return MOE_ERR_UNSUPPORTED;
    if (L->n_shared > 0 && L->d_ff_shared % r != 0) return MOE_ERR_UNSUPPORTED;
  }
  if (L->router_layout == MOE_ROUTER_PACKED && !router_packable(L)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Required pointer: non-null and 16-byte aligned.
int need(const void* p) {
  if (p == nullptr) return MOE_ERR_INVALID_ARG;
  return aligned16(p) ? MOE_OK : MOE_ERR_UNSUPPORTED;
}
// Pointer to a buffer with T rows: required unless T == 0.
int needT(const void* p, int64_t T) { return T == 0 ? (p == nullptr || aligned16(p) ? MOE_OK : MOE_ERR_UNSUPPORTED) : need(p); }
// Optional pointer: null, or 16-byte aligned.
int opt(const void* p) { return (p == nullptr || aligned16(p)) ? MOE_OK : MOE_ERR_UNSUPPORTED; }

#define MOE_TRY(expr)             \
  do {                            \
    const int _st = (expr);       \
    if (_st != MOE_OK) return _st; \
  } while (0)

#define MOE_HIP(expr)                          \
  do {                                         \
    const hipError_t _e = (expr);              \
    if (_e != hipSuccess) {                    \
      g_last_hip_error = static_cast<int>(_e); \
      return MOE_ERR_HIP;                      \
    }                                          \
  } while (0)

char* at(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

// The first projection of an expert: silu(W1 u) * (W3 u), or for the ReLU
// FFN ReLU(wi u) with wi in the W1 slot (one matrix, the plain GEMM with a
// clamped epilogue).
moe::GemmArgs first_projection(const moe_layer* L, moe::GemmArgs g) {
  g.packed = L->weight_layout == MOE_WEIGHTS_PACKED;
  if (L->ffn == MOE_FFN_RELU) {
    g.mode = moe::kDown;
    g.relu = true;
    g.B1 = nullptr;
    g.Bx1 = nullptr;
  }
  return g;
}

moe::GemmArgs routed_gate_up(const moe_layer* L, int64_t T, const int32_t* offsets,
                             const void* A, const int32_t* gather, const void* w_gate,
                             const void* w_up, void* H) {
  moe::GemmArgs g{};
  g.offsets = offsets;
  g.n_groups = L->n_routed;
  g.rows_total = T * L->top_k;
  g.A = A;
  g.lda = L->d_model;
  g.gather = gather;
  g.a_bytes = (gather ? T : T * L->top_k) * static_cast<int64_t>(L->d_model) * elt_bytes(L);
  g.b_bytes = static_cast<int64_t>(L->d_ff) * L->d_model * elt_bytes(L);
  g.B0 = w_gate;
  g.B1 = w_up;
  g.ldb = L->d_model;
  g.b_group_stride = static_cast<int64_t>(L->d_ff) * L->d_model;
  g.k_sub = L->d_model;
  g.b_sub_stride = 0;
  g.N = L->d_ff;
  g.K = L->d_model;
  g.C = H;
  g.ldc = L->d_ff;
  g.mode = moe::kGateUp;
  return first_projection(L, g);
}

moe::GemmArgs routed_down(const moe_layer* L, int64_t T, const int32_t* offsets, const void* H,
                          const void* w_down, void* y_perm) {
  moe::GemmArgs g{};
  g.offsets = offsets;
  g.n_groups = L->n_routed;
  g.rows_total = T * L->top_k;
  g.A = H;
  g.lda = L->d_ff;
  g.gather = nullptr;
  g.a_bytes = T * L->top_k * static_cast<int64_t>(L->d_ff) * elt_bytes(L);
  g.b_bytes = static_cast<int64_t>(L->d_model) * L->d_ff * elt_bytes(L);
  g.B0 = w_down;
  g.B1 = nullptr;
  g.ldb = L->d_ff;
  g.b_group_stride = static_cast<int64_t>(L->d_model) * L->d_ff;
  g.k_sub = L->d_ff;
  g.b_sub_stride = 0;
  g.N = L->d_model;
  g.K = L->d_ff;
  g.C = y_perm;
  g.ldc = L->d_model;
  g.mode = moe::kDown;
  g.packed = L->weight_layout == MOE_WEIGHTS_PACKED;
  return g;
}

// The K_s shared experts as extra groups of T rows after the routed rows
// (rows P + s*T + t), in the routed gate/up and down launches.
void add_shared_groups(const moe_layer* L, int64_t T, moe::GemmArgs& g, const void* b0,
                       const void* b1, bool down) {
  const int64_t e = elt_bytes(L);
  g.n_extra = L->n_shared;
  g.extra_rows = static_cast<int>(T);
  g.extra_base = T * L->top_k;
  g.rows_total = forward_rows(L, T);
  g.Bx0 = b0;
  g.Bx1 = L->ffn == MOE_FFN_RELU ? nullptr : b1;
  g.bx_group_stride = static_cast<int64_t>(L->d_ff_shared) * L->d_model;
  g.bx_bytes = g.bx_group_stride * e;
  if (down) g.a_bytes = g.rows_total * static_cast<int64_t>(L->d_ff) * e;
}

int gemm(const moe_layer* L, const moe::GemmArgs& g, hipStream_t s, moe::StageEvents ev = {}) {
  if (L->dtype == MOE_BF16) {
    MOE_HIP(moe::launch_gemm_bf16(g, s, ev));
    return MOE_OK;
  }
  if (ev.start != nullptr) MOE_HIP(hipEventRecord(ev.start, s));
  MOE_HIP(moe::launch_gemm_f32(g, s));
  if (ev.stop != nullptr) MOE_HIP(hipEventRecord(ev.stop, s));
  return MOE_OK;
}

// Shared experts as one FFN of width K_s*I_s: [K_s, I_s, d] is [K_s*I_s, d].
moe::GemmArgs shared_gate_up(const moe_layer* L, int64_t T, const void* x, const void* ws_gate,
                             const void* ws_up, void* h_shared) {
  const int wsh = L->n_shared * L->d_ff_shared;
  moe::GemmArgs g{};
  g.offsets = nullptr;
  g.n_groups = 1;
  g.rows_total = T;
  g.A = x;
  g.lda = L->d_model;
  g.a_bytes = T * static_cast<int64_t>(L->d_model) * elt_bytes(L);
  g.b_bytes = static_cast<int64_t>(wsh) * L->d_model * elt_bytes(L);
  g.B0 = ws_gate;
  g.B1 = ws_up;
  g.ldb = L->d_model;
  g.k_sub = L->d_model;
  g.N = wsh;
  g.K = L->d_model;
  g.C = h_shared;
  g.ldc = wsh;
  g.mode = moe::kGateUp;
  return first_projection(L, g);
}

// The down projection's K runs over the K_s matrices [d, I_s] in turn.
moe::GemmArgs shared_down(const moe_layer* L, int64_t T, const void* h_shared,
                          const void* ws_down, void* y_shared) {
  const int wsh = L->n_shared * L->d_ff_shared;
  moe::GemmArgs h{};
  h.offsets = nullptr;
  h.n_groups = 1;
  h.rows_total = T;
  h.A = h_shared;
  h.lda = wsh;
  h.a_bytes = T * static_cast<int64_t>(wsh) * elt_bytes(L);
  h.b_bytes = static_cast<int64_t>(wsh) * L->d_model * elt_bytes(L);
  h.B0 = ws_down;
  h.ldb = L->d_ff_shared;
  h.k_sub = L->d_ff_shared;
  h.b_sub_stride = static_cast<int64_t>(L->d_model) * L->d_ff_shared;
  h.N = L->d_model;
  h.K = wsh;
  h.C = y_shared;
  h.ldc = L->d_model;
  h.mode = moe::kDown;
  h.packed = L->weight_layout == MOE_WEIGHTS_PACKED;
  return h;
}

// Optional stage markers for moe_forward_timed.
struct Marks {
  hipEvent_t const* ev;
  hipStream_t s;
  int mark(int i) const {
    if (ev != nullptr && ev[i] != nullptr) MOE_HIP(hipEventRecord(ev[i], s));
    return MOE_OK;
  }
  // Stage `st` as one kernel launch that carries its own start/end events.
  moe::StageEvents launch(int st) const {
    moe::StageEvents e;
    if (ev != nullptr) {
      e.start = ev[2 * st];
      e.stop = ev[2 * st + 1];
    }
    return e;
  }
};

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape, dtype or alignment";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_ERR_HIP: return "HIP error";
    case MOE_ERR_SCRATCH_TOO_SMALL:
      return "the layer needs more scratch than the static buffer of moe_forward_noalloc holds";
    default: return "unknown status";
  }
}

int moe_last_hip_error(void) { return g_last_hip_error; }

int moe_workspace_size(const moe_layer* layer, int64_t T, size_t* bytes) {
  MOE_TRY(check_layer(layer, T));
  if (bytes == nullptr) return MOE_ERR_INVALID_ARG;
  *bytes = layout_of(layer, T).total;
  return MOE_OK;
}

static moe::RouteArgs route_args(const moe_layer* layer, int64_t T, const void* x,
                                 const float* w_router, const float* logit_bias, int32_t* topk_idx,
                                 float* topk_w, float* partial);

static int route_impl(const moe_layer* layer, int64_t T, const void* x, const float* w_router,
                      const float* logit_bias, int32_t* topk_idx, float* topk_w, float* partial,
                      void* stream) {
  MOE_TRY(check_layer(layer, T));
  MOE_TRY(needT(x, T));
  MOE_TRY(need(w_router));
  MOE_TRY(opt(logit_bias));
  MOE_TRY(needT(topk_idx, T));
  MOE_TRY(needT(topk_w, T));
  if (T == 0) return MOE_OK;
  MOE_HIP(moe::launch_route(route_args(layer, T, x, w_router, logit_bias, topk_idx, topk_w, partial),
                            static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

static moe::RouteArgs route_args(const moe_layer* layer, int64_t T, const void* x,
                                 const float* w_router, const float* logit_bias, int32_t* topk_idx,
                                 float* topk_w, float* partial) {
  moe::RouteArgs a{};
  a.partial = partial;
  a.x = x;
  a.w_router = w_router;
  a.bias = logit_bias;
  a.T = static_cast<int>(T);
  a.d = layer->d_model;
  a.n_routed = layer->n_routed;
  a.top_k = layer->top_k;
  a.gate = layer->gate;
  a.bias_sel = layer->bias_mode == MOE_BIAS_SELECTION;
  a.x_bf16 = layer->dtype == MOE_BF16;
  a.w_packed = layer->router_layout == MOE_ROUTER_PACKED;
  a.topk_idx = topk_idx;
  a.topk_w = topk_w;
  return a;
}

int moe_route(const moe_layer* layer, int64_t T, const void* x, const float* w_router,
              const float* logit_bias, int32_t* topk_idx, float* topk_w, void* stream) {
  return route_impl(layer, T, x, w_router, logit_bias, topk_idx, topk_w, nullptr, stream);
}

int moe_pack_weights(const moe_layer* layer, int64_t count, int32_t rows, int32_t cols,
                     const void* src, void* dst, void* stream) {
  MOE_TRY(check_layer(layer, 0));
  if (count < 0 || rows <= 0 || cols <= 0) return MOE_ERR_INVALID_ARG;
  if (layer->dtype != MOE_BF16 || rows % moe::kPackRows != 0 || cols % 64 != 0)
    return MOE_ERR_UNSUPPORTED;
  if (count * rows * static_cast<int64_t>(cols) * 2 >= (int64_t{1} << 40)) return MOE_ERR_UNSUPPORTED;
  if (count == 0) return MOE_OK;   // e.g. the shared weights of a layer with K_s = 0
  if (src == dst) return MOE_ERR_INVALID_ARG;
  MOE_TRY(need(src));
  MOE_TRY(need(dst));
  MOE_HIP(moe::launch_pack(src, dst, count, rows, cols, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

int moe_pack_router(const moe_layer* layer, const float* w_router, float* dst, void* stream) {
  MOE_TRY(check_layer(layer, 0));
  if (!router_packable(layer)) return MOE_ERR_UNSUPPORTED;
  MOE_TRY(need(w_router));
  MOE_TRY(need(dst));
  const int64_t nsrc = static_cast<int64_t>(layer->n_routed) * layer->d_model * 4;
  const int64_t ndst = static_cast<int64_t>(moe::router_pad_rows(layer->n_routed)) * layer->d_model * 4;
  const auto s0 = reinterpret_cast<uintptr_t>(w_router), d0 = reinterpret_cast<uintptr_t>(dst);
  if (s0 < d0 + ndst && d0 < s0 + nsrc) return MOE_ERR_INVALID_ARG;
  MOE_HIP(moe::launch_pack_router(w_router, dst, layer->d_model, layer->n_routed,
                                  static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

int moe_route_noisy(const moe_layer* layer, int64_t T, const void* x, const float* w_router,
                    const float* logit_bias, const float* w_noise, const float* noise,
                    int32_t* topk_idx, float* topk_w, void* stream) {
  MOE_TRY(check_layer(layer, T));
  if (layer->router_layout != MOE_ROUTER_ROW_MAJOR) return MOE_ERR_UNSUPPORTED;
  MOE_TRY(needT(x, T));
  MOE_TRY(need(w_router));
  MOE_TRY(opt(logit_bias));
  MOE_TRY(need(w_noise));
  MOE_TRY(needT(noise, T));
  MOE_TRY(needT(topk_idx, T));
  MOE_TRY(needT(topk_w, T));
  if (T == 0) return MOE_OK;
  moe::RouteArgs a = route_args(layer, T, x, w_router, logit_bias, topk_idx, topk_w, nullptr);
  a.w_noise = w_noise;
  a.noise = noise;
  MOE_HIP(moe::launch_route(a, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

int moe_route_stats(const moe_layer* layer, int64_t T, const void* x, const float* w_router,
                    const float* logit_bias, int32_t n_devices, int32_t* topk_idx, float* topk_w,
                    float* stats, float* lse, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_layer(layer, T));
  MOE_TRY(needT(x, T));
  MOE_TRY(need(w_router));
  MOE_TRY(opt(logit_bias));
  MOE_TRY(needT(topk_idx, T));
  MOE_TRY(needT(topk_w, T));
  MOE_TRY(need(stats));
  MOE_TRY(opt(lse));
  if (n_devices < 1 || layer->n_routed % n_devices != 0) return MOE_ERR_INVALID_ARG;
  const Layout lo = layout_of(layer, T);
  MOE_TRY(need(ws));
  if (ws_bytes < lo.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  moe::RouteArgs a = route_args(layer, T, x, w_router, logit_bias, topk_idx, topk_w, nullptr);
  a.stats_part = reinterpret_cast<double*>(at(ws, lo.stats_part));
  a.lse = lse;
  MOE_HIP(moe::launch_route_stats(a, n_devices, stats, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

static moe::PermuteArgs permute_args(const moe_layer* layer, int64_t T, const int32_t* topk_idx,
                                     const void* x, int32_t* counts, int32_t* offsets,
                                     int32_t* row_token, int32_t* slot_row, void* x_perm, void* ws,
                                     const Layout& lo) {
  moe::PermuteArgs a{};
  a.topk_idx = topk_idx;
  a.x = x;
  a.T = static_cast<int>(T);
  a.d = layer->d_model;
  a.n_routed = layer->n_routed;
  a.top_k = layer->top_k;
  a.elt_bytes = static_cast<int>(elt_bytes(layer));
  a.counts = counts;
  a.offsets = offsets;
  a.row_token = row_token;
  a.slot_row = slot_row;
  a.x_perm = x_perm;
  a.block_counts = reinterpret_cast<int32_t*>(at(ws, lo.block_counts));
  a.block_base = reinterpret_cast<int32_t*>(at(ws, lo.block_base));
  a.local_rank = reinterpret_cast<int32_t*>(at(ws, lo.local_rank));
  a.capacity = layer->capacity;
  a.group_len = static_cast<int>(cap_group_len(layer, T));
  a.n_groups = static_cast<int>(cap_groups(layer, T));
  a.full_counts = reinterpret_cast<int32_t*>(at(ws, lo.cap_counts));
  a.full_offsets = reinterpret_cast<int32_t*>(at(ws, lo.cap_offsets));
  a.full_row_token = reinterpret_cast<int32_t*>(at(ws, lo.cap_row_token));
  a.full_slot_row = reinterpret_cast<int32_t*>(at(ws, lo.cap_slot_row));
  a.group_start = reinterpret_cast<int32_t*>(at(ws, lo.cap_start));
  a.group_base = reinterpret_cast<int32_t*>(at(ws, lo.cap_base));
  return a;
}

static int permute_impl(const moe_layer* layer, int64_t T, const int32_t* topk_idx,
                        const void* x, int32_t* counts, int32_t* offsets, int32_t* row_token,
                        int32_t* slot_row, void* x_perm, void* ws, const Layout& lo,
                        hipStream_t s) {
  MOE_HIP(moe::launch_permute(permute_args(layer, T, topk_idx, x, counts, offsets, row_token,
                                           slot_row, x_perm, ws, lo),
                              s));
  return MOE_OK;
}

int moe_permute(const moe_layer* layer, int64_t T, const int32_t* topk_idx, const void* x,
                int32_t* counts, int32_t* offsets, int32_t* row_token, int32_t* slot_row,
                void* x_perm, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_layer(layer, T));
  MOE_TRY(needT(topk_idx, T));
  MOE_TRY(need(counts));
  MOE_TRY(need(offsets));
  MOE_TRY(needT(row_token, T));
  MOE_TRY(needT(slot_row, T));
  MOE_TRY(opt(x_perm));
  if (x_perm != nullptr) MOE_TRY(needT(x, T));
  MOE_TRY(need(ws));
  const Layout lo = layout_of(layer, T);
  if (ws_bytes < lo.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
#ifdef MOE_DEBUG
  // Checked build: the caller's ids are verified on the device before the
  // dispatch indexes with them (the flag sits in the block-local rank
  // scratch, which the dispatch overwrites later); this waits for the stream.
  if (T > 0) {
    int32_t* bad = reinterpret_cast<int32_t*>(at(ws, lo.local_rank));
    hipStream_t s = static_cast<hipStream_t>(stream);
    MOE_HIP(moe::launch_check_topk(topk_idx, static_cast<int>(T), layer->top_k, layer->n_routed, bad, s));
    int32_t h = 0;
    MOE_HIP(hipMemcpyAsync(&h, bad, sizeof(h), hipMemcpyDeviceToHost, s));
    MOE_HIP(hipStreamSynchronize(s));
    if (h != 0) return MOE_ERR_INVALID_ARG;
  }
#endif
  return permute_impl(layer, T, topk_idx, x, counts, offsets, row_token, slot_row, x_perm, ws,
                      lo, static_cast<hipStream_t>(stream));
}

int moe_expert_ffn(const moe_layer* layer, int64_t T, const int32_t* offsets, const void* x_perm,
                   const void* w_gate, const void* w_up, const void* w_down, void* y_perm,
                   void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_layer(layer, T));
  MOE_TRY(need(offsets));
  MOE_TRY(needT(x_perm, T));
  MOE_TRY(need(w_gate));
  MOE_TRY(layer->ffn == MOE_FFN_SILU_GATED ? need(w_up) : opt(w_up));
  MOE_TRY(need(w_down));
  MOE_TRY(needT(y_perm, T));
  MOE_TRY(need(ws));
  const Layout lo = layout_of(layer, T);
  if (ws_bytes < lo.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (T == 0) return MOE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* H = at(ws, lo.h);
  MOE_TRY(gemm(layer, routed_gate_up(layer, T, offsets, x_perm, nullptr, w_gate, w_up, H), s));
  return gemm(layer, routed_down(layer, T, offsets, H, w_down, y_perm), s);
}

int moe_shared_ffn(const moe_layer* layer, int64_t T, const void* x, const void* ws_gate,
                   const void* ws_up, const void* ws_down, void* y_shared, void* ws,
                   size_t ws_bytes, void* stream) {
  MOE_TRY(check_layer(layer, T));
  MOE_TRY(needT(y_shared, T));
  MOE_TRY(need(ws));
  if (layer->n_shared > 0) {
    MOE_TRY(needT(x, T));
    MOE_TRY(need(ws_gate));
    MOE_TRY(layer->ffn == MOE_FFN_SILU_GATED ? need(ws_up) : opt(ws_up));
    MOE_TRY(need(ws_down));
  }
  const Layout lo = layout_of(layer, T);
  if (ws_bytes < lo.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (T == 0) return MOE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (layer->n_shared == 0) {
    MOE_HIP(moe::launch_zero(y_shared, static_cast<size_t>(T) * layer->d_model * elt_bytes(layer), s));
    return MOE_OK;
  }
  void* hs = at(ws, lo.h_shared);
  MOE_TRY(gemm(layer, shared_gate_up(layer, T, x, ws_gate, ws_up, hs), s));
  return gemm(layer, shared_down(layer, T, hs, ws_down, y_shared), s);
}

int moe_combine(const moe_layer* layer, int64_t T, const void* y_perm, const int32_t* slot_row,
                const float* topk_w, const void* y_shared, const void* residual, void* y,
                void* stream) {
  MOE_TRY(check_layer(layer, T));
  MOE_TRY(needT(y_perm, T));
  MOE_TRY(needT(slot_row, T));
  MOE_TRY(needT(topk_w, T));
  MOE_TRY(opt(y_shared));
  MOE_TRY(opt(residual));
  MOE_TRY(needT(y, T));
  if (T == 0) return MOE_OK;
  moe::CombineArgs a{};
  a.y_perm = y_perm;
  a.slot_row = slot_row;
  a.topk_w = topk_w;
  a.y_shared = y_shared;
  a.shared_blocks = 1;
  a.residual = residual;
  a.y = y;
  a.T = static_cast<int>(T);
  a.d = layer->d_model;
  a.top_k = layer->top_k;
  a.bf16 = layer->dtype == MOE_BF16;
  MOE_HIP(moe::launch_combine(a, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

static int forward_impl(const moe_layer* layer, int64_t T, const void* x,
                        const float* w_router, const float* logit_bias, const void* w_gate,
                        const void* w_up, const void* w_down, const void* ws_gate,
                        const void* ws_up, const void* ws_down, const void* residual, void* y,
                        int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                        void* ws, size_t ws_bytes, void* stream, hipEvent_t const* events) {
  MOE_TRY(check_layer(layer, T));
  MOE_TRY(needT(x, T));
  MOE_TRY(need(w_router));
  MOE_TRY(opt(logit_bias));
  MOE_TRY(need(w_gate));
  MOE_TRY(layer->ffn == MOE_FFN_SILU_GATED ? need(w_up) : opt(w_up));
  MOE_TRY(need(w_down));
  if (layer->n_shared > 0) {
    MOE_TRY(need(ws_gate));
    MOE_TRY(layer->ffn == MOE_FFN_SILU_GATED ? need(ws_up) : opt(ws_up));
    MOE_TRY(need(ws_down));
  }
  MOE_TRY(opt(residual));
  MOE_TRY(needT(y, T));
  MOE_TRY(opt(topk_idx));
  MOE_TRY(opt(topk_w));
  MOE_TRY(opt(counts));
  MOE_TRY(opt(offsets));
  MOE_TRY(need(ws));
  const Layout lo = layout_of(layer, T);
  if (ws_bytes < lo.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Marks m{events, s};
  if (topk_idx == nullptr) topk_idx = reinterpret_cast<int32_t*>(at(ws, lo.topk_idx));
  if (topk_w == nullptr) topk_w = reinterpret_cast<float*>(at(ws, lo.topk_w));
  if (counts == nullptr) counts = reinterpret_cast<int32_t*>(at(ws, lo.counts));
  if (offsets == nullptr) offsets = reinterpret_cast<int32_t*>(at(ws, lo.offsets));
  if (T == 0) {
    for (int i = 0; i < 2 * MOE_NUM_STAGES; ++i) MOE_TRY(m.mark(i));
    return permute_impl(layer, T, nullptr, nullptr, counts, offsets, nullptr, nullptr, nullptr,
                        ws, lo, s);
  }
  int32_t* row_token = reinterpret_cast<int32_t*>(at(ws, lo.row_token));
  int32_t* slot_row = reinterpret_cast<int32_t*>(at(ws, lo.slot_row));
  void* H = at(ws, lo.h);
  void* y_perm = at(ws, lo.y_perm);
  void* h_shared = at(ws, lo.h_shared);
  void* y_shared = layer->n_shared > 0 ? at(ws, lo.y_shared) : nullptr;

  // With the workspace at hand, small batches may split the router's K.
  const moe::RouteArgs ra = route_args(layer, T, x, w_router, logit_bias, topk_idx, topk_w,
                                       reinterpret_cast<float*>(at(ws, lo.router_part)));
  const moe::PermuteArgs pa = permute_args(layer, T, topk_idx, nullptr, counts, offsets, row_token,
                                           slot_row, nullptr, ws, lo);
  MOE_TRY(m.mark(0));
  MOE_HIP(moe::launch_route(ra, s));
  MOE_TRY(m.mark(1));
  MOE_TRY(m.mark(2));
  MOE_HIP(moe::launch_permute(pa, s));
  MOE_TRY(m.mark(3));
  // Routed experts; the gather x[row_token[r]] happens inside the A-tile load.
  moe::GemmArgs gu = routed_gate_up(layer, T, offsets, x, row_token, w_gate, w_up, H);
  moe::GemmArgs dn = routed_down(layer, T, offsets, H, w_down, y_perm);
  const bool fold = fold_shared(layer);
  if (fold) {
    // Shared experts ride in the routed launches: their rows of y_perm are
    // summed by the combine, one block of T rows per shared expert.
    add_shared_groups(layer, T, gu, ws_gate, ws_up, false);
    add_shared_groups(layer, T, dn, ws_down, nullptr, true);
  }
  // Each GEMM stage is one launch; its events time the kernel itself.
  MOE_TRY(gemm(layer, gu, s, m.launch(2)));
  MOE_TRY(gemm(layer, dn, s, m.launch(3)));
  if (layer->n_shared > 0 && !fold) {
    MOE_TRY(gemm(layer, shared_gate_up(layer, T, x, ws_gate, ws_up, h_shared), s, m.launch(4)));
    MOE_TRY(gemm(layer, shared_down(layer, T, h_shared, ws_down, y_shared), s, m.launch(5)));
  } else {
    MOE_HIP(moe::record_stage(m.launch(4), s));
    MOE_HIP(moe::record_stage(m.launch(5), s));
  }
  MOE_TRY(m.mark(12));
  moe::CombineArgs c{};
  c.y_perm = y_perm;
  c.slot_row = slot_row;
  c.topk_w = topk_w;
  if (fold) {
    c.y_shared = static_cast<char*>(y_perm) + T * layer->top_k * layer->d_model * elt_bytes(layer);
    c.shared_blocks = layer->n_shared;
    c.shared_stride = T * layer->d_model;
  } else {
    c.y_shared = y_shared;
    c.shared_blocks = 1;
  }
  c.residual = residual;
  c.y = y;
  c.T = static_cast<int>(T);
  c.d = layer->d_model;
  c.top_k = layer->top_k;
  c.bf16 = layer->dtype == MOE_BF16;
  MOE_HIP(moe::launch_combine(c, s));
  return m.mark(13);
}

int moe_forward(const moe_layer* layer, int64_t T, const void* x, const float* w_router,
                const float* logit_bias, const void* w_gate, const void* w_up,
                const void* w_down, const void* ws_gate, const void* ws_up,
                const void* ws_down, const void* residual, void* y, int32_t* topk_idx,
                float* topk_w, int32_t* counts, int32_t* offsets, void* ws, size_t ws_bytes,
                void* stream) {
  return forward_impl(layer, T, x, w_router, logit_bias, w_gate, w_up, w_down, ws_gate, ws_up,
                      ws_down, residual, y, topk_idx, topk_w, counts, offsets, ws, ws_bytes,
                      stream, nullptr);
}

int moe_forward_timed(const moe_layer* layer, int64_t T, const void* x, const float* w_router,
                      const float* logit_bias, const void* w_gate, const void* w_up,
                      const void* w_down, const void* ws_gate, const void* ws_up,
                      const void* ws_down, const void* residual, void* y, int32_t* topk_idx,
                      float* topk_w, int32_t* counts, int32_t* offsets, void* ws,
                      size_t ws_bytes, void* stream, void* const* events) {
  if (events == nullptr) return MOE_ERR_INVALID_ARG;
  return forward_impl(layer, T, x, w_router, logit_bias, w_gate, w_up, w_down, ws_gate, ws_up,
                      ws_down, residual, y, topk_idx, topk_w, counts, offsets, ws, ws_bytes,
                      stream, reinterpret_cast<hipEvent_t const*>(events));
}


}  // extern "C"

// ---- moe_forward_noalloc: scratch from a static device array ------------
//
// For callers that cannot allocate.  The forward's scratch (the same layout
// moe_workspace_size describes) comes from `scratch`, a file-scope device
// array of MOE_STATIC_SCRATCH_BYTES that each GPU holds from the first call
// on it until the process ends.  In host code `scratch` names a host-side
// stand-in, so the device address of each GPU's copy is looked up once
// (hipGetSymbolAddress, with that device current) and only that address is
// handed to the kernels.
namespace {

static __device__ __align__(256) unsigned char scratch[MOE_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array, looked up on the
// first call on that device.
int scratch_of_current_device(void** out) {
  int dev = -1;
  MOE_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    MOE_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
    if (ptr == nullptr) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_forward_noalloc(const moe_layer* layer, int64_t T, const void* x, const float* w_router,
                        const float* logit_bias, const void* w_gate, const void* w_up,
                        const void* w_down, const void* ws_gate, const void* ws_up,
                        const void* ws_down, const void* residual, void* y, int32_t* topk_idx,
                        float* topk_w, int32_t* counts, int32_t* offsets, void* stream) {
  MOE_TRY(check_layer(layer, T));
  // Refused before the GPU is touched.
  if (layout_of(layer, T).total > static_cast<size_t>(MOE_STATIC_SCRATCH_BYTES))
    return MOE_ERR_SCRATCH_TOO_SMALL;
  void* ws = nullptr;
  MOE_TRY(scratch_of_current_device(&ws));
  return forward_impl(layer, T, x, w_router, logit_bias, w_gate, w_up, w_down, ws_gate, ws_up,
                      ws_down, residual, y, topk_idx, topk_w, counts, offsets, ws,
                      static_cast<size_t>(MOE_STATIC_SCRATCH_BYTES), stream, nullptr);
}

}  // extern "C"
