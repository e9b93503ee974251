/*
 * moe.h -- C ABI of libmoe.so: forward pass of one DeepSeekMoE layer on a
 * gfx950 (MI355X) GPU.
 *
 * The layer (DeepSeekMoE paper page, section 3.2, eq. 9-11):
 *   z_t   = W_g u_t (+ b)                      router logits, fp32
 *   S_t   = top-K' routed experts of token t
 *   g     = s on S_t, s = Softmax over the N_r routed experts       (eq. 10-11)
 *        or Softmax over S_t of z (KeepTopK, noise 0; MoE-survey blog page,
 *           section 2, noisy top-k gating)
 *   y_t   = sum_{i in S_t} g_i FFN_i(u_t) + sum_{s < K_s} FFN^sh_s(u_t) (+ u_t)
 *   FFN(u)= W2 (silu(W1 u) * (W3 u))
 * Only the chosen experts are evaluated (MoE-survey blog page, section 2:
 * E_i is skipped where G(x)_i = 0), which is why the work is split into
 * route -> permute (dispatch) -> expert FFN -> combine.
 *
 * Conventions shared by every entry point
 *   - Tensors are dense and row-major.  Every data pointer is a device
 *     pointer owned by the caller; the library never allocates, frees or
 *     synchronises.  Scratch memory comes from the caller's `ws` buffer,
 *     sized by moe_workspace_size(), except in moe_forward_noalloc, which
 *     takes it from a static device array (its global state, with the
 *     per-device address of that array and the thread-local last HIP
 *     error).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call only enqueues work on it and returns.
 *   - Weights are [out_features, in_features] (in_features contiguous):
 *       w_router [N_r, d] fp32 (row i is the centroid e_i; with
 *         layer->router_layout == MOE_ROUTER_PACKED, the order written by
 *         moe_pack_router instead),
 *       w_gate, w_up [N_r, I, d], w_down [N_r, d, I],
 *       ws_gate, ws_up [K_s, I_s, d], ws_down [K_s, d, I_s].
 *     x, y, expert weights and intermediate buffers use layer->dtype
 *     (MOE_BF16: bfloat16 with fp32 accumulation; MOE_F32: float32).
 *   - Routing outputs: topk_idx [T, K'] int32 ascending within a token,
 *     topk_w [T, K'] fp32 aligned with it.  Rows of expert e occupy
 *     [offsets[e], offsets[e+1]) in ascending token order.  P = T*K'.
 *   - Errors: every argument check runs on the host before anything is
 *     enqueued; on failure nothing is launched.  A failed launch returns
 *     MOE_ERR_HIP and moe_last_hip_error() gives the hipError_t.  Faults
 *     inside kernels surface at the caller's next synchronisation.
 *   - Requirements (else MOE_ERR_UNSUPPORTED): N_r <= 256, 1 <= K' <= 16,
 *     K' <= N_r; for MOE_BF16, d % 8 == 0, I % 16 == 0, I_s % 16 == 0;
 *     for MOE_F32, d % 4 == 0, I % 4 == 0, I_s % 4 == 0; T < 2^31 / 16;
 *     every activation and weight matrix (x, x_perm, y_perm, the T*K' x I
 *     and T x K_s*I_s intermediates, one expert's weights) below 4 GB;
 *     all pointers 16-byte aligned.  T == 0 returns MOE_OK with no work.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 4

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,          /* null required pointer, T < 0, bad enum, K' out of range,
                                       negative capacity or group_size, bad ffn, bias_mode or
                                       weight_layout                                             */
  MOE_ERR_UNSUPPORTED = 2,          /* shape/alignment outside the supported set above         */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,  /* ws_bytes below moe_workspace_size()                      */
  MOE_ERR_HIP = 4,                  /* a HIP launch or query failed                              */
  MOE_ERR_SCRATCH_TOO_SMALL = 5     /* moe_forward_noalloc: the layer at T needs more scratch than
                                       MOE_STATIC_SCRATCH_BYTES                                  */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Expert FFN form. */
typedef enum {
  /* W2 (silu(W1 u) * (W3 u)): w_gate = W1, w_up = W3, w_down = W2.       */
  MOE_FFN_SILU_GATED = 0,
  /* wo ReLU(wi u), GShard's position-wise FFN (MoE-survey blog page,
     section 3): w_gate = wi, w_down = wo; w_up and ws_up are not read
     (NULL allowed).                                                      */
  MOE_FFN_RELU = 1
} moe_ffn;

/* Where logit_bias enters. */
typedef enum {
  /* Added to the logits before both the selection and the gate values. */
  MOE_BIAS_LOGITS = 0,
  /* Selection only: the top-K' is taken on z + b, the gate values (and the
     routing statistics) use the unbiased z.  This is the per-expert bias of
     the load balancing without an auxiliary loss in the Tencent Cloud
     article "DeepSeek MoE: innovations and breakthroughs of the mixture-of-
     experts architecture" (section on auxiliary-loss-free balancing), which
     leaves the gate values unstated.                                      */
  MOE_BIAS_SELECTION = 1
} moe_bias_mode;

/* Storage order of the expert weights (w_gate, w_up, w_down, ws_*). */
typedef enum {
  /* [out_features, in_features] row-major, as described above.          */
  MOE_WEIGHTS_ROW_MAJOR = 0,
  /* The packed order written by moe_pack_weights (bf16 only): every matrix
     is cut into 128-row tiles, and a tile stores its 64-wide K steps one
     after another, each as 128 rows x 64 values row-major.  Element (n, k)
     of an [N, K] matrix sits at (n/128)*128*K + (k/64)*128*64 +
     (n%128)*64 + k%64.  A K step of a tile is then 16 KB of contiguous
     memory, which the weight stream of the expert GEMMs reads faster.
     Requires d % 128 == 0, I % 128 == 0 and I_s % 128 == 0.              */
  MOE_WEIGHTS_PACKED = 1
} moe_weight_layout;

/* Storage order of the router weights w_router. */
typedef enum {
  /* [N_r, d] fp32 row-major.                                             */
  MOE_ROUTER_ROW_MAJOR = 0,
  /* The order written by moe_pack_router: the order in which the bf16
     matrix-core router reads W_g, so that every load instruction of it
     reads 1 KB of contiguous memory.  The N_r rows are padded to
     R = MOE_ROUTER_PAD_ROWS(N_r) rows (rows N_r .. R-1 repeat row N_r - 1)
     and element (e, k) of the padded [R, d] matrix sits at float index
       ((k/16 * R/32 + e/32) * 2 + (k%8)/4) * 256 + (e%32 + 32*((k%16)/8)) * 4
       + k%4.
     Requires dtype MOE_BF16, d % 64 == 0 and N_r <= 128; moe_route_noisy
     does not take it (MOE_ERR_UNSUPPORTED).  No arithmetic changes: the
     router's results are bit-identical to the row-major order.            */
  MOE_ROUTER_PACKED = 1
} moe_router_layout;

/* Rows of the packed router matrix for N_r routed experts (N_r <= 128). */
#define MOE_ROUTER_PAD_ROWS(n_routed) ((n_routed) <= 32 ? 32 : (n_routed) <= 64 ? 64 : 128)

typedef enum {
  /* g_i = s_i on the top-K' of s = Softmax over N_r routed experts, not
     renormalised (DeepSeekMoE page, section 3.2, eq. 10-11).            */
  MOE_GATE_SOFTMAX_TOPK = 0,
  /* g = Softmax(KeepTopK(z, K')) with zero noise (MoE-survey blog page,
     section 2, noisy top-k gating).                                      */
  MOE_GATE_TOPK_SOFTMAX = 1
} moe_gate;

/* Shape of one layer.  n_routed = N_r = mN - K_s, top_k = K' = mK - K_s.
 *
 * Expert capacity (MoE-survey blog page, section 3, GShard: expert capacity
 * with a running counter per expert and local group dispatching; section 4,
 * Switch: capacity = tokens / experts x capacity factor).  With capacity
 * C > 0 the tokens are cut into groups of S = group_size consecutive tokens
 * (the last group may be shorter; group_size 0, or >= T, is one group), and
 * in every group each expert keeps its first C assignments in token order.
 * A dropped assignment has gate zero: moe_permute gives it slot_row -1 and no
 * row, the expert FFN never sees it and moe_combine adds nothing for it, so a
 * token with all K' assignments dropped gets only the shared experts and the
 * residual.  topk_w keeps the router's gate values.  capacity 0 = dropless. */
typedef struct {
  int32_t d_model;      /* d                                  */
  int32_t n_routed;     /* N_r                                */
  int32_t n_shared;     /* K_s (0 allowed)                    */
  int32_t top_k;        /* K'                                 */
  int32_t d_ff;         /* I, width of one routed expert      */
  int32_t d_ff_shared;  /* I_s, width of one shared expert    */
  int32_t gate;         /* moe_gate                           */
  int32_t dtype;        /* moe_dtype                          */
  int32_t capacity;     /* C, slots per expert per group; 0 = no limit */
  int32_t group_size;   /* S, tokens per capacity group; 0 = all T     */
  int32_t ffn;          /* moe_ffn                                     */
  int32_t bias_mode;    /* moe_bias_mode                               */
  int32_t weight_layout;/* moe_weight_layout                           */
  int32_t router_layout;/* moe_router_layout                           */
} moe_layer;

int moe_abi_version(void);
const char* moe_status_str(int status);
/* hipError_t of the last failed HIP call made by this thread (0 if none). */
int moe_last_hip_error(void);

/* Bytes of scratch that every entry point below needs for T tokens (host
 * only, no GPU call).  One buffer of this size serves all of them. */
int moe_workspace_size(const moe_layer* layer, int64_t T, size_t* bytes);

/* Router: logits z = x W_g^T (+ logit_bias) in fp32, gate values and the
 * top-K' choice per token (eq. 10-11; KeepTopK variant per layer->gate).
 * Ties between equal logits go to the lower expert id.
 *   x [T, d] (dtype), w_router [N_r, d] fp32, logit_bias [N_r] fp32 or NULL
 *   (added to the logits before both selection and softmax)
 *   -> topk_idx [T, K'] int32 (ascending), topk_w [T, K'] fp32. */
int moe_route(const moe_layer* layer, int64_t T, const void* x, const float* w_router,
              const float* logit_bias, int32_t* topk_idx, float* topk_w, void* stream);

/* moe_route with noisy top-k gating (MoE-survey blog page, section 2):
 *   H_t,i = (x_t W_g^T)_i + noise[t, i] * Softplus((x_t W_noise^T)_i)
 * takes the place of the logits for both the selection and the gate values
 * (logit_bias is added to H as layer->bias_mode says).  The method's random
 * numbers are an input: noise [T, N_r] fp32 holds the caller's standard
 * normal draws; w_noise [N_r, d] fp32.  Softplus(v) = log(1 + e^v).
 * w_router must be row-major (layer->router_layout MOE_ROUTER_ROW_MAJOR,
 * else MOE_ERR_UNSUPPORTED).  The
 * rest of the layer is the staged path: moe_permute, moe_expert_ffn,
 * moe_shared_ffn, moe_combine. */
int moe_route_noisy(const moe_layer* layer, int64_t T, const void* x, const float* w_router,
                    const float* logit_bias, const float* w_noise, const float* noise,
                    int32_t* topk_idx, float* topk_w, void* stream);

/* Weight packing (once, before inference; no compute of the layer): dst =
 * the MOE_WEIGHTS_PACKED form of `count` row-major bf16 matrices [rows,
 * cols] at src (e.g. w_gate: count N_r, rows I, cols d; w_down: count N_r,
 * rows d, cols I; ws_gate: count K_s, rows I_s, cols d).  dst has the same
 * size and must not overlap src.  layer->dtype must be MOE_BF16; rows % 128
 * == 0 and cols % 64 == 0, else MOE_ERR_UNSUPPORTED.  The other layer
 * fields are checked as everywhere but not used. */
int moe_pack_weights(const moe_layer* layer, int64_t count, int32_t rows, int32_t cols,
                     const void* src, void* dst, void* stream);

/* Router weight packing (once, before inference; no compute of the layer):
 * dst [MOE_ROUTER_PAD_ROWS(N_r) * d] fp32 = w_router [N_r, d] fp32 in the
 * MOE_ROUTER_PACKED order.  dst must not overlap w_router.  The layer must
 * meet that layout's requirements (dtype MOE_BF16, d % 64 == 0, N_r <= 128;
 * else MOE_ERR_UNSUPPORTED) whatever its router_layout field says. */
int moe_pack_router(const moe_layer* layer, const float* w_router, float* dst, void* stream);

/* Floats written to `stats` by moe_route_stats for N_r experts, D groups. */
#define MOE_STATS_LEN(n_routed, n_devices) (2 * (n_routed) + 2 * (n_devices) + 3)

/* moe_route plus the routing statistics of the batch, for training: the
 * balance terms of the DeepSeekMoE page, section 3.3 (eq. 12-14 expert
 * level, eq. 15-17 device level) and the router z-loss of the MoE-survey
 * blog page, section 5.  topk_idx and topk_w are bit-identical to
 * moe_route's.  stats [MOE_STATS_LEN(N_r, D)] fp32, device pointer:
 *   [0, N_r)             P_i = (1/T) sum_t s_{i,t}, s_t = Softmax over the N_r
 *                        routed experts of the logits incl. logit_bias (for
 *                        both gate kinds)
 *   [N_r, 2 N_r)         f_i = N_r / (K' T) * #{t : i among t's top-K'}
 *   [2 N_r, +D)          f'_g = mean of f_i over group g, the experts
 *                        [g N_r/D, (g+1) N_r/D)
 *   [2 N_r + D, +D)      P'_g = sum of P_i over group g
 *   [2 N_r + 2D]         L_ExpBal = sum_i f_i P_i        (alpha_1 = 1)
 *   [2 N_r + 2D + 1]     L_DevBal = sum_g f'_g P'_g      (alpha_2 = 1)
 *   [2 N_r + 2D + 2]     z-loss = (1/T) sum_t lse_t^2
 * lse [T] fp32 or NULL: lse_t = log sum_i exp z_{t,i} over the routed
 * experts.  With K' = 1, L_ExpBal is the Switch balance loss (MoE-survey
 * blog page, section 4) at alpha = 1.  n_devices = D must divide N_r
 * (else MOE_ERR_INVALID_ARG).  Sums run in fp64 in a fixed order, so
 * repeated calls return identical bits.  T == 0 writes zeros. */
int moe_route_stats(const moe_layer* layer, int64_t T, const void* x, const float* w_router,
                    const float* logit_bias, int32_t n_devices, int32_t* topk_idx,
                    float* topk_w, float* stats, float* lse, void* ws, size_t ws_bytes,
                    void* stream);

/* Dispatch: stable counting sort of the T*K' (token, expert) assignments by
 * expert (the per-expert token lists that let only chosen experts run).
 * Passage: MoE-survey blog page, section 2 (sparsely-gated MoE): y is
 * sum_i G(x)_i E_i(x) and E_i is not evaluated where G(x)_i is zero, so each
 * expert needs the list of tokens whose gate for it is non-zero; the
 * DeepSeekMoE page, section 3.2, eq. 10, fixes K' such experts per token.
 *   topk_idx [T, K'] with 0 <= id < N_r and distinct ids per token, x [T, d]
 *   (dtype).  Other ids are undefined behaviour in libmoe.so; the checked
 *   build libmoe_debug.so (MOE_DEBUG) verifies them on the device first and
 *   returns MOE_ERR_INVALID_ARG with no output written, waiting for the
 *   stream to read the result (the one call that synchronises there).
 *   -> counts [N_r], offsets [N_r + 1] (exclusive scan, offsets[N_r] = P),
 *      row_token [P] (token of each row), slot_row [P] (row of slot t*K'+j),
 *      x_perm [P, d] (x_perm[r] = x[row_token[r]]; NULL skips the copy).
 * With layer->capacity > 0 only the kept assignments get rows: counts and
 * offsets count kept rows (offsets[N_r] <= P), rows past offsets[N_r] of
 * row_token and x_perm are left unwritten, and slot_row is -1 for a dropped
 * slot. */
int moe_permute(const moe_layer* layer, int64_t T, const int32_t* topk_idx, const void* x,
                int32_t* counts, int32_t* offsets, int32_t* row_token, int32_t* slot_row,
                void* x_perm, void* ws, size_t ws_bytes, void* stream);

/* Routed experts: for every expert e and row r in [offsets[e], offsets[e+1]):
 *   y_perm[r] = W2_e (silu(W1_e x_perm[r]) * (W3_e x_perm[r]))
 * (FFN_i of eq. 9, unweighted; the gate is applied by moe_combine).
 * Intermediate activations are rounded to dtype.  Reads offsets on the
 * device (no host synchronisation).  y_perm [P, d]. */
int moe_expert_ffn(const moe_layer* layer, int64_t T, const int32_t* offsets, const void* x_perm,
                   const void* w_gate, const void* w_up, const void* w_down, void* y_perm,
                   void* ws, size_t ws_bytes, void* stream);

/* Shared experts (eq. 9, first sum, gate 1), evaluated as one FFN of width
 * K_s*I_s: y_shared[t] = sum_s FFN^sh_s(x[t]).  y_shared [T, d].
 * With K_s == 0 it writes zeros. */
int moe_shared_ffn(const moe_layer* layer, int64_t T, const void* x, const void* ws_gate,
                   const void* ws_up, const void* ws_down, void* y_shared, void* ws,
                   size_t ws_bytes, void* stream);

/* Gate-weighted combine (eq. 9):
 *   y[t] = sum_j topk_w[t,j] * y_perm[slot_row[t*K'+j]] + y_shared[t] + residual[t]
 * in fp32, j ascending, one rounding to dtype.  A slot with slot_row -1 (an
 * assignment dropped by the expert capacity) adds nothing.  y_shared and
 * residual may be NULL (then omitted).  y [T, d]. */
int moe_combine(const moe_layer* layer, int64_t T, const void* y_perm, const int32_t* slot_row,
                const float* topk_w, const void* y_shared, const void* residual, void* y,
                void* stream);

/* The whole layer: route, dispatch, routed and shared experts, combine.
 * Passage: DeepSeekMoE page, section 3.2, eq. 9-11 (h_t = sum of the K_s
 * shared FFNs + sum of g_{i,t} FFN_i(u_t) over the routed experts, with
 * the gates of eq. 10-11); MoE-survey blog page, section 2 (y = sum_i
 * G(x)_i E_i(x), only experts with non-zero gate evaluated).
 * The gather of x rows is fused into the routed gate/up GEMM, so no x_perm
 * is materialised.  When I_s == I the K_s shared experts run inside the
 * routed gate/up and down launches as K_s extra groups of all T tokens,
 * and the combine adds their K_s output rows per token (each rounded to
 * dtype) instead of one y_shared row; otherwise they run as in
 * moe_shared_ffn.  residual (NULL or [T, d], usually x itself) is added
 * last.  topk_idx, topk_w, counts and offsets are written for inspection
 * and may be NULL (then they live in ws).  The expert capacity of the
 * layer applies as in moe_permute.  y [T, d]. */
int moe_forward(const moe_layer* layer, int64_t T, const void* x, const float* w_router,
                const float* logit_bias, const void* w_gate, const void* w_up,
                const void* w_down, const void* ws_gate, const void* ws_up,
                const void* ws_down, const void* residual, void* y, int32_t* topk_idx,
                float* topk_w, int32_t* counts, int32_t* offsets, void* ws, size_t ws_bytes,
                void* stream);

/* Stages of moe_forward, in launch order. */
#define MOE_NUM_STAGES 7
enum {
  MOE_STAGE_ROUTE = 0,          /* router logits, softmax, top-K'             */
  MOE_STAGE_DISPATCH = 1,       /* histogram, scan, scatter of row indices    */
  MOE_STAGE_ROUTED_GATE_UP = 2, /* grouped GEMM x W1/W3 + silu(gate) * up
                                   (shared experts too when I_s == I)        */
  MOE_STAGE_ROUTED_DOWN = 3,    /* grouped GEMM H W2 (likewise)               */
  MOE_STAGE_SHARED_GATE_UP = 4, /* shared experts of width K_s*I_s when
                                   I_s != I (else empty, as for K_s == 0)    */
  MOE_STAGE_SHARED_DOWN = 5,
  MOE_STAGE_COMBINE = 6
};

/* moe_forward with per-stage timing markers, for measurement.  `events`
 * holds 2*MOE_NUM_STAGES hipEvent_t handles (as void*) created by the caller
 * (with timing enabled); hipEventElapsedTime(events[2s], events[2s+1]) is
 * stage s's GPU time.  The four GEMM stages are one kernel launch each
 * (bf16 layers), and their two events are bound to that launch
 * (hipExtLaunchKernel): they take the kernel's own start and end, and add
 * no marker between the kernels.  The other stages, the GEMM stages of fp32
 * layers and GEMM stages with nothing to launch have their events recorded
 * on `stream` right before and right after the stage.  A NULL handle skips
 * that marker (to time only some stages); a NULL array is
 * MOE_ERR_INVALID_ARG.  Everything else is exactly moe_forward. */
int moe_forward_timed(const moe_layer* layer, int64_t T, const void* x, const float* w_router,
                      const float* logit_bias, const void* w_gate, const void* w_up,
                      const void* w_down, const void* ws_gate, const void* ws_up,
                      const void* ws_down, const void* residual, void* y, int32_t* topk_idx,
                      float* topk_w, int32_t* counts, int32_t* offsets, void* ws,
                      size_t ws_bytes, void* stream, void* const* events);

/* Bytes of the static device scratch array of moe_forward_noalloc. */
#define MOE_STATIC_SCRATCH_BYTES (64 * 1024 * 1024)

/* moe_forward for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * launches and results as moe_forward, bit for bit, with the scratch taken
 * from a static device array of MOE_STATIC_SCRATCH_BYTES instead of a `ws`
 * argument.  The caller still passes inputs and outputs.  Each GPU the
 * library runs this on holds its own array from the first call on that GPU
 * (which also looks up the array's address, with the current device) until
 * the process ends; the array of the current device is used, so `stream`
 * must belong to it.  The call allocates nothing: no hipMalloc, no hipFree.
 *   - A layer whose moe_workspace_size(layer, T) exceeds
 *     MOE_STATIC_SCRATCH_BYTES is refused with MOE_ERR_SCRATCH_TOO_SMALL
 *     before anything touches the GPU (the 16B-shaped layer fits up to about
 *     1100 tokens, the decode batch of 128 with room to spare).
 *   - Every call on a GPU shares that GPU's array and leaves its contents
 *     behind; nothing in it needs to start at zero (each value the forward
 *     reads from it is written earlier in the same call).  Calls that
 *     overlap on one GPU (on different streams, or from several threads
 *     without ordering) race on the array and give undefined results.
 * Other arguments, checks and errors as moe_forward. */
int moe_forward_noalloc(const moe_layer* layer, int64_t T, const void* x, const float* w_router,
                        const float* logit_bias, const void* w_gate, const void* w_up,
                        const void* w_down, const void* ws_gate, const void* ws_up,
                        const void* ws_down, const void* residual, void* y, int32_t* topk_idx,
                        float* topk_w, int32_t* counts, int32_t* offsets, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
