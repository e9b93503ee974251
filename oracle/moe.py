"""Plain fp64 evaluation of one DeepSeekMoE layer (test infrastructure only).

Sources (titles and sections of the pages the method is taken from):
  [P1] "DeepSeekMoE" translated paper page: section 2 eq. 3-5 (top-K MoE
       layer), section 3.1 eq. 6-8 (fine-grained experts), section 3.2
       eq. 9-11 (shared experts, routed top-(mK-K_s) gates).
  [P4] MoE-survey blog page ("six MoE papers"): section 2 (sparsely-gated
       MoE: y = sum_i G(x)_i E_i(x), experts with zero gate are skipped;
       noisy top-k gating G = Softmax(KeepTopK(H, k))), section 4 (Switch
       routing: p = softmax over all N experts, y = sum over the top-k of
       p_i E_i(x)), section 5 (router probabilities kept in float32).

Everything is float64.  Inputs are the exact values the GPU consumes (bf16
bit patterns or float32 decoded losslessly), so the only difference between
this and the GPU is rounding inside the computation.

Readings taken where the pages leave a step open:
  * softmax runs over the N_r routed experts only; shared experts have no
    centroid (eq. 10-11 index the gates from K_s+1).
  * "softmax_topk" gates are s_i on the chosen experts, not renormalised
    (eq. 10); "topk_softmax" is Softmax(KeepTopK(z, K')) with no noise.
  * expert FFN is the SiLU-gated form W2 (silu(W1 u) * (W3 u)); with
    cfg.ffn == "relu" it is GShard's wo ReLU(wi u) ([P4] section 3), with
    wi in the w_gate slot and wo in the w_down slot.
  * top-k ties break toward the lower expert id; chosen ids are reported
    in ascending order.
  * shared experts enter with weight 1 (eq. 9, first sum); the residual
    u_t of eq. 9 is added only when asked for.
  * noisy top-k gating ([P4] section 2) when the inputs carry w_noise and
    noise: the standard normal draws are an input [T, N_r] (the method's
    random numbers come from outside), the noise term is part of the logits
    for both the selection and the gates, and the bias is added after it.
  * with cfg.bias_mode == "selection" the bias steers only the top-K'
    choice and the gates come from the unbiased logits (the article that
    describes the bias does not say whether it enters the gate value);
    "logits" (default) adds it before both.
  * with cfg.capacity > 0 the dispatch keeps at most that many assignments
    per expert and token group ([P4] section 3, expert capacity; readings in
    oracle/capacity.py) and a dropped assignment contributes nothing.
"""
from __future__ import annotations

import numpy as np

from .capacity import dispatch_capacity

GATES = ("softmax_topk", "topk_softmax")


def decode(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array -> float64.  bf16 arrive as uint16 bit patterns."""
    if a is None:
        return None
    if dtype == "bf16" and a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def router_logits(x: np.ndarray, w_router: np.ndarray, bias=None) -> np.ndarray:
    """Token-to-centroid affinities u_t^T e_i for every routed expert ([P1] eq. 5/11),
    plus an optional per-expert bias.  x [T, d], w_router [N_r, d] (row i = e_i)."""
    z = x @ w_router.T
    if bias is not None:
        z = z + bias[None, :]
    return z


def softplus(v: np.ndarray) -> np.ndarray:
    """log(1 + e^v), evaluated without overflow."""
    return np.logaddexp(0.0, v)


def noisy_logits(x: np.ndarray, w_router: np.ndarray, w_noise: np.ndarray, eps: np.ndarray) -> np.ndarray:
    """Noisy top-k gating's H(x)_i = (x W_g)_i + StandardNormal() * Softplus((x W_noise)_i)
    ([P4] section 2), with the standard normal draws given as eps [T, N_r]."""
    return x @ w_router.T + eps * softplus(x @ w_noise.T)


def selection_and_gate_logits(cfg, inputs: dict, x: np.ndarray):
    """(logits the top-K' is taken on, logits the gate values come from) for
    the rows x: the affinities (plus the noise term of noisy gating when the
    inputs carry w_noise and noise), with the bias added to both, or to the
    selection logits only when cfg.bias_mode == "selection"."""
    wr = np.asarray(inputs["w_router"], dtype=np.float64)
    b = None if inputs.get("bias") is None else np.asarray(inputs["bias"], dtype=np.float64)
    if inputs.get("w_noise") is not None:
        eps = np.asarray(inputs["noise"], dtype=np.float64)
        if eps.shape[0] != x.shape[0]:
            raise ValueError("noise rows must match x rows")
        z = noisy_logits(x, wr, np.asarray(inputs["w_noise"], dtype=np.float64), eps)
        zb = z if b is None else z + b[None, :]
    else:
        z = router_logits(x, wr)
        zb = z if b is None else router_logits(x, wr, b)
    if b is not None and getattr(cfg, "bias_mode", "logits") == "selection":
        return zb, z
    return zb, zb


def softmax(z: np.ndarray) -> np.ndarray:
    """Row-wise softmax over the last axis."""
    m = np.max(z, axis=-1, keepdims=True)
    e = np.exp(z - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def select_topk(score: np.ndarray, k: int) -> np.ndarray:
    """Ids of the k largest scores per row, ties to the lower id, ascending ids.

    Topk(., K) of [P1] eq. 4/7/10 and KeepTopK of [P4] section 2."""
    order = np.argsort(-score, axis=1, kind="stable")[:, :k]
    return np.sort(order, axis=1)


def gate_values(z: np.ndarray, idx: np.ndarray, gate: str) -> np.ndarray:
    """Gate values g_{i,t} on the chosen experts idx [T, K'] from logits z [T, N_r]."""
    if gate == "softmax_topk":
        # g = s on the kept experts, s = Softmax over all routed experts ([P1] eq. 10-11).
        s = softmax(z)
        return np.take_along_axis(s, idx, axis=1)
    if gate == "topk_softmax":
        # KeepTopK sets the others to -inf, so the softmax runs over the kept set ([P4] sec. 2).
        zk = np.take_along_axis(z, idx, axis=1)
        return softmax(zk)
    raise ValueError(f"unknown gate {gate!r}")


def route(z: np.ndarray, k: int, gate: str):
    """Selection + gate values.  Selection is on s for softmax_topk ([P1] eq. 10)
    and on the logits for topk_softmax ([P4] KeepTopK); both orders agree."""
    if gate == "softmax_topk":
        idx = select_topk(softmax(z), k)
    elif gate == "topk_softmax":
        idx = select_topk(z, k)
    else:
        raise ValueError(f"unknown gate {gate!r}")
    return idx.astype(np.int32), gate_values(z, idx, gate)


def route_selection_bias(z: np.ndarray, bias: np.ndarray, k: int, gate: str):
    """Selection-only bias: the top-K' is taken on z + b (a per-expert bias that
    steers the load, the balancing without an auxiliary loss of the Tencent
    Cloud "DeepSeek MoE" article), the gate values on the unbiased z.  z are
    the logits without the bias."""
    return route_on(z + bias[None, :], z, k, gate)


def route_on(zs: np.ndarray, z: np.ndarray, k: int, gate: str):
    """Top-K' chosen on the logits zs, gate values from the logits z."""
    idx, _ = route(zs, k, gate)
    return idx, gate_values(z, idx, gate)


def dispatch(idx: np.ndarray, n_routed: int):
    """Per-expert token lists for evaluating only the chosen experts ([P4] sec. 2).

    Returns counts [N_r], offsets [N_r+1] (exclusive scan), row_token [P]
    (the token of each row; rows grouped by expert, tokens ascending within an
    expert) and slot_row [P] (row of slot t*K'+j)."""
    T, k = idx.shape
    flat = idx.reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=n_routed).astype(np.int32)
    offsets = np.zeros(n_routed + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    order = np.argsort(flat, kind="stable")          # slot ids sorted by expert, then slot
    row_token = (order // k).astype(np.int32)
    slot_row = np.empty(T * k, dtype=np.int32)
    slot_row[order] = np.arange(T * k, dtype=np.int32)
    return counts, offsets, row_token, slot_row


def silu(a: np.ndarray) -> np.ndarray:
    return a / (1.0 + np.exp(-a))


def expert_ffn(X: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """SiLU-gated FFN_i(u) = W2 (silu(W1 u) * (W3 u)) on the rows of X.
    w_gate, w_up [I, d]; w_down [d, I]."""
    return (silu(X @ w_gate.T) * (X @ w_up.T)) @ w_down.T


def relu_ffn(X: np.ndarray, wi: np.ndarray, wo: np.ndarray) -> np.ndarray:
    """GShard's position-wise FFN_e(x) = wo ReLU(wi x) ([P4] section 3) on the
    rows of X.  wi [I, d]; wo [d, I]."""
    return np.maximum(X @ wi.T, 0.0) @ wo.T


def ffn_of(kind: str, X, w_gate, w_up, w_down):
    """One expert of either form: SiLU-gated (three matrices) or ReLU (wi =
    w_gate, wo = w_down)."""
    if kind == "relu":
        return relu_ffn(X, w_gate, w_down)
    if kind == "silu":
        return expert_ffn(X, w_gate, w_up, w_down)
    raise ValueError(f"unknown ffn {kind!r}")


def shared_ffn(X: np.ndarray, ws_gate, ws_up, ws_down, ffn: str = "silu") -> np.ndarray:
    """Sum over the K_s shared experts, each with weight 1 ([P1] eq. 9, first sum)."""
    y = np.zeros((X.shape[0], X.shape[1]), dtype=np.float64)
    for s in range(ws_gate.shape[0]):
        y += ffn_of(ffn, X, ws_gate[s], None if ws_up is None else ws_up[s], ws_down[s])
    return y


def forward(cfg, inputs: dict, tokens=None, residual: bool = False) -> dict:
    """The layer forward ([P1] eq. 9-11) on storage-form inputs from synth.

    tokens: optional array of token ids; y is then computed for those tokens
    only (routing and dispatch are always for the whole batch).
    """
    dt = cfg.dtype
    x = decode(inputs["x"], dt)
    T, d = x.shape
    Nr, k = cfg.n_routed, cfg.top_k
    kind = getattr(cfg, "ffn", "silu")

    zs, z = selection_and_gate_logits(cfg, inputs, x)
    idx, g = route(z, k, cfg.gate) if zs is z else route_on(zs, z, k, cfg.gate)
    cap = getattr(cfg, "capacity", 0)
    if cap > 0:
        # Expert capacity ([P4] section 3): dropped assignments get gate 0.
        counts, offsets, row_token, slot_row, kept = dispatch_capacity(idx, Nr, cap, cfg.group_size)
    else:
        counts, offsets, row_token, slot_row = dispatch(idx, Nr)
        kept = np.ones(idx.shape, dtype=bool)

    sel = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    pos = np.full(T, -1, dtype=np.int64)
    pos[sel] = np.arange(sel.size)
    y = np.zeros((sel.size, d), dtype=np.float64)

    # Routed experts, ascending expert id, each on the tokens that chose it.
    for e in range(Nr):
        rows = np.arange(offsets[e], offsets[e + 1])
        toks = row_token[rows]
        want = pos[toks] >= 0
        if not np.any(want):
            continue
        toks = toks[want]
        slots = np.nonzero(idx[toks] == e)[1]   # rows hold kept assignments only
        ge = g[toks, slots]
        w_up = inputs.get("w_up")
        F = ffn_of(kind, x[toks], decode(inputs["w_gate"][e], dt),
                   None if w_up is None else decode(w_up[e], dt), decode(inputs["w_down"][e], dt))
        y[pos[toks]] += ge[:, None] * F

    if cfg.n_shared > 0:
        y += shared_ffn(x[sel], decode(inputs["ws_gate"], dt), decode(inputs.get("ws_up"), dt),
                        decode(inputs["ws_down"], dt), kind)
    if residual:
        y += x[sel]

    return {
        "logits": z, "topk_idx": idx, "topk_w": g, "counts": counts, "offsets": offsets,
        "row_token": row_token, "slot_row": slot_row, "tokens": sel, "y": y, "kept": kept,
    }
