"""Pure-Python brute force of the MoE layer for tiny shapes (pins the oracle).

Written independently of oracle/: plain loops and the math module, no
numpy, no dispatch.  Every routed expert is evaluated for every token and
multiplied by its gate, which is zero for the experts not chosen; this is the
dense form y = sum_i G(x)_i E_i(x) of the sparsely-gated MoE (MoE-survey blog
page, section 2) and eq. 9 of the DeepSeekMoE page, section 3.2.
"""
from __future__ import annotations

import math


def _dot(a, b):
    s = 0.0
    for p, q in zip(a, b):
        s += p * q
    return s


def _ffn(u, w1, w3, w2):
    # w1, w3: I rows of length d; w2: d rows of length I
    h = []
    for r1, r3 in zip(w1, w3):
        a = _dot(r1, u)
        h.append(a * (1.0 / (1.0 + math.exp(-a))) * _dot(r3, u))
    return [_dot(row, h) for row in w2]


def _ffn_relu(u, wi, wo):
    # GShard position-wise FFN: wo . ReLU(wi . u)
    h = [max(0.0, _dot(r, u)) for r in wi]
    return [_dot(row, h) for row in wo]


def _gates(z, k, gate):
    n = len(z)
    g = [0.0] * n
    if gate == "softmax_topk":
        m = max(z)
        ex = [math.exp(v - m) for v in z]
        tot = sum(ex)
        s = [v / tot for v in ex]
        chosen = sorted(range(n), key=lambda i: (-s[i], i))[:k]
        for i in chosen:
            g[i] = s[i]
    elif gate == "topk_softmax":
        chosen = sorted(range(n), key=lambda i: (-z[i], i))[:k]
        m = max(z[i] for i in chosen)
        tot = sum(math.exp(z[i] - m) for i in chosen)
        for i in chosen:
            g[i] = math.exp(z[i] - m) / tot
    else:
        raise ValueError(gate)
    return sorted(chosen), g


def brute_forward(x, w_router, bias, w_gate, w_up, w_down, ws_gate, ws_up, ws_down,
                  top_k, gate, residual=False, capacity=0, group_size=0, ffn="silu",
                  bias_mode="logits", w_noise=None, noise=None):
    """All arguments are nested Python lists of floats (bias may be None).

    capacity > 0: each expert takes at most `capacity` tokens per group of
    `group_size` consecutive tokens (0: the whole batch), first come first
    served in token order; a token that finds a chosen expert full loses that
    expert's gate (MoE-survey blog page, section 3, expert capacity).

    w_noise, noise: noisy top-k gating (MoE-survey blog page, section 2): the
    logit of expert i becomes u . w_i + noise[t][i] * log(1 + exp(u . wn_i)).

    bias_mode "selection": the bias takes part in choosing the experts only;
    the gate values come from the logits without it.

    ffn "relu": every expert is wo . ReLU(wi . u) with wi = w_gate, wo = w_down
    (w_up unused; MoE-survey blog page, section 3).

    Returns (chosen ids per token, ascending; dense gates per token; y)."""
    def expert(u, w1, w3, w2):
        return _ffn_relu(u, w1, w2) if ffn == "relu" else _ffn(u, w1, w3, w2)

    chosen_all, g_all, y_all = [], [], []
    n = len(w_router)
    S = group_size if 0 < group_size < len(x) else len(x)
    taken = {}
    for t, u in enumerate(x):
        base = [_dot(w_router[i], u) for i in range(n)]
        if w_noise is not None:
            base = [base[i] + noise[t][i] * math.log1p(math.exp(_dot(w_noise[i], u)))
                    for i in range(n)]
        z = [base[i] + (bias[i] if bias is not None else 0.0) for i in range(n)]
        chosen, g = _gates(z, top_k, gate)
        if bias_mode == "selection" and bias is not None:
            z0 = base
            _, g0 = _gates(z0, n, gate)            # gates of every expert, unbiased
            if gate == "topk_softmax":
                m = max(z0[i] for i in chosen)
                tot = sum(math.exp(z0[i] - m) for i in chosen)
                g0 = [math.exp(z0[i] - m) / tot if i in chosen else 0.0 for i in range(n)]
            g = [g0[i] if i in chosen else 0.0 for i in range(n)]
        if capacity > 0:
            for i in chosen:
                key = (t // S, i)
                if taken.get(key, 0) < capacity:
                    taken[key] = taken.get(key, 0) + 1
                else:
                    g[i] = 0.0
        y = [0.0] * len(u)
        for i in range(n):                       # dense: every routed expert
            f = expert(u, w_gate[i], None if w_up is None else w_up[i], w_down[i])
            for c in range(len(u)):
                y[c] += g[i] * f[c]
        for s in range(len(ws_gate)):            # shared experts, gate 1
            f = expert(u, ws_gate[s], None if ws_up is None else ws_up[s], ws_down[s])
            for c in range(len(u)):
                y[c] += f[c]
        if residual:
            for c in range(len(u)):
                y[c] += u[c]
        chosen_all.append(chosen)
        g_all.append(g)
        y_all.append(y)
    return chosen_all, g_all, y_all
