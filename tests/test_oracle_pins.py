"""Pins of the fp64 oracle to what the pages and the mathematics fix.

Every check here compares the oracle with something other than itself: a
pure-Python brute force that evaluates every expert densely, closed forms
derived by hand (tests/golden), special cases that reduce to textbook
forms, and invariants the pages state.  A last group plants plausible
mistakes into the oracle and checks that these pins catch each one.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import oracle.moe as om
from _brute import brute_forward
from synth import LayerConfig, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny(**kw):
    base = dict(name="pin", tokens=12, d_model=6, n_routed=5, n_shared=1, top_k=2,
                d_ff=4, d_ff_shared=3, gate="softmax_topk", dtype="f32", seed=777, gap=1e-3)
    base.update(kw)
    return LayerConfig(**base)


def inputs_for(cfg, scale_router=1.0):
    inp = make_inputs(cfg)
    inp["w_router"] = (inp["w_router"] * np.float32(scale_router)).astype(np.float32)
    oracle.enforce_gap(cfg, inp)
    return inp


def as_lists(inp):
    f = lambda a: None if a is None else np.asarray(a, dtype=np.float64).tolist()
    return {k: f(v) for k, v in inp.items()}


def run_brute(cfg, inp, residual=False):
    L = as_lists(inp)
    return brute_forward(L["x"], L["w_router"], L["bias"], L["w_gate"], L["w_up"], L["w_down"],
                         L["ws_gate"], L["ws_up"], L["ws_down"], cfg.top_k, cfg.gate, residual)


def rel(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


BRUTE_CASES = [
    dict(),                                               # DeepSeekMoE: shared + fine-grained top-k
    dict(gate="topk_softmax"),
    dict(n_shared=0, top_k=1),                            # Switch top-1
    dict(n_shared=2, top_k=3, n_routed=7, d_ff=2),
    dict(n_shared=0, top_k=5),                            # k = N_r, dense mixture
    dict(gate="topk_softmax", zipf_s=1.2, n_shared=0),    # GShard-style with skew bias
    dict(tokens=1),
]


@pytest.mark.parametrize("kw", BRUTE_CASES, ids=[str(c) for c in BRUTE_CASES])
def test_oracle_matches_dense_brute_force(kw):
    cfg = tiny(**kw)
    inp = inputs_for(cfg)
    r = oracle.forward(cfg, inp)
    chosen, g_dense, y = run_brute(cfg, inp)
    assert r["topk_idx"].tolist() == chosen
    g = np.take_along_axis(np.asarray(g_dense), r["topk_idx"], axis=1)
    np.testing.assert_allclose(r["topk_w"], g, rtol=1e-13, atol=0)
    assert rel(r["y"], y) < 1e-12


def test_residual_adds_u():
    cfg = tiny()
    inp = inputs_for(cfg)
    r = oracle.forward(cfg, inp, residual=True)
    _, _, y = run_brute(cfg, inp, residual=True)
    assert rel(r["y"], y) < 1e-12


# --- pin (a): k = N_r, no shared experts -> dense softmax mixture -------------
def test_pin_a_dense_softmax_mixture():
    """MoE-survey page, section 2: G_sigma(x) = Softmax(x W_g), y = sum_i G_i E_i(x)."""
    cfg = tiny(n_shared=0, top_k=5, n_routed=5)
    inp = inputs_for(cfg)
    x = inp["x"].astype(np.float64)
    z = x @ inp["w_router"].astype(np.float64).T
    ez = np.exp(z - z.max(1, keepdims=True))
    G = ez / ez.sum(1, keepdims=True)
    y = np.zeros_like(x)
    for i in range(cfg.n_routed):
        h = x @ inp["w_gate"][i].astype(np.float64).T
        u = x @ inp["w_up"][i].astype(np.float64).T
        y += G[:, i:i + 1] * ((h * 0.5 * (1 + np.tanh(h / 2))) * u) @ inp["w_down"][i].astype(np.float64).T
    r = oracle.forward(cfg, inp)
    assert rel(r["y"], y) < 1e-12
    np.testing.assert_allclose(r["topk_w"].sum(1), 1.0, rtol=1e-14)
    rb = oracle.forward(cfg.with_(gate="topk_softmax"), inp)          # same at k = N_r
    assert rel(rb["y"], r["y"]) < 1e-13


# --- pin (b): splitting the intermediate dim into m pieces --------------------
@pytest.mark.parametrize("m", [2, 4])
def test_pin_b_split_ffn_sums_to_unsplit(m):
    """DeepSeekMoE page, section 3.1: an expert split along its intermediate
    dim into m smaller experts; with equal gates the pieces add up to the FFN."""
    rng = np.random.default_rng(5)
    d, I = 6, 8
    X = rng.standard_normal((9, d))
    w1, w3 = rng.standard_normal((I, d)), rng.standard_normal((I, d))
    w2 = rng.standard_normal((d, I))
    full = om.expert_ffn(X, w1, w3, w2)
    p = I // m
    parts = sum(om.expert_ffn(X, w1[j * p:(j + 1) * p], w3[j * p:(j + 1) * p], w2[:, j * p:(j + 1) * p])
                for j in range(m))
    assert rel(parts, full) < 1e-13


@pytest.mark.parametrize("gate", ["softmax_topk", "topk_softmax"])
@pytest.mark.parametrize("m", [2, 3])
def test_pin_b_fine_layer_equals_coarse_layer(gate, m):
    """Coarse layer (N experts, top-K) == fine layer (mN pieces, top-mK) when the m
    pieces of a base expert share its centroid and each piece's W2 is scaled by m
    (the replicated softmax gives each piece s/m)."""
    N, K, I = 4, 2, 6
    coarse = tiny(n_routed=N, top_k=K, d_ff=I, n_shared=1, gate=gate, tokens=10)
    inp = inputs_for(coarse, scale_router=3.0)
    p = I // m
    fine = coarse.with_(n_routed=m * N, top_k=m * K, d_ff=p)
    finp = dict(inp)
    finp["w_router"] = np.repeat(inp["w_router"], m, axis=0)
    finp["w_gate"] = inp["w_gate"].reshape(N * m, p, -1)
    finp["w_up"] = inp["w_up"].reshape(N * m, p, -1)
    w2 = inp["w_down"].astype(np.float64)                         # [N, d, I]; x m exact in fp64
    finp["w_down"] = np.stack([w2[b][:, j * p:(j + 1) * p] * m for b in range(N) for j in range(m)])
    rc, rf = oracle.forward(coarse, inp), oracle.forward(fine, finp)
    assert rel(rf["y"], rc["y"]) < 1e-12
    np.testing.assert_array_equal(rf["counts"], np.repeat(rc["counts"], m))
    np.testing.assert_array_equal(rf["topk_idx"] // m, np.repeat(rc["topk_idx"], m, axis=1))
    np.testing.assert_allclose(rf["topk_w"] * m, np.repeat(rc["topk_w"], m, axis=1), rtol=1e-13)


def test_parameter_count_constant_under_segmentation():
    """Section 3.1: splitting keeps the expert parameter count (16 x width 32 == 8 x width 64)."""
    per = lambda n, d, I: n * 3 * d * I
    assert per(16, 64, 32) == per(8, 64, 64)


# --- pin (c): m = 1, no shared experts -> GShard / Switch top-K ---------------
@pytest.mark.parametrize("k", [1, 2, 3])
def test_pin_c_gshard_topk(k):
    cfg = tiny(n_shared=0, top_k=k, n_routed=6)
    inp = inputs_for(cfg)
    r = oracle.forward(cfg, inp)
    chosen, g_dense, y = run_brute(cfg, inp)
    assert r["topk_idx"].tolist() == chosen
    assert rel(r["y"], y) < 1e-12
    if k == 1:
        # Switch top-1: y = p_max * E_argmax(x)
        x = inp["x"].astype(np.float64)
        for t in range(cfg.tokens):
            e = int(r["topk_idx"][t, 0])
            F = om.expert_ffn(x[t:t + 1], inp["w_gate"][e].astype(np.float64),
                              inp["w_up"][e].astype(np.float64), inp["w_down"][e].astype(np.float64))
            assert rel(r["y"][t], max(g_dense[t]) * F[0]) < 1e-13


# --- pin (d): the two gate variants -----------------------------------------
@pytest.mark.parametrize("k", [1, 2, 4])
def test_pin_d_gate_variants(k):
    cfg = tiny(n_shared=0, top_k=k, n_routed=6)
    inp = inputs_for(cfg)
    a = oracle.forward(cfg, inp)
    b = oracle.forward(cfg.with_(gate="topk_softmax"), inp)
    np.testing.assert_array_equal(a["topk_idx"], b["topk_idx"])          # softmax is monotone
    np.testing.assert_allclose(b["topk_w"], a["topk_w"] / a["topk_w"].sum(1, keepdims=True), rtol=1e-13)
    np.testing.assert_allclose(b["topk_w"].sum(1), 1.0, rtol=1e-14)
    assert np.all(a["topk_w"].sum(1) < 1.0)                            # k < N_r
    assert np.all(a["topk_w"] > 0)


# --- invariants stated on the pages -------------------------------------------
def test_dispatch_invariants():
    cfg = tiny(tokens=40, n_routed=7, top_k=3)
    inp = inputs_for(cfg)
    r = oracle.forward(cfg, inp)
    idx, P = r["topk_idx"], cfg.tokens * cfg.top_k
    assert r["counts"].sum() == P                                        # sum of counts = T K'
    assert all(len(set(row)) == cfg.top_k for row in idx.tolist())       # K' distinct per token
    assert np.all(np.diff(idx, axis=1) > 0)                              # ascending
    assert sorted(r["slot_row"].tolist()) == list(range(P))              # bijection
    for t in range(cfg.tokens):
        for j in range(cfg.top_k):
            row = r["slot_row"][t * cfg.top_k + j]
            assert r["row_token"][row] == t
            e = idx[t, j]
            assert r["offsets"][e] <= row < r["offsets"][e + 1]
    for e in range(cfg.n_routed):                                        # tokens ascending per expert
        seg = r["row_token"][r["offsets"][e]:r["offsets"][e + 1]]
        assert np.all(np.diff(seg) > 0)
        assert len(seg) == r["counts"][e]


def test_shared_only_is_dense_ffn_of_concatenated_width():
    """Routed contributions zeroed: the layer is one plain FFN of width K_s*I_s
    (textbook form with the shared experts' weights stacked)."""
    cfg = tiny(n_shared=3, d_ff_shared=4)
    inp = inputs_for(cfg)
    inp["w_down"] = np.zeros_like(inp["w_down"])
    x = inp["x"].astype(np.float64)
    W1 = inp["ws_gate"].reshape(-1, cfg.d_model).astype(np.float64)
    W3 = inp["ws_up"].reshape(-1, cfg.d_model).astype(np.float64)
    W2 = np.concatenate(list(inp["ws_down"].astype(np.float64)), axis=1)
    a = x @ W1.T
    y = ((a * (1.0 / (1.0 + np.exp(-a)))) * (x @ W3.T)) @ W2.T
    assert rel(oracle.forward(cfg, inp)["y"], y) < 1e-13


def test_tokens_are_independent():
    """Each token is routed and computed on its own (Switch section: per-token routing)."""
    cfg = tiny(tokens=16)
    inp = inputs_for(cfg)
    full = oracle.forward(cfg, inp)
    for t in (0, 7, 15):
        one = dict(inp)
        one["x"] = inp["x"][t:t + 1]
        r = oracle.forward(cfg.with_(tokens=1), one)
        assert rel(r["y"][0], full["y"][t]) < 1e-13
    sub = oracle.forward(cfg, inp, tokens=[3, 9])
    assert rel(sub["y"], full["y"][[3, 9]]) < 1e-13


def test_relabelling_experts_permutes_ids_only():
    cfg = tiny(tokens=20, n_routed=6, top_k=2)
    inp = inputs_for(cfg)
    perm = np.array([3, 0, 5, 1, 4, 2])
    pinp = dict(inp)
    for k in ("w_router", "w_gate", "w_up", "w_down"):
        pinp[k] = inp[k][perm]
    a, b = oracle.forward(cfg, inp), oracle.forward(cfg, pinp)
    inv = np.argsort(perm)
    np.testing.assert_array_equal(np.sort(inv[a["topk_idx"]], axis=1), b["topk_idx"])
    assert rel(b["y"], a["y"]) < 1e-13


# --- closed forms --------------------------------------------------------------
def _expr(v):
    if isinstance(v, (int, float)):
        return float(v)
    v = v.strip()
    if v.startswith("-ln(") or v.startswith("ln("):
        sign = -1.0 if v[0] == "-" else 1.0
        return sign * math.log(float(v[v.index("(") + 1:-1]))
    return float(Fraction(v))


def _tensor(x):
    if isinstance(x, list):
        return [_tensor(v) for v in x]
    return _expr(x)


@pytest.mark.parametrize("gate", ["softmax_topk", "topk_softmax"])
def test_worked_example_closed_form(gate):
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    I = g["inputs"]
    inp = {k: np.array(_tensor(I[k]), dtype=np.float64) for k in
           ("x", "w_router", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")}
    inp["bias"] = None
    cfg = LayerConfig(name="worked", tokens=1, d_model=2, n_routed=4, n_shared=1, top_k=2,
                      d_ff=1, d_ff_shared=1, gate=gate, dtype="f64")
    r = oracle.forward(cfg, inp)
    exp = g["expected"]
    assert r["topk_idx"].tolist() == exp["topk_idx"]
    np.testing.assert_allclose(r["topk_w"], _tensor(exp[gate]["topk_w"]), rtol=1e-15)
    np.testing.assert_allclose(r["y"] / math.log(3.0), _tensor(exp[gate]["y_over_ln3"]), rtol=1e-14)


def test_combination_counts_printed_on_page():
    g = json.load(open(os.path.join(GOLDEN, "combinations.json")))
    for v in g["values"]:
        assert math.comb(v["n"], v["k"]) == v["count"]
    # The oracle's top-2 selection over 16 experts reaches exactly 120 distinct sets.
    n, k = 16, 2
    seen = set()
    for a in range(n):
        for b in range(a + 1, n):
            z = np.zeros((1, n))
            z[0, a], z[0, b] = 2.0, 1.0
            seen.add(tuple(om.select_topk(z, k)[0].tolist()))
    assert len(seen) == g["values"][0]["count"]


def test_softmax_and_silu_closed_forms():
    z = np.log(np.array([[2.0, 4.0, 1.0, 1.0]]))
    np.testing.assert_allclose(om.softmax(z), [[0.25, 0.5, 0.125, 0.125]], rtol=1e-15)
    np.testing.assert_allclose(om.softmax(z + 123.0), om.softmax(z), rtol=1e-13)
    np.testing.assert_allclose(om.softmax(np.zeros((1, 7))), np.full((1, 7), 1 / 7), rtol=1e-15)
    a = np.array([math.log(3.0), -math.log(3.0), 0.0, 2.5])
    np.testing.assert_allclose(om.silu(a)[:3], [0.75 * math.log(3.0), -0.25 * math.log(3.0), 0.0],
                               rtol=1e-15, atol=1e-300)
    np.testing.assert_allclose(om.silu(-a) , om.silu(a) - a, rtol=1e-14)   # silu(-a) = silu(a) - a


def test_topk_tie_breaks_to_lower_id():
    z = np.array([[1.0, 3.0, 3.0, 0.5, 3.0]])
    assert om.select_topk(z, 2).tolist() == [[1, 2]]
    assert om.select_topk(z, 3).tolist() == [[1, 2, 4]]


def test_gap_rule_holds_and_is_deterministic():
    cfg = tiny(tokens=300, n_routed=8, top_k=3, d_model=16, gap=0.05)
    a, b = make_inputs(cfg), make_inputs(cfg)
    na, nb = oracle.enforce_gap(cfg, a), oracle.enforce_gap(cfg, b)
    assert na == nb and na > 0
    np.testing.assert_array_equal(a["x"], b["x"])
    z = om.router_logits(a["x"].astype(np.float64), a["w_router"].astype(np.float64))
    assert np.all(oracle.topk_gap(z, cfg.top_k) >= cfg.gap)


# --- planted mistakes: each must make a pin above fail ----------------------
def _renorm_gate(z, idx, gate):
    g = om.softmax(z)
    g = np.take_along_axis(g, idx, axis=1)
    return g / g.sum(1, keepdims=True)


MISTAKES = {
    "gate A renormalised": ("gate_values", lambda: _renorm_gate),
    "softmax sign flipped": ("softmax", lambda: (lambda z: np.exp(-z) / np.exp(-z).sum(-1, keepdims=True))),
    "shared experts dropped": ("shared_ffn", lambda: (lambda X, a, b, c: np.zeros_like(X))),
    "top-k picks smallest": ("select_topk", lambda: (lambda s, k: np.sort(np.argsort(s, axis=1, kind="stable")[:, :k], axis=1))),
    "silu applied to up": ("expert_ffn", lambda: (lambda X, w1, w3, w2: (om.silu(X @ w3.T) * (X @ w1.T)) @ w2.T)),
    "sigmoid for silu": ("silu", lambda: (lambda a: 1.0 / (1.0 + np.exp(-a)))),
    "bias ignored": ("router_logits", lambda: (lambda x, w, b=None: x @ w.T)),
}


@pytest.mark.parametrize("name", sorted(MISTAKES))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, make = MISTAKES[name]
    caught = False
    for kw in BRUTE_CASES:
        cfg = tiny(**kw)
        inp = inputs_for(cfg)
        _, g_dense, y = run_brute(cfg, inp)
        with monkeypatch.context() as mp:
            mp.setattr(om, attr, make())
            try:
                r = om.forward(cfg, inp)
                bad = rel(r["y"], y) > 1e-9
            except Exception:
                bad = True
        if bad:
            caught = True
            break
    assert caught, f"planted mistake {name!r} passed every brute-force pin"
