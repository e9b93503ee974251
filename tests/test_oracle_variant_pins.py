"""Pins of the oracle's gate and FFN variants.

GShard's position-wise ReLU FFN, FFN_e(x) = wo ReLU(wi x) (MoE-survey blog
page, section 3).  Checked against the dense pure-Python brute force, the
split identity of the intermediate dimension (DeepSeekMoE page, section 3.1,
which holds for any FFN that acts element-wise on the intermediate), and
closed forms where the ReLU is the identity or zero.  Planted mistakes
close the file.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import oracle.moe as om
from _brute import brute_forward
from synth import LayerConfig, make_inputs


def cfg_of(**kw):
    base = dict(name="variant", tokens=10, d_model=6, n_routed=5, n_shared=1, top_k=2, d_ff=4,
                d_ff_shared=3, dtype="f32", seed=931, gap=1e-3, ffn="relu")
    base.update(kw)
    return LayerConfig(**base)


def inputs(cfg):
    inp = make_inputs(cfg)
    oracle.enforce_gap(cfg, inp)
    return inp


RELU_CASES = [dict(), dict(gate="topk_softmax"), dict(n_shared=0, top_k=1), dict(n_shared=2, top_k=3),
              dict(zipf_s=1.2, capacity=3)]


@pytest.mark.parametrize("kw", RELU_CASES, ids=[str(c) for c in RELU_CASES])
def test_relu_layer_matches_dense_brute_force(kw):
    cfg = cfg_of(**kw)
    inp = inputs(cfg)
    assert inp["w_up"] is None and inp["ws_up"] is None
    L = {k: (None if v is None else np.asarray(v, np.float64).tolist()) for k, v in inp.items()}
    _, _, y = brute_forward(L["x"], L["w_router"], L["bias"], L["w_gate"], None, L["w_down"],
                            L["ws_gate"], None, L["ws_down"], cfg.top_k, cfg.gate, True,
                            cfg.capacity, cfg.group_size, ffn="relu")
    np.testing.assert_allclose(om.forward(cfg, inp, residual=True)["y"], np.array(y),
                               rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("m", [2, 4])
def test_relu_split_identity(m):
    rng = np.random.default_rng(5)
    X, wi, wo = rng.normal(size=(7, 6)), rng.normal(size=(8, 6)), rng.normal(size=(6, 8))
    whole = om.relu_ffn(X, wi, wo)
    parts = sum(om.relu_ffn(X, wi[j::m], wo[:, j::m]) for j in range(m))
    np.testing.assert_allclose(parts, whole, rtol=1e-13, atol=1e-13)


def test_relu_identity_and_zero_regions():
    # Non-negative x and wi: every pre-activation is >= 0, ReLU is the identity
    # and the FFN is the linear map wo wi.  With wi <= 0 it is exactly zero.
    rng = np.random.default_rng(6)
    X, wi, wo = np.abs(rng.normal(size=(5, 4))), np.abs(rng.normal(size=(3, 4))), rng.normal(size=(4, 3))
    np.testing.assert_allclose(om.relu_ffn(X, wi, wo), X @ (wo @ wi).T, rtol=1e-13)
    assert not om.relu_ffn(X, -wi, wo).any()


def test_relu_expert_rows_closed_form():
    # One token, one hidden unit per expert: FFN(x) = wo * max(0, wi . x).
    x = np.array([[1.0, -2.0, 0.5]])
    wi = np.array([[0.5, 0.25, 2.0]])      # wi . x = 0.5 - 0.5 + 1.0 = 1.0
    wo = np.array([[3.0], [-1.0], [0.0]])
    np.testing.assert_array_equal(om.relu_ffn(x, wi, wo), [[3.0, -1.0, 0.0]])
    np.testing.assert_array_equal(om.relu_ffn(x, -wi, wo), [[0.0, 0.0, 0.0]])


# --- planted mistakes --------------------------------------------------------
MISTAKES = {
    "relu after wo": lambda X, wi, wo: np.maximum(X @ wi.T @ wo.T, 0.0),
    "silu instead of relu": lambda X, wi, wo: om.silu(X @ wi.T) @ wo.T,
    "leaky": lambda X, wi, wo: np.where(X @ wi.T > 0, X @ wi.T, 0.01 * (X @ wi.T)) @ wo.T,
}
PINS = [lambda: [test_relu_layer_matches_dense_brute_force(c) for c in RELU_CASES],
        test_relu_identity_and_zero_regions, test_relu_expert_rows_closed_form]


@pytest.mark.parametrize("name", sorted(MISTAKES))
def test_planted_mistake_is_caught(name, monkeypatch):
    monkeypatch.setattr(om, "relu_ffn", MISTAKES[name])
    failed = 0
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0, f"planted mistake {name!r} passed every pin"


# --- selection-only bias ------------------------------------------------------
SEL_CASES = [dict(ffn="silu", zipf_s=1.2, bias_mode="selection"),
             dict(ffn="silu", zipf_s=1.2, bias_mode="selection", gate="topk_softmax"),
             dict(ffn="relu", zipf_s=2.0, bias_mode="selection", top_k=1, n_shared=0)]


@pytest.mark.parametrize("kw", SEL_CASES, ids=[str(c) for c in SEL_CASES])
def test_selection_bias_matches_dense_brute_force(kw):
    cfg = cfg_of(**kw)
    inp = inputs(cfg)
    L = {k: (None if v is None else np.asarray(v, np.float64).tolist()) for k, v in inp.items()}
    chosen, g, y = brute_forward(L["x"], L["w_router"], L["bias"], L["w_gate"], L.get("w_up"),
                                 L["w_down"], L["ws_gate"], L.get("ws_up"), L["ws_down"], cfg.top_k,
                                 cfg.gate, False, ffn=cfg.ffn, bias_mode="selection")
    r = om.forward(cfg, inp)
    np.testing.assert_array_equal(r["topk_idx"], np.array(chosen))
    np.testing.assert_allclose(r["y"], np.array(y), rtol=1e-12, atol=1e-12)
    dense = np.zeros((cfg.tokens, cfg.n_routed))
    dense[np.arange(cfg.tokens)[:, None], r["topk_idx"]] = r["topk_w"]
    np.testing.assert_allclose(dense, np.array(g), rtol=1e-12, atol=0)


def test_selection_bias_forced_experts_closed_form():
    """A bias of 40 on experts 1 and 3 makes every token choose them; with the
    bias in the logits their softmax_topk gates are ~1/2 each and sum to ~1,
    with a selection-only bias they are the unbiased s_1, s_3."""
    cfg = cfg_of(ffn="silu", bias_mode="selection", tokens=8)
    inp = inputs(cfg)
    bias = np.zeros(cfg.n_routed)
    bias[[1, 3]] = 40.0
    z = om.router_logits(inp["x"].astype(np.float64), inp["w_router"].astype(np.float64))
    idx, g = om.route_selection_bias(z, bias, 2, "softmax_topk")
    assert (idx == [1, 3]).all()
    s = np.exp(z - z.max(1, keepdims=True))
    s /= s.sum(1, keepdims=True)
    np.testing.assert_allclose(g, s[:, [1, 3]], rtol=1e-14)
    _, gl = om.route(z + bias, 2, "softmax_topk")
    assert np.all(np.abs(gl.sum(1) - 1) < 1e-12) and np.all(g.sum(1) < 0.99)


def test_zero_bias_is_the_plain_route():
    rng = np.random.default_rng(8)
    z = rng.normal(size=(20, 7))
    for gate in ("softmax_topk", "topk_softmax"):
        a, b = om.route(z, 3, gate), om.route_selection_bias(z, np.zeros(7), 3, gate)
        np.testing.assert_array_equal(a[0], b[0])
        np.testing.assert_array_equal(a[1], b[1])


SEL_MISTAKES = {
    "gates from biased logits": lambda z, b, k, gate: om.route(z + b[None, :], k, gate),
    "selection ignores bias": lambda z, b, k, gate: om.route(z, k, gate),
}
SEL_PINS = [lambda: [test_selection_bias_matches_dense_brute_force(c) for c in SEL_CASES],
            test_selection_bias_forced_experts_closed_form]


@pytest.mark.parametrize("name", sorted(SEL_MISTAKES))
def test_planted_selection_mistake_is_caught(name, monkeypatch):
    monkeypatch.setattr(om, "route_selection_bias", SEL_MISTAKES[name])
    failed = 0
    for pin in SEL_PINS:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0, f"planted mistake {name!r} passed every pin"


# --- noisy top-k gating -----------------------------------------------------
NOISY_CASES = [dict(ffn="silu", noisy=True, gate="topk_softmax"),
               dict(ffn="silu", noisy=True),
               dict(ffn="relu", noisy=True, zipf_s=1.2, bias_mode="selection", gate="topk_softmax")]


@pytest.mark.parametrize("kw", NOISY_CASES, ids=[str(c) for c in NOISY_CASES])
def test_noisy_gating_matches_dense_brute_force(kw):
    cfg = cfg_of(**kw)
    inp = inputs(cfg)
    L = {k: (None if v is None else np.asarray(v, np.float64).tolist()) for k, v in inp.items()}
    chosen, g, y = brute_forward(L["x"], L["w_router"], L["bias"], L["w_gate"], L.get("w_up"),
                                 L["w_down"], L["ws_gate"], L.get("ws_up"), L["ws_down"], cfg.top_k,
                                 cfg.gate, False, ffn=cfg.ffn, bias_mode=cfg.bias_mode,
                                 w_noise=L["w_noise"], noise=L["noise"])
    r = om.forward(cfg, inp)
    np.testing.assert_array_equal(r["topk_idx"], np.array(chosen))
    np.testing.assert_allclose(r["y"], np.array(y), rtol=1e-12, atol=1e-12)


def test_softplus_closed_forms():
    np.testing.assert_allclose(om.softplus(np.array([0.0])), [np.log(2.0)], rtol=1e-15)
    np.testing.assert_allclose(om.softplus(np.array([50.0, 800.0])), [50.0, 800.0], rtol=1e-15)
    np.testing.assert_allclose(om.softplus(np.array([-40.0])), [np.exp(-40.0)], rtol=1e-12)
    v = np.linspace(-5, 5, 11)
    np.testing.assert_allclose(om.softplus(v) - om.softplus(-v), v, atol=1e-14)   # sp(v) - sp(-v) = v


def test_noise_term_closed_form():
    # W_noise = 0 makes every Softplus ln 2, so H = x W_g + eps ln 2; eps = 0
    # gives the noiseless logits.
    rng = np.random.default_rng(9)
    x, wg, eps = rng.normal(size=(6, 5)), rng.normal(size=(4, 5)), rng.normal(size=(6, 4))
    np.testing.assert_allclose(om.noisy_logits(x, wg, np.zeros((4, 5)), eps), x @ wg.T + eps * np.log(2.0),
                               rtol=1e-14, atol=1e-14)
    np.testing.assert_array_equal(om.noisy_logits(x, wg, rng.normal(size=(4, 5)), np.zeros((6, 4))), x @ wg.T)


def test_zero_noise_is_the_noiseless_layer():
    cfg = cfg_of(ffn="silu", noisy=True)
    inp = inputs(cfg)
    inp["noise"] = np.zeros_like(inp["noise"])
    a = om.forward(cfg, inp)
    b = om.forward(cfg.with_(noisy=False), {k: v for k, v in inp.items() if k not in ("w_noise", "noise")})
    np.testing.assert_array_equal(a["topk_idx"], b["topk_idx"])
    np.testing.assert_allclose(a["y"], b["y"], rtol=1e-15, atol=0)


NOISE_MISTAKES = {
    "noise without softplus": lambda x, wg, wn, eps: x @ wg.T + eps * (x @ wn.T),
    "exp instead of softplus": lambda x, wg, wn, eps: x @ wg.T + eps * np.exp(x @ wn.T),
    "noise scaled by the clean logit": lambda x, wg, wn, eps: x @ wg.T + eps * om.softplus(x @ wg.T),
}
NOISE_PINS = [lambda: [test_noisy_gating_matches_dense_brute_force(c) for c in NOISY_CASES],
              test_noise_term_closed_form]


@pytest.mark.parametrize("name", sorted(NOISE_MISTAKES))
def test_planted_noise_mistake_is_caught(name, monkeypatch):
    monkeypatch.setattr(om, "noisy_logits", NOISE_MISTAKES[name])
    failed = 0
    for pin in NOISE_PINS:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0, f"planted mistake {name!r} passed every pin"
