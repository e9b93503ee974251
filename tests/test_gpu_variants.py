"""GPU parity of the gate and FFN variants against the oracle, through the C ABI.

  ReLU expert FFN, wo ReLU(wi x) (MoE-survey blog page, section 3, GShard's
  position-wise FFN): the gate/up launch runs the single wi projection with
  a clamped epilogue.
  Selection-only bias (the Tencent Cloud "DeepSeek MoE" article, balancing
  without an auxiliary loss): top-K' on z + b, gate values and routing
  statistics from z.
Tolerances as in tests/_parity.py (routing bit-exact) and tests/test_gpu_stats.py.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from _parity import check_gates, check_y, host, prepare, upload
from mixture_experts_layer_43_amd import ops
from test_gpu_parity import MID, announce, cfg_of, check_routing, run_forward, sample_tokens
from test_gpu_stats import check_stats

pytestmark = pytest.mark.gpu

RELU = [("mid-ragged", {}), ("mid-gshard", {}), ("mid-f32", {}), ("16b-decode", {}),
        ("mid-smallm", dict(capacity=6, group_size=100)), ("tiny-f32", {}), ("mid-ragged-k", {}),
        ("decode-ragged-k", {})]


@pytest.mark.parametrize("name,kw", RELU, ids=[f"{n}{'-cap' if kw else ''}" for n, kw in RELU])
def test_relu_forward_matches_oracle(name, kw):
    cfg = cfg_of(name).with_(ffn="relu", **kw)
    announce(f"relu forward {name} {kw}")
    inp = prepare(cfg)
    assert inp["w_up"] is None
    ref = oracle.forward(cfg, inp)
    f = run_forward(cfg, upload(inp))
    np.testing.assert_array_equal(host(f.topk_idx), ref["topk_idx"])
    np.testing.assert_array_equal(host(f.counts), ref["counts"])
    check_y(host(f.y), ref["y"], cfg.dtype)


def test_relu_gshard_full_size():
    """The GShard-shaped layer (8 experts, top-2, Zipf skew) in its own FFN
    form: wo ReLU(wi x), at full size, y on sampled tokens."""
    cfg = cfg_of("gshard-zipf").with_(ffn="relu")
    sample = sample_tokens(cfg.tokens)
    announce("relu forward gshard-zipf full size")
    inp = prepare(cfg)
    ref = oracle.forward(cfg, inp, tokens=np.asarray(sample))
    d = upload(inp)
    f = run_forward(cfg, d)
    check_routing(f, ref)
    check_y(host(f.y)[list(sample)], ref["y"], cfg.dtype)
    del d, f
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["mid-ragged", "mid-f32"])
def test_relu_expert_and_shared_ffn_alone(name):
    cfg = cfg_of(name).with_(ffn="relu")
    announce(f"relu expert_ffn / shared_ffn {name}")
    inp = prepare(cfg)
    ref = oracle.forward(cfg, inp)
    d = upload(inp)
    lay = ops.Layer.of(cfg)
    idx = torch.from_numpy(ref["topk_idx"]).cuda()
    pm = ops.permute(lay, idx, d["x"])
    y_perm = ops.expert_ffn(lay, cfg.tokens, pm["offsets"], pm["x_perm"], d["w_gate"], None,
                            d["w_down"])
    y_sh = ops.shared_ffn(lay, d["x"], d["ws_gate"], None, d["ws_down"])
    torch.cuda.synchronize()
    x = oracle.decode(inp["x"], cfg.dtype)
    rows = ref["row_token"]
    want = np.zeros((rows.size, cfg.d_model))
    for e in range(cfg.n_routed):
        r = slice(ref["offsets"][e], ref["offsets"][e + 1])
        want[r] = oracle.relu_ffn(x[rows[r]], oracle.decode(inp["w_gate"][e], cfg.dtype),
                                  oracle.decode(inp["w_down"][e], cfg.dtype))
    check_y(host(y_perm), want, cfg.dtype, "y_perm")
    sh = oracle.shared_ffn(x, oracle.decode(inp["ws_gate"], cfg.dtype), None,
                           oracle.decode(inp["ws_down"], cfg.dtype), "relu")
    check_y(host(y_sh), sh, cfg.dtype, "y_shared")


SEL = ["mid-gshard", "mid-ragged", "mid-f32", "mid-many-experts", "16b-decode", "2b"]


@pytest.mark.parametrize("name", SEL)
def test_selection_bias_route_and_stats(name):
    cfg = cfg_of(name).with_(zipf_s=1.5, bias_mode="selection")
    announce(f"selection-only bias route {name}")
    inp = prepare(cfg)
    x = oracle.decode(inp["x"], cfg.dtype)
    z = oracle.router_logits(x, np.asarray(inp["w_router"], np.float64))
    idx, g = oracle.route_selection_bias(z, np.asarray(inp["bias"], np.float64), cfg.top_k, cfg.gate)
    lay = ops.Layer.of(cfg)
    d = upload(inp)
    gi, gw = ops.route(lay, d["x"], d["w_router"], d["bias"])
    D = 4 if cfg.n_routed % 4 == 0 else 1
    si, sw, stats, lse = ops.route_stats(lay, d["x"], d["w_router"], d["bias"], D, lse=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(gi), idx)
    check_gates(host(gw), g)
    assert torch.equal(si, gi) and torch.equal(sw, gw)
    check_stats(lay, D, stats, lse, oracle.routing_stats(z, idx, D))


@pytest.mark.parametrize("name", ["mid-gshard", "mid-ragged", "16b-decode"])
def test_selection_bias_forward(name):
    cfg = cfg_of(name).with_(zipf_s=1.5, bias_mode="selection")
    announce(f"selection-only bias forward {name}")
    inp = prepare(cfg)
    ref = oracle.forward(cfg, inp)
    f = run_forward(cfg, upload(inp))
    check_routing(f, ref)
    check_y(host(f.y), ref["y"], cfg.dtype)


def test_selection_bias_changes_gates_only_where_bias_is_set():
    """Without a bias both modes give identical bits."""
    cfg = MID["mid-ragged"]
    announce("bias modes without a bias")
    inp = prepare(cfg)
    d = upload(inp)
    a = ops.route(ops.Layer.of(cfg), d["x"], d["w_router"], None)
    b = ops.route(ops.Layer.of(cfg.with_(bias_mode="selection")), d["x"], d["w_router"], None)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ---- noisy top-k gating --------------------------------------------------------
NOISY = ["mid-gshard", "mid-ragged", "16b-decode", "2b", "mid-f32", "mid-many-experts", "mid-wide-k"]


def noisy_ref(cfg, inp):
    x = oracle.decode(inp["x"], cfg.dtype)
    zs, z = oracle.selection_and_gate_logits(cfg, inp, x)
    return oracle.route_on(zs, z, cfg.top_k, cfg.gate)


@pytest.mark.parametrize("name", NOISY)
def test_noisy_route_matches_oracle(name):
    cfg = cfg_of(name).with_(noisy=True)
    announce(f"noisy route {name}")
    inp = prepare(cfg)
    idx, g = noisy_ref(cfg, inp)
    d = upload(inp)
    gi, gw = ops.route_noisy(ops.Layer.of(cfg), d["x"], d["w_router"], d["bias"], d["w_noise"],
                             d["noise"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(gi), idx)
    check_gates(host(gw), g)


def test_noisy_route_with_selection_bias_and_zero_noise():
    cfg = MID["mid-gshard"].with_(noisy=True, bias_mode="selection", zipf_s=1.5)
    announce("noisy route, selection-only bias; zero noise = moe_route")
    inp = prepare(cfg)
    idx, g = noisy_ref(cfg, inp)
    d = upload(inp)
    lay = ops.Layer.of(cfg)
    gi, gw = ops.route_noisy(lay, d["x"], d["w_router"], d["bias"], d["w_noise"], d["noise"])
    zi, zw = ops.route_noisy(lay, d["x"], d["w_router"], d["bias"], d["w_noise"],
                             torch.zeros_like(d["noise"]))
    ri, rw = ops.route(lay, d["x"], d["w_router"], d["bias"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(gi), idx)
    check_gates(host(gw), g)
    assert torch.equal(zi, ri)
    np.testing.assert_allclose(host(zw), host(rw), rtol=1e-6)


@pytest.mark.parametrize("name", ["mid-ragged", "mid-gshard"])
def test_noisy_layer_through_the_staged_calls(name):
    """route_noisy -> permute -> expert_ffn -> shared_ffn -> combine gives the
    oracle's noisy-gated layer."""
    cfg = cfg_of(name).with_(noisy=True)
    announce(f"noisy layer, staged {name}")
    inp = prepare(cfg)
    ref = oracle.forward(cfg, inp)
    d = upload(inp)
    lay = ops.Layer.of(cfg)
    idx, w = ops.route_noisy(lay, d["x"], d["w_router"], d["bias"], d["w_noise"], d["noise"])
    pm = ops.permute(lay, idx, d["x"])
    y_perm = ops.expert_ffn(lay, cfg.tokens, pm["offsets"], pm["x_perm"], d["w_gate"], d["w_up"],
                            d["w_down"])
    y_sh = ops.shared_ffn(lay, d["x"], d["ws_gate"], d["ws_up"], d["ws_down"]) if cfg.n_shared else None
    y = ops.combine(lay, y_perm, pm["slot_row"], w, y_sh)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(idx), ref["topk_idx"])
    check_y(host(y), ref["y"], cfg.dtype)
