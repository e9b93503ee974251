"""Seeded random layers through moe_forward against the oracle.

Forty layer shapes drawn from a fixed seed over what the boundary accepts
(include/moe.h): bf16 with d % 8 == 0 and I, I_s % 16 == 0, fp32 with
multiples of 4; 1..256 routed experts, top-1..16, 0..3 shared experts of the
routed width or another one; 1..3000 tokens; both gates, the SiLU and ReLU
FFNs, both bias modes and sometimes an expert capacity.  Routing and counts
must match bit for bit and y within the layer's tolerance (tests/_parity.py),
as for the hand-picked shapes.  Sizes stay small enough for the oracle to
finish each case in well under a second.  Where the layer admits the packed
router order (bf16, d % 64 == 0, N_r <= 128) the forward on packed W_g must
also equal the row-major one bit for bit."""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import oracle
from _parity import check_gates, check_y, host, prepare, upload
from mixture_experts_layer_43_amd import ops
from synth import LayerConfig
from test_gpu_parity import announce, run_forward

pytestmark = pytest.mark.gpu

N_CASES = 40


def draw(i: int) -> LayerConfig:
    rng = np.random.default_rng(9100 + i)
    f32 = rng.random() < 0.2
    qd, qi = (4, 4) if f32 else (8, 16)
    d = int(qd * rng.integers(1, 320 // qd + 1))
    I = int(qi * rng.integers(1, 320 // qi + 1))
    n_routed = int(rng.choice([1, 2, 3, 8, 16, 33, 64, 100, 200, 256]))
    top_k = int(rng.integers(1, min(16, n_routed) + 1))
    n_shared = int(rng.integers(0, 4))
    I_s = I if rng.random() < 0.6 else int(qi * rng.integers(1, 320 // qi + 1))
    tokens = int(rng.choice([1, 2, 7, 31, 64, 129, 300, 777, 1500, 3000]))
    # Keep the oracle's work (tokens x experts per token x widths) small.
    while tokens * (top_k + n_shared) * d * max(I, I_s) > 4e8 and tokens > 1:
        tokens //= 2
    cap = 0
    group = 0
    if rng.random() < 0.2:
        cap = int(rng.integers(1, max(2, tokens * top_k // n_routed + 2)))
        group = int(rng.choice([0, max(1, tokens // 3)]))
    return LayerConfig(
        name=f"fuzz-{i}", tokens=tokens, d_model=d, n_routed=n_routed, n_shared=n_shared,
        top_k=top_k, d_ff=I, d_ff_shared=I_s,
        gate=str(rng.choice(["softmax_topk", "topk_softmax"])), dtype="f32" if f32 else "bf16",
        bias_mode=str(rng.choice(["logits", "selection"])), ffn=str(rng.choice(["silu", "relu"])),
        capacity=cap, group_size=group, seed=9200 + i)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_layer_matches_oracle(i):
    cfg = draw(i)
    announce(f"fuzz {i}: T={cfg.tokens} d={cfg.d_model} N_r={cfg.n_routed} K'={cfg.top_k} "
             f"K_s={cfg.n_shared} I={cfg.d_ff} I_s={cfg.d_ff_shared} {cfg.dtype} {cfg.gate} "
             f"{cfg.ffn} bias={cfg.bias_mode} C={cfg.capacity} S={cfg.group_size}")
    inp = prepare(cfg)
    ref = oracle.forward(cfg, inp)
    d = upload(inp)
    f = run_forward(cfg, d)
    np.testing.assert_array_equal(host(f.topk_idx), ref["topk_idx"])
    np.testing.assert_array_equal(host(f.counts), ref["counts"])
    np.testing.assert_array_equal(host(f.offsets), ref["offsets"])
    check_gates(host(f.topk_w), ref["topk_w"])
    check_y(host(f.y), ref["y"], cfg.dtype)
    if cfg.dtype == "bf16" and cfg.d_model % 64 == 0 and cfg.n_routed <= 128:
        lay = ops.Layer.of(cfg)
        wp = ops.pack_router(lay, d["w_router"])
        fp = ops.Forward(dataclasses.replace(lay, router_layout="packed"), cfg.tokens, torch.device("cuda"))
        fp(d["x"], wp, d["bias"], d["w_gate"], d["w_up"], d["w_down"], d.get("ws_gate"), d.get("ws_up"),
           d.get("ws_down"))
        torch.cuda.synchronize()
        assert torch.equal(fp.topk_idx, f.topk_idx)
        assert torch.equal(fp.topk_w, f.topk_w)
        assert torch.equal(fp.y, f.y)
