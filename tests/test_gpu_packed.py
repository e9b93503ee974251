"""GPU tests of the packed weight layout (moe_pack_weights and
MOE_WEIGHTS_PACKED).  Packing only reorders memory, and the GEMMs multiply
the same values in the same order, so every packed result must equal the
row-major one bit for bit; the forward is also checked against the oracle.
Every call goes through the C ABI."""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import oracle
from _parity import check_y, host, prepare, upload
from mixture_experts_layer_43_amd import ops
from synth import LayerConfig
from test_gpu_parity import announce, cfg_of, run_forward

pytestmark = pytest.mark.gpu

WEIGHTS = ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")


def packed_position(n, k, N, K):
    """Element offset of (n, k) of an [N, K] matrix in the packed order (include/moe.h)."""
    return (n // 128) * 128 * K + (k // 64) * 128 * 64 + (n % 128) * 64 + k % 64


def test_pack_layout_is_the_documented_one():
    announce("pack layout")
    g = torch.Generator().manual_seed(11)
    w = torch.randn(3, 256, 192, generator=g).to(torch.bfloat16)
    lay = ops.Layer(256, 4, 0, 2, 256, 256, dtype="bf16")
    p = ops.pack_weights(lay, w.cuda())
    torch.cuda.synchronize()
    src = w.view(torch.int16).numpy().reshape(3, -1)
    got = p.cpu().view(torch.int16).numpy().reshape(3, -1)
    n, k = np.meshgrid(np.arange(256), np.arange(192), indexing="ij")
    pos = packed_position(n, k, 256, 192)
    want = np.empty_like(src)
    want[:, pos.ravel()] = src[:, (n * 192 + k).ravel()]
    np.testing.assert_array_equal(got, want)


def packed_inputs(lay, d):
    out = dict(d)
    for k in WEIGHTS:
        out[k] = ops.pack_weights(lay, d.get(k))
    return out


CASES = {
    "unfolded-shared": LayerConfig(name="pk1", tokens=700, d_model=256, n_routed=16, n_shared=2, top_k=4,
                                   d_ff=256, d_ff_shared=128, seed=801),
    "folded-shared": LayerConfig(name="pk2", tokens=333, d_model=384, n_routed=12, n_shared=1, top_k=3,
                                 d_ff=128, d_ff_shared=128, seed=802),
}


@pytest.mark.parametrize("name,kw", [("16b-decode", {}), ("unfolded-shared", {}), ("folded-shared", {}),
                                     ("folded-shared", dict(ffn="relu")),
                                     ("unfolded-shared", dict(capacity=120, group_size=256)),
                                     ("2b", {}), ("16b", {})],
                         ids=["decode", "unfolded", "folded", "relu", "capacity", "2b", "16b"])
def test_packed_forward_equals_row_major(name, kw):
    cfg = (CASES[name] if name in CASES else cfg_of(name)).with_(**kw)
    announce(f"packed forward {name} {kw}")
    inp = prepare(cfg)
    d = upload(inp)
    ref = run_forward(cfg, d)
    y0, idx0 = ref.y.clone(), ref.topk_idx.clone()
    del ref
    lay = ops.Layer.of(cfg)
    lay_p = dataclasses.replace(lay, weight_layout="packed")
    dp = packed_inputs(lay, d)
    f = ops.Forward(lay_p, cfg.tokens, torch.device("cuda"))
    f(dp["x"], dp["w_router"], dp["bias"], dp["w_gate"], dp["w_up"], dp["w_down"], dp["ws_gate"],
      dp["ws_up"], dp["ws_down"])
    torch.cuda.synchronize()
    assert torch.equal(f.topk_idx, idx0)
    assert torch.equal(f.y, y0)
    y = host(f.y)
    del f, dp
    torch.cuda.empty_cache()
    if cfg.tokens <= 1000:
        check_y(y, oracle.forward(cfg, inp)["y"], cfg.dtype)


def test_packed_expert_and_shared_ffn_equal_row_major():
    cfg = CASES["unfolded-shared"]
    announce("packed expert_ffn / shared_ffn")
    inp = prepare(cfg)
    d = upload(inp)
    lay = ops.Layer.of(cfg)
    lay_p = dataclasses.replace(lay, weight_layout="packed")
    dp = packed_inputs(lay, d)
    idx, _ = ops.route(lay, d["x"], d["w_router"], d["bias"])
    pm = ops.permute(lay, idx, d["x"])
    a = ops.expert_ffn(lay, cfg.tokens, pm["offsets"], pm["x_perm"], d["w_gate"], d["w_up"], d["w_down"])
    b = ops.expert_ffn(lay_p, cfg.tokens, pm["offsets"], pm["x_perm"], dp["w_gate"], dp["w_up"], dp["w_down"])
    sa = ops.shared_ffn(lay, d["x"], d["ws_gate"], d["ws_up"], d["ws_down"])
    sb = ops.shared_ffn(lay_p, d["x"], dp["ws_gate"], dp["ws_up"], dp["ws_down"])
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(sa, sb)
