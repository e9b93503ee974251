"""GPU tests of the packed router order (moe_pack_router, MOE_ROUTER_PACKED).
Packing only reorders W_g in memory, and the matrix-core router multiplies the
same values in the same order, so topk_idx, topk_w, the routing statistics and
the whole forward must equal the row-major results bit for bit (the parity
tests compare those with the oracle).  Every call goes through the C ABI."""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

from _parity import host, prepare, upload
from mixture_experts_layer_43_amd import ops
from mixture_experts_layer_43_amd._lib import router_pad_rows
from synth import make_inputs
from test_gpu_parity import announce, cfg_of, run_forward
from test_gpu_packed import packed_inputs

pytestmark = pytest.mark.gpu


def packed_router_position(e, k, R):
    """Float index of element (e, k) of the padded [R, d] router matrix in the
    packed order (include/moe.h, MOE_ROUTER_PACKED)."""
    return (((k // 16) * (R // 32) + e // 32) * 2 + (k % 8) // 4) * 256 + \
        (e % 32 + 32 * ((k % 16) // 8)) * 4 + k % 4


@pytest.mark.parametrize("n_routed,d", [(8, 64), (63, 192), (64, 128), (100, 64), (128, 192)])
def test_pack_router_layout_is_the_documented_one(n_routed, d):
    announce(f"pack router layout N_r={n_routed} d={d}")
    g = torch.Generator().manual_seed(n_routed * 1000 + d)
    w = torch.randn(n_routed, d, generator=g)
    lay = ops.Layer(d, n_routed, 0, 2, 64, 64, dtype="bf16")
    p = ops.pack_router(lay, w.cuda())
    torch.cuda.synchronize()
    R = router_pad_rows(n_routed)
    assert tuple(p.shape) == (R, d)
    e, k = np.meshgrid(np.arange(R), np.arange(d), indexing="ij")
    want = np.empty(R * d, dtype=np.float32)
    want[packed_router_position(e, k, R).ravel()] = w.numpy()[np.minimum(e, n_routed - 1), k].ravel()
    np.testing.assert_array_equal(p.cpu().numpy().ravel(), want)


# Every path of the matrix-core router: 64-token workgroups with streamed K
# ranges (16b, and a ragged last token block), 32-token ones with streamed
# ranges (GShard-shaped, one 32-row expert block), ranges taken round by
# round (2b: d = 1280 gives 10 slices per wavefront), split K with the
# separate selection (decode), four expert blocks (N_r = 100), and the
# selection-only bias.
ROUTE_CASES = [
    ("16b", {}), ("16b", dict(tokens=16384 + 37)), ("gshard-zipf", {}),
    ("gshard-zipf", dict(bias_mode="selection")), ("2b", {}), ("16b-decode", {}),
    ("mid-wide-k", {}), ("mid-smallm", {}),
]


@pytest.mark.parametrize("name,kw", ROUTE_CASES,
                         ids=[n + ("-" + "-".join(f"{k}{v}" for k, v in kw.items()) if kw else "")
                              for n, kw in ROUTE_CASES])
def test_packed_router_equals_row_major(name, kw):
    cfg = cfg_of(name).with_(**kw)
    announce(f"packed router {name} {kw} T={cfg.tokens}")
    d = upload(make_inputs(cfg, experts=False))
    lay = ops.Layer.of(cfg)
    lay_p = dataclasses.replace(lay, router_layout="packed")
    wp = ops.pack_router(lay, d["w_router"])
    i0, w0 = ops.route(lay, d["x"], d["w_router"], d["bias"])
    i1, w1 = ops.route(lay_p, d["x"], wp, d["bias"])
    torch.cuda.synchronize()
    assert torch.equal(i0, i1)
    assert torch.equal(w0.view(torch.int32), w1.view(torch.int32))
    n_dev = 4 if cfg.n_routed % 4 == 0 else 1
    r0 = ops.route_stats(lay, d["x"], d["w_router"], d["bias"], n_devices=n_dev, lse=True)
    r1 = ops.route_stats(lay_p, d["x"], wp, d["bias"], n_devices=n_dev, lse=True)
    torch.cuda.synchronize()
    for a, b in zip(r0, r1):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    assert torch.equal(r1[0], i1) and torch.equal(r1[1], w1)


@pytest.mark.parametrize("name", ["16b-decode", "16b"])
def test_packed_router_forward_equals_row_major(name):
    """The forward with packed expert weights and packed W_g, as the bench
    times it, against the all-row-major forward."""
    cfg = cfg_of(name)
    announce(f"packed router forward {name}")
    d = upload(prepare(cfg))
    ref = run_forward(cfg, d)
    y0, idx0, w0 = ref.y.clone(), ref.topk_idx.clone(), ref.topk_w.clone()
    del ref
    lay = ops.Layer.of(cfg)
    lay_p = dataclasses.replace(lay, weight_layout="packed", router_layout="packed")
    dp = packed_inputs(lay, d)
    dp["w_router"] = ops.pack_router(lay, d["w_router"])
    f = ops.Forward(lay_p, cfg.tokens, torch.device("cuda"))
    f(dp["x"], dp["w_router"], dp["bias"], dp["w_gate"], dp["w_up"], dp["w_down"], dp["ws_gate"],
      dp["ws_up"], dp["ws_down"])
    torch.cuda.synchronize()
    assert torch.equal(f.topk_idx, idx0)
    assert torch.equal(f.topk_w, w0)
    assert torch.equal(f.y, y0)
    assert np.isfinite(host(f.y)).all()
    del f, dp, d
    torch.cuda.empty_cache()
