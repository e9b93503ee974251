"""moe_forward (and moe_forward_noalloc, which exists for such callers)
captured in a HIP graph: every replay, with eager work and synchronisations
between the replays, equals the eager forward bit for bit, and the eager
forward is within the layer rules of the oracle.  Every call goes through the
C ABI; PyTorch only supplies the graph object and the capture stream."""
from __future__ import annotations

import dataclasses

import pytest
import torch

import oracle
from _parity import check_y, host, prepare, upload
from mixture_experts_layer_43_amd import ops
from test_gpu_parity import announce, cfg_of

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,noalloc,packed", [("16b-decode", False, False), ("16b-decode", True, False),
                                                 ("16b-decode", False, True),
                                                 ("mid-ragged", False, False), ("mid-ragged", True, False),
                                                 ("mid-f32", False, False)])
def test_graph_replays_equal_the_eager_forward(name, noalloc, packed):
    """packed: expert weights and W_g in their packed orders, as bench.py
    captures the decode-shaped forward."""
    cfg = cfg_of(name)
    announce(f"graph capture {name} noalloc={noalloc} packed={packed}")
    inp = prepare(cfg)
    d = upload(inp)
    lay = ops.Layer.of(cfg)
    if packed:
        for k in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down"):
            d[k] = ops.pack_weights(lay, d[k])
        d["w_router"] = ops.pack_router(lay, d["w_router"])
        lay = dataclasses.replace(lay, weight_layout="packed", router_layout="packed")
    f = ops.Forward(lay, cfg.tokens, torch.device("cuda"), noalloc=noalloc)
    args = [d[k] for k in ("x", "w_router", "bias", "w_gate", "w_up", "w_down", "ws_gate", "ws_up",
                           "ws_down")]
    f(*args)
    torch.cuda.synchronize()
    y0, idx0, w0, c0 = f.y.clone(), f.topk_idx.clone(), f.topk_w.clone(), f.counts.clone()
    check_y(host(y0), oracle.forward(cfg, inp)["y"], cfg.dtype)

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        f(*args, checked=True)
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(g):
        f(*args, checked=True)
    for _ in range(4):
        # eager work between replays: clear the outputs with torch's fill kernel
        for t in (f.y, f.topk_idx, f.topk_w, f.counts):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(f.y, y0)
        assert torch.equal(f.topk_idx, idx0)
        assert torch.equal(f.topk_w, w0)
        assert torch.equal(f.counts, c0)
    del g
