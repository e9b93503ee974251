"""moe_forward_noalloc: the forward with its scratch in the library's static
device array, for callers that cannot allocate.  Checked through the C ABI
against moe_forward (bit for bit: the same launches on the same values) and
against the fp64 oracle (routing bit-exact, y under the layer rules), on two
calls in a row, the second with a smaller batch."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import oracle
from _parity import check_gates, check_y, host, prepare, upload
from mixture_experts_layer_43_amd import _lib, ops
from test_gpu_parity import MID, announce, cfg_of

pytestmark = pytest.mark.gpu

# (layer, first batch, second smaller batch)
CASES = [("16b-decode", 128, 37), ("mid-ragged", 1000, 300), ("tiny-f32", 64, 17),
         ("mid-gshard", 777, 129)]


def sub_inputs(inp, T):
    out = dict(inp)
    out["x"] = inp["x"][:T]
    return out


@pytest.mark.parametrize("name,T1,T2", CASES)
def test_noalloc_forward_equals_forward(name, T1, T2):
    cfg = cfg_of(name)
    announce(f"noalloc forward {name} T={T1} then T={T2}")
    inp = prepare(cfg)
    d = upload(inp)
    lay = ops.Layer.of(cfg)
    w = [d[k] for k in ("w_router", "bias", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")]
    ref = {}
    for T in (T1, T2):
        f = ops.Forward(lay, T, torch.device("cuda"))
        f(d["x"][:T].contiguous(), *w)
        torch.cuda.synchronize()
        ref[T] = {k: getattr(f, k).clone() for k in ("y", "topk_idx", "topk_w", "counts", "offsets")}
        del f
    # Two calls in a row on the static scratch, the second with fewer tokens.
    na = {T: ops.Forward(lay, T, torch.device("cuda"), noalloc=True) for T in (T1, T2)}
    assert na[T1].ws is None and na[T2].ws is None
    for T in (T1, T2):
        na[T](d["x"][:T].contiguous(), *w)
    torch.cuda.synchronize()
    for T in (T1, T2):
        for k, v in ref[T].items():
            assert torch.equal(getattr(na[T], k), v), f"T={T}: {k} differs from moe_forward"
        want = oracle.forward(cfg.with_(tokens=T), sub_inputs(inp, T))
        np.testing.assert_array_equal(host(na[T].topk_idx), want["topk_idx"])
        np.testing.assert_array_equal(host(na[T].counts), want["counts"])
        np.testing.assert_array_equal(host(na[T].offsets), want["offsets"])
        check_gates(host(na[T].topk_w), want["topk_w"])
        check_y(host(na[T].y), want["y"], cfg.dtype)


def test_noalloc_refuses_a_batch_beyond_the_static_scratch():
    cfg = cfg_of("16b-decode")
    announce("noalloc refuses an oversized batch")
    lay = ops.Layer.of(cfg)
    T = 4096
    assert ops.workspace_size(lay, T) > _lib.MOE_STATIC_SCRATCH_BYTES
    x = torch.zeros((T, cfg.d_model), dtype=torch.bfloat16, device="cuda")
    y = torch.full((T, cfg.d_model), 7.0, dtype=torch.bfloat16, device="cuda")
    p = ops._p
    st = _lib.lib().moe_forward_noalloc(
        ctypes.byref(lay.c()), T, p(x), p(x), None, p(x), p(x), p(x), p(x), p(x), p(x), None, p(y),
        None, None, None, None, ops._stream())
    torch.cuda.synchronize()
    assert st == _lib.MOE_ERR_SCRATCH_TOO_SMALL
    assert torch.all(y == 7.0)      # nothing was launched
