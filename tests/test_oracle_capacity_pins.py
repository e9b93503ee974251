"""Pins of the capacity-limited dispatch in the oracle (oracle/capacity.py and
the capacity branch of oracle.forward).

MoE-survey blog page, section 3 (GShard expert capacity, running counter,
overflowed tokens, local group dispatching) and section 4 (Switch expert
capacity).  The checks compare the oracle with a dense pure-Python forward
that masks gates token by token (tests/_brute.py), closed forms for forced
routing, counts that follow from the definition (min(count, C) per group and
expert), the C >= T case that must equal the dropless layer, and group
independence.  The last test plants plausible mistakes.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import oracle.capacity as ocap
import oracle.moe as om
from _brute import brute_forward
from synth import LayerConfig, make_inputs


def cfg_of(**kw):
    base = dict(name="cap", tokens=24, d_model=8, n_routed=6, n_shared=1, top_k=2, d_ff=4,
                d_ff_shared=3, dtype="f32", seed=901, gap=1e-3, zipf_s=1.2, capacity=5)
    base.update(kw)
    return LayerConfig(**base)


def inputs(cfg):
    inp = make_inputs(cfg)
    oracle.enforce_gap(cfg, inp)
    return inp


def routed(cfg, inp):
    z = om.router_logits(inp["x"].astype(np.float64), inp["w_router"].astype(np.float64),
                         None if inp["bias"] is None else inp["bias"].astype(np.float64))
    return om.route(z, cfg.top_k, cfg.gate)


def brute(cfg, inp, residual=False):
    L = {k: (None if v is None else np.asarray(v, np.float64).tolist()) for k, v in inp.items()}
    return brute_forward(L["x"], L["w_router"], L["bias"], L["w_gate"], L["w_up"], L["w_down"],
                         L["ws_gate"], L["ws_up"], L["ws_down"], cfg.top_k, cfg.gate, residual,
                         cfg.capacity, cfg.group_size)


CASES = [dict(), dict(capacity=2), dict(capacity=3, group_size=8), dict(capacity=1, group_size=5),
         dict(capacity=4, gate="topk_softmax"), dict(capacity=2, top_k=1, n_shared=0)]


@pytest.mark.parametrize("kw", CASES, ids=[str(c) for c in CASES])
def test_forward_matches_masked_dense_brute_force(kw):
    cfg = cfg_of(**kw)
    inp = inputs(cfg)
    _, g, y = brute(cfg, inp, residual=True)
    r = om.forward(cfg, inp, residual=True)
    np.testing.assert_allclose(r["y"], np.array(y), rtol=1e-12, atol=1e-12)
    # the dense gates left after the capacity are the kept routing gates
    dense = np.zeros((cfg.tokens, cfg.n_routed))
    rows = np.arange(cfg.tokens)[:, None]
    dense[rows, r["topk_idx"]] = r["topk_w"] * r["kept"]
    np.testing.assert_allclose(dense, np.array(g), rtol=1e-12, atol=0)


@pytest.mark.parametrize("S", [0, 7, 8])
@pytest.mark.parametrize("C", [1, 2, 5])
def test_kept_counts_are_min_of_count_and_capacity(C, S):
    cfg = cfg_of(tokens=40, capacity=C, group_size=S)
    idx, _ = routed(cfg, inputs(cfg))
    counts, offsets, row_token, slot_row, keep = ocap.dispatch_capacity(idx, cfg.n_routed, C, S)
    G = 1 if S == 0 else -(-40 // S)
    L = 40 if S == 0 else S
    want = np.zeros(cfg.n_routed, int)
    for g in range(G):
        c = np.bincount(idx[g * L:(g + 1) * L].ravel(), minlength=cfg.n_routed)
        want += np.minimum(c, C)
    np.testing.assert_array_equal(counts, want)
    assert offsets[-1] == keep.sum() == (slot_row >= 0).sum()
    # kept assignments of (group, expert) are the C lowest token ids among its takers
    for g in range(G):
        for e in range(cfg.n_routed):
            toks = sorted(t for t in range(g * L, min((g + 1) * L, 40)) if e in idx[t])
            mine = sorted(t for t in range(g * L, min((g + 1) * L, 40))
                          for j in range(cfg.top_k) if idx[t, j] == e and keep[t, j])
            assert mine == toks[:C]
    # rows: grouped by expert, tokens ascending, slot_row the inverse
    for e in range(cfg.n_routed):
        seg = row_token[offsets[e]:offsets[e + 1]]
        assert (np.diff(seg) > 0).all()
    for a in np.nonzero(slot_row >= 0)[0]:
        assert row_token[slot_row[a]] == a // cfg.top_k


def test_large_capacity_is_dropless():
    cfg = cfg_of(capacity=24)
    inp = inputs(cfg)
    a, b = om.forward(cfg, inp), om.forward(cfg.with_(capacity=0), inp)
    for k in ("counts", "offsets", "row_token", "slot_row"):
        np.testing.assert_array_equal(a[k], b[k])
    np.testing.assert_array_equal(a["y"], b["y"])
    assert a["kept"].all()


def test_one_token_groups_drop_nothing():
    # S = 1: every group is one token, whose K' experts are distinct.
    cfg = cfg_of(capacity=1, group_size=1)
    r = om.forward(cfg, inputs(cfg))
    assert r["kept"].all()


@pytest.mark.parametrize("S,C", [(0, 3), (4, 3), (5, 1)])
def test_forced_routing_closed_form(S, C):
    """Every token is sent to experts 1 and 4 by a large bias.  With capacity C
    per group of S tokens, exactly the first C tokens of each group keep both
    experts; every other token overflows and gets y = shared(x) + x."""
    cfg = cfg_of(tokens=13, capacity=C, group_size=S, zipf_s=0.0)
    inp = inputs(cfg)
    bias = np.zeros(cfg.n_routed, np.float32)
    bias[[1, 4]] = 40.0
    inp["bias"] = bias
    r = om.forward(cfg, inp, residual=True)
    L = 13 if S == 0 else S
    first = np.array([(t % L) < C for t in range(13)])
    np.testing.assert_array_equal(r["kept"], np.repeat(first[:, None], 2, axis=1))
    np.testing.assert_array_equal(r["counts"], [0, first.sum(), 0, 0, first.sum(), 0])
    x = om.decode(inp["x"], "f32")
    sh = om.shared_ffn(x, inp["ws_gate"].astype(np.float64), inp["ws_up"].astype(np.float64),
                       inp["ws_down"].astype(np.float64))
    np.testing.assert_allclose(r["y"][~first], (sh + x)[~first], rtol=1e-13, atol=1e-13)
    assert not np.allclose(r["y"][first], (sh + x)[first])


def test_groups_are_independent():
    cfg = cfg_of(tokens=30, capacity=2, group_size=10)
    idx, _ = routed(cfg, inputs(cfg))
    whole = ocap.keep_mask(idx, cfg.n_routed, 2, 10)
    parts = np.concatenate([ocap.keep_mask(idx[g:g + 10], cfg.n_routed, 2, 0) for g in (0, 10, 20)])
    np.testing.assert_array_equal(whole, parts)


def test_capacity_formulas():
    # Switch: tokens per batch / experts x factor (K' = 1).
    assert ocap.capacity_for(8192, 8, 1, 1.25) == 1280
    # GShard: 2N/(G E) per group for top-2 and factor 1.
    assert ocap.capacity_for(8192, 8, 2, 1.0, group_size=1024) == 2 * 1024 // 8
    assert ocap.capacity_for(100, 64, 6, 1.0) == 10          # ceil(600/64)


# --- planted mistakes: each must make a pin above fail ----------------------
def _keep_last(idx, n, C, S=0):
    return _orig_keep(idx[::-1], n, C, S)[::-1]


def _no_reset(idx, n, C, S=0):
    return _orig_keep(idx, n, C, 0)


def _whole_token(idx, n, C, S=0):
    keep = _orig_keep(idx, n, C, S)
    return np.repeat(keep.all(axis=1, keepdims=True), idx.shape[1], axis=1)


def _per_token_budget(idx, n, C, S=0):
    return _orig_keep(idx, n, C + 1, S)


_orig_keep = ocap.keep_mask
MISTAKES = {"keeps the last C": _keep_last, "counter never reset": _no_reset,
            "drops the whole token": _whole_token, "off by one": _per_token_budget}

PINS = [lambda: [test_forward_matches_masked_dense_brute_force(c) for c in CASES],
        lambda: [test_kept_counts_are_min_of_count_and_capacity(C, S) for C in (1, 2) for S in (0, 7)],
        lambda: [test_forced_routing_closed_form(S, C) for S, C in [(0, 3), (4, 3), (5, 1)]],
        test_groups_are_independent]


@pytest.mark.parametrize("name", sorted(MISTAKES))
def test_planted_mistake_is_caught(name, monkeypatch):
    monkeypatch.setattr(ocap, "keep_mask", MISTAKES[name])
    failed = 0
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0, f"planted mistake {name!r} passed every pin"
