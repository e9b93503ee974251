"""Pins of the routing-statistics oracle (oracle/stats.py).

DeepSeekMoE page, section 3.3, eq. 12-17; MoE-survey blog page, section 4
(Switch balance loss) and section 5 (router z-loss).  Each check compares the
oracle with something other than itself: a hand-derived closed form,
invariants that follow from the definitions, special cases that reduce to
another page's formula computed along an independent path (arg-max and
bincount for Switch), and a pure-Python loop evaluation.  The last test
plants plausible mistakes and checks that a pin fails for each.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
import oracle.moe as om
import oracle.stats as ost
from synth import LayerConfig, make_inputs


def case(T=40, n=8, k=2, gate="softmax_topk", seed=5, bias=True):
    cfg = LayerConfig(name="stats", tokens=T, d_model=16, n_routed=n, n_shared=1, top_k=k,
                      d_ff=4, d_ff_shared=4, gate=gate, dtype="f32", seed=seed, gap=1e-3,
                      zipf_s=1.2 if bias else 0.0)
    inp = make_inputs(cfg)
    oracle.enforce_gap(cfg, inp)
    x = inp["x"].astype(np.float64)
    b = None if inp["bias"] is None else inp["bias"].astype(np.float64)
    z = om.router_logits(x, inp["w_router"].astype(np.float64), b)
    idx, _ = om.route(z, k, gate)
    return z, idx


def test_worked_example_closed_form():
    # T = 2 tokens, N' = 4 experts, K' = 1, D = 2 groups {0,1}, {2,3}.
    # Logits (ln 5, 0, 0, 0) and (0, 0, ln 5, 0): each token picks the expert
    # holding ln 5, with probability a = 5/8; the other three get b = 1/8.
    #   P = ((a+b)/2, b, (a+b)/2, b) = (3/8, 1/8, 3/8, 1/8)       eq. 14
    #   f = 4/(1*2) * (1, 0, 1, 0) = (2, 0, 2, 0)                  eq. 13
    #   L_ExpBal = 2*3/8 + 2*3/8 = 3/2                             eq. 12
    #   f' = (1, 1), P' = (1/2, 1/2), L_DevBal = 1                 eq. 15-17
    #   log-sum-exp = ln 8 for both tokens, z-loss = (ln 8)^2      z-loss
    z = np.array([[math.log(5), 0, 0, 0], [0, 0, math.log(5), 0]])
    idx = np.array([[0], [2]])
    r = oracle.routing_stats(z, idx, 2)
    np.testing.assert_allclose(r["P"], [3 / 8, 1 / 8, 3 / 8, 1 / 8], rtol=1e-15)
    np.testing.assert_array_equal(r["f"], [2, 0, 2, 0])
    np.testing.assert_array_equal(r["f_dev"], [1, 1])
    np.testing.assert_allclose(r["P_dev"], [0.5, 0.5], rtol=1e-15)
    assert abs(r["l_exp"] - 1.5) < 1e-15
    assert abs(r["l_dev"] - 1.0) < 1e-15
    assert abs(r["z_loss"] - math.log(8) ** 2) < 1e-14
    np.testing.assert_allclose(r["lse"], [math.log(8)] * 2, rtol=1e-15)


@pytest.mark.parametrize("gate", ["softmax_topk", "topk_softmax"])
@pytest.mark.parametrize("k", [1, 2, 3])
def test_sums_fixed_by_the_definitions(gate, k):
    # sum_i f_i = N'/(K'T) * T K' = N' and sum_i P_i = 1 (each s_t sums to 1).
    z, idx = case(k=k, gate=gate)
    r = oracle.routing_stats(z, idx, 4)
    assert abs(r["f"].sum() - 8) < 1e-12
    assert abs(r["P"].sum() - 1) < 1e-12
    assert abs(r["P_dev"].sum() - 1) < 1e-12
    assert abs(r["f_dev"].mean() - 1) < 1e-12


def test_device_groups_at_the_extremes():
    # D = N': every group is one expert, so eq. 15-17 reduce to eq. 12.
    # D = 1: f' = mean f = 1 and P' = sum P = 1, so L_DevBal = 1.
    z, idx = case()
    assert abs(oracle.routing_stats(z, idx, 8)["l_dev"] - oracle.routing_stats(z, idx, 8)["l_exp"]) < 1e-15
    assert abs(oracle.routing_stats(z, idx, 1)["l_dev"] - 1.0) < 1e-12
    with pytest.raises(ValueError):
        oracle.routing_stats(z, idx, 3)


def test_uniform_router():
    # All logits equal: P_i = 1/N', so L_ExpBal = sum f_i / N' = 1 whatever f
    # is, and log-sum-exp = c + ln N' for logits all equal to c.
    T, n, k, c = 10, 6, 2, 0.75
    z = np.full((T, n), c)
    idx = om.select_topk(om.softmax(z), k)
    r = oracle.routing_stats(z, idx, 3)
    np.testing.assert_allclose(r["P"], 1 / n, rtol=1e-15)
    assert abs(r["l_exp"] - 1) < 1e-15
    assert abs(r["z_loss"] - (c + math.log(n)) ** 2) < 1e-13


def test_balanced_assignment():
    # Every expert chosen equally often: f_i = 1, so L_ExpBal = sum P = 1.
    T, n, k = 12, 6, 2
    rng = np.random.default_rng(3)
    z = rng.normal(size=(T, n))
    idx = np.array([[(2 * t) % n, (2 * t + 1) % n] for t in range(T)])
    r = oracle.routing_stats(z, idx, 2)
    np.testing.assert_allclose(r["f"], 1.0, rtol=1e-15)
    assert abs(r["l_exp"] - 1) < 1e-12


def test_top1_is_the_switch_loss():
    # MoE-survey blog page, section 4: loss = alpha N sum_i f_i P_i with f_i the
    # share of tokens whose arg-max probability is expert i, P_i the mean router
    # probability.  With K' = 1 eq. 13 is N' times that share, so eq. 12 equals
    # the Switch loss at alpha = 1.  Computed here by arg-max and bincount.
    z, idx = case(T=64, n=8, k=1, bias=False)
    p = np.exp(z - z.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    share = np.bincount(np.argmax(p, axis=1), minlength=8) / z.shape[0]
    switch = 8 * float(np.dot(share, p.mean(0)))
    r = oracle.routing_stats(z, idx, 1)
    assert abs(r["l_exp"] - switch) < 1e-12


def test_load_fraction_agrees_with_dispatch_counts():
    z, idx = case(T=50, k=3)
    counts = om.dispatch(idx, 8)[0]
    np.testing.assert_allclose(oracle.routing_stats(z, idx, 2)["f"], counts * 8 / (3 * 50), rtol=1e-15)


def test_shift_of_all_logits():
    # Softmax and top-K' ignore a common shift c; log-sum-exp moves by c.
    z, idx = case()
    a, b = oracle.routing_stats(z, idx, 2), oracle.routing_stats(z + 2.5, idx, 2)
    np.testing.assert_allclose(b["P"], a["P"], rtol=1e-12)
    np.testing.assert_array_equal(b["f"], a["f"])
    np.testing.assert_allclose(b["lse"], a["lse"] + 2.5, rtol=1e-14)
    assert abs(b["z_loss"] - float(np.mean((a["lse"] + 2.5) ** 2))) < 1e-12


def test_matches_plain_loops():
    z, idx = case(T=9, n=6, k=2)
    T, n = z.shape
    P = [0.0] * n
    cnt = [0] * n
    zl = 0.0
    for t in range(T):
        e = [math.exp(v) for v in z[t]]
        tot = math.fsum(e)
        for i in range(n):
            P[i] += e[i] / tot / T
        for i in idx[t]:
            cnt[int(i)] += 1
        zl += math.log(tot) ** 2 / T
    f = [n / (2 * T) * c for c in cnt]
    r = oracle.routing_stats(z, idx, 2)
    np.testing.assert_allclose(r["P"], P, rtol=1e-13)
    np.testing.assert_allclose(r["f"], f, rtol=1e-15)
    assert abs(r["z_loss"] - zl) < 1e-12 * zl
    fd = [sum(f[3 * g:3 * g + 3]) / 3 for g in range(2)]
    Pd = [sum(P[3 * g:3 * g + 3]) for g in range(2)]
    assert abs(r["l_dev"] - sum(a * b for a, b in zip(fd, Pd))) < 1e-13
    assert abs(r["l_exp"] - sum(a * b for a, b in zip(f, P))) < 1e-13


def test_empty_batch():
    r = oracle.routing_stats(np.zeros((0, 4)), np.zeros((0, 2), np.int64), 2)
    assert r["l_exp"] == 0 and r["l_dev"] == 0 and r["z_loss"] == 0 and r["lse"].size == 0


# --- planted mistakes: each must make a pin above fail ----------------------
MISTAKES = {
    "P divided by N' not T": ("mean_probability", lambda: (lambda z: om.softmax(z).sum(0) / z.shape[1])),
    "f without N'/K'": ("load_fraction", lambda: (lambda idx, n: np.bincount(idx.ravel(), minlength=n) / idx.shape[0])),
    "strided device groups": ("device_fold", lambda: (lambda f, P, D: (f.reshape(-1, D).mean(0), P.reshape(-1, D).sum(0)))),
    "z-loss not squared": ("z_loss", lambda: (lambda z: float(np.mean(ost.logsumexp(z))))),
    "P from the chosen gates only": ("mean_probability", lambda: (lambda z: np.where(
        om.softmax(z) >= np.sort(om.softmax(z), 1)[:, [-1]], om.softmax(z), 0).sum(0) / z.shape[0])),
    "max subtracted, not added back": ("logsumexp", lambda: (lambda z: np.log(np.sum(np.exp(z - z.max(1, keepdims=True)), 1)))),
}

PINS = [test_worked_example_closed_form, lambda: test_sums_fixed_by_the_definitions("softmax_topk", 2),
        test_device_groups_at_the_extremes, test_uniform_router, test_balanced_assignment,
        test_top1_is_the_switch_loss, test_shift_of_all_logits, test_matches_plain_loops]


@pytest.mark.parametrize("name", sorted(MISTAKES))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, make = MISTAKES[name]
    monkeypatch.setattr(ost, attr, make())
    failed = 0
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError):
            failed += 1
    assert failed > 0, f"planted mistake {name!r} passed every pin"
