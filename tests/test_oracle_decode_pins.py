"""Pins of the oracle's storage decoding (`oracle.decode`) and of its bf16 path.

Every bf16 tensor of the bf16 layers (x and the expert weights) enters the
oracle through `decode(a, "bf16")`, which turns uint16 bit patterns into
float64.  The checks below tie it to things other than itself:
  * hand values of the bfloat16 format (sign, 8-bit exponent with bias 127,
    7 stored fraction bits, subnormals below 2^-126);
  * PyTorch's own bfloat16 type, reading the same bit patterns;
  * a whole bf16 layer through the oracle against the pure-Python brute
    force fed with values PyTorch decoded (DeepSeekMoE page, section 3.2,
    eq. 9-11);
  * planted mistakes in decode (raw integers, a wrong shift, a half-precision
    reading) and in the top-k tie-break, each caught by a pin.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import oracle.moe as om
from _brute import brute_forward
from synth import LayerConfig, f32_to_bf16_bits, make_inputs

# (bit pattern, value) written out from the format's definition.
HAND = [
    (0x3F80, 1.0),                                  # exponent 127, fraction 0
    (0xC020, -2.5),                                 # sign, exponent 128, fraction .01b
    (0x4049, 3.140625),                             # 2 * (1 + 73/128)
    (0x3EAB, 0.333984375),                          # 2^-2 * (1 + 43/128)
    (0x0080, 2.0 ** -126),                          # smallest normal
    (0x0001, 2.0 ** -133),                          # smallest subnormal: 2^-126 * 2^-7
    (0x007F, 127 * 2.0 ** -133),                    # largest subnormal
    (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127),       # largest finite
    (0x0000, 0.0),
    (0x4300, 128.0),
    (0xBF00, -0.5),
]


def test_decode_hand_values():
    bits = np.array([b for b, _ in HAND], dtype=np.uint16)
    got = oracle.decode(bits, "bf16")
    assert got.dtype == np.float64
    for (b, want), g in zip(HAND, got.tolist()):
        assert g == want, f"0x{b:04X}: {g!r} != {want!r}"


def test_decode_negative_zero_keeps_its_sign():
    z = oracle.decode(np.array([0x8000], dtype=np.uint16), "bf16")
    assert z[0] == 0.0 and math.copysign(1.0, z[0]) == -1.0


def test_decode_agrees_with_torch_bfloat16_on_every_finite_pattern():
    # All 65536 patterns except NaN/Inf (exponent field 255).
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = ((bits >> 7) & 0xFF) != 0xFF
    bits = bits[finite]
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = oracle.decode(bits, "bf16")
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(np.signbit(got), np.signbit(want))


def test_round_trip_through_storage_rounding():
    """f32 -> bf16 bits (round to nearest even) -> decode equals PyTorch's own
    float32 -> bfloat16 -> float64 conversion."""
    rng = np.random.default_rng(5)
    a = (rng.standard_normal(200_000) * np.exp(rng.uniform(-20, 20, 200_000))).astype(np.float32)
    got = oracle.decode(f32_to_bf16_bits(a), "bf16")
    want = torch.from_numpy(a).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(got, want)


def test_decode_f32_and_none():
    a = np.array([[1.5, -3.25e-8], [7e30, 0.0]], dtype=np.float32)
    got = oracle.decode(a, "f32")
    assert got.dtype == np.float64
    np.testing.assert_array_equal(got, a.astype(np.float64))
    assert oracle.decode(None, "bf16") is None


def _torch_decoded_lists(inp):
    """Inputs as nested lists of float64, the bf16 tensors read by PyTorch."""
    out = {}
    for k, v in inp.items():
        if v is None:
            out[k] = None
        elif v.dtype == np.uint16:
            t = torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).view(torch.bfloat16)
            out[k] = t.double().numpy().tolist()
        else:
            out[k] = np.asarray(v, dtype=np.float64).tolist()
    return out


BF16_CASES = [
    dict(),
    dict(gate="topk_softmax", n_shared=0, top_k=1),
]


@pytest.mark.parametrize("kw", BF16_CASES)
def test_bf16_layer_matches_brute_force_on_torch_decoded_values(kw):
    base = dict(name="pin-bf16", tokens=10, d_model=8, n_routed=6, n_shared=1, top_k=2, d_ff=4,
                d_ff_shared=4, dtype="bf16", seed=913)
    base.update(kw)
    cfg = LayerConfig(**base)
    inp = make_inputs(cfg)
    oracle.enforce_gap(cfg, inp)
    assert inp["x"].dtype == np.uint16 and inp["w_gate"].dtype == np.uint16
    L = _torch_decoded_lists(inp)
    idx, _, y = brute_forward(L["x"], L["w_router"], L["bias"], L["w_gate"], L["w_up"], L["w_down"],
                              L["ws_gate"], L["ws_up"], L["ws_down"], cfg.top_k, cfg.gate)
    r = oracle.forward(cfg, inp)
    assert r["topk_idx"].tolist() == idx
    np.testing.assert_allclose(r["y"], np.asarray(y), rtol=1e-12, atol=1e-14)


# --- planted mistakes -------------------------------------------------------
DECODE_MISTAKES = {
    "raw integers": lambda a, dtype: None if a is None else np.asarray(a, dtype=np.float64),
    "shift by 15": lambda a, dtype: None if a is None else (
        (a.astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)
        if a.dtype == np.uint16 else np.asarray(a, dtype=np.float64)),
    "read as half": lambda a, dtype: None if a is None else (
        a.view(np.float16).astype(np.float64) if a.dtype == np.uint16 else np.asarray(a, dtype=np.float64)),
}


@pytest.mark.parametrize("name", sorted(DECODE_MISTAKES))
def test_planted_decode_mistake_is_caught(name, monkeypatch):
    caught = []
    with monkeypatch.context() as mp:
        mp.setattr(om, "decode", DECODE_MISTAKES[name])
        mp.setattr(oracle, "decode", DECODE_MISTAKES[name])
        for pin in (test_decode_hand_values, test_round_trip_through_storage_rounding,
                    lambda: test_bf16_layer_matches_brute_force_on_torch_decoded_values({})):
            try:
                pin()
            except AssertionError:
                caught.append(pin)
            except Exception:
                caught.append(pin)
    assert caught, f"planted mistake {name!r} passed every decode pin"


def test_planted_tie_break_mistake_is_caught(monkeypatch):
    """Ties broken toward the higher expert id fail the tie-break pin."""
    from test_oracle_pins import test_topk_tie_breaks_to_lower_id

    def higher_id_first(score, k):
        n = score.shape[1]
        order = np.argsort(-score[:, ::-1], axis=1, kind="stable")[:, :k]
        return np.sort(n - 1 - order, axis=1)

    monkeypatch.setattr(om, "select_topk", higher_id_first)
    with pytest.raises(AssertionError):
        test_topk_tie_breaks_to_lower_id()
