"""The seeded input generator: determinism, rounding and distributions."""
import numpy as np
import pytest
import torch

from synth import CONFIGS, bf16_bits_to_f32, f32_to_bf16_bits, get_config, make_inputs, zipf_bias


def test_bf16_rounding_is_round_to_nearest_even():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.0, -2.5, 1e-30, 3.0e38], dtype=np.float32)])
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(f32_to_bf16_bits(a), ref)
    # exact ties: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 -> to even (1.0)
    tie_down = np.array([1.0 + 2.0 ** -8], dtype=np.float32)
    tie_up = np.array([1.0 + 3 * 2.0 ** -8], dtype=np.float32)          # -> 1 + 2^-6 (even)
    assert bf16_bits_to_f32(f32_to_bf16_bits(tie_down))[0] == 1.0
    assert bf16_bits_to_f32(f32_to_bf16_bits(tie_up))[0] == 1.0 + 2.0 ** -6


def test_inputs_are_deterministic_and_shaped():
    cfg = get_config("tiny-f32")
    a, b = make_inputs(cfg), make_inputs(cfg)
    for k in a:
        if a[k] is None:
            assert b[k] is None
            continue
        np.testing.assert_array_equal(a[k], b[k])
    assert a["x"].shape == (64, 64) and a["x"].dtype == np.float32
    assert a["w_gate"].shape == (16, 32, 64) and a["w_down"].shape == (16, 64, 32)
    assert a["ws_gate"].shape == (1, 32, 64)
    c = make_inputs(cfg, seed=cfg.seed + 1)
    assert not np.array_equal(a["x"], c["x"])


def test_bf16_layer_inputs_and_scales():
    cfg = get_config("16b-decode").with_(tokens=256)
    inp = make_inputs(cfg)
    assert inp["x"].dtype == np.uint16 and inp["w_gate"].dtype == np.uint16
    assert inp["w_router"].dtype == np.float32 and inp["bias"] is None
    x = bf16_bits_to_f32(inp["x"])
    assert abs(x.std() - 1.0) < 0.01
    assert abs(inp["w_router"].std() * np.sqrt(cfg.d_model) - 1.0) < 0.02
    assert abs(bf16_bits_to_f32(inp["w_gate"][3]).std() * np.sqrt(cfg.d_model) - 1.0) < 0.01
    assert abs(bf16_bits_to_f32(inp["w_down"][5]).std() * np.sqrt(cfg.d_ff) - 1.0) < 0.01


def test_zipf_bias():
    b = zipf_bias(8, 1.2)
    np.testing.assert_allclose(b, -1.2 * np.log(np.arange(1, 9)), rtol=1e-6)
    cfg = get_config("gshard-zipf")
    assert cfg.zipf_s == 1.2 and cfg.gate == "topk_softmax"


@pytest.mark.parametrize("name", sorted(CONFIGS))
def test_config_shapes(name):
    c = get_config(name)
    assert 1 <= c.top_k <= c.n_routed
    assert c.dtype in ("f32", "bf16")
