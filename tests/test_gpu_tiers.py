"""The expert GEMMs' tile configurations give the same bits.

moe_expert_ffn picks its tiles from the rows per expert group: 32-row tiles
up to 16 rows, 64-row tiles up to 63, and from 64 rows whichever of the
128-, 192- and 256-row tiles leaves the least work for groups of that mean
size, with non-temporal weight copies where the groups fit in one row tile.
Every configuration sums each output over K in the same order (16-wide
slices of 64-wide steps, in order, fp32 accumulation), so the choice must
not change any result.  With every expert holding the same weights, cutting
the same 4096 dispatched rows into 2 ... 256 groups moves the launch through
every configuration while the FFN of each row stays the same (DeepSeekMoE
page, section 3.2, eq. 9: FFN_i applied to the rows routed to expert i):
y_perm must be bit-identical across the cuts, and within the bf16 tolerance
of the oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from _parity import check_y, dev, host
from mixture_experts_layer_43_amd import ops
from synth import LayerConfig, make_inputs
from test_gpu_parity import announce

pytestmark = pytest.mark.gpu

ROWS = 4096
# Groups per cut and the tiles their mean rows (4096 / n) select: 256 rows
# (2, 8, 20), 192 rows with plain (14) and non-temporal copies (26, 34), 128
# rows (40, 64), 64 rows (65, 100, 200) and 32 rows (241, 256).
CUTS = [2, 8, 14, 20, 26, 34, 40, 64, 65, 100, 200, 241, 256]


def cut_offsets(n: int, seed: int) -> np.ndarray:
    """ROWS rows cut into n groups at sorted random points (some groups may be empty)."""
    rng = np.random.default_rng(seed)
    inner = np.sort(rng.integers(0, ROWS + 1, size=n - 1))
    return np.concatenate([[0], inner, [ROWS]]).astype(np.int32)


@pytest.mark.parametrize("layout,d,I", [("row_major", 256, 192), ("row_major", 200, 176),
                                        ("packed", 256, 256)],
                         ids=["aligned", "ragged-k", "packed"])
def test_tile_configurations_give_identical_bits(layout, d, I):
    announce(f"tile configurations d={d} I={I} {layout}")
    one = LayerConfig(name="tiers", tokens=ROWS, d_model=d, n_routed=1, n_shared=0, top_k=1,
                      d_ff=I, d_ff_shared=I, seed=901)
    inp = make_inputs(one)
    x = dev(inp["x"])
    w = {k: dev(inp[k]) for k in ("w_gate", "w_up", "w_down")}
    # The oracle's FFN of every row (one expert's weights serve every group).
    ref = oracle.expert_ffn(oracle.decode(inp["x"], "bf16"), oracle.decode(inp["w_gate"][0], "bf16"),
                            oracle.decode(inp["w_up"][0], "bf16"), oracle.decode(inp["w_down"][0], "bf16"))
    first = None
    for n in CUTS:
        lay = ops.Layer(d_model=d, n_routed=n, n_shared=0, top_k=1, d_ff=I, d_ff_shared=I,
                        weight_layout=layout)
        ws = {k: v.expand(n, *v.shape[1:]).contiguous() for k, v in w.items()}
        if layout == "packed":
            ws = {k: ops.pack_weights(lay, v) for k, v in ws.items()}
        offsets = torch.from_numpy(cut_offsets(n, 1000 + n)).cuda()
        y = ops.expert_ffn(lay, ROWS, offsets, x, ws["w_gate"], ws["w_up"], ws["w_down"])
        torch.cuda.synchronize()
        if first is None:
            first = y
            check_y(host(y), ref, "bf16", f"y_perm, {n} groups")
        else:
            same = torch.equal(y.view(torch.int16), first.view(torch.int16))
            assert same, f"{n} groups (mean {ROWS // n} rows) differ from {CUTS[0]} groups"
        del ws
    torch.cuda.empty_cache()
