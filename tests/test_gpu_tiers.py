"""The expert GEMMs' tile configurations give the same bits.

moe_expert_ffn picks its tiles per launch from the rows per expert group:
32-row tiles up to 16 rows, 64-row tiles up to 63, and from 64 rows whichever
of the 128-, 192- and 256-row tiles finishes first for groups of that mean
size and that grid (rounds of tiles over the CUs), with non-temporal weight
copies where the groups fit in one row tile; gate/up and down may choose
differently.  Every configuration sums each output over K in the same order
(16-wide slices of 64-wide steps, in order, fp32 accumulation), so the choice
must not change any result.  With every expert holding the same weights,
cutting the same dispatched rows into 1 ... 256 groups moves the launches
through every configuration while the FFN of each row stays the same
(DeepSeekMoE page, section 3.2, eq. 9: FFN_i applied to the rows routed to
expert i): y_perm must be bit-identical across the cuts, and within the bf16
tolerance of the oracle."""
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

# 8192 rows of a 16B-like expert (d = 2048, I = 1408; ragged: 2040, 1392).
# Groups per cut and the tiles (gate/up, down) their mean rows select: 256
# rows (1, 8, 40, 46 / 1, 40, 64), 192 rows with plain copies (2 / 2, 8),
# with non-temporal copies (47, 64, 65 / 46, 47), 128 rows (70, 128 / 65,
# 70, 128) and 64 rows (129).  4096 rows of a small expert (d = 256,
# I = 192): 64 rows (100) and 32 rows (241, 256).
WIDE = [1, 2, 8, 40, 46, 47, 64, 65, 70, 128, 129]
SMALL = [100, 241, 256]


def cut_offsets(rows: int, n: int, seed: int) -> np.ndarray:
    """rows cut into n groups at sorted random points (some groups may be empty)."""
    rng = np.random.default_rng(seed)
    inner = np.sort(rng.integers(0, rows + 1, size=n - 1))
    return np.concatenate([[0], inner, [rows]]).astype(np.int32)


@pytest.mark.parametrize("layout,d,I,rows,cuts", [
    ("row_major", 2048, 1408, 8192, WIDE),
    ("row_major", 2040, 1392, 8192, WIDE),
    ("packed", 2048, 1408, 8192, WIDE),
    ("row_major", 256, 192, 4096, SMALL),
], ids=["aligned", "ragged-k", "packed", "small"])
def test_tile_configurations_give_identical_bits(layout, d, I, rows, cuts):
    announce(f"tile configurations d={d} I={I} rows={rows} {layout}")
    one = LayerConfig(name="tiers", tokens=rows, d_model=d, n_routed=1, n_shared=0, top_k=1,
                      d_ff=I, d_ff_shared=I, seed=901)
    inp = make_inputs(one)
    x = dev(inp["x"])
    w = {k: dev(inp[k]) for k in ("w_gate", "w_up", "w_down")}
    # The oracle's FFN of every row (one expert's weights serve every group).
    ref = oracle.expert_ffn(oracle.decode(inp["x"], "bf16"), oracle.decode(inp["w_gate"][0], "bf16"),
                            oracle.decode(inp["w_up"][0], "bf16"), oracle.decode(inp["w_down"][0], "bf16"))
    first = None
    for n in cuts:
        lay = ops.Layer(d_model=d, n_routed=n, n_shared=0, top_k=1, d_ff=I, d_ff_shared=I,
                        weight_layout=layout)
        ws = {k: v.expand(n, *v.shape[1:]).contiguous() for k, v in w.items()}
        if layout == "packed":
            ws = {k: ops.pack_weights(lay, v) for k, v in ws.items()}
        offsets = torch.from_numpy(cut_offsets(rows, n, 1000 + n)).cuda()
        y = ops.expert_ffn(lay, rows, offsets, x, ws["w_gate"], ws["w_up"], ws["w_down"])
        torch.cuda.synchronize()
        if first is None:
            first = y
            check_y(host(y), ref, "bf16", f"y_perm, {n} groups")
        else:
            same = torch.equal(y.view(torch.int16), first.view(torch.int16))
            assert same, f"{n} groups (mean {rows // n} rows) differ from {cuts[0]} groups"
        del ws, y
        torch.cuda.empty_cache()
