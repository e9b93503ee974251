"""Keep only tokens whose routing decision is far from a tie (test infrastructure).

The top-k choice is an integer decision taken from floating-point logits.
The GPU takes it from fp32 logits, this oracle from fp64 ones.  Both agree
whenever the K'-th and (K'+1)-th largest logits are at least `cfg.gap`
apart, far more than the fp32 accumulation error of a length-d dot product
(about 1e-6 here).  Rows of x that miss the gap are replaced by fresh draws
from the seeded generator until they meet it.  The selection order is the
same for both gate kinds (softmax is monotone), so the test is on logits.
"""
from __future__ import annotations

import numpy as np

from synth import redraw_x_rows

from .moe import decode, selection_and_gate_logits


def topk_gap(z: np.ndarray, k: int) -> np.ndarray:
    """z_(k) - z_(k+1) per row (inf when k equals the number of experts)."""
    if k >= z.shape[1]:
        return np.full(z.shape[0], np.inf)
    part = -np.sort(-z, axis=1)
    return part[:, k - 1] - part[:, k]


def enforce_gap(cfg, inputs: dict, max_attempts: int = 64) -> int:
    """Redraw x rows in place until every token meets the gap; returns #tokens redrawn."""
    x = inputs["x"]

    def sel_logits(rows):
        sub = dict(inputs)
        if inputs.get("noise") is not None:
            sub["noise"] = inputs["noise"][rows]
        return selection_and_gate_logits(cfg, sub, decode(x[rows], cfg.dtype))[0]

    z = sel_logits(np.arange(x.shape[0]))
    bad = np.nonzero(topk_gap(z, cfg.top_k) < cfg.gap)[0]
    redrawn = int(bad.size)
    attempt = 0
    while bad.size:
        if attempt >= max_attempts:
            raise RuntimeError(f"gap rule not met for {bad.size} tokens after {max_attempts} redraws")
        x[bad] = redraw_x_rows(cfg, bad, attempt)
        zb = sel_logits(bad)
        bad = bad[topk_gap(zb, cfg.top_k) < cfg.gap]
        attempt += 1
    return redrawn
