"""Plain fp64 routing statistics of one batch (test infrastructure only).

Sources (titles and sections of the pages these follow):
  [P1] "DeepSeekMoE" translated paper page, section 3.3:
       eq. 12-14, expert-level balance: f_i = N'/(K'T) * (number of tokens
       that chose routed expert i), P_i = mean over the batch of the gate
       probability s_{i,t}, L_ExpBal = alpha_1 * sum_i f_i P_i;
       eq. 15-17, device-level balance over D groups of routed experts:
       f'_g = mean of f over group g, P'_g = sum of P over group g,
       L_DevBal = alpha_2 * sum_g f'_g P'_g.
  [P4] MoE-survey blog page ("six MoE papers"), section 4 (Switch
       Transformer: alpha * N * sum_i f_i P_i, f_i = share of tokens whose
       arg-max expert is i) and section 5 (ST-MoE router z-loss: mean over
       tokens of (log sum_j exp z_j)^2, on the logits entering the router
       softmax).

Readings taken where the pages leave a step open:
  * alpha_1 = alpha_2 = 1: the losses are returned unscaled and the caller
    multiplies by its balance factors.
  * s_{i,t} of eq. 14 is the softmax over all N' routed experts of the
    logits the router selects from (bias included), for both gate kinds;
    the indicator of eq. 13 is membership in the chosen top-K' set.
  * the D device groups are contiguous equal ranges of expert ids,
    group g = [g N'/D, (g+1) N'/D); D must divide N'.
  * the z-loss is taken on the same logits (bias included), over the N'
    routed experts (shared experts have no logit).
  * the Switch loss is the K' = 1 case of eq. 12 (f of eq. 13 is then N
    times the Switch token share), so it is not a separate output.
"""
from __future__ import annotations

import numpy as np

from .moe import softmax


def logsumexp(z: np.ndarray) -> np.ndarray:
    """log sum_j exp z_j per row, shifted by the row maximum."""
    m = np.max(z, axis=-1)
    return m + np.log(np.sum(np.exp(z - m[:, None]), axis=-1))


def load_fraction(idx: np.ndarray, n: int) -> np.ndarray:
    """[P1] eq. 13: f_i = N'/(K'T) * #{t : expert i is among token t's top-K'}."""
    T, k = idx.shape
    chosen = np.zeros((T, n))
    chosen[np.arange(T)[:, None], idx] = 1.0
    return chosen.sum(axis=0) * (n / (k * T))


def mean_probability(z: np.ndarray) -> np.ndarray:
    """[P1] eq. 14: P_i = (1/T) sum_t s_{i,t}, s = softmax over the routed experts."""
    return softmax(z).sum(axis=0) / z.shape[0]


def device_fold(f: np.ndarray, P: np.ndarray, n_devices: int):
    """[P1] eq. 16-17 over contiguous equal groups: (mean of f, sum of P) per group."""
    g = f.shape[0] // n_devices
    return f.reshape(n_devices, g).mean(axis=1), P.reshape(n_devices, g).sum(axis=1)


def balance(f: np.ndarray, P: np.ndarray) -> float:
    """[P1] eq. 12 and eq. 15 with alpha = 1: sum_i f_i P_i."""
    return float(np.sum(f * P))


def z_loss(z: np.ndarray) -> float:
    """[P4] section 5: mean over tokens of (log sum_j exp z_j)^2."""
    return float(np.mean(logsumexp(z) ** 2))


def routing_stats(z: np.ndarray, idx: np.ndarray, n_devices: int) -> dict:
    """Statistics of one routed batch.

    z   [T, N'] router logits (bias included), idx [T, K'] chosen experts.
    Returns P [N'], f [N'], f_dev [D], P_dev [D], l_exp, l_dev, z_loss and
    lse [T] (the per-token log-sum-exp that the z-loss squares).  An empty
    batch gives zeros everywhere.
    """
    T, n = z.shape
    if n_devices < 1 or n % n_devices != 0:
        raise ValueError("the number of device groups must divide the routed expert count")
    if T == 0:
        zero = np.zeros(n)
        fd, pd = device_fold(zero, zero, n_devices)
        return {"P": zero, "f": zero, "f_dev": fd, "P_dev": pd, "l_exp": 0.0,
                "l_dev": 0.0, "z_loss": 0.0, "lse": np.zeros(0)}
    P = mean_probability(z)
    f = load_fraction(idx, n)
    f_dev, P_dev = device_fold(f, P, n_devices)
    return {"P": P, "f": f, "f_dev": f_dev, "P_dev": P_dev, "l_exp": balance(f, P),
            "l_dev": balance(f_dev, P_dev), "z_loss": z_loss(z), "lse": logsumexp(z)}
