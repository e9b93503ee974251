"""Seeded input generator (PCG64 streams keyed by tensor and expert).

Recipe (every draw is float32 standard normal from numpy's PCG64):
  x           [T, d]          N(0, 1), rows drawn in blocks of 1024 rows,
                              block b from stream (seed, 0, b)
  w_router    [N_r, d] f32    N(0, 1/d)                 stream (seed, 1)
  bias        [N_r]    f32    -s * ln(e + 1) for Zipf(s) skew, else absent
  w_noise     [N_r, d] f32    N(0, 1/d), noisy gating only   stream (seed, 10)
  noise       [T, N_r] f32    N(0, 1), the gating noise draws  stream (seed, 11)
  w_gate      [N_r, I, d]     N(0, 1/d)   expert e from stream (seed, 2, e)
  w_up        [N_r, I, d]     N(0, 1/d)                  stream (seed, 3, e)
  w_down      [N_r, d, I]     N(0, 1/I)                  stream (seed, 4, e)
  ws_gate     [K_s, I_s, d]   N(0, 1/d)                  stream (seed, 5, s)
  ws_up       [K_s, I_s, d]   N(0, 1/d)                  stream (seed, 6, s)
  ws_down     [K_s, d, I_s]   N(0, 1/I_s)                stream (seed, 7, s)
  redraw of row t, attempt a  N(0, 1)                    stream (seed, 9, t, a)
Each N(0, v) draw is a float32 standard normal times float32(sqrt(v)).
bf16 layers then round x and every expert weight to bfloat16 with
round-to-nearest-even and hand them over as uint16 bit patterns; the router
weights and bias stay float32.  fp32 layers keep everything float32.

Nothing here computes any part of the layer.  Keeping only tokens whose
top-k logit gap is wide enough is done by the caller, which asks for
replacement rows through `redraw_x_rows`.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import LayerConfig

_ROW_BLOCK = 1024


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even.

    Inputs here are finite normal draws, so NaN/Inf handling is not needed.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exact float32 values."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _stream(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def _normal(shape, std: float, *key: int) -> np.ndarray:
    g = _stream(*key)
    a = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a) if dtype == "bf16" else a


def zipf_bias(n_routed: int, s: float) -> np.ndarray:
    """Per-expert router bias -s*ln(e+1): a Zipf(s)-like preference for low ids."""
    e = np.arange(n_routed, dtype=np.float64)
    return (-s * np.log(e + 1.0)).astype(np.float32)


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _fill_experts(out: np.ndarray, std: float, seed: int, tensor: int, dtype: str, pool) -> None:
    def one(e: int) -> None:
        out[e] = _store(_normal(out.shape[1:], std, seed, tensor, e), dtype)
    list(pool.map(one, range(out.shape[0])))


def make_x(cfg: LayerConfig, seed: int | None = None, pool=None) -> np.ndarray:
    seed = cfg.seed if seed is None else seed
    T, d = cfg.tokens, cfg.d_model
    sdt = np.uint16 if cfg.dtype == "bf16" else np.float32
    x = np.empty((T, d), dtype=sdt)
    nblk = (T + _ROW_BLOCK - 1) // _ROW_BLOCK

    def one(b: int) -> None:
        r0, r1 = b * _ROW_BLOCK, min(T, (b + 1) * _ROW_BLOCK)
        x[r0:r1] = _store(_normal((r1 - r0, d), 1.0, seed, 0, b), cfg.dtype)

    if pool is None:
        for b in range(nblk):
            one(b)
    else:
        list(pool.map(one, range(nblk)))
    return x


def make_inputs(cfg: LayerConfig, seed: int | None = None, experts: bool = True) -> dict:
    """All layer inputs in storage form (uint16 bf16 bits, or float32).

    experts=False skips the routed/shared expert weights (router-only work).
    """
    seed = cfg.seed if seed is None else seed
    T, d, Nr, Ks, I, Is = (cfg.tokens, cfg.d_model, cfg.n_routed, cfg.n_shared,
                           cfg.d_ff, cfg.d_ff_shared)
    sdt = np.uint16 if cfg.dtype == "bf16" else np.float32
    out = {}
    with ThreadPoolExecutor(_workers()) as pool:
        out["x"] = make_x(cfg, seed, pool)
        out["w_router"] = _normal((Nr, d), 1.0 / np.sqrt(d), seed, 1)
        out["bias"] = zipf_bias(Nr, cfg.zipf_s) if cfg.zipf_s > 0 else None
        if cfg.noisy:
            # Noisy top-k gating: W_noise like W_g, and the standard normal
            # draws of every (token, expert), an input of the method.
            out["w_noise"] = _normal((Nr, d), 1.0 / np.sqrt(d), seed, 10)
            out["noise"] = _normal((T, Nr), 1.0, seed, 11)
        if experts:
            for name, tensor, shape, std in (
                ("w_gate", 2, (Nr, I, d), 1.0 / np.sqrt(d)),
                ("w_up", 3, (Nr, I, d), 1.0 / np.sqrt(d)),
                ("w_down", 4, (Nr, d, I), 1.0 / np.sqrt(I)),
                ("ws_gate", 5, (Ks, Is, d), 1.0 / np.sqrt(d)),
                ("ws_up", 6, (Ks, Is, d), 1.0 / np.sqrt(d)),
                ("ws_down", 7, (Ks, d, Is), 1.0 / np.sqrt(Is)),
            ):
                if cfg.ffn == "relu" and name in ("w_up", "ws_up"):
                    out[name] = None          # the ReLU FFN has two matrices
                    continue
                a = np.empty(shape, dtype=sdt)
                _fill_experts(a, std, seed, tensor, cfg.dtype, pool)
                out[name] = a
    return out


def redraw_x_rows(cfg: LayerConfig, tokens, attempt: int, seed: int | None = None) -> np.ndarray:
    """Fresh N(0,1) rows for the given token ids (storage form), one stream per (token, attempt)."""
    seed = cfg.seed if seed is None else seed
    rows = [_store(_normal((cfg.d_model,), 1.0, seed, 9, int(t), attempt), cfg.dtype)
            for t in tokens]
    sdt = np.uint16 if cfg.dtype == "bf16" else np.float32
    return np.stack(rows).astype(sdt, copy=False) if rows else np.empty((0, cfg.d_model), sdt)
