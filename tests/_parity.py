"""Shared helpers for the GPU parity tests: seeded inputs, device upload and
the tolerance rules (written here, applied to every comparison).

Tolerances (fixed rules):
  routing (topk_idx, counts, offsets, row_token, slot_row): bit-exact
  topk_w: |gpu - ref| <= 2e-5 * ref
  y, fp32 layers: ||d||/||ref|| <= 1e-5 and |d| <= 1e-4 * (|ref| + rms(ref))
  y, bf16 layers: ||d||/||ref|| <= 1e-2, per-row ||d_t||/||ref_t|| <= 2e-2 and
                  |d| <= 0.05 * rms(ref) + 0.02 * |ref|
The bf16 budget comes from three bf16 roundings on the GPU side (H, y_perm,
y; unit roundoff 2^-8 each, about 4e-3 relative RMS together) against an
exact fp64 reference.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from synth import make_inputs


def prepare(cfg):
    inp = make_inputs(cfg)
    oracle.enforce_gap(cfg, inp)
    return inp


def dev(a, device="cuda"):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:                      # bf16 bit patterns
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def host(t) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def upload(inp, device="cuda"):
    return {k: dev(v, device) for k, v in inp.items()}


def check_gates(w_gpu, w_ref):
    w_gpu, w_ref = np.asarray(w_gpu, np.float64), np.asarray(w_ref, np.float64)
    bad = np.abs(w_gpu - w_ref) > 2e-5 * np.abs(w_ref)
    assert not bad.any(), f"{bad.sum()} gate values off; worst {np.abs(w_gpu - w_ref).max():.3e}"


def check_y(y_gpu, y_ref, dtype, what="y"):
    y_gpu, y_ref = np.asarray(y_gpu, np.float64), np.asarray(y_ref, np.float64)
    assert y_gpu.shape == y_ref.shape
    if y_ref.size == 0:
        return
    d = y_gpu - y_ref
    rms = float(np.sqrt(np.mean(y_ref ** 2)))
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(y_ref), 1e-300))
    if dtype == "f32":
        assert rel <= 1e-5, f"{what}: relative error {rel:.3e}"
        bad = np.abs(d) > 1e-4 * (np.abs(y_ref) + rms)
    else:
        assert rel <= 1e-2, f"{what}: relative error {rel:.3e}"
        rows = y_ref.reshape(y_ref.shape[0], -1)
        dr = d.reshape(d.shape[0], -1)
        rr = np.linalg.norm(dr, axis=1) / np.maximum(np.linalg.norm(rows, axis=1), 1e-300)
        assert rr.max() <= 2e-2, f"{what}: worst row error {rr.max():.3e} at row {rr.argmax()}"
        bad = np.abs(d) > 0.05 * rms + 0.02 * np.abs(y_ref)
    assert not bad.any(), f"{what}: {bad.sum()} elements outside tolerance; max |d| {np.abs(d).max():.3e}, rms {rms:.3e}"
    return rel
