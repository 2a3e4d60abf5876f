"""Shared helpers for the parity tests: run the oracle on the exact values the GPU receives and
compare with the tolerance rule max|x - x_ref| <= tol * rms(x_ref) over a whole tensor."""
from __future__ import annotations

import numpy as np
import torch

from gated_deltanet_delta_amd import synth
from oracle import oracle as O

TOL_BF16 = 2e-2   # bf16 inputs
TOL_F32 = 1e-4    # fp32 inputs


def tol_for(dtype: torch.dtype) -> float:
    return TOL_BF16 if dtype == torch.bfloat16 else TOL_F32


def to_gpu(x: dict, device: str = "cuda") -> dict:
    out = {}
    for key in ("q", "k", "v", "g", "beta", "initial_state", "cu_seqlens"):
        t = x.get(key)
        out[key] = None if t is None else t.to(device).contiguous()
    return out


def oracle_of(x: dict, unit_mask=None):
    f = synth.to_f64
    cu = None if x.get("cu_seqlens") is None else x["cu_seqlens"].cpu().numpy()
    return O.forward(f(x["q"]), f(x["k"]), f(x["v"]), f(x["g"]), f(x["beta"]),
                     f(x.get("initial_state")), cu, unit_mask=unit_mask)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    ok = ~np.isnan(ref)
    got, ref = got[ok], ref[ok]
    rms = float(np.sqrt(np.mean(np.square(ref))))
    return float(np.max(np.abs(got - ref))) / max(rms, 1e-300)


def assert_close_blocked(name: str, got: torch.Tensor, ref: np.ndarray, tol: float, rows: int = 2048) -> float:
    """assert_close for tensors of several GB: the same whole-tensor rule, max|x - x_ref| over every
    element against tol * rms(x_ref) over every element, evaluated a block of leading-axis rows at a
    time (after flattening the leading axes) so that no full-size temporary is made."""
    g = got.detach().to("cpu")
    assert tuple(g.shape) == ref.shape, (name, tuple(g.shape), ref.shape)
    lead = int(np.prod(ref.shape[:2])) if ref.ndim > 2 else ref.shape[0]
    gf = g.reshape(lead, -1)
    rf = ref.reshape(lead, -1)
    max_err, sum_sq, count = 0.0, 0.0, 0
    for a in range(0, lead, rows):
        gb = gf[a:a + rows].to(torch.float64).numpy()
        rb = rf[a:a + rows]
        assert np.all(np.isfinite(gb)), f"{name}: non-finite values in rows {a}..{a + rows}"
        max_err = max(max_err, float(np.max(np.abs(gb - rb))) if gb.size else 0.0)
        sum_sq += float(np.sum(np.square(rb)))
        count += rb.size
    rms = np.sqrt(sum_sq / max(count, 1))
    e = max_err / max(rms, 1e-300)
    print(f"  {name}: max err {e:.3e} x rms (tol {tol:g}, {count} elements)", flush=True)
    assert e <= tol, f"{name}: max|err| = {e:.3e} * rms > {tol:g} * rms"
    return e


def assert_close(name: str, got, ref: np.ndarray, tol: float) -> float:
    g = got.detach().to("cpu", torch.float64).numpy() if isinstance(got, torch.Tensor) else got
    assert g.shape == ref.shape, (name, g.shape, ref.shape)
    assert np.all(np.isfinite(g[~np.isnan(ref)])), f"{name}: non-finite values"
    e = rel_err(g, ref)
    print(f"  {name}: max err {e:.3e} x rms (tol {tol:g})", flush=True)
    assert e <= tol, f"{name}: max|err| = {e:.3e} * rms > {tol:g} * rms"
    return e
