"""Seeded synthetic workloads for the gated delta rule (inputs only; no part of the rule itself).

The tests, the smoke check and the benchmark draw their inputs here, and both sides of every parity
check (the HIP library and the CPU oracle) receive the very same values.  Nothing here evaluates the
state recurrence.

Workloads (Qwen3-Next Gated DeltaNet shapes: 16 q/k heads, 32 v heads, head dim 128):

  ``tiny``     B=1, T=256, 2 heads, d=64, all fp32, zero initial state.
  ``prefill``  B=1, T=4096, Hk=16, Hv=32, d=128, bf16 q/k/v/g/beta, zero initial state.
  ``long``     as ``prefill`` with T=32768 and an initial state ~ N(0, 0.02^2).
  ``decode``   B=256 sequences, Hk=16, Hv=32, d=128, state ~ N(0, 0.02^2) (512 MiB fp32), 128 one-token
               steps with fresh bf16 q/k/v and fp32 g/beta per step.
  ``varlen``   64 packed sequences, lengths ~ U{300..8192} (not multiples of 64), per-sequence initial
               states ~ N(0, 0.02^2), bf16 inputs.

Value distributions, drawn in fp32 with NumPy's PCG64 (``default_rng(seed)``) in this order: (lengths,
``varlen`` only), q, k, v, b, A_log, a, initial state.

  q, k ~ N(0,1), then scaled to unit L2 norm per (token, head) vector;  v ~ N(0,1);
  b ~ N(0,1), beta = sigmoid(b);  A_log = log U(1,16) per head;  a ~ N(0,1) per (token, head);
  dt_bias = 0;  g = -exp(A_log) * softplus(a + dt_bias)   (the log-decay distribution the workloads
  specify; the oracle evaluates the same gate formula independently in fp64 and the tests pin one
  against the other).

Values are then rounded to the workload's dtype with round-to-nearest-even (torch's cast).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    Hk: int
    Hv: int
    dk: int
    dv: int
    dtype: torch.dtype          # q, k, v
    gate_dtype: torch.dtype     # g, beta
    init_state: bool            # False: zero (NULL) initial state
    seed: int
    n_seqs: int = 0             # >0: packed varlen with this many sequences (B == 1)
    len_range: tuple = (0, 0)   # inclusive length range for packed sequences
    steps: int = 0              # >0: decode workload with this many one-token steps
    notes: str = field(default="", compare=False)


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 1, 256, 2, 2, 64, 64, torch.float32, torch.float32, False, 0,
                     notes="single fp32 sequence, chunk-aligned, parity at 1e-4 rms"),
    "prefill": Workload("prefill", 1, 4096, 16, 32, 128, 128, torch.bfloat16, torch.bfloat16, False, 1,
                        notes="Qwen3-Next-shaped prefill"),
    "long": Workload("long", 1, 32768, 16, 32, 128, 128, torch.bfloat16, torch.bfloat16, True, 2,
                     notes="long-context prefill with a carried state"),
    "decode": Workload("decode", 256, 1, 16, 32, 128, 128, torch.bfloat16, torch.float32, True, 3,
                       steps=128, notes="batched decode, 2 MiB of state per sequence"),
    "varlen": Workload("varlen", 1, 0, 16, 32, 128, 128, torch.bfloat16, torch.bfloat16, True, 4,
                       n_seqs=64, len_range=(300, 8192), notes="packed variable-length prefill"),
}


def _unit_rows(x: np.ndarray) -> np.ndarray:
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def draw(rng: np.random.Generator, B: int, T: int, Hk: int, Hv: int, dk: int, dv: int,
         init_state: bool, N: int, A_log: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Raw fp32 draws for one batch in the fixed order q, k, v, b, A_log, a, initial state."""
    f32 = np.float32
    q = _unit_rows(rng.standard_normal((B, T, Hk, dk), dtype=f32))
    k = _unit_rows(rng.standard_normal((B, T, Hk, dk), dtype=f32))
    v = rng.standard_normal((B, T, Hv, dv), dtype=f32)
    b = rng.standard_normal((B, T, Hv), dtype=f32)
    if A_log is None:
        A_log = np.log(rng.uniform(1.0, 16.0, size=Hv)).astype(f32)
    a = rng.standard_normal((B, T, Hv), dtype=f32)
    dt_bias = np.zeros(Hv, dtype=f32)
    s0 = (0.02 * rng.standard_normal((N, Hv, dk, dv), dtype=f32)) if init_state else None
    beta = (1.0 / (1.0 + np.exp(-b.astype(np.float64)))).astype(f32)
    g = (-np.exp(A_log.astype(np.float64)) * _softplus(a.astype(np.float64) + dt_bias)).astype(f32)
    return dict(q=q, k=k, v=v, b=b, A_log=A_log, a=a, dt_bias=dt_bias, g=g, beta=beta, s0=s0)


def _lengths(rng: np.random.Generator, wl: Workload) -> np.ndarray:
    lo, hi = wl.len_range
    return rng.integers(lo, hi + 1, size=wl.n_seqs).astype(np.int64)


def make(wl: Workload, T: Optional[int] = None, seed: Optional[int] = None,
         lengths: Optional[np.ndarray] = None, A_log: Optional[np.ndarray] = None,
         init_state: Optional[bool] = None) -> Dict[str, object]:
    """Inputs for one prefill call (or the first decode step) as CPU torch tensors.

    Returns q, k, v (wl.dtype), g, beta (wl.gate_dtype), initial_state (fp32 or None), cu_seqlens
    (int32 or None), plus the raw fp32 draws under ``raw``.  ``T``, ``seed``, ``lengths`` and
    ``A_log`` override the workload's defaults (for reduced-size parity cases and for custom decay
    ranges); ``init_state`` overrides whether an initial state is drawn.
    """
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    cu = None
    if wl.n_seqs:
        lens = _lengths(rng, wl) if lengths is None else np.asarray(lengths, dtype=np.int64)
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        TT, N = int(cu[-1]), len(lens)
    elif lengths is not None:
        lens = np.asarray(lengths, dtype=np.int64)
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        TT, N = int(cu[-1]), len(lens)
    else:
        TT, N = (wl.T if T is None else T), wl.B
    B = 1 if cu is not None else wl.B
    raw = draw(rng, B, TT, wl.Hk, wl.Hv, wl.dk, wl.dv,
               wl.init_state if init_state is None else init_state, N, A_log)
    out = dict(
        q=torch.from_numpy(raw["q"]).to(wl.dtype),
        k=torch.from_numpy(raw["k"]).to(wl.dtype),
        v=torch.from_numpy(raw["v"]).to(wl.dtype),
        g=torch.from_numpy(raw["g"]).to(wl.gate_dtype),
        beta=torch.from_numpy(raw["beta"]).to(wl.gate_dtype),
        initial_state=None if raw["s0"] is None else torch.from_numpy(raw["s0"]),
        cu_seqlens=None if cu is None else torch.from_numpy(cu),
        raw=raw,
    )
    return out


def decode_step(wl: Workload, step: int, A_log: np.ndarray) -> Dict[str, torch.Tensor]:
    """Fresh one-token inputs for decode step ``step`` (seeded by (workload seed, step))."""
    rng = np.random.default_rng([wl.seed, step + 1])
    raw = draw(rng, wl.B, 1, wl.Hk, wl.Hv, wl.dk, wl.dv, False, wl.B, A_log)
    return dict(
        q=torch.from_numpy(raw["q"]).to(wl.dtype),
        k=torch.from_numpy(raw["k"]).to(wl.dtype),
        v=torch.from_numpy(raw["v"]).to(wl.dtype),
        g=torch.from_numpy(raw["g"]).to(wl.gate_dtype),
        beta=torch.from_numpy(raw["beta"]).to(wl.gate_dtype),
        raw=raw,
    )


def to_f64(t: Optional[torch.Tensor]) -> Optional[np.ndarray]:
    """Exact fp64 copy of a CPU tensor (bf16 and fp32 both widen without rounding)."""
    return None if t is None else t.detach().to("cpu", torch.float64).numpy()
