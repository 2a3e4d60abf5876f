"""GPU parity of the backward pass (gdn_chunk_bwd) against the oracle's fp64 reverse-mode gradients
on the same inputs (the oracle's backward is pinned by finite differences of its forward).

The GPU computes in fp32 from the exact input values, so the bound is the forward's fp32 one:
max |x - x_ref| <= 1e-4 rms(x_ref) per gradient tensor (measured: below 1e-5 everywhere, the
largest on dg, a reverse running sum of up to 64 terms of either sign).  Weak-decay gates keep the
state, and with it the gradients, alive across many chunks."""
import numpy as np
import pytest
import torch

from gated_deltanet_delta_amd import gdn_chunk_bwd, synth
from helpers import assert_close
from oracle import oracle as O

pytestmark = pytest.mark.gpu

WL = synth.WORKLOADS
TOL = 1e-4
NAMES = ("dq", "dk", "dv", "dg", "dbeta", "d_initial")
f64 = synth.to_f64


def with_dims(wl, **kw):
    d = dict(wl.__dict__)
    d.update(kw)
    return synth.Workload(**d)


def grads_of_outputs(x, seed, with_final=True):
    """Seeded gradients of a loss with respect to o (and the final state)."""
    rng = np.random.default_rng(seed)
    B, T, Hv = x["g"].shape
    dv = x["v"].shape[-1]
    dk = x["q"].shape[-1]
    N = B if x.get("cu_seqlens") is None else x["cu_seqlens"].numel() - 1
    d_o = torch.from_numpy(rng.standard_normal((B, T, Hv, dv)).astype(np.float32))
    d_final = torch.from_numpy(rng.standard_normal((N, Hv, dk, dv)).astype(np.float32)) if with_final else None
    return d_o, d_final


def check(x, d_o, d_final, what, tol=TOL):
    dev = "cuda"
    s0 = x.get("initial_state")
    cu = x.get("cu_seqlens")
    got = gdn_chunk_bwd(x["q"].to(dev), x["k"].to(dev), x["v"].to(dev), x["g"].to(dev), x["beta"].to(dev),
                        d_o.to(dev), None if s0 is None else s0.to(dev),
                        None if d_final is None else d_final.to(dev), None if cu is None else cu.to(dev))
    torch.cuda.synchronize()
    ref = O.backward(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["g"]), f64(x["beta"]), f64(d_o),
                     f64(s0), f64(d_final), None if cu is None else cu.numpy())
    for name, a, b in zip(NAMES, got, ref):
        if b.size == 0:
            assert a.numel() == 0, name
            continue
        assert_close(f"{what} {name}", a, b, tol)
    return got


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_backward_weak_decay(dtype):
    wl = with_dims(WL["prefill"], B=2, Hk=2, Hv=4, dtype=dtype, gate_dtype=dtype, init_state=True)
    A_log = np.log(np.linspace(0.1, 0.9, wl.Hv)).astype(np.float32)
    x = synth.make(wl, T=150, seed=81, A_log=A_log)          # three chunks, the last one ragged
    d_o, d_final = grads_of_outputs(x, 82)
    check(x, d_o, d_final, f"bwd {dtype}")


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 64), (64, 128)])
def test_backward_head_sizes(dk, dv):
    wl = with_dims(WL["prefill"], Hk=1, Hv=2, dk=dk, dv=dv, init_state=True)
    A_log = np.log(np.linspace(0.1, 0.9, wl.Hv)).astype(np.float32)
    x = synth.make(wl, T=97, seed=83, A_log=A_log)
    d_o, d_final = grads_of_outputs(x, 84)
    check(x, d_o, d_final, f"bwd dk={dk} dv={dv}")


@pytest.mark.parametrize("G", [1, 3, 4])
def test_backward_head_groupings(G):
    """G v-heads per q/k head other than 2: the per-chunk kernels loop over a q/k head's v-heads and
    sum dq, dk over them."""
    wl = with_dims(WL["prefill"], Hk=2, Hv=2 * G, init_state=True)
    A_log = np.log(np.linspace(0.1, 0.9, wl.Hv)).astype(np.float32)
    x = synth.make(wl, T=130, seed=92 + G, A_log=A_log)
    d_o, d_final = grads_of_outputs(x, 95 + G)
    check(x, d_o, d_final, f"bwd G={G}")


def test_backward_packed_sequences():
    """Packed ragged sequences (empty ones among them, one of a single token), no gradient on the
    final state, the workloads' own strong-decay gates."""
    wl = with_dims(WL["varlen"], Hk=2, Hv=4, n_seqs=6)
    x = synth.make(wl, lengths=np.array([64, 0, 1, 200, 0, 129]), seed=85)
    d_o, _ = grads_of_outputs(x, 86, with_final=False)
    check(x, d_o, None, "bwd packed")


def test_backward_no_tokens_passes_the_state_gradient_through():
    wl = with_dims(WL["prefill"], B=2, Hk=1, Hv=2, dk=64, dv=64, init_state=True)
    x = synth.make(wl, T=0, seed=87)
    d_o, d_final = grads_of_outputs(x, 88)
    got = check(x, d_o, d_final, "bwd T=0")
    assert torch.equal(got[5].cpu(), d_final)


def test_backward_full_prefill_T4096():
    """The 4096-token, 32-v-head prefill with a weak decay and a carried initial state."""
    wl = with_dims(WL["prefill"], init_state=True)
    A_log = np.log(np.random.default_rng(89).uniform(0.01, 0.05, wl.Hv)).astype(np.float32)
    x = synth.make(wl, seed=90, A_log=A_log)
    d_o, d_final = grads_of_outputs(x, 91)
    check(x, d_o, d_final, "bwd full prefill")
