"""GPU parity of the gating entry points (gates formed inside the kernels from the raw projections)
against the oracle: the oracle's fp64 gate formula applied to the very a, b values the GPU receives,
then its token-by-token recurrence.  Same tolerance rule as the other parity tests."""
import numpy as np
import pytest
import torch

from gated_deltanet_delta_amd import gdn_chunk_fwd_gating, gdn_recurrent_step_gating, synth
from helpers import assert_close, tol_for
from oracle import oracle as O

pytestmark = pytest.mark.gpu

WL = synth.WORKLOADS


def with_dims(wl, **kw):
    d = dict(wl.__dict__)
    d.update(kw)
    return synth.Workload(**d)


def raw_gates(x, gate_dtype, seed):
    """a, b in the gate dtype, A_log from the draw, and a nonzero dt_bias (so that its add is
    exercised; the workloads themselves use dt_bias = 0)."""
    raw = x["raw"]
    a = torch.from_numpy(raw["a"]).to(gate_dtype)
    b = torch.from_numpy(raw["b"]).to(gate_dtype)
    A_log = torch.from_numpy(np.asarray(raw["A_log"], dtype=np.float32))
    dt_bias = torch.from_numpy(
        (0.5 * np.random.default_rng(seed).standard_normal(A_log.shape[0])).astype(np.float32))
    return a, b, A_log, dt_bias


def oracle_gated(x, a, b, A_log, dt_bias):
    f = synth.to_f64
    g, beta = O.gates(f(a), f(b), f(A_log), f(dt_bias))
    cu = None if x.get("cu_seqlens") is None else x["cu_seqlens"].numpy()
    return O.forward(f(x["q"]), f(x["k"]), f(x["v"]), g, beta, f(x.get("initial_state")), cu)


def run_gated_chunk(x, a, b, A_log, dt_bias):
    dev = "cuda"
    s0 = x.get("initial_state")
    cu = x.get("cu_seqlens")
    o, fs = gdn_chunk_fwd_gating(x["q"].to(dev), x["k"].to(dev), x["v"].to(dev), a.to(dev), b.to(dev),
                                 A_log.to(dev), dt_bias.to(dev), None if s0 is None else s0.to(dev),
                                 None if cu is None else cu.to(dev))
    torch.cuda.synchronize()
    return o, fs


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_gating_prefill_ragged(dtype):
    wl = with_dims(WL["prefill"], Hk=2, Hv=4, dtype=dtype, gate_dtype=dtype, init_state=True)
    x = synth.make(wl, T=300, seed=11)
    a, b, A_log, dt_bias = raw_gates(x, dtype, 12)
    o, fs = run_gated_chunk(x, a, b, A_log, dt_bias)
    o_ref, s_ref = oracle_gated(x, a, b, A_log, dt_bias)
    assert_close(f"gating prefill {dtype} o", o, o_ref, tol_for(dtype))
    assert_close(f"gating prefill {dtype} final_state", fs, s_ref, tol_for(dtype))


def test_gating_packed_sequences():
    wl = with_dims(WL["varlen"], Hk=2, Hv=4, n_seqs=5)
    x = synth.make(wl, lengths=np.array([64, 1, 200, 0, 129]), seed=13)
    a, b, A_log, dt_bias = raw_gates(x, torch.bfloat16, 14)
    o, fs = run_gated_chunk(x, a, b, A_log, dt_bias)
    o_ref, s_ref = oracle_gated(x, a, b, A_log, dt_bias)
    assert_close("gating packed o", o, o_ref, tol_for(torch.bfloat16))
    assert_close("gating packed final_state", fs, s_ref, tol_for(torch.bfloat16))


def test_gating_large_pre_activations():
    """softplus and sigmoid far into their tails: a + dt_bias of +-40 (softplus equal to its argument
    or to exp of it, sigmoid saturated) must give finite gates and the oracle's result."""
    wl = with_dims(WL["prefill"], Hk=1, Hv=2, dtype=torch.float32, gate_dtype=torch.float32,
                   init_state=True)
    x = synth.make(wl, T=130, seed=15)
    raw = x["raw"]
    sign = np.where(np.arange(raw["a"].size).reshape(raw["a"].shape) % 2 == 0, 1.0, -1.0)
    a = torch.from_numpy((40.0 * sign).astype(np.float32))
    b = torch.from_numpy((40.0 * sign).astype(np.float32))
    A_log = torch.tensor([-3.0, 0.5], dtype=torch.float32)
    dt_bias = torch.tensor([0.0, -0.25], dtype=torch.float32)
    o, fs = run_gated_chunk(x, a, b, A_log, dt_bias)
    o_ref, s_ref = oracle_gated(x, a, b, A_log, dt_bias)
    assert_close("gating tails o", o, o_ref, tol_for(torch.float32))
    assert_close("gating tails final_state", fs, s_ref, tol_for(torch.float32))


def test_gating_decode_steps():
    wd = with_dims(WL["decode"], B=8)
    x0 = synth.make(wd)
    A_log_np = x0["raw"]["A_log"]
    state = x0["initial_state"].clone()
    dev_state = state.cuda()
    f = synth.to_f64
    ref_state = f(state)
    for step in range(4):
        x = x0 if step == 0 else synth.decode_step(wd, step, A_log_np)
        a, b, A_log, dt_bias = raw_gates(x, wd.gate_dtype, 16)
        o, _ = gdn_recurrent_step_gating(x["q"].cuda(), x["k"].cuda(), x["v"].cuda(), a.cuda(), b.cuda(),
                                         A_log.cuda(), dt_bias.cuda(), dev_state)
        g, beta = O.gates(f(a), f(b), f(A_log), f(dt_bias))
        o_ref, ref_state = O.forward(f(x["q"]), f(x["k"]), f(x["v"]), g, beta, ref_state, None)
        torch.cuda.synchronize()
        assert_close(f"gating decode step {step} o", o, o_ref, tol_for(wd.dtype))
    assert_close("gating decode state", dev_state, ref_state, tol_for(wd.dtype))
