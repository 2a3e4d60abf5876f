"""GPU parity of the q/k L2 normalisation option (gdn_chunk_fwd_ex / gdn_recurrent_step_ex with
qk_l2norm) against the oracle: q and k are handed over at arbitrary lengths, the oracle normalises
the very values the GPU receives (fp64, x / sqrt(|x|^2 + 1e-6)) and runs its token-by-token
recurrence.  Same tolerance rule as the other parity tests.  With the option off, the option-taking
calls are checked to give exactly the plain calls' results."""
import numpy as np
import pytest
import torch

from gated_deltanet_delta_amd import (gdn_chunk_fwd, gdn_chunk_fwd_ex, gdn_recurrent_step,
                                      gdn_recurrent_step_ex, synth)
from helpers import assert_close, tol_for
from oracle import oracle as O

pytestmark = pytest.mark.gpu

WL = synth.WORKLOADS
f64 = synth.to_f64


def with_dims(wl, **kw):
    d = dict(wl.__dict__)
    d.update(kw)
    return synth.Workload(**d)


def unnormalise(x, seed, zero_rows=True):
    """Rescale every q and k head vector by its own factor, log-uniform in [0.05, 20], and round back
    to the input dtype; one key row and one query row of the first sequence are zeroed (they
    normalise to zero through eps)."""
    rng = np.random.default_rng(seed)
    for key in ("q", "k"):
        t = x[key]
        s = np.exp(rng.uniform(np.log(0.05), np.log(20.0), size=tuple(t.shape[:-1]) + (1,)))
        t = (t.float() * torch.from_numpy(s.astype(np.float32))).to(t.dtype)
        if zero_rows and t.shape[1] > 5:
            t[0, 3 if key == "k" else 5] = 0
        x[key] = t
    return x


def oracle_l2(x, g=None, beta=None, s0=None):
    cu = None if x.get("cu_seqlens") is None else x["cu_seqlens"].numpy()
    g = f64(x["g"]) if g is None else g
    beta = f64(x["beta"]) if beta is None else beta
    s0 = f64(x.get("initial_state")) if s0 is None else s0
    return O.forward(O.l2norm(f64(x["q"])), O.l2norm(f64(x["k"])), f64(x["v"]), g, beta, s0, cu)


def run_ex(x, **kw):
    dev = "cuda"
    s0 = x.get("initial_state")
    cu = x.get("cu_seqlens")
    o, fs = gdn_chunk_fwd_ex(x["q"].to(dev), x["k"].to(dev), x["v"].to(dev), x["g"].to(dev),
                             x["beta"].to(dev), initial_state=None if s0 is None else s0.to(dev),
                             cu_seqlens=None if cu is None else cu.to(dev), **kw)
    torch.cuda.synchronize()
    return o, fs


@pytest.mark.parametrize("dtype,dk,dv", [(torch.bfloat16, 128, 128), (torch.bfloat16, 128, 64),
                                         (torch.bfloat16, 64, 64), (torch.bfloat16, 64, 128),
                                         (torch.float32, 128, 128)])
def test_l2norm_prefill_ragged(dtype, dk, dv):
    wl = with_dims(WL["prefill"], Hk=2, Hv=4, dk=dk, dv=dv, dtype=dtype, gate_dtype=dtype, init_state=True)
    x = unnormalise(synth.make(wl, T=300, seed=61), 62)
    o, fs = run_ex(x, qk_l2norm=True)
    o_ref, s_ref = oracle_l2(x)
    assert_close(f"l2norm prefill {dtype} dk={dk} dv={dv} o", o, o_ref, tol_for(dtype))
    assert_close(f"l2norm prefill {dtype} dk={dk} dv={dv} final_state", fs, s_ref, tol_for(dtype))


@pytest.mark.parametrize("scale", [1e-3, 3e3])
def test_l2norm_keys_far_from_unit_length(scale):
    """Raw q and k with norms around 1e-3 and 3e3 (|k|^2 up to ~1e7): with the option the rule sees
    unit vectors, so the result must match the oracle at the usual bound whatever the raw scale."""
    wl = with_dims(WL["prefill"], Hk=2, Hv=4, init_state=True)
    x = synth.make(wl, T=200, seed=64)
    for key in ("q", "k"):
        x[key] = (x[key].float() * scale).to(x[key].dtype)
    o, fs = run_ex(x, qk_l2norm=True)
    o_ref, s_ref = oracle_l2(x)
    assert_close(f"l2norm |k| ~ {scale:g} o", o, o_ref, tol_for(wl.dtype))
    assert_close(f"l2norm |k| ~ {scale:g} final_state", fs, s_ref, tol_for(wl.dtype))


def test_l2norm_with_gating_pool_and_packed_sequences():
    """Every option at once: packed ragged sequences (an empty one, one of a single token), raw gate
    projections, a state pool with a padding row, and the normalisation."""
    wl = with_dims(WL["varlen"], Hk=2, Hv=4, n_seqs=5)
    lengths = np.array([64, 1, 200, 0, 129])
    x = unnormalise(synth.make(wl, lengths=lengths, seed=63), 64)
    raw = x["raw"]
    a = torch.from_numpy(raw["a"]).to(torch.bfloat16)
    b = torch.from_numpy(raw["b"]).to(torch.bfloat16)
    A_log = torch.from_numpy(np.asarray(raw["A_log"], dtype=np.float32))
    dt_bias = torch.from_numpy((0.3 * np.random.default_rng(65).standard_normal(wl.Hv)).astype(np.float32))
    num_slots = 7
    pool = torch.from_numpy((0.02 * np.random.default_rng(66).standard_normal(
        (num_slots, wl.Hv, wl.dk, wl.dv))).astype(np.float32))
    idx = torch.tensor([4, 0, -1, 6, 2], dtype=torch.int32)
    dev = "cuda"
    pool_d = pool.to(dev)
    o, _ = gdn_chunk_fwd_ex(x["q"].to(dev), x["k"].to(dev), x["v"].to(dev), a.to(dev), b.to(dev),
                            A_log=A_log.to(dev), dt_bias=dt_bias.to(dev), initial_state=pool_d,
                            state_indices=idx.to(dev), cu_seqlens=x["cu_seqlens"].to(dev), qk_l2norm=True)
    torch.cuda.synchronize()
    g, beta = O.gates(f64(a), f64(b), f64(A_log), f64(dt_bias))
    s0 = np.zeros((len(lengths), wl.Hv, wl.dk, wl.dv))
    for n, i in enumerate(idx.tolist()):
        if 0 <= i < num_slots:
            s0[n] = f64(pool[i])
    o_ref, s_ref = oracle_l2(x, g, beta, s0)
    tol = tol_for(torch.bfloat16)
    assert_close("l2norm all options o", o, o_ref, tol)
    got = pool_d.cpu()
    for n, i in enumerate(idx.tolist()):
        if 0 <= i < num_slots:
            if lengths[n] > 0:
                assert_close(f"l2norm all options slot {i}", got[i], s_ref[n], tol)
            else:
                assert torch.equal(got[i], pool[i]), f"slot {i} of an empty sequence changed"
    for i in set(range(num_slots)) - set(i for i in idx.tolist() if 0 <= i < num_slots):
        assert torch.equal(got[i], pool[i]), f"slot {i} was not named but changed"


def test_l2norm_full_prefill_T4096():
    """The 4096-token, 32-v-head prefill in the benchmark's configuration, q and k unnormalised."""
    x = unnormalise(synth.make(WL["prefill"]), 67)
    o, fs = run_ex(x, qk_l2norm=True)
    o_ref, s_ref = oracle_l2(x)
    assert_close("l2norm full prefill o", o, o_ref, tol_for(torch.bfloat16))
    assert_close("l2norm full prefill final_state", fs, s_ref, tol_for(torch.bfloat16))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_l2norm_decode_steps(dtype):
    """Three one-token decode calls plus one three-token call, each against the oracle run from the
    state the previous call left."""
    wl = with_dims(WL["decode"], B=3, Hk=2, Hv=4, dtype=dtype)
    A_log = np.log(np.random.default_rng(68).uniform(1.0, 16.0, wl.Hv)).astype(np.float32)
    state = torch.from_numpy((0.02 * np.random.default_rng(69).standard_normal(
        (wl.B, wl.Hv, wl.dk, wl.dv))).astype(np.float32))
    dev = "cuda"
    sd = state.to(dev)
    s_ref = f64(state)
    for step in range(3):
        x = unnormalise(synth.decode_step(wl, step, A_log), 70 + step, zero_rows=False)
        o, _ = gdn_recurrent_step_ex(x["q"].to(dev), x["k"].to(dev), x["v"].to(dev), x["g"].to(dev),
                                     x["beta"].to(dev), sd, qk_l2norm=True)
        torch.cuda.synchronize()
        o_ref, s_ref = O.forward(O.l2norm(f64(x["q"])), O.l2norm(f64(x["k"])), f64(x["v"]), f64(x["g"]),
                                 f64(x["beta"]), s_ref)
        assert_close(f"l2norm decode {dtype} step {step} o", o, o_ref, tol_for(dtype))
    assert_close(f"l2norm decode {dtype} state", sd, s_ref, tol_for(dtype))
    # several tokens in one call
    x = unnormalise(synth.make(with_dims(wl, T=3), T=3, seed=73, init_state=False), 74, zero_rows=False)
    o, _ = gdn_recurrent_step_ex(x["q"].to(dev), x["k"].to(dev), x["v"].to(dev), x["g"].to(dev),
                                 x["beta"].to(dev), sd, qk_l2norm=True)
    torch.cuda.synchronize()
    o_ref, s_ref = O.forward(O.l2norm(f64(x["q"])), O.l2norm(f64(x["k"])), f64(x["v"]), f64(x["g"]),
                             f64(x["beta"]), s_ref)
    assert_close(f"l2norm decode {dtype} 3-token o", o, o_ref, tol_for(dtype))
    assert_close(f"l2norm decode {dtype} 3-token state", sd, s_ref, tol_for(dtype))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_ex_without_options_equals_plain_calls_bitwise(dtype):
    wl = with_dims(WL["prefill"], Hk=2, Hv=4, dtype=dtype, gate_dtype=dtype, init_state=True)
    x = synth.make(wl, T=200, seed=75)
    dev = "cuda"
    args = [x[key].to(dev) for key in ("q", "k", "v", "g", "beta")]
    s0 = x["initial_state"].to(dev)
    o1, f1 = gdn_chunk_fwd(*args, s0)
    o2, f2 = gdn_chunk_fwd_ex(*args, initial_state=s0)
    st1 = s0.clone()
    st2 = s0.clone()
    r1, _ = gdn_recurrent_step(*(t[:, :3].contiguous() for t in args), st1)
    r2, _ = gdn_recurrent_step_ex(*(t[:, :3].contiguous() for t in args), st2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)
    assert torch.equal(r1, r2) and torch.equal(st1, st2)
