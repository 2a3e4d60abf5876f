"""GPU parity of the state-pool entry points (continuous batching) against the oracle: each
sequence or batch row starts from its named slot of the pool and writes its final state back
there; padding rows (indices outside the pool) and slots no row names are checked to be left alone
bit for bit."""
import numpy as np
import pytest
import torch

from gated_deltanet_delta_amd import gdn_chunk_fwd_indexed, gdn_recurrent_step_indexed, synth
from helpers import assert_close, tol_for
from oracle import oracle as O

pytestmark = pytest.mark.gpu

WL = synth.WORKLOADS


def with_dims(wl, **kw):
    d = dict(wl.__dict__)
    d.update(kw)
    return synth.Workload(**d)


def pool_of(num_slots, Hv, dk, dv, seed):
    rng = np.random.default_rng(seed)
    return torch.from_numpy((0.02 * rng.standard_normal((num_slots, Hv, dk, dv))).astype(np.float32))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_indexed_prefill_packed(dtype):
    wl = with_dims(WL["varlen"], Hk=2, Hv=4, n_seqs=5, dtype=dtype, gate_dtype=dtype, init_state=False)
    lengths = np.array([70, 1, 0, 130, 64])
    x = synth.make(wl, lengths=lengths, seed=21)
    num_slots = 9
    pool = pool_of(num_slots, wl.Hv, wl.dk, wl.dv, 22)
    idx = torch.tensor([5, 2, 8, -1, 9], dtype=torch.int32)   # -1 and 9: padding rows
    dev = "cuda"
    pool_d = pool.to(dev)
    o = gdn_chunk_fwd_indexed(x["q"].to(dev), x["k"].to(dev), x["v"].to(dev), x["g"].to(dev),
                              x["beta"].to(dev), pool_d, idx.to(dev), x["cu_seqlens"].to(dev))
    torch.cuda.synchronize()
    f = synth.to_f64
    # the oracle's initial states: the named slots, zero for padding rows
    s0 = np.zeros((len(lengths), wl.Hv, wl.dk, wl.dv))
    for n, i in enumerate(idx.tolist()):
        if 0 <= i < num_slots:
            s0[n] = f(pool[i])
    o_ref, s_ref = O.forward(f(x["q"]), f(x["k"]), f(x["v"]), f(x["g"]), f(x["beta"]), s0,
                             x["cu_seqlens"].numpy())
    tol = tol_for(dtype)
    assert_close(f"indexed prefill {dtype} o", o, o_ref, tol)
    got = pool_d.cpu()
    named = [i for i in idx.tolist() if 0 <= i < num_slots]
    for n, i in enumerate(idx.tolist()):
        if 0 <= i < num_slots:
            assert_close(f"indexed prefill {dtype} slot {i}", got[i], s_ref[n], tol)
    for i in range(num_slots):
        if i not in named:
            assert torch.equal(got[i], pool[i]), f"slot {i} was not named but changed"


def test_indexed_decode_steps():
    wd = with_dims(WL["decode"], B=6)
    x0 = synth.make(wd)
    A_log = x0["raw"]["A_log"]
    num_slots = 12
    pool = pool_of(num_slots, wd.Hv, wd.dk, wd.dv, 23)
    idx = torch.tensor([3, 0, 11, -1, 7, 12], dtype=torch.int32)   # rows 3 and 5 are padding
    pool_d = pool.cuda()
    f = synth.to_f64
    ref = {i: f(pool[i]) for i in idx.tolist() if 0 <= i < num_slots}
    for step in range(3):
        x = x0 if step == 0 else synth.decode_step(wd, step, A_log)
        o = gdn_recurrent_step_indexed(x["q"].cuda(), x["k"].cuda(), x["v"].cuda(), x["g"].cuda(),
                                       x["beta"].cuda(), pool_d, idx.cuda())
        torch.cuda.synchronize()
        for b, i in enumerate(idx.tolist()):
            if 0 <= i < num_slots:
                o_ref, s_ref = O.forward(f(x["q"][b:b + 1]), f(x["k"][b:b + 1]), f(x["v"][b:b + 1]),
                                         f(x["g"][b:b + 1]), f(x["beta"][b:b + 1]), ref[i][None], None)
                ref[i] = s_ref[0]
                assert_close(f"indexed decode step {step} row {b} o", o[b:b + 1], o_ref, tol_for(wd.dtype))
            else:
                assert torch.all(o[b] == 0), f"padding row {b} has nonzero outputs"
    got = pool_d.cpu()
    for i in range(num_slots):
        if i in ref:
            assert_close(f"indexed decode slot {i}", got[i], ref[i], tol_for(wd.dtype))
        else:
            assert torch.equal(got[i], pool[i]), f"slot {i} was not named but changed"
