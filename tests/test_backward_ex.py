"""GPU parity of the backward pass with the forward's input options (gdn_chunk_bwd_ex: gates formed
from the raw projections a, b with A_log and dt_bias; q/k L2 normalisation; a state pool) against
the oracle's fp64 gradients of the composed layer call (``oracle.backward_ex``, itself pinned by
central differences of the composed forward).

Same bound as the plain backward: max |x - x_ref| <= 1e-4 rms(x_ref) per gradient tensor.  Weak-decay
gates keep the state, and with it the gradients, alive across chunks; q and k are handed over at
arbitrary lengths so that the normalisation's gradient is not the identity."""
import numpy as np
import pytest
import torch

from gated_deltanet_delta_amd import gdn_chunk_bwd, gdn_chunk_bwd_ex, synth
from helpers import assert_close
from oracle import oracle as O

pytestmark = pytest.mark.gpu

WL = synth.WORKLOADS
TOL = 1e-4
NAMES = ("dq", "dk", "dv", "da", "db", "dA_log", "ddt_bias", "d_initial")
f64 = synth.to_f64
DEV = "cuda"


def with_dims(wl, **kw):
    d = dict(wl.__dict__)
    d.update(kw)
    return synth.Workload(**d)


def unnormalise(x, seed):
    """Rescale every q and k head vector by its own log-uniform factor in [0.05, 20] (rounded back to
    the input dtype) and zero one key row, which normalises to zero through eps."""
    rng = np.random.default_rng(seed)
    for key in ("q", "k"):
        t = x[key]
        s = np.exp(rng.uniform(np.log(0.05), np.log(20.0), size=tuple(t.shape[:-1]) + (1,)))
        t = (t.float() * torch.from_numpy(s.astype(np.float32))).to(t.dtype)
        if key == "k" and t.shape[1] > 3:
            t[0, 3] = 0
        x[key] = t
    return x


def raw_gates(x, dtype, seed):
    """The raw projections a, b the workload's gates were formed from, in ``dtype``, with A_log and a
    non-zero dt_bias."""
    raw = x["raw"]
    a = torch.from_numpy(raw["a"]).to(dtype)
    b = torch.from_numpy(raw["b"]).to(dtype)
    A_log = torch.from_numpy(np.asarray(raw["A_log"], dtype=np.float32))
    Hv = A_log.numel()
    dt_bias = torch.from_numpy((0.3 * np.random.default_rng(seed).standard_normal(Hv)).astype(np.float32))
    return a, b, A_log, dt_bias


def output_grads(shape_o, shape_s, seed):
    rng = np.random.default_rng(seed)
    d_o = torch.from_numpy(rng.standard_normal(shape_o).astype(np.float32))
    d_final = None if shape_s is None else torch.from_numpy(rng.standard_normal(shape_s).astype(np.float32))
    return d_o, d_final


def gpu(t):
    return None if t is None else t.to(DEV)


def run(x, a, b, A_log, dt_bias, d_o, d_final, s0, idx=None, qk_l2norm=False):
    got = gdn_chunk_bwd_ex(gpu(x["q"]), gpu(x["k"]), gpu(x["v"]), gpu(a), gpu(b), gpu(d_o), A_log=gpu(A_log),
                           dt_bias=gpu(dt_bias), initial_state=gpu(s0), state_indices=gpu(idx),
                           d_final=gpu(d_final), cu_seqlens=gpu(x.get("cu_seqlens")), qk_l2norm=qk_l2norm)
    torch.cuda.synchronize()
    return got


def reference(x, a, b, A_log, dt_bias, d_o, d_final, s0, qk_l2norm):
    """Oracle gradients of the composed call (without raw gates, A_log None, a and b are g and beta)."""
    cu = None if x.get("cu_seqlens") is None else x["cu_seqlens"].numpy()
    return O.backward_ex(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(a), f64(b), f64(A_log), f64(dt_bias),
                         f64(d_o), s0, f64(d_final), cu, qk_l2norm=qk_l2norm)


def compare(what, got, ref, tol=TOL):
    for name, a, r in zip(NAMES, got, ref):
        if r is None:
            assert a is None, name
            continue
        assert_close(f"{what} {name}", a, r, tol)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_backward_ex_raw_gates_and_l2norm(dtype):
    wl = with_dims(WL["prefill"], B=2, Hk=2, Hv=4, dtype=dtype, gate_dtype=dtype, init_state=True)
    A_log = np.log(np.linspace(0.1, 0.9, wl.Hv)).astype(np.float32)
    x = unnormalise(synth.make(wl, T=150, seed=101, A_log=A_log), 102)   # three chunks, the last ragged
    a, b, A, dt = raw_gates(x, dtype, 103)
    d_o, d_final = output_grads((wl.B, 150, wl.Hv, wl.dv), (wl.B, wl.Hv, wl.dk, wl.dv), 104)
    s0 = x["initial_state"]
    got = run(x, a, b, A, dt, d_o, d_final, s0, qk_l2norm=True)
    compare(f"bwd_ex {dtype}", got, reference(x, a, b, A, dt, d_o, d_final, f64(s0), True))
    again = run(x, a, b, A, dt, d_o, d_final, s0, qk_l2norm=True)
    for name, u, w in zip(NAMES, got, again):
        assert torch.equal(u, w), f"{name} differs between two identical calls"


@pytest.mark.parametrize("option", ["gates", "l2norm"])
def test_backward_ex_one_option(option):
    wl = with_dims(WL["prefill"], Hk=1, Hv=2, dk=64, dv=128, init_state=True)
    A_log = np.log(np.linspace(0.2, 0.6, wl.Hv)).astype(np.float32)
    x = synth.make(wl, T=97, seed=105, A_log=A_log)
    if option == "l2norm":
        x = unnormalise(x, 106)
        a, b, A, dt = x["g"], x["beta"], None, None
    else:
        a, b, A, dt = raw_gates(x, torch.bfloat16, 107)
    d_o, d_final = output_grads((1, 97, wl.Hv, wl.dv), (1, wl.Hv, wl.dk, wl.dv), 108)
    s0 = x["initial_state"]
    l2 = option == "l2norm"
    got = run(x, a, b, A, dt, d_o, d_final, s0, qk_l2norm=l2)
    compare(f"bwd_ex {option}", got, reference(x, a, b, A, dt, d_o, d_final, f64(s0), l2))


def test_backward_ex_without_options_is_the_plain_call_bitwise():
    wl = with_dims(WL["prefill"], Hk=2, Hv=4, init_state=True)
    x = synth.make(wl, T=130, seed=109)
    d_o, d_final = output_grads((1, 130, wl.Hv, wl.dv), (1, wl.Hv, wl.dk, wl.dv), 110)
    s0 = x["initial_state"]
    ex = run(x, x["g"], x["beta"], None, None, d_o, d_final, s0)
    plain = gdn_chunk_bwd(gpu(x["q"]), gpu(x["k"]), gpu(x["v"]), gpu(x["g"]), gpu(x["beta"]), gpu(d_o), gpu(s0),
                          gpu(d_final))
    torch.cuda.synchronize()
    assert ex[5] is None and ex[6] is None
    for name, u, w in zip(("dq", "dk", "dv", "dg", "dbeta"), ex[:5], plain[:5]):
        assert torch.equal(u, w), name
    assert torch.equal(ex[7], plain[5])


def test_backward_ex_every_option_packed_with_a_pool():
    """Packed ragged sequences (an empty one, one of a single token), raw gates, the normalisation and
    a state pool with a padding row: each sequence starts from its slot (zeros for the padding row)
    and d_initial_state is per sequence."""
    wl = with_dims(WL["varlen"], Hk=2, Hv=4, n_seqs=5)
    lengths = np.array([64, 1, 200, 0, 129])
    A_log = np.log(np.linspace(0.1, 0.9, wl.Hv)).astype(np.float32)
    x = unnormalise(synth.make(wl, lengths=lengths, seed=111, A_log=A_log), 112)
    a, b, A, dt = raw_gates(x, torch.bfloat16, 113)
    num_slots = 7
    pool = torch.from_numpy((0.02 * np.random.default_rng(114).standard_normal(
        (num_slots, wl.Hv, wl.dk, wl.dv))).astype(np.float32))
    idx = torch.tensor([4, 0, -1, 6, 2], dtype=torch.int32)
    T = int(lengths.sum())
    d_o, d_final = output_grads((1, T, wl.Hv, wl.dv), (len(lengths), wl.Hv, wl.dk, wl.dv), 115)
    got = run(x, a, b, A, dt, d_o, d_final, pool, idx=idx, qk_l2norm=True)
    s0 = np.zeros((len(lengths), wl.Hv, wl.dk, wl.dv))
    for n, i in enumerate(idx.tolist()):
        if 0 <= i < num_slots:
            s0[n] = f64(pool[i])
    compare("bwd_ex packed pool", got, reference(x, a, b, A, dt, d_o, d_final, s0, True))


def test_backward_ex_full_prefill_T4096():
    """The 4096-token, 32-v-head prefill through every option (bf16 raw gates and q/k normalisation),
    a weak decay and a carried initial state."""
    wl = with_dims(WL["prefill"], init_state=True)
    A_log = np.log(np.random.default_rng(116).uniform(0.01, 0.05, wl.Hv)).astype(np.float32)
    x = unnormalise(synth.make(wl, seed=117, A_log=A_log), 118)
    a, b, A, dt = raw_gates(x, torch.bfloat16, 119)
    d_o, d_final = output_grads((1, wl.T, wl.Hv, wl.dv), (1, wl.Hv, wl.dk, wl.dv), 120)
    s0 = x["initial_state"]
    got = run(x, a, b, A, dt, d_o, d_final, s0, qk_l2norm=True)
    compare("bwd_ex full prefill", got, reference(x, a, b, A, dt, d_o, d_final, f64(s0), True))


def test_backward_ex_no_tokens():
    """No tokens with every option: the start-state gradient is d_final itself, dA_log and ddt_bias
    are zero, and a padding row of the pool still gets its (passed-through) gradient."""
    wl = with_dims(WL["prefill"], B=2, Hk=1, Hv=2, dk=64, dv=64, init_state=True)
    x = synth.make(wl, T=0, seed=121)
    a, b, A, dt = raw_gates(x, torch.bfloat16, 122)
    pool = torch.from_numpy((0.02 * np.random.default_rng(123).standard_normal(
        (3, wl.Hv, wl.dk, wl.dv))).astype(np.float32))
    idx = torch.tensor([2, -1], dtype=torch.int32)
    d_o, d_final = output_grads((2, 0, wl.Hv, wl.dv), (2, wl.Hv, wl.dk, wl.dv), 124)
    got = run(x, a, b, A, dt, d_o, d_final, pool, idx=idx, qk_l2norm=True)
    assert all(t.numel() == 0 for t in got[:5])
    assert torch.equal(got[5].cpu(), torch.zeros(wl.Hv)) and torch.equal(got[6].cpu(), torch.zeros(wl.Hv))
    assert torch.equal(got[7].cpu(), d_final)
