"""GPU parity: libgdn (through its C ABI) against the fp64 CPU oracle on the same seeded inputs.

Tolerance (whole-tensor): max|x - x_ref| <= 2e-2 * rms(x_ref) for bf16 inputs, 1e-4 * rms(x_ref)
for fp32 inputs, on the outputs o and on the final states.
"""
import numpy as np
import pytest
import torch

from gated_deltanet_delta_amd import gdn_chunk_fwd, gdn_recurrent_step, synth
from helpers import assert_close, assert_close_blocked, oracle_of, to_gpu, tol_for

pytestmark = pytest.mark.gpu

WL = synth.WORKLOADS


def run_chunk(x, initial_state="from_inputs"):
    d = to_gpu(x)
    s0 = d["initial_state"] if isinstance(initial_state, str) else initial_state
    o, fs = gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], s0, d["cu_seqlens"])
    torch.cuda.synchronize()
    return o, fs


def check_chunk(x, tag, tol=None):
    tol = tol_for(x["q"].dtype) if tol is None else tol
    o, fs = run_chunk(x)
    o_ref, s_ref = oracle_of(x)
    assert_close(f"{tag} o", o, o_ref, tol)
    assert_close(f"{tag} final_state", fs, s_ref, tol)


def with_dims(wl, **kw):
    d = dict(wl.__dict__)
    d.update(kw)
    return synth.Workload(**d)


# ---------------------------------------------------------------------------------------------
# small and ragged cases

def test_tiny_fp32_workload():
    check_chunk(synth.make(WL["tiny"]), "tiny")


@pytest.mark.parametrize("T", [1, 17, 64, 65, 200])
def test_prefill_heads_ragged_lengths(T):
    check_chunk(synth.make(WL["prefill"], T=T, seed=100 + T), f"prefill T={T}")


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_head_sizes(dk, dv, dtype):
    wl = with_dims(WL["prefill"], Hk=2, Hv=4, dk=dk, dv=dv, dtype=dtype, gate_dtype=dtype,
                   init_state=True)
    check_chunk(synth.make(wl, T=150, seed=7), f"dk={dk} dv={dv} {dtype}")


@pytest.mark.parametrize("dv", [64, 128])
def test_dk64_bf16_matrix_core_path(dv):
    """Head size 64 on the bf16 matrix-core path: the 4096-token prefill with the Qwen3-Next head
    counts, then packed ragged sequences with a carried state and a weak decay (512 + 4 chunks)."""
    wl = with_dims(WL["prefill"], dk=64, dv=dv)
    check_chunk(synth.make(wl, seed=140 + dv), f"dk=64 dv={dv} T=4096")
    wv = with_dims(WL["varlen"], dk=64, dv=dv, Hk=4, Hv=8, n_seqs=4)
    A_log = np.log(np.linspace(0.1, 0.9, wv.Hv)).astype(np.float32)
    x = synth.make(wv, lengths=np.array([2000, 0, 65, 63]), seed=150 + dv, A_log=A_log)
    check_chunk(x, f"dk=64 dv={dv} packed weak decay")


@pytest.mark.parametrize("G", [1, 3, 4, 8])
def test_head_groupings(G):
    """G v-heads per q/k head other than the Qwen3-Next layout's 2 (each q/k head shared by G
    v-heads, v-head h reading q/k head h // G), packed ragged sequences with a carried state and a
    weak decay, bf16 inputs."""
    wl = with_dims(WL["varlen"], Hk=2, Hv=2 * G, n_seqs=3)
    A_log = np.log(np.linspace(0.1, 0.9, wl.Hv)).astype(np.float32)
    x = synth.make(wl, lengths=np.array([150, 1, 70]), seed=60 + G, A_log=A_log)
    check_chunk(x, f"G={G}")


@pytest.mark.parametrize("G", [1, 3])
def test_head_groupings_decode(G):
    wl = with_dims(WL["decode"], B=3, Hk=2, Hv=2 * G)
    x = synth.make(wl, seed=70 + G)
    o_ref, s_ref = oracle_of(x)
    d = to_gpu(x)
    state = d["initial_state"].clone()
    o, _ = gdn_recurrent_step(d["q"], d["k"], d["v"], d["g"], d["beta"], state)
    torch.cuda.synchronize()
    assert_close(f"decode G={G} o", o, o_ref, tol_for(torch.bfloat16))
    assert_close(f"decode G={G} state", state, s_ref, tol_for(torch.bfloat16))


@pytest.mark.parametrize("decay", ["zero", "linspace", "small"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_weak_decay(decay, dtype):
    """Slow decay keeps the carried state alive across many chunks, so a dropped or mis-scaled
    inter-chunk carry shows up in the final state as well as in o."""
    wl = with_dims(WL["prefill"], Hk=4, Hv=8, dtype=dtype, gate_dtype=dtype, init_state=True)
    Hv = wl.Hv
    A_log = None
    if decay == "linspace":
        A_log = np.log(np.linspace(0.1, 0.9, Hv)).astype(np.float32)
    elif decay == "small":
        A_log = np.log(np.random.default_rng(5).uniform(0.01, 0.05, Hv)).astype(np.float32)
    x = synth.make(wl, T=333, seed=11, A_log=A_log)
    if decay == "zero":
        x["g"] = torch.zeros_like(x["g"])
    check_chunk(x, f"weak decay {decay} {dtype}")


def test_split_and_carry_matches_one_pass():
    wl = with_dims(WL["long"], Hk=4, Hv=8)
    x = synth.make(wl, T=1700, seed=21, A_log=np.log(np.linspace(0.1, 0.9, 8)).astype(np.float32))
    o_ref, s_ref = oracle_of(x)
    d = to_gpu(x)
    T1 = 1000
    part = lambda t, a, b: t[:, a:b].contiguous()  # noqa: E731
    o1, s1 = gdn_chunk_fwd(*(part(d[n], 0, T1) for n in ("q", "k", "v", "g", "beta")), d["initial_state"])
    o2, s2 = gdn_chunk_fwd(*(part(d[n], T1, 1700) for n in ("q", "k", "v", "g", "beta")), s1)
    torch.cuda.synchronize()
    tol = tol_for(x["q"].dtype)
    assert_close("split o", torch.cat([o1, o2], 1), o_ref, tol)
    assert_close("split final_state", s2, s_ref, tol)


def test_packed_sequences_ragged():
    lens = np.array([1, 0, 64, 65, 130, 7, 200, 63])
    wl = with_dims(WL["varlen"], n_seqs=len(lens))
    x = synth.make(wl, lengths=lens, seed=31)
    check_chunk(x, "varlen ragged")
    # zero-length sequence: final state is the initial state, exactly
    _, fs = run_chunk(x)
    assert torch.equal(fs[1].cpu(), x["initial_state"][1])


def test_packed_matches_separate_calls_bitwise_per_sequence():
    lens = np.array([100, 37, 64])
    wl = with_dims(WL["varlen"], n_seqs=3, Hk=2, Hv=4)
    x = synth.make(wl, lengths=lens, seed=41)
    o, fs = run_chunk(x)
    cu = x["cu_seqlens"].numpy()
    for n in range(3):
        a, b = int(cu[n]), int(cu[n + 1])
        y = {key: x[key][:, a:b].contiguous() for key in ("q", "k", "v", "g", "beta")}
        y["initial_state"] = x["initial_state"][n:n + 1].contiguous()
        y["cu_seqlens"] = None
        on, sn = run_chunk(y)
        assert torch.equal(on.cpu(), o[:, a:b].cpu()), n
        assert torch.equal(sn.cpu(), fs[n:n + 1].cpu()), n


@pytest.mark.parametrize("packed", [False, True])
def test_prepare_then_scan_equals_full_call_bitwise(packed):
    # gdn_chunk_fwd is gdn_chunk_fwd_prepare followed by gdn_chunk_fwd_scan on one stream
    if packed:
        wl = with_dims(WL["varlen"], n_seqs=3, Hk=2, Hv=4)
        x = synth.make(wl, lengths=np.array([130, 0, 64]), seed=43)
    else:
        x = synth.make(with_dims(WL["long"], Hk=2, Hv=4), T=200, seed=44)
    d = to_gpu(x)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"], d["cu_seqlens"])
    o1, s1 = gdn_chunk_fwd(*args)
    ws = torch.empty(1 << 24, dtype=torch.uint8, device="cuda")
    o2 = torch.full_like(o1, float("nan"))
    s2 = torch.full_like(s1, float("nan"))
    gdn_chunk_fwd(*args, o=o2, final_state=s2, workspace=ws, stage="prepare")
    gdn_chunk_fwd(*args, o=o2, final_state=s2, workspace=ws, stage="scan")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_final_state_in_place():
    wl = with_dims(WL["long"], Hk=2, Hv=4)
    x = synth.make(wl, T=300, seed=51)
    o_ref, s_ref = oracle_of(x)
    d = to_gpu(x)
    state = d["initial_state"].clone()
    o, fs = gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], state, final_state=state)
    torch.cuda.synchronize()
    assert fs.data_ptr() == state.data_ptr()
    assert_close("in-place o", o, o_ref, 2e-2)
    assert_close("in-place state", state, s_ref, 2e-2)


def test_zero_tokens():
    wl = with_dims(WL["long"], Hk=2, Hv=4)
    x = synth.make(wl, T=0, seed=61)
    o, fs = run_chunk(x)
    assert o.shape == (1, 0, 4, 128)
    assert torch.equal(fs.cpu(), x["initial_state"])
    x["initial_state"] = None
    o, fs = run_chunk(x)
    assert torch.count_nonzero(fs).item() == 0


def test_nan_propagates_without_crash():
    wl = with_dims(WL["prefill"], Hk=2, Hv=4)
    x = synth.make(wl, T=130, seed=71)
    x["v"][0, 70, 1, 5] = float("nan")  # v-head 1 only
    o, fs = run_chunk(x)
    assert torch.isnan(o[0, 70:, 1]).any()
    assert torch.isnan(fs[0, 1]).any()
    others = [0, 2, 3]
    assert torch.isfinite(o[0, :, others]).all() and torch.isfinite(fs[0, others]).all()


def test_deterministic_and_chunk_equals_recurrent():
    wl = with_dims(WL["long"], Hk=4, Hv=8)
    x = synth.make(wl, T=256, seed=81)
    o1, s1 = run_chunk(x)
    o2, s2 = run_chunk(x)
    assert torch.equal(o1, o2) and torch.equal(s1, s2), "chunk path is not bitwise deterministic"
    d = to_gpu(x)
    state = d["initial_state"].clone()
    o_r, _ = gdn_recurrent_step(d["q"], d["k"], d["v"], d["g"], d["beta"], state)
    torch.cuda.synchronize()
    ref = o_r.cpu().double().numpy()
    assert_close("chunk vs recurrent o", o1, ref, 2e-2)
    assert_close("chunk vs recurrent state", s1, state.cpu().double().numpy(), 2e-2)


# ---------------------------------------------------------------------------------------------
# decode (recurrent) path

@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_recurrent_tokens_one_call(dk, dv):
    wl = with_dims(WL["tiny"], Hk=2, Hv=4, dk=dk, dv=dv, init_state=True)
    x = synth.make(wl, T=40, seed=91)
    o_ref, s_ref = oracle_of(x)
    d = to_gpu(x)
    state = d["initial_state"].clone()
    o, _ = gdn_recurrent_step(d["q"], d["k"], d["v"], d["g"], d["beta"], state)
    torch.cuda.synchronize()
    assert_close("recurrent o", o, o_ref, 1e-4)
    assert_close("recurrent state", state, s_ref, 1e-4)


def test_tiny_fp32_stepped_one_token_at_a_time():
    x = synth.make(WL["tiny"])
    o_ref, s_ref = oracle_of(x)
    d = to_gpu(x)
    B, T, Hk, dk = d["q"].shape
    state = torch.zeros((B, d["v"].shape[2], dk, d["v"].shape[3]), device="cuda")
    outs = []
    for t in range(T):
        o, _ = gdn_recurrent_step(*(d[n][:, t:t + 1].contiguous() for n in ("q", "k", "v", "g", "beta")), state)
        outs.append(o)
    torch.cuda.synchronize()
    assert_close("stepped o", torch.cat(outs, 1), o_ref, 1e-4)
    assert_close("stepped state", state, s_ref, 1e-4)


# ---------------------------------------------------------------------------------------------
# full-size workloads, in the launch configuration the benchmark times

def test_full_prefill_T4096():
    check_chunk(synth.make(WL["prefill"]), "prefill T=4096")


def check_chunk_whole(x, tag, tol=None, per_sequence=False):
    """check_chunk for the full-size workloads: o and every final state compared over the whole
    tensor, a block of rows at a time (the long and packed workloads' o is several GB in fp64)."""
    tol = tol_for(x["q"].dtype) if tol is None else tol
    o, fs = run_chunk(x)
    o, fs = o.cpu(), fs.cpu()
    torch.cuda.empty_cache()
    o_ref, s_ref = oracle_of(x)
    assert_close_blocked(f"{tag} o", o, o_ref, tol)
    del o_ref
    assert_close_blocked(f"{tag} final_state", fs, s_ref, tol)
    if per_sequence:
        rms = float(np.sqrt(np.mean(np.square(s_ref))))
        per = [float(np.max(np.abs(fs[n].double().numpy() - s_ref[n]))) / rms for n in range(len(s_ref))]
        print(f"  {tag} final_state per sequence: worst {max(per):.3e} x rms (sequence {int(np.argmax(per))})",
              flush=True)


def test_full_long_T32768():
    """The long-context workload as specified: T = 32768 (512 chunks) carried from a drawn initial
    state, every v-head, o and the final state over the whole tensors."""
    check_chunk_whole(synth.make(WL["long"]), "long T=32768")


@pytest.mark.parametrize("decay", ["linspace", "small"])
def test_full_long_T32768_weak_decay(decay):
    """The long workload's shape with a slow decay, A = linspace(0.1, 0.9) or A ~ U(0.01, 0.05)
    per v-head: the carried state then survives across hundreds of chunks, so the bf16 rounding of
    the chunk chain accumulates over 512 carried chunks and a wrong inter-chunk carry moves the final
    state, which the workload's own strong decay would hide."""
    wl = WL["long"]
    if decay == "linspace":
        A_log = np.log(np.linspace(0.1, 0.9, wl.Hv)).astype(np.float32)
    else:
        A_log = np.log(np.random.default_rng(5).uniform(0.01, 0.05, wl.Hv)).astype(np.float32)
    check_chunk_whole(synth.make(wl, seed=200 + len(decay), A_log=A_log), f"long T=32768 weak decay {decay}")


@pytest.mark.timeout(600)
def test_full_varlen():
    """The packed workload as specified: 64 sequences of 300..8192 tokens with their own initial
    states, o over every token and every final state, the whole tensors."""
    x = synth.make(WL["varlen"])
    print(f"  varlen: {int(x['cu_seqlens'][-1])} tokens", flush=True)
    check_chunk_whole(x, "varlen", per_sequence=True)


def test_full_decode_128_steps():
    """The decode workload as specified: 256 sequences, 128 successive one-token steps against the
    cached state; o of every sequence at every step and the whole state after step 128."""
    wl = WL["decode"]
    x0 = synth.make(wl)
    A_log = x0["raw"]["A_log"]
    steps = [x0] + [synth.decode_step(wl, s, A_log) for s in range(1, wl.steps)]
    state = x0["initial_state"].cuda().contiguous()
    outs = []
    for s in steps:
        d = to_gpu(s)
        o, _ = gdn_recurrent_step(d["q"], d["k"], d["v"], d["g"], d["beta"], state)
        outs.append(o.cpu())
    torch.cuda.synchronize()
    cat = lambda key: torch.cat([s[key] for s in steps], 1)  # noqa: E731
    ref_in = dict(q=cat("q"), k=cat("k"), v=cat("v"), g=cat("g"), beta=cat("beta"),
                  initial_state=x0["initial_state"], cu_seqlens=None)
    o_ref, s_ref = oracle_of(ref_in)
    assert_close_blocked("decode o (256 sequences x 128 steps)", torch.cat(outs, 1), o_ref, 2e-2)
    assert_close_blocked("decode state after 128 steps", state, s_ref, 2e-2)


@pytest.mark.parametrize("dv,T", [(128, 4096), (64, 1000)])
def test_repeat_calls_alternating_inputs_are_bitwise_stable(dv, T):
    """Two input sets called alternately through one shared workspace, three times each: every
    repeat is bitwise equal to the set's first call (the scan's staging copies and L2 prefetches
    are waited for by exact counts, so a miscount would show as run-to-run differences).  The
    first call of each set is also checked against the oracle."""
    wl = with_dims(WL["prefill"], dv=dv)
    xs = [synth.make(wl, T=T, seed=130 + i) for i in range(2)]
    ds = [{k: x[k].to("cuda") for k in ("q", "k", "v", "g", "beta")} for x in xs]
    from gated_deltanet_delta_amd import workspace_size
    ws = torch.empty(workspace_size(1, T, wl.Hk, wl.Hv, wl.dk, dv, 1, wl.dtype), dtype=torch.uint8, device="cuda")
    first = [None, None]
    for r in range(6):
        d = ds[r % 2]
        o, fs = gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], workspace=ws)
        torch.cuda.synchronize()
        got = (o.cpu(), fs.cpu())
        if first[r % 2] is None:
            first[r % 2] = got
        else:
            assert torch.equal(got[0], first[r % 2][0]) and torch.equal(got[1], first[r % 2][1]), f"call {r}"
    x = xs[0]
    o_ref, s_ref = oracle_of(x)
    assert_close("repeat o", first[0][0], o_ref, tol_for(wl.dtype))
    assert_close("repeat state", first[0][1], s_ref, tol_for(wl.dtype))
