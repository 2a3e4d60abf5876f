"""gdn_chunk_fwd_noalloc (through the C ABI) against gdn_chunk_fwd with a caller's workspace: the
same kernels, so the results must agree bit for bit, on two calls in a row (the second smaller, so
it meets the first call's leftovers in the static scratch), and both within the parity bound of the
oracle.  A call whose scratch need exceeds the static array is refused and writes nothing."""
import ctypes

import numpy as np
import pytest
import torch

from gated_deltanet_delta_amd import _lib, gdn_chunk_fwd, synth, workspace_size
from helpers import assert_close, oracle_of, to_gpu, tol_for

pytestmark = pytest.mark.gpu

WL = synth.WORKLOADS


def _noalloc(lib, d, o, fs, B, T, Hk, Hv, dk, dv, N):
    p = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    return lib.gdn_chunk_fwd_noalloc(p(d["q"]), p(d["k"]), p(d["v"]), p(d["g"]), p(d["beta"]),
                                     p(d["initial_state"]), p(d["cu_seqlens"]), B, T, Hk, Hv, dk, dv, N,
                                     _lib.GDN_BF16, _lib.GDN_BF16, p(o), p(fs),
                                     torch.cuda.current_stream().cuda_stream)


def test_noalloc_equals_workspace_call_on_two_calls():
    lib = _lib.load()
    cap = int(lib.gdn_chunk_fwd_noalloc_max_bytes())
    assert cap == 64 << 20
    cases = [dict(wl=WL["long"], T=3000, seed=401),                                   # larger first
             dict(wl=WL["varlen"], lengths=np.array([70, 0, 129, 1, 64]), seed=402)]  # then smaller, packed
    for c in cases:
        wl = c["wl"]
        x = synth.make(wl, T=c.get("T"), lengths=c.get("lengths"), seed=c["seed"])
        d = to_gpu(x)
        B, T = d["q"].shape[:2]
        N = B if d["cu_seqlens"] is None else d["cu_seqlens"].numel() - 1
        assert 0 < workspace_size(B, T, wl.Hk, wl.Hv, wl.dk, wl.dv, N, wl.dtype) <= cap
        o = torch.full((B, T, wl.Hv, wl.dv), float("nan"), device="cuda")
        fs = torch.full((N, wl.Hv, wl.dk, wl.dv), float("nan"), device="cuda")
        st = _noalloc(lib, d, o, fs, B, T, wl.Hk, wl.Hv, wl.dk, wl.dv, N)
        assert st == 0, _lib.status_string(st)
        o_ref, s_ref = gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"], d["cu_seqlens"])
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(fs, s_ref), f"T={T}"
        oo, so = oracle_of(x)
        assert_close(f"noalloc T={T} o", o, oo, tol_for(wl.dtype))
        assert_close(f"noalloc T={T} final_state", fs, so, tol_for(wl.dtype))


def test_noalloc_refuses_more_than_its_scratch():
    lib = _lib.load()
    wl = WL["prefill"]
    T = 16384
    need = workspace_size(1, T, wl.Hk, wl.Hv, wl.dk, wl.dv, 1, wl.dtype)
    assert need > int(lib.gdn_chunk_fwd_noalloc_max_bytes())
    x = synth.make(wl, T=T, seed=403)
    d = to_gpu(x)
    o = torch.full((1, T, wl.Hv, wl.dv), 7.0, device="cuda")
    fs = torch.full((1, wl.Hv, wl.dk, wl.dv), 7.0, device="cuda")
    st = _noalloc(lib, d, o, fs, 1, T, wl.Hk, wl.Hv, wl.dk, wl.dv, 1)
    torch.cuda.synchronize()
    assert st == _lib.GDN_ERROR_WORKSPACE
    assert bool((o == 7.0).all()) and bool((fs == 7.0).all())
