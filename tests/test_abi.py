"""Host-side tests of the C ABI: the library loads, exports every function include/gdn.h declares,
and rejects bad arguments on the host before anything reaches a GPU.  No kernel runs here: every
call below fails validation, which happens before the first HIP call."""
import ctypes
import os
import re

import pytest

from gated_deltanet_delta_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

F32, BF16 = _lib.GDN_F32, _lib.GDN_BF16
INVALID, UNSUPPORTED, WORKSPACE = (_lib.GDN_ERROR_INVALID_VALUE, _lib.GDN_ERROR_NOT_SUPPORTED,
                                   _lib.GDN_ERROR_WORKSPACE)
P = 0x10000  # stand-in device address; never dereferenced because every call here is rejected


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTED), names
    for name in names:
        assert hasattr(lib, name), f"{name} declared in gdn.h but not exported"


def test_status_strings_and_version(lib):
    for code, name in [(0, "GDN_SUCCESS"), (1, "GDN_ERROR_INVALID_VALUE"), (2, "GDN_ERROR_NOT_SUPPORTED"),
                       (3, "GDN_ERROR_WORKSPACE"), (4, "GDN_ERROR_LAUNCH_FAILURE")]:
        assert _lib.status_string(code) == name
    assert _lib.status_string(77) == "GDN_ERROR_UNKNOWN"
    assert lib.gdn_version() >= 100


CHUNK_CALLS = ("gdn_chunk_fwd", "gdn_chunk_fwd_prepare", "gdn_chunk_fwd_scan")


def chunk(lib, q=P, k=P, v=P, g=P, beta=P, s0=None, cu=None, B=1, T=64, Hk=1, Hv=1, dk=64, dv=64,
          N=1, qkv=F32, gate=F32, o=P, fs=P, ws=None, ws_bytes=0, fn="gdn_chunk_fwd"):
    return getattr(lib, fn)(q, k, v, g, beta, s0, cu, B, T, Hk, Hv, dk, dv, N, qkv, gate, o, fs, ws,
                            ctypes.c_size_t(ws_bytes), None)


def rec(lib, q=P, k=P, v=P, g=P, beta=P, state=P, B=1, T=1, Hk=1, Hv=1, dk=64, dv=64, qkv=F32,
        gate=F32, o=P):
    return lib.gdn_recurrent_step(q, k, v, g, beta, state, B, T, Hk, Hv, dk, dv, qkv, gate, o, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID),
    (dict(g=None), INVALID), (dict(beta=None), INVALID), (dict(o=None), INVALID),
    (dict(fs=None), INVALID), (dict(fs=None, T=0), INVALID),
    (dict(B=0), INVALID), (dict(T=-1), INVALID), (dict(Hk=0), INVALID), (dict(Hv=3, Hk=2), INVALID),
    (dict(N=0), INVALID), (dict(N=2), INVALID),                       # N must equal B without cu_seqlens
    (dict(cu=P, B=2, N=2), INVALID),                                  # cu_seqlens needs B == 1
    (dict(qkv=7), INVALID), (dict(gate=-1), INVALID),
    (dict(q=P + 4), INVALID), (dict(s0=P + 8), INVALID), (dict(fs=P + 4), INVALID),  # 16-byte
    (dict(g=P + 2), INVALID), (dict(cu=P + 2, N=1), INVALID),        # element alignment
    (dict(dk=96), UNSUPPORTED), (dict(dv=32), UNSUPPORTED), (dict(dk=256, dv=256), UNSUPPORTED),
    (dict(dk=0), INVALID),
])
@pytest.mark.parametrize("fn", CHUNK_CALLS)
def test_chunk_rejects(lib, kw, status, fn):
    # the two halves of gdn_chunk_fwd check exactly what the whole call checks
    assert chunk(lib, fn=fn, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(state=None), INVALID), (dict(o=None), INVALID),
    (dict(B=0), INVALID), (dict(T=0), INVALID), (dict(Hv=4, Hk=3), INVALID),
    (dict(qkv=2), INVALID), (dict(state=P + 4), INVALID), (dict(o=P + 8), INVALID),
    (dict(q=P + 2), INVALID), (dict(q=P + 2, qkv=BF16, gate=BF16, g=P + 1), INVALID),
    (dict(dk=32), UNSUPPORTED), (dict(dv=256), UNSUPPORTED),
])
def test_recurrent_rejects(lib, kw, status):
    assert rec(lib, **kw) == status


def chunk_gating(lib, A_log=P, dt_bias=P, **kw):
    a = dict(q=P, k=P, v=P, g=P, beta=P, s0=None, cu=None, B=1, T=64, Hk=1, Hv=1, dk=64, dv=64, N=1,
             qkv=F32, gate=F32, o=P, fs=P, ws=None, ws_bytes=0)
    a.update(kw)
    return lib.gdn_chunk_fwd_gating(a["q"], a["k"], a["v"], a["g"], a["beta"], A_log, dt_bias, a["s0"],
                                    a["cu"], a["B"], a["T"], a["Hk"], a["Hv"], a["dk"], a["dv"], a["N"],
                                    a["qkv"], a["gate"], a["o"], a["fs"], a["ws"],
                                    ctypes.c_size_t(a["ws_bytes"]), None)


def rec_gating(lib, A_log=P, dt_bias=P, **kw):
    a = dict(q=P, k=P, v=P, g=P, beta=P, state=P, B=1, T=1, Hk=1, Hv=1, dk=64, dv=64, qkv=F32,
             gate=F32, o=P)
    a.update(kw)
    return lib.gdn_recurrent_step_gating(a["q"], a["k"], a["v"], a["g"], a["beta"], A_log, dt_bias,
                                         a["state"], a["B"], a["T"], a["Hk"], a["Hv"], a["dk"], a["dv"],
                                         a["qkv"], a["gate"], a["o"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(A_log=None), INVALID), (dict(dt_bias=None), INVALID),
    (dict(A_log=P + 2), INVALID), (dict(dt_bias=P + 1), INVALID),
    (dict(g=None), INVALID), (dict(Hv=3, Hk=2), INVALID), (dict(dk=96), UNSUPPORTED),
])
def test_gating_calls_reject(lib, kw, status):
    # the gating calls check their two extra pointers and everything the plain calls check
    assert chunk_gating(lib, **kw) == status
    assert rec_gating(lib, **kw) == status


def test_workspace_query_is_host_only(lib):
    # fp32 inputs take the fp32 chunk kernel, which needs no workspace
    assert lib.gdn_chunk_fwd_workspace_size(1, 256, 2, 2, 64, 64, 1, F32) == 0
    # invalid sizes report 0 rather than failing
    assert lib.gdn_chunk_fwd_workspace_size(1, 256, 2, 3, 64, 64, 1, BF16) == 0
    assert lib.gdn_chunk_fwd_workspace_size(0, 256, 2, 2, 64, 64, 1, BF16) == 0
    # the bf16 path's workspace grows with the token count and never shrinks below the small case
    small = lib.gdn_chunk_fwd_workspace_size(1, 4096, 16, 32, 128, 128, 1, BF16)
    big = lib.gdn_chunk_fwd_workspace_size(1, 32768, 16, 32, 128, 128, 1, BF16)
    assert big >= small


@pytest.mark.parametrize("fn", CHUNK_CALLS)
def test_too_small_workspace_is_rejected(lib, fn):
    need = lib.gdn_chunk_fwd_workspace_size(1, 4096, 16, 32, 128, 128, 1, BF16)
    if need == 0:
        pytest.skip("this build's bf16 path needs no workspace")
    kw = dict(T=4096, Hk=16, Hv=32, dk=128, dv=128, qkv=BF16, gate=BF16, fn=fn)
    assert chunk(lib, ws=None, ws_bytes=0, **kw) == WORKSPACE
    assert chunk(lib, ws=P, ws_bytes=need - 1, **kw) == WORKSPACE
    assert chunk(lib, ws=P + 16, ws_bytes=need, **kw) == WORKSPACE    # 256-byte alignment


def test_binding_refuses_cpu_tensors():
    import torch
    from gated_deltanet_delta_amd import gdn_chunk_fwd, gdn_recurrent_step
    x = torch.zeros(1, 4, 1, 64)
    gg = torch.zeros(1, 4, 1)
    with pytest.raises(ValueError):
        gdn_chunk_fwd(x, x, x, gg, gg)
    with pytest.raises(ValueError):
        gdn_recurrent_step(x, x, x, gg, gg, torch.zeros(1, 1, 64, 64))


def chunk_indexed(lib, pool=P, idx=P, num_slots=4, **kw):
    a = dict(q=P, k=P, v=P, g=P, beta=P, cu=None, B=1, T=64, Hk=1, Hv=1, dk=64, dv=64, N=1, qkv=F32,
             gate=F32, o=P, ws=None, ws_bytes=0)
    a.update(kw)
    return lib.gdn_chunk_fwd_indexed(a["q"], a["k"], a["v"], a["g"], a["beta"], pool, idx, num_slots,
                                     a["cu"], a["B"], a["T"], a["Hk"], a["Hv"], a["dk"], a["dv"], a["N"],
                                     a["qkv"], a["gate"], a["o"], a["ws"], ctypes.c_size_t(a["ws_bytes"]),
                                     None)


def rec_indexed(lib, pool=P, idx=P, num_slots=4, **kw):
    a = dict(q=P, k=P, v=P, g=P, beta=P, B=1, T=1, Hk=1, Hv=1, dk=64, dv=64, qkv=F32, gate=F32, o=P)
    a.update(kw)
    return lib.gdn_recurrent_step_indexed(a["q"], a["k"], a["v"], a["g"], a["beta"], pool, idx, num_slots,
                                          a["B"], a["T"], a["Hk"], a["Hv"], a["dk"], a["dv"], a["qkv"],
                                          a["gate"], a["o"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(idx=None), INVALID), (dict(pool=None), INVALID), (dict(num_slots=0), INVALID),
    (dict(idx=P + 2), INVALID), (dict(pool=P + 4), INVALID), (dict(q=None), INVALID),
    (dict(Hv=3, Hk=2), INVALID), (dict(dv=32), UNSUPPORTED),
])
def test_indexed_calls_reject(lib, kw, status):
    # the pool calls check the pool, the indices and everything the plain calls check
    assert chunk_indexed(lib, **kw) == status
    assert rec_indexed(lib, **kw) == status


def chunk_ex(lib, A_log=None, dt_bias=None, s0=None, fs=P, idx=None, num_slots=0, flags=0, **kw):
    a = dict(q=P, k=P, v=P, g=P, beta=P, cu=None, B=1, T=64, Hk=1, Hv=1, dk=64, dv=64, N=1, qkv=F32,
             gate=F32, o=P, ws=None, ws_bytes=0)
    a.update(kw)
    return lib.gdn_chunk_fwd_ex(a["q"], a["k"], a["v"], a["g"], a["beta"], A_log, dt_bias, s0, fs, idx,
                                num_slots, a["cu"], a["B"], a["T"], a["Hk"], a["Hv"], a["dk"], a["dv"],
                                a["N"], a["qkv"], a["gate"], flags, a["o"], a["ws"],
                                ctypes.c_size_t(a["ws_bytes"]), None)


def rec_ex(lib, A_log=None, dt_bias=None, state=P, idx=None, num_slots=0, flags=0, **kw):
    a = dict(q=P, k=P, v=P, g=P, beta=P, B=1, T=1, Hk=1, Hv=1, dk=64, dv=64, qkv=F32, gate=F32, o=P)
    a.update(kw)
    return lib.gdn_recurrent_step_ex(a["q"], a["k"], a["v"], a["g"], a["beta"], A_log, dt_bias, state,
                                     idx, num_slots, a["B"], a["T"], a["Hk"], a["Hv"], a["dk"], a["dv"],
                                     a["qkv"], a["gate"], flags, a["o"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(flags=2), INVALID), (dict(flags=0x80000001), INVALID),     # unknown flag bits
    (dict(dt_bias=P), INVALID),                                       # dt_bias without A_log
    (dict(A_log=P), INVALID),                                         # A_log without dt_bias
    (dict(A_log=P + 2, dt_bias=P), INVALID),
    (dict(idx=P, num_slots=0, s0=P), INVALID), (dict(idx=P + 2, num_slots=4, s0=P), INVALID),
    (dict(q=None, flags=1), INVALID), (dict(Hv=3, Hk=2, flags=1), INVALID),
    (dict(dk=96, flags=1), UNSUPPORTED),
])
def test_ex_calls_reject(lib, kw, status):
    # the option-taking calls check their options and everything the plain calls check
    assert chunk_ex(lib, **kw) == status
    rkw = {key: val for key, val in kw.items() if key != "s0"}
    assert rec_ex(lib, **rkw) == status


def test_ex_chunk_pool_must_be_both_states(lib):
    # with state_indices the chunk call's initial and final state are one pool
    assert chunk_ex(lib, idx=P, num_slots=4, s0=P, fs=P + 256) == INVALID
    assert chunk_ex(lib, idx=P, num_slots=4, s0=None, fs=P) == INVALID


def fused(lib, z=P, w=P, eps=1e-6, y=P, zt=BF16, yt=BF16, A_log=None, dt_bias=None, s0=None, fs=P,
          idx=None, num_slots=0, flags=0, **kw):
    a = dict(q=P, k=P, v=P, g=P, beta=P, cu=None, B=1, T=64, Hk=1, Hv=1, dk=64, dv=64, N=1, qkv=BF16,
             gate=F32, ws=P, ws_bytes=1 << 40)
    a.update(kw)
    return lib.gdn_chunk_fwd_gated_norm(a["q"], a["k"], a["v"], a["g"], a["beta"], A_log, dt_bias, s0, fs,
                                        idx, num_slots, a["cu"], z, w, ctypes.c_float(eps), a["B"], a["T"],
                                        a["Hk"], a["Hv"], a["dk"], a["dv"], a["N"], a["qkv"], a["gate"], zt,
                                        yt, flags, y, a["ws"], ctypes.c_size_t(a["ws_bytes"]), None)


@pytest.mark.parametrize("kw,status", [
    (dict(z=None), INVALID), (dict(w=None), INVALID), (dict(y=None), INVALID),
    (dict(eps=-1.0), INVALID), (dict(eps=float("nan")), INVALID), (dict(eps=float("inf")), INVALID),
    (dict(zt=5), INVALID), (dict(yt=7), INVALID),
    (dict(z=P + 8), INVALID), (dict(y=P + 4), INVALID), (dict(w=P + 4), INVALID),   # 16-byte alignment
    (dict(flags=2), INVALID), (dict(dt_bias=P), INVALID), (dict(q=None), INVALID),
    (dict(idx=P, num_slots=4, s0=P, fs=P + 256), INVALID),                          # pool: one tensor
    (dict(dk=96), UNSUPPORTED), (dict(dv=32), UNSUPPORTED),
    (dict(ws=None), WORKSPACE), (dict(ws_bytes=16), WORKSPACE), (dict(ws=P + 16), WORKSPACE),
    (dict(qkv=F32, ws=None), WORKSPACE),                                             # fp32: o needs room
])
def test_fused_norm_rejects(lib, kw, status):
    assert fused(lib, **kw) == status


def test_fused_norm_workspace_sizes(lib):
    size = lib.gdn_chunk_fwd_gated_norm_workspace_size
    plain = lib.gdn_chunk_fwd_workspace_size
    for dk, dv in ((128, 128), (64, 64), (128, 64)):
        # bf16: the prefill's scratch plus one fp32 sum of squares per row and 16-channel slice
        extra = size(1, 4096, 16, 32, dk, dv, 1, BF16) - plain(1, 4096, 16, 32, dk, dv, 1, BF16)
        assert extra == (4096 // 64 + 1) * 32 * 64 * (dv // 16) * 4, (dk, dv, extra)
    # fp32: o between the prefill and the norm pass
    assert size(2, 100, 2, 4, 128, 64, 2, F32) == (2 * 100 * 4 * 64 * 4 + 255) // 256 * 256
    assert size(0, 100, 2, 4, 128, 64, 2, F32) == 0 and size(1, 100, 2, 4, 96, 64, 1, BF16) == 0


def bwd(lib, q=P, k=P, v=P, g=P, beta=P, s0=None, cu=None, do=P, dfin=None, B=1, T=64, Hk=1, Hv=1,
        dk=64, dv=64, N=1, qkv=F32, gate=F32, dq=P, dkk=P, dvv=P, dg=P, db=P, ds0=None, ws=P,
        ws_bytes=1 << 40):
    return lib.gdn_chunk_bwd(q, k, v, g, beta, s0, cu, do, dfin, B, T, Hk, Hv, dk, dv, N, qkv, gate, dq, dkk,
                             dvv, dg, db, ds0, ws, ctypes.c_size_t(ws_bytes), None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(do=None), INVALID), (dict(dq=None), INVALID), (dict(db=None), INVALID),
    (dict(B=0), INVALID), (dict(Hv=3, Hk=2), INVALID), (dict(N=2), INVALID), (dict(cu=P, B=2, N=2), INVALID),
    (dict(qkv=5), INVALID), (dict(do=P + 2), INVALID), (dict(q=P + 1, qkv=BF16), INVALID),
    (dict(k=P + 8, qkv=BF16), INVALID), (dict(v=P + 2), INVALID),   # q, k 16-byte; v its element
    (dict(dk=96), UNSUPPORTED), (dict(dv=32), UNSUPPORTED),
    (dict(ws=None), WORKSPACE), (dict(ws_bytes=16), WORKSPACE), (dict(ws=P + 16), WORKSPACE),
])
def test_backward_rejects(lib, kw, status):
    assert bwd(lib, **kw) == status


def test_backward_workspace_query_is_host_only(lib):
    assert lib.gdn_chunk_bwd_workspace_size(1, 4096, 16, 32, 128, 128, 1) > 0
    assert lib.gdn_chunk_bwd_workspace_size(1, 4096, 16, 33, 128, 128, 1) == 0   # Hv % Hk
    assert lib.gdn_chunk_bwd_workspace_size(1, 4096, 16, 32, 96, 128, 1) == 0    # head size


def bwd_ex(lib, q=P, k=P, v=P, g=P, beta=P, A_log=None, dt_bias=None, s0=None, idx=None, num_slots=0,
           cu=None, do=P, dfin=None, B=1, T=64, Hk=1, Hv=1, dk=64, dv=64, N=1, qkv=F32, gate=F32, flags=0,
           dq=P, dkk=P, dvv=P, dg=P, db=P, dA=None, ddt=None, ds0=None, ws=P, ws_bytes=1 << 40):
    return lib.gdn_chunk_bwd_ex(q, k, v, g, beta, A_log, dt_bias, s0, idx, num_slots, cu, do, dfin, B, T, Hk,
                                Hv, dk, dv, N, qkv, gate, flags, dq, dkk, dvv, dg, db, dA, ddt, ds0, ws,
                                ctypes.c_size_t(ws_bytes), None)


@pytest.mark.parametrize("kw,status", [
    (dict(flags=2), INVALID), (dict(dt_bias=P), INVALID),                       # unknown flag; bias alone
    (dict(A_log=P, dt_bias=P), INVALID), (dict(A_log=P, dt_bias=P, dA=P), INVALID),  # no gate gradients
    (dict(A_log=P + 2, dt_bias=P, dA=P, ddt=P), INVALID),                        # misaligned A_log
    (dict(idx=P, num_slots=4), INVALID), (dict(idx=P, num_slots=0, s0=P), INVALID),  # pool without states
    (dict(idx=P, num_slots=4, s0=P + 4), INVALID),                               # pool not 16-byte aligned
    (dict(idx=P + 2, num_slots=4, s0=P), INVALID),                               # misaligned indices
    (dict(A_log=P, dt_bias=P, dA=P, ddt=P, Hk=2050, Hv=4100), UNSUPPORTED),       # raw gates, > 2048 v-heads
    (dict(q=None, flags=1), INVALID), (dict(dk=96, flags=1), UNSUPPORTED),
    (dict(ws_bytes=16, flags=1), WORKSPACE), (dict(ws=None, idx=P, num_slots=2, s0=P), WORKSPACE),
])
def test_backward_ex_rejects(lib, kw, status):
    assert bwd_ex(lib, **kw) == status


def test_backward_ex_workspace_grows_with_each_option(lib):
    base = lib.gdn_chunk_bwd_workspace_size(1, 4096, 16, 32, 128, 128, 1)
    size = lambda *o: lib.gdn_chunk_bwd_ex_workspace_size(1, 4096, 16, 32, 128, 128, 1, BF16, *o)  # noqa: E731
    assert size(0, 0, 0) >= base
    assert size(1, 0, 0) >= size(0, 0, 0) + 2 * 4 * 4096 * 32             # formed g and beta, fp32
    assert size(0, 0, 1) >= size(0, 0, 0) + 4 * 4096 * (2 * 16 + 32) * 128  # q^, k^ and v as fp32
    assert size(0, 1, 0) >= size(0, 0, 0) + 4 * 32 * 128 * 128               # one gathered state
    assert lib.gdn_chunk_bwd_ex_workspace_size(1, 4096, 16, 33, 128, 128, 1, BF16, 1, 1, 1) == 0


def norm(lib, x=P, z=P, w=P, eps=1e-6, rows=8, d=128, zt=BF16, ot=BF16, out=P):
    return lib.gdn_gated_rmsnorm(x, z, w, eps, rows, d, zt, ot, out, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), INVALID), (dict(z=None), INVALID), (dict(w=None), INVALID), (dict(out=None), INVALID),
    (dict(rows=-1), INVALID), (dict(d=0), INVALID), (dict(zt=5), INVALID), (dict(ot=-1), INVALID),
    (dict(eps=-1.0), INVALID), (dict(eps=float("nan")), INVALID), (dict(eps=float("inf")), INVALID),
    (dict(x=P + 8), INVALID), (dict(w=P + 4), INVALID), (dict(z=P + 4), INVALID),
    (dict(out=P + 2, ot=F32), INVALID), (dict(d=96), UNSUPPORTED), (dict(d=256), UNSUPPORTED),
])
def test_gated_rmsnorm_rejects(lib, kw, status):
    assert norm(lib, **kw) == status


def test_gated_rmsnorm_zero_rows_is_a_no_op(lib):
    # nothing to do: accepted without touching (or even needing) any buffer
    assert norm(lib, x=None, z=None, w=None, out=None, rows=0) == _lib.GDN_SUCCESS


def conv(lib, x=P, w=P, b=None, st=None, idx=None, ns=0, cu=None, B=1, T=8, C=64, W=4, N=1, xt=BF16, silu=0,
         y=P):
    return lib.gdn_causal_conv1d(x, w, b, st, idx, ns, cu, B, T, C, W, N, xt, silu, y, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), INVALID), (dict(w=None), INVALID), (dict(y=None), INVALID),
    (dict(B=0), INVALID), (dict(T=-1), INVALID), (dict(C=0), INVALID), (dict(C=6), INVALID), (dict(N=0), INVALID),
    (dict(N=2), INVALID), (dict(cu=P, B=2, N=2), INVALID), (dict(xt=9), INVALID),
    (dict(idx=P), INVALID), (dict(idx=P, st=P, ns=0), INVALID), (dict(idx=P + 2, st=P, ns=3), INVALID),
    (dict(x=P + 2), INVALID), (dict(y=P + 4), INVALID), (dict(st=P + 2), INVALID), (dict(b=P + 4), INVALID),
    (dict(w=P + 2), INVALID), (dict(cu=P + 2), INVALID),
    (dict(W=0), UNSUPPORTED), (dict(W=17), UNSUPPORTED),
])
def test_causal_conv1d_rejects(lib, kw, status):
    assert conv(lib, **kw) == status
