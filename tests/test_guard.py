"""Writes stay inside the memory a call owns (every entry point, the fused-norm prefill included).

Every output, state and workspace of a call is carved out of one device arena, each region between
bands of a fixed NaN bit pattern that no kernel produces.  After each call every band (and the
alignment padding after each region) must still hold that pattern, the results must equal the same
call with ordinarily allocated buffers bit for bit (so every output element was written), and
outputs of earlier calls, both in their arenas and as separate device copies, must still hold what
those calls wrote after later calls of every entry point have run.
"""
import ctypes

import numpy as np
import pytest
import torch

from gated_deltanet_delta_amd import (_lib, gdn_causal_conv1d, gdn_chunk_fwd, gdn_chunk_fwd_gated_norm,
                                      gdn_gated_rmsnorm, gdn_recurrent_step, synth, workspace_size)
from helpers import assert_close, oracle_of, to_gpu, tol_for

pytestmark = pytest.mark.gpu

CANARY = 0x7FA5A5A5        # a quiet-NaN payload: no kernel writes this bit pattern
BAND = 4096                # int32 words of canary before and after every region
WL = synth.WORKLOADS


class Arena:
    """One int32 device buffer: band | region 0 | pad + band | region 1 | ... ; regions start on
    256-byte boundaries and are handed out as typed views."""

    def __init__(self, regions):          # regions: list of (name, shape, dtype)
        self.views, spans, pos = {}, [], BAND
        for _, shape, dtype in regions:
            nbytes = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
            words = (nbytes + 3) // 4
            spans.append((pos, words, shape, dtype, nbytes))
            pos += (words + 63) // 64 * 64 + BAND
        self.buf = torch.full((pos,), CANARY, dtype=torch.int32, device="cuda")
        self.mask = torch.ones(pos, dtype=torch.bool, device="cuda")
        for (name, _, _), (off, words, shape, dtype, nbytes) in zip(regions, spans):
            self.mask[off:off + words] = False
            raw = self.buf[off:off + words].view(torch.uint8)[:nbytes]
            self.views[name] = raw.view(dtype).view(shape) if shape else raw.view(dtype)

    def __getitem__(self, name):
        return self.views[name]

    def check(self, what):
        torch.cuda.synchronize()
        bad = int((self.buf[self.mask] != CANARY).sum().item())
        assert bad == 0, f"{what}: {bad} guard words overwritten"


def ws_region(nbytes):
    return ("ws", (max(int(nbytes), 1),), torch.uint8)


def prefill_case(lengths=None, T=None, seed=0):
    wl = WL["varlen"] if lengths is not None else WL["long"]
    x = synth.make(wl, lengths=lengths, T=T, seed=seed)
    d = to_gpu(x)
    B, TT = d["q"].shape[:2]
    N = len(lengths) if lengths is not None else B
    return wl, x, d, B, TT, N


def run_prefill_in_arena(wl, d, B, TT, N):
    ws_bytes = workspace_size(B, TT, wl.Hk, wl.Hv, wl.dk, wl.dv, N, wl.dtype)
    ar = Arena([("o", (B, TT, wl.Hv, wl.dv), torch.float32),
                ("fs", (N, wl.Hv, wl.dk, wl.dv), torch.float32), ws_region(ws_bytes)])
    gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"], d["cu_seqlens"],
                  o=ar["o"], final_state=ar["fs"], workspace=ar["ws"])
    ar.check("gdn_chunk_fwd")
    return ar


def test_guard_bands_and_earlier_outputs_survive_every_entry_point():
    keep = []     # (description, device tensor, host copy) to re-check after every later call

    def recheck(after):
        torch.cuda.synchronize()
        for what, dev_t, host in keep:
            assert torch.equal(dev_t.cpu(), host), f"{what} changed after {after}"

    def remember(what, t):
        keep.append((what + " (arena)", t, t.cpu()))
        keep.append((what + " (copy)", t.clone(), t.cpu()))

    # 1. packed ragged prefill, Qwen3-Next heads: arena results == ordinary call, bit for bit,
    #    and within the parity bound of the oracle
    lens = np.array([1, 0, 64, 65, 130, 7, 200, 63])
    wl, x, d, B, TT, N = prefill_case(lengths=lens, seed=301)
    ar1 = run_prefill_in_arena(wl, d, B, TT, N)
    o_ref, s_ref = gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"], d["cu_seqlens"])
    torch.cuda.synchronize()
    assert torch.equal(ar1["o"], o_ref) and torch.equal(ar1["fs"], s_ref)
    oo, so = oracle_of(x)
    assert_close("packed o", ar1["o"], oo, tol_for(wl.dtype))
    assert_close("packed final_state", ar1["fs"], so, tol_for(wl.dtype))
    remember("packed prefill o", ar1["o"])
    remember("packed prefill final state", ar1["fs"])

    # 1b. the prefill with the gated norm fused onto o, on the same inputs: y, final state and its
    #     (larger) workspace in one arena; equal to the same call with ordinary buffers, bit for bit
    zr = np.random.default_rng(308)
    zf = torch.from_numpy(zr.standard_normal((B, TT, wl.Hv, wl.dv), dtype=np.float32)).to(torch.bfloat16).cuda()
    wf = torch.from_numpy(zr.uniform(0.5, 1.5, wl.dv).astype(np.float32)).cuda()
    fws = int(_lib.load().gdn_chunk_fwd_gated_norm_workspace_size(B, TT, wl.Hk, wl.Hv, wl.dk, wl.dv, N,
                                                                   _lib.GDN_BF16))
    arf = Arena([("y", (B, TT, wl.Hv, wl.dv), torch.bfloat16), ("fs", (N, wl.Hv, wl.dk, wl.dv), torch.float32),
                 ws_region(fws)])
    gdn_chunk_fwd_gated_norm(d["q"], d["k"], d["v"], d["g"], d["beta"], zf, wf, 1e-6,
                             initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"], y=arf["y"],
                             final_state=arf["fs"], workspace=arf["ws"])
    arf.check("gdn_chunk_fwd_gated_norm")
    ar1.check("gdn_chunk_fwd_gated_norm (earlier arena)")
    recheck("gdn_chunk_fwd_gated_norm")
    y_ref, s_ref2 = gdn_chunk_fwd_gated_norm(d["q"], d["k"], d["v"], d["g"], d["beta"], zf, wf, 1e-6,
                                             initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"])
    torch.cuda.synchronize()
    assert torch.equal(arf["y"], y_ref) and torch.equal(arf["fs"], s_ref2)
    assert torch.equal(arf["fs"], ar1["fs"])
    remember("fused norm y", arf["y"])

    # 2. a longer single sequence with a carried state, then a shorter one through the same call
    for T, seed in ((1000, 302), (130, 303)):
        wl, x, d, B, TT, N = prefill_case(T=T, seed=seed)
        ar = run_prefill_in_arena(wl, d, B, TT, N)
        ar1.check(f"prefill T={T} (earlier arena)")
        recheck(f"prefill T={T}")
        o_ref, s_ref = gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"])
        torch.cuda.synchronize()
        assert torch.equal(ar["o"], o_ref) and torch.equal(ar["fs"], s_ref), T
        remember(f"prefill T={T} o", ar["o"])
        remember(f"prefill T={T} final state", ar["fs"])

    # 3. the backward pass, every output and its workspace in one arena (through the C ABI)
    wl, x, d, B, TT, N = prefill_case(T=200, seed=304)
    rng = np.random.default_rng(305)
    d_o = torch.from_numpy(rng.standard_normal((B, TT, wl.Hv, wl.dv), dtype=np.float32)).cuda()
    d_fin = torch.from_numpy(rng.standard_normal((N, wl.Hv, wl.dk, wl.dv), dtype=np.float32)).cuda()
    clib = _lib.load()
    bws = int(clib.gdn_chunk_bwd_workspace_size(B, TT, wl.Hk, wl.Hv, wl.dk, wl.dv, N))
    f32 = torch.float32
    names = ("dq", "dk", "dv", "dg", "db", "ds0")
    shapes = ((B, TT, wl.Hk, wl.dk), (B, TT, wl.Hk, wl.dk), (B, TT, wl.Hv, wl.dv), (B, TT, wl.Hv),
              (B, TT, wl.Hv), (N, wl.Hv, wl.dk, wl.dv))
    ar = Arena([(n, s, f32) for n, s in zip(names, shapes)] + [ws_region(bws)])
    p = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    st = clib.gdn_chunk_bwd(p(d["q"]), p(d["k"]), p(d["v"]), p(d["g"]), p(d["beta"]), p(d["initial_state"]),
                            None, p(d_o), p(d_fin), B, TT, wl.Hk, wl.Hv, wl.dk, wl.dv, N, _lib.GDN_BF16,
                            _lib.GDN_BF16, *(p(ar[n]) for n in names), p(ar["ws"]), ctypes.c_size_t(bws),
                            torch.cuda.current_stream().cuda_stream)
    assert st == 0, _lib.status_string(st)
    ar.check("gdn_chunk_bwd")
    ar1.check("gdn_chunk_bwd (earlier arena)")
    recheck("gdn_chunk_bwd")
    from gated_deltanet_delta_amd import gdn_chunk_bwd
    ref = gdn_chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d_o, d["initial_state"], d_fin)
    torch.cuda.synchronize()
    for n, r in zip(names, ref):
        assert torch.equal(ar[n], r), n
    remember("backward dk", ar["dk"])

    # 4. the decode step: state and o in an arena, the state advanced in place
    wd = synth.Workload(**{**WL["decode"].__dict__, "B": 5})
    y = synth.make(wd, seed=306)
    dy = to_gpu(y)
    ar = Arena([("o", (wd.B, 1, wd.Hv, wd.dv), f32), ("state", (wd.B, wd.Hv, wd.dk, wd.dv), f32)])
    ar["state"].copy_(dy["initial_state"])
    gdn_recurrent_step(dy["q"], dy["k"], dy["v"], dy["g"], dy["beta"], ar["state"], o=ar["o"])
    ar.check("gdn_recurrent_step")
    recheck("gdn_recurrent_step")
    s2 = dy["initial_state"].clone()
    o2, _ = gdn_recurrent_step(dy["q"], dy["k"], dy["v"], dy["g"], dy["beta"], s2)
    torch.cuda.synchronize()
    assert torch.equal(ar["o"], o2) and torch.equal(ar["state"], s2)

    # 5. the causal conv1d (packed, with a cache) and the gated norm, outputs in arenas
    lens_c = [5, 0, 300, 70]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens_c)]), dtype=torch.int32, device="cuda")
    Tc, C, W = int(sum(lens_c)), 384, 4
    crng = np.random.default_rng(307)
    xc = torch.from_numpy(crng.standard_normal((1, Tc, C), dtype=np.float32)).to(torch.bfloat16).cuda()
    wc = torch.from_numpy(crng.standard_normal((C, W), dtype=np.float32)).cuda()
    cache0 = torch.from_numpy(crng.standard_normal((len(lens_c), W - 1, C), dtype=np.float32)).to(torch.bfloat16).cuda()
    ar = Arena([("y", (1, Tc, C), torch.bfloat16), ("cache", (len(lens_c), W - 1, C), torch.bfloat16)])
    ar["cache"].copy_(cache0)
    gdn_causal_conv1d(xc, wc, None, ar["cache"], cu, silu=True, y=ar["y"])
    ar.check("gdn_causal_conv1d")
    recheck("gdn_causal_conv1d")
    c2 = cache0.clone()
    y2 = gdn_causal_conv1d(xc, wc, None, c2, cu, silu=True)
    torch.cuda.synchronize()
    assert torch.equal(ar["y"], y2) and torch.equal(ar["cache"], c2)

    xo = keep[0][1]                      # the packed prefill's o (fp32), normalised per head vector
    zn = torch.from_numpy(crng.standard_normal(tuple(xo.shape), dtype=np.float32)).to(torch.bfloat16).cuda()
    wn = torch.from_numpy(crng.uniform(0.5, 1.5, xo.shape[-1]).astype(np.float32)).cuda()
    ar = Arena([("out", tuple(xo.shape), torch.bfloat16)])
    gdn_gated_rmsnorm(xo, zn, wn, 1e-6, out=ar["out"])
    ar.check("gdn_gated_rmsnorm")
    recheck("gdn_gated_rmsnorm")
    assert torch.equal(ar["out"], gdn_gated_rmsnorm(xo, zn, wn, 1e-6))
    ar1.check("every entry point (first arena)")
