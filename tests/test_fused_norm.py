"""GPU parity of gdn_chunk_fwd_gated_norm: the prefill with the layer's gated output norm fused onto
o, y = o / sqrt(mean(o^2) + eps) * weight * silu(z) per (token, v-head) row.

Each case is checked twice on the same seeded inputs:

* Against the oracle's gated norm of the library's own o (gdn_chunk_fwd_ex on the same arguments,
  normalised in fp64 on the CPU): this isolates the fusion.  bf16 y: |err| <= (2^-8 + 1e-4) |y_ref|
  + 1e-6 rms(y_ref) element by element (one bf16 rounding of the result, plus fp32 arithmetic in
  another order: the sum of squares is taken per 16-channel slice, then over the slices); fp32 y:
  max|err| <= 1e-4 rms(y_ref).
* Against oracle.gated_rmsnorm(oracle.forward(...)), element by element, with the bound that the
  prefill's own tolerance implies: with |o - o_ref| <= tol_o rms(o_ref) over the tensor (the parity
  rule of the prefill, 2e-2 for bf16 inputs), a row of rms r moves by at most
  tol_o rms(o_ref) / r relative, so |y - y_ref| <= tol_o (rms(o_ref) / r) (|weight silu(z)| + |y_ref|)
  + the bf16 rounding above.  The test prints the worst ratio of error to that bound.

z is drawn standard normal (a projection of the hidden state, as the z branch of the Qwen3.5 page's
flowchart), the weight uniform in [0.5, 1.5].
"""
import numpy as np
import pytest
import torch

from gated_deltanet_delta_amd import gdn_chunk_fwd_ex, gdn_chunk_fwd_gated_norm, synth
from helpers import oracle_of, tol_for
from oracle import oracle as O

pytestmark = pytest.mark.gpu

WL = synth.WORKLOADS
f64 = synth.to_f64
EPS = 1e-6
BF16_REL = 2.0 ** -8 + 1e-4


def with_dims(wl, **kw):
    d = dict(wl.__dict__)
    d.update(kw)
    return synth.Workload(**d)


def norm_inputs(shape, z_dtype, seed):
    rng = np.random.default_rng(seed)
    z = torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(z_dtype)
    w = torch.from_numpy(rng.uniform(0.5, 1.5, shape[-1]).astype(np.float32))
    return z, w


def silu64(z):
    return z / (1.0 + np.exp(-z))


def check_fusion(name, y, o_lib, z, w, y_dtype):
    """y against the oracle's gated norm of the library's own o (the fusion's arithmetic alone)."""
    ref = O.gated_rmsnorm(f64(o_lib), f64(z), f64(w), EPS)
    got = y.double().cpu().numpy()
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = np.abs(got - ref)
    if y_dtype == torch.float32:
        worst = float(err.max()) / rms
        print(f"  {name} vs norm(own o): max err {worst:.3e} x rms (tol 1e-4)", flush=True)
        assert worst <= 1e-4
    else:
        bound = BF16_REL * np.abs(ref) + 1e-6 * rms
        worst = float(np.max(err / bound))
        print(f"  {name} vs norm(own o): worst err / bound {worst:.3f}", flush=True)
        assert worst <= 1.0


def check_oracle(name, y, o_ref, z, w, tol_o, y_dtype):
    """y against oracle.gated_rmsnorm(oracle.forward(...)) with the bound the prefill's tolerance implies."""
    ref = O.gated_rmsnorm(o_ref, f64(z), f64(w), EPS)
    got = y.double().cpu().numpy()
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    g_rms = float(np.sqrt(np.nanmean(o_ref * o_ref)))
    r = np.sqrt(np.mean(o_ref * o_ref, axis=-1, keepdims=True) + EPS)
    gate = np.abs(f64(w) * silu64(f64(z)))
    bound = tol_o * (g_rms / r) * (gate + np.abs(ref))
    if y_dtype != torch.float32:
        bound = bound + BF16_REL * np.abs(ref)
    bound = bound + 1e-30
    ratio = float(np.max(np.abs(got - ref) / bound))
    e_rms = float(np.max(np.abs(got - ref))) / float(np.sqrt(np.mean(ref * ref)))
    print(f"  {name} vs oracle: max err {e_rms:.3e} x rms(y), worst err / bound {ratio:.3f}", flush=True)
    assert ratio <= 1.0


def run(x, z, w, y_dtype=torch.bfloat16, **kw):
    dev = "cuda"
    s0 = x.get("initial_state")
    cu = x.get("cu_seqlens")
    args = (x["q"].to(dev), x["k"].to(dev), x["v"].to(dev), kw.pop("a", x["g"]).to(dev),
            kw.pop("b", x["beta"]).to(dev))
    common = dict(initial_state=None if s0 is None else s0.to(dev), cu_seqlens=None if cu is None else cu.to(dev))
    common.update({k_: (v_.to(dev) if isinstance(v_, torch.Tensor) else v_) for k_, v_ in kw.items()})
    y, fs = gdn_chunk_fwd_gated_norm(*args, z.to(dev), w.to(dev), EPS, y_dtype=y_dtype, **common)
    o, fs2 = gdn_chunk_fwd_ex(*args, **common)
    torch.cuda.synchronize()
    assert torch.equal(fs, fs2), "final state differs from the unfused call"
    return y, o, fs


def test_fused_norm_prefill_T4096():
    """The 4096-token Qwen3-Next-shaped prefill the benchmark times (bf16 z and y)."""
    wl = WL["prefill"]
    x = synth.make(wl)
    z, w = norm_inputs((wl.B, wl.T, wl.Hv, wl.dv), torch.bfloat16, 501)
    y, o, fs = run(x, z, w)
    assert y.dtype == torch.bfloat16
    check_fusion("T=4096", y, o, z, w, torch.bfloat16)
    o_ref, _ = oracle_of(x)
    check_oracle("T=4096", y, o_ref, z, w, tol_for(wl.dtype), torch.bfloat16)


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64)])
def test_fused_norm_packed_ragged(dk, dv):
    """Packed sequences with carried states: empty, one-token, partial and multi-chunk lengths."""
    wl = with_dims(WL["varlen"], Hk=4, Hv=8, dk=dk, dv=dv, n_seqs=9)
    lengths = np.array([1, 0, 64, 65, 130, 7, 200, 63, 300])
    x = synth.make(wl, lengths=lengths, seed=510 + dk + dv)
    z, w = norm_inputs((1, int(lengths.sum()), wl.Hv, dv), torch.bfloat16, 511)
    y, o, _ = run(x, z, w)
    check_fusion(f"packed dk={dk} dv={dv}", y, o, z, w, torch.bfloat16)
    o_ref, _ = oracle_of(x)
    check_oracle(f"packed dk={dk} dv={dv}", y, o_ref, z, w, tol_for(wl.dtype), torch.bfloat16)


def test_fused_norm_many_packed_sequences():
    """More workgroups than the GPU holds at once (40 packed sequences at the Qwen3-Next head
    layout: 10,240 scan workgroups): the slices of a v-head still find each other's sums."""
    wl = WL["varlen"]
    rng = np.random.default_rng(550)
    lengths = rng.integers(300, 2000, size=40)
    lengths[7] = 0
    lengths[19] = 1
    x = synth.make(wl, lengths=lengths, seed=551)
    z, w = norm_inputs((1, int(lengths.sum()), wl.Hv, wl.dv), torch.bfloat16, 552)
    y, o, _ = run(x, z, w)
    check_fusion("40 packed sequences", y, o, z, w, torch.bfloat16)
    o_ref, _ = oracle_of(x)
    check_oracle("40 packed sequences", y, o_ref, z, w, tol_for(wl.dtype), torch.bfloat16)


@pytest.mark.parametrize("z_dtype,y_dtype", [(torch.float32, torch.float32), (torch.bfloat16, torch.float32),
                                             (torch.float32, torch.bfloat16)])
def test_fused_norm_every_option(z_dtype, y_dtype):
    """Raw gate projections, q/k normalisation, a ragged batch, and the other z / y dtypes."""
    wl = with_dims(WL["prefill"], B=2, T=333, Hk=2, Hv=4)
    x = synth.make(wl, seed=520)
    raw = x["raw"]
    a = torch.from_numpy(raw["a"]).to(torch.bfloat16)
    b = torch.from_numpy(raw["b"]).to(torch.bfloat16)
    A_log = torch.from_numpy(np.asarray(raw["A_log"], dtype=np.float32))
    dt_bias = torch.from_numpy((0.3 * np.random.default_rng(521).standard_normal(wl.Hv)).astype(np.float32))
    z, w = norm_inputs((wl.B, wl.T, wl.Hv, wl.dv), z_dtype, 522)
    y, o, _ = run(x, z, w, y_dtype=y_dtype, a=a, b=b, A_log=A_log, dt_bias=dt_bias, qk_l2norm=True)
    assert y.dtype == y_dtype
    check_fusion(f"options z {z_dtype} y {y_dtype}", y, o, z, w, y_dtype)
    g, beta = O.gates(f64(a), f64(b), f64(A_log), f64(dt_bias))
    o_ref, _ = O.forward(O.l2norm(f64(x["q"])), O.l2norm(f64(x["k"])), f64(x["v"]), g, beta,
                         f64(x.get("initial_state")), None)
    check_oracle(f"options z {z_dtype} y {y_dtype}", y, o_ref, z, w, tol_for(wl.dtype), y_dtype)


def test_fused_norm_fp32_inputs():
    """fp32 q, k, v take the prefill then a separate norm pass (o held in the workspace)."""
    wl = with_dims(WL["prefill"], B=1, T=200, Hk=2, Hv=4, dtype=torch.float32)
    x = synth.make(wl, seed=530)
    z, w = norm_inputs((wl.B, wl.T, wl.Hv, wl.dv), torch.bfloat16, 531)
    y, o, _ = run(x, z, w)
    check_fusion("fp32 inputs", y, o, z, w, torch.bfloat16)
    o_ref, _ = oracle_of(x)
    check_oracle("fp32 inputs", y, o_ref, z, w, tol_for(wl.dtype), torch.bfloat16)


def test_fused_norm_zero_length_sequence_passes_state():
    """T = 0: nothing is written to y and the state passes through."""
    wl = with_dims(WL["prefill"], B=1, T=0, Hk=2, Hv=4)
    x = synth.make(wl, seed=540)
    z, w = norm_inputs((1, 0, wl.Hv, wl.dv), torch.bfloat16, 541)
    y, _, fs = run(x, z, w)
    assert y.shape == (1, 0, wl.Hv, wl.dv)
    s0 = x.get("initial_state")
    assert torch.equal(fs.cpu(), s0 if s0 is not None else torch.zeros_like(fs.cpu()))
