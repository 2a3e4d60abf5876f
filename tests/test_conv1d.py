"""GPU parity of the depthwise causal conv1d (gdn_causal_conv1d) against the oracle's fp64 version on
the same (already rounded) inputs, per sequence, including the carried cache.

Tolerance, element by element: |y - y_ref| <= r |y_ref| + 1e-6 * s, with s = sum_j |w x| + |bias| the
magnitude the fp32 sum works at (cancellation), r = 2^-8 + 1e-5 for bf16 outputs (one rounding,
up to 2^-8 of the value just above a power of two) and 0 for fp32.  Caches hold copies of inputs:
they must match exactly."""
import numpy as np
import pytest
import torch

from gated_deltanet_delta_amd import gdn_causal_conv1d
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def close(got, ref, scale, dtype, what):
    r = 2.0 ** -8 + 1e-5 if dtype == torch.bfloat16 else 0.0
    err = np.abs(got - ref)
    bound = r * np.abs(ref) + 1e-6 * scale
    worst = float(np.max(err / np.maximum(bound, 1e-300)))
    print(f"  {what}: max err / bound {worst:.3f}", flush=True)
    assert np.all(err <= bound), what


def reference(x, w, b, states, lens, silu):
    """Per sequence oracle over the packed rows of x [L, C]; states [N, W-1, C] (None: zeros)."""
    ys, scales, new = [], [], []
    start = 0
    for n, ln in enumerate(lens):
        st = None if states is None else states[n]
        y, s1 = O.causal_conv1d(x[start:start + ln], w, b, st, silu)
        ya, _ = O.causal_conv1d(np.abs(x[start:start + ln]), np.abs(w), None if b is None else np.abs(b),
                                None if st is None else np.abs(st))
        ys.append(y)
        scales.append(ya)
        new.append(s1)
        start += ln
    return np.concatenate(ys), np.concatenate(scales), new


def draw(rng, L, C, W, N, dtype):
    x = torch.from_numpy(rng.standard_normal((L, C)).astype(np.float32)).to(dtype)
    w = torch.from_numpy((0.5 * rng.standard_normal((C, W))).astype(np.float32))
    b = torch.from_numpy((0.1 * rng.standard_normal(C)).astype(np.float32))
    st = torch.from_numpy(rng.standard_normal((N, W - 1, C)).astype(np.float32)).to(dtype)
    return x, w, b, st


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("silu", [False, True])
@pytest.mark.parametrize("B,T", [(3, 150), (4, 16)])
def test_conv1d_batched(dtype, silu, B, T):
    """Equal-length batch rows.  T = 150: sequence starts fall inside tiles, and the first tokens of
    the later rows straddle two tiles (their caches rewritten by the second launch).  T = 16: every row
    starts on a tile boundary, so every cache is rewritten in the first launch and the second skipped."""
    rng = np.random.default_rng(31 + T)
    C, W = 1040, 4                          # C spans two workgroups
    x, w, b, st = draw(rng, B * T, C, W, B, dtype)
    dev = "cuda"
    st_d = st.to(dev)
    y = gdn_causal_conv1d(x.view(B, T, C).to(dev), w.to(dev), b.to(dev), st_d, silu=silu)
    torch.cuda.synchronize()
    f = lambda t: t.double().cpu().numpy()
    ref, scale, new = reference(f(x), f(w), f(b), f(st), [T] * B, silu)
    close(f(y).reshape(B * T, C), ref, scale, dtype, f"batched {dtype} silu={silu} y")
    for n in range(B):
        assert np.array_equal(f(st_d)[n], new[n]), f"cache of sequence {n}"


@pytest.mark.parametrize("W", [1, 2, 5, 16])
def test_conv1d_packed_pool(W):
    """Packed ragged sequences (empty ones and ones shorter than the cache), caches in a pool addressed
    by slot indices, padding rows with no slot; slots no sequence names are left alone."""
    rng = np.random.default_rng(32 + W)
    lens = [1, 0, 3, 70, 130, 2, 64]
    N, C, L = len(lens), 72, sum(lens)
    x, w, b, _ = draw(rng, L, C, W, N, torch.float32)
    num_slots = 9
    pool = torch.from_numpy(rng.standard_normal((num_slots, W - 1, C)).astype(np.float32))
    idx = torch.tensor([4, 0, 8, -1, 2, 9, 6], dtype=torch.int32)      # -1 and 9: no slot
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    dev = "cuda"
    pool_d = pool.to(dev)
    y = gdn_causal_conv1d(x.view(1, L, C).to(dev), w.to(dev), None, pool_d, cu.to(dev), idx.to(dev))
    torch.cuda.synchronize()
    f = lambda t: t.double().cpu().numpy()
    states = np.zeros((N, W - 1, C))
    for n, i in enumerate(idx.tolist()):
        if 0 <= i < num_slots:
            states[n] = f(pool[i])
    ref, scale, new = reference(f(x), f(w), None, states, lens, False)
    close(f(y).reshape(L, C), ref, scale, torch.float32, f"packed pool W={W} y")
    got = f(pool_d)
    named = {}
    for n, i in enumerate(idx.tolist()):
        if 0 <= i < num_slots:
            named[i] = n
    for i in range(num_slots):
        if i in named and lens[named[i]] > 0:
            assert np.array_equal(got[i], new[named[i]]), f"slot {i}"
        else:
            assert np.array_equal(got[i], f(pool[i])), f"slot {i} should be untouched"


@pytest.mark.parametrize("W", [2, 4, 7])
def test_conv1d_short_sequences(W):
    """Packed sequences of a few tokens each (a decode batch mixed with short requests): the kernel
    takes them one token per thread; one-token sequences rewrite their cache in the same launch, the
    25-token one in the second."""
    rng = np.random.default_rng(50 + W)
    lens = [1, 1, 0, 2, 1, 5, 1, 1, 25, 1, 3, 1]
    N, C, L = len(lens), 264, sum(lens)
    x, w, b, st = draw(rng, L, C, W, N, torch.bfloat16)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    dev = "cuda"
    st_d = st.to(dev)
    y = gdn_causal_conv1d(x.view(1, L, C).to(dev), w.to(dev), b.to(dev), st_d, cu.to(dev), silu=True)
    torch.cuda.synchronize()
    f = lambda t: t.double().cpu().numpy()
    ref, scale, new = reference(f(x), f(w), f(b), f(st), lens, True)
    close(f(y).reshape(L, C), ref, scale, torch.bfloat16, f"short sequences W={W} y")
    for n in range(N):
        want = new[n] if lens[n] > 0 else f(st)[n]
        assert np.array_equal(f(st_d)[n], want), f"cache of sequence {n}"


def test_conv1d_decode_steps_equal_prefill_bitwise():
    """Feeding a sequence one token per call (the decode path) gives bit-identical outputs and cache
    to one call over the whole sequence."""
    rng = np.random.default_rng(40)
    B, T, C, W = 2, 20, 128, 4
    x, w, b, st = draw(rng, B * T, C, W, B, torch.bfloat16)
    dev = "cuda"
    xd = x.view(B, T, C).to(dev)
    s_all = st.to(dev)
    y_all = gdn_causal_conv1d(xd, w.to(dev), b.to(dev), s_all, silu=True)
    s_step = st.to(dev)
    ys = [gdn_causal_conv1d(xd[:, t:t + 1].contiguous(), w.to(dev), b.to(dev), s_step, silu=True)
          for t in range(T)]
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(ys, dim=1), y_all)
    assert torch.equal(s_step, s_all)
