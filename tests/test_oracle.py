"""Pins for the CPU oracle: closed forms, a hand-worked example, brute force and invariants.

None of these re-types the oracle's own loop.  Each pin fixes the answer by other means: a value
worked by hand, a closed form of a special case, the explicit product of per-token transition
matrices, or an identity the rule must satisfy.  ``test_pins_catch_planted_mistakes`` plants typical
mistakes in a copy of the oracle's C source and shows that every one of them fails some pin.
"""
import json
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------------------------
# input helpers (plain random draws; nothing here evaluates the rule)

def rand_inputs(rng, B=1, T=16, Hk=1, Hv=1, dk=8, dv=8, init=True, gscale=1.0):
    q = rng.standard_normal((B, T, Hk, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((B, T, Hk, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, Hv, dv))
    g = -gscale * rng.uniform(0.0, 1.0, (B, T, Hv))
    beta = rng.uniform(0.05, 0.95, (B, T, Hv))
    s0 = rng.standard_normal((B, Hv, dk, dv)) if init else None
    return q, k, v, g, beta, s0


def rel(a, b):
    return float(np.max(np.abs(a - b)) / max(1e-300, np.sqrt(np.mean(np.square(b)))))


# ----------------------------------------------------------------------------------------------
# pins, written against an oracle object so the mutation test can reuse them

def pin_golden(orc):
    d = json.load(open(os.path.join(GOLDEN, "hand_worked_two_tokens.json")))
    x = d["inputs"]
    q = np.array(x["q"])[None, :, None, :]
    k = np.array(x["k"])[None, :, None, :]
    v = np.array(x["v"])[None, :, None, :]
    g = np.array(x["g"])[None, :, None]
    beta = np.array(x["beta"])[None, :, None]
    s0 = np.array(x["initial_state"])[None, None]
    o, fs = orc.forward(q, k, v, g, beta, s0)
    tol = d["tolerance"]
    assert np.allclose(o[0, :, 0, :], np.array(d["expected"]["o"]), atol=tol, rtol=0)
    assert np.allclose(fs[0, 0], np.array(d["expected"]["final_state"]), atol=tol, rtol=0)


def pin_pure_decay(orc):
    """beta = 0: nothing is written, S_t = exp(G_t) S0 and o_t = exp(G_t) S0^T q_t."""
    rng = np.random.default_rng(1)
    q, k, v, g, beta, s0 = rand_inputs(rng, T=12, dk=6, dv=5)
    beta[:] = 0.0
    o, fs = orc.forward(q, k, v, g, beta, s0)
    G = np.cumsum(g[0, :, 0])
    expect_o = np.exp(G)[:, None] * (q[0, :, 0, :] @ s0[0, 0])
    assert np.allclose(o[0, :, 0, :], expect_o, atol=1e-12)
    assert np.allclose(fs[0, 0], np.exp(G[-1]) * s0[0, 0], atol=1e-12)


def pin_retrieval_overwrite(orc):
    """g = 0, beta = 1, orthonormal keys, S0 = 0: the state stores each (key, value) pair exactly;
    a query equal to a stored key returns its value; writing a key again keeps only the later value."""
    rng = np.random.default_rng(2)
    dk, dv = 8, 5
    basis, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = basis.T  # orthonormal rows
    order = [0, 3, 5, 3, 7]  # key 3 is written twice
    T = len(order)
    k = keys[order][None, :, None, :]
    v = rng.standard_normal((1, T, 1, dv))
    q = keys[[0, 0, 5, 3, 3]][None, :, None, :]
    g = np.zeros((1, T, 1))
    beta = np.ones((1, T, 1))
    o, fs = orc.forward(q, k, v, g, beta, None)
    S = fs[0, 0]
    assert np.allclose(keys[0] @ S, v[0, 0, 0], atol=1e-12)
    assert np.allclose(keys[5] @ S, v[0, 2, 0], atol=1e-12)
    assert np.allclose(keys[3] @ S, v[0, 3, 0], atol=1e-12)  # the later write wins
    assert np.allclose(keys[7] @ S, v[0, 4, 0], atol=1e-12)
    assert np.allclose(keys[1] @ S, 0.0, atol=1e-12)         # never written
    assert np.allclose(o[0, 0, 0], v[0, 0, 0], atol=1e-12)   # read-out includes the current token
    assert np.allclose(o[0, 1, 0], v[0, 0, 0], atol=1e-12)
    assert np.allclose(o[0, 2, 0], v[0, 2, 0], atol=1e-12)
    assert np.allclose(o[0, 3, 0], v[0, 3, 0], atol=1e-12)   # overwritten on this very token
    assert np.allclose(o[0, 4, 0], v[0, 3, 0], atol=1e-12)
    # S equals the sum of outer products of the surviving pairs
    expect = np.outer(keys[0], v[0, 0, 0]) + np.outer(keys[5], v[0, 2, 0]) + \
        np.outer(keys[3], v[0, 3, 0]) + np.outer(keys[7], v[0, 4, 0])
    assert np.allclose(S, expect, atol=1e-12)


def pin_single_direction(orc):
    """k_t = e_0 for all t: row 0 of S follows the scalar EMA s <- e^g (1 - beta) s + beta v,
    every other row only decays by e^(sum g); o_t = S_t^T q_t reads those rows."""
    rng = np.random.default_rng(3)
    T, dk, dv = 10, 4, 3
    q, k, v, g, beta, s0 = rand_inputs(rng, T=T, dk=dk, dv=dv)
    k[:] = 0.0
    k[..., 0] = 1.0
    o, fs = orc.forward(q, k, v, g, beta, s0)
    s = s0[0, 0].copy()
    for t in range(T):
        a, b = np.exp(g[0, t, 0]), beta[0, t, 0]
        s[0] = a * (1 - b) * s[0] + b * v[0, t, 0]
        s[1:] = a * s[1:]
        assert np.allclose(o[0, t, 0], q[0, t, 0] @ s, atol=1e-12)
    assert np.allclose(fs[0, 0], s, atol=1e-12)


def pin_brute_force(orc):
    """T <= 8: S_T = A_T...A_1 S0 + sum_j A_T...A_{j+1} beta_j k_j v_j^T with the explicit dk x dk
    transitions A_t = e^{g_t} (I - beta_t k_t k_t^T); o_t from the same unrolled products."""
    rng = np.random.default_rng(4)
    for T in (1, 2, 5, 8):
        dk, dv = 5, 4
        q, k, v, g, beta, s0 = rand_inputs(rng, T=T, dk=dk, dv=dv, gscale=2.0)
        o, fs = orc.forward(q, k, v, g, beta, s0)
        A = [np.exp(g[0, t, 0]) * (np.eye(dk) - beta[0, t, 0] * np.outer(k[0, t, 0], k[0, t, 0]))
             for t in range(T)]
        Bt = [beta[0, t, 0] * np.outer(k[0, t, 0], v[0, t, 0]) for t in range(T)]

        def prod(lo, hi):  # A_hi ... A_lo (inclusive, 0-based), identity if empty
            P = np.eye(dk)
            for t in range(lo, hi + 1):
                P = A[t] @ P
            return P

        for t in range(T):
            St = prod(0, t) @ s0[0, 0] + sum(prod(j + 1, t) @ Bt[j] for j in range(t + 1))
            assert np.allclose(o[0, t, 0], St.T @ q[0, t, 0], atol=1e-12)
        assert np.allclose(fs[0, 0], St, atol=1e-12)


def pin_split_and_carry(orc):
    """Running T1 tokens, then T2 tokens from the carried state, equals running T1+T2 at once
    (the jsqmd.com article's segment loop, §2.2)."""
    rng = np.random.default_rng(5)
    q, k, v, g, beta, s0 = rand_inputs(rng, B=2, T=23, Hk=2, Hv=4, dk=6, dv=7)
    o, fs = orc.forward(q, k, v, g, beta, s0)
    T1 = 9
    o1, s1 = orc.forward(q[:, :T1], k[:, :T1], v[:, :T1], g[:, :T1], beta[:, :T1], s0)
    o2, s2 = orc.forward(q[:, T1:], k[:, T1:], v[:, T1:], g[:, T1:], beta[:, T1:], s1)
    assert np.allclose(np.concatenate([o1, o2], axis=1), o, atol=1e-12)
    assert np.allclose(s2, fs, atol=1e-12)


def pin_varlen_is_separate(orc):
    """Packed sequences (cu_seqlens) give the same results as separate calls; a zero-length sequence
    returns its initial state."""
    rng = np.random.default_rng(6)
    lens = [5, 0, 11, 1, 7]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q, k, v, g, beta, _ = rand_inputs(rng, T=T, Hk=1, Hv=2, dk=4, dv=3)
    s0 = rng.standard_normal((len(lens), 2, 4, 3))
    o, fs = orc.forward(q, k, v, g, beta, s0, cu_seqlens=cu)
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        if b == a:
            assert np.array_equal(fs[n], s0[n])
            continue
        on, sn = orc.forward(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b], beta[:, a:b], s0[n:n + 1])
        assert np.allclose(o[:, a:b], on, atol=1e-12)
        assert np.allclose(fs[n], sn[0], atol=1e-12)


def pin_padding_neutral(orc):
    """Tokens with g = 0 and beta = 0 leave the state exactly unchanged."""
    rng = np.random.default_rng(7)
    q, k, v, g, beta, s0 = rand_inputs(rng, T=9, dk=5, dv=4)
    _, fs = orc.forward(q, k, v, g, beta, s0)
    q2, k2, v2, _, _, _ = rand_inputs(rng, T=6, dk=5, dv=4)
    cat = lambda a, b: np.concatenate([a, b], axis=1)  # noqa: E731
    _, fs2 = orc.forward(cat(q, q2), cat(k, k2), cat(v, v2), cat(g, np.zeros((1, 6, 1))),
                         cat(beta, np.zeros((1, 6, 1))), s0)
    assert np.array_equal(fs2, fs)


def pin_linearity(orc):
    """For fixed q, k, g, beta the map (S0, V) -> (o, S_T) is linear."""
    rng = np.random.default_rng(8)
    q, k, v1, g, beta, sa = rand_inputs(rng, T=14, Hk=1, Hv=2, dk=5, dv=4)
    v2 = rng.standard_normal(v1.shape)
    sb = rng.standard_normal(sa.shape)
    a, b = 0.7, -1.3
    o1, f1 = orc.forward(q, k, v1, g, beta, sa)
    o2, f2 = orc.forward(q, k, v2, g, beta, sb)
    o3, f3 = orc.forward(q, k, a * v1 + b * v2, g, beta, a * sa + b * sb)
    assert np.allclose(o3, a * o1 + b * o2, atol=1e-11)
    assert np.allclose(f3, a * f1 + b * f2, atol=1e-11)


def pin_norm_bound(orc):
    """With |k| = 1 and beta in [0,1], (I - beta k k^T) is a contraction, so
    ||S_t||_2 <= e^{g_t} ||S_{t-1}||_2 + beta_t ||v_t||; checked along every prefix."""
    rng = np.random.default_rng(9)
    T = 20
    q, k, v, g, beta, s0 = rand_inputs(rng, T=T, dk=6, dv=6)
    prev = np.linalg.norm(s0[0, 0], 2)
    for t in range(1, T + 1):
        _, fs = orc.forward(q[:, :t], k[:, :t], v[:, :t], g[:, :t], beta[:, :t], s0)
        cur = np.linalg.norm(fs[0, 0], 2)
        assert cur <= np.exp(g[0, t - 1, 0]) * prev + beta[0, t - 1, 0] * np.linalg.norm(v[0, t - 1, 0]) + 1e-12
        prev = cur


def pin_head_grouping(orc):
    """v-head h reads q/k head h // (Hv/Hk): a grouped call equals per-v-head calls that are handed
    that q/k head explicitly."""
    rng = np.random.default_rng(10)
    Hk, Hv = 2, 6
    q, k, v, g, beta, s0 = rand_inputs(rng, T=7, Hk=Hk, Hv=Hv, dk=4, dv=3)
    o, fs = orc.forward(q, k, v, g, beta, s0)
    for h in range(Hv):
        kh = h // (Hv // Hk)
        oh, sh = orc.forward(q[:, :, kh:kh + 1], k[:, :, kh:kh + 1], v[:, :, h:h + 1],
                             g[:, :, h:h + 1], beta[:, :, h:h + 1], s0[:, h:h + 1])
        assert np.allclose(o[:, :, h:h + 1], oh, atol=1e-12)
        assert np.allclose(fs[:, h:h + 1], sh, atol=1e-12)


def pin_chunked_form(orc):
    """The chunk-parallel (WY/UT) form reaches the token-by-token result for every chunk length,
    including a ragged last chunk, with and without an initial state."""
    rng = np.random.default_rng(11)
    for T, C, init, gscale in ((37, 1, True, 1.0), (37, 5, True, 1.0), (64, 16, False, 4.0),
                               (100, 64, True, 6.0), (37, 37, True, 0.01), (130, 64, True, 0.0)):
        q, k, v, g, beta, s0 = rand_inputs(rng, T=T, Hk=1, Hv=2, dk=8, dv=6, init=init, gscale=gscale)
        o, fs = orc.forward(q, k, v, g, beta, s0)
        oc, fc = O.chunked(q[0], k[0], v[0], g[0], beta[0], None if s0 is None else s0[0], C)
        assert rel(oc, o[0]) < 1e-11, (T, C)
        assert rel(fc, fs[0]) < 1e-11, (T, C)


PINS = [pin_golden, pin_pure_decay, pin_retrieval_overwrite, pin_single_direction, pin_brute_force,
        pin_split_and_carry, pin_varlen_is_separate, pin_padding_neutral, pin_linearity,
        pin_norm_bound, pin_head_grouping, pin_chunked_form]


@pytest.fixture(scope="module")
def orc():
    return O.Oracle()


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(orc, pin):
    pin(orc)


# ----------------------------------------------------------------------------------------------
# gates

def test_gates_closed_forms():
    g, beta = O.gates(np.zeros(3), np.zeros(3), np.zeros(3), np.zeros(3))
    assert np.allclose(beta, 0.5, atol=0, rtol=1e-15)
    assert np.allclose(g, -np.log(2.0), atol=0, rtol=1e-15)   # softplus(0) = ln 2, exp(A_log=0) = 1
    # A_log = log 3, a = large: softplus(a) -> a, so g -> -3a
    g, _ = O.gates(np.array([40.0]), np.array([0.0]), np.log(np.array([3.0])), np.zeros(1))
    assert np.isclose(g[0], -120.0, rtol=1e-15)
    # a very negative: softplus(a) ~ e^a (tiny but positive), g stays < 0
    g, _ = O.gates(np.array([-30.0]), np.array([0.0]), np.zeros(1), np.zeros(1))
    assert g[0] < 0 and np.isclose(g[0], -np.exp(-30.0), rtol=1e-12)
    # beta = sigmoid(b): symmetric, limits 0 and 1
    _, bb = O.gates(np.zeros(3), np.array([-50.0, 2.0, 50.0]), np.zeros(3), np.zeros(3))
    assert bb[0] < 1e-20 and np.isclose(bb[1], 1 / (1 + np.exp(-2.0))) and bb[2] == 1.0
    # dt_bias shifts a
    ga, _ = O.gates(np.array([0.3]), np.zeros(1), np.array([0.5]), np.array([0.2]))
    gb, _ = O.gates(np.array([0.5]), np.zeros(1), np.array([0.5]), np.zeros(1))
    assert np.isclose(ga[0], gb[0], rtol=1e-15)


def test_synth_gates_follow_oracle_gates():
    """The workload generator's fp32 g and beta agree with the oracle's fp64 gate formula."""
    from gated_deltanet_delta_amd import synth
    wl = synth.WORKLOADS["prefill"]
    x = synth.make(wl, T=64)
    raw = x["raw"]
    g, beta = O.gates(raw["a"], raw["b"], raw["A_log"], raw["dt_bias"])
    assert np.max(np.abs(raw["g"] - g) / np.abs(g)) < 1e-6
    assert np.max(np.abs(raw["beta"] - beta)) < 1e-6
    assert np.all(raw["g"] < 0)


# ----------------------------------------------------------------------------------------------
# gated RMSNorm

def test_gated_rmsnorm_hand_worked():
    """d = 2 by hand: x = (3, 4) has mean square 12.5, so x / rms = (3, 4) / sqrt(12.5) =
    (0.848528..., 1.131370...); weight (2, 0.5); z = (0, 2): silu(0) = 0, silu(2) = 2 / (1 + e^-2)
    = 1.761594...; so y = (0, 1.131371 * 0.5 * 1.761594) = (0, 0.996508...)."""
    y = O.gated_rmsnorm(np.array([3.0, 4.0]), np.array([0.0, 2.0]), np.array([2.0, 0.5]), 0.0)
    assert y[0] == 0.0
    assert np.isclose(y[1], 4.0 / np.sqrt(12.5) * 0.5 * 2.0 / (1.0 + np.exp(-2.0)), rtol=1e-15)
    assert np.isclose(y[1], 0.9965081, rtol=1e-6)


def test_gated_rmsnorm_closed_forms():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 7, 64))
    w = rng.uniform(0.5, 1.5, 64)
    big = np.full_like(x, 40.0)                 # silu(z) = z (to 1e-17) for z = 40
    y = O.gated_rmsnorm(x, big, np.ones(64), 0.0)
    # with weight 1 and a constant gate, the rows have rms exactly 40
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 40.0, rtol=1e-12)
    # scale invariance (eps = 0), sign equivariance
    assert np.allclose(O.gated_rmsnorm(3.7 * x, big, w, 0.0), O.gated_rmsnorm(x, big, w, 0.0), rtol=1e-12)
    assert np.allclose(O.gated_rmsnorm(-x, big, w, 0.0), -O.gated_rmsnorm(x, big, w, 0.0), rtol=1e-12)
    # a zero gate closes the output, a very negative gate nearly does
    assert np.all(O.gated_rmsnorm(x, np.zeros_like(x), w, 1e-6) == 0.0)
    assert np.max(np.abs(O.gated_rmsnorm(x, np.full_like(x, -40.0), w, 1e-6))) < 1e-14
    # the gate and the weight act per channel and commute
    z = rng.standard_normal(x.shape)
    assert np.allclose(O.gated_rmsnorm(x, z, w, 1e-6), O.gated_rmsnorm(x, z, np.ones(64), 1e-6) * w)
    # eps only matters against the mean square: a zero row stays zero, a tiny row is damped
    assert np.all(O.gated_rmsnorm(np.zeros(8), np.ones(8), np.ones(8), 1e-6) == 0.0)
    small = O.gated_rmsnorm(np.full(8, 1e-6), np.full(8, 40.0), np.ones(8), 1e-6)
    assert np.allclose(small, 40.0 * 1e-6 / np.sqrt(1e-12 + 1e-6), rtol=1e-12)


# ----------------------------------------------------------------------------------------------
# causal conv1d

def test_conv1d_impulse_response():
    """A unit impulse at t0 in channel c returns that channel's taps reversed: y[t0 + i] = w[c, W-1-i]."""
    rng = np.random.default_rng(4)
    C, W, L, t0 = 3, 5, 12, 4
    w = rng.standard_normal((C, W))
    x = np.zeros((L, C))
    x[t0, 1] = 1.0
    y, st = O.causal_conv1d(x, w)
    for i in range(W):
        assert y[t0 + i, 1] == w[1, W - 1 - i]
    assert np.all(y[:t0] == 0) and np.all(y[t0 + W:] == 0) and np.all(y[:, [0, 2]] == 0)
    assert st.shape == (W - 1, C) and np.all(st == x[L - W + 1:])


def test_conv1d_equals_numpy_convolve():
    """Per channel the causal conv is the full convolution with the taps reversed, cut to the first L."""
    rng = np.random.default_rng(5)
    C, W, L = 4, 4, 30
    w, x, b = rng.standard_normal((C, W)), rng.standard_normal((L, C)), rng.standard_normal(C)
    y, _ = O.causal_conv1d(x, w, b)
    for c in range(C):
        ref = np.convolve(x[:, c], w[c, ::-1])[:L] + b[c]
        assert np.allclose(y[:, c], ref, rtol=1e-13, atol=1e-13)


def test_conv1d_split_and_carry():
    """Two calls carrying the cache equal one call over the concatenation, for every cut, including
    pieces shorter than the W-1 rows of the cache (and empty ones)."""
    rng = np.random.default_rng(6)
    C, W, L = 3, 6, 17
    w, x, s0 = rng.standard_normal((C, W)), rng.standard_normal((L, C)), rng.standard_normal((W - 1, C))
    y, s = O.causal_conv1d(x, w, None, s0, silu=True)
    for cut in range(L + 1):
        y1, s1 = O.causal_conv1d(x[:cut], w, None, s0, silu=True)
        y2, s2 = O.causal_conv1d(x[cut:], w, None, s1, silu=True)
        assert np.allclose(np.concatenate([y1, y2]), y, rtol=1e-13, atol=1e-13)
        assert np.array_equal(s2, s)
    # an empty piece leaves the cache as it was
    _, same = O.causal_conv1d(x[:0], w, None, s0)
    assert np.array_equal(same, s0)


def test_conv1d_silu_and_width_one():
    rng = np.random.default_rng(7)
    x, w = rng.standard_normal((9, 2)), rng.standard_normal((2, 1))
    y, st = O.causal_conv1d(x, w, silu=True)             # W = 1: a per-channel scale, no cache
    lin = x * w[:, 0]
    assert np.allclose(y, lin / (1.0 + np.exp(-lin)), rtol=1e-14) and st.shape == (0, 2)


# ----------------------------------------------------------------------------------------------
# q/k L2 normalisation

def test_l2norm_hand_worked_and_library():
    """(3, 4) has length 5; at eps = 0 the step is x / numpy.linalg.norm(x); a zero vector stays zero."""
    y = O.l2norm(np.array([3.0, 4.0]), eps=0.0)
    assert np.array_equal(y, np.array([0.6, 0.8]))
    y = O.l2norm(np.array([3.0, 4.0]))                    # eps = 1e-6 inside the root: 5.0000001
    assert np.allclose(y, np.array([3.0, 4.0]) / np.sqrt(25.000001), rtol=1e-15)
    rng = np.random.default_rng(8)
    x = rng.standard_normal((5, 3, 16))
    ref = x / np.linalg.norm(x, axis=-1, keepdims=True)
    assert np.allclose(O.l2norm(x, eps=0.0), ref, rtol=1e-14, atol=0)
    assert np.array_equal(O.l2norm(np.zeros((2, 4))), np.zeros((2, 4)))


def test_l2norm_scale_invariance_and_unit_inputs():
    """Rescaling a vector leaves its normalised form unchanged up to eps; unit vectors only lose the
    factor 1 / sqrt(1 + eps)."""
    rng = np.random.default_rng(9)
    x = rng.standard_normal((4, 32))
    for c in (1e-2, 7.0, 1e3):
        assert np.allclose(O.l2norm(c * x, eps=0.0), O.l2norm(x, eps=0.0), rtol=1e-14, atol=0)
    u = x / np.linalg.norm(x, axis=-1, keepdims=True)
    assert np.allclose(O.l2norm(u), u / np.sqrt(1.0 + 1e-6), rtol=1e-14, atol=0)


def test_l2norm_makes_the_correction_an_overwrite(orc):
    """With a key of length 3 along e0 and beta = 1, g = 0, normalising the key turns the correction
    into an exact overwrite: from S0 = e0 w^T the state becomes e0 v^T and a query along e0 reads v.
    Unnormalised, (I - 9 e0 e0^T) would flip and amplify the stored row instead."""
    dk = dv = 4
    q = np.zeros((1, 1, 1, dk)); q[..., 0] = 2.0
    k = np.zeros((1, 1, 1, dk)); k[..., 0] = 3.0
    v = np.arange(1.0, dv + 1).reshape(1, 1, 1, dv)
    g, beta = np.zeros((1, 1, 1)), np.ones((1, 1, 1))
    s0 = np.zeros((1, 1, dk, dv)); s0[0, 0, 0] = [5.0, -1.0, 2.0, 0.5]
    o, fs = orc.forward(O.l2norm(q, eps=0.0), O.l2norm(k, eps=0.0), v, g, beta, s0)
    want = np.zeros((dk, dv)); want[0] = v[0, 0, 0]
    assert np.array_equal(fs[0, 0], want) and np.array_equal(o[0, 0, 0], v[0, 0, 0])
    _, raw = orc.forward(q, k, v, g, beta, s0)
    assert raw[0, 0, 0, 0] == (1 - 9) * 5.0 + 3.0 * 1.0


# ----------------------------------------------------------------------------------------------
# backward pass

def _fd_case(rng, lens, Hk, Hv, dk, dv, with_state):
    T = int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    N = len(lens)
    k = rng.standard_normal((1, T, Hk, dk))
    k = 0.9 * k / np.linalg.norm(k, axis=-1, keepdims=True)
    x = dict(q=rng.standard_normal((1, T, Hk, dk)), k=k, v=rng.standard_normal((1, T, Hv, dv)),
             g=-rng.uniform(0.01, 0.5, (1, T, Hv)), beta=rng.uniform(0.1, 0.9, (1, T, Hv)),
             s0=rng.standard_normal((N, Hv, dk, dv)) if with_state else None)
    return x, cu


def pin_backward_fd(orc, lens=(5, 0, 70), with_state=True, with_dfinal=True):
    """Every gradient element equals the central difference of L = <w_o, o> + <w_S, S_T> computed with
    the forward oracle (h = 1e-5, error O(h^2)): packed sequences (an empty one, one longer than the
    backward's 64-token recompute pieces), two v-heads sharing a q/k head (dq, dk sum over both)."""
    rng = np.random.default_rng(20 + len(lens))
    Hk, Hv, dk, dv = 1, 2, 3, 2
    x, cu = _fd_case(rng, lens, Hk, Hv, dk, dv, with_state)
    wo = rng.standard_normal((1, int(sum(lens)), Hv, dv))
    ws = rng.standard_normal((len(lens), Hv, dk, dv)) if with_dfinal else None

    def loss(xx):
        o, fs = orc.forward(xx["q"], xx["k"], xx["v"], xx["g"], xx["beta"], xx["s0"], cu)
        return float(np.sum(wo * o) + (np.sum(ws * fs) if ws is not None else 0.0))

    grads = dict(zip(("q", "k", "v", "g", "beta", "s0"),
                     orc.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], wo, x["s0"], ws, cu)))
    h = 1e-5
    for name in ("q", "k", "v", "g", "beta", "s0"):
        if x[name] is None:
            continue
        fd = np.zeros_like(x[name])
        for idx in np.ndindex(x[name].shape):
            xp = {key: (val.copy() if val is not None else None) for key, val in x.items()}
            xm = {key: (val.copy() if val is not None else None) for key, val in x.items()}
            xp[name][idx] += h
            xm[name][idx] -= h
            fd[idx] = (loss(xp) - loss(xm)) / (2 * h)
        assert np.allclose(grads[name], fd, rtol=1e-6, atol=1e-8), (name, np.max(np.abs(grads[name] - fd)))


@pytest.mark.parametrize("lens,with_state,with_dfinal", [((5, 0, 70), True, True), ((12,), False, False)])
def test_backward_matches_finite_differences(orc, lens, with_state, with_dfinal):
    pin_backward_fd(orc, lens, with_state, with_dfinal)


@pytest.mark.parametrize("qk_l2norm,raw", [(False, True), (True, True), (True, False)])
def test_backward_ex_matches_finite_differences(orc, qk_l2norm, raw):
    """The gradients through the input steps (raw gates a, b, A_log, dt_bias; q, k normalised) equal
    central differences of the composed forward oracle, for every element of every input.  Without
    raw gates (A_log None) the gates enter as g and beta themselves."""
    rng = np.random.default_rng(30 + qk_l2norm + 2 * raw)
    lens, Hk, Hv, dk, dv = (3, 0, 9), 1, 2, 3, 2
    T, N = sum(lens), len(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    x = dict(q=rng.standard_normal((1, T, Hk, dk)), k=rng.standard_normal((1, T, Hk, dk)),
             v=rng.standard_normal((1, T, Hv, dv)), a=rng.standard_normal((1, T, Hv)),
             b=rng.standard_normal((1, T, Hv)), A_log=np.log(rng.uniform(0.2, 2.0, Hv)),
             dt_bias=0.3 * rng.standard_normal(Hv), s0=rng.standard_normal((N, Hv, dk, dv)))
    if not raw:   # g <= 0 and beta in (0, 1) drawn directly
        x["a"] = -rng.uniform(0.0, 1.5, (1, T, Hv))
        x["b"] = rng.uniform(0.05, 0.95, (1, T, Hv))
        del x["A_log"], x["dt_bias"]
    wo = rng.standard_normal((1, T, Hv, dv))
    ws = rng.standard_normal((N, Hv, dk, dv))

    def loss(xx):
        if raw:
            g, beta = O.gates(xx["a"], xx["b"], xx["A_log"], xx["dt_bias"])
        else:
            g, beta = xx["a"], xx["b"]
        q, k = (O.l2norm(xx["q"]), O.l2norm(xx["k"])) if qk_l2norm else (xx["q"], xx["k"])
        o, fs = orc.forward(q, k, xx["v"], g, beta, xx["s0"], cu)
        return float(np.sum(wo * o) + np.sum(ws * fs))

    out = O.backward_ex(x["q"], x["k"], x["v"], x["a"], x["b"], x.get("A_log"), x.get("dt_bias"), wo, x["s0"],
                        ws, cu, qk_l2norm=qk_l2norm)
    got = dict(zip(("q", "k", "v", "a", "b", "A_log", "dt_bias", "s0"), out))
    if not raw:
        assert got["A_log"] is None and got["dt_bias"] is None
    h = 1e-5
    for name, val in x.items():
        fd = np.zeros_like(val)
        for idx in np.ndindex(val.shape):
            xp = {key: vv.copy() for key, vv in x.items()}
            xm = {key: vv.copy() for key, vv in x.items()}
            xp[name][idx] += h
            xm[name][idx] -= h
            fd[idx] = (loss(xp) - loss(xm)) / (2 * h)
        assert np.allclose(got[name], fd, rtol=1e-6, atol=1e-8), (name, np.max(np.abs(got[name] - fd)))


def test_backward_without_writes_is_a_pure_decay(orc):
    """beta = 0: nothing is written, so k and v get no gradient at all and S_t = e^{G_t} S0, whence
    dq_t = e^{G_t} S0 do_t and dS0 = sum_t e^{G_t} q_t do_t^T (one sequence, one head)."""
    rng = np.random.default_rng(27)
    T, dk, dv = 9, 3, 4
    q, k = rng.standard_normal((1, T, 1, dk)), rng.standard_normal((1, T, 1, dk))
    v = rng.standard_normal((1, T, 1, dv))
    g = -rng.uniform(0.0, 0.7, (1, T, 1))
    beta = np.zeros((1, T, 1))
    s0 = rng.standard_normal((1, 1, dk, dv))
    do = rng.standard_normal((1, T, 1, dv))
    dq, dkk, dvv, dg, db, ds0 = orc.backward(q, k, v, g, beta, do, s0)
    assert np.all(dkk == 0.0) and np.all(dvv == 0.0)
    G = np.cumsum(g[0, :, 0])
    for t in range(T):
        assert np.allclose(dq[0, t, 0], np.exp(G[t]) * s0[0, 0] @ do[0, t, 0], rtol=1e-13)
    want = sum(np.exp(G[t]) * np.outer(q[0, t, 0], do[0, t, 0]) for t in range(T))
    assert np.allclose(ds0[0, 0], want, rtol=1e-13)


# ----------------------------------------------------------------------------------------------
# sampling and threading do not change results

def test_unit_mask_and_threads(orc):
    rng = np.random.default_rng(12)
    q, k, v, g, beta, s0 = rand_inputs(rng, B=3, T=11, Hk=2, Hv=4, dk=5, dv=3)
    o, fs = orc.forward(q, k, v, g, beta, s0, threads=1)
    mask = np.zeros((3, 4), bool)
    mask[1, 2] = mask[2, 0] = True
    om, fm = orc.forward(q, k, v, g, beta, s0, unit_mask=mask, threads=3)
    for n, h in zip(*np.nonzero(mask)):
        assert np.array_equal(om[n, :, h], o[n, :, h])
        assert np.array_equal(fm[n, h], fs[n, h])
    assert np.isnan(om[0, :, 0]).all()


def test_rejects_bad_arguments(orc):
    rng = np.random.default_rng(13)
    q, k, v, g, beta, s0 = rand_inputs(rng, T=4, Hk=2, Hv=3)
    with pytest.raises(ValueError):
        orc.forward(q, k, v, g, beta, None)  # Hv % Hk != 0
    q, k, v, g, beta, s0 = rand_inputs(rng, T=4)
    with pytest.raises(ValueError):
        orc.forward(q, k, v, g, beta, None, cu_seqlens=np.array([0, 3, 2], np.int32))


# ----------------------------------------------------------------------------------------------
# the pins are strong enough: planted mistakes in the C oracle each fail at least one of them

MUTANTS = {
    "no_decay": ("for (size_t e = 0; e < SS; ++e) S[e] *= a;", ";"),
    "decay_sign": ("const double a = exp(gt);", "const double a = exp(-gt);"),
    "delta_sign": ("u[j] = bt * (vt[j] - p[j]);", "u[j] = bt * (vt[j] + p[j]);"),
    "no_beta": ("u[j] = bt * (vt[j] - p[j]);", "u[j] = (vt[j] - p[j]);"),
    "predict_with_q": ("p[j] += Si[j] * ki;", "p[j] += Si[j] * qt[i];"),
    "correct_with_q": ("Si[j] += ki * u[j];", "Si[j] += qt[i] * u[j];"),
    "read_transposed": ("ot[j] += Si[j] * qi;", "ot[j] += S[(size_t)j * dv + i] * qi;"),
    "read_with_k": ("ot[j] += Si[j] * qi;", "ot[j] += Si[j] * kt[i];"),
    "interleaved_heads": ("const int kh = h / (Hv / Hk);", "const int kh = h % Hk;"),
    "ignore_initial_state": ("if (s0) memcpy", "if (0) memcpy"),
    "gate_of_head0": ("const double gt = g[row * Hv + h];", "const double gt = g[row * Hv];"),
    "drop_last_token": ("const int t1 = cu_seqlens ? cu_seqlens[n + 1] : T;",
                        "const int t1 = cu_seqlens ? cu_seqlens[n + 1] : T - 1;"),
}


BACKWARD_MUTANTS = {
    "bw_drop_predict_term": ("dkt[i] += st * dp[j];", ";"),
    "bw_dg_sign": ("dgt += st * dS[e];", "dgt -= st * dS[e];"),
    "bw_undecayed_D": ("for (size_t e = 0; e < SS; ++e) D[e] = a * dS[e];",
                       "for (size_t e = 0; e < SS; ++e) D[e] = dS[e];"),
    "bw_dbeta_from_v": ("db += du[j] * pv[j];", "db += du[j] * vt[j];"),
    "bw_dq_from_previous_state": ("dqt[i] += St[(size_t)i * dv + j] * dot[j];",
                                  "dqt[i] += Sp[(size_t)i * dv + j] * dot[j];"),
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name", sorted(BACKWARD_MUTANTS))
def test_backward_pin_catches_planted_mistakes(tmp_path, name):
    """The finite-difference pin fails for each typical slip planted in the backward pass (the
    mutant's forward is untouched, so its differences are still the true gradients)."""
    src = open(O.SOURCE).read()
    find, repl = BACKWARD_MUTANTS[name]
    assert src.count(find) == 1, f"mutation site for {name} no longer in the oracle source"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(find, repl))
    lib = str(tmp_path / "libmutant.so")
    subprocess.run(["gcc", "-O1", "-fopenmp", "-shared", "-fPIC", "-std=c99", str(path), "-o", lib, "-lm"],
                   check=True)
    with pytest.raises(AssertionError):
        pin_backward_fd(O.Oracle(lib))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(tmp_path, name):
    src = open(O.SOURCE).read()
    find, repl = MUTANTS[name]
    assert src.count(find) == 1, f"mutation site for {name} no longer in the oracle source"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(find, repl))
    lib = str(tmp_path / "libmutant.so")
    subprocess.run(["gcc", "-O1", "-fopenmp", "-shared", "-fPIC", "-std=c99", str(path), "-o", lib, "-lm"],
                   check=True)
    mutant = O.Oracle(lib)
    caught = []
    for pin in PINS:
        try:
            pin(mutant)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name}"
