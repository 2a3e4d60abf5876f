"""The oracle: plain, slow, obviously correct CPU versions of what the GPU path computes.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module.  It shares no code with the HIP library (``gated_deltanet_delta_amd``) and never
imports it; the library never imports this.

Contents
--------
``forward``  the gated delta rule token by token in fp64 (``gdn_oracle.c``, compiled with gcc).  It
             serves both entry points: a prefill is one call over whole sequences, a decode step is
             the same call over length-1 sequences.
``gates``    the gate formulas of the Qwen3.5 Gated DeltaNet flowchart (wanger-sjtu.github.io,
             "Qwen3.5 Gated DeltaNet core-mechanism" page, flowchart nodes "Sigmoid -> beta",
             "Softplus + dt_bias", "Exp and Neg", "Mul -> g") and of the Qwen3-Next architecture
             write-up (intelliparadigm.com, section 2.2 "linear attention module", step 2 "gate
             generation"), in fp64.
``gated_rmsnorm``  the output norm of the layer (the Qwen3.5 page's "Output and gated RMSNorm"
             section): each head vector of the core output is RMS-normalised, scaled by a learned
             per-channel weight and gated by the z branch through SiLU, in fp64 numpy.
``causal_conv1d``  the depthwise causal convolution the QKV mixture passes through before the rule
             (the Qwen3.5 page's flowchart node "conv1d, Depthwise Causal Conv" and its
             conv_states cache), per sequence, carrying the last inputs in fp64 numpy.
``backward`` the gradients of ``forward`` (reverse-mode over its token steps, fp64, in
             ``gdn_oracle.c``), for the training direction of the chunked call.
``backward_ex`` the same with the layer's input steps (raw gates, q/k normalisation) differentiated
             through as well.
``l2norm``   the optional normalisation of each q and k head vector to unit length before the rule
             (a reading: the pages do not state how q and k are scaled), in fp64 numpy.
``chunked``  the chunk-parallel (WY/UT) form of the same rule in fp64 numpy.  It is not the
             definition: it exists to show, against ``forward``, that the block algebra a chunked
             kernel uses reaches the token-by-token result exactly (up to rounding order).

Every function here is pinned by ``tests/test_oracle.py`` against closed forms, a hand-worked example
(``tests/golden/``), brute-force transition products and invariants.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "gdn_oracle.c")
LIBRARY = os.path.join(HERE, "libgdn_oracle.so")


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the C oracle with gcc (plain -O2, OpenMP, no target-specific flags)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99", "-Wall", source, "-o", output, "-lm"]
    subprocess.run(cmd, check=True)
    return output


class Oracle:
    """ctypes view of one compiled oracle library (the real one, or a test's mutant)."""

    def __init__(self, path: str = LIBRARY):
        if path == LIBRARY and (
            not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(SOURCE)
        ):
            build()
        self.path = path
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.gdn_oracle_forward.restype = ctypes.c_int
        lib.gdn_oracle_forward.argtypes = [
            dp, dp, dp, dp, dp, dp, ctypes.POINTER(ctypes.c_int32),
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.POINTER(ctypes.c_ubyte), ctypes.c_int, dp, dp,
        ]
        lib.gdn_oracle_default_threads.restype = ctypes.c_int
        lib.gdn_oracle_backward.restype = ctypes.c_int
        lib.gdn_oracle_backward.argtypes = [
            dp, dp, dp, dp, dp, dp, ctypes.POINTER(ctypes.c_int32),
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, dp, dp, ctypes.c_int, dp, dp, dp, dp, dp, dp,
        ]
        self._lib = lib

    def default_threads(self) -> int:
        return int(self._lib.gdn_oracle_default_threads())

    def forward(
        self,
        q: np.ndarray,
        k: np.ndarray,
        v: np.ndarray,
        g: np.ndarray,
        beta: np.ndarray,
        initial_state: Optional[np.ndarray] = None,
        cu_seqlens: Optional[np.ndarray] = None,
        unit_mask: Optional[np.ndarray] = None,
        threads: int = 0,
    ) -> Tuple[np.ndarray, np.ndarray]:
        """(o, final_state) in fp64 for q,k [B,T,Hk,dk], v [B,T,Hv,dv], g,beta [B,T,Hv].

        ``initial_state`` is [N,Hv,dk,dv] or None (zeros).  ``cu_seqlens`` (int32 [N+1], B == 1)
        packs N sequences along T; without it N == B.  ``unit_mask`` (bool [N,Hv]) restricts the run
        to a sample of (sequence, v-head) units; o rows and states of skipped units are NaN.
        """
        B, T, Hk, dk = q.shape
        Hv, dv = v.shape[2], v.shape[3]
        if k.shape != q.shape or v.shape[:2] != (B, T) or g.shape != (B, T, Hv) or beta.shape != g.shape:
            raise ValueError("inconsistent shapes")
        N = B if cu_seqlens is None else len(cu_seqlens) - 1
        arrs = [np.ascontiguousarray(x, dtype=np.float64) for x in (q, k, v, g, beta)]
        s0 = None if initial_state is None else np.ascontiguousarray(initial_state, dtype=np.float64)
        if s0 is not None and s0.shape != (N, Hv, dk, dv):
            raise ValueError("initial_state shape")
        cu = None if cu_seqlens is None else np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        mask = None if unit_mask is None else np.ascontiguousarray(unit_mask, dtype=np.uint8).reshape(N * Hv)
        o = np.full((B, T, Hv, dv), np.nan)
        fs = np.full((N, Hv, dk, dv), np.nan)
        dp = ctypes.POINTER(ctypes.c_double)
        ptr = lambda a: a.ctypes.data_as(dp)  # noqa: E731
        rc = self._lib.gdn_oracle_forward(
            *(ptr(a) for a in arrs),
            None if s0 is None else ptr(s0),
            None if cu is None else cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
            B, T, Hk, Hv, dk, dv, N,
            None if mask is None else mask.ctypes.data_as(ctypes.POINTER(ctypes.c_ubyte)),
            int(threads), ptr(o), ptr(fs),
        )
        if rc != 0:
            raise ValueError(f"gdn_oracle_forward returned {rc}")
        return o, fs


    def backward(
        self,
        q: np.ndarray,
        k: np.ndarray,
        v: np.ndarray,
        g: np.ndarray,
        beta: np.ndarray,
        d_o: np.ndarray,
        initial_state: Optional[np.ndarray] = None,
        d_final: Optional[np.ndarray] = None,
        cu_seqlens: Optional[np.ndarray] = None,
        threads: int = 0,
    ) -> Tuple[np.ndarray, ...]:
        """Gradients (dq, dk, dv, dg, dbeta, d_initial_state) in fp64 of a scalar loss whose
        gradients with respect to the outputs are ``d_o`` [B,T,Hv,dv] and ``d_final``
        [N,Hv,dk,dv] (None: zero): reverse-mode differentiation of ``forward``'s token steps
        (``gdn_oracle_backward`` in ``gdn_oracle.c``)."""
        B, T, Hk, dk = q.shape
        Hv, dv = v.shape[2], v.shape[3]
        if k.shape != q.shape or v.shape[:2] != (B, T) or g.shape != (B, T, Hv) or beta.shape != g.shape:
            raise ValueError("inconsistent shapes")
        if d_o.shape != v.shape:
            raise ValueError("d_o shape")
        N = B if cu_seqlens is None else len(cu_seqlens) - 1
        arrs = [np.ascontiguousarray(x, dtype=np.float64) for x in (q, k, v, g, beta)]
        s0 = None if initial_state is None else np.ascontiguousarray(initial_state, dtype=np.float64)
        df = None if d_final is None else np.ascontiguousarray(d_final, dtype=np.float64)
        for x, what in ((s0, "initial_state"), (df, "d_final")):
            if x is not None and x.shape != (N, Hv, dk, dv):
                raise ValueError(what + " shape")
        do = np.ascontiguousarray(d_o, dtype=np.float64)
        cu = None if cu_seqlens is None else np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        outs = [np.full(a.shape, np.nan) for a in arrs] + [np.full((N, Hv, dk, dv), np.nan)]
        dp = ctypes.POINTER(ctypes.c_double)
        ptr = lambda a: a.ctypes.data_as(dp)  # noqa: E731
        rc = self._lib.gdn_oracle_backward(
            *(ptr(a) for a in arrs),
            None if s0 is None else ptr(s0),
            None if cu is None else cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
            B, T, Hk, Hv, dk, dv, N, ptr(do), None if df is None else ptr(df), int(threads),
            *(ptr(a) for a in outs),
        )
        if rc != 0:
            raise ValueError(f"gdn_oracle_backward returned {rc}")
        return tuple(outs)


_default: Optional[Oracle] = None


def _oracle() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def forward(*args, **kwargs) -> Tuple[np.ndarray, np.ndarray]:
    """Token-by-token fp64 gated delta rule; see ``Oracle.forward``."""
    return _oracle().forward(*args, **kwargs)


def backward(*args, **kwargs) -> Tuple[np.ndarray, ...]:
    """Gradients of the token-by-token rule; see ``Oracle.backward``."""
    return _oracle().backward(*args, **kwargs)


def backward_ex(q, k, v, a, b, A_log, dt_bias, d_o, initial_state=None, d_final=None, cu_seqlens=None,
                qk_l2norm=False, eps=1e-6):
    """Gradients of the layer call with its options, fp64: q, k raw (normalised first when
    ``qk_l2norm``), gates from the raw projections a, b [B,T,Hv] and A_log, dt_bias [Hv] (with
    ``A_log`` None, a and b are g and beta themselves and there is no gate step).

    Returns (dq, dk, dv, da, db, dA_log, ddt_bias, d_initial_state), dA_log and ddt_bias None without
    a gate step.  Composition of ``backward`` with the derivatives of the two input steps, written
    from their formulas:
      beta = sigmoid(b):                     db = dbeta * beta (1 - beta)
      g = -exp(A_log) softplus(a + dt_bias):  da = dg * (-exp(A_log) sigmoid(a + dt_bias)),
                                              dA_log = sum over tokens of dg * g, ddt_bias = sum of da
      x^ = x r, r = 1 / sqrt(|x|^2 + eps):    dx = r dx^ - r^3 (x . dx^) x
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if A_log is None:
        g, beta = a, b
    else:
        A_log = np.asarray(A_log, dtype=np.float64)
        dt_bias = np.asarray(dt_bias, dtype=np.float64)
        g, beta = gates(a, b, A_log, dt_bias)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    qn, kn = (l2norm(q, eps), l2norm(k, eps)) if qk_l2norm else (q, k)
    dqn, dkn, dv, dg, dbeta, ds0 = backward(qn, kn, v, g, beta, d_o, initial_state, d_final, cu_seqlens)

    def through_norm(x, dxn):
        r = 1.0 / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)
        return r * dxn - r ** 3 * np.sum(x * dxn, axis=-1, keepdims=True) * x

    dq = through_norm(q, dqn) if qk_l2norm else dqn
    dk = through_norm(k, dkn) if qk_l2norm else dkn
    if A_log is None:
        return dq, dk, dv, dg, dbeta, None, None, ds0
    db = dbeta * beta * (1.0 - beta)
    da = dg * (-np.exp(A_log) / (1.0 + np.exp(-(a + dt_bias))))
    if cu_seqlens is not None:   # tokens outside every sequence carry no gradient
        inside = np.zeros(a.shape[1], dtype=bool)
        inside[int(cu_seqlens[0]):int(cu_seqlens[-1])] = True
        da = np.where(inside[None, :, None], da, 0.0)
        dg = np.where(inside[None, :, None], dg, 0.0)
        db = np.where(inside[None, :, None], db, 0.0)
    dA_log = np.sum(dg * g, axis=(0, 1))
    ddt = np.sum(da, axis=(0, 1))
    return dq, dk, dv, da, db, dA_log, ddt, ds0


def default_threads() -> int:
    return _oracle().default_threads()


def gates(a: np.ndarray, b: np.ndarray, A_log: np.ndarray, dt_bias: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """(g, beta) in fp64 from the raw per-token projections a, b [..., H] and per-head A_log, dt_bias [H].

    Qwen3.5 flowchart (wanger-sjtu.github.io) and the Qwen3-Next write-up (intelliparadigm.com §2.2):
    beta = sigmoid(b) is the write strength; g = -exp(A_log) * softplus(a + dt_bias) is the log-decay,
    always <= 0, so the per-token decay factor exp(g) lies in (0, 1].  (The jsqmd.com article's §2.1
    swaps the two names; its "beta" is negative and cannot be a strength in (0,1), so its labels are
    not followed.)
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    x = a + np.asarray(dt_bias, dtype=np.float64)
    softplus = np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))
    g = -np.exp(np.asarray(A_log, dtype=np.float64)) * softplus
    beta = 1.0 / (1.0 + np.exp(-b))
    return g, beta


def gated_rmsnorm(x: np.ndarray, z: np.ndarray, weight: np.ndarray, eps: float) -> np.ndarray:
    """y = x / sqrt(mean(x^2) + eps) * weight * silu(z) over the last axis (one head vector), fp64.

    Qwen3.5 Gated DeltaNet page (wanger-sjtu.github.io), section "Output and gated RMSNorm" and the
    flowchart nodes "AttnOut -> Norm (Qwen3_5MoeRMSNormGated or FusedRMSNormGated)", "Z -> Norm":
    the core output is normalised and then gated by z in the manner of SwiGLU, i.e. multiplied by
    silu(z) = z * sigmoid(z).  The normalisation is RMSNorm over the head dimension with a learned
    per-channel weight; the Qwen3-Next article's section 3.2 shows the same rsqrt(mean(x^2) + eps)
    normalisation for the model's other norms.  (Reading taken: the weight multiplies directly; the
    "1 + weight" zero-centred form of that section belongs to the non-gated norms.)
    """
    x = np.asarray(x, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    inv_rms = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    silu = z / (1.0 + np.exp(-z))
    return x * inv_rms * w * silu


def l2norm(x: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """x / sqrt(sum(x^2) + eps) over the last axis (one q or k head vector), fp64.

    Not on the pages, which feed q and k to the rule without stating their scale.  The rule corrects
    the state along the current key (Qwen3.5 page, "core mechanism": the old value stored along k is
    replaced by the new one in proportion beta); that correction is an exact partial overwrite only
    for a unit key, for which I - beta k k^T scales the state's component along k by 1 - beta.  This
    step makes q and k unit vectors before the rule.  Reading taken for its form: a plain L2
    normalisation with eps inside the square root, eps = 1e-6 (the eps the Qwen3-Next article's
    section 3.2 uses for the model's RMS norms).
    """
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def causal_conv1d(x: np.ndarray, weight: np.ndarray, bias: Optional[np.ndarray] = None,
                  state: Optional[np.ndarray] = None, silu: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """One sequence: x [L, C], weight [C, W], bias [C] or None, state [W-1, C] (the W-1 inputs before
    this sequence, oldest first) or None for zeros.  Returns (y [L, C], new state [W-1, C]), fp64.

    Qwen3.5 Gated DeltaNet page (wanger-sjtu.github.io): the flowchart sends the QKV mixture through
    "conv1d, Depthwise Causal Conv" before it splits into q, k, v, reads "conv_states" on the decode
    path and ends in "Update Conv Cache"; its section on the convolution layer describes a causal
    convolution that gathers local context.  Depthwise: each channel has its own W taps.  Causal:
    output t sees inputs t-W+1 .. t only, the inputs before the sequence coming from the cache (zeros
    without one):
        y[t, c] = sum_j weight[c, j] * xp[t + j, c] + bias[c],   xp = [state; x]
    and the new cache holds the last W-1 rows of xp.  The kernel width varies across the pages (4, 8,
    12-16 by context length; 5 elsewhere), so W is a parameter.  The pages name no activation after
    the convolution: none is the default reading; ``silu`` applies x * sigmoid(x) to y for callers
    whose model has one.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    L, C = x.shape
    W = w.shape[1]
    st = np.zeros((W - 1, C)) if state is None else np.asarray(state, dtype=np.float64)
    xp = np.concatenate([st, x], axis=0)
    y = np.zeros((L, C))
    for t in range(L):
        for j in range(W):
            y[t] += w[:, j] * xp[t + j]
    if bias is not None:
        y += np.asarray(bias, dtype=np.float64)
    if silu:
        y = y / (1.0 + np.exp(-y))
    return y, xp[xp.shape[0] - (W - 1):].copy()


def chunked(
    q: np.ndarray,
    k: np.ndarray,
    v: np.ndarray,
    g: np.ndarray,
    beta: np.ndarray,
    initial_state: Optional[np.ndarray],
    chunk: int,
) -> Tuple[np.ndarray, np.ndarray]:
    """The chunk-parallel form, fp64, for one sequence: q,k [T,Hk,dk], v [T,Hv,dv], g,beta [T,Hv].

    Within a chunk of C tokens starting from state S0, with G_t the running sum of g inside the chunk,
    unrolling the per-token rule gives (rows are tokens):

        (I + A) U = diag(beta) V - diag(beta e^G) K S0,   A_tj = beta_t (k_t.k_j) e^(G_t - G_j), j < t
        O   = diag(e^G) Q S0 + P U,                         P_tj = (q_t.k_j) e^(G_t - G_j), j <= t
        S_C = e^(G_C) S0 + K^T diag(e^(G_C - G)) U

    so U = W~ - W S0 with W = (I+A)^-1 diag(beta e^G) K and W~ = (I+A)^-1 diag(beta) V.  Every decay
    factor is exp of a non-positive number.  The last chunk may be shorter than C.
    """
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    grp = Hv // Hk
    o = np.zeros((T, Hv, dv))
    fs = np.zeros((Hv, dk, dv))
    for h in range(Hv):
        kh = h // grp
        S = np.zeros((dk, dv)) if initial_state is None else np.array(initial_state[h], dtype=np.float64)
        for c0 in range(0, T, chunk):
            c1 = min(T, c0 + chunk)
            Q = np.asarray(q[c0:c1, kh], dtype=np.float64)
            K = np.asarray(k[c0:c1, kh], dtype=np.float64)
            V = np.asarray(v[c0:c1, h], dtype=np.float64)
            bt = np.asarray(beta[c0:c1, h], dtype=np.float64)
            G = np.cumsum(np.asarray(g[c0:c1, h], dtype=np.float64))
            L = c1 - c0
            diff = G[:, None] - G[None, :]
            lower_strict = np.tril(np.ones((L, L)), -1)
            lower = np.tril(np.ones((L, L)))
            decay_strict = np.exp(np.where(lower_strict > 0, diff, -np.inf))
            decay = np.exp(np.where(lower > 0, diff, -np.inf))
            A = bt[:, None] * (K @ K.T) * decay_strict
            Tinv = np.linalg.solve(np.eye(L) + A, np.eye(L))
            W = Tinv @ ((bt * np.exp(G))[:, None] * K)
            Wt = Tinv @ (bt[:, None] * V)
            U = Wt - W @ S
            P = (Q @ K.T) * decay
            o[c0:c1, h] = np.exp(G)[:, None] * (Q @ S) + P @ U
            S = np.exp(G[-1]) * S + K.T @ (np.exp(G[-1] - G)[:, None] * U)
        fs[h] = S
    return o, fs
