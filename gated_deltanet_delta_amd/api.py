"""Python binding of libgdn: argument marshalling only.

Every function here checks that the torch tensors it is handed have the shapes, dtypes, devices and
layouts the C ABI expects (the C library sees only pointers), allocates outputs and workspace with
torch when the caller does not pass them, and calls the library on torch's current stream.  All
arithmetic runs in the HIP kernels.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from . import _lib

_DTYPES = {torch.float32: _lib.GDN_F32, torch.bfloat16: _lib.GDN_BF16}


def _code(t: torch.Tensor, what: str) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"{what}: dtype {t.dtype} not supported (bfloat16 or float32)") from None


def _check(t: torch.Tensor, shape, what: str, device: torch.device, dtype=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what}: shape {tuple(t.shape)} != expected {tuple(shape)}")
    if t.device != device:
        raise ValueError(f"{what}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what}: dtype {t.dtype}, expected {dtype}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def workspace_size(B: int, T: int, Hk: int, Hv: int, dk: int, dv: int, N: int,
                   qkv_dtype: torch.dtype) -> int:
    """Bytes of workspace gdn_chunk_fwd needs (0 if none)."""
    return int(_lib.load().gdn_chunk_fwd_workspace_size(B, T, Hk, Hv, dk, dv, N, _DTYPES[qkv_dtype]))


def _chunk_call(fn, q, k, v, x, y, A_log, dt_bias, initial_state, cu_seqlens, o, final_state,
                workspace, gating: bool):
    lib = _lib.load()
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, T, H, d]")
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError(f"{fn.__name__} runs on a GPU; tensors must be on a cuda device")
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    xn, yn = ("a", "b") if gating else ("g", "beta")
    _check(q, (B, T, Hk, dk), "q", dev)
    _check(k, (B, T, Hk, dk), "k", dev, q.dtype)
    _check(v, (B, T, Hv, dv), "v", dev, q.dtype)
    _check(x, (B, T, Hv), xn, dev)
    _check(y, (B, T, Hv), yn, dev, x.dtype)
    if gating:
        _check(A_log, (Hv,), "A_log", dev, torch.float32)
        _check(dt_bias, (Hv,), "dt_bias", dev, torch.float32)
    if cu_seqlens is not None:
        _check(cu_seqlens, (N + 1,), "cu_seqlens", dev, torch.int32)
    if initial_state is not None:
        _check(initial_state, (N, Hv, dk, dv), "initial_state", dev, torch.float32)
    if o is None:
        o = torch.empty((B, T, Hv, dv), dtype=torch.float32, device=dev)
    _check(o, (B, T, Hv, dv), "o", dev, torch.float32)
    if final_state is None:
        final_state = torch.empty((N, Hv, dk, dv), dtype=torch.float32, device=dev)
    _check(final_state, (N, Hv, dk, dv), "final_state", dev, torch.float32)
    qkv, gate = _code(q, "q"), _code(x, xn)
    ws_bytes = int(lib.gdn_chunk_fwd_workspace_size(B, T, Hk, Hv, dk, dv, N, qkv))
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    if workspace is not None:
        if workspace.device != dev or workspace.numel() * workspace.element_size() < ws_bytes:
            raise ValueError(f"workspace must hold {ws_bytes} bytes on {dev}")
    gates = (_ptr(A_log), _ptr(dt_bias)) if gating else ()
    st = fn(
        _ptr(q), _ptr(k), _ptr(v), _ptr(x), _ptr(y), *gates, _ptr(initial_state), _ptr(cu_seqlens),
        B, T, Hk, Hv, dk, dv, N, qkv, gate, _ptr(o), _ptr(final_state), _ptr(workspace),
        ctypes.c_size_t(0 if workspace is None else workspace.numel() * workspace.element_size()),
        _stream(dev))
    if st != _lib.GDN_SUCCESS:
        raise _lib.GdnError(st, fn.__name__)
    return o, final_state


def gdn_chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                  beta: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
                  cu_seqlens: Optional[torch.Tensor] = None, *, o: Optional[torch.Tensor] = None,
                  final_state: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None,
                  stage: str = "all") -> Tuple[torch.Tensor, torch.Tensor]:
    """Chunk-parallel prefill.  q,k [B,T,Hk,dk]; v [B,T,Hv,dv]; g,beta [B,T,Hv];
    initial_state [N,Hv,dk,dv] fp32 or None; cu_seqlens int32 [N+1] (B == 1) or None.
    Returns (o [B,T,Hv,dv] fp32, final_state [N,Hv,dk,dv] fp32).

    ``stage`` selects gdn_chunk_fwd ("all"), gdn_chunk_fwd_prepare ("prepare") or
    gdn_chunk_fwd_scan ("scan"); the halves must be called in that order with the same tensors
    and workspace."""
    lib = _lib.load()
    try:
        fn = {"all": lib.gdn_chunk_fwd, "prepare": lib.gdn_chunk_fwd_prepare,
              "scan": lib.gdn_chunk_fwd_scan}[stage]
    except KeyError:
        raise ValueError(f"stage must be 'all', 'prepare' or 'scan', not {stage!r}") from None
    return _chunk_call(fn, q, k, v, g, beta, None, None, initial_state, cu_seqlens, o, final_state,
                       workspace, gating=False)


def gdn_chunk_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                          beta: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
                          cu_seqlens: Optional[torch.Tensor] = None, *, o: torch.Tensor,
                          final_state: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """gdn_chunk_fwd with its scratch in the library's static device array (no workspace, nothing
    allocated by the library; the caller passes o and final_state).  Raises GdnError
    (GDN_ERROR_WORKSPACE) when the call needs more scratch than the array holds."""
    lib = _lib.load()
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, T, H, d]")
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    dev = q.device
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    for t, shape, what in ((k, (B, T, Hk, dk), "k"), (v, (B, T, Hv, dv), "v"), (g, (B, T, Hv), "g"),
                           (beta, (B, T, Hv), "beta"), (o, (B, T, Hv, dv), "o"),
                           (final_state, (N, Hv, dk, dv), "final_state")):
        _check(t, shape, what, dev)
    _check(q, (B, T, Hk, dk), "q", dev)
    if initial_state is not None:
        _check(initial_state, (N, Hv, dk, dv), "initial_state", dev, torch.float32)
    if cu_seqlens is not None:
        _check(cu_seqlens, (N + 1,), "cu_seqlens", dev, torch.int32)
    st = lib.gdn_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                                   _ptr(cu_seqlens), B, T, Hk, Hv, dk, dv, N, _code(q, "q"), _code(g, "g"),
                                   _ptr(o), _ptr(final_state), _stream(dev))
    if st != _lib.GDN_SUCCESS:
        raise _lib.GdnError(st, "gdn_chunk_fwd_noalloc")
    return o, final_state


def gdn_chunk_fwd_gating(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, a: torch.Tensor,
                         b: torch.Tensor, A_log: torch.Tensor, dt_bias: torch.Tensor,
                         initial_state: Optional[torch.Tensor] = None,
                         cu_seqlens: Optional[torch.Tensor] = None, *,
                         o: Optional[torch.Tensor] = None,
                         final_state: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """gdn_chunk_fwd with the gates formed in the kernels: a, b [B,T,Hv] the raw projections;
    A_log, dt_bias [Hv] fp32.  beta = sigmoid(b), g = -exp(A_log) softplus(a + dt_bias)."""
    lib = _lib.load()
    return _chunk_call(lib.gdn_chunk_fwd_gating, q, k, v, a, b, A_log, dt_bias, initial_state,
                       cu_seqlens, o, final_state, workspace, gating=True)


def _recurrent_call(fn, q, k, v, x, y, A_log, dt_bias, state, o, gating: bool):
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, T, H, d]")
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError(f"{fn.__name__} runs on a GPU; tensors must be on a cuda device")
    xn, yn = ("a", "b") if gating else ("g", "beta")
    _check(q, (B, T, Hk, dk), "q", dev)
    _check(k, (B, T, Hk, dk), "k", dev, q.dtype)
    _check(v, (B, T, Hv, dv), "v", dev, q.dtype)
    _check(x, (B, T, Hv), xn, dev)
    _check(y, (B, T, Hv), yn, dev, x.dtype)
    if gating:
        _check(A_log, (Hv,), "A_log", dev, torch.float32)
        _check(dt_bias, (Hv,), "dt_bias", dev, torch.float32)
    _check(state, (B, Hv, dk, dv), "state", dev, torch.float32)
    if o is None:
        o = torch.empty((B, T, Hv, dv), dtype=torch.float32, device=dev)
    _check(o, (B, T, Hv, dv), "o", dev, torch.float32)
    gates = (_ptr(A_log), _ptr(dt_bias)) if gating else ()
    st = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(x), _ptr(y), *gates, _ptr(state), B, T, Hk, Hv, dk, dv,
            _code(q, "q"), _code(x, xn), _ptr(o), _stream(dev))
    if st != _lib.GDN_SUCCESS:
        raise _lib.GdnError(st, fn.__name__)
    return o, state


def gdn_recurrent_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                       beta: torch.Tensor, state: torch.Tensor, *,
                       o: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Decode step(s) against a cached state, updated in place.  q,k [B,T,Hk,dk]; v [B,T,Hv,dv];
    g,beta [B,T,Hv]; state [B,Hv,dk,dv] fp32.  Returns (o [B,T,Hv,dv] fp32, state)."""
    lib = _lib.load()
    return _recurrent_call(lib.gdn_recurrent_step, q, k, v, g, beta, None, None, state, o,
                           gating=False)


def gdn_recurrent_step_gating(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, a: torch.Tensor,
                              b: torch.Tensor, A_log: torch.Tensor, dt_bias: torch.Tensor,
                              state: torch.Tensor, *,
                              o: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """gdn_recurrent_step with the gates formed in the kernel from a, b [B,T,Hv] and A_log,
    dt_bias [Hv] fp32."""
    lib = _lib.load()
    return _recurrent_call(lib.gdn_recurrent_step_gating, q, k, v, a, b, A_log, dt_bias, state, o,
                           gating=True)


def gdn_chunk_fwd_indexed(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                          beta: torch.Tensor, state_pool: torch.Tensor, state_indices: torch.Tensor,
                          cu_seqlens: Optional[torch.Tensor] = None, *,
                          o: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Prefill against a pool of states: sequence n starts from state_pool[state_indices[n]] and its
    final state is written back there.  state_pool [num_slots,Hv,dk,dv] fp32; state_indices int32
    [N] (an index outside [0, num_slots) is a padding row: zero start state, no write).  Returns o."""
    lib = _lib.load()
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, T, H, d]")
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("gdn_chunk_fwd_indexed runs on a GPU; tensors must be on a cuda device")
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    _check(q, (B, T, Hk, dk), "q", dev)
    _check(k, (B, T, Hk, dk), "k", dev, q.dtype)
    _check(v, (B, T, Hv, dv), "v", dev, q.dtype)
    _check(g, (B, T, Hv), "g", dev)
    _check(beta, (B, T, Hv), "beta", dev, g.dtype)
    if state_pool.dim() != 4:
        raise ValueError("state_pool must be [num_slots, Hv, dk, dv]")
    num_slots = state_pool.shape[0]
    _check(state_pool, (num_slots, Hv, dk, dv), "state_pool", dev, torch.float32)
    _check(state_indices, (N,), "state_indices", dev, torch.int32)
    if cu_seqlens is not None:
        _check(cu_seqlens, (N + 1,), "cu_seqlens", dev, torch.int32)
    if o is None:
        o = torch.empty((B, T, Hv, dv), dtype=torch.float32, device=dev)
    _check(o, (B, T, Hv, dv), "o", dev, torch.float32)
    qkv, gate = _code(q, "q"), _code(g, "g")
    ws_bytes = int(lib.gdn_chunk_fwd_workspace_size(B, T, Hk, Hv, dk, dv, N, qkv))
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    if workspace is not None:
        if workspace.device != dev or workspace.numel() * workspace.element_size() < ws_bytes:
            raise ValueError(f"workspace must hold {ws_bytes} bytes on {dev}")
    st = lib.gdn_chunk_fwd_indexed(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_pool), _ptr(state_indices),
        num_slots, _ptr(cu_seqlens), B, T, Hk, Hv, dk, dv, N, qkv, gate, _ptr(o), _ptr(workspace),
        ctypes.c_size_t(0 if workspace is None else workspace.numel() * workspace.element_size()),
        _stream(dev))
    if st != _lib.GDN_SUCCESS:
        raise _lib.GdnError(st, "gdn_chunk_fwd_indexed")
    return o


def gdn_recurrent_step_indexed(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                               beta: torch.Tensor, state_pool: torch.Tensor,
                               state_indices: torch.Tensor, *,
                               o: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decode step(s) against a pool of states, updated in place: row b uses slot state_indices[b]
    (outside [0, num_slots): a padding row, left alone, zero outputs).  Returns o."""
    lib = _lib.load()
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, T, H, d]")
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("gdn_recurrent_step_indexed runs on a GPU; tensors must be on a cuda device")
    _check(q, (B, T, Hk, dk), "q", dev)
    _check(k, (B, T, Hk, dk), "k", dev, q.dtype)
    _check(v, (B, T, Hv, dv), "v", dev, q.dtype)
    _check(g, (B, T, Hv), "g", dev)
    _check(beta, (B, T, Hv), "beta", dev, g.dtype)
    if state_pool.dim() != 4:
        raise ValueError("state_pool must be [num_slots, Hv, dk, dv]")
    num_slots = state_pool.shape[0]
    _check(state_pool, (num_slots, Hv, dk, dv), "state_pool", dev, torch.float32)
    _check(state_indices, (B,), "state_indices", dev, torch.int32)
    if o is None:
        o = torch.empty((B, T, Hv, dv), dtype=torch.float32, device=dev)
    _check(o, (B, T, Hv, dv), "o", dev, torch.float32)
    st = lib.gdn_recurrent_step_indexed(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_pool), _ptr(state_indices),
        num_slots, B, T, Hk, Hv, dk, dv, _code(q, "q"), _code(g, "g"), _ptr(o), _stream(dev))
    if st != _lib.GDN_SUCCESS:
        raise _lib.GdnError(st, "gdn_recurrent_step_indexed")
    return o


def _ex_args(name, q, k, v, g, beta, A_log, dt_bias, initial_state, final_state, state_indices,
             cu_seqlens):
    """Shape and dtype checks shared by the option-complete chunked calls; returns the sizes, the
    pool size and the final-state tensor (allocated when not given)."""
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, T, H, d]")
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError(f"{name} runs on a GPU; tensors must be on a cuda device")
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    gating = A_log is not None
    xn, yn = ("a", "b") if gating else ("g", "beta")
    _check(q, (B, T, Hk, dk), "q", dev)
    _check(k, (B, T, Hk, dk), "k", dev, q.dtype)
    _check(v, (B, T, Hv, dv), "v", dev, q.dtype)
    _check(g, (B, T, Hv), xn, dev)
    _check(beta, (B, T, Hv), yn, dev, g.dtype)
    if gating:
        _check(A_log, (Hv,), "A_log", dev, torch.float32)
        _check(dt_bias, (Hv,), "dt_bias", dev, torch.float32)
    elif dt_bias is not None:
        raise ValueError("dt_bias needs A_log")
    if cu_seqlens is not None:
        _check(cu_seqlens, (N + 1,), "cu_seqlens", dev, torch.int32)
    num_slots = 0
    if state_indices is not None:
        if initial_state is None or initial_state.dim() != 4 or final_state is not None:
            raise ValueError("with state_indices, initial_state is the pool [num_slots, Hv, dk, dv] "
                             "and final_state is not given")
        num_slots = initial_state.shape[0]
        _check(initial_state, (num_slots, Hv, dk, dv), "state pool", dev, torch.float32)
        _check(state_indices, (N,), "state_indices", dev, torch.int32)
        final_state = initial_state
    else:
        if initial_state is not None:
            _check(initial_state, (N, Hv, dk, dv), "initial_state", dev, torch.float32)
        if final_state is None:
            final_state = torch.empty((N, Hv, dk, dv), dtype=torch.float32, device=dev)
        _check(final_state, (N, Hv, dk, dv), "final_state", dev, torch.float32)
    return B, T, Hk, Hv, dk, dv, N, num_slots, final_state, dev, xn


def _workspace(ws_bytes: int, workspace, dev):
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    if workspace is not None:
        if workspace.device != dev or workspace.numel() * workspace.element_size() < ws_bytes:
            raise ValueError(f"workspace must hold {ws_bytes} bytes on {dev}")
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return workspace, ctypes.c_size_t(nbytes)


def gdn_chunk_fwd_ex(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                     beta: torch.Tensor, *, A_log: Optional[torch.Tensor] = None,
                     dt_bias: Optional[torch.Tensor] = None,
                     initial_state: Optional[torch.Tensor] = None,
                     final_state: Optional[torch.Tensor] = None,
                     state_indices: Optional[torch.Tensor] = None,
                     cu_seqlens: Optional[torch.Tensor] = None, qk_l2norm: bool = False,
                     o: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """The chunked call with every option: A_log, dt_bias [Hv] fp32 make g, beta the raw projections
    a, b; state_indices int32 [N] makes initial_state a pool [num_slots,Hv,dk,dv] read and written in
    place (it is then also the returned final state); qk_l2norm normalises q and k to unit length
    inside the kernels.  Returns (o, final_state)."""
    lib = _lib.load()
    B, T, Hk, Hv, dk, dv, N, num_slots, final_state, dev, xn = _ex_args(
        "gdn_chunk_fwd_ex", q, k, v, g, beta, A_log, dt_bias, initial_state, final_state, state_indices,
        cu_seqlens)
    if o is None:
        o = torch.empty((B, T, Hv, dv), dtype=torch.float32, device=dev)
    _check(o, (B, T, Hv, dv), "o", dev, torch.float32)
    qkv, gate = _code(q, "q"), _code(g, xn)
    workspace, nbytes = _workspace(int(lib.gdn_chunk_fwd_workspace_size(B, T, Hk, Hv, dk, dv, N, qkv)),
                                   workspace, dev)
    flags = _lib.GDN_FLAG_QK_L2NORM if qk_l2norm else 0
    st = lib.gdn_chunk_fwd_ex(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(A_log), _ptr(dt_bias), _ptr(initial_state),
        _ptr(final_state), _ptr(state_indices), num_slots, _ptr(cu_seqlens), B, T, Hk, Hv, dk, dv, N,
        qkv, gate, flags, _ptr(o), _ptr(workspace), nbytes, _stream(dev))
    if st != _lib.GDN_SUCCESS:
        raise _lib.GdnError(st, "gdn_chunk_fwd_ex")
    return o, final_state


def gdn_chunk_fwd_gated_norm(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                             beta: torch.Tensor, z: torch.Tensor, weight: torch.Tensor, eps: float = 1e-6,
                             *, A_log: Optional[torch.Tensor] = None,
                             dt_bias: Optional[torch.Tensor] = None,
                             initial_state: Optional[torch.Tensor] = None,
                             final_state: Optional[torch.Tensor] = None,
                             state_indices: Optional[torch.Tensor] = None,
                             cu_seqlens: Optional[torch.Tensor] = None, qk_l2norm: bool = False,
                             y: Optional[torch.Tensor] = None, y_dtype: torch.dtype = torch.bfloat16,
                             workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """gdn_chunk_fwd_ex with the gated output norm fused onto o: returns (y, final_state), y [B,T,Hv,dv]
    = o / sqrt(mean(o^2) + eps) * weight * silu(z) per (token, v-head) row, o being gdn_chunk_fwd_ex's
    output for the same arguments.  z [B,T,Hv,dv] bf16 or fp32, weight [dv] fp32, y bf16 or fp32."""
    lib = _lib.load()
    B, T, Hk, Hv, dk, dv, N, num_slots, final_state, dev, xn = _ex_args(
        "gdn_chunk_fwd_gated_norm", q, k, v, g, beta, A_log, dt_bias, initial_state, final_state,
        state_indices, cu_seqlens)
    _check(z, (B, T, Hv, dv), "z", dev)
    _check(weight, (dv,), "weight", dev, torch.float32)
    if y is None:
        y = torch.empty((B, T, Hv, dv), dtype=y_dtype, device=dev)
    _check(y, (B, T, Hv, dv), "y", dev)
    qkv, gate = _code(q, "q"), _code(g, xn)
    workspace, nbytes = _workspace(
        int(lib.gdn_chunk_fwd_gated_norm_workspace_size(B, T, Hk, Hv, dk, dv, N, qkv)), workspace, dev)
    flags = _lib.GDN_FLAG_QK_L2NORM if qk_l2norm else 0
    st = lib.gdn_chunk_fwd_gated_norm(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(A_log), _ptr(dt_bias), _ptr(initial_state),
        _ptr(final_state), _ptr(state_indices), num_slots, _ptr(cu_seqlens), _ptr(z), _ptr(weight),
        ctypes.c_float(eps), B, T, Hk, Hv, dk, dv, N, qkv, gate, _code(z, "z"), _code(y, "y"), flags,
        _ptr(y), _ptr(workspace), nbytes, _stream(dev))
    if st != _lib.GDN_SUCCESS:
        raise _lib.GdnError(st, "gdn_chunk_fwd_gated_norm")
    return y, final_state


def gdn_recurrent_step_ex(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                          beta: torch.Tensor, state: torch.Tensor, *,
                          A_log: Optional[torch.Tensor] = None,
                          dt_bias: Optional[torch.Tensor] = None,
                          state_indices: Optional[torch.Tensor] = None, qk_l2norm: bool = False,
                          o: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """The decode call with every option: raw gates (A_log, dt_bias), a state pool (state_indices
    int32 [B]; state is then [num_slots,Hv,dk,dv]) and qk_l2norm.  Returns (o, state)."""
    lib = _lib.load()
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, T, H, d]")
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("gdn_recurrent_step_ex runs on a GPU; tensors must be on a cuda device")
    gating = A_log is not None
    xn, yn = ("a", "b") if gating else ("g", "beta")
    _check(q, (B, T, Hk, dk), "q", dev)
    _check(k, (B, T, Hk, dk), "k", dev, q.dtype)
    _check(v, (B, T, Hv, dv), "v", dev, q.dtype)
    _check(g, (B, T, Hv), xn, dev)
    _check(beta, (B, T, Hv), yn, dev, g.dtype)
    if gating:
        _check(A_log, (Hv,), "A_log", dev, torch.float32)
        _check(dt_bias, (Hv,), "dt_bias", dev, torch.float32)
    elif dt_bias is not None:
        raise ValueError("dt_bias needs A_log")
    num_slots = 0
    if state_indices is not None:
        if state.dim() != 4:
            raise ValueError("state must be the pool [num_slots, Hv, dk, dv]")
        num_slots = state.shape[0]
        _check(state, (num_slots, Hv, dk, dv), "state pool", dev, torch.float32)
        _check(state_indices, (B,), "state_indices", dev, torch.int32)
    else:
        _check(state, (B, Hv, dk, dv), "state", dev, torch.float32)
    if o is None:
        o = torch.empty((B, T, Hv, dv), dtype=torch.float32, device=dev)
    _check(o, (B, T, Hv, dv), "o", dev, torch.float32)
    flags = _lib.GDN_FLAG_QK_L2NORM if qk_l2norm else 0
    st = lib.gdn_recurrent_step_ex(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(A_log), _ptr(dt_bias), _ptr(state),
        _ptr(state_indices), num_slots, B, T, Hk, Hv, dk, dv, _code(q, "q"), _code(g, xn), flags,
        _ptr(o), _stream(dev))
    if st != _lib.GDN_SUCCESS:
        raise _lib.GdnError(st, "gdn_recurrent_step_ex")
    return o, state


def gdn_chunk_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                  beta: torch.Tensor, d_o: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
                  d_final: Optional[torch.Tensor] = None, cu_seqlens: Optional[torch.Tensor] = None, *,
                  need_d_initial: bool = True,
                  workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, ...]:
    """Backward pass of gdn_chunk_fwd: (dq, dk, dv, dg, dbeta, d_initial_state) in fp32 from the
    gradients d_o [B,T,Hv,dv] and d_final [N,Hv,dk,dv] (None: zero) of the outputs.  d_initial_state
    is None when need_d_initial is False."""
    lib = _lib.load()
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, T, H, d]")
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("gdn_chunk_bwd runs on a GPU; tensors must be on a cuda device")
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    _check(q, (B, T, Hk, dk), "q", dev)
    _check(k, (B, T, Hk, dk), "k", dev, q.dtype)
    _check(v, (B, T, Hv, dv), "v", dev, q.dtype)
    _check(g, (B, T, Hv), "g", dev)
    _check(beta, (B, T, Hv), "beta", dev, g.dtype)
    _check(d_o, (B, T, Hv, dv), "d_o", dev, torch.float32)
    if initial_state is not None:
        _check(initial_state, (N, Hv, dk, dv), "initial_state", dev, torch.float32)
    if d_final is not None:
        _check(d_final, (N, Hv, dk, dv), "d_final", dev, torch.float32)
    if cu_seqlens is not None:
        _check(cu_seqlens, (N + 1,), "cu_seqlens", dev, torch.int32)
    f32 = dict(dtype=torch.float32, device=dev)
    dq = torch.empty((B, T, Hk, dk), **f32)
    dk_ = torch.empty((B, T, Hk, dk), **f32)
    dv_ = torch.zeros((B, T, Hv, dv), **f32)
    dg = torch.empty((B, T, Hv), **f32)
    db = torch.empty((B, T, Hv), **f32)
    ds0 = torch.empty((N, Hv, dk, dv), **f32) if need_d_initial else None
    ws_bytes = int(lib.gdn_chunk_bwd_workspace_size(B, T, Hk, Hv, dk, dv, N))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    if workspace.device != dev or workspace.numel() * workspace.element_size() < ws_bytes:
        raise ValueError(f"workspace must hold {ws_bytes} bytes on {dev}")
    st = lib.gdn_chunk_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(cu_seqlens), _ptr(d_o),
        _ptr(d_final), B, T, Hk, Hv, dk, dv, N, _code(q, "q"), _code(g, "g"), _ptr(dq), _ptr(dk_), _ptr(dv_),
        _ptr(dg), _ptr(db), _ptr(ds0), _ptr(workspace),
        ctypes.c_size_t(workspace.numel() * workspace.element_size()), _stream(dev))
    if st != _lib.GDN_SUCCESS:
        raise _lib.GdnError(st, "gdn_chunk_bwd")
    return dq, dk_, dv_, dg, db, ds0


def gdn_chunk_bwd_ex(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                     beta: torch.Tensor, d_o: torch.Tensor, *, A_log: Optional[torch.Tensor] = None,
                     dt_bias: Optional[torch.Tensor] = None,
                     initial_state: Optional[torch.Tensor] = None,
                     state_indices: Optional[torch.Tensor] = None,
                     d_final: Optional[torch.Tensor] = None, cu_seqlens: Optional[torch.Tensor] = None,
                     qk_l2norm: bool = False, need_d_initial: bool = True,
                     workspace: Optional[torch.Tensor] = None) -> Tuple[Optional[torch.Tensor], ...]:
    """Backward pass of gdn_chunk_fwd_ex with the same options.  Returns (dq, dk, dv, dg, dbeta,
    dA_log, ddt_bias, d_initial_state): with A_log set, g and beta are the raw projections a, b and
    dg, dbeta are da, db, and dA_log, ddt_bias [Hv] are returned (else None); with state_indices,
    initial_state is the pool [num_slots,Hv,dk,dv] and d_initial_state is per sequence; with
    qk_l2norm, dq and dk are with respect to the raw q and k."""
    lib = _lib.load()
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, T, H, d]")
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("gdn_chunk_bwd_ex runs on a GPU; tensors must be on a cuda device")
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    gating = A_log is not None
    xn, yn = ("a", "b") if gating else ("g", "beta")
    _check(q, (B, T, Hk, dk), "q", dev)
    _check(k, (B, T, Hk, dk), "k", dev, q.dtype)
    _check(v, (B, T, Hv, dv), "v", dev, q.dtype)
    _check(g, (B, T, Hv), xn, dev)
    _check(beta, (B, T, Hv), yn, dev, g.dtype)
    _check(d_o, (B, T, Hv, dv), "d_o", dev, torch.float32)
    if gating:
        _check(A_log, (Hv,), "A_log", dev, torch.float32)
        _check(dt_bias, (Hv,), "dt_bias", dev, torch.float32)
    elif dt_bias is not None:
        raise ValueError("dt_bias needs A_log")
    num_slots = 0
    if state_indices is not None:
        if initial_state is None or initial_state.dim() != 4:
            raise ValueError("with state_indices, initial_state is the pool [num_slots, Hv, dk, dv]")
        num_slots = initial_state.shape[0]
        _check(initial_state, (num_slots, Hv, dk, dv), "state pool", dev, torch.float32)
        _check(state_indices, (N,), "state_indices", dev, torch.int32)
    elif initial_state is not None:
        _check(initial_state, (N, Hv, dk, dv), "initial_state", dev, torch.float32)
    if d_final is not None:
        _check(d_final, (N, Hv, dk, dv), "d_final", dev, torch.float32)
    if cu_seqlens is not None:
        _check(cu_seqlens, (N + 1,), "cu_seqlens", dev, torch.int32)
    f32 = dict(dtype=torch.float32, device=dev)
    dq = torch.empty((B, T, Hk, dk), **f32)
    dk_ = torch.empty((B, T, Hk, dk), **f32)
    dv_ = torch.zeros((B, T, Hv, dv), **f32)
    dg = torch.empty((B, T, Hv), **f32)
    db = torch.empty((B, T, Hv), **f32)
    dA = torch.empty((Hv,), **f32) if gating else None
    ddt = torch.empty((Hv,), **f32) if gating else None
    ds0 = torch.empty((N, Hv, dk, dv), **f32) if need_d_initial else None
    flags = _lib.GDN_FLAG_QK_L2NORM if qk_l2norm else 0
    qkv, gate = _code(q, "q"), _code(g, xn)
    ws_bytes = int(lib.gdn_chunk_bwd_ex_workspace_size(B, T, Hk, Hv, dk, dv, N, qkv, int(gating),
                                                       int(state_indices is not None), flags))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    if workspace.device != dev or workspace.numel() * workspace.element_size() < ws_bytes:
        raise ValueError(f"workspace must hold {ws_bytes} bytes on {dev}")
    st = lib.gdn_chunk_bwd_ex(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(A_log), _ptr(dt_bias), _ptr(initial_state),
        _ptr(state_indices), num_slots, _ptr(cu_seqlens), _ptr(d_o), _ptr(d_final), B, T, Hk, Hv, dk, dv, N,
        qkv, gate, flags, _ptr(dq), _ptr(dk_), _ptr(dv_), _ptr(dg), _ptr(db), _ptr(dA), _ptr(ddt), _ptr(ds0),
        _ptr(workspace), ctypes.c_size_t(workspace.numel() * workspace.element_size()), _stream(dev))
    if st != _lib.GDN_SUCCESS:
        raise _lib.GdnError(st, "gdn_chunk_bwd_ex")
    return dq, dk_, dv_, dg, db, dA, ddt, ds0


def gdn_gated_rmsnorm(x: torch.Tensor, z: torch.Tensor, weight: torch.Tensor, eps: float = 1e-6, *,
                      out_dtype: torch.dtype = torch.bfloat16,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The layer's gated output norm over the last axis: x fp32 [..., d] (e.g. o of
    gdn_chunk_fwd), z [..., d] bf16 or fp32, weight [d] fp32.
    Returns x / sqrt(mean(x^2) + eps) * weight * silu(z) in ``out_dtype``."""
    lib = _lib.load()
    if x.dim() < 1:
        raise ValueError("x must have a channel axis")
    d = x.shape[-1]
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("gdn_gated_rmsnorm runs on a GPU; tensors must be on a cuda device")
    _check(x, tuple(x.shape), "x", dev, torch.float32)
    _check(z, tuple(x.shape), "z", dev)
    _check(weight, (d,), "weight", dev, torch.float32)
    if out is None:
        out = torch.empty(tuple(x.shape), dtype=out_dtype, device=dev)
    _check(out, tuple(x.shape), "out", dev)
    rows = x.numel() // d if d else 0
    st = lib.gdn_gated_rmsnorm(_ptr(x), _ptr(z), _ptr(weight), float(eps), rows, d, _code(z, "z"),
                               _code(out, "out"), _ptr(out), _stream(dev))
    if st != _lib.GDN_SUCCESS:
        raise _lib.GdnError(st, "gdn_gated_rmsnorm")
    return out


def gdn_causal_conv1d(x: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor] = None,
                      conv_state: Optional[torch.Tensor] = None,
                      cu_seqlens: Optional[torch.Tensor] = None,
                      state_indices: Optional[torch.Tensor] = None, *, silu: bool = False,
                      y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Depthwise causal convolution over time: x [B, T, C] (bf16 or fp32; packed sequences with
    cu_seqlens use B == 1), weight [C, W] fp32, bias [C] fp32 or None, conv_state [N, W-1, C] in x's
    dtype (or a pool [num_slots, W-1, C] with state_indices [N] int32), updated in place; None: zero
    history, nothing kept.  Returns y [B, T, C] in x's dtype."""
    lib = _lib.load()
    if x.dim() != 3 or weight.dim() != 2:
        raise ValueError("x must be [B, T, C] and weight [C, W]")
    B, T, C = x.shape
    W = weight.shape[1]
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("gdn_causal_conv1d runs on a GPU; tensors must be on a cuda device")
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    _check(x, (B, T, C), "x", dev)
    _check(weight, (C, W), "weight", dev, torch.float32)
    if bias is not None:
        _check(bias, (C,), "bias", dev, torch.float32)
    if cu_seqlens is not None:
        _check(cu_seqlens, (N + 1,), "cu_seqlens", dev, torch.int32)
    num_slots = 0
    if state_indices is not None:
        if conv_state is None:
            raise ValueError("state_indices needs a conv_state pool")
        _check(state_indices, (N,), "state_indices", dev, torch.int32)
        num_slots = conv_state.shape[0]
    if conv_state is not None:
        _check(conv_state, (num_slots if state_indices is not None else N, W - 1, C), "conv_state", dev,
               x.dtype)
    if y is None:
        y = torch.empty((B, T, C), dtype=x.dtype, device=dev)
    _check(y, (B, T, C), "y", dev, x.dtype)
    st = lib.gdn_causal_conv1d(_ptr(x), _ptr(weight), _ptr(bias), _ptr(conv_state), _ptr(state_indices),
                               num_slots, _ptr(cu_seqlens), B, T, C, W, N, _code(x, "x"), int(bool(silu)),
                               _ptr(y), _stream(dev))
    if st != _lib.GDN_SUCCESS:
        raise _lib.GdnError(st, "gdn_causal_conv1d")
    return y


def chunk_gated_delta_rule(q, k, v, g, beta, initial_state=None, cu_seqlens=None):
    """The prefill entry point under its model-side name; see gdn_chunk_fwd."""
    return gdn_chunk_fwd(q, k, v, g, beta, initial_state, cu_seqlens)


def recurrent_gated_delta_rule(q, k, v, g, beta, initial_state):
    """The decode entry point under its model-side name: advances ``initial_state`` in place and
    returns (o, the same state tensor); see gdn_recurrent_step."""
    return gdn_recurrent_step(q, k, v, g, beta, initial_state)
