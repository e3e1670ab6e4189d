"""CPU fp64 oracle for the gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never loads it, and it
imports nothing from the GPU library: the two share no code.

The arithmetic lives in ``gdn_oracle.c`` (plain C, fp64, the sequential
per-token recurrence of the Qwen3.5-9B-npu model page, "How it works" ->
"Gated DeltaNet on the NPU").  This module only marshals arrays: it upcasts
whatever it is given (bf16/fp32 tensors or arrays) to contiguous fp64 and calls
the C code through ctypes.

Parity pins for every function here are in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import LIB_PATH, build as _build

__all__ = ["prefill", "decode", "gated_rmsnorm", "preop", "default_threads", "load"]

_lib = None


def load():
    """Load (building once if absent) the oracle's shared library."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        _build()
    lib = ctypes.CDLL(LIB_PATH)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int64)
    i64 = ctypes.c_int64
    lib.gdn_oracle_prefill.argtypes = [dp, dp, dp, dp, dp, dp, ip, i64, i64, i64,
                                       i64, i64, dp, dp, ctypes.c_int]
    lib.gdn_oracle_prefill.restype = ctypes.c_int
    lib.gdn_oracle_prefill_states.argtypes = [dp, dp, dp, dp, dp, dp, ip, i64, i64, i64,
                                              i64, i64, dp, dp, dp, ctypes.c_int]
    lib.gdn_oracle_prefill_states.restype = ctypes.c_int
    lib.gdn_oracle_decode.argtypes = [dp, dp, dp, dp, dp, dp, i64, i64, i64, i64,
                                      i64, dp, ctypes.c_int]
    lib.gdn_oracle_decode.restype = ctypes.c_int
    lib.gdn_oracle_gated_rmsnorm.argtypes = [dp, dp, dp, i64, i64, ctypes.c_double, dp]
    lib.gdn_oracle_gated_rmsnorm.restype = ctypes.c_int
    lib.gdn_oracle_preop.argtypes = [dp, dp, dp, dp, dp, dp, dp, ip, i64, i64, i64, i64, i64,
                                     i64, ctypes.c_double, dp, dp, dp, dp, dp, dp]
    lib.gdn_oracle_preop.restype = ctypes.c_int
    _lib = lib
    return lib


def default_threads() -> int:
    """Threads the oracle uses by default: every core this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux
        return os.cpu_count() or 1


def _f64(x):
    """Exact fp64 copy of a numpy array or a (CPU or device) torch tensor."""
    if x is None:
        return None
    if not isinstance(x, np.ndarray) and hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a, ctype=ctypes.c_double):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def prefill(q, k, v, g, beta, S0=None, cu_seqlens=None, nthreads=None, states=False):
    """Run the per-token recurrence over whole sequences.

    q, k: [B, T, H, dk]; v: [B, T, H, dv]; g, beta: [B, T, H].
    S0: [N, H, dk, dv] or None (zero state).
    cu_seqlens: None (N = B sequences of length T) or [N+1] int offsets into
    the packed token axis (then B must be 1 and T = cu_seqlens[-1]).
    Returns (O [B, T, H, dv], S_T [N, H, dk, dv]) as fp64 numpy arrays; with
    states=True also S_tok [B, T, H, dk, dv], the state after every token.
    """
    q, k, v, g, beta, S0 = map(_f64, (q, k, v, g, beta, S0))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != (B, T, H) or g.shape != (B, T, H) \
            or beta.shape != (B, T, H):
        raise ValueError("oracle.prefill: inconsistent shapes")
    cu = None
    if cu_seqlens is not None:
        if B != 1:
            raise ValueError("oracle.prefill: packed batches need B == 1")
        cu = np.ascontiguousarray(np.asarray(
            cu_seqlens.cpu().numpy() if hasattr(cu_seqlens, "cpu") else cu_seqlens,
            dtype=np.int64))
        N = cu.shape[0] - 1
    else:
        N = B
    if S0 is not None and S0.shape != (N, H, dk, dv):
        raise ValueError("oracle.prefill: S0 must be [N, H, dk, dv]")
    O = np.zeros((B, T, H, dv), dtype=np.float64)
    S_T = np.zeros((N, H, dk, dv), dtype=np.float64)
    if states:
        S_tok = np.zeros((B, T, H, dk, dv), dtype=np.float64)
        rc = load().gdn_oracle_prefill_states(
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0),
            _ptr(cu, ctypes.c_int64), N, T, H, dk, dv, _ptr(O), _ptr(S_T), _ptr(S_tok),
            nthreads or default_threads())
    else:
        rc = load().gdn_oracle_prefill(
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0),
            _ptr(cu, ctypes.c_int64), N, T, H, dk, dv, _ptr(O), _ptr(S_T),
            nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle.prefill failed with code {rc}")
    return (O, S_T, S_tok) if states else (O, S_T)


def decode(q, k, v, g, beta, S, nthreads=None):
    """Run consecutive one-token steps on a batch of states.

    q, k: [steps, B, H, dk] (or [B, H, dk] for one step); v likewise with dv;
    g, beta: [steps, B, H] (or [B, H]); S: [B, H, dk, dv].
    Returns (o with v's shape, S after the last step) as fp64 numpy arrays;
    the input S is not modified.
    """
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    S = _f64(S).copy()
    single = q.ndim == 3
    if single:
        q, k, v, g, beta = (x[None] for x in (q, k, v, g, beta))
    steps, B, H, dk = q.shape
    dv = v.shape[-1]
    if S.shape != (B, H, dk, dv) or g.shape != (steps, B, H) or beta.shape != g.shape:
        raise ValueError("oracle.decode: inconsistent shapes")
    o = np.zeros((steps, B, H, dv), dtype=np.float64)
    rc = load().gdn_oracle_decode(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S), steps, B, H, dk,
        dv, _ptr(o), nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle.decode failed with code {rc}")
    return (o[0] if single else o), S


def gated_rmsnorm(o, z, w, eps):
    """Gated RMS norm over the last axis: y = w * o / sqrt(mean(o^2) + eps) * silu(z).

    o and z: any shape [..., dv] (the same); w: [dv].  Returns fp64 numpy y.
    """
    o, z, w = map(_f64, (o, z, w))
    if z.shape != o.shape or w.shape != (o.shape[-1],):
        raise ValueError("oracle.gated_rmsnorm: inconsistent shapes")
    y = np.zeros_like(o)
    dv = o.shape[-1]
    rows = o.size // dv if dv else 0
    rc = load().gdn_oracle_gated_rmsnorm(_ptr(o), _ptr(z), _ptr(w), rows, dv, float(eps), _ptr(y))
    if rc != 0:
        raise ValueError(f"oracle.gated_rmsnorm failed with code {rc}")
    return y


def preop(xq, xk, xv, a, b, conv_w, state, cu_seqlens=None, eps=1e-6):
    """The block's pre-operations: causal depthwise conv over the carried FIFO,
    silu, L2 norm of q and k, g = -softplus(a), beta = sigmoid(b).

    xq, xk: [B, T, H, dk]; xv: [B, T, H, dv]; a, b: [B, T, H];
    conv_w: [3, H, dmax, K]; state: [N, 3, H, K-1, dmax] (dmax = max(dk, dv));
    cu_seqlens as for prefill.  Returns fp64 (q, k, v, g, beta, state_out).
    """
    xq, xk, xv, a, b, conv_w, state = map(_f64, (xq, xk, xv, a, b, conv_w, state))
    B, T, H, dk = xq.shape
    dv = xv.shape[-1]
    K = conv_w.shape[-1]
    dmax = max(dk, dv)
    cu = None
    if cu_seqlens is not None:
        if B != 1:
            raise ValueError("oracle.preop: packed batches need B == 1")
        cu = np.ascontiguousarray(np.asarray(
            cu_seqlens.cpu().numpy() if hasattr(cu_seqlens, "cpu") else cu_seqlens,
            dtype=np.int64))
        N = cu.shape[0] - 1
    else:
        N = B
    if xk.shape != xq.shape or xv.shape[:3] != (B, T, H) or a.shape != (B, T, H) \
            or b.shape != (B, T, H) or conv_w.shape != (3, H, dmax, K) \
            or state.shape != (N, 3, H, K - 1, dmax):
        raise ValueError("oracle.preop: inconsistent shapes")
    q, k = np.zeros_like(xq), np.zeros_like(xk)
    v = np.zeros_like(xv)
    g, beta = np.zeros_like(a), np.zeros_like(b)
    state_out = np.zeros_like(state)
    rc = load().gdn_oracle_preop(_ptr(xq), _ptr(xk), _ptr(xv), _ptr(a), _ptr(b), _ptr(conv_w),
                                 _ptr(state), _ptr(cu, ctypes.c_int64), N, T, H, dk, dv, K,
                                 float(eps), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                 _ptr(state_out))
    if rc != 0:
        raise ValueError(f"oracle.preop failed with code {rc}")
    return q, k, v, g, beta, state_out
