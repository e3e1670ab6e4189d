"""ctypes binding for libgdn's C ABI (include/gdn.h).

Argument marshalling only: each function checks that the torch tensors it is
given are device tensors of the dtype and contiguity the ABI expects, then
passes their data pointers, the sizes and torch's current HIP stream to the
C entry point of the same name.  Every step of the computation runs in the
library's HIP kernels.  If ``libgdn.so`` has not been built the first call
raises; there is no other code path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch  # imported first so that libgdn binds to torch's HIP runtime

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgdn.so")

GDN_OK, GDN_ERR_INVALID_ARG, GDN_ERR_UNSUPPORTED, GDN_ERR_ALIAS, GDN_ERR_HIP, GDN_ERR_SCRATCH = range(6)
GDN_F32, GDN_BF16, GDN_BF16_F32_OUT = 0, 1, 2
EXPORTED = ("gdn_version", "gdn_status_string", "gdn_chunk_prefill", "gdn_chunk_prefill_ex",
            "gdn_chunk_prefill_segmented", "gdn_chunk_prefill_segmented_workspace",
            "gdn_chunk_prefill_segmented_noalloc", "gdn_noalloc_scratch_bytes",
            "gdn_chunk_prefill_gated", "gdn_prefill_states", "gdn_preop", "gdn_decode_step",
            "gdn_decode_step_ex", "gdn_decode_step_preop", "gdn_chunk_prefill_preop")
GDN_INVERSE_DEFAULT, GDN_INVERSE_SUBSTITUTION, GDN_INVERSE_DOUBLING = 0, 1, 2
GDN_COLUMNS_DEFAULT, GDN_COLUMNS_WHOLE, GDN_COLUMNS_SPLIT = 0, 1, 2
GDN_STATE_CACHED, GDN_STATE_STREAMING = 0, 1

_lib = None


class GdnError(RuntimeError):
    """A libgdn call returned a non-zero status."""

    def __init__(self, status: int, msg: str):
        super().__init__(f"libgdn status {status}: {msg}")
        self.status = status


def load_library(path: Optional[str] = None):
    """Load libgdn.so (raises FileNotFoundError if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise FileNotFoundError(
            f"{p} not found: build it with `python -m linear_attention_recurrence_02_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.gdn_version.argtypes = []
    lib.gdn_version.restype = ctypes.c_int
    lib.gdn_status_string.argtypes = [ctypes.c_int]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_chunk_prefill.argtypes = [vp, vp, vp, ctypes.c_int, vp, vp, vp, vp, i64, i64,
                                      i64, i64, i64, i64, vp, vp, vp]
    lib.gdn_chunk_prefill.restype = ctypes.c_int
    lib.gdn_preop.argtypes = [vp, vp, vp, ctypes.c_int, vp, vp, vp, vp, vp, vp, i64, i64, i64,
                              i64, i64, i64, ctypes.c_float, vp, vp, vp, vp, vp, vp]
    lib.gdn_preop.restype = ctypes.c_int
    lib.gdn_chunk_prefill_ex.argtypes = [vp, vp, vp, ctypes.c_int, vp, vp, vp, vp, i64, i64,
                                         i64, i64, i64, i64, ctypes.c_int, ctypes.c_int, vp, vp,
                                         vp]
    lib.gdn_chunk_prefill_ex.restype = ctypes.c_int
    lib.gdn_chunk_prefill_segmented.argtypes = [vp, vp, vp, ctypes.c_int, vp, vp, vp, vp, i64,
                                                i64, i64, i64, i64, i64, i64, vp, i64, vp, vp,
                                                vp]
    lib.gdn_chunk_prefill_segmented.restype = ctypes.c_int
    lib.gdn_chunk_prefill_segmented_noalloc.argtypes = [vp, vp, vp, ctypes.c_int, vp, vp, vp, vp,
                                                        i64, i64, i64, i64, i64, i64, i64, vp,
                                                        vp, vp]
    lib.gdn_chunk_prefill_segmented_noalloc.restype = ctypes.c_int
    lib.gdn_noalloc_scratch_bytes.argtypes = []
    lib.gdn_noalloc_scratch_bytes.restype = i64
    lib.gdn_chunk_prefill_segmented_workspace.argtypes = [ctypes.c_int, vp, i64, i64, i64, i64]
    lib.gdn_chunk_prefill_segmented_workspace.restype = i64
    lib.gdn_chunk_prefill_gated.argtypes = [vp, vp, vp, ctypes.c_int, vp, vp, vp, vp, i64,
                                            i64, i64, i64, i64, i64, vp, vp, ctypes.c_float,
                                            vp, vp, vp]
    lib.gdn_chunk_prefill_gated.restype = ctypes.c_int
    lib.gdn_prefill_states.argtypes = [vp, vp, vp, ctypes.c_int, vp, vp, vp, vp, i64, i64,
                                       i64, i64, i64, vp, vp, vp]
    lib.gdn_prefill_states.restype = ctypes.c_int
    lib.gdn_decode_step.argtypes = [vp, vp, vp, ctypes.c_int, vp, vp, vp, i64, i64, i64,
                                    i64, vp, vp]
    lib.gdn_decode_step.restype = ctypes.c_int
    lib.gdn_decode_step_ex.argtypes = [vp, vp, vp, ctypes.c_int, vp, vp, vp, i64, i64, i64,
                                       i64, ctypes.c_int, vp, vp]
    lib.gdn_decode_step_ex.restype = ctypes.c_int
    lib.gdn_decode_step_preop.argtypes = [vp, vp, vp, ctypes.c_int, vp, vp, vp, vp, vp,
                                          ctypes.c_float, vp, vp, ctypes.c_float, vp, i64, i64,
                                          i64, i64, ctypes.c_int, vp, vp]
    lib.gdn_decode_step_preop.restype = ctypes.c_int
    lib.gdn_chunk_prefill_preop.argtypes = [vp, vp, vp, ctypes.c_int, vp, vp, vp, vp, vp,
                                            ctypes.c_float, vp, vp, i64, i64, i64, i64, i64,
                                            i64, i64, vp, vp, vp]
    lib.gdn_chunk_prefill_preop.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def gdn_version() -> int:
    return load_library().gdn_version()


def gdn_status_string(status: int) -> str:
    return load_library().gdn_status_string(status).decode()


def _check(status: int):
    if status != GDN_OK:
        raise GdnError(status, gdn_status_string(status))


def _io_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise TypeError(f"unsupported io dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor], dtype=None, name="tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def gdn_chunk_prefill(q, k, v, g, beta, S0=None, cu_seqlens=None, chunk=64, *,
                      O=None, S_T=None, stream=None, inverse=None, columns=None,
                      out_dtype=None):
    """Chunkwise-parallel prompt form over whole sequences.

    q, k, v: [B, T, H, 128] (bf16 or fp32; packed batches B = 1);
    g, beta: [B, T, H] fp32; S0: [N, H, 128, 128] fp32 or None;
    cu_seqlens: int32 [N+1] device offsets or None.
    inverse, columns: both None (gdn_chunk_prefill), or GDN_INVERSE_* and
    GDN_COLUMNS_* values, None standing for the DEFAULT one
    (gdn_chunk_prefill_ex).
    out_dtype: O's dtype; q's by default, or torch.float32 for bf16 inputs
    (GDN_BF16_F32_OUT).
    Returns (O, S_T); O/S_T may be given to write in place (S_T may be S0).
    """
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if cu_seqlens is not None and B != 1:
        raise ValueError("packed batches (cu_seqlens) need B == 1")
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or k.dtype != q.dtype \
            or v.dtype != q.dtype:
        raise ValueError("q, k, v must share shape [B, T, H, d] and dtype")
    if g.shape != (B, T, H) or beta.shape != (B, T, H):
        raise ValueError("g and beta must be [B, T, H]")
    if out_dtype is None:
        out_dtype = q.dtype if O is None else O.dtype
    if O is None:
        O = torch.empty(v.shape, dtype=out_dtype, device=v.device)
    if S_T is None:
        S_T = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    f32_out = q.dtype == torch.bfloat16 and out_dtype == torch.float32
    if O.shape != v.shape or O.dtype != out_dtype or not (O.dtype == q.dtype or f32_out):
        raise ValueError("O must match v's shape, with q's dtype (or fp32 for bf16 inputs)")
    if S_T.shape != (N, H, dk, dv) or (S0 is not None and S0.shape != (N, H, dk, dv)):
        raise ValueError("S0 / S_T must be [N, H, dk, dv]")
    args = (_ptr(q, name="q"), _ptr(k, name="k"), _ptr(v, name="v"),
            GDN_BF16_F32_OUT if f32_out else _io_dtype(q),
            _ptr(g, torch.float32, "g"), _ptr(beta, torch.float32, "beta"),
            _ptr(S0, torch.float32, "S0"), _ptr(cu_seqlens, torch.int32, "cu_seqlens"),
            N, T, H, dk, dv, int(chunk))
    out = (_ptr(O, name="O"), _ptr(S_T, torch.float32, "S_T"), _stream(stream))
    if inverse is None and columns is None:
        st = load_library().gdn_chunk_prefill(*args, *out)
    else:
        st = load_library().gdn_chunk_prefill_ex(
            *args, GDN_INVERSE_DEFAULT if inverse is None else int(inverse),
            GDN_COLUMNS_DEFAULT if columns is None else int(columns), *out)
    _check(st)
    return O, S_T


def segmented_workspace_bytes(q, segment_len, cu_seqlens=None):
    """Bytes of workspace gdn_chunk_prefill_segmented needs for q's shape and
    dtype ([B, T, H, 128], or a packed [1, T, H, 128] with ``cu_seqlens``), or
    ValueError for sizes it cannot take."""
    B, T, H, _ = q.shape
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    need = load_library().gdn_chunk_prefill_segmented_workspace(
        _io_dtype(q), _ptr(cu_seqlens, torch.int32, "cu_seqlens"), N, T, H, int(segment_len))
    if need < 0:
        raise ValueError("invalid sizes for the segmented prompt form")
    return need


def gdn_chunk_prefill_segmented(q, k, v, g, beta, S0=None, chunk=64, segment_len=256, *,
                                cu_seqlens=None, workspace=None, O=None, S_T=None, stream=None):
    """The prompt form with each sequence cut into segments walked in parallel
    (see include/gdn.h); a uniform batch, or a packed one with ``cu_seqlens``
    (int32 [N+1] device offsets, B == 1).  ``workspace``: a uint8 device tensor
    of at least gdn_chunk_prefill_segmented_workspace bytes, or None to allocate
    one here.  Returns (O, S_T)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if cu_seqlens is not None and B != 1:
        raise ValueError("packed batches (cu_seqlens) need B == 1")
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or k.dtype != q.dtype \
            or v.dtype != q.dtype:
        raise ValueError("q, k, v must share shape [B, T, H, d] and dtype")
    if g.shape != (B, T, H) or beta.shape != (B, T, H):
        raise ValueError("g and beta must be [B, T, H]")
    lib = load_library()
    cu = _ptr(cu_seqlens, torch.int32, "cu_seqlens")
    need = segmented_workspace_bytes(q, segment_len, cu_seqlens)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if O is None:
        O = torch.empty_like(v)
    if S_T is None:
        S_T = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    if O.dtype != q.dtype or O.shape != v.shape:
        raise ValueError("O must match v's shape and dtype")
    if S_T.shape != (N, H, dk, dv) or (S0 is not None and S0.shape != (N, H, dk, dv)):
        raise ValueError("S0 / S_T must be [N, H, dk, dv]")
    st = lib.gdn_chunk_prefill_segmented(
        _ptr(q, name="q"), _ptr(k, name="k"), _ptr(v, name="v"), _io_dtype(q),
        _ptr(g, torch.float32, "g"), _ptr(beta, torch.float32, "beta"),
        _ptr(S0, torch.float32, "S0"), cu, N, T, H, dk, dv, int(chunk), int(segment_len),
        _ptr(workspace, name="workspace"), workspace.numel() * workspace.element_size(),
        _ptr(O, name="O"), _ptr(S_T, torch.float32, "S_T"), _stream(stream))
    _check(st)
    return O, S_T


def gdn_chunk_prefill_segmented_noalloc(q, k, v, g, beta, S0=None, chunk=64, segment_len=256, *,
                                        cu_seqlens=None, O=None, S_T=None, stream=None):
    """gdn_chunk_prefill_segmented with the library's own per-GPU scratch instead
    of a workspace (see include/gdn.h): nothing is allocated by the call except
    O / S_T here when they are not given.  Returns (O, S_T)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if cu_seqlens is not None and B != 1:
        raise ValueError("packed batches (cu_seqlens) need B == 1")
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or k.dtype != q.dtype \
            or v.dtype != q.dtype:
        raise ValueError("q, k, v must share shape [B, T, H, d] and dtype")
    if g.shape != (B, T, H) or beta.shape != (B, T, H):
        raise ValueError("g and beta must be [B, T, H]")
    if O is None:
        O = torch.empty_like(v)
    if S_T is None:
        S_T = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    if O.dtype != q.dtype or O.shape != v.shape:
        raise ValueError("O must match v's shape and dtype")
    if S_T.shape != (N, H, dk, dv) or (S0 is not None and S0.shape != (N, H, dk, dv)):
        raise ValueError("S0 / S_T must be [N, H, dk, dv]")
    st = load_library().gdn_chunk_prefill_segmented_noalloc(
        _ptr(q, name="q"), _ptr(k, name="k"), _ptr(v, name="v"), _io_dtype(q),
        _ptr(g, torch.float32, "g"), _ptr(beta, torch.float32, "beta"),
        _ptr(S0, torch.float32, "S0"), _ptr(cu_seqlens, torch.int32, "cu_seqlens"),
        N, T, H, dk, dv, int(chunk), int(segment_len), _ptr(O, name="O"),
        _ptr(S_T, torch.float32, "S_T"), _stream(stream))
    _check(st)
    return O, S_T


def noalloc_scratch_bytes() -> int:
    """Bytes of the per-GPU scratch gdn_chunk_prefill_segmented_noalloc holds."""
    return load_library().gdn_noalloc_scratch_bytes()


def gdn_chunk_prefill_gated(q, k, v, g, beta, z, norm_w, eps, S0=None, cu_seqlens=None,
                            chunk=64, *, Y=None, S_T=None, stream=None):
    """The prompt form with the gated RMS norm applied to each output row.

    Inputs as for gdn_chunk_prefill, plus z: [B, T, H, 128] with q's dtype (the
    gate), norm_w: [128] fp32 and eps >= 0.  Returns (Y, S_T) with
    Y = norm_w * O / sqrt(mean(O^2) + eps) * silu(z) per token row and head.
    """
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if cu_seqlens is not None and B != 1:
        raise ValueError("packed batches (cu_seqlens) need B == 1")
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or k.dtype != q.dtype \
            or v.dtype != q.dtype:
        raise ValueError("q, k, v must share shape [B, T, H, d] and dtype")
    if g.shape != (B, T, H) or beta.shape != (B, T, H):
        raise ValueError("g and beta must be [B, T, H]")
    if z.shape != v.shape or z.dtype != q.dtype:
        raise ValueError("z must match v's shape and q's dtype")
    if norm_w.shape != (dv,):
        raise ValueError("norm_w must be [dv]")
    if Y is None:
        Y = torch.empty_like(v)
    if S_T is None:
        S_T = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    if Y.dtype != q.dtype or Y.shape != v.shape:
        raise ValueError("Y must match v's shape and dtype")
    if S_T.shape != (N, H, dk, dv) or (S0 is not None and S0.shape != (N, H, dk, dv)):
        raise ValueError("S0 / S_T must be [N, H, dk, dv]")
    st = load_library().gdn_chunk_prefill_gated(
        _ptr(q, name="q"), _ptr(k, name="k"), _ptr(v, name="v"), _io_dtype(q),
        _ptr(g, torch.float32, "g"), _ptr(beta, torch.float32, "beta"),
        _ptr(S0, torch.float32, "S0"), _ptr(cu_seqlens, torch.int32, "cu_seqlens"),
        N, T, H, dk, dv, int(chunk), _ptr(z, name="z"), _ptr(norm_w, torch.float32, "norm_w"),
        float(eps), _ptr(Y, name="Y"), _ptr(S_T, torch.float32, "S_T"), _stream(stream))
    _check(st)
    return Y, S_T


def gdn_preop(xq, xk, xv, a, b, conv_w, state, cu_seqlens=None, eps=1e-6, *, state_out=None,
              out=None, stream=None):
    """The block's pre-operations (conv FIFO, silu, L2 norm of q and k, gates).

    xq, xk, xv: [B, T, H, 128] (bf16 or fp32); a, b: [B, T, H] fp32;
    conv_w: [3, H, 128, 4] fp32; state: [N, 3, H, 3, 128] with xq's dtype.
    state_out: None updates ``state`` in place; else a tensor of its shape.
    out: optional (q, k, v, g, beta) to write into.
    Returns (q, k, v, g, beta).
    """
    B, T, H, dk = xq.shape
    dv = xv.shape[-1]
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if cu_seqlens is not None and B != 1:
        raise ValueError("packed batches (cu_seqlens) need B == 1")
    if xk.shape != xq.shape or xv.shape[:3] != xq.shape[:3] or xk.dtype != xq.dtype \
            or xv.dtype != xq.dtype:
        raise ValueError("xq, xk, xv must share shape [B, T, H, d] and dtype")
    if a.shape != (B, T, H) or b.shape != (B, T, H):
        raise ValueError("a and b must be [B, T, H]")
    if state.shape != (N, 3, H, 3, max(dk, dv)) or state.dtype != xq.dtype:
        raise ValueError("state must be [N, 3, H, 3, d] with the projections' dtype")
    if state_out is None:
        state_out = state
    if out is None:
        out = (torch.empty_like(xq), torch.empty_like(xk), torch.empty_like(xv),
               torch.empty_like(a), torch.empty_like(b))
    q, k, v, g, beta = out
    st = load_library().gdn_preop(
        _ptr(xq, name="xq"), _ptr(xk, name="xk"), _ptr(xv, name="xv"), _io_dtype(xq),
        _ptr(a, torch.float32, "a"), _ptr(b, torch.float32, "b"),
        _ptr(conv_w, torch.float32, "conv_w"), _ptr(state, name="state"),
        _ptr(state_out, name="state_out"), _ptr(cu_seqlens, torch.int32, "cu_seqlens"),
        N, T, H, dk, dv, conv_w.shape[-1], float(eps), _ptr(q, name="q"), _ptr(k, name="k"),
        _ptr(v, name="v"), _ptr(g, torch.float32, "g"), _ptr(beta, torch.float32, "beta"),
        _stream(stream))
    _check(st)
    return q, k, v, g, beta


def gdn_chunk_prefill_preop(xq, xk, xv, a, b, conv_w, state, S0=None, cu_seqlens=None,
                            eps=1e-6, *, state_out=None, O=None, S_T=None, stream=None):
    """The prompt form from the raw projections: gdn_preop's pre-operations
    inside the 64-token kernel's chunk load (bf16 only).

    xq, xk, xv, a, b, conv_w, state, cu_seqlens, eps: as for gdn_preop (the
    FIFO ``state`` is advanced in place unless ``state_out`` is given);
    S0: optional [N, H, 128, 128] fp32.  Returns (O, S_T) as gdn_chunk_prefill.
    """
    B, T, H, dk = xq.shape
    dv = xv.shape[-1]
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if cu_seqlens is not None and B != 1:
        raise ValueError("packed batches (cu_seqlens) need B == 1")
    if xk.shape != xq.shape or xv.shape[:3] != xq.shape[:3] or xk.dtype != xq.dtype \
            or xv.dtype != xq.dtype:
        raise ValueError("xq, xk, xv must share shape [B, T, H, d] and dtype")
    if a.shape != (B, T, H) or b.shape != (B, T, H):
        raise ValueError("a and b must be [B, T, H]")
    if state.shape != (N, 3, H, 3, max(dk, dv)) or state.dtype != xq.dtype:
        raise ValueError("state must be [N, 3, H, 3, d] with the projections' dtype")
    if state_out is None:
        state_out = state
    if O is None:
        O = torch.empty(B, T, H, dv, dtype=xq.dtype, device=xq.device)
    if S_T is None:
        S_T = torch.empty(N, H, dk, dv, dtype=torch.float32, device=xq.device)
    st = load_library().gdn_chunk_prefill_preop(
        _ptr(xq, name="xq"), _ptr(xk, name="xk"), _ptr(xv, name="xv"), _io_dtype(xq),
        _ptr(a, torch.float32, "a"), _ptr(b, torch.float32, "b"),
        _ptr(conv_w, torch.float32, "conv_w"), _ptr(state, name="state"),
        _ptr(state_out, name="state_out"), float(eps), _ptr(S0, torch.float32, "S0"),
        _ptr(cu_seqlens, torch.int32, "cu_seqlens"), N, T, H, dk, dv, conv_w.shape[-1], 64,
        _ptr(O, name="O"), _ptr(S_T, torch.float32, "S_T"), _stream(stream))
    _check(st)
    return O, S_T


def gdn_prefill_states(q, k, v, g, beta, S0=None, cu_seqlens=None, *, O=None, S_tok=None,
                       stream=None):
    """The prompt form that also keeps the state after every token.

    Inputs as for gdn_chunk_prefill.  Returns (O, S_tok) with S_tok
    [B, T, H, 128, 128] fp32: the state after each token row within its
    sequence.  O/S_tok may be given to write in place.
    """
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if cu_seqlens is not None and B != 1:
        raise ValueError("packed batches (cu_seqlens) need B == 1")
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or k.dtype != q.dtype \
            or v.dtype != q.dtype:
        raise ValueError("q, k, v must share shape [B, T, H, d] and dtype")
    if g.shape != (B, T, H) or beta.shape != (B, T, H):
        raise ValueError("g and beta must be [B, T, H]")
    if O is None:
        O = torch.empty_like(v)
    if S_tok is None:
        S_tok = torch.empty((B, T, H, dk, dv), dtype=torch.float32, device=q.device)
    if O.dtype != q.dtype or O.shape != v.shape:
        raise ValueError("O must match v's shape and dtype")
    if S_tok.shape != (B, T, H, dk, dv) or (S0 is not None and S0.shape != (N, H, dk, dv)):
        raise ValueError("S_tok must be [B, T, H, dk, dv] and S0 [N, H, dk, dv]")
    st = load_library().gdn_prefill_states(
        _ptr(q, name="q"), _ptr(k, name="k"), _ptr(v, name="v"), _io_dtype(q),
        _ptr(g, torch.float32, "g"), _ptr(beta, torch.float32, "beta"),
        _ptr(S0, torch.float32, "S0"), _ptr(cu_seqlens, torch.int32, "cu_seqlens"),
        N, T, H, dk, dv, _ptr(O, name="O"), _ptr(S_tok, torch.float32, "S_tok"),
        _stream(stream))
    _check(st)
    return O, S_tok


def gdn_decode_step(q, k, v, g, beta, S, *, o=None, stream=None, streaming=False):
    """One token for each of B x H states, S [B, H, 128, 128] fp32 updated in
    place.  q, k, v: [B, H, 128]; g, beta: [B, H] fp32.  Returns o [B, H, 128].
    streaming=True moves the state with non-temporal loads and stores
    (gdn_decode_step_ex with GDN_STATE_STREAMING): same result, faster when
    the state is not in cache."""
    B, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:2] != (B, H) or k.dtype != q.dtype \
            or v.dtype != q.dtype:
        raise ValueError("q, k, v must share shape [B, H, d] and dtype")
    if g.shape != (B, H) or beta.shape != (B, H) or S.shape != (B, H, dk, dv):
        raise ValueError("g, beta must be [B, H]; S [B, H, dk, dv]")
    if o is None:
        o = torch.empty_like(v)
    args = (_ptr(q, name="q"), _ptr(k, name="k"), _ptr(v, name="v"), _io_dtype(q),
            _ptr(g, torch.float32, "g"), _ptr(beta, torch.float32, "beta"),
            _ptr(S, torch.float32, "S"), B, H, dk, dv)
    tail = (_ptr(o, q.dtype, "o"), _stream(stream))
    if streaming:
        st = load_library().gdn_decode_step_ex(*args, GDN_STATE_STREAMING, *tail)
    else:
        st = load_library().gdn_decode_step(*args, *tail)
    _check(st)
    return o


def gdn_decode_step_preop(xq, xk, xv, a, b, conv_w, state, S, eps=1e-6, *, state_out=None,
                          gate=None, o=None, stream=None, streaming=False):
    """One decode step from the raw projections: the pre-operations (conv FIFO,
    silu, L2 norm of q and k, gates) and the step in one launch.

    xq, xk, xv: [B, H, 128] (bf16 or fp32); a, b: [B, H] fp32;
    conv_w: [3, H, 128, 4] fp32; state: [B, 3, H, 3, 128] with xq's dtype,
    advanced in place unless ``state_out`` is given; S: [B, H, 128, 128] fp32,
    updated in place.  gate = (z, norm_w, norm_eps) applies the gated RMS norm
    to the output row (z [B, H, 128] with xq's dtype, norm_w [128] fp32).
    streaming=True moves S with non-temporal loads and stores.  Returns o
    [B, H, 128]."""
    B, H, dk = xq.shape
    dv = xv.shape[-1]
    if xk.shape != xq.shape or xv.shape[:2] != (B, H) or xk.dtype != xq.dtype \
            or xv.dtype != xq.dtype:
        raise ValueError("xq, xk, xv must share shape [B, H, d] and dtype")
    if a.shape != (B, H) or b.shape != (B, H) or S.shape != (B, H, dk, dv):
        raise ValueError("a, b must be [B, H]; S [B, H, dk, dv]")
    if conv_w.shape != (3, H, dk, 4) or state.shape != (B, 3, H, 3, dk) or state.dtype != xq.dtype:
        raise ValueError("conv_w must be [3, H, 128, 4]; state [B, 3, H, 3, 128] with xq's dtype")
    if state_out is None:
        state_out = state
    elif state_out.shape != state.shape or state_out.dtype != state.dtype:
        raise ValueError("state_out must match state")
    if o is None:
        o = torch.empty_like(xv)
    z, norm_w, norm_eps = gate if gate is not None else (None, None, 0.0)
    if z is not None and (z.shape != xv.shape or z.dtype != xq.dtype
                          or norm_w.shape != (dv,)):
        raise ValueError("gate: z must match xv, norm_w be [128]")
    st = load_library().gdn_decode_step_preop(
        _ptr(xq, name="xq"), _ptr(xk, name="xk"), _ptr(xv, name="xv"), _io_dtype(xq),
        _ptr(a, torch.float32, "a"), _ptr(b, torch.float32, "b"),
        _ptr(conv_w, torch.float32, "conv_w"), _ptr(state, xq.dtype, "state"),
        _ptr(state_out, xq.dtype, "state_out"), float(eps), _ptr(z, xq.dtype, "z"),
        _ptr(norm_w, torch.float32, "norm_w"), float(norm_eps), _ptr(S, torch.float32, "S"),
        B, H, dk, dv, GDN_STATE_STREAMING if streaming else GDN_STATE_CACHED,
        _ptr(o, xq.dtype, "o"), _stream(stream))
    _check(st)
    return o
