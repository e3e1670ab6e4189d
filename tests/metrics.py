"""Error measures used by the GPU parity tests.

Per-slice normwise error: for each (sequence, head) slice of an output,
max|x - r| / max|r|; the report is the worst slice.  The outputs' own
rounding to bf16 is allowed for separately: an element of a bf16 output may
differ from the fp64 reference by tol * max_slice|r| plus half a bf16 unit in
the last place of max(|x|, |r|).
"""
from __future__ import annotations

import numpy as np

TOL_BF16 = 2e-3     # bf16 inputs
TOL_F32 = 1e-5      # fp32 inputs


def f64(x):
    if hasattr(x, "detach"):
        x = x.detach().float().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def bf16_half_ulp(a):
    """Half a bf16 ulp (8 significant bits) of |a|, elementwise."""
    a = np.abs(a)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - 8), 0.0)


def slices_tokens(x, spans, H):
    """Yield [L, d] slices of a [B, T, H, d] array for spans (b, start, end)."""
    for (b, s, e) in spans:
        for h in range(H):
            yield x[b, s:e, h]


def spans_of(B, T, cu_seqlens=None):
    if cu_seqlens is None:
        return [(b, 0, T) for b in range(B)]
    cu = [int(c) for c in np.asarray(f64(cu_seqlens)).astype(np.int64)]
    return [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]


def worst_slice_error(x, r, spans=None, H=None):
    """max over slices of max|x-r|/max|r|.  Token outputs [B,T,H,d] need spans
    and H; states [N,H,dk,dv] (or any [..., a, b]) are sliced on the last two."""
    x, r = f64(x), f64(r)
    worst = 0.0
    if spans is None:
        xs = x.reshape(-1, x.shape[-2], x.shape[-1])
        rs = r.reshape(-1, r.shape[-2], r.shape[-1])
        pairs = zip(xs, rs)
    else:
        pairs = zip(slices_tokens(x, spans, H), slices_tokens(r, spans, H))
    for a, b in pairs:
        if b.size == 0:
            continue
        den = np.max(np.abs(b))
        err = np.max(np.abs(a - b)) / (den if den > 0 else 1.0)
        worst = max(worst, float(err))
    return worst


def bf16_output_ok(x, r, tol, spans, H):
    """Elementwise bound for a bf16 token output against the fp64 reference.
    Returns (ok, worst excess ratio)."""
    x, r = f64(x), f64(r)
    worst = 0.0
    for a, b in zip(slices_tokens(x, spans, H), slices_tokens(r, spans, H)):
        if b.size == 0:
            continue
        bound = tol * np.max(np.abs(b)) + bf16_half_ulp(np.maximum(np.abs(a), np.abs(b)))
        ratio = np.max(np.abs(a - b) / np.where(bound > 0, bound, 1e-300))
        worst = max(worst, float(ratio))
    return worst <= 1.0, worst


def gated_output_ok(Y, Yr, Or, z, w, eps, tol, spans, H):
    """Bound for the gated RMS norm's output y = w o / rho silu(z),
    rho = sqrt(mean(o^2) + eps) per (token, head) row, derived from the bar on
    O: if each element of O is within D = tol * max_slice|O_ref| of the
    reference, then to first order
        |y_j - r_j| <= |w_j silu(z_j)| (D / rho) (1 + |o_j| / rho)
    (the Jacobian of the norm is (w silu(z) / rho)(I - o o^T / (n rho^2)), and
    sum_i |o_i| <= n rho).  A bf16 output may also differ by half an ulp.
    Returns (ok, worst ratio of |y - r| to the bound)."""
    Y, Yr, Or, z = f64(Y), f64(Yr), f64(Or), f64(z)
    w = f64(w)
    worst = 0.0
    for yy, rr, oo, zz in zip(slices_tokens(Y, spans, H), slices_tokens(Yr, spans, H),
                              slices_tokens(Or, spans, H), slices_tokens(z, spans, H)):
        if oo.size == 0:
            continue
        d = tol * np.max(np.abs(oo))
        rho = np.sqrt(np.mean(oo * oo, axis=-1, keepdims=True) + eps)
        gate = np.abs(w * zz / (1.0 + np.exp(-zz)))
        bound = gate * (d / rho) * (1.0 + np.abs(oo) / rho) \
            + bf16_half_ulp(np.maximum(np.abs(yy), np.abs(rr)))
        ratio = np.max(np.abs(yy - rr) / np.where(bound > 0, bound, 1e-300))
        worst = max(worst, float(ratio))
    return worst <= 1.0, worst
