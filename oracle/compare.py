"""Error metric used to compare a result with the oracle -- TEST INFRASTRUCTURE ONLY.

A pure element-wise relative error |y - r| / |r| is unusable for these operators: the
WKV output is a ratio whose numerator can cancel to ~0 at isolated time steps, and a
perfectly rounded float32 evaluation then shows element-wise relative errors of order
one.  The metric therefore floors the denominator at the root-mean-square of the
oracle output over the time axis of the same (batch, channel) sequence:

    err = max_i |y_i - r_i| / max(|r_i|, RMS_t(r[b, :, c]), 1e-30)

For per-channel vectors (the w and u gradients) the floor is the RMS over channels.
Complex values use the modulus.  ``quantiles`` reports the plain element-wise relative
error distribution alongside, for transparency.

The w and u gradients are also held channel by channel (``chan_ratio``): each channel's
error against tol times its own value, floored by kappa times the sum of the magnitudes of
the products its terms are made of (its conditioning, ``wkv4_backward_cond``), which bounds
what float32 evaluation of those terms can resolve.
"""

from __future__ import annotations

import numpy as np


def rel_err(out, ref, time_axis: int | None = 1) -> float:
    """RMS-floored maximum relative error of ``out`` against the oracle ``ref``.

    ``time_axis`` is the axis the RMS floor is taken over (1 for (B,T,C) tensors);
    ``None`` takes it over the whole array (used for (C,) vectors).
    """
    out = np.asarray(out)
    ref = np.asarray(ref)
    if out.shape != ref.shape:
        raise ValueError("shape mismatch %s vs %s" % (out.shape, ref.shape))
    if ref.size == 0:
        return 0.0
    mag = np.abs(ref.astype(np.complex128 if np.iscomplexobj(ref) else np.float64))
    diff = np.abs(out.astype(np.complex128 if np.iscomplexobj(out) else np.float64) - ref)
    if time_axis is None:
        rms = np.sqrt(np.mean(mag * mag))
    else:
        rms = np.sqrt(np.mean(mag * mag, axis=time_axis, keepdims=True))
    denom = np.maximum(np.maximum(mag, rms), 1e-30)
    with np.errstate(invalid="ignore"):
        e = diff / denom
    if not np.all(np.isfinite(e)):
        return float("inf")
    return float(np.max(e))


# kappa of chan_ratio: a term of dL/dw or dL/du evaluated in float32 passes through about a
# dozen roundings (the weights' exponentials and their float32 arguments, the reciprocal of
# the denominator, the products, the in-chunk float32 partial sums), each of at most 2^-24
# relative to the magnitudes of the products involved.
KAPPA_F32_TERMS = 2.0 ** -20


def chan_ratio(out, ref, cond, tol: float, kappa: float = KAPPA_F32_TERMS) -> float:
    """max_c |out_c - ref_c| / max(tol |ref_c|, kappa cond_c): at most 1 when every channel
    is within tol of its own value or within kappa of its conditioning sum cond_c."""
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    cond = np.asarray(cond, np.float64)
    if ref.size == 0:
        return 0.0
    bound = np.maximum(np.maximum(tol * np.abs(ref), kappa * cond), 1e-300)
    e = np.abs(out - ref) / bound
    return float(np.max(e)) if np.all(np.isfinite(e)) else float("inf")


def plain_rel(out, ref) -> float:
    """max |out - ref| / |ref| (no floor), reported next to the floored metrics."""
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        e = np.abs(out - ref) / np.abs(ref)
    e = e[np.isfinite(e)]
    return float(np.max(e)) if e.size else 0.0


def quantiles(out, ref) -> dict:
    """Median, 99.99th percentile and maximum of the plain element-wise relative error."""
    out = np.asarray(out)
    ref = np.asarray(ref)
    mag = np.abs(ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        e = np.abs(out - ref) / np.maximum(mag, 1e-30)
    e = e[np.isfinite(e)]
    if e.size == 0:
        return {"median": 0.0, "p9999": 0.0, "max": 0.0}
    return {"median": float(np.median(e)), "p9999": float(np.quantile(e, 0.9999)),
            "max": float(np.max(e))}
