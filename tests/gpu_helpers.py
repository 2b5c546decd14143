"""Shared helpers for the GPU parity tests (comparison against the CPU oracle)."""
import numpy as np
import torch


def f64(t):
    """Exact host float64 copy of a tensor (bf16/fp32 promote exactly)."""
    return None if t is None else t.detach().to("cpu", torch.float64).numpy()


def half_ulp(a, dtype):
    """Half a unit in the last place of |a| in ``dtype`` (bf16: 8 significant bits,
    fp32: 24): the largest error of round-to-nearest into that format."""
    bits = {torch.bfloat16: 8, torch.float32: 24}[dtype]
    a = np.abs(np.asarray(a, dtype=np.float64))
    _, e = np.frexp(a)                       # a = m * 2^e, m in [0.5, 1)
    return np.where(a > 0, np.ldexp(1.0, e - bits - 1), 0.0)


def rel_max_err(x, ref, out_dtype=None):
    """max|x - ref| / RMS(ref), the parity measure.

    With ``out_dtype`` set, x was stored in that dtype, and the half-ulp of that
    final rounding (taken at the larger of |x|, |ref|) is not counted: the
    tolerance bounds the computation, not the storage format of its result.
    """
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    d = np.abs(x - ref)
    if out_dtype is not None:
        d = np.maximum(d - half_ulp(np.maximum(np.abs(x), np.abs(ref)), out_dtype), 0.0)
    return float(np.max(d)) / max(rms, 1e-300)


def assert_close(x, ref, tol, what, out_dtype=None):
    """max|x - ref| <= tol * RMS(ref), net of the final rounding's half-ulp when
    ``out_dtype`` is given.  Prints both the raw and the net error, so that the
    margin where the elements are largest can be read off the log."""
    err = rel_max_err(x, ref, out_dtype)
    raw = rel_max_err(x, ref) if out_dtype is not None else err
    print(f"[parity] {what}: max|d|/RMS = {err:.3e} net, {raw:.3e} raw (tol {tol:.0e})")
    assert np.all(np.isfinite(np.asarray(x, dtype=np.float64))), f"{what}: non-finite values"
    assert err <= tol, f"{what}: max|d|/RMS = {err:.3e} > {tol:.1e}"
    return err


def dev():
    return torch.device("cuda:0")
