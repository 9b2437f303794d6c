"""Comparison helpers for the GPU-vs-oracle parity tests.

Tolerance readings (fp32 path against the fp64 oracle):
- loss: |a - o| <= 1e-5 * |o|;
- logits and gradients ("1e-3 max relative error with an absolute floor of 1e-6"): per
  tensor, max|a - o| <= 1e-3 * max(max|o|, 1e-6), i.e. the largest error relative to the
  tensor's scale, with the scale floored at 1e-6. An elementwise reading cannot hold for
  fp32: an output that is a K-term sum carries about sqrt(K) * 2^-24 * sum|terms| of
  rounding whatever its own size, so outputs that cancel to near zero have large relative
  error in any fp32 implementation. As a second, elementwise gate every entry must satisfy
  |a - o| <= 1e-3 * |o| + 1e-4 * rms(o);
- parameters after AdamW: max |a - o| <= 1e-5.
Per-kernel tests on arbitrary inputs use assert_close_mag, an elementwise bound derived
from the arithmetic of the sum that produces each output.
"""
from __future__ import annotations

import numpy as np

LOSS_RTOL = 1e-5
RTOL = 1e-3
ATOL = 1e-6
PARAM_ATOL = 1e-5


def stats(a, o, rtol=RTOL, atol=ATOL) -> dict:
    a = np.asarray(a, dtype=np.float64).ravel()
    o = np.asarray(o, dtype=np.float64).ravel()
    err = np.abs(a - o)
    bound = rtol * np.abs(o) + atol
    worst = int(np.argmax(err - bound)) if err.size else 0
    return {
        "n": int(err.size),
        "max_abs": float(err.max()) if err.size else 0.0,
        "allclose_ratio": float((err / bound).max()) if err.size else 0.0,
        "literal_rel": float((err / np.maximum(np.abs(o), atol)).max()) if err.size else 0.0,
        "normwise": float(np.linalg.norm(a - o) / max(np.linalg.norm(o), 1e-300)),
        "violations": int((err > bound).sum()),
        "worst_index": worst,
        "worst": (float(a[worst]), float(o[worst])) if err.size else None,
    }


def assert_close(name, a, o, rtol=RTOL, atol=ATOL):
    s = stats(a, o, rtol, atol)
    assert s["violations"] == 0, f"{name}: {s}"
    return s


def assert_tensor_close(name, a, o, rtol=RTOL, floor=ATOL, elem_rms=1e-4):
    """The model-level gate described in the module docstring; returns the statistics."""
    a = np.asarray(a, dtype=np.float64).ravel()
    o = np.asarray(o, dtype=np.float64).ravel()
    err = np.abs(a - o)
    scale = max(float(np.abs(o).max()) if o.size else 0.0, floor)
    rms = float(np.sqrt(np.mean(o * o))) if o.size else 0.0
    s = stats(a, o)
    s["max_rel_to_scale"] = float(err.max() / scale) if err.size else 0.0
    assert s["max_rel_to_scale"] <= rtol, f"{name}: {s}"
    bound = rtol * np.abs(o) + elem_rms * rms
    bad = err > bound
    assert not bad.any(), f"{name}: {int(bad.sum())} entries above 1e-3|o| + 1e-4 rms: {s}"
    return s


U32 = 2.0 ** -24  # fp32 unit roundoff


def assert_close_mag(name, a, o, mag, K, rtol=RTOL, atol=ATOL, operand_u=0.0):
    """allclose with an extra absolute term from the arithmetic of a K-term fp32 sum.

    ``mag`` is the same sum taken over absolute values (sum_k |x_k y_k|); rounding in a
    K-term fp32 accumulation is below K*u*mag in the worst case and about sqrt(K)*u*mag in
    practice, so cancellation (|o| << mag) is allowed 4*sqrt(K)*u*mag of absolute error.
    ``operand_u``: unit roundoff of an operand the kernel rounds before the products (bf16:
    2^-9), which moves the sum by at most operand_u * mag.
    """
    a = np.asarray(a, dtype=np.float64).ravel()
    o = np.asarray(o, dtype=np.float64).ravel()
    mag = np.asarray(mag, dtype=np.float64).ravel()
    err = np.abs(a - o)
    bound = rtol * np.abs(o) + atol + (4.0 * np.sqrt(K) * U32 + operand_u) * mag
    bad = err > bound
    if bad.any():
        i = int(np.argmax(err - bound))
        raise AssertionError(f"{name}: {int(bad.sum())} of {err.size} outside the bound; worst "
                             f"at {i}: got {a[i]!r} want {o[i]!r} (bound {bound[i]:.3e}, "
                             f"mag {mag[i]:.3e})")
    return stats(a, o, rtol, atol)


def assert_loss(a, o, rtol=LOSS_RTOL):
    assert abs(a - o) <= rtol * abs(o), f"loss {a} vs oracle {o} (rel {abs(a - o) / abs(o):.3e})"
