"""Comparison helpers for the GPU-vs-oracle parity tests.

Tolerance readings (fp32 path against the fp64 oracle):
- loss: |a - o| <= 1e-5 * |o|;
- logits and gradients: elementwise |a - o| <= 1e-3 * |o| + 1e-6 (the "1e-3 relative with
  an absolute floor of 1e-6" read as an allclose bound). The literal statistic
  max |a - o| / max(|o|, 1e-6) and the normwise error are reported next to it;
- gradients whose magnitude is near the floor (e.g. dwte rows, which scale as 1/(B*T)) are
  also compared after multiplying both sides by B*T, a power of two, so the floor does not
  make the comparison vacuous;
- parameters after AdamW: max |a - o| <= 1e-5.
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


def assert_loss(a, o, rtol=LOSS_RTOL):
    assert abs(a - o) <= rtol * abs(o), f"loss {a} vs oracle {o} (rel {abs(a - o) / abs(o):.3e})"
