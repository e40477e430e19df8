"""Element-by-element comparison of an attention result with the float64 oracle.

Tolerance for 16-bit outputs computed with fp32 accumulation: max abs error
<= 1.5e-2 and median relative error <= 4e-3 (median over elements whose oracle
value is nonzero).  Elements where the oracle is nonfinite must match in class
(+Inf, -Inf, NaN) and are left out of both metrics.  The diagnostic
max |x - ref| / (1 + |ref|) is the error form TensorFold PR #1009 uses for its
router logits (Receipt).
"""

import numpy as np

MAX_ABS = 1.5e-2
MED_REL = 4e-3


def compare(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if x.shape != ref.shape:
        raise AssertionError(f"shape {x.shape} != {ref.shape}")
    fin = np.isfinite(ref)
    class_ok = bool(np.all(np.isnan(x[~fin]) == np.isnan(ref[~fin]))
                    and np.all(np.where(np.isnan(ref[~fin]), True, x[~fin] == ref[~fin])))
    xf, rf = x[fin], ref[fin]
    if xf.size == 0:
        return {"max_abs": 0.0, "med_rel": 0.0, "diag": 0.0, "class_ok": class_ok, "ok": class_ok, "n": 0}
    err = np.abs(xf - rf)
    err = np.where(np.isnan(err), np.inf, err)
    nz = rf != 0
    med_rel = float(np.median(err[nz] / np.abs(rf[nz]))) if nz.any() else 0.0
    max_abs = float(err.max())
    diag = float((err / (1.0 + np.abs(rf))).max())
    ok = class_ok and max_abs <= MAX_ABS and med_rel <= MED_REL
    return {"max_abs": max_abs, "med_rel": med_rel, "diag": diag, "class_ok": class_ok, "ok": ok, "n": int(xf.size)}


def assert_close(x, ref, what=""):
    res = compare(x, ref)
    assert res["ok"], f"{what}: {res}"
    return res
