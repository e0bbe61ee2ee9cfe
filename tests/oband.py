"""The forward output's error split by the size of the exact output.

A bf16 output is the exact result rounded to 8 significant bits, so its
rounding alone costs up to 2^-8 |O|: under 1e-2 while |O| < 2, up to 7.8e-3
for |O| in [2, 4) and up to 1.6e-2 at |O| >= 4.  Reporting the largest error
per band shows which band spends the output bar.  The report lines are kept in
``REPORT`` and printed at the end of the test session.
"""

import numpy as np

BANDS = ((0.0, 2.0, "|O|<2"), (2.0, 4.0, "2<=|O|<4"), (4.0, np.inf, "|O|>=4"))
REPORT = []


def split(got, ref):
    """[(label, count, max-abs error)] over the three |O| bands of ``ref``."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    mag = np.abs(ref)
    err = np.abs(got - ref)
    out = []
    for lo, hi, label in BANDS:
        sel = (mag >= lo) & (mag < hi)
        n = int(np.count_nonzero(sel))
        out.append((label, n, float(np.max(err[sel])) if n else 0.0))
    return out


def record(what, got, ref):
    """Add ``what``'s band split to the session report and return it."""
    parts = split(got, ref)
    line = f"{what:<40s} " + "  ".join(
        f"{label}: n={n} max err {e:.2e}" for label, n, e in parts)
    REPORT.append(line)
    print("O error by band:", line, flush=True)
    return parts
