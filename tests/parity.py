"""The acceptance rule for GPU log-mel against the fp64 oracle.

Per element: where the oracle's mel energy is at least 1e-7, the GPU log-mel
must be within 1e-3 of the oracle's; below that, the GPU value must lie below
ln(1e-7) + 1 (the oracle's own value is then at most ln(1e-7)). No NaN is
allowed for finite input. Frame counts and offsets are compared exactly
elsewhere.
"""

import math

import numpy as np

E_LOUD = 1e-7
ABS_TOL = 1e-3
QUIET_CEIL = math.log(1e-7) + 1.0      # -15.118095650958319


def parity_report(L_gpu, L_ref, E_ref):
    L_gpu = np.asarray(L_gpu, dtype=np.float64)
    L_ref = np.asarray(L_ref, dtype=np.float64)
    E_ref = np.asarray(E_ref, dtype=np.float64)
    assert L_gpu.shape == L_ref.shape == E_ref.shape, (L_gpu.shape, L_ref.shape)
    loud = E_ref >= E_LOUD
    err = np.abs(L_gpu - L_ref)
    max_err = float(err[loud].max()) if loud.any() else 0.0
    n_bad_loud = int(np.count_nonzero(~(err[loud] <= ABS_TOL)))
    quiet_vals = L_gpu[~loud]
    n_bad_quiet = int(np.count_nonzero(~(quiet_vals < QUIET_CEIL)))
    n_nan = int(np.count_nonzero(np.isnan(L_gpu)))
    return {
        "elements": int(L_gpu.size), "loud": int(loud.sum()),
        "max_abs_err_loud": max_err, "bad_loud": n_bad_loud,
        "bad_quiet": n_bad_quiet, "nan": n_nan,
        "ok": n_bad_loud == 0 and n_bad_quiet == 0 and n_nan == 0,
    }


def assert_parity(L_gpu, L_ref, E_ref, what=""):
    rep = parity_report(L_gpu, L_ref, E_ref)
    assert rep["ok"], f"parity failed {what}: {rep}"
    return rep
