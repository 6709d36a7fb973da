"""Acceptance rule for GPU results against the oracle.  Test infrastructure only.

An output element d (bf16, widened to float) passes against the oracle value
r (fp64) when

    |d - r| <= 8e-3 * |r| + 1e-3 * rms(r)

where rms(r) is the root mean square of r over the valid elements of the
call.  The relative term allows the bf16 rounding of the output (half an ulp
is 2^-9 ~= 1.95e-3 relative) plus fp32 accumulation-order differences; the
absolute term covers elements whose value is cancelled to near zero.  The
pages print no accuracy figure for the GEMM, so the rule is a reading derived
from the output precision.
"""

import numpy as np

REL_TOL = 8e-3
ABS_TOL_RMS = 1e-3


def bf16_bits_to_float(bits):
    """Widen raw bf16 bit patterns (uint16) to float32, exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def bf16_round(x):
    """Round float64 values to the nearest bf16 (ties to even), returned as
    float32.  Used only for diagnostics: the share of outputs that equal the
    correctly rounded result."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)  # one rounding to fp32
    # The fp32 rounding first can only matter in a double-rounding tie, which is
    # harmless for a diagnostic.
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) >> 16
    return bf16_bits_to_float(u.astype(np.uint16))


def tolerance_check(d, r, valid=None, rms=None):
    """Check GPU values d against oracle values r.

    d, r: arrays of equal shape; valid: optional boolean mask (same shape or
    broadcastable) of elements that have a result; rms: optional precomputed
    rms(r) (for sampled checks the caller passes the rms of its sample).
    Returns a dict with 'ok', 'n', 'n_bad', 'max_ratio' (largest
    |d - r| / bound), 'rms', 'frac_bf16_exact'.
    """
    d = np.asarray(d, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if valid is None:
        valid = np.ones(r.shape, dtype=bool)
    valid = np.broadcast_to(valid, r.shape)
    dv = d[valid]
    rv = r[valid]
    if rv.size == 0:
        return {"ok": True, "n": 0, "n_bad": 0, "max_ratio": 0.0, "rms": 0.0,
                "frac_bf16_exact": 1.0}
    if rms is None:
        rms = float(np.sqrt(np.mean(rv * rv)))
    bound = REL_TOL * np.abs(rv) + ABS_TOL_RMS * rms
    err = np.abs(dv - rv)
    bad = ~(err <= bound)  # NaN in d counts as bad
    ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err > 0, np.inf, 0.0))
    exact = np.mean(dv.astype(np.float32) == bf16_round(rv))
    return {"ok": not bool(bad.any()), "n": int(rv.size), "n_bad": int(bad.sum()),
            "max_ratio": float(np.nanmax(np.where(np.isnan(ratio), np.inf, ratio))),
            "rms": rms, "frac_bf16_exact": float(exact)}
