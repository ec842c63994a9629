"""Shared helpers of the parity tests (no arithmetic of the layer itself)."""
import numpy as np

# Layer-output tolerance: |got - want| <= REL * max(|want|, floor), floor = 2^-3 * max_c |want[t, c]|.
# The relative bound 2e-3 applies after FP16 rounding of the output.  The floor
# exists because the SwiGLU output h is rounded to FP16 before the down
# projection: FP32 and fp64 evaluations of the same h round differently when
# the value sits next to an FP16 rounding midpoint (about 1 element in 300),
# and each such 1-ulp flip moves every output of that pair by |w_d| * ulp(h)
# in absolute terms.  Outputs that are small through cancellation then see a
# large relative change.  tests/test_fp32_floor_model.py evaluates the layer
# with plain FP32 matmuls (any FP32 order is as valid as the kernels') on each
# workload shape and asserts that the floor each one needs stays below FLOOR.
# Normwise errors are reported as well.
REL = 2e-3
FLOOR = 2.0 ** -3

# FP16 activations h (SwiGLU outputs, routed and shared): the GPU's value must
# be within one FP16 ulp of the oracle's, with the ulp taken no smaller than
# that of 2^-6 (2^-16): an FP32 sum of ~2^11 products of this layer carries an
# absolute error around 2^-21, so below 2^-6 an FP16 ulp is no longer far
# above the summation-order noise.  Beyond that, at least H_MIN_EQUAL of the
# elements must be bit-identical (a flip needs the FP32 value within its
# error of an FP16 rounding midpoint; a wrong index, scale or rounding point
# would change nearly all of them).
H_ULP_FLOOR_AT = 2.0 ** -6
H_MIN_EQUAL = 0.97

# Floor of the stage-wise comparison (the oracle's down projection and combine
# applied to the GPU's own h): without the h rounding flips only FP32
# summation-order noise remains, and the proposed 2^-8 floor holds.
STAGE_FLOOR = 2.0 ** -8


def f16_to_f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.float16)
    return a.astype(np.float64)


def ulp16(v):
    """Spacing of FP16 numbers at |v| (2^-24 in the subnormal range)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - 10)


def assert_h_close(got_bits, want_bits, what, min_equal=H_MIN_EQUAL):
    """FP16 activations: elementwise within one ulp (floored at ulp(2^-6)), and
    at least `min_equal` of them bit-identical."""
    g = np.asarray(got_bits).view(np.uint16)
    w = np.asarray(want_bits).view(np.uint16)
    assert g.shape == w.shape, f"{what}: shape {g.shape} vs {w.shape}"
    if g.size == 0:
        return
    gv, wv = f16_to_f64(g), f16_to_f64(w)
    allow = np.maximum(ulp16(wv), ulp16(H_ULP_FLOOR_AT))
    d = np.abs(gv - wv)
    bad = ~(d <= allow)
    if bad.any():
        idx = np.argwhere(bad)[:5].tolist()
        raise AssertionError(f"{what}: {int(bad.sum())} of {g.size} FP16 values beyond one ulp, e.g. "
                             + ", ".join(f"{tuple(i)}: got {gv[tuple(i)]:.6g} want {wv[tuple(i)]:.6g}" for i in idx))
    eq = float(np.mean(g == w))
    assert eq >= min_equal, f"{what}: only {eq:.4f} of the FP16 values bit-identical (need {min_equal})"
    return eq


def rowwise_violations(got, want, rel=REL, floor=FLOOR):
    """Boolean mask of elements outside the tolerance, rows = tokens (or pairs)."""
    g, w = f16_to_f64(got), f16_to_f64(want)
    m = np.abs(w).max(axis=-1, keepdims=True)
    return np.abs(g - w) > rel * np.maximum(np.abs(w), m * floor)


def assert_close_rows(got, want, what, rel=REL, floor=FLOOR):
    bad = rowwise_violations(got, want, rel, floor)
    if bad.any():
        g, w = f16_to_f64(got), f16_to_f64(want)
        idx = np.argwhere(bad)[:5].tolist()
        raise AssertionError(f"{what}: {int(bad.sum())} elements outside tolerance, e.g. "
                             + ", ".join(f"{tuple(i)}: got {g[tuple(i)]:.6g} want {w[tuple(i)]:.6g}" for i in idx))


def error_report(got, want):
    """(max relative error without floor over |want|>0, max normwise error per row)."""
    g, w = f16_to_f64(got), f16_to_f64(want)
    nz = np.abs(w) > 0
    rel = float(np.max(np.abs(g - w)[nz] / np.abs(w)[nz])) if nz.any() else 0.0
    m = np.abs(w).max(axis=-1, keepdims=True)
    norm = float(np.max(np.abs(g - w).max(axis=-1, keepdims=True) / np.where(m > 0, m, 1)))
    return rel, norm
