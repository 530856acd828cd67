"""Acceptance checks shared by the GPU parity tests.

The bar: relative Frobenius error <= 1e-5 and, element by element,
|C_gpu - C_ref| <= 1e-4 * sum_k |a_ik * b_kj|, both evaluated in float64. A
reference of all zeros requires an exact-zero result.
"""

import numpy as np

REL_FRO = 1e-5
ELEM = 1e-4


def check(c_gpu, c_ref, s_ref, what=""):
    g = np.asarray(c_gpu, dtype=np.float64)
    r = np.asarray(c_ref, dtype=np.float64)
    s = np.asarray(s_ref, dtype=np.float64)
    assert g.shape == r.shape == s.shape, (g.shape, r.shape, s.shape)
    assert np.isfinite(g).all(), "%s: non-finite output" % what
    d = np.abs(g - r)
    nr = float(np.linalg.norm(r))
    if nr == 0.0:
        assert (g == 0).all(), "%s: reference is zero, output is not" % what
        return 0.0, 0.0
    rel = float(np.linalg.norm(g - r)) / nr
    worst = float(np.max(d / np.maximum(s, 1e-300))) if d.size else 0.0
    bad = d > ELEM * s
    assert rel <= REL_FRO, "%s: relative Frobenius error %.3e > %.0e" % (what, rel, REL_FRO)
    assert not bad.any(), "%s: %d elements beyond 1e-4*sum|ab| (worst ratio %.3e)" % (
        what, int(bad.sum()), worst)
    return rel, worst


# bf16 output. The kernel rounds its fp32 result c32 once to the nearest bf16
# (ties to even). c32 meets the fp32 bar, |c32 - ref| <= 1e-4 * S, and rounding
# to nearest is monotone, so the bf16 result must lie between the bf16
# roundings of ref - 1e-4*S and ref + 1e-4*S (both computed by the oracle's
# binary64 -> bf16 rounding). Whole-array sanity: rounding to 8 significant
# bits moves a value by at most 2^-8 of itself (unit roundoff), so the relative
# Frobenius error stays within 2^-8 plus the fp32 bar (twice, for the cross
# term).
REL_FRO_BF16 = 2.0 ** -8 + 2 * REL_FRO


def check_bf16(c_gpu, c_ref, s_ref, what=""):
    import oracle
    g = np.asarray(c_gpu, dtype=np.float64)
    r = np.asarray(c_ref, dtype=np.float64)
    s = np.asarray(s_ref, dtype=np.float64)
    assert g.shape == r.shape == s.shape, (g.shape, r.shape, s.shape)
    assert np.isfinite(g).all(), "%s: non-finite output" % what
    lo = oracle.round_to_bf16(r - ELEM * s)
    hi = oracle.round_to_bf16(r + ELEM * s)
    bad = (g < lo) | (g > hi)
    assert not bad.any(), "%s: %d bf16 elements outside [rnd(ref - 1e-4 S), rnd(ref + 1e-4 S)]" % (
        what, int(bad.sum()))
    nr = float(np.linalg.norm(r))
    if nr == 0.0:
        assert (g == 0).all(), "%s: reference is zero, output is not" % what
        return 0.0
    rel = float(np.linalg.norm(g - r)) / nr
    assert rel <= REL_FRO_BF16, "%s: relative Frobenius error %.3e" % (what, rel)
    return rel
