"""Acceptance check shared by the GPU parity tests.

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
