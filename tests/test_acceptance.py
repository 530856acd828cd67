"""The GPU acceptance checks themselves, on the CPU.

A float32 product computed by numpy (another summation order than the
oracle's binary64 loop) stands in for a kernel result that meets the bar;
each check must accept it and reject it once a plausible mistake is planted
(a wrong sign, one element off, a transposed pairing). Nothing here runs on
the GPU.
"""

import numpy as np
import pytest

import oracle
import workloads as wl
from tests import parity


def _bf16_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


@pytest.fixture(scope="module")
def case():
    w = wl.make_workload(E=3, K=384, N=264, sizes=[40, 0, 77], seed=31)
    ref, s, _ = oracle.grouped_gemm(w.A, w.B, w.offsets)
    A = _bf16_to_f32(w.A)
    B = _bf16_to_f32(w.B)
    c32 = np.zeros((w.M_cap, w.N), dtype=np.float32)
    for e in range(w.E):
        r0, r1 = int(w.offsets[e]), int(w.offsets[e + 1])
        c32[r0:r1] = A[r0:r1] @ B[e]
    m = w.M_tot
    return c32[:m], ref[:m], s[:m]


def test_fp32_check_accepts_float32_product_and_rejects_mistakes(case):
    c32, ref, s = case
    parity.check(c32, ref, s, "float32 product")
    with pytest.raises(AssertionError):
        parity.check(-c32, ref, s, "sign")
    bad = c32.copy()
    bad[5, 17] *= 1.01
    with pytest.raises(AssertionError):
        parity.check(bad, ref, s, "one element")


def test_bf16_check_accepts_rounded_product_and_rejects_mistakes(case):
    c32, ref, s = case
    c16 = oracle.round_to_bf16(c32.astype(np.float64))
    parity.check_bf16(c16, ref, s, "bf16 product")
    bad = c16.copy()
    bad[3, 9] = oracle.round_to_bf16(bad[3, 9] * 1.02)
    with pytest.raises(AssertionError):
        parity.check_bf16(bad, ref, s, "one element")
    with pytest.raises(AssertionError):
        parity.check_bf16(c16[:, ::-1], ref, s, "columns reversed")


def _swiglu_f32(c32):
    g = c32[:, 0::2].astype(np.float32)
    u = c32[:, 1::2].astype(np.float32)
    with np.errstate(over="ignore"):
        return (g / (np.float32(1) + np.exp(-g))) * u


def test_swiglu_check_accepts_float32_activation_and_rejects_mistakes(case):
    c32, ref, s = case
    h = oracle.round_to_bf16(_swiglu_f32(c32).astype(np.float64))
    parity.check_swiglu_bf16(h, ref, s, "float32 swiglu")
    swapped = oracle.round_to_bf16(_swiglu_f32(c32[:, [i ^ 1 for i in range(c32.shape[1])]])
                                   .astype(np.float64))
    with pytest.raises(AssertionError):
        parity.check_swiglu_bf16(swapped, ref, s, "gate and up swapped")
    bad = h.copy()
    bad[7, 4] = oracle.round_to_bf16(bad[7, 4] * 1.02 + 1e-3)
    with pytest.raises(AssertionError):
        parity.check_swiglu_bf16(bad, ref, s, "one element")
    with pytest.raises(AssertionError):  # sigmoid instead of silu
        g, u = c32[:, 0::2].astype(np.float64), c32[:, 1::2].astype(np.float64)
        parity.check_swiglu_bf16(oracle.round_to_bf16(u / (1 + np.exp(-g))), ref, s, "sigmoid")


def test_silu_range_brackets_samples():
    rng = np.random.default_rng(4)
    lo = rng.normal(0, 3, 2000)
    hi = lo + rng.exponential(1.0, 2000)
    smin, smax = parity.silu_range(lo, hi)
    t = rng.random((2000, 64))
    x = lo[:, None] + t * (hi - lo)[:, None]
    v = oracle.silu(x)
    assert (v.min(axis=1) >= smin - 1e-15).all()
    assert (v.max(axis=1) <= smax + 1e-15).all()
    # the interior minimum is attained: silu(x*) = -W(1/e) ~ -0.2785
    m = (lo < -1.3) & (hi > -1.25)
    assert m.any() and np.allclose(smin[m], -0.2784645427610738, rtol=1e-12)


def test_swiglu_bounds_cover_saturated_gates():
    # a gate of -200: e^200 overflows float32, the kernel returns -0 * u; the
    # exact value is about -2.8e-85 * u; both must be inside the bracket
    c = np.array([[-200.0, 3.0, 150.0, -2.0]])
    s = np.array([[1.0, 1.0, 1.0, 1.0]])
    parity.check_swiglu_bf16(np.array([[-0.0, -300.0]]), c, s, "saturated, kernel")
    exact = oracle.swiglu_pairs(c)
    assert -1e-80 < exact[0, 0] < 0.0
    parity.check_swiglu_bf16(oracle.round_to_bf16(exact), c, s, "saturated, exact")
    with pytest.raises(AssertionError):
        parity.check_swiglu_bf16(np.array([[-1e-3, -300.0]]), c, s, "saturated, wrong")


def test_combine_check_accepts_float32_atomics_and_rejects_mistakes():
    rng = np.random.default_rng(15)
    n_tokens, E, K, N, topk = 40, 6, 256, 40, 3
    pairs = sorted((int(e), t) for t in range(n_tokens) for e in rng.choice(E, topk, replace=False))
    sizes = np.bincount([p[0] for p in pairs], minlength=E)
    src = np.array([p[1] for p in pairs], dtype=np.int32)
    w = wl.make_workload(E=E, K=K, N=N, sizes=[int(x) for x in sizes], seed=16)
    X = wl.make_workload(E=1, K=K, N=8, sizes=[n_tokens], seed=17).A
    gate = rng.random(len(src)).astype(np.float32)
    Y, SW, AY, terms = oracle.grouped_gemm_combine(X, src, w.B, w.offsets, src, gate, n_tokens)
    # float32 stand-in: float32 products, weights applied in float32, terms
    # added in a shuffled order in float32
    xf, bf = _bf16_to_f32(X), _bf16_to_f32(w.B)
    experts = np.repeat(np.arange(E), sizes)
    y32 = np.zeros((n_tokens, N), dtype=np.float32)
    for r in rng.permutation(len(src)):
        y32[src[r]] += gate[r] * (xf[src[r]] @ bf[experts[r]])
    parity.check_combine(y32, Y, SW, AY, terms, "float32 combine")
    with pytest.raises(AssertionError):  # a route dropped
        y_bad = y32.copy()
        y_bad[src[0]] -= gate[0] * (xf[src[0]] @ bf[experts[0]])
        parity.check_combine(y_bad, Y, SW, AY, terms, "dropped route")
    with pytest.raises(AssertionError):  # weights ignored
        y_bad = np.zeros_like(y32)
        for r in range(len(src)):
            y_bad[src[r]] += xf[src[r]] @ bf[experts[r]]
        parity.check_combine(y_bad, Y, SW, AY, terms, "unweighted")


def test_fp8_group_bound_and_check():
    rng = np.random.default_rng(18)
    m, K, N = 6, 64, 5
    a = rng.normal(size=(m, K)) * np.where(rng.random((m, K)) < 0.1, 300.0, 1.0)
    w = rng.normal(size=(K, N))
    # G by brute force
    G = parity.fp8_group_max_sum(a, w)
    for r in range(m):
        for n in range(N):
            want = sum(max(abs(a[r, k] * w[k, n]) for k in range(g, g + 8)) for g in range(0, K, 8))
            assert abs(G[r, n] - want) <= 1e-12 * want
    exact = a @ w
    S = np.abs(a) @ np.abs(w)
    # emulate the observed hardware sum: in each group of 8, products at or
    # below 2^-14 of the group's largest are dropped
    hw = np.zeros((m, N))
    for r in range(m):
        for n in range(N):
            for g in range(0, K, 8):
                p = a[r, g:g + 8] * w[g:g + 8, n]
                big = np.abs(p).max()
                hw[r, n] += p[np.abs(p) > 2.0 ** -14 * big].sum()
    parity.check_fp8(exact, exact, S, G, K, "exact")
    parity.check_fp8(hw, exact, S, G, K, "group-truncated")
    with pytest.raises(AssertionError):
        parity.check_fp8(exact * 1.01, exact, S, G, K, "scaled by 1.01")
    # without outliers, losing one whole product is far outside the bound
    a2 = rng.normal(size=(m, K))
    e2 = a2 @ w
    S2, G2 = np.abs(a2) @ np.abs(w), parity.fp8_group_max_sum(a2, w)
    parity.check_fp8(e2, e2, S2, G2, K, "exact, no outliers")
    with pytest.raises(AssertionError):
        parity.check_fp8(e2 - a2[:, 5:6] @ w[5:6, :], e2, S2, G2, K, "one k dropped")
