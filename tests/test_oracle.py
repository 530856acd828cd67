"""Pins for the CPU oracle (no GPU).

Each test checks the oracle against something other than itself: a scalar
brute force written from the textbook definition, numpy's float64 matrix
product (a library routine), closed forms (identity and permutation weights,
the multiply-add count) and the figures the worklog prints (tests/golden).
A dropped term, a wrong index, a transposed operand or a wrong expert slice
in the oracle fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


def _decode(bits):
    return wl.bf16_bits_to_f32(bits).astype(np.float64)


def _py_brute(A, B, off):
    """Scalar triple loop from the definition, pure Python floats, no numpy math."""
    E, K, N = B.shape
    Af = _decode(A).tolist()
    Bf = _decode(B).tolist()
    out = {}
    for e in range(E):
        for i in range(int(off[e]), int(off[e + 1])):
            for j in range(N):
                acc = 0.0
                for k in range(K):
                    acc += Af[i][k] * Bf[e][k][j]
                out[(i, j)] = acc
    return out


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_brute_force_integer_inputs(seed):
    rng = np.random.default_rng(100 + seed)
    E = int(rng.integers(1, 4))
    K = int(rng.integers(1, 9))
    N = int(rng.integers(1, 9))
    sizes = rng.integers(0, 6, size=E)
    w = wl.make_workload(E=E, K=K, N=N, sizes=sizes, seed=seed, values="int", M_cap=int(sizes.sum()) + 2)
    C, S, madds = oracle.grouped_gemm(w.A, w.B, w.offsets)
    ref = _py_brute(w.A, w.B, w.offsets)
    for (i, j), v in ref.items():
        assert C[i, j] == v  # integers below 2^24: exact in any order
    # rows outside every group untouched
    assert np.isnan(C[w.M_tot:]).all()
    assert madds == int(sizes.sum()) * K * N


@pytest.mark.parametrize("name", ["tiny"])
def test_tiny_against_python_brute_force(name):
    w = wl.make_workload(name)
    C, _, _ = oracle.grouped_gemm(w.A, w.B, w.offsets)
    ref = _py_brute(w.A[:, :64], w.B[:, :64, :8], w.offsets)  # K,N cut for speed
    Cc, _, _ = oracle.grouped_gemm(np.ascontiguousarray(w.A[:, :64]), np.ascontiguousarray(w.B[:, :64, :8]), w.offsets)
    for (i, j), v in ref.items():
        assert Cc[i, j] == pytest.approx(v, rel=1e-15, abs=1e-300)
    assert np.isfinite(C).all()


def _numpy_per_expert(w):
    Af = _decode(w.A)
    Bf = _decode(w.B)
    out = np.full((w.M_cap, w.N), np.nan)
    sab = np.full((w.M_cap, w.N), np.nan)
    for e in range(w.E):
        r0, r1 = int(w.offsets[e]), int(w.offsets[e + 1])
        out[r0:r1] = Af[r0:r1] @ Bf[e]
        sab[r0:r1] = np.abs(Af[r0:r1]) @ np.abs(Bf[e])
    return out, sab


@pytest.mark.parametrize("case", [
    dict(name="tiny"),
    dict(E=5, K=96, N=40, sizes=[7, 0, 33, 1, 12], seed=11),
    dict(E=3, K=200, N=24, sizes=[0, 50, 0], seed=12),
    dict(E=1, K=64, N=64, sizes=[65], seed=13),
])
def test_equals_separate_dense_products(case):
    w = wl.make_workload(case.pop("name")) if "name" in case else wl.make_workload(**case)
    C, S, _ = oracle.grouped_gemm(w.A, w.B, w.offsets)
    ref, sref = _numpy_per_expert(w)
    m = w.M_tot
    # different summation orders of the same fp64 sum: |diff| <= K * 2^-53 * S
    bound = w.K * 2.0 ** -53 * sref[:m] + 1e-300
    assert (np.abs(C[:m] - ref[:m]) <= bound).all()
    assert np.allclose(S[:m], sref[:m], rtol=w.K * 2.0 ** -52, atol=0)
    assert (S[:m] >= np.abs(C[:m])).all()


def test_transposed_or_wrong_expert_is_caught():
    # the dense-product pin really distinguishes a transposed B or a shifted expert
    w = wl.make_workload(E=3, K=32, N=32, sizes=[5, 6, 7], seed=21)
    C, _, _ = oracle.grouped_gemm(w.A, w.B, w.offsets)
    Bt = np.ascontiguousarray(np.transpose(w.B, (0, 2, 1)))
    Ct, _, _ = oracle.grouped_gemm(w.A, Bt, w.offsets)
    assert not np.allclose(C, Ct)
    Bs = np.ascontiguousarray(np.roll(w.B, 1, axis=0))
    Cs, _, _ = oracle.grouped_gemm(w.A, Bs, w.offsets)
    assert not np.allclose(C, Cs)


@pytest.mark.parametrize("sizes", [
    [0, 0, 5, 3], [4, 2, 0, 0], [3, 0, 0, 4], [0, 0, 0, 0], [7], [0], [0, 9, 0],
])
def test_empty_groups_write_no_rows(sizes):
    E = len(sizes)
    w = wl.make_workload(E=E, K=16, N=24, sizes=sizes, seed=5, M_cap=sum(sizes) + 3)
    C, S, madds = oracle.grouped_gemm(w.A, w.B, w.offsets)
    m = w.M_tot
    assert np.isfinite(C[:m]).all() and np.isfinite(S[:m]).all()
    assert np.isnan(C[m:]).all() and np.isnan(S[m:]).all()
    assert madds == m * 16 * 24


def test_identity_weights_reproduce_a_exactly():
    w = wl.make_workload("tiny")
    eye = wl.f32_to_bf16_bits(np.eye(256, dtype=np.float32))
    B = np.broadcast_to(eye, (4, 256, 256)).copy()
    C, _, _ = oracle.grouped_gemm(w.A, B, w.offsets)
    assert (C == wl.bf16_bits_to_f32(w.A).astype(np.float64)).all()


def test_permutation_weights_permute_columns_exactly():
    w = wl.make_workload("tiny")
    rng = np.random.default_rng(7)
    B = np.zeros((4, 256, 256), dtype=np.uint16)
    perms = []
    for e in range(4):
        p = rng.permutation(256)
        P = np.zeros((256, 256), dtype=np.float32)
        P[p, np.arange(256)] = 1.0  # column j takes input column p[j]
        B[e] = wl.f32_to_bf16_bits(P)
        perms.append(p)
    C, _, _ = oracle.grouped_gemm(w.A, B, w.offsets)
    Af = wl.bf16_bits_to_f32(w.A).astype(np.float64)
    for e in range(4):
        r0, r1 = int(w.offsets[e]), int(w.offsets[e + 1])
        assert (C[r0:r1] == Af[r0:r1][:, perms[e]]).all()


def test_group_split_invariance_bitwise():
    w = wl.make_workload(E=2, K=80, N=48, sizes=[20, 9], seed=31)
    C, S, _ = oracle.grouped_gemm(w.A, w.B, w.offsets)
    # split expert 0 into rows [0,8) and [8,20), both using B_0
    off2 = np.array([0, 8, 20, 29], dtype=np.int32)
    B2 = np.ascontiguousarray(np.stack([w.B[0], w.B[0], w.B[1]]))
    C2, S2, _ = oracle.grouped_gemm(w.A, B2, off2)
    assert (C2 == C).all() and (S2 == S).all()


def test_flop_count_closed_form():
    w = wl.make_workload(E=4, K=40, N=8, sizes=[3, 0, 11, 2], seed=3)
    _, _, madds = oracle.grouped_gemm(w.A, w.B, w.offsets, want_s=False)
    assert 2 * madds == oracle.useful_flops(16, 40, 8) == 2 * 16 * 40 * 8
    g = json.load(open(GOLDEN))["useful_work"][0]
    f = oracle.useful_flops(g["m_tot"], g["K"], g["N"])
    assert f == 90_194_313_216
    assert round(f / 1e9, 1) == g["gflop_rounded_1dp"]


def test_entries_match_full_and_numpy():
    w = wl.make_workload(E=3, K=300, N=50, sizes=[10, 0, 25], seed=41)
    C, S, _ = oracle.grouped_gemm(w.A, w.B, w.offsets)
    rng = np.random.default_rng(0)
    rows = rng.integers(0, w.M_tot, size=40)
    cols = rng.integers(0, w.N, size=40)
    c, s = oracle.grouped_gemm_entries(w.A, w.B, w.offsets, rows, cols)
    assert (c == C[rows, cols]).all() and (s == S[rows, cols]).all()
    Af = _decode(w.A)
    Bf = _decode(w.B)
    for t in range(40):
        e = int(np.searchsorted(w.offsets, rows[t], side="right") - 1)
        assert c[t] == pytest.approx(float(np.dot(Af[rows[t]], Bf[e][:, cols[t]])), rel=1e-13, abs=1e-15)


def test_malformed_offsets_rejected():
    w = wl.make_workload(E=2, K=8, N=8, sizes=[2, 2], seed=1)
    for bad in ([1, 2, 4], [0, 3, 2], [0, 2, 9]):
        with pytest.raises(ValueError):
            oracle.grouped_gemm(w.A, w.B, np.array(bad, dtype=np.int32))


# ---- tile list, eta and byte model against the worklog's printed figures ----

def _golden_sizes(name):
    if name == "uniform16k":
        return [256] * 64
    if name == "skew16k_page":
        return list(wl.page_skew_sizes(16384, 64, 1.2))
    if name == "uniform2k":
        return [32] * 64
    raise KeyError(name)


def test_page_skew_law_figures():
    for g in json.load(open(GOLDEN))["skew_law"]:
        s = wl.page_skew_sizes(g["m_tot"], g["experts"], g["s"])
        assert int(s.sum()) == g["m_tot"]
        assert int(s.max()) == g["largest"] and int(s.min()) == g["smallest"]


def test_tile_counts_from_pages():
    for g in json.load(open(GOLDEN))["tile_counts"]:
        sizes = _golden_sizes(g["workload"])
        off = wl.offsets_from_sizes(sizes)
        tiles = oracle.tile_list(off, 2688, g["bm"], g["bn"])
        assert len(tiles) == g["count"], g["cite"]


def test_tile_list_structure():
    off = wl.offsets_from_sizes([3, 0, 17, 9, 0])
    tiles = oracle.tile_list(off, 256, 16, 128)
    # expert 1 and 4 empty: no tiles; expert 2 -> 2 M tiles x 2 N tiles
    assert tiles == [
        (0, 0, 3, 0), (0, 0, 3, 128),
        (2, 3, 16, 0), (2, 3, 16, 128), (2, 19, 1, 0), (2, 19, 1, 128),
        (3, 20, 9, 0), (3, 20, 9, 128),
    ]
    # every valid (row, col-block) is covered exactly once, never past the expert
    cover = {}
    for e, r0, rows, c0 in oracle.tile_list(off, 200, 16, 64):
        assert rows >= 1 and r0 >= off[e] and r0 + rows <= off[e + 1]
        for r in range(r0, r0 + rows):
            cover[(r, c0)] = cover.get((r, c0), 0) + 1
    assert set(cover.values()) == {1} and len(cover) == 29 * 4


def test_eta_from_pages():
    for g in json.load(open(GOLDEN))["eta"]:
        v = oracle.eta(_golden_sizes(g["workload"]), g["bm"])
        if "waste_pct" in g:
            assert round(100 * (1 - v), 1) == g["waste_pct"], g["cite"]
        if "eta" in g:
            assert round(v, 3) == g["eta"], g["cite"]


def test_eta_estimates_from_pages():
    for g in json.load(open(GOLDEN))["eta_estimates"]:
        # the page multiplies by eta as it prints it, to three places (0.780, 0.250)
        v = round(oracle.eta(_golden_sizes(g["workload"]), g["bm"]), 3)
        assert round(oracle.eta_estimate(g["balanced"], v), 1) == g["estimate"], g["cite"]


def test_compulsory_bytes_from_pages():
    for g in json.load(open(GOLDEN))["compulsory_bytes"]:
        b = oracle.algorithmic_bytes(_golden_sizes(g["workload"]), 1024, 2688, c_bytes=g["c_bytes"])
        assert b == 473_956_352
        assert round(b / 1e6) == g["mb_rounded"]
    # the fp32-output figure used for this library, and empty experts' B not counted
    assert oracle.algorithmic_bytes([256] * 64, 1024, 2688) == 562_036_736
    assert oracle.algorithmic_bytes([3, 0, 17, 9], 256, 256) == (2 * 29 * 256 + 2 * 256 * 256 * 3 + 4 * 29 * 256)


def test_adaptive_bm_special_cases():
    # multiples of the largest height and very small experts are decided by padding alone
    assert oracle.adaptive_bm([256, 512, 4096]) == [256, 256, 256]
    assert oracle.adaptive_bm([1, 5, 16]) == [16, 16, 16]
    assert oracle.adaptive_bm([32]) == [32]
    assert oracle.adaptive_bm([0]) == [16]
    # worked by hand: m=48 -> costs 16:3*80=240, 32:2*96=192, 64:1*128=128, 128:192, 256:320 -> 64
    assert oracle.adaptive_bm([48]) == [64]
    # m=128 -> 64:2*128=256, 128:1*192=192, 256:320 -> 128
    assert oracle.adaptive_bm([128]) == [128]
    # m=130 -> 64:3*128=384, 128:2*192=384, 256:1*320=320 -> 256
    assert oracle.adaptive_bm([130]) == [256]
    # m=100 -> 64:2*128=256, 128:192, 256:320 -> 128
    assert oracle.adaptive_bm([100]) == [128]
    # eta never below the uniform-BM=128 eta on the page skew law
    s = _golden_sizes("skew16k_page")
    assert oracle.eta(s, oracle.adaptive_bm(s)) >= oracle.eta(s, 128)


def test_tile_widths_hand_worked():
    # every expert with rows takes 16-row tiles: those tiles are 512 wide
    assert oracle.tile_widths([16, 16, 16], [3, 16, 0]) == [512, 512, 512]
    # one expert with rows takes taller tiles: every width stays 256
    assert oracle.tile_widths([16, 32, 16], [5, 20, 1]) == [256, 256, 256]
    # an expert without rows does not take part, whatever its height
    assert oracle.tile_widths([16, 256], [7, 0]) == [512, 256]
    # no rows at all: nothing is tall, 16-row experts would be wide
    assert oracle.tile_widths([16, 16], [0, 0]) == [512, 512]
    # a fixed height above 16 never gives wide tiles
    assert oracle.tile_widths([64, 64], [1, 1]) == [256, 256]
    # with the adaptive height rule: 32 experts x 16 rows (the decode shape)
    # are all 16 high, hence 512 wide; one 17-row expert makes all narrow
    hs = oracle.adaptive_bm([16] * 32)
    assert oracle.tile_widths(hs, [16] * 32) == [512] * 32
    sz = [16] * 31 + [17]
    assert oracle.tile_widths(oracle.adaptive_bm(sz), sz) == [256] * 32
    with pytest.raises(ValueError):
        oracle.tile_widths([16], [1, 2])


def test_tile_widths_tile_counts():
    # the decode shape: 32 experts x ceil(4096/512) = 256 tiles; with the
    # 256-wide rule it would be 512 (one per CU pair)
    sizes = [16] * 32
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    hs = oracle.adaptive_bm(sizes)
    assert len(oracle.tile_list(off, 4096, hs, oracle.tile_widths(hs, sizes))) == 256
    assert len(oracle.tile_list(off, 4096, hs, oracle.TILE_WIDTH)) == 512


def test_round_to_bf16_definition_cases():
    # values of the format map to themselves; ties go to the even significand;
    # anything past a tie goes up; the subnormal spacing is 2^-133; the largest
    # finite bf16 is (2 - 2^-7) * 2^127 and a value that rounds past it is inf
    cases = [
        (1.0, 1.0), (1.0 + 2 ** -7, 1.0 + 2 ** -7), (-3.5, -3.5), (2.0 ** -126, 2.0 ** -126),
        (1.0 + 2 ** -8, 1.0),                          # tie, 1.0 is even
        (1.0 + 3 * 2 ** -8, 1.0 + 2 ** -6),            # tie, 1 + 2^-6 is even
        (1.0 + 2 ** -8 + 2 ** -30, 1.0 + 2 ** -7),     # just past the tie
        (-(1.0 + 2 ** -8 + 2 ** -30), -(1.0 + 2 ** -7)),
        (255.0, 255.0), (257.0, 256.0), (259.0, 260.0),  # integers: spacing 2 above 256
        (2.0 ** -130 + 2.0 ** -134, 2.0 ** -130),      # subnormal tie to even
        (3 * 2.0 ** -134, 2.0 ** -132),                # 1.5 units of 2^-133: tie to 2
        ((2 - 2 ** -7) * 2.0 ** 127, (2 - 2 ** -7) * 2.0 ** 127),
        ((2 - 2 ** -9) * 2.0 ** 127, math.inf),
        (0.0, 0.0),
    ]
    x = np.array([c[0] for c in cases])
    want = np.array([c[1] for c in cases])
    assert (oracle.round_to_bf16(x) == want).all(), (oracle.round_to_bf16(x), want)


def test_round_to_bf16_matches_torch_on_fp32_values():
    # on binary32 inputs the binary64 rounding must agree with torch's fp32 ->
    # bf16 conversion (a library routine; no double rounding is possible since
    # the inputs are exact in both formats)
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(200000) * s for s in (1e-3, 1.0, 37.0, 1e5)])
    x32 = x.astype(np.float32)
    want = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    assert (oracle.round_to_bf16(x32.astype(np.float64)) == want).all()
    # monotone nondecreasing
    xs = np.sort(x)
    assert (np.diff(oracle.round_to_bf16(xs)) >= 0).all()


def test_indexed_identity_is_the_grouped_product():
    w = wl.make_workload(E=3, K=40, N=24, sizes=[5, 0, 9], seed=31)
    src = np.arange(w.M_cap)
    c1, s1 = oracle.grouped_gemm_indexed(w.A, src, w.B, w.offsets)
    c0, s0, _ = oracle.grouped_gemm(w.A, w.B, w.offsets)
    m = w.M_tot
    assert np.array_equal(c1[:m], c0[:m]) and np.array_equal(s1[:m], s0[:m])
    assert np.isnan(c1[m:]).all()


def test_indexed_brute_force_gather_scatter():
    # integer inputs, so every sum is exact; a scalar Python definition of
    # gather -> per-expert product -> scatter, with an out-of-range source
    # (zero row) and an out-of-range destination (row not written)
    rng = np.random.default_rng(32)
    E, K, N, n_src = 3, 6, 5, 7
    X = wl.f32_to_bf16_bits(rng.integers(-3, 4, size=(n_src, K)).astype(np.float32))
    B = wl.f32_to_bf16_bits(rng.integers(-3, 4, size=(E, K, N)).astype(np.float32))
    off = np.array([0, 3, 3, 8], dtype=np.int32)
    src = np.array([4, 0, 6, 2, 2, 99, 1, 5, 0, 0])
    dst = np.array([9, 7, 5, 3, 1, 0, 2, -1, 4, 6])
    got, _ = oracle.grouped_gemm_indexed(X, src, B, off, dst, M_cap=10)
    xf, bf = wl.bf16_bits_to_f32(X), wl.bf16_bits_to_f32(B)
    want = np.full((10, N), np.nan)
    for e in range(E):
        for r in range(off[e], off[e + 1]):
            if not 0 <= dst[r] < 10:
                continue
            for j in range(N):
                acc = 0.0
                for k in range(K):
                    a = float(xf[src[r], k]) if 0 <= src[r] < n_src else 0.0
                    acc += a * float(bf[e, k, j])
                want[dst[r], j] = acc
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.array_equal(got[~np.isnan(got)], want[~np.isnan(want)])
    assert (got[0] == 0).all()  # grouped row 5 reads source 99 -> zero row


def test_indexed_permutation_invariance():
    # permuting the source rows and the index list together changes nothing
    w = wl.make_workload(E=4, K=48, N=32, sizes=[7, 3, 0, 11], seed=33)
    rng = np.random.default_rng(34)
    perm = rng.permutation(w.M_cap)
    X = w.A[perm]
    inv = np.argsort(perm)
    c1, _ = oracle.grouped_gemm_indexed(X, inv, w.B, w.offsets)
    c0, _, _ = oracle.grouped_gemm(w.A, w.B, w.offsets)
    m = w.M_tot
    assert np.array_equal(c1[:m], c0[:m])


def test_decode_e4m3_against_torch_and_definition():
    torch = pytest.importorskip("torch")
    codes = np.arange(256)
    d = oracle.decode_e4m3(codes)
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    both_nan = np.isnan(d) & np.isnan(ref)
    assert ((d == ref) | both_nan).all()
    assert np.isnan(d[[0x7F, 0xFF]]).all() and np.isnan(d).sum() == 2
    assert d[0x7E] == 448.0 and d[0xFE] == -448.0     # largest finite
    assert d[0x38] == 1.0 and d[0xB8] == -1.0
    assert d[0x01] == 2.0 ** -9 and d[0x08] == 2.0 ** -6  # smallest subnormal / normal


def _int_codes(vals):
    # E4M3 codes of small integers: 1 = 0x38, 2 = 0x40, 3 = 0x44, sign in bit 7
    table = {0: 0x00, 1: 0x38, 2: 0x40, 3: 0x44}
    v = np.asarray(vals)
    return (np.vectorize(table.get)(np.abs(v)) | ((v < 0) << 7)).astype(np.uint8)


def test_fp8w_brute_force_integers():
    rng = np.random.default_rng(35)
    E, K, N = 3, 7, 5
    sizes = [2, 0, 4]
    off = wl.offsets_from_sizes(sizes)
    A = wl.f32_to_bf16_bits(rng.integers(-3, 4, size=(6, K)).astype(np.float32))
    qv = rng.integers(-3, 4, size=(E, K, N))
    Bq = _int_codes(qv)
    scale = np.ldexp(1.0, rng.integers(-3, 4, size=(E, N))).astype(np.float32)
    c, s = oracle.grouped_gemm_fp8w(A, Bq, scale, off)
    af = wl.bf16_bits_to_f32(A)
    for e in range(E):
        for r in range(off[e], off[e + 1]):
            for n in range(N):
                acc = 0.0
                for k in range(K):
                    acc += float(af[r, k]) * float(qv[e, k, n])
                assert c[r, n] == acc * float(scale[e, n])


def test_fp8w_unit_scale_reduces_to_bf16_product():
    # every E4M3 value is a bf16 value, so with unit scales the fp8-weight
    # product is the bf16 grouped product of the decoded weights
    w = wl.make_workload(E=3, K=96, N=40, sizes=[9, 4, 0], seed=36)
    rng = np.random.default_rng(37)
    Bq = rng.integers(0, 256, size=(3, 96, 40)).astype(np.uint8)
    Bq[(Bq & 0x7F) == 0x7F] = 0x3C  # no NaN codes
    ones = np.ones((3, 40), dtype=np.float32)
    c, s = oracle.grouped_gemm_fp8w(w.A, Bq, ones, w.offsets)
    Bbf = wl.f32_to_bf16_bits(oracle.decode_e4m3(Bq).astype(np.float32))
    c0, s0, _ = oracle.grouped_gemm(w.A, Bbf, w.offsets)
    m = w.M_tot
    assert np.allclose(c[:m], c0[:m], rtol=0, atol=1e-12 * s0[:m].max())
    assert np.allclose(s[:m], s0[:m], rtol=1e-14)


def test_e4m3_bf16_table_against_torch():
    # the bfloat16 pattern of every finite code is torch's own conversion of
    # the same value, and widening it back gives the code's value exactly
    torch = pytest.importorskip("torch")
    t = oracle.e4m3_bf16_table()
    vals = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float()
    ref = vals.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    finite = np.isfinite(vals.numpy())
    assert (t[finite] == ref[finite]).all()
    back = wl.bf16_bits_to_f32(t).astype(np.float64)
    assert (back[finite] == oracle.decode_e4m3(np.arange(256))[finite]).all()
    assert t[0x38] == 0x3F80 and t[0xB8] == 0xBF80 and t[0x7E] == 0x43E0  # 1, -1, 448


def test_fp8w_whole_matches_definition():
    # the whole-size route (codes as bf16 patterns, C triple loop, column
    # scales) against the definition written with numpy products
    w = wl.make_workload(E=4, K=72, N=48, sizes=[6, 0, 13, 2], seed=40, M_cap=24)
    q, scale = wl.fp8_weights(w)
    c0, s0 = oracle.grouped_gemm_fp8w(w.A, q, scale, w.offsets)
    c1, s1 = oracle.grouped_gemm_fp8w_whole(w.A, q, scale, w.offsets)
    m = w.M_tot
    tol = 72 * 2.0 ** -52 * s0[:m]
    assert (np.abs(c1[:m] - c0[:m]) <= tol).all()
    assert np.allclose(s1[:m], s0[:m], rtol=1e-14, atol=0)
    assert np.isnan(c1[m:]).all()
    # integer codes with power-of-two scales: exact, both ways
    rng = np.random.default_rng(41)
    qv = rng.integers(-3, 4, size=(2, 9, 7))
    Bq = _int_codes(qv)
    sc = np.ldexp(1.0, rng.integers(-2, 3, size=(2, 7))).astype(np.float32)
    A = wl.f32_to_bf16_bits(rng.integers(-3, 4, size=(5, 9)).astype(np.float32))
    off = wl.offsets_from_sizes([3, 2])
    a, _ = oracle.grouped_gemm_fp8w(A, Bq, sc, off)
    b, _ = oracle.grouped_gemm_fp8w_whole(A, Bq, sc, off)
    assert np.array_equal(a, b)
    with pytest.raises(ValueError):
        bad = Bq.copy()
        bad[0, 0, 0] = 0x7F
        oracle.grouped_gemm_fp8w_whole(A, bad, sc, off)


def test_fp8w_column_scale_is_linear_and_entries_match():
    w = wl.make_workload(E=2, K=64, N=24, sizes=[5, 7], seed=38)
    q, scale = wl.fp8_weights(w)
    c, _ = oracle.grouped_gemm_fp8w(w.A, q, scale, w.offsets)
    scale2 = scale.copy()
    scale2[:, 3] *= 2
    c2, _ = oracle.grouped_gemm_fp8w(w.A, q, scale2, w.offsets)
    assert np.array_equal(c2[:, 3], 2 * c[:, 3])
    rows = np.arange(w.M_tot).repeat(3)
    cols = np.tile([0, 11, 23], w.M_tot)
    ce, _ = oracle.grouped_gemm_fp8w_entries(w.A, q, scale, w.offsets, rows, cols)
    assert np.allclose(ce, c[rows, cols], rtol=1e-14, atol=1e-14)


def test_fp8_weight_recipe_is_close_to_bf16_weights():
    # the input recipe: per-column scale maps the largest |w| to 448, and the
    # quantized weight is within half an E4M3 spacing (2^-4 relative) of it
    w = wl.make_workload(E=2, K=128, N=32, sizes=[1, 1], seed=39)
    q, scale = wl.fp8_weights(w)
    b = wl.bf16_bits_to_f32(w.B).astype(np.float64)
    deq = oracle.decode_e4m3(q) * scale[:, None, :]
    assert (np.abs(oracle.decode_e4m3(q)).max(axis=1) == 448.0).all()
    assert (np.abs(deq - b) <= 2.0 ** -4 * np.abs(b) + 2.0 ** -10 * scale[:, None, :]).all()


# ---- SwiGLU on (gate, up) column pairs ------------------------------------------

def test_silu_against_library_sigmoid():
    # silu(x) = x * sigmoid(x); scipy's expit is an independent sigmoid
    special = pytest.importorskip("scipy.special")
    x = np.concatenate([np.linspace(-60, 60, 2401), [-700.0, -30.5, -1e-12, 0.0, 1e-12, 30.5, 700.0]])
    want = x * special.expit(x)
    got = oracle.silu(x)
    assert np.allclose(got, want, rtol=4e-16, atol=0.0)
    assert oracle.silu(0.0) == 0.0


def test_silu_closed_forms():
    rng = np.random.default_rng(3)
    x = rng.normal(0, 4, 10000)
    # sigmoid(-x) = 1 - sigmoid(x), so silu(x) - silu(-x) = x
    assert np.allclose(oracle.silu(x) - oracle.silu(-x), x, rtol=1e-14, atol=1e-14)
    # silu(x) -> x for large x, -> 0 (from below) for very negative x
    assert oracle.silu(40.0) == 40.0
    assert -1e-300 < oracle.silu(-800.0) <= 0.0
    # sigmoid(1) = e / (1 + e)
    assert abs(oracle.silu(1.0) - math.e / (1.0 + math.e)) < 1e-16


def test_silu_minimum_is_minus_lambert_w():
    # silu'(x) = 0 where 1 + x + e^x = 0, i.e. x* = -1 - W(1/e); there
    # silu(x*) = -W(1/e), the global minimum
    special = pytest.importorskip("scipy.special")
    w = float(special.lambertw(1.0 / math.e).real)
    x_star = -1.0 - w
    assert abs(oracle.silu(x_star) + w) < 1e-15
    near = oracle.silu(np.array([x_star - 1e-4, x_star + 1e-4, -5.0, 0.0, 5.0]))
    assert (near > -w).all()


def test_swiglu_pairs_gate_even_up_odd():
    special = pytest.importorskip("scipy.special")
    C = np.array([[2.0, 3.0, -1.0, 5.0], [0.5, -4.0, 7.0, 0.25]])
    want = np.array([[2.0 * special.expit(2.0) * 3.0, -1.0 * special.expit(-1.0) * 5.0],
                     [0.5 * special.expit(0.5) * -4.0, 7.0 * special.expit(7.0) * 0.25]])
    got = oracle.swiglu_pairs(C)
    assert got.shape == (2, 2)
    assert np.allclose(got, want, rtol=1e-15, atol=0.0)
    # swapping gate and up changes the result (the layout is not symmetric)
    assert not np.allclose(oracle.swiglu_pairs(C[:, [1, 0, 3, 2]]), want)
    with pytest.raises(ValueError):
        oracle.swiglu_pairs(np.zeros((2, 3)))


def test_swiglu_of_identity_product_is_swiglu_of_a():
    # B[e] = I: the product is A (exact), so H = silu(A[:, even]) * A[:, odd],
    # computed here one scalar at a time with the math module
    w = wl.make_workload(E=3, K=16, N=16, sizes=[3, 0, 4], seed=9)
    B = np.zeros_like(w.B)
    one = np.uint16(0x3F80)  # bf16 1.0
    for e in range(3):
        B[e][np.arange(16), np.arange(16)] = one
    C, _, _ = oracle.grouped_gemm(w.A, B, w.offsets, want_s=False)
    H = oracle.swiglu_pairs(C[: w.M_tot])
    a = (w.A[: w.M_tot].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for r in range(w.M_tot):
        for j in range(8):
            g, u = a[r, 2 * j], a[r, 2 * j + 1]
            assert H[r, j] == pytest.approx(g / (1.0 + math.exp(-g)) * u, rel=1e-15, abs=0.0)


# ---- weighted combine after the grouped product ----------------------------------

def _routing(n_tokens, E, topk, rng):
    pairs = sorted((int(e), t, k) for t in range(n_tokens)
                   for k, e in enumerate(rng.choice(E, size=topk, replace=False)))
    sizes = np.bincount([p[0] for p in pairs], minlength=E)
    src = np.array([p[1] for p in pairs], dtype=np.int32)
    slot = np.array([p[2] for p in pairs], dtype=np.int32)
    expert = np.array([p[0] for p in pairs], dtype=np.int32)
    return sizes, src, slot, expert


def test_combine_brute_force_token_major():
    # Y[t] = sum over token t's routes (e, w) of w * (x_t @ B[e]), computed
    # token by token with scalar Python loops, independent of the grouped
    # layout the oracle works in
    rng = np.random.default_rng(12)
    n_tokens, E, K, N, topk = 7, 4, 6, 5, 2
    sizes, src, slot, expert = _routing(n_tokens, E, topk, rng)
    w = wl.make_workload(E=E, K=K, N=N, sizes=[int(x) for x in sizes], seed=5, values="int")
    X = wl.make_workload(E=1, K=K, N=8, sizes=[n_tokens], seed=6, values="int").A
    gate = rng.choice([0.25, 0.5, 0.75, 1.0, -0.5], size=len(src))
    Y, _, _, terms = oracle.grouped_gemm_combine(X, src, w.B, w.offsets, src, gate, n_tokens)
    xf = (X.astype(np.uint32) << 16).view(np.float32)
    bf = (w.B.astype(np.uint32) << 16).view(np.float32)
    for t in range(n_tokens):
        for n in range(N):
            want = 0.0
            for r in range(len(src)):
                if src[r] == t:
                    want += gate[r] * sum(float(xf[t, k]) * float(bf[expert[r], k, n]) for k in range(K))
            assert Y[t, n] == want
    assert (terms == topk).all()


def test_combine_top1_unit_weight_is_the_scatter():
    rng = np.random.default_rng(13)
    sizes, src, _, _ = _routing(20, 5, 1, rng)
    w = wl.make_workload(E=5, K=40, N=24, sizes=[int(x) for x in sizes], seed=7)
    X = wl.make_workload(E=1, K=40, N=8, sizes=[20], seed=8).A
    Y, SW, _, _ = oracle.grouped_gemm_combine(X, src, w.B, w.offsets, src, np.ones(len(src)), 20)
    C, S = oracle.grouped_gemm_indexed(X, src, w.B, w.offsets, dst_rows=src, M_cap=20)
    assert np.array_equal(Y, C) and np.array_equal(SW, S)


def test_combine_linear_in_weights_and_start_values():
    rng = np.random.default_rng(14)
    sizes, src, _, _ = _routing(16, 6, 3, rng)
    w = wl.make_workload(E=6, K=32, N=16, sizes=[int(x) for x in sizes], seed=9)
    X = wl.make_workload(E=1, K=32, N=8, sizes=[16], seed=10).A
    g = rng.random(len(src))
    Y1, _, _, _ = oracle.grouped_gemm_combine(X, src, w.B, w.offsets, src, g, 16)
    Y2, _, _, _ = oracle.grouped_gemm_combine(X, src, w.B, w.offsets, src, 2.0 * g, 16)
    assert np.array_equal(Y2, 2.0 * Y1)  # scaling by 2 is exact
    Y0 = rng.normal(size=(16, 16))
    Y3, _, AY, terms = oracle.grouped_gemm_combine(X, src, w.B, w.offsets, src, g, 16, Y0=Y0)
    assert np.allclose(Y3, Y0 + Y1, rtol=1e-13, atol=1e-13)
    assert (terms == 4).all() and (AY >= np.abs(Y0)).all()
    # destinations out of range are dropped; a negative weight subtracts
    dst = src.copy()
    dst[0] = 16
    Y4, _, _, _ = oracle.grouped_gemm_combine(X, src, w.B, w.offsets, dst, g, 16)
    C, _ = oracle.grouped_gemm_indexed(X, src, w.B, w.offsets, dst_rows=None, M_cap=len(src))
    assert np.allclose(Y4[src[0]], Y1[src[0]] - g[0] * C[0], rtol=1e-12, atol=1e-12)


# ---- fp8 activations and fp8 weights ---------------------------------------------

def test_fp8_brute_force_integers():
    # small integers are exact E4M3 codes; scales are powers of two, so every
    # product and sum is exact and the scalar loop must agree bit for bit
    rng = np.random.default_rng(36)
    E, K, N = 3, 9, 5
    sizes = [2, 0, 4]
    off = wl.offsets_from_sizes(sizes)
    av = rng.integers(-3, 4, size=(6, K))
    qv = rng.integers(-3, 4, size=(E, K, N))
    Aq, Bq = _int_codes(av), _int_codes(qv)
    a_scale = np.ldexp(1.0, rng.integers(-2, 3, size=6)).astype(np.float32)
    b_scale = np.ldexp(1.0, rng.integers(-3, 4, size=(E, N))).astype(np.float32)
    c, s = oracle.grouped_gemm_fp8(Aq, a_scale, Bq, b_scale, off)
    for e in range(E):
        for r in range(off[e], off[e + 1]):
            for n in range(N):
                acc = 0.0
                for k in range(K):
                    acc += float(av[r, k]) * float(qv[e, k, n])
                assert c[r, n] == acc * float(a_scale[r]) * float(b_scale[e, n])
                assert s[r, n] >= abs(c[r, n])


def test_fp8_unit_activation_scale_reduces_to_fp8_weight_product():
    # every E4M3 value is a bf16 value: with unit activation scales the fp8 x
    # fp8 product is the fp8-weight product of the decoded activations
    rng = np.random.default_rng(37)
    E, K, N = 4, 64, 24
    sizes = [5, 0, 9, 3]
    off = wl.offsets_from_sizes(sizes)
    Aq = rng.integers(0, 256, size=(17, K)).astype(np.uint8)
    Aq[(Aq & 0x7F) == 0x7F] = 0x38  # no NaN codes
    Bq = rng.integers(0, 256, size=(E, K, N)).astype(np.uint8)
    Bq[(Bq & 0x7F) == 0x7F] = 0x40
    b_scale = rng.uniform(0.01, 2.0, size=(E, N)).astype(np.float32)
    c1, s1 = oracle.grouped_gemm_fp8(Aq, np.ones(17, np.float32), Bq, b_scale, off)
    A_bf16 = wl.f32_to_bf16_bits(oracle.decode_e4m3(Aq).astype(np.float32))
    c2, s2 = oracle.grouped_gemm_fp8w(A_bf16, Bq, b_scale, off)
    m = int(off[-1])
    assert np.allclose(c1[:m], c2[:m], rtol=1e-12, atol=1e-12 * np.abs(s1[:m]).max())
    assert np.allclose(s1[:m], s2[:m], rtol=1e-12)
    # the activation scale multiplies whole rows; a power of two is exact
    a_scale = np.ldexp(1.0, rng.integers(-4, 5, size=17)).astype(np.float32)
    c3, _ = oracle.grouped_gemm_fp8(Aq, a_scale, Bq, b_scale, off)
    assert np.array_equal(c3[:m], c1[:m] * a_scale[:m, None].astype(np.float64))


def test_fp8_entries_match_full_product():
    rng = np.random.default_rng(38)
    w = wl.make_workload(E=3, K=48, N=32, sizes=[7, 0, 12], seed=39)
    Aq, a_scale = wl.fp8_activations(w)
    Bq, b_scale = wl.fp8_weights(w)
    C, S = oracle.grouped_gemm_fp8(Aq, a_scale, Bq, b_scale, w.offsets)
    rows = rng.integers(0, w.M_tot, size=40)
    cols = rng.integers(0, w.N, size=40)
    c, s = oracle.grouped_gemm_fp8_entries(Aq, a_scale, Bq, b_scale, w.offsets, rows, cols)
    assert np.allclose(c, C[rows, cols], rtol=1e-13, atol=1e-15)
    assert np.allclose(s, S[rows, cols], rtol=1e-13)


def test_fp8_activation_recipe_is_close_to_bf16_activations():
    # E4M3 keeps 4 significant bits: each activation is within 2^-4 of its
    # value relative to the row scale's range, and the scale is max|row|/448
    w = wl.make_workload(E=2, K=96, N=16, sizes=[9, 4], seed=40)
    Aq, a_scale = wl.fp8_activations(w)
    a = wl.bf16_bits_to_f32(w.A).astype(np.float64)
    back = oracle.decode_e4m3(Aq) * a_scale[:, None]
    rowmax = np.abs(a).max(axis=1, keepdims=True)
    assert np.allclose(a_scale, (np.abs(a).max(axis=1) / 448).astype(np.float32))
    assert (np.abs(back - a) <= 2.0 ** -4 * np.maximum(np.abs(a), rowmax * 2.0 ** -6) + 1e-30).all()
