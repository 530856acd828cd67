"""CPU oracle for the ragged-M grouped GEMM -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The HIP library never uses it, and it
never uses the HIP library: the two share nothing but the seeded input
generators in ``workloads``.

Contents
--------
* ``grouped_gemm`` / ``grouped_gemm_entries``: the fp64 product, from the C
  file ``oracle.c`` (plain triple loop, one expert at a time). Definition:
  "Grouped GEMM for Imbalanced Experts on Blackwell: A WIP Worklog", section
  "What I am measuring" and section 2; InferenceX glossary "Grouped GEMM",
  "Technical definition".
* ``tile_list``: the flat, expert-major tile descriptor list of the same
  worklog, section 2 (the descriptor holds expert, first row, valid rows and
  first column; tiles stop at expert boundaries; experts with no rows give no
  tiles). Written here as the plain nested loop over experts, M tiles, N tiles.
* ``eta``: tile efficiency of section 2.1 -- the share of scheduled rows that
  hold routed rows. The printed formula did not survive extraction; the
  reading taken is valid rows over scheduled rows, sum_e m_e / (BM * sum_e
  ceil(m_e/BM)), which reproduces the printed waste figures (10.2% at BM=64,
  22.0% at BM=128, skew 1.2, 16k rows) and the 50%/75% padding at 2,048
  uniform rows.
* ``eta_estimate``: the section-2.1 skew estimate, balanced throughput times
  eta (also lost in extraction; pinned by the printed 343.3 and 110.0).
* ``useful_flops`` / ``algorithmic_bytes``: the worklog's useful-work count
  (section 1: 2*M_tot*K*N) and the compulsory byte count of section 2.1
  (A once, B once per expert that has rows, C once).
* ``adaptive_bm`` / ``tile_widths``: the per-expert tile-height rule and
  tile-width rule of the HIP path, each written from its stated definition
  (see the functions).
* ``grouped_gemm_indexed``: the same product with A rows gathered from X by a
  row index list and C rows scattered by a second list -- the definition
  written out: A = X[src] (zero rows for indices out of range), the grouped
  product, then C[dst[r]] = C_grouped[r]. The permutation around the GEMM is
  the worklog's "What I am measuring" scope note; the indexed form is the
  plain reading of folding it into the loads and stores.
* ``e4m3_bf16_table`` / ``grouped_gemm_fp8w_whole``: every E4M3 value is
  exactly a bfloat16 value, so the fp8-weight product of any size is the
  binary64 triple loop above on the codes' bfloat16 patterns, each column
  then times its scale (pinned against ``grouped_gemm_fp8w``).
* ``decode_e4m3`` / ``grouped_gemm_fp8w`` / ``grouped_gemm_fp8w_entries``:
  the fp8-weight product C[r][n] = scale[e][n] * sum_k a[r][k] * dec(q[e][k][n])
  with the OCP E4M3 decode written from the format's definition, and the sum
  in binary64 (numpy float64 matmul per expert; the decoded weight times its
  fp32 scale is exact in binary64). The Pearl Pulse page "Pearl's grouped
  GEMM kernel for MoE models, explained" (section "What the 15% measures")
  mentions an FP8 scheme without details; per-output-column scales are the
  reading taken.
* ``grouped_gemm_fp8`` / ``grouped_gemm_fp8_entries``: fp8 activations and
  fp8 weights, C[r][n] = a_scale[r] * b_scale[e][n] * sum_k dec(Aq[r][k]) *
  dec(Bq[e][k][n]), the same E4M3 decode, one fp32 scale per activation row
  and per weight column (the reading taken of the article's unspecified FP8
  scheme), the sum in binary64 (every scaled operand is exact in binary64).
* ``round_to_bf16``: binary64 -> bfloat16 rounding to nearest, ties to even,
  written from the IEEE-754 definition of the format (8 significant bits,
  fp32's exponent range). It turns the fp64 reference into the bf16 values a
  bf16-output product may return (the worklog's traffic model, section 2.1,
  counts C in 2-byte values).

* ``grouped_gemm_combine``: the weighted combine after the grouped product:
  Y[dst[r]] += w[r] * C_grouped[r] for every routed row r whose destination
  is in range, starting from Y0 (zeros by default), in binary64. The
  permutation and combine are the steps either side of the measured GEMM in
  the worklog's "What I am measuring"; the InferenceX glossary's
  "Engineering details" name the weighted combine after the expert
  products. Also returns, per element, sum_r |w[r]| * S[r] (the product's
  error budget carried through the weights), |Y0| + sum_r |w[r] * C[r]| and
  the number of terms.
* ``silu`` / ``swiglu_pairs``: the SwiGLU activation between the gate and up
  projections the Pearl Pulse page benchmarks ("What the 15% measures"):
  silu(x) = x * sigmoid(x) = x / (1 + e^-x), and H[:, j] = silu(C[:, 2j]) *
  C[:, 2j+1] for a product whose columns interleave gate (even) and up (odd)
  -- the column layout of the fused entry point, written out directly.

Every function is pinned by ``tests/test_oracle.py`` (brute force, library
products, closed forms, the pages' printed figures); none is unpinned.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        i32 = ctypes.c_int
        lib.oracle_grouped_gemm.argtypes = [p, p, p, i32, i32, i32, i32, p, p, p]
        lib.oracle_grouped_gemm.restype = i32
        lib.oracle_grouped_gemm_entries.argtypes = [p, p, p, i32, i32, i32, i32, p, p,
                                                    ctypes.c_int64, p, p]
        lib.oracle_grouped_gemm_entries.restype = i32
        lib.oracle_threads.argtypes = []
        lib.oracle_threads.restype = i32
        lib.oracle_set_threads.argtypes = [i32]
        lib.oracle_set_threads.restype = None
        _lib = lib
    return _lib


def threads() -> int:
    """OpenMP threads the oracle runs on."""
    return int(_load().oracle_threads())


def set_threads(n: int) -> None:
    """Run later oracle calls on n OpenMP threads (n >= 1)."""
    _load().oracle_set_threads(int(n))


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def grouped_gemm(A, B, offsets, M_cap=None, C=None, S=None, want_s=True):
    """fp64 grouped product. A uint16 [M_cap,K], B uint16 [E,K,N], offsets int32 [E+1].

    Returns (C, S, madds). C and S are float64 [M_cap, N]; rows outside every
    group keep whatever C/S held on entry (NaN when allocated here).
    """
    A = np.ascontiguousarray(A, dtype=np.uint16)
    B = np.ascontiguousarray(B, dtype=np.uint16)
    off = np.ascontiguousarray(offsets, dtype=np.int32)
    E, K, N = B.shape
    if M_cap is None:
        M_cap = A.shape[0]
    assert A.shape == (M_cap, K) and off.shape == (E + 1,)
    if C is None:
        C = np.full((M_cap, N), np.nan)
    if want_s and S is None:
        S = np.full((M_cap, N), np.nan)
    madds = ctypes.c_int64(0)
    rc = _load().oracle_grouped_gemm(_ptr(A), _ptr(B), _ptr(off), E, K, N, M_cap, _ptr(C),
                                     _ptr(S) if want_s else None, ctypes.byref(madds))
    if rc != 0:
        raise ValueError("oracle: malformed problem (offsets or sizes)")
    return C, S, int(madds.value)


def grouped_gemm_entries(A, B, offsets, rows, cols):
    """C and S at selected (row, col) pairs, one fp64 dot product each."""
    A = np.ascontiguousarray(A, dtype=np.uint16)
    B = np.ascontiguousarray(B, dtype=np.uint16)
    off = np.ascontiguousarray(offsets, dtype=np.int32)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    E, K, N = B.shape
    n = rows.shape[0]
    c = np.empty(n)
    s = np.empty(n)
    rc = _load().oracle_grouped_gemm_entries(_ptr(A), _ptr(B), _ptr(off), E, K, N, A.shape[0],
                                             _ptr(rows), _ptr(cols), n, _ptr(c), _ptr(s))
    if rc != 0:
        raise ValueError("oracle: malformed problem (offsets or sizes)")
    return c, s


def grouped_gemm_indexed(X, src_rows, B, offsets, dst_rows=None, M_cap=None):
    """Gather, grouped product, scatter (all in the plain definition).

    X: bf16 bits [n_src, K]; src_rows: int [M_cap]; B: bf16 bits [E, K, N];
    offsets: [E+1]; dst_rows: int [M_cap] or None (identity). Returns (C, S)
    with C, S float64 [M_cap, N]; rows no grouped row writes are NaN.
    """
    X = np.asarray(X)
    src = np.asarray(src_rows, dtype=np.int64)
    off = np.asarray(offsets, dtype=np.int64)
    M_cap = len(src) if M_cap is None else int(M_cap)
    n_src, K = X.shape
    m_tot = int(off[-1])
    A = np.zeros((max(m_tot, 1), K), dtype=np.uint16)
    for r in range(m_tot):
        if 0 <= src[r] < n_src:
            A[r] = X[src[r]]
    Cg, Sg, _ = grouped_gemm(A, B, off, M_cap=max(m_tot, 1))
    C = np.full((M_cap, B.shape[2]), np.nan)
    S = np.full((M_cap, B.shape[2]), np.nan)
    dst = np.arange(M_cap) if dst_rows is None else np.asarray(dst_rows, dtype=np.int64)
    for r in range(m_tot):
        d = int(dst[r])
        if 0 <= d < M_cap:
            C[d] = Cg[r]
            S[d] = Sg[r]
    return C, S


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def tile_list(offsets, N: int, bm, bn):
    """Expert-major flat tile list: [(expert, row0, rows, col0), ...].

    bm, bn: one tile height / width for all experts, or a sequence with one
    entry per expert. Order: expert, then M tile, then N tile innermost.
    """
    off = [int(x) for x in offsets]
    E = len(off) - 1
    bms = [int(bm)] * E if np.isscalar(bm) else [int(x) for x in bm]
    bns = [int(bn)] * E if np.isscalar(bn) else [int(x) for x in bn]
    tiles = []
    for e in range(E):
        m_e = off[e + 1] - off[e]
        BM, BN = bms[e], bns[e]
        for mt in range(_cdiv(m_e, BM)):
            for nt in range(_cdiv(N, BN)):
                tiles.append((e, off[e] + mt * BM, min(BM, m_e - mt * BM), nt * BN))
    return tiles


def eta(sizes, bm) -> float:
    """Valid rows over scheduled rows for tile height bm (scalar or per expert)."""
    sizes = [int(x) for x in sizes]
    bms = [int(bm)] * len(sizes) if np.isscalar(bm) else [int(x) for x in bm]
    sched = sum(b * _cdiv(m, b) for m, b in zip(sizes, bms))
    valid = sum(sizes)
    return valid / sched if sched else 1.0


def eta_estimate(balanced_rate: float, eta_value: float) -> float:
    """Skewed-run throughput estimated from a balanced run: rate * eta."""
    return balanced_rate * eta_value


def useful_flops(m_tot: int, K: int, N: int) -> int:
    return 2 * int(m_tot) * int(K) * int(N)


def algorithmic_bytes(sizes, K: int, N: int, c_bytes: int = 4, in_bytes: int = 2) -> int:
    """Compulsory bytes: A once, B once per expert with rows, C once."""
    sizes = [int(x) for x in sizes]
    m_tot = sum(sizes)
    active = sum(1 for m in sizes if m > 0)
    return in_bytes * m_tot * K + in_bytes * K * N * active + c_bytes * m_tot * N


# Tile heights the HIP path supports, smallest first.
BM_CHOICES = (16, 32, 64, 128, 256)

# Tile widths (output columns per tile) of the HIP path.
TILE_WIDTH = 256
TILE_WIDTH_WIDE = 512


def tile_widths(heights, sizes):
    """Per-expert tile width, as the HIP path defines it.

    Tiles are TILE_WIDTH columns wide. In a launch where every expert that
    has rows takes 16-row tiles (the weight-streaming case of many small
    groups), those 16-row tiles are TILE_WIDTH_WIDE columns wide instead.
    Experts without rows have no tiles and do not take part in the decision.
    heights and sizes hold one entry per expert (the tile height chosen for
    it and its row count m_e).
    """
    heights = [int(h) for h in heights]
    sizes = [int(m) for m in sizes]
    if len(heights) != len(sizes):
        raise ValueError("one height and one size per expert")
    every_16 = True
    for h, m in zip(heights, sizes):
        if m > 0 and h != 16:
            every_16 = False
    widths = []
    for h in heights:
        widths.append(TILE_WIDTH_WIDE if (every_16 and h == 16) else TILE_WIDTH)
    return widths


def adaptive_bm(sizes, choices=BM_CHOICES):
    """Per-expert tile height, as the HIP path defines it.

    For each expert the rule takes the height that minimises the cost
        ceil(m_e / BM) * (BM + H)
    where H = 64 rows stands for the fixed per-tile work that does not grow
    with the tile height (streaming the expert's weight slice through the
    tile, the barriers and the epilogue set-up). Ties go to the larger
    height. An expert with no rows gets the smallest height (and no tiles).
    The worklog (sections 2.1, 6 and 7) motivates the trade -- padding falls
    with BM while per-tile staging work rises -- and proposes choosing BM
    from the expert sizes; the constant H is this implementation's own.
    """
    H = 64
    out = []
    for m in (int(x) for x in sizes):
        if m <= 0:
            out.append(choices[0])
            continue
        best, best_cost = None, None
        for b in choices:
            cost = _cdiv(m, b) * (b + H)
            if best_cost is None or cost <= best_cost:
                best, best_cost = b, cost
        out.append(best)
    return out


def round_to_bf16(x):
    """Round binary64 values to bfloat16 (nearest, ties to even); float64 out.

    bfloat16 keeps fp32's 8 exponent bits and 8 significant bits. A finite
    x with 2^(e-1) <= |x| < 2^e (numpy.frexp) has a unit in the last place of
    2^(e-8) while it is normal (|x| >= 2^-126); below that the spacing stays
    2^-133 (subnormals). Scaling by a power of two is exact in binary64, so
    x / ulp is exact and numpy's round (half to even) applies the tie rule.
    A result at or above 2^128 overflows to infinity.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = (x != 0) & np.isfinite(x)
    _, e = np.frexp(x[nz])
    ulp = np.ldexp(1.0, np.maximum(e - 8, -133))
    r = np.round(x[nz] / ulp) * ulp
    r[np.abs(r) >= 2.0 ** 128] = np.inf * np.sign(r[np.abs(r) >= 2.0 ** 128])
    out[nz] = r
    out[~np.isfinite(x)] = x[~np.isfinite(x)]
    return out


def decode_e4m3(codes):
    """OCP fp8 E4M3 codes (uint8) -> float64 values.

    Bit 7 is the sign, bits 6..3 the exponent field (bias 7), bits 2..0 the
    mantissa. Field 0: subnormal m/8 * 2^-6. Field 15 with mantissa 7: NaN
    (E4M3 has no infinities). Otherwise (1 + m/8) * 2^(field - 7).
    """
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    f = (c >> 3) & 15
    m = c & 7
    mag = np.where(f == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.ldexp(1.0, f - 7))
    out = sign * mag
    out[(f == 15) & (m == 7)] = np.nan
    return out


def e4m3_bf16_table():
    """bfloat16 bit pattern of every OCP E4M3 code's value, indexed by code.

    An E4M3 value has at most 4 significant bits and an exponent between
    2^-9 and 2^8, so it is exactly a bfloat16 value (8 significant bits,
    fp32's exponent range): its binary32 form has zero low 16 bits, and the
    high 16 bits are its bfloat16 pattern. The two NaN codes map to the
    bfloat16 quiet NaN 0x7FC0 (sign kept).
    """
    v = decode_e4m3(np.arange(256)).astype(np.float32)
    u = v.view(np.uint32)
    finite = np.isfinite(v)
    assert (u[finite] & 0xFFFF == 0).all(), "an E4M3 value that is not a bfloat16 value"
    bits = (u >> 16).astype(np.uint16)
    bits[~finite] = np.where(np.arange(256)[~finite] >> 7, 0xFFC0, 0x7FC0).astype(np.uint16)
    return bits


def grouped_gemm_fp8w_whole(A, Bq, scale, offsets, M_cap=None):
    """The fp8-weight product at any size, through the binary64 triple loop.

    C[r][n] = scale[e][n] * sum_k a[r][k] * dec(q[e][k][n]): dec(q) is taken
    as the exact bfloat16 value of each code (e4m3_bf16_table), the sum is the
    C oracle's grouped_gemm, and each column is then multiplied by its scale
    in binary64. Returns (C, S) like grouped_gemm_fp8w (S scaled by |scale|).
    Codes must not be NaN.
    """
    Bq = np.asarray(Bq, dtype=np.uint8)
    nan_codes = (Bq & 0x7F) == 0x7F
    if nan_codes.any():
        raise ValueError("NaN weight codes")
    table = e4m3_bf16_table()
    off = np.asarray(offsets, dtype=np.int32)
    E, K, N = Bq.shape
    Bbits = np.empty((E, K, N), dtype=np.uint16)
    for e in range(E):
        np.take(table, Bq[e], out=Bbits[e])
    C, S, _ = grouped_gemm(A, Bbits, off, M_cap=M_cap)
    sc = np.asarray(scale, dtype=np.float64)
    for e in range(E):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 > r0:
            C[r0:r1] *= sc[e][None, :]
            S[r0:r1] *= np.abs(sc[e])[None, :]
    return C, S


def _fp8_expert_weights(Bq, scale, e):
    return decode_e4m3(Bq[e]) * np.asarray(scale[e], dtype=np.float64)[None, :]


def grouped_gemm_fp8w(A, Bq, scale, offsets, M_cap=None):
    """fp64 fp8-weight grouped product. Returns (C, S), float64 [M_cap, N];
    S[r][n] = sum_k |a[r][k] * dec(q[e][k][n]) * scale[e][n]|; rows outside
    every group are NaN."""
    A = np.asarray(A)
    off = np.asarray(offsets, dtype=np.int64)
    E, K, N = Bq.shape
    M_cap = A.shape[0] if M_cap is None else int(M_cap)
    C = np.full((M_cap, N), np.nan)
    S = np.full((M_cap, N), np.nan)
    for e in range(E):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 <= r0:
            continue
        a = _bf16_to_f64(A[r0:r1])
        w = _fp8_expert_weights(Bq, scale, e)
        C[r0:r1] = a @ w
        S[r0:r1] = np.abs(a) @ np.abs(w)
    return C, S


def grouped_gemm_fp8w_entries(A, Bq, scale, offsets, rows, cols):
    """Selected entries of the fp8-weight product, one dot product each."""
    off = np.asarray(offsets, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    c = np.empty(len(rows))
    s = np.empty(len(rows))
    for i, (r, n) in enumerate(zip(rows, cols)):
        e = int(np.searchsorted(off, r, side="right") - 1)
        a = _bf16_to_f64(A[r])
        w = decode_e4m3(Bq[e, :, n]) * float(scale[e, n])
        c[i] = a @ w
        s[i] = np.abs(a) @ np.abs(w)
    return c, s


def grouped_gemm_fp8(Aq, a_scale, Bq, b_scale, offsets, M_cap=None):
    """fp64 product of fp8 activations and fp8 weights. Returns (C, S), float64
    [M_cap, N]; S[r][n] = sum_k |a_scale[r] dec(Aq[r][k]) * dec(Bq[e][k][n])
    b_scale[e][n]|; rows outside every group are NaN."""
    Aq = np.asarray(Aq)
    a_scale = np.asarray(a_scale, dtype=np.float64)
    off = np.asarray(offsets, dtype=np.int64)
    E, K, N = Bq.shape
    M_cap = Aq.shape[0] if M_cap is None else int(M_cap)
    C = np.full((M_cap, N), np.nan)
    S = np.full((M_cap, N), np.nan)
    for e in range(E):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 <= r0:
            continue
        a = decode_e4m3(Aq[r0:r1]) * a_scale[r0:r1, None]
        w = _fp8_expert_weights(Bq, b_scale, e)
        C[r0:r1] = a @ w
        S[r0:r1] = np.abs(a) @ np.abs(w)
    return C, S


def grouped_gemm_fp8_entries(Aq, a_scale, Bq, b_scale, offsets, rows, cols):
    """Selected entries of the fp8 x fp8 product, one dot product each."""
    off = np.asarray(offsets, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    c = np.empty(len(rows))
    s = np.empty(len(rows))
    for i, (r, n) in enumerate(zip(rows, cols)):
        e = int(np.searchsorted(off, r, side="right") - 1)
        a = decode_e4m3(Aq[r]) * float(a_scale[r])
        w = decode_e4m3(Bq[e, :, n]) * float(b_scale[e, n])
        c[i] = a @ w
        s[i] = np.abs(a) @ np.abs(w)
    return c, s


def _bf16_to_f64(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def silu(x):
    """silu(x) = x * sigmoid(x) = x / (1 + e^-x), in binary64.

    For x below about -709, e^-x overflows to infinity and the quotient is
    -0, while the exact value has magnitude below 1e-305.
    """
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def swiglu_pairs(C):
    """H[:, j] = silu(C[:, 2j]) * C[:, 2j+1]: gate in the even columns, up in
    the odd ones; binary64 in and out."""
    C = np.asarray(C, dtype=np.float64)
    if C.shape[-1] % 2:
        raise ValueError("an even number of columns is needed (gate, up pairs)")
    return silu(C[..., 0::2]) * C[..., 1::2]


def grouped_gemm_combine(X, src_rows, B, offsets, dst_rows, weights, n_dst, Y0=None):
    """Gather, grouped product, weighted scatter-add (binary64).

    X: bf16 bits [n_src, K]; src_rows, dst_rows: int [M_cap]; weights: float
    [M_cap]; B: bf16 bits [E, K, N]; offsets: [E+1]; Y0: optional [n_dst, N]
    starting values. Returns (Y, SW, AY, terms): Y[d] = Y0[d] + sum of
    weights[r] * C[r] over routed rows r < off[E] with dst_rows[r] = d;
    SW[d] = sum |weights[r]| * S[r]; AY[d] = |Y0[d]| + sum |weights[r] * C[r]|;
    terms[d] = the number of additions into row d (Y0 counts as one).
    """
    off = np.asarray(offsets, dtype=np.int64)
    m_tot = int(off[-1])
    src = np.asarray(src_rows, dtype=np.int64)
    dst = np.asarray(dst_rows, dtype=np.int64)
    w = np.asarray(weights, dtype=np.float64)
    N = B.shape[2]
    Cg, Sg = grouped_gemm_indexed(X, src, B, off, dst_rows=None, M_cap=max(m_tot, 1))
    Y = np.zeros((n_dst, N)) if Y0 is None else np.array(Y0, dtype=np.float64)
    AY = np.abs(Y)
    SW = np.zeros((n_dst, N))
    terms = np.zeros(n_dst, dtype=np.int64) if Y0 is None else np.ones(n_dst, dtype=np.int64)
    for r in range(m_tot):
        d = int(dst[r])
        if 0 <= d < n_dst:
            Y[d] += w[r] * Cg[r]
            SW[d] += abs(w[r]) * Sg[r]
            AY[d] += np.abs(w[r] * Cg[r])
            terms[d] += 1
    return Y, SW, AY, terms
