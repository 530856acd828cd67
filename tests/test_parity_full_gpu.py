"""Full-size workloads: the HIP path against the CPU oracle on whole outputs.

Every entry point runs on every full-size workload (decode, uniform16k,
skew16k, skew16k_page, skew2k_wide) in the launch configuration the
benchmark times (bm=0, the device's per-expert tile height). The oracle
computes the whole fp32 product once per workload; the fp32, bf16, SwiGLU,
gather/scatter, weighted-combine and fp8-weight outputs are then compared
element by element with it, each output followed by guard rows that must
stay untouched. The fp8 x fp8 product gets an oracle of its own, also once
per workload: its fp32 output is compared on sampled entries at its tight
bound (which needs each group's largest product, computed one entry at a
time) and whole at a looser one, and its bf16 and SwiGLU outputs whole.

The workload fixture is module-scoped and parametrized, so pytest runs all
tests of one workload before drawing the next.
"""

import dataclasses
import sys

import numpy as np
import pytest

import oracle
import workloads as wl
from tests import parity

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

FULL = ["decode", "uniform16k", "skew16k", "skew16k_page", "skew2k_wide"]
GUARD = 16  # rows after every output that must stay untouched


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def gg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_ragged_grouped_amd as m
    m.load_library()
    return m


@dataclasses.dataclass
class Full:
    name: str
    w: object
    ref: np.ndarray   # oracle C, float64 [M_tot, N]
    s: np.ndarray     # oracle sum_k |a b|, float64 [M_tot, N]
    A: object         # device tensors
    B: object
    off: object


@pytest.fixture(scope="module", params=FULL)
def full(request, gg):
    name = request.param
    _say("drawing workload %s" % name)
    w = wl.make_workload(name)
    m = w.M_tot
    _say("oracle: whole %s product E=%d K=%d N=%d M_tot=%d" % (name, w.E, w.K, w.N, m))
    ref, s, madds = oracle.grouped_gemm(w.A, w.B, w.offsets)
    assert madds == m * w.K * w.N
    dev = torch.device("cuda:0")
    A = torch.from_numpy(w.A.view(np.int16)).to(dev).view(torch.bfloat16)
    B = torch.from_numpy(w.B.view(np.int16)).to(dev).view(torch.bfloat16)
    off = torch.from_numpy(w.offsets).to(dev)
    f = Full(name, w, ref[:m], s[:m], A, B, off)
    yield f
    del f, A, B, off
    torch.cuda.empty_cache()


def _guarded(rows, cols, dtype, fill=float("nan")):
    big = torch.full((rows + GUARD, cols), fill, dtype=dtype, device="cuda:0")
    return big, big[:rows]


def _host(t):
    return t.float().cpu().numpy().astype(np.float64)


def test_fp32_whole(gg, full):
    w = full.w
    _say("case full fp32 %s" % full.name)
    big, C = _guarded(w.M_cap, w.N, torch.float32)
    gg.grouped_gemm(full.A, full.B, full.off, out=C, bm=0)
    torch.cuda.synchronize()
    out = _host(big)
    rel, worst = parity.check(out[: w.M_tot], full.ref, full.s, full.name)
    _say("  %s: rel_fro %.2e, worst |diff| / (1e-4 S) %.3f" % (full.name, rel, worst / parity.ELEM))
    assert np.isnan(out[w.M_tot:]).all(), "rows past the last group were written"


def test_bf16_out_whole(gg, full):
    w = full.w
    _say("case full bf16-out %s" % full.name)
    big, C = _guarded(w.M_cap, w.N, torch.bfloat16)
    gg.grouped_gemm(full.A, full.B, full.off, out=C, bm=0)
    torch.cuda.synchronize()
    out = _host(big)
    parity.check_bf16(out[: w.M_tot], full.ref, full.s, full.name + " bf16")
    assert np.isnan(out[w.M_tot:]).all()


def test_swiglu_whole(gg, full):
    w = full.w
    _say("case full swiglu %s" % full.name)
    big, H = _guarded(w.M_cap, w.N // 2, torch.bfloat16)
    gg.grouped_gemm_swiglu(full.A, full.B, full.off, out=H, bm=0)
    torch.cuda.synchronize()
    out = _host(big)
    # the bracket is built in row blocks to bound the host memory it needs
    step = 2048
    for r0 in range(0, w.M_tot, step):
        r1 = min(w.M_tot, r0 + step)
        parity.check_swiglu_bf16(out[r0:r1], full.ref[r0:r1], full.s[r0:r1],
                                 "%s swiglu rows %d..%d" % (full.name, r0, r1))
    assert np.isnan(out[w.M_tot:]).all()


def _permutation(w):
    # the benchmark's top-1 routing: grouped row r is token row perm[r]
    return np.random.default_rng(w.seed + 500).permutation(w.M_cap).astype(np.int32)


def test_gather_scatter_whole(gg, full):
    w = full.w
    perm = _permutation(w)
    dev = torch.device("cuda:0")
    pd = torch.from_numpy(perm).to(dev)
    X = torch.empty_like(full.A)
    X[pd.long()] = full.A
    _say("case full gather/scatter %s" % full.name)
    big, C = _guarded(w.M_cap, w.N, torch.float32)
    gg.grouped_gemm_gather(X, pd, full.B, full.off, dst_rows=pd, out=C, bm=0)
    torch.cuda.synchronize()
    out = _host(big)
    m = w.M_tot
    # C[perm[r]] is grouped row r's product; the M_cap = M_tot rows are a
    # permutation, so every output row is written exactly once
    parity.check(out[perm[:m]], full.ref, full.s, full.name + " gather")
    assert np.isnan(out[w.M_cap:]).all()


def test_combine_top2_whole(gg, full):
    # top-2 routing: grouped row r reads token row perm[r] of X and adds
    # gate[r] * C[r] into output token perm[r] // 2, so each of the M_tot/2
    # output rows receives exactly two products, on top of start values
    w = full.w
    m = w.M_tot
    perm = _permutation(w)
    gate = np.random.default_rng(w.seed + 501).uniform(0.05, 1.0, w.M_cap).astype(np.float32)
    dst = (perm // 2).astype(np.int32)
    n_dst = (w.M_cap + 1) // 2
    dev = torch.device("cuda:0")
    pd = torch.from_numpy(perm).to(dev)
    X = torch.empty_like(full.A)
    X[pd.long()] = full.A
    big, Y = _guarded(n_dst, w.N, torch.float32, fill=0.5)
    _say("case full combine top-2 %s" % full.name)
    gg.grouped_gemm_gather_combine(X, pd, full.B, full.off, torch.from_numpy(dst).to(dev),
                                   torch.from_numpy(gate).to(dev), out=Y, bm=0)
    torch.cuda.synchronize()
    out = _host(big)
    # binary64 reference: Y0 = 0.5, then gate * C of each routed row
    g = gate[:m].astype(np.float64)[:, None]
    Yref = np.full((n_dst, w.N), 0.5)
    SW = np.zeros((n_dst, w.N))
    AY = np.full((n_dst, w.N), 0.5)
    np.add.at(Yref, dst[:m], g * full.ref)
    np.add.at(SW, dst[:m], g * full.s)
    np.add.at(AY, dst[:m], np.abs(g * full.ref))
    terms = 1 + np.bincount(dst[:m], minlength=n_dst)
    assert terms.max() <= 3
    parity.check_combine(out[:n_dst], Yref, SW, AY, terms, full.name + " combine")
    assert (out[n_dst:] == 0.5).all(), "guard rows after the output were written"


def test_fp8w_whole(gg, full):
    w = full.w
    _say("case full fp8w %s: quantizing weights" % full.name)
    Bq, scale = wl.fp8_weights(w)
    _say("oracle: whole fp8-weight %s product" % full.name)
    ref, s = oracle.grouped_gemm_fp8w_whole(w.A, Bq, scale, w.offsets)
    dev = torch.device("cuda:0")
    Bd = torch.from_numpy(Bq).to(dev)
    sd = torch.from_numpy(scale).to(dev)
    del Bq
    big, C = _guarded(w.M_cap, w.N, torch.float32)
    gg.grouped_gemm_fp8w(full.A, Bd, sd, full.off, out=C, bm=0)
    torch.cuda.synchronize()
    out = _host(big)
    m = w.M_tot
    rel, worst = parity.check(out[:m], ref[:m], s[:m], full.name + " fp8w")
    _say("  %s fp8w: rel_fro %.2e, worst |diff| / (1e-4 S) %.3f" % (full.name, rel,
                                                                    worst / parity.ELEM))
    assert np.isnan(out[w.M_cap:]).all()


def _samples(w, rng, n_random=3000):
    # boundary rows of every expert at both ends and the middle of the column
    # range and around the first column-tile edges, plus uniform random entries
    rows, cols = [], []
    off = w.offsets
    for e in range(w.E):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 > r0:
            for r in {r0, r1 - 1, (r0 + r1) // 2}:
                for c in (0, 1, 255, 256, 511, 512, w.N - 1, int(rng.integers(0, w.N))):
                    if c < w.N:
                        rows.append(r)
                        cols.append(c)
    rows += list(rng.integers(0, w.M_tot, size=n_random))
    cols += list(rng.integers(0, w.N, size=n_random))
    return np.array(rows, dtype=np.int64), np.array(cols, dtype=np.int64)


@dataclasses.dataclass
class Q8:
    Aq: np.ndarray      # host codes and scales
    a_scale: np.ndarray
    Bq: np.ndarray
    b_scale: np.ndarray
    dev: list           # the same four on the device
    ref: np.ndarray     # oracle C, float64 [M_tot, N]
    S: np.ndarray       # oracle sum |products|, float64 [M_tot, N]
    loose: np.ndarray   # the fp8 bound with each group's largest product replaced by its sum


@pytest.fixture(scope="module")
def q8(full):
    # the fp8 x fp8 inputs of a workload and the oracle's whole product, once
    w = full.w
    _say("fp8 x fp8 %s: quantizing" % full.name)
    Aq, a_scale = wl.fp8_activations(w)
    Bq, b_scale = wl.fp8_weights(w)
    _say("oracle: whole fp8 x fp8 %s product" % full.name)
    ref, S = oracle.grouped_gemm_fp8(Aq, a_scale, Bq, b_scale, w.offsets, M_cap=w.M_cap)
    m = w.M_tot
    dev = torch.device("cuda:0")
    d = [torch.from_numpy(x).to(dev) for x in (Aq, a_scale, Bq, b_scale)]
    # G <= S for every group, so this bound is never below the tight one
    q = Q8(Aq, a_scale, Bq, b_scale, d, ref[:m], S[:m], parity.fp8_bound(S[:m], S[:m], w.K))
    yield q
    del q, d
    torch.cuda.empty_cache()


def _fp8_run(gg, full, q8, out, swiglu=False):
    f = gg.grouped_gemm_fp8_swiglu if swiglu else gg.grouped_gemm_fp8
    f(*q8.dev, full.off, out=out, bm=0)
    torch.cuda.synchronize()


def test_fp8_sampled(gg, full, q8):
    w = full.w
    Aq, a_scale, Bq, b_scale = q8.Aq, q8.a_scale, q8.Bq, q8.b_scale
    _say("case full fp8 x fp8 %s" % full.name)
    big, C = _guarded(w.M_cap, w.N, torch.float32)
    _fp8_run(gg, full, q8, C)
    out = _host(big)
    assert np.isfinite(out[: w.M_tot]).all()
    assert np.isnan(out[w.M_cap:]).all()
    rows, cols = _samples(w, np.random.default_rng(11))
    c, s = oracle.grouped_gemm_fp8_entries(Aq, a_scale, Bq, b_scale, w.offsets, rows, cols)
    G = np.empty(len(rows))
    for i, (r, n) in enumerate(zip(rows, cols)):
        e = int(np.searchsorted(w.offsets, r, side="right") - 1)
        a = oracle.decode_e4m3(Aq[r:r + 1]) * float(a_scale[r])
        wt = oracle.decode_e4m3(Bq[e][:, n:n + 1]) * float(b_scale[e, n])
        G[i] = parity.fp8_group_max_sum(a, wt)[0, 0]
    worst = parity.check_fp8(out[rows, cols], c, s, G, w.K, full.name + " fp8 sampled")
    _say("  %s fp8 sampled: worst error / bound %.3e" % (full.name, worst))
    assert worst <= parity.FP8_TRIPWIRE, "%s: worst error / bound %.3e" % (full.name, worst)


def test_fp8_whole(gg, full, q8):
    # Every output of the fp8 x fp8 product against the oracle. The bound is
    # check_fp8's with each group's largest product replaced by the group's
    # sum (G <= S): looser than the sampled check above, but over the whole
    # output, so a wrong tile, row, column or scale anywhere fails it.
    w = full.w
    _say("case full fp8 x fp8 whole %s" % full.name)
    big, C = _guarded(w.M_cap, w.N, torch.float32)
    _fp8_run(gg, full, q8, C)
    out = _host(big)
    assert np.isnan(out[w.M_cap:]).all()
    m = w.M_tot
    assert np.isfinite(out[:m]).all()
    ratio = np.abs(out[:m] - q8.ref) / np.maximum(q8.loose, 1e-300)
    worst = float(ratio.max()) if ratio.size else 0.0
    _say("  %s fp8 whole: worst error / loose bound %.3e" % (full.name, worst))
    assert worst <= 1.0, "%s: %d outputs beyond the fp8 bound" % (full.name, int((ratio > 1).sum()))
    # the loose bound is never below the tight one, so the tight check's
    # tripwire holds here too wherever the tight one holds
    assert worst <= parity.FP8_TRIPWIRE, "%s: worst error / loose bound %.3e" % (full.name, worst)


def test_fp8_bf16_out_whole(gg, full, q8):
    # bf16 C of the fp8 x fp8 product: bit for bit the fp32 entry point's
    # output rounded by torch, and inside the bf16 roundings of the oracle's
    # value -/+ the loose fp8 bound, everywhere
    w = full.w
    m = w.M_tot
    _say("case full fp8 x fp8 bf16-out %s" % full.name)
    big, C = _guarded(w.M_cap, w.N, torch.bfloat16)
    _fp8_run(gg, full, q8, C)
    c32 = torch.empty((w.M_cap, w.N), dtype=torch.float32, device="cuda:0")
    _fp8_run(gg, full, q8, c32)
    assert torch.equal(c32[:m].to(torch.bfloat16).view(torch.int16), C[:m].view(torch.int16))
    out = _host(big)
    assert np.isnan(out[m:]).all()
    step = 2048  # brackets built in row blocks to bound the host memory they need
    for r0 in range(0, m, step):
        r1 = min(m, r0 + step)
        parity.check_fp8_bf16(out[r0:r1], q8.ref[r0:r1], q8.S[r0:r1], q8.S[r0:r1], w.K,
                              "%s fp8 bf16-out rows %d..%d" % (full.name, r0, r1))


def test_fp8_swiglu_whole(gg, full, q8):
    # SwiGLU of the fp8 x fp8 gate/up product: bracketed by silu's range over
    # the loose fp8 bound around the oracle's product, and equal to the SwiGLU
    # of the fp32 entry point's output within the fp32 evaluation error
    w = full.w
    m = w.M_tot
    _say("case full fp8 x fp8 swiglu %s" % full.name)
    big, H = _guarded(w.M_cap, w.N // 2, torch.bfloat16)
    _fp8_run(gg, full, q8, H, swiglu=True)
    c32 = torch.empty((w.M_cap, w.N), dtype=torch.float32, device="cuda:0")
    _fp8_run(gg, full, q8, c32)
    out = _host(big)
    c64 = _host(c32[:m])
    assert np.isnan(out[m:]).all()
    step = 2048
    for r0 in range(0, m, step):
        r1 = min(m, r0 + step)
        what = "%s fp8 swiglu rows %d..%d" % (full.name, r0, r1)
        parity.check_swiglu_bf16(out[r0:r1], q8.ref[r0:r1], q8.S[r0:r1], what,
                                 err=q8.loose[r0:r1])
        h64 = oracle.swiglu_pairs(c64[r0:r1])
        slack = parity.swiglu_eval_slack(c64[r0:r1], h64)
        assert (out[r0:r1] >= oracle.round_to_bf16(h64 - slack)).all(), what
        assert (out[r0:r1] <= oracle.round_to_bf16(h64 + slack)).all(), what


@pytest.mark.parametrize("full", ["decode"], indirect=True)
def test_gather_routed_top8_decode(gg, full):
    # the decode shape reached through routing: 64 tokens, top-8 over 32
    # experts (16 rows each), K=6144, N=4096, output row token*8 + slot
    w = full.w
    E, K, N, topk, n_tokens = 32, 6144, 4096, 8, 64
    pairs = sorted(((t * topk + j) % E, t, j) for t in range(n_tokens) for j in range(topk))
    sizes = np.bincount([p[0] for p in pairs], minlength=E)
    assert (sizes == w.sizes).all()
    src = np.array([p[1] for p in pairs], dtype=np.int32)
    dst = np.array([p[1] * topk + p[2] for p in pairs], dtype=np.int32)
    X = wl.make_workload(E=1, K=K, N=8, sizes=[n_tokens], seed=46).A
    dev = torch.device("cuda:0")
    big, C = _guarded(512, N, torch.float32)
    _say("case gather routed top-8 decode")
    gg.grouped_gemm_gather(torch.from_numpy(X.view(np.int16)).to(dev).view(torch.bfloat16),
                           torch.from_numpy(src).to(dev), full.B, full.off,
                           dst_rows=torch.from_numpy(dst).to(dev), out=C, bm=0)
    torch.cuda.synchronize()
    out = _host(big)
    ref, s, _ = oracle.grouped_gemm(np.ascontiguousarray(X[src]), w.B, w.offsets)
    parity.check(out[dst], ref, s, "gather routed top-8 decode")
    assert np.isnan(out[512:]).all()
