"""The tracing build (include/grouped_gemm_trace.h) on the GPU: it computes the
product's result bit for bit, and its records describe the launch the
library makes (every tile once, on the workgroup the stride order gives it,
with the descriptor of the device-built tile list)."""

import numpy as np
import pytest

import workloads as wl
from tests.test_parity_gpu import _dev, _say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

XCDS = 8


@pytest.fixture(scope="module")
def gg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_ragged_grouped_amd as m
    m.load_library()
    m.load_trace_library()
    return m


@pytest.mark.parametrize("bm", [0, 16, 256])
def test_trace_matches_product_and_schedule(gg, bm):
    w = wl.make_workload(E=9, K=520, N=1800, sizes=[0, 700, 3, 129, 0, 64, 1000, 17, 250],
                         seed=61, M_cap=2200)
    A, B, off = _dev(w)
    _say("case trace bm=%d" % bm)
    ref = gg.grouped_gemm(A, B, off, bm=bm)
    tiles, n = gg.tile_schedule(off, w.N, w.M_cap, bm=bm)
    C, tr, khz = gg.traced_grouped_gemm(A, B, off, n, bm=bm)
    torch.cuda.synchronize()
    m = w.M_tot
    assert torch.equal(C[:m], ref[:m])
    assert khz > 0
    tr = tr.cpu().numpy()
    tl = tiles.cpu().numpy()
    W = gg.TRACE_WORKGROUPS
    wg = tr[:W]
    G = int((wg[:, 0] > 0).sum())
    assert G % XCDS == 0 and (wg[:G, 0] > 0).all() and (wg[G:] == 0).all()
    assert int(wg[:G, 3].sum()) == n
    assert (wg[:G, 1] >= wg[:G, 0]).all()
    assert ((wg[:G, 2] >> 6) < XCDS).all()
    assert (wg[:G, 4:] == 0).all()
    rec = tr[W:W + n]
    assert (rec[:, 0] > 0).all() and (rec[:, 1] >= rec[:, 0]).all() and (rec[:, 2] >= rec[:, 1]).all()
    # the descriptor of tile t is the device tile list's entry t
    # (expert, row0, rows, col0, bm)
    assert np.array_equal(rec[:, 3], tl[:, 4])
    assert np.array_equal(rec[:, 5], tl[:, 0])
    assert np.array_equal(rec[:, 6], tl[:, 2])
    assert np.array_equal(rec[:, 7], tl[:, 3])
    # workgroup b runs tiles slot(b), slot(b) + G, ... in that order
    owner = rec[:, 4]
    slot = (owner % XCDS) * (G // XCDS) + owner // XCDS
    assert np.array_equal(slot, np.arange(n) % G)
    for b in set(owner.tolist()):
        mine = rec[owner == b]
        assert (mine[1:, 0] >= mine[:-1, 2]).all(), "tiles of one workgroup overlap"
    assert tr.shape[1] == gg.TRACE_RECORD and (tr[W + n:] == 0).all()


def test_tracing_build_runs_the_plain_entry_point(gg):
    # the tracing library also exports the product's entry points; called
    # without a trace buffer they record nothing and compute the same result
    import ctypes
    w = wl.make_workload(E=4, K=256, N=512, sizes=[100, 0, 37, 260], seed=62, M_cap=400)
    A, B, off = _dev(w)
    ref = gg.grouped_gemm(A, B, off, bm=0)
    lib = gg.load_trace_library()
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    fn = lib.gg_grouped_gemm_bf16
    fn.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
    fn.restype = ctypes.c_int
    C = torch.full_like(ref, float("nan"))
    _say("case tracing build, plain entry point")
    st = fn(A.data_ptr(), B.data_ptr(), off.data_ptr(), C.data_ptr(), w.E, w.K, w.N, w.M_cap, 0,
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == 0
    m = w.M_tot
    assert torch.equal(C[:m], ref[:m]) and torch.isnan(C[m:]).all()
