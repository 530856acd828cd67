"""The C-ABI library (no GPU): it loads, exports every declared symbol, and its
host-side argument checks return the documented status without enqueuing work.

None of the calls below reaches the HIP runtime: each is rejected by the host
checks before any device call.
"""

import ctypes
import os
import re

import pytest

import moe_ragged_grouped_amd as gg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER_DIR = os.path.join(ROOT, "include")


TRACE_HEADER = "grouped_gemm_trace.h"  # the tracing build's own entry points


def _declared_symbols(trace=False):
    names = set()
    for fn in os.listdir(HEADER_DIR):
        if fn.endswith(".h") and (fn == TRACE_HEADER) == trace:
            text = open(os.path.join(HEADER_DIR, fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names.update(re.findall(r"\b(gg_[a-z0-9_]+)\s*\(", text))
    return names


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gg.library_path()):
        import moe_ragged_grouped_amd.build as b
        b.build()
    return gg.load_library()


@pytest.fixture(scope="module")
def trace_lib():
    if not os.path.exists(gg.trace_library_path()):
        import moe_ragged_grouped_amd.build as b
        b.build_trace()
    return gg.load_trace_library()


def test_exports_every_declared_symbol(lib):
    declared = _declared_symbols()
    assert declared == set(gg.SYMBOLS), declared
    for name in declared:
        assert hasattr(lib, name), name


def test_tracing_build_exports_its_symbols(lib, trace_lib):
    declared = _declared_symbols(trace=True)
    assert declared == set(gg.TRACE_SYMBOLS), declared
    for name in declared:
        assert hasattr(trace_lib, name), name
        assert not hasattr(lib, name), "the product library carries no tracing entry point"


@pytest.mark.parametrize("kw,status", [
    (dict(trace=0), 1), (dict(max_tiles=-1), 1), (dict(trace=260), 2), (dict(A=0), 1),
    (dict(E=0), 1), (dict(bm=48), 1), (dict(K=12), 2), (dict(E=1025), 3),
])
def test_trace_host_checks(trace_lib, kw, status):
    a = dict(GOOD, trace=256, max_tiles=16)
    a.update(kw)
    assert trace_lib.gg_trace_grouped_gemm_bf16(a["A"], a["B"], a["off"], a["C"], a["E"], a["K"],
                                                a["N"], a["M_cap"], a["bm"], a["trace"],
                                                a["max_tiles"], None) == status
    assert trace_lib.gg_trace_clock_khz(None) == 1


def test_status_strings(lib):
    for code in range(5):
        assert lib.gg_status_string(code)
    assert lib.gg_status_string(99) == b"unknown status"


GOOD = dict(A=16, B=32, off=64, C=128, E=4, K=256, N=256, M_cap=29, bm=0)


def _call(lib, fn="gg_grouped_gemm_bf16", **kw):
    a = dict(GOOD)
    a.update(kw)
    # fake but aligned device addresses: every call below is rejected on the host
    return getattr(lib, fn)(a["A"], a["B"], a["off"], a["C"], a["E"], a["K"], a["N"],
                                    a["M_cap"], a["bm"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(A=0), 1), (dict(B=0), 1), (dict(C=0), 1), (dict(off=0), 1),
    (dict(E=0), 1), (dict(E=-3), 1), (dict(K=0), 1), (dict(N=0), 1), (dict(M_cap=-1), 1),
    (dict(bm=8), 1), (dict(bm=512), 1), (dict(bm=48), 1),
    (dict(A=24), 2), (dict(B=40), 2), (dict(C=8), 2), (dict(off=66), 2),
    (dict(K=12), 2), (dict(N=100), 2),
    (dict(E=1025), 3), (dict(M_cap=2**31 - 100), 3),
    (dict(K=2**22 + 8), 3), (dict(N=2**24 + 8), 3),
])
@pytest.mark.parametrize("fn", ["gg_grouped_gemm_bf16", "gg_grouped_gemm_bf16_bf16out",
                                "gg_grouped_gemm_bf16_swiglu"])
def test_host_checks(lib, kw, status, fn):
    assert _call(lib, fn, **kw) == status


@pytest.mark.parametrize("fn", ["gg_grouped_gemm_bf16", "gg_grouped_gemm_bf16_bf16out",
                                "gg_grouped_gemm_bf16_swiglu"])
def test_empty_problem_enqueues_nothing(lib, fn):
    # M_cap == 0: nothing to compute; returns before touching the device
    assert _call(lib, fn, M_cap=0) == 0


def test_tile_schedule_host_checks(lib):
    f = lib.gg_tile_schedule
    assert f(64, 4, 256, 29, 0, 128, 0, 10, None) == 1     # n_tiles NULL
    assert f(64, 4, 256, 29, 0, 0, 128, 10, None) == 1     # tiles NULL with max_tiles > 0
    assert f(64, 4, 256, 29, 0, 128, 128, -1, None) == 1   # negative max
    assert f(64, 4, 256, 29, 7, 128, 128, 10, None) == 1   # bad bm
    assert f(64, 4, 250, 29, 0, 128, 128, 10, None) == 2   # N not multiple of 8
    assert f(0, 4, 256, 29, 0, 128, 128, 10, None) == 1    # offsets NULL


def test_gather_host_checks(lib):
    f = lib.gg_grouped_gemm_bf16_gather
    #      X   n_src src  B   off  C    dst  E  K    N    M_cap bm
    ok = [16, 10, 64, 32, 64, 128, 0, 4, 256, 256, 29, 0]
    def call(**kw):
        a = list(ok)
        names = ["X", "n_src", "src", "B", "off", "C", "dst", "E", "K", "N", "M_cap", "bm"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return f(*a, None)
    assert call(src=0) == 1                    # src_rows NULL
    assert call(n_src=-1) == 1
    assert call(X=0) == 1
    assert call(src=66) == 2                   # misaligned index list
    assert call(dst=70) == 2
    assert call(n_src=2 ** 22 + 1) == 3        # n_src * K * 2 > 2^31
    assert call(M_cap=0) == 0                  # nothing to do


def test_gather_combine_host_checks(lib):
    f = lib.gg_grouped_gemm_bf16_gather_combine
    names = ["X", "n_src", "src", "B", "off", "dst", "w", "Y", "n_dst", "E", "K", "N", "M_cap",
             "bm"]
    ok = [16, 10, 64, 32, 64, 96, 48, 128, 10, 4, 256, 256, 29, 0]

    def call(**kw):
        a = list(ok)
        for k, v in kw.items():
            a[names.index(k)] = v
        return f(*a, None)
    assert call(dst=0) == 1                    # the combine needs destinations
    assert call(w=0) == 1                      # and weights
    assert call(n_dst=-1) == 1
    assert call(Y=0) == 1
    assert call(src=0) == 1
    assert call(w=50) == 2                     # misaligned weights
    assert call(Y=136) == 2                    # misaligned Y
    assert call(dst=98) == 2
    assert call(N=100) == 2
    assert call(bm=48) == 1
    assert call(n_src=2 ** 22 + 1) == 3
    assert call(M_cap=0) == 0                  # nothing to do


@pytest.mark.parametrize("fn", ["gg_grouped_gemm_fp8", "gg_grouped_gemm_fp8_bf16out",
                                "gg_grouped_gemm_fp8_swiglu"])
def test_fp8_host_checks(lib, fn):
    f = getattr(lib, fn)
    names = ["Aq", "a_scale", "Bq", "b_scale", "off", "C", "E", "K", "N", "M_cap", "bm"]
    ok = [16, 48, 32, 64, 96, 128, 4, 256, 256, 29, 0]

    def call(**kw):
        a = list(ok)
        for k, v in kw.items():
            a[names.index(k)] = v
        return f(*a, None)
    assert call(a_scale=0) == 1                # scales are required
    assert call(b_scale=0) == 1
    assert call(Aq=0) == 1
    assert call(a_scale=50) == 2               # misaligned row scales
    assert call(b_scale=72) == 2               # column scales need 16 bytes
    assert call(K=264) == 2                    # K a multiple of 16
    assert call(N=264) == 2                    # N a multiple of 16
    assert call(bm=48) == 1
    assert call(E=1025) == 3
    assert call(M_cap=0) == 0                  # nothing to do
