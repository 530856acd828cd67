"""Random workloads through every entry point, each against the oracle.

Each seed draws one ragged problem (the generator of test_parity_gpu.py: E up
to 96, K and N any multiple of 8, empty and large experts, spare rows, a
random tile height) and runs it through the fp32, bf16 and SwiGLU products,
fp8 weights, fp8 activations and weights (where K and N are multiples of 16),
and a random top-k gather/scatter and weighted combine of the same shape.
Every output is checked as the dedicated tests check it.

The default is a short run of 8 seeds. GG_SWEEP="lo:hi" runs seeds lo..hi-1
instead (seeds 100..549 have been run through this module in full).
"""

import os

import numpy as np
import pytest

import workloads as wl
from tests.test_parity_gpu import (_combine_case, _fp8_compare, _full_compare,
                                   _full_compare_bf16, _full_compare_swiglu, _gather_case,
                                   _q8_compare, _random_workload, _say)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _seeds():
    lo, hi = (int(x) for x in os.environ.get("GG_SWEEP", "100:108").split(":"))
    return range(lo, hi)


@pytest.fixture(scope="module")
def gg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_ragged_grouped_amd as m
    m.load_library()
    return m


@pytest.mark.parametrize("seed", _seeds())
def test_every_entry_point(gg, seed):
    w, bm = _random_workload(seed)
    rng = np.random.default_rng(5000 + seed)
    _say("sweep seed %d: E=%d K=%d N=%d M_tot=%d M_cap=%d bm=%d"
         % (seed, w.E, w.K, w.N, w.M_tot, w.M_cap, bm))
    _full_compare(gg, w, bm, "seed %d" % seed)
    _full_compare_bf16(gg, w, bm, "seed %d bf16" % seed)
    _full_compare_swiglu(gg, w, bm, "seed %d swiglu" % seed)
    Bq, scale = wl.fp8_weights(w)
    _fp8_compare(gg, w, Bq, scale, bm, "seed %d fp8w" % seed)
    if w.K % 16 == 0 and w.N % 16 == 0:
        _q8_compare(gg, w, bm, "seed %d fp8" % seed)
    # top-k routing of a random token count onto the same experts and shape,
    # with the product kept at or below 4e8 multiply-adds
    topk = int(rng.integers(1, min(8, w.E) + 1))
    n_max = int(max(1, min(400, 4e8 / (topk * w.K * w.N))))
    n_tokens = int(rng.integers(1, n_max + 1))
    _gather_case(gg, n_tokens, w.E, w.K, w.N, topk, 7000 + seed, bm,
                 use_dst=bool(rng.integers(2)), pad=int(rng.integers(0, 20)))
    _combine_case(gg, n_tokens, w.E, w.K, w.N, topk, 8000 + seed, bm)
