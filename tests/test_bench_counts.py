"""bench.py's per-launch accounting, pinned to the figures written out by hand
(and, last, its summary of a traced launch's timeline on a hand-made record set).

The roofline fractions in every bench line divide these counts by the
measured time, so each count is checked here against its parts:
A = routed rows x K, B = experts with rows x K x N, C = routed rows x N, at
each operand's element size (fp8 codes carry one fp32 scale per row or
column). The literal totals below are those sums done by hand; the 16k and
decode totals are the 562.0 MB and 1,625.3 MB of the workload tables.
"""
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as wl  # noqa: E402


def _args(out="fp32", weights="bf16", acts="bf16", gather=False, combine=False):
    return SimpleNamespace(out=out, weights=weights, acts=acts, gather=gather, combine=combine)


def test_decode_counts():
    sizes = wl.config_sizes("decode")  # 32 experts x 16 rows
    useful, alg, peak = bench.launch_counts(sizes, 6144, 4096, _args())
    assert useful == 25_769_803_776  # 2 * 512 * 6144 * 4096
    # A 6,291,456 + B 1,610,612,736 + C 8,388,608
    assert alg == 1_625_292_800
    assert peak == bench.MFMA_BF16_PEAK_TFLOPS


def test_uniform16k_counts():
    sizes = wl.config_sizes("uniform16k")  # 64 experts x 256 rows
    useful, alg, _ = bench.launch_counts(sizes, 1024, 2688, _args())
    assert useful == 90_194_313_216  # 2 * 16384 * 1024 * 2688
    # A 33,554,432 + B 352,321,536 + C 176,160,768
    assert alg == 562_036_736
    # bf16 C: C 88,080,384; SwiGLU H: one bf16 per (gate, up) pair, 44,040,192
    assert bench.launch_counts(sizes, 1024, 2688, _args(out="bf16"))[1] == 473_956_352
    assert bench.launch_counts(sizes, 1024, 2688, _args(out="swiglu"))[1] == 429_916_160


def test_skewed_counts_every_expert_active():
    # every expert of the seeded skewed draws has rows, so B counts all of them
    s16 = wl.config_sizes("skew16k")
    assert (s16 > 0).all() and s16.sum() == 16384
    assert bench.launch_counts(s16, 1024, 2688, _args())[1] == 562_036_736
    s2k = wl.config_sizes("skew2k_wide")
    assert (s2k > 0).all() and s2k.sum() == 2048
    useful, alg, _ = bench.launch_counts(s2k, 6144, 4096, _args())
    assert useful == 103_079_215_104  # 2 * 2048 * 6144 * 4096
    # A 25,165,824 + B 1,610,612,736 + C 33,554,432
    assert alg == 1_669_332_992


def test_empty_expert_weights_not_counted():
    # tiny: m = [3, 0, 17, 9]; three experts with rows, K = N = 256
    sizes = wl.config_sizes("tiny")
    useful, alg, _ = bench.launch_counts(sizes, 256, 256, _args())
    assert useful == 2 * 29 * 256 * 256
    # A 2*29*256 = 14,848 + B 2*256*256*3 = 393,216 + C 4*29*256 = 29,696
    assert alg == 437_760


def test_fp8_counts_and_peaks():
    sizes = wl.config_sizes("decode")
    # fp8 weights: B (6144 codes + one fp32 scale per column's 4 bytes) * 4096 * 32
    _, alg, peak = bench.launch_counts(sizes, 6144, 4096, _args(weights="fp8"))
    assert alg == 6_291_456 + 805_830_656 + 8_388_608
    assert peak == bench.MFMA_BF16_PEAK_TFLOPS  # widened to bf16 for the matrix cores
    # fp8 activations too: A (6144 + 4) * 512 = 3,147,776, on the fp8 matrix cores
    _, alg, peak = bench.launch_counts(sizes, 6144, 4096, _args(weights="fp8", acts="fp8"))
    assert alg == 3_147_776 + 805_830_656 + 8_388_608
    assert peak == bench.MFMA_FP8_PEAK_TFLOPS


def test_indexed_rows_add_their_lists_and_the_combine_its_reads():
    sizes = np.array([5, 0, 7])
    K, N, M = 64, 32, 12
    base = 2 * M * K + 2 * K * N * 2 + 4 * M * N
    assert bench.launch_counts(sizes, K, N, _args())[1] == base
    # two int32 index lists
    assert bench.launch_counts(sizes, K, N, _args(gather=True))[1] == base + 8 * M
    # plus a read of each output element and one fp32 weight per row
    assert (bench.launch_counts(sizes, K, N, _args(gather=True, combine=True))[1]
            == base + 8 * M + 4 * M * N + 4 * M)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_tile_trace_summary_of_a_known_timeline():
    # two workgroups (XCDs 0 and 1), three tiles on a 100 MHz counter:
    # workgroup 0 runs tiles 0 and 2, workgroup 1 tile 1
    import moe_ragged_grouped_amd as gg
    W, R = gg.TRACE_WORKGROUPS, gg.TRACE_RECORD
    tr = np.zeros((W + 3, R), dtype=np.int64)
    t0 = 10 ** 9
    tr[0, :4] = [t0, t0 + 200, 0 << 6, 2]
    tr[1, :4] = [t0 + 100, t0 + 300, 1 << 6, 1]
    # start, decoded, end, bm, workgroup, expert, rows, col0 (ticks of 10 ns)
    tr[W + 0] = [t0 + 250, t0 + 320, t0 + 4250, 256, 0, 0, 256, 0]
    tr[W + 1] = [t0 + 350, t0 + 410, t0 + 2350, 64, 1, 1, 40, 0]
    tr[W + 2] = [t0 + 4266, t0 + 4330, t0 + 8266, 256, 0, 2, 256, 256]
    s = bench.tile_trace_summary(tr, 100000, 2, 3)
    assert s["span_us"] == 82.66
    assert s["workgroup_finish_us"] == {"min": 23.5, "mean": 53.1, "max": 82.7}
    assert s["workgroup_busy_us"] == {"mean": 50.0, "max": 80.0}
    assert s["gap_between_tiles_us"] == {"median": 0.16, "p90": 0.16, "count": 1}
    assert s["schedule_build_us"] == 2.0
    assert s["entry_to_first_tile_us"] == 2.5
    assert s["tile_decode_us"]["median"] == 0.64
    assert s["tiles_by_height"] == {64: {"count": 1, "mean_us": 20.0},
                                    256: {"count": 2, "mean_us": 40.0}}
    assert s["xcd_busy_mean_us"][:2] == [80.0, 20.0] and s["xcd_busy_mean_us"][2] is None
    assert s["workgroups_on_xcd_b_mod_8"] == 1.0
    assert s["tile_us_by_col0"] == {0: 30.0, 256: 40.0}
