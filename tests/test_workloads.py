"""The seeded input generators (no GPU): bf16 rounding, group sizes, determinism."""

import numpy as np
import torch

import workloads as wl


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        (rng.standard_normal(1000) * 1e-30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 65504.0, 3.0e38], dtype=np.float32),
    ])
    ours = wl.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (ours == ref).all()


def test_bf16_ties_to_even():
    # 1 + 2^-8 lies exactly half way between bf16 neighbours 1 and 1 + 2^-7
    half = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8], dtype=np.float32)
    got = wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(half))
    assert got[0] == 1.0 and got[1] == 1.0 + 2 * 2.0 ** -7


def test_offsets_and_sizes():
    off = wl.offsets_from_sizes([3, 0, 17, 9])
    assert off.dtype == np.int32 and list(off) == [0, 3, 3, 20, 29]
    for name in wl.CONFIGS:
        s = wl.config_sizes(name)
        assert len(s) == wl.CONFIGS[name]["E"] and (s >= 0).all()
    assert wl.config_sizes("skew16k").sum() == 16384
    assert wl.config_sizes("skew2k_wide").sum() == 2048
    assert (wl.config_sizes("decode") == 16).all()


def test_deterministic_draws():
    a = wl.make_workload("tiny")
    b = wl.make_workload("tiny")
    assert (a.A == b.A).all() and (a.B == b.B).all()
    assert a.A.shape == (29, 256) and a.B.shape == (4, 256, 256)
    # values have the stated scale: N(0,1)/sqrt(256)
    v = wl.bf16_bits_to_f32(a.B)
    assert abs(float(v.std()) - 1 / 16) < 0.002


def test_e4m3_rounding_matches_torch():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(50000).astype(np.float32) * s for s in (1e-3, 0.1, 3, 100)])
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (wl.f32_to_e4m3_bits(x) == ref).all()
    # saturation above the largest finite value
    assert (wl.f32_to_e4m3_bits(np.array([500.0, -1e6], dtype=np.float32)) == [0x7E, 0xFE]).all()
