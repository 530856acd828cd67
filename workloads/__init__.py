"""Seeded synthetic inputs for the ragged-M grouped GEMM.

This module only draws inputs. It holds none of the method's arithmetic (no
products, no sums over K, no tile bookkeeping) and is shared by both sides:
the CPU oracle under ``oracle/`` and the HIP path in ``moe_ragged_grouped_amd``.

What is drawn, and why it looks like the pages' workloads:

* Group sizes. "Grouped GEMM for Imbalanced Experts on Blackwell: A WIP
  Worklog" (section 2.1, "Skew and tile efficiency") gives expert e rows in
  proportion to (e+1)^-s; the rounding to integers is not printed.
  ``page_skew_sizes`` takes the reading that reproduces every printed figure
  (largest expert 4,793 rows, smallest 32 at 16,384 rows / 64 experts / s=1.2):
  floor of the proportional share, then the leftover rows one each to experts
  0, 1, 2, ...  ``routed_skew_sizes`` is the stochastic law of the measured
  skewed workloads: every routed row picks an expert with probability
  proportional to rank^-s, ranks being a seeded shuffle of 1..E.
* Values. float32 standard normals, scaled in float32 (by 1/sqrt(K) or by
  0.02), then rounded to the nearest bfloat16 with ties to even. bfloat16 is
  the top 16 bits of an IEEE binary32 word; the rounding below is the
  textbook round-half-even on the 16 discarded bits (inputs are finite).

* fp8 weights. ``fp8_weights`` turns a workload's bf16 weights into OCP fp8
  E4M3 codes with one fp32 scale per expert and output column: the scale
  maps the column's largest magnitude to 448 (the largest finite E4M3 value)
  and every weight divided by it is rounded to the nearest E4M3 value, ties
  to even. This is the input recipe of the fp8-weight product, not part of
  the product itself.

Streams: the group sizes come from numpy's PCG64 generator seeded with the
workload seed; A from ``default_rng([seed, 1])``; expert e's weight slice
from ``default_rng([seed, 2, e])``. Giving every expert its own stream keeps
the 805M-element weight tensors of the 6144x4096 shapes deterministic while
they are drawn in parallel threads, one bounded slice at a time.
"""

from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "Workload",
    "CONFIGS",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "page_skew_sizes",
    "routed_skew_sizes",
    "offsets_from_sizes",
    "make_workload",
    "config_sizes",
    "f32_to_e4m3_bits",
    "fp8_weights",
]


def f32_to_bf16_bits(x: np.ndarray, out: np.ndarray = None) -> np.ndarray:
    """Round finite float32 -> bfloat16 bit patterns (uint16), nearest, ties to even.

    Works in uint32: for every finite pattern u, u + 0x7FFF + 1 < 2^32, so the
    biased sum cannot wrap.
    """
    u = np.array(x, dtype=np.float32, copy=True, order="C").view(np.uint32)
    lsb = u >> np.uint32(16)
    lsb &= np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u >>= np.uint32(16)
    if out is None:
        return u.astype(np.uint16)
    out[...] = u
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def page_skew_sizes(m_tot: int, n_experts: int, s: float) -> np.ndarray:
    """Deterministic power-law split: rows of expert e proportional to (e+1)^-s.

    Floor of each share, leftover rows handed out one each to experts 0,1,...
    """
    w = np.array([(e + 1.0) ** (-s) for e in range(n_experts)], dtype=np.float64)
    base = np.floor(m_tot * w / w.sum()).astype(np.int64)
    left = int(m_tot - base.sum())
    for e in range(left):
        base[e % n_experts] += 1
    return base


def routed_skew_sizes(rng: np.random.Generator, m_tot: int, n_experts: int, s: float) -> np.ndarray:
    """Stochastic routing: each row picks expert e with p proportional to rank_e^-s.

    ranks = a seeded shuffle of 1..E. With s=0 this is uniform random routing.
    """
    ranks = rng.permutation(n_experts) + 1
    p = ranks.astype(np.float64) ** (-s)
    p /= p.sum()
    tok = rng.choice(n_experts, size=m_tot, p=p)
    return np.bincount(tok, minlength=n_experts).astype(np.int64)


def offsets_from_sizes(sizes) -> np.ndarray:
    """int32 group offsets [E+1]: off[0]=0, off[e+1]=off[e]+m_e."""
    sizes = np.asarray(sizes, dtype=np.int64)
    off = np.zeros(len(sizes) + 1, dtype=np.int64)
    np.cumsum(sizes, out=off[1:])
    if off[-1] > np.iinfo(np.int32).max:
        raise ValueError("row count exceeds int32")
    return off.astype(np.int32)


@dataclasses.dataclass
class Workload:
    """One grouped-GEMM problem as raw bfloat16 bits on the host."""

    name: str
    E: int
    K: int
    N: int
    sizes: np.ndarray        # int64 [E]
    offsets: np.ndarray      # int32 [E+1]
    M_cap: int               # rows allocated for A and C (>= offsets[-1])
    A: np.ndarray            # uint16 [M_cap, K]  (bf16 bits; rows >= M_tot are zero)
    B: np.ndarray            # uint16 [E, K, N]   (bf16 bits)
    seed: int

    @property
    def M_tot(self) -> int:
        return int(self.offsets[-1])

    @property
    def useful_flops(self) -> int:
        return 2 * self.M_tot * self.K * self.N


# name -> (E, K, N, sizes rule, value scale rule, seed)
#   sizes rule: ("list", [...]) | ("uniform", m) | ("routed", M_tot, s) | ("page", M_tot, s)
#   scale rule: "rsqrtk" -> N(0,1)/sqrt(K) ; "0.02" -> N(0, 0.02)
CONFIGS = {
    "tiny":        dict(E=4,  K=256,  N=256,  sizes=("list", [3, 0, 17, 9]),  scale="rsqrtk", seed=0),
    "decode":      dict(E=32, K=6144, N=4096, sizes=("uniform", 16),         scale="0.02",   seed=1),
    "uniform16k":  dict(E=64, K=1024, N=2688, sizes=("uniform", 256),        scale="rsqrtk", seed=2),
    "skew16k":     dict(E=64, K=1024, N=2688, sizes=("routed", 16384, 1.2),  scale="rsqrtk", seed=3),
    "skew2k_wide": dict(E=32, K=6144, N=4096, sizes=("routed", 2048, 1.2),   scale="0.02",   seed=4),
    # the page's deterministic skew law at the 16k shape (pins tile counts and eta)
    "skew16k_page": dict(E=64, K=1024, N=2688, sizes=("page", 16384, 1.2),   scale="rsqrtk", seed=3),
}


def _sizes(rule, E, rng):
    kind = rule[0]
    if kind == "list":
        return np.asarray(rule[1], dtype=np.int64)
    if kind == "uniform":
        return np.full(E, rule[1], dtype=np.int64)
    if kind == "routed":
        return routed_skew_sizes(rng, rule[1], E, rule[2])
    if kind == "page":
        return page_skew_sizes(rule[1], E, rule[2])
    raise ValueError(rule)


def _scale(rule, K):
    if rule == "rsqrtk":
        return np.float32(1.0) / np.float32(math.sqrt(K))
    if rule == "0.02":
        return np.float32(0.02)
    raise ValueError(rule)


def config_sizes(name: str) -> np.ndarray:
    """Group sizes of a named config without drawing A and B."""
    c = CONFIGS[name]
    rng = np.random.default_rng(c["seed"])
    return _sizes(c["sizes"], c["E"], rng)


def make_workload(name: str = None, *, E=None, K=None, N=None, sizes=None, scale="rsqrtk",
                  seed=0, M_cap=None, values="normal") -> Workload:
    """Draw a workload, either a named config or an explicit shape.

    values: "normal" (scaled N(0,1) rounded to bf16) or "int" (integers in
    [-3, 3], exact in bf16; every product and partial sum of a small problem
    is then an exact integer in float32).
    """
    if name is not None:
        c = CONFIGS[name]
        E, K, N, seed, scale = c["E"], c["K"], c["N"], c["seed"], c["scale"]
        rng = np.random.default_rng(seed)
        sizes = _sizes(c["sizes"], E, rng)
    else:
        rng = np.random.default_rng(seed)
        sizes = np.asarray(sizes, dtype=np.int64)
    assert len(sizes) == E
    off = offsets_from_sizes(sizes)
    m_tot = int(off[-1])
    if M_cap is None:
        M_cap = m_tot
    assert M_cap >= m_tot
    A = np.zeros((M_cap, K), dtype=np.uint16)
    B = np.empty((E, K, N), dtype=np.uint16)
    sc = _scale(scale, K)

    def draw(r, shape):
        if values == "int":
            return r.integers(-3, 4, size=shape).astype(np.float32)
        x = r.standard_normal(shape, dtype=np.float32)
        x *= sc
        return x

    f32_to_bf16_bits(draw(np.random.default_rng([seed, 1]), (m_tot, K)), out=A[:m_tot])

    def draw_expert(e):
        f32_to_bf16_bits(draw(np.random.default_rng([seed, 2, e]), (K, N)), out=B[e])

    workers = max(1, min(16, os.cpu_count() or 1, E))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(draw_expert, range(E)))
    return Workload(name=name or "custom", E=E, K=K, N=N, sizes=sizes, offsets=off,
                    M_cap=M_cap, A=A, B=B, seed=seed)


def f32_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to OCP fp8 E4M3 codes (uint8): nearest, ties to even,
    magnitudes above 448 saturated to 448.

    E4M3: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; normal values
    (1 + m/8) * 2^(e-7) for exponent fields 1..15 (field 15 with m = 7 is NaN,
    so the largest finite value is 1.75 * 2^8 = 448); subnormals m/8 * 2^-6.
    Values in [2^p, 2^(p+1)) are spaced 2^(p-3) apart, and below 2^-6 the
    spacing stays 2^-9. Scaling by powers of two is exact in binary64, so the
    division by the spacing is exact and numpy's round applies the tie rule.
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    neg = np.signbit(x)
    a = np.abs(x)
    _, ex = np.frexp(a)                       # a = f * 2^ex, f in [0.5, 1)
    spacing = np.ldexp(1.0, np.maximum(ex - 1, -6) - 3)
    q = np.minimum(np.round(a / spacing) * spacing, 448.0)
    code = np.zeros(a.shape, dtype=np.int64)
    normal = q >= 2.0 ** -6
    _, eq = np.frexp(q[normal])
    p = eq - 1                                # q = (1 + m/8) * 2^p
    m = np.round(np.ldexp(q[normal], -p) * 8).astype(np.int64) - 8
    code[normal] = ((p + 7) << 3) | m
    code[~normal] = np.round(q[~normal] / 2.0 ** -9).astype(np.int64)
    code |= neg.astype(np.int64) << 7
    return code.astype(np.uint8)


def fp8_activations(w: "Workload"):
    """fp8 E4M3 codes and per-row fp32 scales for w.A (rows past the last group
    included).

    scale[r] = max_k |A[r, k]| / 448 (1 for an all-zero row), computed in
    float32; codes = E4M3 rounding of A[r, k] / scale[r] (float32 division).
    Returns (codes uint8 [M_cap, K], scale float32 [M_cap]).
    """
    a = bf16_bits_to_f32(w.A)
    scale = (np.abs(a).max(axis=1) / np.float32(448.0)).astype(np.float32)
    scale[scale == 0] = 1.0
    codes = f32_to_e4m3_bits(a / scale[:, None])
    return codes, scale


def fp8_weights(w: "Workload"):
    """fp8 E4M3 codes and per-(expert, column) fp32 scales for w.B.

    scale[e, n] = max_k |B[e, k, n]| / 448 (1 for an all-zero column), computed
    in float32; codes = E4M3 rounding of B[e, k, n] / scale[e, n] (float32
    division). Returns (codes uint8 [E, K, N], scale float32 [E, N]).
    """
    E, K, N = w.B.shape
    codes = np.empty((E, K, N), dtype=np.uint8)
    scale = np.empty((E, N), dtype=np.float32)

    def one(e):
        b = bf16_bits_to_f32(w.B[e])
        s_e = (np.abs(b).max(axis=0) / np.float32(448.0)).astype(np.float32)
        s_e[s_e == 0] = 1.0
        scale[e] = s_e
        codes[e] = f32_to_e4m3_bits(b / s_e)

    workers = max(1, min(8, os.cpu_count() or 1, E))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(one, range(E)))
    return codes, scale
