"""Pins of the oracle's counter-based noise: Philox4x32-10 against the
known-answer vectors published with its reference implementation, the
23-bit uniforms, and the Box-Muller normals against the standard normal
distribution (moments and a Kolmogorov-Smirnov test).  CPU only."""
import json
import math
import os

import numpy as np
import scipy.stats

import oracle
from sparsely_gated_mixture_noisy_amd.inputs import CONFIGS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_philox_known_answers():
    with open(os.path.join(GOLDEN, "philox_kat.json"), encoding="utf-8") as f:
        g = json.load(f)
    for v in g["vectors"]:
        ctr = np.array([int(h, 16) for h in v["ctr"]], dtype=np.uint64)
        key = np.array([int(h, 16) for h in v["key"]], dtype=np.uint64)
        out = oracle.philox4x32_10(ctr, key)
        assert [f"{int(w):08x}" for w in out] == v["out"]


def test_uniform23_range_and_exactness():
    x = np.array([0, 511, 512, 0xFFFFFFFF, 0x80000000], dtype=np.uint32)
    u = oracle.uniform23(x)
    assert u[0] == u[1] == 0.5 * 2.0 ** -23
    assert u[2] == 1.5 * 2.0 ** -23
    assert u[3] == 1.0 - 0.5 * 2.0 ** -23
    assert u[4] == 0.5 + 0.5 * 2.0 ** -23
    rng = np.random.default_rng(0)
    u = oracle.uniform23(rng.integers(0, 2 ** 32, 100000, dtype=np.uint64).astype(np.uint32))
    assert (u.astype(np.float32).astype(np.float64) == u).all()       # exact in float32
    assert ((u > 0) & (u < 1)).all()


def test_normals_are_standard():
    z = oracle.philox_normals(np.arange(400), 500, seed=12345).ravel()
    assert abs(z.mean()) < 4 / math.sqrt(z.size)
    assert abs(z.var() - 1.0) < 6 * math.sqrt(2.0 / z.size)
    assert scipy.stats.kstest(z, "norm").pvalue > 1e-3
    # the cos and sin halves of each pair are uncorrelated
    zz = z.reshape(-1, 2)
    assert abs(np.corrcoef(zz[:, 0], zz[:, 1])[0, 1]) < 5 / math.sqrt(zz.shape[0])


def test_normals_follow_the_counter_layout():
    """Element i of row t is word pair (i % 4) // 2 of counter (i // 4, t,
    sub, stream); streams, groups, rows and seeds give different draws."""
    seed = (7 << 32) | 99
    z = oracle.philox_normals([5], 8, seed)[0]
    w = oracle.philox4x32_10(np.array([1, 5, 0, 0], dtype=np.uint64),
                             np.array([99, 7], dtype=np.uint64))
    r = math.sqrt(-2.0 * math.log(oracle.uniform23(w[0])))
    a = 2.0 * math.pi * oracle.uniform23(w[1])
    assert abs(z[4] - r * math.cos(a)) < 1e-12 and abs(z[5] - r * math.sin(a)) < 1e-12
    base = oracle.philox_normals([5], 8, seed)
    for other in (oracle.philox_normals([6], 8, seed), oracle.philox_normals([5], 8, seed + 1),
                  oracle.philox_normals([5], 8, seed, sub=1),
                  oracle.philox_normals([5], 8, seed, stream=1)):
        assert not np.allclose(other, base)


def _element(seed, ctr):
    """The four normals of one Philox counter, written out from the
    documented mapping: words (0, 1) give elements 0 and 1 (cos and sin of
    one Box-Muller pair), words (2, 3) give elements 2 and 3, each word
    mapped to (top 23 bits + 1/2) / 2^23."""
    w = oracle.philox4x32_10(np.array(ctr, dtype=np.uint64),
                             np.array([seed & 0xFFFFFFFF, seed >> 32], dtype=np.uint64))
    u = [((int(v) >> 9) + 0.5) / 8388608.0 for v in w]
    out = []
    for a, b in ((u[0], u[1]), (u[2], u[3])):
        r = math.sqrt(-2.0 * math.log(a))
        out += [r * math.cos(2.0 * math.pi * b), r * math.sin(2.0 * math.pi * b)]
    return out


def test_draw_noise_counter_layout():
    """Every element of a layer's noise against Philox computed at the
    documented counter: flat element j of token t at (j // 4, t, 0, 0); the
    hierarchy's secondary element j of group g at (j // 4, t, g, 0) and its
    primary element g at (g // 4, t, 0, 1).  The rows are ragged (6 and 10
    elements, not multiples of 4), the seed uses both key words."""
    seed = (0x1234 << 32) | 0xABCDEF
    flat = oracle.draw_noise(CONFIGS["tiny"].replace(tokens=3, n_experts=10, top_k=2), seed)
    assert flat["eps"].shape == (3, 10) and flat["eps_p"] is None
    for t in range(3):
        for j in range(10):
            want = _element(seed, [j // 4, t, 0, 0])[j % 4]
            assert abs(flat["eps"][t, j] - want) < 1e-12, (t, j)
    hc = CONFIGS["hier4096"].replace(tokens=3, n_experts=18, n_groups=3, k_groups=2,
                                     k_per_group=2, top_k=4)
    h = oracle.draw_noise(hc, seed)
    assert h["eps"].shape == (3, 3, 6) and h["eps_p"].shape == (3, 3)
    for t in range(3):
        for g in range(3):
            want = _element(seed, [g // 4, t, 0, 1])[g % 4]
            assert abs(h["eps_p"][t, g] - want) < 1e-12, (t, g)
            for j in range(6):
                want = _element(seed, [j // 4, t, g, 0])[j % 4]
                assert abs(h["eps"][t, g, j] - want) < 1e-12, (t, g, j)
