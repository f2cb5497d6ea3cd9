"""Pins of the oracle's next-token selection: defined exp, Philox, nucleus draw.

* The defined exp's constants equal the nearest binary32 values of the exact
  mathematical constants (checked with exact rationals), and E(x) is within one
  ulp of fp64 exp over the whole [-23, 0] range it is used on.
* Philox4x32-10 equals rocRAND's independent implementation (its public header
  compiled and run, not copied).
* The nucleus draw equals a brute-force re-derivation with Python integers on
  tiny vocabularies; top-p -> 0 reduces to argmax; with T = 1 and top-p = 1 the
  draws follow softmax(logits) (chi-square test).
* The defined log L is within two ulps of fp64 log over the inputs the Gumbel
  noise feeds it; the noise follows the standard Gumbel law (Kolmogorov-Smirnov
  against exp(-exp(-g))); Gumbel-max equals a brute-force re-derivation from
  Philox words and fp64 logs on tiny vocabularies, reduces to argmax for large
  logit gaps and T = 0, and its draws follow softmax(logits / T) (chi-square).
"""
import math
import os
import shutil
import subprocess
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


# ---------------------------------------------------------------- defined exp

def _nearest_f32(x: Fraction) -> float:
    c = np.float32(float(x))
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    return float(min(cands, key=lambda f: abs(Fraction(float(f)) - x)))


def test_expdef_constants_are_nearest_binary32(orc):
    getcontext().prec = 60
    ln2 = Fraction(Decimal(2).ln())
    c = orc.expdef_constants().astype(np.float64)
    assert c[0] == _nearest_f32(1 / ln2)                     # log2(e)
    assert c[1] == _nearest_f32(ln2)                         # ln 2 (high part)
    assert c[2] == _nearest_f32(ln2 - Fraction(c[1]))         # ln 2 - high part
    for n in range(8):
        assert c[3 + n] == _nearest_f32(Fraction(1, math.factorial(n))), n


def test_expdef_within_one_ulp_of_exp(orc):
    x = np.concatenate([np.linspace(-23, 0, 1_000_001, dtype=np.float32),
                        -np.random.default_rng(0).random(200_000).astype(np.float32) * 23,
                        np.float32([0.0, -0.0, -1e-30, -1e-7, -23.0, -0.34657359, -0.34657362])])
    y = orc.expdef(x).astype(np.float64)
    ref = np.exp(x.astype(np.float64))
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    assert np.max(np.abs(y - ref) / ulp) <= 1.0
    assert orc.expdef([0.0])[0] == 1.0


# ---------------------------------------------------------------- Philox

def test_philox_matches_rocrand():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND cross-check")
    import oracle
    exe = os.path.join(os.environ.get("TMPDIR", "/tmp"), f"lf_philox_check_{os.getpid()}")
    subprocess.run([hipcc, "-O1", "-o", exe, os.path.join(HERE, "helpers", "philox_rocrand_check.cpp")],
                   check=True, capture_output=True)
    rng = np.random.default_rng(11)
    cases = [(0, 0), (1234, 0), (1234, 16384), (1234, 16511), (2 ** 64 - 1, 2 ** 32 - 1), (2 ** 32, 7)]
    cases += [(int(s), int(p)) for s, p in zip(rng.integers(0, 2 ** 63, 40), rng.integers(0, 2 ** 31, 40))]
    inp = "".join(f"{s} {p}\n" for s, p in cases)
    out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout.split("\n")
    os.unlink(exe)
    for (s, p), line in zip(cases, out):
        ref = [int(v) for v in line.split()]
        ours = oracle.philox4x32_10([p & 0xFFFFFFFF, p >> 32, 0, 0], [s & 0xFFFFFFFF, s >> 32])
        assert list(map(int, ours)) == ref, (s, p)


# ---------------------------------------------------------------- nucleus draw

def _brute_force_token(orc, logits, T, top_p, seed, pos):
    """Re-derivation with Python integers and an explicit sort."""
    n = len(logits)
    invT = np.float32(1.0 / float(np.float32(T)))
    z = [np.float32(l) * invT for l in np.float32(logits)]
    zs = max(z)
    dz = np.array([np.float32(zi - zs) for zi in z], dtype=np.float32)
    e = orc.expdef(dz)
    q = [0 if dz[i] < -23 else int(np.float64(e[i]) * 2 ** 32) for i in range(n)]
    order = sorted(range(n), key=lambda i: (-float(z[i]), i))
    m_star = math.ceil(float(np.float32(top_p)) * float(sum(q)))
    nucleus, run = [], 0
    for i in order:
        nucleus.append(i)
        run += q[i]
        if run >= m_star:
            break
    cn = sum(q[i] for i in nucleus)
    x = orc.philox4x32_10([pos, 0, 0, 0], [seed & 0xFFFFFFFF, seed >> 32])
    r = (int(x[1]) << 32) | int(x[0])
    t = (r * cn) >> 64
    run = 0
    for i in sorted(nucleus):
        run += q[i]
        if run > t:
            return i


def test_nucleus_draw_brute_force_tiny_vocab(orc):
    rng = np.random.default_rng(12)
    for trial in range(300):
        n = int(rng.integers(1, 17))
        logits = (rng.standard_normal(n) * rng.choice([0.1, 1, 5, 30])).astype(np.float32)
        if trial % 5 == 0:                       # exact ties in the logits
            logits = np.round(logits).astype(np.float32)
        T = float(rng.choice([0.3, 0.8, 1.0, 2.0]))
        top_p = float(rng.choice([0.05, 0.5, 0.9, 1.0]))
        seed, pos = int(rng.integers(0, 2 ** 63)), int(rng.integers(0, 2 ** 20))
        assert orc.sample(logits, T, top_p, seed, pos) == _brute_force_token(orc, logits, T, top_p, seed, pos)


def test_greedy_when_temperature_zero(orc):
    logits = np.float32([0.5, 2.0, 2.0, -1.0])
    assert orc.sample(logits, 0.0, 0.9, 1234, 3) == 1


def test_tiny_top_p_reduces_to_argmax(orc):
    rng = np.random.default_rng(13)
    for _ in range(50):
        logits = rng.standard_normal(4096).astype(np.float32)
        assert orc.sample(logits, 0.8, 1e-9, 1234, int(rng.integers(0, 1 << 20))) == orc.argmax(logits)


def test_nucleus_is_minimal_top_mass_prefix(orc):
    rng = np.random.default_rng(14)
    logits = rng.standard_normal(32768).astype(np.float32)
    d = orc.sample_detail(logits, 0.8, 0.9, 1234, 16384)
    q, inn = d["q"].astype(np.float64), d["in_nucleus"]
    assert d["c_v"] == int(d["q"].sum()) and d["c_n"] == int(d["q"][inn].sum())
    z = logits * np.float32(1.25)
    assert z[inn].min() >= z[~inn].max()                     # a top set by z
    assert d["c_n"] >= math.ceil(np.float64(np.float32(0.9)) * d["c_v"])
    smallest = np.where(inn)[0][np.argmin(z[inn])]
    assert d["c_n"] - int(d["q"][smallest]) < math.ceil(np.float64(np.float32(0.9)) * d["c_v"])
    assert inn[d["token"]] and d["t"] < d["c_n"]
    assert d["nucleus_size"] == int(inn.sum())


def test_draws_follow_softmax(orc):
    """T = 1, top-p = 1: frequencies over 10^5 counters match softmax (chi-square)."""
    logits = np.float32([1.0, 0.0, -0.5, 2.0, 0.25, -3.0, 1.5, 0.9])
    p = np.exp(logits.astype(np.float64) - logits.max())
    p /= p.sum()
    N = 100_000
    counts = np.zeros(len(logits))
    for pos in range(N):
        counts[orc.sample(logits, 1.0, 1.0, 42, pos)] += 1
    chi2 = float(((counts - N * p) ** 2 / (N * p)).sum())
    assert chi2 < 30.0, (chi2, counts / N, p)        # 7 dof: P(chi2 > 30) ~ 1e-4


# ---------------------------------------------------------------- Gumbel-max

def test_logdef_within_two_ulp_of_log(orc):
    rng = np.random.default_rng(5)
    x = np.concatenate([
        (2 * np.arange(0, 2 ** 23, 97, dtype=np.float64) + 1) * 2.0 ** -24,    # the u grid
        np.linspace(1e-7, 17.0, 400_001),                                     # -L(u) range
        rng.random(200_000) * 2.0 ** rng.integers(-126, 127, 200_000),        # all exponents
        2.0 ** np.arange(-126, 128, dtype=np.float64),
        [1.0, 1.0 - 2.0 ** -24, 1.0 + 2.0 ** -23, float.fromhex("0x1.6a09e6p+0"), float.fromhex("0x1.6a09e8p+0"), 0.5, 2.0]])
    x = x.astype(np.float32)
    x = x[(x > 0) & np.isfinite(x) & (x >= np.float32(2.0 ** -126))]
    y = orc.logdef(x).astype(np.float64)
    ref = np.log(x.astype(np.float64))
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    ulp = np.maximum(ulp, np.float64(2.0 ** -149))
    err = np.abs(y - ref) / ulp
    assert err.max() <= 2.0, (err.max(), x[np.argmax(err)])
    assert orc.logdef([1.0])[0] == 0.0


def test_gumbel_noise_follows_gumbel_law(orc):
    """Kolmogorov-Smirnov: 2*10^5 noise values against F(g) = exp(-exp(-g))."""
    g = np.array([orc.gumbel_noise(99, pos, i) for pos in range(2000) for i in range(100)])
    assert np.isfinite(g).all()
    g.sort()
    n = g.size
    F = np.exp(-np.exp(-g))
    ks = max(np.max(np.arange(1, n + 1) / n - F), np.max(F - np.arange(n) / n))
    assert ks < 1.95 / math.sqrt(n), ks            # P(D > 1.95/sqrt(n)) ~ 1e-3
    assert abs(g.mean() - 0.5772156649) < 0.01      # Euler-Mascheroni constant


def _gumbel_brute(orc, logits, T, seed, pos):
    """argmax(z + g) with g from the Philox words and fp64 logs; also the gap
    between the two largest scores."""
    key = np.uint32([seed & 0xFFFFFFFF, seed >> 32])
    invT = np.float32(1.0 / T)
    y = []
    for i, l in enumerate(logits):
        x0 = int(orc.philox4x32_10(np.uint32([pos, i, 1, 0]), key)[0])
        u = (2 * (x0 >> 9) + 1) * 2.0 ** -24
        y.append(float(np.float32(l) * invT) - math.log(-math.log(u)))
    y = np.array(y)
    top = np.sort(y)[-2:]
    return int(np.argmax(y)), (top[1] - top[0]) if len(y) > 1 else math.inf


def test_gumbel_brute_force_tiny_vocab(orc):
    rng = np.random.default_rng(8)
    checked = 0
    for case in range(300):
        V = int(rng.integers(1, 12))
        logits = (rng.standard_normal(V) * 2).astype(np.float32)
        T, seed, pos = float(rng.choice([0.5, 0.8, 1.0, 1.7])), int(rng.integers(0, 2 ** 63)), int(rng.integers(0, 2 ** 31))
        tok = orc.sample_gumbel(logits, T, seed, pos)
        ref, gap = _gumbel_brute(orc, logits, T, seed, pos)
        if gap > 1e-4:
            assert tok == ref, (case, tok, ref, gap)
            checked += 1
    assert checked > 250


def test_gumbel_greedy_limits(orc):
    logits = np.float32([0.0, 3.0, -1.0, 2.5])
    assert all(orc.sample_gumbel(logits, 0.0, 7, pos) == 1 for pos in range(50))
    logits = np.float32([0.0, 100.0, -1.0, 2.5])   # gap beyond any noise difference (< 40)
    assert all(orc.sample_gumbel(logits, 1.0, 7, pos) == 1 for pos in range(500))
    assert orc.sample_gumbel(np.float32([]), 1.0, 7, 0) == -1


def test_gumbel_draws_follow_softmax(orc):
    """T = 0.7: frequencies over 10^5 counters match softmax(logits / T) (chi-square)."""
    logits = np.float32([1.0, 0.0, -0.5, 2.0, 0.25, -3.0, 1.5, 0.9])
    z = logits.astype(np.float64) * float(np.float32(1.0 / 0.7))
    p = np.exp(z - z.max())
    p /= p.sum()
    N = 100_000
    counts = np.zeros(len(logits))
    for pos in range(N):
        counts[orc.sample_gumbel(logits, 0.7, 42, pos)] += 1
    chi2 = float(((counts - N * p) ** 2 / (N * p)).sum())
    assert chi2 < 30.0, (chi2, counts / N, p)        # 7 dof: P(chi2 > 30) ~ 1e-4
