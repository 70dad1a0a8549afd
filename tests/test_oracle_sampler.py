"""Pins of the sampling-suffix oracle (oracle/sampler.py) against what the mathematics and the published generator
fix: the SplitMix64 reference outputs from state 0, uniformity of u, the penalty and bias readings on a hand-worked
example, greedy and top-k = 1 limits, the exact distribution of an unrestricted draw on a uniform grid of u, the
top-p / min-p cut points on a distribution with known cumulative sums, rank ties, the inverse CDF boundaries, and
log-softmax identities."""
import numpy as np
import pytest

from oracle import sampler as S


def test_splitmix64_reference_outputs():
    # the generator's first outputs from state 0 (the published reference implementation's sequence)
    assert S.splitmix64(0, 0) == 0xE220A8397B1DCDAF
    assert S.splitmix64(0, 1) == 0x6E789E6AA1B965F4
    assert S.splitmix64(0, 2) == 0x06C45D188009454F


def test_uniform_is_uniform_and_exact_in_float32():
    u = np.array([S.uniform(12345, d) for d in range(100000)])
    assert u.min() >= 0.0 and u.max() < 1.0
    assert np.all(u.astype(np.float32).astype(np.float64) == u)   # 24 bits: exact in float32
    counts, _ = np.histogram(u, bins=64, range=(0, 1))
    chi2 = float(np.sum((counts - 100000 / 64) ** 2 / (100000 / 64)))
    assert chi2 < 120, chi2   # 63 degrees of freedom; the 99.99% point is about 115
    assert abs(u.mean() - 0.5) < 0.005


def test_adjust_hand_example():
    logits = np.array([2.0, -2.0, 1.0, 0.0, np.nan])
    counts = np.array([1, 2, 0, 3, 0])
    bias = np.array([0.0, 0.5, 0.0, 0.0, 0.0])
    z = S.adjust(logits, counts, bias, rep=2.0, presence=0.1, frequency=0.2)
    # seen 2 > 0: 2 / 2 - 0.1 - 0.2; seen -2: -2 * 2 - 0.1 - 0.4 + 0.5; unseen 1; seen 0: 0 * 2 - 0.1 - 0.6; NaN
    assert np.allclose(z[:4], [0.7, -4.0, 1.0, -0.7], atol=1e-15)
    assert z[4] == -np.inf


def test_greedy_and_top1_limits():
    rng = np.random.default_rng(0)
    for _ in range(20):
        l = rng.normal(size=50)
        c = rng.integers(0, 3, size=50)
        want = int(np.argmax(S.adjust(l, c, None, rep=1.3, presence=0.2, frequency=0.1)))
        assert S.sample(l, c, None, temperature=0.0, rep=1.3, presence=0.2, frequency=0.1) == want
        for d in range(5):
            assert S.sample(l, c, None, temperature=0.7, top_k=1, rep=1.3, presence=0.2, frequency=0.1,
                            seed=9, d=d) == want
            assert S.sample(l, c, None, temperature=1e-6, rep=1.3, presence=0.2, frequency=0.1, seed=9, d=d) == want
    assert S.sample([1.0, 3.0, 3.0, 2.0], [0] * 4, None, temperature=0.0) == 1   # ties: lowest index


def test_unrestricted_draw_has_the_softmax_distribution():
    l = np.array([0.3, -1.0, 2.0, 0.0, 1.5])
    T = 0.8
    p = np.exp(l / T) / np.exp(l / T).sum()
    kept, w = S.keep_set(S.adjust(l, np.zeros(5), None), T)
    assert list(kept) == [0, 1, 2, 3, 4]
    N = 20000
    picks = np.array([S.draw(kept, w, (i + 0.5) / N) for i in range(N)])
    freq = np.bincount(picks, minlength=5) / N
    assert np.max(np.abs(freq - p)) <= 1.0 / N + 1e-12


def test_top_p_and_min_p_cut_points():
    q = np.array([0.05, 0.5, 0.15, 0.3])   # ranks: 1, 3, 2, 0 -> cumulative 0.5, 0.8, 0.95, 1.0
    z = np.log(q)
    kept, _ = S.keep_set(z, 1.0, top_p=0.79)   # (0.8 itself sits on a rounding boundary)
    assert list(kept) == [1, 3]
    kept, _ = S.keep_set(z, 1.0, top_p=0.81)
    assert list(kept) == [1, 2, 3]
    kept, _ = S.keep_set(z, 1.0, top_p=0.01)
    assert list(kept) == [1]                       # at least the top token
    kept, w = S.keep_set(z, 1.0, min_p=0.2)        # q >= 0.1
    assert list(kept) == [1, 2, 3] and np.allclose(w / w.sum(), np.array([0.5, 0.15, 0.3]) / 0.95)
    kept, _ = S.keep_set(z, 1.0, top_k=2, top_p=0.9)   # top-k first: renormalized 0.625, 0.375
    assert list(kept) == [1, 3]
    kept, _ = S.keep_set(z, 1.0, top_k=2, top_p=0.6)
    assert list(kept) == [1]


def test_rank_ties_and_inverse_cdf_boundaries():
    z = np.array([1.0, 2.0, 2.0, 2.0, 0.0])
    kept, _ = S.keep_set(z, 1.0, top_k=2)
    assert list(kept) == [1, 2]                    # equal values: lower index ranks first
    kept, w = np.array([2, 5, 7]), np.array([0.2, 0.5, 0.3])
    assert [S.draw(kept, w, u) for u in (0.0, 0.1999, 0.2, 0.69, 0.7, 0.9999)] == [2, 2, 5, 5, 7, 7]


def test_logprobs_identities():
    z = np.array([0.5, 2.0, -1.0, 2.0])
    top, lp, lt = S.logprobs(z, 0.0, 3, token=2)
    full = z - np.log(np.sum(np.exp(z)))
    assert list(top) == [1, 3, 0] and np.allclose(lp, full[[1, 3, 0]]) and np.isclose(lt, full[2])
    top, lp, _ = S.logprobs(z, 2.0, 4, token=0)
    assert np.isclose(np.sum(np.exp(lp)), 1.0)
