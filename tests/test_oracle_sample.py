"""Pins for the oracle's single-step sampling (CPU only).

* The joint filter reduces to the renormalisation already pinned when only
  one of top-k and top-p is active (so the sequential and joint orders agree).
* A hand-worked row where the orders differ: logits (3, 2, 1, 0), k = 2,
  top_p = 0.7.  The top-2 mass renormalised gives e^3 / (e^3 + e^2) = 0.731
  >= 0.7, so the sequential order keeps {3}; the whole row gives
  e^3 / (e^3 + e^2 + e + 1) = 0.644 < 0.7 and 0.644 + 0.237 >= 0.7, so the
  joint nucleus is {3, 2}, and with the top-2 set the joint filter keeps {3, 2}.
* Min-p keeps exactly the tokens whose softmax probability (scipy) is at
  least min_p times the largest; at min_p >= 1 that is the set of maximal
  probabilities (ties included).
* The sampled token follows the renormalised kept distribution (chi-square
  over Philox streams); greedy rows give the argmax.
"""
import numpy as np
from scipy.special import softmax

from oracle import joint_filter_row, renorm_row, sample


def test_single_filters_reduce_to_renorm():
    rng = np.random.default_rng(80)
    for _ in range(30):
        V = int(rng.integers(2, 40))
        z = np.round(rng.standard_normal(V) * 2, 1)
        T = float(rng.uniform(0.3, 1.5))
        k = int(rng.integers(0, V + 2))
        tp = float(rng.uniform(0.05, 1.0))
        w, _ = joint_filter_row(z, T, k, 1.0, 0.0)
        want, _ = renorm_row(z, T, k, 1.0)
        assert np.allclose(w / w.sum(), want, rtol=0, atol=1e-12)
        w, _ = joint_filter_row(z, T, 0, tp, 0.0)
        want, _ = renorm_row(z, T, 0, tp)
        assert np.allclose(w / w.sum(), want, rtol=0, atol=1e-12)


def test_joint_differs_from_sequential_worked_row():
    z = np.array([0.0, 3.0, 1.0, 2.0])
    w, _ = joint_filter_row(z, 1.0, 2, 0.7, 0.0)
    assert list(np.nonzero(w)[0]) == [1, 3]
    seq, _ = renorm_row(z, 1.0, 2, 0.7)
    assert list(np.nonzero(seq)[0]) == [1]


def test_min_p_matches_softmax_probabilities():
    rng = np.random.default_rng(81)
    for _ in range(40):
        V = int(rng.integers(2, 60))
        z = rng.standard_normal(V) * 3
        T = float(rng.uniform(0.4, 1.4))
        mp = float(rng.uniform(0.001, 0.9))
        p = softmax(z / T)
        w, fl = joint_filter_row(z, T, 0, 1.0, mp)
        if fl:
            continue
        assert np.array_equal(w > 0, p >= mp * p.max())


def test_min_p_at_or_above_one_keeps_the_maximal_set():
    """min_p = 1 keeps {p >= p_max}; min_p = 1.5 asks for p >= 1.5 p_max, which
    no token meets, and the reading clamps it to the same set (the page's
    name gives no formula past 1).  Rows with tied maxima keep every tie."""
    rng = np.random.default_rng(83)
    for t in range(40):
        V = int(rng.integers(2, 50))
        z = np.round(rng.standard_normal(V) * 2, 1)
        if t % 2 == 0:
            z[rng.integers(0, V, 3)] = z.max()          # tied maxima
        T = float(rng.uniform(0.3, 1.5))
        p = softmax(z / T)
        want = p >= p.max()
        for mp in (1.0, 1.5):
            w, fl = joint_filter_row(z, T, 0, 1.0, mp)
            assert np.array_equal(w > 0, want), (t, mp)
            # combined with top-k = V - 1 and a top-p of 0.99 the maximal set survives unchanged
            w2, _ = joint_filter_row(z, T, V - 1, 0.99, mp)
            assert np.array_equal(w2 > 0, want & (w2 > 0)) and (w2 > 0).any()


def test_sampled_law_and_greedy_rows():
    rng = np.random.default_rng(82)
    V, trials = 7, 30000
    z = (rng.standard_normal(V) * 1.5).astype(np.float32)
    T, k, tp, mp = 0.8, 5, 0.9, 0.02
    w, _ = joint_filter_row(z, T, k, tp, mp)
    law = w / w.sum()
    assert 2 <= np.count_nonzero(law) < V
    logits = np.tile(z, (trials, 1))
    out = sample(logits, "f32", np.full(trials, T), np.full(trials, k), np.full(trials, tp),
                 np.full(trials, mp), np.arange(1, trials + 1, dtype=np.uint64),
                 (np.arange(trials, dtype=np.uint64) * 7919) % 1000)
    obs = np.bincount(out["tokens"], minlength=V).astype(float)
    assert np.all(obs[law == 0] == 0)
    exp = law * trials
    m = exp > 5
    chi2 = ((obs[m] - exp[m]) ** 2 / exp[m]).sum()
    assert chi2 < 25, (chi2, obs, exp)
    g = sample(logits[:5], "f32", np.zeros(5), None, None, None, np.arange(5, dtype=np.uint64),
               np.zeros(5, np.uint64))
    assert np.all(g["tokens"] == int(np.argmax(z)))
