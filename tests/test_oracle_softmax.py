"""Pins for the oracle's temperature softmax and top-k / top-p renormalisation.

* scipy.special.softmax (library routine) for the temperature softmax.
* Hugging Face transformers' TemperatureLogitsWarper, TopKLogitsWarper and
  TopPLogitsWarper applied in sequence (library routines) on tie-free rows.
* Brute force over every subset of a tiny vocabulary with ties: the kept set is
  the smallest tie-closed, upward-closed set reaching k elements (top-k) and
  then the smallest one reaching top_p of the top-k mass (top-p).
"""
import itertools
import math

import numpy as np
import pytest
import scipy.special

from oracle import renorm_row, softmax_renorm, temperature_softmax


def test_softmax_matches_scipy():
    rng = np.random.default_rng(1)
    for V in (1, 2, 7, 1000):
        for T in (0.25, 0.7, 1.0, 3.0):
            z = rng.standard_normal(V) * 3
            got = temperature_softmax(z, T)
            want = scipy.special.softmax(z / T)
            np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-16)
            assert abs(got.sum() - 1.0) < 1e-14


def test_softmax_shift_invariance_and_greedy_limit():
    rng = np.random.default_rng(2)
    z = rng.standard_normal(50)
    np.testing.assert_allclose(temperature_softmax(z, 0.8), temperature_softmax(z + 123.0, 0.8), atol=1e-14)
    zt = np.array([0.0, 3.0, -1.0, 3.0])
    for T in (0.0, 1e-6, 9.99e-6, -1.0):
        assert list(temperature_softmax(zt, T)) == [0.0, 1.0, 0.0, 0.0]
    # just above the threshold it is a (very sharp) softmax, not a one-hot
    sharp = temperature_softmax(np.array([0.0, 1e-5]), 1.0000001e-5)
    assert 0.0 < sharp[0] < sharp[1] < 1.0


def test_renorm_disabled_filters_is_softmax():
    rng = np.random.default_rng(3)
    z = rng.standard_normal(300)
    for k in (0, -5, 300, 1000):
        for tp in (1.0, 1.5):
            got, flag = renorm_row(z, 0.9, k, tp)
            np.testing.assert_allclose(got, temperature_softmax(z, 0.9), atol=1e-15)
            assert not flag


def _hf_renorm(z, T, k, top_p):
    torch = pytest.importorskip("torch")
    lp = pytest.importorskip("transformers.generation.logits_process")
    s = torch.tensor(z[None, :], dtype=torch.float64)
    s = lp.TemperatureLogitsWarper(T)(None, s)
    if 0 < k < z.shape[0]:
        s = lp.TopKLogitsWarper(top_k=k)(None, s)
    if top_p < 1.0:
        s = lp.TopPLogitsWarper(top_p=top_p)(None, s)
    return torch.softmax(s, dim=-1)[0].numpy()


def test_renorm_matches_transformers_warpers():
    rng = np.random.default_rng(4)
    checked = 0
    for trial in range(60):
        V = int(rng.choice([5, 17, 64, 300]))
        z = rng.standard_normal(V) * rng.choice([0.5, 2.0, 4.0])
        T = float(rng.choice([0.5, 1.0, 1.7]))
        k = int(rng.choice([0, 1, 2, 5, V - 1, V]))
        tp = float(rng.choice([0.05, 0.3, 0.7, 0.9, 0.99, 1.0]))
        got, flag = renorm_row(z, T, k, tp)
        if flag:
            continue
        want = _hf_renorm(z, T, k, tp)
        np.testing.assert_allclose(got, want, atol=1e-12, err_msg=f"V={V} T={T} k={k} p={tp}")
        assert np.array_equal(got > 0, want > 0)
        checked += 1
    assert checked > 50


def _brute_kept(z, w, k, tp):
    """Smallest tie-closed upward-closed subsets by exhaustive search (float64 masses)."""
    V = len(z)

    def closed(S):
        return all((u in S) for v in S for u in range(V) if z[u] >= z[v])

    subsets = [frozenset(c) for r in range(1, V + 1) for c in itertools.combinations(range(V), r)]
    subsets = [S for S in subsets if closed(S)]
    kept_k = frozenset(range(V))
    if 0 < k < V:
        kept_k = min((S for S in subsets if len(S) >= k), key=len)
    if tp < 1.0:
        s_k = math.fsum(w[list(kept_k)])
        cands = [S for S in subsets if S <= kept_k and math.fsum(w[list(S)]) >= tp * s_k]
        kept = min(cands, key=len)
    else:
        kept = kept_k
    return kept


def test_renorm_brute_force_with_ties():
    vals = [-2.0, -1.0, 0.0, 1.0, 2.0]
    n = 0
    for V in (1, 2, 3, 4):
        for z in itertools.product(vals, repeat=V):
            z = np.array(z)
            for T in (0.6, 1.3):
                w = np.exp((z - z.max()) / T)
                for k in range(0, V + 1):
                    for tp in (0.2, 0.5, 0.75, 0.95, 1.0):
                        got, flag = renorm_row(z, T, k, tp)
                        if flag:
                            continue
                        kept = _brute_kept(z, w, k, tp)
                        assert set(np.nonzero(got > 0)[0].tolist()) == set(kept), (z, T, k, tp)
                        ws = np.array([w[i] if i in kept else 0.0 for i in range(V)])
                        np.testing.assert_allclose(got, ws / ws.sum(), atol=1e-15)
                        n += 1
    assert n > 3000


def test_topk_one_keeps_all_tied_maxima_and_top_p_zero_keeps_max_set():
    z = np.array([1.0, 4.0, 2.0, 4.0, 4.0, -3.0])
    got, _ = renorm_row(z, 1.0, 1, 1.0)
    np.testing.assert_allclose(got, [0, 1 / 3, 0, 1 / 3, 1 / 3, 0], atol=1e-15)
    got, _ = renorm_row(z, 1.0, 0, 0.0)
    np.testing.assert_allclose(got, [0, 1 / 3, 0, 1 / 3, 1 / 3, 0], atol=1e-15)
    # top-p sees the top-k-renormalised distribution: k=2 keeps {4,4,4} (ties) only
    got, _ = renorm_row(z, 1.0, 2, 0.5)
    np.testing.assert_allclose(got, [0, 1 / 3, 0, 1 / 3, 1 / 3, 0], atol=1e-15)


def test_batch_form_and_bf16_decode():
    from workloads import f32_to_bf16_bits
    rng = np.random.default_rng(5)
    z = rng.standard_normal((2, 3, 40)).astype(np.float32)
    zb = f32_to_bf16_bits(z)
    probs, flags = softmax_renorm(zb, "bf16", np.array([1.0, 0.0], np.float32),
                                  np.array([5, 0], np.int32), np.array([0.8, 1.0], np.float32))
    sub, _ = softmax_renorm(zb, "bf16", np.array([1.0, 0.0], np.float32), np.array([5, 0], np.int32),
                            np.array([0.8, 1.0], np.float32), requests=[1])
    assert np.array_equal(sub[0], probs[1])
    assert probs.shape == (2, 3, 40)
    np.testing.assert_allclose(probs.sum(-1), 1.0, atol=1e-13)
    assert np.all((probs[1] == 0) | (probs[1] == 1))
    assert np.all((probs[0] > 0).sum(-1) <= 5 + 3)
