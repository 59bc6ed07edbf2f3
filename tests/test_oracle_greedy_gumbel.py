"""Pins for the oracle's greedy chain verify and Gumbel-max sampling (CPU only).

* Argmax: a pure-Python first-maximum scan (brute force) and torch.argmax
  (library routine), including ties, signed zeros and NaN.
* Greedy chain verify: a hand-worked example of predict / accept_index /
  accept_length, and the planted-maximum workload where the target token is
  known by construction.
* Gumbel-max: the sampled token's law equals softmax(z / T) (chi-square over
  Philox seeds); rows below the greedy threshold are the argmax; strict
  acceptance over rows.
"""
import math

import numpy as np
import scipy.special
import scipy.stats

from oracle import greedy_verify, gumbel_row, gumbel_sample
from workloads import f32_to_bf16_bits, make_config


def _first_max(row):
    best, arg = None, 0
    for i, v in enumerate(row):
        if math.isnan(v):
            return i
        if best is None or v > best:
            best, arg = v, i
    return arg


def test_argmax_brute_force_and_torch():
    torch = __import__("torch")
    rng = np.random.default_rng(20)
    cases = [np.round(rng.standard_normal((3, 40))).astype(np.float32) for _ in range(20)]
    special = np.array([[-0.0, 0.0, -0.0, 0.0],
                        [1.0, np.nan, 3.0, np.nan],
                        [-np.inf, -np.inf, -np.inf, -np.inf],
                        [2.0, 5.0, 5.0, np.inf]], dtype=np.float32)
    cases.append(special)
    for z in cases:
        N = z.shape[0]
        out = greedy_verify(z[None], "f32", np.full((1, N - 1), -7, np.int32))
        for j in range(N):
            assert out["argmax"][0, j] == _first_max([float(v) for v in z[j]])
            assert out["argmax"][0, j] == int(torch.argmax(torch.from_numpy(z[j])))


def test_greedy_worked_example():
    V, N = 12, 4
    z = np.zeros((2, N, V), np.float32)
    y = [[5, 7, 9, 2], [1, 1, 0, 11]]
    for b in range(2):
        for j in range(N):
            z[b, j, y[b][j]] = 1.0
    x = np.array([[5, 7, 1], [3, 1, 0]], np.int32)
    out = greedy_verify(z, "f32", x)
    assert list(out["accept_length"]) == [2, 0]
    assert out["accepted_tokens"].tolist() == [[5, 7, 9, -1], [1, -1, -1, -1]]
    assert out["predict"].tolist() == [[5, 7, 9, -1], [1, -1, -1, -1]]
    assert out["accept_index"].tolist() == [[0, 1, 2, -1], [4, -1, -1, -1]]
    assert out["argmax"].tolist() == y
    xa = np.array([[5, 7, 9], [1, 1, 0]], np.int32)
    out = greedy_verify(z, "f32", xa)
    assert list(out["accept_length"]) == [3, 3]
    assert out["accepted_tokens"].tolist() == y


def test_greedy_planted_maximum_workload_subset():
    cfg = make_config(4, B=64)
    reqs = [0, 17, 31, 63]
    out = greedy_verify(cfg["logits"], "bf16", cfg["draft_ids"], requests=reqs)
    for b in reqs:
        assert list(out["argmax"][b]) == list(cfg["planted"][b])
        L = out["accept_length"][b]
        assert all(cfg["draft_ids"][b, :L] == cfg["planted"][b, :L])
        assert L == 3 or cfg["draft_ids"][b, L] != cfg["planted"][b, L]


def test_gumbel_law_is_temperature_softmax():
    z = np.array([0.3, -1.2, 2.0, 0.0, 1.1], np.float32)
    for T in (0.6, 1.5):
        n = 40000
        ys = np.array([gumbel_row(z, T, s, 5)[0] for s in range(n)])
        obs = np.bincount(ys, minlength=z.size)
        exp = scipy.special.softmax(z.astype(np.float64) / np.float64(np.float32(T))) * n
        chi2 = ((obs - exp) ** 2 / exp).sum()
        assert chi2 < scipy.stats.chi2.ppf(1 - 1e-4, z.size - 1), (T, chi2)


def test_gumbel_greedy_rows_and_strict_accept():
    rng = np.random.default_rng(21)
    B, D, V = 6, 3, 64
    z = rng.standard_normal((B, D + 1, V)).astype(np.float32) * 3
    T = np.array([0.0, 1e-6, 0.9, 1.2, 0.5, 0.0], np.float32)
    x = rng.integers(0, V, size=(B, D)).astype(np.int32)
    am = z.argmax(-1)
    x[0] = am[0, :D]                    # greedy request that accepts everything
    x[5, 0] = am[5, 0]
    x[5, 1] = (am[5, 1] + 1) % V         # greedy request that stops at position 1
    seed = np.arange(B, dtype=np.uint64) * np.uint64(3) + np.uint64(1)
    off = np.arange(B, dtype=np.uint64) * np.uint64(1 << 20)
    out = gumbel_sample(z, "f32", T, x, seed, off)
    full = gumbel_sample(z, "f32", T, x, seed, off, all_rows=True)
    assert out["accepted_tokens"].tolist() == full["accepted_tokens"].tolist()
    assert list(out["accept_length"]) == list(full["accept_length"])
    assert out["accepted_tokens"][0].tolist() == am[0].tolist() and out["accept_length"][0] == D
    assert out["accept_length"][5] == 1 and out["accepted_tokens"][5].tolist() == [am[5, 0], am[5, 1], -1, -1]
    assert full["sampled"][1].tolist() == am[1].tolist()
    for b in range(B):
        L = full["accept_length"][b]
        s = full["sampled"][b]
        assert all(x[b, :L] == s[:L]) and (L == D or x[b, L] != s[L])
    # the drafted token is accepted when it is the sample: feed the samples back as drafts
    x2 = full["sampled"][:, :D].astype(np.int32)
    again = gumbel_sample(z, "f32", T, x2, seed, off)
    assert list(again["accept_length"]) == [D] * B


def test_gumbel_band_covers_float32_scores():
    """An implementation that forms the scores in float32 (division and
    logarithms each correctly rounded) picks a different token than the
    float64 oracle only on rows the oracle flags as near ties.  Rows mix
    small and large |z/T| (T down to 0.02) so the scaled band is exercised;
    most rows get a planted runner-up whose logit is set so its score trails
    the best one by 0 to 1e-5 of its size, where float32 rounding decides."""
    from oracle import philox
    rng = np.random.default_rng(23)
    diff = 0
    for t in range(600):
        V = int(rng.integers(2, 3000))
        z = (rng.standard_normal(V) * rng.choice([0.5, 3.0, 30.0])).astype(np.float32)
        T = np.float32(rng.choice([0.02, 0.3, 1.0, 1.7]))
        seed, sub = int(rng.integers(1, 2 ** 40)), int(rng.integers(0, 2 ** 20))
        u32 = philox.uniform(philox.words(seed, sub, V)).astype(np.float32)
        if t % 4 and V > 2:
            g64 = -np.log(-np.log(u32.astype(np.float64)))
            s64 = z.astype(np.float64) / float(T) + g64
            top = int(np.argmax(s64))
            j2 = (top + 1 + int(rng.integers(0, V - 1))) % V
            gap = abs(s64[top]) * float(rng.choice([0.0, 1e-8, 1e-7, 1e-6, 1e-5]))
            z[j2] = np.float32((s64[top] - g64[j2] - gap) * float(T))
        y, near = gumbel_row(z, float(T), seed, sub)
        s32 = z / T + (-np.log(-np.log(u32)))
        if int(np.argmax(s32)) != y:
            diff += 1
            assert near, (t, V, float(T))
    assert diff > 0                                        # the planted runner-ups do reach the band
    print(f"float32 choices that differ: {diff} (all flagged)")


def test_gumbel_rows_use_distinct_streams():
    z = np.zeros((1, 8, 1000), np.float32)
    out = gumbel_sample(z, "f32", np.array([1.0], np.float32), np.zeros((1, 7), np.int32),
                        np.array([9], np.uint64), np.array([0], np.uint64), all_rows=True)
    assert len(set(out["sampled"][0].tolist())) > 4


def test_bf16_inputs_decode_exactly():
    z = np.array([[[1.0, 3.0, 2.0, -5.0], [0.5, 0.25, 0.125, 8.0]]], np.float32)
    out = greedy_verify(f32_to_bf16_bits(z), "bf16", np.array([[1]], np.int32))
    assert out["accepted_tokens"].tolist() == [[1, 3]]
