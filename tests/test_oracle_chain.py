"""Pins for the oracle's chain rejection sampling (CPU only).

* Closed forms: P(accept x) = min(1, p(x)/q(x)); P(accept at i) = sum min(p_i, q_i)
  when x_i ~ q_i; the emitted token's law equals the target row (the
  rejection-sampling identity min(p, q) + max(0, p - q) = p); P(L >= j) =
  prod_{i<j} alpha_i.  Checked on deterministic grids of uniforms through the
  oracle's core, and by Monte Carlo through its Philox streams.
* Special cases: q = p accepts every draft; disjoint supports reject at 0;
  invalid ids reject; all-zero rows fall back to p, then to a uniform index.
"""
import math

import numpy as np
import pytest

from oracle import chain_reject, chain_reject_core, chain_uniforms, residual_draw

GRID = 1 << 12
UGRID = (2 * np.arange(GRID) + 1) / (2.0 * GRID)          # midpoints of a 2**12 grid


def _core(q, x, p, ua, uf):
    code = int(round(uf * 2 ** 24)) | 1
    return chain_reject_core(q, np.asarray(x), p, np.asarray(ua, dtype=np.float64), float(uf), code)


def _rows(rng, V, n, zero_frac=0.0):
    w = rng.random((n, V)) ** 3
    w[rng.random((n, V)) < zero_frac] = 0.0
    w[:, 0] += 1e-3
    return (w / w.sum(-1, keepdims=True)).astype(np.float32)


def test_accept_probability_is_min_ratio():
    rng = np.random.default_rng(10)
    V = 5
    for _ in range(5):
        p = _rows(rng, V, 2)
        q = _rows(rng, V, 1, zero_frac=0.3)
        alpha = 0.0
        for x in range(V):
            acc = np.mean([_core(q, [x], p, [u], 0.5)["L"] == 1 for u in UGRID])
            c, a = float(q[0, x]), float(p[0, x])
            want = 1.0 if c == 0 and a > 0 else (0.0 if c == 0 else min(1.0, a / c))
            assert abs(acc - want) <= 1.0 / GRID + 1e-12, (x, acc, want)
            alpha += c * acc
        assert abs(alpha - np.minimum(p[0], q[0]).astype(np.float64).sum()) < 2.0 / GRID


def test_emitted_token_law_is_target_row():
    """Law of the first emitted token, integrated over the draft and both uniforms."""
    rng = np.random.default_rng(11)
    for V in (2, 3, 6):
        p = _rows(rng, V, 2, zero_frac=0.2)
        q = _rows(rng, V, 1, zero_frac=0.2)
        law = np.zeros(V)
        for x in range(V):
            if q[0, x] == 0:
                continue
            acc = np.mean([_core(q, [x], p, [u], 0.5)["L"] == 1 for u in UGRID])
            law[x] += q[0, x] * acc
            if acc < 1.0:
                # a rejecting uniform for this x: the largest on the grid
                ys = [_core(q, [x], p, [UGRID[-1]], uf)["tokens"][0] for uf in UGRID]
                law += q[0, x] * (1.0 - acc) * np.bincount(ys, minlength=V) / GRID
        np.testing.assert_allclose(law, p[0].astype(np.float64), atol=4.0 / GRID)


def test_bonus_law_is_last_target_row():
    rng = np.random.default_rng(12)
    V, D = 4, 2
    p = _rows(rng, V, D + 1)
    q = p[:D].copy()
    x = [1, 2]
    ys = [_core(q, x, p, [0.9, 0.9], uf)["tokens"] for uf in UGRID]
    assert all(list(t[:D]) == x for t in ys)
    law = np.bincount([t[D] for t in ys], minlength=V) / GRID
    np.testing.assert_allclose(law, p[D], atol=2.0 / GRID)


def test_equal_rows_always_accept():
    rng = np.random.default_rng(13)
    V, D = 50, 4
    p = _rows(rng, V, D + 1)
    for s in range(200):
        x = rng.integers(0, V, size=D)
        ua, uf, code = chain_uniforms(s, 7 * s, D)
        out = chain_reject_core(p[:D], x, p, ua, uf, code)
        assert out["L"] == D and list(out["tokens"][:D]) == list(x)


def test_disjoint_supports_reject_first_and_draw_from_target():
    rng = np.random.default_rng(14)
    V, D = 8, 3
    p = _rows(rng, V, D + 1)
    p[:, 4:] = 0
    p /= p.sum(-1, keepdims=True)
    q = _rows(rng, V, D)
    q[:, :4] = 0
    q /= q.sum(-1, keepdims=True)
    ys = []
    for s in range(400):
        x = rng.integers(4, 8, size=D)
        ua, uf, code = chain_uniforms(1000 + s, 0, D)
        out = chain_reject_core(q, x, p, ua, uf, code)
        assert out["L"] == 0 and list(out["tokens"][1:]) == [-1] * D
        ys.append(out["tokens"][0])
    assert set(ys) <= {0, 1, 2, 3}


def test_invalid_ids_reject_at_their_position():
    rng = np.random.default_rng(15)
    V, D = 16, 4
    p = _rows(rng, V, D + 1)
    for bad in (-1, V, 2 ** 31 - 1, -(2 ** 31)):
        for pos in range(D):
            x = np.array([3, 4, 5, 6])
            x[pos] = bad
            ua, uf, code = chain_uniforms(5, 9, D)
            out = chain_reject_core(p[:D], x, p, ua, uf, code)      # q = p: valid ids accept
            assert out["L"] == pos
            assert 0 <= out["tokens"][pos] < V


def test_zero_residual_falls_back_to_target_then_uniform():
    V = 10
    p = np.zeros((2, V), np.float32)
    p[0, 3] = 0.25
    p[0, 7] = 0.75
    # reject forced by an invalid id; residual max(0, p - q) with q = p is empty -> draws from p
    ys = [_core(p[:1], [-1], p, [0.5], uf)["tokens"][0] for uf in UGRID]
    law = np.bincount(ys, minlength=V) / GRID
    np.testing.assert_allclose(law, p[0], atol=1.0 / GRID)
    # all-zero target row: uniform index floor(u * V), exact from the uniform's code
    z = np.zeros((2, V), np.float32)
    for code in (1, 3, 2 ** 23 + 1, 2 ** 24 - 1):
        y, margin = residual_draw(np.zeros(V), np.zeros(V), code * 2.0 ** -24, code)
        assert y == (code * V) >> 24 and 0 <= y < V and margin == math.inf
    out = chain_reject_core(z[:1], np.array([2]), z, np.array([0.3]), 0.999, 2 ** 24 - 1)
    assert out["L"] == 0 and out["tokens"][0] == V - 1


def test_monte_carlo_through_philox_streams():
    """Law of L and of the emitted tokens over seeds; catches stream-layout mistakes."""
    rng = np.random.default_rng(16)
    V, D, trials = 6, 3, 30000
    p = _rows(rng, V, D + 1, zero_frac=0.2)
    q = _rows(rng, V, D, zero_frac=0.2)
    alpha = np.minimum(p[:D], q[:D]).astype(np.float64).sum(-1)
    Ls = np.empty(trials, int)
    first = np.empty(trials, int)
    toks = np.empty((trials, D + 1), int)
    qc = np.cumsum(q.astype(np.float64), -1)
    for t in range(trials):
        x = np.array([min(int(np.searchsorted(qc[i], rng.random() * qc[i, -1], side="right")), V - 1)
                      for i in range(D)])
        ua, uf, code = chain_uniforms(t, (t * 2654435761) & (2 ** 64 - 1), D)
        out = chain_reject_core(q, x, p, ua, uf, code)
        Ls[t] = out["L"]
        first[t] = out["tokens"][0]
        toks[t] = out["tokens"]
    # P(L >= j) = prod_{i<j} alpha_i
    for j in range(1, D + 1):
        want = np.prod(alpha[:j])
        got = np.mean(Ls >= j)
        assert abs(got - want) < 5 * np.sqrt(want * (1 - want) / trials) + 1e-3, (j, got, want)
    assert abs(Ls.mean() - sum(np.prod(alpha[:j]) for j in range(1, D + 1))) < 0.03
    # emitted token at position j (given L >= j) ~ p_j : chi-square
    for j in range(D + 1):
        sel = Ls >= j
        obs = np.bincount(toks[sel, j], minlength=V).astype(float)
        exp = p[j].astype(np.float64) * sel.sum()
        m = exp > 5
        chi2 = ((obs[m] - exp[m]) ** 2 / exp[m]).sum()
        assert chi2 < 30, (j, chi2)                       # < 1e-4 tail for <= 5 dof
        assert obs[~m].sum() < 5 + 5 * np.sqrt(exp[~m].sum() + 1)


def test_batch_form_layout_and_request_subset():
    rng = np.random.default_rng(17)
    B, D, V = 5, 2, 30
    p = _rows(rng, V, B * (D + 1)).reshape(B, D + 1, V)
    q = _rows(rng, V, B * D).reshape(B, D, V)
    x = rng.integers(0, V, size=(B, D)).astype(np.int32)
    seed = np.arange(B, dtype=np.uint64) + np.uint64(77)
    off = np.arange(B, dtype=np.uint64) * np.uint64(4096)
    full = chain_reject(q, x, p, seed, off)
    sub = chain_reject(q, x, p, seed, off, requests=[3, 1])
    for b in (1, 3):
        assert np.array_equal(full["accepted_tokens"][b], sub["accepted_tokens"][b])
    assert np.all(sub["accepted_tokens"][[0, 2, 4]] == -2)
    for b in range(B):
        L = full["accept_length"][b]
        row = full["accepted_tokens"][b]
        assert 0 <= L <= D
        assert list(row[:L]) == list(x[b, :L]) and np.all(row[L + 1:] == -1) and 0 <= row[L] < V


def test_inverse_cdf_exact_boundary_convention():
    """token = min{j : C_j > u R}: a uniform landing exactly on C_j moves past j,
    and zero-mass tokens are never drawn (dyadic weights make the sums exact)."""
    e = 2.0 ** -24
    y, _ = residual_draw(np.array([e, 1 - e]), np.zeros(2), 1 * e, 1)
    assert y == 1
    y, _ = residual_draw(np.array([3 * e, 0.0, 1 - 3 * e]), np.zeros(3), 3 * e, 3)
    assert y == 2
    y, _ = residual_draw(np.array([0.0, 0.25, 0.0, 0.75]), np.zeros(4), e, 1)
    assert y == 1


def test_target_only_first_token_law_is_target_row():
    """Point-mass drafts (no draft probabilities): for a fixed draft id the
    first emitted token follows p_0 exactly (accept x w.p. p_0(x), otherwise
    draw from p_0 without x), and the accept rate at position 0 is p_0(x)."""
    rng = np.random.default_rng(61)
    V, D, trials = 6, 2, 30000
    p = _rows(rng, V, D + 1, zero_frac=0.1)[None]
    x = np.array([[2, 4]], np.int32)
    first = np.zeros(V)
    acc0 = 0
    for t in range(trials):
        out = chain_reject(None, x, p, np.array([t + 1], np.uint64), np.array([(7 * t) & 0xFFFF], np.uint64))
        first[out["accepted_tokens"][0, 0]] += 1
        acc0 += out["accept_length"][0] >= 1
    exp = p[0, 0].astype(np.float64) * trials
    m = exp > 5
    chi2 = ((first[m] - exp[m]) ** 2 / exp[m]).sum()
    assert chi2 < 25, (chi2, first, exp)
    pa = float(p[0, 0, 2])
    assert abs(acc0 / trials - pa) < 5 * np.sqrt(pa * (1 - pa) / trials) + 1e-3


def test_target_only_is_the_one_hot_draft_case():
    rng = np.random.default_rng(62)
    B, D, V = 8, 3, 40
    p = np.stack([_rows(rng, V, D + 1) for _ in range(B)])
    x = rng.integers(-2, V + 2, (B, D)).astype(np.int32)
    seed = rng.integers(1, 2 ** 40, B).astype(np.uint64)
    off = rng.integers(0, 2 ** 20, B).astype(np.uint64)
    a = chain_reject(None, x, p, seed, off)
    # acceptance at position i is exactly u_i < p_i(x_i) for a valid id
    for b in range(B):
        ua, _, _ = chain_uniforms(int(seed[b]), int(off[b]), D)
        L = 0
        while L < D and 0 <= x[b, L] < V and ua[L] < p[b, L, x[b, L]]:
            L += 1
        assert a["accept_length"][b] == L
        if L < D and 0 <= x[b, L] < V:
            assert a["accepted_tokens"][b, L] != x[b, L] or p[b, L, x[b, L]] > 1.0


def test_draw_margin_worked_example():
    """The margin is the distance of u to the two CDF values bracketing the token."""
    r = np.array([0.25, 0.5, 0.25])
    y, m = residual_draw(r, r, 0.3, 1)
    assert y == 1 and abs(m - 0.05) < 1e-15
    y, m = residual_draw(r, r, 0.74, 1)
    assert y == 1 and abs(m - 0.01) < 1e-15
    # u exactly on a boundary: the token moves past it and the margin is 0
    y, m = residual_draw(r, r, 0.25, 1)
    assert y == 1 and m == 0.0


def _orders(r):
    """Prefix sums and totals of r in four association orders: sequential,
    blocked (per-1024 block sums, then a running sum of blocks), pairwise
    (numpy's reduction inside blocks of 64) and reversed-within-block."""
    V = r.size
    seq = np.cumsum(r)
    out = [(seq, seq[-1])]
    for blk in (1024, 64):
        n = (V + blk - 1) // blk
        pad = np.zeros(n * blk)
        pad[:V] = r
        tiles = pad.reshape(n, blk)
        sums = tiles.sum(axis=1)                        # pairwise inside a tile
        base = np.concatenate([[0.0], np.cumsum(sums)[:-1]])
        pre = (base[:, None] + np.cumsum(tiles, axis=1)).reshape(-1)[:V]
        out.append((pre, float(np.cumsum(sums)[-1])))
    rev = np.cumsum(r[::-1])[::-1]                       # suffix sums, converted to prefixes
    tot = float(rev[0])
    out.append((tot - np.concatenate([rev[1:], [0.0]]), tot))
    return out


def test_cdf_sum_band_covers_summation_order():
    """The exclusion band is a real bound: across association orders the
    normalised CDF values C_j / R never differ by more than a quarter of
    cdf_sum_band(V) (the band keeps a factor 2 over the two-sided bound),
    on row shapes with the largest rounding: many tiny weights behind a
    large one, Zipf rows and rows with exact zeros."""
    from oracle import cdf_sum_band
    rng = np.random.default_rng(91)
    for V in (1000, 32000, 128256):
        rows = [rng.random(V) ** 6,
                np.concatenate([[1.0], rng.random(V - 1) * 1e-12]),
                1.0 / np.arange(1, V + 1) ** 1.1]
        z = rng.random(V)
        z[rng.random(V) < 0.5] = 0.0
        rows.append(z)
        band = cdf_sum_band(V)
        for r in rows:
            r = r.astype(np.float32).astype(np.float64)
            ref, rt = _orders(r)[0]
            for pre, tot in _orders(r)[1:]:
                d = np.max(np.abs(pre / tot - ref / rt))
                assert d <= band / 4, (V, d, band)
    # the band grows with V: a constant band would be wrong for long rows
    assert cdf_sum_band(2 ** 20) > 100 * cdf_sum_band(1000)


def test_cdf_exclusion_band_is_sufficient_against_another_order():
    """A draw outside the exclusion band gives the same token under a
    different summation order (blocked sums, as an implementation that sums
    per tile would form them); only draws inside the band may differ."""
    from oracle import cdf_sum_band
    rng = np.random.default_rng(92)
    V = 4096
    band = cdf_sum_band(V)
    differ = 0
    scale = V * 2.0 ** -53                      # the size of a worst-case summation error
    for t in range(300):
        r = (rng.random(V) ** 8).astype(np.float32).astype(np.float64)
        tot_seq = np.cumsum(r)
        # uniforms placed right at a boundary, then nudged by multiples of that size
        j = int(rng.integers(0, V))
        for k in (-8, -2, -0.5, -0.05, -0.005, 0.0, 0.005, 0.05, 0.5, 2, 8):
            u = float(np.clip(tot_seq[j] / tot_seq[-1] + k * scale, 1e-12, 1 - 1e-12))
            y, m = residual_draw(r, r, u, 1)
            pre, tot = _orders(r)[1]
            y2 = int(np.searchsorted(pre, u * tot, side="right"))
            y2 = min(y2, V - 1)
            if y2 != y:
                differ += 1
                assert m < band, (t, k, m, band)
    print(f"draws that another order changes: {differ} (all inside the band)")
