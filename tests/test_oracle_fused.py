"""Pins for the oracle's fused target-rows + chain rejection call (CPU only).

* Reductions to other pinned definitions: at temperature below the greedy
  threshold, and with top-k = 1 on untied logits, every target row is one-hot,
  so the fused call must give the greedy verify's tokens and accept lengths.
* Closed form: draft probabilities equal to the renormalised target rows
  accept every draft (u * q < q for u < 1).
* Law: over Philox streams, the first emitted token follows the renormalised
  target row 0 (top-k and top-p applied), not the plain softmax.
"""
import numpy as np

from oracle import chain_uniforms, greedy_verify, renorm_row, verify_fused


def _case(rng, B, D, V, scale=2.0):
    z = (rng.standard_normal((B, D + 1, V)) * scale).astype(np.float32)
    q = rng.random((B, D, V)) ** 2
    q = (q / q.sum(-1, keepdims=True)).astype(np.float32)
    seed = rng.integers(0, 2 ** 63, B, dtype=np.int64).astype(np.uint64)
    off = rng.integers(0, 2 ** 40, B, dtype=np.int64).astype(np.uint64)
    return z, q, seed, off


def _planted_drafts(rng, z, match=0.7):
    B, N, V = z.shape
    y = z.argmax(-1)[:, :N - 1]
    x = np.where(rng.random(y.shape) < match, y, rng.integers(0, V, y.shape))
    return x.astype(np.int32)


def test_greedy_rows_reduce_to_greedy_verify():
    rng = np.random.default_rng(41)
    B, D, V = 40, 4, 37
    z, q, seed, off = _case(rng, B, D, V)
    x = _planted_drafts(rng, z)
    g = greedy_verify(z, "f32", x)
    for T, k in ((0.0, 0), (1e-6, 0), (0.8, 1), (1.7, 1)):
        tp = np.full(B, 0.9, np.float32)
        f = verify_fused(z, "f32", np.full(B, T, np.float32), np.full(B, k, np.int32), tp, q, x, seed, off)
        assert np.array_equal(f["accept_length"], g["accept_length"]), (T, k)
        assert np.array_equal(f["accepted_tokens"], g["accepted_tokens"]), (T, k)
        assert np.all(f["flag_pos"] == D + 1)


def test_drafts_equal_to_target_rows_accept_everything():
    rng = np.random.default_rng(42)
    B, D, V = 12, 3, 50
    z, _, seed, off = _case(rng, B, D, V)
    T = rng.uniform(0.5, 1.5, B).astype(np.float32)
    k = rng.choice([0, 5, 20], B).astype(np.int32)
    tp = rng.choice([1.0, 0.9, 0.7], B).astype(np.float32)
    q = np.zeros((B, D, V), np.float32)
    x = np.zeros((B, D), np.int32)
    for b in range(B):
        for i in range(D):
            p, _ = renorm_row(z[b, i], float(T[b]), int(k[b]), float(tp[b]))
            q[b, i] = p.astype(np.float32)
            x[b, i] = int(np.argmax(p))
    # float32 q may round above the float64 target: compare with the margin the product needs
    f = verify_fused(z, "f32", T, k, tp, q, x, seed, off)
    for b in range(B):
        ok = all(q[b, i, x[b, i]] <= renorm_row(z[b, i], float(T[b]), int(k[b]), float(tp[b]))[0][x[b, i]]
                 for i in range(D))
        if ok:
            assert f["accept_length"][b] == D
            pD, _ = renorm_row(z[b, D], float(T[b]), int(k[b]), float(tp[b]))
            assert pD[f["accepted_tokens"][b, D]] > 0


def test_first_token_law_is_renormalised_target_row():
    rng = np.random.default_rng(43)
    V, D, trials = 7, 2, 12000
    z = np.array([[2.0, 1.5, 1.4, 0.3, -1.0, 0.9, 1.1],
                  [0.5, 0.1, 1.2, -0.4, 0.8, 0.0, 0.6],
                  [1.0, 0.9, 0.8, 0.7, 0.6, 0.5, 0.4]], np.float32)[None]
    T, k, tp = 0.9, 4, 0.8
    p0, _ = renorm_row(z[0, 0], T, k, tp)
    assert np.count_nonzero(p0) < V          # the filters bite: plain softmax would differ
    q = np.full((1, D, V), 1.0 / V, np.float32)
    first = np.zeros(V)
    for t in range(trials):
        x = rng.integers(0, V, (1, D)).astype(np.int32)
        out = verify_fused(z, "f32", np.array([T], np.float32), np.array([k], np.int32),
                           np.array([tp], np.float32), q, x,
                           np.array([t], np.uint64), np.array([(t * 2654435761) & (2 ** 63 - 1)], np.uint64))
        first[out["accepted_tokens"][0, 0]] += 1
    exp = p0 * trials
    m = exp > 0
    chi2 = ((first[m] - exp[m]) ** 2 / exp[m]).sum()
    assert chi2 < 25, (chi2, first, exp)
    assert first[~m].sum() == 0


def test_only_rows_up_to_the_rejection_matter():
    """Rows after position L never change the outputs (they are not read)."""
    rng = np.random.default_rng(44)
    B, D, V = 30, 5, 40
    z, q, seed, off = _case(rng, B, D, V)
    x = rng.integers(0, V, (B, D)).astype(np.int32)
    T = np.full(B, 1.0, np.float32)
    k = np.zeros(B, np.int32)
    tp = np.ones(B, np.float32)
    a = verify_fused(z, "f32", T, k, tp, q, x, seed, off)
    z2 = z.copy()
    for b in range(B):
        z2[b, a["accept_length"][b] + 1:] = rng.standard_normal((D - a["accept_length"][b], V))
    c = verify_fused(z2, "f32", T, k, tp, q, x, seed, off)
    assert np.array_equal(a["accepted_tokens"], c["accepted_tokens"])
    # and the accept tests use the same uniforms as the two-call form
    ua, uf, code = chain_uniforms(int(seed[0]), int(off[0]), D)
    assert ua.shape == (D,) and 0 < uf < 1 and code & 1
