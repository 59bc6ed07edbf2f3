"""Pins for the oracle's ragged chain rejection (CPU only).

* Reduction: when every request verifies all D + 1 positions the ragged form
  is the dense chain verify on the same rows.
* Law: at a request's own last position the padded one-hot rows make the
  emitted token follow that position's target row exactly (accept token 0
  with probability p(0), otherwise draw from p with token 0 removed), the
  argument the TensorRT-LLM page gives for its padding; checked by
  chi-square over Philox streams, together with the accept event itself.
* Clamp: no request emits more tokens than it verified; padding after the
  emitted tokens is -1; requests with an invalid length are marked -1.
"""
import numpy as np

from oracle import chain_reject, chain_reject_ragged, chain_uniforms


def _rows(rng, V, n, zero_frac=0.0):
    w = rng.random((n, V)) ** 3
    w[rng.random((n, V)) < zero_frac] = 0.0
    w[:, 0] += 1e-3
    return (w / w.sum(-1, keepdims=True)).astype(np.float32)


def _pack(p_dense, lens):
    """Packed rows and qo_indptr from a dense [B, D+1, V] batch and per-request lengths."""
    rows = np.concatenate([p_dense[b, :n] for b, n in enumerate(lens)], axis=0)
    ind = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return rows, ind


def test_full_length_reduces_to_dense():
    rng = np.random.default_rng(70)
    B, D, V = 7, 3, 50
    p = np.stack([_rows(rng, V, D + 1, 0.2) for _ in range(B)])
    q = np.stack([_rows(rng, V, D, 0.2) for _ in range(B)])
    x = rng.integers(-1, V + 1, (B, D)).astype(np.int32)
    seed = rng.integers(1, 2 ** 40, B).astype(np.uint64)
    off = rng.integers(0, 2 ** 20, B).astype(np.uint64)
    rows, ind = _pack(p, [D + 1] * B)
    for qq in (q, None):
        a = chain_reject(qq, x, p, seed, off)
        r = chain_reject_ragged(qq, x, rows, ind, seed, off)
        assert np.array_equal(a["accepted_tokens"], r["accepted_tokens"])
        assert np.array_equal(a["accept_length"], r["accept_length"])


def test_request_local_bonus_follows_its_target_row():
    """len = 1 (no drafts verified): the one emitted token follows p_0, and it
    is token 0 exactly when the position's accept uniform falls below p_0(0).
    len = 2 with q_0 = p_0 (always accepted): position 1's token follows p_1."""
    rng = np.random.default_rng(71)
    V, D, trials = 6, 3, 30000
    p = _rows(rng, V, D + 1, 0.15)
    p[:, 0] = np.float32(0.2)
    p = (p / p.sum(-1, keepdims=True)).astype(np.float32)
    q = _rows(rng, V, D, 0.1)
    q[0] = p[0]
    for n, pos in ((1, 0), (2, 1)):
        rows, ind = _pack(p[None], [n])
        x = np.array([[3, 1, 2]], np.int32)
        if n == 2:
            x[0, 0] = 4                       # q_0 = p_0: always accepted
        first = np.zeros(V)
        for t in range(trials):
            seed = np.array([t + 11], np.uint64)
            off = np.array([(13 * t) & 0xFFFFF], np.uint64)
            out = chain_reject_ragged(q[None], x, rows, ind, seed, off)
            assert out["accept_length"][0] == pos
            tok = out["accepted_tokens"][0]
            assert np.all(tok[pos + 1:] == -1)
            first[tok[pos]] += 1
            ua, _, _ = chain_uniforms(int(seed[0]), int(off[0]), D)
            assert (tok[pos] == 0) == (ua[pos] < p[pos, 0]), (t, tok, ua[pos], p[pos, 0])
        exp = p[pos].astype(np.float64) * trials
        m = exp > 5
        chi2 = ((first[m] - exp[m]) ** 2 / exp[m]).sum()
        assert chi2 < 30, (n, chi2, first, exp)


def test_clamp_padding_and_invalid_lengths():
    rng = np.random.default_rng(72)
    B, D, V = 40, 4, 30
    lens = rng.integers(1, D + 2, B)
    p = np.stack([_rows(rng, V, D + 1, 0.2) for _ in range(B)])
    q = np.stack([_rows(rng, V, D, 0.2) for _ in range(B)])
    # drafts mostly at the target's mode so that long acceptances happen
    x = np.where(rng.random((B, D)) < 0.7, p[:, :D].argmax(-1), rng.integers(0, V, (B, D))).astype(np.int32)
    rows, ind = _pack(p, lens)
    seed = rng.integers(1, 2 ** 40, B).astype(np.uint64)
    off = rng.integers(0, 2 ** 20, B).astype(np.uint64)
    for qq in (q, None):
        out = chain_reject_ragged(qq, x, rows, ind, seed, off)
        for b in range(B):
            L = out["accept_length"][b]
            t = out["accepted_tokens"][b]
            assert 0 <= L <= lens[b] - 1
            assert np.array_equal(t[:L], x[b, :L])
            assert 0 <= t[L] < V
            assert np.all(t[L + 1:] == -1)
    # lengths 0 and D + 2, and rows past the packed array, are invalid
    bad = ind.copy()
    bad[1] = bad[0]                          # request 0: length 0
    bad[3] = bad[2] + D + 2                  # request 2: length D + 2
    bad[-1] = rows.shape[0] + 1              # last request: past the end
    out = chain_reject_ragged(q, x, rows, bad, seed, off)
    for b in (0, 2, B - 1):
        assert out["accept_length"][b] == -1 and np.all(out["accepted_tokens"][b] == -1)


def test_d2t_expand_placement_and_mass():
    """Draft -> target placement: with a zero table and equal vocabularies it
    is the identity; otherwise every draft entry lands at (s + d2t[s]) mod V
    (negative offsets wrap as a floor modulus), every other target entry is
    zero, and each row keeps its mass."""
    from oracle import d2t_expand
    rng = np.random.default_rng(73)
    q = _rows(rng, 8, 6)
    assert np.array_equal(d2t_expand(q, np.zeros(8, np.int64), 8), q)
    assert np.array_equal(d2t_expand(q, None, 8), q)
    # a hand-worked table: V = 11, draft ids 0..7 at targets 3, 4, 10, 0, 1, 5, 6, 9
    d2t = np.array([3, 3, 8, -3, -3, 0, 0, 2], np.int64)
    want = [3, 4, 10, 0, 1, 5, 6, 9]
    out = d2t_expand(q, d2t, 11)
    for s_, t in enumerate(want):
        assert np.array_equal(out[:, t], q[:, s_])
    others = np.setdiff1d(np.arange(11), want)
    assert np.all(out[:, others] == 0)
    assert np.allclose(out.astype(np.float64).sum(-1), q.astype(np.float64).sum(-1), rtol=0, atol=1e-12)
    # without a table the draft vocabulary is the first Vd target entries
    out = d2t_expand(q, None, 11)
    assert np.array_equal(out[:, :8], q) and np.all(out[:, 8:] == 0)


def test_d2t_shared_targets_keep_the_last_draft_entry():
    """A table that sends several draft entries to one target: the target
    holds the highest-numbered of them (computed here with np.maximum.at on
    the draft index, independently of the oracle's scatter), every other
    target holds its unique entry or 0."""
    from oracle import d2t_expand
    rng = np.random.default_rng(74)
    for Vd, V in ((50, 60), (200, 200), (7, 5)):
        tgt = rng.integers(0, V, Vd)                       # collisions certain at these sizes
        d2t = (tgt - np.arange(Vd)).astype(np.int64)      # (s + d2t[s]) mod V = tgt[s]
        if Vd == 7:
            d2t = d2t - 3 * V                              # negative offsets wrap (floor modulus)
        q = rng.random((3, Vd)).astype(np.float32)
        out = d2t_expand(q, d2t, V)
        winner = np.full(V, -1, np.int64)
        np.maximum.at(winner, tgt, np.arange(Vd))
        want = np.where(winner >= 0, q[:, np.maximum(winner, 0)], 0.0).astype(np.float32)
        assert np.array_equal(out, want), (Vd, V)
