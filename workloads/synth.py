"""Seeded generators for the five verification workloads and for fuzz shapes.

Every array is produced from ``numpy.random.Generator(PCG64(SeedSequence([cfg,
replica])))`` in a fixed order (workloads 3 and 5 draw each request's rows from
its own stream ``SeedSequence([cfg, replica, b])``, so requests can be
generated in parallel), so a (cfg, replica) pair names one input set.
Logits are drawn in float32 and stored as float32 or as bfloat16 bit patterns
(uint16, round-to-nearest-even from float32).  Draft token ids are drawn from
the draft distribution by inverse CDF on float64 weights with the data RNG; this
randomness is independent of the Philox streams the verification path uses.

Workloads (B requests, D draft tokens, N = D + 1 verified positions, V vocab):

1. tiny: B=4 D=3 V=1000, float32 logits ~ N(0, 2), temperature 1; draft
   distribution = normalised exp(z + N(0, 0.5)); greedy draft ids equal the
   row argmax with probability 0.7, else uniform.  Philox seed_b = b, offset 0.
2. top-k/top-p: B=64 D=3 V=32000, bf16 logits ~ N(0, 3) plus 8 on a
   Bernoulli(0.01) mask; T=0.7, top_k=50, top_p=0.9 for every request; draft
   distribution = normalised exp(z + N(0, 0.3)) (unfiltered, temperature 1).
3. large-vocab rejection: B=256 D=5 V=128256, float32 target probabilities
   from a Zipf law (weight r**-1.1 over ranks r = 1..V placed at a fresh random
   permutation per row); draft rows = target row times exp(N(0, 0.4)) per
   entry, renormalised (a N(0, 0.4) logit-space perturbation).
4. greedy: B=512 D=3 V=151936, bf16 logits ~ N(0, 2) with one planted maximum
   per row (max of the row + 6, at a uniform position); draft ids equal the
   planted position with probability 0.8, else uniform.
5. mixed: B=1024 D=7 V=129280, bf16 logits ~ N(0, 2.5); a seeded permutation
   gives exactly B/4 requests to each mode: greedy (T=0), temperature-only,
   top-k (k in {20, 100}) and top-p (top_p ~ U[0.8, 0.95]), with T ~ U[0.5, 1.2]
   for non-greedy requests.  Draft distributions for non-greedy requests are
   normalised exp((z + N(0, 0.3)) / T), unfiltered; greedy requests draw draft
   ids like workload 4 (the row's largest logit with probability 0.8).
"""
from __future__ import annotations

import numpy as np

CONFIGS = {
    1: dict(workload="tiny_chain_and_greedy", B=4, D=3, V=1000),
    2: dict(workload="topk_topp_chain", B=64, D=3, V=32000),
    3: dict(workload="large_vocab_chain_reject", B=256, D=5, V=128256),
    4: dict(workload="greedy_chain_verify", B=512, D=3, V=151936),
    5: dict(workload="mixed_modes_gumbel", B=1024, D=7, V=129280),
}

MODE_GREEDY, MODE_TEMPERATURE, MODE_TOPK, MODE_TOPP = 0, 1, 2, 3


def data_rng(cfg: int, replica: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg, replica])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1).view(np.uint32)
    out = np.empty(flat.shape, np.uint16)
    step = 1 << 22
    for i in range(0, flat.size, step):
        b = flat[i:i + step]
        t = b >> np.uint32(16)
        t &= np.uint32(1)
        t += np.uint32(0x7FFF)
        t += b                      # finite values and infinities stay below 2**32
        t >>= np.uint32(16)
        out[i:i + step] = t
        nan = (b & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
        if nan.any():
            out[i:i + step][nan] = np.uint16(0x7FC0)
    return out.reshape(x.shape)


def bf16_bits_to_f32(u16: np.ndarray) -> np.ndarray:
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normalised(w: np.ndarray) -> np.ndarray:
    """Rows of non-negative weights scaled to sum to one (float64)."""
    return w / w.sum(axis=-1, keepdims=True)


def _exp_weights(z: np.ndarray) -> np.ndarray:
    """exp(z - rowmax) in float64, the synthetic draft model's unnormalised weights."""
    z = np.asarray(z, dtype=np.float64)
    return np.exp(z - z.max(axis=-1, keepdims=True))


def _draw_from_rows(rng: np.random.Generator, w: np.ndarray) -> np.ndarray:
    """One index per row of ``w`` (float64 weights), by inverse CDF with the data RNG."""
    rows = w.reshape(-1, w.shape[-1])
    out = np.empty(rows.shape[0], dtype=np.int32)
    for i, row in enumerate(rows):
        c = np.cumsum(row)
        t = rng.random() * c[-1]
        out[i] = min(int(np.searchsorted(c, t, side="right")), row.shape[0] - 1)
    return out.reshape(w.shape[:-1])


def _seeds(cfg: int, B: int) -> np.ndarray:
    return (np.uint64(cfg) << np.uint64(32)) + np.arange(B, dtype=np.uint64)


def _cfg1(rng, replica):
    B, D, V = 4, 3, 1000
    z = (rng.standard_normal((B, D + 1, V)) * 2.0).astype(np.float32)
    noise = rng.standard_normal((B, D, V)) * 0.5
    q = _normalised(_exp_weights(z[:, :D].astype(np.float64) + noise))
    x = _draw_from_rows(rng, q)
    am = np.argmax(z[:, :D], axis=-1).astype(np.int32)
    keep = rng.random((B, D)) < 0.7
    xg = np.where(keep, am, rng.integers(0, V, size=(B, D))).astype(np.int32)
    return dict(
        dtype="f32", logits=z, temperature=np.ones(B, np.float32),
        top_k=np.zeros(B, np.int32), top_p=np.ones(B, np.float32),
        draft_probs=q.astype(np.float32), draft_ids=x, greedy_draft_ids=xg,
        seed=np.arange(B, dtype=np.uint64), offset=np.zeros(B, np.uint64),
    )


def _cfg2(rng, replica):
    B, D, V = 64, 3, 32000
    z = rng.standard_normal((B, D + 1, V), dtype=np.float32) * np.float32(3.0)
    z += np.where(rng.random((B, D + 1, V)) < 0.01, np.float32(8.0), np.float32(0.0))
    zb = f32_to_bf16_bits(z)
    zd = bf16_bits_to_f32(zb).astype(np.float64)
    noise = rng.standard_normal((B, D, V)) * 0.3
    q = _normalised(_exp_weights(zd[:, :D] + noise))
    x = _draw_from_rows(rng, q)
    return dict(
        dtype="bf16", logits=zb, temperature=np.full(B, 0.7, np.float32),
        top_k=np.full(B, 50, np.int32), top_p=np.full(B, 0.9, np.float32),
        draft_probs=q.astype(np.float32), draft_ids=x,
        seed=_seeds(2, B), offset=np.full(B, 4096 * replica, np.uint64),
    )


def _cfg3(rng, replica, B=256):
    D, V = 5, 128256
    zipf = np.arange(1, V + 1, dtype=np.float64) ** -1.1
    zipf /= zipf.sum()
    p = np.empty((B, D + 1, V), np.float32)
    q = np.empty((B, D, V), np.float32)
    x = np.empty((B, D), np.int32)
    base = np.arange(V)

    def one(b):
        r = _request_rng(3, replica, b)
        perms = r.permuted(np.broadcast_to(base, (D + 1, V)), axis=1)
        pb = zipf[perms]
        p[b] = pb
        qb = _normalised(pb[:D] * np.exp(r.standard_normal((D, V)) * 0.4))
        q[b] = qb
        x[b] = _draw_from_rows(r, qb)

    _parallel_rows(B, one)
    return dict(
        dtype="f32", target_probs=p, draft_probs=q, draft_ids=x,
        temperature=np.ones(B, np.float32),
        seed=_seeds(3, B), offset=np.full(B, 4096 * replica, np.uint64),
    )


def _planted_logits(rng, rows, V, sigma, chunk=128):
    """bf16 logits ~ N(0, sigma) with one planted strict maximum per row."""
    zb = np.empty((rows, V), np.uint16)
    pos = rng.integers(0, V, size=rows)
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        z = rng.standard_normal((r1 - r0, V), dtype=np.float32)
        z *= np.float32(sigma)
        zc = f32_to_bf16_bits(z)
        top = bf16_bits_to_f32(zc).max(axis=1) + np.float32(6.0)
        zc[np.arange(r1 - r0), pos[r0:r1]] = f32_to_bf16_bits(top.astype(np.float32))
        zb[r0:r1] = zc
    return zb, pos.astype(np.int32)


def _cfg4(rng, replica, B=512):
    D, V = 3, 151936
    zb, pos = _planted_logits(rng, B * (D + 1), V, 2.0)
    zb = zb.reshape(B, D + 1, V)
    pos = pos.reshape(B, D + 1)
    keep = rng.random((B, D)) < 0.8
    x = np.where(keep, pos[:, :D], rng.integers(0, V, size=(B, D))).astype(np.int32)
    return dict(dtype="bf16", logits=zb, draft_ids=x, planted=pos)


def _request_rng(cfg: int, replica: int, b: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg, replica, b])))


def _parallel_rows(n: int, fn, threads: int | None = None):
    """Run fn(b) for b in range(n) on a thread pool (numpy releases the GIL)."""
    import concurrent.futures
    import os
    threads = threads or min(16, os.cpu_count() or 1)
    with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(fn, range(n)))


def _cfg5(rng, replica, B=1024):
    D, V = 7, 129280
    N = D + 1
    modes = np.empty(B, np.int32)
    perm = rng.permutation(B)
    for m in range(4):
        modes[perm[m * (B // 4):(m + 1) * (B // 4)]] = m
    T = rng.uniform(0.5, 1.2, size=B).astype(np.float32)
    T[modes == MODE_GREEDY] = 0.0
    top_k = np.where(modes == MODE_TOPK, rng.choice([20, 100], size=B), 0).astype(np.int32)
    top_p = np.where(modes == MODE_TOPP, rng.uniform(0.8, 0.95, size=B), 1.0).astype(np.float32)
    zb = np.empty((B, N, V), np.uint16)
    q = np.zeros((B, D, V), np.float32)
    x = np.empty((B, D), np.int32)

    def one(b):
        r = _request_rng(5, replica, b)
        z = r.standard_normal((N, V), dtype=np.float32)
        z *= np.float32(2.5)
        zb[b] = f32_to_bf16_bits(z)
        zd = bf16_bits_to_f32(zb[b])
        if modes[b] == MODE_GREEDY:
            am = np.argmax(zd[:D], axis=-1)
            keep = r.random(D) < 0.8
            x[b] = np.where(keep, am, r.integers(0, V, size=D))
        else:
            a = zd[:D] + r.standard_normal((D, V), dtype=np.float32) * np.float32(0.3)
            a *= np.float32(1.0 / float(T[b]))
            a -= a.max(axis=-1, keepdims=True)
            w = np.exp(a)
            w /= w.sum(axis=-1, keepdims=True, dtype=np.float64).astype(np.float32)
            q[b] = w
            x[b] = _draw_from_rows(r, w.astype(np.float64))

    _parallel_rows(B, one)
    return dict(
        dtype="bf16", logits=zb, temperature=T, top_k=top_k, top_p=top_p, modes=modes,
        draft_probs=q, draft_ids=x,
        seed=_seeds(5, B), offset=np.full(B, 4096 * replica, np.uint64),
    )


def make_config(cfg: int, replica: int = 0, **kw) -> dict:
    """Inputs of workload ``cfg`` (1..5), replica ``replica``; see module docstring."""
    rng = data_rng(cfg, replica)
    gen = {1: _cfg1, 2: _cfg2, 3: _cfg3, 4: _cfg4, 5: _cfg5}[cfg]
    out = gen(rng, replica, **kw)
    out.update(CONFIGS[cfg])
    if "B" in kw:
        out["B"] = kw["B"]
    return out


def make_ragged_config(replica: int = 0) -> dict:
    """The large-vocab inputs with per-request verify lengths: request b
    verifies len_b ~ U{1..D+1} positions (data RNG, independent of the rest),
    and its first len_b target rows are packed in request order
    (``target_rows`` [sum len, V], ``qo_indptr`` [B+1])."""
    out = make_config(3, replica)
    B, D = out["B"], out["D"]
    lens = data_rng(30, replica).integers(1, D + 2, B)
    out["verify_lens"] = lens
    out["qo_indptr"] = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    out["target_rows"] = np.ascontiguousarray(
        np.concatenate([out["target_probs"][b, :n] for b, n in enumerate(lens)], axis=0))
    return out


def make_ragged_d2t_config(replica: int = 0, Vd: int = 32000) -> dict:
    """The ragged large-vocab inputs with a draft model over a Vd-entry draft
    vocabulary: an ascending d2t table (``make_d2t``), draft rows = the
    config's draft rows at the mapped target ids, renormalised
    (``draft_probs_d`` [B, D, Vd]), and draft ids drawn from those rows (data
    RNG) and given as target ids."""
    out = make_ragged_config(replica)
    V = out["V"]
    d2t = make_d2t(0, Vd, V)
    tgt = (np.arange(Vd, dtype=np.int64) + d2t) % V
    qd = out["draft_probs"][:, :, tgt].astype(np.float64)
    qd /= qd.sum(axis=-1, keepdims=True)
    rng = data_rng(31, replica)
    out["d2t"] = d2t
    out["draft_probs_d"] = qd.astype(np.float32)
    out["draft_ids"] = tgt[_draw_from_rows(rng, qd)].astype(np.int32)
    return out


def make_sample_config(replica: int = 0, B: int = 1024, V: int = 129280) -> dict:
    """Single-step sampling rows at the mixed workload's shape: bf16 logits
    ~ N(0, 2.5) [B, V]; per row (data RNG) a quarter greedy (T = 0), the rest
    T ~ U[0.5, 1.2] with top_k in {0, 20, 100}, top_p 1 or U[0.8, 0.95] and
    min_p in {0, 0.05}; Philox seed_b = 6 * 2^32 + b."""
    rng = data_rng(6, replica)
    z = np.empty((B, V), np.uint16)
    for b0 in range(0, B, 128):
        blk = rng.standard_normal((min(128, B - b0), V), dtype=np.float32)
        blk *= np.float32(2.5)
        z[b0:b0 + blk.shape[0]] = f32_to_bf16_bits(blk)
    T = rng.uniform(0.5, 1.2, B).astype(np.float32)
    T[rng.random(B) < 0.25] = 0.0
    top_k = rng.choice([0, 20, 100], B).astype(np.int32)
    top_p = np.where(rng.random(B) < 0.5, rng.uniform(0.8, 0.95, B), 1.0).astype(np.float32)
    min_p = np.where(rng.random(B) < 0.5, 0.05, 0.0).astype(np.float32)
    return dict(dtype="bf16", logits=z, temperature=T, top_k=top_k, top_p=top_p, min_p=min_p,
                seed=_seeds(6, B), offset=np.full(B, 4096 * replica, np.uint64))


def make_d2t(seed: int, Vd: int, V: int, shuffled: bool = False) -> np.ndarray:
    """A one-to-one draft -> target offset table: draft id s maps to target id
    t_s = s + d2t[s] (mod V), the t_s a seeded sample of Vd distinct target
    ids, ascending (a reduced-vocabulary drafter keeps the target's order) or
    shuffled."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([2000, seed, Vd, V])))
    t = rng.choice(V, size=Vd, replace=False)
    if not shuffled:
        t = np.sort(t)
    return (t.astype(np.int64) - np.arange(Vd, dtype=np.int64))


def fuzz_case(seed: int, B: int, D: int, V: int, dtype: str = "f32", sigma: float = 2.0,
              draft_noise: float = 0.5, special: str | None = None) -> dict:
    """A small random case for parity fuzzing.

    ``special`` plants a degenerate structure: "ties" (logits on a coarse grid
    so rows hold repeated maxima), "zeros" (all-zero logits and probability
    rows), "onehot" (one-hot target and draft rows), "disjoint" (draft and
    target supports disjoint), "equal" (draft rows equal to target rows),
    "invalid_ids" (some draft ids outside [0, V)), "mostly_zero" (nine in ten
    logits exactly zero, so one value fills most of a row), "wide" (logits
    uniform over [-3e4, 3e4]), "signed_zeros" (logits drawn from -1, -0.0,
    +0.0 and 1).
    """
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([1000, seed, B, D, V])))
    N = D + 1
    z = rng.standard_normal((B, N, V)).astype(np.float32) * np.float32(sigma)
    if special == "ties":
        z = np.round(z).astype(np.float32)
    if special == "zeros":
        z = np.zeros_like(z)
    if special == "mostly_zero":
        z = np.where(rng.random(z.shape) < 0.9, np.float32(0.0), z).astype(np.float32)
    if special == "wide":
        z = rng.uniform(-3e4, 3e4, size=z.shape).astype(np.float32)
    if special == "signed_zeros":
        z = rng.choice(np.array([-1.0, -0.0, 0.0, 1.0], np.float32), size=z.shape, p=[0.3, 0.2, 0.2, 0.3])
    if dtype == "bf16":
        zs = f32_to_bf16_bits(z)
        zd = bf16_bits_to_f32(zs).astype(np.float64)
    else:
        zs = z
        zd = z.astype(np.float64)
    p = _normalised(_exp_weights(zd)).astype(np.float32)
    q64 = _normalised(_exp_weights(zd[:, :D] + rng.standard_normal((B, D, V)) * draft_noise)) \
        if D > 0 else np.zeros((B, 0, V))
    if special == "zeros":
        p = np.zeros_like(p)
    if special == "onehot":
        hot = rng.integers(0, V, size=(B, N))
        p = np.zeros((B, N, V), np.float32)
        p[np.arange(B)[:, None], np.arange(N)[None, :], hot] = 1.0
        hq = np.where(rng.random((B, D)) < 0.5, hot[:, :D], rng.integers(0, V, size=(B, D)))
        q64 = np.zeros((B, D, V))
        q64[np.arange(B)[:, None], np.arange(D)[None, :], hq] = 1.0
    if special == "disjoint" and V >= 2:
        half = V // 2
        pw = p.astype(np.float64)
        pw[..., half:] = 0.0
        p = _normalised(pw).astype(np.float32)
        qw = q64.copy()
        qw[..., :half] = 0.0
        q64 = _normalised(qw + 1e-300)
        q64[..., :half] = 0.0
    if special == "equal":
        q64 = p[:, :D].astype(np.float64)
    q = q64.astype(np.float32)
    if D > 0:
        x = _draw_from_rows(rng, np.maximum(q64, 0) + 1e-300)
    else:
        x = np.zeros((B, 0), np.int32)
    if special == "invalid_ids" and D > 0:
        bad = rng.random((B, D)) < 0.3
        x = np.where(bad, rng.choice([-1, V, V + 7, -(2 ** 31)], size=(B, D)), x).astype(np.int32)
    T = rng.uniform(0.3, 1.5, size=B).astype(np.float32)
    return dict(
        dtype=dtype, logits=zs, target_probs=p, draft_probs=q, draft_ids=x.astype(np.int32),
        temperature=T,
        seed=rng.integers(0, 2 ** 63, size=B, dtype=np.uint64) * np.uint64(2) + np.uint64(1),
        offset=rng.integers(0, 2 ** 40, size=B, dtype=np.uint64),
        B=B, D=D, V=V,
    )
