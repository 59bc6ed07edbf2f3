"""Plain CPU definitions of the verification path (numpy, float64).

TEST INFRASTRUCTURE: see the package docstring.

Sources (pages, by title and section):

* TensorRT-LLM ``_torch/speculative/interface.py`` -- ``rejection_sampling_one_model``
  (docstring: draft probs [batch, D, vocab], draft ids [batch, D], target probs
  [batch, D+1, vocab], per-request Philox seed/offset; returns accepted tokens
  [batch, D+1] = accepted drafts, the corrected or bonus token, then -1);
  ``_sample_and_accept_draft_tokens_base`` (strict acceptance: count the leading
  draft tokens equal to the target's); ``_sample_sharded_temperature``
  (Gumbel-max is an exact temperature sample; rows below the greedy
  temperature threshold stay greedy); the key-exchange comments in the draft
  sampler (global argmax, lowest index on ties); ``_RNG_SLOT_SPAN`` (32 offsets
  between consecutive rows of one request).
* tokenspeed ``sampling/backends/flashinfer.py`` -- ``FlashInferSamplingBackend.verify``
  (temperature softmax, then top-k renormalisation followed by top-p
  renormalisation; greedy batches take the row argmax and a chain verify that
  fills accept_index with -1 first; per-position coins plus one final coin).
* The verification rule itself (accept x with probability min(1, p(x)/q(x)),
  otherwise draw from the normalised residual max(0, p - q); a bonus token from
  the last target row when every draft is accepted) is the one the pages'
  rejection op implements.

Readings where the pages are silent (each is listed with its reason in the
design notes):

* temperature below 1e-5 means greedy (one-hot at the lowest-index argmax);
* top-k keeps every value >= the k-th largest (ties kept), disabled when k <= 0
  or k >= V; top-p then keeps the smallest set of largest values whose mass
  reaches top_p times the top-k mass (ties at the threshold kept), active iff
  top_p < 1; selection compares logits, not rounded probabilities;
* acceptance is ``u * q(x) < p(x)`` (product form; exact in float64);
* the residual/bonus draw is an inverse CDF over ascending vocabulary index
  with float64 running sums; an empty residual falls back to the target row,
  and an all-zero target row to a uniform index floor(u * V);
* a draft id outside [0, V) is rejected at its position;
* uniforms: chain request b uses words 0..D-1 of stream (seed_b, offset_b) for
  the accept tests and word D for the final draw; Gumbel row j of request b
  uses word v of stream (seed_b, offset_b + 32 j) for vocabulary entry v.

Decisions that floating point takes carry a margin; a decision inside its band
flags the request (category and first affected output position).  Two widths
exist for the inverse-CDF boundary: ``CDF_BAND`` (1e-6) is the reporting
category; a draw is excluded from bit-exact comparison only inside
``cdf_sum_band(V)``, the rounding bound of two double-precision sums of V
non-negative terms taken in different orders (see ``cdf_sum_band``), unless
the draw's inputs were themselves rounded differently (the fused verify and
single-step sampling, whose target probabilities a float32 implementation
rounds: there the 1e-6 band is the exclusion).  Gumbel scores are float64.
"""
from __future__ import annotations

import math

import numpy as np

from . import philox

GREEDY_TEMPERATURE = 1e-5
RNG_SLOT_SPAN = 32
ACCEPT_BAND = 1e-6
CDF_BAND = 1e-6
TOPP_BAND = 1e-5
GUMBEL_BAND = 1e-4
_MASK64 = (1 << 64) - 1
_U53 = 2.0 ** -53          # unit roundoff of float64


def cdf_sum_band(V: int) -> float:
    """Exclusion band, relative to the total R, for an inverse-CDF draw over V exact double weights.

    Any summation order of n non-negative doubles has relative error at most
    (n - 1) u (u = 2^-53; Higham, Accuracy and Stability of Numerical
    Algorithms, Sec. 4.2, for every summation tree).  Two implementations that
    form the prefix C_j and the total R in different orders can therefore
    decide ``C_j > u_f * R`` differently only when |C_j / R - u_f| <= 2 g + u
    with g = V u (each side's C_j and R off by at most g R, plus one rounding
    of the product).  The oracle's own margin |C_j / R - u_f| is off from the
    exact one by at most another 2 g + u, so a draw whose oracle margin is at
    least 4 g + 2 u cannot differ.  The band is twice that: 8 (V + 1) u.
    """
    return 8.0 * (int(V) + 1) * _U53


# --------------------------------------------------------------------------- inputs
def decode_logits(logits, dtype: str) -> np.ndarray:
    """bf16 bit patterns (uint16) or float32 values -> float64 (exact)."""
    if dtype == "bf16":
        bits = np.asarray(logits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    return np.asarray(logits, dtype=np.float32).astype(np.float64)


def is_greedy(temperature) -> bool:
    return float(temperature) < GREEDY_TEMPERATURE


# --------------------------------------------------------------------------- softmax + renorm
def temperature_softmax(z: np.ndarray, temperature: float) -> np.ndarray:
    """softmax(z / T) of one row; T below the greedy threshold gives a one-hot at argmax.

    tokenspeed flashinfer.py, ``verify``: ``softmax(logits, temperature=...)``.
    """
    z = np.asarray(z, dtype=np.float64)
    if is_greedy(temperature):
        out = np.zeros_like(z)
        out[int(np.argmax(z))] = 1.0
        return out
    w = np.exp((z - z.max()) / float(temperature))
    return w / math.fsum(w)


def renorm_row(z: np.ndarray, temperature: float, top_k: int, top_p: float):
    """Temperature softmax, then top-k, then top-p renormalisation of one row.

    tokenspeed flashinfer.py, ``verify``: ``top_k_renorm_prob`` followed by
    ``top_p_renorm_prob`` (the fused kernel is a drop-in for that pair).
    Returns (probs float64 [V], flagged: bool).  ``flagged`` marks a row whose
    top-p threshold sits within TOPP_BAND (relative to the top-k mass) of a
    mass boundary.
    """
    z = np.asarray(z, dtype=np.float64)
    V = z.shape[0]
    if is_greedy(temperature):
        return temperature_softmax(z, temperature), False
    m = z.max()
    w = np.exp((z - m) / float(temperature))
    kept = np.ones(V, dtype=bool)
    k = int(top_k)
    if 0 < k < V:
        kth = np.partition(z, V - k)[V - k]          # k-th largest, counted with multiplicity
        kept = z >= kth
    flagged = False
    tp = float(top_p)
    if tp < 1.0:
        s_k = math.fsum(w[kept])
        vals, inv = np.unique(z[kept], return_inverse=True)   # ascending distinct values
        mass = np.bincount(inv.reshape(-1), weights=w[kept])
        cum = np.cumsum(mass[::-1])                  # mass of values >= each distinct value, descending
        target = tp * s_k
        hit = np.nonzero(cum >= target)[0]
        i = int(hit[0]) if hit.size else cum.shape[0] - 1
        tau = vals[::-1][i]
        kept &= z >= tau
        if s_k > 0:
            near = abs(cum[i] / s_k - tp) < TOPP_BAND
            if i > 0:
                near = near or abs(cum[i - 1] / s_k - tp) < TOPP_BAND
            flagged = bool(near)
    ws = np.where(kept, w, 0.0)
    return ws / math.fsum(ws), flagged


def softmax_renorm(logits, dtype, temperature, top_k=None, top_p=None, requests=None):
    """Batch form: logits [B, N, V] -> (probs float64, flags bool).

    Per-request parameters are arrays of length B.  With ``requests`` None the
    result covers every row ([B, N, V] and [B, N]); otherwise it holds the
    listed requests in the given order ([len(requests), N, V]).
    """
    B, N, V = np.shape(logits)
    reqs = list(range(B)) if requests is None else [int(r) for r in requests]
    out = np.empty((len(reqs), N, V))
    flags = np.zeros((len(reqs), N), dtype=bool)
    for i, b in enumerate(reqs):
        z = decode_logits(logits[b], dtype)
        k = 0 if top_k is None else int(top_k[b])
        tp = 1.0 if top_p is None else float(top_p[b])
        for j in range(N):
            out[i, j], flags[i, j] = renorm_row(z[j], float(temperature[b]), k, tp)
    return out, flags


# --------------------------------------------------------------------------- single-step sampling
MINP_BAND = 1e-9


def joint_filter_row(z: np.ndarray, temperature: float, top_k: int, top_p: float, min_p: float):
    """Weights of one row after the joint top-k / top-p / min-p filter.

    tokenspeed flashinfer.py, ``sample``: ``softmax(logits, temperature)``
    then ``top_k_top_p_sampling_from_probs(..., filter_apply_order="joint")``:
    both filters judge the unfiltered distribution and a token is kept when
    it passes both -- top-k keeps every value >= the k-th largest (ties kept,
    off when k <= 0 or k >= V), top-p keeps the smallest set of largest values
    whose mass reaches top_p of the row's whole mass (ties at the threshold
    kept, active iff top_p < 1).  TensorRT-LLM interface.py passes per-request
    ``min_ps`` to its fused sampler; read plainly, min-p keeps p_v >= min_p *
    p_max, i.e. (z_v - max z) >= T ln(min(min_p, 1)), compared on logits in
    float64 (off when min_p <= 0; min_p >= 1 keeps the maximal values).
    Returns (unnormalised kept weights exp((z - max) / T) float64 [V], flagged):
    ``flagged`` marks a row with a top-p threshold within TOPP_BAND of a mass
    boundary or a logit within MINP_BAND of the min-p threshold.
    """
    z = np.asarray(z, dtype=np.float64)
    V = z.shape[0]
    m = z.max()
    T = float(temperature)
    w = np.exp((z - m) / T)
    kept = np.ones(V, dtype=bool)
    k = int(top_k)
    if 0 < k < V:
        kth = np.partition(z, V - k)[V - k]
        kept &= z >= kth
    flagged = False
    tp = float(top_p)
    if tp < 1.0:
        total = math.fsum(w)
        vals, inv = np.unique(z, return_inverse=True)
        mass = np.bincount(inv.reshape(-1), weights=w)
        cum = np.cumsum(mass[::-1])
        hit = np.nonzero(cum >= tp * total)[0]
        i = int(hit[0]) if hit.size else cum.shape[0] - 1
        kept &= z >= vals[::-1][i]
        near = abs(cum[i] / total - tp) < TOPP_BAND
        if i > 0:
            near = near or abs(cum[i - 1] / total - tp) < TOPP_BAND
        flagged = bool(near)
    mp = float(min_p)
    if mp > 0.0:
        thr = T * math.log(min(mp, 1.0))      # min_p >= 1 keeps the maximal value(s)
        d = z - m
        kept &= d >= thr
        flagged = flagged or bool(np.any(np.abs(d - thr) < MINP_BAND * max(1.0, abs(thr))))
    return np.where(kept, w, 0.0), flagged


def sample(logits, dtype, temperature, top_k, top_p, min_p, seed, offset, requests=None):
    """Single-step sampling of one token per request from logits [B, V].

    tokenspeed flashinfer.py, ``sample``: all-greedy batches take the row
    argmax; otherwise the joint-filtered, renormalised temperature softmax is
    sampled with the request's Philox (seed, offset).  Here a row below the
    greedy temperature takes its argmax; every other row draws by inverse CDF
    over ascending vocabulary index with the uniform of word 0 of its stream
    (the bonus draw of a verify without drafts).  Per-request arrays may be
    None (top_k off, top_p 1, min_p 0).
    Returns dict(tokens [B] int64 (-2 where not computed), flagged [B] bool).
    """
    B, V = np.shape(logits)
    tokens = np.full(B, -2, dtype=np.int64)
    flagged = np.zeros(B, dtype=bool)
    reqs = range(B) if requests is None else [int(r) for r in requests]
    for b in reqs:
        z = decode_logits(logits[b], dtype)
        T = float(temperature[b])
        if is_greedy(T):
            tokens[b] = int(np.argmax(z))
            continue
        k = 0 if top_k is None else int(top_k[b])
        tp = 1.0 if top_p is None else float(top_p[b])
        mp = 0.0 if min_p is None else float(min_p[b])
        r, fl = joint_filter_row(z, T, k, tp, mp)
        wd = philox.words(int(seed[b]), int(offset[b]), 1)
        u = float(philox.uniform(wd)[0])
        code = int(philox.uniform_code(wd)[0])
        y, margin = residual_draw(r, r, u, code)
        tokens[b] = y
        flagged[b] = fl or margin < CDF_BAND
    return dict(tokens=tokens, flagged=flagged)


# --------------------------------------------------------------------------- chain rejection
def chain_uniforms(seed: int, offset: int, D: int):
    """Accept uniforms u_0..u_{D-1} and the final uniform (with its odd code) of one request."""
    w = philox.words(seed, offset, D + 1)
    u = philox.uniform(w)
    code = int(philox.uniform_code(w[D:D + 1])[0])
    return u[:D], float(u[D]), code


def residual_draw(r: np.ndarray, fallback: np.ndarray, u_final: float, code: int):
    """Inverse-CDF draw of one index from non-negative weights ``r``.

    token = min{ j : sum_{v <= j} r_v > u * R }, R = sum r (float64 running sum
    in ascending index order).  If R is not positive the target row
    ``fallback`` is used instead; if that too has no positive mass the draw is
    uniform: floor(u * V) computed exactly from the uniform's code.
    Returns (token, margin): margin = min |u - C / R| over the two CDF values
    that bracket the token (C_{y-1} and C_y), 0 when rounding left u * R past
    every positive weight (the token is then the last positive entry), and
    infinity for the uniform fallback (no float decision).
    """
    V = r.shape[0]
    c = np.cumsum(r)
    total = c[-1] if V else 0.0
    if not total > 0.0:
        r = fallback
        c = np.cumsum(r)
        total = c[-1] if V else 0.0
    if not total > 0.0:
        return int((code * V) >> 24), math.inf
    t = u_final * total
    y = int(np.searchsorted(c, t, side="right"))
    if y >= V:
        return int(np.nonzero(r > 0)[0][-1]), 0.0
    lo = c[y - 1] if y > 0 else 0.0
    hi = c[y]
    return y, float(min(abs(u_final - lo / total), abs(u_final - hi / total)))


def chain_reject_core(q: np.ndarray, x: np.ndarray, p: np.ndarray,
                      u_accept: np.ndarray, u_final: float, code: int, cdf_band=None):
    """Chain rejection of one request given its uniforms.

    q [D, V] draft probs, x [D] draft ids, p [D+1, V] target probs (float32 or
    float64 values).  For i = 0..D-1: accept x_i iff u_i * q_i(x_i) < p_i(x_i);
    stop at the first rejection and draw the correction from max(0, p_i - q_i);
    if all D are accepted draw the bonus from p_D.
    Returns dict(tokens [D+1], L, near_accept (position or None), near_cdf
    (the draw's margin is below the 1e-6 reporting band), cdf_excluded (below
    ``cdf_band``; default ``cdf_sum_band(V)``, for inputs both sides hold as
    the same float values), cdf_margin).
    """
    D = x.shape[0]
    V = p.shape[-1]
    L = D
    near_accept = None
    for i in range(D):
        xi = int(x[i])
        if 0 <= xi < V:
            a = float(p[i, xi])
            c = float(q[i, xi])
            if near_accept is None and c > 0 and abs(float(u_accept[i]) - a / c) < ACCEPT_BAND:
                near_accept = i
            if float(u_accept[i]) * c < a:
                continue
        L = i
        break
    target_row = np.asarray(p[L], dtype=np.float64)
    if L < D:
        r = np.maximum(0.0, target_row - np.asarray(q[L], dtype=np.float64))
    else:
        r = target_row
    y, margin = residual_draw(r, target_row, u_final, code)
    band = cdf_sum_band(V) if cdf_band is None else float(cdf_band)
    tokens = np.full(D + 1, -1, dtype=np.int64)
    tokens[:L] = x[:L]
    tokens[L] = y
    return dict(tokens=tokens, L=L, near_accept=near_accept, near_cdf=margin < CDF_BAND,
                cdf_excluded=margin < band, cdf_margin=margin)


def one_hot_drafts(x: np.ndarray, V: int) -> np.ndarray:
    """Draft distributions of a target-only verify: row i is one-hot at x_i
    (all zeros when x_i lies outside [0, V)).

    tokenspeed flashinfer.py, ``verify``: without draft probabilities the
    chain kernel is given the draft tokens alone, with acceptance thresholds
    (``threshold_single``, ``threshold_acc``); at thresholds of one that is the
    rejection rule with a point-mass draft, which is what this builds.
    """
    x = np.asarray(x)
    q = np.zeros((x.shape[0], V))
    for i, xi in enumerate(x):
        if 0 <= int(xi) < V:
            q[i, int(xi)] = 1.0
    return q


def chain_reject(draft_probs, draft_ids, target_probs, seed, offset, requests=None, cdf_band=None):
    """Batch form of ``rejection_sampling_one_model``.

    ``draft_probs`` None is the target-only verify: every draft distribution is
    one-hot at its draft id (``one_hot_drafts``).  ``cdf_band`` is the draw's
    exclusion band (default ``cdf_sum_band(V)``: both sides hold the same
    float32 rows; pass ``CDF_BAND`` when the other side's rows were rounded
    from these, e.g. float32 probabilities against float64 ones).

    Returns accepted_tokens [B, D+1] (int64, -1 padded; rows not computed are
    -2), accept_length [B] (number of accepted drafts, -2 if not computed),
    flag_pos [B] (first output position whose value a float decision inside
    its exclusion band may change -- here only the drawn token at L, inside
    ``cdf_sum_band(V)``; D+1 when none), near_accept [B] (position of an
    accept test within 1e-6 of its threshold, -1 when none; accept tests are
    exact products, so this is reported only) and near_cdf [B] (the draw lies
    within the 1e-6 reporting band of a CDF boundary).  accept_length never
    depends on a sum, so it is exact for every request.
    """
    B, D = np.asarray(draft_ids).shape
    tokens = np.full((B, D + 1), -2, dtype=np.int64)
    L = np.full(B, -2, dtype=np.int64)
    flag_pos = np.full(B, D + 1, dtype=np.int64)
    near_accept = np.full(B, -1, dtype=np.int64)
    near_cdf = np.zeros(B, dtype=bool)
    reqs = range(B) if requests is None else [int(r) for r in requests]
    for b in reqs:
        ua, uf, code = chain_uniforms(int(seed[b]), int(offset[b]), D)
        q = one_hot_drafts(draft_ids[b], np.shape(target_probs)[-1]) if draft_probs is None else draft_probs[b]
        res = chain_reject_core(q, draft_ids[b], target_probs[b], ua, uf, code, cdf_band=cdf_band)
        tokens[b] = res["tokens"]
        L[b] = res["L"]
        near_cdf[b] = res["near_cdf"]
        if res["cdf_excluded"]:
            flag_pos[b] = res["L"]
        if res["near_accept"] is not None:
            near_accept[b] = res["near_accept"]
    return dict(accepted_tokens=tokens, accept_length=L, flag_pos=flag_pos, near_accept=near_accept,
                near_cdf=near_cdf)


# --------------------------------------------------------------------------- draft -> target vocabulary
def d2t_expand(draft_probs, d2t, V: int) -> np.ndarray:
    """Draft distributions over a reduced draft vocabulary, placed in the target vocabulary.

    TensorRT-LLM interface.py, one-model sampler: draft entry s goes to
    target index (s + d2t[s]) mod V (a floor modulus, as torch's ``%``) of a
    zero-filled row; without a d2t table the draft vocabulary is the first Vd
    target entries.  The page's scatter assumes the mapping is one-to-one and
    says nothing of shared targets; here the scatter runs in ascending draft
    order, so when several draft entries share a target the highest-numbered
    one is what that target holds.
    draft_probs [..., Vd] -> [..., V] (same dtype).
    """
    draft_probs = np.asarray(draft_probs)
    Vd = draft_probs.shape[-1]
    out = np.zeros(draft_probs.shape[:-1] + (V,), dtype=draft_probs.dtype)
    if d2t is None:
        out[..., :Vd] = draft_probs
        return out
    target = (np.arange(Vd, dtype=np.int64) + np.asarray(d2t, dtype=np.int64)) % V
    if np.unique(target).size == Vd:
        out[..., target] = draft_probs            # one-to-one: a single scatter
    else:
        for s in range(Vd):                       # shared targets: each later entry overwrites
            out[..., target[s]] = draft_probs[..., s]
    return out


# --------------------------------------------------------------------------- ragged chain rejection
def ragged_pad(draft_probs, draft_ids, target_packed, qo_indptr, D: int):
    """The padded rectangle a ragged verify batch is scattered into.

    TensorRT-LLM interface.py, the ragged branch of the one-model sampler
    (``scatter_ragged_to_padded`` then ``fill_padded_rows_onehot``, for target
    and draft rows alike): request r owns packed target rows
    [qo_indptr[r], qo_indptr[r+1]), verify_lens[r] = their count.  Target rows
    at positions >= verify_lens[r] and draft rows at positions >=
    verify_lens[r] - 1 are one-hot at token 0, and missing draft ids are 0:
    at the request's own last position acceptance emits token 0 with
    probability p(0) and a rejection samples p with token 0 removed, which
    together sample p.

    ``draft_probs`` None is the target-only verify (point masses at the draft
    ids).  Returns (q [B, D, V], x [B, D], p [B, D+1, V], lens [B]); a request
    whose length is outside [1, D+1] or whose rows fall outside the packed
    array gets length -1 (and is not verified).
    """
    target_packed = np.asarray(target_packed)
    T, V = target_packed.shape
    ind = np.asarray(qo_indptr, dtype=np.int64)
    B = ind.shape[0] - 1
    p = np.zeros((B, D + 1, V))
    q = np.zeros((B, D, V))
    x = np.zeros((B, D), dtype=np.int64)
    lens = np.full(B, -1, dtype=np.int64)
    for b in range(B):
        base, n = int(ind[b]), int(ind[b + 1] - ind[b])
        if not (1 <= n <= D + 1 and 0 <= base and base + n <= T):
            continue
        lens[b] = n
        d = n - 1
        p[b, :n] = target_packed[base:base + n]
        p[b, n:, 0] = 1.0
        x[b, :d] = np.asarray(draft_ids)[b, :d]
        if draft_probs is None:
            q[b, :d] = one_hot_drafts(x[b, :d], V)
        else:
            q[b, :d] = np.asarray(draft_probs)[b, :d]
        q[b, d:, 0] = 1.0
    return q, x, p, lens


def chain_reject_ragged(draft_probs, draft_ids, target_packed, qo_indptr, seed, offset, requests=None):
    """Ragged (per-request verify length) chain rejection.

    TensorRT-LLM interface.py, ragged branch of the one-model sampler: the
    packed rows are padded as ``ragged_pad`` states, the chain verify runs on
    the padded rectangle, and the number of emitted tokens is capped at the
    request's verify length, since positions past it were never scored by the
    target.  Returned accept_length is the number of accepted draft tokens
    after the cap (emitted - 1); tokens after the emitted ones are -1.
    Requests with an invalid length get accept_length -1 and all tokens -1.

    Same return dict as ``chain_reject``.
    """
    B, D = np.asarray(draft_ids).shape
    q, x, p, lens = ragged_pad(draft_probs, draft_ids, target_packed, qo_indptr, D)
    tokens = np.full((B, D + 1), -2, dtype=np.int64)
    L = np.full(B, -2, dtype=np.int64)
    flag_pos = np.full(B, D + 1, dtype=np.int64)
    near_accept = np.full(B, -1, dtype=np.int64)
    near_cdf = np.zeros(B, dtype=bool)
    reqs = range(B) if requests is None else [int(r) for r in requests]
    for b in reqs:
        if lens[b] < 0:
            tokens[b] = -1
            L[b] = -1
            continue
        ua, uf, code = chain_uniforms(int(seed[b]), int(offset[b]), D)
        res = chain_reject_core(q[b], x[b], p[b], ua, uf, code)
        emitted = min(res["L"] + 1, int(lens[b]))
        t = res["tokens"].copy()
        t[emitted:] = -1
        tokens[b] = t
        L[b] = emitted - 1
        if res["L"] < emitted:
            near_cdf[b] = res["near_cdf"]
            if res["cdf_excluded"]:
                flag_pos[b] = res["L"]
        if res["near_accept"] is not None and res["near_accept"] < emitted:
            near_accept[b] = res["near_accept"]
    return dict(accepted_tokens=tokens, accept_length=L, flag_pos=flag_pos, near_accept=near_accept,
                near_cdf=near_cdf)


# --------------------------------------------------------------------------- fused target rows + chain rejection
def verify_fused(logits, dtype, temperature, top_k, top_p, draft_probs, draft_ids, seed, offset, requests=None):
    """Target rows from logits, then chain rejection, as one call.

    tokenspeed flashinfer.py, ``verify``: the target probabilities are the
    temperature softmax of the logits followed by top-k and then top-p
    renormalisation, and the chain verify consumes them; TensorRT-LLM's
    fused sampling ops are the pages' reason to compute both without
    materialising the probabilities.  Definition: row j of request b is
    ``renorm_row(z_bj, T_b, k_b, top_p_b)`` (float64) and the outputs are
    ``chain_reject_core`` on those rows with the request's draft probs, draft
    ids and uniforms.  Only rows 0..L are needed, and only those are
    computed.

    Returns the ``chain_reject`` dictionary.  Here ``flag_pos`` also covers
    the decisions a float32 implementation takes from differently rounded
    target probabilities: a near-threshold accept test at position i (from i
    on), a top-p boundary flag on a row j <= L (from j on), and a CDF boundary
    within 1e-6 (from L on; the draw's weights are probabilities that a
    float32 implementation rounds, so the double-sum band does not cover it).
    """
    B, N, V = np.shape(logits)
    D = N - 1
    x = np.asarray(draft_ids)
    tokens = np.full((B, N), -2, dtype=np.int64)
    L = np.full(B, -2, dtype=np.int64)
    flag_pos = np.full(B, N, dtype=np.int64)
    near_accept = np.full(B, -1, dtype=np.int64)
    near_cdf = np.zeros(B, dtype=bool)
    reqs = range(B) if requests is None else [int(r) for r in requests]
    for b in reqs:
        z = decode_logits(logits[b], dtype)
        k = 0 if top_k is None else int(top_k[b])
        tp = 1.0 if top_p is None else float(top_p[b])
        T = float(temperature[b])
        ua, uf, code = chain_uniforms(int(seed[b]), int(offset[b]), D)
        rows, row_flag = [], []
        # rows 0..L: row j is needed once positions 0..j-1 are accepted
        for j in range(N):
            pj, fj = renorm_row(z[j], T, k, tp)
            rows.append(pj)
            row_flag.append(fj)
            if j < D:
                xj = int(x[b, j])
                if not (0 <= xj < V and float(ua[j]) * float(draft_probs[b, j, xj]) < pj[xj]):
                    break
        P = np.zeros((N, V))
        P[:len(rows)] = np.array(rows)
        res = chain_reject_core(draft_probs[b], x[b], P, ua, uf, code, cdf_band=CDF_BAND)
        tokens[b] = res["tokens"]
        L[b] = res["L"]
        near_cdf[b] = res["near_cdf"]
        fp = N
        if res["cdf_excluded"]:
            fp = res["L"]
        if res["near_accept"] is not None:
            near_accept[b] = res["near_accept"]
            fp = min(fp, res["near_accept"])
        for j in range(res["L"] + 1):
            if row_flag[j]:
                fp = min(fp, j)
                break
        flag_pos[b] = fp
    return dict(accepted_tokens=tokens, accept_length=L, flag_pos=flag_pos, near_accept=near_accept,
                near_cdf=near_cdf)


# --------------------------------------------------------------------------- greedy verify
def greedy_verify(logits, dtype, draft_ids, requests=None):
    """Greedy chain verify.

    tokenspeed flashinfer.py, ``verify`` (all-greedy branch): target tokens are
    the row argmax (lowest index on ties, as the TensorRT-LLM draft sampler's
    key-exchange comments state); L = number of leading draft ids equal to the
    target tokens.  Outputs: accepted_tokens = y_0..y_L then -1; predict[b, j] =
    y_j for j <= L else -1; accept_index[b, j] = b*N + j (flat index into
    predict) for j <= L else -1; argmax [B, N] = y for every row.
    """
    B, N, V = np.shape(logits)
    D = N - 1
    x = np.asarray(draft_ids)
    tokens = np.full((B, N), -2, dtype=np.int64)
    predict = np.full((B, N), -2, dtype=np.int64)
    accept_index = np.full((B, N), -2, dtype=np.int64)
    argmax = np.full((B, N), -2, dtype=np.int64)
    L = np.full(B, -2, dtype=np.int64)
    reqs = range(B) if requests is None else [int(r) for r in requests]
    for b in reqs:
        z = decode_logits(logits[b], dtype)
        y = np.array([int(np.argmax(z[j])) for j in range(N)], dtype=np.int64)
        n_acc = 0
        while n_acc < D and int(x[b, n_acc]) == y[n_acc]:
            n_acc += 1
        L[b] = n_acc
        tokens[b] = -1
        tokens[b, :n_acc + 1] = y[:n_acc + 1]
        predict[b] = tokens[b]
        accept_index[b] = -1
        accept_index[b, :n_acc + 1] = b * N + np.arange(n_acc + 1)
        argmax[b] = y
    return dict(accepted_tokens=tokens, accept_length=L, predict=predict,
                accept_index=accept_index, argmax=argmax)


# --------------------------------------------------------------------------- Gumbel-max
def gumbel_row(z32: np.ndarray, temperature: float, seed: int, subseq: int):
    """Temperature sample of one row by Gumbel-max, in float64.

    s_v = z_v / T + G_v with G_v = -ln(-ln u_v), u_v = uniform of word v of
    stream (seed, subseq); token = lowest-index argmax of s.  Returns (token,
    near_tie).  near_tie marks a gap between the two largest scores below
    ``gumbel_band`` of those two entries: an implementation that forms the
    scores in float32 is off by a few float32 ulps of |z/T| + |G| per score,
    and only a gap that small can reorder the top two.
    """
    z = np.asarray(z32, dtype=np.float32).astype(np.float64)
    V = z.shape[0]
    u = philox.uniform(philox.words(seed, subseq, V))
    g = -np.log(-np.log(u))
    zt = z / float(temperature)
    s = zt + g
    y = int(np.argmax(s))
    near = False
    if V > 1:
        i2 = np.argpartition(s, V - 2)[V - 2:]
        scale = float(np.max(np.abs(zt[i2]) + np.abs(g[i2])))
        near = bool(abs(float(s[i2[1]]) - float(s[i2[0]])) < gumbel_band(scale))
    return y, near


def gumbel_band(scale: float) -> float:
    """Near-tie band of two Gumbel scores whose terms |z/T| + |G| are at most ``scale``.

    1e-4 for scale <= 16, growing in proportion beyond: 1e-4 / 16 = 6.25e-6
    of the scale is about 52 float32 ulps (2^-23 relative each), an order of
    magnitude above the error of a float32 score from a correctly rounded
    product and logarithms within a few ulps.
    """
    return GUMBEL_BAND * max(1.0, float(scale) / 16.0)


def gumbel_sample(logits, dtype, temperature, draft_ids, seed, offset, requests=None,
                  all_rows=False):
    """Temperature-only target sampling by Gumbel-max, then strict chain acceptance.

    TensorRT-LLM interface.py, ``_sample_sharded_temperature`` and
    ``_sample_and_accept_draft_tokens_base``.  Row j of request b draws from
    stream (seed_b, offset_b + 32 j); rows with T below the greedy threshold
    take the plain argmax.  Rows are computed up to the first mismatch unless
    ``all_rows``.  Returns accepted_tokens, accept_length, sampled [B, N] (-2
    where not computed), flag_pos [B] (first row whose decision is a near tie,
    N when none).
    """
    B, N, V = np.shape(logits)
    D = N - 1
    x = np.asarray(draft_ids)
    tokens = np.full((B, N), -2, dtype=np.int64)
    sampled = np.full((B, N), -2, dtype=np.int64)
    L = np.full(B, -2, dtype=np.int64)
    flag_pos = np.full(B, N, dtype=np.int64)
    reqs = range(B) if requests is None else [int(r) for r in requests]
    for b in reqs:
        z = decode_logits(logits[b], dtype).astype(np.float32)
        T = float(np.float32(temperature[b]))
        n_acc = None
        for j in range(N):
            if is_greedy(T):
                yj, near = int(np.argmax(z[j])), False
            else:
                sub = (int(offset[b]) + RNG_SLOT_SPAN * j) & _MASK64
                yj, near = gumbel_row(z[j], T, int(seed[b]), sub)
            sampled[b, j] = yj
            if near and flag_pos[b] == N:
                flag_pos[b] = j
            if n_acc is None and (j == D or int(x[b, j]) != yj):
                n_acc = j
                if not all_rows:
                    break
        L[b] = n_acc
        tokens[b] = -1
        tokens[b, :n_acc + 1] = sampled[b, :n_acc + 1]
    return dict(accepted_tokens=tokens, accept_length=L, sampled=sampled, flag_pos=flag_pos)
