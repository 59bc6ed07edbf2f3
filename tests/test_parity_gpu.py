"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Integer results (tokens, accept lengths, predict, accept_index, argmax) must be
bit-exact except decisions the oracle flags as falling inside their exclusion
band: an inverse-CDF draw within the double-sum rounding bound of a boundary
(8 (V + 1) 2^-53 of the row mass when both sides sum the same float32 rows;
1e-6 when one side's rows are float64), a top-p boundary within 1e-5 of the
top-k mass, a Gumbel near tie (1e-4, scaled with the scores' size).  Flagged
requests are compared up to the flagged position.  Chain-rejection accept
lengths come from exact products and are compared for every request.
Probabilities must agree within 1e-5 absolute.  Every test prints its case
before launching.
"""
import itertools

import numpy as np
import pytest

import oracle
from gpu_helpers import dev, dev_logits, guard_intact, guarded_i32, log, np_i, SENTINEL
from workloads import MODE_GREEDY, MODE_TEMPERATURE, MODE_TOPK, MODE_TOPP, fuzz_case, make_config

pytestmark = pytest.mark.gpu

PROB_ATOL = 1e-5


@pytest.fixture(scope="module")
def sv():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import token_sampling_temp_amd as m
    m.lib()   # raises when the HIP library is missing: there is no fallback
    return m


# --------------------------------------------------------------------------- comparison helpers
def assert_chain_match(gpu_tok, gpu_len, ref, reqs, ctx, len_exact=True, max_excluded=None):
    """Accept lengths and tokens bit-exact, except tokens from the oracle's
    flagged position on.  len_exact: every accept length must match (chain
    rejection, where L follows from exact products); otherwise a flag at or
    before L may move it (Gumbel rows).  max_excluded bounds the number of
    requests with an excluded decision (default: 1 + 1% of them).  Returns
    that number."""
    reqs = list(reqs)
    flagged = 0
    for b in reqs:
        L = int(ref["accept_length"][b])
        fp = int(ref["flag_pos"][b])
        if len_exact or fp > L:
            assert int(gpu_len[b]) == L, (ctx, b, int(gpu_len[b]), L, fp)
        n = min(fp, L + 1)
        assert list(gpu_tok[b, :n]) == list(ref["accepted_tokens"][b, :n]), (ctx, b, gpu_tok[b], ref["accepted_tokens"][b])
        if int(gpu_len[b]) == L:
            assert np.all(gpu_tok[b, L + 1:] == -1), (ctx, b)
        flagged += fp <= L
    bound = 1 + len(reqs) // 100 if max_excluded is None else max_excluded
    assert flagged <= bound, (ctx, "excluded decisions", flagged, bound)
    return flagged


def greedy_drafts(rng, z, dtype, D, p_match=0.7):
    y = oracle.greedy_verify(z, dtype, np.zeros((z.shape[0], D), np.int32))["argmax"]
    V = z.shape[-1]
    rnd = rng.integers(0, V, size=(z.shape[0], D))
    return np.where(rng.random((z.shape[0], D)) < p_match, y[:, :D], rnd).astype(np.int32)


# --------------------------------------------------------------------------- greedy verify
GREEDY_CASES = list(itertools.product(
    [1, 2, 3, 7, 9, 31, 1000, 1001, 4099, 32000], [0, 1, 3, 16], ["f32", "bf16"], [None, "ties"]))


def test_greedy_verify_fuzz(sv):
    rng = np.random.default_rng(100)
    for i, (V, D, dt, sp) in enumerate(GREEDY_CASES):
        B = 5
        log(f"greedy fuzz {i}: V={V} D={D} dtype={dt} special={sp}")
        c = fuzz_case(i, B, D, V, dt, special=sp)
        x = greedy_drafts(rng, c["logits"], dt, D)
        ref = oracle.greedy_verify(c["logits"], dt, x)
        z = dev_logits(c["logits"], dt)
        acc, acc_full = guarded_i32((B, D + 1))
        out = sv.greedy_verify(z, dev(x), argmax=True, out={"accepted_tokens": acc})
        for k in ("accepted_tokens", "accept_length", "predict", "accept_index", "argmax"):
            assert np.array_equal(np_i(out[k]), ref[k]), (k, V, D, dt, sp, np_i(out[k]), ref[k])
        assert guard_intact(acc_full, B * (D + 1))
        # without argmax: rows after the first mismatch are skipped, same results
        out2 = sv.greedy_verify(z, dev(x))
        for k in ("accepted_tokens", "accept_length", "predict", "accept_index"):
            assert np.array_equal(np_i(out2[k]), ref[k]), (k, V, D, dt)
        # the one-workgroup-per-request form (no workspace), with and without every argmax
        for am in (True, False):
            out3 = sv.greedy_verify(z, dev(x), argmax=am, workspace=False)
            for k in ("accepted_tokens", "accept_length", "predict", "accept_index") + (("argmax",) if am else ()):
                assert np.array_equal(np_i(out3[k]), ref[k]), (k, V, D, dt, am)


def test_greedy_special_values(sv):
    torch = __import__("torch")
    rows = np.array([
        [-0.0, 0.0, 0.0, -0.0, -1.0, -0.0, 0.0, -5.0, 0.0],        # signed zeros tie
        [1.0, np.nan, 3.0, np.nan, 2.0, 3.0, 0.0, 1.0, 1.0],       # first NaN wins
        [-np.inf] * 9,                                             # all -inf -> index 0
        [2.0, 5.0, 5.0, np.inf, 1.0, np.inf, 0.0, 0.0, -np.inf],   # +inf, tie
        [3.0, 3.0, 3.0, 3.0, 3.0, 3.0, 3.0, 3.0, 3.0],
        [-1.0, -2.0, -3.0, -4.0, -5.0, -6.0, -7.0, -8.0, -0.5],
    ], dtype=np.float32)
    from workloads import f32_to_bf16_bits
    for dt in ("f32", "bf16"):
        for V in (9, 8 * 9):
            z = np.tile(rows, (1, V // 9))[None].astype(np.float32)      # [1, 6, V]
            zz = f32_to_bf16_bits(z) if dt == "bf16" else z
            log(f"greedy special values dtype={dt} V={V}")
            ref = oracle.greedy_verify(zz, dt, np.zeros((1, 5), np.int32) - 1)
            out = sv.greedy_verify(dev_logits(zz, dt), dev(np.zeros((1, 5), np.int32) - 1), argmax=True)
            assert np.array_equal(np_i(out["argmax"]), ref["argmax"]), (dt, V, np_i(out["argmax"]), ref["argmax"])
            t = torch.from_numpy(oracle.decode_logits(zz, dt)[0])
            assert list(ref["argmax"][0]) == [int(torch.argmax(r)) for r in t]


def test_greedy_unaligned_rows_and_offsets(sv):
    """Rows starting at every 2/4-byte offset modulo 16 (tensor views with a storage offset)."""
    torch = __import__("torch")
    rng = np.random.default_rng(7)
    for dt in ("f32", "bf16"):
        B, D, V = 3, 2, 517
        c = fuzz_case(55, B, D, V, dt, special="ties")
        x = greedy_drafts(rng, c["logits"], dt, D, 0.9)
        ref = oracle.greedy_verify(c["logits"], dt, x)
        z = dev_logits(c["logits"], dt).reshape(-1)
        for shift in range(1, 8):
            log(f"greedy unaligned dtype={dt} shift={shift}")
            buf = torch.empty(z.numel() + 8, dtype=z.dtype, device=z.device)
            view = buf[shift:shift + z.numel()]
            view.copy_(z)
            out = sv.greedy_verify(view.view(B, D + 1, V), dev(x), argmax=True)
            assert np.array_equal(np_i(out["argmax"]), ref["argmax"])
            assert np.array_equal(np_i(out["accepted_tokens"]), ref["accepted_tokens"])


def test_greedy_config4_full(sv):
    c = make_config(4)
    log("greedy config 4 full: B=512 N=4 V=151936 bf16")
    ref = oracle.greedy_verify(c["logits"], "bf16", c["draft_ids"])
    out = sv.greedy_verify(dev_logits(c["logits"], "bf16"), dev(c["draft_ids"]), argmax=True)
    for k in ("accepted_tokens", "accept_length", "predict", "accept_index", "argmax"):
        assert np.array_equal(np_i(out[k]), ref[k]), k
    assert np.array_equal(ref["argmax"], c["planted"])
    out2 = sv.greedy_verify(dev_logits(c["logits"], "bf16"), dev(c["draft_ids"]))
    assert np.array_equal(np_i(out2["accepted_tokens"]), ref["accepted_tokens"])
    out3 = sv.greedy_verify(dev_logits(c["logits"], "bf16"), dev(c["draft_ids"]), workspace=False)
    for k in ("accepted_tokens", "accept_length", "predict", "accept_index"):
        assert np.array_equal(np_i(out3[k]), ref[k]), k


def _rowpar_subset_case(sv, fn, ws_query, check):
    """Both strict-acceptance calls through an explicit workspace: a request
    subset with a repeated row and indices outside [0, B), then a smaller
    batch on the same workspace; outputs against the one-workgroup-per-request
    form (bit-exact: same row arithmetic), untouched rows keep their sentinel,
    and the workspace is zero after every call."""
    torch = __import__("torch")
    B, D, V = 40, 5, 4099
    c = fuzz_case(77, B, D, V, "bf16")
    rng = np.random.default_rng(77)
    x = greedy_drafts(rng, c["logits"], "bf16", D, 0.9)
    T = np.where(np.arange(B) % 3 == 0, 0.0, 0.8).astype(np.float32)
    z = dev_logits(c["logits"], "bf16")
    for idx in (np.array([3, 7, 7, 39, -1, 40, 0, 12, 5, 6, 8, 9, 10, 11, 13, 2], np.int32),
                np.array([1, 4], np.int32)):
        n = len(idx)
        ws = torch.zeros((ws_query(n, D),), dtype=torch.uint8, device="cuda")
        outs = []
        for w in (ws, False):
            acc = torch.full((B, D + 1), SENTINEL, dtype=torch.int32, device="cuda")
            alen = torch.full((B,), SENTINEL, dtype=torch.int32, device="cuda")
            fn(z, dev(x), dev(T), c, dev(idx), {"accepted_tokens": acc, "accept_length": alen}, w)
            outs.append((np_i(acc), np_i(alen)))
            if w is not False:
                assert int(ws.cpu().numpy().astype(np.int64).sum()) == 0, "workspace left non-zero"
        assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
        valid = sorted(set(int(b) for b in idx if 0 <= b < B))
        untouched = np.setdiff1d(np.arange(B), valid)
        assert np.all(outs[0][1][untouched] == SENTINEL)
        check(outs[0][0], outs[0][1], c, x, T, valid)


def test_greedy_rowpar_workspace_subset(sv):
    def fn(z, x, T, c, idx, out, w):
        sv.greedy_verify(z, x, req_index=idx, predict=False, accept_index=False, out=out, workspace=w)
    def check(A, Ls, c, x, T, valid):
        ref = oracle.greedy_verify(c["logits"], "bf16", x, requests=valid)
        for b in valid:
            assert list(A[b]) == list(ref["accepted_tokens"][b]) and Ls[b] == ref["accept_length"][b], b
    log("greedy row-parallel: subset with repeats and invalid indices, explicit workspace")
    _rowpar_subset_case(sv, fn, sv.greedy_verify_workspace_bytes, check)


def test_gumbel_rowpar_workspace_subset(sv):
    def fn(z, x, T, c, idx, out, w):
        sv.gumbel_sample(z, T, x, dev(c["seed"]), dev(c["offset"]), req_index=idx, out=out, workspace=w)
    def check(A, Ls, c, x, T, valid):
        ref = oracle.gumbel_sample(c["logits"], "bf16", T, x, c["seed"], c["offset"], requests=valid)
        assert_chain_match(A, Ls, ref, valid, "gumbel row-parallel subset", len_exact=False, max_excluded=1)
    log("Gumbel row-parallel: subset with repeats and invalid indices, explicit workspace")
    _rowpar_subset_case(sv, fn, sv.gumbel_sample_workspace_bytes, check)


# --------------------------------------------------------------------------- chain rejection
CHAIN_CASES = (
    [(V, D, None) for V in (1, 2, 3, 5, 31, 1000, 1001, 4097, 32000) for D in (0, 1, 3, 5)]
    + [(V, 16, None) for V in (7, 1030)]
    + [(V, D, sp) for sp in ("equal", "disjoint", "onehot", "zeros", "invalid_ids")
       for V in (2, 33, 1000, 4099) for D in (1, 4)]
)


def test_chain_reject_fuzz(sv):
    flagged = 0
    for i, (V, D, sp) in enumerate(CHAIN_CASES):
        B = 6
        log(f"chain fuzz {i}: V={V} D={D} special={sp}")
        c = fuzz_case(200 + i, B, D, V, "f32", special=sp)
        ref = oracle.chain_reject(c["draft_probs"], c["draft_ids"], c["target_probs"], c["seed"], c["offset"])
        acc, acc_full = guarded_i32((B, D + 1))
        alen, alen_full = guarded_i32((B,))
        sv.chain_reject(dev(c["draft_probs"]), dev(c["draft_ids"]), dev(c["target_probs"]), dev(c["seed"]),
                        dev(c["offset"]), out=(acc, alen))
        flagged += assert_chain_match(np_i(acc), np_i(alen), ref, range(B), (V, D, sp))
        assert guard_intact(acc_full, B * (D + 1)) and guard_intact(alen_full, B)
        if sp == "equal":
            assert np.all(np_i(alen) == D)
        if sp == "disjoint" and V >= 2:
            assert np.all(np_i(alen) == 0)
    log(f"chain fuzz flagged requests: {flagged}")


def test_chain_reject_unaligned_rows(sv):
    torch = __import__("torch")
    B, D, V = 4, 3, 1003
    c = fuzz_case(77, B, D, V, "f32")
    ref = oracle.chain_reject(c["draft_probs"], c["draft_ids"], c["target_probs"], c["seed"], c["offset"])
    for shift in (1, 2, 3):
        log(f"chain unaligned shift={shift}")
        p = torch.empty(B * (D + 1) * V + 4, device="cuda")[shift:shift + B * (D + 1) * V]
        q = torch.empty(B * D * V + 4, device="cuda")[shift:shift + B * D * V]
        p.copy_(dev(c["target_probs"]).reshape(-1))
        q.copy_(dev(c["draft_probs"]).reshape(-1))
        acc, alen = sv.chain_reject(q.view(B, D, V), dev(c["draft_ids"]), p.view(B, D + 1, V), dev(c["seed"]),
                                    dev(c["offset"]))
        assert_chain_match(np_i(acc), np_i(alen), ref, range(B), ("unaligned", shift))


def test_chain_reject_one_workgroup_per_request(sv):
    """Batches large enough that each request gets one workgroup (chunk sums
    kept in LDS), on aligned rows with a partial last round, odd V, and the
    degenerate-row fallbacks."""
    for B, D, V, special in ((260, 5, 20000, None), (300, 3, 5003, None), (258, 2, 4096, "zeros"),
                             (257, 4, 12288, "disjoint")):
        c = fuzz_case(500 + V, B, D, V, "f32", special=special)
        log(f"chain one workgroup per request: B={B} D={D} V={V} special={special}")
        ref = oracle.chain_reject(c["draft_probs"], c["draft_ids"], c["target_probs"], c["seed"], c["offset"])
        acc, alen = sv.chain_reject(dev(c["draft_probs"]), dev(c["draft_ids"]), dev(c["target_probs"]),
                                    dev(c["seed"]), dev(c["offset"]))
        assert_chain_match(np_i(acc), np_i(alen), ref, range(B), (B, D, V, special))


def test_chain_reject_large_batches(sv):
    """Batches of long rows, with rows split over several workgroups (partial
    sums published, last workgroup locates) and with one workgroup per
    request: a ragged last chunk, up to 1024 requests, all-bonus and
    all-residual batches, degenerate rows, a row of 293 chunks, and a
    request subset with skipped and repeated indices.  (64, 3, 49148) and
    (40, 5, 60000) split rows into segments of three 4096-entry rounds: the
    load pipeline pads a segment to an even number of rounds, and the padding
    round lies in the next segment, so it must read zeros, not that
    segment's entries."""
    cases = ((64, 5, 65536, None), (300, 3, 16424, None), (1024, 3, 4096, None), (130, 4, 32768, "zeros"),
             (110, 2, 40000, "equal"), (140, 2, 30000, "disjoint"), (70, 7, 60000, None), (160, 0, 65536, None),
             (64, 3, 49148, None), (40, 5, 60000, None),
             # one workgroup per request: no drafts, all accepted, a row of 293 chunks
             (300, 0, 8192, None), (270, 2, 8000, "equal"), (256, 1, 300000, None))
    flagged = 0
    for B, D, V, special in cases:
        c = fuzz_case(900 + B + V, B, D, V, "f32", special=special)
        log(f"chain large batch: B={B} D={D} V={V} special={special}")
        ref = oracle.chain_reject(c["draft_probs"], c["draft_ids"], c["target_probs"], c["seed"], c["offset"])
        acc, acc_full = guarded_i32((B, D + 1))
        alen, alen_full = guarded_i32((B,))
        sv.chain_reject(dev(c["draft_probs"]), dev(c["draft_ids"]), dev(c["target_probs"]), dev(c["seed"]),
                        dev(c["offset"]), out=(acc, alen))
        flagged += assert_chain_match(np_i(acc), np_i(alen), ref, range(B), (B, D, V, special))
        assert guard_intact(acc_full, B * (D + 1)) and guard_intact(alen_full, B)
        if special == "equal":
            assert np.all(np_i(alen) == D)
        if special == "disjoint":
            assert np.all(np_i(alen) == 0)
    # request subset: skipped (-1, B) and repeated entries
    B, D, V = 400, 4, 20000
    c = fuzz_case(977, B, D, V, "f32")
    rng = np.random.default_rng(5)
    reqs = rng.permutation(B)[:300].astype(np.int32)
    reqs[10], reqs[20], reqs[30] = -1, B, reqs[40]
    log(f"chain large batch subset: B={B} D={D} V={V} n_req={len(reqs)}")
    ref = oracle.chain_reject(c["draft_probs"], c["draft_ids"], c["target_probs"], c["seed"], c["offset"])
    acc = __import__("torch").full((B, D + 1), SENTINEL, dtype=__import__("torch").int32, device="cuda")
    alen = __import__("torch").full((B,), SENTINEL, dtype=__import__("torch").int32, device="cuda")
    sv.chain_reject(dev(c["draft_probs"]), dev(c["draft_ids"]), dev(c["target_probs"]), dev(c["seed"]),
                    dev(c["offset"]), req_index=dev(reqs), out=(acc, alen))
    done = sorted({int(r) for r in reqs if 0 <= r < B})
    flagged += assert_chain_match(np_i(acc), np_i(alen), ref, done, "large batch subset")
    rest = np.setdiff1d(np.arange(B), done)
    assert np.all(np_i(acc)[rest] == SENTINEL) and np.all(np_i(alen)[rest] == SENTINEL)
    log(f"chain large batch flagged requests: {flagged}")


def test_chain_reject_target_only(sv):
    """Target-only verify (no draft probabilities: point-mass drafts), on the
    split-row and one-workgroup-per-request paths, aligned and unaligned rows,
    with invalid ids, all-zero and one-hot target rows."""
    torch = __import__("torch")
    flagged = 0
    cases = [(6, 3, V, sp, 0) for V in (1, 7, 1000, 4097, 32000) for sp in (None, "invalid_ids", "onehot")]
    cases += [(6, 4, 3001, "zeros", 0), (5, 3, 1003, None, 1), (300, 5, 20000, None, 0), (260, 2, 4096, "onehot", 0),
              (40, 5, 60000, None, 0), (64, 3, 49148, "invalid_ids", 0)]
    for i, (B, D, V, sp, shift) in enumerate(cases):
        c = fuzz_case(1100 + i, B, D, V, "f32", special=sp)
        if sp is None and i % 2 == 0:
            # drafts at each row's most likely token half of the time, so acceptances happen
            c["draft_ids"] = np.where(np.random.default_rng(i).random((B, D)) < 0.5,
                                      c["target_probs"][:, :D].argmax(-1), c["draft_ids"]).astype(np.int32)
        log(f"chain target-only {i}: B={B} D={D} V={V} special={sp} shift={shift}")
        p = dev(c["target_probs"])
        if shift:
            flat = torch.empty(p.numel() + 4, device="cuda")
            pp = flat[shift:shift + p.numel()].view(B, D + 1, V)
            pp.copy_(p)
            p = pp
        ref = oracle.chain_reject(None, c["draft_ids"], c["target_probs"], c["seed"], c["offset"])
        acc, acc_full = guarded_i32((B, D + 1))
        alen, alen_full = guarded_i32((B,))
        sv.chain_reject(None, dev(c["draft_ids"]), p, dev(c["seed"]), dev(c["offset"]), out=(acc, alen))
        flagged += assert_chain_match(np_i(acc), np_i(alen), ref, range(B), (B, D, V, sp, shift))
        assert guard_intact(acc_full, B * (D + 1)) and guard_intact(alen_full, B)
    log(f"chain target-only flagged requests: {flagged}")


def test_chain_workspace_reuse_and_zero_after_use(sv):
    """One caller workspace serves split launches of different layouts (the
    counter region of a later call overlaps where an earlier call kept
    partial sums): every call leaves it all zero, and results match the
    oracle.  Also the ragged call through the same workspace."""
    torch = __import__("torch")
    cases = ((10, 3, 60000), (100, 2, 20000), (7, 5, 100003), (200, 1, 40000), (40, 5, 60000))
    ws = torch.zeros(max(sv.chain_workspace_bytes(B, V) for B, _, V in cases), dtype=torch.uint8, device="cuda")
    for B, D, V in cases:
        c = fuzz_case(1700 + B, B, D, V, "f32")
        log(f"chain with a shared caller workspace: B={B} D={D} V={V} need={sv.chain_workspace_bytes(B, V)}")
        ref = oracle.chain_reject(c["draft_probs"], c["draft_ids"], c["target_probs"], c["seed"], c["offset"])
        acc, alen = sv.chain_reject(dev(c["draft_probs"]), dev(c["draft_ids"]), dev(c["target_probs"]),
                                    dev(c["seed"]), dev(c["offset"]), workspace=ws)
        assert_chain_match(np_i(acc), np_i(alen), ref, range(B), ("shared workspace", B, V))
        assert not bool((ws != 0).any().item()), ("workspace not zero after the call", B, V)
        lens = np.random.default_rng(B).integers(1, D + 2, B)
        rows, ind = _ragged_pack(c, lens)
        refr = oracle.chain_reject_ragged(c["draft_probs"], c["draft_ids"], rows, ind, c["seed"], c["offset"])
        acc, alen = sv.chain_reject_ragged(dev(c["draft_probs"]), dev(c["draft_ids"]), dev(rows), dev(ind),
                                           dev(c["seed"]), dev(c["offset"]), workspace=ws)
        assert_chain_match(np_i(acc), np_i(alen), refr, range(B), ("shared workspace ragged", B, V))
        assert not bool((ws != 0).any().item()), ("workspace not zero after the ragged call", B, V)


def test_chain_reject_graph_capture_and_replay(sv):
    """Split-row chain rejection captured in a HIP graph with a caller
    workspace (no allocation or memset inside the call): three replays,
    with eager work and synchronisation between them, each equal to the
    eager result."""
    torch = __import__("torch")
    B, D, V = 40, 5, 60000
    c = fuzz_case(1777, B, D, V, "f32")
    args = [dev(c["draft_probs"]), dev(c["draft_ids"]), dev(c["target_probs"]), dev(c["seed"]), dev(c["offset"])]
    ws = sv.chain_workspace(B, V, "cuda")
    assert ws is not None
    log("chain graph capture: B=40 D=5 V=60000 (split rows), eager reference")
    acc0, len0 = sv.chain_reject(*args, workspace=ws)
    eager = (np_i(acc0), np_i(len0))
    acc = torch.empty((B, D + 1), dtype=torch.int32, device="cuda")
    alen = torch.empty((B,), dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        sv.chain_reject(*args, workspace=ws, out=(acc, alen))        # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sv.chain_reject(*args, workspace=ws, out=(acc, alen))
    for r in range(3):
        acc.fill_(-7)
        alen.fill_(-7)
        torch.cuda.synchronize()
        log(f"chain graph replay {r}")
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(np_i(acc), eager[0]) and np.array_equal(np_i(alen), eager[1]), r
        assert not bool((ws != 0).any().item())
        # eager work between replays, on the same workspace
        a2, l2 = sv.chain_reject(*args, workspace=ws)
        assert np.array_equal(np_i(a2), eager[0])


def _ragged_pack(c, lens):
    """Packed target rows and qo_indptr from a dense fuzz case and per-request lengths."""
    p = c["target_probs"]
    rows = np.concatenate([p[b, :n] for b, n in enumerate(lens)], axis=0)
    ind = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return np.ascontiguousarray(rows), ind


def test_chain_reject_ragged(sv):
    """Per-request verify lengths over packed target rows, with and without
    draft probabilities, on split rows and one workgroup per request, aligned
    and unaligned V, degenerate rows, all lengths 1, invalid lengths, and a
    request subset."""
    torch = __import__("torch")
    flagged = 0
    cases = [(6, 3, 1000, None), (5, 4, 32000, None), (6, 2, 4097, "zeros"), (7, 5, 3001, "disjoint"),
             (300, 5, 20000, None), (260, 3, 5003, None), (258, 4, 8192, "onehot"), (256, 2, 4096, "len1")]
    for i, (B, D, V, sp) in enumerate(cases):
        c = fuzz_case(1300 + i, B, D, V, "f32", special=None if sp == "len1" else sp)
        rng = np.random.default_rng(1300 + i)
        lens = np.ones(B, np.int64) if sp == "len1" else rng.integers(1, D + 2, B)
        if sp is None and i % 2 == 0:
            # drafts at each row's most likely token half of the time, so long acceptances happen
            c["draft_ids"] = np.where(rng.random((B, D)) < 0.5, c["target_probs"][:, :D].argmax(-1),
                                      c["draft_ids"]).astype(np.int32)
        rows, ind = _ragged_pack(c, lens)
        if i == 1:
            ind[2] = ind[1]                    # request 1: length 0 (request 2 then reads past its rows)
        for q in (c["draft_probs"], None):
            log(f"chain ragged {i}: B={B} D={D} V={V} special={sp} draft_probs={q is not None}")
            ref = oracle.chain_reject_ragged(q, c["draft_ids"], rows, ind, c["seed"], c["offset"])
            acc, acc_full = guarded_i32((B, D + 1))
            alen, alen_full = guarded_i32((B,))
            sv.chain_reject_ragged(None if q is None else dev(q), dev(c["draft_ids"]), dev(rows), dev(ind),
                                   dev(c["seed"]), dev(c["offset"]), out=(acc, alen))
            flagged += assert_chain_match(np_i(acc), np_i(alen), ref, range(B), (B, D, V, sp, q is not None))
            assert guard_intact(acc_full, B * (D + 1)) and guard_intact(alen_full, B)
    # request subset on the one-workgroup path: other rows untouched
    B, D, V = 300, 4, 12288
    c = fuzz_case(1399, B, D, V, "f32")
    lens = np.random.default_rng(9).integers(1, D + 2, B)
    rows, ind = _ragged_pack(c, lens)
    reqs = np.random.default_rng(8).permutation(B)[:270].astype(np.int32)
    log(f"chain ragged subset: B={B} D={D} V={V} n_req={len(reqs)}")
    ref = oracle.chain_reject_ragged(c["draft_probs"], c["draft_ids"], rows, ind, c["seed"], c["offset"])
    acc = torch.full((B, D + 1), SENTINEL, dtype=torch.int32, device="cuda")
    alen = torch.full((B,), SENTINEL, dtype=torch.int32, device="cuda")
    sv.chain_reject_ragged(dev(c["draft_probs"]), dev(c["draft_ids"]), dev(rows), dev(ind), dev(c["seed"]),
                           dev(c["offset"]), req_index=dev(reqs), out=(acc, alen))
    flagged += assert_chain_match(np_i(acc), np_i(alen), ref, sorted(set(reqs.tolist())), "ragged subset")
    rest = np.setdiff1d(np.arange(B), reqs)
    assert np.all(np_i(acc)[rest] == SENTINEL) and np.all(np_i(alen)[rest] == SENTINEL)
    log(f"chain ragged flagged requests: {flagged}")


def test_chain_reject_ragged_large_vocab_full(sv):
    """The large-vocab workload with per-request verify lengths drawn from {1..D+1}."""
    from workloads import make_ragged_config
    c = make_ragged_config()
    B, D, V = c["B"], c["D"], c["V"]
    log(f"chain ragged large vocab: B={B} D={D} V={V} rows={c['target_rows'].shape[0]}")
    ref = oracle.chain_reject_ragged(c["draft_probs"], c["draft_ids"], c["target_rows"], c["qo_indptr"], c["seed"],
                                     c["offset"])
    acc, alen = sv.chain_reject_ragged(dev(c["draft_probs"]), dev(c["draft_ids"]), dev(c["target_rows"]),
                                       dev(c["qo_indptr"]), dev(c["seed"]), dev(c["offset"]))
    flagged = assert_chain_match(np_i(acc), np_i(alen), ref, range(B), "ragged large vocab")
    log(f"ragged large vocab: mean accept length {np_i(alen).mean():.3f}, flagged {flagged}")


def test_d2t_expand(sv):
    """Draft -> target placement, bit-exact, through the inverse table:
    ascending and shuffled tables, negative offsets, no table, odd and
    unaligned row lengths."""
    torch = __import__("torch")
    from workloads import make_d2t
    rng = np.random.default_rng(1401)
    for i, (rows, Vd, V, kind) in enumerate([(7, 100, 1000, "sorted"), (5, 999, 1003, "shuffled"),
                                             (3, 1000, 1000, "shuffled"), (6, 37, 4097, None),
                                             (1280, 3200, 12826, "sorted"), (4, 32000, 128256, "sorted"),
                                             (1281, 3200, 12824, "shuffled"), (37, 32000, 128256, "sorted")]):
        q = rng.random((rows, Vd)).astype(np.float32)
        d2t = None if kind is None else make_d2t(i, Vd, V, shuffled=kind == "shuffled")
        log(f"d2t expand {i}: rows={rows} Vd={Vd} V={V} table={kind}")
        ref = oracle.d2t_expand(q, d2t, V)
        t2d = sv.d2t_inverse(None if d2t is None else dev(d2t), Vd, V, device="cuda")
        want = np.full(V, -1, np.int64)
        want[np.arange(Vd) if d2t is None else (np.arange(Vd) + d2t) % V] = np.arange(Vd)
        assert np.array_equal(np_i(t2d).astype(np.int64), want), i
        out = sv.d2t_expand(dev(q), t2d)
        assert np.array_equal(out.cpu().numpy(), ref), i
    # an output row view that is not 16-byte aligned, guard bands intact
    rows, Vd, V = 4, 300, 1001
    q = rng.random((rows, Vd)).astype(np.float32)
    d2t = make_d2t(9, Vd, V)
    flat = torch.full((rows * V + 6,), 7.0, device="cuda")
    out = flat[3:3 + rows * V].view(rows, V)
    log(f"d2t expand unaligned output: rows={rows} Vd={Vd} V={V}")
    sv.d2t_expand(dev(q), sv.d2t_inverse(dev(d2t), Vd, V), out=out)
    assert np.array_equal(out.cpu().numpy(), oracle.d2t_expand(q, d2t, V))
    f = flat.cpu().numpy()
    assert np.all(f[:3] == 7.0) and np.all(f[3 + rows * V:] == 7.0)
    # an aligned output view (column tiles, a partial last tile) inside guard bands
    rows, Vd, V = 9, 3000, 5004
    q = rng.random((rows, Vd)).astype(np.float32)
    d2t = make_d2t(10, Vd, V, shuffled=True)
    flat = torch.full((rows * V + 8,), 7.0, device="cuda")
    out = flat[4:4 + rows * V].view(rows, V)
    log(f"d2t expand aligned view in guard bands: rows={rows} Vd={Vd} V={V}")
    sv.d2t_expand(dev(q), sv.d2t_inverse(dev(d2t), Vd, V), out=out)
    assert np.array_equal(out.cpu().numpy(), oracle.d2t_expand(q, d2t, V))
    f = flat.cpu().numpy()
    assert np.all(f[:4] == 7.0) and np.all(f[4 + rows * V:] == 7.0)


def test_d2t_shared_targets(sv):
    """A table whose draft entries share targets: the inverse table keeps the
    highest-numbered draft entry per target (the oracle's in-order scatter),
    on every launch, and the expansion matches the oracle's placement."""
    rng = np.random.default_rng(1402)
    for Vd, V in ((50, 60), (3000, 3000), (20000, 25000)):
        tgt = rng.integers(0, V, Vd)
        d2t = (tgt - np.arange(Vd)).astype(np.int64)
        q = rng.random((4, Vd)).astype(np.float32)
        log(f"d2t shared targets: Vd={Vd} V={V}")
        want = np.full(V, -1, np.int64)
        np.maximum.at(want, tgt, np.arange(Vd))
        for rep in range(3):
            t2d = sv.d2t_inverse(dev(d2t), Vd, V)
            assert np.array_equal(np_i(t2d), want), (Vd, V, rep)
        out = sv.d2t_expand(dev(q), t2d)
        assert np.array_equal(out.cpu().numpy(), oracle.d2t_expand(q, d2t, V)), (Vd, V)


def test_ragged_verify_with_reduced_draft_vocab(sv):
    """The reduced-vocabulary drafter end to end: d2t placement then the
    ragged chain verify, and the verify reading the draft rows through the
    inverse table, against the oracle's placement and ragged verify; split
    and one-workgroup rows, aligned and odd V.  Draft rows that fit LDS are
    staged there when a workgroup covers at least Vd target entries: an odd
    Vd (unaligned draft rows, copied entry by entry), a shuffled table, Vd at
    the staging limit (38400) and one past it (gathered from global memory)."""
    from workloads import make_d2t
    for B, D, Vd, V, shuffled in ((6, 3, 300, 1000, False), (260, 4, 3200, 12288, False), (5, 2, 333, 1001, False),
                                  (257, 3, 5000, 20001, False), (258, 3, 1003, 4096, False),
                                  (260, 3, 3000, 12288, True), (256, 1, 38400, 40000, False),
                                  (256, 1, 38401, 40000, True)):
        rng = np.random.default_rng(B + V)
        c = fuzz_case(1500 + B, B, D, V, "f32")
        d2t = make_d2t(B, Vd, V, shuffled)
        tgt = (np.arange(Vd) + d2t) % V
        # draft distributions over the draft vocabulary: the fuzz draft rows restricted to the mapped ids
        qd = c["draft_probs"][:, :, tgt].astype(np.float64)
        qd = (qd / qd.sum(-1, keepdims=True)).astype(np.float32)
        x = tgt[rng.integers(0, Vd, (B, D))].astype(np.int32)          # draft ids are target ids
        lens = rng.integers(1, D + 2, B)
        rows, ind = _ragged_pack(c, lens)
        log(f"ragged verify with a reduced draft vocabulary: B={B} D={D} Vd={Vd} V={V} shuffled={shuffled}")
        q_full = oracle.d2t_expand(qd, d2t, V)
        ref = oracle.chain_reject_ragged(q_full, x, rows, ind, c["seed"], c["offset"])
        t2d = sv.d2t_inverse(dev(d2t), Vd, V)
        qg = sv.d2t_expand(dev(qd), t2d)
        acc, alen = sv.chain_reject_ragged(qg, dev(x), dev(rows), dev(ind), dev(c["seed"]), dev(c["offset"]))
        assert_chain_match(np_i(acc), np_i(alen), ref, range(B), (B, D, Vd, V, "expanded"))
        # the same verify reading the draft rows through t2d, with nothing expanded
        acc, alen = sv.chain_reject_ragged(dev(qd), dev(x), dev(rows), dev(ind), dev(c["seed"]), dev(c["offset"]),
                                           t2d=t2d)
        assert_chain_match(np_i(acc), np_i(alen), ref, range(B), (B, D, Vd, V, "through t2d"))


def _sample_params(rng, B, V):
    T = rng.uniform(0.4, 1.3, B).astype(np.float32)
    T[rng.random(B) < 0.15] = 0.0                                            # greedy rows
    k = np.where(rng.random(B) < 0.5, rng.choice([1, 2, 5, 20, 100, V, V + 3], B), 0).astype(np.int32)
    tp = np.where(rng.random(B) < 0.6, rng.uniform(0.0, 1.0, B), 1.0).astype(np.float32)
    mp = np.where(rng.random(B) < 0.4, rng.choice([0.001, 0.02, 0.1, 0.5, 1.0, 1.5], B), 0.0).astype(np.float32)
    return T, k, tp, mp


def test_sample_fuzz(sv):
    """Single-step sampling against the oracle: f32 and bf16 rows, greedy
    rows, every filter alone and together (k = 1, k >= V, top_p 0, min_p >= 1),
    ties, all-zero rows, odd V, optional parameter arrays absent."""
    flagged = 0
    for i, (B, V, dt, sp) in enumerate([(40, 1000, "f32", None), (40, 1000, "bf16", None), (33, 4097, "bf16", "ties"),
                                        (20, 32000, "bf16", None), (17, 3001, "f32", "zeros"), (9, 7, "f32", None),
                                        (12, 129280, "bf16", None), (8, 1, "bf16", None)]):
        c = fuzz_case(1600 + i, B, 0, V, dt, special=sp)
        z = c["logits"][:, 0]
        rng = np.random.default_rng(1600 + i)
        T, k, tp, mp = _sample_params(rng, B, V)
        for opt in ((k, tp, mp), (None, None, None), (k, None, mp)):
            log(f"sample fuzz {i}: B={B} V={V} dtype={dt} special={sp} filters={[o is not None for o in opt]}")
            ref = oracle.sample(z, dt, T, opt[0], opt[1], opt[2], c["seed"], c["offset"])
            tok = sv.sample(dev_logits(np.ascontiguousarray(z), dt), dev(T), dev(c["seed"]), dev(c["offset"]),
                            top_k=None if opt[0] is None else dev(opt[0]),
                            top_p=None if opt[1] is None else dev(opt[1]),
                            min_p=None if opt[2] is None else dev(opt[2]))
            got = np_i(tok)
            ok = (got == ref["tokens"]) | ref["flagged"]
            assert np.all(ok), (i, np.nonzero(~ok)[0], got[~ok], ref["tokens"][~ok])
            flagged += int(ref["flagged"].sum())
    log(f"sample flagged rows: {flagged}")


def test_sample_mixed_batch_and_subset(sv):
    """The mixed workload's rows (B=1024, V=129280 bf16), sampled through a
    request subset; rows outside it are untouched."""
    torch = __import__("torch")
    from workloads import make_sample_config
    c = make_sample_config()
    B, V = c["logits"].shape
    reqs = np.random.default_rng(3).permutation(B)[:200].astype(np.int32)
    log(f"sample mixed batch: B={B} V={V} n_req={len(reqs)}")
    ref = oracle.sample(c["logits"], "bf16", c["temperature"], c["top_k"], c["top_p"], c["min_p"], c["seed"],
                        c["offset"], requests=reqs)
    out = torch.full((B,), SENTINEL, dtype=torch.int32, device="cuda")
    sv.sample(dev_logits(c["logits"], "bf16"), dev(c["temperature"]), dev(c["seed"]), dev(c["offset"]),
              top_k=dev(c["top_k"]), top_p=dev(c["top_p"]), min_p=dev(c["min_p"]), req_index=dev(reqs), out=out)
    got = np_i(out)
    ok = (got[reqs] == ref["tokens"][reqs]) | ref["flagged"][reqs]
    assert np.all(ok), np.nonzero(~ok)
    rest = np.setdiff1d(np.arange(B), reqs)
    assert np.all(got[rest] == SENTINEL)


def test_ragged_verify_reduced_vocab_large(sv):
    """The large-vocab ragged workload with a 32000-entry draft vocabulary,
    the draft rows read through the inverse table."""
    from workloads import make_ragged_d2t_config
    c = make_ragged_d2t_config()
    B, D, V = c["B"], c["D"], c["V"]
    Vd = c["draft_probs_d"].shape[-1]
    log(f"ragged verify through t2d, large vocab: B={B} D={D} Vd={Vd} V={V}")
    q_full = oracle.d2t_expand(c["draft_probs_d"], c["d2t"], V)
    ref = oracle.chain_reject_ragged(q_full, c["draft_ids"], c["target_rows"], c["qo_indptr"], c["seed"],
                                     c["offset"])
    t2d = sv.d2t_inverse(dev(c["d2t"]), Vd, V)
    acc, alen = sv.chain_reject_ragged(dev(c["draft_probs_d"]), dev(c["draft_ids"]), dev(c["target_rows"]),
                                       dev(c["qo_indptr"]), dev(c["seed"]), dev(c["offset"]), t2d=t2d)
    flagged = assert_chain_match(np_i(acc), np_i(alen), ref, range(B), "ragged through t2d")
    log(f"mean accept length {np_i(alen).mean():.3f}, flagged {flagged}")


def test_chain_reject_request_subset_and_determinism(sv):
    B, D, V = 9, 4, 3001
    c = fuzz_case(91, B, D, V, "f32")
    args = [dev(c["draft_probs"]), dev(c["draft_ids"]), dev(c["target_probs"]), dev(c["seed"]), dev(c["offset"])]
    log("chain subset/determinism")
    acc1, len1 = sv.chain_reject(*args)
    acc2, len2 = sv.chain_reject(*args)
    assert np.array_equal(np_i(acc1), np_i(acc2)) and np.array_equal(np_i(len1), np_i(len2))
    reqs = np.array([7, 2, 5], np.int32)
    acc3, acc3_full = guarded_i32((B, D + 1))
    acc3.fill_(SENTINEL)
    len3, _ = guarded_i32((B,))
    len3.fill_(SENTINEL)
    sv.chain_reject(*args, req_index=dev(reqs), out=(acc3, len3))
    a3, l3 = np_i(acc3), np_i(len3)
    for b in range(B):
        if b in reqs:
            assert np.array_equal(a3[b], np_i(acc1)[b]) and l3[b] == np_i(len1)[b]
        else:
            assert np.all(a3[b] == SENTINEL) and l3[b] == SENTINEL
    # a request's draws follow its own (seed, offset), not its batch position
    perm = np.array([3, 0, 8, 1, 6, 2, 5, 7, 4])
    pargs = [dev(c["draft_probs"][perm]), dev(c["draft_ids"][perm]), dev(c["target_probs"][perm]),
             dev(c["seed"][perm]), dev(c["offset"][perm])]
    acc4, len4 = sv.chain_reject(*pargs)
    assert np.array_equal(np_i(acc4), np_i(acc1)[perm]) and np.array_equal(np_i(len4), np_i(len1)[perm])


def test_chain_reject_config3_full(sv):
    """The large-vocab batch in full, at the four Philox offsets the benchmark
    rotates through (4096 r): every accept length exact, every token exact
    outside the double-sum exclusion band; the 1e-6 CDF category is counted."""
    c = make_config(3)
    B, D, V = 256, 5, 128256
    args = [dev(c["draft_probs"]), dev(c["draft_ids"]), dev(c["target_probs"]), dev(c["seed"])]
    near, excl, Ls = 0, 0, []
    for r in range(4):
        off = np.full(B, 4096 * r, np.uint64)
        log(f"chain config 3 full: B=256 D=5 V=128256 f32, offset {4096 * r}")
        ref = oracle.chain_reject(c["draft_probs"], c["draft_ids"], c["target_probs"], c["seed"], off)
        acc, alen = sv.chain_reject(*args, dev(off))
        excl += assert_chain_match(np_i(acc), np_i(alen), ref, range(B), ("cfg3", r), max_excluded=1)
        near += int(ref["near_cdf"].sum())
        Ls.append(np_i(alen))
    L = np.concatenate(Ls)
    log(f"config 3: mean L={L.mean():.3f} P(L=D)={np.mean(L == D):.3f} within 1e-6 of a CDF boundary={near} "
        f"excluded={excl} of {4 * B}")
    assert 2.0 < L.mean() < 4.5


# --------------------------------------------------------------------------- softmax + top-k/top-p
SOFTMAX_CASES = [
    (V, dt, T, k, p)
    for V in (1, 7, 100, 1001, 32000)
    for dt in ("f32", "bf16")
    for (T, k, p) in ((1.0, 0, 1.0), (0.7, 50, 0.9), (0.0, 0, 1.0), (1.3, 5, 1.0), (0.5, 0, 0.8),
                      (0.9, 1, 0.5), (1.1, V - 1, 0.95), (0.8, V, 0.3), (2.0, 0, 0.0), (0.6, 3, 0.99))
]


def assert_probs_match(gpu, ref, flags, ctx):
    ok_rows = ~flags
    g, r = gpu[ok_rows], ref[ok_rows]
    err = np.abs(g - r).max() if g.size else 0.0
    assert err <= PROB_ATOL, (ctx, err)
    # kept sets: zero exactly where the oracle is zero; non-zero where the oracle is not negligible
    assert np.all(g[r == 0] == 0), ctx
    assert np.all(g[r > 1e-30] > 0), ctx
    return int(flags.sum())


def test_softmax_renorm_fuzz(sv):
    flagged = 0
    for i, (V, dt, T, k, p) in enumerate(SOFTMAX_CASES):
        B, npos = 3, 2
        c = fuzz_case(300 + i, B, npos - 1, V, dt, special="ties" if i % 3 == 0 else None)
        Ts = np.array([T, T * 1.1 if T > 0 else 0.0, T], np.float32)
        ks = np.array([k, k, 0], np.int32)
        ps = np.array([p, p, p], np.float32)
        log(f"softmax fuzz {i}: V={V} dtype={dt} T={T} k={k} top_p={p}")
        ref, fl = oracle.softmax_renorm(c["logits"], dt, Ts, ks, ps)
        out = sv.softmax_renorm(dev_logits(c["logits"], dt), dev(Ts), dev(ks), dev(ps))
        flagged += assert_probs_match(out.cpu().numpy().astype(np.float64), ref, fl, (V, dt, T, k, p))
    log(f"softmax fuzz flagged rows: {flagged}")


# bf16 rows held in registers: every register-count variant (V a multiple of
# 8), rows of odd V (redone by the streamed algorithm),
# a row whose most common value overflows a 16-bit histogram counter (redone by
# the streamed algorithm), a key span too wide for the probability table, and
# signed zeros at a top-k threshold.
RR_CASES = [
    (4096, "ties", ((1.0, 0, 1.0), (0.8, 100, 0.9), (1.2, 0, 0.6), (0.7, 3, 1.0))),
    (8200, None, ((1.0, 0, 1.0), (0.8, 100, 0.9), (1.2, 0, 0.6), (0.0, 0, 1.0))),
    (8193, None, ((1.0, 0, 1.0), (0.8, 100, 0.9), (1.2, 0, 0.6), (0.0, 0, 1.0))),
    (40000, "ties", ((1.0, 0, 1.0), (0.8, 100, 0.9), (1.2, 7, 0.6), (0.0, 0, 1.0))),
    (100000, None, ((1.0, 0, 1.0), (0.8, 20, 0.95), (1.2, 0, 0.8), (0.0, 0, 1.0))),
    (100003, None, ((1.0, 0, 1.0), (0.8, 20, 0.95), (1.2, 0, 0.8), (0.9, 0, 0.7))),
    (129280, None, ((0.7, 0, 1.0), (0.8, 100, 1.0), (1.1, 0, 0.9), (0.9, 50, 0.5))),
    (150000, None, ((1.0, 0, 1.0), (0.8, 100, 0.9), (1.2, 0, 0.6), (0.5, 30000, 0.99))),
    (80000, "mostly_zero", ((1.0, 0, 1.0), (0.8, 100, 0.9), (1.0, 20000, 1.0), (1.2, 0, 0.3))),
    (140000, "mostly_zero", ((1.0, 0, 1.0), (0.8, 100, 0.9), (1.0, 20000, 0.99), (0.0, 0, 1.0))),
    (50000, "wide", ((3e3, 0, 1.0), (1e4, 500, 0.9), (5e4, 0, 0.7), (2e3, 0, 1.0))),
    (20000, "signed_zeros", ((1.0, 7000, 1.0), (0.5, 7000, 0.9), (2.0, 0, 0.5), (0.0, 0, 1.0))),
]


def test_softmax_register_resident_paths(sv):
    flagged = 0
    for i, (V, special, modes) in enumerate(RR_CASES):
        c = fuzz_case(700 + i, 4, 1, V, "bf16", special=special)
        Ts = np.array([m[0] for m in modes], np.float32)
        ks = np.array([m[1] for m in modes], np.int32)
        ps = np.array([m[2] for m in modes], np.float32)
        log(f"register-resident softmax {i}: V={V} special={special}")
        ref, fl = oracle.softmax_renorm(c["logits"], "bf16", Ts, ks, ps)
        out = sv.softmax_renorm(dev_logits(c["logits"], "bf16"), dev(Ts), dev(ks), dev(ps))
        flagged += assert_probs_match(out.cpu().numpy().astype(np.float64), ref, fl, (V, special))
    log(f"register-resident softmax flagged rows: {flagged}")


def test_softmax_renorm_optional_filters_and_subset(sv):
    torch = __import__("torch")
    B, npos, V = 5, 3, 2000
    c = fuzz_case(333, B, npos - 1, V, "bf16")
    T = np.array([1.0, 0.5, 0.0, 2.0, 0.8], np.float32)
    log("softmax without top_k/top_p arrays, and via req_index")
    ref, fl = oracle.softmax_renorm(c["logits"], "bf16", T)
    out = sv.softmax_renorm(dev_logits(c["logits"], "bf16"), dev(T))
    assert_probs_match(out.cpu().numpy().astype(np.float64), ref, fl, "no filters")
    full = torch.full((B, npos, V), -3.0, device="cuda")
    sv.softmax_renorm(dev_logits(c["logits"], "bf16"), dev(T), req_index=dev(np.array([4, 1], np.int32)), out=full)
    f = full.cpu().numpy()
    assert np.array_equal(f[[4, 1]], out.cpu().numpy()[[4, 1]])
    assert np.all(f[[0, 2, 3]] == -3.0)


def test_softmax_then_chain_config2_full(sv):
    c = make_config(2)
    B, D, V = 64, 3, 32000
    log("config 2 full: softmax_renorm(T=0.7, k=50, p=0.9) -> chain_reject, bf16 V=32000")
    z = dev_logits(c["logits"], "bf16")
    probs = sv.softmax_renorm(z, dev(c["temperature"]), dev(c["top_k"]), dev(c["top_p"]))
    ref, fl = oracle.softmax_renorm(c["logits"], "bf16", c["temperature"], c["top_k"], c["top_p"])
    g = probs.cpu().numpy()
    n_flag = assert_probs_match(g.astype(np.float64), ref, fl, "cfg2")
    kept = (g > 0).sum(-1)
    log(f"config 2: kept per row mean={kept.mean():.2f} flagged rows={n_flag}")
    acc, alen = sv.chain_reject(dev(c["draft_probs"]), dev(c["draft_ids"]), probs, dev(c["seed"]), dev(c["offset"]))
    # stage parity: the oracle chain on the GPU's own probabilities
    ref_c = oracle.chain_reject(c["draft_probs"], c["draft_ids"], g, c["seed"], c["offset"])
    assert_chain_match(np_i(acc), np_i(alen), ref_c, range(B), "cfg2 stage")
    # end to end: the oracle chain on the oracle's probabilities (near-threshold accepts flagged)
    ref_e = oracle.chain_reject(c["draft_probs"], c["draft_ids"], ref, c["seed"], c["offset"],
                                cdf_band=oracle.CDF_BAND)
    ok = [b for b in range(B) if not fl[b].any() and ref_e["near_accept"][b] < 0]
    assert_chain_match(np_i(acc), np_i(alen), ref_e, ok, "cfg2 end-to-end")
    log(f"config 2: mean L={np_i(alen).mean():.3f}")


def test_config1_end_to_end(sv):
    c = make_config(1)
    B, D, V = 4, 3, 1000
    log("config 1: softmax(T=1) -> chain_reject, and greedy verify")
    probs = sv.softmax_renorm(dev_logits(c["logits"], "f32"), dev(c["temperature"]))
    ref, fl = oracle.softmax_renorm(c["logits"], "f32", c["temperature"])
    assert_probs_match(probs.cpu().numpy().astype(np.float64), ref, fl, "cfg1")
    acc, alen = sv.chain_reject(dev(c["draft_probs"]), dev(c["draft_ids"]), probs, dev(c["seed"]), dev(c["offset"]))
    ref_c = oracle.chain_reject(c["draft_probs"], c["draft_ids"], probs.cpu().numpy(), c["seed"], c["offset"])
    assert_chain_match(np_i(acc), np_i(alen), ref_c, range(B), "cfg1 stage")
    g = sv.greedy_verify(dev_logits(c["logits"], "f32"), dev(c["greedy_draft_ids"]), argmax=True)
    rg = oracle.greedy_verify(c["logits"], "f32", c["greedy_draft_ids"])
    for k in ("accepted_tokens", "accept_length", "predict", "accept_index", "argmax"):
        assert np.array_equal(np_i(g[k]), rg[k]), k


# --------------------------------------------------------------------------- Gumbel-max
GUMBEL_CASES = [(V, D, dt) for V in (1, 3, 100, 1001, 32000) for D in (0, 1, 3, 7) for dt in ("f32", "bf16")]


def test_gumbel_sample_fuzz(sv):
    rng = np.random.default_rng(400)
    flagged = 0
    for i, (V, D, dt) in enumerate(GUMBEL_CASES):
        B = 6
        c = fuzz_case(400 + i, B, D, V, dt)
        T = np.array([0.7, 1.0, 0.0, 1.5, 0.3, 1e-6], np.float32)
        log(f"gumbel fuzz {i}: V={V} D={D} dtype={dt}")
        # drafts: the oracle's own samples with probability 0.8 so chains run deep
        full = oracle.gumbel_sample(c["logits"], dt, T, np.zeros((B, D), np.int32), c["seed"], c["offset"],
                                    all_rows=True)
        x = np.where(rng.random((B, D)) < 0.8, full["sampled"][:, :D], rng.integers(0, V, size=(B, D)))
        x = x.astype(np.int32)
        ref = oracle.gumbel_sample(c["logits"], dt, T, x, c["seed"], c["offset"], all_rows=True)
        out = sv.gumbel_sample(dev_logits(c["logits"], dt), dev(T), dev(x), dev(c["seed"]), dev(c["offset"]),
                               sampled=True)
        s_gpu = np_i(out["sampled"])
        for b in range(B):
            fp = int(ref["flag_pos"][b])
            assert list(s_gpu[b, :fp]) == list(ref["sampled"][b, :fp]), (V, D, dt, b, s_gpu[b], ref["sampled"][b])
            flagged += fp < D + 1
        assert_chain_match(np_i(out["accepted_tokens"]), np_i(out["accept_length"]), ref, range(B), (V, D, dt),
                           len_exact=False, max_excluded=B)
        out2 = sv.gumbel_sample(dev_logits(c["logits"], dt), dev(T), dev(x), dev(c["seed"]), dev(c["offset"]))
        assert np.array_equal(np_i(out2["accepted_tokens"]), np_i(out["accepted_tokens"]))
        # the one-workgroup-per-request form computes the same rows
        for smp in (True, False):
            out3 = sv.gumbel_sample(dev_logits(c["logits"], dt), dev(T), dev(x), dev(c["seed"]), dev(c["offset"]),
                                    sampled=smp, workspace=False)
            assert np.array_equal(np_i(out3["accepted_tokens"]), np_i(out["accepted_tokens"]))
            assert np.array_equal(np_i(out3["accept_length"]), np_i(out["accept_length"]))
            if smp:
                assert np.array_equal(np_i(out3["sampled"]), s_gpu)
    log(f"gumbel fuzz flagged requests: {flagged}")


def test_gumbel_staged_many_continuing(sv):
    """The staged Gumbel form when most requests continue past row 0 (drafts
    are the oracle's own samples, so chains run to the bonus row): the
    helpers then take whole later rows, not pieces.  Against the oracle and
    the one-workgroup-per-request form, two calls on one workspace, which is
    zero afterwards."""
    torch = __import__("torch")
    B, D, V = 96, 7, 8192
    c = fuzz_case(470, B, D, V, "bf16")
    rng = np.random.default_rng(470)
    T = rng.uniform(0.5, 1.5, B).astype(np.float32)
    T[::7] = 0.0   # some greedy rows among them
    full = oracle.gumbel_sample(c["logits"], "bf16", T, np.zeros((B, D), np.int32), c["seed"], c["offset"],
                                all_rows=True)
    x = np.where(rng.random((B, D)) < 0.95, full["sampled"][:, :D], rng.integers(0, V, size=(B, D))).astype(np.int32)
    ref = oracle.gumbel_sample(c["logits"], "bf16", T, x, c["seed"], c["offset"], all_rows=True)
    ws = torch.zeros((sv.gumbel_sample_workspace_bytes(B, D),), dtype=torch.uint8, device="cuda")
    args = (dev_logits(c["logits"], "bf16"), dev(T), dev(x), dev(c["seed"]), dev(c["offset"]))
    log(f"gumbel staged, many continuing: B={B} D={D} V={V}")
    for _ in range(2):
        out = sv.gumbel_sample(*args, workspace=ws)
        torch.cuda.synchronize()
        assert int(ws.count_nonzero()) == 0
        assert_chain_match(np_i(out["accepted_tokens"]), np_i(out["accept_length"]), ref, range(B), (V, D),
                           len_exact=False, max_excluded=B)
        per = sv.gumbel_sample(*args, workspace=False)
        assert np.array_equal(np_i(per["accepted_tokens"]), np_i(out["accepted_tokens"]))
        assert np.array_equal(np_i(per["accept_length"]), np_i(out["accept_length"]))
    assert float(np.mean(np_i(out["accept_length"]))) > 3.0   # most chains run deep


# --------------------------------------------------------------------------- config 5 (mixed modes)
def test_config5_mixed_modes_full(sv):
    """The mixed batch (B=1024 D=7 V=129280 bf16), each mode through
    req_index into shared outputs, compared with the oracle for every
    request: all 256 greedy requests, all 256 Gumbel requests, the chain
    stage of all 512 top-k/top-p requests on the GPU's probabilities, and the
    renormalised probabilities of 128 of those requests (every row)."""
    torch = __import__("torch")
    c = make_config(5)
    B, D, V = 1024, 7, 129280
    N = D + 1
    modes = c["modes"]
    log("config 5 full launch: B=1024 D=7 V=129280 bf16, each mode via req_index")
    z = dev_logits(c["logits"], "bf16")
    T = dev(c["temperature"])
    x = dev(c["draft_ids"])
    seed, off = dev(c["seed"]), dev(c["offset"])
    idx = {m: np.nonzero(modes == m)[0].astype(np.int32) for m in range(4)}
    acc = torch.full((B, N), SENTINEL, dtype=torch.int32, device="cuda")
    alen = torch.full((B,), SENTINEL, dtype=torch.int32, device="cuda")
    sv.greedy_verify(z, x, req_index=dev(idx[MODE_GREEDY]), predict=False, accept_index=False,
                     out={"accepted_tokens": acc, "accept_length": alen})
    sv.gumbel_sample(z, T, x, seed, off, req_index=dev(idx[MODE_TEMPERATURE]),
                     out={"accepted_tokens": acc, "accept_length": alen})
    filt = np.concatenate([idx[MODE_TOPK], idx[MODE_TOPP]]).astype(np.int32)
    probs = torch.zeros((B, N, V), dtype=torch.float32, device="cuda")
    sv.softmax_renorm(z, T, dev(c["top_k"]), dev(c["top_p"]), req_index=dev(filt), out=probs)
    sv.chain_reject(dev(c["draft_probs"]), x, probs, seed, off, req_index=dev(filt), out=(acc, alen))
    A, Ls = np_i(acc), np_i(alen)
    # greedy and Gumbel in their one-workgroup-per-request form: identical outputs
    acc1 = torch.full((B, N), SENTINEL, dtype=torch.int32, device="cuda")
    alen1 = torch.full((B,), SENTINEL, dtype=torch.int32, device="cuda")
    sv.greedy_verify(z, x, req_index=dev(idx[MODE_GREEDY]), predict=False, accept_index=False,
                     out={"accepted_tokens": acc1, "accept_length": alen1}, workspace=False)
    sv.gumbel_sample(z, T, x, seed, off, req_index=dev(idx[MODE_TEMPERATURE]),
                     out={"accepted_tokens": acc1, "accept_length": alen1}, workspace=False)
    both = np.concatenate([idx[MODE_GREEDY], idx[MODE_TEMPERATURE]])
    assert np.array_equal(np_i(acc1)[both], A[both]) and np.array_equal(np_i(alen1)[both], Ls[both])
    assert np.all((Ls >= 0) & (Ls <= D))
    for b in range(B):
        assert np.all(A[b, Ls[b] + 1:] == -1) and np.all(A[b, :Ls[b] + 1] >= 0)
    log("config 5: greedy requests against the oracle (256)")
    rg = oracle.greedy_verify(c["logits"], "bf16", c["draft_ids"], requests=idx[MODE_GREEDY])
    for b in idx[MODE_GREEDY]:
        assert list(A[b]) == list(rg["accepted_tokens"][b]) and Ls[b] == rg["accept_length"][b], b
    log("config 5: Gumbel requests against the oracle (256)")
    ru = oracle.gumbel_sample(c["logits"], "bf16", c["temperature"], c["draft_ids"], c["seed"], c["offset"],
                              requests=idx[MODE_TEMPERATURE])
    ng = assert_chain_match(A, Ls, ru, idx[MODE_TEMPERATURE], "cfg5 gumbel", len_exact=False, max_excluded=3)
    log("config 5: chain stage against the oracle on the GPU's probabilities (512)")
    gp = probs.cpu().numpy()
    rc = oracle.chain_reject(c["draft_probs"], c["draft_ids"], gp, c["seed"], c["offset"], requests=filt)
    nc = assert_chain_match(A, Ls, rc, filt, "cfg5 chain stage", max_excluded=1)
    sreq = np.concatenate([idx[MODE_TOPK][:64], idx[MODE_TOPP][:64]])
    log(f"config 5: renormalised probabilities against the oracle ({len(sreq)} requests x {N} rows)")
    rp, fl = oracle.softmax_renorm(c["logits"], "bf16", c["temperature"], c["top_k"], c["top_p"], requests=sreq)
    nf = assert_probs_match(gp[sreq].astype(np.float64), rp, fl, "cfg5 softmax")
    log(f"config 5: excluded Gumbel near ties {ng}, excluded CDF draws {nc}, "
        f"within 1e-6 of a CDF boundary {int(rc['near_cdf'][filt].sum())}, top-p flagged rows {nf}")
    for m, name in ((MODE_GREEDY, "greedy"), (MODE_TEMPERATURE, "temperature"), (MODE_TOPK, "top-k"),
                    (MODE_TOPP, "top-p")):
        log(f"config 5 {name}: mean L={Ls[idx[m]].mean():.3f}")
