"""GPU parity of the fused target-rows + chain-rejection call.

Each case is checked two ways: against the oracle (bit-exact tokens and
accept lengths outside the oracle's flagged positions), and against the
library's own two-call form, softmax_renorm followed by chain_reject on the
same inputs, which must give identical outputs for every request.
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import SENTINEL, dev, dev_logits, guard_intact, guarded_i32, log, np_i
from workloads import MODE_TOPK, MODE_TOPP, fuzz_case, make_config

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sv():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import token_sampling_temp_amd as m
    m.lib()
    return m


def assert_match(gpu_tok, gpu_len, ref, reqs, ctx):
    flagged = 0
    for b in reqs:
        L = int(ref["accept_length"][b])
        fp = int(ref["flag_pos"][b])
        n = min(fp, L + 1)
        if fp > L:
            assert int(gpu_len[b]) == L, (ctx, b, int(gpu_len[b]), L)
        assert list(gpu_tok[b, :n]) == list(ref["accepted_tokens"][b, :n]), (ctx, b, gpu_tok[b],
                                                                            ref["accepted_tokens"][b])
        if int(gpu_len[b]) == L:
            assert np.all(gpu_tok[b, L + 1:] == -1), (ctx, b)
        flagged += fp <= L
    return flagged


def two_call(sv, z, T, k, p, q, x, seed, off, req=None, B=None, N=None, V=None):
    torch = __import__("torch")
    probs = torch.zeros((B, N, V), dtype=torch.float32, device="cuda")
    sv.softmax_renorm(z, T, k, p, req_index=req, out=probs)
    acc = torch.full((B, N), SENTINEL, dtype=torch.int32, device="cuda")
    alen = torch.full((B,), SENTINEL, dtype=torch.int32, device="cuda")
    sv.chain_reject(q, x, probs, seed, off, req_index=req, out=(acc, alen))
    return np_i(acc), np_i(alen)


PARAMS = ((1.0, 0, 1.0), (0.7, 50, 0.9), (0.0, 0, 1.0), (1.3, 5, 1.0), (0.5, 0, 0.8), (0.9, 1, 0.5))
FUSED_CASES = [(V, dt, D, sp) for V in (1, 7, 1000, 1001, 8192, 32000, 40001) for dt in ("f32", "bf16")
               for (D, sp) in ((0, None), (3, None), (5, "ties"), (2, "invalid_ids"))]


def test_verify_fused_fuzz(sv):
    flagged = 0
    for i, (V, dt, D, sp) in enumerate(FUSED_CASES):
        B = len(PARAMS)
        N = D + 1
        c = fuzz_case(700 + i, B, D, V, dt, special=sp)
        T = np.array([t for t, _, _ in PARAMS], np.float32)
        k = np.array([kk for _, kk, _ in PARAMS], np.int32)
        p = np.array([pp for _, _, pp in PARAMS], np.float32)
        log(f"fused fuzz {i}: V={V} dtype={dt} D={D} special={sp}")
        z = dev_logits(c["logits"], dt)
        args = (dev(T), dev(c["draft_probs"]), dev(c["draft_ids"]), dev(c["seed"]), dev(c["offset"]))
        acc, acc_full = guarded_i32((B, N))
        alen, alen_full = guarded_i32((B,))
        sv.verify_fused(z, args[0], *args[1:], top_k=dev(k), top_p=dev(p), out=(acc, alen))
        assert guard_intact(acc_full, B * N) and guard_intact(alen_full, B)
        A, Ls = np_i(acc), np_i(alen)
        ref = oracle.verify_fused(c["logits"], dt, T, k, p, c["draft_probs"], c["draft_ids"], c["seed"],
                                  c["offset"])
        flagged += assert_match(A, Ls, ref, range(B), (V, dt, D, sp))
        A2, L2 = two_call(sv, z, dev(T), dev(k), dev(p), *args[1:], B=B, N=N, V=V)
        assert np.array_equal(A, A2) and np.array_equal(Ls, L2), (V, dt, D, sp, A, A2)
    log(f"fused fuzz flagged requests: {flagged}")


def test_verify_fused_degenerate_rows(sv):
    """All-zero logits (uniform target rows), disjoint supports, one-hot drafts,
    and drafts equal to the library's own target rows (every draft accepted)."""
    torch = __import__("torch")
    for V, dt, sp in ((1000, "f32", "zeros"), (4096, "bf16", "zeros"), (3000, "f32", "disjoint"),
                      (8192, "bf16", "onehot"), (20000, "bf16", None)):
        B, D = 5, 4
        N = D + 1
        c = fuzz_case(800 + V, B, D, V, dt, special=sp)
        T = np.array([1.0, 0.8, 1.2, 0.6, 1.0], np.float32)
        k = np.array([0, 10, 0, 100, 0], np.int32)
        p = np.array([1.0, 1.0, 0.7, 0.9, 1.0], np.float32)
        z = dev_logits(c["logits"], dt)
        q = dev(c["draft_probs"])
        x = dev(c["draft_ids"])
        if sp is None:
            # drafts equal to the target rows the library computes, ids at their maxima
            probs = sv.softmax_renorm(z, dev(T), dev(k), dev(p))
            q = probs[:, :D].contiguous()
            x = probs[:, :D].argmax(-1).to(torch.int32).contiguous()
        log(f"fused degenerate: V={V} dtype={dt} special={sp}")
        acc, alen = sv.verify_fused(z, dev(T), q, x, dev(c["seed"]), dev(c["offset"]), top_k=dev(k), top_p=dev(p))
        A, Ls = np_i(acc), np_i(alen)
        A2, L2 = two_call(sv, z, dev(T), dev(k), dev(p), q, x, dev(c["seed"]), dev(c["offset"]), B=B, N=N, V=V)
        assert np.array_equal(A, A2) and np.array_equal(Ls, L2), (V, dt, sp)
        qn = q.cpu().numpy()
        xn = x.cpu().numpy()
        ref = oracle.verify_fused(c["logits"], dt, T, k, p, qn, xn, c["seed"], c["offset"])
        assert_match(A, Ls, ref, range(B), (V, dt, sp))
        if sp is None:
            assert np.all(Ls == D)


def test_verify_fused_config5_filtered_rows(sv):
    """The mixed batch's top-k and top-p requests through req_index at the full
    shape (B=1024, D=7, V=129280 bf16): identical to the two-call form and
    to the oracle for all 512 of them."""
    torch = __import__("torch")
    c = make_config(5)
    B, D, V = 1024, 7, 129280
    N = D + 1
    modes = c["modes"]
    filt = np.nonzero((modes == MODE_TOPK) | (modes == MODE_TOPP))[0].astype(np.int32)
    log(f"config 5 fused: {len(filt)} filtered requests, bf16 V={V}")
    z = dev_logits(c["logits"], "bf16")
    T, k, p = dev(c["temperature"]), dev(c["top_k"]), dev(c["top_p"])
    q, x = dev(c["draft_probs"]), dev(c["draft_ids"])
    seed, off = dev(c["seed"]), dev(c["offset"])
    acc = torch.full((B, N), SENTINEL, dtype=torch.int32, device="cuda")
    alen = torch.full((B,), SENTINEL, dtype=torch.int32, device="cuda")
    sv.verify_fused(z, T, q, x, seed, off, top_k=k, top_p=p, req_index=dev(filt), out=(acc, alen))
    A, Ls = np_i(acc), np_i(alen)
    rest = np.setdiff1d(np.arange(B), filt)
    assert np.all(A[rest] == SENTINEL) and np.all(Ls[rest] == SENTINEL)
    A2, L2 = two_call(sv, z, T, k, p, q, x, seed, off, req=dev(filt), B=B, N=N, V=V)
    assert np.array_equal(A[filt], A2[filt]) and np.array_equal(Ls[filt], L2[filt])
    log("config 5 fused: all filtered requests against the oracle")
    ref = oracle.verify_fused(c["logits"], "bf16", c["temperature"], c["top_k"], c["top_p"], c["draft_probs"],
                              c["draft_ids"], c["seed"], c["offset"], requests=filt)
    flagged = assert_match(A, Ls, ref, filt, "cfg5 fused")
    assert flagged <= 1 + len(filt) // 20, flagged     # top-p boundary (1e-5) and 1e-6 CDF flags
    log(f"config 5 fused: mean L={Ls[filt].mean():.3f}, flagged={flagged} of {len(filt)}, "
        f"within 1e-6 of a CDF boundary {int(ref['near_cdf'][filt].sum())}")


def test_verify_fused_other_row_paths(sv):
    """bf16 rows too long for the register-resident statistics (streamed),
    logits whose rows are not 16-byte aligned (streamed), the largest
    vocabulary the call accepts, and 16 drafts."""
    torch = __import__("torch")
    for V, dt, D, shift in ((200000, "bf16", 3, 0), (32000, "bf16", 2, 1), (524288, "f32", 1, 0),
                            (5000, "bf16", 16, 0), (9000, "f32", 16, 3)):
        B = 3
        N = D + 1
        c = fuzz_case(900 + V + D, B, D, V, dt)
        T = np.array([0.9, 1.1, 0.0], np.float32)
        k = np.array([40, 0, 0], np.int32)
        p = np.array([0.95, 0.85, 1.0], np.float32)
        zt = dev_logits(c["logits"], dt)
        if shift:
            flat = torch.empty(zt.numel() + 8, dtype=zt.dtype, device="cuda")
            z = flat[shift:shift + zt.numel()].view(B, N, V)
            z.copy_(zt)
        else:
            z = zt
        log(f"fused other paths: V={V} dtype={dt} D={D} shift={shift}")
        args = (dev(c["draft_probs"]), dev(c["draft_ids"]), dev(c["seed"]), dev(c["offset"]))
        acc, alen = sv.verify_fused(z, dev(T), *args, top_k=dev(k), top_p=dev(p))
        A, Ls = np_i(acc), np_i(alen)
        A2, L2 = two_call(sv, z, dev(T), dev(k), dev(p), *args, B=B, N=N, V=V)
        assert np.array_equal(A, A2) and np.array_equal(Ls, L2), (V, dt, D, shift)
        ref = oracle.verify_fused(c["logits"], dt, T, k, p, c["draft_probs"], c["draft_ids"], c["seed"],
                                  c["offset"])
        assert_match(A, Ls, ref, range(B), (V, dt, D, shift))


def test_verify_fused_row_mode_matches_serial(sv):
    """Small batches evaluate every row at once (one workgroup per row, the
    caller's counters); with no workspace the same call walks each request's
    rows in order.  Both must agree bit for bit, also through a request
    subset that lists requests twice, and the counters must be zero after
    every call; the oracle is checked as well."""
    import ctypes
    torch = __import__("torch")
    L = sv.lib()
    for i, (B, D, V, dt) in enumerate(((64, 3, 32000, "bf16"), (20, 7, 4096, "bf16"), (6, 16, 1001, "f32"),
                                       (40, 5, 8192, "bf16"))):
        N = D + 1
        c = fuzz_case(1900 + i, B, D, V, dt)
        rng = np.random.default_rng(1900 + i)
        T = rng.uniform(0.5, 1.3, B).astype(np.float32)
        T[::7] = 0.0
        k = np.where(rng.random(B) < 0.5, rng.choice([0, 5, 50, 200], B), 0).astype(np.int32)
        p = np.where(rng.random(B) < 0.5, rng.uniform(0.6, 0.99, B), 1.0).astype(np.float32)
        z = dev_logits(c["logits"], dt)
        args = [dev(T), dev(c["draft_probs"]), dev(c["draft_ids"]), dev(c["seed"]), dev(c["offset"])]
        log(f"fused row mode vs serial {i}: B={B} D={D} V={V} dtype={dt}")
        ws = torch.zeros(sv.verify_fused_workspace_bytes(B, D), dtype=torch.uint8, device="cuda")
        assert ws.numel() > 0
        acc, alen = sv.verify_fused(z, args[0], *args[1:], top_k=dev(k), top_p=dev(p), workspace=ws)
        assert not bool((ws != 0).any().item())
        acc2 = torch.full((B, N), SENTINEL, dtype=torch.int32, device="cuda")
        alen2 = torch.full((B,), SENTINEL, dtype=torch.int32, device="cuda")
        dtype_code = sv.BF16 if dt == "bf16" else sv.F32
        kk, pp = dev(k), dev(p)
        st = L.specverify_verify_fused(
            ctypes.c_void_p(z.data_ptr()), dtype_code, ctypes.c_void_p(args[0].data_ptr()),
            ctypes.c_void_p(kk.data_ptr()), ctypes.c_void_p(pp.data_ptr()), ctypes.c_void_p(args[1].data_ptr()),
            ctypes.c_void_p(args[2].data_ptr()), ctypes.c_void_p(args[3].data_ptr()),
            ctypes.c_void_p(args[4].data_ptr()), B, D, V, None, B, ctypes.c_void_p(acc2.data_ptr()),
            ctypes.c_void_p(alen2.data_ptr()), None, 0, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == 0, L.specverify_last_error()
        assert np.array_equal(np_i(acc), np_i(acc2)) and np.array_equal(np_i(alen), np_i(alen2)), (B, D, V)
        ref = oracle.verify_fused(c["logits"], dt, T, k, p, c["draft_probs"], c["draft_ids"], c["seed"],
                                  c["offset"])
        assert_match(np_i(acc), np_i(alen), ref, range(B), ("row mode", B, D, V))
        # a subset listing requests twice: each listed request as in the full call, others untouched
        reqs = np.array([3, 1, 3, 0, 1, 5], np.int32)
        acc3 = torch.full((B, N), SENTINEL, dtype=torch.int32, device="cuda")
        alen3 = torch.full((B,), SENTINEL, dtype=torch.int32, device="cuda")
        sv.verify_fused(z, args[0], *args[1:], top_k=kk, top_p=pp, req_index=dev(reqs), out=(acc3, alen3),
                        workspace=ws)
        a3, l3 = np_i(acc3), np_i(alen3)
        for b in range(B):
            if b in reqs:
                assert np.array_equal(a3[b], np_i(acc)[b]) and l3[b] == np_i(alen)[b], (b, B, D, V)
            else:
                assert np.all(a3[b] == SENTINEL) and l3[b] == SENTINEL
        assert not bool((ws != 0).any().item())
