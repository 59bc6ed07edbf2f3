"""The C-ABI library loads, exports every symbol the header declares, and
rejects invalid arguments on the host before any HIP call (CPU only)."""
import ctypes
import os
import re

import pytest

import token_sampling_temp_amd as sv

HERE = os.path.dirname(os.path.abspath(__file__))
HEADER = os.path.join(os.path.dirname(HERE), "include", "specverify.h")

pytestmark = pytest.mark.skipif(not os.path.exists(sv.LIB_PATH),
                                reason="libspecverify.so not built (run __graft_entry__.build())")

P = ctypes.c_void_p(0x1000)     # never dereferenced: validation fails first


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"\b(specverify_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert set(names) == set(sv.SYMBOLS)
    L = sv.lib()
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings():
    L = sv.lib()
    assert sv.version() == 202
    assert L.specverify_status_string(0) == b"SPECVERIFY_OK"
    assert L.specverify_status_string(1) == b"SPECVERIFY_INVALID_ARGUMENT"
    assert L.specverify_status_string(2) == b"SPECVERIFY_UNSUPPORTED"
    assert L.specverify_status_string(3) == b"SPECVERIFY_HIP_ERROR"
    assert L.specverify_status_string(77) == b"SPECVERIFY_UNKNOWN_STATUS"


def _chain(**kw):
    a = dict(q=P, x=P, p=P, seed=P, off=P, B=4, D=3, V=100, req=None, n=4, acc=P, alen=P, ws=None, wsb=0)
    a.update(kw)
    return sv.lib().specverify_chain_reject(a["q"], a["x"], a["p"], a["seed"], a["off"], a["B"], a["D"], a["V"],
                                            a["req"], a["n"], a["acc"], a["alen"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,msg", [
    (dict(D=-1), "D=-1"),
    (dict(D=17), "D=17"),
    (dict(V=0), "V=0"),
    (dict(V=2 ** 31), "V="),
    (dict(B=-2, n=0), "B=-2"),
    (dict(n=3), "n_req=3"),
    (dict(n=5, req=P), "n_req=5"),
    (dict(p=None), "target_probs"),
    (dict(x=None), "draft_ids"),
    (dict(seed=None), "seed"),
    (dict(off=None), "offset"),
    (dict(acc=None), "accepted_tokens"),
    (dict(alen=None), "accept_length"),
    (dict(B=2 ** 40, n=2 ** 40, V=2 ** 30), "grid limit"),
    (dict(B=2 ** 30, n=2 ** 30, V=2 ** 30), "overflow"),
])
def test_chain_reject_invalid_arguments(kw, msg):
    assert _chain(**kw) == sv.INVALID_ARGUMENT
    err = sv.lib().specverify_last_error().decode()
    assert msg in err and "specverify_chain_reject" in err


def test_chain_reject_zero_draft_allows_null_draft_buffers_and_empty_batch_is_noop():
    # n_req = 0 returns OK without touching any device
    assert _chain(B=0, n=0) == sv.OK
    assert _chain(n=0, req=P) == sv.OK
    # draft_probs NULL with D > 0 is the target-only verify: not an argument error
    assert _chain(q=None, p=None) == sv.INVALID_ARGUMENT
    assert "target_probs" in sv.lib().specverify_last_error().decode()
    # D = 0: draft buffers may be NULL (the failure is then a missing target buffer)
    assert _chain(D=0, q=None, x=None, p=None) == sv.INVALID_ARGUMENT
    assert "target_probs" in sv.lib().specverify_last_error().decode()


def _ws_bytes(n_req, V):
    out = ctypes.c_int64(-1)
    st = sv.lib().specverify_chain_workspace_bytes(n_req, V, ctypes.byref(out))
    return st, out.value


def test_chain_workspace_query():
    # one workgroup per request with chunk sums on chip: no workspace
    assert _ws_bytes(256, 128256) == (sv.OK, 0)
    assert _ws_bytes(1024, 4096) == (sv.OK, 0)
    assert _ws_bytes(0, 100) == (sv.OK, 0)
    # small batches split rows: 256 bytes of counters, then one double per 1024 entries per request
    assert _ws_bytes(64, 32000) == (sv.OK, 256 + 64 * 32 * 8)
    assert _ws_bytes(65, 32000) == (sv.OK, 512 + 65 * 32 * 8)
    # rows longer than 262144 entries split even for large batches
    assert _ws_bytes(256, 262144) == (sv.OK, 0)
    assert _ws_bytes(256, 262145)[1] == 1024 + 256 * 257 * 8
    assert _ws_bytes(-1, 10)[0] == sv.INVALID_ARGUMENT
    assert _ws_bytes(4, 0)[0] == sv.INVALID_ARGUMENT
    assert sv.lib().specverify_chain_workspace_bytes(4, 10, None) == sv.INVALID_ARGUMENT
    assert sv.chain_workspace_bytes(40, 60000) == 256 + 40 * 59 * 8


def test_chain_reject_workspace_validation():
    # B = 4 over V = 100000 splits each row: the call needs the caller's workspace
    assert _chain(V=100000) == sv.INVALID_ARGUMENT
    assert "workspace is NULL" in sv.lib().specverify_last_error().decode()
    need = _ws_bytes(4, 100000)[1]
    assert _chain(V=100000, ws=P, wsb=need - 8) == sv.INVALID_ARGUMENT
    assert "needs %d" % need in sv.lib().specverify_last_error().decode()
    assert _chain(V=100000, ws=ctypes.c_void_p(0x1004), wsb=need) == sv.INVALID_ARGUMENT
    assert "8-byte aligned" in sv.lib().specverify_last_error().decode()
    # a large batch needs none, and the empty batch never looks at it
    assert _chain(B=0, n=0, ws=None) == sv.OK


def test_greedy_and_gumbel_and_softmax_invalid_arguments():
    L = sv.lib()
    assert L.specverify_greedy_verify(P, 2, P, 4, 3, 10, None, 4, P, P, None, None, None, None, 0, None) == 1
    assert "dtype=2" in L.specverify_last_error().decode()
    assert L.specverify_greedy_verify(None, 1, P, 4, 3, 10, None, 4, P, P, None, None, None, None, 0, None) == 1
    assert L.specverify_greedy_verify(P, 0, None, 4, 3, 10, None, 4, P, P, None, None, None, None, 0, None) == 1
    assert L.specverify_greedy_verify(P, 0, P, 4, 3, 10, None, 0, P, P, None, None, None, None, 0, None) == 1
    assert L.specverify_gumbel_sample(P, 1, None, P, P, P, 4, 3, 10, None, 4, P, P, None, None, 0, None) == 1
    assert "temperature" in L.specverify_last_error().decode()
    assert L.specverify_gumbel_sample(P, 1, P, P, P, P, 4, 20, 10, None, 4, P, P, None, None, 0, None) == 1
    assert L.specverify_softmax_renorm(P, 0, 4, 0, 10, P, None, None, None, 4, P, None) == 1
    assert "npos=0" in L.specverify_last_error().decode()
    assert L.specverify_softmax_renorm(P, 0, 4, 2, 10, None, None, None, None, 4, P, None) == 1
    assert L.specverify_softmax_renorm(P, 5, 4, 2, 10, P, None, None, None, 4, P, None) == 1
    assert L.specverify_softmax_renorm(P, 1, 4, 2, 10, P, None, None, None, 0, P, None) == 1
    assert L.specverify_softmax_renorm(None, 1, 0, 2, 10, None, None, None, None, 0, None, None) == 0


def test_rowpar_workspace_query_and_validation():
    out = ctypes.c_int64(-1)
    L = sv.lib()
    # greedy: one 128-byte line (ended rows, row count, D + 1 tokens) per request, rounded up to 256
    q = L.specverify_greedy_verify_workspace_bytes
    assert q(256, 7, ctypes.byref(out)) == 0 and out.value == 256 * 128
    assert q(5, 3, ctypes.byref(out)) == 0 and out.value == 768
    assert q(100, 16, ctypes.byref(out)) == 0 and out.value == 12800
    # Gumbel: the same lines, a 256-byte count, then a 128-byte line per (request, later row)
    q = L.specverify_gumbel_sample_workspace_bytes
    assert q(256, 7, ctypes.byref(out)) == 0 and out.value == 256 * 128 + 256 + 256 * 7 * 128
    assert q(5, 3, ctypes.byref(out)) == 0 and out.value == 2816   # 640 + 256 + 1920 = 2816
    assert q(100, 16, ctypes.byref(out)) == 0 and out.value == 12800 + 256 + 204800
    for q in (L.specverify_greedy_verify_workspace_bytes, L.specverify_gumbel_sample_workspace_bytes):
        # no drafts or no requests: the one-row form needs none
        assert q(100, 0, ctypes.byref(out)) == 0 and out.value == 0
        assert q(0, 3, ctypes.byref(out)) == 0 and out.value == 0
        assert q(-1, 3, ctypes.byref(out)) == 1
        assert q(4, 17, ctypes.byref(out)) == 1
        assert q(4, 3, None) == 1
    assert sv.greedy_verify_workspace_bytes(512, 3) == 512 * 128
    assert sv.gumbel_sample_workspace_bytes(256, 7) == 256 * 128 + 256 + 256 * 7 * 128
    # (logits, dtype, x, B, D, V, req_index, n_req, acc, alen, predict, accept_index, argmax, ws, ws_bytes, stream)
    assert L.specverify_greedy_verify(P, 0, P, 4, 3, 10, None, 4, P, P, None, None, None, P, 8, None) == 1
    assert "needs 512" in L.specverify_last_error().decode()
    assert L.specverify_greedy_verify(P, 0, P, 4, 3, 10, None, 4, P, P, None, None, None,
                                      ctypes.c_void_p(0x1004), 512, None) == 1
    assert "aligned" in L.specverify_last_error().decode()
    assert L.specverify_gumbel_sample(P, 1, P, P, P, P, 4, 3, 10, None, 4, P, P, None, P, 2303, None) == 1
    assert "needs 2304" in L.specverify_last_error().decode()
    # the empty batch never looks at the workspace
    assert L.specverify_greedy_verify(None, 0, None, 4, 3, 10, P, 0, None, None, None, None, None, P, 0, None) == 0


def test_verify_fused_invalid_arguments():
    L = sv.lib()
    # (logits, dtype, T, top_k, top_p, q, x, seed, offset, B, D, V, req_index, n_req, acc, alen, workspace,
    #  workspace_bytes, stream)
    assert L.specverify_verify_fused(P, 3, P, None, None, P, P, P, P, 4, 3, 10, None, 4, P, P, None, 0, None) == 1
    assert "dtype=3" in L.specverify_last_error().decode()
    assert L.specverify_verify_fused(P, 1, None, None, None, P, P, P, P, 4, 3, 10, None, 4, P, P, None, 0, None) == 1
    assert "temperature" in L.specverify_last_error().decode()
    assert L.specverify_verify_fused(P, 1, P, None, None, None, P, P, P, 4, 3, 10, None, 4, P, P, None, 0, None) == 1
    assert "draft_probs" in L.specverify_last_error().decode()
    assert L.specverify_verify_fused(P, 1, P, None, None, P, P, P, P, 4, 17, 10, None, 4, P, P, None, 0, None) == 1
    assert L.specverify_verify_fused(P, 1, P, None, None, P, P, P, P, 4, 3, 600000, None, 4, P, P, None, 0, None) == 1
    assert "exceeds" in L.specverify_last_error().decode()
    assert L.specverify_verify_fused(P, 1, P, None, None, P, P, None, P, 4, 3, 10, None, 4, P, P, None, 0, None) == 1
    assert "seed" in L.specverify_last_error().decode()
    # n_req = 0 is a no-op that touches no device
    assert L.specverify_verify_fused(None, 0, None, None, None, None, None, None, None, 4, 3, 10, P, 0, None, None,
                                     None, 0, None) == 0
    # a workspace shorter than the query, or misaligned, is refused before any device call
    assert L.specverify_verify_fused(P, 1, P, None, None, P, P, P, P, 4, 3, 10, None, 4, P, P, P, 8, None) == 1
    assert "needs 512" in L.specverify_last_error().decode()
    assert L.specverify_verify_fused(P, 1, P, None, None, P, P, P, P, 4, 3, 10, None, 4, P, P,
                                     ctypes.c_void_p(0x1004), 512, None) == 1
    assert "aligned" in L.specverify_last_error().decode()


def test_verify_fused_workspace_query():
    out = ctypes.c_int64(-1)
    L = sv.lib()
    # one 128-byte line per request, rounded up to 256
    assert L.specverify_verify_fused_workspace_bytes(64, 3, ctypes.byref(out)) == 0 and out.value == 8192
    assert L.specverify_verify_fused_workspace_bytes(85, 2, ctypes.byref(out)) == 0 and out.value == 11008
    # any batch with drafts takes one; without drafts none is used
    assert L.specverify_verify_fused_workspace_bytes(65, 3, ctypes.byref(out)) == 0 and out.value == 8448
    assert L.specverify_verify_fused_workspace_bytes(100, 0, ctypes.byref(out)) == 0 and out.value == 0
    assert L.specverify_verify_fused_workspace_bytes(-1, 3, ctypes.byref(out)) == 1
    assert L.specverify_verify_fused_workspace_bytes(4, 17, ctypes.byref(out)) == 1
    assert sv.verify_fused_workspace_bytes(64, 3) == 8192


def test_chain_reject_ragged_invalid_arguments():
    L = sv.lib()
    # (q, t2d, Vd, x, p, qo_indptr, n_rows, seed, offset, B, D, V, req_index, n_req, acc, alen, workspace,
    #  workspace_bytes, stream)
    assert L.specverify_chain_reject_ragged(P, None, 0, P, P, None, 8, P, P, 4, 3, 10, None, 4, P, P, None, 0, None) == 1
    assert "qo_indptr" in L.specverify_last_error().decode()
    assert L.specverify_chain_reject_ragged(P, None, 0, P, P, P, -1, P, P, 4, 3, 10, None, 4, P, P, None, 0, None) == 1
    assert "n_rows" in L.specverify_last_error().decode()
    assert L.specverify_chain_reject_ragged(P, None, 0, P, P, P, 8, P, P, 4, 17, 10, None, 4, P, P, None, 0, None) == 1
    assert L.specverify_chain_reject_ragged(P, None, 0, None, P, P, 8, P, P, 4, 3, 10, None, 4, P, P, None, 0, None) == 1
    assert "draft_ids" in L.specverify_last_error().decode()
    assert L.specverify_chain_reject_ragged(P, None, 0, P, None, P, 8, P, P, 4, 3, 10, None, 4, P, P, None, 0, None) == 1
    assert L.specverify_chain_reject_ragged(None, P, 5, P, P, P, 8, P, P, 4, 3, 10, None, 4, P, P, None, 0, None) == 1
    assert "t2d needs draft_probs" in L.specverify_last_error().decode()
    assert L.specverify_chain_reject_ragged(P, P, 0, P, P, P, 8, P, P, 4, 3, 10, None, 4, P, P, None, 0, None) == 1
    assert "Vd=0" in L.specverify_last_error().decode()
    assert L.specverify_chain_reject_ragged(None, None, 0, None, None, None, 0, None, None, 4, 3, 10, P, 0, None,
                                            None, None, 0, None) == 0
    # a split launch needs the caller's workspace: missing, short or misaligned is an argument error
    assert L.specverify_chain_reject_ragged(P, None, 0, P, P, P, 8, P, P, 4, 3, 100000, None, 4, P, P, None, 0,
                                            None) == 1
    assert "workspace is NULL" in L.specverify_last_error().decode()
    assert L.specverify_chain_reject_ragged(P, None, 0, P, P, P, 8, P, P, 4, 3, 100000, None, 4, P, P, P, 8,
                                            None) == 1
    assert "needs" in L.specverify_last_error().decode()


def test_d2t_invalid_arguments():
    L = sv.lib()
    # inverse: (d2t, Vd, V, t2d, stream)
    assert L.specverify_d2t_inverse(None, 12, 10, P, None) == 1
    assert "Vd=12" in L.specverify_last_error().decode()
    # a table cannot map more draft entries than the target has one-to-one
    assert L.specverify_d2t_inverse(P, 12, 10, P, None) == 1
    assert "Vd=12" in L.specverify_last_error().decode()
    assert L.specverify_d2t_inverse(P, 0, 10, P, None) == 1
    assert L.specverify_d2t_inverse(P, 8, 0, P, None) == 1
    assert L.specverify_d2t_inverse(P, 8, 10, None, None) == 1
    assert "t2d" in L.specverify_last_error().decode()
    # expand: (draft_probs, t2d, rows, Vd, V, out, stream)
    assert L.specverify_d2t_expand(P, P, -1, 8, 10, P, None) == 1
    assert L.specverify_d2t_expand(P, P, 4, 0, 10, P, None) == 1
    assert L.specverify_d2t_expand(None, P, 4, 8, 10, P, None) == 1
    assert "draft_probs" in L.specverify_last_error().decode()
    assert L.specverify_d2t_expand(P, None, 4, 8, 10, P, None) == 1
    assert "t2d" in L.specverify_last_error().decode()
    assert L.specverify_d2t_expand(P, P, 4, 8, 10, None, None) == 1
    assert L.specverify_d2t_expand(None, None, 0, 8, 10, None, None) == 0


def test_sample_invalid_arguments():
    L = sv.lib()
    # (logits, dtype, T, top_k, top_p, min_p, seed, offset, B, V, req_index, n_req, tokens, stream)
    assert L.specverify_sample(P, 2, P, None, None, None, P, P, 4, 10, None, 4, P, None) == 1
    assert "dtype=2" in L.specverify_last_error().decode()
    assert L.specverify_sample(P, 1, None, None, None, None, P, P, 4, 10, None, 4, P, None) == 1
    assert "temperature" in L.specverify_last_error().decode()
    assert L.specverify_sample(P, 1, P, None, None, None, P, P, 4, 600000, None, 4, P, None) == 1
    assert "exceeds" in L.specverify_last_error().decode()
    assert L.specverify_sample(P, 1, P, None, None, None, P, P, 4, 10, None, 4, None, None) == 1
    assert "tokens" in L.specverify_last_error().decode()
    assert L.specverify_sample(P, 1, P, None, None, None, None, P, 4, 10, None, 4, P, None) == 1
    assert L.specverify_sample(None, 0, None, None, None, None, None, None, 4, 10, P, 0, None, None) == 0


def test_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    z = torch.zeros(2, 3, 8)
    with pytest.raises(ValueError, match="GPU"):
        sv.softmax_renorm(z, torch.ones(2))
    with pytest.raises(ValueError, match="GPU"):
        sv.greedy_verify(z, torch.zeros(2, 2, dtype=torch.int32))
