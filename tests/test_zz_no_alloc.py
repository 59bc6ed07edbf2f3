"""The chain-rejection entry point that allocates nothing (the library's
static scratch) against the entry point with a caller workspace, through the
C ABI: two calls in a row on split rows, the second smaller, each bit-exact
with the workspace call and matching the oracle; a call too large for the
scratch is refused before any launch."""
import ctypes

import numpy as np
import pytest

import oracle
from gpu_helpers import dev, guard_intact, guarded_i32, log, np_i
from workloads import fuzz_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sv():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import token_sampling_temp_amd as m
    m.lib()
    return m


def _check(sv, B, D, V, seed):
    c = fuzz_case(seed, B, D, V, "f32")
    args = [dev(c["draft_probs"]), dev(c["draft_ids"]), dev(c["target_probs"]), dev(c["seed"]), dev(c["offset"])]
    need = sv.chain_workspace_bytes(B, V)
    log(f"no-alloc chain: B={B} D={D} V={V} scratch bytes needed {need}")
    assert 0 < need <= sv.STATIC_SCRATCH_BYTES
    acc, acc_full = guarded_i32((B, D + 1))
    alen, alen_full = guarded_i32((B,))
    sv.chain_reject_noalloc(*args, out=(acc, alen))
    ws = sv.chain_workspace(B, V, "cuda")
    acc_ws, alen_ws = sv.chain_reject(*args, workspace=ws)
    assert np.array_equal(np_i(acc), np_i(acc_ws)) and np.array_equal(np_i(alen), np_i(alen_ws)), (B, D, V)
    assert guard_intact(acc_full, B * (D + 1)) and guard_intact(alen_full, B)
    ref = oracle.chain_reject(c["draft_probs"], c["draft_ids"], c["target_probs"], c["seed"], c["offset"])
    L = ref["accept_length"]
    assert np.array_equal(np_i(alen), L)
    for b in range(B):
        n = min(int(ref["flag_pos"][b]), int(L[b]) + 1)
        assert list(np_i(acc)[b, :n]) == list(ref["accepted_tokens"][b, :n]), (b, B, V)


def test_no_alloc_matches_workspace_call_twice_second_smaller(sv):
    _check(sv, 40, 5, 60000, 1801)
    _check(sv, 10, 3, 20000, 1802)


def test_no_alloc_refuses_more_than_its_scratch(sv):
    B, V = 255, 3_000_000
    assert sv.chain_workspace_bytes(B, V) > sv.STATIC_SCRATCH_BYTES
    P = ctypes.c_void_p(0x1000)
    st = sv.lib().specverify_chain_reject_noalloc(P, P, P, P, P, B, 3, V, None, B, P, P, None)
    assert st == sv.INVALID_ARGUMENT
    assert "static scratch" in sv.lib().specverify_last_error().decode()
