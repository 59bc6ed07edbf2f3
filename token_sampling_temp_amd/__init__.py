"""specverify: speculative-decoding draft verification on MI355X (gfx950).

Thin ctypes binding over ``libspecverify.so`` (C ABI declared in
``include/specverify.h``).  This module only marshals arguments: it checks
tensor placement, dtype and contiguity, allocates outputs with torch, and
passes raw device pointers plus the current HIP stream.  Every step of the
verification runs in the library's HIP kernels; there is no CPU fallback, and
a missing library raises.

Functions mirror the C entry points:

* ``softmax_renorm(logits, temperature, top_k=None, top_p=None, req_index=None)``
* ``chain_reject(draft_probs, draft_ids, target_probs, seed, offset, req_index=None, workspace=None)``
* ``chain_reject_ragged(draft_probs, draft_ids, target_probs, qo_indptr, seed, offset, req_index=None,
  workspace=None)``: per-request verify lengths over packed target rows
* ``chain_workspace_bytes(n_req, V)`` and ``chain_workspace(n_req, V, device)``: the caller-owned
  workspace the two chain calls need when rows are split over workgroups (small batches)
* ``chain_reject_noalloc(draft_probs, draft_ids, target_probs, seed, offset, req_index=None)``:
  chain rejection that allocates nothing, using the library's static scratch
* ``sample(logits, temperature, seed, offset, top_k=None, top_p=None, min_p=None, req_index=None)``:
  single-step sampling with the joint top-k/top-p filter and min-p
* ``d2t_inverse(d2t, Vd, V)`` and ``d2t_expand(draft_probs, t2d)``: draft distributions over a
  reduced draft vocabulary placed in the target vocabulary
* ``greedy_verify(target_logits, draft_ids, req_index=None, ..., workspace=None)``
* ``gumbel_sample(target_logits, temperature, draft_ids, seed, offset, req_index=None, ..., workspace=None)``;
  ``greedy_verify_workspace_bytes(n_req, D)`` and ``gumbel_sample_workspace_bytes(n_req, D)``: the
  per-request words of their one-workgroup-per-row form (``workspace=False`` takes the
  one-workgroup-per-request form)
* ``verify_fused(target_logits, temperature, draft_probs, draft_ids, seed, offset, top_k=None,
  top_p=None, req_index=None, workspace=None)``: softmax_renorm followed by chain_reject in one call;
  ``verify_fused_workspace_bytes(n_req, D)``: the per-request lines of its one-workgroup-per-row form

``accept_length`` is the number of accepted drafts L in [0, D]; a request
emits L + 1 tokens.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libspecverify.so")

OK, INVALID_ARGUMENT, UNSUPPORTED, HIP_ERROR = 0, 1, 2, 3
F32, BF16 = 0, 1
MAX_DRAFT = 16
STATIC_SCRATCH_BYTES = 4 << 20
RNG_SLOT_SPAN = 32

SYMBOLS = (
    "specverify_softmax_renorm",
    "specverify_chain_reject",
    "specverify_chain_workspace_bytes",
    "specverify_chain_reject_noalloc",
    "specverify_chain_reject_ragged",
    "specverify_d2t_inverse",
    "specverify_d2t_expand",
    "specverify_greedy_verify",
    "specverify_greedy_verify_workspace_bytes",
    "specverify_gumbel_sample",
    "specverify_gumbel_sample_workspace_bytes",
    "specverify_verify_fused",
    "specverify_verify_fused_workspace_bytes",
    "specverify_sample",
    "specverify_status_string",
    "specverify_last_error",
    "specverify_version",
)

_lib = None


class SpecVerifyError(RuntimeError):
    """A specverify call returned a non-zero status."""

    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn}: {message} (status {status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libspecverify.so (built in-tree); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m token_sampling_temp_amd.build` "
            "(there is no CPU fallback)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    L.specverify_softmax_renorm.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp, vp, i64, vp, vp]
    L.specverify_chain_reject.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp, i64, vp, vp, vp, i64, vp]
    L.specverify_chain_workspace_bytes.argtypes = [i64, i64, ctypes.POINTER(ctypes.c_int64)]
    L.specverify_chain_reject_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp, i64, vp, vp, vp]
    L.specverify_chain_reject_ragged.argtypes = [vp, vp, i64, vp, vp, vp, i64, vp, vp, i64, i64, i64, vp, i64, vp,
                                                 vp, vp, i64, vp]
    L.specverify_d2t_inverse.argtypes = [vp, i64, i64, vp, vp]
    L.specverify_d2t_expand.argtypes = [vp, vp, i64, i64, i64, vp, vp]
    L.specverify_greedy_verify.argtypes = [vp, i32, vp, i64, i64, i64, vp, i64, vp, vp, vp, vp, vp, vp, i64, vp]
    L.specverify_greedy_verify_workspace_bytes.argtypes = [i64, i64, ctypes.POINTER(ctypes.c_int64)]
    L.specverify_gumbel_sample.argtypes = [vp, i32, vp, vp, vp, vp, i64, i64, i64, vp, i64, vp, vp, vp, vp, i64,
                                           vp]
    L.specverify_gumbel_sample_workspace_bytes.argtypes = [i64, i64, ctypes.POINTER(ctypes.c_int64)]
    L.specverify_verify_fused.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, vp, i64, vp, vp, vp,
                                          i64, vp]
    L.specverify_verify_fused_workspace_bytes.argtypes = [i64, i64, ctypes.POINTER(ctypes.c_int64)]
    L.specverify_sample.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, i64, i64, vp, i64, vp, vp]
    for name in ("specverify_softmax_renorm", "specverify_chain_reject", "specverify_chain_workspace_bytes",
                 "specverify_chain_reject_noalloc", "specverify_chain_reject_ragged",
                 "specverify_d2t_inverse", "specverify_d2t_expand", "specverify_greedy_verify",
                 "specverify_greedy_verify_workspace_bytes", "specverify_gumbel_sample",
                 "specverify_gumbel_sample_workspace_bytes", "specverify_verify_fused",
                 "specverify_verify_fused_workspace_bytes",
                 "specverify_sample"):
        getattr(L, name).restype = ctypes.c_int
    L.specverify_status_string.argtypes = [ctypes.c_int]
    L.specverify_status_string.restype = ctypes.c_char_p
    L.specverify_last_error.argtypes = []
    L.specverify_last_error.restype = ctypes.c_char_p
    L.specverify_version.argtypes = []
    L.specverify_version.restype = ctypes.c_int
    _lib = L
    return L


def _check(fn: str, status: int):
    if status != OK:
        msg = lib().specverify_last_error().decode(errors="replace")
        raise SpecVerifyError(fn, status, msg)


# --------------------------------------------------------------------------- marshalling
def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_ptr(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtypes, device=None, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    return t


def _logit_dtype(t):
    torch = _torch()
    return BF16 if t.dtype == torch.bfloat16 else F32


def _req(req_index, B, device):
    torch = _torch()
    if req_index is None:
        return None, B
    _need(req_index, "req_index", (torch.int32,), device, 1)
    return req_index, int(req_index.shape[0])


def _u64(t, name, B, device):
    torch = _torch()
    _need(t, name, (torch.int64, torch.uint64), device, 1)
    if t.shape[0] != B:
        raise ValueError(f"{name} must have shape [{B}], got {tuple(t.shape)}")
    return t


def chain_workspace_bytes(n_req, V) -> int:
    """Bytes of workspace a chain call over n_req requests and V entries needs (0: none)."""
    out = ctypes.c_int64(0)
    _check("specverify_chain_workspace_bytes", lib().specverify_chain_workspace_bytes(int(n_req), int(V),
                                                                                       ctypes.byref(out)))
    return int(out.value)


def chain_workspace(n_req, V, device):
    """A zero-filled workspace for chain calls over n_req requests and V entries (None when none is
    needed).  Every call leaves the bytes it used zero, so it can be reused by any later chain call
    on the same stream that fits in it."""
    torch = _torch()
    n = chain_workspace_bytes(n_req, V)
    if n == 0:
        return None
    return torch.zeros((n,), dtype=torch.uint8, device=device)


# Workspaces made for callers that pass none, one per (device, stream), replaced by a larger one when a
# call needs more.  A replaced tensor goes back to torch's stream-ordered caching allocator, so kernels
# already queued on that stream finish with it before its memory is handed out again there.
_workspaces = {}


def _workspace(workspace, n_req, V, device):
    torch = _torch()
    n = chain_workspace_bytes(n_req, V)
    if n == 0:
        return None, 0
    if workspace is not None:
        _need(workspace, "workspace", (torch.uint8,), device, 1)
        return workspace, int(workspace.numel())
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < n:
        ws = torch.zeros((n,), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws, int(ws.numel())


# --------------------------------------------------------------------------- entry points
def softmax_renorm(logits, temperature, top_k=None, top_p=None, req_index=None, out=None):
    """Temperature softmax then top-k then top-p renormalisation: [B, npos, V] -> float32 probs."""
    torch = _torch()
    _need(logits, "logits", (torch.float32, torch.bfloat16), None, 3)
    dev = logits.device
    B, npos, V = logits.shape
    _need(temperature, "temperature", (torch.float32,), dev, 1)
    if top_k is not None:
        _need(top_k, "top_k", (torch.int32,), dev, 1)
    if top_p is not None:
        _need(top_p, "top_p", (torch.float32,), dev, 1)
    for name, t in (("temperature", temperature), ("top_k", top_k), ("top_p", top_p)):
        if t is not None and t.shape[0] != B:
            raise ValueError(f"{name} must have shape [{B}]")
    req_index, n_req = _req(req_index, B, dev)
    if out is None:
        out = torch.empty((B, npos, V), dtype=torch.float32, device=dev)
    else:
        _need(out, "out", (torch.float32,), dev, 3)
        if tuple(out.shape) != (B, npos, V):
            raise ValueError("out has the wrong shape")
    st = lib().specverify_softmax_renorm(
        _ptr(logits), _logit_dtype(logits), B, npos, V, _ptr(temperature), _ptr(top_k), _ptr(top_p),
        _ptr(req_index), n_req, _ptr(out), _stream_ptr(dev))
    _check("specverify_softmax_renorm", st)
    return out


def chain_reject(draft_probs, draft_ids, target_probs, seed, offset, req_index=None, out=None, workspace=None):
    """Chain rejection sampling; returns (accepted_tokens [B, D+1] int32, accept_length [B] int32).

    ``draft_probs`` None is the target-only verify: each draft is a point mass at its id.
    ``workspace``: a uint8 tensor from ``chain_workspace`` (zero-filled once, reused); when None and
    the call needs one, a zero-filled tensor kept per (device, stream) is used."""
    torch = _torch()
    _need(target_probs, "target_probs", (torch.float32,), None, 3)
    dev = target_probs.device
    B, N, V = target_probs.shape
    D = N - 1
    if draft_probs is not None:
        _need(draft_probs, "draft_probs", (torch.float32,), dev, 3)
        if tuple(draft_probs.shape) != (B, D, V):
            raise ValueError(f"draft_probs must be [{B},{D},{V}]")
    _need(draft_ids, "draft_ids", (torch.int32,), dev, 2)
    if tuple(draft_ids.shape) != (B, D):
        raise ValueError(f"draft_ids must be [{B},{D}]")
    _u64(seed, "seed", B, dev)
    _u64(offset, "offset", B, dev)
    req_index, n_req = _req(req_index, B, dev)
    if out is None:
        acc = torch.empty((B, N), dtype=torch.int32, device=dev)
        alen = torch.empty((B,), dtype=torch.int32, device=dev)
    else:
        acc, alen = out
    ws, ws_bytes = _workspace(workspace, n_req, V, dev)
    st = lib().specverify_chain_reject(
        _ptr(draft_probs), _ptr(draft_ids), _ptr(target_probs), _ptr(seed), _ptr(offset), B, D, V,
        _ptr(req_index), n_req, _ptr(acc), _ptr(alen), _ptr(ws), ws_bytes, _stream_ptr(dev))
    _check("specverify_chain_reject", st)
    return acc, alen


def chain_reject_noalloc(draft_probs, draft_ids, target_probs, seed, offset, req_index=None, out=None):
    """Chain rejection through the entry point that allocates nothing (the library's static scratch of
    STATIC_SCRATCH_BYTES per device; calls overlapping on one device race).  ``out`` must be given to
    allocate nothing here either."""
    torch = _torch()
    _need(target_probs, "target_probs", (torch.float32,), None, 3)
    dev = target_probs.device
    B, N, V = target_probs.shape
    D = N - 1
    if draft_probs is not None:
        _need(draft_probs, "draft_probs", (torch.float32,), dev, 3)
        if tuple(draft_probs.shape) != (B, D, V):
            raise ValueError(f"draft_probs must be [{B},{D},{V}]")
    _need(draft_ids, "draft_ids", (torch.int32,), dev, 2)
    if tuple(draft_ids.shape) != (B, D):
        raise ValueError(f"draft_ids must be [{B},{D}]")
    _u64(seed, "seed", B, dev)
    _u64(offset, "offset", B, dev)
    req_index, n_req = _req(req_index, B, dev)
    if out is None:
        acc = torch.empty((B, N), dtype=torch.int32, device=dev)
        alen = torch.empty((B,), dtype=torch.int32, device=dev)
    else:
        acc, alen = out
    st = lib().specverify_chain_reject_noalloc(
        _ptr(draft_probs), _ptr(draft_ids), _ptr(target_probs), _ptr(seed), _ptr(offset), B, D, V,
        _ptr(req_index), n_req, _ptr(acc), _ptr(alen), _stream_ptr(dev))
    _check("specverify_chain_reject_noalloc", st)
    return acc, alen


def _query(fn, n_req, D) -> int:
    out = ctypes.c_int64(0)
    _check(fn, getattr(lib(), fn)(int(n_req), int(D), ctypes.byref(out)))
    return int(out.value)


def verify_fused_workspace_bytes(n_req, D) -> int:
    """Bytes of the per-request lines verify_fused's one-workgroup-per-row form uses (0: none)."""
    return _query("specverify_verify_fused_workspace_bytes", n_req, D)


def greedy_verify_workspace_bytes(n_req, D) -> int:
    """Bytes of the per-request words of greedy_verify's one-workgroup-per-row form (0: none)."""
    return _query("specverify_greedy_verify_workspace_bytes", n_req, D)


def gumbel_sample_workspace_bytes(n_req, D) -> int:
    """Bytes of gumbel_sample's workspace: request lines, a helper count and a line per later row (0: none)."""
    return _query("specverify_gumbel_sample_workspace_bytes", n_req, D)


_counter_workspaces = {}


def _counter_workspace(kind, n, workspace, device):
    """(tensor, bytes) for a workspace of n bytes: the caller's tensor, none for n == 0 or
    workspace=False, else a zeroed buffer kept per (kind, device, stream); the library leaves it zero."""
    torch = _torch()
    if n == 0 or workspace is False:
        return None, 0
    if workspace is not None:
        _need(workspace, "workspace", (torch.uint8,), device, 1)
        return workspace, int(workspace.numel())
    key = (kind, device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _counter_workspaces.get(key)
    if ws is None or ws.numel() < n:
        ws = torch.zeros((n,), dtype=torch.uint8, device=device)
        _counter_workspaces[key] = ws
    return ws, int(ws.numel())


def _fused_workspace(workspace, n_req, D, device):
    return _counter_workspace("fused", verify_fused_workspace_bytes(n_req, D), workspace, device)


def verify_fused(target_logits, temperature, draft_probs, draft_ids, seed, offset, top_k=None, top_p=None,
                 req_index=None, out=None, workspace=None):
    """Target rows from logits (softmax, top-k, top-p) then chain rejection, in one call;
    returns (accepted_tokens [B, D+1] int32, accept_length [B] int32).  With a zero-filled uint8
    workspace of verify_fused_workspace_bytes(n_req, D) bytes (kept per device and stream when
    ``workspace`` is None; False for none) every target row gets a workgroup of its own."""
    torch = _torch()
    _need(target_logits, "target_logits", (torch.float32, torch.bfloat16), None, 3)
    dev = target_logits.device
    B, N, V = target_logits.shape
    D = N - 1
    _need(temperature, "temperature", (torch.float32,), dev, 1)
    if top_k is not None:
        _need(top_k, "top_k", (torch.int32,), dev, 1)
    if top_p is not None:
        _need(top_p, "top_p", (torch.float32,), dev, 1)
    for name, t in (("temperature", temperature), ("top_k", top_k), ("top_p", top_p)):
        if t is not None and t.shape[0] != B:
            raise ValueError(f"{name} must have shape [{B}]")
    _need(draft_probs, "draft_probs", (torch.float32,), dev, 3)
    _need(draft_ids, "draft_ids", (torch.int32,), dev, 2)
    if tuple(draft_probs.shape) != (B, D, V) or tuple(draft_ids.shape) != (B, D):
        raise ValueError(f"draft_probs must be [{B},{D},{V}] and draft_ids [{B},{D}]")
    _u64(seed, "seed", B, dev)
    _u64(offset, "offset", B, dev)
    req_index, n_req = _req(req_index, B, dev)
    if out is None:
        acc = torch.empty((B, N), dtype=torch.int32, device=dev)
        alen = torch.empty((B,), dtype=torch.int32, device=dev)
    else:
        acc, alen = out
    ws, ws_bytes = _fused_workspace(workspace, n_req, D, dev)
    st = lib().specverify_verify_fused(
        _ptr(target_logits), _logit_dtype(target_logits), _ptr(temperature), _ptr(top_k), _ptr(top_p),
        _ptr(draft_probs), _ptr(draft_ids), _ptr(seed), _ptr(offset), B, D, V, _ptr(req_index), n_req, _ptr(acc),
        _ptr(alen), _ptr(ws), ws_bytes, _stream_ptr(dev))
    _check("specverify_verify_fused", st)
    return acc, alen


def chain_reject_ragged(draft_probs, draft_ids, target_probs, qo_indptr, seed, offset, req_index=None, out=None,
                        t2d=None, workspace=None):
    """Ragged chain rejection over packed target rows [n_rows, V]; request b owns rows
    [qo_indptr[b], qo_indptr[b+1]).  Returns (accepted_tokens [B, D+1] int32,
    accept_length [B] int32); ``draft_probs`` None means point-mass drafts.  With ``t2d``
    (from ``d2t_inverse``) the draft rows are [B, D, Vd] over a smaller draft vocabulary."""
    torch = _torch()
    _need(target_probs, "target_probs", (torch.float32,), None, 2)
    dev = target_probs.device
    n_rows, V = target_probs.shape
    _need(draft_ids, "draft_ids", (torch.int32,), dev, 2)
    B, D = draft_ids.shape
    Vd = V
    if t2d is not None:
        if draft_probs is None:
            raise ValueError("t2d needs draft_probs")
        _need(t2d, "t2d", (torch.int32,), dev, 1)
        if t2d.shape[0] != V:
            raise ValueError(f"t2d must have shape [{V}]")
        Vd = int(draft_probs.shape[-1])
    if draft_probs is not None:
        _need(draft_probs, "draft_probs", (torch.float32,), dev, 3)
        if tuple(draft_probs.shape) != (B, D, Vd):
            raise ValueError(f"draft_probs must be [{B},{D},{Vd}]")
    _need(qo_indptr, "qo_indptr", (torch.int32,), dev, 1)
    if qo_indptr.shape[0] != B + 1:
        raise ValueError(f"qo_indptr must have shape [{B + 1}]")
    _u64(seed, "seed", B, dev)
    _u64(offset, "offset", B, dev)
    req_index, n_req = _req(req_index, B, dev)
    if out is None:
        acc = torch.empty((B, D + 1), dtype=torch.int32, device=dev)
        alen = torch.empty((B,), dtype=torch.int32, device=dev)
    else:
        acc, alen = out
    ws, ws_bytes = _workspace(workspace, n_req, V, dev)
    st = lib().specverify_chain_reject_ragged(
        _ptr(draft_probs), _ptr(t2d), Vd, _ptr(draft_ids), _ptr(target_probs), _ptr(qo_indptr), n_rows, _ptr(seed),
        _ptr(offset), B, D, V, _ptr(req_index), n_req, _ptr(acc), _ptr(alen), _ptr(ws), ws_bytes,
        _stream_ptr(dev))
    _check("specverify_chain_reject_ragged", st)
    return acc, alen


def d2t_inverse(d2t, Vd, V, device=None, out=None):
    """Inverse map t2d [V] int32 (draft entry of each target entry, -1 for none) of the offset
    table d2t [Vd] int64 (None: the first Vd target entries); built once per table."""
    torch = _torch()
    if d2t is not None:
        _need(d2t, "d2t", (torch.int64,), None, 1)
        if d2t.shape[0] != Vd:
            raise ValueError(f"d2t must have shape [{Vd}]")
        device = d2t.device
    if device is None:
        raise ValueError("device is required when d2t is None")
    if out is None:
        out = torch.empty((int(V),), dtype=torch.int32, device=device)
    else:
        _need(out, "out", (torch.int32,), torch.device(device), 1)
    st = lib().specverify_d2t_inverse(_ptr(d2t), int(Vd), int(V), _ptr(out), _stream_ptr(torch.device(device)))
    _check("specverify_d2t_inverse", st)
    return out


def d2t_expand(draft_probs, t2d, out=None):
    """Place draft_probs [..., Vd] into the target vocabulary with the inverse map t2d [V]:
    [..., V], entry t = draft_probs[..., t2d[t]] (0 where t2d[t] < 0)."""
    torch = _torch()
    _need(draft_probs, "draft_probs", (torch.float32,), None)
    dev = draft_probs.device
    _need(t2d, "t2d", (torch.int32,), dev, 1)
    Vd, V = int(draft_probs.shape[-1]), int(t2d.shape[0])
    rows = draft_probs.numel() // Vd if Vd else 0
    shape = tuple(draft_probs.shape[:-1]) + (V,)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=dev)
    else:
        _need(out, "out", (torch.float32,), dev)
        if tuple(out.shape) != shape:
            raise ValueError(f"out must be {shape}")
    st = lib().specverify_d2t_expand(_ptr(draft_probs), _ptr(t2d), rows, Vd, V, _ptr(out), _stream_ptr(dev))
    _check("specverify_d2t_expand", st)
    return out


def sample(logits, temperature, seed, offset, top_k=None, top_p=None, min_p=None, req_index=None, out=None):
    """Single-step sampling: one token per row of logits [B, V] (float32 or bfloat16); returns tokens [B] int32."""
    torch = _torch()
    _need(logits, "logits", (torch.float32, torch.bfloat16), None, 2)
    dev = logits.device
    B, V = logits.shape
    _need(temperature, "temperature", (torch.float32,), dev, 1)
    if top_k is not None:
        _need(top_k, "top_k", (torch.int32,), dev, 1)
    if top_p is not None:
        _need(top_p, "top_p", (torch.float32,), dev, 1)
    if min_p is not None:
        _need(min_p, "min_p", (torch.float32,), dev, 1)
    _u64(seed, "seed", B, dev)
    _u64(offset, "offset", B, dev)
    req_index, n_req = _req(req_index, B, dev)
    if out is None:
        out = torch.empty((B,), dtype=torch.int32, device=dev)
    st = lib().specverify_sample(_ptr(logits), _logit_dtype(logits), _ptr(temperature), _ptr(top_k), _ptr(top_p),
                                 _ptr(min_p), _ptr(seed), _ptr(offset), B, V, _ptr(req_index), n_req, _ptr(out),
                                 _stream_ptr(dev))
    _check("specverify_sample", st)
    return out


def greedy_verify(target_logits, draft_ids, req_index=None, predict=True, accept_index=True,
                  argmax=False, out=None, workspace=None):
    """Greedy chain verify; returns a dict of int32 tensors:
    accepted_tokens [B, N], accept_length [B], and optionally predict [B, N],
    accept_index [B, N] (flat index into predict), argmax [B, N] (forces every row).
    workspace: uint8 tensor of greedy_verify_workspace_bytes(n_req, D) bytes (zero before the
    first call; kept per device and stream when None; False for the one-workgroup-per-request form)."""
    torch = _torch()
    _need(target_logits, "target_logits", (torch.float32, torch.bfloat16), None, 3)
    dev = target_logits.device
    B, N, V = target_logits.shape
    D = N - 1
    _need(draft_ids, "draft_ids", (torch.int32,), dev, 2)
    if tuple(draft_ids.shape) != (B, D):
        raise ValueError(f"draft_ids must be [{B},{D}]")
    req_index, n_req = _req(req_index, B, dev)
    o = dict(out) if out is not None else {}

    def mk(key, shape, want=True):
        if not want:
            return None
        if key not in o:
            o[key] = torch.empty(shape, dtype=torch.int32, device=dev)
        return o[key]

    acc = mk("accepted_tokens", (B, N))
    alen = mk("accept_length", (B,))
    pr = mk("predict", (B, N), predict)
    ai = mk("accept_index", (B, N), accept_index)
    am = mk("argmax", (B, N), argmax)
    ws, ws_bytes = _counter_workspace("rows", greedy_verify_workspace_bytes(n_req, D), workspace, dev)
    st = lib().specverify_greedy_verify(
        _ptr(target_logits), _logit_dtype(target_logits), _ptr(draft_ids), B, D, V, _ptr(req_index), n_req,
        _ptr(acc), _ptr(alen), _ptr(pr), _ptr(ai), _ptr(am), _ptr(ws), ws_bytes, _stream_ptr(dev))
    _check("specverify_greedy_verify", st)
    return o


def gumbel_sample(target_logits, temperature, draft_ids, seed, offset, req_index=None, sampled=False,
                  out=None, workspace=None):
    """Gumbel-max temperature sampling + strict acceptance; returns a dict of
    int32 tensors accepted_tokens [B, N], accept_length [B] and optionally
    sampled [B, N] (forces every row).  workspace: as for greedy_verify, of
    gumbel_sample_workspace_bytes(n_req, D) bytes."""
    torch = _torch()
    _need(target_logits, "target_logits", (torch.float32, torch.bfloat16), None, 3)
    dev = target_logits.device
    B, N, V = target_logits.shape
    D = N - 1
    _need(temperature, "temperature", (torch.float32,), dev, 1)
    _need(draft_ids, "draft_ids", (torch.int32,), dev, 2)
    if tuple(draft_ids.shape) != (B, D) or temperature.shape[0] != B:
        raise ValueError(f"draft_ids must be [{B},{D}] and temperature [{B}]")
    _u64(seed, "seed", B, dev)
    _u64(offset, "offset", B, dev)
    req_index, n_req = _req(req_index, B, dev)
    o = dict(out) if out is not None else {}
    for key, shape, want in (("accepted_tokens", (B, N), True), ("accept_length", (B,), True),
                             ("sampled", (B, N), sampled)):
        if want and key not in o:
            o[key] = torch.empty(shape, dtype=torch.int32, device=dev)
    ws, ws_bytes = _counter_workspace("rows", gumbel_sample_workspace_bytes(n_req, D), workspace, dev)
    st = lib().specverify_gumbel_sample(
        _ptr(target_logits), _logit_dtype(target_logits), _ptr(temperature), _ptr(draft_ids), _ptr(seed),
        _ptr(offset), B, D, V, _ptr(req_index), n_req, _ptr(o["accepted_tokens"]), _ptr(o["accept_length"]),
        _ptr(o.get("sampled")), _ptr(ws), ws_bytes, _stream_ptr(dev))
    _check("specverify_gumbel_sample", st)
    return o


def version() -> int:
    return int(lib().specverify_version())
