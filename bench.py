#!/usr/bin/env python3
"""Benchmark of the speculative-decoding verify path on one MI355X.

Default workload: chain rejection sampling on the large-vocabulary batch
(B=256 requests, D=5 drafts, V=128256, float32 target and draft
probabilities).  One step = one ``specverify_chain_reject`` call over the
whole batch.  Metric: verified vocab rows per second, B * (D + 1) per step,
plus the dominant kernel's achieved HBM bandwidth (algorithmic bytes / kernel
time) against the 8 TB/s peak.

Inputs are synthetic (see workloads/), resident in HBM before timing; R
replicas (copies at distinct addresses with distinct Philox offsets) rotate
so consecutive calls never hit the 256 MB Infinity Cache with the previous
call's rows.  Timing uses HIP events on the stream the kernels run on.

Other workloads (``--workload``) exist for profiling: ``topk_topp_chain``
(softmax_renorm -> chain_reject, B=64 D=3 V=32000 bf16), ``greedy`` (greedy
verify, B=512 N=4 V=151936 bf16), ``mixed`` (B=1024 D=7 V=129280 bf16: 256
requests each greedy, temperature-only (Gumbel), top-k and top-p, every mode
dispatched through req_index; per-call times are reported), ``mixed_fused``
(the same with the fused verify for the top-k/top-p requests),
``large_vocab_target_only`` (the default inputs without draft
probabilities), ``large_vocab_ragged`` (per-request verify lengths U{1..6}
over packed rows; rows/s counts the verified rows), ``large_vocab_ragged_d2t``
(the same with draft rows over a 32000-entry draft vocabulary read through
the inverse d2t table), ``d2t_expand`` (1280
draft rows of a 32000-entry draft vocabulary placed in V=128256),
``sample`` (single-step sampling of 1024 bf16 rows of V=129280) and
``gumbel`` (the mixed batch's 256 temperature-only requests through the
Gumbel-max call alone; arithmetic-bound, so its roofline is the vector
ALU's: entries/s against the issue rate of the kernel's instruction mix and
against a probe running the same arithmetic with no memory traffic).

The CPU baseline is the numpy oracle timed on this host on the same inputs
(whole batches repeated for --cpu-seconds), single threaded.  For the chain
workloads that leg also compares the oracle's outputs with the GPU's outputs
of the same replicas and reports the counts (``parity``).

Beside the 8 TB/s data-sheet peak, the roofline reports the fraction of a
read rate measured on the same GPU in the same run by a plain read-stream
kernel (``libsvprobe.so``, best of a small sweep of grid sizes and loads in
flight), once reading 1 GiB per launch (the asymptotic rate) and once
reading the kernel's own algorithmic byte count (what a pure stream of that
size reaches, start-up and tail included), and the per-call time distribution (p10 / median / p90 over groups
of 10 consecutive calls, one HIP event pair per group).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "verified vocab rows/sec (batch×(D+1)) + achieved HBM GB/s vs MI355X peak"
PEAK_HBM_GBS = 8000.0
PROBE_GRANULE = 64     # bytes a single-element probe costs in HBM (one 64-byte line)
# Vector ALU issue of MI355X: 256 CUs x 4 SIMDs at 2.4 GHz, one wave64
# instruction per SIMD every 4 cycles (16 lanes per cycle).
SIMD_CYCLES_PER_S = 256 * 4 * 2.4e9
# The Gumbel-max hot loop as compiled for gfx950 (one pipelined iteration of
# gumbel_sample.hip = 4 groups of 4 entries per lane) issues 473 VALU
# instructions: 136 v_xor, 68 v_mad_u64_u32 (the Philox products), 48
# v_mul_f32, 32 v_log_f32, 16 v_fmac_f32 and 173 others (compares, selects,
# adds, shifts, conversions).  On gfx950 the 64-bit multiply-add and the
# logarithm issue at the full rate like the rest (the arithmetic probe,
# svprobe_gumbel_alu, runs this mix at 3.9 cycles per wave64 instruction), so
# a group costs 473 / 4 instructions x 4 cycles per wave64.
GUMBEL_VALU_PER_GROUP = 473 / 4
GUMBEL_CYCLES_PER_GROUP = GUMBEL_VALU_PER_GROUP * 4
# entries per second with every SIMD issuing that loop without a stall
GUMBEL_ALU_PEAK_GES = SIMD_CYCLES_PER_S * 64 * 4 / GUMBEL_CYCLES_PER_GROUP / 1e9


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="large_vocab_chain_reject",
                    choices=["large_vocab_chain_reject", "large_vocab_target_only", "large_vocab_ragged",
                             "large_vocab_ragged_d2t", "d2t_expand",
                             "sample", "topk_topp_chain", "topk_topp_fused", "greedy",
                             "mixed", "mixed_fused", "gumbel"])
    ap.add_argument("--replicas", type=int, default=0, help="input replicas (0 = workload default)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle baseline budget (0 disables)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB -> 1 GiB elementwise copy 5 times (HBM counter calibration)")
    return ap.parse_args()


def copy_calibration():
    """A plain copy kernel of known size: 2**28 floats read and written per launch."""
    import torch
    a = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        torch.mul(a, 1.0, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read_per_launch": 4 << 28,
                      "copy_calibration_bytes_written_per_launch": 4 << 28, "launches": 5}), flush=True)


# --------------------------------------------------------------------------- device helpers
def _t(a, dev):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint64:
        a = a.view(np.int64)
    return torch.from_numpy(a).to(dev)


def _bf16(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)


def _source_digest(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "token_sampling_temp_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(summary, digest):
    """HBM bytes per launch from a committed counter summary, if it was taken on this kernel source."""
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_src = re.search(r"source_digest:\s*([0-9a-f]+)", txt)
    m_b = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m_src or not m_b or m_src.group(1) != digest:
        return None
    return float(m_b.group(1))


def cpu_info():
    """Host CPU facts for the baseline: logical CPUs, CPUs this process may run on, model name."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {"cpu_count": os.cpu_count(), "affinity": affinity, "cpu_model": model}


class ParityCount:
    """Request-level comparison of GPU chain outputs with the oracle's: accept lengths always
    exact (they follow from exact products), tokens exact up to the oracle's excluded position."""

    def __init__(self):
        self.requests = self.exact = self.near_accept = self.near_cdf = self.excluded = self.mismatches = 0

    def add(self, acc, alen, ref, reqs=None):
        reqs = range(len(alen)) if reqs is None else reqs
        for b in reqs:
            L, fp = int(ref["accept_length"][b]), int(ref["flag_pos"][b])
            ok = int(alen[b]) == L
            n = min(fp, L + 1)
            ok = ok and list(acc[b, :n]) == list(ref["accepted_tokens"][b, :n]) and bool(np.all(acc[b, L + 1:] == -1))
            self.requests += 1
            self.mismatches += not ok
            self.exact += bool(ok and list(acc[b]) == list(ref["accepted_tokens"][b]))
            self.near_accept += int(ref["near_accept"][b]) >= 0
            self.near_cdf += bool(ref["near_cdf"][b])
            self.excluded += fp <= L

    def report(self):
        return {"requests": self.requests, "exact": self.exact, "flagged_accept": self.near_accept,
                "flagged_cdf": self.near_cdf, "excluded": self.excluded, "mismatches": self.mismatches,
                "bands": "flagged_*: within 1e-6 of an accept threshold / CDF boundary (reported); excluded: "
                         "draws within 8 (V + 1) 2^-53 of a CDF boundary, tokens from there not compared"}


def stream_peak(dev, nbytes=1 << 30):
    """The HBM read rate a plain read-stream kernel reaches here (GB/s) when it reads `nbytes` per launch:
    best over grids of 256..2048 workgroups and 4..16 loads in flight, four buffers rotating so nothing
    is served from the 256 MB Infinity Cache.  At 1 GiB this is the asymptotic read rate; at a kernel's
    own byte count it is the rate a pure stream of that size reaches, start-up and tail included."""
    import ctypes
    import torch
    L = ctypes.CDLL(os.path.join(ROOT, "token_sampling_temp_amd", "libsvprobe.so"))
    L.svprobe_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_void_p, ctypes.c_void_p]
    L.svprobe_read_stream.restype = ctypes.c_int
    nbytes = max(16, int(nbytes) // 16 * 16)
    bufs = [torch.zeros(nbytes // 4, dtype=torch.float32, device=dev) for _ in range(4)]
    sink = torch.zeros(4 * 4096, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    best = (0.0, None)
    for grid in (256, 512, 1024, 2048):
        for loads in (4, 8, 16):
            def run(i):
                st = L.svprobe_read_stream(ctypes.c_void_p(bufs[i % 4].data_ptr()), nbytes, grid, loads,
                                           ctypes.c_void_p(sink.data_ptr()), sp)
                assert st == 0, st
            for i in range(4):
                run(i)
            s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s0.record(stream)
            n = 12
            for i in range(n):
                run(i)
            s1.record(stream)
            torch.cuda.synchronize()
            gbs = nbytes * n / (s0.elapsed_time(s1) * 1e-3) / 1e9
            if gbs > best[0]:
                best = (gbs, {"grid": grid, "loads_in_flight": loads})
    del bufs
    torch.cuda.empty_cache()
    return best


# --------------------------------------------------------------------------- workloads
class ChainWorkload:
    """B=256 D=5 V=128256 chain rejection on float32 probabilities."""
    name = "large_vocab_chain_reject"
    kernel = "chain_reject_kernel"
    sources = ("chain_reject.hip", "sv_draw.hpp", "sv_common.hpp")
    counters = "chain_reject_large_vocab_counters.txt"
    dtype = "f32"

    def __init__(self, dev, replicas):
        from workloads import make_config
        t0 = time.time()
        self.host = make_config(3)
        log(f"generated inputs in {time.time() - t0:.1f}s")
        h = self.host
        self.B, self.D, self.V = h["B"], h["D"], h["V"]
        self.R = replicas or 4
        self.reps = []
        for r in range(self.R):
            off = np.full(self.B, 4096 * r, np.uint64)
            self.reps.append(dict(q=_t(h["draft_probs"], dev), x=_t(h["draft_ids"], dev),
                                  p=_t(h["target_probs"], dev), seed=_t(h["seed"], dev), off=_t(off, dev),
                                  off_host=off))
        import token_sampling_temp_amd as sv
        self.sv = sv
        import torch
        self.acc = torch.empty((self.B, self.D + 1), dtype=torch.int32, device=dev)
        self.alen = torch.empty((self.B,), dtype=torch.int32, device=dev)
        self.rows = self.B * (self.D + 1)

    def step(self, i):
        r = self.reps[i % self.R]
        self.sv.chain_reject(r["q"], r["x"], r["p"], r["seed"], r["off"], out=(self.acc, self.alen))

    def algorithmic_bytes(self):
        """Bytes the method must move per call, from each replica's realised accept lengths."""
        per = []
        self.L = []
        self.gpu_out = []
        for i in range(self.R):
            self.step(i)
            L = self.alen.cpu().numpy().astype(np.int64)
            self.L.append(L)
            self.gpu_out.append((self.acc.cpu().numpy().astype(np.int64), L))
            D, V = self.D, self.V
            rows = np.where(L < D, 8 * V, 4 * V)
            probes = 2 * PROBE_GRANULE * np.minimum(L + 1, D)
            per.append(int(rows.sum() + probes.sum() + self.B * (8 * D + 24)))
        return float(np.mean(per))

    def oracle_call(self, r):
        import oracle
        h = self.host
        return oracle.chain_reject(h["draft_probs"], h["draft_ids"], h["target_probs"], h["seed"],
                                   self.reps[r]["off_host"])

    def extra(self):
        L = np.concatenate(self.L)
        # realised acceptance rate at position i: requests accepting i, among those that reached i
        alpha = [round(float(np.mean(L[L >= i] > i)), 4) for i in range(self.D) if np.any(L >= i)]
        return {"mean_accept_length": round(float(L.mean()), 4),
                "frac_all_accepted": round(float(np.mean(L == self.D)), 4), "alpha_per_position": alpha}

    def config(self):
        return {"workload": self.name, "batch": self.B, "draft_tokens": self.D, "vocab": self.V,
                "input": "float32 target/draft probabilities", "replicas": self.R}

    def cpu_baseline(self, seconds):
        """The oracle on whole batches, replicas rotating, for ``seconds``; each replica's first pass is
        also compared with the GPU's outputs of that replica (timed all the same: the comparison is a
        few ms against ~0.1 s of oracle work per batch)."""
        par = ParityCount()
        rows, t0, passes = 0, time.perf_counter(), 0
        while True:
            r = passes % self.R
            ref = self.oracle_call(r)
            if passes < self.R:
                par.add(*self.gpu_out[r], ref)
            rows += self.rows
            passes += 1
            el = time.perf_counter() - t0
            if el >= seconds and passes >= self.R:
                break
        self.parity = par.report()
        return dict({"value": rows / el, "unit": "rows/s", "cores": 1, "kind": "oracle",
                     "sample": f"{passes} full batches of {self.B} requests (replica offsets rotating), "
                               f"{el:.1f}s single-threaded numpy"}, **cpu_info())


class TargetOnlyWorkload(ChainWorkload):
    """The large-vocab chain inputs verified without draft probabilities (point-mass drafts)."""
    name = "large_vocab_target_only"
    counters = "chain_reject_target_only_counters.txt"

    def step(self, i):
        r = self.reps[i % self.R]
        self.sv.chain_reject(None, r["x"], r["p"], r["seed"], r["off"], out=(self.acc, self.alen))

    def algorithmic_bytes(self):
        """Per request: one target line per probed position, one target row (p_L or the bonus row p_D)."""
        per = []
        self.L = []
        self.gpu_out = []
        for i in range(self.R):
            self.step(i)
            L = self.alen.cpu().numpy().astype(np.int64)
            self.L.append(L)
            self.gpu_out.append((self.acc.cpu().numpy().astype(np.int64), L))
            D, V = self.D, self.V
            probes = PROBE_GRANULE * np.minimum(L + 1, D)
            per.append(int(4 * V * self.B + probes.sum() + self.B * (8 * D + 24)))
        return float(np.mean(per))

    def config(self):
        c = super().config()
        c["input"] = "float32 target probabilities, draft ids only (no draft probabilities)"
        return c

    def oracle_call(self, r):
        import oracle
        h = self.host
        return oracle.chain_reject(None, h["draft_ids"], h["target_probs"], h["seed"], self.reps[r]["off_host"])


class RaggedWorkload:
    """The large-vocab chain inputs with per-request verify lengths len_b ~ U{1..6} over packed target rows."""
    name = "large_vocab_ragged"
    kernel = "chain_reject_kernel"
    sources = ("chain_reject.hip", "sv_draw.hpp", "sv_common.hpp")
    counters = "chain_reject_ragged_counters.txt"
    dtype = "f32"

    def __init__(self, dev, replicas):
        from workloads import make_ragged_config
        t0 = time.time()
        self.host = make_ragged_config()
        log(f"generated inputs in {time.time() - t0:.1f}s")
        h = self.host
        self.B, self.D, self.V = h["B"], h["D"], h["V"]
        self.R = replicas or 4
        self.reps = []
        for r in range(self.R):
            off = np.full(self.B, 4096 * r, np.uint64)
            self.reps.append(dict(q=_t(h["draft_probs"], dev), x=_t(h["draft_ids"], dev),
                                  p=_t(h["target_rows"], dev), ind=_t(h["qo_indptr"], dev), seed=_t(h["seed"], dev),
                                  off=_t(off, dev), off_host=off))
        import token_sampling_temp_amd as sv
        self.sv = sv
        import torch
        self.acc = torch.empty((self.B, self.D + 1), dtype=torch.int32, device=dev)
        self.alen = torch.empty((self.B,), dtype=torch.int32, device=dev)
        self.rows = int(h["verify_lens"].sum())

    def step(self, i):
        r = self.reps[i % self.R]
        self.sv.chain_reject_ragged(r["q"], r["x"], r["p"], r["ind"], r["seed"], r["off"], out=(self.acc, self.alen))

    def algorithmic_bytes(self):
        """Per request: one target and one draft line per probed position, then the row pass its outcome
        needs: p_L and q_L after a rejection before its last position d, p_d after a rejection at d (or the
        bonus when d = D), nothing when token 0 was accepted at d."""
        per = []
        self.L = []
        d = self.host["verify_lens"] - 1
        self.gpu_out = []
        for i in range(self.R):
            self.step(i)
            L = self.alen.cpu().numpy().astype(np.int64)
            tok = self.acc.cpu().numpy()
            self.L.append(L)
            self.gpu_out.append((tok.astype(np.int64), L))
            D, V = self.D, self.V
            at_d = tok[np.arange(self.B), np.minimum(L, D)]
            rows = np.where(L < d, 8 * V, np.where((d < D) & (at_d == 0), 0, 4 * V))
            probes = 2 * PROBE_GRANULE * np.minimum(L + 1, D)
            per.append(int(rows.sum() + probes.sum() + self.B * (8 * D + 32)))
        return float(np.mean(per))

    def extra(self):
        L = np.concatenate(self.L)
        return {"mean_accept_length": round(float(L.mean()), 4),
                "mean_verify_length": round(float(self.host["verify_lens"].mean()), 4)}

    def config(self):
        return {"workload": self.name, "batch": self.B, "draft_tokens": self.D, "vocab": self.V,
                "verified_rows": self.rows, "input": "float32 packed target rows, per-request verify lengths "
                "U{1..6}, float32 draft probabilities", "replicas": self.R}

    def oracle_call(self, r):
        import oracle
        h = self.host
        return oracle.chain_reject_ragged(h["draft_probs"], h["draft_ids"], h["target_rows"], h["qo_indptr"],
                                          h["seed"], self.reps[r]["off_host"])

    cpu_baseline = ChainWorkload.cpu_baseline


class RaggedD2tWorkload(RaggedWorkload):
    """The ragged large-vocab inputs with a draft model over a 32000-entry draft vocabulary: the verify reads
    the draft rows [256, 5, 32000] through the inverse d2t table, with no expanded rows."""
    name = "large_vocab_ragged_d2t"
    counters = "chain_reject_ragged_d2t_counters.txt"

    def __init__(self, dev, replicas):
        from workloads import make_ragged_d2t_config
        t0 = time.time()
        self.host = make_ragged_d2t_config()
        log(f"generated inputs in {time.time() - t0:.1f}s")
        h = self.host
        self.B, self.D, self.V = h["B"], h["D"], h["V"]
        self.Vd = h["draft_probs_d"].shape[-1]
        self.R = replicas or 4
        import token_sampling_temp_amd as sv
        import torch
        self.sv = sv
        self.t2d = sv.d2t_inverse(_t(h["d2t"], dev), self.Vd, self.V)   # once per table
        self.reps = []
        for r in range(self.R):
            off = np.full(self.B, 4096 * r, np.uint64)
            self.reps.append(dict(q=_t(h["draft_probs_d"], dev), x=_t(h["draft_ids"], dev),
                                  p=_t(h["target_rows"], dev), ind=_t(h["qo_indptr"], dev), seed=_t(h["seed"], dev),
                                  off=_t(off, dev), off_host=off))
        self.acc = torch.empty((self.B, self.D + 1), dtype=torch.int32, device=dev)
        self.alen = torch.empty((self.B,), dtype=torch.int32, device=dev)
        self.rows = int(h["verify_lens"].sum())

    def step(self, i):
        r = self.reps[i % self.R]
        self.sv.chain_reject_ragged(r["q"], r["x"], r["p"], r["ind"], r["seed"], r["off"], out=(self.acc, self.alen),
                                    t2d=self.t2d)

    def algorithmic_bytes(self):
        """As the ragged workload, with a draft row costing 4 Vd (read through the table) and the table
        (4 V) read once per launch."""
        per = []
        self.L = []
        d = self.host["verify_lens"] - 1
        self.gpu_out = []
        for i in range(self.R):
            self.step(i)
            L = self.alen.cpu().numpy().astype(np.int64)
            tok = self.acc.cpu().numpy()
            self.L.append(L)
            self.gpu_out.append((tok.astype(np.int64), L))
            D, V, Vd = self.D, self.V, self.Vd
            at_d = tok[np.arange(self.B), np.minimum(L, D)]
            rows = np.where(L < d, 4 * V + 4 * Vd, np.where((d < D) & (at_d == 0), 0, 4 * V))
            probes = 3 * PROBE_GRANULE * np.minimum(L + 1, D)
            per.append(int(rows.sum() + probes.sum() + self.B * (8 * D + 32) + 4 * V))
        return float(np.mean(per))

    def config(self):
        c = super().config()
        c["input"] = ("float32 packed target rows, per-request verify lengths U{1..6}, float32 draft rows over a "
                      "32000-entry draft vocabulary read through the inverse d2t table")
        return c

    def oracle_call(self, r):
        import oracle
        h = self.host
        q_full = oracle.d2t_expand(h["draft_probs_d"], h["d2t"], self.V)
        return oracle.chain_reject_ragged(q_full, h["draft_ids"], h["target_rows"], h["qo_indptr"], h["seed"],
                                          self.reps[r]["off_host"])


class DraftVocabWorkload:
    """Draft distributions over a 32000-entry draft vocabulary placed into the 128256-entry target
    vocabulary (ascending d2t table), 256 requests x 5 drafts."""
    name = "d2t_expand"
    kernel = "d2t_expand_kernel"
    sources = ("d2t_expand.hip", "sv_common.hpp")
    counters = "d2t_expand_counters.txt"
    dtype = "f32"

    def __init__(self, dev, replicas):
        from workloads import make_d2t
        self.B, self.D, self.Vd, self.V = 256, 5, 32000, 128256
        rows = self.B * self.D
        rng = np.random.default_rng(7)
        q = rng.random((rows, self.Vd), dtype=np.float32)
        self.d2t_host = make_d2t(0, self.Vd, self.V)
        self.q_host = q
        self.R = replicas or 4
        import torch
        self.reps = [dict(q=_t(q, dev), out=torch.empty((rows, self.V), dtype=torch.float32, device=dev))
                     for _ in range(self.R)]
        import token_sampling_temp_amd as sv
        self.sv = sv
        self.t2d = sv.d2t_inverse(_t(self.d2t_host, dev), self.Vd, self.V)   # once per table
        self.rows = rows

    def step(self, i):
        r = self.reps[i % self.R]
        self.sv.d2t_expand(r["q"], self.t2d, out=r["out"])

    def algorithmic_bytes(self):
        """Per row: the target row written (4 V) and the draft row read (4 Vd); the inverse table
        (4 V) once."""
        return float(self.rows * (4 * self.V + 4 * self.Vd) + 4 * self.V)

    def extra(self):
        return {}

    def config(self):
        return {"workload": self.name, "rows": self.rows, "draft_vocab": self.Vd, "vocab": self.V,
                "input": "float32 draft probabilities, inverse table of an ascending d2t table", "replicas": self.R}

    def cpu_baseline(self, seconds):
        import oracle
        rows, t0, passes = 0, time.perf_counter(), 0
        while True:
            oracle.d2t_expand(self.q_host, self.d2t_host, self.V)
            rows += self.rows
            passes += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
        return {"value": rows / el, "unit": "rows/s", "cores": 1, "kind": "oracle",
                "sample": f"{passes} full expansions of {self.rows} rows, {el:.1f}s single-threaded numpy"}


class SampleWorkload:
    """Single-step sampling of 1024 bf16 rows of V=129280: a quarter greedy, the rest T ~ U[0.5, 1.2]
    with top-k in {0, 20, 100}, top-p 1 or U[0.8, 0.95] and min-p in {0, 0.05} (joint filter)."""
    name = "sample"
    kernel = "sample_kernel"
    sources = ("fused_verify.hip", "sv_softmax.hpp", "sv_draw.hpp", "sv_argmax.hpp", "sv_rowpar.hpp", "sv_common.hpp")
    counters = "sample_counters.txt"
    dtype = "bf16"

    def __init__(self, dev, replicas):
        from workloads import make_sample_config
        t0 = time.time()
        self.host = make_sample_config()
        log(f"generated inputs in {time.time() - t0:.1f}s")
        h = self.host
        self.B, self.V = h["logits"].shape
        self.R = replicas or 2
        self.reps = []
        for r in range(self.R):
            off = np.full(self.B, 4096 * r, np.uint64)
            self.reps.append(dict(z=_bf16(h["logits"], dev), T=_t(h["temperature"], dev), k=_t(h["top_k"], dev),
                                  p=_t(h["top_p"], dev), mp=_t(h["min_p"], dev), seed=_t(h["seed"], dev),
                                  off=_t(off, dev), off_host=off))
        import token_sampling_temp_amd as sv
        import torch
        self.sv = sv
        self.out = torch.empty((self.B,), dtype=torch.int32, device=dev)
        self.rows = self.B

    def step(self, i):
        r = self.reps[i % self.R]
        self.sv.sample(r["z"], r["T"], r["seed"], r["off"], top_k=r["k"], top_p=r["p"], min_p=r["mp"], out=self.out)

    def algorithmic_bytes(self):
        """One read of every logit row (2 V bytes) and the token written."""
        return float(self.B * (2 * self.V + 4) + self.B * 32)

    def extra(self):
        return {}

    def config(self):
        return {"workload": self.name, "batch": self.B, "vocab": self.V, "input": "bf16 logits, per-row "
                "temperature, top-k, top-p, min-p (joint filter)", "replicas": self.R}

    def cpu_baseline(self, seconds):
        import oracle
        h = self.host
        rows, t0, n = 0, time.perf_counter(), 0
        while True:
            reqs = [(n * 16 + j) % self.B for j in range(16)]
            oracle.sample(h["logits"], "bf16", h["temperature"], h["top_k"], h["top_p"], h["min_p"], h["seed"],
                          h["offset"], requests=reqs)
            rows += len(reqs)
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
        return {"value": rows / el, "unit": "rows/s", "cores": 1, "kind": "oracle",
                "sample": f"{rows} rows in groups of 16, {el:.1f}s single-threaded numpy"}


class GreedyWorkload:
    name = "greedy"
    kernel = "greedy_verify_kernel"
    sources = ("greedy_verify.hip", "sv_argmax.hpp", "sv_rowpar.hpp", "sv_common.hpp")
    counters = "greedy_verify_counters.txt"
    dtype = "bf16"

    def __init__(self, dev, replicas):
        from workloads import make_config
        import torch
        import token_sampling_temp_amd as sv
        self.sv = sv
        h = make_config(4)
        self.host = h
        self.B, self.D, self.V = h["B"], h["D"], h["V"]
        self.R = replicas or 2
        self.reps = [dict(z=_bf16(h["logits"], dev), x=_t(h["draft_ids"], dev)) for _ in range(self.R)]
        self.out = {"accepted_tokens": torch.empty((self.B, self.D + 1), dtype=torch.int32, device=dev),
                    "accept_length": torch.empty((self.B,), dtype=torch.int32, device=dev)}
        self.rows = self.B * (self.D + 1)

    def step(self, i):
        r = self.reps[i % self.R]
        self.sv.greedy_verify(r["z"], r["x"], predict=False, accept_index=False, out=self.out)

    def algorithmic_bytes(self):
        self.step(0)
        L = self.out["accept_length"].cpu().numpy().astype(np.int64)
        self.L = L
        return float(((L + 1) * self.V * 2).sum() + self.B * (4 * self.D + 4 * (self.D + 1) + 4))

    def extra(self):
        return {"mean_accept_length": round(float(self.L.mean()), 4)}

    def config(self):
        return {"workload": self.name, "batch": self.B, "draft_tokens": self.D, "vocab": self.V,
                "input": "bf16 logits", "replicas": self.R}

    def cpu_baseline(self, seconds):
        import oracle
        h = self.host
        rows, t0, n = 0, time.perf_counter(), 0
        while True:
            b = n % self.B
            oracle.greedy_verify(h["logits"], "bf16", h["draft_ids"], requests=[b])
            rows += self.D + 1
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
        return {"value": rows / el, "unit": "rows/s", "cores": 1, "kind": "oracle",
                "sample": f"{n} requests, {el:.1f}s single-threaded numpy"}


class TopkToppWorkload:
    name = "topk_topp_chain"
    kernel = "softmax_renorm_rr_kernel"
    dominant_call = "softmax_renorm"
    sources = ("softmax_renorm.hip", "sv_softmax.hpp", "sv_argmax.hpp", "sv_common.hpp")
    counters = "softmax_renorm_topk_topp_counters.txt"
    dtype = "bf16"

    def __init__(self, dev, replicas):
        from workloads import make_config
        import torch
        import token_sampling_temp_amd as sv
        self.sv = sv
        h = make_config(2)
        self.host = h
        self.B, self.D, self.V = h["B"], h["D"], h["V"]
        self.R = replicas or 8
        self.reps = [dict(z=_bf16(h["logits"], dev), q=_t(h["draft_probs"], dev), x=_t(h["draft_ids"], dev),
                          T=_t(h["temperature"], dev), k=_t(h["top_k"], dev), p=_t(h["top_p"], dev),
                          seed=_t(h["seed"], dev), off=_t(np.full(self.B, 4096 * r, np.uint64), dev))
                     for r in range(self.R)]
        N = self.D + 1
        self.probs = [torch.empty((self.B, N, self.V), dtype=torch.float32, device=dev) for _ in range(self.R)]
        self.acc = torch.empty((self.B, N), dtype=torch.int32, device=dev)
        self.alen = torch.empty((self.B,), dtype=torch.int32, device=dev)
        self.rows = self.B * N

        self.calls = {"softmax_renorm": self.softmax, "chain_reject": self.chain}

    def softmax(self, i):
        r = self.reps[i % self.R]
        self.sv.softmax_renorm(r["z"], r["T"], r["k"], r["p"], out=self.probs[i % self.R])

    def chain(self, i):
        r = self.reps[i % self.R]
        self.sv.chain_reject(r["q"], r["x"], self.probs[i % self.R], r["seed"], r["off"], out=(self.acc, self.alen))

    def step(self, i):
        self.softmax(i)
        self.chain(i)

    def algorithmic_bytes(self):
        # softmax_renorm: read bf16 logits, write float32 probabilities (every row)
        N = self.D + 1
        self.step(0)
        L = self.alen.cpu().numpy().astype(np.int64)
        self.bytes_by_call = {
            "softmax_renorm": float(self.B * N * self.V * (2 + 4)),
            "chain_reject": float((np.where(L < self.D, 8 * self.V, 4 * self.V)
                                   + 2 * PROBE_GRANULE * np.minimum(L + 1, self.D)).sum()),
        }
        return self.bytes_by_call["softmax_renorm"]

    def extra(self):
        return {}

    def config(self):
        return {"workload": self.name, "batch": self.B, "draft_tokens": self.D, "vocab": self.V,
                "temperature": 0.7, "top_k": 50, "top_p": 0.9, "input": "bf16 logits", "replicas": self.R}

    def cpu_baseline(self, seconds):
        import oracle
        h = self.host
        rows, t0, n = 0, time.perf_counter(), 0
        while True:
            b = n % self.B
            probs, _ = oracle.softmax_renorm(h["logits"], "bf16", h["temperature"], h["top_k"], h["top_p"],
                                             requests=[b])
            full = np.zeros((self.B,) + probs.shape[1:])
            full[b] = probs[0]
            oracle.chain_reject(h["draft_probs"], h["draft_ids"], full, h["seed"], np.zeros(self.B, np.uint64),
                                requests=[b])
            rows += self.D + 1
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
        return {"value": rows / el, "unit": "rows/s", "cores": 1, "kind": "oracle",
                "sample": f"{n} requests, {el:.1f}s single-threaded numpy"}


class TopkToppFusedWorkload(TopkToppWorkload):
    """The top-k/top-p batch (B=64 D=3 V=32000 bf16, T 0.7, k 50, top_p 0.9) through the fused call: target rows
    from logits and chain rejection in one call, no probabilities stored.  64 x 4 rows fit one per CU, so the
    call evaluates every row of a request at once; the request's last row to finish assembles its outputs."""
    name = "topk_topp_fused"
    kernel = "verify_fused_rows_kernel"
    dominant_call = "verify_fused"
    sources = ("fused_verify.hip", "sv_softmax.hpp", "sv_draw.hpp", "sv_argmax.hpp", "sv_rowpar.hpp", "sv_common.hpp")
    counters = "verify_fused_topk_topp_counters.txt"

    def __init__(self, dev, replicas):
        super().__init__(dev, replicas)
        self.calls = {"verify_fused": self.fused}

    def fused(self, i):
        r = self.reps[i % self.R]
        self.sv.verify_fused(r["z"], r["T"], r["q"], r["x"], r["seed"], r["off"], top_k=r["k"], top_p=r["p"],
                             out=(self.acc, self.alen))

    def step(self, i):
        self.fused(i)

    def algorithmic_bytes(self):
        """The method's bytes: logit rows 0..L, the draft row at the entries row L keeps (one 64-byte line
        each) on a rejection, q at the probed ids.  (The call reads every row of a request to evaluate them at
        once; the counters show that.)"""
        import torch
        N, D, V = self.D + 1, self.D, self.V
        self.step(0)
        L = self.alen.cpu().numpy().astype(np.int64)
        r = self.reps[0]
        probs = self.sv.softmax_renorm(r["z"], r["T"], r["k"], r["p"])
        kept = (probs > 0).sum(-1).cpu().numpy().astype(np.int64)[np.arange(self.B), np.minimum(L, D)]
        del probs
        torch.cuda.empty_cache()
        self.bytes_by_call = {"verify_fused": float(((L + 1) * V * 2 + np.where(L < D, np.minimum(
            4 * V, PROBE_GRANULE * kept), 0) + PROBE_GRANULE * np.minimum(L + 1, D)).sum())}
        self.L = L
        return self.bytes_by_call["verify_fused"]

    def extra(self):
        return {"mean_accept_length": round(float(self.L.mean()), 4)}


class MixedWorkload:
    """B=1024 D=7 V=129280 bf16 logits, 256 requests per mode, each mode through req_index.  R = 4
    replicas (logits, draft rows and probability buffers at distinct addresses, Philox offsets
    4096 r apart) rotate so that no call finds the previous call's rows in the Infinity Cache."""
    name = "mixed"
    kernel = "softmax_renorm_rr_kernel"
    dominant_call = "softmax_renorm"
    sources = ("softmax_renorm.hip", "sv_softmax.hpp", "sv_argmax.hpp", "sv_common.hpp")
    counters = "softmax_renorm_mixed_counters.txt"
    dtype = "bf16"
    needs_probs = True

    def __init__(self, dev, replicas):
        from workloads import MODE_GREEDY, MODE_TEMPERATURE, MODE_TOPK, MODE_TOPP, make_config
        import torch
        import token_sampling_temp_amd as sv
        self.sv = sv
        t0 = time.time()
        h = make_config(5)
        log(f"generated inputs in {time.time() - t0:.1f}s")
        self.host = h
        self.B, self.D, self.V = h["B"], h["D"], h["V"]
        N = self.D + 1
        self.R = replicas or 4
        self.x = _t(h["draft_ids"], dev)
        self.T = _t(h["temperature"], dev)
        self.k = _t(h["top_k"], dev)
        self.p = _t(h["top_p"], dev)
        self.seed = _t(h["seed"], dev)
        self.reps = []
        for r in range(self.R):
            off = (h["offset"] + np.uint64(4096 * r)).astype(np.uint64)
            rep = dict(z=_bf16(h["logits"], dev), q=_t(h["draft_probs"], dev), off=_t(off, dev), off_host=off)
            if self.needs_probs:
                rep["probs"] = torch.zeros((self.B, N, self.V), dtype=torch.float32, device=dev)
            self.reps.append(rep)
        modes = h["modes"]
        self.idx_host = {m: np.nonzero(modes == m)[0].astype(np.int32) for m in range(4)}
        self.greedy_idx = _t(self.idx_host[MODE_GREEDY], dev)
        self.temp_idx = _t(self.idx_host[MODE_TEMPERATURE], dev)
        filt = np.concatenate([self.idx_host[MODE_TOPK], self.idx_host[MODE_TOPP]]).astype(np.int32)
        self.filt_host = filt
        self.filt_idx = _t(filt, dev)
        self.acc = torch.empty((self.B, N), dtype=torch.int32, device=dev)
        self.alen = torch.empty((self.B,), dtype=torch.int32, device=dev)
        self.out = {"accepted_tokens": self.acc, "accept_length": self.alen}
        self.rows = self.B * N
        self.calls = {"greedy_verify": self.greedy, "gumbel_sample": self.gumbel,
                      "softmax_renorm": self.softmax, "chain_reject": self.chain}

    def greedy(self, i=0):
        r = self.reps[i % self.R]
        self.sv.greedy_verify(r["z"], self.x, req_index=self.greedy_idx, predict=False, accept_index=False,
                              out=self.out)

    def gumbel(self, i=0):
        r = self.reps[i % self.R]
        self.sv.gumbel_sample(r["z"], self.T, self.x, self.seed, r["off"], req_index=self.temp_idx, out=self.out)

    def softmax(self, i=0):
        r = self.reps[i % self.R]
        self.sv.softmax_renorm(r["z"], self.T, self.k, self.p, req_index=self.filt_idx, out=r["probs"])

    def chain(self, i=0):
        r = self.reps[i % self.R]
        self.sv.chain_reject(r["q"], self.x, r["probs"], self.seed, r["off"], req_index=self.filt_idx,
                             out=(self.acc, self.alen))

    def step(self, i):
        self.greedy(i)
        self.gumbel(i)
        self.softmax(i)
        self.chain(i)

    def _lengths(self):
        """Realised accept lengths of every replica (one step each)."""
        Ls = []
        for i in range(self.R):
            self.step(i)
            Ls.append(self.alen.cpu().numpy().astype(np.int64))
        self.L = np.concatenate(Ls)
        return Ls

    def algorithmic_bytes(self):
        from workloads import MODE_GREEDY, MODE_TEMPERATURE
        D, V, N = self.D, self.V, self.D + 1
        g = self.idx_host[MODE_GREEDY]
        t = self.idx_host[MODE_TEMPERATURE]
        f = self.filt_host
        by = {"greedy_verify": [], "gumbel_sample": [], "softmax_renorm": [], "chain_reject": []}
        for L in self._lengths():
            by["greedy_verify"].append(((L[g] + 1) * V * 2).sum())
            by["gumbel_sample"].append(((L[t] + 1) * V * 2).sum())
            by["softmax_renorm"].append(f.size * N * V * (2 + 4))
            by["chain_reject"].append((np.where(L[f] < D, 8 * V, 4 * V)
                                       + 2 * PROBE_GRANULE * np.minimum(L[f] + 1, D)).sum())
        self.bytes_by_call = {k: float(np.mean(v)) for k, v in by.items()}
        return self.bytes_by_call["softmax_renorm"]

    def extra(self):
        from workloads import MODE_GREEDY, MODE_TEMPERATURE, MODE_TOPK, MODE_TOPP
        L = self.L.reshape(-1, self.B)
        return {"mean_accept_length_by_mode": {
            name: round(float(L[:, self.idx_host[m]].mean()), 4)
            for m, name in ((MODE_GREEDY, "greedy"), (MODE_TEMPERATURE, "temperature"), (MODE_TOPK, "top_k"),
                            (MODE_TOPP, "top_p"))}}

    def config(self):
        return {"workload": self.name, "batch": self.B, "draft_tokens": self.D, "vocab": self.V,
                "input": "bf16 logits; float32 draft probabilities", "modes": "256 greedy / 256 temperature / "
                "256 top-k / 256 top-p", "replicas": self.R}

    def cpu_baseline(self, seconds):
        import oracle
        h = self.host
        rows, t0, n = 0, time.perf_counter(), 0
        order = np.random.default_rng(0).permutation(self.B)
        while True:
            b = int(order[n % self.B])
            if h["modes"][b] == 0:
                oracle.greedy_verify(h["logits"], "bf16", h["draft_ids"], requests=[b])
            elif h["modes"][b] == 1:
                oracle.gumbel_sample(h["logits"], "bf16", h["temperature"], h["draft_ids"], h["seed"], h["offset"],
                                     requests=[b])
            else:
                probs, _ = oracle.softmax_renorm(h["logits"], "bf16", h["temperature"], h["top_k"], h["top_p"],
                                                 requests=[b])
                one = slice(b, b + 1)
                oracle.chain_reject(h["draft_probs"][one], h["draft_ids"][one], probs, h["seed"][one],
                                    h["offset"][one])
            rows += self.D + 1
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
        return {"value": rows / el, "unit": "rows/s", "cores": 1, "kind": "oracle",
                "sample": f"{n} requests (random order over all modes), {el:.1f}s single-threaded numpy"}


class GumbelWorkload:
    """The mixed batch's 256 temperature-only requests (B=1024 D=7 V=129280 bf16) through
    gumbel_sample alone, R = 4 replicas.  Arithmetic-bound: each entry costs a quarter of a
    Philox4x32-10 block and two hardware logarithms, so its roofline is the vector ALU's."""
    name = "gumbel"
    kernel = "gumbel_staged_kernel"
    sources = ("gumbel_sample.hip", "sv_gumbel.hpp", "sv_rowpar.hpp", "sv_argmax.hpp", "sv_common.hpp")
    counters = "gumbel_sample_counters.txt"
    valu_counters = "gumbel_sample_valu_counters.txt"
    dtype = "bf16"
    bound = "alu"

    def __init__(self, dev, replicas):
        from workloads import MODE_TEMPERATURE, make_config
        import torch
        import token_sampling_temp_amd as sv
        self.sv = sv
        h = make_config(5)
        self.host = h
        self.B, self.D, self.V = h["B"], h["D"], h["V"]
        self.R = replicas or 4
        self.x = _t(h["draft_ids"], dev)
        self.T = _t(h["temperature"], dev)
        self.seed = _t(h["seed"], dev)
        self.idx_host = np.nonzero(h["modes"] == MODE_TEMPERATURE)[0].astype(np.int32)
        self.idx = _t(self.idx_host, dev)
        self.reps = []
        for r in range(self.R):
            off = (h["offset"] + np.uint64(4096 * r)).astype(np.uint64)
            self.reps.append(dict(z=_bf16(h["logits"], dev), off=_t(off, dev)))
        N = self.D + 1
        self.out = {"accepted_tokens": torch.empty((self.B, N), dtype=torch.int32, device=dev),
                    "accept_length": torch.empty((self.B,), dtype=torch.int32, device=dev)}
        self.rows = len(self.idx_host) * N

    def step(self, i):
        r = self.reps[i % self.R]
        self.sv.gumbel_sample(r["z"], self.T, self.x, self.seed, r["off"], req_index=self.idx, out=self.out)

    def _lengths(self):
        Ls = []
        for i in range(self.R):
            self.step(i)
            Ls.append(self.out["accept_length"].cpu().numpy().astype(np.int64)[self.idx_host])
        return Ls

    def algorithmic_bytes(self):
        """The rows strict acceptance needs (L + 1 per request), read once."""
        Ls = self._lengths()
        self.L = np.concatenate(Ls)
        self.entries = float(np.mean([((L + 1) * self.V).sum() for L in Ls]))
        return self.entries * 2

    def extra(self):
        return {"mean_accept_length": round(float(self.L.mean()), 4)}

    def config(self):
        return {"workload": self.name, "batch": self.B, "requests": len(self.idx_host), "draft_tokens": self.D,
                "vocab": self.V, "input": "bf16 logits, per-request temperature in [0.5, 1.2]",
                "replicas": self.R}

    def cpu_baseline(self, seconds):
        import oracle
        h = self.host
        rows, t0, n = 0, time.perf_counter(), 0
        while True:
            b = int(self.idx_host[n % len(self.idx_host)])
            r = oracle.gumbel_sample(h["logits"], "bf16", h["temperature"], h["draft_ids"], h["seed"], h["offset"],
                                     requests=[b])
            rows += int(r["accept_length"][b]) + 1
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
        return {"value": rows / el, "unit": "rows/s", "cores": 1, "kind": "oracle",
                "sample": f"{n} requests ({rows} sampled rows), {el:.1f}s single-threaded numpy float64"}


def gumbel_alu_ceiling(dev):
    """Entries/s the Gumbel-max arithmetic reaches with no memory traffic (the sampling kernel's
    per-group function on 1024-thread workgroups, logits made in registers), best of a few grids."""
    import ctypes
    import torch
    L = ctypes.CDLL(os.path.join(ROOT, "token_sampling_temp_amd", "libsvprobe.so"))
    L.svprobe_gumbel_alu.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    L.svprobe_gumbel_alu.restype = ctypes.c_int
    sink = torch.zeros(16 * 4096, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    best = (0.0, None)
    groups = 256
    for grid in (256, 512, 1024):
        def run():
            st = L.svprobe_gumbel_alu(groups, grid, 1 << 30, ctypes.c_void_p(sink.data_ptr()), sp)
            assert st == 0, st
        for _ in range(3):
            run()
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        n = 10
        for _ in range(n):
            run()
        s1.record(stream)
        torch.cuda.synchronize()
        ges = grid * 1024 * groups * 4 * n / (s0.elapsed_time(s1) * 1e-3) / 1e9
        if ges > best[0]:
            best = (ges, {"grid": grid, "groups_per_thread": groups})
    return best


def load_valu_cycles(summary, digest):
    """Weighted VALU cycles per launch from a committed counter summary taken on this kernel source."""
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_src = re.search(r"source_digest:\s*([0-9a-f]+)", txt)
    m_c = re.search(r"weighted_valu_cycles_per_launch:\s*([0-9.eE+]+)", txt)
    if not m_src or not m_c or m_src.group(1) != digest:
        return None
    return float(m_c.group(1))


class MixedFusedWorkload(MixedWorkload):
    """The mixed batch with its top-k and top-p requests through the fused call
    (target rows from logits and chain rejection in one launch, no probabilities
    stored): greedy_verify, gumbel_sample, verify_fused."""
    name = "mixed_fused"
    kernel = "verify_fused_rows_kernel"
    dominant_call = "verify_fused"
    sources = ("fused_verify.hip", "sv_softmax.hpp", "sv_draw.hpp", "sv_argmax.hpp", "sv_rowpar.hpp", "sv_common.hpp")
    counters = "verify_fused_mixed_counters.txt"
    needs_probs = False

    def __init__(self, dev, replicas):
        super().__init__(dev, replicas)
        self.calls = {"greedy_verify": self.greedy, "gumbel_sample": self.gumbel, "verify_fused": self.fused}

    def fused(self, i=0):
        r = self.reps[i % self.R]
        self.sv.verify_fused(r["z"], self.T, r["q"], self.x, self.seed, r["off"], top_k=self.k, top_p=self.p,
                             req_index=self.filt_idx, out=(self.acc, self.alen))

    def step(self, i):
        self.greedy(i)
        self.gumbel(i)
        self.fused(i)

    def algorithmic_bytes(self):
        from workloads import MODE_GREEDY, MODE_TEMPERATURE
        D, V = self.D, self.V
        g = self.idx_host[MODE_GREEDY]
        t = self.idx_host[MODE_TEMPERATURE]
        f = self.filt_host
        by = {"greedy_verify": [], "gumbel_sample": [], "verify_fused": []}
        # logit rows 0..L; on a rejection the draft row q_L at the entries row L keeps (the residual
        # max(0, p - q) is zero wherever p is), one 64-byte line per kept entry, at most the whole row;
        # q at the ids probed
        kept = self._kept_counts()
        for r, L in enumerate(self._lengths()):
            qbytes = np.minimum(4 * V, PROBE_GRANULE * kept[r][np.arange(self.B), np.minimum(L, D)][f])
            by["greedy_verify"].append(((L[g] + 1) * V * 2).sum())
            by["gumbel_sample"].append(((L[t] + 1) * V * 2).sum())
            by["verify_fused"].append(((L[f] + 1) * V * 2 + np.where(L[f] < D, qbytes, 0)
                                       + PROBE_GRANULE * np.minimum(L[f] + 1, D)).sum())
        self.bytes_by_call = {k: float(np.mean(v)) for k, v in by.items()}
        return self.bytes_by_call["verify_fused"]

    def _kept_counts(self):
        """Entries each target row keeps after top-k/top-p, per replica [B, N] (rows of other modes: 0),
        counted on the library's own renormalised rows (setup only, not timed)."""
        import torch
        out = []
        for r in self.reps:
            probs = torch.zeros((self.B, self.D + 1, self.V), dtype=torch.float32, device=r["z"].device)
            self.sv.softmax_renorm(r["z"], self.T, self.k, self.p, req_index=self.filt_idx, out=probs)
            out.append((probs > 0).sum(-1).cpu().numpy().astype(np.int64))
            del probs
        torch.cuda.empty_cache()
        return out


WORKLOADS = {c.name: c for c in (ChainWorkload, TargetOnlyWorkload, RaggedWorkload, RaggedD2tWorkload,
                                 DraftVocabWorkload,
                                 SampleWorkload, GreedyWorkload, TopkToppWorkload, TopkToppFusedWorkload,
                                 MixedWorkload, MixedFusedWorkload, GumbelWorkload)}


def _spread(us):
    us = np.asarray(us)
    return {"p10_us": round(float(np.percentile(us, 10)), 2), "median_us": round(float(np.median(us)), 2),
            "p90_us": round(float(np.percentile(us, 90)), 2)}


def timed_calls(fn, steps, stream, group=10):
    """Per-call times (us): one HIP event pair on `stream` around each group of `group` consecutive calls,
    the group's time divided by `group`.  (A pair around every single call adds about 2 us per call here,
    so single-call pairs would report the event overhead, not the kernel.)"""
    import torch
    n = max(1, steps // group)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    ev[0].record(stream)
    for g in range(n):
        for i in range(group):
            fn(g * group + i)
        ev[g + 1].record(stream)
    torch.cuda.synchronize()
    return [ev[g].elapsed_time(ev[g + 1]) * 1e3 / group for g in range(n)]


def per_call_times(wl, steps, stream):
    """Time of each call type of a multi-call step, each call type timed alone with replicas rotating."""
    out = {}
    for name, fn in getattr(wl, "calls", {}).items():
        for i in range(3):
            fn(i)
        us = timed_calls(fn, steps, stream)
        entry = {"us": round(float(np.mean(us)), 2), **_spread(us)}
        b = getattr(wl, "bytes_by_call", {}).get(name)
        if b is not None:
            entry["algorithmic_GBps"] = round(b / (entry["us"] * 1e-6) / 1e9, 1)
            entry["frac_of_peak"] = round(b / (entry["us"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
        out[name] = entry
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU: this build has no multi-GPU path "
              f"(--gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        copy_calibration()
        return
    import token_sampling_temp_amd as sv
    sv.lib()
    dev = torch.device("cuda:0")
    wl = WORKLOADS[args.workload](dev, args.replicas)
    log(f"workload {wl.name}: warmup {args.warmup}, steps {args.steps}")
    alg_bytes = wl.algorithmic_bytes()
    # the read-stream ceilings first: they also bring the GPU to its working clocks before the timed region
    log("measuring the read-stream ceilings")
    peak_read, peak_cfg = stream_peak(dev)
    same_read, same_cfg = stream_peak(dev, alg_bytes)
    log(f"read stream: {peak_read:.0f} GB/s at {peak_cfg} (1 GiB); {same_read:.0f} GB/s at {same_cfg} "
        f"({alg_bytes / 1e6:.0f} MB, the kernel's algorithmic bytes)")
    for i in range(args.warmup):
        wl.step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        wl.step(i)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    log(f"timed {args.steps} steps: {ms * 1e3:.2f} us/step")
    spread = _spread(timed_calls(wl.step, args.steps, stream))
    log(f"per-step spread: {spread}")
    rows_per_s = wl.rows / (ms * 1e-3)
    achieved = alg_bytes / (ms * 1e-3) / 1e9
    calls = per_call_times(wl, max(5, args.steps // 4), stream) if hasattr(wl, "calls") else None
    digest = _source_digest(*wl.sources)
    traffic = load_traffic(wl.counters, digest)
    cpu = None
    if args.cpu_seconds > 0:
        log("timing the CPU oracle baseline")
        cpu = wl.cpu_baseline(args.cpu_seconds)
        for k, v in cpu_info().items():
            cpu.setdefault(k, v)
    out = {
        "metric": METRIC,
        "value": rows_per_s,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": wl.config(),
        "roofline": {"bound": "hbm", "kernel": wl.kernel, "achieved": achieved, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": alg_bytes, "kernel_source_digest": digest},
        "per_step": spread,
        "cpu_baseline": cpu,
    }
    if calls:
        out["per_call"] = calls
        dom = calls.get(getattr(wl, "dominant_call", wl.kernel.replace("_kernel", "")))
        if dom:   # the dominant kernel timed on its own
            us = dom["us"]
            out["roofline"]["achieved"] = alg_bytes / (us * 1e-6) / 1e9
            out["roofline"]["frac"] = out["roofline"]["achieved"] / PEAK_HBM_GBS
    if getattr(wl, "bound", "hbm") == "alu":
        # arithmetic-bound: entries per second against the vector ALU's issue rate for the
        # kernel's instruction mix, and against the same arithmetic with no memory traffic
        ges = wl.entries / (ms * 1e-3) / 1e9
        log("measuring the Gumbel arithmetic ceiling")
        ceil, ceil_cfg = gumbel_alu_ceiling(dev)
        hbm = out["roofline"]
        out["roofline"] = {"bound": "alu", "kernel": wl.kernel, "achieved": ges, "peak": GUMBEL_ALU_PEAK_GES,
                           "unit": "G entries/s", "frac": ges / GUMBEL_ALU_PEAK_GES, "traffic": traffic,
                           "peak_derivation": f"{SIMD_CYCLES_PER_S / 1e9:.1f} G SIMD-cycles/s x 64 lanes x 4 "
                           f"entries per {GUMBEL_CYCLES_PER_GROUP:.0f} cycles (one wave64 group)",
                           "algorithmic_entries_per_launch": wl.entries, "kernel_source_digest": digest,
                           "measured_alu_ceiling_Gentries": round(ceil, 1), "alu_ceiling_config": ceil_cfg,
                           "frac_of_alu_ceiling": ges / ceil,
                           "hbm_GBps": hbm["achieved"], "hbm_frac": hbm["frac"]}
        cyc = load_valu_cycles(wl.valu_counters, digest)
        if cyc is not None:   # every VALU instruction the kernel issued, from the counter summary
            out["roofline"]["valu_busy_frac"] = cyc / SIMD_CYCLES_PER_S / (ms * 1e-3)
        if getattr(wl, "parity", None) is not None:
            out["parity"] = wl.parity
        out.update(wl.extra())
        print(json.dumps(out), flush=True)
        return
    out["roofline"]["measured_read_stream_GBps"] = round(peak_read, 1)
    out["roofline"]["read_stream_config"] = peak_cfg
    out["roofline"]["frac_of_stream_peak"] = out["roofline"]["achieved"] / peak_read
    out["roofline"]["read_stream_same_bytes_GBps"] = round(same_read, 1)
    out["roofline"]["frac_of_same_bytes_stream"] = out["roofline"]["achieved"] / same_read
    if getattr(wl, "parity", None) is not None:
        out["parity"] = wl.parity
    out.update(wl.extra())
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
