#!/usr/bin/env python3
"""Benchmark: MoE token dispatch + combine on one MI355X (one EP rank's share).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dsv3_prefill]

A step is one pass of the hot path over one batch of synthetic input already
resident in HBM: the permute (routing layout -- counts, seg_indptr, src2dst,
reorder ids -- and the normal bf16 row scatter, one call of two kernels) ->
combine (top-k-weighted gather-sum) of the dispatched rows (identity
expert).  The same step through the separate layout / dispatch calls is
timed too, for comparison.  The default workload is the
DeepSeek-V3-shaped prefill share: T=4096 tokens, H=7168, 256 experts of
which 32 are local, top-8.

Reported (one JSON line on stdout):
  value        algorithmic GB/s of the whole step (bytes of the step's
               definition / measured step time), unit GB/s
  tokens_per_s T / step time
  roofline     the dominant kernel (combine): algorithmic bytes per launch /
               its average duration inside the timed step loop, from HIP
               events carried by the combine's own launch (cdl_combine_timed),
               against the 8 TB/s HBM3E peak; `traffic` = HBM bytes per launch
               from rocprofv3 FETCH_SIZE + WRITE_SIZE when a summary taken on
               the current kernel source is committed, else null
  cpu_baseline the CPU oracle (single-threaded C) on host copies of the same
               input, over a bounded number of full steps; all_cores: the
               oracle's loops on every host core this job may use (OpenMP
               timing build)
Input/output sets rotate between steps (default 6 sets, > 1 GB in total) so
that no step finds its input in the 256 MB Infinity Cache; the warm
(single-set) rate is reported beside it for context.

Only one GPU is supported: --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
METRIC = ("dispatch+combine HBM GB/s and tokens/sec at T=4096,H=7168,k=8 "
          "(fraction of peak)")
KERNEL_SOURCE = os.path.join(ROOT, "combine_dispatch_layout_amd", "csrc", "cdl.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "combine_dsv3_prefill_traffic.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="dsv3_prefill")
    p.add_argument("--sets", type=int, default=6,
                   help="rotating input/output sets (defeats the 256 MB Infinity Cache)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-modes", action="store_true",
                   help="skip the side measurements (fp8, low-latency, Zipf, next rows)")
    p.add_argument("--only", choices=["fp8_dispatch", "ll_decode", "zipf_prefill", "next_rows"],
                   help="run just this side measurement and print its JSON (for profiling)")
    p.add_argument("--calibration-copy", type=int, default=0, metavar="MB",
                   help="first run 5 plain device copies of MB MiB (torch copy_), the "
                        "known-size reference for scaling rocprofv3 byte counters")
    return p.parse_args()


def source_digest() -> str:
    """sha256 prefix of the kernel source with comments and whitespace
    removed: a comment edit does not change a kernel, so it keeps a counter
    summary valid; any change to the code does not."""
    import re
    with open(KERNEL_SOURCE) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    src = " ".join(src.split())
    return hashlib.sha256(src.encode()).hexdigest()[:16]


def committed_traffic():
    """HBM bytes per combine launch from a committed rocprofv3 summary, if it
    was taken on the current kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                kv[key.strip()] = val.strip()
    if kv.get("source_sha256") != source_digest():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------
# one input/output set with pre-bound C calls
# ---------------------------------------------------------------------------

class NormalSet:
    """Device buffers of one batch and the three C calls of a step, with
    every pointer argument bound up front (ctypes overhead only)."""

    def __init__(self, torch, cdl, W, w, dev):
        self.torch = torch
        lib = cdl.library()
        self.lib = lib
        x, ids, wts = W.make_inputs(w)
        T, k, L, H = w.T, w.k, w.L, w.H
        self.T, self.k, self.L, self.H = T, k, L, H
        self.x_host, self.ids_host, self.w_host = x, ids, wts
        self.x = x.to(dev)
        self.ids = ids.to(dev)
        self.wts = wts.to(dev)
        i32, i64 = torch.int32, torch.int64
        self.counts = torch.empty(L, dtype=i32, device=dev)
        self.seg = torch.empty(L + 1, dtype=i64, device=dev)
        self.src2dst = torch.empty(T * k, dtype=i32, device=dev)
        self.reorder = torch.empty(max(T * k, 1), dtype=i32, device=dev)
        wsb = cdl.layout_workspace_size(T, k, L)
        self.ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        self.status = torch.zeros(1, dtype=i32, device=dev)
        stream = torch.cuda.current_stream(dev).cuda_stream
        P = ctypes.c_void_p
        self.stream = P(stream)
        self.a_layout = (P(self.ids.data_ptr()), T, k, w.expert_begin, L,
                         P(self.counts.data_ptr()), P(self.seg.data_ptr()),
                         P(self.src2dst.data_ptr()), P(self.reorder.data_ptr()),
                         P(self.ws.data_ptr()), wsb, self.stream)
        self.layout()
        torch.cuda.synchronize()
        self.R = int(self.seg[L].item())
        valid = (self.src2dst.view(T, k) >= 0).any(dim=1)
        self.U = int(valid.sum().item())
        self.P = torch.empty(max(self.R, 1), H, dtype=torch.bfloat16, device=dev)
        self.out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
        self.a_dispatch = (P(self.x.data_ptr()), T, H, k, P(self.src2dst.data_ptr()),
                           P(self.P.data_ptr()), self.R, P(self.status.data_ptr()), self.stream)
        self.a_permute = (P(self.x.data_ptr()), T, H, k, P(self.ids.data_ptr()), w.expert_begin, L,
                          1, P(self.counts.data_ptr()), P(self.seg.data_ptr()),
                          P(self.src2dst.data_ptr()), P(self.reorder.data_ptr()), T * k,
                          P(self.P.data_ptr()), self.R, P(self.status.data_ptr()),
                          P(self.ws.data_ptr()), wsb, self.stream)
        self.a_combine = (P(self.P.data_ptr()), self.R, H, P(self.src2dst.data_ptr()),
                          P(self.wts.data_ptr()), T, k, P(self.out.data_ptr()),
                          P(self.status.data_ptr()), self.stream)

    def layout(self):
        rc = self.lib.cdl_dispatch_layout(*self.a_layout)
        if rc:
            raise RuntimeError("cdl_dispatch_layout failed: %d" % rc)

    def dispatch(self):
        rc = self.lib.cdl_dispatch(*self.a_dispatch)
        if rc:
            raise RuntimeError("cdl_dispatch failed: %d" % rc)

    def combine(self):
        rc = self.lib.cdl_combine(*self.a_combine)
        if rc:
            raise RuntimeError("cdl_combine failed: %d" % rc)

    def combine_timed(self, start, stop):
        """The combine with its kernel's own begin / end recorded into two
        torch.cuda.Event objects (created with enable_timing)."""
        P = ctypes.c_void_p
        a = self.a_combine
        rc = self.lib.cdl_combine_timed(*a[:-1], P(start.cuda_event), P(stop.cuda_event), a[-1])
        if rc:
            raise RuntimeError("cdl_combine_timed failed: %d" % rc)

    def permute(self):
        rc = self.lib.cdl_permute(*self.a_permute)
        if rc:
            raise RuntimeError("cdl_permute failed: %d" % rc)

    def step(self):
        self.permute()
        self.combine()

    def step_unfused(self):
        self.layout()
        self.dispatch()
        self.combine()

    # algorithmic bytes (definitions of the steps; per instance R, U)
    def bytes_layout(self):
        T, k, L = self.T, self.k, self.L
        return 4 * T * k + 4 * T * k + 4 * self.R + 4 * L + 8 * (L + 1)

    def bytes_scatter(self):
        return 4 * self.T * self.k + 2 * self.U * self.H + 2 * self.R * self.H

    def bytes_combine(self):
        T, k, H = self.T, self.k, self.H
        return 4 * T * k + 4 * T * k + 2 * self.R * H + 2 * T * H

    def bytes_step(self):
        # dispatch (layout + scatter, the ids read once) + combine
        return (self.bytes_layout() + 2 * self.U * self.H + 2 * self.R * self.H
                + self.bytes_combine())


def time_steps(torch, sets, fn, steps, warmup):
    """Average ms per call of fn(set) over `steps` calls rotating the sets,
    bracketed by synchronisations; events on the launch stream."""
    n = len(sets)
    for i in range(warmup):
        fn(sets[i % n])
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        fn(sets[i % n])
    end.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3
    return start.elapsed_time(end) / steps, wall / steps


def time_kernels(torch, sets, steps, warmup, lag=0):
    """The combine kernel's average duration inside a step loop: its launch
    carries two HIP events that receive the kernel's own begin and end
    (cdl_combine_timed), so nothing is added to the stream between the
    kernels.  Also returns the mean step time of that same loop, to show the
    events do not perturb it.

    lag = 0: each step combines the rows its own permute just wrote, as the
    timed step does; about 59 MB of the combine's reads then come from the
    256 MB Infinity Cache.  lag = len(sets) - 1 (cold source): step i
    permutes set i and combines the set permuted len(sets) - 1 steps earlier,
    whose rows the later permutes' (4 x 59 MB at 6 sets) and the other
    traffic have evicted, so the combine reads them from HBM (an explicit
    eviction write would leave dirty lines whose write-back competes with
    the combine)."""
    n = len(sets)
    assert 0 <= lag < n
    for i in range(warmup):
        sets[i % n].step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:             # torch creates the HIP event at its first record
        a.record()
        b.record()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        sets[i % n].permute()
        sets[(i - lag) % n].combine_timed(*ev[i])
    end.record()
    torch.cuda.synchronize()
    com = [a.elapsed_time(b) * 1e3 for a, b in ev]
    return {"combine_us": statistics.mean(com), "combine_us_median": statistics.median(com),
            "step_us_same_loop": start.elapsed_time(end) * 1e3 / steps}


# ---------------------------------------------------------------------------
# side measurements: fp8 dispatch, low latency, Zipf prefill
# ---------------------------------------------------------------------------

def measure_fp8(torch, cdl, sets, steps):
    """fp8 dispatch on the same-shaped sets: the fused permute (layout + fp8
    quantise-on-scatter) and the scatter kernel alone from a given layout."""
    lib = cdl.library()
    P = ctypes.c_void_p
    bufs = []
    for s in sets:
        q = torch.empty(max(s.R, 1), s.H, dtype=torch.uint8, device=s.x.device)
        sc = torch.empty(max(s.R, 1), s.H // 128, dtype=torch.float32, device=s.x.device)
        a_scatter = (P(s.x.data_ptr()), s.T, s.H, s.k, P(s.src2dst.data_ptr()), P(q.data_ptr()),
                     P(sc.data_ptr()), s.R, P(s.status.data_ptr()), s.stream)
        a_perm = (P(s.x.data_ptr()), s.T, s.H, s.k, P(s.ids.data_ptr()), 0, s.L, 1,
                  P(s.counts.data_ptr()), P(s.seg.data_ptr()), P(s.src2dst.data_ptr()),
                  P(s.reorder.data_ptr()), s.T * s.k, P(q.data_ptr()), P(sc.data_ptr()), 0, s.R,
                  P(s.status.data_ptr()), P(s.ws.data_ptr()), s.ws.numel(), s.stream)
        # per-tensor cast (the w8a8 buffer), no scale given
        a_tens = (P(s.x.data_ptr()), s.T, s.H, s.k, P(s.ids.data_ptr()), 0, s.L, 1,
                  P(s.counts.data_ptr()), P(s.seg.data_ptr()), P(s.src2dst.data_ptr()),
                  P(s.reorder.data_ptr()), s.T * s.k, P(q.data_ptr()), None, s.R,
                  P(s.status.data_ptr()), P(s.ws.data_ptr()), s.ws.numel(), s.stream)
        bufs.append((s, a_scatter, a_perm, q, sc, a_tens))

    def scatter(b):
        if lib.cdl_dispatch_fp8(*b[1]):
            raise RuntimeError("cdl_dispatch_fp8 failed")

    def perm(b):
        if lib.cdl_permute_fp8(*b[2]):
            raise RuntimeError("cdl_permute_fp8 failed")

    def perm_tensor(b):
        if lib.cdl_permute_fp8_tensor(*b[5]):
            raise RuntimeError("cdl_permute_fp8_tensor failed")

    ms_s, _ = time_steps(torch, bufs, scatter, steps, 5)
    ms_p, _ = time_steps(torch, bufs, perm, steps, 5)
    ms_t, _ = time_steps(torch, bufs, perm_tensor, steps, 5)
    tens_bytes = statistics.mean(x.bytes_layout() + 2 * x.U * x.H + x.R * x.H for x in sets)
    scat_bytes = statistics.mean(4 * x.T * x.k + 2 * x.U * x.H + x.R * (x.H + 4 * x.H // 128)
                                 for x in sets)
    perm_bytes = statistics.mean(x.bytes_layout() + 2 * x.U * x.H + x.R * (x.H + 4 * x.H // 128)
                                 for x in sets)
    # a device copy moving the permute's algorithmic bytes: the streaming
    # rate of a transfer of this size, launch and ramp included
    ceiling = copy_ceiling(torch, sets[0].x.device, perm_bytes)
    return {"workload": "fp8_dispatch (T=4096, H=7168, 32 of 256 experts, top-8, e4m3fn "
                        "groups of 128)",
            "permute_fp8_us": ms_p * 1e3, "permute_fp8_gbps": perm_bytes / (ms_p * 1e-3) / 1e9,
            "scatter_fp8_us": ms_s * 1e3, "scatter_fp8_gbps": scat_bytes / (ms_s * 1e-3) / 1e9,
            "permute_fp8_tensor_us": ms_t * 1e3,
            "permute_fp8_tensor_gbps": tens_bytes / (ms_t * 1e-3) / 1e9,
            "fp8_tensor_format": "per-tensor cast, no scale (w8a8 permuted buffer)",
            "copy_same_bytes": {**ceiling, "permute_fp8_frac_of_copy":
                                round(ceiling["us"] / (ms_p * 1e3), 4)}}


def measure_next_rows(torch, cdl, sets, E, steps):
    """The rows built beyond the hot path, at the same shape and on the same
    rotating sets: the rank layout that precedes an exchange (8 ranks on one
    node), the layout + bf16 scatter with expert segments padded to 128 rows,
    and the fused fp8 permute in the DeepGEMM format (segments padded to 128,
    UE8M0 exponents packed four to a word, column-major, TMA-aligned)."""
    lib = cdl.library()
    P = ctypes.c_void_p
    i32, u8 = torch.int32, torch.uint8
    A, R_RANKS, RPN = 128, 8, 8
    flags = cdl.FP8_SCALE_UE8M0 | cdl.FP8_SCALE_COLMAJOR | cdl.FP8_SCALE_PACKED
    bufs = []
    for s in sets:
        T, k, L, H, dev = s.T, s.k, s.L, s.H, s.x.device
        ntr = torch.empty(R_RANKS, dtype=i32, device=dev)
        ntn = torch.empty(R_RANKS // RPN, dtype=i32, device=dev)
        nte = torch.empty(E, dtype=i32, device=dev)
        itr = torch.empty(T, R_RANKS, dtype=u8, device=dev)
        rwsb = lib.cdl_rank_layout_workspace_size(T, k, E, R_RANKS, RPN)
        rws = torch.empty(max(rwsb, 1), dtype=u8, device=dev)
        a_rank = (P(s.ids.data_ptr()), T, k, E, R_RANKS, RPN, P(ntr.data_ptr()), P(ntn.data_ptr()),
                  P(nte.data_ptr()), P(itr.data_ptr()), P(rws.data_ptr()), rwsb, s.stream)
        reo_cap = T * k + L * (A - 1)
        cnt = torch.empty(L, dtype=i32, device=dev)
        seg = torch.empty(L + 1, dtype=torch.int64, device=dev)
        s2d = torch.empty(T * k, dtype=i32, device=dev)
        reo = torch.empty(reo_cap, dtype=i32, device=dev)
        lay = (P(s.ids.data_ptr()), T, k, 0, L, A, P(cnt.data_ptr()), P(seg.data_ptr()),
               P(s2d.data_ptr()), P(reo.data_ptr()), reo_cap, None, P(s.ws.data_ptr()),
               s.ws.numel(), s.stream)
        if lib.cdl_dispatch_layout_aligned(*lay):
            raise RuntimeError("cdl_dispatch_layout_aligned failed")
        torch.cuda.synchronize()
        Rp = int(seg[L].item())                       # padded rows, sized exactly
        out = torch.empty(max(Rp, 1), H, dtype=torch.bfloat16, device=dev)
        a_al = (P(s.x.data_ptr()), T, H, k, P(s.ids.data_ptr()), 0, L, A, P(cnt.data_ptr()),
                P(seg.data_ptr()), P(s2d.data_ptr()), P(reo.data_ptr()), reo_cap,
                P(out.data_ptr()), Rp, P(s.status.data_ptr()), P(s.ws.data_ptr()), s.ws.numel(),
                s.stream)
        q = torch.empty(max(Rp, 1), H, dtype=u8, device=dev)
        sb = torch.empty(max(cdl.fp8_scale_bytes(Rp, H, flags, Rp), 1), dtype=u8, device=dev)
        # workspace with room to stage the column-major scales
        fws = torch.empty(cdl.permute_fp8_workspace_size(T, k, L, H, flags, Rp), dtype=u8,
                          device=dev)
        a_f8 = (P(s.x.data_ptr()), T, H, k, P(s.ids.data_ptr()), 0, L, A, P(cnt.data_ptr()),
                P(seg.data_ptr()), P(s2d.data_ptr()), P(reo.data_ptr()), reo_cap, P(q.data_ptr()),
                P(sb.data_ptr()), flags, Rp, P(s.status.data_ptr()), P(fws.data_ptr()),
                fws.numel(), s.stream)
        bufs.append((s, a_rank, a_al, a_f8, Rp,
                     (ntr, ntn, nte, itr, rws, cnt, seg, s2d, reo, out, q, sb, fws)))

    def call(name, fn):
        def f(b):
            if fn(*b):
                raise RuntimeError(name + " failed")
        return f

    ms_rank, _ = time_steps(torch, bufs, lambda b: call("cdl_rank_layout", lib.cdl_rank_layout)(b[1]), steps, 5)
    ms_al, _ = time_steps(torch, bufs, lambda b: call("cdl_permute", lib.cdl_permute)(b[2]), steps, 5)
    ms_f8, _ = time_steps(torch, bufs, lambda b: call("cdl_permute_fp8", lib.cdl_permute_fp8)(b[3]), steps, 5)
    if sum(int(b[0].status.item()) for b in bufs):
        raise SystemExit("device status word set in the next-row measurements")
    G = sets[0].H // 128
    al_bytes = statistics.mean(b[0].bytes_layout() + 4 * (b[4] - b[0].R) + 2 * b[0].U * b[0].H
                               + 2 * b[0].R * b[0].H for b in bufs)
    f8_bytes = statistics.mean(b[0].bytes_layout() + 4 * (b[4] - b[0].R) + 2 * b[0].U * b[0].H
                               + b[0].R * (b[0].H + 4 * ((G + 3) // 4)) for b in bufs)
    s0 = sets[0]
    rank_bytes = 4 * s0.T * s0.k + s0.T * R_RANKS + 4 * (R_RANKS + R_RANKS // RPN + E)
    return {"workload": "dsv3_prefill shape (T=4096, H=7168, 32 of 256 experts, top-8)",
            "rank_layout_us": ms_rank * 1e3,
            "rank_layout_gbps": rank_bytes / (ms_rank * 1e-3) / 1e9,
            "rank_layout_config": "8 ranks, 1 node, 256 experts",
            "permute_aligned128_us": ms_al * 1e3,
            "permute_aligned128_gbps": al_bytes / (ms_al * 1e-3) / 1e9,
            "permute_fp8_deepgemm_us": ms_f8 * 1e3,
            "permute_fp8_deepgemm_gbps": f8_bytes / (ms_f8 * 1e-3) / 1e9,
            "fp8_deepgemm_format": "segments padded to 128, UE8M0 exponents packed 4 per int32, "
                                   "column-major, TMA-aligned"}


def measure_ll(torch, cdl, W, dev, steps):
    w = W.WORKLOADS["ll_decode"]
    lib = cdl.library()
    P = ctypes.c_void_p
    runs = []
    for s in range(2):
        base = NormalSet(torch, cdl, W, w.scaled(seed_base=w.seed_base + 7919 * s), dev)
        B = torch.empty(w.L, w.cap, w.H, dtype=torch.bfloat16, device=dev)
        mm = torch.empty(w.L, dtype=torch.int32, device=dev)
        llm = torch.empty(w.T * w.k, dtype=torch.int32, device=dev)
        a_ll = (P(base.x.data_ptr()), w.T, w.H, w.k, P(base.ids.data_ptr()), w.expert_begin,
                w.L, P(base.src2dst.data_ptr()), P(base.seg.data_ptr()),
                P(base.counts.data_ptr()), w.cap, P(B.data_ptr()), P(mm.data_ptr()),
                P(llm.data_ptr()), P(base.status.data_ptr()), base.stream)
        a_cb = (P(B.data_ptr()), w.L * w.cap, w.H, P(llm.data_ptr()), P(base.wts.data_ptr()),
                w.T, w.k, P(base.out.data_ptr()), P(base.status.data_ptr()), base.stream)
        a_pll = (P(base.x.data_ptr()), w.T, w.H, w.k, P(base.ids.data_ptr()), w.expert_begin, w.L,
                 P(base.counts.data_ptr()), P(base.seg.data_ptr()), P(base.src2dst.data_ptr()),
                 P(base.reorder.data_ptr()), base.reorder.numel(), w.cap, P(B.data_ptr()),
                 P(mm.data_ptr()), P(llm.data_ptr()), P(base.status.data_ptr()),
                 P(base.ws.data_ptr()), base.ws.numel(), base.stream)
        # the same dispatch with fp8 rows, UE8M0 exponents packed four to a
        # word, column-major per expert (the DeepGEMM masked-GEMM format)
        f8 = cdl.FP8_SCALE_UE8M0 | cdl.FP8_SCALE_COLMAJOR | cdl.FP8_SCALE_PACKED
        Bq = torch.empty(w.L, w.cap, w.H, dtype=torch.uint8, device=dev)
        Bs = torch.empty(cdl.fp8_scale_bytes(w.L * w.cap, w.H, f8, w.cap), dtype=torch.uint8,
                         device=dev)
        fws = torch.empty(cdl.permute_fp8_workspace_size(w.T, w.k, w.L, w.H, f8, w.L * w.cap),
                          dtype=torch.uint8, device=dev)
        a_pll8 = (P(base.x.data_ptr()), w.T, w.H, w.k, P(base.ids.data_ptr()), w.expert_begin,
                  w.L, P(base.counts.data_ptr()), P(base.seg.data_ptr()),
                  P(base.src2dst.data_ptr()), P(base.reorder.data_ptr()), base.reorder.numel(),
                  w.cap, P(Bq.data_ptr()), P(Bs.data_ptr()), f8, P(mm.data_ptr()),
                  P(llm.data_ptr()), P(base.status.data_ptr()), P(fws.data_ptr()), fws.numel(),
                  base.stream)
        runs.append((base, a_ll, a_cb, B, mm, llm, a_pll, a_pll8, Bq, Bs, fws))

    def fn(r):
        if lib.cdl_permute_ll(*r[6]) or lib.cdl_combine(*r[2]):
            raise RuntimeError("low-latency step failed")

    def fn_separate(r):
        r[0].layout()
        if lib.cdl_dispatch_ll(*r[1]) or lib.cdl_combine(*r[2]):
            raise RuntimeError("low-latency step failed")

    def dispatch_bf16(r):
        if lib.cdl_permute_ll(*r[6]):
            raise RuntimeError("cdl_permute_ll failed")

    def dispatch_fp8(r):
        if lib.cdl_permute_ll_fp8(*r[7]):
            raise RuntimeError("cdl_permute_ll_fp8 failed")

    ms_d16, _ = time_steps(torch, runs, dispatch_bf16, steps, 5)
    ms_d8, _ = time_steps(torch, runs, dispatch_fp8, steps, 5)
    ms, _ = time_steps(torch, runs, fn, steps, 5)
    ms_sep, _ = time_steps(torch, runs, fn_separate, steps, 5)
    b = runs[0][0]
    byts = (b.bytes_layout() + 4 * w.L + 4 * w.T * w.k + 2 * b.U * w.H + 2 * b.R * w.H
            + b.bytes_combine())
    return {"workload": "ll_decode (T=128, H=7168, 32 of 256 experts, top-8, cap 1024; "
                        "layout + padded dispatch (one call) + combine)",
            "us_per_step": ms * 1e3, "gbps": byts / (ms * 1e-3) / 1e9,
            "us_per_step_separate_calls": ms_sep * 1e3,
            "us_dispatch_one_call": ms_d16 * 1e3,
            "us_dispatch_fp8_one_call": ms_d8 * 1e3,
            "fp8_format": "UE8M0 exponents packed 4 per int32, column-major per expert",
            "expected_m": cdl.ll_expected_m(w.T, w.num_ranks, w.k, w.E)}


def measure_zipf(torch, cdl, W, dev, steps):
    w = W.WORKLOADS["zipf_prefill"]
    sets = [NormalSet(torch, cdl, W, w.scaled(seed_base=w.seed_base + 7919 * s), dev)
            for s in range(2)]
    ms, _ = time_steps(torch, sets, NormalSet.step, steps, 3)
    byts = statistics.mean(s.bytes_step() for s in sets)
    counts = sets[0].counts.cpu()
    return {"workload": "zipf_prefill (T=16384, H=4096, 128 local experts, top-8 Zipf 1.2; "
                        "layout + dispatch + combine)",
            "us_per_step": ms * 1e3, "gbps": byts / (ms * 1e-3) / 1e9,
            "tokens_per_s": w.T / (ms * 1e-3),
            "expert_rows_max": int(counts.max()), "expert_rows_min": int(counts.min())}


# ---------------------------------------------------------------------------
# CPU baseline (the oracle as it stands)
# ---------------------------------------------------------------------------

def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads() -> int:
    """Host cores this process may use: its CPU affinity, capped by
    OMP_NUM_THREADS when that is set (the GPU machines give one GPU's job a
    share of the host's cores)."""
    n = len(os.sched_getaffinity(0))
    try:
        cap = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        cap = 0
    return min(n, cap) if cap > 0 else n


def cpu_baseline_all_cores(W, s, threads, budget_s=6.0, max_reps=64):
    """The oracle's dispatch and combine loops on `threads` host threads
    (the OpenMP timing build, bit-identical to the oracle; the layout, under
    0.1% of a step, stays the single-threaded oracle's) on full steps of the
    timed workload until about budget_s seconds have passed."""
    import oracle

    xb = W.bf16_bits(s.x_host)
    ids = s.ids_host.numpy()
    wts = s.w_host.numpy()
    times, parts = [], []
    t_start = time.perf_counter()
    while len(times) < max_reps and (not times or time.perf_counter() - t_start < budget_s):
        t0 = time.perf_counter()
        c, seg, d, r = oracle.layout(ids, 0, s.L)
        t1 = time.perf_counter()
        P = oracle.omp_dispatch(xb, d, s.k, int(seg[-1]), threads)
        t2 = time.perf_counter()
        oracle.omp_combine(P, d, wts, s.T, s.k, threads)
        t3 = time.perf_counter()
        times.append(t3 - t0)
        parts.append((t1 - t0, t2 - t1, t3 - t2))
    t = statistics.median(times)
    return {"value": s.bytes_step() / t / 1e9, "unit": "GB/s", "cores": threads,
            "kind": "oracle loops, OpenMP timing build",
            "tokens_per_s": s.T / t, "ms_per_step": t * 1e3,
            "ms_layout_dispatch_combine": [round(statistics.median(p[i] for p in parts) * 1e3, 3)
                                           for i in range(3)],
            "sample": "%d full steps of the same T=%d workload on %d threads, %.1f s, median "
                      "step" % (len(times), s.T, threads, sum(times))}


def cpu_baseline(W, s, budget_s=12.0, max_reps=64):
    """The oracle as it stands, single-threaded, on full steps of the timed
    workload until about budget_s seconds of CPU work are done (a bounded
    sample: at least one step, at most max_reps)."""
    import numpy as np  # noqa: F401
    import oracle

    xb = W.bf16_bits(s.x_host)
    ids = s.ids_host.numpy()
    wts = s.w_host.numpy()
    times, parts = [], []
    t_start = time.perf_counter()
    while len(times) < max_reps and (not times or time.perf_counter() - t_start < budget_s):
        t0 = time.perf_counter()
        c, seg, d, r = oracle.layout(ids, 0, s.L)
        t1 = time.perf_counter()
        P = oracle.dispatch(xb, d, s.k, int(seg[-1]))
        t2 = time.perf_counter()
        oracle.combine(P, d, wts, s.T, s.k)
        t3 = time.perf_counter()
        times.append(t3 - t0)
        parts.append((t1 - t0, t2 - t1, t3 - t2))
    t = statistics.median(times)
    return {"value": s.bytes_step() / t / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "tokens_per_s": s.T / t, "ms_per_step": t * 1e3,
            "ms_layout_dispatch_combine": [round(statistics.median(p[i] for p in parts) * 1e3, 3)
                                           for i in range(3)],
            "cpu_model": cpu_model(),
            "sample": "%d full steps (layout+dispatch+combine) of the same T=%d workload, "
                      "%.1f s of single-threaded C oracle work, median step" % (
                          len(times), s.T, sum(times))}


def step_spread(torch, sets, fn, steps, warmup, loops=10, min_per_loop=20):
    """Median, p10 and p90 (us) of the mean step time of `loops` separate
    loops of max(steps // loops, min_per_loop) steps each (no event inside a
    loop).  Every loop pays one launch gap at its start, so loops of a few
    steps would read slower than the steady state; a fixed minimum keeps the
    spread comparable whatever --steps is."""
    per = max(steps // loops, min_per_loop)
    vals = sorted(time_steps(torch, sets, fn, per, warmup if i == 0 else 2)[0] * 1e3
                  for i in range(loops))
    q = lambda f: vals[min(int(f * (len(vals) - 1) + 0.5), len(vals) - 1)]
    return {"loops": loops, "steps_per_loop": per, "p10_us": round(q(0.1), 3),
            "median_us": round(q(0.5), 3), "p90_us": round(q(0.9), 3)}


def copy_ceiling(torch, dev, step_bytes, sets=6, reps=50):
    """A device-to-device copy moving the step's algorithmic bytes (half read,
    half written), rotating `sets` buffer pairs so no copy finds its source in
    the Infinity Cache: its GB/s is the achievable ceiling of this part."""
    n = int(step_bytes // 2) // 16 * 16
    pairs = [(torch.empty(n, dtype=torch.uint8, device=dev).fill_(i + 1),
              torch.empty(n, dtype=torch.uint8, device=dev)) for i in range(sets)]
    ms, _ = time_steps(torch, pairs, lambda p: p[1].copy_(p[0]), reps, 5)
    del pairs
    torch.cuda.empty_cache()
    return {"bytes_moved": 2 * n, "us": round(ms * 1e3, 3), "gbps": round(2 * n / (ms * 1e-3) / 1e9, 2)}


def inputs_digest(torch, s):
    import hashlib as hl
    h = {}
    for name, t in (("hidden_bf16", s.x_host), ("topk_ids", s.ids_host), ("topk_weights", s.w_host)):
        h[name] = hl.sha256(t.contiguous().view(torch.uint8).numpy().tobytes()).hexdigest()[:16]
    h["torch"] = torch.__version__
    return h


# ---------------------------------------------------------------------------

def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only (one expert-parallel rank's share); "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch

    import combine_dispatch_layout_amd as cdl
    from combine_dispatch_layout_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibration_copy:
        nbytes = args.calibration_copy << 20
        a = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        log("calibration copies: 5 x %d bytes read + %d bytes written" % (nbytes, nbytes))
        del a, b
    if args.only:
        if args.only == "fp8_dispatch":
            wf = W.WORKLOADS["fp8_dispatch"].scaled(mode="normal")
            fsets = [NormalSet(torch, cdl, W, wf.scaled(seed_base=wf.seed_base + 7919 * i), dev)
                     for i in range(args.sets)]
            r = measure_fp8(torch, cdl, fsets, args.steps)
        elif args.only == "ll_decode":
            r = measure_ll(torch, cdl, W, dev, args.steps)
        elif args.only == "next_rows":
            wn = W.WORKLOADS["dsv3_prefill"]
            nsets = [NormalSet(torch, cdl, W, wn.scaled(seed_base=wn.seed_base + 7919 * i), dev)
                     for i in range(args.sets)]
            r = measure_next_rows(torch, cdl, nsets, wn.E, args.steps)
        else:
            r = measure_zipf(torch, cdl, W, dev, args.steps)
        print(json.dumps({"only": args.only, **r}), flush=True)
        return
    w = W.WORKLOADS[args.workload]
    if w.mode != "normal":
        raise SystemExit("the timed step is the normal-mode path; pick a normal workload")
    log("building %d input sets of %s ..." % (args.sets, w.name))
    sets = [NormalSet(torch, cdl, W, w.scaled(seed_base=w.seed_base + 7919 * i), dev)
            for i in range(args.sets)]
    log("sets ready: R=%s U=%s" % ([s.R for s in sets], [s.U for s in sets]))

    # the spread over separate loops (at least 200 steps of this workload)
    # runs first: it brings the GPU to its working clocks before the timed
    # loop, with the timed step's own work
    spread = step_spread(torch, sets, NormalSet.step, args.steps, args.warmup)
    ms, wall_ms = time_steps(torch, sets, NormalSet.step, args.steps, args.warmup)
    log("cold step: %.2f us (wall %.2f us)" % (ms * 1e3, wall_ms * 1e3))
    warm_ms, _ = time_steps(torch, sets[:1], NormalSet.step, args.steps, args.warmup)
    unfused_ms, _ = time_steps(torch, sets, NormalSet.step_unfused, args.steps, args.warmup)
    kern = time_kernels(torch, sets, args.steps, args.warmup)
    cold = time_kernels(torch, sets, args.steps, args.warmup, lag=len(sets) - 1)
    log("kernels: %s; cold source: %s" % (kern, cold))
    st = int(sum(int(s.status.item()) for s in sets))
    if st:
        raise SystemExit("device status word set: %d" % st)

    step_bytes = statistics.mean(s.bytes_step() for s in sets)
    gbps = step_bytes / (ms * 1e-3) / 1e9
    comb_bytes = statistics.mean(s.bytes_combine() for s in sets)
    comb_gbps = comb_bytes / (kern["combine_us"] * 1e-6) / 1e9
    cold_gbps = comb_bytes / (cold["combine_us"] * 1e-6) / 1e9
    traffic = committed_traffic()
    ceiling = copy_ceiling(torch, dev, step_bytes)

    result = {
        "metric": METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "H": w.H, "E": w.E, "L": w.L, "k": w.k,
                   "expert_begin": w.expert_begin, "rotating_sets": args.sets,
                   "step": "permute (layout + bf16 scatter) + weighted combine (identity expert)"},
        "tokens_per_s": round(w.T / (ms * 1e-3), 1),
        "frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4),
        "algorithmic_bytes_per_step": int(step_bytes),
        "step_spread": spread,
        "copy_ceiling": {**ceiling, "frac_of_copy": round(gbps / ceiling["gbps"], 4)},
        "inputs_sha256": inputs_digest(torch, sets[0]),
        "warm_single_set": {"ms_per_step": round(warm_ms, 6),
                            "gbps": round(step_bytes / (warm_ms * 1e-3) / 1e9, 2)},
        "unfused_step": {"ms_per_step": round(unfused_ms, 6),
                         "gbps": round(step_bytes / (unfused_ms * 1e-3) / 1e9, 2),
                         "calls": "dispatch_layout + dispatch + combine"},
        "kernels_us": {k_: round(v, 3) for k_, v in kern.items()},
        "kernels_us_cold_source": {k_: round(v, 3) for k_, v in cold.items()},
        # frac: inside the timed step, where about 59 MB of the combine's reads
        # (the rows the permute just wrote) come from the Infinity Cache;
        # frac_cold_source: the same launch over the rows of the set permuted
        # five steps earlier, evicted by then, so read from HBM
        "roofline": {"kernel": "combine_rows_pipe", "bound": "hbm",
                     "achieved": round(comb_gbps, 2), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(comb_gbps / PEAK_HBM_GBPS, 4),
                     "traffic": traffic, "algorithmic_bytes_per_launch": int(comb_bytes),
                     "source_rows": "in step (Infinity Cache hits)",
                     "cold_source": "rows permuted %d steps earlier (evicted)" % (len(sets) - 1),
                     "achieved_cold_source": round(cold_gbps, 2),
                     "frac_cold_source": round(cold_gbps / PEAK_HBM_GBPS, 4)},
    }
    if not args.no_modes:
        result["modes"] = {
            "fp8_dispatch": measure_fp8(torch, cdl, sets, args.steps),
            "ll_decode": measure_ll(torch, cdl, W, dev, args.steps),
            "zipf_prefill": measure_zipf(torch, cdl, W, dev, max(args.steps // 4, 10)),
            "next_rows": measure_next_rows(torch, cdl, sets, w.E, args.steps),
        }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        base = cpu_baseline(W, sets[0])
        threads = host_threads()
        log("timing the oracle's loops on %d host threads ..." % threads)
        base["all_cores"] = cpu_baseline_all_cores(W, sets[0], threads)
        result["cpu_baseline"] = base
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
