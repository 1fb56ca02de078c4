#!/usr/bin/env python3
"""Benchmark of the 4-bit dequantize-fused GEMV library on one MI355X.

Headline (the JSON line's `value`): effective HBM bandwidth of the Q4_K GEMV at
M = 1, N = K = 4096 (an o_proj-sized decode product), i.e.
    (weight bytes + x bytes + y bytes) / time per call.

Timing protocol (every workload): the weights are rotated over >= 1 GiB of
distinct device copies so that the 256 MB Infinity Cache cannot serve them.
One timed replay is a HIP graph of ceil(copies / K) passes of K calls (K =
--steps), call i reading copy i % copies, so every replay touches every copy
whatever K is; the time per call is the replay time (HIP events on the launch
stream) divided by the calls in it.  The first of five timed replays is the
figure reported, the median, p10 and p90 over the five give the spread, and
one cold call after a 512 MiB cache flush is reported beside it.

Beside each workload: the same protocol applied to a plain device copy
(torch.mul(src, 1.0, out=dst)) that moves the workload's byte count (half read,
half written) and to a plain streaming read of that byte count
(libqg_read.so), as measured ceilings for a memory-bound kernel of that size;
beside the matrix-core workloads, the vendor bf16 GEMM of the shape they issue;
and (unless --no-cpu) the f64 CPU oracle timed on the host at 1 thread and at
all cores.  The headline's `cpu_baseline` is the oracle on a bounded sample of
full headline calls.  `roofline.traffic` comes from the committed rocprofv3
counter summary when it was taken on the current kernel source.

Workloads: Q4_0 GEMV 1024^2, Q4_K GEMV 4096^2, dual Q4_0 at M = 1/4/8, affine
12288x4096 at M = 1/8, prefill affine GEMM 512x8192x2048 (also through the
allocation-free entry point) + qkv split, and the
follow-on paths: multi-part Q4_K, packed 4-bit affine, Q4_0 prefill on the
matrix cores, the fused projection + split.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME] [--no-cpu] [--no-ceiling]
                       [--profile]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published
ROTATE_BYTES = 1 << 30
REPS = 5  # timed replays of the K-call graph per workload
HEADLINE = "q4_k_gemv_4096"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "q4_k_gemv_4096_traffic.json")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in ("gemm_qgemv_q4_amd/csrc/kernels/gemv.hpp", "gemm_qgemv_q4_amd/csrc/kernels/common.hpp",
                "gemm_qgemv_q4_amd/csrc/api.hip"):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Case:
    """One workload: device inputs rotated over copies, a launch closure,
    byte/flop counts, and the oracle call on the same host inputs."""

    def __init__(self, name, desc, nbytes, flops, copies, launch, bound="hbm", oracle=None, context=None,
                 gemm_shape=None, bias_groups=0):
        self.name, self.desc, self.nbytes, self.flops = name, desc, nbytes, flops
        self.copies, self.launch, self.bound = copies, launch, bound
        self.oracle, self.context = oracle, context
        # (M, N, K') of the bf16 GEMM that the matrix-core path issues (x split
        # into hi + lo: K' = 2K), for the vendor-GEMM reference ceiling
        self.gemm_shape = gemm_shape
        self.bias_groups = bias_groups  # K / group size for formats with a bias product, else 0


def _orc():
    import oracle  # the cpu_baseline leg only
    return oracle


def n_copies(weight_bytes):
    return max(2, min(4096, -(-ROTATE_BYTES // weight_bytes)))


def build_cases(qg, torch, only=None):
    import synth
    cfg = synth.CONFIGS
    cases = []
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()

    # groups of workloads by the config they come from, and the workloads of each
    groups = {"q4_k_gemv_4096": ["q4_k_gemv_4096"], "q4_0_gemv_1024": ["q4_0_gemv_1024"],
              "dual_q4_0_4096": [f"dual_q4_0_4096_m{m}" for m in (1, 4, 8)],
              "affine_12288x4096_gs64": [f"affine_12288x4096_gs64_m{m}" for m in (1, 8)],
              "prefill_qkv_512x2048": ["prefill_gemm_512x8192x2048", "prefill_gemm_512x8192x2048_noalloc",
                                       "qkv_split_512x8192"],
              "q4_k_qkv_multi_4096": ["q4_k_qkv_multi_4096", "q4_k_qkv_separate_4096"],
              "affine_b4_12288x4096_gs64": [f"affine_b4_12288x4096_gs64_m{m}" for m in (1, 8)],
              "q4_0_prefill_512x4096": ["q4_0_prefill_512x4096"],
              "prefill_qkv_fused_512x2048": ["prefill_qkv_fused_512x2048"]}

    def want(n):
        return only is None or n.startswith(only) or any(c.startswith(only) for c in groups[n])

    def rot(t, r):
        # r distinct device copies of one tensor (HBM does not deduplicate)
        return [t] + [t.clone() for _ in range(r - 1)]

    # --- Q4_K GEMV 4096^2, M = 1 (headline)
    if want("q4_k_gemv_4096"):
        c = cfg["q4_k_gemv_4096"]
        w, x = synth.q4_k_case(c["seed"], c["m"], c["n"], c["k"])
        r = n_copies(w.nbytes)
        ws, dx = rot(dev(w), r), dev(x)
        y = torch.empty((c["m"], c["n"]), dtype=torch.float32, device="cuda")
        nb = w.nbytes + x.nbytes + y.numel() * 4
        cases.append(Case("q4_k_gemv_4096", "Q4_K GEMV M=1 N=4096 K=4096", nb, 2 * c["n"] * c["k"], r,
                          lambda i, ws=ws, dx=dx, y=y, r=r, n=c["n"], k=c["k"]:
                          qg.qgemv_q4_k(ws[i % r], dx, n, k, y=y),
                          oracle=lambda w=w, x=x, c=c: _orc().qgemv_q4_k(w, x, c["m"], c["n"], c["k"])))
    # --- Q4_0 GEMV 1024^2, M = 1
    if want("q4_0_gemv_1024"):
        c = cfg["q4_0_gemv_1024"]
        w, x = synth.q4_0_case(c["seed"], c["m"], c["n"], c["k"])
        r = n_copies(w.nbytes)
        ws, dx = rot(dev(w), r), dev(x)
        y = torch.empty((c["m"], c["n"]), dtype=torch.float32, device="cuda")
        nb = w.nbytes + x.nbytes + y.numel() * 4
        cases.append(Case("q4_0_gemv_1024", "Q4_0 GEMV M=1 N=1024 K=1024", nb, 2 * c["n"] * c["k"], r,
                          lambda i, ws=ws, dx=dx, y=y, r=r, n=c["n"], k=c["k"]:
                          qg.qgemv_q4_0(ws[i % r], dx, n, k, y=y),
                          oracle=lambda w=w, x=x, c=c: _orc().qgemv_q4_0(w, x, c["m"], c["n"], c["k"])))
    # --- dual Q4_0 4096 -> 2 x 4096, M = 1, 4, 8
    if want("dual_q4_0_4096"):
        c = cfg["dual_q4_0_4096"]
        wa, wb, x8 = synth.dual_q4_0_case(c["seed"], c["m"], c["n"], c["k"])
        r = n_copies(wa.nbytes + wb.nbytes)
        was, wbs = rot(dev(wa), r), rot(dev(wb), r)
        for m in (1, 4, 8):
            dx = dev(x8[:m])
            ya = torch.empty((m, c["n"]), dtype=torch.float32, device="cuda")
            yb = torch.empty_like(ya)
            nb = wa.nbytes + wb.nbytes + m * c["k"] * 4 + 2 * m * c["n"] * 4
            cases.append(Case(f"dual_q4_0_4096_m{m}", f"dual Q4_0 M={m} N=4096 K=4096", nb,
                              4 * m * c["n"] * c["k"], r,
                              lambda i, was=was, wbs=wbs, dx=dx, ya=ya, yb=yb, r=r, n=c["n"], k=c["k"]:
                              qg.qgemv_dual_q4_0(was[i % r], wbs[i % r], dx, n, k, y_a=ya, y_b=yb),
                              oracle=lambda wa=wa, wb=wb, x=x8[:m], m=m, c=c:
                              _orc().qgemv_dual_q4_0(wa, wb, x, m, c["n"], c["k"])))
    # --- affine 12288 x 4096 gs 64, M = 1, 8
    if want("affine_12288x4096_gs64"):
        c = cfg["affine_12288x4096_gs64"]
        x8, q, s, b = synth.affine_case(c["seed"], c["m"], c["n"], c["k"], c["gs"])
        wbytes = q.nbytes + s.nbytes + b.nbytes
        r = n_copies(wbytes)
        qs_, ss_, bs_ = rot(dev(q), r), rot(dev(s), r), rot(dev(b), r)
        for m in (1, 8):
            dx = dev(x8[:m])
            y = torch.empty((m, c["n"]), dtype=torch.float32, device="cuda")
            nb = wbytes + m * c["k"] * 4 + m * c["n"] * 4
            cases.append(Case(f"affine_12288x4096_gs64_m{m}", f"affine gs64 M={m} N=12288 K=4096", nb,
                              2 * m * c["n"] * c["k"], r,
                              lambda i, qs_=qs_, ss_=ss_, bs_=bs_, dx=dx, y=y, r=r, gs=c["gs"]:
                              qg.qmm_affine_t(dx, qs_[i % r], ss_[i % r], bs_[i % r], gs, y=y),
                              oracle=lambda x=x8[:m], q=q, s=s, b=b, m=m, c=c:
                              _orc().qmm_affine_t(x, q, s, b, m, c["n"], c["k"], c["gs"])))
    # --- prefill affine GEMM 512 x 8192 x 2048 (matrix cores) + qkv split
    if want("prefill_qkv_512x2048"):
        c = cfg["prefill_qkv_512x2048"]
        x, q, s, b = synth.affine_case(c["seed"], c["m"], c["n"], c["k"], c["gs"])
        wbytes = q.nbytes + s.nbytes + b.nbytes
        r = n_copies(wbytes)
        qs_, ss_, bs_ = rot(dev(q), r), rot(dev(s), r), rot(dev(b), r)
        dx = dev(x)
        qkv = torch.empty((c["m"], c["n"]), dtype=torch.float32, device="cuda")
        nb = wbytes + x.nbytes + qkv.numel() * 4
        cases.append(Case("prefill_gemm_512x8192x2048", "affine gs64 M=512 N=8192 K=2048 (MFMA)", nb,
                          2 * c["m"] * c["n"] * c["k"], r,
                          lambda i, qs_=qs_, ss_=ss_, bs_=bs_, dx=dx, qkv=qkv, r=r, gs=c["gs"]:
                          qg.qmm_affine_t(dx, qs_[i % r], ss_[i % r], bs_[i % r], gs, y=qkv),
                          bound="mfma", gemm_shape=(c["m"], c["n"], 2 * c["k"]), bias_groups=c["k"] // c["gs"],
                          oracle=lambda x=x, q=q, s=s, b=b, c=c:
                          _orc().qmm_affine_t(x, q, s, b, c["m"], c["n"], c["k"], c["gs"])))
        # the same product through the allocation-free entry point (static
        # scratch instead of a stream-ordered allocation per call)
        cases.append(Case("prefill_gemm_512x8192x2048_noalloc",
                          "affine gs64 M=512 N=8192 K=2048 (MFMA), allocation-free entry point", nb,
                          2 * c["m"] * c["n"] * c["k"], r,
                          lambda i, qs_=qs_, ss_=ss_, bs_=bs_, dx=dx, qkv=qkv, r=r, gs=c["gs"]:
                          qg.qmm_affine_t_noalloc(dx, qs_[i % r], ss_[i % r], bs_[i % r], gs, qkv),
                          bound="mfma"))
        qkv_r = rot(qkv, max(2, min(64, -(-ROTATE_BYTES // (qkv.numel() * 4)))))
        rr = len(qkv_r)
        qo = torch.empty((c["m"], c["q_sp"]), dtype=torch.float32, device="cuda")
        ko = torch.empty((c["m"], c["k_sp"]), dtype=torch.float32, device="cuda")
        vo = torch.empty((c["m"], c["v_sp"]), dtype=torch.float32, device="cuda")
        cases.append(Case("qkv_split_512x8192", "qkv_split seq=512 2048|2048|4096", 2 * qkv.numel() * 4, 0, rr,
                          lambda i, qkv_r=qkv_r, rr=rr, c=c, qo=qo, ko=ko, vo=vo:
                          qg.qkv_split_f32(qkv_r[i % rr], c["m"], c["q_sp"], c["k_sp"], c["v_sp"],
                                           q=qo, k=ko, v=vo),
                          oracle=lambda qk=synth.qkv_payload(c["m"], c["q_sp"], c["k_sp"], c["v_sp"]), c=c:
                          _orc().qkv_split_f32(qk, c["m"], c["q_sp"], c["k_sp"], c["v_sp"]),
                          context={"pages_figure": "838 ms in total, 17.5 ms per layer: the layer.qkv_deinterleave "
                                                   "bucket of the CPU download -> split -> 3x upload round trip "
                                                   "that the pages' GPU split kernel replaces (mlx-native "
                                                   "qkv_split.rs, module doc); hardware not stated (Metal host "
                                                   "code), sequence length not stated, no figure after the change",
                                   "vs_pages": None}))
    # ---- follow-on paths
    nxt = synth.NEXT_CONFIGS
    # multi-part Q4_K: a q|k|v decode projection (4096 + 1024 + 1024 rows) in one
    # launch, and the same three products as three separate calls
    if want("q4_k_qkv_multi_4096"):
        c = nxt["q4_k_qkv_multi_4096"]
        ws, x = synth.q4_k_multi_case(c["seed"], c["m"], c["ns"], c["k"])
        wbytes = sum(w.nbytes for w in ws)
        r = n_copies(wbytes)
        wss = [rot(dev(w), r) for w in ws]
        dx = dev(x)
        ntot = sum(c["ns"])
        y = torch.empty((c["m"], ntot), dtype=torch.float32, device="cuda")
        nb = wbytes + x.nbytes + y.numel() * 4
        ns, k = list(c["ns"]), c["k"]
        cases.append(Case("q4_k_qkv_multi_4096", "Q4_K multi-part 4096+1024+1024 x 4096, M=1, one launch", nb,
                          2 * ntot * k, r,
                          lambda i, wss=wss, dx=dx, y=y, r=r, ns=ns, k=k:
                          qg.qgemv_q4_k_multi([wl[i % r] for wl in wss], dx, ns, k, y=y),
                          oracle=lambda ws=ws, x=x, ns=ns, k=k, m=c["m"]:
                          _orc().qgemv_multi(_orc().decode_q4_k, list(zip(ws, ns)), x, m, k)))
        ys = [y[:, sum(ns[:j]):sum(ns[:j + 1])] for j in range(len(ns))]
        outs = [torch.empty((c["m"], n), dtype=torch.float32, device="cuda") for n in ns]
        cases.append(Case("q4_k_qkv_separate_4096", "the same three Q4_K products as three calls", nb,
                          2 * ntot * k, r,
                          lambda i, wss=wss, dx=dx, outs=outs, r=r, ns=ns, k=k:
                          [qg.qgemv_q4_k(wl[i % r], dx, n, k, y=o) for wl, n, o in zip(wss, ns, outs)],
                          oracle=lambda ws=ws, x=x, ns=ns, k=k, m=c["m"]:
                          [_orc().qgemv_q4_k(w, x, m, n, k) for w, n in zip(ws, ns)]))
    # packed 4-bit affine codes, 12288 x 4096 gs 64, M = 1 and 8
    if want("affine_b4_12288x4096_gs64"):
        c = nxt["affine_b4_12288x4096_gs64"]
        x8, q, s, b = synth.affine_case(c["seed"], c["m"], c["n"], c["k"], c["gs"])
        wp = synth.pack_b4_u32(q).view(np.int32)
        wbytes = wp.nbytes + s.nbytes + b.nbytes
        r = n_copies(wbytes)
        wps, ss_, bs_ = rot(dev(wp), r), rot(dev(s), r), rot(dev(b), r)
        for m in (1, 8):
            dx = dev(x8[:m])
            y = torch.empty((m, c["n"]), dtype=torch.float32, device="cuda")
            nb = wbytes + m * c["k"] * 4 + m * c["n"] * 4
            cases.append(Case(f"affine_b4_12288x4096_gs64_m{m}", f"packed affine gs64 M={m} N=12288 K=4096", nb,
                              2 * m * c["n"] * c["k"], r,
                              lambda i, wps=wps, ss_=ss_, bs_=bs_, dx=dx, y=y, r=r, gs=c["gs"]:
                              qg.qmm_affine_t_packed(dx, wps[i % r], ss_[i % r], bs_[i % r], gs, y=y),
                              oracle=lambda x=x8[:m], wp=wp, s=s, b=b, m=m, c=c:
                              _orc().qmm_affine_t_packed(x, wp, s, b, m, c["n"], c["k"], c["gs"])))
    # Q4_0 prefill on the matrix cores, 512 x 4096 x 4096
    if want("q4_0_prefill_512x4096"):
        c = nxt["q4_0_prefill_512x4096"]
        w, x = synth.q4_0_case(c["seed"], c["m"], c["n"], c["k"])
        r = n_copies(w.nbytes)
        ws, dx = rot(dev(w), r), dev(x)
        y = torch.empty((c["m"], c["n"]), dtype=torch.float32, device="cuda")
        nb = w.nbytes + x.nbytes + y.numel() * 4
        cases.append(Case("q4_0_prefill_512x4096", "Q4_0 M=512 N=4096 K=4096 (MFMA)", nb,
                          2 * c["m"] * c["n"] * c["k"], r,
                          lambda i, ws=ws, dx=dx, y=y, r=r, n=c["n"], k=c["k"]:
                          qg.qgemv_q4_0(ws[i % r], dx, n, k, y=y), bound="mfma",
                          gemm_shape=(c["m"], c["n"], 2 * c["k"]),
                          oracle=lambda w=w, x=x, c=c: _orc().qgemv_q4_0(w, x, c["m"], c["n"], c["k"])))
    # fused projection + q|k|v split on the prefill workload
    if want("prefill_qkv_fused_512x2048"):
        c = cfg["prefill_qkv_512x2048"]
        x, q, s, b = synth.affine_case(c["seed"], c["m"], c["n"], c["k"], c["gs"])
        wbytes = q.nbytes + s.nbytes + b.nbytes
        r = n_copies(wbytes)
        qs_, ss_, bs_ = rot(dev(q), r), rot(dev(s), r), rot(dev(b), r)
        dx = dev(x)
        qo = torch.empty((c["m"], c["q_sp"]), dtype=torch.float32, device="cuda")
        ko = torch.empty((c["m"], c["k_sp"]), dtype=torch.float32, device="cuda")
        vo = torch.empty((c["m"], c["v_sp"]), dtype=torch.float32, device="cuda")
        nb = wbytes + x.nbytes + c["m"] * c["n"] * 4
        cases.append(Case("prefill_qkv_fused_512x2048", "affine gs64 M=512 N=8192 K=2048 -> q|k|v (MFMA, split epilogue)",
                          nb, 2 * c["m"] * c["n"] * c["k"], r,
                          lambda i, qs_=qs_, ss_=ss_, bs_=bs_, dx=dx, qo=qo, ko=ko, vo=vo, r=r, c=c:
                          qg.qmm_affine_t_qkv(dx, qs_[i % r], ss_[i % r], bs_[i % r], c["gs"], c["q_sp"],
                                              c["k_sp"], c["v_sp"], q_out=qo, k_out=ko, v_out=vo),
                          bound="mfma",
                          oracle=lambda x=x, q=q, s=s, b=b, c=c:
                          _orc().qmm_affine_t_qkv(x, q, s, b, c["m"], c["k"], c["gs"], c["q_sp"], c["k_sp"],
                                                  c["v_sp"])))
    # a workload name selects that workload alone
    return [c for c in cases if only is None or c.name.startswith(only)] or cases


def _replay_timing(torch, launch, calls, warmup, reps_n=None):
    """Capture `calls` launches (launch(i), i = 0 .. calls-1) in one graph,
    replay it once untimed, then time REPS replays with events on the launch
    stream.  Returns the per-call times (us) of the replays and whether the
    graph could be captured."""
    s = torch.cuda.current_stream()
    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    graph = None
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(calls):
                launch(i)
        graph = g
    except Exception as e:  # capture not possible for this call: time eager launches
        log(f"[bench] graph capture failed ({e}); timing eager launches")
        torch.cuda.synchronize()
    run = (lambda: graph.replay()) if graph is not None else (lambda: [launch(i) for i in range(calls)])
    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = []
    for _ in range(reps_n or REPS):
        torch.cuda.synchronize()
        e0.record(s)
        run()
        e1.record(s)
        torch.cuda.synchronize()
        reps.append(e0.elapsed_time(e1) * 1e3 / calls)
    graphed = graph is not None
    del graph
    return reps, graphed


def copy_ceiling(torch, nbytes, calls, warmup):
    """The timing protocol applied to a plain device copy moving `nbytes`
    (nbytes/2 read, nbytes/2 written) over >= 1 GiB of rotating buffers:
    us per copy and GB/s of nbytes."""
    n = max(1, nbytes // 8)  # floats per half
    pairs = max(2, min(4096, -(-ROTATE_BYTES // (8 * n))))
    src = [torch.ones(n, dtype=torch.float32, device="cuda") for _ in range(pairs)]
    dst = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(pairs)]
    reps, _ = _replay_timing(torch, lambda i: torch.mul(src[i % pairs], 1.0, out=dst[i % pairs]), calls, warmup)
    del src, dst
    us = min(reps)  # a ceiling: the fastest replay (a slow first replay would inflate the fractions)
    return {"us": round(us, 3), "GBps": round(8 * n / (us * 1e-6) / 1e9, 1), "copies": pairs}


_READ_LIB = None


def read_ceiling(torch, nbytes, calls, warmup):
    """The plain streaming read of the workload's byte count (libqg_read.so,
    16-byte loads, nothing written), rotated over >= 1 GiB of buffers and
    timed with the same graph protocol: the read-only counterpart of the copy
    ceiling, for kernels that read far more than they write."""
    import ctypes
    global _READ_LIB
    if _READ_LIB is None:
        path = os.path.join(ROOT, "gemm_qgemv_q4_amd", "lib", "libqg_read.so")
        _READ_LIB = ctypes.CDLL(path)
        _READ_LIB.qg_stream_read.restype = ctypes.c_int
        _READ_LIB.qg_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p, ctypes.c_int,
                                             ctypes.c_void_p]
    n16 = max(16, nbytes // 16 * 16)
    copies = max(2, min(4096, -(-ROTATE_BYTES // n16)))
    bufs = [torch.empty(n16, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    # 4 blocks of 256 threads per CU (16 waves) walking the buffer: the best of
    # a sweep of 144 to 4096 blocks at 9.5 MB (3.48 us) and 57 MB (9.84 us)
    blocks = 4 * cus
    out = torch.zeros(blocks, dtype=torch.int32, device="cuda")

    def launch(i):
        rc = _READ_LIB.qg_stream_read(bufs[i % copies].data_ptr(), n16, out.data_ptr(), blocks,
                                      torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError(f"qg_stream_read failed ({rc})")

    reps, _ = _replay_timing(torch, launch, calls, warmup)
    del bufs, out
    us = min(reps)  # a ceiling: the fastest replay
    return {"us": round(us, 3), "GBps": round(n16 / (us * 1e-6) / 1e9, 1), "copies": copies}


def gemm_ceiling(torch, m, n, k, calls, warmup):
    """The vendor bf16 GEMM (torch.matmul, hipBLASLt) of the matrix-core
    path's issued shape: x [m, k] times a bf16 weight [n, k] transposed, f32
    accumulation, with the weight rotated over >= 1 GiB of copies like the
    quantized weights.  A reference ceiling for the matrix-core kernels: the
    same MFMA work on operands that need no decode."""
    a = torch.randn(m, k, device="cuda", dtype=torch.bfloat16)
    copies = max(2, min(64, -(-ROTATE_BYTES // (n * k * 2))))
    bs = [torch.randn(n, k, device="cuda", dtype=torch.bfloat16) for _ in range(copies)]
    reps, _ = _replay_timing(torch, lambda i: torch.matmul(a, bs[i % copies].t()), calls, warmup)
    del a, bs
    us = min(reps)  # a ceiling: the fastest replay
    return {"us": round(us, 3), "TFLOPs": round(2 * m * n * k / (us * 1e-6) / 1e12, 1), "copies": copies,
            "shape": f"bf16 [{m}, {k}] x [{n}, {k}]^T"}


def time_case(torch, case, steps, warmup, ceiling=True, profile=False):
    """Time ceil(copies / steps) passes of `steps` calls per replay (so that
    every replay reads every rotation copy), plus one cold call, and the copy
    ceiling at the same byte count.  profile: one timed replay, no cold calls,
    no ceiling (fewer dispatches under a profiler)."""
    passes = max(1, -(-case.copies // steps))
    calls = passes * steps
    reps, graphed = _replay_timing(torch, case.launch, calls, warmup, 1 if profile else None)
    us = reps[0]  # the first timed replay is the figure reported; the others give the spread
    per_call = sorted(reps)
    # single cold call: write a 512 MiB buffer to push the operands out of the
    # caches, then time one call.  The events and the call are queued while the
    # fill still runs, so the events bracket GPU time only (no host launch gap).
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    flush = torch.empty(128 << 20, dtype=torch.float32, device="cuda")
    cold = []
    for i in range(0 if profile else 3):
        torch.cuda.synchronize()
        flush.fill_(float(i))
        e0.record(s)
        case.launch(i)
        e1.record(s)
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1) * 1e3)
    del flush
    gbps = case.nbytes / (us * 1e-6) / 1e9
    out = {
        "desc": case.desc, "us_per_call": round(us, 3), "us_per_call_reps": [round(r, 3) for r in reps],
        "us_median": round(float(np.median(per_call)), 3),
        "us_p10": round(float(np.percentile(per_call, 10)), 3),
        "us_p90": round(float(np.percentile(per_call, 90)), 3),
        "us_cold_single_call": round(float(np.median(cold)), 3) if cold else None,
        "bytes": case.nbytes, "GBps": round(gbps, 1),
        "frac_hbm_peak": round(gbps / HBM_PEAK_GBS, 4),
        "graph": graphed, "rotation_copies": case.copies, "calls_per_replay": calls,
        "copies_touched": min(calls, case.copies),
        "bytes_touched_per_replay": min(calls, case.copies) * case.nbytes,
    }
    if ceiling and not profile and case.bound == "hbm":
        cc = copy_ceiling(torch, case.nbytes, calls, warmup)
        out["copy_ceiling"] = cc
        out["copy_ceiling_GBps"] = cc["GBps"]
        out["frac_of_copy_ceiling"] = round(gbps / cc["GBps"], 4)
        rc = read_ceiling(torch, case.nbytes, calls, warmup)
        out["read_ceiling"] = rc
        out["read_ceiling_GBps"] = rc["GBps"]
        out["frac_of_read_ceiling"] = round(gbps / rc["GBps"], 4)
    if ceiling and not profile and case.bound == "mfma" and case.gemm_shape:
        gc = gemm_ceiling(torch, *case.gemm_shape, min(calls, 200), warmup)
        out["vendor_bf16_gemm"] = gc
        out["frac_of_vendor_bf16_gemm_time"] = round(gc["us"] / us, 4)
    if case.flops:
        out["TFLOPs"] = round(case.flops / (us * 1e-6) / 1e12, 2)
    if case.bound == "mfma":
        out["frac_mfma_bf16_peak_useful"] = round(case.flops / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
        if case.gemm_shape:
            # issued by the matrix cores: the product with x split into hi + lo
            # (2x the useful flops) plus, for formats with a bias term, the bias
            # product over the group index (hi*hi, hi*lo, lo*hi, groups padded
            # to 32)
            m, n, k2 = case.gemm_shape
            issued = 2 * m * n * k2 + (3 * 2 * m * n * -(-case.bias_groups // 32) * 32 if case.bias_groups else 0)
            out["flops_issued"] = issued
            out["TFLOPs_issued"] = round(issued / (us * 1e-6) / 1e12, 2)
            out["frac_mfma_bf16_peak_issued"] = round(issued / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
    if case.context:
        out.update(case.context)
    return us, out


def _threads(n):
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=n)
    except Exception:  # pragma: no cover
        return None


def _time_calls(fn, budget_s, max_calls=200):
    """Call fn until about budget_s seconds have passed (at least once)."""
    calls, t0 = 0, time.perf_counter()
    while True:
        fn()
        calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s or calls >= max_calls:
            return calls, el


def oracle_timing(case, budget_s):
    """The oracle on the workload's own inputs: us per call at 1 BLAS thread
    and at all the host's cores."""
    host_cores = len(os.sched_getaffinity(0))
    out = {"kind": "oracle", "cores_all": host_cores}
    for key, n in (("1_thread", 1), ("all_cores", host_cores)):
        lim = _threads(n)
        calls, el = _time_calls(case.oracle, budget_s)
        if lim is not None:
            lim.unregister()
        per = el / calls
        out[key] = {"us_per_call": round(per * 1e6, 1), "GBps": round(case.nbytes / per / 1e9, 4),
                    "calls": calls, "threads": n}
    return out


def cpu_baseline(budget_s=10.0):
    """The oracle as it stands on the host, on full headline calls: one BLAS
    thread (the reported value) and all the host's cores (reported beside it)."""
    import synth
    oracle = _orc()
    host_cores = len(os.sched_getaffinity(0))
    c = synth.CONFIGS[HEADLINE]
    w, x = synth.q4_k_case(c["seed"], c["m"], c["n"], c["k"])
    nb = w.nbytes + x.nbytes + c["m"] * c["n"] * 4
    call = lambda: oracle.qgemv_q4_k(w, x, c["m"], c["n"], c["k"])
    lim = _threads(1)
    calls, el = _time_calls(call, budget_s)
    # one more call split into its two steps: f64 decode, then the f64 product
    t0 = time.perf_counter()
    w64 = oracle.decode_q4_k(w, c["n"], c["k"])
    t1 = time.perf_counter()
    oracle.gemv_f64(w64, x)
    t2 = time.perf_counter()
    if lim is not None:
        lim.unregister()
    per = el / calls
    out = {"value": round(nb / per / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": f"{calls} full Q4_K GEMV calls (M=1, N=K=4096) in {el:.1f}s, numpy f64 decode + matvec, "
                     f"1 BLAS thread; {per * 1e6:.0f} us/call (decode {(t1 - t0) * 1e6:.0f} us, "
                     f"product {(t2 - t1) * 1e6:.0f} us); host has {host_cores} cores"}
    lim = _threads(host_cores)
    calls, el = _time_calls(call, budget_s)
    if lim is not None:
        lim.unregister()
    per = el / calls
    out["all_cores"] = {"value": round(nb / per / 1e9, 4), "unit": "GB/s", "cores": host_cores,
                        "sample": f"{calls} calls in {el:.1f}s with {host_cores} BLAS threads; {per * 1e6:.0f} us/call"}
    return out


def read_traffic():
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--only", default=None, help="run only workloads whose name starts with this")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU timings")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the plain-copy, plain-read and vendor-GEMM ceilings")
    ap.add_argument("--profile", action="store_true",
                    help="for counter runs: one timed replay per workload, no cold calls, no ceilings, no oracle")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (x*1 -> y), the reference the HBM "
                         "byte counters of the profiles are scaled by")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (got --gpus {args.gpus}); "
              "the path shards by output rows: each GPU would hold N/G rows of the weights", file=sys.stderr)
        sys.exit(2)

    import torch
    import gemm_qgemv_q4_amd as qg
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)

    cases = build_cases(qg, torch, args.only)
    per = {}
    head_us = None
    for case in cases:
        log(f"[bench] {case.name}: {case.desc} ({case.copies} rotating copies)")
        us, res = time_case(torch, case, args.steps, args.warmup, ceiling=not args.no_ceiling, profile=args.profile)
        per[case.name] = res
        cc = (f", copy ceiling {res['copy_ceiling_GBps']} GB/s, read ceiling {res['read_ceiling_GBps']} GB/s"
              if "copy_ceiling_GBps" in res else "")
        log(f"[bench] {case.name}: {res['us_per_call']} us/call, {res['GBps']} GB/s{cc}")
        if case.name == HEADLINE:
            head_us = us
    torch.cuda.synchronize()
    if args.calibrate_copy:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")  # 256 MiB
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 3 x (read 268435456 B, write 268435456 B) in elementwise mul kernels")
        del src, dst
    if args.profile:
        args.no_cpu = True
    if not args.no_cpu:
        for case in cases:
            if case.oracle is not None:
                log(f"[bench] oracle on the host: {case.name}")
                per[case.name]["oracle"] = oracle_timing(case, 0.5)

    if HEADLINE not in per:
        print(json.dumps({"per_config": per}))
        return
    h = per[HEADLINE]
    ms_per_step = head_us * 1e-3
    value = h["bytes"] / (ms_per_step * 1e-3) / 1e9
    line = {
        "metric": "effective HBM GB/s (weights+acts) and % of peak; us per GEMV at M=1",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "us_per_gemv": round(ms_per_step * 1e3, 3),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "Q4_K GEMV M=1 N=4096 K=4096 (o_proj-sized decode)", "M": 1, "N": 4096,
                   "K": 4096, "weight_format": "Q4_K", "bytes_per_call": h["bytes"],
                   "rotation_copies": h["rotation_copies"], "copies_touched": h["copies_touched"],
                   "timing": f"hip graph of {h['calls_per_replay']} calls "
                             f"({h['calls_per_replay'] // args.steps} passes of {args.steps} steps, every "
                             f"rotation copy read), hip events on the launch stream; ms_per_step = replay "
                             f"time / calls"},
        "roofline": {"bound": "hbm", "kernel": "gemv_ks_kernel<Q4_K>", "achieved": round(value, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(value / HBM_PEAK_GBS, 4),
                     "traffic": read_traffic(),
                     "copy_ceiling_GBps": h.get("copy_ceiling_GBps"),
                     "frac_of_copy_ceiling": h.get("frac_of_copy_ceiling"),
                     "read_ceiling_GBps": h.get("read_ceiling_GBps"),
                     "frac_of_read_ceiling": h.get("frac_of_read_ceiling")},
        "per_config": per,
    }
    if not args.no_cpu:
        log("[bench] cpu baseline (oracle, headline)")
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
