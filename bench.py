#!/usr/bin/env python3
"""Benchmark of the compressed-key scoring hot path on one MI355X.

One step = the whole path over one batch: tq_query_transform (A = Pi q,
T = S_mat q) then tq_score (raw scores of every query against every compressed
key). The default workload is the decode shape: B=32 queries, S=32768 keys,
D=128, 2-bit indices + 1-bit QJL signs (3 bits per coordinate), unpacked bytes.

Inputs are synthetic and already resident in HBM when timing starts. A ring of
distinct buffer sets totalling at least 512 MB is cycled so that no step finds
its keys in the 256 MiB Infinity Cache. The K timed steps are replayed from
captured HIP graphs (host launch overhead would otherwise dominate microsecond
kernels): per chunk of the ring, one graph holding each set's transform and
then its score. A second pass of K steps in phased graphs (per chunk, one graph
of its query transforms and one of its scores, HIP events between the graph
launches) gives each kernel's average duration. The CPU oracle is timed on a bounded sample
as a reported baseline.

Prints ONE JSON line. ``--gpus N`` with N > 1 exits: the benchmark runs on one GPU.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "query-key scores/sec + achieved HBM GB/s, B=32 S=32768 D=128 3-bit keys"
HBM_PEAK_GBS = 8000.0
FP64_MATRIX_PEAK_TFLOPS = 78.6
RING_BYTES = 512 * 1024 * 1024


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="decode",
                    help="decode (default, the quoted configuration); others for profiling")
    ap.add_argument("--kernel", default="auto",
                    choices=["auto", "valu", "mfma", "mfma_lds", "mfma_reg", "mfma16", "mfma_shared", "mfma_f16"],
                    help="kernel family of tq_score; mfma_f16 is the single-pass f16 form (2e-2 accuracy)")
    ap.add_argument("--path", default="score", choices=["score", "compress", "attend", "mse", "split", "fused"],
                    help="score (default): the scoring hot path; compress: the key compressor "
                         "(tq_compress_keys) on the workload's key set; attend: softmax and value "
                         "aggregation (tq_attend) over the workload's scores and values; mse: the "
                         "MSE-only variant (tq_query_transform_hadamard + tq_score_mse); split: the "
                         "outlier split, 32 hot channels at 3 bits + the rest at 2 (tq_query_transform_split "
                         "+ tq_score_split); fused: the whole decode step, tq_query_transform + "
                         "tq_score_attend (scores never written), against the two-call form")
    ap.add_argument("--no-stream-probe", action="store_true",
                    help="skip the streaming probes and the same-size device copy (for profiler runs of the kernels)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU oracle timing (profiling runs)")
    ap.add_argument("--eager", action="store_true", help="launch every step eagerly (no HIP graphs)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time for the oracle baseline sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy a 256 MiB device buffer 20 times (known bytes, to scale "
                         "memory counters read under a profiler), then exit")
    return ap.parse_args()


def source_digest(files) -> str:
    """sha256 over the code of the listed sources with comments and blank lines
    taken out, so that a record taken on a kernel stays valid through edits
    of its comments but not of its code. String and character literals are
    kept whole (a "//" inside one is not a comment)."""
    import hashlib

    h = hashlib.sha256()
    for p in files:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            text = f.read()
        out, i, n = [], 0, len(text)
        while i < n:
            c = text[i]
            if c in "\"'":
                j = i + 1
                while j < n and text[j] != c:
                    j += 2 if text[j] == "\\" else 1
                out.append(text[i:j + 1])
                i = j + 1
            elif text.startswith("//", i):
                j = text.find("\n", i)
                i = n if j < 0 else j
            elif text.startswith("/*", i):
                j = text.find("*/", i + 2)
                i = n if j < 0 else j + 2
            else:
                out.append(c)
                i += 1
        lines = [ln.rstrip() for ln in "".join(out).split("\n")]
        h.update(("\n".join(ln for ln in lines if ln) + "\n").encode())
    return h.hexdigest()


def record_matches(rec, kname=None) -> bool:
    """True if a committed profile record was taken on the sources as they are
    now (and, given a kernel name, on that kernel)."""
    try:
        digest = source_digest(rec["source_files"])
    except (OSError, KeyError, ValueError, UnicodeDecodeError):
        return False
    return digest == rec.get("source_sha256") and (kname is None or rec.get("kernel_id") == kname)


def counters_path(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"tq_score_{workload}_counters.json")


def measured_traffic(w, kname):
    """HBM bytes per score launch from the committed counter record of this
    workload, if it was taken on the kernel that runs now with its source as it
    is now; else None."""
    try:
        with open(counters_path(w.name)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if not record_matches(rec, kname):
        return None
    return rec["per_dispatch"]["traffic_bytes"]


def copy_calibration() -> int:
    """Device-to-device copies of a known size, for calibrating FETCH_SIZE/WRITE_SIZE."""
    import torch

    n = 256 * 1024 * 1024
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(20):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read_per_copy": n, "bytes_written_per_copy": n,
                                           "copies": 20}}), flush=True)
    return 0


def build_ring(w, device, seed_base):
    """Distinct input/output buffer sets, each a full batch of workload w."""
    import numpy as np
    import torch

    import compressed_attention_scoring_amd as tq
    import synth

    per_set = w.key_bytes() + w.score_bytes() + 4 * w.P * w.B * w.D * 3
    nsets = max(2, math.ceil(RING_BYTES / per_set))
    if w.name not in ("decode", "tiny", "packed"):
        nsets = max(2, min(nsets, 8))
    Pi, S_mat = synth.head_matrices(w.seed, w.H, w.D)
    cb = synth.timing_codebook(w.seed, w.C, w.D)
    q = synth.queries(w.seed, w.P, w.B, w.D)
    idx, sign, gamma = synth.timing_code_streams(w.seed, w.P, w.S, w.D, w.C, w.layout, w.bits)
    base = {
        "q": torch.from_numpy(q).to(device),
        "idx": torch.from_numpy(idx).to(device),
        "sign": torch.from_numpy(sign).to(device),
        "gamma": torch.from_numpy(gamma).to(device),
    }
    shared = {
        "Pi": torch.from_numpy(Pi).to(device),
        "S_mat": torch.from_numpy(S_mat).to(device),
        "codebook": torch.from_numpy(cb).to(device),
    }
    ring = []
    for _ in range(nsets):
        s = {k: v.clone() for k, v in base.items()}
        s["A"] = torch.empty((w.P, w.B, w.D), dtype=torch.float32, device=device)
        s["T"] = torch.empty_like(s["A"])
        s["scores"] = torch.empty((w.P, w.B, w.S), dtype=torch.float32, device=device)
        s["keys"] = tq.Keys(w.layout, s["idx"], s["sign"], s["gamma"], w.bits if w.layout == "packed" else 0)
        ring.append(s)
    torch.cuda.synchronize()
    host = {"q": q, "Pi": Pi, "S_mat": S_mat, "codebook": cb, "idx": idx, "sign": sign, "gamma": gamma}
    return ring, shared, host, per_set


def make_step(w, shared, kernel):
    import compressed_attention_scoring_amd as tq

    def step(s, ev=None):
        if ev is not None:
            ev[0].record()
        tq.tq_query_transform(s["q"], shared["Pi"], shared["S_mat"], s["A"], s["T"])
        if ev is not None:
            ev[1].record()
        tq.tq_score_with_kernel(s["A"], s["T"], s["keys"], shared["codebook"], kernel, s["scores"])
        if ev is not None:
            ev[2].record()
    return step


def time_step_graphs(w, ring, shared, kernel, steps):
    """Run exactly `steps` steps from captured HIP graphs, one graph per chunk of
    consecutive ring sets holding each set's transform and then its score (the
    path's own order). Returns (seconds between synchronisations, mean us per
    step on the GPU from HIP events around the graph launches)."""
    import torch

    import compressed_attention_scoring_amd as tq

    G = len(ring)
    chunks = [G] * (steps // G) + ([steps % G] if steps % G else [])
    graphs = {}
    for n in sorted(set(chunks)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                s = ring[i]
                tq.tq_query_transform(s["q"], shared["Pi"], shared["S_mat"], s["A"], s["T"])
                tq.tq_score_with_kernel(s["A"], s["T"], s["keys"], shared["codebook"], kernel, s["scores"])
        graphs[n] = g
    for g in graphs.values():           # one untimed replay of each graph
        g.replay()
    torch.cuda.synchronize()
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(2)) for _ in chunks]
    t0 = time.perf_counter()
    for n, ev in zip(chunks, evs):
        ev[0].record()
        graphs[n].replay()
        ev[1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    return elapsed, 1e3 * sum(a.elapsed_time(b) for a, b in evs) / steps


def time_phased_graphs(w, ring, shared, kernel, steps):
    """Run exactly `steps` steps from captured HIP graphs and time each kernel.

    The ring is cut into chunks of consecutive buffer sets. For a chunk, one graph
    holds the query transforms of its sets and a second graph their scores, so
    each batch still gets its transform and then its score. HIP events recorded
    on the kernels' stream between the graph launches bracket runs of
    back-to-back kernels of one kind, giving each kernel's average duration
    without per-launch event overhead. Returns (seconds between synchronisations,
    mean transform us, mean score us)."""
    import torch

    import compressed_attention_scoring_amd as tq

    G = len(ring)
    chunks = [G] * (steps // G) + ([steps % G] if steps % G else [])
    graphs = {}
    for n in sorted(set(chunks)):
        gq, gs = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(gq):
            for i in range(n):
                tq.tq_query_transform(ring[i]["q"], shared["Pi"], shared["S_mat"], ring[i]["A"], ring[i]["T"])
        with torch.cuda.graph(gs):
            for i in range(n):
                s = ring[i]
                tq.tq_score_with_kernel(s["A"], s["T"], s["keys"], shared["codebook"], kernel, s["scores"])
        graphs[n] = (gq, gs)
    for gq, gs in graphs.values():      # one untimed replay of each graph
        gq.replay()
        gs.replay()
    torch.cuda.synchronize()
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in chunks]
    t0 = time.perf_counter()
    for n, ev in zip(chunks, evs):
        gq, gs = graphs[n]
        ev[0].record()
        gq.replay()
        ev[1].record()
        gs.replay()
        ev[2].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    qt_ms = sum(a.elapsed_time(b) for a, b, _ in evs)
    sc_ms = sum(b.elapsed_time(c) for _, b, c in evs)
    return elapsed, 1e3 * qt_ms / steps, 1e3 * sc_ms / steps


def stream_probe(device, nbytes: int) -> dict:
    """A same-size reference for what one launch can move on this GPU: a
    device-to-device copy of nbytes / 2 bytes (so nbytes are read and written
    in total, like one tq_score launch's algorithmic bytes), replayed back to
    back from a captured graph over distinct buffer pairs (>= 512 MB in all, so
    no copy finds its source in the caches), timed with HIP events."""
    import torch

    half = max(256, (nbytes // 2) // 256 * 256)
    npairs = max(2, min(64, math.ceil(RING_BYTES / (2 * half))))
    pairs = [(torch.empty(half, dtype=torch.uint8, device=device), torch.empty(half, dtype=torch.uint8, device=device))
             for _ in range(npairs)]
    for src, _ in pairs:
        src.fill_(1)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for src, dst in pairs:
            dst.copy_(src)
    g.replay()
    torch.cuda.synchronize()
    reps = max(2, 2000 // npairs)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = 1e3 * e0.elapsed_time(e1) / (reps * npairs)
    return {"kind": "device-to-device copy (torch copy_), graph-replayed over distinct buffers",
            "bytes": 2 * half, "us": us, "GB_s": 2 * half / (us * 1e-6) / 1e9}


def stream_probes(device, read_bytes: int, write_bytes: int, steps: int, tile=None) -> dict:
    """The library's streaming probes at the workload's byte counts: tq_probe_read
    over read_bytes (the key codes of one launch), tq_probe_write over
    write_bytes (its scores), and tq_probe_read_write (each workgroup reads its
    slice of the codes, then writes its slice of the scores from what it read).
    With tile = (B, S, D) (unpacked keys, one 32-query tile) also tq_probe_tile:
    the unpacked scorer's own loads and stores in its own grid, without its
    arithmetic (the read buffer holds the index rows, the sign rows and gamma).
    Each is launched over a ring of distinct buffers (>= 512 MB, so no launch
    finds its bytes in the caches), captured in a graph and replayed back to
    back, timed with HIP events on the launching stream -- the same method as
    the score kernel's figure."""
    import ctypes

    import torch

    import compressed_attention_scoring_amd as tq

    rb = (read_bytes + 15) // 16 * 16
    wb = (write_bytes + 15) // 16 * 16
    npairs = max(2, min(64, math.ceil(RING_BYTES / (rb + wb))))
    pairs = [(torch.empty(rb, dtype=torch.uint8, device=device), torch.empty(wb, dtype=torch.uint8, device=device))
             for _ in range(npairs)]
    for src, _ in pairs:
        src.fill_(3)
    sink = torch.zeros(4, dtype=torch.int32, device=device)
    lib = tq._lib
    vp = ctypes.c_void_p

    def launch(kind, src, dst):
        st = vp(torch.cuda.current_stream(device).cuda_stream)
        if kind == "read":
            rc = lib.tq_probe_read(vp(src.data_ptr()), ctypes.c_size_t(rb), vp(sink.data_ptr()), st)
        elif kind == "write":
            rc = lib.tq_probe_write(vp(dst.data_ptr()), ctypes.c_size_t(wb), st)
        elif kind == "tile":
            B, S, D = tile
            ck = tq._CKeys(0, 0, src.data_ptr(), src.data_ptr() + S * D, src.data_ptr() + 2 * S * D)
            rc = lib.tq_probe_tile(ctypes.byref(ck), vp(dst.data_ptr()), B, S, D, st)
        else:
            rc = lib.tq_probe_read_write(vp(src.data_ptr()), ctypes.c_size_t(rb), vp(dst.data_ptr()),
                                         ctypes.c_size_t(wb), st)
        if rc != 0:
            raise tq.TqError(rc, f"tq_probe_{kind}")

    out = {"kind": "the library's streaming probe kernels (tq_probe_*), graph-replayed over distinct buffers, "
                   "HIP events",
           "ring_pairs": npairs}
    reps = max(2, steps // npairs)
    kinds = [("read", rb), ("write", wb), ("read_write", rb + wb)] + ([("tile", rb + wb)] if tile else [])
    for kind, nbytes in kinds:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for src, dst in pairs:
                launch(kind, src, dst)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = 1e3 * e0.elapsed_time(e1) / (reps * npairs)
        out[kind] = {"bytes": nbytes, "us": us, "GB_s": nbytes / (us * 1e-6) / 1e9}
    return out


def trace_record(w, kname):
    """Per-dispatch durations of this workload's score kernel from the committed
    rocprofv3 kernel-trace record, if it was taken on the kernel that runs now
    with its source as it is now; else None."""
    try:
        with open(os.path.join(ROOT, "profiles", f"tq_score_{w.name}_kernel_trace.json")) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if not record_matches(rec, kname):
        return None
    return rec


def cpu_baseline(w, host, target_s):
    """The float64 oracle (explicit key reconstruction) on the host cores."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import score as osc

    from threadpoolctl import threadpool_limits

    threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    P = 1
    S = w.S

    def timed_runs(budget_s):
        times = []
        t_start = time.perf_counter()
        while True:
            t0 = time.perf_counter()
            for p in range(P):
                osc.scores_by_reconstruction(host["q"][p], host["idx"][p], host["sign"][p],
                                             host["gamma"][p].astype(np.float64), host["Pi"][p % w.H],
                                             host["S_mat"][p % w.H], host["codebook"])
            times.append(time.perf_counter() - t0)
            if time.perf_counter() - t_start >= budget_s and len(times) >= 3:
                break
            if len(times) >= 5000:
                break
        return sorted(times)[len(times) // 2], times

    med, times = timed_runs(target_s)
    with threadpool_limits(limits=1, user_api="blas"):
        med1, times1 = timed_runs(min(target_s, 3.0))
    pairs = P * w.B * S
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            model = next(line.split(":", 1)[1].strip() for line in f if line.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return {
        "value": pairs / med,
        "unit": "scores/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{'problem 0 of ' + str(w.P) if w.P > 1 else 'the full batch'} "
                   f"(B={w.B}, S={S}, D={w.D}) scored by float64 explicit reconstruction, "
                   f"median of {len(times)} runs ({sum(times):.1f} s total); host {model}"),
        "value_1_thread": pairs / med1,
        "runs_1_thread": len(times1),
        "cpu_model": model,
    }


def bench_compress(args, w, device) -> dict:
    """Time tq_compress_keys on the workload's P*S keys (float64 arithmetic,
    three D x D products per key on the fp64 matrix cores)."""
    import numpy as np
    import torch

    import compressed_attention_scoring_amd as tq
    import synth
    from oracle.codebook import codebook_fp32

    Pi, S_mat = synth.head_matrices(w.seed, w.H, w.D)
    cb = codebook_fp32(w.D, w.C)
    one = synth.unit_keys(synth.keys_rng(w.seed, 0), w.S, w.D, w.keys).astype(np.float32)
    keys_dev = torch.from_numpy(one).to(device).unsqueeze(0).expand(w.P, w.S, w.D).contiguous()
    shared = [torch.from_numpy(a).to(device) for a in (Pi, S_mat, cb)]
    per_set = keys_dev.numel() * 4 + w.key_bytes()
    nsets = max(2, min(32, math.ceil(RING_BYTES / per_set)))
    ring = [keys_dev.clone() for _ in range(nsets)]
    bits = w.bits if w.layout == "packed" else 0
    outs = [tq.tq_compress_keys(k, *shared, w.layout, bits) for k in ring]   # allocates the outputs once
    torch.cuda.synchronize()

    def launch(i):
        k, o = ring[i], outs[i]
        out = tq._CKeysOut(tq.TQ_UNPACKED if w.layout == "unpacked" else tq.TQ_PACKED, bits,
                           o.idx.data_ptr(), o.sign.data_ptr(), o.gamma.data_ptr())
        st = torch.cuda.current_stream(device).cuda_stream
        rc = tq._lib.tq_compress_keys(k.data_ptr(), shared[0].data_ptr(), shared[1].data_ptr(),
                                      shared[2].data_ptr(), w.C, ctypes.byref(out), w.P, w.H, w.S, w.D, st)
        if rc != 0:
            raise tq.TqError(rc, "tq_compress_keys")

    for i in range(args.warmup):
        launch(i % nsets)
    torch.cuda.synchronize()
    steps = args.steps
    chunks = [nsets] * (steps // nsets) + ([steps % nsets] if steps % nsets else [])
    graphs = {}
    for n in sorted(set(chunks)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                launch(i)
        graphs[n] = g
    for g in graphs.values():
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for n in chunks:
        graphs[n].replay()
    e1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    us = 1e3 * e0.elapsed_time(e1) / steps
    nkeys = w.P * w.S
    flops = 6 * w.D * w.D * nkeys          # y = Pi k, x = Pi^T c, p = S_mat r
    achieved = flops / (us * 1e-6) / 1e12
    log(f"compress: {steps} launches, {us:.2f} us per launch ({nkeys} keys), {achieved:.1f} TFLOP/s fp64")
    out = {
        "metric": "keys compressed/sec (TurboQuant_prod, float64 arithmetic)",
        "value": nkeys / (us * 1e-6),
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed * 1e3 / steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic: seeded unit keys (Gaussian with outlier channels), Haar rotation, Gaussian projection",
        "config": {"workload": w.name, "path": "compress", "P": w.P, "S": w.S, "D": w.D, "C": w.C,
                   "layout": w.layout, "bits": w.bits},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": FP64_MATRIX_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / FP64_MATRIX_PEAK_TFLOPS, "traffic": None,
                     "kernel": f"compress_{w.layout}{bits if bits else ''}", "flops_per_launch": flops,
                     "avg_launch_us": us},
        "ring_sets": nsets,
    }
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_info

        from oracle import compress as oc
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
        k64 = one.astype(np.float64)
        times = []
        t_start = time.perf_counter()
        while time.perf_counter() - t_start < args.cpu_seconds or len(times) < 3:
            t1 = time.perf_counter()
            oc.quantize_prod_unit(k64, Pi[0], S_mat[0], cb)
            times.append(time.perf_counter() - t1)
        med = sorted(times)[len(times) // 2]
        out["cpu_baseline"] = {"value": w.S / med, "unit": "keys/s", "cores": int(threads), "kind": "oracle",
                               "sample": f"one problem's {w.S} keys (D={w.D}) compressed by the float64 oracle, "
                                         f"median of {len(times)} runs ({sum(times):.1f} s total)"}
    return out


def attend_bytes(w) -> int:
    """Bytes tq_attend must move once: fp32 scores, value indices and norms,
    the value codebook and rotations in, fp32 outputs out."""
    if w.layout == "unpacked":
        per_value = w.D + 4
    else:
        per_value = w.D * w.bits // 8 + 2
    return (w.P * w.B * w.S * 4 + w.P * w.S * per_value + w.C * 4 + w.H * w.D * w.D * 4
            + w.P * w.B * w.D * 4)


def attend_traffic(w):
    """HBM bytes per tq_attend call (both kernels) from the committed counter
    record of this workload, if taken with attend.hip as it is now; else None."""
    try:
        with open(os.path.join(ROOT, "profiles", f"tq_attend_{w.name}_counters.json")) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if not record_matches(rec):
        return None
    return rec["traffic_bytes_per_call"]


def bench_attend(args, w, device) -> dict:
    """Time tq_attend (partial and combine kernels) on the workload's shape:
    scores [P,B,S] and values in the workload's key layout and codebook size."""
    import numpy as np
    import torch

    import compressed_attention_scoring_amd as tq
    import synth

    bits = w.bits if w.layout == "packed" else 0
    rng = np.random.default_rng([w.seed, 7])
    Pi_v = np.stack([synth.haar_rotation(rng, w.D) for _ in range(w.H)])
    cb = synth.timing_codebook(w.seed, w.C, w.D)
    idx, norm = synth.timing_value_streams(w.seed, w.P, w.S, w.D, w.C, w.layout, bits)
    scores = synth.timing_scores(w.seed, w.P, w.B, w.S)
    shared = {"Pi_v": torch.from_numpy(Pi_v).to(device), "cb": torch.from_numpy(cb).to(device)}
    base = {"idx": torch.from_numpy(idx).to(device), "norm": torch.from_numpy(norm).to(device),
            "scores": torch.from_numpy(scores).to(device)}
    nbytes = attend_bytes(w)
    nsets = max(2, min(64, math.ceil(RING_BYTES / nbytes)))
    wsb = tq.tq_attend_workspace_bytes(w.P, w.B, w.S, w.D)
    ring = []
    for _ in range(nsets):
        s = {k: v.clone() for k, v in base.items()}
        s["values"] = tq.Values(w.layout, s["idx"], s["norm"], bits)
        s["out"] = torch.empty((w.P, w.B, w.D), dtype=torch.float32, device=device)
        s["ws"] = torch.empty(wsb, dtype=torch.uint8, device=device)
        ring.append(s)
    scale = 1.0 / math.sqrt(w.D)

    def launch(s):
        tq.tq_attend(s["scores"], s["values"], shared["cb"], shared["Pi_v"], scale, s["out"], s["ws"])

    for i in range(args.warmup):
        launch(ring[i % nsets])
    torch.cuda.synchronize()
    steps = args.steps
    chunks = [nsets] * (steps // nsets) + ([steps % nsets] if steps % nsets else [])
    graphs = {}
    for n in sorted(set(chunks)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                launch(ring[i])
        graphs[n] = g
    for g in graphs.values():
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for n in chunks:
        graphs[n].replay()
    e1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    us = 1e3 * e0.elapsed_time(e1) / steps
    achieved = nbytes / (us * 1e-6) / 1e9
    log(f"attend: {steps} calls, {us:.2f} us per call, {achieved:.0f} GB/s algorithmic")
    out = {
        "metric": "attention outputs/sec (softmax over scores, compressed-value aggregation)",
        "value": w.P * w.B / (us * 1e-6),
        "unit": "query outputs/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed * 1e3 / steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 MFMA on hi/lo-split fp32 operands, f32 accumulate",
        "data": "synthetic: seeded random value codes and norms, N(0, 16) scores, Haar value rotation",
        "config": {"workload": w.name, "path": "attend", "P": w.P, "H": w.H, "B": w.B, "S": w.S, "D": w.D,
                   "C": w.C, "layout": w.layout, "bits": w.bits, "scale": scale},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": attend_traffic(w),
                     "kernel": "attend_partial + attend_combine", "bytes_per_launch": nbytes,
                     "avg_launch_us": us, "workspace_bytes": wsb},
        "ring_sets": nsets,
    }
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_info

        from oracle import attend as oa
        from oracle import pack as opk
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
        idx0 = idx[0] if w.layout == "unpacked" else opk.unpack_indices(idx[0], w.bits, w.D)
        n0 = norm[0].astype(np.float64)
        times = []
        t_start = time.perf_counter()
        while time.perf_counter() - t_start < args.cpu_seconds or len(times) < 3:
            t1 = time.perf_counter()
            oa.attend_rotated(scores[0], idx0, n0, Pi_v[0], cb, scale)
            times.append(time.perf_counter() - t1)
        med = sorted(times)[len(times) // 2]
        out["cpu_baseline"] = {"value": w.B / med, "unit": "query outputs/s", "cores": int(threads),
                               "kind": "oracle",
                               "sample": f"problem 0 (B={w.B}, S={w.S}, D={w.D}) through the float64 oracle, "
                                         f"median of {len(times)} runs ({sum(times):.1f} s total)"}
    return out


def mse_bytes(w) -> int:
    """Bytes tq_score_mse must move once: key indices and norms, A and the
    codebook in, fp32 scores out."""
    per_key = w.D + 4 if w.layout == "unpacked" else w.D * w.bits // 8 + 2
    return w.P * w.S * per_key + w.P * w.B * w.D * 4 + w.C * 4 + w.P * w.B * w.S * 4


def score_dtype(kname) -> str:
    """The arithmetic of a score kernel, from its name: the four-query kernel for
    packed keys multiplies int8 limbs on the integer matrix cores, the others
    f16 hi/lo parts on the f16 ones."""
    if kname and "i8" in kname:
        return "i8 MFMA on int8-limb-split fp32 operands (4 query limbs, 3 codebook limbs), i32 accumulate"
    return "f16 MFMA on hi/lo-split fp32 operands, f32 accumulate"


def bench_mse(args, w, device) -> dict:
    """One step = tq_query_transform_hadamard + tq_score_mse over the workload's
    shape with MSE-only keys (its index layout and codebook size, one norm per
    key, no signs). Per-kernel times from phased graph replays, as for the
    scoring path."""
    import numpy as np
    import torch

    import compressed_attention_scoring_amd as tq
    import synth

    bits = w.bits if w.layout == "packed" else 0
    rng = np.random.default_rng([w.seed, 11])
    signs = np.where(rng.integers(0, 2, size=(w.H, w.D)) == 1, 1.0, -1.0).astype(np.float32)
    cb = synth.timing_codebook(w.seed, w.C, w.D)
    idx, norm = synth.timing_value_streams(w.seed, w.P, w.S, w.D, w.C, w.layout, bits)
    q = synth.queries(w.seed, w.P, w.B, w.D)
    shared = {"signs": torch.from_numpy(signs).to(device), "cb": torch.from_numpy(cb).to(device)}
    base = {"q": torch.from_numpy(q).to(device), "idx": torch.from_numpy(idx).to(device),
            "norm": torch.from_numpy(norm).to(device)}
    nbytes = mse_bytes(w)
    # tq_score_mse picks its kernel form by the same rule as tq_score
    mse_kernel = tq.tq_score_kernel_name(w.layout, bits, w.C, w.P, w.B, w.S, w.D)
    nsets = max(2, min(64, math.ceil(RING_BYTES / nbytes)))
    ring = []
    for _ in range(nsets):
        s = {k: v.clone() for k, v in base.items()}
        s["keys"] = tq.Values(w.layout, s["idx"], s["norm"], bits)
        s["A"] = torch.empty((w.P, w.B, w.D), dtype=torch.float32, device=device)
        s["scores"] = torch.empty((w.P, w.B, w.S), dtype=torch.float32, device=device)
        ring.append(s)

    def transform(s):
        tq.tq_query_transform_hadamard(s["q"], shared["signs"], s["A"])

    def score(s):
        tq.tq_score_mse(s["A"], s["keys"], shared["cb"], s["scores"])

    for i in range(args.warmup):
        transform(ring[i % nsets])
        score(ring[i % nsets])
    torch.cuda.synchronize()
    steps = args.steps
    chunks = [nsets] * (steps // nsets) + ([steps % nsets] if steps % nsets else [])
    graphs = {}
    for n in sorted(set(chunks)):
        gt, gs = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(gt):
            for i in range(n):
                transform(ring[i])
        with torch.cuda.graph(gs):
            for i in range(n):
                score(ring[i])
        graphs[n] = (gt, gs)
    for gt, gs in graphs.values():
        gt.replay()
        gs.replay()
    torch.cuda.synchronize()
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in chunks]
    t0 = time.perf_counter()
    for n, ev in zip(chunks, evs):
        gt, gs = graphs[n]
        ev[0].record()
        gt.replay()
        ev[1].record()
        gs.replay()
        ev[2].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    qt_us = 1e3 * sum(a.elapsed_time(b) for a, b, _ in evs) / steps
    sc_us = 1e3 * sum(b.elapsed_time(c) for _, b, c in evs) / steps
    ms_per_step = elapsed * 1e3 / steps
    achieved = nbytes / (sc_us * 1e-6) / 1e9
    log(f"mse: transform {qt_us:.2f} us, score {sc_us:.2f} us per launch, {achieved:.0f} GB/s algorithmic")
    out = {
        "metric": "query-key scores/sec, MSE-only keys (randomized Hadamard queries)",
        "value": w.pairs / (ms_per_step * 1e-3),
        "unit": "scores/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": score_dtype(mse_kernel),
        "data": "synthetic: seeded random MSE codes and norms, N(0,1) queries, random Hadamard signs",
        "config": {"workload": w.name, "path": "mse", "P": w.P, "H": w.H, "B": w.B, "S": w.S, "D": w.D, "C": w.C,
                   "layout": w.layout, "bits": w.bits},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None, "kernel": f"{mse_kernel} (MSE-only form)",
                     "bytes_per_launch": nbytes, "avg_launch_us": sc_us},
        "tq_score_mse_us": sc_us,
        "tq_query_transform_hadamard_us": qt_us,
        "ring_sets": nsets,
    }
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_info

        from oracle import mse as om
        from oracle import pack as opk
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
        idx0 = idx[0] if w.layout == "unpacked" else opk.unpack_indices(idx[0], w.bits, w.D)
        R = om.hadamard_rotation(signs[0].astype(np.float64))
        n0 = norm[0].astype(np.float64)
        times = []
        t_start = time.perf_counter()
        while time.perf_counter() - t_start < args.cpu_seconds or len(times) < 3:
            t1 = time.perf_counter()
            om.scores_mse_by_reconstruction(q[0], idx0, n0, R, cb)
            times.append(time.perf_counter() - t1)
        med = sorted(times)[len(times) // 2]
        out["cpu_baseline"] = {"value": w.B * w.S / med, "unit": "scores/s", "cores": int(threads), "kind": "oracle",
                               "sample": f"problem 0 (B={w.B}, S={w.S}, D={w.D}) scored by float64 explicit "
                                         f"reconstruction, median of {len(times)} runs ({sum(times):.1f} s total)"}
    return out


def bench_split(args, w, device) -> dict:
    """One step = tq_query_transform_split + tq_score_split over the workload's
    shape (P, B, S, D) with outlier-split keys: the 32 hot channels at 3 bits
    (C=8) and the other D-32 at 2 bits (C=4), both packed with fp16 norms."""
    import numpy as np
    import torch

    import compressed_attention_scoring_amd as tq
    import synth

    d_hi, d_lo = 32, w.D - 32
    rng = np.random.default_rng([w.seed, 21])
    perm = np.concatenate([np.arange(0, w.D, w.D // d_hi), np.setdiff1d(np.arange(w.D), np.arange(0, w.D, w.D // d_hi))])
    perm = perm.astype(np.int32)
    Pi_hi = np.stack([synth.haar_rotation(rng, d_hi) for _ in range(w.H)])
    Pi_lo = np.stack([synth.haar_rotation(rng, d_lo) for _ in range(w.H)])
    cb_hi = synth.timing_codebook(w.seed, 8, d_hi)
    cb_lo = synth.timing_codebook(w.seed + 1, 4, d_lo)
    ih, nh = synth.timing_value_streams(w.seed, w.P, w.S, d_hi, 8, "packed", 3)
    il, nl = synth.timing_value_streams(w.seed + 1, w.P, w.S, d_lo, 4, "packed", 2)
    q = synth.queries(w.seed, w.P, w.B, w.D)
    shared = {k: torch.from_numpy(v).to(device) for k, v in
              {"perm": perm, "Pi_hi": Pi_hi, "Pi_lo": Pi_lo, "cb_hi": cb_hi, "cb_lo": cb_lo}.items()}
    base = {k: torch.from_numpy(v).to(device) for k, v in {"q": q, "ih": ih, "nh": nh, "il": il, "nl": nl}.items()}
    nbytes = (w.P * w.S * (d_hi * 3 // 8 + 2 + d_lo * 2 // 8 + 2) + w.P * w.B * w.D * 4 + 12 * 4
              + w.P * w.B * w.S * 4)
    flops = 2 * w.P * w.B * w.S * w.D
    nsets = max(2, min(64, math.ceil(RING_BYTES / nbytes)))
    ring = []
    for _ in range(nsets):
        s = {k: v.clone() for k, v in base.items()}
        s["keys"] = tq.SplitKeys(tq.Values("packed", s["ih"], s["nh"], 3), tq.Values("packed", s["il"], s["nl"], 2))
        s["A"] = None
        s["scores"] = torch.empty((w.P, w.B, w.S), dtype=torch.float32, device=device)
        ring.append(s)

    def transform(s):
        s["A"] = tq.tq_query_transform_split(s["q"], shared["perm"], shared["Pi_hi"], shared["Pi_lo"])

    def score(s):
        tq.tq_score_split(s["A"][0], s["A"][1], s["keys"], shared["cb_hi"], shared["cb_lo"], s["scores"])

    for s in ring:                      # allocates each set's A once, before capture
        transform(s)
    A_fixed = [s["A"] for s in ring]

    def transform_into(i):
        A_hi, A_lo = A_fixed[i]
        tq.tq_query_transform_split(ring[i]["q"], shared["perm"], shared["Pi_hi"], shared["Pi_lo"], A_hi, A_lo)

    for i in range(args.warmup):
        transform_into(i % nsets)
        score(ring[i % nsets])
    torch.cuda.synchronize()
    steps = args.steps
    chunks = [nsets] * (steps // nsets) + ([steps % nsets] if steps % nsets else [])
    graphs = {}
    for n in sorted(set(chunks)):
        gt, gs = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(gt):
            for i in range(n):
                transform_into(i)
        with torch.cuda.graph(gs):
            for i in range(n):
                score(ring[i])
        graphs[n] = (gt, gs)
    for gt, gs in graphs.values():
        gt.replay()
        gs.replay()
    torch.cuda.synchronize()
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in chunks]
    t0 = time.perf_counter()
    for n, ev in zip(chunks, evs):
        gt, gs = graphs[n]
        ev[0].record()
        gt.replay()
        ev[1].record()
        gs.replay()
        ev[2].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    qt_us = 1e3 * sum(a.elapsed_time(b) for a, b, _ in evs) / steps
    sc_us = 1e3 * sum(b.elapsed_time(c) for _, b, c in evs) / steps
    ms_per_step = elapsed * 1e3 / steps
    tflops = flops / (sc_us * 1e-6) / 1e12
    gbs = nbytes / (sc_us * 1e-6) / 1e9
    log(f"split: transform {qt_us:.2f} us, score {sc_us:.2f} us per launch, {tflops:.1f} TFLOP/s, "
        f"{gbs:.0f} GB/s algorithmic")
    out = {
        "metric": "query-key scores/sec, outlier-split keys (32 channels at 3 bits + the rest at 2)",
        "value": w.pairs / (ms_per_step * 1e-3),
        "unit": "scores/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic: seeded random packed codes and fp16 norms per instance, N(0,1) queries, Haar rotations",
        "config": {"workload": w.name, "path": "split", "P": w.P, "H": w.H, "B": w.B, "S": w.S, "D": w.D,
                   "D_hi": d_hi, "bits_hi": 3, "D_lo": d_lo, "bits_lo": 2},
        # the 2.5-bit setting at D = 128 runs on the matrix cores (score_split_mfma_kernel):
        # bound by the bytes it moves, not by its f16 MFMA work (well under 1% of that peak)
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "score_split_mfma_kernel" if w.D == 128 else "score_split_kernel",
                     "bytes_per_launch": nbytes, "flops_per_launch": flops, "tflops": tflops,
                     "avg_launch_us": sc_us},
        "tq_score_split_us": sc_us,
        "tq_query_transform_split_us": qt_us,
        "ring_sets": nsets,
    }
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_info

        from oracle import pack as opk
        from oracle import split as osp
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
        u_hi = opk.unpack_indices(ih[0], 3, d_hi)
        u_lo = opk.unpack_indices(il[0], 2, d_lo)
        times = []
        t_start = time.perf_counter()
        while time.perf_counter() - t_start < args.cpu_seconds or len(times) < 3:
            t1 = time.perf_counter()
            osp.scores_split_by_reconstruction(q[0], perm, d_hi, u_hi, nh[0].astype(np.float64), Pi_hi[0], cb_hi,
                                               u_lo, nl[0].astype(np.float64), Pi_lo[0], cb_lo)
            times.append(time.perf_counter() - t1)
        med = sorted(times)[len(times) // 2]
        out["cpu_baseline"] = {"value": w.B * w.S / med, "unit": "scores/s", "cores": int(threads), "kind": "oracle",
                               "sample": f"problem 0 (B={w.B}, S={w.S}, D={w.D}) scored by float64 explicit "
                                         f"reconstruction, median of {len(times)} runs ({sum(times):.1f} s total)"}
    return out


def bench_fused(args, w, device) -> dict:
    """One step = tq_query_transform + tq_score_attend over the workload: its
    keys, and values in the same layout and codebook size. Timed beside the
    unfused form (tq_score then tq_attend) on the same inputs; per-kernel times
    from phased graph replays."""
    import numpy as np
    import torch

    import compressed_attention_scoring_amd as tq
    import synth

    bits = w.bits if w.layout == "packed" else 0
    Pi, S_mat = synth.head_matrices(w.seed, w.H, w.D)
    rng = np.random.default_rng([w.seed, 7])
    Pi_v = np.stack([synth.haar_rotation(rng, w.D) for _ in range(w.H)])
    cb = synth.timing_codebook(w.seed, w.C, w.D)
    cbv = synth.timing_codebook(w.seed + 1, w.C, w.D)
    q = synth.queries(w.seed, w.P, w.B, w.D)
    idx, sign, gamma = synth.timing_code_streams(w.seed, w.P, w.S, w.D, w.C, w.layout, w.bits)
    vidx, vnorm = synth.timing_value_streams(w.seed, w.P, w.S, w.D, w.C, w.layout, bits)
    shared = {k: torch.from_numpy(v).to(device) for k, v in
              {"Pi": Pi, "S_mat": S_mat, "Pi_v": Pi_v, "cb": cb, "cbv": cbv}.items()}
    base = {k: torch.from_numpy(v).to(device) for k, v in
            {"q": q, "idx": idx, "sign": sign, "gamma": gamma, "vidx": vidx, "vnorm": vnorm}.items()}
    per_set = w.key_bytes() + base["vidx"].numel() + base["vnorm"].numel() * base["vnorm"].element_size()
    nsets = max(2, min(64, math.ceil(RING_BYTES / per_set)))
    wsf = tq.tq_score_attend_workspace_bytes(w.P, w.B, w.S, w.D, "fused")
    wsa = tq.tq_attend_workspace_bytes(w.P, w.B, w.S, w.D)
    ring = []
    for _ in range(nsets):
        s = {k: v.clone() for k, v in base.items()}
        s["keys"] = tq.Keys(w.layout, s["idx"], s["sign"], s["gamma"], bits)
        s["values"] = tq.Values(w.layout, s["vidx"], s["vnorm"], bits)
        s["A"] = torch.empty((w.P, w.B, w.D), dtype=torch.float32, device=device)
        s["T"] = torch.empty_like(s["A"])
        s["out"] = torch.empty_like(s["A"])
        ring.append(s)
    ws_f = torch.empty(wsf, dtype=torch.uint8, device=device)     # calls on one stream run in order
    ws_auto = torch.empty(tq.tq_score_attend_workspace_bytes(w.P, w.B, w.S, w.D), dtype=torch.uint8, device=device)
    ws_a = torch.empty(wsa, dtype=torch.uint8, device=device)
    scores = torch.empty((w.P, w.B, w.S), dtype=torch.float32, device=device)
    scale = 1.0 / math.sqrt(w.D)

    def transform(s):
        tq.tq_query_transform(s["q"], shared["Pi"], shared["S_mat"], s["A"], s["T"])

    def fused(s):
        tq.tq_score_attend(s["A"], s["T"], s["keys"], shared["cb"], s["values"], shared["cbv"], shared["Pi_v"],
                           scale, s["out"], ws_f, mode="fused")

    def automatic(s):
        tq.tq_score_attend(s["A"], s["T"], s["keys"], shared["cb"], s["values"], shared["cbv"], shared["Pi_v"],
                           scale, s["out"], ws_auto)

    def unfused(s):
        tq.tq_score(s["A"], s["T"], s["keys"], shared["cb"], scores)
        tq.tq_attend(scores, s["values"], shared["cbv"], shared["Pi_v"], scale, s["out"], ws_a)

    for i in range(args.warmup):
        transform(ring[i % nsets])
        fused(ring[i % nsets])
        unfused(ring[i % nsets])
        automatic(ring[i % nsets])
    torch.cuda.synchronize()
    steps = args.steps
    chunks = [nsets] * (steps // nsets) + ([steps % nsets] if steps % nsets else [])

    def phased(second):
        graphs = {}
        for n in sorted(set(chunks)):
            g1, g2 = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
            with torch.cuda.graph(g1):
                for i in range(n):
                    transform(ring[i])
            with torch.cuda.graph(g2):
                for i in range(n):
                    second(ring[i])
            graphs[n] = (g1, g2)
        for g1, g2 in graphs.values():
            g1.replay()
            g2.replay()
        torch.cuda.synchronize()
        evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in chunks]
        t0 = time.perf_counter()
        for n, ev in zip(chunks, evs):
            g1, g2 = graphs[n]
            ev[0].record()
            g1.replay()
            ev[1].record()
            g2.replay()
            ev[2].record()
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        return (el, 1e3 * sum(a.elapsed_time(b) for a, b, _ in evs) / steps,
                1e3 * sum(b.elapsed_time(c) for _, b, c in evs) / steps)

    el_a, qt_us, auto_us = phased(automatic)
    _, _, fused_us = phased(fused)
    el_u, _, unfused_us = phased(unfused)
    if w.layout == "unpacked":
        vb = w.D + 4
    else:
        vb = w.D * w.bits // 8 + 2
    nbytes = w.key_bytes() + w.P * w.S * vb + 2 * w.P * w.B * w.D * 4 + 2 * w.C * 4 + w.H * w.D * w.D * 4 \
        + w.P * w.B * w.D * 4
    achieved = nbytes / (fused_us * 1e-6) / 1e9
    ms_per_step = el_a * 1e3 / steps
    log(f"fused: transform {qt_us:.2f} us, tq_score_attend {auto_us:.2f} us per call (one-pass form "
        f"{fused_us:.2f}, score then attend {unfused_us:.2f}); one-pass {achieved:.0f} GB/s algorithmic")
    out = {
        "metric": "decode steps/sec (query transform + tq_score_attend: scores, softmax and value sum)",
        "value": w.P * w.B / (ms_per_step * 1e-3),
        "unit": "query outputs/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 MFMA on hi/lo-split fp32 operands, f32 accumulate",
        "data": "synthetic: seeded random key and value codes, N(0,1) queries, Haar rotations, Gaussian projection",
        "config": {"workload": w.name, "path": "fused", "P": w.P, "H": w.H, "B": w.B, "S": w.S, "D": w.D, "C": w.C,
                   "layout": w.layout, "bits": w.bits, "scale": scale},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "score_attend_kernel + attend_combine", "bytes_per_launch": nbytes,
                     "avg_launch_us": fused_us, "workspace_bytes": wsf},
        "tq_score_attend_us": auto_us,
        "one_pass_form_us": fused_us,
        "unfused_score_then_attend_us": unfused_us,
        "ms_per_step_unfused": el_u * 1e3 / steps,
        "tq_query_transform_us": qt_us,
        "ring_sets": nsets,
    }
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_info

        from oracle import attend as oa
        from oracle import score as osc
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
        from oracle import pack as opk
        if w.layout == "unpacked":
            iu, su, vu = idx[0], sign[0], vidx[0]
        else:
            iu, su = opk.unpack_indices(idx[0], w.bits, w.D), opk.unpack_signs(sign[0], w.D)
            vu = opk.unpack_indices(vidx[0], w.bits, w.D)
        times = []
        t_start = time.perf_counter()
        while time.perf_counter() - t_start < args.cpu_seconds or len(times) < 3:
            t1 = time.perf_counter()
            sco = osc.scores_by_reconstruction(q[0], iu, su, gamma[0].astype(np.float64), Pi[0], S_mat[0], cb)
            oa.attend_rotated(sco, vu, vnorm[0].astype(np.float64), Pi_v[0], cbv, scale)
            times.append(time.perf_counter() - t1)
        med = sorted(times)[len(times) // 2]
        out["cpu_baseline"] = {"value": w.B / med, "unit": "query outputs/s", "cores": int(threads), "kind": "oracle",
                               "sample": f"problem 0 (B={w.B}, S={w.S}, D={w.D}): float64 scores by reconstruction, "
                                         f"then softmax and value sum, median of {len(times)} runs "
                                         f"({sum(times):.1f} s total)"}
    return out


def main() -> int:
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only: the path would shard by key "
                                   "ranges or problems with no exchange between GPUs, but no multi-GPU "
                                   "run is built",
                          "n_gpus": args.gpus}), flush=True)
        return 2
    if args.copy_calibration:
        return copy_calibration()
    import torch

    import compressed_attention_scoring_amd as tq
    import synth

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    device = torch.device("cuda:0")
    w = synth.workload(args.workload)
    if args.path == "compress":
        print(json.dumps(bench_compress(args, w, device)), flush=True)
        return 0
    if args.path == "attend":
        print(json.dumps(bench_attend(args, w, device)), flush=True)
        return 0
    if args.path == "mse":
        print(json.dumps(bench_mse(args, w, device)), flush=True)
        return 0
    if args.path == "split":
        print(json.dumps(bench_split(args, w, device)), flush=True)
        return 0
    if args.path == "fused":
        print(json.dumps(bench_fused(args, w, device)), flush=True)
        return 0
    kname = tq.tq_score_kernel_name(w.layout, w.bits, w.C, w.P, w.B, w.S, w.D, args.kernel)
    log(f"workload {w.describe()} kernel {kname}")
    ring, shared, host, per_set = build_ring(w, device, w.seed)
    log(f"ring of {len(ring)} buffer sets, {len(ring) * per_set / 1e6:.0f} MB")
    step = make_step(w, shared, args.kernel)

    for i in range(args.warmup):
        step(ring[i % len(ring)])
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    mode = "eager" if args.eager else "hipgraph"
    step_gpu_us = None
    if mode == "hipgraph":
        # the K timed steps: each batch's transform then its score, from graphs
        elapsed, step_gpu_us = time_step_graphs(w, ring, shared, args.kernel, args.steps)
        # the per-kernel split from a second pass of K steps in phased graphs
        _, qt_us, score_us = time_phased_graphs(w, ring, shared, args.kernel, args.steps)
    else:
        evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(ring[i % len(ring)], evs[i])
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        qt_us = 1e3 * sum(a.elapsed_time(b) for a, b, _ in evs) / args.steps
        score_us = 1e3 * sum(b.elapsed_time(c) for _, b, c in evs) / args.steps
    log(f"timed {args.steps} steps in {elapsed * 1e3:.2f} ms ({mode}); "
        f"transform {qt_us:.2f} us, score {score_us:.2f} us per launch")

    ms_per_step = elapsed * 1e3 / args.steps
    pairs = w.pairs
    alg_bytes = w.algorithmic_bytes()
    achieved = alg_bytes / (score_us * 1e-6) / 1e9
    out = {
        "metric": METRIC,
        "value": pairs / (ms_per_step * 1e-3),
        "unit": "scores/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": score_dtype(kname),
        "data": "synthetic: seeded random codes, N(0,1) queries, Haar rotation, Gaussian projection",
        "config": {"workload": w.name, "P": w.P, "B": w.B, "S": w.S, "D": w.D, "C": w.C,
                   "layout": w.layout, "bits": w.bits},
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": measured_traffic(w, kname),
            "kernel": kname,
            "bytes_per_launch": alg_bytes,
            "avg_launch_us": score_us,
        },
        "achieved_hbm_gbs": achieved,
        "tq_score_us": score_us,
        "tq_query_transform_us": qt_us,
        "timing": mode,
        "step_gpu_us": step_gpu_us,
        "step_timing": ("wall clock between synchronisations around graph launches of K steps, each a "
                        "transform then its score"),
        "kernel_timing": ("HIP events on the kernels' stream around graph launches of back-to-back "
                          "transforms and back-to-back scores, a second pass of K steps"),
        "ring_sets": len(ring),
    }
    rec = trace_record(w, kname)
    if rec is not None:
        med = rec["per_dispatch_us"]["median"]
        out["roofline"]["trace"] = {"source": rec["profile"], "median_us": med, "avg_us": rec["per_dispatch_us"]["avg"],
                                    "frac_at_median": alg_bytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBS}
    f16_name = tq.tq_score_kernel_name(w.layout, w.bits, w.C, w.P, w.B, w.S, w.D, "mfma_f16")
    if args.kernel == "auto" and mode == "hipgraph" and f16_name is not None:
        # the single-pass f16 form of the same kernel, reported beside the fp32-accurate one
        _, _, f16_us = time_phased_graphs(w, ring, shared, "mfma_f16", args.steps)
        f16_gbs = alg_bytes / (f16_us * 1e-6) / 1e9
        out["f16_single_pass"] = {
            "kernel": f16_name, "tq_score_us": f16_us, "achieved_hbm_gbs": f16_gbs,
            "frac": f16_gbs / HBM_PEAK_GBS, "accuracy": "max |err| / (1 + |exact|) <= 2e-2 (tests/test_gpu_f16.py)",
            "scores_per_s_score_only": pairs / (f16_us * 1e-6),
        }
        log(f"f16 single pass ({f16_name}): {f16_us:.2f} us per tq_score launch ({f16_gbs:.0f} GB/s)")
    if not args.no_stream_probe:
        tile = (w.B, w.S, w.D) if (w.layout == "unpacked" and w.P == 1 and w.B <= 32 and w.D in (64, 128, 256)) else None
        probes = stream_probes(device, w.key_bytes(), w.score_bytes(), args.steps, tile)
        rw = probes["read_write"]
        probes["tq_score_time_over_read_write"] = score_us / rw["us"]
        if tile:
            probes["tq_score_time_over_tile"] = score_us / probes["tile"]["us"]
        out["stream_probes"] = probes
        log(f"probes: read {probes['read']['bytes'] / 1e6:.2f} MB in {probes['read']['us']:.2f} us, "
            f"write {probes['write']['bytes'] / 1e6:.2f} MB in {probes['write']['us']:.2f} us, "
            f"read-then-write {rw['us']:.2f} us ({rw['GB_s']:.0f} GB/s); tq_score takes "
            f"{probes['tq_score_time_over_read_write']:.2f}x the read-then-write probe")
        if tile:
            log(f"tile-pattern probe (the scorer's loads and stores, no arithmetic): {probes['tile']['us']:.2f} us; "
                f"tq_score takes {probes['tq_score_time_over_tile']:.2f}x it")
        probe = stream_probe(device, alg_bytes)
        probe["tq_score_frac_of_probe"] = achieved / probe["GB_s"]
        out["stream_probe"] = probe
        log(f"copy probe: {probe['bytes'] / 1e6:.1f} MB copied in {probe['us']:.2f} us ({probe['GB_s']:.0f} GB/s); "
            f"tq_score at {probe['tq_score_frac_of_probe']:.2f} of it")
    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline")
        out["cpu_baseline"] = cpu_baseline(w, host, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
