"""Benchmark of the Binade hot path on one MI355X.

Workload: the Llama-3.2-3B-shaped linear stack (28 layers x {q, o 3072x3072;
k, v 1024x3072; gate, up 8192x3072; down 3072x8192}; bf16 N(0, 0.02) with
0.1% outliers x20; seeds 1000 + tensor index). One step = format 2 -> R4
decode of all 196 tensors, then the batch-1 R4 GEMV of every tensor with an
N(0, 1) bf16 input of its width. Inputs and planes are resident in HBM before
the timed region; every kernel is timed with HIP events on its stream.

Before timing, parity is checked (and the run refuses to time if it fails):
every tensor's device decode unpacks to its original bits and its R4 GEMV
equals the bf16-weight twin bit for bit; the first layer's R4 planes equal
the oracle's byte for byte and sampled GEMV rows equal the oracle's replay.

    python bench.py [--gpus 1] [--steps 10] [--warmup 2]

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import subprocess
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from decode_gemv_tensor_amd import binade as B  # noqa: E402
from decode_gemv_tensor_amd import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemv_bytes(r4: B.R4Tensor) -> int:
    """Algorithmic bytes of one R4 GEMV: sign/mantissa + nibbles + escape
    entries + escape prefixes + x (bf16) + y (fp32)."""
    n, k = r4.rows, r4.cols
    return n * k + n * k // 2 + 4 * r4.n_esc + 4 * r4.esc_pre.numel() + 2 * k + 4 * n


def gemv_b_total(tensors) -> int:
    return sum(gemv_bytes(t["r4"]) for t in tensors)


def twin_bytes(n: int, k: int) -> int:
    return 2 * n * k + 2 * k + 4 * n


def decode_bytes(p: B.RicePlanes) -> int:
    """Algorithmic bytes of one format 2 -> R4 decode: the unary and
    remainder bits, anchors and escape prefixes read; nibbles and escape
    entries written. The sign/mantissa plane is not touched."""
    n = p.rows * p.cols
    unary = 4 * ((p.unary_bits + 31) // 32)
    rem = 4 * ((n * p.k + 31) // 32)
    chunks = p.anchor.numel()
    return unary + rem + 12 * chunks + n // 2 + 4 * p.n_esc


class Timer:
    """Pairs of HIP events recorded on one stream."""

    def __init__(self, stream):
        self.stream = stream
        self.pairs: dict[str, list] = {}

    def start(self):
        e = torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        return e

    def stop(self, key, e0):
        e1 = torch.cuda.Event(enable_timing=True)
        e1.record(self.stream)
        self.pairs.setdefault(key, []).append((e0, e1))
        return e1

    def add(self, key, e0, e1):
        """Another interval between two events already recorded."""
        self.pairs.setdefault(key, []).append((e0, e1))

    def total_ms(self, key):
        return sum(a.elapsed_time(b) for a, b in self.pairs.get(key, []))

    def count(self, key):
        return len(self.pairs.get(key, []))

    def spread_us(self, key):
        """p10 / median / p90 of the single intervals, in us."""
        v = [a.elapsed_time(b) * 1e3 for a, b in self.pairs.get(key, [])]
        return {k: round(x, 3) for k, x in spread(v).items()}


def spread(v) -> dict:
    v = sorted(v)
    if not v:
        return {}
    at = lambda q: v[min(len(v) - 1, int(round(q * (len(v) - 1))))]
    return {"p10": at(0.1), "median": at(0.5), "p90": at(0.9)}


def host_cpu() -> tuple[int, dict]:
    """Threads the CPU baseline may use -- this process's CPU affinity, at
    most 16 (one GPU's share of the host) -- and what the host reports."""
    aff = len(os.sched_getaffinity(0))
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return max(1, min(16, aff)), {"os_cpu_count": os.cpu_count(), "affinity_cpus": aff,
                                  "model": model}


def oracle_rate(items, fn, threads: int, min_s: float):
    """Runs fn(item) over `items` (cycling) on `threads` host threads until
    min_s seconds have passed; returns (sum of the values fn returns, seconds).
    The oracle is a C library called through ctypes, which releases the GIL,
    and it keeps no global state, so items run truly in parallel."""
    import threading
    lock = threading.Lock()
    state = {"i": 0, "done": 0.0}
    t0 = time.perf_counter()

    def worker():
        while time.perf_counter() - t0 < min_s:
            with lock:
                it = items[state["i"] % len(items)]
                state["i"] += 1
            v = fn(it)
            with lock:
                state["done"] += v

    ts = [threading.Thread(target=worker) for _ in range(threads)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    return state["done"], time.perf_counter() - t0


def cpu_baseline(tensors, host_bits, xs, log_fn) -> dict:
    """The oracle timed on this host: its fp32-order GEMV replay over the
    stack tensors (the metric's unit, GB/s of the R4 GEMV's bytes) and its
    format 2 -> R4 decode (bit-by-bit Rice decode, then the R4 layout) over
    row blocks of one gate tensor, each on one thread and on every thread
    this process may use. Results do not depend on the thread count: the
    items are independent tensors or row blocks."""
    import oracle  # test infrastructure: cpu baseline only
    cores, host = host_cpu()
    gemv_items = []
    for t in tensors:
        wn = host_bits[t["spec"].name].view(torch.int16).numpy().view(np.uint16)
        xb = xs[t["spec"].cols].cpu().view(torch.int16).numpy().view(np.uint16)
        gemv_items.append((wn, xb, gemv_bytes(t["r4"])))

    def gemv_one(it):
        oracle.gemv_replay(it[0], it[1])
        return it[2]

    gate = next(t for t in tensors if t["spec"].name.endswith(".gate"))
    gw = host_bits[gate["spec"].name].view(torch.int16).numpy().view(np.uint16)
    blocks = [np.ascontiguousarray(gw[r:r + 256]) for r in range(0, gw.shape[0], 256)]

    def pack(b):
        tab = oracle.build_table(b)
        return tab, oracle.pack_rice(b, tab)

    with ThreadPoolExecutor(max_workers=cores) as ex:
        packed = list(ex.map(pack, blocks))

    def dec_bytes_of(pk):
        n = pk["rows"] * pk["cols"]
        return (4 * ((pk["unary_bits"] + 31) // 32) + 4 * ((n * pk["k"] + 31) // 32)
                + 12 * pk["anchor"].size + n // 2 + 4 * pk["n_esc"])

    dec_items = [(tab, pk, pk["rows"] * pk["cols"], dec_bytes_of(pk)) for tab, pk in packed]

    def dec_one(it):
        bits = oracle.rice_decode(it[1])
        oracle.make_r4(bits, it[0])
        return it[2]

    res = {}
    for name, items, fn, secs in (("gemv", gemv_items, gemv_one, 5.0), ("decode", dec_items, dec_one, 4.0)):
        for th in (1, cores):
            done, el = oracle_rate(items, fn, th, secs)
            res[(name, th)] = (done, el)
            log_fn(f"cpu baseline {name} x{th}: {done / el / 1e9:.3f} G/s over {el:.1f}s")
    g1, gn = res[("gemv", 1)], res[("gemv", cores)]
    d1, dn = res[("decode", 1)], res[("decode", cores)]
    sym_b = sum(it[3] for it in dec_items) / sum(it[2] for it in dec_items)   # bytes per symbol
    return {"value": round(gn[0] / gn[1] / 1e9, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": (f"oracle fp32-order GEMV replay (C, one tensor per thread) cycling over the "
                       f"{len(gemv_items)} stack tensors for {gn[1]:.1f} s on {cores} threads; bytes "
                       "counted as the R4 GEMV's"),
            "single_thread_GBs": round(g1[0] / g1[1] / 1e9, 3),
            "decode": {"kernel": "rice_to_r4",
                       "gsym_per_s": round(dn[0] / dn[1] / 1e9, 4),
                       "GBs": round(dn[0] * sym_b / dn[1] / 1e9, 4),
                       "single_thread_gsym_per_s": round(d1[0] / d1[1] / 1e9, 4),
                       "cores": cores,
                       "sample": (f"oracle bit-by-bit Rice decode + R4 layout over {len(dec_items)} "
                                  f"row blocks (256 x {gw.shape[1]}) of {gate['spec'].name}, "
                                  f"{dn[1]:.1f} s on {cores} threads")},
            "host": host}


MFMA_BF16_PEAK_TFS = 2500.0   # MI355X dense bf16 matrix peak

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "decode_gemv_tensor_amd", "csrc")
# sources whose text decides each kernel's memory traffic
KERNEL_SOURCES = {"rice_to_r4": ["rice_to_r4.hip", "device_common.h"],
                  "r4_gemv": ["gemv.hip", "device_common.h"]}


def source_sha(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE runs
    (profiles/traffic.json), if they were taken on this kernel's current
    source; else None."""
    path = os.path.join(HERE, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != source_sha(kernel):
        return None
    return rec.get("bytes_per_launch")


def copy_probe(dev) -> None:
    """A plain elementwise copy of 1 GiB (fp32 x 1), five times: the counter
    runs read FETCH_SIZE and WRITE_SIZE on it to scale the kernels' readings."""
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    log(f"copy probe: 5 x {n * 4} bytes read and written")


def graph_replays_ms(stream, body, reps: int = 15) -> list:
    """`body` captured once in a HIP graph and replayed `reps` times; the
    duration of each replay in ms (events recorded on the stream the graph
    replays on)."""
    with torch.cuda.stream(stream):
        body()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        body()
    with torch.cuda.stream(stream):
        g.replay()
    torch.cuda.synchronize()
    out = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1))
    del g
    return out


def graph_time_ms(stream, body, reps: int = 15) -> float:
    """Median replay of `body` captured in a HIP graph, in ms."""
    return spread(graph_replays_ms(stream, body, reps))["median"]


def r4_bytes(r4: B.R4Tensor) -> int:
    return r4.rows * r4.cols * 3 // 2 + 4 * r4.n_esc + 4 * r4.esc_pre.numel()


ROTATE_BYTES = 1 << 30   # working set per timed GEMM replay: well past the 256 MiB last-level cache


def r4_replica(r4: B.R4Tensor) -> B.R4Tensor:
    return B.R4Tensor(r4.rows, r4.cols, r4.lut, r4.sm.clone(), r4.nib.clone(),
                      r4.esc_pre.clone(), r4.esc.clone(), r4.n_esc)


def measure_gemm(dev, stream) -> dict:
    """Prompt GEMM on the 12B-class FFN shapes (R4 and its bf16 twin).

    Each HIP-graph replay runs one launch on each of several weight copies, so
    that the replay reads at least 1 GiB of weights and no launch finds its
    weights in the last-level cache; the median replay is reported with p10 /
    p90, and cache-hot figures (one copy launched ten times) beside it.
    torch.nn.functional.linear on the same bf16 weights (bf16 output, the
    vendor BLAS) is timed the same way as an outside reference; it is not
    bit-identical to the path. Outputs of R4 and twin are checked equal."""
    out = {}
    for spec in synth.gemma_12b_ffn()[1:]:   # up 15360x3840, down 3840x15360
        w = synth.normal_bf16(spec, device=dev)
        r4 = B.rice_to_r4(B.pack_rice(w.cpu()).to(dev))
        N, K = spec.rows, spec.cols
        n_r4 = -(-ROTATE_BYTES // r4.nbytes())
        n_bf = -(-ROTATE_BYTES // (2 * N * K))
        r4s = [r4] + [r4_replica(r4) for _ in range(n_r4 - 1)]
        wts = [w] + [w.clone() for _ in range(n_bf - 1)]
        for M in synth.GEMM_ROWS:
            x = synth.vector_bf16(K, 500 + M, device=dev, count=M)
            y = torch.empty(M, N, dtype=torch.float32, device=dev)
            y2 = torch.empty_like(y)
            ws = torch.empty(B.gemm_workspace_bytes(M, N, K), dtype=torch.uint8, device=dev)
            reps = 5 if M >= 2048 else 15

            def r4_rot():
                for t in r4s:
                    B.r4_gemm(t, x, y=y, stream=stream, workspace=ws)

            def bf_rot():
                for t in wts:
                    B.bf16_gemm(t, x, y=y2, stream=stream, workspace=ws)

            def lin_rot():
                for t in wts:
                    torch.nn.functional.linear(x, t)

            def r4_hot():
                for _ in range(10):
                    B.r4_gemm(r4, x, y=y, stream=stream, workspace=ws)

            def bf_hot():
                for _ in range(10):
                    B.bf16_gemm(w, x, y=y2, stream=stream, workspace=ws)

            def per_launch(body, n):
                v = graph_replays_ms(stream, body, reps)
                return {k: x_ / n for k, x_ in spread(v).items()}

            tr = per_launch(r4_rot, len(r4s))
            tt = per_launch(bf_rot, len(wts))
            tl = per_launch(lin_rot, len(wts))
            hr = per_launch(r4_hot, 10)
            ht = per_launch(bf_hot, 10)
            torch.cuda.synchronize()
            if not torch.equal(y.view(torch.int32), y2.view(torch.int32)):
                raise SystemExit(f"parity gate: R4 GEMM differs from its twin ({N}x{K}, M={M})")
            fl = 2.0 * M * N * K
            nbytes = r4_bytes(r4) + 2 * M * K + 4 * M * N
            m = tr["median"]
            us = lambda d: {k: round(v * 1e3, 2) for k, v in d.items()}
            out[f"{N}x{K}_M{M}"] = {
                "r4_us": round(m * 1e3, 2), "r4_us_spread": us(tr),
                "r4_TFLOPs": round(fl / m / 1e9, 1),
                "mfma_frac": round(fl / m / 1e9 / MFMA_BF16_PEAK_TFS, 4),
                "r4_GBs": round(nbytes / m / 1e6, 1),
                "bf16_twin_us": round(tt["median"] * 1e3, 2), "bf16_twin_us_spread": us(tt),
                "speedup_vs_twin": round(tt["median"] / m, 3),
                "torch_linear_bf16_us": round(tl["median"] * 1e3, 2),
                "speedup_vs_torch_linear": round(tl["median"] / m, 3),
                "cache_hot": {"r4_us": round(hr["median"] * 1e3, 2),
                              "bf16_twin_us": round(ht["median"] * 1e3, 2)},
                "weight_copies": {"r4": len(r4s), "bf16": len(wts)}}
        del w, r4, r4s, wts
        torch.cuda.empty_cache()
    return out


def f1_decode_bytes(p: B.F1Planes) -> int:
    """Algorithmic bytes of one format 1 -> R4 decode: codes, width bytes,
    escape bytes and the per-chunk index (anchor, two prefixes) read;
    nibbles and R4 side-list entries written. sm is not touched."""
    n = p.rows * p.cols
    return ((p.code_bits + 7) // 8 + p.width.numel() + p.n_f1esc + 16 * p.anchor.numel()
            + n // 2 + 4 * p.n_esc)


def planes_replica(p: B.RicePlanes, dev) -> B.RicePlanes:
    """Device copies of a format 2 tensor's planes (the sm plane shared)."""
    return B.RicePlanes(rows=p.rows, cols=p.cols, table=p.table, sm=p.sm, unary=p.unary.clone(),
                        rem=None if p.rem is None else p.rem.clone(), anchor=p.anchor.clone(),
                        esc_pre=p.esc_pre.clone(), unary_bits=p.unary_bits, n_esc=p.n_esc)


def measure_configs(dev, stream) -> dict:
    """The single 1024 x 1024 tensor (table, pack, decode, GEMV), and the
    12B-class shapes: bulk decode of the 262144 x 256 tensor (67,108,864
    symbols) and the batch-1 GEMV of 15360 x 3840 and 3840 x 15360. Each
    timed HIP-graph replay works on copies whose total is >= 1 GiB (decode:
    planes in, nibbles and escapes out; GEMV: weights), so no launch finds its
    data in the last-level cache; medians of 15 replays, per launch."""
    out = {}
    # ---- single 1024 x 1024 tensor (launch-bound; reported, not a roofline)
    sp = synth.single_1024()[0]
    w = synth.normal_bf16(sp, device=dev)
    wh = w.cpu()
    t0 = time.perf_counter()
    table = B.build_table(wh)
    t1 = time.perf_counter()
    planes = B.pack_rice(wh, table)
    t2 = time.perf_counter()
    dp = planes.to(dev)
    r4 = B.rice_to_r4(dp)
    x = synth.vector_bf16(sp.cols, 1, device=dev)
    y = torch.empty(sp.rows, dtype=torch.float32, device=dev)
    tdec = graph_time_ms(stream, lambda: B.rice_to_r4(dp, stream=stream, out=r4))
    tgv = graph_time_ms(stream, lambda: B.r4_gemv(r4, x, y=y, stream=stream))
    ttw = graph_time_ms(stream, lambda: B.bf16_gemv(w, x, y=y, stream=stream))
    torch.cuda.synchronize()
    if not torch.equal(B.unpack(r4).view(torch.int16), w.view(torch.int16)):
        raise SystemExit("parity gate: 1024 x 1024 unpack differs")
    out["single_1024x1024"] = {
        "host_table_ms": round((t1 - t0) * 1e3, 3), "host_pack_ms": round((t2 - t1) * 1e3, 3),
        "format2_bits_per_weight": round(planes.bits_per_weight(), 4),
        "r4_bits_per_weight": round(r4.bits_per_weight(), 4),
        "decode_us": round(tdec * 1e3, 2), "gemv_us": round(tgv * 1e3, 2),
        "bf16_twin_gemv_us": round(ttw * 1e3, 2),
        "note": "1.5 MB of weights: one launch is bound by launch and cache latency, not HBM"}
    # ---- 64M-symbol bulk decode
    sp = synth.embedding_64m()
    w = synth.normal_bf16(sp, device=dev)
    planes = B.pack_rice(w.cpu())
    dp = planes.to(dev)
    ref = B.rice_to_r4(dp)
    per_copy = decode_bytes(dp) + dp.rows * dp.cols   # + the sm plane it leaves alone
    n = max(2, -(-ROTATE_BYTES // per_copy))
    copies = [dp] + [planes_replica(dp, dev) for _ in range(n - 1)]
    outs = [ref] + [B.R4Tensor(dp.rows, dp.cols, bytes(16), dp.sm, torch.empty_like(ref.nib),
                               dp.esc_pre, torch.empty_like(ref.esc), dp.n_esc) for _ in range(n - 1)]
    status = torch.zeros(1, dtype=torch.int32, device=dev)

    def dec_rot():
        for p_, o_ in zip(copies, outs):
            B.rice_to_r4(p_, status=status, stream=stream, out=o_)

    v = spread(graph_replays_ms(stream, dec_rot))
    torch.cuda.synchronize()
    if int(status.item()) != 0 or not all(torch.equal(o_.nib, ref.nib) for o_ in outs):
        raise SystemExit("parity gate: bulk decode copies differ")
    if not torch.equal(B.unpack(ref).view(torch.int16), w.view(torch.int16)):
        raise SystemExit("parity gate: bulk decode unpack differs")
    t = v["median"] / n
    syms = dp.rows * dp.cols
    ach = decode_bytes(dp) / (t * 1e-3) / 1e9
    out["bulk_decode_262144x256"] = {
        "symbols": syms, "us_per_launch": round(t * 1e3, 2),
        "us_spread": {k: round(x_ / n * 1e3, 2) for k, x_ in v.items()},
        "gsym_per_s": round(syms / (t * 1e-3) / 1e9, 1), "GBs": round(ach, 1),
        "frac_of_hbm_peak": round(ach / HBM_PEAK_GBS, 4), "copies": n,
        "bytes_per_launch": decode_bytes(dp)}
    del copies, outs, ref, dp, w
    torch.cuda.empty_cache()
    # ---- format 1 -> R4 (the second file format) on the 64M tensor and a
    # 12B FFN weight
    for sp in (synth.embedding_64m(), synth.gemma_12b_ffn()[1]):
        w = synth.normal_bf16(sp, device=dev)
        f1 = B.pack_f1(w.cpu())
        dp = f1.to(dev)
        ref = B.f1_to_r4(dp)
        per_copy = f1_decode_bytes(dp) + dp.rows * dp.cols
        n = max(2, -(-ROTATE_BYTES // per_copy))
        copies = [dp] + [B.F1Planes(**{**dp.__dict__, "codes": dp.codes.clone(),
                                       "width": dp.width.clone(), "esc_rank": dp.esc_rank.clone(),
                                       "anchor": dp.anchor.clone(), "f1_pre": dp.f1_pre.clone()})
                         for _ in range(n - 1)]
        outs = [ref] + [B.R4Tensor(dp.rows, dp.cols, bytes(16), dp.sm, torch.empty_like(ref.nib),
                                   dp.esc_pre, torch.empty_like(ref.esc), dp.n_esc) for _ in range(n - 1)]
        status = torch.zeros(1, dtype=torch.int32, device=dev)

        def f1_rot():
            for p_, o_ in zip(copies, outs):
                B.f1_to_r4(p_, status=status, stream=stream, out=o_)

        v = spread(graph_replays_ms(stream, f1_rot))
        torch.cuda.synchronize()
        if int(status.item()) != 0 or not all(torch.equal(o_.nib, ref.nib) for o_ in outs):
            raise SystemExit("parity gate: format 1 decode copies differ")
        if not torch.equal(B.unpack(ref).view(torch.int16), w.view(torch.int16)):
            raise SystemExit("parity gate: format 1 decode unpack differs")
        t = v["median"] / n
        syms = dp.rows * dp.cols
        ach = f1_decode_bytes(dp) / (t * 1e-3) / 1e9
        out[f"format1_decode_{dp.rows}x{dp.cols}"] = {
            "symbols": syms, "format1_bits_per_weight": round(f1.bits_per_weight(), 4),
            "us_per_launch": round(t * 1e3, 2),
            "us_spread": {k: round(x_ / n * 1e3, 2) for k, x_ in v.items()},
            "gsym_per_s": round(syms / (t * 1e-3) / 1e9, 1), "GBs": round(ach, 1),
            "frac_of_hbm_peak": round(ach / HBM_PEAK_GBS, 4), "copies": n,
            "bytes_per_launch": f1_decode_bytes(dp)}
        del copies, outs, ref, dp, w, f1
        torch.cuda.empty_cache()
    # ---- the Huffman comparison decoder on the 64M-symbol tensor (the pages'
    # own timing workload: an embedding-like 64M-symbol sample)
    sp = synth.embedding_64m()
    w = synth.normal_bf16(sp)
    hp = B.pack_huff(w)
    hd = hp.to(dev)
    n_copy = max(2, -(-ROTATE_BYTES // (hp.n * 3)))
    copies = [hd] + [B.HuffPlanes(hd.n, hd.len, hd.sm.clone(), hd.stream.clone(), hd.stream_bytes,
                                  hd.block_len.clone(), hd.group_off.clone())
                     for _ in range(n_copy - 1)]
    hws = torch.empty(int(B.lib().binade_huff_workspace_bytes()), dtype=torch.uint8, device=dev)
    houts = [torch.empty(hp.n, dtype=torch.bfloat16, device=dev) for _ in range(2)]
    hstatus = torch.zeros(1, dtype=torch.int32, device=dev)

    def huff_rot():
        for i, c_ in enumerate(copies):
            B.huff_decode(c_, out=houts[i & 1], status=hstatus, workspace=hws, stream=stream)

    v = spread(graph_replays_ms(stream, huff_rot))
    torch.cuda.synchronize()
    if int(hstatus.item()) != 0 or not torch.equal(houts[0].cpu().view(torch.int16),
                                                   w.reshape(-1).view(torch.int16)):
        raise SystemExit("parity gate: Huffman decode differs from the weights")
    t = v["median"] / n_copy
    hbytes = hp.stream_bytes + hp.block_len.numel() + 8 * hp.group_off.numel() + hp.n + 2 * hp.n
    gb = hbytes / (t * 1e-3) / 1e9
    out["huffman_decode_262144x256"] = {
        "symbols": hp.n, "huffman_bits_per_weight": round(hp.bits_per_weight(), 4),
        "us_per_launch": round(t * 1e3, 2),
        "us_spread": {k: round(x_ / n_copy * 1e3, 2) for k, x_ in v.items()},
        "gsym_per_s": round(hp.n / (t * 1e-3) / 1e9, 1), "GBs": round(gb, 1),
        "frac_of_hbm_peak": round(gb / HBM_PEAK_GBS, 4), "bytes_per_launch": hbytes,
        "copies": n_copy,
        "pages_context_ms": {"A100": 0.47, "RTX 4090": 0.19},
        "note": "bytes: stream + 8-bit block lengths + group offsets + sm read, bf16 written "
                "(the comparison decoder outputs whole bf16 weights; Rice->R4 writes 4-bit ranks)"}
    del copies, hd, houts, w, hp
    torch.cuda.empty_cache()
    # ---- the table and the format 2 pack on the device
    for sp in [synth.gemma_12b_ffn()[0], synth.embedding_64m()]:
        w = synth.normal_bf16(sp, device=dev)
        rows, cols = sp.rows, sp.cols
        n_copy = max(2, -(-ROTATE_BYTES // (2 * rows * cols)))
        wcopies = [w] + [w.clone() for _ in range(n_copy - 1)]
        ref = B.pack_rice_gpu(w)          # table on the device, planes, status-free run
        table = ref.table
        wsb = int(B.lib().binade_pack_gpu_workspace_bytes(rows, cols))
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        dtab = torch.empty(ctypes.sizeof(B.Table), dtype=torch.uint8, device=dev)
        outp = B.RicePlanes(rows, cols, table, torch.empty_like(ref.sm), torch.empty_like(ref.unary),
                            None if ref.rem is None else torch.empty_like(ref.rem),
                            torch.empty_like(ref.anchor), torch.empty_like(ref.esc_pre), 0, 0)
        d = outp.desc()
        st = ctypes.c_void_p(stream.cuda_stream)

        def table_rot():
            for w_ in wcopies:
                B._call("binade_build_table_gpu", B._ptr(w_), w_.numel(), B._ptr(ws), B._ptr(dtab), st)

        def pack_rot():
            for w_ in wcopies:
                B._call("binade_pack_rice_gpu", B._ptr(w_), rows, cols, ctypes.byref(table),
                        ctypes.byref(d), B._ptr(ws), None, st)

        tt = spread(graph_replays_ms(stream, table_rot))["median"] / n_copy
        tp = spread(graph_replays_ms(stream, pack_rot))["median"] / n_copy
        torch.cuda.synchronize()
        if not (torch.equal(outp.unary, ref.unary) and torch.equal(outp.sm, ref.sm)
                and torch.equal(outp.anchor, ref.anchor)):
            raise SystemExit("parity gate: device pack replays differ")
        host = B.pack_rice(w.cpu())
        if not (torch.equal(host.unary, ref.unary.cpu()) and torch.equal(host.sm, ref.sm.cpu())):
            raise SystemExit("parity gate: device pack differs from the host pack")
        t0 = time.perf_counter()
        B.pack_rice(w.cpu())
        host_ms = (time.perf_counter() - t0) * 1e3
        planes_b = sum(ref.nbytes().values())
        pack_b = 2 * rows * cols + planes_b        # bf16 read once + planes written
        gbp = pack_b / (tp * 1e-3) / 1e9
        out[f"gpu_table_and_pack_{rows}x{cols}"] = {
            "table_us": round(tt * 1e3, 2), "pack_us": round(tp * 1e3, 2),
            "table_GBs_read": round(2 * rows * cols / (tt * 1e-3) / 1e9, 1),
            "pack_GBs": round(gbp, 1), "pack_frac_of_hbm_peak": round(gbp / HBM_PEAK_GBS, 4),
            "bytes_per_pack": pack_b, "host_pack_ms_one_thread": round(host_ms, 1),
            "speedup_vs_host_pack": round(host_ms / ((tt + tp)), 1), "copies": n_copy,
            "note": "pack bytes: the bf16 weights read once plus the planes written; the kernels "
                    "read the weights twice (count, then write)"}
        del w, wcopies, ref, outp, ws
        torch.cuda.empty_cache()
    # ---- 12B FFN batch-1 GEMV
    for sp in synth.gemma_12b_ffn()[1:]:
        w = synth.normal_bf16(sp, device=dev)
        r4 = B.rice_to_r4(B.pack_rice(w.cpu()).to(dev))
        N, K = sp.rows, sp.cols
        x = synth.vector_bf16(K, 700 + N, device=dev)
        y = torch.empty(N, dtype=torch.float32, device=dev)
        y2 = torch.empty_like(y)
        n_r4 = -(-ROTATE_BYTES // r4.nbytes())
        n_bf = -(-ROTATE_BYTES // (2 * N * K))
        r4s = [r4] + [r4_replica(r4) for _ in range(n_r4 - 1)]
        wts = [w] + [w.clone() for _ in range(n_bf - 1)]

        def r4_rot():
            for t_ in r4s:
                B.r4_gemv(t_, x, y=y, stream=stream)

        def bf_rot():
            for t_ in wts:
                B.bf16_gemv(t_, x, y=y2, stream=stream)

        tr = spread(graph_replays_ms(stream, r4_rot))["median"] / len(r4s)
        tt = spread(graph_replays_ms(stream, bf_rot))["median"] / len(wts)
        torch.cuda.synchronize()
        if not torch.equal(y.view(torch.int32), y2.view(torch.int32)):
            raise SystemExit(f"parity gate: 12B GEMV differs from its twin ({N}x{K})")
        gb = gemv_bytes(r4) / (tr * 1e-3) / 1e9
        line = {
            "us_per_launch": round(tr * 1e3, 2), "GBs": round(gb, 1),
            "frac_of_hbm_peak": round(gb / HBM_PEAK_GBS, 4),
            "bf16_twin_us": round(tt * 1e3, 2), "speedup_vs_twin": round(tt / tr, 3),
            "copies": {"r4": len(r4s), "bf16": len(wts)}}
        # the decode step of m sequences: one launch reads W once for m rows
        small = {}
        for m in (2, 4, 8):
            xm = synth.vector_bf16(K, 800 + N + m, device=dev, count=m)
            ym = torch.empty(m, N, dtype=torch.float32, device=dev)
            ym2 = torch.empty_like(ym)

            def r4_rows_rot():
                for t_ in r4s:
                    B.r4_gemv_rows(t_, xm, y=ym, stream=stream)

            def bf_rows_rot():
                for t_ in wts:
                    B.bf16_gemv_rows(t_, xm, y=ym2, stream=stream)

            trm = spread(graph_replays_ms(stream, r4_rows_rot))["median"] / len(r4s)
            ttm = spread(graph_replays_ms(stream, bf_rows_rot))["median"] / len(wts)
            torch.cuda.synchronize()
            if not torch.equal(ym.view(torch.int32), ym2.view(torch.int32)):
                raise SystemExit(f"parity gate: {m}-row GEMV differs from its twin ({N}x{K})")
            if not torch.equal(ym[0].view(torch.int32),
                               B.r4_gemv(r4, xm[0].contiguous()).view(torch.int32)):
                raise SystemExit(f"parity gate: {m}-row GEMV row 0 differs from batch 1")
            bm = gemv_bytes(r4) + (m - 1) * (2 * K + 4 * N)
            gbm = bm / (trm * 1e-3) / 1e9
            small[f"m{m}"] = {
                "us_per_launch": round(trm * 1e3, 2), "GBs": round(gbm, 1),
                "frac_of_hbm_peak": round(gbm / HBM_PEAK_GBS, 4),
                "bf16_twin_us": round(ttm * 1e3, 2), "speedup_vs_twin": round(ttm / trm, 3),
                "speedup_vs_m_batch1_launches": round(m * tr / trm, 3)}
        line["small_batch_rows"] = small
        out[f"gemv_{N}x{K}"] = line
        del w, r4, r4s, wts
        torch.cuda.empty_cache()
    return out


def measure_moe(dev, stream) -> dict:
    """One gathered MoE step: 8 tokens x top-8 of 128 experts through gate,
    up (shared token input) and down (per-slot input) in R4 and bf16."""
    specs = synth.moe_layer()
    ws = [synth.normal_bf16(sp, device=dev) for sp in specs]
    r4s = [B.rice_to_r4(B.pack_rice(w.cpu()).to(dev)) for w in ws]
    E, T, k = synth.MOE_EXPERTS, synth.MOE_TOKENS, synth.MOE_TOP_K
    idx = synth.topk_indices(T, k, E, 3100, device=dev)
    xh = synth.vector_bf16(synth.MOE_HIDDEN, 3101, device=dev, count=T)
    xf = synth.vector_bf16(synth.MOE_FFN, 3102, device=dev, count=T * k)
    ins = [(xh, False), (xh, False), (xf, True)]
    ys = [torch.empty(T * k, sp.rows // E, dtype=torch.float32, device=dev) for sp in specs]
    ys2 = [torch.empty_like(y) for y in ys]

    def r4_step():
        for r4, (x, per), y in zip(r4s, ins, ys):
            B.r4_moe_gemv(r4, E, x, idx, x_per_slot=per, y=y, stream=stream)

    def twin_step():
        for w, (x, per), y in zip(ws, ins, ys2):
            B.bf16_moe_gemv(w, E, x, idx, x_per_slot=per, y=y, stream=stream)

    tr = graph_time_ms(stream, r4_step)
    tt = graph_time_ms(stream, twin_step)
    torch.cuda.synchronize()
    for y, y2 in zip(ys, ys2):
        if not torch.equal(y.view(torch.int32), y2.view(torch.int32)):
            raise SystemExit("parity gate: R4 MoE differs from its twin")
    used = int(torch.unique(idx).numel())
    nbytes = sum(r4_bytes(r4) * used // E for r4 in r4s)
    nbytes += 2 * (xh.numel() * 2 + xf.numel()) + 4 * sum(y.numel() for y in ys)
    # the whole layer with its epilogue: gate, up, silu*up (bf16), down on the
    # per-slot activations, router-weighted combine
    rw = synth.router_weights(T, k, 3103, device=dev).reshape(-1)
    h = torch.empty(T * k, synth.MOE_FFN, dtype=torch.bfloat16, device=dev)
    comb = torch.empty(T, synth.MOE_HIDDEN, dtype=torch.float32, device=dev)

    reps = 20   # launches per replay: a lone small launch is dominated by the replay's own cost

    def silu_only():
        for _ in range(reps):
            B.moe_silu_mul(ys[0], ys[1], h=h, stream=stream)

    def combine_only():
        for _ in range(reps):
            B.moe_combine(ys[2], rw, k, out=comb, stream=stream)

    def r4_layer():
        B.r4_moe_gemv(r4s[0], E, xh, idx, y=ys[0], stream=stream)
        B.r4_moe_gemv(r4s[1], E, xh, idx, y=ys[1], stream=stream)
        B.moe_silu_mul(ys[0], ys[1], h=h, stream=stream)
        B.r4_moe_gemv(r4s[2], E, h, idx, x_per_slot=True, y=ys[2], stream=stream)
        B.moe_combine(ys[2], rw, k, out=comb, stream=stream)

    t_silu = graph_time_ms(stream, silu_only) / reps
    t_comb = graph_time_ms(stream, combine_only) / reps
    t_layer = graph_time_ms(stream, r4_layer)
    torch.cuda.synchronize()
    return {"workload": "128 experts, gate/up 704x2816 and down 2816x704; 8 tokens x top-8",
            "unique_experts": used, "r4_us_per_step": round(tr * 1e3, 2),
            "r4_GBs": round(nbytes / tr / 1e6, 1), "bf16_twin_us_per_step": round(tt * 1e3, 2),
            "speedup_vs_twin": round(tt / tr, 3),
            "bytes": "unique experts' R4 bytes once + inputs + fp32 outputs",
            "epilogue": {"silu_mul_us": round(t_silu * 1e3, 2),
                         "combine_us": round(t_comb * 1e3, 2),
                         "r4_layer_us": round(t_layer * 1e3, 2),
                         "layer": "gate, up, silu*up -> bf16, down per slot, weighted top-8 "
                                  "combine; one HIP graph"}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--layers", type=int, default=synth.LLAMA_3B_LAYERS)
    ap.add_argument("--skip-cpu-baseline", action="store_true")
    ap.add_argument("--skip-twin", action="store_true")
    ap.add_argument("--skip-gemm", action="store_true")
    ap.add_argument("--skip-configs", action="store_true")
    ap.add_argument("--skip-moe", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run the 1 GiB copy used to scale memory counters")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: "
              "the library runs on a single GPU (no sharding across GPUs)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe:
        copy_probe(dev)
        return
    stream = torch.cuda.Stream()
    L = B.lib()

    # ------------------------------------------------------------ inputs
    t0 = time.time()
    specs = synth.llama32_3b_stack(args.layers)
    host_bits = {}

    def prepare(spec):
        w = synth.normal_bf16(spec, device=dev)
        wh = w.cpu()
        planes = B.pack_rice(wh)
        return spec, w, wh, planes

    with ThreadPoolExecutor(max_workers=16) as ex:
        prepared = list(ex.map(prepare, specs))
    tensors = []
    for spec, w, wh, planes in prepared:
        dplanes = planes.to(dev)
        nib = torch.empty(spec.rows * spec.cols // 2, dtype=torch.uint8, device=dev)
        esc = torch.empty(max(planes.n_esc, 1), dtype=torch.int32, device=dev)
        r4 = B.R4Tensor(spec.rows, spec.cols, bytes(16), dplanes.sm, nib,
                        dplanes.esc_pre, esc, planes.n_esc)
        if spec.name.startswith("L0.") or not args.skip_cpu_baseline:
            host_bits[spec.name] = wh
        tensors.append({"spec": spec, "w": w if not args.skip_twin else None,
                        "planes": dplanes, "r4": r4,
                        "y": torch.empty(spec.rows, dtype=torch.float32, device=dev)})
    xs = {k: synth.vector_bf16(k, 1 + k, device=dev) for k in sorted({s.cols for s in specs})}
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    log(f"setup {time.time() - t0:.1f}s: {len(tensors)} tensors")

    # pre-built C arguments: the timed loop calls the library directly.
    # Decode: the whole stack in one launch, from a plan written once and
    # kept in device memory. GEMV: 16 tensors per launch; per layer the
    # groups a decoder issues together -- q, k, v; o; gate, up; down -- one
    # launch each.
    n_t = len(tensors)
    plan = B.RicePlan([t["planes"] for t in tensors], outs=[t["r4"] for t in tensors])
    plan.run(status=status, stream=stream)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "device decode flagged corrupt planes"
    dec_in = (B.RiceDesc * n_t)(*[t["planes"].desc() for t in tensors])
    dec_out = (B.R4Desc * n_t)()
    for i, t in enumerate(tensors):
        dec_out[i].nib = t["r4"].nib.data_ptr()
        dec_out[i].esc = t["r4"].esc.data_ptr()
    plan_dev = ctypes.c_void_p(plan.dev.data_ptr())
    # the timed step takes the stack 16 tensors per launch (the kernel's
    # streaming rate over the whole stack); a second, untimed-by-the-step
    # schedule issues per layer what a decoder can issue together
    names = [t["spec"].name.split(".")[1] for t in tensors]
    layer_groups = []
    i = 0
    while i < n_t:
        g = [i]
        if names[i] == "q":
            g = [i, i + 1, i + 2]
        elif names[i] == "gate":
            g = [i, i + 1]
        layer_groups.append(g)
        i += len(g)
    stack_groups = [list(range(s0, min(s0 + 16, n_t))) for s0 in range(0, n_t, 16)]

    def make_args(groups):
        out = []
        for g in groups:
            ws = (B.R4Desc * len(g))(*[tensors[j]["r4"].desc() for j in g])
            xs_ = (ctypes.c_void_p * len(g))(*[xs[tensors[j]["spec"].cols].data_ptr() for j in g])
            ys_ = (ctypes.c_void_p * len(g))(*[tensors[j]["y"].data_ptr() for j in g])
            out.append((ws, xs_, ys_, len(g), sum(gemv_bytes(tensors[j]["r4"]) for j in g)))
        return out
    gemv_args = make_args(stack_groups)
    layer_args = make_args(layer_groups)
    sptr = ctypes.c_void_p(stream.cuda_stream)
    stat_p = ctypes.c_void_p(status.data_ptr())
    RD = ctypes.sizeof(B.RiceDesc)
    R4D = ctypes.sizeof(B.R4Desc)

    def decode():
        rc = L.binade_rice_to_r4_run(plan.host, plan_dev, stat_p, sptr)
        if rc:
            raise B.BinadeError("binade_rice_to_r4_run", rc)

    def decode_16(s0):
        # the batched call: 16 tensors per launch
        rc = L.binade_rice_to_r4_batch(ctypes.byref(dec_in, s0 * RD), ctypes.byref(dec_out, s0 * R4D),
                                       min(16, n_t - s0), stat_p, sptr)
        if rc:
            raise B.BinadeError("binade_rice_to_r4_batch", rc)

    def gemv(gi, args_list=None):
        ws, xs_, ys_, n, _ = (args_list or gemv_args)[gi]
        rc = L.binade_r4_gemv_batch(ws, xs_, ys_, n, B.F32, sptr)
        if rc:
            raise B.BinadeError("binade_r4_gemv_batch", rc)

    # ------------------------------------------------------------ parity gate
    t0 = time.time()
    with torch.cuda.stream(stream):
        for gi in range(len(gemv_args)):
            gemv(gi)
    torch.cuda.synchronize()
    for t in tensors:
        if t["w"] is not None:
            back = B.unpack(t["r4"], stream=stream)
            yt = B.bf16_gemv(t["w"], xs[t["spec"].cols], stream=stream)
            y1 = B.r4_gemv(t["r4"], xs[t["spec"].cols], stream=stream)
            torch.cuda.synchronize()
            if not torch.equal(back.view(torch.int16), t["w"].view(torch.int16)):
                raise SystemExit(f"parity gate: unpack differs for {t['spec'].name}")
            if not torch.equal(yt.view(torch.int32), t["y"].view(torch.int32)):
                raise SystemExit(f"parity gate: R4 GEMV differs from bf16 twin for {t['spec'].name}")
            if not torch.equal(y1.view(torch.int32), t["y"].view(torch.int32)):
                raise SystemExit(f"parity gate: batched GEMV differs from single for {t['spec'].name}")
    import oracle  # test infrastructure: parity gate and cpu baseline only
    for t in tensors[:7]:
        name = t["spec"].name
        wn = host_bits[name].view(torch.int16).numpy().view(np.uint16)
        ref = oracle.make_r4(wn, oracle.build_table(wn))
        if not np.array_equal(t["r4"].nib.cpu().numpy(), ref["nib"].reshape(-1)):
            raise SystemExit(f"parity gate: nibbles differ from the oracle for {name}")
        if ref["n_esc"] and not np.array_equal(
                t["r4"].esc[: ref["n_esc"]].cpu().numpy().view(np.uint32), ref["esc"]):
            raise SystemExit(f"parity gate: escapes differ from the oracle for {name}")
        rows = np.arange(0, wn.shape[0], 97)
        xb = xs[t["spec"].cols].cpu().view(torch.int16).numpy().view(np.uint16)
        yref = oracle.gemv_replay(wn[rows], xb)
        if not np.array_equal(t["y"].cpu().numpy()[rows].view(np.uint32), yref.view(np.uint32)):
            raise SystemExit(f"parity gate: GEMV rows differ from the oracle for {name}")
    log(f"parity gate passed ({time.time() - t0:.1f}s)")

    # ------------------------------------------------------------ timed
    timer = Timer(stream)
    for _ in range(args.warmup):
        with torch.cuda.stream(stream):
            decode()
            for gi in range(len(gemv_args)):
                gemv(gi)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    torch.cuda.synchronize()
    # One event between consecutive launches: launch i's interval runs from
    # the event before it to the event after it, so the intervals of a phase
    # add up to the phase and no launch waits behind a second event.
    with torch.cuda.stream(stream):
        for _ in range(args.steps):
            s0 = timer.start()
            decode()
            e = timer.stop("decode", s0)
            timer.add("decode_phase", s0, e)
            p1 = e
            for gi in range(len(gemv_args)):
                gemv(gi)
                e = timer.stop("gemv", e)
            timer.add("gemv_phase", p1, e)
            timer.add("step", s0, e)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    assert int(status.item()) == 0
    # the batched call over the same stack, 16 tensors per launch (outside
    # the step): what the single launch saves in ramp-up and tail per launch
    t16 = Timer(stream)
    with torch.cuda.stream(stream):
        for _ in range(3):
            e = t16.start()
            for s0_ in range(0, n_t, 16):
                decode_16(s0_)
                e = t16.stop("decode16", e)
    torch.cuda.synchronize()
    assert int(status.item()) == 0

    K = args.steps
    gemv_b = sum(gemv_bytes(t["r4"]) for t in tensors)
    dec_b = sum(decode_bytes(t["planes"]) for t in tensors)
    syms = sum(t["spec"].rows * t["spec"].cols for t in tensors)
    step_ms_avg = timer.total_ms("step") / K
    gemv_phase_ms = timer.total_ms("gemv_phase") / K
    dec_phase_ms = timer.total_ms("decode_phase") / K
    gemv_kernel_ms = timer.total_ms("gemv") / K
    dec_kernel_ms = timer.total_ms("decode") / K
    n_gemv_launch = len(gemv_args)
    n_dec_launch = 1
    gemv_ach = gemv_b / (gemv_kernel_ms * 1e-3) / 1e9      # GB/s over kernel time
    dec_ach = dec_b / (dec_kernel_ms * 1e-3) / 1e9
    value = gemv_b / (gemv_phase_ms * 1e-3) / 1e9           # whole GEMV phase

    # Per token, as a decoder loop would run it: each schedule captured once
    # in a HIP graph and replayed. The per-layer schedule, and one launch per
    # tensor on both sides of the bf16-twin comparison.
    def graph_ms(body):
        return graph_time_ms(stream, body)

    def layer_schedule():
        for gi in range(len(layer_args)):
            gemv(gi, layer_args)

    layer_ms = graph_ms(layer_schedule)
    sched = {"schedule": "per layer: q|k|v, o, gate|up, down (4 launches per layer), HIP graph",
             "launches": len(layer_args), "ms_per_token": round(layer_ms, 4),
             "GBs": round(gemv_b_total(tensors) / (layer_ms * 1e-3) / 1e9, 1)}
    twin = None
    if not args.skip_twin:
        def r4_single():
            for t in tensors:
                B.r4_gemv(t["r4"], xs[t["spec"].cols], y=t["y"], stream=stream)

        def bf16_single():
            for t in tensors:
                B.bf16_gemv(t["w"], xs[t["spec"].cols], y=t["y"], stream=stream)

        twin_args = []
        for g in stack_groups:
            n = len(g)
            twin_args.append((
                (ctypes.c_void_p * n)(*[tensors[j]["w"].data_ptr() for j in g]),
                (ctypes.c_int64 * n)(*[tensors[j]["spec"].rows for j in g]),
                (ctypes.c_int64 * n)(*[tensors[j]["spec"].cols for j in g]),
                (ctypes.c_void_p * n)(*[xs[tensors[j]["spec"].cols].data_ptr() for j in g]),
                (ctypes.c_void_p * n)(*[tensors[j]["y"].data_ptr() for j in g]), n))

        def r4_batched():
            for gi in range(len(gemv_args)):
                gemv(gi)

        def bf16_batched():
            for a in twin_args:
                rc = L.binade_bf16_gemv_batch(*a, B.F32, sptr)
                if rc:
                    raise B.BinadeError("binade_bf16_gemv_batch", rc)

        def torch_linear():
            for t in tensors:
                torch.nn.functional.linear(xs[t["spec"].cols].view(1, -1), t["w"])

        twin_b = sum(twin_bytes(t["spec"].rows, t["spec"].cols) for t in tensors)
        lin_ms = graph_ms(torch_linear)
        r4s_ms = graph_ms(r4_single)
        twin_ms = graph_ms(bf16_single)
        r4b_ms = graph_ms(r4_batched)
        twinb_ms = graph_ms(bf16_batched)
        twin = {"one_launch_per_tensor": {
                    "bf16_ms_per_token": round(twin_ms, 4), "r4_ms_per_token": round(r4s_ms, 4),
                    "speedup": round(twin_ms / r4s_ms, 4),
                    "bf16_GBs": round(twin_b / (twin_ms * 1e-3) / 1e9, 1)},
                "sixteen_tensors_per_launch": {
                    "bf16_ms_per_token": round(twinb_ms, 4), "r4_ms_per_token": round(r4b_ms, 4),
                    "speedup": round(twinb_ms / r4b_ms, 4),
                    "bf16_GBs": round(twin_b / (twinb_ms * 1e-3) / 1e9, 1),
                    "r4_GBs": round(gemv_b_total(tensors) / (r4b_ms * 1e-3) / 1e9, 1)},
                "torch_linear_bf16": {
                    "ms_per_token": round(lin_ms, 4),
                    "GBs": round(twin_b / (lin_ms * 1e-3) / 1e9, 1),
                    "r4_sixteen_per_launch_speedup": round(lin_ms / r4b_ms, 4),
                    "note": "nn.functional.linear, bf16 output, one call per tensor; an outside "
                            "reference, not bit-identical"},
                "note": "HIP-graph replays of the same schedule, median of 15; bytes per side "
                        "are that side's own weight bytes"}

    # ------------------------------------------------------------ GEMM, MoE
    # (the other rows of the path, reported beside the step; not in `value`)
    configs = None if args.skip_configs else measure_configs(dev, stream)
    gemm = None if args.skip_gemm else measure_gemm(dev, stream)
    moe = None if args.skip_moe else measure_moe(dev, stream)

    # ------------------------------------------------------------ CPU oracle
    cpu = None
    if not args.skip_cpu_baseline:
        cpu = cpu_baseline(tensors, host_bits, xs, log)

    dominant = "gemv" if gemv_kernel_ms >= dec_kernel_ms else "rice_to_r4"
    roof_g = {"kernel": "r4_gemv", "bound": "hbm", "achieved": round(gemv_ach, 1),
              "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gemv_ach / HBM_PEAK_GBS, 4),
              "traffic": measured_traffic("r4_gemv"), "launches_per_step": n_gemv_launch,
              "avg_launch_us": round(gemv_kernel_ms * 1e3 / n_gemv_launch, 3),
              "launch_us_spread": timer.spread_us("gemv"),
              "bytes_per_launch": gemv_b // n_gemv_launch}
    roof_d = {"kernel": "rice_to_r4", "bound": "hbm", "achieved": round(dec_ach, 1),
              "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dec_ach / HBM_PEAK_GBS, 4),
              "traffic": measured_traffic("rice_to_r4"), "launches_per_step": n_dec_launch,
              "avg_launch_us": round(dec_kernel_ms * 1e3 / n_dec_launch, 3),
              "launch_us_spread": timer.spread_us("decode"),
              "bytes_per_launch": dec_b // n_dec_launch,
              "gsym_per_s": round(syms / (dec_kernel_ms * 1e-3) / 1e9, 1)}
    out = {
        "metric": "R4 GEMV effective GB/s and % of HBM peak; Rice->R4 Gsym/s; GEMM TFLOP/s",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms_avg, 4),
        "step_us_spread": timer.spread_us("step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 weights (R4), fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": f"llama-3.2-3b linear stack, {args.layers} layers x 7 tensors: "
                               "Rice->R4 decode + batch-1 R4 GEMV per tensor",
                   "launches": "decode: the whole stack in one launch (a plan in device memory); "
                               "GEMV 16 tensors per launch",
                   "tensors": len(tensors), "weights": syms,
                   "r4_bytes": sum(t["r4"].nbytes() for t in tensors),
                   "parallelism": "single GPU"},
        "gemv_frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "rice_to_r4_gsym_s": round(syms / (dec_phase_ms * 1e-3) / 1e9, 1),
        "roofline": roof_g if dominant == "gemv" else roof_d,
        "roofline_other": roof_d if dominant == "gemv" else roof_g,
        "bf16_twin": twin,
        "gemv_per_layer_schedule": sched,
        "decode_16_per_launch": {
            "launches": t16.count("decode16") // 3,
            "avg_launch_us": round(t16.total_ms("decode16") * 1e3 / t16.count("decode16"), 3),
            "ms_per_stack": round(t16.total_ms("decode16") / 3, 4),
            "frac": round(dec_b / (t16.total_ms("decode16") / 3 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "note": "binade_rice_to_r4_batch over the same stack, 16 tensors per launch, "
                    "outside the step"},
        "other_configs": configs,
        "prompt_gemm": gemm,
        "moe_gather": moe,
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
