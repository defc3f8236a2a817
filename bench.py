#!/usr/bin/env python3
"""Benchmark of the W4A16 small-M linear layer on one MI355X.

One step = one decode token's weight sweep of a 64-layer 27B-class decoder:
64 layers x (fused QKV 5120->7168, o_proj 5120->5120, fused gate_up
5120->34816, down 17408->5120), 256 distinct packed weight buffers (11.00 GB),
M = 1, fp16 x, group 128, fp32 y, all 256 w4a16_gemv calls captured in one
HIP graph and replayed.  `value` is the effective bandwidth of that sweep
(algorithmic bytes / time; bytes = packed weights + fp16 scales + 4-bit zeros
+ x + y), with inputs resident in HBM.

Also reported: the same sweep at M = 4 (bf16 x with 1% outliers of magnitude
20), microseconds per call for each shape (a graph of that shape's 64 calls on
distinct buffers, replayed; replay time / 64), the read-only bandwidth probe, a
roofline object for the dominant kernel instantiation (the one with the most
time in the M = 1 sweep) and the CPU oracle timed on a bounded sample.  Under
`extra`: the skinny sweep (M in 1, 2, 3, 4, 6, 8 x group 64, 128 x K = N in
4096, 5120, 8192, and an lm_head-like N = 152064, K = 5120) and the ternary
variant (K = 5120, N in 7168, 34816 and K = 17408, N = 5120 at M = 1, 4, 8),
each shape packed into enough distinct copies to span 2 GiB and timed as a
graph over them (one fp16 x per M), each with a sampled parity check.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3]

HBM traffic of the dominant kernel comes from two rocprofv3 counter runs of
this same script (FETCH_SIZE, then WRITE_SIZE), each calibrated by the counter
value of a plain 1 GiB device copy made in the same run, folded into
profiles/w4_gemv_traffic.json by

    python bench.py --ingest-pmc FETCH.csv WRITE.csv --pmc-command "..."
"""
from __future__ import annotations

import argparse
import csv
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

PEAK_GBPS = 8000.0          # MI355X HBM3E, published
GROUP = 128
SHAPES = (("qkv", 5120, 7168), ("o_proj", 5120, 5120), ("gate_up", 5120, 34816),
          ("down", 17408, 5120))
N_LAYERS = 64
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "w4_gemv_traffic.json")
# The sources that define the 4-bit GEMV kernel (its counters are only valid
# for the code they were taken on).
KERNEL_SRCS = [os.path.join(ROOT, "bit_weight_only_03_amd", "csrc", f) for f in ("w4_gemv.hip", "common.h")]
CALIB_BYTES = 1 << 30       # the plain device copy the counter runs are calibrated with
KERNEL_RE = re.compile(r"(?:w4_gemv_kernel|w4_gemm_kernel|w16_gemv_kernel|w16_ksplit_kernel|w16_dot_kernel|w16_dot_bal_kernel|w2t_gemv_kernel|"
                       r"w2t_gemv_direct_kernel)<[^>]*>")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def alg_bytes(M, N, K, g, x_bytes=2, y_bytes=4):
    """Algorithmic bytes of one call: packed q + fp16 scales + 4-bit zeros + x + y."""
    G = K // g
    return N * K // 2 + G * N * 2 + G * N // 2 + M * K * x_bytes + M * N * y_bytes


def gbps(nbytes, seconds):
    return nbytes / seconds / 1e9


def kernel_source_hash():
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def kernel_key(name):
    """'w4_gemv_kernel<false, 4, 5>' out of a variant string or a profiler's
    demangled kernel name (spaces normalised)."""
    m = KERNEL_RE.search(name)
    if not m:
        return None
    k = re.sub(r"\s+", " ", m.group(0))
    # The 4-bit GEMV's template arguments after the fourth (MXFP4 mode,
    # per-unit x staging, balanced plan) default to false and the variant
    # strings leave trailing defaults out; profiler names spell them.
    if k.startswith("w4_gemv_kernel<"):
        while k.count(",") > 3 and k.endswith(", false>"):
            k = k[: -len(", false>")] + ">"
    return k


def load_traffic(kernel):
    """Mean HBM bytes per dispatch of `kernel` from the committed rocprofv3
    counter summary, if it was taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_dispatch")


def _pmc_rows(path, counter):
    """(kernel name, value) per dispatch from a rocprofv3 counter_collection
    CSV holding one counter."""
    out = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name", counter) != counter:
                continue
            out.append((r["Kernel_Name"], float(r["Counter_Value"])))
    if not out:
        raise SystemExit(f"{path}: no {counter} rows")
    return out


def ingest_pmc(fetch_csv, write_csv, command):
    """Fold two counter runs into TRAFFIC_FILE.  FETCH_SIZE and WRITE_SIZE are
    KiB per dispatch; each is scaled by known / counted bytes of the largest
    plain device copy in its run (the 1 GiB calibration copy), and the result
    is the mean per dispatch of every w4_gemv_kernel instantiation seen."""
    res = {"kernel_source_sha256_16": kernel_source_hash(), "command": command,
           "calibration": {}, "kernels": {}}
    per = {}
    for label, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"),
                                 ("write", write_csv, "WRITE_SIZE")):
        rows = _pmc_rows(path, counter)
        # torch runs the contiguous 1 GiB device copy as the runtime's own
        # copy kernel; it is by far the largest copy dispatch in the run.
        copies = [(v, n) for n, v in rows if "copy" in n.lower()]
        if not copies:
            raise SystemExit(f"{path}: no device copy kernel to calibrate against")
        v, cname = max(copies)
        counted = v * 1024.0
        factor = CALIB_BYTES / counted
        if not 0.25 <= factor <= 4.0:
            raise SystemExit(f"{path}: largest copy ({cname[:60]}) counted {counted:.3e} B, "
                             f"not the {CALIB_BYTES} B calibration copy")
        res["calibration"][label] = {"counter": counter, "kernel": cname[:80],
                                     "known_bytes": CALIB_BYTES, "counted_bytes": counted,
                                     "factor": round(factor, 5)}
        for n, v in rows:
            k = kernel_key(n)
            if k:
                per.setdefault(k, {}).setdefault(label, []).append(v * 1024.0 * factor)
    for k, d in sorted(per.items()):
        f, w = d.get("fetch", []), d.get("write", [])
        if not f or not w:
            continue
        res["kernels"][k] = {"dispatches": [len(f), len(w)],
                             "fetch_bytes_per_dispatch": round(float(np.mean(f))),
                             "write_bytes_per_dispatch": round(float(np.mean(w))),
                             "bytes_per_dispatch": round(float(np.mean(f) + np.mean(w)))}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(res, fh, indent=1)
        fh.write("\n")
    print(json.dumps(res, indent=1))


class Sweep:
    """256 packed matrices plus per-call x and y buffers for one M."""

    def __init__(self, L, torch, synth, M, x_dtype, outliers, mats=None):
        self.L, self.torch = L, torch
        self.M, self.x_dtype = M, x_dtype
        self.mats = mats if mats is not None else self._make_mats(synth)
        self.xs, self.ys = [], []
        for i, (layer, name, K, N, _) in enumerate(self.mats_meta):
            self.xs.append(synth.gen_x_torch((2, M, layer, i), M, K, x_dtype,
                                             outlier_frac=0.01 if outliers else 0.0))
            self.ys.append(torch.empty((M, N), dtype=torch.float32, device="cuda"))
        self.bytes = sum(alg_bytes(M, N, K, GROUP) for (_, _, K, N, _) in self.mats_meta)
        # One workspace serves every call: calls on one stream run one after another.
        self.ws_bytes = max(L.w4a16_workspace_bytes(M, N, K, GROUP) for (_, _, K, N, _) in self.mats)
        self.ws = torch.zeros(self.ws_bytes, dtype=torch.uint8, device="cuda") if self.ws_bytes else None

    @property
    def mats_meta(self):
        return self.mats

    def _make_mats(self, synth):
        torch, L = self.torch, self.L
        mats = []
        for layer in range(N_LAYERS):
            for mi, (name, K, N) in enumerate(SHAPES):
                w = synth.gen_w4_torch((1, layer, mi), N, K, GROUP)
                qb, sb, zb = L.w4a16_packed_sizes(N, K, GROUP)
                q = torch.empty(qb, dtype=torch.uint8, device="cuda")
                s = torch.empty(sb, dtype=torch.uint8, device="cuda")
                z = torch.empty(zb, dtype=torch.uint8, device="cuda")
                L.w4a16_pack(w["qweight"], w["scales"], w["zeros"], q, s, z, N, K, GROUP)
                mats.append((layer, name, K, N, (q, s, z)))
                del w
            if layer % 16 == 15:
                torch.cuda.synchronize()
                log(f"packed {layer + 1}/{N_LAYERS} layers")
        return mats

    def launch(self, i, stream):
        layer, name, K, N, (q, s, z) = self.mats[i]
        self.L.w4a16_gemv(self.xs[i], self.x_dtype, q, s, z, self.ys[i], "f32", self.M, N, K,
                          GROUP, self.ws, self.ws_bytes, stream)

    def run_all(self, stream):
        for i in range(len(self.mats)):
            self.launch(i, stream)

    def capture(self, stream, calls=None):
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in (range(len(self.mats)) if calls is None else calls):
                self.launch(i, stream)
        return g

    def per_shape(self, stream, steps, warmup):
        """Microseconds per call of each shape: a graph of that shape's
        N_LAYERS calls (distinct buffers), timed with events over replays.
        Also the kernel instantiation each shape dispatches to."""
        out = {}
        for mi, (name, K, N) in enumerate(SHAPES):
            self.launch(mi, stream)
            variant = self.L.w4a16_last_variant()
            calls = list(range(mi, len(self.mats), len(SHAPES)))
            g = self.capture(stream, calls)
            t = self.time_graph(g, stream, steps, warmup) / len(calls)
            del g
            b = alg_bytes(self.M, N, K, GROUP, x_bytes=2, y_bytes=4)
            out[name] = {"us": round(t * 1e6, 3), "GBps": round(gbps(b, t), 1),
                         "bytes": b, "kernel": kernel_key(variant), "variant": variant}
        return out

    def time_graph(self, graph, stream, steps, warmup):
        torch = self.torch
        with torch.cuda.stream(stream):
            for _ in range(warmup):
                graph.replay()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(steps):
                graph.replay()
            e1.record(stream)
            torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / steps

    def time_eager(self, stream, steps):
        torch = self.torch
        with torch.cuda.stream(stream):
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(steps):
                self.run_all(stream)
            e1.record(stream)
            torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / steps


def parity_guard(L, torch, synth, oracle_mod, sweep):
    """Sampled columns of a few calls against the oracle, so a timing is never
    reported for wrong results."""
    rng = np.random.default_rng(0)
    worst = 0.0
    for i in (0, 1, 2, 3, len(sweep.mats) - 1):
        layer, name, K, N, _ = sweep.mats[i]
        mi = i % 4
        w = synth.gen_w4_torch((1, layer, mi), N, K, GROUP)
        wq = w["qweight"].cpu().numpy()
        ws = w["scales"].cpu().numpy().view(np.uint16)
        wz = w["zeros"].cpu().numpy()
        x = sweep.xs[i].cpu().numpy().view(np.uint16)
        cols = np.sort(rng.choice(N, size=64, replace=False)).astype(np.int64)
        ref = oracle_mod.w4_gemv(x, sweep.x_dtype, wq, ws, wz, sweep.M, N, K, GROUP, cols=cols)
        got = sweep.ys[i].cpu().numpy().astype(np.float64)[:, cols]
        rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        mx = np.max(np.abs(got - ref)) / np.max(np.abs(ref))
        if rel > 1e-3 or mx > 4e-3:
            raise SystemExit(f"parity guard failed on call {i} ({name}): rel={rel:.2e} max={mx:.2e}")
        worst = max(worst, rel)
    return worst


def cpu_baseline(torch, synth, oracle_mod, budget_s=12.0):
    """The fp64 oracle on the host cores, on a bounded sample: whole layers of
    the sweep (4 matrices, M = 1) until about budget_s seconds of oracle time
    have passed."""
    t_total, nbytes, layers = 0.0, 0, 0
    while t_total < budget_s and layers < N_LAYERS:
        for mi, (name, K, N) in enumerate(SHAPES):
            w = synth.gen_w4_torch((1, layers, mi), N, K, GROUP)
            wq = w["qweight"].cpu().numpy()
            ws = w["scales"].cpu().numpy().view(np.uint16)
            wz = w["zeros"].cpu().numpy()
            x = synth.gen_x_torch((2, 1, layers, 4 * layers + mi), 1, K, "f16").cpu().numpy().view(np.uint16)
            t0 = time.perf_counter()
            oracle_mod.w4_gemv(x, "f16", wq, ws, wz, 1, N, K, GROUP)
            t_total += time.perf_counter() - t0
            nbytes += alg_bytes(1, N, K, GROUP)
        layers += 1
        if layers % 16 == 0:
            log(f"cpu oracle: {layers} layer(s), {t_total:.1f} s")
    return {"value": round(gbps(nbytes, t_total), 4), "unit": "GB/s",
            "cores": oracle_mod.num_threads(), "kind": "oracle",
            "sample": f"{layers} full decoder layer(s) of the M=1 sweep (qkv, o_proj, gate_up, "
                      f"down; {nbytes / 1e9:.3f} GB algorithmic), fp64 oracle, "
                      f"{t_total:.1f} s; GB/s over that sample"}


ROT_BYTES = 2 << 30   # distinct copies per shape, so no shape sits in the 256 MB cache
SKINNY_M = (1, 2, 3, 4, 6, 8)
BATCH_M = (16, 32, 64)            # rows of the batch sweeps (M-tiled kernel)
W16_M = (1, 2, 4, 8)               # rows of the W16A16 measurements
MX_M = (1, 4, 8, 64)               # rows of the MXFP4 sweep (64: the M-tiled kernel)
SKINNY_KN = (4096, 5120, 8192)
LM_HEAD = (5120, 152064)
TERNARY = ((5120, 7168), (5120, 34816), (17408, 5120))
TERNARY_M = (1, 4, 8)


def w2t_bytes(M, N, K, g, x_bytes=2, y_bytes=4):
    """Algorithmic bytes of one ternary call: 2-bit codes + fp16 scales + x + y."""
    return N * K // 4 + (K // g) * N * 2 + M * K * x_bytes + M * N * y_bytes


def mx_bytes(M, N, K, g=32, x_bytes=2, y_bytes=4):
    """Algorithmic bytes of one MXFP4 call: 4-bit elements + one E8M0 byte per
    32 elements + x + y."""
    return N * K // 2 + (K // 32) * N + M * K * x_bytes + M * N * y_bytes


def residual_fusion(L, torch, synth, oracle_mod, K, N, g, steps, warmup, stream, key):
    """µs per call of h += x . W (fp16 hidden state h, M = 1) two ways: fused
    (w4a16_gemv_add in place) and unfused (w4a16_gemv into an fp16 temporary,
    then torch's add), each as a graph over copies of one packed matrix."""
    M = 1
    w = synth.gen_w4_torch(key, N, K, g)
    sizes = L.w4a16_packed_sizes(N, K, g)
    copies = max(2, -(-ROT_BYTES // sum(sizes)))
    mats = []
    for _ in range(copies):
        bufs = [torch.empty(b, dtype=torch.uint8, device="cuda") for b in sizes]
        L.w4a16_pack(w["qweight"], w["scales"], w["zeros"], *bufs, N, K, g)
        mats.append(bufs)
    torch.cuda.synchronize()
    x = synth.gen_x_torch(key + (M,), M, K, "f16")
    h0 = (torch.randn((M, N), generator=torch.Generator().manual_seed(7)) * 4).half().cuda()
    h = h0.clone()
    t = torch.empty((M, N), dtype=torch.float16, device="cuda")
    wsb = L.w4a16_workspace_bytes(M, N, K, g)
    ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device="cuda")

    def fused(bufs):
        L.w4a16_gemv_add(x, "f16", *bufs, h, "f16", h, "f16", M, N, K, g, ws, wsb, stream)

    def unfused(bufs):
        L.w4a16_gemv(x, "f16", *bufs, t, "f16", M, N, K, g, ws, wsb, stream)
        h.add_(t)

    xh = x.cpu().numpy().view(np.uint16)
    cols = np.sort(np.random.default_rng(3).choice(N, size=64, replace=False)).astype(np.int64)
    ref = oracle_mod.w4_gemv(xh, "f16", w["qweight"].cpu().numpy(),
                             w["scales"].cpu().numpy().view(np.uint16),
                             w["zeros"].cpu().numpy(), M, N, K, g, cols=cols)
    ref = ref + h0.double().cpu().numpy()[:, cols]
    out = {"K": K, "N": N, "group": g, "M": M, "copies": copies}
    for name, call in (("fused", fused), ("unfused", unfused)):
        h.copy_(h0)
        with torch.cuda.stream(stream):
            call(mats[0])
        torch.cuda.synchronize()
        got = h.double().cpu().numpy()[:, cols]
        rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
        if rel > 1e-3 + 2.0 ** -11:
            raise SystemExit(f"parity guard failed: residual {name} K={K} N={N}: rel={rel:.2e}")
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for bufs in mats:
                call(bufs)
        with torch.cuda.stream(stream):
            for _ in range(warmup):
                graph.replay()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(steps):
                graph.replay()
            e1.record(stream)
            torch.cuda.synchronize()
        del graph
        out[name + "_us"] = round(e0.elapsed_time(e1) * 1e3 / steps / copies, 3)
        out[name + "_parity_rel"] = rel
    return out


def w16_sweep(L, torch, synth, oracle_mod, K, N, Ms, steps, warmup, stream, key):
    """µs per call of the W16A16 layer (fp16 weights [N][K]) at each M: copies
    of one weight matrix spanning ROT_BYTES, a graph of one call per copy."""
    w = synth.gen_w16_torch(key, N, K, "f16")
    copies = max(2, -(-ROT_BYTES // (N * K * 2)))
    mats = [w.clone() for _ in range(copies)]
    torch.cuda.synchronize()
    out = []
    rng = np.random.default_rng(2)
    wh = w.cpu().numpy().view(np.uint16)
    for M in Ms:
        x = synth.gen_x_torch(key + (M,), M, K, "f16")
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        wsb = L.w16a16_workspace_bytes(M, N, K)
        ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device="cuda")

        def call(wm):
            L.w16a16_gemv(x, wm, "f16", y, "f32", M, N, K, ws, wsb, stream)

        with torch.cuda.stream(stream):
            call(mats[0])
        torch.cuda.synchronize()
        variant = L.w4a16_last_variant()
        cols = np.sort(rng.choice(N, size=min(32, N), replace=False)).astype(np.int64)
        ref = oracle_mod.w16_gemv(x.cpu().numpy().view(np.uint16), "f16", wh, M, N, K, cols=cols)
        got = y.cpu().numpy().astype(np.float64)[:, cols]
        rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
        if rel > 1e-3:
            raise SystemExit(f"parity guard failed: w16 M={M} K={K} N={N}: rel={rel:.2e}")
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for wm in mats:
                call(wm)
        with torch.cuda.stream(stream):
            for _ in range(warmup):
                graph.replay()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(steps):
                graph.replay()
            e1.record(stream)
            torch.cuda.synchronize()
        del graph
        t = e0.elapsed_time(e1) / 1e3 / steps / copies
        b = N * K * 2 + M * K * 2 + M * N * 4
        out.append({"M": M, "K": K, "N": N, "us": round(t * 1e6, 3), "GBps": round(gbps(b, t), 1),
                    "pct_of_peak": round(100 * gbps(b, t) / PEAK_GBPS, 2), "bytes": b,
                    "copies": copies, "parity_rel": rel, "kernel": kernel_key(variant)})
    return out


def rotation_sweep(L, torch, synth, oracle_mod, kind, K, N, g, Ms, steps, warmup, stream, key):
    """µs per call of one shape at each M: copies of one packed matrix spanning
    ROT_BYTES, a graph of one call per copy, events around the replays."""
    if kind == "w4":
        w = synth.gen_w4_torch(key, N, K, g)
        sizes = L.w4a16_packed_sizes(N, K, g)
    elif kind == "mx":
        w = synth.gen_mx_torch(key, N, K)
        sizes = L.mxfp4_packed_sizes(N, K)
    else:
        w = synth.gen_w2t_torch(key, N, K, g)
        sizes = L.w2t_packed_sizes(N, K, g)
    copies = max(2, -(-ROT_BYTES // sum(sizes)))
    mats = []
    for _ in range(copies):
        bufs = [torch.empty(b, dtype=torch.uint8, device="cuda") for b in sizes]
        if kind == "w4":
            L.w4a16_pack(w["qweight"], w["scales"], w["zeros"], *bufs, N, K, g)
        elif kind == "mx":
            L.mxfp4_pack(w["qweight"], w["scales"], *bufs, N, K)
        else:
            L.w2t_pack(w["codes"], w["scales"], *bufs, N, K, g)
        mats.append(bufs)
    # The packs ran on torch's current stream; the calls below use `stream`.
    torch.cuda.synchronize()
    out = []
    rng = np.random.default_rng(1)
    for M in Ms:
        x = synth.gen_x_torch(key + (M,), M, K, "f16")
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        if kind == "w4":
            wsb = L.w4a16_workspace_bytes(M, N, K, g)
        elif kind == "mx":
            wsb = L.mxfp4_workspace_bytes(M, N, K)
        else:
            wsb = L.w2t_workspace_bytes(M, N, K, g)
        ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device="cuda")

        def call(bufs):
            if kind == "w4":
                L.w4a16_gemv(x, "f16", *bufs, y, "f32", M, N, K, g, ws, wsb, stream)
            elif kind == "mx":
                L.mxfp4_gemv(x, "f16", *bufs, y, "f32", M, N, K, ws, wsb, stream)
            else:
                L.w2t_gemv(x, "f16", *bufs, y, "f32", M, N, K, g, ws, wsb, stream)

        with torch.cuda.stream(stream):
            call(mats[0])
        torch.cuda.synchronize()
        variant = L.w4a16_last_variant()
        cols = np.sort(rng.choice(N, size=min(32, N), replace=False)).astype(np.int64)
        xh = x.cpu().numpy().view(np.uint16)
        if kind == "w4":
            ref = oracle_mod.w4_gemv(xh, "f16", w["qweight"].cpu().numpy(),
                                     w["scales"].cpu().numpy().view(np.uint16),
                                     w["zeros"].cpu().numpy(), M, N, K, g, cols=cols)
        elif kind == "mx":
            ref = oracle_mod.mx_gemv(xh, "f16", w["qweight"].cpu().numpy(),
                                     w["scales"].cpu().numpy(), M, N, K, cols=cols)
        else:
            ref = oracle_mod.w2t_gemv(xh, "f16", w["codes"].cpu().numpy(),
                                      w["scales"].cpu().numpy().view(np.uint16), M, N, K, g,
                                      cols=cols)
        got = y.cpu().numpy().astype(np.float64)[:, cols]
        rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
        mx = float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
        if rel > 1e-3 or mx > 4e-3:
            raise SystemExit(f"parity guard failed: {kind} M={M} K={K} N={N} g={g}: rel={rel:.2e}")
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for bufs in mats:
                call(bufs)
        with torch.cuda.stream(stream):
            for _ in range(warmup):
                graph.replay()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(steps):
                graph.replay()
            e1.record(stream)
            torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / 1e3 / steps / copies
        del graph
        b = {"w4": alg_bytes, "mx": mx_bytes, "w2t": w2t_bytes}[kind](M, N, K, g)
        out.append({"M": M, "K": K, "N": N, "group": g, "us": round(t * 1e6, 3),
                    "GBps": round(gbps(b, t), 1), "pct_of_peak": round(100 * gbps(b, t) / PEAK_GBPS, 2),
                    "bytes": b, "copies": copies, "parity_rel": rel,
                    "kernel": variant.split("kernel=")[1].split(">")[0] + ">" if "kernel=" in variant else variant})
    del mats
    torch.cuda.synchronize()
    return out


def bw_probe(L, torch, nbytes=4 << 30, reps=5):
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.empty(L.w4a16_bw_probe_sink_floats(), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream()
    L.w4a16_bw_probe(buf, nbytes, sink, s)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(reps):
        L.w4a16_bw_probe(buf, nbytes, sink, s)
    e1.record(s)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3 / reps
    # The plain device copy of known size that the counter runs calibrate
    # FETCH_SIZE and WRITE_SIZE against (1 GiB read, 1 GiB written).
    dst = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda")
    dst.copy_(buf[:CALIB_BYTES])
    torch.cuda.synchronize()
    del buf, dst
    return gbps(nbytes, t)


def dominant(per_shape):
    """The kernel instantiation with the most time in one sweep, and its
    algorithmic GB/s per launch (equal call counts per shape, so total bytes
    over total time of its shapes)."""
    tot = {}
    for name, d in per_shape.items():
        b, t = tot.get(d["kernel"], (0, 0.0))
        tot[d["kernel"]] = (b + d["bytes"], t + d["us"] * 1e-6)
    k = max(tot, key=lambda k: tot[k][1])
    shapes = [n for n, d in per_shape.items() if d["kernel"] == k]
    b, t = tot[k]
    return k, shapes, b / len(shapes), t / len(shapes)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-m4", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the skinny-sweep and ternary measurements")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="fold two rocprofv3 counter runs of this script into "
                         "profiles/w4_gemv_traffic.json and exit (no GPU work)")
    ap.add_argument("--pmc-command", default="", help="the command the counter runs used")
    ap.add_argument("--extra-json", default=EXTRA_JSON,
                    help="where to write the detailed measurements (`extra`) as JSON")
    args = ap.parse_args()
    if args.ingest_pmc:
        ingest_pmc(args.ingest_pmc[0], args.ingest_pmc[1], args.pmc_command)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this library has no multi-GPU path "
              f"(--gpus {args.gpus} is not supported)", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_weight_only_03_amd as L
    import synth

    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    dev_name = torch.cuda.get_device_name(0)
    log(f"device: {dev_name}")
    stream = torch.cuda.Stream()

    log("building the M=1 sweep (64 layers x 4 matrices, packed on device)")
    s1 = Sweep(L, torch, synth, 1, "f16", outliers=False)
    torch.cuda.synchronize()
    s1.run_all(stream)
    torch.cuda.synchronize()

    import oracle as oracle_mod
    worst = parity_guard(L, torch, synth, oracle_mod, s1)
    log(f"parity guard ok (worst sampled rel Frobenius {worst:.2e})")

    g1 = s1.capture(stream)
    t1 = s1.time_graph(g1, stream, args.steps, args.warmup)
    log(f"M=1 sweep: {t1 * 1e3:.4f} ms/token, {gbps(s1.bytes, t1):.1f} GB/s")
    del g1
    te1 = s1.time_eager(stream, max(2, args.steps // 4))
    shapes1 = s1.per_shape(stream, args.steps, args.warmup)
    for name, d in shapes1.items():
        log(f"  {name}: {d['us']:.2f} us/call, {d['GBps']:.0f} GB/s  [{d['kernel']}]")
    kern, kshapes, kbytes, ktime = dominant(shapes1)
    achieved = gbps(kbytes, ktime)
    traffic = load_traffic(kern)

    extra = {"device": dev_name, "sweep_bytes": s1.bytes,
             "pct_of_peak": round(100 * gbps(s1.bytes, t1) / PEAK_GBPS, 2),
             "m1_eager_ms": round(te1 * 1e3, 4), "m1_per_shape": shapes1}

    if not args.no_m4:
        log("M=4 sweep (bf16 x, 1% outliers), same weights")
        s4 = Sweep(L, torch, synth, 4, "bf16", outliers=True, mats=s1.mats)
        s4.run_all(stream)
        torch.cuda.synchronize()
        w4 = parity_guard(L, torch, synth, oracle_mod, s4)
        g4 = s4.capture(stream)
        t4 = s4.time_graph(g4, stream, args.steps, args.warmup)
        del g4
        shapes4 = s4.per_shape(stream, args.steps, args.warmup)
        extra["m4_sweep"] = {"ms_per_token": round(t4 * 1e3, 4), "GBps": round(gbps(s4.bytes, t4), 1),
                             "pct_of_peak": round(100 * gbps(s4.bytes, t4) / PEAK_GBPS, 2),
                             "bytes": s4.bytes, "parity_worst_rel": w4, "per_shape": shapes4}
        log(f"M=4 sweep: {t4 * 1e3:.4f} ms/token, {gbps(s4.bytes, t4):.1f} GB/s")
        for name, d in shapes4.items():
            log(f"  {name}: {d['us']:.2f} us/call, {d['GBps']:.0f} GB/s  [{d['kernel']}]")
        del s4

    if not args.no_extra:
        # Several rows at once (a batch of decode tokens): the same 64 layers
        # at M = 16, 32 and 64, which the M-tiled kernel serves.
        batch = []
        for mb in BATCH_M:
            sb = Sweep(L, torch, synth, mb, "f16", outliers=False, mats=s1.mats)
            sb.run_all(stream)
            torch.cuda.synchronize()
            wb = parity_guard(L, torch, synth, oracle_mod, sb)
            gb = sb.capture(stream)
            tb = sb.time_graph(gb, stream, args.steps, args.warmup)
            del gb
            shb = sb.per_shape(stream, args.steps, args.warmup)
            batch.append({"M": mb, "ms_per_step": round(tb * 1e3, 4), "tokens_per_s": round(mb / tb, 1),
                          "GBps": round(gbps(sb.bytes, tb), 1), "bytes": sb.bytes,
                          "parity_worst_rel": wb, "per_shape": shb})
            log(f"M={mb} sweep (fp16 x): {tb * 1e3:.4f} ms/step, {mb / tb:.0f} tokens/s, "
                f"{gbps(sb.bytes, tb):.1f} GB/s; " + ", ".join(
                    f"{k} {d['us']:.1f}us" for k, d in shb.items()))
            del sb
        extra["batch_sweeps"] = batch
        # The residual add of o_proj and down, fused into the GEMV's output
        # stage or done as a separate add.
        fusion = []
        for (name, K, N) in (("o_proj", 5120, 5120), ("down", 17408, 5120)):
            r = residual_fusion(L, torch, synth, oracle_mod, K, N, GROUP, max(5, args.steps // 2),
                                max(2, args.warmup), stream, (5, K, N))
            r["shape"] = name
            fusion.append(r)
            log(f"residual add {name}: fused {r['fused_us']:.2f} us, unfused {r['unfused_us']:.2f} us")
        extra["residual_fusion"] = fusion
        # 16-bit weights (W16A16) on the same layer shapes.
        w16 = []
        for (name, K, N) in SHAPES:
            rows = w16_sweep(L, torch, synth, oracle_mod, K, N, W16_M, max(5, args.steps // 2),
                             max(2, args.warmup), stream, (6, K, N))
            for r in rows:
                r["shape"] = name
            w16 += rows
            log(f"w16a16 {name}: " + ", ".join(f"M{r['M']} {r['us']:.2f}us {r['GBps']:.0f}GB/s"
                                               for r in rows))
        extra["w16a16"] = w16
        # MXFP4 weights on the same layer shapes.
        mx = []
        for (name, K, N) in SHAPES:
            rows = rotation_sweep(L, torch, synth, oracle_mod, "mx", K, N, 32, MX_M,
                                  max(5, args.steps // 2), max(2, args.warmup), stream, (7, K, N))
            for r in rows:
                r["shape"] = name
            mx += rows
            log(f"mxfp4 {name}: " + ", ".join(f"M{r['M']} {r['us']:.2f}us {r['GBps']:.0f}GB/s"
                                              for r in rows))
        extra["mxfp4"] = mx
        steps_x, warm_x = max(5, args.steps // 2), max(2, args.warmup)
        skinny = []
        for kn in SKINNY_KN:
            for g in (128, 64):
                skinny += rotation_sweep(L, torch, synth, oracle_mod, "w4", kn, kn, g, SKINNY_M,
                                         steps_x, warm_x, stream, (4, kn, g))
                log(f"skinny K=N={kn} g={g}: " + ", ".join(
                    f"M{r['M']} {r['us']:.2f}us" for r in skinny[-len(SKINNY_M):]))
        for g in (128, 64):
            skinny += rotation_sweep(L, torch, synth, oracle_mod, "w4", LM_HEAD[0], LM_HEAD[1], g,
                                     SKINNY_M, steps_x, warm_x, stream, (4, 152064, g))
            log(f"lm_head g={g}: " + ", ".join(f"M{r['M']} {r['us']:.2f}us"
                                               for r in skinny[-len(SKINNY_M):]))
        extra["skinny_sweep"] = skinny
        tern = []
        for K, N in TERNARY:
            tern += rotation_sweep(L, torch, synth, oracle_mod, "w2t", K, N, GROUP, TERNARY_M,
                                   steps_x, warm_x, stream, (5, K, N))
            log(f"ternary K={K} N={N}: " + ", ".join(
                f"M{r['M']} {r['us']:.2f}us {r['GBps']:.0f}GB/s" for r in tern[-len(TERNARY_M):]))
        extra["ternary"] = tern

    probe = bw_probe(L, torch)
    extra["bw_probe_GBps"] = round(probe, 1)
    extra["value_pct_of_probe"] = round(100 * gbps(s1.bytes, t1) / probe, 2)
    log(f"bw_probe read ceiling: {probe:.1f} GB/s")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(torch, synth, oracle_mod)

    result = {
        "metric": "W4A16 GEMV effective HBM GB/s (% of peak) + µs/call at M=1,4; ms/token sweep",
        "value": round(gbps(s1.bytes, t1), 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t1 * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "27B-class decoder weight sweep: 64 layers x (qkv K5120 N7168, "
                               "o_proj K5120 N5120, gate_up K5120 N34816, down K17408 N5120), "
                               "M=1, group 128, 256 distinct packed buffers, hipGraph replay",
                   "M": 1, "group": GROUP, "layers": N_LAYERS, "x": "f16", "y": "f32"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_GBPS, 4),
                     "traffic": traffic, "kernel": kern, "shapes": kshapes,
                     "per_launch_alg_bytes": round(kbytes), "per_launch_us": round(ktime * 1e6, 3),
                     "timing": "HIP events around replays of a graph of the shape's 64 calls"},
        "cpu_baseline": cpu,
    }
    emit(result, extra, args.extra_json)


HEADLINE_MAX_BYTES = 3072
EXTRA_JSON = os.path.join(ROOT, "gpurun_out", "bench_extra.json")


def summary(extra):
    """The few figures of `extra` that belong on the headline line: the
    sweep's share of peak and of the read probe, µs per call of each shape at
    M = 1 and M = 4, and the M = 4 sweep."""
    out = {"pct_of_peak": extra.get("pct_of_peak"), "bw_probe_GBps": extra.get("bw_probe_GBps"),
           "value_pct_of_probe": extra.get("value_pct_of_probe"),
           "m1_us": {k: d["us"] for k, d in extra.get("m1_per_shape", {}).items()}}
    m4 = extra.get("m4_sweep")
    if m4:
        out["m4_ms_per_token"] = m4["ms_per_token"]
        out["m4_pct_of_peak"] = m4["pct_of_peak"]
        out["m4_us"] = {k: d["us"] for k, d in m4["per_shape"].items()}
    return out


def emit(result, extra, extra_json=None):
    """Write the detail (`extra`) to a JSON file, then print the headline as
    the last stdout line: one JSON object of at most HEADLINE_MAX_BYTES
    bytes (a reader that keeps only the tail of the output still gets it
    whole)."""
    if extra_json:
        os.makedirs(os.path.dirname(os.path.abspath(extra_json)), exist_ok=True)
        with open(extra_json, "w") as f:
            json.dump(extra, f, indent=1)
            f.write("\n")
        log(f"detailed measurements written to {extra_json}")
    head = dict(result)
    head["summary"] = summary(extra)
    line = json.dumps(head)
    if len(line.encode()) > HEADLINE_MAX_BYTES:
        head.pop("summary")
        line = json.dumps(head)
    print(line, flush=True)
    return line


if __name__ == "__main__":
    main()
