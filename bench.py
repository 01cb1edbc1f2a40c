"""Benchmark of the additive-codebook decode GEMV on one MI355X.

Workload: the 4096 x 14336 down-projection linear (d_out 4096, d_in 14336) at
batch 1, M = 4 code planes of uint8, g = 8, fp16 codebooks, Hadamard block
256, evaluated at k = 1, 2, 3 and 4 codebooks (1..4 bits per weight).

One step = one pass of the decode hot path over one token: the online block
Hadamard rotation of the activation, then the GEMV at k = 1, 2, 3 and 4, each
reading its own cold copy of the packed codes (64 copies, 1.9 GB in total,
cycled so the 256 MB last-level cache cannot serve them).  Inputs are resident
in HBM before timing starts.

Reported (one JSON line): mean microseconds per GEMV over the four bitwidths
(`value`), per-k timings and HBM-roofline fractions, a roofline object for the
k = 4 GEMV kernel (algorithmic bytes per launch / average launch time measured
with HIP events on the launch stream around a graph of K back-to-back
launches), the same launches issued eagerly from Python, the 32-layer stack
latency, the small-batch matrix-core path, and the CPU oracle timed on the host
cores on a bounded sample (which also checks the GPU outputs of the timed
configuration).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
D_OUT, D_IN, M, BLOCK, BATCH = 4096, 14336, 4, 256, 1
KS = (1, 2, 3, 4)
N_COPIES = 64
CONFIG_ID = 3            # the MLP workload family (gate/up/down 14336 x 4096 and 4096 x 14336)

# HBM bytes per k=4 launch from rocprofv3 FETCH_SIZE + WRITE_SIZE (each scaled by a 64 MiB copy), valid
# only for the kernel sources they were taken on: the summary under profiles/ gives the commands.
TRAFFIC_K4_BYTES = 30674934
TRAFFIC_K4_SOURCE_SHA256_PREFIX = "4f14952b0c17a702"
TIMING_ROUNDS = 4          # rounds the timed steps are split into (see main)
# the batch-1 GEMV kernel's source and the headers it includes
HEADLINE_SOURCES = ("gemv_lut.hip", "lut_device.h", "fixed_sum.h", "fwht_device.h", "aqd_internal.h")


def source_code_text(text: str) -> str:
    """The code of a C/C++/HIP source: block and line comments removed, trailing blanks and empty lines
    dropped (the kernel sources hold no string literal that contains a comment marker)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip()) + "\n"


def headline_source_digest() -> str:
    """SHA-256 over the code (comments removed) of the batch-1 GEMV kernel's source files, concatenated in
    HEADLINE_SOURCES order: a comment edit leaves it, and the traffic figure taken for it, unchanged."""
    import hashlib
    h = hashlib.sha256()
    for name in HEADLINE_SOURCES:
        with open(os.path.join(ROOT, "additive_codebook_gemv_amd", "csrc", name), encoding="utf-8") as f:
            h.update(source_code_text(f.read()).encode("utf-8"))
    return h.hexdigest()


def measured_traffic():
    return TRAFFIC_K4_BYTES if headline_source_digest().startswith(TRAFFIC_K4_SOURCE_SHA256_PREFIX) else None


def algorithmic_bytes(k: int, d_out: int = D_OUT, d_in: int = D_IN, batch: int = BATCH) -> int:
    """Bytes the k-codebook GEMV must move: codes, codebooks, scales, activation in, output out."""
    return k * d_out * (d_in // 8) + k * 256 * 8 * 2 + 2 * d_out + 2 * batch * d_in + 2 * batch * d_out


def code_bytes(k: int) -> int:
    return k * D_OUT * (D_IN // 8)


def cpu_model() -> str:
    """The host CPU's model name (first 'model name' line of /proc/cpuinfo), or the platform string."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def cpu_baseline(codes, cb, s, x, budget_s: float, y_gpu=None):
    """The fp64 oracle on the host cores: full-size GEMVs (rotation included), k = 1..4 round-robin,
    first on every core this process may use, then on one thread.

    The all-core leg takes about two thirds of the budget and the one-thread leg the rest (at least one
    GEMV per k).  The oracle's rows are independent and it gives the same bits at any thread count.  Its
    first all-core output per k is also compared with the GPU result of the timed configuration
    (normwise max relative error), so the baseline and the measured kernels are seen to compute the same
    thing.
    """
    import oracle
    orc = oracle.load()
    affinity = len(os.sched_getaffinity(0))
    want = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or affinity

    def leg(threads: int, budget: float, check: bool):
        used = orc.set_threads(threads)
        times = {k: [] for k in KS}
        worst = 0.0
        t_start = time.perf_counter()
        while True:
            for k in KS:
                t0 = time.perf_counter()
                ref = orc.forward(codes, cb, s, k, x, BLOCK)
                times[k].append(time.perf_counter() - t0)
                if check and y_gpu is not None and len(times[k]) == 1:
                    worst = max(worst, float(np.max(np.abs(y_gpu[k].astype(np.float64) - ref)) /
                                       np.max(np.abs(ref))))
            if time.perf_counter() - t_start >= budget:
                break
        per_k = {k: float(np.median(v)) * 1e6 for k, v in times.items()}
        return used, per_k, len(times[1]), time.perf_counter() - t_start, worst

    threads, per_k, reps, spent, worst = leg(want, budget_s * 2 / 3, True)
    one, per_k1, reps1, spent1, _ = leg(1, budget_s / 3, False)
    orc.set_threads(want)
    out = {
        "value": float(np.mean(list(per_k.values()))),
        "unit": "us per GEMV",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{reps} full {D_OUT}x{D_IN} batch-1 decode linears (rotation + explicit W_k fp64 matvec) "
                  f"per k in 1..4 on {threads} threads ({spent:.1f} s), then {reps1} per k on 1 thread "
                  f"({spent1:.1f} s); median per k",
        "per_k_us": {str(k): v for k, v in per_k.items()},
        "one_thread": {"value": float(np.mean(list(per_k1.values()))), "unit": "us per GEMV", "cores": one,
                       "per_k_us": {str(k): v for k, v in per_k1.items()}},
        "cpu_model": cpu_model(),
        "nproc": os.cpu_count(),
        "affinity_cpus": affinity,
    }
    if y_gpu is not None:
        out["gpu_vs_oracle_worst_err"] = worst
        assert worst <= 2e-3, f"GPU output of the timed configuration disagrees with the oracle: {worst}"
    return out


def measure_stack(aqd, wl, torch, dev, replays: int = 20):
    """One decode token through the synthetic 32-layer stack of 8B shape (linears and rotations only).

    Per layer: q/k/v share one rotated input, o, gate/up (shared) and down get their own; every linear
    uses the layer's seeded k.  Three schedules of the same work, each captured in one graph and replayed:
    fused (each launch rotates its own input; q, k, v in one launch, gate and up in one launch: 4 launches
    per layer), grouped (4 rotations + 4 GEMV launches per layer) and separate (4 rotations + 7 GEMV
    launches per layer).
    """
    lins = wl.config(4)
    ks = wl.stack_ks()
    layers = []
    code_bytes = 0
    for lin in lins:
        codes, cb, sc, _ = wl.layer_inputs(4, lin)
        packed = aqd.aqd_pack_codes(torch.from_numpy(codes).to(dev))
        layers.append((lin, packed, torch.from_numpy(cb).to(dev), torch.from_numpy(sc).to(dev)))
        code_bytes += lin.ks[0] * lin.d_out * (lin.d_in // 8)
        del codes
    ws_need = max(aqd.aqd_gemv_workspace_bytes(l.d_out, l.d_in, l.M, 1) for l in lins)
    ws_need = max(ws_need, aqd.aqd_gemv_grouped_workspace_bytes([4096, 1024, 1024], 4096, [4, 4, 4]),
                  aqd.aqd_gemv_grouped_workspace_bytes([14336, 14336], 4096, [4, 4]))
    ws = torch.zeros(max(ws_need, 16), dtype=torch.uint8, device=dev)
    g = np.random.Generator(np.random.PCG64(0xA0D00004))
    inputs = {}
    for layer in range(32):
        for name, d_in in (("qkv", 4096), ("o", 4096), ("mlp", 4096), ("down", 14336)):
            x = g.standard_normal((1, d_in)).astype(np.float16)
            inputs[(layer, name)] = (torch.from_numpy(x).to(dev), torch.empty((1, d_in), dtype=torch.float16, device=dev))
    outs = [torch.empty((1, l.d_out), dtype=torch.float16, device=dev) for l in lins]
    src = {"q": "qkv", "k": "qkv", "v": "qkv", "o": "o", "gate": "mlp", "up": "mlp", "down": "down"}

    def rotations(layer):
        for name in ("qkv", "o", "mlp", "down"):
            x, xr = inputs[(layer, name)]
            aqd.aqd_hadamard_rotate(x, wl.block_for(x.shape[1]), aqd.AQD_F16, out=xr)

    def token_separate():
        for layer in range(32):
            rotations(layer)
            for j in range(7):
                lin, packed, cb, sc = layers[layer * 7 + j]
                xr = inputs[(layer, src[lin.proj])][1]
                aqd.aqd_gemv(packed, cb, sc, lin.ks[0], xr, lin.d_out, lin.d_in, lin.M, out=outs[layer * 7 + j],
                             workspace=ws)

    def token_grouped():
        for layer in range(32):
            rotations(layer)
            for group in ((0, 1, 2), (3,), (4, 5), (6,)):
                lin0 = layers[layer * 7 + group[0]][0]
                xr = inputs[(layer, src[lin0.proj])][1]
                if len(group) == 1:
                    lin, packed, cb, sc = layers[layer * 7 + group[0]]
                    aqd.aqd_gemv(packed, cb, sc, lin.ks[0], xr, lin.d_out, lin.d_in, lin.M,
                                 out=outs[layer * 7 + group[0]], workspace=ws)
                else:
                    parts = [(p, c, s_, l.d_out, l.M, outs[layer * 7 + j])
                             for j in group for (l, p, c, s_) in [layers[layer * 7 + j]]]
                    aqd.aqd_gemv_grouped(parts, lin0.ks[0], xr, lin0.d_in, workspace=ws)

    def token_fused():
        for layer in range(32):
            for group in ((0, 1, 2), (3,), (4, 5), (6,)):
                lin0 = layers[layer * 7 + group[0]][0]
                x = inputs[(layer, src[lin0.proj])][0]
                parts = [(p, c, s_, l.d_out, l.M, outs[layer * 7 + j])
                         for j in group for (l, p, c, s_) in [layers[layer * 7 + j]]]
                aqd.aqd_rotate_gemv_grouped(parts, lin0.ks[0], x, lin0.d_in, wl.block_for(lin0.d_in), workspace=ws)

    stream = torch.cuda.current_stream()

    def timed(token):
        token()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                token()
        stream.wait_stream(side)
        graph.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(replays):
            graph.replay()
        b.record(stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / replays
        a2, b2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a2.record(stream)
        for _ in range(3):
            token()
        b2.record(stream)
        torch.cuda.synchronize()
        return us, a2.elapsed_time(b2) * 1e3 / 3

    us, us_eager = timed(token_fused)
    us_grp, us_grp_eager = timed(token_grouped)
    us_sep, us_sep_eager = timed(token_separate)
    return {
        "workload": "32-layer decoder stack of 8B shape (q,o 4096x4096; k,v 1024x4096; gate,up 14336x4096; "
                    "down 4096x14336), batch 1, M=4, per-layer k from {2,3,4} (seeded), linears and rotations "
                    "only; each launch rotates its own input, q/k/v and gate/up grouped into one launch each",
        "layer_k": ks,
        "launches_per_token": 32 * 4,
        "code_bytes_per_token": code_bytes,
        "us_per_token_graph": us,
        "tokens_per_s_graph": 1e6 / us,
        "us_per_token_eager": us_eager,
        "frac_hbm_peak_graph": code_bytes / us / 1e3 / HBM_PEAK_GBPS,
        "grouped_rotations_apart": {"launches_per_token": 32 * 8, "us_per_token_graph": us_grp,
                                    "us_per_token_eager": us_grp_eager},
        "separate_launches": {"launches_per_token": 32 * 11, "us_per_token_graph": us_sep,
                              "us_per_token_eager": us_sep_eager},
    }


def measure_tiered(aqd, wl, torch, dev, copies: int = 32, reps: int = 2):
    """Tiered batch on the 4096x14336 down projection: 16 requests at k = 4, 3, 2, 1 (four each) in one
    launch, against the same requests as four single-k launches of four columns each."""
    lin = [l for l in wl.config(5) if l.name == "down4096x14336_sb"][0]
    codes, cb, sc, _ = wl.layer_inputs(5, lin, batch=64)
    packed0 = aqd.aqd_pack_codes(torch.from_numpy(codes).to(dev))
    cps = [packed0] + [packed0.clone() for _ in range(copies - 1)]
    cbd, sd = torch.from_numpy(cb).to(dev), torch.from_numpy(sc).to(dev)
    g = np.random.Generator(np.random.PCG64(0x7E))
    xr = torch.from_numpy(g.standard_normal((16, lin.d_in)).astype(np.float16)).to(dev)
    ks = [4] * 4 + [3] * 4 + [2] * 4 + [1] * 4
    y = torch.empty((16, lin.d_out), dtype=torch.float32, device=dev)
    ys = [torch.empty((4, lin.d_out), dtype=torch.float32, device=dev) for _ in range(4)]
    xs = [xr[4 * t:4 * t + 4].contiguous() for t in range(4)]
    ws = torch.zeros(max(aqd.aqd_gemm_small_batch_workspace_bytes(lin.d_out, lin.d_in, lin.M, 16), 16),
                     dtype=torch.uint8, device=dev)

    def one(c):
        aqd.aqd_gemm_small_batch_tiered(cps[c], cbd, sd, ks, xr, lin.d_out, lin.d_in, lin.M, out=y, workspace=ws)

    def split(c):
        for t, k in enumerate((4, 3, 2, 1)):
            aqd.aqd_gemm_small_batch(cps[c], cbd, sd, k, xs[t], lin.d_out, lin.d_in, lin.M, aqd.AQD_F16,
                                     out=ys[t], workspace=ws)

    res = {"workload": "4096x14336, 16 requests: k = 4, 3, 2, 1 for four each, fp16 activations", "ks": ks}
    for name, fn in (("one_launch", one), ("four_single_k_launches", split)):
        for c in range(copies):
            fn(c)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            for c in range(copies):
                fn(c)
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / (reps * copies)
        res[name] = {"us": us, "requests_per_s": 16 * 1e6 / us}
    del cps, packed0
    torch.cuda.empty_cache()
    return res


def measure_batched_gemv(aqd, torch, dev, copies, cbd, sd, stream, reps: int = 3):
    """The GEMV at batch 2, 4 and 8 on the timed layer (the code stream is read once for all columns),
    k = 1..4, each over a captured graph of back-to-back launches on the cold copies."""
    res = []
    g = np.random.Generator(np.random.PCG64(0xB2))
    for B in (2, 4, 8):
        xr = torch.from_numpy(g.standard_normal((B, D_IN)).astype(np.float16)).to(dev)
        y = torch.empty((B, D_OUT), dtype=torch.float16, device=dev)
        need = aqd.aqd_gemv_workspace_bytes(D_OUT, D_IN, M, B)
        ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=dev)
        for k in KS:
            def run():
                for c in copies:
                    aqd.aqd_gemv(c, cbd, sd, k, xr, D_OUT, D_IN, M, out=y, workspace=ws)
            run()
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                with torch.cuda.graph(graph, stream=side):
                    run()
            stream.wait_stream(side)
            graph.replay()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                graph.replay()
            b.record(stream)
            torch.cuda.synchronize()
            us = a.elapsed_time(b) * 1e3 / (reps * len(copies))
            byts = algorithmic_bytes(k, batch=B)
            res.append({"batch": B, "k": k, "us": us, "tokens_per_s": B * 1e6 / us,
                        "frac_hbm_peak": byts / us / 1e3 / HBM_PEAK_GBPS})
            del graph
    return res


def time_graph(torch, stream, run, reps: int) -> float:
    """Capture run() in one graph, replay it once untimed, then reps times between events on the launch
    stream; returns microseconds per replay."""
    run()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            run()
    stream.wait_stream(side)
    graph.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        graph.replay()
    b.record(stream)
    torch.cuda.synchronize()
    del graph
    return a.elapsed_time(b) * 1e3 / reps


# launch shapes of the streaming-read probe: (workgroups, waves per workgroup, loads in flight per lane,
# contiguous segment per workgroup)
PROBE_SHAPES = [(wg, w, u, c) for wg in (256, 512, 1024, 2048) for w in (4, 8, 16) for u in (4, 8) for c in (0, 1)]


def measure_read_probe(aqd, torch, dev, copies, stream, reps: int = 3):
    """The plain streaming-read kernel over the same bytes the k-codebook GEMV streams (the first k planes
    of each cold copy), 64 back-to-back launches per graph, every launch shape in PROBE_SHAPES; per k the
    fastest shape is what one launch can stream on this part."""
    sink = torch.zeros(65536, dtype=torch.int32, device=dev)
    res = {}
    for k in KS:
        nbytes = code_bytes(k)
        best = None
        for shape in PROBE_SHAPES:
            def run():
                for c in copies:
                    aqd.aqd_read_probe(c, nbytes, sink, *shape)
            us = time_graph(torch, stream, run, reps) / len(copies)
            if best is None or us < best[0]:
                best = (us, shape)
        us, (wg, w, u, c) = best
        res[str(k)] = {"bytes": nbytes, "us": us, "GBps": nbytes / us / 1e3,
                       "frac_hbm_peak": nbytes / us / 1e3 / HBM_PEAK_GBPS,
                       "best_shape": {"workgroups": wg, "waves": w, "loads_in_flight": u, "contiguous": bool(c)}}
    res["shapes_tried"] = len(PROBE_SHAPES)
    res["sink_written"] = int(torch.count_nonzero(sink).item())
    return res


def measure_small_batch(aqd, wl, torch, dev, copies: int = 32, reps: int = 2):
    """The matrix-core path on the 14336x4096 and 4096x14336 shapes at batch 16/32/64, k = 4 and 2, with
    the activation as bf16 hi/lo planes (three bf16 passes) and as fp16 (one pass)."""
    res = []
    for lin in wl.config(5):
        codes, cb, sc, _ = wl.layer_inputs(5, lin, batch=64)
        packed0 = aqd.aqd_pack_codes(torch.from_numpy(codes).to(dev))
        cps = [packed0] + [packed0.clone() for _ in range(copies - 1)]
        cbd, sd = torch.from_numpy(cb).to(dev), torch.from_numpy(sc).to(dev)
        g = np.random.Generator(np.random.PCG64(0x5B))
        x = torch.from_numpy(g.standard_normal((64, lin.d_in)).astype(np.float32)).to(dev).to(torch.bfloat16)
        xr = {"bf16x2": aqd.aqd_hadamard_rotate(x, lin.block, aqd.AQD_BF16X2),
              "f16": aqd.aqd_hadamard_rotate(x, lin.block, aqd.AQD_F16)}
        dts = {"bf16x2": aqd.AQD_BF16X2, "f16": aqd.AQD_F16}
        for mode in ("f16", "bf16x2"):
            for k in lin.ks:
                for B in lin.batches:
                    xb = xr[mode][..., :B, :].contiguous()
                    y = torch.empty((B, lin.d_out), dtype=torch.float32, device=dev)
                    need = aqd.aqd_gemm_small_batch_workspace_bytes(lin.d_out, lin.d_in, lin.M, B)
                    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)

                    def run(c):
                        aqd.aqd_gemm_small_batch(cps[c], cbd, sd, k, xb, lin.d_out, lin.d_in, lin.M, dts[mode],
                                                 out=y, workspace=ws)
                    for c in range(copies):
                        run(c)
                    torch.cuda.synchronize()
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record()
                    for _ in range(reps):
                        for c in range(copies):
                            run(c)
                    b.record()
                    torch.cuda.synchronize()
                    us = a.elapsed_time(b) * 1e3 / (reps * copies)
                    xbytes = (4 if mode == "bf16x2" else 2) * B * lin.d_in
                    byts = k * lin.d_out * (lin.d_in // 8) + xbytes + 4 * B * lin.d_out
                    flops = 2.0 * B * lin.d_out * lin.d_in
                    res.append({"shape": [lin.d_out, lin.d_in], "mode": mode, "k": k, "batch": B, "us": us,
                                "tokens_per_s": B * 1e6 / us,
                                "frac_hbm_peak": byts / us / 1e3 / HBM_PEAK_GBPS,
                                "frac_mfma_peak": flops / us / 1e6 / 2500.0})
        del cps, packed0
        torch.cuda.empty_cache()
    return res


FP32_VECTOR_PEAK_TFLOPS = 157.3


def measure_encode(aqd, wl, torch, dev, reps: int = 3):
    """Greedy residual encoding of the 4096x14336 layer (M = 4, N(0, 0.05) codebooks, rotated Gaussian
    weights and their row scales): time per layer, and the weight error of the encoded layer per k.
    Work per code group and codebook: 256 squared distances of 8 elements (8 subtractions and 8 fmas,
    24 flops each) plus the residual update; the kernel is fp32 ALU-bound."""
    d_out, d_in, M = 4096, 14336, 4
    g = wl.rng(0xE1)
    cb = wl.gen_codebooks(g, M)
    w, s, target = wl.gen_encode_targets(g, d_out, d_in, M)
    td, cbd = torch.from_numpy(target).to(dev), torch.from_numpy(cb).to(dev)
    codes = torch.empty((d_out, d_in // 8, M), dtype=torch.uint8, device=dev)
    aqd.aqd_encode_greedy(td, cbd, out=codes)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        aqd.aqd_encode_greedy(td, cbd, out=codes)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / reps
    groups = d_out * (d_in // 8)
    flops = groups * M * (256 * 24 + 8)
    # weight error of the encoded layer per k (a diagnostic, computed with torch on the device)
    wd = torch.from_numpy(w).to(dev)
    cbf = cbd.float()
    sd = torch.from_numpy(s).to(dev).float()[:, None]
    acc = torch.zeros((d_out, d_in // 8, 8), dtype=torch.float32, device=dev)
    errs = []
    for m in range(M):
        acc += cbf[m][codes[:, :, m].long()]
        errs.append(float(torch.linalg.norm(sd * acc.reshape(d_out, d_in) - wd) / torch.linalg.norm(wd)))
    del td, codes, wd, acc
    torch.cuda.empty_cache()
    return {"workload": "encode 4096x14336 (M = 4, g = 8): rotated N(0,1) weights, fp16 row scales, "
                        "N(0, 0.05) fp16 codebooks; greedy residual codes",
            "us": us, "weights_per_s": d_out * d_in * 1e6 / us,
            "roofline": {"bound": "alu", "achieved": flops / us / 1e6, "peak": FP32_VECTOR_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": flops / us / 1e6 / FP32_VECTOR_PEAK_TFLOPS},
            "rel_weight_error_per_k": errs}


def measure_prefill(aqd, wl, torch, dev, reps: int = 5):
    """Prefill (batch 128 / 512 / 2048 prompt tokens) through aqd_gemm_prefill (weights rebuilt per workgroup,
    or staged once as fp16 at the larger batches, then the matrix cores) on
    the 4096x14336 and 14336x4096 shapes, k = 2 and 4.  Beside each, the dense fp16 GEMM of the same shape
    through torch.matmul (the vendor GEMM library) on an uncompressed weight, as a reference point for what
    the matrix cores deliver on a plain GEMM here.  At these sizes the work is compute-bound, so no cold
    copies are needed."""
    res = []
    M = 4
    for d_out, d_in in ((4096, 14336), (14336, 4096)):
        g = wl.rng(0x9F, extra=d_out)
        packed = aqd.aqd_pack_codes(torch.from_numpy(wl.gen_codes(g, d_out, d_in, M)).to(dev))
        cbd = torch.from_numpy(wl.gen_codebooks(g, M)).to(dev)
        sd = torch.from_numpy(wl.gen_scales(g, d_out)).to(dev)
        W = torch.randn((d_out, d_in), device=dev, dtype=torch.float32).to(torch.float16)
        for B in (128, 512, 2048):
            x = torch.randn((B, d_in), device=dev, dtype=torch.float32).to(torch.float16)
            y = torch.empty((B, d_out), dtype=torch.float32, device=dev)
            need = aqd.aqd_gemm_prefill_workspace_bytes(d_out, d_in, M, B)
            ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)

            def timed(fn):
                # a short idle gap first, so that no case starts on a clock the previous one (the dense
                # GEMM in particular, at full matrix-core load) has pushed down
                torch.cuda.synchronize()
                time.sleep(0.25)
                for _ in range(2):
                    fn()
                torch.cuda.synchronize()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                for _ in range(reps):
                    fn()
                b.record()
                torch.cuda.synchronize()
                return a.elapsed_time(b) * 1e3 / reps
            us_dense = timed(lambda: torch.matmul(x, W.t()))
            flops = 2.0 * B * d_out * d_in
            for k in (2, 4):
                us = timed(lambda: aqd.aqd_gemm_prefill(packed, cbd, sd, k, x, d_out, d_in, M, out=y, workspace=ws))
                res.append({"shape": [d_out, d_in], "k": k, "batch": B, "us": us, "tokens_per_s": B * 1e6 / us,
                            "tflops": flops / us / 1e6, "frac_mfma_peak": flops / us / 1e6 / 2500.0,
                            "dense_fp16_gemm_us": us_dense, "dense_fp16_gemm_tflops": flops / us_dense / 1e6})
            del x, y, ws
        del packed, W
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of CPU work for the oracle baseline")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline (profiling runs)")
    ap.add_argument("--no-eager", action="store_true", help="skip the eager (one Python call per launch) timing")
    ap.add_argument("--no-stack", action="store_true", help="skip the 32-layer decoder-stack measurement")
    ap.add_argument("--no-small-batch", action="store_true", help="skip the small-batch matrix-core measurement")
    ap.add_argument("--no-batched", action="store_true", help="skip the batch 2/4/8 GEMV measurement")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill (batch 128..2048) measurement")
    ap.add_argument("--no-encode", action="store_true", help="skip the encoder measurement")
    ap.add_argument("--no-probe", action="store_true", help="skip the streaming-read probe")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one plain 64 MiB device copy first (scale reference for memory counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU only: the library has no multi-GPU path "
                                   "(each GPU would run the same kernels on its own shard of rows)"}))
        sys.exit(2)

    import torch

    import additive_codebook_gemv_amd as aqd
    import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    lin = [l for l in wl.config(CONFIG_ID) if l.name == "down4096x14336"][0]
    codes, cb, s, x = wl.layer_inputs(CONFIG_ID, lin, batch=BATCH)

    packed0 = aqd.aqd_pack_codes(torch.from_numpy(codes).to(dev))
    copies = [packed0] + [packed0.clone() for _ in range(N_COPIES - 1)]
    cbd = torch.from_numpy(cb).to(dev)
    sd = torch.from_numpy(s).to(dev)
    xd = torch.from_numpy(x).to(dev)
    xr = torch.empty((BATCH, D_IN), dtype=torch.float16, device=dev)
    ys = {k: torch.empty((BATCH, D_OUT), dtype=torch.float16, device=dev) for k in KS}
    ws = None
    need = aqd.aqd_gemv_workspace_bytes(D_OUT, D_IN, M, BATCH)
    if need:
        ws = torch.zeros(need, dtype=torch.uint8, device=dev)

    if args.calibrate_copy:
        src = torch.ones(64 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    aqd.aqd_hadamard_rotate(xd, BLOCK, aqd.AQD_F16, out=xr)
    y_check = {k: aqd.aqd_gemv(copies[5], cbd, sd, k, xr, D_OUT, D_IN, M, out=ys[k], workspace=ws).cpu().numpy()
               for k in KS}

    stream = torch.cuda.current_stream()
    ctr = [0]

    def gemv(k):
        c = copies[ctr[0] % N_COPIES]
        ctr[0] += 1
        aqd.aqd_gemv(c, cbd, sd, k, xr, D_OUT, D_IN, M, out=ys[k], workspace=ws)

    def rotate():
        aqd.aqd_hadamard_rotate(xd, BLOCK, aqd.AQD_F16, out=xr)

    for _ in range(args.warmup):
        rotate()
        for k in KS:
            gemv(k)
    torch.cuda.synchronize()

    # The K timed steps are issued in TIMING_ROUNDS rounds.  Each round replays, in turn, a graph of
    # about K / TIMING_ROUNDS rotations and one of about K / TIMING_ROUNDS GEMVs at each k (a Python
    # launch costs more than a short kernel takes), with an event after every graph.  Every step's
    # work is done exactly once, each kernel's time is the sum of its graphs' event intervals, and no
    # kernel is always the one timed last (after milliseconds of back-to-back streaming the part can
    # sustain less than at the start).
    rounds = max(1, min(TIMING_ROUNDS, args.steps))
    seg = [args.steps // rounds + (1 if r < args.steps % rounds else 0) for r in range(rounds)]

    def capture(fn, n):
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for _ in range(n):
                    fn()
        stream.wait_stream(side)
        return g

    kernels = [rotate] + [lambda k=k: gemv(k) for k in KS]
    graphs = [[capture(fn, seg[r]) for fn in kernels] for r in range(rounds)]
    for row in graphs:
        for g in row:
            g.replay()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(rounds * len(kernels) + 1)]
    t0 = time.perf_counter()
    evs[0].record(stream)
    i = 0
    for row in graphs:
        for g in row:
            g.replay()
            i += 1
            evs[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = evs[0].elapsed_time(evs[-1])
    kernel_ms = [0.0] * len(kernels)
    for r in range(rounds):
        for j in range(len(kernels)):
            e = r * len(kernels) + j
            kernel_ms[j] += evs[e].elapsed_time(evs[e + 1])
    rot_us = kernel_ms[0] * 1e3 / args.steps
    per_k = {}
    for i, k in enumerate(KS):
        us = kernel_ms[i + 1] * 1e3 / args.steps
        per_k[k] = {
            "us_per_gemv": us,
            "code_bytes": code_bytes(k),
            "algorithmic_bytes": algorithmic_bytes(k),
            "GBps": algorithmic_bytes(k) / us / 1e3,
            "frac_hbm_peak": algorithmic_bytes(k) / us / 1e3 / HBM_PEAK_GBPS,
            "frac_hbm_peak_code_stream": code_bytes(k) / us / 1e3 / HBM_PEAK_GBPS,
        }
    del graphs

    # the same launches issued one by one from Python (launch-rate bound for the short kernels)
    if not args.no_eager:
        reps = 50
        for k in KS:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                gemv(k)
            b.record(stream)
            torch.cuda.synchronize()
            per_k[k]["us_per_gemv_eager"] = a.elapsed_time(b) * 1e3 / reps

    probe = None if args.no_probe else measure_read_probe(aqd, torch, dev, copies, stream)
    if probe is not None:
        for k in KS:
            per_k[k]["read_probe_us"] = probe[str(k)]["us"]
            per_k[k]["frac_of_read_probe"] = probe[str(k)]["us"] / per_k[k]["us_per_gemv"]
    batched = None if args.no_batched else measure_batched_gemv(aqd, torch, dev, copies, cbd, sd, stream)
    stack = None if args.no_stack else measure_stack(aqd, wl, torch, dev)
    small = None if args.no_small_batch else measure_small_batch(aqd, wl, torch, dev)
    tiered = None if args.no_small_batch else measure_tiered(aqd, wl, torch, dev)
    prefill = None if args.no_prefill else measure_prefill(aqd, wl, torch, dev)
    encode = None if args.no_encode else measure_encode(aqd, wl, torch, dev)

    value = float(np.mean([per_k[k]["us_per_gemv"] for k in KS]))
    k4 = per_k[4]
    result = {
        "metric": "µs per GEMV and % of HBM roofline at k=1..4 codebooks, 4096×14336 batch 1",
        "value": value,
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": gpu_ms / args.steps,
        "ms_per_step_host_wall": wall * 1e3 / args.steps,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "down-projection decode linear 4096x14336 (d_out 4096, d_in 14336), batch 1, "
                        "M=4 uint8 code planes, g=8, fp16 codebooks N(0,0.05), fp16 scales U(0.5,1.5), "
                        "Hadamard block 256, k=1..4, 64 cold copies of the codes",
            "d_out": D_OUT, "d_in": D_IN, "M": M, "k": list(KS), "batch": BATCH, "block": BLOCK,
            "accumulate": "f32", "cold_copies": N_COPIES,
        },
        "us_rotation": rot_us,
        "per_k": {str(k): v for k, v in per_k.items()},
        "roofline": {
            "bound": "hbm",
            "kernel": "gemv k=4",
            "achieved": k4["GBps"],
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": k4["frac_hbm_peak"],
            "traffic": measured_traffic(),
        },
    }
    if probe is not None:
        result["read_probe"] = probe
    if batched is not None:
        result["gemv_batch_2_4_8"] = batched
    if stack is not None:
        result["stack"] = stack
    if small is not None:
        result["small_batch"] = small
    if tiered is not None:
        result["tiered_batch"] = tiered
    if prefill is not None:
        result["prefill"] = prefill
    if encode is not None:
        result["encode"] = encode
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(codes, cb, s, x, args.cpu_budget, y_check)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
