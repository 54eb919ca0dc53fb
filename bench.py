#!/usr/bin/env python3
"""Benchmark of the integer-dot block-quantized matmul on one MI355X.

Default workload: Qwen3-8B-shaped decode (hidden 4096, 36 layers; Q 4096x4096,
K/V 1024x4096, O 4096x4096, gate/up 12288x4096, down 4096x12288; V and down in
Q6_K, the rest Q4_K), seeded synthetic weights resident in HBM.  One step is one
pass of the whole path for M = 1, 2, 4 and 8 token rows: per layer, four
activation quantizations (qkv input, o input, gate/up input, down input) and the
seven qmatmuls.  At M = 1 (--fused-max-m) the quantizations run inside the
matmul launches (qdot_quantize_qmatmul[_multi], bitwise the same results),
which measured faster there than a separate quantize launch, except with
IQ4_XS weights and for launches whose workgroups would repeat more than 4 M
quantized values (gate+up); elsewhere, one quantize launch per input.  Every matrix is cold in the 256 MB Infinity Cache because a
36-layer sweep streams 4.4 GB.

Timing: each M's 36-layer sweep is captured once in a HIP graph; the timed
region replays the step graphs between HIP events (no host launch overhead in
the measurement).  Per-kernel durations come from graphs holding one
projection's 36 launches, replayed between HIP events on the same stream
(ROCm does not allow timing events inside a captured graph); they include the
graph's sub-microsecond dispatch gaps, so they are slightly conservative
against the rocprofv3 kernel trace.

Output: one JSON line (metric, value = whole-step weight GB/s, roofline of the
dominant kernel, the CPU oracle's rate on a bounded sample, per-M details).
"""
import argparse
import ctypes
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_I8_PEAK_TOPS = 5000.0     # MI355X dense int8 MFMA, published (TOP/s)
METRIC = "weight GB/s (% HBM peak) and µs per qmatmul at M=1,2,4,8; Qwen3-8B shapes"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="qwen3-8b-decode",
                   choices=["qwen3-8b-decode", "qwen3-8b-prefill-512", "iq4xs-h5120-decode",
                            "qwen2.5-1.5b-decode", "qwen3-8b-q4_0-q8_0-decode", "qwen3-8b-mid-batch",
                            "qwen3-8b-rmsnorm-q8_1", "q4k-matvec-1536", "qwen3-8b-attn-kv4-32k",
                            "qwen3-8b-tp8-shard-decode"])
    p.add_argument("--ms", default=None, help="comma-separated M values (default per workload)")
    p.add_argument("--ctx", type=int, default=32768,
                   help="context length of the attention workload (tokens in the KV cache)")
    p.add_argument("--layers", type=int, default=None, help="override the layer count")
    p.add_argument("--same-weights", action="store_true",
                   help="every layer reads layer 0's weights (cache-hot timing of the same launches)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-check", action="store_true", help="skip the sampled oracle check")
    p.add_argument("--kernel-reps", type=int, default=None,
                   help="replays of each per-projection graph, the median of which is reported "
                        "(default: 20 or --steps, whichever is larger)")
    p.add_argument("--fused-max-m", type=int, default=1,
                   help="largest M whose launches quantize the activations in the matmul kernel "
                        "(qdot_quantize_qmatmul[_multi]) instead of a separate quantize launch; 0 = never")
    p.add_argument("--no-shard-rows", action="store_true",
                   help="skip the tensor-parallel share rows of the decode workload")
    p.add_argument("--no-prefill-row", action="store_true",
                   help="skip the M = 512 prefill row of the decode workload")
    p.add_argument("--separate", action="store_true",
                   help="one launch per projection (default: projections sharing an input in one "
                        "qdot_qmatmul_multi launch for M <= 8)")
    p.add_argument("--eager-only", action="store_true",
                   help="run the sweep eagerly --steps times per M and exit (for counter passes)")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="run only a plain device copy of this size (PMC calibration) and exit")
    return p.parse_args()


def workload_def(name):
    from quant_integer_dot_amd import synth
    if name == "qwen3-8b-decode":
        return 2, synth.QWEN3_8B, 36, [1, 2, 4, 8]
    if name == "qwen3-8b-prefill-512":
        return 4, synth.QWEN3_8B, 36, [512]
    if name == "iq4xs-h5120-decode":
        return 3, synth.IQ4XS_H5120, 64, [1, 2, 4, 8]
    if name == "qwen2.5-1.5b-decode":
        return 1, synth.QWEN25_1P5B, 28, [1, 2, 4, 8]
    if name == "qwen3-8b-q4_0-q8_0-decode":
        return 5, synth.QWEN3_8B_Q40_Q80, 36, [1, 2, 4, 8]
    if name == "qwen3-8b-mid-batch":
        return 6, synth.QWEN3_8B, 36, [16, 32, 64, 96]
    if name == "qwen3-8b-tp8-shard-decode":
        return 7, synth.QWEN3_8B_TP8, 36, list(range(1, 9))
    if name == "q4k-matvec-1536":
        # One 1536 x 1536 Q4_K matrix at M = 1, as 400 distinct seeded copies
        # (531 MB, over twice the 256 MB Infinity Cache) launched in turn, so
        # every launch reads its weights from HBM; --layers 1 repeats a single
        # copy, which then stays in cache (the hot figure).
        return 0, [("w", 1536, 1536, synth.Q4_K)], 400, [1]
    raise ValueError(name)


# The HIP kernel function behind each kernel label of qdot_kernel_name (and
# of the grouped decode launch).
KERNEL_FUNCTION = {"qmv_dot4": "qmv_kernel", "qmv_mfma": "qmv_kernel", "qmv_multi": "qmv_multi_kernel",
                   "qmv_dot4q": "qmv_kernel",
                   "qmm_skinny": "qmm_skinny_kernel", "qmm_mfma": "qmm_mfma_kernel",
                   "quantize_q8_1": "quantize_q8_1_kernel"}

# The input each projection reads: projections sharing an input share one
# activation quantization (xLLM v0.7 log, section C: one d_xn_q8 per step).
INPUT_OF = {"q": "attn", "k": "attn", "v": "attn", "qkv": "attn", "o": "o",
            "gate": "ffn", "up": "ffn", "down": "down", "w": "attn"}


def kernel_source_digest(files):
    """First 16 hex digits of sha256 over the named csrc/ files (in order)."""
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "quant_integer_dot_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel, workload):
    """HBM bytes per launch from a committed counter summary (profiles/hbm_traffic_*.md),
    or None when there is none for this kernel and workload or when the kernel's
    sources have changed since the counters were taken."""
    import glob
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "hbm_traffic_*.md"))):
        kv = {}
        with open(path) as fh:
            for line in fh:
                if ": " in line and not line.startswith(("|", "#", " ")):
                    k, v = line.rstrip("\n").split(": ", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("kernel") != kernel or kv.get("workload") != workload:
            continue
        files = kv.get("source_files", "").split()
        if not files or kernel_source_digest(files) != kv.get("source_digest"):
            return None
        return int(kv["traffic_bytes_per_launch"])
    return None


def graph_median_ms(g, reps):
    """Median over `reps` replays of a captured graph, each replay between its
    own pair of HIP events on the current stream (ms per replay)."""
    import numpy as np
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in evs]))


def copy_calibration(mib):
    import torch
    n = mib * 1024 * 1024
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)


def copy_reference(dev, launch_bytes, reps=10):
    """Measured HBM reference for the decode roofline: device-to-device copies
    (torch copy_, i.e. the runtime's copy kernel), counting the bytes read plus
    the bytes written.  Once as one 512 MiB copy (streaming rate), once as 36
    copies of the dominant kernel's bytes per launch, each from its own buffer
    (every copy cold in the Infinity Cache), timed together between HIP events
    (what a single launch of that size reaches)."""
    import torch
    out = {}
    n = 512 << 20
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty(n, dtype=torch.uint8, device=dev)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    out["copy_512MiB_GBps"] = round(2 * n * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    del a, b
    m = int(launch_bytes) // 256 * 256
    srcs = [torch.ones(m, dtype=torch.uint8, device=dev) for _ in range(36)]
    dsts = [torch.empty(m, dtype=torch.uint8, device=dev) for _ in range(36)]
    for s_, d_ in zip(srcs, dsts):
        d_.copy_(s_)
    torch.cuda.synchronize()
    e0.record()
    for s_, d_ in zip(srcs, dsts):
        d_.copy_(s_)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / 36
    out["copy_at_launch_size"] = {"bytes_per_copy": m, "us": round(t * 1e6, 3),
                                  "GBps": round(2 * m / t / 1e9, 1)}
    return out


def cpu_info():
    """Host CPU model (from /proc/cpuinfo) and the cores this process may use."""
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:
        nproc = os.cpu_count()
    return model, nproc


def cpu_baseline(shapes, cfg_idx, Ms, prefill=False, layers=36):
    """The CPU oracle (plain scalar C, fp64) timed on a bounded sample of the
    same workload, twice: on one thread and on every thread OpenMP gives it
    (OMP_NUM_THREADS, else all cores), with the loop over output rows split
    across threads (no change to any output's arithmetic).  It is a
    correctness reference, not a tuned CPU kernel.
      decode:  layer 0's projections, whole matmuls at every M (quantize +
               qmatmul), in weight GB/s;
      prefill: the full q (4096 x 4096) and down (4096 x 12288) matrices at
               M = 512 on all threads, 256 weight rows of each on one thread,
               in int8 TOP/s (2 ops per MAC); the 36-layer sweep time is
               extrapolated from that rate and labelled as such."""
    import numpy as np
    import oracle
    from quant_integer_dot_amd import synth
    model, nproc = cpu_info()

    def timed(threads, jobs):
        oracle.set_threads(threads)
        used = oracle.max_threads()
        t0 = time.perf_counter()
        for fn in jobs:
            fn()
        return time.perf_counter() - t0, used

    note = "the oracle: plain scalar C, fp64; a correctness reference, not a tuned CPU kernel"
    if prefill:
        picks = [(pi, sh) for pi, sh in enumerate(shapes) if sh[0] in ("q", "down")]
        M = Ms[0]
        data = []
        for pi, (name, N, K, t) in picks:
            W = synth.weights(t, N, K, synth.weight_seed(cfg_idx, 0, pi))
            x = synth.activations(M, K, synth.act_seed(cfg_idx, K, M))
            data.append((name, N, K, t, W, x))
        rows = np.arange(256)
        one = [lambda d=d: oracle.qmatmul_rows(d[4], d[3], d[1], d[2], oracle.quantize_q8_1(d[5]), M, rows)
               for d in data]
        full = [lambda d=d: oracle.qmatmul(d[4], d[3], d[1], d[2], oracle.quantize_q8_1(d[5]), M) for d in data]
        ops_one = sum(2 * M * rows.size * d[2] for d in data)
        ops_full = sum(2 * M * d[1] * d[2] for d in data)
        t1, _ = timed(1, one)
        tn, used = timed(0, full)
        oracle.set_threads(0)
        rate = ops_full / tn / 1e12
        sweep_ops = sum(2 * M * N * K for _, N, K, _ in shapes) * layers
        names = " and ".join(f"{d[0]} {d[1]}x{d[2]}" for d in data)
        return {"value": round(rate, 6), "unit": "TOP/s", "cores": used, "kind": "oracle",
                "sample": f"layer 0 of the same workload: the full {names} matrices at M={M} "
                          f"({ops_full / 1e9:.1f} G int8 ops, {tn:.1f} s on {used} threads); single thread: "
                          f"256 weight rows of each ({ops_one / 1e9:.1f} G ops, {t1:.1f} s)",
                "single_thread": {"value": round(ops_one / t1 / 1e12, 6), "unit": "TOP/s", "cores": 1},
                "sweep_s_extrapolated": round(sweep_ops / (rate * 1e12), 1),
                "sweep_note": f"extrapolated: {sweep_ops / 1e12:.2f} T int8 ops per {layers}-layer sweep "
                              f"at the all-threads rate",
                "nproc": nproc, "cpu_model": model, "note": note}
    jobs, parts, wbytes = [], [], 0
    for M in Ms:
        for pi, (name, N, K, t) in enumerate(shapes):
            W = synth.weights(t, N, K, synth.weight_seed(cfg_idx, 0, pi))
            x = synth.activations(M, K, synth.act_seed(cfg_idx, K, M))
            jobs.append(lambda W=W, t=t, N=N, K=K, x=x, M=M:
                        oracle.qmatmul(W, t, N, K, oracle.quantize_q8_1(x), M))
            wbytes += W.nbytes
            parts.append(f"{name}@M={M}")
    t1, _ = timed(1, jobs)
    tn, used = timed(0, jobs)
    oracle.set_threads(0)
    return {"value": round(wbytes / tn / 1e9, 4), "unit": "GB/s", "cores": used, "kind": "oracle",
            "sample": f"layer 0 of the same workload, whole matmuls: {', '.join(parts)} "
                      f"({wbytes / 1e6:.1f} MB of weights, quantize + qmatmul per projection; "
                      f"{tn:.2f} s on {used} threads, {t1:.1f} s on one)",
            "single_thread": {"value": round(wbytes / t1 / 1e9, 4), "unit": "GB/s", "cores": 1},
            "nproc": nproc, "cpu_model": model, "note": note}


def stream_reference(dev, launch_bytes, reps=10):
    """Measured read-only reference for the decode roofline: the library's
    plain streaming read kernel (qdot_stream_read), once over 512 MiB (the
    streaming rate) and once as 36 reads of the dominant kernel's bytes per
    launch, each from its own buffer (cold in the Infinity Cache), timed
    together between HIP events (what one launch of that size reaches)."""
    import torch
    from quant_integer_dot_amd import binding as qd
    out = {}
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    n = 512 << 20
    a = torch.ones(n, dtype=torch.uint8, device=dev)
    for _ in range(3):
        qd.qdot_stream_read(a, n, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        qd.qdot_stream_read(a, n, sink)
    e1.record()
    torch.cuda.synchronize()
    out["read_512MiB_GBps"] = round(n * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    del a
    m = int(launch_bytes) // 256 * 256
    srcs = [torch.ones(m, dtype=torch.uint8, device=dev) for _ in range(36)]
    for b_ in srcs:
        qd.qdot_stream_read(b_, m, sink)
    torch.cuda.synchronize()
    e0.record()
    for b_ in srcs:
        qd.qdot_stream_read(b_, m, sink)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / 36
    out["read_at_launch_size"] = {"bytes_per_read": m, "us": round(t * 1e6, 3), "GBps": round(m / t / 1e9, 1)}
    return out


def shard_rows_shapes():
    """The FFN matrices of one GPU's 8-way tensor-parallel share: gate and up
    column-parallel (1536 x 4096), down row-parallel (4096 x 1536)."""
    from quant_integer_dot_amd import synth
    return [s for s in synth.QWEN3_8B_TP8 if s[0] in ("gate", "up", "down")]


def shard_rows(dev, fused_max_m, reps, per_m_full, check=True):
    """Per-launch timing of the tensor-parallel FFN share at M = 1..8 on this
    one GPU: gate+up (one grouped launch) and down, 36 distinct seeded layers
    (440 MB, cold in the 256 MB Infinity Cache), each launch list captured in
    a graph and replayed between HIP events, with the full-shape rows of the
    same step beside them where that M is in the step."""
    import numpy as np
    import torch
    from quant_integer_dot_amd import binding as qd
    from quant_integer_dot_amd import synth

    shapes = shard_rows_shapes()
    cfg_idx, layers = 7, 36
    pidx = {n: i for i, (n, *_) in enumerate(synth.QWEN3_8B_TP8)}
    W = [[torch.from_numpy(synth.weights(t, N, K, synth.weight_seed(cfg_idx, layer, pidx[n]))).to(dev)
          for n, N, K, t in shapes] for layer in range(layers)]
    out = {}
    bad = nchk = 0
    for M in range(1, 9):
        fz = M <= fused_max_m
        xs, xqs, ys = {}, {}, {}
        for K in (4096, 1536):
            x = torch.from_numpy(synth.activations(M, K, synth.act_seed(cfg_idx, K, M))).to(dev)
            xq = torch.empty(qd.qdot_q8_1_bytes(M, K), dtype=torch.uint8, device=dev)
            qd.qdot_quantize_q8_1(x, M, K, xq)
            xs[K], xqs[K] = x, xq
        for n, N, K, t in shapes:
            ys[n] = torch.empty((M, N), dtype=torch.float32, device=dev)
        gate, up, down = shapes

        def launch(label, layer):
            if label == "gate+up":
                Ws, ts, Ns = W[layer][:2], [gate[3], up[3]], [gate[1], up[1]]
                if fz:
                    qd.qdot_quantize_qmatmul_multi(Ws, ts, Ns, 4096, xs[4096], M, [ys["gate"], ys["up"]])
                else:
                    qd.qdot_qmatmul_multi(Ws, ts, Ns, 4096, xqs[4096], M, [ys["gate"], ys["up"]])
            else:
                _, N, K, t = down
                if fz:
                    qd.qdot_quantize_qmatmul(W[layer][2], t, N, K, xs[K], M, ys["down"])
                else:
                    qd.qdot_qmatmul(W[layer][2], t, N, K, xqs[K], M, ys["down"])

        rows = {}
        for label in ("gate+up", "down"):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for layer in range(layers):
                    launch(label, layer)
            g.replay()
            torch.cuda.synchronize()
            us = graph_median_ms(g, reps) * 1e3 / layers
            mats = shapes[:2] if label == "gate+up" else shapes[2:]
            wb = sum(qd.qdot_weight_bytes(t, N, K) for _, N, K, t in mats)
            K = mats[0][2]
            if fz:
                tiles = [f"qmv_dot4q<{synth.TYPE_NAMES[t]},{M}>" for *_, t in mats]
            elif len(mats) == 2:
                tiles = [qd.qdot_multi_kernel_name([t for *_, t in mats], [N for _, N, _, _ in mats], K, M, i)
                         for i in range(2)]
            else:
                tiles = [qd.qdot_kernel_name_shape(mats[0][3], mats[0][1], K, M)]
            row = {"shape": " + ".join(f"{N}x{K} {synth.TYPE_NAMES[t]}" for _, N, K, t in mats),
                   "us": round(us, 3), "weight_GBps": round(wb / us / 1e3, 1),
                   "pct_hbm_peak": round(100 * wb / us / 1e3 / HBM_PEAK_GBS, 1), "tiles": tiles}
            full = (per_m_full or {}).get(str(M), {}).get("qmatmul", {}).get(label)
            if full:
                row["full_shape"] = {"us": full["us"], "pct_hbm_peak": full["pct_hbm_peak"]}
            rows[label] = row
        if check:
            import oracle
            for layer_label in ("gate+up", "down"):
                launch(layer_label, layers - 1)
            torch.cuda.synchronize()
            for i, (n, N, K, t) in enumerate(shapes):
                Wh = synth.weights(t, N, K, synth.weight_seed(cfg_idx, layers - 1, pidx[n]))
                xq = oracle.quantize_q8_1(xs[K].cpu().numpy())
                r = np.random.default_rng(700 + 10 * M + i).integers(0, N, 8)
                y64, _ = oracle.qmatmul_rows(Wh, t, N, K, xq, M, r)
                yg = ys[n].cpu().numpy()[:, r].astype(np.float64)
                bad += int((np.abs(yg - y64) > 1e-5 * np.abs(y64)).sum())
                nchk += y64.size
        out[str(M)] = rows
    res = {"what": "one GPU's share of 8-way tensor parallelism: gate/up split by rows (column-parallel), "
                   "down by K (row-parallel); 36 distinct layers, cold; no collective runs",
           "per_M": out}
    if check:
        res["sampled_check"] = {"outputs_checked": nchk, "outside_1e-5_rel": bad}
        if bad:
            log(f"[bench] SHARD ROWS CHECK FAILED: {bad} of {nchk} outputs")
    return res


def prefill_row(dev, Wdev, shapes, cfg_idx, layers, reps, check=True):
    """The M = 512 prefill sweep on the decode line's resident weights (the
    same 36 Qwen3-8B layers): one quantize launch per input and layer, then
    one qdot_qmatmul per projection, captured in a graph and replayed between
    HIP events; int8 TOP/s against the MFMA int8 peak, with a sampled oracle
    check of the last layer."""
    import numpy as np
    import torch
    from quant_integer_dot_amd import binding as qd
    from quant_integer_dot_amd import synth

    M = 512
    inputs = sorted({INPUT_OF[name] for name, *_ in shapes})
    in_K = {INPUT_OF[name]: K for name, N, K, t in shapes}
    xs = {i: torch.from_numpy(synth.activations(M, in_K[i], synth.act_seed(cfg_idx, in_K[i], M))).to(dev)
          for i in inputs}
    xqs = {i: torch.empty(qd.qdot_q8_1_bytes(M, in_K[i]), dtype=torch.uint8, device=dev) for i in inputs}
    ys = {name: torch.empty((M, N), dtype=torch.float32, device=dev) for name, N, K, t in shapes}

    def sweep():
        for layer in range(layers):
            for i in inputs:
                qd.qdot_quantize_q8_1(xs[i], M, in_K[i], xqs[i])
                for pi, (name, N, K, t) in enumerate(shapes):
                    if INPUT_OF[name] == i:
                        qd.qdot_qmatmul(Wdev[layer][pi], t, N, K, xqs[i], M, ys[name])

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sweep()
    g.replay()
    torch.cuda.synchronize()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    a, b = ev(), ev()
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    ops = sum(2 * M * N * K for _, N, K, _ in shapes) * layers
    tops = ops / (ms * 1e-3) / 1e12
    res = {"what": "M = 512 prefill sweep over the same resident weights (quantize launches included)",
           "M": M, "ms_per_sweep": round(ms, 3), "int8_TOPs": round(tops, 1),
           "pct_mfma_i8_peak": round(100 * tops / MFMA_I8_PEAK_TOPS, 2),
           "kernels": sorted({qd.qdot_kernel_name_shape(t, N, K, M) for _, N, K, t in shapes})}
    if check:
        import oracle
        bad = nchk = 0
        for pi, (name, N, K, t) in enumerate(shapes):
            Wh = synth.weights(t, N, K, synth.weight_seed(cfg_idx, layers - 1, pi))
            xq = oracle.quantize_q8_1(xs[INPUT_OF[name]].cpu().numpy())
            r = np.random.default_rng(900 + pi).integers(0, N, 4)
            y64, _ = oracle.qmatmul_rows(Wh, t, N, K, xq, M, r)
            yg = ys[name].cpu().numpy()[:, r].astype(np.float64)
            bad += int((np.abs(yg - y64) > 1e-5 * np.abs(y64)).sum())
            nchk += y64.size
        res["sampled_check"] = {"outputs_checked": nchk, "outside_1e-5_rel": bad}
        if bad:
            log(f"[bench] PREFILL ROW CHECK FAILED: {bad} of {nchk} outputs")
    return res


def producer_bench(args):
    """The fused RMSNorm + Q8_1 producer at the Qwen3-8B hidden size (K = 4096):
    one step = 36 layers x 2 norms (attention and FFN input) for each M in
    1, 2, 4, 8, captured in HIP graphs like the matmul step; the standalone
    quantizer on the same rows is timed beside it.  Bytes per launch: x read
    (4MK), w read (4K), Q8_1 written (36MK/32)."""
    import numpy as np
    import torch
    from quant_integer_dot_amd import binding as qd
    from quant_integer_dot_amd import synth
    L = qd.load()
    dev = torch.device("cuda:0")
    K, layers, Ms = 4096, 36, [int(v) for v in args.ms.split(",")] if args.ms else [1, 2, 4, 8]
    if args.layers:
        layers = args.layers
    n = 2 * layers
    bufs = {}
    for M in Ms:
        xs = [torch.from_numpy(synth.activations(M, K, (2026, 90, M, i))).to(dev) for i in range(n)]
        ws = [torch.from_numpy((1.0 + 0.1 * synth.activations(1, K, (2026, 91, i))[0]).astype(np.float32)).to(dev)
              for i in range(n)]
        qs = [torch.empty(qd.qdot_q8_1_bytes(M, K), dtype=torch.uint8, device=dev) for _ in range(n)]
        bufs[M] = (xs, ws, qs)

    def sweep(M, fused):
        s = torch.cuda.current_stream(dev).cuda_stream
        xs, ws, qs = bufs[M]
        for i in range(n):
            if fused:
                rc = L.qdot_rmsnorm_quantize_q8_1(xs[i].data_ptr(), ws[i].data_ptr(), ctypes.c_float(1e-6), M, K,
                                                  qs[i].data_ptr(), s)
            else:
                rc = L.qdot_quantize_q8_1(xs[i].data_ptr(), M, K, qs[i].data_ptr(), s)
            assert rc == 0, rc

    def timed(fused):
        graphs = {}
        for M in Ms:
            sweep(M, fused)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                sweep(M, fused)
            graphs[M] = g
        for _ in range(args.warmup):
            for M in Ms:
                graphs[M].replay()
        torch.cuda.synchronize()
        per = {}
        for M in Ms:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(args.steps):
                graphs[M].replay()
            b.record()
            torch.cuda.synchronize()
            per[M] = a.elapsed_time(b) / args.steps
        return per

    fused = timed(True)
    quant = timed(False)
    # sampled check: last launch of each M against the oracle
    check = None
    if not args.no_check:
        import oracle
        bad = 0
        for M in Ms:
            xs, ws, qs = bufs[M]
            sweep(M, True)
            torch.cuda.synchronize()
            exp = oracle.rmsnorm_quantize_q8_1(xs[-1].cpu().numpy(), ws[-1].cpu().numpy(), np.float32(1e-6))
            bad += int((qs[-1].cpu().numpy() != exp.reshape(-1)).sum())
        check = {"bytes_differing": bad}
    ms_step = sum(fused.values())
    byt = {M: 4 * M * K + 4 * K + qd.qdot_q8_1_bytes(M, K) for M in Ms}
    total = sum(byt[M] * n for M in Ms)
    per_launch_us = ms_step * 1e3 / (n * len(Ms))
    achieved = total / (ms_step * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < 10.0:
            for M in Ms:
                xs, ws, _ = bufs[M]
                oracle.rmsnorm_quantize_q8_1(xs[0].cpu().numpy(), ws[0].cpu().numpy(), np.float32(1e-6))
            reps += 1
        dt = time.perf_counter() - t0
        cpu = {"value": round(reps * sum(byt.values()) / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
               "kind": "oracle", "sample": f"{reps} passes over one launch per M ({dt:.1f} s, single thread)"}
    print(json.dumps({
        "metric": "GB/s (x and w read, Q8_1 written) of the fused RMSNorm + Q8_1 producer, Qwen3-8B hidden 4096",
        "value": round(achieved, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": args.workload, "K": K, "layers": layers, "M": Ms, "launches_per_step": n * len(Ms)},
        "roofline": {"bound": "hbm", "kernel": "rmsnorm_q8_1_kernel", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 5),
                     "traffic": recorded_traffic("rmsnorm_q8_1_kernel", args.workload),
                     "launches": n * len(Ms), "avg_launch_us": round(per_launch_us, 3),
                     "algorithmic_bytes_per_launch": round(total / (n * len(Ms)))},
        "per_M_us": {str(M): {"fused_rmsnorm_q8_1": round(fused[M] * 1e3 / n, 3),
                              "quantize_q8_1_alone": round(quant[M] * 1e3 / n, 3)} for M in Ms},
        "cpu_baseline": cpu, "sampled_check": check}), flush=True)


def attention_bench(args):
    """Decode attention over the 4-bit KV cache (qdot_attn_decode_kv4) with
    Qwen3-8B heads (32 query heads, 8 KV heads, D = 128) at a 32K-token
    context: one step = 36 layers, each quantizing its query (Q8_1) and
    attending over its own cache, captured in one HIP graph.  The cache of
    every layer is distinct (36 x 37.7 MB), so each step streams it from HBM
    as on the pages' long-context path.  Algorithmic bytes per attention
    call: K and V once, the Q8_1 query, the fp32 output."""
    import numpy as np
    import torch
    from quant_integer_dot_amd import binding as qd
    from quant_integer_dot_amd import synth
    L = qd.load()
    dev = torch.device("cuda:0")
    Hq, Hkv, D, T = 32, 8, 128, args.ctx
    layers = args.layers or 36
    row = qd.qdot_attn_kv4_row_bytes(D)
    scale = np.float32(1 / np.sqrt(D))
    t0 = time.time()
    Ks, Vs, xs, qs, outs = [], [], [], [], []
    for layer in range(layers):
        Ks.append(torch.from_numpy(synth.kv4_cache(Hkv, T, D, (2026, 80, layer, 1))).to(dev))
        Vs.append(torch.from_numpy(synth.kv4_cache(Hkv, T, D, (2026, 80, layer, 2))).to(dev))
        xs.append(torch.from_numpy(synth.activations(Hq, D, (2026, 80, layer, 3))).to(dev))
        qs.append(torch.empty(qd.qdot_q8_1_bytes(Hq, D), dtype=torch.uint8, device=dev))
        outs.append(torch.empty((Hq, D), dtype=torch.float32, device=dev))
    wsb = qd.qdot_attn_kv4_workspace_bytes(Hq, T)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    kv_bytes = 2 * Hkv * T * row
    log(f"[bench] workload {args.workload}: {layers} layers, Hq={Hq} Hkv={Hkv} D={D} T={T}; KV cache "
        f"{layers * kv_bytes / 1e9:.3f} GB resident in {time.time() - t0:.1f} s; library {qd.qdot_build_id()}")

    def step(quantize=True):
        s = torch.cuda.current_stream(dev).cuda_stream
        for i in range(layers):
            if quantize:
                assert L.qdot_quantize_q8_1(xs[i].data_ptr(), Hq, D, qs[i].data_ptr(), s) == 0
            rc = L.qdot_attn_decode_kv4(qs[i].data_ptr(), Hq, Ks[i].data_ptr(), Vs[i].data_ptr(), Hkv, T, D,
                                        ctypes.c_float(scale), outs[i].data_ptr(), ws.data_ptr(), wsb, s)
            assert rc == 0, rc

    if args.eager_only:   # counter runs: plain launches, no graphs, no timing
        for _ in range(max(args.steps, 1)):
            step(True)
        torch.cuda.synchronize()
        print(json.dumps({"eager_only": True, "workload": args.workload, "layers": layers, "ctx": T}), flush=True)
        return

    def graph_ms(quantize):
        step(quantize)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(quantize)
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps

    ms_step = graph_ms(True)
    ms_attn = graph_ms(False)   # the attention calls alone (queries already quantized)
    per_call_us = ms_attn * 1e3 / layers
    alg = kv_bytes + qd.qdot_q8_1_bytes(Hq, D) + Hq * D * 4
    achieved = alg / (per_call_us * 1e-6) / 1e9
    value = layers * kv_bytes / (ms_step * 1e-3) / 1e9
    check = None
    if not args.no_check:
        import oracle
        step(True)
        torch.cuda.synchronize()
        i = layers - 1
        o64, _ = oracle.attn_decode_kv4(qs[i].cpu().numpy(), Hq, Ks[i].cpu().numpy(), Vs[i].cpu().numpy(), Hkv,
                                        T, D, float(scale))
        got = outs[i].cpu().numpy().astype(np.float64)
        d = np.abs(Vs[i].cpu().numpy().reshape(Hkv, T, D // 32, 18)[..., 0:2].copy().view(np.float16)
                   .astype(np.float64))
        vmax = np.repeat((8 * d).reshape(Hkv, -1).max(axis=1), Hq // Hkv)[:, None]
        bad = int((np.abs(got - o64) > 1e-4 * vmax).sum())
        check = {"outputs_checked": int(got.size), "outside_1e-4_of_max_v": bad, "layer": i}
        if bad:
            log(f"[bench] SAMPLED CHECK FAILED: {bad} of {got.size} outputs")
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        K0, V0, q0 = Ks[0].cpu().numpy(), Vs[0].cpu().numpy(), qs[0].cpu().numpy()
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < 10.0:
            oracle.attn_decode_kv4(q0, Hq, K0, V0, Hkv, T, D, float(scale))
            reps += 1
        dt = time.perf_counter() - t0
        cpu = {"value": round(reps * kv_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"{reps} attention calls of layer 0 (all {Hq} heads, T = {T}) in {dt:.1f} s, "
                         "single thread"}
    log(f"[bench] step {ms_step:.3f} ms -> {value:.1f} GB/s of KV cache; attention call {per_call_us:.2f} us "
        f"({achieved:.1f} GB/s)")
    print(json.dumps({
        "metric": "KV-cache GB/s of int4-KV decode attention, Qwen3-8B heads",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8/f32", "data": "synthetic",
        "config": {"workload": args.workload, "layers": layers, "Hq": Hq, "Hkv": Hkv, "D": D, "ctx": T,
                   "kv_bytes_per_layer": kv_bytes, "launches_per_step": 3 * layers},
        "roofline": {"bound": "hbm", "kernel": "attn_kv4_partial_kernel+attn_kv4_combine_kernel",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 5),
                     "traffic": recorded_traffic("attn_kv4_partial_kernel+attn_kv4_combine_kernel", args.workload),
                     "launches": layers, "avg_launch_us": round(per_call_us, 3),
                     "algorithmic_bytes_per_launch": alg,
                     "note": "one launch = one qdot_attn_decode_kv4 call (the partial and combine kernels)"},
        "cpu_baseline": cpu, "sampled_check": check}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        log(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU sharding "
            "of this path is a design note, not a measured configuration.")
        sys.exit(2)
    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)
        return
    if args.workload == "qwen3-8b-rmsnorm-q8_1":
        producer_bench(args)
        return
    if args.workload == "qwen3-8b-attn-kv4-32k":
        attention_bench(args)
        return

    import numpy as np
    import torch
    from quant_integer_dot_amd import binding as qd
    from quant_integer_dot_amd import synth

    qd.load()
    dev = torch.device("cuda:0")
    cfg_idx, shapes, layers, Ms = workload_def(args.workload)
    prefill = args.workload.endswith("prefill-512")
    if args.layers:
        layers = args.layers
    if args.ms:
        Ms = [int(v) for v in args.ms.split(",")]
    log(f"[bench] workload {args.workload}: {len(shapes)} projections x {layers} layers, M={Ms}; "
        f"library {qd.qdot_build_id()}")

    # ---------------------------------------------------------- weights
    t0 = time.time()
    Wdev = []   # [layer][proj] device tensors
    for layer in range(layers):
        if args.same_weights and layer > 0:
            Wdev.append(Wdev[0])
            continue
        row = []
        for pi, (name, N, K, t) in enumerate(shapes):
            row.append(torch.from_numpy(synth.weights(t, N, K, synth.weight_seed(cfg_idx, layer, pi))).to(dev))
        Wdev.append(row)
    torch.cuda.synchronize()
    wbytes_sweep = sum(int(w.numel()) for row in Wdev for w in row)
    log(f"[bench] weights resident: {wbytes_sweep / 1e9:.3f} GB in {time.time() - t0:.1f} s")

    # ------------------------------------------------ activations, buffers
    inputs = sorted({INPUT_OF[name] for name, *_ in shapes})
    in_K = {INPUT_OF[name]: K for name, N, K, t in shapes}
    bufs = {}
    for M in Ms:
        b = {"x": {}, "xq": {}, "y": {}}
        for inp in inputs:
            K = in_K[inp]
            b["x"][inp] = torch.from_numpy(synth.activations(M, K, synth.act_seed(cfg_idx, K, M))).to(dev)
            b["xq"][inp] = torch.empty(qd.qdot_q8_1_bytes(M, K), dtype=torch.uint8, device=dev)
        for name, N, K, t in shapes:
            b["y"][name] = torch.empty((M, N), dtype=torch.float32, device=dev)
        bufs[M] = b

    lib = qd.load()
    stream = torch.cuda.current_stream(dev)

    # Projections that read the same quantized input share one quantization
    # per layer (q/k/v, gate/up), and for M <= 8 one qdot_qmatmul_multi launch
    # (unless --separate).  Everything runs in order on one stream: running
    # the q/k/v and gate/up launches as parallel graph branches on side
    # streams measured slower on MI355X (12.5 vs 10.3 ms per step).
    groups = []
    for pi, (name, N, K, t) in enumerate(shapes):
        inp = INPUT_OF[name]
        if not groups or groups[-1][0] != inp:
            groups.append((inp, []))
        groups[-1][1].append(pi)

    def units(M):
        """The launches of one layer after each quantization: (label, [proj indices])."""
        out = []
        for inp, pis in groups:
            if not args.separate and M <= 8 and len(pis) > 1:
                out.append(("+".join(shapes[pi][0] for pi in pis), pis))
            else:
                out.extend((shapes[pi][0], [pi]) for pi in pis)
        return out

    # IQ4_XS's dot4 tile already spends its VALU on the codebook lookups: its
    # launches with the quantization inside measured slower than a separate
    # quantize launch (hidden-5120 sweep at M = 1: 4.29 vs 4.09 ms), so
    # workloads with IQ4_XS weights keep the separate launch.
    fusable = not prefill and all(t != synth.IQ4_XS for *_, t in shapes)

    # Quantizing inside the matmul repeats the work in every workgroup (16
    # weight rows each): M*K values per workgroup.  Above about 4 M values per
    # launch that costs more than the separate launch it saves (12288 x 4096
    # gate+up at M = 1, 6.3 M: 16.1 us against 14.0 + 1.8; down 4096 x 12288,
    # 3.1 M: 13.7 against 12.5 + 1.8).
    REDUNDANT_MAX = 4_000_000

    def fused(M, inp):
        """Whether M's launches reading input `inp` quantize it themselves."""
        if M > args.fused_max_m or not fusable:
            return False
        pis = [pi for pi, (name, *_r) in enumerate(shapes) if INPUT_OF[name] == inp]
        work = sum((shapes[pi][1] + 15) // 16 * shapes[pi][2] * M for pi in pis)
        return work <= REDUNDANT_MAX

    def unit_kernel(M, pis):
        if fused(M, INPUT_OF[shapes[pis[0]][0]]):
            names = [f"qmv_dot4q<{synth.TYPE_NAMES[shapes[pi][3]]},{M}>" for pi in pis]
            return names[0] if len(pis) == 1 else "qmv_multi<" + "+".join(names) + ">"
        if len(pis) == 1:
            _, N, K, t = shapes[pis[0]]
            return qd.qdot_kernel_name_shape(t, N, K, M)
        types = [shapes[pi][3] for pi in pis]
        Ns = [shapes[pi][1] for pi in pis]
        K = shapes[pis[0]][2]
        return "qmv_multi<" + "+".join(qd.qdot_multi_kernel_name(types, Ns, K, M, i)
                                       for i in range(len(pis))) + ">"

    P_, I32_, I64_ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    multi_args = {}   # (M, layer, label) -> prebuilt ctypes arrays

    def sweep(M, only=None):
        """Launch one M's sweep on the current stream (all layers)."""
        b = bufs[M]
        s = torch.cuda.current_stream(dev).cuda_stream
        us = units(M)
        for layer in range(layers):
            for inp, pis in groups:
                K = shapes[pis[0]][2]
                fz = fused(M, inp)
                if not fz and (only is None or only == "quantize"):
                    rc = lib.qdot_quantize_q8_1(b["x"][inp].data_ptr(), M, K, b["xq"][inp].data_ptr(), s)
                    assert rc == 0, rc
                src = b["x"][inp] if fz else b["xq"][inp]
                for label, upis in us:
                    if upis[0] not in pis or (only is not None and only != label):
                        continue
                    if len(upis) == 1:
                        name, N, K, t = shapes[upis[0]]
                        fn = lib.qdot_quantize_qmatmul if fz else lib.qdot_qmatmul
                        rc = fn(Wdev[layer][upis[0]].data_ptr(), t, N, K, src.data_ptr(), M,
                                b["y"][name].data_ptr(), s)
                    else:
                        key = (M, layer, label)
                        if key not in multi_args:
                            n = len(upis)
                            multi_args[key] = (
                                (P_ * n)(*[Wdev[layer][pi].data_ptr() for pi in upis]),
                                (I32_ * n)(*[shapes[pi][3] for pi in upis]),
                                (I64_ * n)(*[shapes[pi][1] for pi in upis]),
                                (P_ * n)(*[b["y"][shapes[pi][0]].data_ptr() for pi in upis]))
                        wa, ta, na, ya = multi_args[key]
                        fn = lib.qdot_quantize_qmatmul_multi if fz else lib.qdot_qmatmul_multi
                        rc = fn(len(upis), wa, ta, na, K, src.data_ptr(), M, ya, s)
                    assert rc == 0, rc

    # eager run once (also fills every xq buffer)
    for M in Ms:
        sweep(M)
    torch.cuda.synchronize()
    if args.eager_only:
        # Plain stream launches, no graphs: what hardware-counter passes profile.
        t0 = time.perf_counter()
        for _ in range(args.steps):
            for M in Ms:
                sweep(M)
        torch.cuda.synchronize()
        print(json.dumps({"eager_only": True, "workload": args.workload, "M": Ms, "layers": layers,
                          "steps": args.steps,
                          "wall_ms_per_step": round((time.perf_counter() - t0) * 1e3 / args.steps, 3)}),
              flush=True)
        return

    # ------------------------------------------------------- step graphs
    graphs = {}
    for M in Ms:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            sweep(M)
        graphs[M] = g
    for _ in range(args.warmup):
        for M in Ms:
            graphs[M].replay()
    torch.cuda.synchronize()

    ev = lambda: torch.cuda.Event(enable_timing=True)
    per_m_ms = {M: [] for M in Ms}
    t_start, t_end = ev(), ev()
    marks = [[ev() for _ in range(len(Ms) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start.record()
    for k in range(args.steps):
        marks[k][0].record()
        for i, M in enumerate(Ms):
            graphs[M].replay()
            marks[k][i + 1].record()
    t_end.record()
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / args.steps
    for k in range(args.steps):
        for i, M in enumerate(Ms):
            per_m_ms[M].append(marks[k][i].elapsed_time(marks[k][i + 1]))
    value = len(Ms) * wbytes_sweep / (ms_per_step * 1e-3) / 1e9
    step_ops = sum(2 * M * N * K for M in Ms for _, N, K, _ in shapes) * layers
    log(f"[bench] step {ms_per_step:.3f} ms -> {value:.1f} GB/s of weights, "
        f"{step_ops / (ms_per_step * 1e-3) / 1e12:.1f} int8 TOP/s")

    # ------------------------------------- per-projection kernel timing
    reps = args.kernel_reps or max(20, args.steps)
    kern = {}      # kernel name -> [bytes, ms, launches]
    per_m = {}
    for M in Ms:
        rows = {}
        for label, upis in units(M):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                sweep(M, only=label)
            g.replay()
            torch.cuda.synchronize()
            us = graph_median_ms(g, reps) * 1e3 / layers
            K = shapes[upis[0]][2]
            Ns = [shapes[pi][1] for pi in upis]
            wb = sum(qd.qdot_weight_bytes(shapes[pi][3], shapes[pi][1], K) for pi in upis)
            # activations read once (fp32 when quantized in the kernel, Q8_1 otherwise), y written once
            fz_u = fused(M, INPUT_OF[shapes[upis[0]][0]])
            alg = wb + (4 * M * K if fz_u else qd.qdot_q8_1_bytes(M, K)) + 4 * M * sum(Ns)
            rows[label] = {"N": Ns[0] if len(Ns) == 1 else Ns, "K": K,
                           "type": "+".join(synth.TYPE_NAMES[shapes[pi][3]] for pi in upis),
                           "us": round(us, 3), "weight_GBps": round(wb / us / 1e3, 1),
                           "pct_hbm_peak": round(100 * wb / us / 1e3 / HBM_PEAK_GBS, 1)}
            rows[label]["TOPs"] = round(2 * M * sum(Ns) * K / us / 1e6, 2)
            kn = unit_kernel(M, upis)
            e = kern.setdefault(kn, [0, 0.0, 0, 0])
            e[0] += alg * layers
            e[1] += us * layers * 1e-3
            e[2] += layers
            e[3] += 2 * M * sum(Ns) * K * layers
        # quantizer (none for inputs the matmul kernels quantize themselves)
        qus = None
        q_inputs = [i for i in inputs if not fused(M, i)]
        if q_inputs:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                sweep(M, only="quantize")
            g.replay()
            torch.cuda.synchronize()
            nq = layers * len(q_inputs)
            qus = graph_median_ms(g, reps) * 1e3 / nq
            qbytes = sum(M * in_K[i] * 4 + qd.qdot_q8_1_bytes(M, in_K[i]) for i in q_inputs) * layers
            e = kern.setdefault("quantize_q8_1", [0, 0.0, 0, 0])
            e[0] += qbytes
            e[1] += qus * nq * 1e-3
            e[2] += nq
        wb_m = wbytes_sweep
        per_m[str(M)] = {"sweep_ms": round(float(np.median(per_m_ms[M])), 4),
                         "sweep_weight_GBps": round(wb_m / (np.median(per_m_ms[M]) * 1e-3) / 1e9, 1),
                         "quantize_us": round(qus, 3) if qus is not None else "in the matmul kernels",
                         "quantized_in_matmul": [i for i in inputs if fused(M, i)],
                         "qmatmul": rows}

    # µs per qmatmul for each projection on its own (one launch per matrix,
    # as `--separate` runs them), beside the grouped launches the step uses.
    per_proj = None
    if not prefill and any(len(u) > 1 for M in Ms for _, u in units(M)):
        per_proj = {}
        for M in Ms:
            b = bufs[M]
            row = {}
            for pi, (name, N, K, t) in enumerate(shapes):
                fz = fused(M, INPUT_OF[name])
                src = b["x"][INPUT_OF[name]] if fz else b["xq"][INPUT_OF[name]]
                fn = lib.qdot_quantize_qmatmul if fz else lib.qdot_qmatmul
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    s_ = torch.cuda.current_stream(dev).cuda_stream
                    for layer in range(layers):
                        rc = fn(Wdev[layer][pi].data_ptr(), t, N, K, src.data_ptr(), M, b["y"][name].data_ptr(), s_)
                        assert rc == 0, rc
                g.replay()
                torch.cuda.synchronize()
                us = graph_median_ms(g, reps) * 1e3 / layers
                wb = qd.qdot_weight_bytes(t, N, K)
                row[name] = {"us": round(us, 3), "pct_hbm_peak": round(100 * wb / us / 1e3 / HBM_PEAK_GBS, 1),
                             "kernel": (f"qmv_dot4q<{synth.TYPE_NAMES[t]},{M}>" if fz
                                        else qd.qdot_kernel_name_shape(t, N, K, M))}
            per_proj[str(M)] = row

    # The dominant kernel is the HIP kernel function with the largest share of
    # the step, summed over its template instances (weight types, M tile,
    # prefetch depth): its rate is its algorithmic bytes (or ops) over all its
    # launches of a step divided by their summed duration.
    fam = {}
    for k, v in kern.items():
        f = fam.setdefault(KERNEL_FUNCTION[k.split("<")[0]], [0, 0.0, 0, 0, []])
        for i in range(4):
            f[i] += v[i]
        f[4].append(k)
    dname, (dbytes, dms, dn, dops, dinst) = max(fam.items(), key=lambda kv: kv[1][1])
    if prefill:
        # a dense int8 contraction: priced against the int8 MFMA peak
        achieved = dops / (dms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "kernel": dname, "instances": dinst, "achieved": round(achieved, 2),
                    "peak": MFMA_I8_PEAK_TOPS, "unit": "TFLOP/s", "frac": round(achieved / MFMA_I8_PEAK_TOPS, 4),
                    "traffic": recorded_traffic(dname, args.workload), "launches": dn,
                    "avg_launch_us": round(dms * 1e3 / dn, 3),
                    "algorithmic_ops_per_launch": round(dops / dn)}
    else:
        achieved = dbytes / (dms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "kernel": dname, "instances": dinst, "achieved": round(achieved, 1),
                    "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": recorded_traffic(dname, args.workload),
                    "launches": dn, "avg_launch_us": round(dms * 1e3 / dn, 3),
                    "algorithmic_bytes_per_launch": round(dbytes / dn)}
        ref = copy_reference(dev, dbytes / dn)
        ref.update(stream_reference(dev, dbytes / dn))
        ref["frac_of_copy_512MiB"] = round(achieved / ref["copy_512MiB_GBps"], 4)
        ref["frac_of_read_512MiB"] = round(achieved / ref["read_512MiB_GBps"], 4)
        ref["frac_of_read_at_launch_size"] = round(achieved / ref["read_at_launch_size"]["GBps"], 4)
        roofline["measured_reference"] = ref
    kernels = {k: {"launches_per_step": v[2], "ms_per_step": round(v[1], 4),
                   "GBps": round(v[0] / (v[1] * 1e-3) / 1e9, 1),
                   **({"TOPs": round(v[3] / (v[1] * 1e-3) / 1e12, 2)} if v[3] else {})}
               for k, v in kern.items()}
    # The sweep aggregate over kernel time alone (the sum of the per-launch
    # figures above), beside the wall time of the step graphs.
    ksum_ms = sum(v[1] for v in kern.values())
    kernel_aggregate = {"sum_of_launch_ms_per_step": round(ksum_ms, 4), "step_wall_ms": round(ms_per_step, 4)}
    if prefill:
        kernel_aggregate["int8_TOPs_over_launch_time"] = round(step_ops / (ksum_ms * 1e-3) / 1e12, 2)
    else:
        kernel_aggregate["weight_GBps_over_launch_time"] = round(len(Ms) * wbytes_sweep / (ksum_ms * 1e-3) / 1e9, 1)

    # ------------------------------------------- sampled oracle check
    check = None
    if not args.no_check:
        import oracle
        bad = 0
        nchk = 0
        for M in Ms:
            graphs[M].replay()
            torch.cuda.synchronize()
            b = bufs[M]
            layer = 0 if args.same_weights else layers - 1   # whose weights the last launches read
            for pi, (name, N, K, t) in enumerate(shapes):
                W = synth.weights(t, N, K, synth.weight_seed(cfg_idx, layer, pi))
                xq = oracle.quantize_q8_1(b["x"][INPUT_OF[name]].cpu().numpy())
                rows = np.random.default_rng(M * 100 + pi).integers(0, N, 8)
                y64, _ = oracle.qmatmul_rows(W, t, N, K, xq, M, rows)
                yg = b["y"][name].cpu().numpy()[:, rows].astype(np.float64)
                bad += int((np.abs(yg - y64) > 1e-5 * np.abs(y64)).sum())
                nchk += y64.size
        check = {"outputs_checked": nchk, "outside_1e-5_rel": bad}
        if bad:
            log(f"[bench] SAMPLED CHECK FAILED: {bad} of {nchk} outputs")

    shard = None
    if args.workload == "qwen3-8b-decode" and not args.no_shard_rows:
        shard = shard_rows(dev, args.fused_max_m, reps, per_m, check=not args.no_check)
    pre_row = None
    if args.workload == "qwen3-8b-decode" and not args.no_prefill_row and not args.same_weights:
        pre_row = prefill_row(dev, Wdev, shapes, cfg_idx, layers, reps, check=not args.no_check)
        log(f"[bench] prefill row: {pre_row['ms_per_sweep']} ms per M = 512 sweep, "
            f"{pre_row['int8_TOPs']} int8 TOP/s ({pre_row['pct_mfma_i8_peak']} % of peak)")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(shapes, cfg_idx, Ms, prefill=prefill, layers=layers)

    if prefill:
        metric, unit = "int8 TOP/s (% of MFMA int8 peak), M=512 prefill chunk, Qwen3-8B shapes", "TOP/s"
        value = step_ops / (ms_per_step * 1e-3) / 1e12
    else:
        metric = METRIC if args.workload == "qwen3-8b-decode" and Ms == [1, 2, 4, 8] else \
            f"weight GB/s, {args.workload}, M={','.join(str(m) for m in Ms)}"
        unit = "GB/s"
    out = {
        "metric": metric,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": args.workload, "layers": layers, "M": Ms,
                   "projections": [f"{n} {N}x{K} {synth.TYPE_NAMES[t]}" for n, N, K, t in shapes],
                   "weight_bytes_per_sweep": wbytes_sweep,
                   "launches_per_step": sum(len(units(M)) for M in Ms) * layers +
                                        sum(0 if fused(M, i) else 1 for M in Ms for i in inputs) * layers,
                   "grouped_launches": not args.separate,
                   "quantized_in_matmul": {str(M): [i for i in inputs if fused(M, i)] for M in Ms
                                           if any(fused(M, i) for i in inputs)},
                   **({"same_weights_every_layer": True} if args.same_weights else {})},
        **({"pct_mfma_i8_peak": round(100 * value / MFMA_I8_PEAK_TOPS, 2)} if prefill else
           {"pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 1)}),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "per_M": per_m,
        **({"per_projection_single_launch": per_proj} if per_proj else {}),
        **({"shard_tp8_rows": shard} if shard else {}),
        **({"prefill_512_row": pre_row} if pre_row else {}),
        "kernels": kernels,
        "kernel_time_aggregate": kernel_aggregate,
        "sampled_check": check,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
