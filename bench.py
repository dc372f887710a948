"""Benchmark of the convrot linear hot path on one MI355X.

One step = the whole hot path on one batch: pack the activation (group-wise
rotation + row absmax + int8 codes) once, then the three attention
projections Q, K, V on that packed activation in one grouped launch (int8
MFMA GEMM with the fused scale/bias epilogue).  Workload: X bf16 [4096, 3072] with LogNormal channel
scales, three weights [3072, 3072], G = 256 (N total 9216).  Weight
preparation is offline and not timed.  Inputs are resident in HBM before the
timed region starts.

Prints one JSON line: value = effective INT8 TOPS of the whole step
(2*M*N*K / step time, the pack included), plus the pack's HBM GB/s, the
roofline of the dominant kernel (the GEMM) from HIP events recorded on the
launch stream around every 4th launch in the timed region, and the CPU
oracle timed on a bounded sample of the same workload.  Measured before
the warm-up steps and reported beside them: the pack alone (warm and
cold), an HBM stream of the pack's bytes in its read:write mix (HBM's
ceiling for such a pass), a register-only MFMA loop on the same operand
codes (the matrix cores' ceiling under the power limit) and the GEMM alone
over back-to-back launches.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0   # MI355X dense INT8 MFMA, 5.0 POP/s
PEAK_HBM_GBPS = 8000.0    # MI355X HBM3E, 8 TB/s

GEMM_SOURCE = os.path.join(ROOT, "hadamard_rotated_int8_amd", "csrc", "gemm.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_qkv_4096x3072x9216_traffic.json")
CALIBRATION_BYTES = 256 * 1024 * 1024  # the plain copy whose counters scale FETCH/WRITE_SIZE
WARM_MS = 25.0  # sustained launches before a back-to-back timing (clock settling)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # The shader clock settles over the first few hundred launches (20 warm-up
    # steps measured ~7 % slower GEMMs than 300), so the default warms up
    # for 300 steps (about 40 ms).
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="qkv_4096x3072x9216")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--all-configs", action="store_true",
                    help="instead of the step line: one JSON line per workload and kernel "
                         "(pack GB/s, linear TOPS, roofline fractions, oracle baseline on a row sample)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device-to-device copy of CALIBRATION_BYTES "
                         "(reads and writes that many bytes), for scaling HBM byte counters")
    return ap.parse_args()


def gemm_traffic():
    """HBM bytes per grouped Q/K/V GEMM launch from the committed counter
    summary, or None when the GEMM source changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        with open(GEMM_SOURCE, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    if t.get("gemm_source_sha256") != sha:
        return None
    return t.get("hbm_bytes_per_launch")


def _time_ms(fn, reps=20, flush=None, warm_ms=WARM_MS):
    """Average ms per call over back-to-back launches, or the median of single
    launches each after a cache-flushing write when ``flush`` is given.
    Back-to-back timings first run the call for about ``warm_ms`` ms: after
    idle time or a short kernel the clock needs some 20 ms of sustained work
    to settle, and the first launches run slower."""
    import torch

    fn()
    torch.cuda.synchronize()
    if flush is None:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        for _ in range(min(5000, int(warm_ms / max(e0.elapsed_time(e1), 1e-3)))):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps
    ts = []
    for _ in range(reps):
        flush.fill_(1.0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    return float(np.median(ts))


def _graph_time_ms(fn, launches=20, reps=6, warm_ms=WARM_MS):
    """Device time per call of a short launch: `launches` calls captured in one
    HIP graph, the graph replayed back to back (median of reps pairs of
    replays, after about warm_ms of replays).  Timing the same calls from
    the host back to back measures the host's call overhead instead once a
    launch is shorter than that overhead (the pack at 4096 rows: ~9 us on
    the device, 12-13 us per call from Python)."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # outside the capture: lazily set-up state, then the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for _ in range(launches):
            fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    for _ in range(min(1000, int(warm_ms / max(e0.elapsed_time(e1), 1e-3)))):
        graph.replay()
    ts = []
    for _ in range(reps):
        e0.record()
        graph.replay()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) / (2 * launches))
    del graph
    return float(np.median(ts))


def stream_beside(m, k, in_bytes, pack_warm_ms, pack_cold_ms, flush):
    """The HBM stream kernel moving the pack's bytes in the pack's read:write
    mix (stream_ceiling), warm and cold, and its time over the pack's (1.0:
    the pack moves its bytes as fast as the stream)."""
    r = stream_ceiling(m, k, in_bytes, flush)
    if r is None:
        return {}
    warm, cold, _, _ = r
    return {"stream_us_warm": round(warm * 1e3, 2), "stream_us_cold": round(cold * 1e3, 2),
            "stream_over_pack_warm": round(warm / pack_warm_ms, 4),
            "stream_over_pack_cold": round(cold / pack_cold_ms, 4)}


def all_configs(args):
    """Every workload: the pack per group size and each linear, as JSON lines."""
    import torch
    from threadpoolctl import threadpool_limits

    import hadamard_rotated_int8_amd as cr
    import workloads as wl
    from oracle import convrot_oracle as orc

    cr.lib()
    cores = len(os.sched_getaffinity(0))
    flush = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")

    def emit(**kw):
        print(json.dumps(kw), flush=True)

    def oracle_tops(x64_rows, qws_or, g, n_total):
        """The oracle (pack + linears) on a row sample, as TOPS on this host."""
        with threadpool_limits(limits=cores):
            t0 = time.perf_counter()
            qx, sx = orc.pack_activations(x64_rows, g)
            for q, sw in qws_or:
                orc.linear(qx, sx, q, sw, None)
            dt = time.perf_counter() - t0
        return 2.0 * x64_rows.shape[0] * n_total * x64_rows.shape[1] / dt / 1e12

    for w in wl.ORDER:
        inp = wl.generate(w)
        x = inp["x"].cuda()
        m, k = w.m, w.k
        xb = x.element_size()
        for g in w.group_sizes:
            qws = [cr.quantize_weights(torch.from_numpy(wt).cuda(), g, torch.from_numpy(b).cuda())
                   for wt, b in zip(inp["weights"], inp["biases"])]
            packed = cr.pack_activations(x, g)
            pbytes = m * k * (xb + 1) + 4 * m
            warm = _graph_time_ms(lambda: cr.pack_activations(x, g, out=packed))
            cold = _time_ms(lambda: cr.pack_activations(x, g, out=packed), reps=10, flush=flush)
            emit(workload=w.name, kernel="pack", m=m, k=k, x_dtype=w.x_dtype, group_size=g,
                 us_warm=round(warm * 1e3, 2), us_cold=round(cold * 1e3, 2),
                 gbps_cold=round(pbytes / (cold * 1e-3) / 1e9, 1),
                 hbm_frac_cold=round(pbytes / (cold * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                 **stream_beside(m, k, xb, warm, cold, flush))
            linears = list(zip(w.linears, qws))
            if w.gelu_chain:
                linears = linears[:1]
            for spec, qw in linears:
                gl = w.gelu_chain
                y = torch.empty((m, spec.n), dtype=torch.float32, device="cuda")
                if gl:
                    # the GELU epilogue's cost: alternate the launch with and
                    # without it (same shape) and take medians
                    tg, tp = [], []
                    for _ in range(6):
                        tg.append(_time_ms(lambda: cr.linear(packed, qw, out=y, gelu=True)))
                        tp.append(_time_ms(lambda: cr.linear(packed, qw, out=y)))
                    t, t_plain = statistics.median(tg), statistics.median(tp)
                else:
                    t = _time_ms(lambda: cr.linear(packed, qw, out=y))
                tops = 2.0 * m * spec.n * k / (t * 1e-3) / 1e12
                extra = {}
                if gl:
                    extra = {"us_without_gelu": round(t_plain * 1e3, 2),
                             "gelu_overhead": round(t / t_plain - 1.0, 4)}
                emit(workload=w.name, kernel="linear", linear=spec.name, m=m, n=spec.n, k=k,
                     group_size=g, gelu=gl, us=round(t * 1e3, 2), tops=round(tops, 1),
                     mfma_frac=round(tops / PEAK_INT8_TOPS, 4), **extra)
                if w.gelu_chain:  # the down projection on this (float32) output
                    dspec, dqw = w.linears[1], qws[1]
                    hp = cr.pack_activations(y, g)
                    hbytes = m * spec.n * 5 + 4 * m
                    hwarm = _graph_time_ms(lambda: cr.pack_activations(y, g, out=hp))
                    hcold = _time_ms(lambda: cr.pack_activations(y, g, out=hp), reps=10, flush=flush)
                    emit(workload=w.name, kernel="pack", m=m, k=spec.n, x_dtype="f32", group_size=g,
                         us_warm=round(hwarm * 1e3, 2), us_cold=round(hcold * 1e3, 2),
                         gbps_cold=round(hbytes / (hcold * 1e-3) / 1e9, 1),
                         hbm_frac_cold=round(hbytes / (hcold * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                         **stream_beside(m, spec.n, 4, hwarm, hcold, flush))
                    yd = torch.empty((m, dspec.n), dtype=torch.float32, device="cuda")
                    td = _time_ms(lambda: cr.linear(hp, dqw, out=yd))
                    dtops = 2.0 * m * dspec.n * spec.n / (td * 1e-3) / 1e12
                    emit(workload=w.name, kernel="linear", linear=dspec.name, m=m, n=dspec.n,
                         k=spec.n, group_size=g, gelu=False, us=round(td * 1e3, 2),
                         tops=round(dtops, 1), mfma_frac=round(dtops / PEAK_INT8_TOPS, 4))
                    del yd, hp
                del y
            if len(qws) > 1 and not w.gelu_chain:
                ys = [torch.empty((m, q.q.shape[0]), dtype=torch.float32, device="cuda") for q in qws]
                t = _time_ms(lambda: cr.linear_grouped(packed, qws, outs=ys))
                n_total = sum(q.q.shape[0] for q in qws)
                tops = 2.0 * m * n_total * k / (t * 1e-3) / 1e12
                emit(workload=w.name, kernel="linear_grouped", n=n_total, m=m, k=k, group_size=g,
                     us=round(t * 1e3, 2), tops=round(tops, 1), mfma_frac=round(tops / PEAK_INT8_TOPS, 4))
                del ys
                # The same weights as one [n_total, k] matrix (codes and scales
                # are per output row, so stacking the rows is the quantised
                # concatenation), one plain launch.
                if len({q.q.shape[1] for q in qws}) == 1 and all(q.bias is not None for q in qws):
                    qcat = cr.QuantizedWeights(torch.cat([q.q for q in qws]),
                                               torch.cat([q.scale for q in qws]),
                                               torch.cat([q.bias for q in qws]), g)
                    ycat = torch.empty((m, n_total), dtype=torch.float32, device="cuda")
                    t = _time_ms(lambda: cr.linear(packed, qcat, out=ycat))
                    tops = 2.0 * m * n_total * k / (t * 1e-3) / 1e12
                    emit(workload=w.name, kernel="linear_concat", n=n_total, m=m, k=k, group_size=g,
                         us=round(t * 1e3, 2), tops=round(tops, 1),
                         mfma_frac=round(tops / PEAK_INT8_TOPS, 4))
                    del qcat, ycat
            # Rank-64 low-rank adapters on the workload's linears (the first,
            # GELU one for the MLP): the down projection of each adapter into
            # one shared U buffer, and the linears with U B^T added in the
            # GEMM epilogue, beside the same launch without adapters.
            if g == 256 and m >= 1024:
                rank = 64
                lqws = qws[:1] if w.gelu_chain else qws
                ads = [wl.lora_adapter(k, q.q.shape[0], rank, m=0, seed=w.seed + 50 + i)
                       for i, q in enumerate(lqws)]
                a_dev = [ad["a"].cuda() for ad in ads]
                b_dev = [ad["b"].cuda() for ad in ads]
                ucat = torch.empty((m, rank * len(ads)), dtype=torch.bfloat16, device="cuda")
                us = [ucat[:, i * rank:(i + 1) * rank] for i in range(len(ads))]

                def down_all():
                    for ad, a_d, u in zip(ads, a_dev, us):
                        cr.lora_down(x, a_d, ad["scale"], out=u)

                td = _time_ms(down_all)
                emit(workload=w.name, kernel="lora_down", m=m, k=k, rank=rank, adapters=len(ads),
                     us=round(td * 1e3, 2),
                     x_gbps=round(len(ads) * m * k * xb / (td * 1e-3) / 1e9, 1))
                # Adapters that share a scale can stack their A matrices into one
                # down projection that reads X once and fills the same U buffer.
                if len(ads) > 1 and len({ad["scale"] for ad in ads}) == 1:
                    a_cat = torch.cat(a_dev)
                    tds = _time_ms(lambda: cr.lora_down(x, a_cat, ads[0]["scale"], out=ucat))
                    emit(workload=w.name, kernel="lora_down_stacked", m=m, k=k,
                         rank=int(a_cat.shape[0]), adapters=len(ads), us=round(tds * 1e3, 2),
                         x_gbps=round(m * k * xb / (tds * 1e-3) / 1e9, 1))
                    del a_cat
                ys = [torch.empty((m, q.q.shape[0]), dtype=torch.float32, device="cuda") for q in lqws]
                gl = w.gelu_chain
                # Alternate the two launches and take medians: the first
                # rounds after a change of kernel run at a lower clock.
                t0s, tls = [], []
                for _ in range(6):
                    t0s.append(_time_ms(lambda: cr.linear_lora(packed, lqws, [None] * len(lqws),
                                                               outs=ys, gelu=gl)))
                    tls.append(_time_ms(lambda: cr.linear_lora(packed, lqws, list(zip(us, b_dev)),
                                                               outs=ys, gelu=gl)))
                t0, tl = statistics.median(t0s), statistics.median(tls)
                n_total = sum(q.q.shape[0] for q in lqws)
                emit(workload=w.name, kernel="linear_lora", m=m, n=n_total, k=k, rank=rank,
                     gelu=gl, us_without_adapters=round(t0 * 1e3, 2), us=round(tl * 1e3, 2),
                     adapter_overhead=round(tl / t0 - 1.0, 4))
                del ys, ucat, us, a_dev, b_dev
            # The oracle on a row sample of the same workload (weights quantised
            # offline and untimed, as on the device).
            rows = min(m, 64)
            qws_or = [orc.quantize_weights(wt, g) for wt in inp["weights"]]
            n_total = sum(wt.shape[0] for wt in inp["weights"])
            if w.gelu_chain:
                qws_or, n_total = qws_or[:1], inp["weights"][0].shape[0]
            emit(workload=w.name, kernel="cpu_baseline", group_size=g, kind="oracle",
                 sample_rows=rows, cores=cores,
                 tops=round(oracle_tops(inp["x64"][:rows], qws_or, g, n_total), 4))
            del qws, packed
        del x, inp
        torch.cuda.empty_cache()


def calibrate_copy():
    import torch

    n = CALIBRATION_BYTES // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": CALIBRATION_BYTES, "launches": 5}), flush=True)


def cpu_baseline(inp, w, g, target_s):
    """The oracle, as it stands, on the same workload, repeated until about
    target_s seconds of CPU time have run (one pass takes well under that)."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import convrot_oracle as orc

    cores = len(os.sched_getaffinity(0))
    qws = [orc.quantize_weights(wt, g) for wt in inp["weights"]]  # offline, untimed

    def run(rows):
        x = inp["x64"][:rows]
        t0 = time.perf_counter()
        qx, sx = orc.pack_activations(x, g)
        for (qw, sw), b in zip(qws, inp["biases"]):
            orc.linear(qx, sx, qw, sw, b)
        return time.perf_counter() - t0

    with threadpool_limits(limits=cores):
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
        probe_rows = min(w.m, 256)
        t_probe = run(probe_rows)
        rows = int(min(w.m, max(probe_rows, probe_rows * target_s / max(t_probe, 1e-3))))
        rows = max(16, (rows // 16) * 16)
        t, passes = 0.0, 0
        while t < target_s and passes < 64:
            t += run(rows)
            passes += 1
    n_total = sum(wt.shape[0] for wt in inp["weights"])
    tops = 2.0 * rows * n_total * w.k * passes / t / 1e12
    return {
        "value": tops, "unit": "TOPS", "cores": int(threads), "kind": "oracle",
        "sample": f"{passes} pass(es) over {rows} of {w.m} rows, pack + "
                  f"{len(inp['weights'])} linears, float64 NumPy oracle, {t:.2f} s wall",
    }


def _ceiling_lib():
    """The measurement library (include/convrot_ceiling.h), or None if absent."""
    import ctypes

    path = os.path.join(ROOT, "hadamard_rotated_int8_amd", "libconvrot_ceiling.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    f = lib.convrot_ceiling_mfma_i8
    f.restype = ctypes.c_int64
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                  ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    f = lib.convrot_ceiling_stream
    f.restype = ctypes.c_int32
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                  ctypes.c_void_p]
    return lib


def mfma_ceiling(qa, qb, reps=5):
    """Rate of a register-only v_mfma_i32_32x32x32_i8 loop in the GEMM's
    per-wave shape, one wave per SIMD on every CU, on fragments of the given
    int8 codes (TOPS, median of reps launches of ~2 ms).  None without the
    measurement library."""
    import torch

    lib = _ceiling_lib()
    if lib is None:
        return None
    grid = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(grid * 256, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    iters = 4000
    ts, ops = [], 0
    for _ in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        ops = lib.convrot_ceiling_mfma_i8(qa.data_ptr(), qa.stride(0), qa.shape[0], qb.data_ptr(),
                                          qb.stride(0), qb.shape[0], iters, grid, sink.data_ptr(),
                                          stream)
        e1.record()
        torch.cuda.synchronize()
        if ops < 0:
            raise RuntimeError("MFMA ceiling kernel refused its arguments")
        ts.append(e0.elapsed_time(e1))
    return ops / (float(np.median(ts[1:])) * 1e-3) / 1e12


def stream_ceiling(m, k, in_bytes, flush, reps=20):
    """The HBM ceiling for a pack of an [m, k] input of in_bytes per element:
    the measurement library's stream kernel reads in_bytes * m * k and writes
    m * k bytes (the pack's bytes but the 4 per row of its scales, in its
    read:write mix) with non-temporal 16-byte accesses.  Returns (warm ms,
    cold ms, warm GB/s, cold GB/s) at the best of four grid sizes, warm =
    graph-replayed back-to-back launches, cold = single launches after a
    cache-flushing write; None without the measurement library."""
    import torch

    lib = _ceiling_lib()
    if lib is None:
        return None
    dst_bytes = m * k // 16 * 16
    src = torch.ones(dst_bytes * in_bytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty(dst_bytes // 4, dtype=torch.float32, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count

    def launch(grid):  # on the current stream (a graph's capture stream too)
        if lib.convrot_ceiling_stream(src.data_ptr(), dst.data_ptr(), dst_bytes, in_bytes, grid,
                                      torch.cuda.current_stream().cuda_stream) != 0:
            raise RuntimeError("stream ceiling kernel refused its arguments")

    best = min((_graph_time_ms(lambda: launch(cus * w)), cus * w) for w in (2, 4, 8, 16))
    warm, grid = best
    cold = _time_ms(lambda: launch(grid), reps=reps, flush=flush)
    del src, dst
    moved = dst_bytes * (in_bytes + 1)
    return warm, cold, moved / (warm * 1e-3) / 1e9, moved / (cold * 1e-3) / 1e9


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.all_configs:
        all_configs(args)
        return

    import torch

    import hadamard_rotated_int8_amd as cr
    import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    cr.lib()  # fails loudly when the HIP library is missing
    w = wl.WORKLOADS[args.workload]
    g = 256
    inp = wl.generate(w)
    x = inp["x"].cuda()
    qws = [cr.quantize_weights(torch.from_numpy(wt).cuda(), g, torch.from_numpy(b).cuda())
           for wt, b in zip(inp["weights"], inp["biases"])]
    m, k = w.m, w.k
    packed = cr.PackedActivation(torch.empty((m, k), dtype=torch.int8, device="cuda"),
                                 torch.empty((m,), dtype=torch.float32, device="cuda"), g)
    ys = [torch.empty((m, q.q.shape[0]), dtype=torch.float32, device="cuda") for q in qws]
    torch.cuda.synchronize()
    pack_bytes = m * k * (2 if x.dtype == torch.bfloat16 else 4) + m * k + 4 * m

    # Before the step loop: the pack alone (warm: graph-replayed back-to-back
    # launches, device time; cold:
    # after a 512 MB cache-flushing write), an HBM stream of the same bytes in
    # the same read:write mix, the matrix cores' rate on these operand codes, and the grouped
    # GEMM alone over 200 back-to-back launches.  Besides their own figures
    # these runs (about 0.1 s) bring the shader clock to the state it holds
    # under sustained work before the warm-up steps begin: from idle, the
    # GEMM needs about 200 launches to settle.
    flush = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
    pack_avg_ms = _graph_time_ms(lambda: cr.pack_activations(x, g, out=packed))
    pack_cold_ms = _time_ms(lambda: cr.pack_activations(x, g, out=packed), reps=20, flush=flush)
    stream = stream_ceiling(m, k, 2 if x.dtype == torch.bfloat16 else 4, flush)
    del flush
    mfma_loop_tops = mfma_ceiling(packed.q, qws[0].q)
    gemm_alone_ms = _time_ms(lambda: cr.linear_grouped(packed, qws, outs=ys), reps=200)
    pack_gbps = pack_bytes / (pack_avg_ms * 1e-3) / 1e9
    pack_cold_gbps = pack_bytes / (pack_cold_ms * 1e-3) / 1e9

    # Events are recorded on the current stream, the one the library launches
    # on.  A timed event costs about 2 us of stream time here, so the GEMM's
    # own duration is sampled on every EVERY-th step of the timed region
    # (none around the pack), which keeps the step time close to that of
    # plain back-to-back launches.
    EVERY = 4

    def step(ev=None):
        cr.pack_activations(x, g, out=packed)
        if ev is not None:
            ev[0].record()
        cr.linear_grouped(packed, qws, outs=ys)
        if ev is not None:
            ev[1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    sampled = list(range(0, args.steps, EVERY))
    events = {s: [torch.cuda.Event(enable_timing=True) for _ in range(2)] for s in sampled}
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for s in range(args.steps):
        step(events.get(s))
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / args.steps

    gemm_ms = np.array([e[0].elapsed_time(e[1]) for e in events.values()])
    n_total = sum(q.q.shape[0] for q in qws)
    ops = 2.0 * m * n_total * k
    value = ops / (ms_per_step * 1e-3) / 1e12
    gemm_ops_per_launch = ops  # one grouped launch covers all three weights
    gemm_avg_ms = float(gemm_ms.mean())
    gemm_tops = gemm_ops_per_launch / (gemm_avg_ms * 1e-3) / 1e12
    traffic = gemm_traffic()

    out = {
        "metric": "convrot linear effective INT8 TOPS at 4096x3072x9216; act-pack HBM GB/s",
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "m": m, "k": k, "n": [q.q.shape[0] for q in qws], "group_size": g,
            "x_dtype": w.x_dtype, "y_dtype": "f32",
            "step": "1 pack + 1 grouped launch of 3 linears on the packed activation",
        },
        "linear_tops": round(gemm_tops, 2),
        "gemm_us_per_launch": round(gemm_avg_ms * 1e3, 3),
        "gemm_launches_timed": len(gemm_ms),
        "pack_us_warm": round(pack_avg_ms * 1e3, 3),
        "pack_gbps_warm": round(pack_gbps, 1),
        "pack_us_cold": round(pack_cold_ms * 1e3, 3),
        "pack_gbps_cold": round(pack_cold_gbps, 1),
        "pack_hbm_frac_cold": round(pack_cold_gbps / PEAK_HBM_GBPS, 4),
        "stream_gbps_warm": None if stream is None else round(stream[2], 1),
        "stream_gbps_cold": None if stream is None else round(stream[3], 1),
        "pack_frac_of_stream_warm": None if stream is None else round(pack_gbps / stream[2], 4),
        "pack_frac_of_stream_cold": None if stream is None else round(pack_cold_gbps / stream[3], 4),
        "gemm_us_back_to_back": round(gemm_alone_ms * 1e3, 3),
        "mfma_loop_tops": None if mfma_loop_tops is None else round(mfma_loop_tops, 1),
        "gemm_frac_of_mfma_loop": (None if mfma_loop_tops is None
                                   else round(gemm_tops / mfma_loop_tops, 4)),
        "wall_s_timed": round(wall, 3),
        "roofline": {
            "bound": "mfma",
            "kernel": "gemm_i8_kernel (grouped Q, K, V: 4096 x 9216 x 3072)",
            "achieved": round(gemm_tops, 2),
            "peak": PEAK_INT8_TOPS,
            # tera-operations per second (int8 multiply-add = 2 operations)
            "unit": "TFLOP/s",
            "frac": round(gemm_tops / PEAK_INT8_TOPS, 4),
            "traffic": traffic,
            "traffic_source": (None if traffic is None else
                               "profiles/gemm_qkv_4096x3072x9216_traffic.json: rocprofv3 FETCH_SIZE + "
                               "WRITE_SIZE per launch, scaled by a plain copy, taken on this gemm.hip"),
        },
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, w, g, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
