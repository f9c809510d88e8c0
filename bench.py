"""Benchmark: effective weight GB/s and fraction of HBM peak of the 4-bit
k-means-palettized (km4) lm_head matvec, 248320 x 2048, batch 1, on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]

A step is one call of the fused dequantize-matvec on the lm_head weights
(the decode hot path; quantize-and-pack is export-time work and is timed once
beside it). Inputs are seeded synthetic tensors of the lm_head's shape, packed
on the GPU, resident in HBM before timing starts. Four copies of the packed
weights (4 x 262 MB) are cycled so that no call finds its weights in the
256 MB Infinity Cache. Time is taken with HIP events on the stream the kernel
runs on, around exactly K calls after W warm-up calls.

Prints one JSON line. `value` = algorithmic bytes per call (codes + tables,
262,225,920 B) / mean time per call. `roofline` compares that to the 8 TB/s
HBM peak; `traffic` comes from rocprofv3 FETCH_SIZE/WRITE_SIZE counters
recorded under profiles/ (null when no counter summary matches this kernel
build). `cpu_baseline` times the plain CPU oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

N_ROWS, K_DIM = 248320, 2048
PEAK_GBS = 8000.0
METRIC = "effective weight GB/s & % HBM peak for 4-bit lm_head matvec (248320×2048, B=1)"
ROOT = os.path.dirname(os.path.abspath(__file__))


def algo_bytes(fmt, N, K):
    """Bytes a call must read from HBM: code plane plus scale/table plane."""
    codes = N * K if fmt in ("int8", "int8km") else N * K // 2
    plane = {"int4": N * (K // 32) * 2, "int8": N * (K // 32) * 2, "fp4": N * (K // 32), "km4": N * 16 * 2,
             "int4aff": N * (K // 32) * 4, "int8km": (N // 32) * 512}[fmt]
    return codes + plane


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=4)
    ap.add_argument("--quick", action="store_true", help="skip the int8 head, the MoE layer and the fp4 4096^2 config")
    ap.add_argument("--all", action="store_true", help="(default; kept for older command lines)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only-metric", action="store_true", help="time the metric kernel only (for profiling)")
    ap.add_argument("--case", default=None,
                    help="time one other kernel only (for profiling): FMT_bB with FMT in fp4, int4, int4aff, "
                         "int8km, km4 and B in 1, 4, 8 (lm_head shape); int8_head; argmax_bB; moe")
    ap.add_argument("--calibrate", action="store_true",
                    help="run a plain 1 GiB device copy and a 1 GiB streaming read, for HBM byte-counter calibration")
    return ap.parse_args()


def calibrate():
    """Known-size traffic for scaling the FETCH_SIZE / WRITE_SIZE counters:
    5 device-to-device copies of 1 GiB (torch's copy kernel: 1 GiB read and
    1 GiB written each) and 5 streaming reads of 1 GiB (qmv_stream_read)."""
    import torch
    import quantized_decode_matvec_amd as qmv
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.random_(0, 255)
    dst = torch.empty_like(src)
    sink = torch.empty((int(qmv.lib().qmv_stream_read_sink_words(n)),), dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    for _ in range(5):
        qmv.qmv_stream_read(src, sink=sink)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_bytes_per_copy": n, "copies": 5, "stream_reads": 5}))


def gpu_warm(fn, seconds=0.2):
    """Run the timed operation itself, untimed, for a moment so the clocks have
    left their idle state before the warm-up steps (a heavier load here, such
    as GEMMs, leaves the chip power-limited for what follows)."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(50):
            fn(i)
            i += 1
        torch.cuda.synchronize()


def timed(fn, steps, warmup):
    """Mean ms per call over `steps` calls, HIP events on the current stream."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for i in range(steps):
        fn(i)
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def per_call_us(fn, steps):
    """p10 / median / p90 of single-call durations (an event pair around each
    of `steps` back-to-back calls, after the timed loop; not used for `value`)."""
    import torch
    st = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(st)
    for i in range(steps):
        fn(i)
        ev[i + 1].record(st)
    torch.cuda.synchronize()
    d = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(steps))
    pick = lambda q: round(d[min(len(d) - 1, int(q * len(d)))], 2)
    return pick(0.1), pick(0.5), pick(0.9)


def timed_graph(fn, steps, per_graph=32):
    """Mean ms per call with `per_graph` calls captured in one HIP graph and the
    graph replayed (removes host launch overhead; for microsecond-scale ops)."""
    import torch
    for i in range(3):
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(per_graph):
            fn(i)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // per_graph)
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        g.replay()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * per_graph)


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


_CASES = {}


def workload(name):
    """A seeded synthetic workload from quantized_decode_matvec_amd.workloads,
    generated once per run (the MoE slabs take about 30 s of numpy)."""
    if name not in _CASES:
        from quantized_decode_matvec_amd import workloads as wl
        _CASES[name] = getattr(wl, name)()
    return _CASES[name]


def traffic_from_profiles(key):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel sources (otherwise None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    from quantized_decode_matvec_amd.rocprof_summary import kernel_source_hash
    try:
        rec = json.load(open(path)).get(key)
    except ValueError:
        return None
    if not rec or rec.get("kernel_source_sha256") != kernel_source_hash(rec.get("kernel_sources") or None):
        return None
    return rec["traffic_bytes"]


def cpu_baseline(c, x1):
    """The oracle, untuned: pack a sample of rows, then time its matvec on them,
    on all cores (the reported baseline) and on one thread (an extra)."""
    import oracle
    rows = 4096
    codes, lut = oracle.pack_km4(c.W[:rows])
    bytes_per_row = algo_bytes("km4", 1, K_DIM)

    def rate(seconds):
        t0 = time.perf_counter()
        reps = 0
        while True:
            oracle.matvec("km4", codes, lut, x1)
            reps += 1
            el = time.perf_counter() - t0
            if el > seconds or reps >= 10000:
                break
        return rows * bytes_per_row * reps / el / 1e9, reps, el

    cores = oracle.num_threads()
    gbs, reps, el = rate(10.0)
    oracle.set_num_threads(1)
    try:
        gbs1, reps1, el1 = rate(5.0)
    finally:
        oracle.set_num_threads(cores)
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": "km4 matvec over the first %d of 248320 lm_head rows (batch 1), %d repetitions, %.1f s"
                      % (rows, reps, el)}, {"cpu_oracle_1thread_GBps": round(gbs1, 4),
                                            "cpu_oracle_1thread_reps": reps1}


def cpu_configs(lm, quick):
    """The oracle as it stands (untuned) on each workload, on all cores and on
    one thread: packing time and matvec rate in GB/s of that workload's
    algorithmic weight bytes. The lm_head and the int8 head are sampled by
    rows (the first 4096 / 8192 rows; rows are independent); the MoE layer
    runs one token through its 8 routed experts (packing only those). The
    tiny int4 and the fp4 4096 x 4096 workloads run whole. With `quick`, the
    int8 head and the MoE layer are left out (they are not generated)."""
    import oracle

    cores = oracle.num_threads()
    out = {"cpu_cores": cores}

    def timed_host(fn, min_s):
        reps, t0 = 0, time.perf_counter()
        while True:
            r = fn()
            reps += 1
            el = time.perf_counter() - t0
            if el >= min_s:
                return r, el / reps

    def dense(name, fmt, W, x, note):
        nb = algo_bytes(fmt, *W.shape)
        for thr, tag in ((cores, "all"), (1, "1thr")):
            oracle.set_num_threads(thr)
            try:
                (codes, plane), tp = timed_host(lambda: oracle.pack(fmt, W), 0.0)
                _, tm = timed_host(lambda: oracle.matvec(fmt, codes, plane, x), 0.3)
            finally:
                oracle.set_num_threads(cores)
            out["cpu_%s_%s_pack_ms" % (name, tag)] = round(tp * 1e3, 2)
            out["cpu_%s_%s_matvec_ms" % (name, tag)] = round(tm * 1e3, 3)
            out["cpu_%s_%s_matvec_GBps" % (name, tag)] = round(nb / tm / 1e9, 4)
        out["cpu_%s_sample" % name] = note

    c1 = workload("tiny_int4")
    dense("tiny_int4", "int4", c1.W, c1.x, "whole 256x512, x fp32 [1, 512]")
    c2 = workload("fp4_square")
    dense("fp4_4096sq", "fp4", c2.W, c2.x[:1], "whole 4096x4096, batch 1")
    dense("km4_lm_head", "km4", lm.W[:4096], lm.x[:1], "first 4096 of 248320 rows, batch 1")
    if not quick:
        c4 = workload("int8_head")
        dense("int8_head", "int8", c4.W[:8192], c4.x, "first 8192 of 130560 rows, batch 1")
        c5 = workload("moe")
        ids, w = oracle.moe_route(c5.logits[:1], c5.topk)
        E, I2, H = c5.W_gate_up.shape
        I = I2 // 2
        experts = sorted(set(int(e) for e in ids.reshape(-1)))
        per_expert = algo_bytes("int4", I2, H) + algo_bytes("int4", H, I)
        for thr, tag in ((cores, "all"), (1, "1thr")):
            oracle.set_num_threads(thr)
            try:
                t0 = time.perf_counter()
                guc = np.zeros((E, I2, H // 2), np.uint8)
                gus = np.zeros((E, I2, H // 32), np.uint16)
                dnc = np.zeros((E, H, I // 2), np.uint8)
                dns = np.zeros((E, H, I // 32), np.uint16)
                for e in experts:
                    guc[e], gus[e] = oracle.pack_int4(c5.W_gate_up[e])
                    dnc[e], dns[e] = oracle.pack_int4(c5.W_down[e])
                tp = time.perf_counter() - t0
                _, tm = timed_host(lambda: oracle.moe_ffn(guc, gus, dnc, dns, c5.x[:1], ids, w), 0.3)
            finally:
                oracle.set_num_threads(cores)
            out["cpu_moe_int4_T1_%s_pack_ms" % tag] = round(tp * 1e3, 2)
            out["cpu_moe_int4_T1_%s_ms" % tag] = round(tm * 1e3, 3)
            out["cpu_moe_int4_T1_%s_GBps" % tag] = round(len(experts) * per_expert / tm / 1e9, 4)
        out["cpu_moe_int4_T1_sample"] = "one token, its %d routed experts packed" % len(experts)
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU (torch.cuda.is_available() is False)", file=sys.stderr)
        sys.exit(1)
    if args.calibrate:
        calibrate()
        return
    if args.case:
        run_case(args)
        return
    import quantized_decode_matvec_amd as qmv
    from quantized_decode_matvec_amd import workloads as wl

    log("generating lm_head weights %dx%d" % (N_ROWS, K_DIM))
    c = wl.lm_head_km4(batch=8)
    W = torch.from_numpy(c.W).cuda()
    x8 = torch.from_numpy(c.x).cuda()
    x1 = x8[:1].contiguous()
    torch.cuda.synchronize()

    ev = lambda: torch.cuda.Event(enable_timing=True)
    e0, e1 = ev(), ev()
    e0.record()
    codes, lut = qmv.qpack_km4(W)
    e1.record()
    torch.cuda.synchronize()
    pack_ms = e0.elapsed_time(e1)
    log("km4 pack %.1f ms" % pack_ms)
    copies = [(codes, lut)] + [(codes.clone(), lut.clone()) for _ in range(args.copies - 1)]
    y = torch.empty((8, N_ROWS), dtype=torch.float32, device="cuda")
    # the row-tiled code plane the batch-1 lm_head kernel reads (a one-time
    # reordering of the same bytes, done when the weights are loaded)
    tiled0 = qmv.qtile_km4(codes)
    # the relayout kernel alone (the first call above also allocates)
    e0.record()
    qmv.qtile_km4(codes, tiled=tiled0)
    e1.record()
    torch.cuda.synchronize()
    tile_ms = e0.elapsed_time(e1)
    tiled = [(tiled0 if i == 0 else qmv.qtile_km4(cc), ll) for i, (cc, ll) in enumerate(copies)]

    # checked once; each call then only launches (a decode loop's hot path)
    calls1 = [qmv.qmatvec_km4_tiled_call(tt, ll, x1, y=y[:1]) for tt, ll in tiled]

    def step(i):
        calls1[i % len(calls1)]()

    gpu_warm(step)
    ms = timed(step, args.steps, args.warmup)
    p10 = p50 = p90 = None
    if not args.only_metric:
        p10, p50, p90 = per_call_us(step, args.steps)
    nbytes = algo_bytes("km4", N_ROWS, K_DIM)
    gbs = nbytes / (ms * 1e-3) / 1e9
    log("km4 B=1: %.2f us/call, %.1f GB/s (%.1f%% of 8 TB/s)" % (ms * 1e3, gbs, gbs / PEAK_GBS * 100))

    extras = {"km4_pack_ms": round(pack_ms, 3), "km4_tile_ms": round(tile_ms, 3)}
    if p50 is not None:
        extras.update({"km4_B1_us_p10": p10, "km4_B1_us_p50": p50, "km4_B1_us_p90": p90})
    if not args.only_metric:
        # the same matvec from the row-major code plane (the row-per-wave kernel)
        callsr = [qmv.qmatvec_call("km4", cc, ll, x1, y=y[:1]) for cc, ll in copies]
        msr = timed(lambda i: callsr[i % len(callsr)](), args.steps, args.warmup)
        extras["km4_rowmajor_B1_us"] = round(msr * 1e3, 2)
        extras["km4_rowmajor_B1_GBps"] = round(nbytes / (msr * 1e-3) / 1e9, 1)
        del callsr
    def stream_rate(nb):
        """GB/s of the plain streaming read over `nb` bytes, cycling the same
        number of buffers as the weight copies (the read each matvec is set
        against: same bytes, same cache behaviour)."""
        buf = torch.empty((len(copies), nb // 16 * 16), dtype=torch.uint8, device="cuda")
        buf.random_(0, 255)
        sink = torch.empty((int(qmv.lib().qmv_stream_read_sink_words(buf[0].numel())),), dtype=torch.int32,
                           device="cuda")
        ms_r = timed(lambda i: qmv.qmv_stream_read(buf[i % len(copies)], sink=sink), args.steps, args.warmup)
        rate = buf[0].numel() / (ms_r * 1e-3) / 1e9
        del buf, sink
        return round(rate, 1)

    if not args.only_metric:
        # plain streaming read over the same footprint
        extras["stream_read_GBps"] = stream_rate(nbytes)
        log("stream read %.1f GB/s" % extras["stream_read_GBps"])

        # batch 2-4 from the row-tiled plane (one table lookup feeds B products)
        for bb in (2, 3, 4):
            ct = [qmv.qmatvec_km4_tiled_call(tt, ll, x8[:bb], y=y[:bb]) for tt, ll in tiled]
            mst = timed(lambda i: ct[i % len(ct)](), args.steps // 2, args.warmup)
            extras["km4_tiled_B%d_us" % bb] = round(mst * 1e3, 2)
            extras["km4_tiled_B%d_GBps" % bb] = round(nbytes / (mst * 1e-3) / 1e9, 1)
            del ct
        cr2 = [qmv.qmatvec_call("km4", cc, ll, x8[:2], y=y[:2]) for cc, ll in copies]
        ms2r = timed(lambda i: cr2[i % len(cr2)](), args.steps // 2, args.warmup)
        extras["km4_B2_us"] = round(ms2r * 1e3, 2)
        extras["km4_B2_GBps"] = round(nbytes / (ms2r * 1e-3) / 1e9, 1)
        del cr2
        calls4 = [qmv.qmatvec_call("km4", cc, ll, x8[:4], y=y[:4]) for cc, ll in copies]
        ms4 = timed(lambda i: calls4[i % len(calls4)](), args.steps // 2, args.warmup)
        extras["km4_B4_us"] = round(ms4 * 1e3, 2)
        extras["km4_B4_GBps"] = round(nbytes / (ms4 * 1e-3) / 1e9, 1)
        calls8 = [qmv.qmatvec_call("km4", cc, ll, x8, y=y) for cc, ll in copies]
        ms8 = timed(lambda i: calls8[i % len(calls8)](), args.steps // 2, args.warmup)
        extras["km4_B8_us"] = round(ms8 * 1e3, 2)
        extras["km4_B8_GBps"] = round(nbytes / (ms8 * 1e-3) / 1e9, 1)
        del calls4

        e0.record()
        pk8 = qmv.qpack_int8km(W)
        e1.record()
        torch.cuda.synchronize()
        extras["int8km_pack_ms"] = round(e0.elapsed_time(e1), 3)
        del pk8
        for fmt in ("fp4", "int4", "int4aff", "int8km"):
            pk = [qmv.qpack(fmt, W)]
            pk += [(a.clone(), b.clone()) for a, b in [pk[0]] * (len(copies) - 1)]
            cf = [qmv.qmatvec_call(fmt, a, b, x1, y=y[:1]) for a, b in pk]
            msf = timed(lambda i: cf[i % len(cf)](), args.steps, args.warmup)
            nb = algo_bytes(fmt, N_ROWS, K_DIM)
            extras["%s_B1_us" % fmt] = round(msf * 1e3, 2)
            extras["%s_B1_GBps" % fmt] = round(nb / (msf * 1e-3) / 1e9, 1)
            extras["%s_stream_read_GBps" % fmt] = stream_rate(nb)
            for bb in (4, 8):
                cb = [qmv.qmatvec_call(fmt, a, b, x8[:bb], y=y[:bb]) for a, b in pk]
                msb = timed(lambda i: cb[i % len(cb)](), args.steps // 2, args.warmup)
                extras["%s_B%d_us" % (fmt, bb)] = round(msb * 1e3, 2)
                extras["%s_B%d_GBps" % (fmt, bb)] = round(nb / (msb * 1e-3) / 1e9, 1)
            del pk, cf, cb
        # km4 rows plus 16 int8 outliers per row (0.8% of the weights)
        e0.record()
        pko = qmv.qpack_km4o(W, 16)
        e1.record()
        torch.cuda.synchronize()
        extras["km4o16_pack_ms"] = round(e0.elapsed_time(e1), 3)
        pks = [pko] + [tuple(a.clone() for a in pko) for _ in range(len(copies) - 1)]
        nbo = algo_bytes("km4", N_ROWS, K_DIM) + N_ROWS * (16 * 3 + 2)
        mso = timed(lambda i: qmv.qmatvec_km4o(*pks[i % len(pks)], x1, y=y[:1]), args.steps, args.warmup)
        extras["km4o16_B1_us"] = round(mso * 1e3, 2)
        extras["km4o16_B1_GBps"] = round(nbo / (mso * 1e-3) / 1e9, 1)
        # the same from the row-tiled codes
        pkt = [(qmv.qtile_km4(p[0]),) + tuple(p[1:]) for p in pks]
        msot = timed(lambda i: qmv.qmatvec_km4o_tiled(*pkt[i % len(pkt)], x1, y=y[:1]), args.steps, args.warmup)
        extras["km4o16_tiled_B1_us"] = round(msot * 1e3, 2)
        extras["km4o16_tiled_B1_GBps"] = round(nbo / (msot * 1e-3) / 1e9, 1)
        msot4 = timed(lambda i: qmv.qmatvec_km4o_tiled(*pkt[i % len(pkt)], x8[:4], y=y[:4]), args.steps // 2,
                      args.warmup)
        extras["km4o16_tiled_B4_us"] = round(msot4 * 1e3, 2)
        del pkt
        del pks, pko
        # fp16 dense GEMV on the same shape (torch), for the per-op ratio against fp16
        wcp = [W] + [W.clone() for _ in range(1)]
        msd = timed(lambda i: torch.matmul(x1, wcp[i % 2].t()), max(10, args.steps // 4), 5)
        extras["fp16_dense_torch_us"] = round(msd * 1e3, 2)
        extras["km4_speedup_vs_fp16_dense"] = round(msd / ms, 2)
        del wcp
        # fused lm_head + argmax (no logits written) against matvec + torch.argmax
        ws = torch.empty((qmv.qmatvec_argmax_workspace_bytes(N_ROWS, 1),), dtype=torch.uint8, device="cuda")
        aidx = torch.empty((1,), dtype=torch.int32, device="cuda")
        aval = torch.empty((1,), dtype=torch.float32, device="cuda")
        msa = timed(lambda i: qmv.qmatvec_argmax("km4", copies[i % len(copies)][0], copies[i % len(copies)][1], x1,
                                                 idx=aidx, val=aval, workspace=ws), args.steps, args.warmup)

        def two_step(i):
            qmv.qmatvec_km4(copies[i % len(copies)][0], copies[i % len(copies)][1], x1, y=y[:1])
            torch.argmax(y[:1], dim=1)

        ms2 = timed(two_step, args.steps, args.warmup)
        extras["km4_argmax_fused_us"] = round(msa * 1e3, 2)
        # the same from the row-tiled plane
        mst = timed(lambda i: qmv.qmatvec_argmax_km4_tiled(tiled[i % len(tiled)][0], tiled[i % len(tiled)][1], x1,
                                                           idx=aidx, val=aval, workspace=ws), args.steps, args.warmup)
        extras["km4_tiled_argmax_fused_us"] = round(mst * 1e3, 2)
        extras["km4_matvec_then_argmax_us"] = round(ms2 * 1e3, 2)
        # batch 8: the matrix-core matvec then the argmax launch
        ws8 = torch.empty((qmv.qmatvec_argmax_workspace_bytes(N_ROWS, 8),), dtype=torch.uint8, device="cuda")
        aidx8 = torch.empty((8,), dtype=torch.int32, device="cuda")
        aval8 = torch.empty((8,), dtype=torch.float32, device="cuda")
        msa8 = timed(lambda i: qmv.qmatvec_argmax("km4", copies[i % len(copies)][0], copies[i % len(copies)][1], x8,
                                                  idx=aidx8, val=aval8, workspace=ws8), max(10, args.steps // 4), 5)
        extras["km4_argmax_fused_B8_us"] = round(msa8 * 1e3, 2)
        del ws, ws8
        # int8 embedding dequant-gather from a table of the same shape, 8 tokens (HIP graphs)
        tq, ts = qmv.qpack_int8_rows(W)
        gids = torch.randint(0, N_ROWS, (8,), dtype=torch.int32, device="cuda",
                             generator=torch.Generator(device="cuda").manual_seed(0))
        gout = torch.empty((8, K_DIM), dtype=torch.float16, device="cuda")
        msg = timed_graph(lambda i: qmv.qembed_gather_int8(tq, ts, gids, out=gout), args.steps, per_graph=64)
        extras["embed_gather_int8_8tok_us"] = round(msg * 1e3, 2)
        del tq, ts
        # attention projections of the pages' shapes (q: 2048 -> 4096, o: 4096 -> 2048)
        for name, (n, k) in {"q_proj": (4096, 2048), "o_proj": (2048, 4096)}.items():
            cc = wl.small_dense("km4", n, k, batch=1, seed=1)
            Wq = torch.from_numpy(cc.W).cuda()
            xq = torch.from_numpy(cc.x).cuda()
            for fmt in ("km4", "fp4"):
                p0 = qmv.qpack(fmt, Wq)
                pk = [p0] + [(p0[0].clone(), p0[1].clone()) for _ in range(127)]
                yq = torch.empty((1, n), dtype=torch.float32, device="cuda")
                msq = timed_graph(lambda i: qmv.qmatvec(fmt, pk[i % 128][0], pk[i % 128][1], xq, y=yq),
                                  4 * args.steps, per_graph=128)
                extras["%s_%s_us" % (name, fmt)] = round(msq * 1e3, 2)
                extras["%s_%s_GBps" % (name, fmt)] = round(algo_bytes(fmt, n, k) / (msq * 1e-3) / 1e9, 1)
                del pk
            # the floor for this size: the plain streaming read of the fp4
            # footprint, 128 distinct buffers in the same graphs
            nbq = algo_bytes("fp4", n, k) // 16 * 16
            rb = torch.empty((128, nbq), dtype=torch.uint8, device="cuda")
            rsink = torch.empty((int(qmv.lib().qmv_stream_read_sink_words(nbq)),), dtype=torch.int32, device="cuda")
            msr = timed_graph(lambda i: qmv.qmv_stream_read(rb[i % 128], sink=rsink), 4 * args.steps, per_graph=128)
            extras["%s_stream_read_fp4_bytes_us" % name] = round(msr * 1e3, 2)
            del rb
        # one GPU's share of an lm_head split by rows over 8 GPUs (31040 x 2048):
        # the 32 distinct row slices of the weight copies, so no call finds its
        # codes in the cache; matvec and the fused argmax, in HIP graphs
        ns = N_ROWS // 8
        sl = [(cc[s * ns:(s + 1) * ns], ll[s * ns:(s + 1) * ns]) for cc, ll in copies for s in range(8)]
        mss = timed_graph(lambda i: qmv.qmatvec_km4(sl[i % len(sl)][0], sl[i % len(sl)][1], x1, y=y[:1, :ns]),
                          4 * args.steps, per_graph=len(sl))
        wss = torch.empty((qmv.qmatvec_argmax_workspace_bytes(ns, 1),), dtype=torch.uint8, device="cuda")
        msx = timed_graph(lambda i: qmv.qmatvec_argmax("km4", sl[i % len(sl)][0], sl[i % len(sl)][1], x1, idx=aidx,
                                                       val=aval, workspace=wss), 4 * args.steps, per_graph=len(sl))
        extras["km4_shard8_%d_us" % ns] = round(mss * 1e3, 2)
        extras["km4_shard8_%d_GBps" % ns] = round(algo_bytes("km4", ns, K_DIM) / (mss * 1e-3) / 1e9, 1)
        extras["km4_shard8_%d_argmax_us" % ns] = round(msx * 1e3, 2)
        # the same shares of the row-tiled planes (31040 rows = 485 whole tiles)
        tb = qmv.qtile_km4_bytes(ns, K_DIM)
        slt = [(tc[s * tb:(s + 1) * tb], ll[s * ns:(s + 1) * ns]) for tc, ll in tiled for s in range(8)]
        mst8 = timed_graph(lambda i: qmv.qmatvec_km4_tiled(slt[i % len(slt)][0], slt[i % len(slt)][1], x1,
                                                           y=y[:1, :ns]), 4 * args.steps, per_graph=len(slt))
        mstx = timed_graph(lambda i: qmv.qmatvec_argmax_km4_tiled(slt[i % len(slt)][0], slt[i % len(slt)][1], x1,
                                                                  idx=aidx, val=aval, workspace=wss),
                           4 * args.steps, per_graph=len(slt))
        extras["km4_tiled_shard8_%d_us" % ns] = round(mst8 * 1e3, 2)
        extras["km4_tiled_shard8_%d_GBps" % ns] = round(algo_bytes("km4", ns, K_DIM) / (mst8 * 1e-3) / 1e9, 1)
        extras["km4_tiled_shard8_%d_argmax_us" % ns] = round(mstx * 1e3, 2)
        del sl, slt, wss
        if not args.quick:
            extras.update(bench_fp4_square(args))
            extras.update(bench_int8_head(args))
            extras.update(bench_moe(args))

    traffic = traffic_from_profiles("km4_tiled_lm_head_b1")
    if not args.only_metric:
        # the fastest whole-HBM read of this run (the plain streaming read over
        # each format's footprint, or a batch-1 matvec when one reads faster):
        # the practical ceiling the batch-1 kernels are judged against
        reads = {k: v for k, v in extras.items()
                 if k.endswith("stream_read_GBps") or k.endswith("_B1_GBps") or k == "int8_head_GBps"}
        best = max(reads, key=reads.get)
        extras["best_read_GBps"], extras["best_read_kernel"] = reads[best], best
        extras["km4_B1_frac_of_best_read"] = round(gbs / reads[best], 4)
    result = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "lm_head km4 matvec 248320x2048, batch 1, fp16 x, fp32 accumulate, "
                               "codes in the row-tiled layout",
                   "N": N_ROWS, "K": K_DIM, "batch": 1, "format": "km4 (4-bit index + 16-entry fp16 table per row)",
                   "algorithmic_bytes_per_call": nbytes, "weight_copies_cycled": len(copies)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_GBS, 4), "traffic": traffic},
        "extras": extras,
    }
    if not args.no_cpu and not args.only_metric:
        log("cpu baseline (oracle)")
        result["cpu_baseline"], one = cpu_baseline(c, c.x[:1])
        extras.update(one)
        log("cpu oracle on each workload")
        extras.update(cpu_configs(c, args.quick))
    print(json.dumps(result), flush=True)


def bench_fp4_square(args):
    """fp4 4096 x 4096 (8.9 MB of codes and scales, batch 1 and 4): 64 weight
    copies cycled so no call finds its weights in the 256 MB cache; HIP graphs
    of 64 calls, since one call is launch-latency bound."""
    import torch
    import quantized_decode_matvec_amd as qmv
    from quantized_decode_matvec_amd import workloads as wl
    c = workload("fp4_square")
    W = torch.from_numpy(c.W).cuda()
    p0 = qmv.qpack_fp4(W)
    del W
    pk = [p0] + [(p0[0].clone(), p0[1].clone()) for _ in range(63)]
    nb = algo_bytes("fp4", 4096, 4096)
    out = {}
    for B in (1, 4):
        x = torch.from_numpy(c.x[:B]).cuda().contiguous()
        y = torch.empty((B, 4096), dtype=torch.float32, device="cuda")
        ms = timed_graph(lambda i: qmv.qmatvec_fp4(pk[i % 64][0], pk[i % 64][1], x, y=y), 4 * args.steps,
                         per_graph=64)
        out["fp4_4096sq_B%d_us" % B] = round(ms * 1e3, 2)
        out["fp4_4096sq_B%d_GBps" % B] = round(nb / (ms * 1e-3) / 1e9, 1)
    return out


def bench_int8_head(args):
    import torch
    import quantized_decode_matvec_amd as qmv
    from quantized_decode_matvec_amd import workloads as wl
    c = workload("int8_head")
    W = torch.from_numpy(c.W).cuda()
    x = torch.from_numpy(c.x).cuda()
    p0 = qmv.qpack_int8(W)
    del W
    pk = [p0] + [(p0[0].clone(), p0[1].clone()) for _ in range(2)]
    cs = [qmv.qmatvec_call("int8", a, b, x) for a, b in pk]
    ms = timed(lambda i: cs[i % 3](), args.steps, args.warmup)
    nb = algo_bytes("int8", *c.W.shape)
    return {"int8_head_us": round(ms * 1e3, 2), "int8_head_GBps": round(nb / (ms * 1e-3) / 1e9, 1)}


def run_case(args):
    """One kernel alone, `args.steps` timed calls (for counter runs under rocprofv3)."""
    import torch
    import quantized_decode_matvec_amd as qmv
    from quantized_decode_matvec_amd import workloads as wl
    case = args.case
    res = {"case": case}
    if case == "moe":
        res.update(bench_moe(args, fmts=("int4",)))
    elif case == "int8_head":
        res.update(bench_int8_head(args))
    else:
        name, b = case.rsplit("_b", 1)
        B = int(b)
        c = wl.lm_head_km4(batch=8)
        W = torch.from_numpy(c.W).cuda()
        x = torch.from_numpy(c.x[:B]).cuda().contiguous()
        fmt = "km4" if name == "argmax" else name
        p0 = qmv.qpack(fmt, W)
        del W
        pk = [p0] + [(p0[0].clone(), p0[1].clone()) for _ in range(args.copies - 1)]
        y = torch.empty((B, N_ROWS), dtype=torch.float32, device="cuda")
        if name == "argmax":
            ws = torch.empty((qmv.qmatvec_argmax_workspace_bytes(N_ROWS, B),), dtype=torch.uint8, device="cuda")
            idx = torch.empty((B,), dtype=torch.int32, device="cuda")
            val = torch.empty((B,), dtype=torch.float32, device="cuda")
            fn = lambda i: qmv.qmatvec_argmax(fmt, pk[i % len(pk)][0], pk[i % len(pk)][1], x, idx=idx, val=val,
                                              workspace=ws)
        else:
            cs = [qmv.qmatvec_call(fmt, a, b, x, y=y) for a, b in pk]
            fn = lambda i: cs[i % len(cs)]()
        gpu_warm(fn)
        ms = timed(fn, args.steps, args.warmup)
        res.update({"us": round(ms * 1e3, 2), "GBps": round(algo_bytes(fmt, N_ROWS, K_DIM) / (ms * 1e-3) / 1e9, 1)})
    print(json.dumps(res), flush=True)


MOE_CALLS, MOE_COPIES = 128, 4


def bench_moe(args, fmts=("int4", "int4aff", "int8km"), tokens=(1, 4, 8)):
    """The MoE layer (E = 256, top-8, H = 2048, I = 512) in the pages' gather
    formats at T = 1, 4, 8 tokens, fused entry point and three-call path, in
    HIP graphs of 128 calls. Each call of a graph routes its own set of router
    logits (128 sets drawn N(0, 1) with numpy default_rng(1)) against one of 4
    copies of the expert slabs, so that what a window of calls reads is spread
    over 4 x 256 expert copies (1.8 GB in int4), far more than twice the 256 MB
    Infinity Cache: a routed expert is rarely still cached from an earlier call.
    GB/s counts each call's distinct routed experts once (the gather reads an
    expert once however many tokens chose it)."""
    import torch
    import quantized_decode_matvec_amd as qmv
    from quantized_decode_matvec_amd import workloads as wl
    c = workload("moe")
    E, I2, H = c.W_gate_up.shape
    I = I2 // 2
    lg_all = np.random.default_rng(1).standard_normal((MOE_CALLS, max(tokens), E), dtype=np.float32)
    out = {}
    for fmt in fmts:
        guc, gus = qmv.qpack(fmt, torch.from_numpy(c.W_gate_up.reshape(E * I2, H)).cuda())
        dnc, dns = qmv.qpack(fmt, torch.from_numpy(c.W_down.reshape(E * H, I)).cuda())
        slab = (guc.view(E, I2, -1), gus.view(E, -1), dnc.view(E, H, -1), dns.view(E, -1))
        copies = [slab] + [tuple(a.clone() for a in slab) for _ in range(MOE_COPIES - 1)]
        per_expert = algo_bytes(fmt, I2, H) + algo_bytes(fmt, H, I)
        for T in tokens:
            x = torch.from_numpy(c.x[:T]).cuda()
            lg = torch.from_numpy(np.ascontiguousarray(lg_all[:, :T])).cuda()
            ids = torch.empty((T, c.topk), dtype=torch.int32, device="cuda")
            w = torch.empty((T, c.topk), dtype=torch.float32, device="cuda")
            h = torch.empty((T, c.topk, I), dtype=torch.float16, device="cuda")
            y = torch.empty((T, H), dtype=torch.float32, device="cuda")
            uniq = []
            for k in range(MOE_CALLS):
                qmv.qmoe_route(lg[k], c.topk, ids=ids, weights=w)
                uniq.append(len(np.unique(ids.cpu().numpy())))
            moved = float(np.mean(uniq)) * per_expert

            def layer(i):
                g, s, d, ds = copies[i % MOE_COPIES]
                qmv.qmoe_ffn(fmt, g, s, d, ds, x, lg[i % MOE_CALLS], c.topk, ids=ids, weights=w, h=h, y=y)

            def layer3(i):
                g, s, d, ds = copies[i % MOE_COPIES]
                qmv.qmoe_route(lg[i % MOE_CALLS], c.topk, ids=ids, weights=w)
                qmv.gather_qmatvec(fmt, g, s, x, ids, epi="swiglu", y=h)
                qmv.gather_qmatvec(fmt, d, ds, h, ids, weights=w, epi="combine", x_per_slot=True, y=y)

            ms = timed_graph(layer, 4 * args.steps, per_graph=MOE_CALLS)
            ms3 = timed_graph(layer3, 4 * args.steps, per_graph=MOE_CALLS)
            out["moe_%s_T%d_us" % (fmt, T)] = round(ms * 1e3, 2)
            out["moe_%s_T%d_GBps" % (fmt, T)] = round(moved / (ms * 1e-3) / 1e9, 1)
            out["moe_%s_T%d_3call_us" % (fmt, T)] = round(ms3 * 1e3, 2)
            out["moe_T%d_experts_per_call" % T] = round(float(np.mean(uniq)), 2)
        del copies, slab, guc, gus, dnc, dns
    return out


if __name__ == "__main__":
    main()
