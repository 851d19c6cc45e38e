#!/usr/bin/env python3
"""Benchmark: N:M SpMV achieved HBM GB/s (% of peak) and speedup over the
dense GEMV, batch 1, on one MI355X.

A step is one decode token's worth of weight projections of Llama-3.1-8B
(32 layers x q, k, v, o, gate, up, down; 2:4, fp16, B = 1).  Each layer is
four launches, as a decoder issues them: q/k/v fused (one x), o, gate/up
fused (one x), down -- every one on its own layer's packed weights, so a step
streams 7.86 GB of distinct packed bytes, far beyond the 256 MB last-level
cache.  The dense baseline runs the same step on the unpruned weights with the
same fusion.  Weights are synthetic, W ~ N(0, 0.02); activations x ~ N(0, 1)
with ceil(1% K) channels x10; all seeded.  The step is captured once into a
HIP graph and replayed.

One JSON line is printed.  ``value`` = algorithmic bytes per step / step time
(bytes = packed values + bitmaps + x + y of every launch).  ``roofline`` is for
the sparse kernel instantiation that carries q/k/v, o and gate/up (all rows of
4096 columns): its launches timed in back-to-back bursts with HIP events on
the launch stream.  ``mlp_shapes`` times the Llama-3.1-8B MLP projections as
single launches.  ``cpu_baseline`` times the CPU oracle on one layer.
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

METRIC = "N:M SpMV achieved HBM GB/s (% of peak) + speedup vs dense GEMV, batch 1"
PEAK_GBS = 8000.0
P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int


# name -> (description, model shapes, layers, dtype, n, m, batch, launch groups, x kind)
ATTN_MLP = [(("q", "k", "v"), "attn"), (("o",), "o"), (("gate", "up"), "mlp"), (("down",), "down")]
MLP_ONLY = [(("gate", "up"), "mlp"), (("down",), "down")]


def workloads(I):
    w = {
        "llama31_8b": ("Llama-3.1-8B decode-step projections: 32 layers x (q+k+v fused, o, gate+up fused, down), "
                       "2:4 sparse, fp16, batch 1", I.LLAMA31_8B, 32, "fp16", 2, 4, 1, ATTN_MLP, "outliers"),
        "llama33_70b": ("Llama-3.3-70B full decode-step weight sweep: 80 layers x (q+k+v fused, o, gate+up fused, "
                        "down), 2:4 sparse, bf16, batch 1", I.LLAMA33_70B, 80, "bf16", 2, 4, 1, ATTN_MLP, "normal"),
    }
    for nmk, (n, m) in (("4of8", (4, 8)), ("2of4", (2, 4))):
        w[f"qwen3_14b_{nmk}"] = (f"Qwen3-14B MLP projections: 40 layers x (gate+up fused, down), {n}:{m} sparse, "
                                 f"bf16, batch 1, Laplace x", I.QWEN3_14B_MLP, 40, "bf16", n, m, 1, MLP_ONLY, "laplace")
        w[f"qwen3_32b_{nmk}"] = (f"Qwen3-32B MLP projections: 64 layers x (gate+up fused, down), {n}:{m} sparse, "
                                 f"bf16, batch 1, Laplace x", I.QWEN3_32B_MLP, 64, "bf16", n, m, 1, MLP_ONLY, "laplace")
    for B in (1, 2, 4, 8, 16, 32):
        w[f"qwen3_32b_b{B}"] = (f"Qwen3-32B MLP projections: 64 layers x (gate+up fused, down), 2:4 sparse, bf16, "
                                f"batch {B}", I.QWEN3_32B_MLP, 64, "bf16", 2, 4, B, MLP_ONLY, "normal")
    return w


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--workload", default="llama31_8b",
                   help="llama31_8b (default), llama33_70b, qwen3_14b_4of8, qwen3_14b_2of4, qwen3_32b_4of8, "
                        "qwen3_32b_2of4, qwen3_32b_b1/b2/b4/b8")
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--layers", type=int, default=0, help="override the workload's layer count")
    p.add_argument("--eager", action="store_true", help="launch from Python each step instead of replaying a graph")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--crossover", action="store_true",
                   help="batch crossover study instead of the step: Qwen3-32B MLP shapes (2:4 bf16) at B = 1..32, "
                        "sparse vs the dense kernel vs torch's matmul; prints one JSON line")
    p.add_argument("--no-configs", action="store_true",
                   help="leave out the other workloads' step figures (extras.configs) from the default run")
    p.add_argument("--no-glu", action="store_true",
                   help="skip the gated gate+up launch (its grid equals the plain gate+up launch's, which would mix "
                        "the two in a kernel trace keyed by kernel and grid)")
    return p.parse_args()


class Launch:
    """One launch of the step: 1-3 projections of one layer sharing one x."""

    def __init__(self, torch, nm, I, spec, tag, layer, names):
        _, shapes, _, dts, n, m, B, _, xkind = spec
        dt = {"fp16": torch.float16, "bf16": torch.bfloat16}[dts]
        self.layer, self.names, self.n, self.m, self.B = layer, names, n, m, B
        self.dtc = 0 if dts == "fp16" else 1
        self.K = K = shapes[names[0]][1]
        xseed = I.seed_of(tag, layer, names[0], "x")
        if xkind == "laplace":
            self.x = I.activation_laplace(B, K, dt, xseed, device="cuda")
        else:
            self.x = I.activation_normal(B, K, dt, xseed, device="cuda",
                                         outlier_frac=0.01 if xkind == "outliers" else 0.0)
        self.R, self.W, self.values, self.masks, self.y, self.yd = [], [], [], [], [], []
        for nme in names:
            R, K2 = shapes[nme]
            assert K2 == K
            W = I.weight(R, K, dt, I.seed_of(tag, layer, nme, "W"), device="cuda")
            v, mk = nm.pack(W, None, n, m)
            self.R.append(R)
            self.W.append(W)
            self.values.append(v)
            self.masks.append(mk)
            self.y.append(torch.empty((B, R), dtype=dt, device="cuda"))
            self.yd.append(torch.empty((B, R), dtype=dt, device="cuda"))

    @property
    def kind(self):
        return "+".join(self.names)

    def sparse_args(self, stream):
        c = len(self.names)
        return (I32(c), (P * c)(*[v.data_ptr() for v in self.values]), (P * c)(*[m.data_ptr() for m in self.masks]),
                (I64 * c)(*self.R), I64(self.K), I32(self.n), I32(self.m), I32(self.dtc), P(self.x.data_ptr()),
                I32(self.B), (P * c)(*[y.data_ptr() for y in self.y]), P(stream))

    def sparse_args_ws(self, stream, ws):
        """nm_spmv_multi_ws arguments: the plain call's, with the K-split workspace."""
        return self.sparse_args(stream)[:-1] + (P(ws.data_ptr()), I64(ws.numel()), P(stream))

    def dense_args_ws(self, stream, ws):
        return self.dense_args(stream)[:-1] + (P(ws.data_ptr()), I64(ws.numel()), P(stream))

    def dense_args(self, stream):
        c = len(self.names)
        return (I32(c), (P * c)(*[W.data_ptr() for W in self.W]), (I64 * c)(*self.R), I64(self.K), I32(self.dtc),
                P(self.x.data_ptr()), I32(self.B), (P * c)(*[y.data_ptr() for y in self.yd]), P(stream))

    def glu_args(self, stream, dense=False):
        """Arguments of nm_spmv_swiglu (or nm_gemv_dense_swiglu) for a gate+up launch."""
        if not hasattr(self, "h"):
            self.h = self.y[0].new_empty((self.B, self.R[0]))
        if dense:
            return (P(self.W[0].data_ptr()), P(self.W[1].data_ptr()), I64(self.R[0]), I64(self.K), I32(self.dtc),
                    P(self.x.data_ptr()), I32(self.B), P(self.h.data_ptr()), P(stream))
        return (P(self.values[0].data_ptr()), P(self.masks[0].data_ptr()), P(self.values[1].data_ptr()),
                P(self.masks[1].data_ptr()), I64(self.R[0]), I64(self.K), I32(self.n), I32(self.m), I32(self.dtc),
                P(self.x.data_ptr()), I32(self.B), P(self.h.data_ptr()), P(stream))

    def part_bytes(self, i):
        R, K = self.R[i], self.K
        return R * K * self.n // self.m * 2 + R * K // 8 + self.B * R * 2

    def sparse_bytes(self):
        return sum(self.part_bytes(i) for i in range(len(self.R))) + self.B * self.K * 2

    def dense_bytes(self):
        return sum(R * self.K * 2 + self.B * R * 2 for R in self.R) + self.B * self.K * 2


def build_step(spec, tag, layers, torch, nm, I):
    launches = []
    for l in range(layers):
        for names, _ in spec[7]:
            launches.append(Launch(torch, nm, I, spec, tag, l, names))
    torch.cuda.synchronize()
    return launches


def run(fn, arg_lists):
    for a in arg_lists:
        st = fn(*a)
        if st != 0:
            raise RuntimeError(f"launch failed with status {st}")


def time_ms(torch, body, reps):
    """HIP events on torch's current stream around `reps` calls of body()."""
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(s)
    for _ in range(reps):
        body()
    e1.record(s)
    e1.synchronize()
    return e0.elapsed_time(e1) / reps


def capture(torch, fn, args_for_stream):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        args = args_for_stream(s.cuda_stream)
        run(fn, args)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            run(fn, args)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


def read_ceiling(torch, cur):
    """Plain 16-byte streaming read of 1 GB regions rotated over 4 GB."""
    from measure import probe
    lib = probe.lib()
    buf = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    nb = 1 << 30
    best = 0.0
    for blocks in (512, 1024, 2048):
        def body():
            for i in range(4):
                if lib.nmp_read(P(buf.data_ptr() + i * nb), nb, P(sink.data_ptr()), blocks, P(cur)) != 0:
                    raise RuntimeError("probe launch failed")
        body()
        ms = time_ms(torch, body, 3) / 4
        best = max(best, nb / (ms * 1e-3) / 1e9)
    del buf
    torch.cuda.empty_cache()
    return best


def copy_calibration(torch, cur, nbytes=256 << 20):
    """One plain 16-byte copy of known size: its FETCH_SIZE / WRITE_SIZE
    counter readings calibrate the counters' units in profiling runs."""
    from measure import probe
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    if probe.lib().nmp_copy(P(src.data_ptr()), P(dst.data_ptr()), nbytes, 1024, P(cur)) != 0:
        raise RuntimeError("probe copy failed")
    torch.cuda.synchronize()
    del src, dst
    return nbytes


def burst(torch, fn, args_for_stream, trials):
    """(min, median, max) per-launch microseconds of a back-to-back burst of
    fn(*args) launches, captured once into a HIP graph and replayed (a
    launch from Python can take longer than a small kernel runs)."""
    g = capture(torch, fn, args_for_stream)
    n = len(args_for_stream(0))
    return trials_us(torch, g.replay, trials, n)


def trials_us(torch, body, trials, launches):
    """(min, median, max) per-launch microseconds over `trials` timed bursts
    of body() (each burst: `launches` launches)."""
    import statistics
    ts = sorted(time_ms(torch, body, 1) / launches * 1e3 for _ in range(trials))
    return ts[0], statistics.median(ts), ts[-1]


def mlp_single(torch, lib, launches, cur, ws, reps=10, trials=20):
    """MLP projections (gate, up, down) as single launches through the
    workspace calls the step uses (nm_spmv_multi_ws / nm_gemv_dense_multi_ws
    on one matrix), back to back over every layer's weights (HIP-graph
    bursts); per-launch time is the median over `trials` bursts (min and max
    beside it)."""
    out = {}
    for name in ("gate", "up", "down"):
        group = [L for L in launches if name in L.names]
        if not group:
            continue
        L0 = group[0]
        i0 = L0.names.index(name)
        R, K, B = L0.R[i0], L0.K, L0.B

        wsa = (P(ws.data_ptr()), I64(ws.numel()))

        def sargs(st):
            out_ = []
            for L in group:
                i = L.names.index(name)
                out_.append((I32(1), (P * 1)(L.values[i].data_ptr()), (P * 1)(L.masks[i].data_ptr()), (I64 * 1)(R),
                             I64(K), I32(L.n), I32(L.m), I32(L.dtc), P(L.x.data_ptr()), I32(L.B),
                             (P * 1)(L.y[i].data_ptr())) + wsa + (P(st),))
            return out_

        def dargs(st):
            return [(I32(1), (P * 1)(L.W[L.names.index(name)].data_ptr()), (I64 * 1)(R), I64(K), I32(L.dtc),
                     P(L.x.data_ptr()), I32(L.B), (P * 1)(L.yd[L.names.index(name)].data_ptr())) + wsa + (P(st),)
                    for L in group]
        nbytes = L0.part_bytes(i0) + B * K * 2
        dbytes = R * K * 2 + B * (K + R) * 2
        ts = burst(torch, lib.nm_spmv_multi_ws, sargs, trials)
        td = burst(torch, lib.nm_gemv_dense_multi_ws, dargs, trials)
        us, usd = ts[1], td[1]
        # torch's own dense product (hipBLASLt / rocBLAS) on the same weights, as context
        pairs = [(L.W[L.names.index(name)], L.x, L.yd[L.names.index(name)]) for L in group]

        def torch_linear():
            for W, x, yd in pairs:
                torch.matmul(x, W.t(), out=yd)
        torch_linear()
        ust = time_ms(torch, torch_linear, reps) / len(pairs) * 1e3
        best_dense = min(usd, ust)
        out[name] = {"shape": [R, K], "us": round(us, 3), "us_min": round(ts[0], 3), "us_max": round(ts[2], 3),
                     "trials": trials, "gbs": round(nbytes / us / 1e3, 1),
                     "pct_of_peak": round(100 * nbytes / us / 1e3 / PEAK_GBS, 2),
                     "dense_us": round(usd, 3), "dense_us_min": round(td[0], 3), "dense_us_max": round(td[2], 3),
                     "dense_gbs": round(dbytes / usd / 1e3, 1),
                     "torch_matmul_us": round(ust, 3), "speedup": round(usd / us, 4),
                     "speedup_vs_best_dense": round(best_dense / us, 4), "bytes": nbytes}
    return out


def launch_floors(torch, sizes, trials=10):
    """For each byte count: the median per-launch time of a one-shot streaming
    read of that many bytes (measure/nmprobe.hip read_shot_kernel: 512-thread
    blocks, four 16-byte loads per thread, no loop), back to back over regions
    rotated past the 256 MB MALL -- the floor for one launch that streams
    those bytes; and the per-launch time of an empty kernel back to back."""
    from measure import probe
    plib = probe.lib()
    region = (max(sizes) + 4095) // 4096 * 4096
    n_inst = max(8, -(-(512 << 20) // region))
    buf = torch.empty(region * n_inst, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    floors = {}
    for nb in sorted(set(sizes)):
        n16 = nb // 16 * 16

        def args(st):
            return [(P(buf.data_ptr() + i * region), I64(n16), P(sink.data_ptr()), I32(512), P(st))
                    for i in range(n_inst)]
        floors[nb] = burst(torch, plib.nmp_read_shot, args, trials)[1]
    empty = burst(torch, plib.nmp_empty, lambda st: [(P(st),) for _ in range(64)], trials)[1]
    del buf, sink
    torch.cuda.empty_cache()
    return floors, empty


def hybrid_gate(torch, nm, lib, launches, cur, fracs=(0.05, 0.10), reps=5):
    """The hybrid sparse + dense row format on the gate projections: the rows
    of largest pruning loss kept dense (5% and 10% of them), the rest 2:4,
    timed back to back over the layers' weights against nm_gemv_dense."""
    out = {}
    Ls = [L for L in launches if "gate" in L.names]
    if not Ls:
        return out
    i = Ls[0].names.index("gate")
    R, K, B = Ls[0].R[i], Ls[0].K, Ls[0].B
    for frac in fracs:
        nd = int(round(frac * R))
        hybs = []
        for L in Ls:
            W = L.W[L.names.index("gate")]
            flags = nm.hybrid_select_rows(nm.hybrid_row_loss(W, L.n, L.m), nd)
            hybs.append((nm.hybrid_pack(W, flags, nd, L.n, L.m), L))
        ys = [torch.empty_like(L.y[i]) for _, L in hybs]     # own outputs: L.y is checked against the oracle later

        def args(st):
            return [(P(h.values.data_ptr()), P(h.masks.data_ptr()), P(h.rows_sparse.data_ptr()),
                     P(h.W_dense.data_ptr()), P(h.rows_dense.data_ptr()), I64(nd), I64(R), I64(K), I32(h.n), I32(h.m),
                     I32(L.dtc), P(L.x.data_ptr()), I32(B), P(y.data_ptr()), P(st)) for (h, L), y in zip(hybs, ys)]
        us = burst(torch, lib.nm_spmv_hybrid, args, reps)[1]
        h0, L0 = hybs[0]
        Rs = R - nd
        nbytes = Rs * K * h0.n // h0.m * 2 + Rs * K // 8 + nd * K * 2 + R * 4 + B * (K + R) * 2
        out[f"{int(frac * 100)}pct_dense_rows"] = {"shape": [R, K], "dense_rows": nd, "us": round(us, 3),
                                                   "gbs": round(nbytes / us / 1e3, 1), "bytes": nbytes}
        del hybs, ys
        torch.cuda.empty_cache()
    return out


def calib_throughput(torch, nm, I, K=4096, T=512, reps=5):
    """nm_calib_accumulate at the Llama-3.1-8B hidden size: H += X^T X over T
    decode rows, timed; matrix-core TFLOP/s and the H read-modify-write rate."""
    X = I.activation_normal(T, K, torch.bfloat16, I.seed_of("bench_calib"), device="cuda")
    H = torch.zeros((K, K), dtype=torch.float32, device="cuda")
    nm.calib_accumulate(X, None, H=H)
    ms = time_ms(torch, lambda: nm.calib_accumulate(X, None, H=H), reps)
    flops = 2.0 * K * K * T
    nbytes = 2 * 4 * K * K + T * K * 2
    return {"K": K, "T": T, "us": round(ms * 1e3, 2), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "pct_of_bf16_peak": round(100 * flops / (ms * 1e-3) / 2.5e15, 2),
            "hbm_gbs": round(nbytes / (ms * 1e-3) / 1e9, 1)}


def cpu_baseline(launches, budget_s, torch, label):
    """CPU oracle (plain C, fp64, one thread) on layer 0's projections, packed
    by the oracle itself from the same weights; repeated until about budget_s
    seconds of oracle time.  Beside it, the same calls split by rows over the
    host's worker threads (up to OMP_NUM_THREADS)."""
    import numpy as np

    import oracle
    work = []
    for L in launches:
        if L.layer != 0:
            continue
        xb = L.x.cpu().view(torch.int16).numpy().view(np.uint16)
        dts = "fp16" if L.dtc == 0 else "bf16"
        for i, R in enumerate(L.R):
            Wb = L.W[i].cpu().view(torch.int16).numpy().view(np.uint16)
            v, m = oracle.pack(Wb, None, L.n, L.m, dts)
            work.append((v, m, L, xb, L.part_bytes(i) + L.B * L.K * 2, dts))
    done, elapsed, reps = 0, 0.0, 0
    while elapsed < budget_s or reps == 0:
        for v, m, L, xb, nbytes, dts in work:
            t0 = time.perf_counter()
            oracle.spmv(v, m, L.K, L.n, L.m, dts, xb)
            elapsed += time.perf_counter() - t0
            done += nbytes
        reps += 1
    # The same oracle calls over row ranges on the host's worker threads (the
    # C oracle runs outside Python's lock), as an all-cores reference figure.
    nthreads = max(1, min(os.cpu_count() or 1, int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))))
    all_threads = None
    if nthreads > 1:
        from concurrent.futures import ThreadPoolExecutor

        def rows_job(job):
            v, m, L, xb, dts, r0, r1 = job
            oracle.spmv(v, m, L.K, L.n, L.m, dts, xb, rows=(r0, r1))
        done_mt, t_mt, reps_mt = 0, 0.0, 0
        with ThreadPoolExecutor(nthreads) as ex:
            while t_mt < min(budget_s, 5.0) or reps_mt == 0:
                for v, m, L, xb, nbytes, dts in work:
                    R = m.shape[0]
                    step = (R + nthreads - 1) // nthreads
                    jobs = [(v, m, L, xb, dts, r0, min(R, r0 + step)) for r0 in range(0, R, step)]
                    t0 = time.perf_counter()
                    list(ex.map(rows_job, jobs))
                    t_mt += time.perf_counter() - t0
                    done_mt += nbytes
                reps_mt += 1
        all_threads = {"value": round(done_mt / t_mt / 1e9, 4), "unit": "GB/s", "cores": nthreads,
                       "sample": f"the same projections x {reps_mt}, rows split over {nthreads} threads, "
                                 f"{t_mt:.1f} s, {t_mt / reps_mt * 1e3:.0f} ms per layer"}
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(done / elapsed / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{label}: layer 0's projections x {reps}, fp64 scalar C oracle, 1 thread, {elapsed:.1f} s, "
                      f"{elapsed / reps * 1e3:.0f} ms per layer; host {cpu}, {os.cpu_count()} logical CPUs",
            "all_threads": all_threads}


def sampled_parity(launches, torch):
    """First 64 rows of every layer-0 projection against the oracle."""
    import numpy as np

    import oracle
    worst = 0.0
    for L in launches:
        if L.layer != 0:
            continue
        xb = L.x.cpu().view(torch.int16).numpy().view(np.uint16)
        dts = "fp16" if L.dtc == 0 else "bf16"
        for i, nme in enumerate(L.names):
            Wb = L.W[i][:64].cpu().view(torch.int16).numpy().view(np.uint16)
            v, m = oracle.pack(Wb, None, L.n, L.m, dts)
            assert np.array_equal(v, L.values[i][:64].cpu().view(torch.int16).numpy().view(np.uint16)), "pack"
            assert np.array_equal(m, L.masks[i][:64].cpu().numpy()), "masks"
            yref, A = oracle.spmv(v, m, L.K, L.n, L.m, dts, xb)
            got = L.y[i][:, :64].cpu().view(torch.int16).numpy().view(np.uint16)
            ok, w, _ = oracle.check(got, yref, A, dts)
            assert ok, f"{nme}: outside tolerance ({w})"
            worst = max(worst, w)
    return worst


def measured_traffic():
    """HBM bytes per launch of the roofline kernel from the committed counter
    summary, or None when the kernel source changed since it was taken."""
    from measure.profsummary import kernel_sources_sha256
    path = os.path.join(ROOT, "profiles", "nm_spmv_llama31_8b_decode_traffic.json")
    try:
        with open(path) as fh:
            rec = json.load(fh)
        sha = kernel_sources_sha256()
    except OSError:
        return None
    return rec["traffic_bytes_per_launch"] if rec.get("source_sha256") == sha else None


# The other workloads, each as a decode step over its own weight instances
# (more than the 256 MB last-level cache holds), in the default run's line.
CONFIG_STEPS = [("qwen3_14b_4of8", 8), ("qwen3_14b_2of4", 8), ("qwen3_32b_4of8", 8), ("qwen3_32b_2of4", 8),
                ("llama33_70b", 8), ("qwen3_32b_b1", 8), ("qwen3_32b_b2", 8), ("qwen3_32b_b4", 8),
                ("qwen3_32b_b8", 8)]


def config_steps(torch, nm, I, specs, steps=10):
    """Each workload of CONFIG_STEPS as a HIP-graph step over `layers` layer
    instances of its projections: GB/s (algorithmic bytes per step / step
    time), share of the 8 TB/s peak, speedup over the same step on the dense
    weights, us per layer, and per launch kind the median us of back-to-back
    bursts.  Sparse and dense steps both run through the K-split workspace
    calls (nm_spmv_multi_ws, nm_gemv_dense_multi_ws), one workspace a step."""
    lib = nm.lib()
    out = {}
    for name, layers in CONFIG_STEPS:
        spec = specs[name]
        launches = build_step(spec, name, layers, torch, nm, I)
        sparse_bytes = sum(L.sparse_bytes() for L in launches)
        dense_bytes = sum(L.dense_bytes() for L in launches)
        ws = nm.workspace()
        gs = capture(torch, lib.nm_spmv_multi_ws, lambda st: [L.sparse_args_ws(st, ws) for L in launches])
        gd = capture(torch, lib.nm_gemv_dense_multi_ws, lambda st: [L.dense_args_ws(st, ws) for L in launches])
        for _ in range(3):
            gs.replay()
        ms = time_ms(torch, gs.replay, steps)
        for _ in range(3):
            gd.replay()
        msd = time_ms(torch, gd.replay, steps)
        kinds = {}
        for names, _ in spec[7]:
            kind = "+".join(names)
            group = [L for L in launches if L.kind == kind]
            kinds[kind] = round(burst(torch, lib.nm_spmv_multi_ws, lambda st: [L.sparse_args_ws(st, ws) for L in group],
                                      5)[1], 3)
        gbs = sparse_bytes / (ms * 1e-3) / 1e9
        out[name] = {"workload": spec[0], "layers": layers, "n_m": f"{spec[4]}:{spec[5]}", "batch": spec[6],
                     "gbs": round(gbs, 1), "pct_of_peak": round(100 * gbs / PEAK_GBS, 2),
                     "speedup_vs_dense": round(msd / ms, 4), "us_per_layer": round(ms * 1e3 / layers, 2),
                     "ms_per_step": round(ms, 4), "dense_ms_per_step": round(msd, 4),
                     "packed_bytes_per_step": sparse_bytes, "per_launch_us": kinds}
        del launches, gs, gd, ws
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def crossover(torch, nm, I, batches=(1, 2, 4, 8, 16, 32)):
    """Sparse 2:4 (nm_spmv), dense (nm_gemv_dense) and torch.matmul (hipBLASLt)
    on the Qwen3-32B MLP shapes over a range of batch sizes, each timed over
    enough weight instances to exceed the 256 MB MALL; beside them the same
    sparse and dense products through the workspace calls (nm_spmv_multi_ws,
    nm_gemv_dense_multi_ws: the K-split plan where it applies)."""
    lib = nm.lib()
    cur = torch.cuda.current_stream().cuda_stream
    dt = torch.bfloat16
    ws = nm.workspace()
    wsa = (P(ws.data_ptr()), I64(ws.numel()))
    out = {}
    for name in ("gate", "down"):
        R, K = I.QWEN3_32B_MLP[name]
        n_inst = 6
        Ws = [I.weight(R, K, dt, I.seed_of("xover", name, i), device="cuda") for i in range(n_inst)]
        packed = [nm.pack(W, None, 2, 4) for W in Ws]
        torch.cuda.synchronize()
        rows = []
        for B in batches:
            x = I.activation_normal(B, K, dt, I.seed_of("xover_x", name, B), device="cuda")
            y = torch.empty((B, R), dtype=dt, device="cuda")
            sargs = [(P(v.data_ptr()), P(mk.data_ptr()), I64(R), I64(K), I32(2), I32(4), I32(1), P(x.data_ptr()),
                      I32(B), P(y.data_ptr()), P(cur)) for v, mk in packed]
            dargs = [(P(W.data_ptr()), I64(R), I64(K), I32(1), P(x.data_ptr()), I32(B), P(y.data_ptr()), P(cur))
                     for W in Ws]
            run(lib.nm_spmv, sargs)
            us = time_ms(torch, lambda: run(lib.nm_spmv, sargs), 5) / n_inst * 1e3
            run(lib.nm_gemv_dense, dargs)
            usd = time_ms(torch, lambda: run(lib.nm_gemv_dense, dargs), 5) / n_inst * 1e3
            smargs = [(I32(1), (P * 1)(v.data_ptr()), (P * 1)(mk.data_ptr()), (I64 * 1)(R), I64(K), I32(2), I32(4),
                       I32(1), P(x.data_ptr()), I32(B), (P * 1)(y.data_ptr())) + wsa + (P(cur),) for v, mk in packed]
            dmargs = [(I32(1), (P * 1)(W.data_ptr()), (I64 * 1)(R), I64(K), I32(1), P(x.data_ptr()), I32(B),
                       (P * 1)(y.data_ptr())) + wsa + (P(cur),) for W in Ws]
            run(lib.nm_spmv_multi_ws, smargs)
            usw = time_ms(torch, lambda: run(lib.nm_spmv_multi_ws, smargs), 5) / n_inst * 1e3
            run(lib.nm_gemv_dense_multi_ws, dmargs)
            usdw = time_ms(torch, lambda: run(lib.nm_gemv_dense_multi_ws, dmargs), 5) / n_inst * 1e3

            def torch_mm():
                for W in Ws:
                    torch.matmul(x, W.t(), out=y)
            torch_mm()
            ust = time_ms(torch, torch_mm, 5) / n_inst * 1e3
            sb = R * K // 2 * 2 + R * K // 8 + B * (R + K) * 2
            db = R * K * 2 + B * (R + K) * 2
            rows.append({"B": B, "sparse_us": round(us, 2), "sparse_gbs": round(sb / us / 1e3, 1),
                         "dense_us": round(usd, 2), "dense_gbs": round(db / usd / 1e3, 1), "torch_us": round(ust, 2),
                         "speedup_vs_dense": round(usd / us, 3), "speedup_vs_torch": round(ust / us, 3),
                         "ws_sparse_us": round(usw, 2), "ws_dense_us": round(usdw, 2),
                         "ws_speedup_vs_dense": round(min(usd, usdw) / min(us, usw), 3)})
        out[name] = {"shape": [R, K], "rows": rows}
        del Ws, packed
        torch.cuda.empty_cache()
    return out


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {a.gpus} is not supported (multi-GPU sharding of this kernel "
              f"is design-only).", file=sys.stderr)
        sys.exit(2)
    import torch

    import sparse_matrix_vector_amd as nm
    from sparse_matrix_vector_amd import inputs as I
    specs = workloads(I)
    if a.workload not in specs:
        print(f"unknown workload {a.workload}; one of {sorted(specs)}", file=sys.stderr)
        sys.exit(2)
    if a.crossover:
        torch.cuda.set_device(0)
        print(json.dumps({"crossover": crossover(torch, nm, I), "workload": "Qwen3-32B MLP, 2:4 sparse, bf16"}),
              flush=True)
        return
    spec = specs[a.workload]
    desc, _, layers, dts, n, m, B = spec[:7]
    layers = a.layers or layers
    lib = nm.lib()
    torch.cuda.set_device(0)
    cur = torch.cuda.current_stream().cuda_stream

    launches = build_step(spec, a.workload, layers, torch, nm, I)
    n_launches = len(launches)
    sparse_bytes = sum(L.sparse_bytes() for L in launches)
    dense_bytes = sum(L.dense_bytes() for L in launches)

    ws = nm.workspace()        # the K-split workspace (used by batched products on few rows)
    if a.eager:
        sl = [L.sparse_args_ws(cur, ws) for L in launches]
        dl = [L.dense_args_ws(cur, ws) for L in launches]
        step_sparse = lambda: run(lib.nm_spmv_multi_ws, sl)       # noqa: E731
        step_dense = lambda: run(lib.nm_gemv_dense_multi_ws, dl)  # noqa: E731
    else:
        gs = capture(torch, lib.nm_spmv_multi_ws, lambda s: [L.sparse_args_ws(s, ws) for L in launches])
        gd = capture(torch, lib.nm_gemv_dense_multi_ws, lambda s: [L.dense_args_ws(s, ws) for L in launches])
        step_sparse, step_dense = gs.replay, gd.replay

    # ---- the timed region: K sparse steps ----
    for _ in range(a.warmup):
        step_sparse()
    torch.cuda.synchronize()
    ms_step = time_ms(torch, step_sparse, a.steps)
    # ---- dense baseline, same step structure ----
    for _ in range(max(1, a.warmup)):
        step_dense()
    ms_dense = time_ms(torch, step_dense, max(5, a.steps // 2))

    # ---- per launch kind: back-to-back bursts over the layers' weights ----
    per = {}
    for names, _ in spec[7]:
        kind = "+".join(names)
        group = [L for L in launches if L.kind == kind]
        ts = burst(torch, lib.nm_spmv_multi_ws, lambda st: [L.sparse_args_ws(st, ws) for L in group], 10)
        td = burst(torch, lib.nm_gemv_dense_multi_ws, lambda st: [L.dense_args_ws(st, ws) for L in group], 10)
        us, usd = ts[1], td[1]
        sb, db = group[0].sparse_bytes(), group[0].dense_bytes()
        per[kind] = {"rows": sum(group[0].R), "K": group[0].K, "us": round(us, 3), "us_min": round(ts[0], 3),
                     "us_max": round(ts[2], 3), "trials": 10, "gbs": round(sb / us / 1e3, 1),
                     "pct_of_peak": round(100 * sb / us / 1e3 / PEAK_GBS, 2), "dense_us": round(usd, 3),
                     "dense_us_min": round(td[0], 3), "dense_us_max": round(td[2], 3),
                     "dense_gbs": round(db / usd / 1e3, 1), "speedup": round(usd / us, 4), "bytes": sb}

    # ---- gated MLP input as one launch: h = SiLU(gate x) * (up x) ----
    group = [L for L in launches if L.names == ("gate", "up")]
    if group and not a.no_glu:
        ts = burst(torch, lib.nm_spmv_swiglu, lambda st: [L.glu_args(st) for L in group], 10)
        td = burst(torch, lib.nm_gemv_dense_swiglu, lambda st: [L.glu_args(st, dense=True) for L in group], 10)
        us, usd = ts[1], td[1]
        L0 = group[0]
        sb = L0.sparse_bytes() - L0.B * L0.R[1] * 2          # one output of R rows instead of two
        db = L0.dense_bytes() - L0.B * L0.R[1] * 2
        per["gate+up+silu"] = {"rows": L0.R[0], "K": L0.K, "us": round(us, 3), "us_min": round(ts[0], 3),
                               "us_max": round(ts[2], 3), "trials": 10, "gbs": round(sb / us / 1e3, 1),
                               "pct_of_peak": round(100 * sb / us / 1e3 / PEAK_GBS, 2), "dense_us": round(usd, 3),
                               "dense_gbs": round(db / usd / 1e3, 1), "speedup": round(usd / us, 4), "bytes": sb}

    if a.workload == "llama31_8b":
        # roofline kernel: the instantiation shared by the K = 4096 launches (3 per layer)
        rk = ("q+k+v", "o", "gate+up")
        kernel = "rowslice_kernel<2:4, fp16, B=1, 4 chunks/lane> (q+k+v, o, gate+up launches)"
        traffic = measured_traffic()
    else:
        rk = ("gate+up",)
        kernel = f"nm_spmv_multi gate+up launch ({n}:{m}, {dts}, B={B})"
        traffic = None
    rbytes = sum(per[k]["bytes"] for k in rk) / len(rk)
    rus = sum(per[k]["us"] for k in rk) / len(rk)
    achieved = rbytes / rus / 1e3

    mlp = mlp_single(torch, lib, launches, cur, ws, reps=10 if layers <= 64 else 3)
    # What no single launch of these sizes can beat: a one-shot read of the
    # same bytes, and an empty kernel (both back to back, as in the step).
    floors, empty_us = launch_floors(torch, [v["bytes"] for v in per.values()] + [v["bytes"] for v in mlp.values()])
    for v in list(per.values()) + list(mlp.values()):
        v["read_floor_us"] = round(floors[v["bytes"]], 3)
        v["above_floor_us"] = round(v["us"] - floors[v["bytes"]], 3)
    extras = {}
    if a.workload == "llama31_8b" and not a.no_glu:
        extras["hybrid_gate"] = hybrid_gate(torch, nm, lib, launches, cur)
        extras["calib_accumulate"] = calib_throughput(torch, nm, I)
    ceiling = read_ceiling(torch, cur)
    copy_bytes = copy_calibration(torch, cur)
    worst = sampled_parity(launches, torch)
    default_workload = a.workload == "llama31_8b"
    cpu = None if (a.no_cpu or not default_workload) else cpu_baseline(launches, a.cpu_seconds, torch, desc)
    if default_workload and not a.no_configs:
        # the step's own weights are no longer needed: free them before the other workloads
        del launches
        step_sparse = step_dense = gs = gd = None                 # noqa: F841 -- releases the step's graphs
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        extras["configs"] = config_steps(torch, nm, I, specs)

    gbs = sparse_bytes / (ms_step * 1e-3) / 1e9
    props = torch.cuda.get_device_properties(0)
    out = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if dts == "fp16" else "bf16",
        "data": "synthetic",
        "config": {"workload": desc, "name": a.workload, "layers": layers, "n_m": f"{n}:{m}", "batch": B,
                   "launches_per_step": n_launches, "mode": "eager" if a.eager else "hip_graph",
                   "packed_bytes_per_step": sparse_bytes, "dense_bytes_per_step": dense_bytes},
        "pct_of_peak": round(100 * gbs / PEAK_GBS, 2),
        "speedup_vs_dense": round(ms_dense / ms_step, 4),
        "dense_ms_per_step": round(ms_dense, 4),
        "dense_gbs": round(dense_bytes / (ms_dense * 1e-3) / 1e9, 1),
        "us_per_layer": round(ms_step * 1e3 / layers, 2),
        "per_launch": per,
        "mlp_shapes": mlp,
        "extras": extras,
        "launch_floor": {"empty_kernel_us": round(empty_us, 3),
                         "read_shot": "one-shot read of each launch's bytes (read_floor_us beside each launch)"},
        "read_ceiling_gbs": round(ceiling, 1),
        "pct_of_read_ceiling": round(100.0 * gbs / ceiling, 2) if ceiling else None,
        "copy_calibration_bytes": copy_bytes,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_GBS, 4), "traffic": traffic, "kernel": kernel,
                     "avg_launch_us": round(rus, 3), "algorithmic_bytes_per_launch": round(rbytes)},
        "cpu_baseline": cpu,
        "parity_sampled_worst_ratio": round(worst, 4),
        "env": {"gpu": props.name, "gcn_arch": getattr(props, "gcnArchName", None), "cus": props.multi_processor_count,
                "torch": torch.__version__, "hip": getattr(torch.version, "hip", None),
                "python": platform.python_version()},
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
