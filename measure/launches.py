"""Run chosen launches of a bench.py workload back to back, for profiler runs.

    python -m measure.launches [--workload llama31_8b] [--layers 8] [--kinds gate,down] [--reps 20] [--ws] [--dense]

Kinds are the step's launch kinds (``q+k+v``, ``o``, ``gate+up``, ``down`` for
the Llama-3.1-8B step) or one projection of a fused kind on its own (``gate``,
``up``).  Each kind runs as a HIP graph of one launch per layer (every layer on
its own weights, as in the step), replayed ``--reps`` times; the per-launch
median of those replays is printed.  Under ``rocprofv3 --pmc`` or
``--kernel-trace`` this gives counter and duration figures for just these
launches (the weights are packed on the GPU first, so the pack kernels show
up too, under their own names).
"""
import argparse
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def main():
    p = argparse.ArgumentParser()
    p.add_argument("--workload", default="llama31_8b")
    p.add_argument("--layers", type=int, default=8)
    p.add_argument("--kinds", default="gate,down")
    p.add_argument("--reps", type=int, default=20)
    p.add_argument("--ws", action="store_true", help="the step's kinds through the workspace calls (_multi_ws)")
    p.add_argument("--dense", action="store_true", help="the dense baseline of the step's kinds (nm_gemv_dense_multi)")
    a = p.parse_args()

    import torch

    import bench
    import sparse_matrix_vector_amd as nm
    from sparse_matrix_vector_amd import inputs as I
    from bench import I32, I64, P
    spec = list(bench.workloads(I)[a.workload])
    kinds = a.kinds.split(",")
    # build only the step's launch kinds that hold a requested kind or projection
    spec[7] = [k for k in spec[7] if "+".join(k[0]) in kinds or any(n in kinds for n in k[0])]
    torch.cuda.set_device(0)
    lib = nm.lib()
    launches = bench.build_step(spec, a.workload, a.layers, torch, nm, I)
    out = {}
    for kind in kinds:
        group = [L for L in launches if L.kind == kind]
        if group and a.dense and a.ws:
            ws = nm.workspace()
            fn, args = lib.nm_gemv_dense_multi_ws, (lambda st, g=group: [L.dense_args_ws(st, ws) for L in g])
        elif group and a.dense:
            fn, args = lib.nm_gemv_dense_multi, (lambda st, g=group: [L.dense_args(st) for L in g])
        elif group and a.ws:
            ws = nm.workspace()
            wsa = (P(ws.data_ptr()), I64(ws.numel()))
            fn, args = lib.nm_spmv_multi_ws, (lambda st, g=group: [L.sparse_args(st)[:-1] + wsa + (P(st),) for L in g])
        elif group:
            fn, args = lib.nm_spmv_multi, (lambda st, g=group: [L.sparse_args(st) for L in g])
        else:
            group = [L for L in launches if kind in L.names]
            if not group:
                raise SystemExit(f"no launch kind or projection named {kind}")

            def args(st, g=group, name=kind):
                res = []
                for L in g:
                    i = L.names.index(name)
                    res.append((P(L.values[i].data_ptr()), P(L.masks[i].data_ptr()), I64(L.R[i]), I64(L.K),
                                I32(L.n), I32(L.m), I32(L.dtc), P(L.x.data_ptr()), I32(L.B), P(L.y[i].data_ptr()),
                                P(st)))
                return res
            fn = lib.nm_spmv
        g = bench.capture(torch, fn, args)
        g.replay()
        torch.cuda.synchronize()
        ts = [bench.time_ms(torch, g.replay, 1) / len(group) * 1e3 for _ in range(a.reps)]
        out[kind] = {"launches_per_replay": len(group), "replays": a.reps, "us_median": round(statistics.median(ts), 3),
                     "us_min": round(min(ts), 3)}
        print(json.dumps({kind: out[kind]}), flush=True)


if __name__ == "__main__":
    main()
