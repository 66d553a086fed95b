"""Throughput of the fused W4A4 + block-sparse INT4 residual layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one pass of the online hot path - fp16 activations to fp16 y
through mq_fused_layer (activation quantisation and the fused GEMM; one
kernel for M <= 4, where the GEMM quantises the token tile itself, else the
act-quant kernel then the fused GEMM) - for every (shape, M) of the
workload, with inputs resident in HBM.  The offline part (Delta-score selection and packing) runs once on
the GPU before timing.  Every (shape, M) in a step reads its own copy of the
packed weights, and whole copies of the step's data rotate between steps so
the footprint is >= 512 MB: the 256 MB Infinity Cache cannot serve weights
from a previous launch.

Printed JSON (one line on stdout):
  value      algorithmic bytes of the step (fp16 X, packed layer, fp16 Y of
             every (shape, M)) / step time (GB/s)
  tops       algorithmic integer ops of the step / step time
  roofline   the fused GEMM (dominant kernel): algorithmic bytes (decode) or
             ops (prefill) per launch / average launch time, from HIP events
             around K replays of a graph holding only the step's GEMM
             launches (the one-kernel layer where M <= 4: its bytes count
             the fp16 activations it reads instead of codes)
Launches are replayed from HIP graphs (one per rotating set) so the timed
region measures the GPU, not Python launch overhead (--no-graph: eager).
  cpu_baseline  the CPU oracle (quantise + fused GEMM) on a bounded sample
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

METRIC = "fused W4A4+10% residual GEMM TOPS & HBM GB/s vs roofline, M=1..4096"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
INT8_MFMA_PEAK_TOPS = 5000.0   # MI355X dense int8 MFMA
ROTATE_BYTES = 512 << 20


def workload(name: str):
    from dense_sparse_w4a4_amd import synthetic as syn
    if name == "llama3-8b-decode":
        return [(syn.llama3_8b(K, N), syn.LLAMA3_8B_DECODE_M) for (K, N) in syn.LLAMA3_8B_SHAPES], "hbm"
    if name == "llama3-8b-prefill":
        return [(syn.llama3_8b(K, N), [syn.LLAMA3_8B_PREFILL_M]) for (K, N) in syn.LLAMA3_8B_SHAPES], "mfma"
    if name.startswith("qwen3-32b"):
        ms = {"qwen3-32b-decode": [1, 16], "qwen3-32b-256": [256], "qwen3-32b-4096": [4096]}.get(name)
        if ms is None:
            raise SystemExit(f"unknown workload {name}")
        return [(syn.qwen3_32b(K, N), ms) for (K, N) in syn.QWEN3_32B_SHAPES], ("hbm" if max(ms) <= 16 else "mfma")
    if name.startswith("llama3-70b"):
        # llama3-70b-b{32,64,128}-r{0,5,10,20}
        parts = name.split("-")
        b = int(parts[2][1:])
        rho = int(parts[3][1:]) / 100.0
        return [(syn.llama3_70b(b, rho), [syn.LLAMA3_70B_M])], "mfma"
    if name == "tiny":
        return [(syn.TINY, [syn.TINY_M])], "hbm"
    raise SystemExit(f"unknown workload {name}")


def weight_bytes(N, K, b, ns):
    """Packed layer: base codes and scales, residual codes and scales, CSR."""
    G = K // 128
    return N * K // 2 + 2 * N * G + ns * (b * b // 2 + 2 * b) + 4 * ns + 4 * (N // b + 1)


def gemm_bytes(M, N, K, b, ns):
    """Compulsory bytes of one fused GEMM call from activation codes (each
    byte counted once)."""
    return weight_bytes(N, K, b, ns) + M * K // 2 + 4 * M * (K // 128) + 2 * M * N


def layer_bytes(M, N, K, b, ns):
    """Compulsory bytes of the online layer from fp16 activations to fp16 y."""
    return weight_bytes(N, K, b, ns) + 2 * M * K + 2 * M * N


def gemm_ops(M, N, K, b, ns):
    return 2 * M * N * K + 2 * M * ns * b * b


def traffic_from_profile(wname: str):
    """HBM bytes per GEMM launch measured with rocprofv3 counters, if the
    stored measurement was taken on the current kernel sources."""
    p = os.path.join(ROOT, "profiles", f"traffic_{wname}.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    from dense_sparse_w4a4_amd.profiling import kernel_sources_sha
    if d.get("sources_sha") != kernel_sources_sha():
        return None
    return d.get("bytes_per_launch")


def cpu_baseline(layers, budget_s: float):
    """Time the oracle's online path (quantise + fused GEMM) on the workload.

    The oracle's packed layers are built first (untimed).  Then whole passes
    over every (shape, M) of the step are timed until about budget_s seconds
    of CPU work have accumulated (at least one pass), so the sample is the
    step itself, repeated; a pass that would exceed four budgets of wall time
    stops early and the sample names what ran."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    from dense_sparse_w4a4_amd import synthetic as syn
    prepared = []
    for spec, ms in layers:
        w = syn.make_weight(spec)
        xc = syn.make_calib(spec)
        sel, _, _ = oracle.select_blocks(w, xc, spec.block, spec.n_select)
        packed = oracle.pack_weights(w, spec.block, sel)
        for M in ms:
            prepared.append((spec, M, len(sel), packed, syn.make_acts(spec, M)))
    tbytes, tops, tsec, passes, partial = 0, 0, 0.0, 0, []
    while True:
        for (spec, M, ns, packed, x) in prepared:
            t0 = time.perf_counter()
            qa, sa = oracle.quantize_act(x)
            oracle.fused_gemm(qa, sa, packed)
            tsec += time.perf_counter() - t0
            tbytes += layer_bytes(M, spec.N, spec.K, spec.block, ns)
            tops += gemm_ops(M, spec.N, spec.K, spec.block, ns)
            if passes == 0:
                partial.append(f"{spec.K}x{spec.N}@M={M}")
            if tsec > 4 * budget_s:
                break
        passes += 1
        if tsec >= budget_s or tsec > 4 * budget_s:
            break
    what = ", ".join(partial)
    return dict(value=tbytes / tsec / 1e9, unit="GB/s", tops=tops / tsec / 1e12, cores=int(threads),
                kind="oracle", seconds=round(tsec, 3),
                sample=f"{passes} pass(es) of oracle quantize_act + fused_gemm (numpy; BLAS "
                       f"threads = cores) over {what}")


def sweep_llama3_70b(args):
    """Llama-3-70B FFN (K=8192, N=28672), M=256: fused-GEMM time for every
    (block edge, budget) pair relative to the same block edge at budget 0,
    next to the output distortion recovered, 1 - D(S_rho)/D(empty), on the
    calibration tokens and on held-out tokens from the same generator.
    Prints one JSON line."""
    import torch
    from dense_sparse_w4a4_amd import evaluate, ops
    from dense_sparse_w4a4_amd import synthetic as syn
    dev = torch.device("cuda:0")
    log = lambda *a: print(*a, file=sys.stderr, flush=True)  # noqa: E731
    M = syn.LLAMA3_70B_M
    rows = []
    base = syn.llama3_70b(64, 0.0)
    w = torch.from_numpy(syn.make_weight(base)).to(dev)
    xc = torch.from_numpy(syn.make_calib(base)).to(dev)
    xh = torch.from_numpy(syn.make_acts(base, 512)).to(dev)   # held-out tokens (same layer, other draw)
    x = torch.from_numpy(syn.make_acts(base, M)).to(dev)
    qa, sa = ops.quantize_act(x)
    y = torch.empty((M, base.N), dtype=torch.float16, device=dev)
    cap = torch.cuda.Stream()
    for b in syn.LLAMA3_70B_BLOCKS:
        t_zero = None
        d0 = {}
        for rho in syn.LLAMA3_70B_RHOS:
            spec = syn.llama3_70b(b, rho)
            sel, _, _ = ops.select_blocks(w, xc, b, spec.n_select)
            L = ops.pack_weights(w, b, sel)
            R = max(2, -(-ROTATE_BYTES // L.nbytes()))
            cs = [L.clone() for _ in range(R)]
            for c in cs:
                ops.fused_gemm(qa, sa, c, out=y)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                for c in cs:
                    ops.fused_gemm(qa, sa, c, out=y)
            torch.cuda.synchronize()
            g.replay()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(args.steps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) * 1e-3 / (args.steps * R)
            if rho == 0.0:
                t_zero = t
                d0 = {k: evaluate.distortion(xe, w, L, with_residual=False) for k, xe in (("calib", xc), ("holdout", xh))}
            d = {k: evaluate.distortion(xe, w, L) for k, xe in (("calib", xc), ("holdout", xh))}
            ops_ = gemm_ops(M, spec.N, spec.K, b, spec.n_select)
            row = dict(block=b, rho=rho, n_select=spec.n_select, us=round(t * 1e6, 2),
                       time_vs_rho0=round(t / t_zero, 4), tops=round(ops_ / t / 1e12, 1),
                       recovered_calib=round(1 - d["calib"] / d0["calib"], 4),
                       recovered_holdout=round(1 - d["holdout"] / d0["holdout"], 4))
            rows.append(row)
            log(f"[sweep] b={b:3d} rho={rho:4.2f} n_sel={spec.n_select:6d}: {t * 1e6:8.2f} us "
                f"(x{t / t_zero:5.3f} vs rho=0)  recovered calib {row['recovered_calib']:.3f} "
                f"held-out {row['recovered_holdout']:.3f}")
            del cs, L, g
            torch.cuda.empty_cache()
    print(json.dumps({"metric": METRIC, "workload": "llama3-70b-ffn-8192x28672-M256-sweep",
                      "unit": "us", "data": "synthetic", "n_gpus": 1, "steps": args.steps,
                      "sweep": rows}), flush=True)


def smooth_study(args):
    """Outlier migration before the decomposition, with and without, on the
    Llama-3-8B decode shapes at M=16 (b=64, 10% residual): the layer's output
    error against the exact X W^T, ||Y - X W^T||_F / ||X W^T||_F, and the
    weight distortion recovered by the residual on held-out tokens.  Every
    step runs through the library (migration, selection, packing, act-quant,
    fused GEMM); the exact product and the error norms are torch float64.
    Prints one JSON line."""
    import torch
    from dense_sparse_w4a4_amd import evaluate, ops
    from dense_sparse_w4a4_amd import synthetic as syn
    dev = torch.device("cuda:0")
    log = lambda *a: print(*a, file=sys.stderr, flush=True)  # noqa: E731
    rows = []
    for (K, N) in syn.LLAMA3_8B_SHAPES:
        spec = syn.llama3_8b(K, N)
        w = torch.from_numpy(syn.make_weight(spec)).to(dev)
        xc = torch.from_numpy(syn.make_calib(spec)).to(dev)
        x = torch.from_numpy(syn.make_acts(spec, 16)).to(dev)
        xe = torch.from_numpy(syn.make_acts(spec, 512)).to(dev)
        exact = x.double() @ w.double().T
        res = {}
        for tag in ("plain", "migrated"):
            if tag == "migrated":
                s, wm, _, _ = ops.smooth_weights(xc, w)
                xcm, xm, xem = ops.smooth_acts(xc, s), ops.smooth_acts(x, s), ops.smooth_acts(xe, s)
            else:
                wm, xcm, xm, xem = w, xc, x, xe
            sel, _, _ = ops.select_blocks(wm, xcm, spec.block, spec.n_select)
            L = ops.pack_weights(wm, spec.block, sel)
            y = ops.layer_forward(xm, L).double()
            err = float(torch.linalg.norm(y - exact) / torch.linalg.norm(exact))
            d0 = evaluate.distortion(xem, wm, L, with_residual=False)
            d1 = evaluate.distortion(xem, wm, L)
            res[tag] = dict(rel_output_error=round(err, 6), recovered_holdout=round(1 - d1 / d0, 4),
                            weight_distortion_base=d0, weight_distortion=d1)
        rows.append(dict(K=K, N=N, M=16, **{f"{t}_{k}": v for t in res for k, v in res[t].items()}))
        log(f"[smooth] K={K:5d} N={N:5d}: output error plain {res['plain']['rel_output_error']:.5f} "
            f"migrated {res['migrated']['rel_output_error']:.5f}; residual recovers "
            f"{res['plain']['recovered_holdout']:.3f} / {res['migrated']['recovered_holdout']:.3f} of the "
            f"weight distortion (held-out tokens)")
    print(json.dumps({"metric": "layer output error with and without outlier migration",
                      "workload": "llama3-8b-decode-M16", "data": "synthetic", "n_gpus": 1,
                      "rows": rows}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama3-8b-decode")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying HIP graphs")
    ap.add_argument("--per-shape", action="store_true", help="also time each (shape, M) on its own")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (for HBM counter calibration)")
    ap.add_argument("--smooth", action="store_true",
                    help="output error with and without outlier migration (Llama-3-8B shapes, M=16)")
    ap.add_argument("--sweep", action="store_true",
                    help="Llama-3-70B FFN block-size x budget grid: time vs rho=0 and distortion recovered")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer shards by output channels with no exchange; see the sharding "
              "design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    from dense_sparse_w4a4_amd import ops
    from dense_sparse_w4a4_amd import synthetic as syn

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.sweep:
        ops.lib()
        sweep_llama3_70b(args)
        return
    if args.smooth:
        ops.lib()
        smooth_study(args)
        return
    dev = torch.device("cuda:0")
    ops.lib()
    layers, bound = workload(args.workload)
    log = lambda *a: print(*a, file=sys.stderr, flush=True)  # noqa: E731

    # ---- offline: select + pack once per shape (GPU), then replicate ----
    t0 = time.perf_counter()
    base = []
    for spec, ms in layers:
        wt = torch.from_numpy(syn.make_weight(spec)).to(dev)
        xct = torch.from_numpy(syn.make_calib(spec)).to(dev)
        sel, _, _ = ops.select_blocks(wt, xct, spec.block, spec.n_select)
        layer = ops.pack_weights(wt, spec.block, sel)
        xs = {M: torch.from_numpy(syn.make_acts(spec, M)).to(dev) for M in ms}
        base.append((spec, ms, layer, xs))
        del wt, xct
    torch.cuda.synchronize()
    pairs = [(spec, M) for spec, ms, _, _ in base for M in ms]
    step_footprint = sum(layer.nbytes() + 2 * xs[M].numel() for spec, ms, layer, xs in base for M in ms)
    R = max(1, -(-ROTATE_BYTES // step_footprint))
    sets = []
    for r in range(R):
        s = []
        for spec, ms, layer, xs in base:
            for M in ms:
                L = layer.clone()
                x = xs[M].clone()
                qa, sa = ops.quantize_act(x)  # codes for the GEMM-only timing
                y = torch.empty((M, spec.N), dtype=torch.float16, device=dev)
                wsb = ops.fused_layer_workspace(M, spec.N, spec.K)
                ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
                s.append((spec, M, L, x, qa, sa, y, ws))
        sets.append(s)
    # pairs the layer runs as one kernel (the GEMM quantises the token tile)
    one_kernel = [ops.fused_layer_workspace(M, s.N, s.K) == 0 for s, M in pairs]
    torch.cuda.synchronize()
    log(f"[bench] workload {args.workload}: {len(pairs)} (shape, M) pairs per step, "
        f"{R} rotating copies x {step_footprint / 2**20:.1f} MiB, setup {time.perf_counter() - t0:.1f}s")

    per_step_bytes = sum(layer_bytes(M, s.N, s.K, s.block, s.n_select) for s, M in pairs)
    per_step_gemm_bytes = sum((layer_bytes if one else gemm_bytes)(M, s.N, s.K, s.block, s.n_select)
                              for (s, M), one in zip(pairs, one_kernel))
    per_step_ops = sum(gemm_ops(M, s.N, s.K, s.block, s.n_select) for s, M in pairs)

    def run_set(i, whole_layer=True):
        # whole_layer: the step (mq_fused_layer); otherwise only the GEMM
        # launches (the one-kernel layer where it applies, else the fused
        # GEMM from precomputed codes)
        for p_idx, (spec, M, L, x, qa, sa, y, ws) in enumerate(sets[i % R]):
            if whole_layer or one_kernel[p_idx]:
                ops.fused_layer(x, L, out=y, workspace=ws)
            else:
                ops.fused_gemm(qa, sa, L, out=y)

    for i in range(max(args.warmup, R)):
        run_set(i)
    torch.cuda.synchronize()

    # One HIP graph per rotating set: the whole step (the layer for every
    # (shape, M)), and the GEMM launches alone for per-launch timing.
    use_graph = not args.no_graph
    if use_graph:
        g_step, g_gemm = [], []
        cap = torch.cuda.Stream()
        for r in range(R):
            for lst, wq in ((g_step, True), (g_gemm, False)):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cap):
                    run_set(r, wq)
                lst.append(g)
        torch.cuda.synchronize()
        for r in range(R):
            g_step[r].replay()
        torch.cuda.synchronize()

    def timed(n, body):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall = time.perf_counter()
        start.record()
        for i in range(n):
            body(i)
        end.record()
        torch.cuda.synchronize()
        return max(start.elapsed_time(end), 0.0), (time.perf_counter() - wall) * 1e3

    # ---- timed region: exactly K steps ----
    if use_graph:
        ev_ms, wall_ms = timed(args.steps, lambda i: g_step[i % R].replay())
    else:
        ev_ms, wall_ms = timed(args.steps, lambda i: run_set(i))
    ms_per_step = ev_ms / args.steps
    log(f"[bench] {args.steps} steps: {ms_per_step * 1e3:.2f} us/step on HIP events "
        f"({wall_ms / args.steps * 1e3:.2f} us/step wall), graphs={'on' if use_graph else 'off'}")

    # ---- fused GEMM alone: average launch time over the same number of steps ----
    if use_graph:
        gem_ms, _ = timed(args.steps, lambda i: g_gemm[i % R].replay())
    else:
        gem_ms, _ = timed(args.steps, lambda i: run_set(i, False))
    gemm_time_s = gem_ms * 1e-3 / args.steps  # per step (all pairs)

    # per-(shape, M) launch times, each pair replayed in its own graph, and
    # the same kernel on a dense-only copy (empty CSR) for the residual cost
    per_shape = []
    if args.per_shape and use_graph:
        def pair_copies(p_idx):
            # enough copies of the pair's packed layer that one pass over
            # them is >= 512 MB, so no launch finds its weights in the
            # 256 MB Infinity Cache
            L = sets[0][p_idx][2]
            n = max(2, -(-ROTATE_BYTES // L.nbytes()))
            return [L.clone() for _ in range(n)]

        def pair_time(p_idx, mode, copies):
            # mode: "fused" (fused GEMM from codes), "dense" (same kernel,
            # empty CSR), "unfused" (dense-only launch + the standalone
            # residual kernel that reloads the activations and merges into
            # y), "layer" (mq_fused_layer from fp16 X), "two" (act-quant
            # kernel then the fused GEMM).  One graph launches every copy
            # once; the time is per launch over several replays.
            (sp_, M_, L0, x, qa, sa, y, ws) = sets[0][p_idx]
            q2, s2 = torch.empty_like(qa), torch.empty_like(sa)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                for L in copies:
                    D = ops.PackedLayer(L.N, L.K, L.block, L.qw, L.sw, torch.zeros_like(L.row_ptr),
                                        L.col_idx[:0], L.qr[:0], L.sr[:0])
                    if mode == "layer":
                        ops.fused_layer(x, L, out=y, workspace=ws)
                    elif mode == "two":
                        ops.quantize_act(x, q2, s2)
                        ops.fused_gemm(q2, s2, L, out=y)
                    else:
                        ops.fused_gemm(qa, sa, L if mode == "fused" else D, out=y)
                    if mode == "unfused":
                        ops.residual_merge(qa, sa, L, y)
            g.replay()
            reps = max(3, -(-200 // len(copies)))
            t_ms, _ = timed(reps, lambda i: g.replay())
            del g
            return t_ms * 1e-3 / (reps * len(copies))
        for p_idx, (spec, M) in enumerate(pairs):
            copies = pair_copies(p_idx)
            t = pair_time(p_idx, "fused", copies)
            t0 = pair_time(p_idx, "dense", copies)
            tu = pair_time(p_idx, "unfused", copies)
            tl = pair_time(p_idx, "layer", copies)
            t2 = pair_time(p_idx, "two", copies)
            del copies
            torch.cuda.empty_cache()
            gb = gemm_bytes(M, spec.N, spec.K, spec.block, spec.n_select)
            lb = layer_bytes(M, spec.N, spec.K, spec.block, spec.n_select)
            go = gemm_ops(M, spec.N, spec.K, spec.block, spec.n_select)
            per_shape.append(dict(K=spec.K, N=spec.N, M=M, us=round(t * 1e6, 3), dense_only_us=round(t0 * 1e6, 3),
                                  residual_cost=round(t / t0 - 1, 4), unfused_us=round(tu * 1e6, 3),
                                  unfused_over_fused=round(tu / t, 4), gbs=round(gb / t / 1e9, 1),
                                  tops=round(go / t / 1e12, 2), layer_us=round(tl * 1e6, 3),
                                  layer_one_kernel=bool(one_kernel[p_idx]),
                                  layer_gbs=round(lb / tl / 1e9, 1), two_kernel_us=round(t2 * 1e6, 3)))
            log(f"[bench]   K={spec.K:6d} N={spec.N:6d} M={M:5d}: gemm {t * 1e6:8.2f} us  "
                f"{gb / t / 1e9:8.1f} GB/s ({gb / t / 1e9 / HBM_PEAK_GBS:5.1%} HBM)  "
                f"{go / t / 1e12:8.2f} TOPS ({go / t / 1e12 / INT8_MFMA_PEAK_TOPS:5.1%} int8 MFMA)  "
                f"dense-only {t0 * 1e6:8.2f} us (residual +{t / t0 - 1:5.1%})  "
                f"unfused {tu * 1e6:8.2f} us (x{tu / t:5.3f})  "
                f"layer {tl * 1e6:8.2f} us ({'one kernel' if one_kernel[p_idx] else 'two kernels'}; "
                f"act-quant + gemm {t2 * 1e6:8.2f} us)")

    launches = len(pairs)
    if bound == "hbm":
        achieved = per_step_gemm_bytes / gemm_time_s / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 2), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4))
    else:
        achieved = per_step_ops / gemm_time_s / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 2), peak=INT8_MFMA_PEAK_TOPS,
                    unit="TOP/s", frac=round(achieved / INT8_MFMA_PEAK_TOPS, 4))
    roof["traffic"] = traffic_from_profile(args.workload)
    # the library runs M <= 32 on the streaming kernel, larger M on the tile kernel
    roof["kernel"] = "gemm_stream_kernel" if max(M for _, M in pairs) <= 32 else "gemm_tile_kernel"
    roof["launches_quantising_in_kernel"] = int(sum(one_kernel))
    roof["avg_launch_us"] = round(gemm_time_s / launches * 1e6, 3)
    roof["alg_bytes_per_launch"] = per_step_gemm_bytes / launches
    roof["alg_ops_per_launch"] = per_step_ops / launches
    if bound == "hbm" and not args.copy_calibration:
        # a plain device copy measured here (outside the timed region): the
        # rate a streaming kernel reaches on this part, beside the datasheet
        # peak (not in counter runs, whose 256 MiB calibration copy must stay
        # the largest copy of the run)
        a = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        for _ in range(10):
            b.copy_(a)
        c1.record()
        torch.cuda.synchronize()
        copy_gbs = 2 * a.numel() / (c0.elapsed_time(c1) * 1e-3 / 10) / 1e9
        roof["measured_copy_gbs"] = round(copy_gbs, 1)
        roof["frac_of_copy"] = round(achieved / copy_gbs, 4)
        del a, b

    if args.copy_calibration:
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    out = {
        "metric": METRIC,
        "value": round(per_step_bytes / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "tops": round(per_step_ops / (ms_per_step * 1e-3) / 1e12, 3),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "shapes_KxN": [[s.K, s.N] for s, _, _, _ in base],
            "M": sorted({M for _, M in pairs}),
            "group": 128, "block": base[0][0].block, "rho": base[0][0].rho,
            "codes": "w4a4 int4 symmetric, int8 MFMA, int32 accumulators, fp32 epilogue, fp16 out",
            "bytes_per_step": per_step_bytes, "ops_per_step": per_step_ops,
            "rotating_copies": R,
            "launch": "hip-graph" if use_graph else "eager",
        },
        "roofline": roof,
    }
    if per_shape:
        out["per_shape"] = per_shape
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        out["cpu_baseline"] = cpu_baseline(layers, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
