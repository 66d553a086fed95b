"""Throughput of the fused W4A4 + block-sparse INT4 residual layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Default workload: the Qwen3-32B MLP shapes (K x N = 5120 x 25600 and
25600 x 5120, 10% residual in 64 x 64 blocks) at M = 1, 16, 256 and 4096 -
decode-shaped launches bounded by HBM and prefill-shaped launches bounded by
the matrix cores in one step.  One step is one pass of the online hot
path - fp16 activations to fp16 y through mq_fused_layer (activation
quantisation and the fused GEMM; one kernel where the GEMM quantises the
token tile itself, else the act-quant kernel then the fused GEMM) - for every
(shape, M) of the workload, with inputs resident in HBM.  The offline part
(Delta-score selection and packing) runs once on the GPU before timing.
Every (shape, M) in a step reads its own copy of the packed weights, and
whole copies of the step's data rotate between steps so the footprint is
>= 512 MB: the 256 MB Infinity Cache cannot serve weights from a previous
launch.

Printed JSON (one line on stdout):
  value      algorithmic integer ops of the step / step time (TOP/s)
  gbs        algorithmic bytes of the step (fp16 X, packed layer, fp16 Y of
             every (shape, M)) / step time
  roofline   per GEMM kernel (streaming kernel for M <= 32; tile kernel,
             int8 route, for 32 < M < 1024; tile kernel, fp6 route, from
             M = 1024), the dominant one (most time per step) first:
             algorithmic bytes (streaming: HBM) or ops (tile: against the
             dense peak of the matrix-core type it runs on, int8 or fp6) per
             launch / average launch time, from HIP events around K replays
             of a graph holding only that kernel's launches of the step (the
             one-kernel layer where it applies: its bytes count the fp16
             activations it reads instead of codes; the fp6 kernel on its
             operand images prepared outside the timing, while the step's
             layer converts them on every call); next to the measured int8
             matrix-core rate, shader clock and device-copy rate
  per_pair   per (shape, M): fused GEMM launch time p10 / median / p90 over
             replays, TOPS, GB/s, roofline fractions, the same kernel with an
             empty CSR (residual cost), act-quant alone, the whole layer
  cpu_baseline  the CPU oracle (quantise + fused GEMM) on a bounded sample
Launches are replayed from HIP graphs (one per rotating set) so the timed
region measures the GPU, not Python launch overhead (--no-graph: eager).
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
FP6_MFMA_PEAK_TOPS = 10100.0   # MI355X dense fp6 / fp4 MFMA
FP6_MIN_M = 1024               # the library's fp6 route: M >= 1024, block 64 or 128
ROTATE_BYTES = 512 << 20


DEFAULT_WORKLOAD = "qwen3-32b-sweep"
PAIR_REPLAYS = 15   # timed replays per (shape, M) and mode


def workload(name: str):
    """[(LayerSpec, [M, ...]), ...] of a named workload."""
    from dense_sparse_w4a4_amd import synthetic as syn
    if name == "qwen3-32b-sweep":
        return [(syn.qwen3_32b(K, N), syn.QWEN3_32B_M) for (K, N) in syn.QWEN3_32B_SHAPES]
    if name == "llama3-8b-decode":
        return [(syn.llama3_8b(K, N), syn.LLAMA3_8B_DECODE_M) for (K, N) in syn.LLAMA3_8B_SHAPES]
    if name == "llama3-8b-prefill":
        return [(syn.llama3_8b(K, N), [syn.LLAMA3_8B_PREFILL_M]) for (K, N) in syn.LLAMA3_8B_SHAPES]
    if name.startswith("qwen3-32b"):
        ms = {"qwen3-32b-decode": [1, 16], "qwen3-32b-256": [256], "qwen3-32b-4096": [4096]}.get(name)
        if ms is None:
            raise SystemExit(f"unknown workload {name}")
        return [(syn.qwen3_32b(K, N), ms) for (K, N) in syn.QWEN3_32B_SHAPES]
    if name.startswith("llama3-70b"):
        # llama3-70b-b{32,64,128}-r{0,5,10,20}
        parts = name.split("-")
        b = int(parts[2][1:])
        rho = int(parts[3][1:]) / 100.0
        return [(syn.llama3_70b(b, rho), [syn.LLAMA3_70B_M])]
    if name == "tiny":
        return [(syn.TINY, [syn.TINY_M])]
    raise SystemExit(f"unknown workload {name}")


def kernel_of(M: int, block: int = 64) -> str:
    """The GEMM kernel the library runs for M tokens (the streaming kernel up
    to 32 tokens, the LDS-tiled kernel above: its fp6 route from 1024 tokens
    with 64- or 128-wide blocks, its int8 route otherwise)."""
    if M <= 32:
        return "gemm_stream_kernel"
    return "gemm_tile6_kernel" if M >= FP6_MIN_M and block in (64, 128) else "gemm_tile_kernel"


def mfma_peak(kernel: str) -> float:
    """Dense MFMA peak of the matrix-core type a tile kernel runs on."""
    return FP6_MFMA_PEAK_TOPS if kernel == "gemm_tile6_kernel" else INT8_MFMA_PEAK_TOPS


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


def traffic_from_profile(wname: str, kernel: str):
    """HBM bytes per launch of `kernel` measured with rocprofv3 counters, if
    the stored measurement was taken on the current kernel sources."""
    p = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{wname}.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    from dense_sparse_w4a4_amd.profiling import kernel_sources_sha
    if d.get("sources_sha") != kernel_sources_sha(kernel) or d.get("kernel") != kernel:
        return None
    return d.get("bytes_per_launch")


def cpu_baseline(layers, budget_s: float, host_layers=None):
    """Time the oracle's online path (quantise + fused GEMM) on the workload.

    The oracle's packed layers are built first (untimed).  Then the (shape, M)
    pairs of the step are timed in order of increasing M, passes over all of
    them repeated while under budget_s seconds; a pair is skipped once the
    time so far plus an estimate of its own (ops x the slowest rate seen
    yet) would pass twice the budget, so the sample stays bounded and names
    what ran.  Rates are algorithmic ops (and bytes) over the oracle's time."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    from dense_sparse_w4a4_amd import synthetic as syn
    prepared = []
    for i, (spec, ms) in enumerate(layers):
        w, xc = host_layers[i] if host_layers else (syn.make_weight(spec), syn.make_calib(spec))
        sel, _, _ = oracle.select_blocks(w, xc, spec.block, spec.n_select)
        packed = oracle.pack_weights(w, spec.block, sel)
        for M in ms:
            prepared.append((spec, M, len(sel), packed))
    prepared.sort(key=lambda p: p[1])
    tbytes, tops, tsec, passes, ran, skipped = 0, 0, 0.0, 0, [], []
    sec_per_op = 0.0
    while True:
        for (spec, M, ns, packed) in prepared:
            ops_ = gemm_ops(M, spec.N, spec.K, spec.block, ns)
            if tsec + ops_ * sec_per_op > 2 * budget_s:
                if passes == 0:
                    skipped.append(f"{spec.K}x{spec.N}@M={M}")
                continue
            x = syn.make_acts(spec, M)
            t0 = time.perf_counter()
            qa, sa = oracle.quantize_act(x)
            oracle.fused_gemm(qa, sa, packed)
            dt = time.perf_counter() - t0
            tsec += dt
            sec_per_op = dt / ops_  # the rate improves with M: the last pair predicts the next
            tbytes += layer_bytes(M, spec.N, spec.K, spec.block, ns)
            tops += ops_
            if passes == 0:
                ran.append(f"{spec.K}x{spec.N}@M={M}")
        passes += 1
        if tsec >= budget_s or not ran or passes >= 50:
            break
    return dict(value=round(tops / tsec / 1e12, 6), unit="TOP/s", gbs=round(tbytes / tsec / 1e9, 4),
                cores=int(threads), kind="oracle", seconds=round(tsec, 3),
                sample=f"{passes} pass(es) of oracle quantize_act + fused_gemm (numpy; BLAS threads = "
                       f"cores) over {', '.join(ran)}"
                       + (f"; not run (over the time bound): {', '.join(skipped)}" if skipped else ""))


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


def exact_selection_study(args):
    """The Delta-score against the exact-distortion greedy selection it stands
    in for, on full-size Llama-3-8B projections (512 calibration tokens, the
    block edges and budgets of the method) and the Qwen3-32B MLP shapes.  Both selections, their exact
    output distortions on the calibration tokens and on 512 held-out tokens,
    and their GPU times come from the library; prints one JSON line."""
    import torch
    from dense_sparse_w4a4_amd import ops
    from dense_sparse_w4a4_amd import synthetic as syn
    dev = torch.device("cuda:0")
    log = lambda *a: print(*a, file=sys.stderr, flush=True)  # noqa: E731

    def timed_ms(fn):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        out = fn()
        b.record()
        torch.cuda.synchronize()
        return out, a.elapsed_time(b)

    cases = [("llama3-8b", (4096, 4096), 64, 0.10), ("llama3-8b", (4096, 4096), 32, 0.10),
             ("llama3-8b", (4096, 4096), 128, 0.10), ("llama3-8b", (4096, 4096), 64, 0.05),
             ("llama3-8b", (4096, 4096), 64, 0.20), ("llama3-8b", (14336, 4096), 64, 0.10),
             ("qwen3-32b", (5120, 25600), 64, 0.10), ("qwen3-32b", (25600, 5120), 64, 0.10)]
    rows = []
    for model, (K, N), b, rho in cases:
        make = syn.llama3_8b if model == "llama3-8b" else syn.qwen3_32b
        spec = make(K, N).with_block(b, rho)
        w = torch.from_numpy(syn.make_weight(spec)).to(dev)
        xc = torch.from_numpy(syn.make_calib(spec)).to(dev)
        xe = torch.from_numpy(syn.make_acts(spec, 512)).to(dev)
        k = spec.n_select
        ops.select_blocks(w, xc, b, k)  # warm the kernels once
        (sd, _, _), t_delta = timed_ms(lambda: ops.select_blocks(w, xc, b, k))
        (sg, _, gains, dist), t_greedy = timed_ms(lambda: ops.select_exact_greedy(w, xc, b, k))
        none = torch.empty(0, dtype=torch.int32, device=dev)
        d = {}
        for tag, x in (("calib", xc), ("holdout", xe)):
            d0 = float(ops.distortion(w, x, b, none).item())
            dd = float(ops.distortion(w, x, b, sd).item())
            dg = float(ops.distortion(w, x, b, sg).item())
            d[tag] = dict(base=d0, greedy=dg, recovered_delta=round(1 - dd / d0, 5),
                          recovered_greedy=round(1 - dg / d0, 5))
        overlap = len(set(sd.tolist()) & set(sg.tolist())) / max(1, k)
        row = dict(model=model, K=K, N=N, block=b, rho=rho, n_select=k, T=spec.T,
                   recovered_calib_delta=d["calib"]["recovered_delta"],
                   recovered_calib_greedy=d["calib"]["recovered_greedy"],
                   recovered_holdout_delta=d["holdout"]["recovered_delta"],
                   recovered_holdout_greedy=d["holdout"]["recovered_greedy"],
                   delta_share_of_greedy_calib=round(
                       d["calib"]["recovered_delta"] / d["calib"]["recovered_greedy"], 4),
                   overlap=round(overlap, 4), delta_ms=round(t_delta, 3),
                   greedy_ms=round(t_greedy, 2),
                   # the greedy's own final distortion against mq_distortion of its
                   # selection (different summation orders: equal to ~1e-12)
                   greedy_dist_rel_diff=float(f"{float(dist[1].item()) / d['calib']['greedy'] - 1:.3e}"))
        rows.append(row)
        log(f"[exact] {model} K={K} N={N} b={b} rho={rho:.2f} n={k}: recovered calib Delta "
            f"{row['recovered_calib_delta']:.4f} / greedy {row['recovered_calib_greedy']:.4f}, held-out "
            f"{row['recovered_holdout_delta']:.4f} / {row['recovered_holdout_greedy']:.4f}, overlap "
            f"{row['overlap']:.3f}, GPU {t_delta:.2f} ms / {t_greedy:.1f} ms")
        del w, xc, xe, sd, sg, gains, dist
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "output distortion recovered: Delta top-K vs exact greedy",
                      "workload": "llama3-8b-and-qwen3-32b-projections-T512", "data": "synthetic", "n_gpus": 1,
                      "rows": rows}), flush=True)


def _pct(v, q):
    v = sorted(v)
    if len(v) == 1:
        return v[0]
    x = (len(v) - 1) * q / 100.0
    i = int(x)
    j = min(i + 1, len(v) - 1)
    return v[i] + (v[j] - v[i]) * (x - i)


def measure_mfma_ceiling(torch, ops):
    """The int8 matrix-core rate and shader clock measured on this device:
    2 workgroups of 4 waves per compute unit, each wave issuing back-to-back
    V_MFMA_I32_16X16X64_I8 (four independent chains), timed with HIP events;
    the clock is the waves' shader-cycle count over the same wall time."""
    blocks, iters = 512, 20000
    ops.measure_mfma(blocks, 200)  # warm-up
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    cycles, _ = ops.measure_mfma(blocks, iters)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3
    total_ops = blocks * 4 * iters * 4 * 2 * 16 * 16 * 64
    cyc = sorted(cycles.cpu().tolist())
    return dict(measured_mfma_int8_tops=round(total_ops / t / 1e12, 1),
                observed_clock_ghz=round(cyc[len(cyc) // 2] / t / 1e9, 3),
                probe="512 workgroups x 4 waves, 20000 rounds of 4 independent v_mfma_i32_16x16x64_i8 each")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying HIP graphs")
    ap.add_argument("--no-per-pair", action="store_true",
                    help="skip the per-(shape, M) launch statistics (counter runs)")
    ap.add_argument("--ablation", action="store_true",
                    help="per (shape, M) also time the unfused design (dense launch + standalone residual kernel)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (for HBM counter calibration)")
    ap.add_argument("--smooth", action="store_true",
                    help="output error with and without outlier migration (Llama-3-8B shapes, M=16)")
    ap.add_argument("--sweep", action="store_true",
                    help="Llama-3-70B FFN block-size x budget grid: time vs rho=0 and distortion recovered")
    ap.add_argument("--exact-selection", action="store_true",
                    help="Delta top-K vs exact-distortion greedy selection (Llama-3-8B projections)")
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
    if args.exact_selection:
        ops.lib()
        exact_selection_study(args)
        return
    dev = torch.device("cuda:0")
    ops.lib()
    layers = workload(args.workload)
    log = lambda *a: print(*a, file=sys.stderr, flush=True)  # noqa: E731

    # ---- offline: select + pack once per shape (GPU), then replicate ----
    t0 = time.perf_counter()
    base, host_layers = [], []
    for spec, ms in layers:
        w_np, xc_np = syn.make_weight(spec), syn.make_calib(spec)
        if not args.no_cpu_baseline:
            host_layers.append((w_np, xc_np))
        wt = torch.from_numpy(w_np).to(dev)
        xct = torch.from_numpy(xc_np).to(dev)
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
                gwsb = ops.fused_gemm_workspace(M, spec.N, spec.K)
                gws = torch.empty(max(gwsb, 1), dtype=torch.uint8, device=dev)
                f6 = None
                if kernel_of(M, spec.block) == "gemm_tile6_kernel":
                    # the fp6 kernel alone: its operand images prepared here,
                    # outside every timed region (the step's mq_fused_layer
                    # converts them itself on every call)
                    _, _, pb = ops.fp6_sizes(M, spec.N, spec.K, spec.block, spec.n_select)
                    f6 = (ops.fp6_prepare_acts(qa, spec.K), ops.fp6_prepare_weights(L),
                          torch.empty(max(pb, 1), dtype=torch.uint8, device=dev))
                s.append((spec, M, L, x, qa, sa, y, ws, gws, f6))
        sets.append(s)
    # pairs the layer runs as one kernel (the GEMM quantises the token tile)
    one_kernel = [ops.fused_layer_workspace(M, s.N, s.K) == 0 for s, M in pairs]
    kern = [kernel_of(M, s.block) for s, M in pairs]
    torch.cuda.synchronize()
    log(f"[bench] workload {args.workload}: {len(pairs)} (shape, M) pairs per step, "
        f"{R} rotating copies x {step_footprint / 2**20:.1f} MiB, setup {time.perf_counter() - t0:.1f}s")

    per_step_bytes = sum(layer_bytes(M, s.N, s.K, s.block, s.n_select) for s, M in pairs)
    per_step_ops = sum(gemm_ops(M, s.N, s.K, s.block, s.n_select) for s, M in pairs)
    # the GEMM launch of a pair: the one-kernel layer (fp16 X in) or the fused
    # GEMM from codes
    launch_bytes = [(layer_bytes if one else gemm_bytes)(M, s.N, s.K, s.block, s.n_select)
                    for (s, M), one in zip(pairs, one_kernel)]
    launch_ops = [gemm_ops(M, s.N, s.K, s.block, s.n_select) for s, M in pairs]

    def run_set(i, which=None):
        # which=None: the step (mq_fused_layer for every pair); otherwise the
        # GEMM launches of the pairs whose kernel is `which` (the one-kernel
        # layer where it applies, else the fused GEMM from precomputed codes)
        for p_idx, (spec, M, L, x, qa, sa, y, ws, gws, f6) in enumerate(sets[i % R]):
            if which is None:
                ops.fused_layer(x, L, out=y, workspace=ws)
            elif kern[p_idx] == which:
                if one_kernel[p_idx]:
                    ops.fused_layer(x, L, out=y, workspace=ws)
                elif f6 is not None:
                    ops.fused_gemm_fp6(f6[0], sa, M, L, f6[1], out=y, split_ws=f6[2])
                else:
                    ops.fused_gemm(qa, sa, L, out=y, workspace=gws)

    for i in range(max(args.warmup, R)):
        run_set(i)
    torch.cuda.synchronize()

    classes = sorted(set(kern))
    use_graph = not args.no_graph
    cap = torch.cuda.Stream()
    if use_graph:
        # one HIP graph per rotating set: the whole step, and per kernel the
        # step's GEMM launches alone (per-launch timing)
        g_step, g_cls = [], {c: [] for c in classes}
        for r in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                run_set(r)
            g_step.append(g)
            for c in classes:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cap):
                    run_set(r, c)
                g_cls[c].append(g)
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

    # ---- each kernel's GEMM launches alone: average launch time over K steps ----
    cls_time = {}
    for c in classes:
        if use_graph:
            t_ms, _ = timed(args.steps, lambda i, c=c: g_cls[c][i % R].replay())
        else:
            t_ms, _ = timed(args.steps, lambda i, c=c: run_set(i, c))
        cls_time[c] = t_ms * 1e-3 / args.steps  # seconds per step
    # (shape, M) launch statistics: each pair's launches replayed from a graph
    # over enough copies of its packed layer that one pass is >= 512 MB (no
    # launch finds its weights in the 256 MB Infinity Cache); every replay is
    # timed on its own and gives one sample of the mean launch time
    per_pair = []
    if use_graph and not args.no_per_pair:
        modes = ["fused", "dense", "actq", "layer"] + (["unfused"] if args.ablation else [])
        for p_idx, (spec, M) in enumerate(pairs):
            (_, _, L0, x, qa, sa, y, ws, gws, f6) = sets[0][p_idx]
            n = max(2, -(-ROTATE_BYTES // L0.nbytes()))
            copies = [L0.clone() for _ in range(n)]
            # pairs on the int8 tile route: also the fp6 kernel on prepared
            # images (a deployment that keeps the converted weights)
            p6 = None
            if f6 is None and kern[p_idx] == "gemm_tile_kernel" and spec.block in (64, 128):
                _, _, pb = ops.fp6_sizes(M, spec.N, spec.K, spec.block, spec.n_select)
                p6 = (ops.fp6_prepare_acts(qa, spec.K), torch.empty(max(pb, 1), dtype=torch.uint8, device=dev))
            # the fp6 kernel reads prepared images: one per copy, so its
            # launches rotate through as many weight bytes as the others
            imgs = [ops.fp6_prepare_weights(L) for L in copies] if (f6 is not None or p6 is not None) else None
            if f6 is not None:
                dimgs = [ops.fp6_prepare_weights(ops.PackedLayer(L.N, L.K, L.block, L.qw, L.sw,
                                                                 torch.zeros_like(L.row_ptr), L.col_idx[:0],
                                                                 L.qr[:0], L.sr[:0])) for L in copies]
            q2, s2 = torch.empty_like(qa), torch.empty_like(sa)
            res = {}
            for mode in modes + (["fp6_prepared"] if p6 is not None else []):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cap):
                    for ci, L in enumerate(copies):
                        D = ops.PackedLayer(L.N, L.K, L.block, L.qw, L.sw, torch.zeros_like(L.row_ptr),
                                            L.col_idx[:0], L.qr[:0], L.sr[:0])
                        if mode == "layer":
                            ops.fused_layer(x, L, out=y, workspace=ws)
                        elif mode == "actq":
                            ops.quantize_act(x, q2, s2)
                        elif mode == "fp6_prepared":
                            ops.fused_gemm_fp6(p6[0], sa, M, L, imgs[ci], out=y, split_ws=p6[1])
                        elif f6 is not None and mode in ("fused", "dense"):
                            ops.fused_gemm_fp6(f6[0], sa, M, L if mode == "fused" else D,
                                               imgs[ci] if mode == "fused" else dimgs[ci], out=y,
                                               split_ws=f6[2])
                        else:
                            ops.fused_gemm(qa, sa, L if mode == "fused" else D, out=y, workspace=gws)
                        if mode == "unfused":
                            ops.residual_merge(qa, sa, L, y)
                g.replay()
                torch.cuda.synchronize()
                samples = []
                for _ in range(PAIR_REPLAYS):
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    g.replay()
                    e1.record()
                    torch.cuda.synchronize()
                    samples.append(e0.elapsed_time(e1) * 1e3 / n)
                res[mode] = samples
                del g
            del copies, imgs, p6
            if f6 is not None:
                del dimgs
            torch.cuda.empty_cache()
            med = {m: _pct(v, 50) for m, v in res.items()}
            gb = gemm_bytes(M, spec.N, spec.K, spec.block, spec.n_select)
            go = gemm_ops(M, spec.N, spec.K, spec.block, spec.n_select)
            row = dict(K=spec.K, N=spec.N, M=M, kernel=kern[p_idx], n_select=spec.n_select,
                       us_p10=round(_pct(res["fused"], 10), 3), us_p50=round(med["fused"], 3),
                       us_p90=round(_pct(res["fused"], 90), 3),
                       tops=round(go / (med["fused"] * 1e-6) / 1e12, 2),
                       dense_equiv_tops=round(2 * M * spec.N * spec.K / (med["fused"] * 1e-6) / 1e12, 2),
                       gbs=round(gb / (med["fused"] * 1e-6) / 1e9, 1),
                       frac_mfma=round(go / (med["fused"] * 1e-6) / 1e12 / mfma_peak(kern[p_idx]), 4),
                       frac_int8_peak=round(go / (med["fused"] * 1e-6) / 1e12 / INT8_MFMA_PEAK_TOPS, 4),
                       frac_hbm=round(gb / (med["fused"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                       dense_only_us_p50=round(med["dense"], 3),
                       residual_cost=round(med["fused"] / med["dense"] - 1, 4),
                       act_quant_us_p50=round(med["actq"], 3),
                       layer_us_p50=round(med["layer"], 3), layer_one_kernel=bool(one_kernel[p_idx]),
                       samples=PAIR_REPLAYS, copies=n)
            if "fp6_prepared" in med:
                row["fp6_prepared_us_p50"] = round(med["fp6_prepared"], 3)
            if "unfused" in med:
                row["unfused_us_p50"] = round(med["unfused"], 3)
                row["unfused_over_fused"] = round(med["unfused"] / med["fused"], 4)
            per_pair.append(row)
            log(f"[bench]   K={spec.K:6d} N={spec.N:6d} M={M:5d}: gemm p50 {med['fused']:9.2f} us "
                f"(p10 {row['us_p10']:.2f}, p90 {row['us_p90']:.2f})  {row['gbs']:8.1f} GB/s "
                f"({row['frac_hbm']:5.1%} HBM)  {row['tops']:8.1f} TOPS ({row['frac_mfma']:5.1%} of "
                f"{'fp6' if kern[p_idx] == 'gemm_tile6_kernel' else 'int8'} peak, {row['frac_int8_peak']:5.1%} int8)  "
                f"dense-only {med['dense']:9.2f} us (residual +{row['residual_cost']:5.1%})  "
                f"act-quant {med['actq']:7.2f} us  layer {med['layer']:9.2f} us"
                + (f"  unfused x{row['unfused_over_fused']:.3f}" if "unfused" in med else "")
                + (f"  fp6 on prepared images {row['fp6_prepared_us_p50']:.2f} us" if "fp6_prepared" in med else ""))

    # ---- rooflines: each kernel's algorithmic work per launch over its
    # average launch time; the dominant kernel (most time per step) first ----
    def roof_of(c):
        idx = [i for i, k in enumerate(kern) if k == c]
        t = cls_time[c]
        nl = len(idx)
        if c == "gemm_stream_kernel":
            achieved = sum(launch_bytes[i] for i in idx) / t / 1e9
            r = dict(bound="hbm", achieved=round(achieved, 2), peak=HBM_PEAK_GBS, unit="GB/s",
                     frac=round(achieved / HBM_PEAK_GBS, 4))
        else:
            achieved = sum(launch_ops[i] for i in idx) / t / 1e12
            r = dict(bound="mfma", achieved=round(achieved, 2), peak=mfma_peak(c), unit="TOP/s",
                     frac=round(achieved / mfma_peak(c), 4))
            if c == "gemm_tile6_kernel":
                r["mfma_dtype"] = "fp6 e2m3 (int4 codes as exact fp6 fields), fp32 accumulate"
                r["frac_of_int8_peak"] = round(achieved / INT8_MFMA_PEAK_TOPS, 4)
            else:
                r["mfma_dtype"] = "int8 (int4 codes widened), int32 accumulate"
        r["traffic"] = traffic_from_profile(args.workload, c)
        r["kernel"] = c
        r["launches_per_step"] = nl
        r["M"] = sorted({pairs[i][1] for i in idx})
        r["avg_launch_us"] = round(t / nl * 1e6, 3)
        r["alg_bytes_per_launch"] = sum(launch_bytes[i] for i in idx) / nl
        r["alg_ops_per_launch"] = sum(launch_ops[i] for i in idx) / nl
        r["launches_quantising_in_kernel"] = int(sum(one_kernel[i] for i in idx))
        return r

    order = sorted(classes, key=lambda c: -cls_time[c])
    roof = roof_of(order[0])
    if len(order) > 1:
        roof["other_kernels"] = [roof_of(c) for c in order[1:]]
    if not args.copy_calibration:
        roof.update(measure_mfma_ceiling(torch, ops))
        if roof["bound"] == "mfma" and roof["kernel"] == "gemm_tile_kernel":
            roof["frac_of_measured_mfma"] = round(roof["achieved"] / roof["measured_mfma_int8_tops"], 4)
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
        for r in [roof] + roof.get("other_kernels", []):
            if r["bound"] == "hbm":
                r["frac_of_copy"] = round(r["achieved"] / copy_gbs, 4)
        del a, b

    if args.copy_calibration:
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    out = {
        "metric": METRIC,
        "value": round(per_step_ops / (ms_per_step * 1e-3) / 1e12, 3),
        "unit": "TOP/s",
        "gbs": round(per_step_bytes / (ms_per_step * 1e-3) / 1e9, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 codes on int8 / fp6 MFMA",
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "shapes_KxN": [[s.K, s.N] for s, _, _, _ in base],
            "M": sorted({M for _, M in pairs}),
            "group": 128, "block": base[0][0].block, "rho": base[0][0].rho,
            "codes": ("w4a4 int4 symmetric; M <= 32: int8 MFMA, int32 accumulators; 32 < M < 1024: int8 MFMA; "
                      "M >= 1024: exact fp6 MFMA on re-encoded codes (converted per call), fp32 group sums; "
                      "fp32 epilogue, fp16 out"),
            "step": "mq_fused_layer (fp16 X -> fp16 Y) for every (shape, M)",
            "bytes_per_step": per_step_bytes, "ops_per_step": per_step_ops,
            "rotating_copies": R,
            "launch": "hip-graph" if use_graph else "eager",
        },
        "roofline": roof,
    }
    if per_pair:
        out["per_pair"] = per_pair
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        out["cpu_baseline"] = cpu_baseline(layers, args.cpu_budget, host_layers)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
