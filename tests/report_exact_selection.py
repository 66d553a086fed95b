"""Report: Delta-score top-K vs exact-distortion greedy selection (CPU oracle).

    python tests/report_exact_selection.py

Prints, per synthetic layer and budget, the output distortion recovered
(1 - D(S)/D(empty)) on the calibration tokens and on held-out tokens of the
same layer, the overlap of the two selections, and their CPU times.
"""
import os
import sys
import time

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import oracle  # noqa: E402
from dense_sparse_w4a4_amd import synthetic as syn  # noqa: E402


def main():
    print("| K x N | b | rho | n_sel | recovered (calib) Delta / greedy | recovered (held-out) Delta / greedy "
          "| overlap | CPU s Delta / greedy |")
    print("|---|---|---|---|---|---|---|---|")
    for K, N in ((512, 512), (1024, 512)):
        for b in (32, 64):
            for rho in (0.05, 0.10, 0.20):
                spec = syn.LayerSpec(f"q{K}", K=K, N=N, w_outlier_frac=0.005, w_outlier_mult=20.0,
                                     T=128, block=b, rho=rho)
                w, xc, xe = syn.make_weight(spec), syn.make_calib(spec), syn.make_acts(spec, 256)
                qw, sw = oracle.quantize_base(w)
                E = oracle.base_error(w, qw, sw)
                _, _, rhat = oracle.residual_all_blocks(E, b)
                t0 = time.perf_counter()
                sd, _, _ = oracle.select_blocks(w, xc, b, spec.n_select)
                t1 = time.perf_counter()
                sg = oracle.select_exact_greedy(w, xc, b, spec.n_select)
                t2 = time.perf_counter()
                rec = {}
                for tag, x in (("c", xc), ("e", xe)):
                    d0 = oracle.distortion(x, w, qw, sw, rhat, [], b)
                    rec[tag] = [1 - oracle.distortion(x, w, qw, sw, rhat, s, b) / d0 for s in (sd, sg)]
                ov = len(set(sd.tolist()) & set(sg.tolist())) / max(1, len(sd))
                print(f"| {K}x{N} | {b} | {rho:.2f} | {spec.n_select} | {rec['c'][0]:.3f} / {rec['c'][1]:.3f} "
                      f"| {rec['e'][0]:.3f} / {rec['e'][1]:.3f} | {ov:.2f} | {t1 - t0:.2f} / {t2 - t1:.2f} |")


if __name__ == "__main__":
    main()
