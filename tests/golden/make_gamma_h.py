"""Writes gamma_h.txt: the per-expert tensor scale of the MLP's intermediate h for the routed-expert MLP
workloads, computed by the CPU oracle alone from the seeded inputs.

Source: paper "Hardware-Native Joint Sparse-Quantization for Trillion-Scale Mixture-of-Experts",
Section 3.4, Eq. 5 (gamma = 448 / (amax / 6) from the tensor's largest magnitude); model card
"Kimi-K2.5-P48NVFP4-MoESQ" (the input scale is stored per expert linear). Reading: the down projection's
input scale of expert e is Eq. 5 over the largest |h| of that expert's routed rows of the batch, with h =
SiLU(g) * u from the oracle's gate_up GEMM (double), rounded to fp32 (the precision the requantization
takes its decisions in).

Run from the repository root:  python tests/golden/make_gamma_h.py [c4 c3_mlp]
Calls only the input generator (gen/) and the oracle (oracle/). c4 takes several minutes: the oracle's
gate_up GEMM over all 65,536 routed rows.
"""
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import gen  # noqa: E402
import oracle as orc  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gamma_h.txt")


def tokens(cfg):
    """The workload's token rows as the oracle quantizes them (bf16 hand-over rounds them first)."""
    x = gen.activations(cfg, 0, cfg.T, cfg.K)
    if cfg.x_bf16:
        import torch  # input preparation only: round-to-nearest-even to bf16 and back
        x = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    return x


def gamma_h_table(name):
    cfg = gen.CONFIGS[name]
    E, H, I2 = cfg.E, cfg.K, cfg.N
    x = tokens(cfg)
    ids, _ = gen.routing(cfg)
    R = orc.route(ids, E)
    off = R["offsets"]
    ga = np.full(E, orc.global_scale_of(x), np.float32)
    q, s = orc.dispatch_quantize(x, R["sorted_slot"], cfg.k, off, ga)
    rows = []
    t0 = time.time()
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            rows.append((e, 0.0, float(orc.global_scale(0.0)), 0))
            continue
        W = orc.compress(gen.weights_expert(cfg, 0, e, I2, H)[None])
        y13 = orc.grouped_gemm(W, q[lo:hi], s[lo:hi], ga[e:e + 1], np.array([0, hi - lo], np.int32))
        amax = float(np.abs(orc.swiglu(y13).astype(np.float32)).max())
        rows.append((e, amax, float(orc.global_scale(amax)), hi - lo))
        if e % 32 == 0:
            print("%s: expert %d/%d (%.0f s)" % (name, e, E, time.time() - t0), flush=True)
    return rows


def main(names):
    have = {}
    if os.path.exists(OUT):
        for line in open(OUT):
            if line.strip() and not line.startswith("#"):
                have.setdefault(line.split()[0], []).append(line)
    for n in names:
        have[n] = ["%s %d %s %s %d\n" % (n, e, float.hex(a), float.hex(g), cnt) for e, a, g, cnt in gamma_h_table(n)]
    with open(OUT, "w") as f:
        f.write("# Per-expert tensor scale gamma_h of the MLP intermediate h (paper Section 3.4, Eq. 5; model card:\n"
                "# input scale stored per expert linear), from the oracle alone: gamma_h = Eq. 5 of the largest |h|\n"
                "# (fp32) over the expert's routed rows of the workload's seeded batch. Written by make_gamma_h.py.\n"
                "# Columns: workload expert amax_h(hex) gamma_h(hex) routed_rows\n")
        for n in sorted(have):
            f.writelines(have[n])


if __name__ == "__main__":
    main(sys.argv[1:] or ["c3_mlp", "c4"])
