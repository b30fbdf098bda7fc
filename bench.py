#!/usr/bin/env python3
"""Benchmark of the paired-4:8 sparse NVFP4 MoE expert path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input, inputs resident in HBM:
  single-projection workloads (c0, c1, c2): route/permute + dispatch quantize -> grouped GEMM;
  decode layer (c3): route/permute + quantize -> gate_up GEMM -> quantize -> down GEMM;
  MLP (c4 prefill, c3_mlp decode from bf16 tokens): route/permute + quantize -> gate_up GEMM + SwiGLU +
    requantize -> down GEMM -> combine.
Weights and input batches rotate over R copies so that repeated steps do not find the weights in the
last-level cache when the weight set would fit there (c1: 8 copies, about 1.1 GB). The R consecutive
steps of one rotation are captured as one HIP graph, the way a decode server captures a sequence of
MoE layers, so a graph launch is paid once per R steps; K timed steps are K // R replays of that
graph plus single-step graphs for the remainder.

Metric (paper Appendix D.2): TFLOP/s_eff = 2 * M * K * sum_e N_e / t with M the output rows and N_e
the tokens of expert e, summed over the step's GEMMs. The roofline object reports the dominant
kernel: its algorithmic bytes (decode: weights of experts with tokens at 2.75 bits per weight, the
quantized activations, bf16 outputs) or algorithmic flops (prefill: the kept products only, half
of the dense-equivalent count) per launch, divided by its mean duration measured with HIP events
on the launch stream.

Prints one JSON line. --gpus N > 1 exits: the path runs on one GPU (no collective or sharded path).
"""
import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "grouped sparse-NVFP4 GEMM eff. TFLOP/s + HBM GB/s (decode & prefill, 1 GPU)"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
F16_PEAK_TFLOPS = 2500.0     # MI355X dense f16 MFMA; the 2:4 sparse MFMA does kept products at this rate x2 eff
FP8_PEAK_TFLOPS = 5000.0      # MI355X dense FP8 MFMA
FP4_PEAK_TFLOPS = 10100.0     # MI355X dense FP4 / FP6 MFMA
BITS_PER_WEIGHT = 2.75       # paper Appendix A, Eq. 7


def tflops_eff(M, K, sum_n, seconds):
    """Paper Appendix D.2: TFLOP/s_eff = 2 M K sum_g N_g / (t * 1e12)."""
    return 2.0 * M * K * sum_n / (seconds * 1e12)


def weight_bytes(N, K):
    return N * K * BITS_PER_WEIGHT / 8.0


def gemm_bytes(n_active, N, K, rows, E, out_bytes=2):
    """Algorithmic HBM bytes of one grouped GEMM launch: compressed weights of the experts that have
    tokens, NVFP4 activations (codes + block scales), outputs, offsets and per-expert scales."""
    return (n_active * weight_bytes(N, K) + rows * (K / 2 + K / 32) + rows * N * out_bytes + (E + 1) * 4 + 2 * E * 4)


def fused_step_bytes(n_active, N, K, T, k, E, x_bytes=4):
    """Algorithmic HBM bytes of the one-launch decode step (route + quantize + GEMM): compressed
    weights of the experts with tokens, the token rows and ids read once, the routing tables, the
    activation codes + block scales and the bf16 outputs written once, per-expert scales."""
    rows = T * k
    return (n_active * weight_bytes(N, K) + T * K * x_bytes + rows * 4 + rows * 8 + (2 * E + 1) * 4 +
            rows * (K / 2 + K / 32) + rows * N * 2 + 2 * E * 4)


FUSED_KERNEL = "dispatch_gemm_kernel"
MLP_KEY = "moesq_expert_mlp (gate_up+SwiGLU+requant, down)"
GATEUP_KERNEL = "gemm_tile_kernel<MLP> (gate_up + SwiGLU + requant)"


def fused_eligible(cfg):
    """The library's one-launch condition for moesq_route_quantize_gemm."""
    rows = cfg.T * cfg.k
    return not cfg.mlp and not cfg.N2 and rows <= 1024 and 2 * rows <= cfg.E and cfg.K <= 2048


def _src_hash():
    h = hashlib.sha256()
    for f in ("gemm.hip", "common.h", "api.hip", "launch.h"):  # the kernels and which operands they get
        with open(os.path.join(ROOT, "sparse_precision_grouped_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


COPY_BYTES = 1 << 30  # payload of the plain-copy calibration launch


def calibrate_copy(torch, iters=5):
    """A plain device copy of COPY_BYTES, run under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE to get the
    counter's reading for a launch whose HBM traffic is known (COPY_BYTES read, COPY_BYTES written)."""
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(iters):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": COPY_BYTES, "iters": iters}))


def _pmc_means(csv_path, match, grid=None):
    """Mean per-dispatch value (KiB) and dispatch count of every counter in a rocprofv3 counter CSV,
    per kernel whose name contains `match` (and, with `grid`, only dispatches of that many work-items)."""
    import csv
    acc = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            k = r["Kernel_Name"]
            if match not in k:
                continue
            if grid is not None and "gemm_" in k and int(r["Grid_Size"]) != grid:
                continue
            key = (k.split("(")[0], r["Counter_Name"])
            acc.setdefault(key, []).append(float(r["Counter_Value"]))
    return {k: (float(np.mean(v)), len(v)) for k, v in acc.items()}


def summarize_pmc(argv):
    """--summarize-pmc WORKLOAD FETCH_CSV WRITE_CSV COPY_FETCH_CSV COPY_WRITE_CSV: scale the GEMM
    kernels' FETCH_SIZE / WRITE_SIZE by the copy calibration and record bytes per dominant launch in
    profiles/traffic.json (keyed by workload and kernel, tagged with the kernel source hash)."""
    wl, fcsv, wcsv, cf, cw = argv
    import gen
    cfg = gen.CONFIGS[wl]
    # two projections with the same weight-streaming kernel: keep the first (gate_up) launches, told
    # apart by their grid (N/64 x E workgroups of 256 threads)
    grid = (cfg.N // 64) * cfg.E * 256 if cfg.N2 and not cfg.mlp else None
    fetch = _pmc_means(fcsv, "gemm_", grid)
    write = _pmc_means(wcsv, "gemm_", grid)
    # the calibration run's copy launch is the one that reads the most (the fill before it reads nothing)
    cf_all = {k: v for (k, c), v in _pmc_means(cf, "").items() if c == "FETCH_SIZE"}
    copy_name = max(cf_all, key=lambda k: cf_all[k][0])
    cfetch_kib = cf_all[copy_name][0]
    cwrite_kib = _pmc_means(cw, "")[(copy_name, "WRITE_SIZE")][0]
    f_fetch = COPY_BYTES / 1024.0 / cfetch_kib
    f_write = COPY_BYTES / 1024.0 / cwrite_kib
    per_kernel = {}
    for (k, c), (v, n) in fetch.items():
        if c == "FETCH_SIZE":
            per_kernel.setdefault(k, {})["fetch_bytes"] = v * 1024.0 * f_fetch
            per_kernel[k]["dispatches"] = n
    for (k, c), (v, n) in write.items():
        if c == "WRITE_SIZE":
            per_kernel.setdefault(k, {})["write_bytes"] = v * 1024.0 * f_write
    entries = {}
    if wl in ("c4", "c3_mlp"):
        # one moesq_expert_mlp call: its gate_up and down kernels (distinct template instances)
        key = MLP_KEY
        # the production forms only: the calibration and dump forms (epilogue template argument 3 or 2) run
        # once at set-up
        import re
        side = re.compile(r"gemm_tile_kernel<[23],|gemm_decode_kernel<.*, [23]>$")
        total = sum(d["fetch_bytes"] + d["write_bytes"] for k, d in per_kernel.items()
                    if ("gemm_tile_kernel" in k or "gemm_decode_kernel" in k) and not side.search(k))
        # the prefill gate_up launch alone (the tiled kernel with the MLP epilogue, template argument 1)
        gu = [d for k, d in per_kernel.items() if "gemm_tile_kernel<1," in k]
        if gu:
            entries[GATEUP_KERNEL] = gu[0]["fetch_bytes"] + gu[0]["write_bytes"]
    else:
        key = next((n for n in (FUSED_KERNEL, "gemm_decode_kernel") if any(n in k for k in per_kernel)),
                   "gemm_tile_kernel")
        total = sum(d["fetch_bytes"] + d["write_bytes"] for k, d in per_kernel.items() if key in k)
    path = os.path.join(ROOT, "profiles", "traffic.json")
    t = json.load(open(path)) if os.path.exists(path) else {}
    entries[key] = total
    for kk, tot in entries.items():
        t["%s:%s" % (wl, kk)] = {"bytes_per_launch": round(tot), "src_hash": _src_hash(), "copy_kernel": copy_name,
                                 "copy_factor_fetch": round(f_fetch, 4), "copy_factor_write": round(f_write, 4),
                                 "kernels": {k: {kv: round(vv) for kv, vv in d.items()} for k, d in per_kernel.items()}}
    with open(path, "w") as f:
        json.dump(t, f, indent=1, sort_keys=True)
    print(json.dumps(t["%s:%s" % (wl, key)]))


# MI355X: 8 XCDs x 32 CUs x 4 SIMDs
N_XCD, N_SIMD = 8, 1024


def summarize_sq(paths):
    """--summarize-sq CSV [CSV ...]: per-dispatch means of the SQ / GRBM counters of the GEMM kernels in
    rocprofv3 counter CSVs (one pass per file), with derived ratios, as a markdown table."""
    import csv
    acc, dur = {}, {}
    for p in paths:
        with open(p) as f:
            for r in csv.DictReader(f):
                k = r["Kernel_Name"].split("(")[0]
                if "gemm_" not in k:
                    continue
                acc.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
                dur.setdefault(k, {})[(p, r["Correlation_Id"])] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    for k, cs in acc.items():
        m = {c: float(np.mean(v)) for c, v in cs.items()}
        n = max(len(v) for v in cs.values())
        t = float(np.mean(list(dur[k].values())))
        print("\n`%s` (%d dispatches per pass, mean duration %.1f us under the profiler)\n" % (k, n, t * 1e6))
        print("| counter | mean per dispatch |\n|---|---|")
        for c in sorted(m):
            print("| %s | %.4g |" % (c, m[c]))
        gui = m.get("GRBM_GUI_ACTIVE")
        rows = []
        if gui:
            rows.append(("GRBM_GUI_ACTIVE / %d XCDs / duration (clock the GUI counter ran at)" % N_XCD,
                         "%.2f GHz" % (gui / N_XCD / t / 1e9)))
            if "SQ_VALU_MFMA_BUSY_CYCLES" in m:
                rows.append(("MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / (%d SIMDs x GUI cycles per XCD)" % N_SIMD,
                             "%.3f" % (m["SQ_VALU_MFMA_BUSY_CYCLES"] / (N_SIMD * gui / N_XCD))))
        if "SQ_INSTS_VALU" in m and "SQ_INSTS_MFMA" in m:
            rows.append(("SQ_INSTS_VALU / SQ_INSTS_MFMA (VALU count includes the MFMAs)",
                         "%.2f" % (m["SQ_INSTS_VALU"] / m["SQ_INSTS_MFMA"])))
        if "SQ_INSTS_LDS" in m and "SQ_INSTS_MFMA" in m:
            rows.append(("SQ_INSTS_LDS / SQ_INSTS_MFMA", "%.2f" % (m["SQ_INSTS_LDS"] / m["SQ_INSTS_MFMA"])))
        if "SQ_INSTS_SALU" in m and "SQ_INSTS_MFMA" in m:
            rows.append(("SQ_INSTS_SALU / SQ_INSTS_MFMA", "%.2f" % (m["SQ_INSTS_SALU"] / m["SQ_INSTS_MFMA"])))
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in m and "SQ_VALU_MFMA_BUSY_CYCLES" in m:
            rows.append(("SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES",
                         "%.3f" % (m["SQ_VALU_MFMA_COEXEC_CYCLES"] / m["SQ_VALU_MFMA_BUSY_CYCLES"])))
        for c in ("SQ_WAIT_INST_ANY", "SQ_WAIT_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU"):
            if c in m and "SQ_WAVE_CYCLES" in m:
                scale = 1.0 if c.startswith("SQ_WAIT") else 0.25  # wait counters and wave cycles in quad-cycles
                rows.append(("%s / SQ_WAVE_CYCLES" % c, "%.3f" % (scale * m[c] / m["SQ_WAVE_CYCLES"])))
        if rows:
            print("\n| derived | value |\n|---|---|")
            for a, b in rows:
                print("| %s | %s |" % (a, b))


def _traffic(kernel_key):
    """HBM traffic per launch from a committed rocprofv3 counter summary, if it was taken on the
    current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    ent = t.get(kernel_key)
    if not ent or ent.get("src_hash") != _src_hash():
        return None
    return ent.get("bytes_per_launch")


class Workload:
    """Device buffers, graphs and accounting for one named config."""

    def __init__(self, name, rotate, torch, gen, mq, f16_operand=False, fused=False, dyn_scale=False):
        self.torch, self.gen, self.mq = torch, gen, mq
        self.cfg = cfg = gen.CONFIGS[name]
        self.name = name
        dev = "cuda"
        self.kind = "mlp" if cfg.mlp else ("pair" if cfg.N2 else "single")
        E, T, k = cfg.E, cfg.T, cfg.k
        self.rows = T * k
        self.tiled = self.kind == "mlp" or self.rows > 16 * E
        # routing, quantization and the GEMM in one launch (moesq_route_quantize_gemm)
        self.fused = fused and fused_eligible(cfg) and not dyn_scale
        # the activation tensor scale computed on the device inside each step (moesq_route_quantize_dyn)
        self.dyn_scale = dyn_scale
        # weights: compressed once on the device, then copied for rotation
        self.W = self._weights(0, cfg.N, cfg.K)
        self.W2 = self._weights(1, cfg.N2, cfg.K2) if self.kind != "single" else None
        wset = self.W.kl.numel() + (self.W2.kl.numel() if self.W2 else 0)
        self.R = max(1, min(rotate, int(np.ceil(1.2e9 / wset)))) if wset < 512e6 else 1
        self.Wc = [self.W] + [self._clone(self.W) for _ in range(self.R - 1)]
        self.W2c = [self.W2] * self.R if self.W2 is None else [self.W2] + [self._clone(self.W2) for _ in
                                                                          range(self.R - 1)]
        self.slots = []
        for r in range(self.R):
            cr = dataclasses.replace(cfg, seed=cfg.seed + 7919 * r)
            ids, wts = gen.routing(cr)
            x = torch.from_numpy(gen.activations(cr, 0, T, cfg.K)).to(dev)
            if cfg.x_bf16:
                x = x.to(torch.bfloat16)
            sl = dict(ids=torch.from_numpy(ids).to(dev), wts=torch.from_numpy(wts).to(dev), x=x,
                      counts_host=np.bincount(ids.ravel(), minlength=E))
            g = mq.moesq_global_scale(x)
            sl["ga"] = g.expand(E).contiguous()
            sl["rt"] = mq.moesq_route_permute(sl["ids"], E)
            sl["ws_route"] = torch.empty(max(1, mq.moesq_workspace_bytes(mq.WS_ROUTE, T, k, E)), dtype=torch.uint8,
                                         device=dev)
            sl["q"] = torch.empty((self.rows, cfg.K // 2), dtype=torch.uint8, device=dev)
            sl["s"] = torch.empty((self.rows, cfg.K // 32), dtype=torch.uint8, device=dev)
            # optional: the quantizer also writes the f16 operand copy that the tiled kernel can stage
            # straight into LDS (more HBM traffic, fewer instructions in the GEMM)
            sl["xk"] = (torch.empty((self.rows, cfg.K), dtype=torch.float16, device=dev)
                        if f16_operand else None)
            if self.kind == "single":
                sl["y"] = torch.empty((self.rows, cfg.N), dtype=torch.bfloat16, device=dev)
            elif self.kind == "pair":
                x2 = torch.from_numpy(gen.activations(cr, 1, T, cfg.K2)).to(dev)
                sl["x2"] = x2
                sl["ga2"] = mq.moesq_global_scale(x2).expand(E).contiguous()
                sl["y"] = torch.empty((self.rows, cfg.N), dtype=torch.bfloat16, device=dev)
                sl["q2"] = torch.empty((self.rows, cfg.K2 // 2), dtype=torch.uint8, device=dev)
                sl["s2"] = torch.empty((self.rows, cfg.K2 // 32), dtype=torch.uint8, device=dev)
                sl["y2"] = torch.empty((self.rows, cfg.N2), dtype=torch.bfloat16, device=dev)
                sl["xk2"] = (torch.empty((self.rows, cfg.K2), dtype=torch.float16, device=dev)
                             if f16_operand else None)
            else:
                I = cfg.N // 2
                sl["gh"] = torch.full((E,), cfg.gamma_h, dtype=torch.float32, device=dev)
                sl["ws_mlp"] = mq.mlp_workspace(self.rows, I, False, dev)
                sl["y2"] = torch.empty((self.rows, cfg.N2), dtype=torch.bfloat16, device=dev)
                sl["out"] = torch.empty((T, cfg.N2), dtype=torch.bfloat16, device=dev)
            self.slots.append(sl)
        if self.kind == "mlp":
            self._calibrate()
        torch.cuda.synchronize()
        self.graphs = []

    def _calibrate(self):
        """Per-expert tensor scales of the intermediate h (the model card's stored per-expert input scale,
        Eq. 5 over the expert's amax of h), calibrated on the device on the first batch before anything
        is timed, then kept for every batch: moesq_expert_mlp with MOESQ_F_CALIBRATE."""
        mq, cfg, sl = self.mq, self.cfg, self.slots[0]
        mq.moesq_route_quantize(sl["ids"], cfg.E, sl["x"], sl["ga"], rt=sl["rt"], q=sl["q"], s=sl["s"], xk=sl["xk"],
                                workspace=sl["ws_route"])
        gam, amax = mq.moesq_calibrate_gamma_h(self.W, self.W2, sl["q"], sl["s"], sl["ga"], sl["rt"]["offsets"],
                                               xk=sl["xk"])
        for slr in self.slots:
            slr["gh"].copy_(gam)
        g = gam.cpu().numpy()
        self.gamma_h_range = (float(g.min()), float(g.max()))

    def _weights(self, proj, N, K):
        torch, gen, mq, cfg = self.torch, self.gen, self.mq, self.cfg
        W = mq.Weights.empty(cfg.E, N, K)
        chunk = max(1, min(cfg.E, int(2e9 // (N * K * 4))))
        buf = torch.empty((chunk, N, K), dtype=torch.float32, device="cuda")
        ws = torch.empty(mq.moesq_workspace_bytes(mq.WS_COMPRESS, 0, 0, chunk), dtype=torch.uint8, device="cuda")
        for e0 in range(0, cfg.E, chunk):
            n = min(chunk, cfg.E - e0)
            for j in range(n):
                gen.gpu_fill_normal(buf[j], cfg.seed, gen.weight_stream(proj, e0 + j), cfg.w_std)
            sub = mq.Weights(W.packed[e0:e0 + n], W.mask[e0:e0 + n], W.scale[e0:e0 + n], W.gscale[e0:e0 + n])
            mq.moesq_compress_weights(buf[:n], out=sub, workspace=ws, prepack=False)
        W.prepack()
        torch.cuda.synchronize()
        del buf
        return W

    def _clone(self, W):
        return self.mq.Weights(W.packed, W.mask, W.scale, W.gscale.clone(), W.kl.clone())

    # ---- one step of the path on slot r (enqueued on the current stream) ----
    def step(self, r):
        mq, cfg, sl = self.mq, self.cfg, self.slots[r]
        rt = sl["rt"]
        if self.fused:
            mq.moesq_route_quantize_gemm(sl["ids"], sl["x"], sl["ga"], self.Wc[r], rt=rt, q=sl["q"], s=sl["s"],
                                         y=sl["y"], workspace=sl["ws_route"])
            return
        # routing + dispatch quantization (one launch for decode-sized batches)
        if self.dyn_scale:
            mq.moesq_route_quantize_dyn(sl["ids"], cfg.E, sl["x"], gamma_out=sl["ga"], rt=rt, q=sl["q"], s=sl["s"],
                                        xk=sl["xk"], workspace=sl["ws_route"])
        else:
            mq.moesq_route_quantize(sl["ids"], cfg.E, sl["x"], sl["ga"], rt=rt, q=sl["q"], s=sl["s"], xk=sl["xk"],
                                    workspace=sl["ws_route"])
        if self.kind != "mlp":
            mq.moesq_grouped_gemm(self.Wc[r], sl["q"], sl["s"], sl["ga"], rt["offsets"], y=sl["y"], xk=sl["xk"])
        if self.kind == "pair":
            mq.moesq_quantize_act(sl["x2"], sl["ga2"], slot_pos=rt["slot_pos"], k=cfg.k, offsets=rt["offsets"],
                                  q=sl["q2"], s=sl["s2"], xk=sl["xk2"])
            mq.moesq_grouped_gemm(self.W2c[r], sl["q2"], sl["s2"], sl["ga2"], rt["offsets"], y=sl["y2"],
                                  xk=sl["xk2"])
        if self.kind == "mlp":
            mq.moesq_expert_mlp(self.Wc[r], self.W2c[r], sl["q"], sl["s"], sl["ga"], sl["gh"], rt["offsets"],
                                y=sl["y2"], workspace=sl["ws_mlp"], xk=sl["xk"])
            mq.moesq_unpermute_combine(sl["y2"], rt["slot_pos"], sl["wts"], out=sl["out"])

    def dominant(self, r):
        """The dominant kernel launch of a step (enqueued on the current stream)."""
        mq, sl = self.mq, self.slots[r]
        rt = sl["rt"]
        if self.fused:
            self.step(r)
        elif self.kind == "mlp":
            mq.moesq_expert_mlp(self.Wc[r], self.W2c[r], sl["q"], sl["s"], sl["ga"], sl["gh"], rt["offsets"],
                                y=sl["y2"], workspace=sl["ws_mlp"], xk=sl["xk"])
        else:
            mq.moesq_grouped_gemm(self.Wc[r], sl["q"], sl["s"], sl["ga"], rt["offsets"], y=sl["y"], xk=sl["xk"])

    def down_only(self, r):
        """The MLP's down GEMM alone (the same kernel and operands as the second launch of
        moesq_expert_mlp: the requantized h codes from the workspace, and for the weight-streaming
        form (rows <= 16 E) their f16 copy; the tiled form stages h from the codes)."""
        mq, cfg, sl = self.mq, self.cfg, self.slots[r]
        I = cfg.N // 2
        hq, hs, _ = mq.mlp_workspace_views(sl["ws_mlp"], self.rows, I)
        hk = mq.mlp_hk_view(sl["ws_mlp"], self.rows, I) if self.rows <= 16 * cfg.E else None
        mq.moesq_grouped_gemm(self.W2c[r], hq, hs, sl["gh"], sl["rt"]["offsets"], y=sl["y2"], xk=hk)

    def capture(self):
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for r in range(self.R):
                self.step(r)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for r in range(self.R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self.step(r)
            self.graphs.append(g)
        self.chain = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.chain):
            for r in range(self.R):
                self.step(r)
        torch.cuda.synchronize()

    def run(self, n):
        """Enqueue n consecutive steps: the R-step graph n // R times, then single-step graphs."""
        for _ in range(n // self.R):
            self.chain.replay()
        for r in range(n % self.R):
            self.graphs[r].replay()

    # ---- accounting ----
    def eff_flops_per_step(self):
        cfg = self.cfg
        if self.kind == "single":
            return 2.0 * cfg.N * cfg.K * self.rows
        if self.kind == "pair":
            return 2.0 * self.rows * (cfg.N * cfg.K + cfg.N2 * cfg.K2)
        return 2.0 * self.rows * (cfg.N * cfg.K + cfg.N2 * cfg.K2)

    def roofline_units(self):
        """(bound, algorithmic units per dominant launch averaged over the slots, unit, peak, kernel)."""
        cfg = self.cfg
        decode = self.rows <= 16 * cfg.E
        if decode and self.kind == "mlp":
            # both weight-streaming GEMMs: the two projections' weights of the experts with tokens, the
            # routed rows' NVFP4 codes, the intermediate h codes written once and read once, bf16 outputs
            I = cfg.N // 2
            b = np.mean([gemm_bytes(int((sl["counts_host"] > 0).sum()), cfg.N, cfg.K, self.rows, cfg.E,
                                    out_bytes=(I / 2 + I / 32) / cfg.N) +
                         gemm_bytes(int((sl["counts_host"] > 0).sum()), cfg.N2, cfg.K2, self.rows, cfg.E)
                         for sl in self.slots])
            return "hbm", b / 1e9, "GB/s", HBM_PEAK_GBS, MLP_KEY
        if self.fused:
            b = np.mean([fused_step_bytes(int((sl["counts_host"] > 0).sum()), cfg.N, cfg.K, cfg.T, cfg.k, cfg.E,
                                          x_bytes=2 if cfg.x_bf16 else 4) for sl in self.slots])
            return "hbm", b / 1e9, "GB/s", HBM_PEAK_GBS, FUSED_KERNEL
        if decode:
            b = np.mean([gemm_bytes(int((sl["counts_host"] > 0).sum()), cfg.N, cfg.K, self.rows, cfg.E)
                         for sl in self.slots])
            return "hbm", b / 1e9, "GB/s", HBM_PEAK_GBS, "gemm_decode_kernel"
        kept = 0.5 * self.eff_flops_per_step() if self.kind == "mlp" else cfg.N * cfg.K * self.rows
        kern = MLP_KEY if self.kind == "mlp" else "gemm_tile_kernel"
        return "mfma", kept / 1e12, "TFLOP/s", F16_PEAK_TFLOPS, kern


def cpu_baseline(wl, orc, gen, max_reps=3):
    """The oracle's step on the host cores, on a bounded sample of the same workload."""
    cfg = wl.cfg
    if wl.kind != "single" or cfg.E * cfg.N * cfg.K > 512 * 1024 * 1024:
        return cpu_baseline_sampled(wl, orc, gen, max_reps)
    E, T, k, N, K = cfg.E, cfg.T, cfg.k, cfg.N, cfg.K
    ids, wts = gen.routing(cfg)
    x = gen.activations(cfg, 0, T, K)
    rows = T * k
    w = np.stack([gen.weights_expert(cfg, 0, e, N, K) for e in range(E)])
    Wo = orc.compress(w)
    row_list = None if rows <= 4096 else np.linspace(0, rows - 1, 512).astype(np.int64)
    sample = "full step (route, dispatch-quantize, GEMM) on %s" % (
        "all %d rows" % rows if row_list is None else "512 of %d rows (GEMM), all rows (route, quantize)" % rows)
    ga = np.full(E, orc.global_scale_of(x), np.float32)
    times = []
    n_rows = rows if row_list is None else row_list.size
    for _ in range(max_reps):
        t0 = time.perf_counter()
        Rr = orc.route(ids, E)
        q, s = orc.dispatch_quantize(x, Rr["sorted_slot"], k, Rr["offsets"], ga)
        orc.grouped_gemm(Wo, q, s, ga, Rr["offsets"], row_list)
        times.append(time.perf_counter() - t0)
        if sum(times) > 20:
            break
    t = float(np.median(times))
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": tflops_eff(N, K, n_rows, t), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": sample + ", median of %d run(s), %.3f s each" % (len(times), t), "cpu_model": _cpu_model()}


# rows of the expert sample per workload kind: the Kimi decode workloads route 1-2 rows to an expert,
# the prefill MLP a few hundred
CPU_SAMPLE = {"pair": (16, 64), "mlp_decode": (16, 64), "mlp": (16, 2048)}   # (max experts, max rows)


def _sub_weights(gen, orc, cfg, proj, N, K, experts):
    """The oracle's compression of the sampled experts' weights (host draw), as a grouped problem of
    its own (expert i of the sample = experts[i])."""
    return orc.compress(np.stack([gen.weights_expert(cfg, proj, int(e), N, K) for e in experts]))


def cpu_baseline_sampled(wl, orc, gen, max_reps=3):
    """Workloads too large for the oracle in seconds (the Kimi shapes: 10-15 MB of weights per expert,
    29.4 M multiply-adds per routed row of the gate_up): the oracle runs the whole step's per-token parts
    (routing, dispatch quantization, for the MLP the combine) on the full batch, and the per-row GEMM
    chain (gate_up, SwiGLU, requantization, down) on the routed rows of a seeded sample of experts,
    which it computes as a grouped problem of its own. The full step's time is extrapolated linearly
    in the rows (the GEMM chain costs the same per row): t = t_per_token_parts + t_sample * rows /
    sample_rows, and value = TFLOP/s_eff of the full step over that time. Weight compression is setup
    (untimed), as in the GPU measurement."""
    cfg = wl.cfg
    E, T, k = cfg.E, cfg.T, cfg.k
    rows = T * k
    decode = rows <= 16 * E
    kind = "mlp_decode" if (wl.kind == "mlp" and decode) else wl.kind
    max_e, max_rows = CPU_SAMPLE[kind]
    ids, wts = gen.routing(cfg)
    x = gen.activations(cfg, 0, T, cfg.K)
    if cfg.x_bf16:
        import torch  # the bf16 hand-over of the tokens, as on the device
        x = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    R = orc.route(ids, E)
    off = np.asarray(R["offsets"])
    counts = np.diff(off)
    rng = np.random.default_rng(cfg.seed)
    experts, n = [], 0
    for e in rng.permutation(np.flatnonzero(counts > 0)):
        if len(experts) == max_e or n >= max_rows:
            break
        experts.append(int(e))
        n += int(min(counts[e], max_rows - n))
    experts = np.array(experts)
    take = [np.arange(off[e], off[e] + min(counts[e], max_rows)) for e in experts]
    per = np.array([t.size for t in take])
    total = int(per.sum())
    while total > max_rows:             # trim the last expert to the row budget
        per[-1] -= total - max_rows
        take[-1] = take[-1][:per[-1]]
        total = int(per.sum())
    sel = np.concatenate(take)
    sub_off = np.concatenate([[0], np.cumsum(per)]).astype(np.int32)
    N, K = cfg.N, cfg.K
    W1 = _sub_weights(gen, orc, cfg, 0, N, K, experts)
    W2 = _sub_weights(gen, orc, cfg, 1, cfg.N2, cfg.K2, experts) if cfg.N2 else None
    x2 = gen.activations(cfg, 1, T, cfg.K2) if wl.kind == "pair" else None
    ga = np.full(E, orc.global_scale_of(x), np.float32)
    ga2 = np.full(E, orc.global_scale_of(x2), np.float32) if x2 is not None else None
    t_tok, t_rows = [], []
    for _ in range(max_reps):
        t0 = time.perf_counter()
        Rr = orc.route(ids, E)
        q, s = orc.dispatch_quantize(x, Rr["sorted_slot"], k, Rr["offsets"], ga)
        if x2 is not None:
            q2, s2 = orc.dispatch_quantize(x2, Rr["sorted_slot"], k, Rr["offsets"], ga2)
        t1 = time.perf_counter()
        y1 = orc.grouped_gemm(W1, q[sel], s[sel], ga[experts], sub_off)
        if wl.kind == "pair":
            y2 = orc.grouped_gemm(W2, q2[sel], s2[sel], ga2[experts], sub_off)
        elif wl.kind == "mlp":
            h = orc.swiglu(y1).astype(np.float32)
            ex = orc.expert_of_rows(sub_off, np.arange(total))
            amax = np.zeros(len(experts), np.float32)
            np.maximum.at(amax, ex, np.abs(h).max(axis=1))
            gh = np.array([orc.global_scale(float(v)) for v in amax], np.float32)
            hq, hs = orc.quantize_rows(h, gh, ex)
            y2 = orc.grouped_gemm(W2, hq, hs, gh, sub_off)
        t2 = time.perf_counter()
        if wl.kind == "mlp":
            yfull = np.zeros((rows, cfg.N2), np.float64)
            yfull[sel] = y2
            orc.combine(yfull, Rr["slot_pos"], wts)
        t3 = time.perf_counter()
        t_tok.append((t1 - t0) + (t3 - t2))
        t_rows.append(t2 - t1)
        if sum(t_tok) + sum(t_rows) > 25:
            break
    tt, tr = float(np.median(t_tok)), float(np.median(t_rows))
    t_full = tt + tr * rows / total
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    flops = wl.eff_flops_per_step()
    parts = {"pair": "routing, dispatch quantization of both projections' inputs",
             "mlp": "routing, dispatch quantization, combine"}[wl.kind]
    chain = {"pair": "gate_up GEMM, down GEMM", "mlp": "gate_up GEMM, SwiGLU, requantization, down GEMM"}[wl.kind]
    sample = ("%s on the full batch (%.3f s); %s on the %d routed rows of %d seeded-random experts (%.3f s), "
              "extrapolated x%.1f to all %d rows: %.2f s per step; median of %d run(s)" % (
                  parts, tt, chain, total, len(experts), tr, rows / total, rows, t_full, len(t_rows)))
    return {"value": flops / t_full / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": sample, "extrapolated": True, "cpu_model": _cpu_model()}


def _cpu_model():
    """The host CPU's model name (Linux), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# Kernel sweep of the pages' Appendix D.2 (Table 8 layer shapes, per-expert token counts following the
# ragged pattern {N, 3N/4, N/2, N/4} repeated over the G experts).
SWEEP_LAYERS = {
    "kimi_gate_up": (4096, 7168, [32, 64, 128, 256, 512, 1024], [24, 48, 96, 192, 384]),
    "kimi_down": (7168, 2048, [32, 64, 128, 256, 512, 1024], [24, 48, 96, 192, 384]),
    "qwen_gate_up": (1536, 2048, [16, 32, 64, 128, 256, 512, 1024], [8, 16, 32, 64, 128]),
    "qwen_down": (2048, 768, [16, 32, 64, 128, 256, 512, 1024], [8, 16, 32, 64, 128]),
}


def sweep_counts(G, N):
    pat = [N, 3 * N // 4, N // 2, N // 4]
    return [pat[g % 4] for g in range(G)]


def run_sweep(layer, torch, gen, mq, reps=20, Ns=None, Gs=None, kernel="auto", dense=False):
    """Median graph-replay time of the grouped GEMM (and of quantize + GEMM from bf16 activations)
    for each (G, N); one JSON line per point."""
    M, K, Nl, Gl = SWEEP_LAYERS[layer]
    Nl = Ns or Nl
    Gl = Gs or Gl
    Gmax = max(Gl)
    cfg = dataclasses.replace(gen.CONFIGS["c0"], E=Gmax, N=M, K=K, seed=4242)
    W = mq.Weights.empty(Gmax, M, K)
    chunk = max(1, min(Gmax, int(2e9 // (M * K * 4))))
    buf = torch.empty((chunk, M, K), dtype=torch.float32, device="cuda")
    ws = torch.empty(mq.moesq_workspace_bytes(mq.WS_COMPRESS, 0, 0, chunk), dtype=torch.uint8, device="cuda")
    for e0 in range(0, Gmax, chunk):
        n = min(chunk, Gmax - e0)
        for j in range(n):
            gen.gpu_fill_normal(buf[j], cfg.seed, gen.weight_stream(0, e0 + j), cfg.w_std)
        sub = mq.Weights(W.packed[e0:e0 + n], W.mask[e0:e0 + n], W.scale[e0:e0 + n], W.gscale[e0:e0 + n])
        mq.moesq_compress_weights(buf[:n], out=sub, workspace=ws, prepack=False)
    W.prepack()
    Wd = None
    if dense:
        # the dense control: the same weights quantized without pruning
        Wd = mq.DenseWeights(torch.empty((Gmax, M, K // 2), dtype=torch.uint8, device="cuda"),
                             torch.empty((Gmax, M, K // 32), dtype=torch.uint8, device="cuda"),
                             torch.empty((Gmax,), dtype=torch.float32, device="cuda"))
        for e in range(Gmax):
            gen.gpu_fill_normal(buf[0], cfg.seed, gen.weight_stream(0, e), cfg.w_std)
            mq.moesq_global_scale(buf[0], out=Wd.gscale[e:e + 1])
            mq.moesq_quantize_act(buf[0], Wd.gscale[e:e + 1], q=Wd.codes[e], s=Wd.scale[e])
        Wd.prepack()
    del buf
    ekl = W.kl.numel() // Gmax
    dkl = Wd.kl.numel() // Gmax if dense else 0
    st = torch.cuda.current_stream()
    first = True
    for G in Gl:
        Wg = mq.Weights(W.packed[:G], W.mask[:G], W.scale[:G], W.gscale[:G], W.kl[:G * ekl])
        Wdg = mq.DenseWeights(Wd.codes[:G], Wd.scale[:G], Wd.gscale[:G], Wd.kl[:G * dkl]) if dense else None
        for N in (Nl[:1] + Nl) if first else Nl:  # the first point twice: clocks and caches settle
            counts = sweep_counts(G, N)
            rows = int(sum(counts))
            offsets = torch.tensor(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32), device="cuda")
            x = torch.empty((rows, K), dtype=torch.float32, device="cuda")
            gen.gpu_fill_normal(x, cfg.seed, gen.act_stream(7), 1.0)
            xb = x.to(torch.bfloat16)
            del x
            g = mq.moesq_global_scale(xb)
            ga = g.expand(G).contiguous()
            decode = rows <= 16 * G if kernel == "auto" else kernel == "decode"
            flags = mq.F_FORCE_DECODE if decode else mq.F_FORCE_PREFILL
            xk = torch.empty((rows, K), dtype=torch.float16, device="cuda") if decode else None
            q = torch.empty((rows, K // 2), dtype=torch.uint8, device="cuda")
            s = torch.empty((rows, K // 32), dtype=torch.uint8, device="cuda")
            y = torch.empty((rows, M), dtype=torch.bfloat16, device="cuda")
            mq.moesq_quantize_act(xb, g, q=q, s=s, xk=xk)

            def gemm():
                mq.moesq_grouped_gemm(Wg, q, s, ga, offsets, y=y, xk=xk, flags=flags)

            def quant_gemm():
                mq.moesq_quantize_act(xb, g, q=q, s=s, xk=xk)
                mq.moesq_grouped_gemm(Wg, q, s, ga, offsets, y=y, xk=xk, flags=flags)

            def dense_gemm():
                mq.moesq_dense_grouped_gemm(Wdg, q, s, ga, offsets, y=y, xk=xk, flags=flags)

            def dense_gemm_fp4():
                mq.moesq_dense_grouped_gemm(Wdg, q, s, ga, offsets, y=y, flags=flags)

            out = {"layer": layer, "M": M, "K": K, "G": G, "N": N, "rows": rows,
                   "kernel": "decode" if decode else "tiled"}
            runs = [("gemm", gemm), ("quant_gemm", quant_gemm)]
            if dense:
                # the control takes its faster activation operand (the f16 copy or the NVFP4 codes)
                runs += [("dense_gemm_f16", dense_gemm)] if xk is not None else []
                runs += [("dense_gemm", dense_gemm_fp4)]
            for name, fn in runs:
                side = torch.cuda.Stream()
                side.wait_stream(st)
                with torch.cuda.stream(side):
                    fn()
                st.wait_stream(side)
                torch.cuda.synchronize()
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph):
                    fn()
                for _ in range(3):
                    graph.replay()
                ts = []
                for _ in range(reps):
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record(st)
                    graph.replay()
                    b.record(st)
                    torch.cuda.synchronize()
                    ts.append(a.elapsed_time(b))
                t = float(np.median(ts)) * 1e-3
                out[name + "_us"] = round(t * 1e6, 2)
                if name == "gemm":
                    out["tflops_eff"] = round(tflops_eff(M, K, rows, t), 1)
                    out["weight_GBs"] = round(G * weight_bytes(M, K) / t / 1e9, 1)
                if name == "dense_gemm":
                    if "dense_gemm_f16_us" in out and out["dense_gemm_f16_us"] < out["dense_gemm_us"]:
                        out["dense_gemm_fp4_us"] = out["dense_gemm_us"]
                        out["dense_gemm_us"] = out["dense_gemm_f16_us"]
                        t = out["dense_gemm_us"] * 1e-6
                    out["dense_tflops_eff"] = round(tflops_eff(M, K, rows, t), 1)
                    out["speedup_vs_dense"] = round(out["dense_gemm_us"] / out["gemm_us"], 3)
            if not first:
                print(json.dumps(out), flush=True)
            first = False
            del q, s, y, xk, xb


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c4", choices=["c0", "c1", "c2", "c3", "c4", "c3_mlp"])
    ap.add_argument("--rotate", type=int, default=8)
    ap.add_argument("--kernel-iters", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--operand", choices=["auto", "nvfp4", "f16"], default="auto",
                    help="activation operand of the GEMMs: NVFP4 codes decoded in the kernel, or the quantizer's "
                         "f16 copy; auto = f16 for weight-streaming (decode-sized) workloads, NVFP4 "
                         "otherwise")
    ap.add_argument("--dispatch", choices=["fused", "separate"], default="fused",
                    help="decode step of a single projection: routing, quantization and the GEMM in one launch "
                         "(moesq_route_quantize_gemm, where it applies) or as two calls")
    ap.add_argument("--act-scale", choices=["static", "dynamic"], default="static",
                    help="activation tensor scale: a per-expert constant computed once (the model card's stored "
                         "scale), or Eq. 5 over each step's tokens on the device inside the step")
    ap.add_argument("--sweep", choices=sorted(SWEEP_LAYERS) + ["all"],
                    help="the pages' G x N kernel sweep on one layer shape (one JSON line per point)")
    ap.add_argument("--sweep-kernel", choices=["auto", "decode", "tiled"], default="auto")
    ap.add_argument("--sweep-n", type=int, nargs="*", help="restrict the sweep's per-expert token counts")
    ap.add_argument("--sweep-dense", action="store_true",
                    help="also time the dense NVFP4 control on the same weights (speedup of the sparse kernel)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB device copy (traffic-counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=5, metavar=("WORKLOAD", "FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV",
                                                         "COPY_WRITE_CSV"),
                    help="host only: write profiles/traffic.json from rocprofv3 counter CSVs")
    ap.add_argument("--summarize-sq", nargs="+", metavar="CSV",
                    help="host only: SQ / GRBM counter table of the GEMM kernels from rocprofv3 counter CSVs")
    args = ap.parse_args(argv)
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc)
        return 0
    if args.summarize_sq:
        summarize_sq(args.summarize_sq)
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the path runs on one GPU only (no collective or sharded path); "
              "rerun with --gpus 1", file=sys.stderr)
        return 2

    import torch
    if args.calibrate_copy:
        calibrate_copy(torch)
        return 0

    import gen
    import sparse_precision_grouped_amd as mq

    if args.sweep:
        torch.cuda.set_device(0)
        for layer in (sorted(SWEEP_LAYERS) if args.sweep == "all" else [args.sweep]):
            run_sweep(layer, torch, gen, mq, Ns=args.sweep_n, kernel=args.sweep_kernel, dense=args.sweep_dense)
        return 0

    torch.cuda.set_device(0)
    cfgw = gen.CONFIGS[args.workload]
    # the f16 copy pays off in the weight-streaming kernels; the tiled kernels keep the NVFP4 codes
    decode_shaped = cfgw.T * cfgw.k <= 16 * cfgw.E
    fused = args.dispatch == "fused" and fused_eligible(cfgw) and args.act_scale == "static"
    # the one-launch step builds its f16 operand in LDS and writes no copy
    f16_operand = args.operand == "f16" or (args.operand == "auto" and decode_shaped and not fused)
    wl = Workload(args.workload, args.rotate, torch, gen, mq, f16_operand, fused, args.act_scale == "dynamic")
    wl.capture()
    wl.run(args.warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    wl.run(args.steps)
    torch.cuda.synchronize()
    t = (time.perf_counter() - t0) / args.steps
    value = wl.eff_flops_per_step() / t / 1e12

    # spread of the step time (outside the timed region): HIP events around each replay of the R-step
    # graph, per step
    st = torch.cuda.current_stream()
    reps = max(5, min(50, args.steps // wl.R))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record(st)
        wl.chain.replay()
        b.record(st)
    torch.cuda.synchronize()
    per_step = np.array([a.elapsed_time(b) * 1e3 / wl.R for a, b in evs])
    pcts = [round(float(np.percentile(per_step, q)), 2) for q in (10, 50, 90)]

    # dominant kernel: one pair of HIP events on the launch stream around kernel_iters back-to-back
    # launches (rotating weight copies), the mean per launch; the median of 3 such blocks
    def block_ms(fn, iters):
        out = []
        for _ in range(3):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(st)
            for i in range(iters):
                fn(i % wl.R)
            b.record(st)
            torch.cuda.synchronize()
            out.append(a.elapsed_time(b) / iters)
        return float(np.median(out))

    kms = block_ms(wl.dominant, args.kernel_iters)
    bound, units, unit, peak, kname = wl.roofline_units()
    mlp_split = None
    if wl.kind == "mlp" and bound == "mfma":
        # the prefill MLP is two launches (gate_up + SwiGLU + requant, then down): the dominant one is the
        # gate_up; its time is the MLP call's minus the down GEMM's, timed alone on the same operands
        cfg = wl.cfg
        down_ms = block_ms(wl.down_only, args.kernel_iters)
        kept_gu, kept_dn = cfg.N * cfg.K * wl.rows / 1e12, cfg.N2 * cfg.K2 * wl.rows / 1e12
        mlp_split = {"kernel": MLP_KEY, "kernel_ms": round(kms, 5), "achieved": round((kept_gu + kept_dn) / (kms * 1e-3), 2),
                     "frac": round((kept_gu + kept_dn) / (kms * 1e-3) / peak, 4),
                     "down_kernel_ms": round(down_ms, 5),
                     "down_frac": round(kept_dn / (down_ms * 1e-3) / peak, 4),
                     "traffic": _traffic("%s:%s" % (args.workload, MLP_KEY))}
        kms = kms - down_ms
        units, kname = kept_gu, GATEUP_KERNEL
    achieved = units / (kms * 1e-3)
    traffic = _traffic("%s:%s" % (args.workload, kname))
    roofline = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": kname,
                "kernel_ms": round(kms, 5)}
    if mlp_split:
        roofline["mlp_two_gemms"] = mlp_split
    if bound == "mfma":
        # the same launch against the chip's dense FP8 and FP4 peaks, on dense-equivalent flops
        # (2 x the kept flops)
        roofline["dense_equivalent_tflops"] = round(2 * achieved, 1)
        roofline["frac_of_fp8_dense_peak"] = round(2 * achieved / FP8_PEAK_TFLOPS, 4)
        roofline["frac_of_fp4_dense_peak"] = round(2 * achieved / FP4_PEAK_TFLOPS, 4)

    cpu = None
    if not args.no_cpu_baseline:
        import oracle as orc
        cpu = cpu_baseline(wl, orc, gen)

    cfg = wl.cfg
    # whole-step algorithmic GEMM bytes per second (weight-streaming workloads only)
    n_act = np.mean([(sl["counts_host"] > 0).sum() for sl in wl.slots])
    step_gbps = None
    if wl.fused:
        step_gbps = round(fused_step_bytes(n_act, cfg.N, cfg.K, cfg.T, cfg.k, cfg.E,
                                           x_bytes=2 if cfg.x_bf16 else 4) / t / 1e9, 1)
    elif wl.kind == "single":
        step_gbps = round(gemm_bytes(n_act, cfg.N, cfg.K, wl.rows, cfg.E) / t / 1e9, 1)
    elif wl.kind == "pair":
        step_gbps = round((gemm_bytes(n_act, cfg.N, cfg.K, wl.rows, cfg.E) +
                           gemm_bytes(n_act, cfg.N2, cfg.K2, wl.rows, cfg.E)) / t / 1e9, 1)
    if wl.kind == "mlp":
        cfgd_extra = {"gamma_h": "per expert, calibrated on the device (Eq. 5 over each expert's amax of h), "
                                 "range %.4g..%.4g" % wl.gamma_h_range}
    else:
        cfgd_extra = {}
    line = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(t * 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "nvfp4 operands, f16 sparse MFMA, f32 accumulate", "data": "synthetic",
        "config": {"workload": "%s: %s (E=%d, K=%d, N=%d, T=%d, top-%d, %s routing%s)" % (
            args.workload, cfg.desc, cfg.E, cfg.K, cfg.N, cfg.T, cfg.k, cfg.routing,
            ", then K=%d N=%d" % (cfg.K2, cfg.N2) if cfg.N2 else ""),
            "rows": wl.rows, "weight_copies": wl.R, "graph_replay": "%d steps per graph" % wl.R,
            "activation_operand": ("f16, quantized into LDS by the GEMM's workgroups" if wl.fused else
                                   "f16 copy" if f16_operand else "nvfp4"),
            "dispatch": "one launch (route+quantize+GEMM)" if wl.fused else "separate launches",
            "activation_scale": ("dynamic: Eq. 5 over the step's tokens, on the device" if wl.dyn_scale else
                                 "static per-expert constant"),
            "step_gbps_algorithmic": step_gbps, "step_us_p10_p50_p90": pcts, **cfgd_extra},
        "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
