"""Benchmark of the W4A16 group-wise hot path on one MI355X, on the 36-layer decoder stack.

Workload (the largest configuration; it fits one GPU): 36 decoder layers at hidden 4096, 32
query / 8 KV heads of dim 128, intermediate 12288 -> 252 linears (q, o 4096x4096; k, v
1024x4096; gate, up 12288x4096; down 4096x12288), 6.95e9 weights; 8192 calibration tokens per
layer input (bf16, lognormal(0,1) channel scales); K = 40 candidates over alpha in [0.4, 1.0];
LSQ on the gate and up weights; prefill at M = 2048 and decode at M = 1 on every linear.  Inputs
are drawn once on the GPU (seeded; synth.device_*) and stay resident in HBM.

One step = one pass of the whole hot path over the stack, in a decoder's order:
  for each layer: quant_hessian of its 4 inputs -> quant_scale_search, quant_pack of its 7
  linears -> lsq_fwd + lsq_bwd (fused forward) on gate and up -> w4a16_gemm_dq at M = 2048
  (prefill, weights dequantized to bf16 in registers) on its 7 linears;
  then the decode pass: w4a16_gemm at M = 1 over all 252 linears as grouped launches per decoder
  phase (q|k|v, o, gate|up, down: the order a decoder issues them in), replayed from a HIP graph.
`value` is the decode pass's HBM bandwidth (bytes of codes, scales, x and y per pass / its
time in the timed region).  Every launch is bracketed by HIP events on its stream; `kernels`
reports each family's algorithmic rate (sum of the work of its launches / sum of their
durations) against its roofline, and `roofline` repeats it for the family with the largest share
of the step.  `components` adds measurements outside the step: the prefill product on exact weights
(w4a16_gemm) beside the dequantizing one, the decode pass in other launch orders, single-launch
rates, and the rows beyond the step (per-channel search, joint descent, GPTQ, fused LSQ + Adam).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--layers L] [--no-cpu] [--no-components]
    python bench.py --pmc-copy                       (copy kernel that calibrates the counters)
    python bench.py --pmc-summary FETCH_DIR WRITE_DIR [MFMA_DIR]   (-> profiles/traffic_*.json)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W4A16 GEMV GB/s (% HBM peak); scale-search groups/s; Hessian+GEMM MFMA util"
WORKLOAD = "decoder36_h4096"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # dense bf16 MFMA
PEAK_FP32_VALU_TFLOPS = 157.3  # fp32 vector (published)
PEAK_FP64_TFLOPS = 78.6        # fp64 vector and matrix (published)
GS = 1.0 / np.sqrt(32 * 7)
PREFILL_M = 2048
CSRC = os.path.join(ROOT, "w4a16_group_wise_amd", "csrc")

# kernel family -> (source file, kernel symbol substrings as they appear in a kernel trace)
KERNELS = {
    "hessian": ("hessian.hip", ["hessian_kernel", "hessian_fixup_kernel"]),
    "scale_search": ("scale_search.hip", ["search_split_kernel", "search_split16_kernel"]),
    "pack": ("pack_lsq.hip", ["pack_kernel"]),
    "lsq_fwd": ("pack_lsq.hip", ["lsq_fwd_kernel"]),
    "lsq_bwd": ("pack_lsq.hip", ["lsq_bwd_kernel"]),
    "prefill_gemm": ("gemm.hip", ["gemm_dq_kernel", "gemm_fixup_kernel"]),
    "decode_gemv": ("gemv.hip", ["gemv_stream_kernel"]),
}


def src_hash(fname: str) -> str:
    h = hashlib.sha256()
    for f in (fname, "common.hpp"):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_peaks(dev):
    """Measured peaks in the same job: a plain streaming read of 2 GiB and loops of independent
    bf16 and fp64 matrix-core products (the library's probe calls), best of 5, timed with HIP
    events."""
    import torch
    import w4a16_group_wise_amd as w4q

    buf = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    best_r, best_m, best_d = 0.0, 0.0, 0.0
    for _ in range(5):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        w4q.probe_read(buf, nontemporal=True)
        e1.record()
        e1.synchronize()
        best_r = max(best_r, buf.numel() / (e0.elapsed_time(e1) * 1e-3))
        e0.record()
        flop = w4q.probe_mfma_bf16(4000, dev)
        e1.record()
        e1.synchronize()
        best_m = max(best_m, flop / (e0.elapsed_time(e1) * 1e-3))
        e0.record()
        flop = w4q.probe_mfma_f64(8000, dev)
        e1.record()
        e1.synchronize()
        best_d = max(best_d, flop / (e0.elapsed_time(e1) * 1e-3))
    del buf
    torch.cuda.empty_cache()
    return {"hbm": best_r, "mfma": best_m, "mfma_f64": best_d}


def gemv_bytes(d_out, d_in, m=1):
    return d_out * d_in * 9 // 16 + 2 * m * d_in + 4 * m * d_out


class Stack:
    """The 36-layer stack's inputs and outputs, resident in HBM, and the launches of one step."""

    def __init__(self, dev, layers):
        import torch
        import w4a16_group_wise_amd as w4q
        from w4a16_group_wise_amd import synth

        self.c = c = synth.WORKLOADS[WORKLOAD]
        self.dev = dev
        self.layers = layers
        g = synth.device_generator(dev, 5)
        f32 = torch.float32
        self.alpha = torch.from_numpy(c.alpha()).to(dev)
        self.K = c.n_cand
        dims = c.inputs()
        self.x = [{inp: synth.device_calib_x(g, c.n_tok, d, c.sigma, dev) for inp, d in dims.items()}
                  for _ in range(layers)]
        self.lin = []
        for layer in range(layers):
            per = {}
            for lin in c.linears:
                G = lin.d_in // 32
                e = dict(lin=lin, w=synth.device_weights(g, lin.d_out, lin.d_in, c.outlier_frac, dev),
                         scale=torch.empty((lin.d_out, G), dtype=f32, device=dev),
                         idx=torch.empty((lin.d_out, G), dtype=torch.uint8, device=dev),
                         obj=torch.empty((lin.d_out, G), dtype=f32, device=dev),
                         packed=torch.empty((lin.d_out, lin.d_in // 2), dtype=torch.uint8, device=dev),
                         s16=torch.empty((lin.d_out, G), dtype=torch.float16, device=dev),
                         y1=torch.empty((1, lin.d_out), dtype=f32, device=dev))
                if lin.name in c.lsq:
                    e["g"] = synth.device_grad(g, lin.d_out, lin.d_in, dev)
                per[lin.name] = e
            self.lin.append(per)
        # per-step scratch reused by every layer: Hessians, LSQ outputs, prefill outputs
        self.h = {inp: torch.empty((d, d), dtype=f32, device=dev) for inp, d in dims.items()}
        big = max(lin.d_out * lin.d_in for lin in c.linears)
        self.w_hat = torch.empty(big, dtype=f32, device=dev)
        self.gw = torch.empty(big, dtype=f32, device=dev)
        self.w_hat2 = torch.empty(big, dtype=f32, device=dev)
        self.gsc = torch.empty(big // 32, dtype=f32, device=dev)
        self.y_pre = torch.empty(PREFILL_M * max(lin.d_out for lin in c.linears), dtype=f32, device=dev)
        ws = max([w4q.workspace_size("quant_hessian", c.n_tok, d) for d in dims.values()] +
                 [w4q.workspace_size("w4a16_gemm", PREFILL_M, lin.d_out, lin.d_in) for lin in c.linears] +
                 [w4q.workspace_size("w4a16_gemm_dq", PREFILL_M, lin.d_out, lin.d_in) for lin in c.linears])
        self.ws = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev)
        self.decode_bytes = sum(gemv_bytes(lin.d_out, lin.d_in) for lin in c.linears) * layers
        self._decode_graph = None

    def view(self, buf, *shape):
        n = int(np.prod(shape))
        return buf[:n].view(*shape)

    def layer_launches(self, layer):
        """(family, work, fn) of one layer's launches, in order."""
        import w4a16_group_wise_amd as w4q

        c = self.c
        out = []
        xs = self.x[layer]
        for inp, xt in xs.items():
            n, d = xt.shape
            out.append(("hessian", n * d * (d + 1),
                        lambda xt=xt, inp=inp: w4q.quant_hessian(xt, h=self.h[inp], workspace=self.ws)))
        for name, e in self.lin[layer].items():
            lin = e["lin"]
            ng = lin.d_out * lin.d_in // 32
            out.append(("scale_search", ng * self.K * 1056,
                        lambda e=e, lin=lin: w4q.quant_scale_search(e["w"], self.h[lin.inp], self.alpha,
                                                                    out=(e["scale"], e["idx"], e["obj"], None))))
            out.append(("pack", lin.d_out * lin.d_in * 4.5 + ng * 6,
                        lambda e=e: w4q.quant_pack(e["w"], e["scale"], out=(e["packed"], e["s16"]))))
            if name in c.lsq:
                nw = lin.d_out * lin.d_in
                shp = (lin.d_out, lin.d_in)
                out.append(("lsq_fwd", nw * 8 + ng * 4,
                            lambda e=e, shp=shp: w4q.lsq_fwd(e["w"], e["scale"], out=self.view(self.w_hat, *shp))))
                out.append(("lsq_bwd", nw * 16 + ng * 8,
                            lambda e=e, shp=shp, ng=ng: w4q.lsq_bwd(
                                e["w"], e["scale"], e["g"], GS,
                                out=(self.view(self.gw, *shp), self.view(self.gsc, shp[0], shp[1] // 32),
                                     self.view(self.w_hat2, *shp)))))
        for name, e in self.lin[layer].items():
            lin = e["lin"]
            xt = xs[lin.inp][:PREFILL_M]
            # prefill: the product with the weights dequantized to bf16 in registers
            out.append(("prefill_gemm", 2 * PREFILL_M * lin.d_out * lin.d_in,
                        lambda e=e, xt=xt, lin=lin: w4q.w4a16_gemm_dq(
                            xt, e["packed"], e["s16"], out=self.view(self.y_pre, PREFILL_M, lin.d_out),
                            workspace=self.ws)))
        return out

    def decode_plans(self):
        """Grouped M = 1 launches per decoder phase, in dependency order: q|k|v share the
        attention input, o follows them, gate|up share the MLP input, down follows them."""
        import w4a16_group_wise_amd as w4q

        plans = []
        for layer in range(self.layers):
            per = self.lin[layer]
            xs = self.x[layer]
            for names in (("q", "k", "v"), ("o",), ("gate", "up"), ("down",)):
                es = [per[n] for n in names]
                plans.append(w4q.GemvGroupPlan([xs[e["lin"].inp][:1] for e in es], [e["packed"] for e in es],
                                               [e["s16"] for e in es], outs=[e["y1"] for e in es]))
        return plans

    def decode_graph(self):
        """The per-phase decode pass captured once in a HIP graph (a decoder replays it per token)."""
        import torch

        if self._decode_graph is None:
            plans = self.decode_plans()
            for p in plans:
                p()
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for p in plans:
                    p()
            self._decode_graph = (graph, plans)
        return self._decode_graph[0]


def run_step(stack, events):
    """One step; when `events` is a dict, each launch is bracketed by two HIP events."""
    import torch

    def timed(fam, work, fn):
        if events is None:
            fn()
            return
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        events.setdefault(fam, []).append((e0, e1, work))

    for layer in range(stack.layers):
        for fam, work, fn in stack.layer_launches(layer):
            timed(fam, work, fn)
    graph = stack.decode_graph()
    timed("decode_pass", stack.decode_bytes, graph.replay)


def components(stack, dev, peaks, reps=5):
    """Measurements outside the step: the prefill product on exact weights beside the step's
    dequantizing one, the decode pass in other launch orders, single launches of the largest
    shapes, and the rows beyond the step."""
    import torch
    import w4a16_group_wise_amd as w4q

    def median_us(fn, n=reps):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(n):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        return float(np.median(ts))

    out = {}
    # prefill on each distinct shape of layer 0: bf16-dequantized weights (the step's) and exact ones
    per = stack.lin[0]
    xs = stack.x[0]
    dq = {}
    for name in ("q", "k", "gate", "down"):
        e = per[name]
        lin = e["lin"]
        xt = xs[lin.inp][:PREFILL_M]
        y = stack.view(stack.y_pre, PREFILL_M, lin.d_out)
        fl = 2 * PREFILL_M * lin.d_out * lin.d_in
        t_dq = median_us(lambda: w4q.w4a16_gemm_dq(xt, e["packed"], e["s16"], out=y, workspace=stack.ws))
        t_ex = median_us(lambda: w4q.w4a16_gemm(xt, e["packed"], e["s16"], out=y, workspace=stack.ws))
        dq[f"{lin.d_out}x{lin.d_in}"] = {"gemm_dq_us": round(t_dq, 1),
                                          "gemm_dq_frac_bf16": round(fl / (t_dq * 1e-6) / (PEAK_BF16_TFLOPS * 1e12), 4),
                                          "gemm_exact_us": round(t_ex, 1),
                                          "gemm_exact_frac_bf16": round(fl / (t_ex * 1e-6) / (PEAK_BF16_TFLOPS * 1e12), 4)}
    out["prefill_m2048_per_shape"] = dq
    # the decode pass in other orders (all 252 linears, weights far beyond the Infinity Cache)
    plans = stack.decode_plans()
    flat = [(e, stack.x[layer][e["lin"].inp][:1]) for layer in range(stack.layers) for e in stack.lin[layer].values()]
    whole = w4q.GemvGroupPlan([x for _, x in flat], [e["packed"] for e, _ in flat], [e["s16"] for e, _ in flat],
                              outs=[e["y1"] for e, _ in flat])

    def singles():
        for e, x in flat:
            w4q.w4a16_gemm(x, e["packed"], e["s16"], out=e["y1"])

    def per_phase():
        for p in plans:
            p()

    B = stack.decode_bytes
    for name, fn in (("one_call_per_linear", singles), ("grouped_per_phase_host", per_phase),
                     ("grouped_per_phase_graph", stack.decode_graph().replay), ("grouped_whole_pass", whole)):
        us = median_us(fn)
        out.setdefault("decode_pass", {})[name] = {"us": round(us, 1), "GBps": round(B / (us * 1e-6) / 1e9, 1),
                                                   "frac_hbm": round(B / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    out["decode_pass"]["bytes"] = B
    out["decode_pass"]["linears"] = len(flat)
    # the ceiling of the per-phase launch structure: the same dependent launches (phase sizes, in
    # a graph) done by a plain streaming read of the library's read probe
    phase_bytes = []
    for layer in range(stack.layers):
        per = stack.lin[layer]
        for names in (("q", "k", "v"), ("o",), ("gate", "up"), ("down",)):
            nb = sum(per[nm]["packed"].numel() + 2 * per[nm]["s16"].numel() for nm in names)
            phase_bytes.append((nb + 15) // 16 * 16)
    buf = torch.empty(sum(phase_bytes), dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.empty(65536, dtype=torch.int32, device=dev)
    offs = np.cumsum([0] + phase_bytes[:-1])
    views = [buf[o:o + b] for o, b in zip(offs, phase_bytes)]

    def reads():
        for v in views:
            w4q.probe_read(v, nontemporal=True, sink=sink)

    reads()
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        reads()
    us = median_us(gr.replay)
    out["decode_pass"]["per_phase_read_floor"] = {
        "us": round(us, 1), "frac_hbm": round(sum(phase_bytes) / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
        "how": "144 dependent streaming reads (w4q_probe_read, non-temporal) of the phase sizes, graph-replayed"}
    del buf, views
    torch.cuda.empty_cache()
    # one M = 1 launch of the largest weight (gate 12288x4096, 28 MB)
    e = per["gate"]
    us = median_us(lambda: w4q.w4a16_gemm(xs["mlp"][:1], e["packed"], e["s16"], out=e["y1"]), n=20)
    gb = gemv_bytes(12288, 4096)
    out["gemv_single_12288x4096"] = {"us": round(us, 2), "frac_hbm": round(gb / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    out["next_rows"] = next_rows(stack, dev, median_us, peaks)
    return out


def next_rows(stack, dev, median_us, peaks):
    """The rows beyond the step, each on one full-size shape of layer 0: the per-channel search,
    the joint objective's coordinate descent and GPTQ on the q projection (4096x4096, its 8192-token
    H, K = 40), and the fused LSQ + Adam update on the gate weight (12288x4096).  Rates are
    algorithmic work over the median duration; the fp64 work is priced against the nominal fp64
    peak and against the fp64 matrix-core rate measured in the same job."""
    import torch
    import w4a16_group_wise_amd as w4q

    per, xs = stack.lin[0], stack.x[0]
    e = per["q"]
    lin = e["lin"]
    n, k = lin.d_out, lin.d_in
    K = stack.K
    h = w4q.quant_hessian(xs[lin.inp], workspace=stack.ws)
    w4q.quant_scale_search(e["w"], h, stack.alpha, out=(e["scale"], e["idx"], e["obj"], None))
    fp64 = PEAK_FP64_TFLOPS * 1e12
    mf64 = peaks["mfma_f64"]
    res = {}
    # per-channel: K candidates x (E H) over the row, 2 K d_in^2 flop per row
    t = median_us(lambda: w4q.quant_scale_search_pc(e["w"], h, stack.alpha), n=3)
    fl = 2.0 * n * K * k * k
    res["scale_search_pc_4096x4096"] = {"us": round(t, 1), "fp64_TFLOPs": round(fl / (t * 1e-6) / 1e12, 3),
                                        "frac_fp64": round(fl / (t * 1e-6) / fp64, 4),
                                        "frac_of_measured_fp64": round(fl / (t * 1e-6) / mf64, 4)}
    # joint: U = E H (2 d_out d_in^2 flop) and the descent; the objective ratio it reached
    ws = torch.empty(w4q.workspace_size("joint", n, k), dtype=torch.uint8, device=dev)
    t_obj = median_us(lambda: w4q.quant_joint_objective(e["w"], e["scale"], h, workspace=ws), n=3)
    res_ref = {}

    def refine():
        res_ref["r"] = w4q.quant_joint_refine(e["w"], h, stack.alpha, e["idx"], n_sweeps=2, workspace=ws)

    t_ref = median_us(refine, n=3)
    _, _, ob, oa, sw = res_ref["r"]
    fl = 2.0 * n * k * k
    res["joint_4096x4096"] = {"objective_us": round(t_obj, 1),
                              "objective_fp64_TFLOPs": round(fl / (t_obj * 1e-6) / 1e12, 3),
                              "objective_frac_fp64": round(fl / (t_obj * 1e-6) / fp64, 4),
                              "objective_frac_of_measured_fp64": round(fl / (t_obj * 1e-6) / mf64, 4),
                              "refine_2_sweeps_us": round(t_ref, 1),
                              "objective_after_over_before": round(float((oa / ob).mean().item()), 5),
                              "rows_converged": int((sw < 2).sum().item())}
    # GPTQ: Cholesky (d^3 / 3 flop) and the feedback sums (d_out d_in^2 flop)
    wsg = torch.empty(w4q.workspace_size("gptq", n, k), dtype=torch.uint8, device=dev)
    t = median_us(lambda: w4q.quant_gptq(e["w"], h, e["scale"], workspace=wsg), n=3)
    fl = k ** 3 / 3.0 + 1.0 * n * k * k
    res["gptq_4096x4096"] = {"us": round(t, 1), "fp64_TFLOPs": round(fl / (t * 1e-6) / 1e12, 3),
                             "frac_fp64": round(fl / (t * 1e-6) / fp64, 4),
                             "frac_of_measured_fp64": round(fl / (t * 1e-6) / mf64, 4)}
    del ws, wsg
    # fused LSQ + Adam on the gate weight (parameters and moments updated in place, next forward)
    g = per["gate"]
    gn, gk = g["lin"].d_out, g["lin"].d_in
    wc, sc = g["w"].clone(), g["scale"].clone()
    mw, vw = torch.zeros_like(wc), torch.zeros_like(wc)
    ms, vs = torch.zeros_like(sc), torch.zeros_like(sc)
    t = median_us(lambda: w4q.lsq_adam_step(wc, sc, g["g"], GS, mw, vw, ms, vs, lr_w=1e-5, lr_s=1e-6, step=1,
                                            with_w_hat_next=True), n=5)
    nb = gn * gk * 32 + gn * gk // 32 * 24      # w, m_w, v_w read+written, g read, w_hat written
    res["lsq_adam_12288x4096"] = {"us": round(t, 1), "GBps": round(nb / (t * 1e-6) / 1e9, 1),
                                  "frac_hbm": round(nb / (t * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    return res


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(budget_s=20.0):
    """The oracle (as it is, untuned) on a bounded sample of the same workload, on the host cores:
    the decode product of one gate linear (12288x4096) repeated for about a quarter of the
    budget, the search on 65536 groups of it, a 256-column slab of an 8192x4096 Hessian, pack and
    LSQ on 4M weights, and the prefill product on 16 output columns.  The inputs are the host
    (numpy) draws of the same recipe."""
    import oracle
    from w4a16_group_wise_amd import synth

    c = synth.WORKLOADS[WORKLOAD]
    lin = [l for l in c.linears if l.name == "gate"][0]
    w = c.weight(0, lin)
    x = c.x(0, lin.inp)
    alpha = c.alpha()
    G = lin.d_in // 32
    rates, t_step = {}, 0.0

    def timed(fn):
        t0 = time.perf_counter()
        r = fn()
        return time.perf_counter() - t0, r

    # Hessian: 256-column slab (unique entries) -> flop/s
    ij = np.stack(np.meshgrid(np.arange(256), np.arange(256), indexing="ij"), -1).reshape(-1, 2)
    ij = ij[ij[:, 0] <= ij[:, 1]]
    th, _ = timed(lambda: oracle.hessian_entries(x, ij))
    rates["hessian_GFLOPs"] = ij.shape[0] * 2 * x.shape[0] / th / 1e9
    # search on the first 65536 groups (needs the H blocks of those groups: the slab covers the
    # first 8 group columns; the rest of H is computed on the GPU's shapes only for its blocks)
    rows = 65536 // G
    h = np.zeros((lin.d_in, lin.d_in), np.float32)
    for g0 in range(G):
        blk = np.stack(np.meshgrid(np.arange(32 * g0, 32 * g0 + 32), np.arange(32 * g0, 32 * g0 + 32),
                                   indexing="ij"), -1).reshape(-1, 2)
        h[blk[:, 0], blk[:, 1]] = oracle.hessian_entries(x, blk)
    ts, (sc, _, _, _) = timed(lambda: oracle.scale_search(w[:rows], h, alpha))
    rates["search_groups_per_s"] = rows * G / ts
    # pack and LSQ on the first 4M weights
    r4 = (4 << 20) // lin.d_in
    scale = np.abs(w[:r4].reshape(r4, G, 32)).max(axis=2).astype(np.float32) / 7
    tp, (packed, s16) = timed(lambda: oracle.pack(w[:r4], scale))
    gr = c.grad(0, lin)[:r4]
    tl, _ = timed(lambda: oracle.lsq_bwd(w[:r4], scale, gr, GS))
    rates["pack_GBps"] = r4 * lin.d_in * 4.5 / tp / 1e9
    rates["lsq_bwd_GBps"] = r4 * lin.d_in * 16 / tl / 1e9
    # decode product over all rows of the packed gate weight, repeated
    scale_all = np.abs(w.reshape(lin.d_out, G, 32)).max(axis=2).astype(np.float32) / 7
    packed_all, s16_all = oracle.pack(w, scale_all)
    reps, t = 0, 0.0
    while t < budget_s * 0.25 or reps < 1:
        dt, _ = timed(lambda: oracle.gemm_cols(x[:1], packed_all, s16_all))
        t += dt
        reps += 1
    decode_gbps = gemv_bytes(lin.d_out, lin.d_in) * reps / t / 1e9
    rates["decode_GBps"] = decode_gbps
    # prefill on 16 output columns
    tg, _ = timed(lambda: oracle.gemm_cols(x[:PREFILL_M], packed_all, s16_all, np.arange(16), dequant_bf16=True))
    rates["prefill_GFLOPs"] = 2 * PREFILL_M * 16 * lin.d_in / tg / 1e9
    # the whole step extrapolated from these rates over the stack's work
    wl = synth.WORKLOADS[WORKLOAD]
    n_w = sum(l.d_out * l.d_in for l in wl.linears) * wl.layers
    hess = sum(wl.n_tok * d * (d + 1) for d in wl.inputs().values()) * wl.layers
    t_step = (hess / (rates["hessian_GFLOPs"] * 1e9) + n_w / 32 / rates["search_groups_per_s"]
              + n_w * 4.5 / (rates["pack_GBps"] * 1e9)
              + 2 * 12288 * 4096 * wl.layers * 24 / (rates["lsq_bwd_GBps"] * 1e9)
              + 2 * PREFILL_M * n_w / (rates["prefill_GFLOPs"] * 1e9)
              + sum(gemv_bytes(l.d_out, l.d_in) for l in wl.linears) * wl.layers / (decode_gbps * 1e9))
    return dict(value=round(decode_gbps, 3), unit="GB/s", cores=oracle.threads(), kind="oracle",
                cpu_model=cpu_model(),
                sample=(f"decode product of one 12288x4096 gate linear x{reps}; search on {rows * G} groups; "
                        f"Hessian {ij.shape[0]} entries of a 256-col slab (8192 tokens); pack/LSQ on {r4 * lin.d_in} "
                        f"weights; prefill M={PREFILL_M} on 16 cols"),
                rates={k: round(v, 3) for k, v in rates.items()},
                step_s_extrapolated=round(t_step, 1))


def traffic_for(kernel):
    """HBM bytes per launch (mean over the family's launches in a step) from the committed
    counters, if the kernel source is unchanged since they were taken."""
    p = os.path.join(ROOT, "profiles", f"traffic_{WORKLOAD}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    k = t.get("kernels", {}).get(kernel)
    if not k or k.get("src_hash") != src_hash(KERNELS[kernel][0]):
        return None
    return k.get("bytes_per_launch")


def run(args):
    import torch
    import w4a16_group_wise_amd as w4q

    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 (how the path "
                          "would shard over several GPUs is described, not built)"}))
        sys.exit(2)
    dev = torch.device("cuda:0")
    print(f"[bench] drawing the {args.layers}-layer stack on the GPU", file=sys.stderr, flush=True)
    stack = Stack(dev, args.layers)
    torch.cuda.synchronize()
    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        run_step(stack, None)
    torch.cuda.synchronize()
    # the timed region: exactly `steps` passes, host clock, synchronised on both sides; every
    # launch between two HIP events on the current stream (the library's launch stream)
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    events = {}
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run_step(stack, events)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    fam_info = {
        "hessian": ("flop", "mfma", PEAK_BF16_TFLOPS * 1e12),
        "scale_search": ("flop", "alu", PEAK_FP32_VALU_TFLOPS * 1e12),
        "pack": ("byte", "hbm", PEAK_HBM_GBS * 1e9),
        "lsq_fwd": ("byte", "hbm", PEAK_HBM_GBS * 1e9),
        "lsq_bwd": ("byte", "hbm", PEAK_HBM_GBS * 1e9),
        "prefill_gemm": ("flop", "mfma", PEAK_BF16_TFLOPS * 1e12),
        "decode_pass": ("byte", "hbm", PEAK_HBM_GBS * 1e9),
    }
    print("[bench] measured peaks", file=sys.stderr, flush=True)
    peaks = measured_peaks(dev)
    kernels = {}
    total_us = 0.0
    for fam, lst in events.items():
        durs = np.array([a.elapsed_time(b) * 1e3 for a, b, _ in lst])
        work = float(sum(w for _, _, w in lst))
        unit, bound, peak = fam_info[fam]
        rate = work / (durs.sum() * 1e-6)
        scale = 1e9 if unit == "byte" else 1e12
        kernels[fam] = dict(launches_per_step=len(lst) // args.steps, us_per_step=round(durs.sum() / args.steps, 1),
                            mean_launch_us=round(float(durs.mean()), 3),
                            work_per_launch=work / len(lst), work_unit=unit, bound=bound,
                            achieved=round(rate / scale, 3), peak=round(peak / scale, 1),
                            rate_unit="GB/s" if unit == "byte" else "TFLOP/s", frac=round(rate / peak, 4))
        mp = peaks["hbm"] if bound == "hbm" else (peaks["mfma"] if bound == "mfma" else None)
        if mp:
            kernels[fam]["frac_of_measured_peak"] = round(rate / mp, 4)
        total_us += durs.sum() / args.steps
    for k in kernels.values():
        k["share_of_step"] = round(k["us_per_step"] / total_us, 4)
    dom = max((f for f in kernels if f != "decode_pass"), key=lambda f: kernels[f]["us_per_step"])
    d = kernels[dom]
    roof = {"kernel": dom, "bound": d["bound"], "achieved": d["achieved"], "peak": d["peak"],
            "unit": d["rate_unit"], "frac": d["frac"], "traffic": traffic_for(dom),
            "launch_us": d["mean_launch_us"], "algorithmic_per_launch": d["work_per_launch"],
            "algorithmic_unit": d["work_unit"]}
    dp = kernels["decode_pass"]
    c = stack.c
    out = {
        "metric": METRIC, "value": dp["achieved"], "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16+fp32",
        "data": "synthetic (seeded, drawn on the GPU; see w4a16_group_wise_amd/synth.py)",
        "config": {"workload": f"{WORKLOAD}: 36-layer decoder stack at hidden 4096 (q, o 4096x4096; k, v "
                               f"1024x4096; gate, up 12288x4096; down 4096x12288; 252 linears); X 8192 tok "
                               f"bf16 per layer input; K=40, alpha in [0.4,1.0]; LSQ on gate/up; prefill "
                               f"M={PREFILL_M}; decode M=1 per-phase grouped, graph-replayed",
                   "layers": args.layers, "linears": args.layers * len(c.linears), "n_tok": c.n_tok,
                   "n_cand": c.n_cand, "prefill_m": PREFILL_M, "parallelism": "single GPU"},
        "roofline": roof,
        "value_detail": {"decode_pass_us": round(dp["mean_launch_us"], 1), "bytes": stack.decode_bytes,
                         "frac_hbm": dp["frac"]},
        "measured_peaks": {"hbm_read_GBps": round(peaks["hbm"] / 1e9, 1),
                           "mfma_bf16_TFLOPs": round(peaks["mfma"] / 1e12, 1),
                           "mfma_f64_TFLOPs": round(peaks["mfma_f64"] / 1e12, 1),
                           "how": "w4q_probe_read (non-temporal) over 2 GiB, w4q_probe_mfma_bf16 and "
                                  "w4q_probe_mfma_f64, best of 5, HIP events"},
        "timing": "timed region: HIP events around every launch on its stream; per family, sum of "
                  "algorithmic work / sum of launch durations",
        "kernels": kernels,
        "components": {"search_groups_per_s": round(
            sum(l.d_out * l.d_in // 32 for l in c.linears) * args.layers / (kernels["scale_search"]["us_per_step"] * 1e-6), 1)},
    }
    if not args.no_components:
        print("[bench] components", file=sys.stderr, flush=True)
        out["components"].update(components(stack, dev, peaks))
    del stack
    torch.cuda.empty_cache()
    if not args.no_cpu:
        print("[bench] cpu baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out))


def pmc_summary(args):
    """Per-kernel FETCH_SIZE / WRITE_SIZE (KiB per dispatch) -> bytes per launch (mean over the
    family's dispatches), scaled by the reading of torch's plain copy of a known size that
    bench.py --pmc-copy runs; with a third directory, the matrix-core busy counters."""
    import csv
    import glob

    def read(dirn, counter):
        rows = {}
        for f in glob.glob(os.path.join(dirn, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    if r.get("Counter_Name") != counter:
                        continue
                    rows.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return rows

    def mean_of(rows, keys):
        """Sum over the launch's kernels of each kernel's mean per dispatch."""
        tot, found = 0.0, False
        for key in keys:
            pat = re.compile(r"\b" + re.escape(key) + r"\b")
            vals = [v for k, vs in rows.items() if pat.search(k) for v in vs]
            if vals:
                tot += float(np.mean(vals))
                found = True
        return tot if found else None

    fetch = read(args.pmc_summary[0], "FETCH_SIZE")
    write = read(args.pmc_summary[1], "WRITE_SIZE")
    copy_bytes = float(args.copy_bytes)
    cf = mean_of(fetch, ["neg_kernel_cuda"])
    cw = mean_of(write, ["neg_kernel_cuda"])
    f_scale = copy_bytes / (cf * 1024) if cf else 1.0
    w_scale = copy_bytes / (cw * 1024) if cw else 1.0
    res = {"workload": WORKLOAD, "copy_bytes": copy_bytes, "fetch_scale": f_scale, "write_scale": w_scale,
           "kernels": {}}
    for name, (src, keys) in KERNELS.items():
        fk = mean_of(fetch, keys)
        wk = mean_of(write, keys)
        if fk is None or wk is None:
            continue
        res["kernels"][name] = {"fetch_kib": fk, "write_kib": wk,
                                "bytes_per_launch": fk * 1024 * f_scale + wk * 1024 * w_scale,
                                "src_hash": src_hash(src)}
    # a family's launches differ in shape: these are means per dispatch over one step's launches,
    # comparable with the mean algorithmic work per launch the bench reports
    if len(args.pmc_summary) > 2:
        # matrix cores: SQ_INSTS_VALU_MFMA_MOPS_* count matrix operations in units of 512 flop;
        # SQ_VALU_MFMA_BUSY_CYCLES / GRBM_GUI_ACTIVE is normalised by the same ratio read for the
        # probe kernel of the same job, which issues independent products back to back on every
        # SIMD (busy fraction 1 by construction)
        mdir = args.pmc_summary[2]
        mops_bf16 = read(mdir, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
        mops_f16 = read(mdir, "SQ_INSTS_VALU_MFMA_MOPS_F16")
        busy = read(mdir, "SQ_VALU_MFMA_BUSY_CYCLES")
        gui = read(mdir, "GRBM_GUI_ACTIVE")
        pb, pg = mean_of(busy, ["mfma_kernel"]), mean_of(gui, ["mfma_kernel"])
        norm = pb / pg if pb and pg else None
        res["mfma_probe"] = {"busy_cycles": pb, "gui_active": pg,
                             "mops_bf16_flop": (mean_of(mops_bf16, ["mfma_kernel"]) or 0) * 512}
        for name, (src, keys) in KERNELS.items():
            b, gact = mean_of(busy, keys), mean_of(gui, keys)
            if b is None or gact is None:
                continue
            ent = res["kernels"].setdefault(name, {"src_hash": src_hash(src)})
            ent["mfma_busy_cycles"] = b
            ent["gui_active"] = gact
            ent["mfma_bf16_flop_issued"] = (mean_of(mops_bf16, keys) or 0) * 512
            ent["mfma_f16_flop_issued"] = (mean_of(mops_f16, keys) or 0) * 512
            if norm:
                ent["mfma_busy_frac"] = b / gact / norm
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    p = os.path.join(ROOT, "profiles", f"traffic_{WORKLOAD}.json")
    with open(p, "w") as f:
        json.dump(res, f, indent=1)
    print(p)


def pmc_copy(args):
    """A plain streaming kernel of known size (b = -a: reads and writes copy_bytes each), to
    calibrate the byte counters."""
    import torch

    n = int(args.copy_bytes) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(3):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    print("copy done", n * 4)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--layers", type=int, default=36, help="layers of the stack (36; fewer for profiling runs)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-components", action="store_true")
    ap.add_argument("--pmc-summary", nargs="+", metavar="DIR")
    ap.add_argument("--pmc-copy", action="store_true")
    ap.add_argument("--copy-bytes", type=float, default=float(1 << 30))
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(args)
    elif args.pmc_copy:
        pmc_copy(args)
    else:
        run(args)


if __name__ == "__main__":
    main()
