"""Bench: one full quantized MoE expert step (forward, data gradient and
weight gradient of both expert linears) through libmx355 on one MI355X.

Workload (synthetic, seeded, resident in HBM before timing): 32 experts,
d_model 2880, expert FFN 2880 (gate_up 2880 -> 5760, down 2880 -> 2880),
16384 tokens routed top-4 with Zipf(1.1) counts (65,536 assignments).  One
step runs, in order:
  Q2D(W1), Q2D(W2)                 32x32 RTNE, both layouts (fprop and dgrad)
  Q1D(X) RTNE -> GEMM  Y1 = X W1   (rows gathered by routing), bf16 out
  Q1D(h) RTNE -> GEMM  Y2 = h W2   bf16 out
  Q1D(dY2) SR -> GEMM dh = dY2 W2^T ; Q1D(dY1) SR -> GEMM dX = dY1 W1^T
  Qcol(h), Qcol(dY2) RHT+SR -> GEMM dW2 = h^T dY2   (groups split K), fp32 out
  Qcol(X), Qcol(dY1) RHT+SR -> GEMM dW1 = X^T dY1   fp32 out
The metric is BASELINE's pair: quantize GB/s and grouped-GEMM TFLOP/s, each
as a fraction of its MI355X roofline; `value` is the whole step's algorithmic
GEMM FLOPs divided by the step time.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_traffic.txt")
# kernel-name prefix (template arguments without spaces) of each GEMM role:
# bf16 output with 2D weight scales, fp32 output with 1D scales
# kernel-name prefixes of each role's launches (the last template argument,
# the quantizing epilogue, is off in the step)
ROLE_KERNEL = {"gemm": "gemm_kernel<true,true,", "gemm_wgrad": "gemm_kernel<false,false,true,"}
PEAK_FP4_TFLOPS = 10100.0      # MI355X dense FP4 MFMA, TFLOP/s
E, D, F2, T, TOPK = 32, 2880, 5760, 16384, 4
ROWS = T * TOPK


def build_inputs(torch, dev):
    """Synthetic tensors on the device.  Distributions follow the workload
    recipe: activations N(0,1) x per-column log-uniform[0.1, 10] (seed 1),
    weights N(0, 0.02), the down-projection input h N(0,1), upstream
    gradients N(0, 1e-3) (seed 5).  Drawn with torch's device generator."""
    from mxfp4_precision_numerics_amd import synth
    g1 = torch.Generator(device=dev).manual_seed(1)
    g5 = torch.Generator(device=dev).manual_seed(5)
    c = torch.exp(torch.empty(D, device=dev).uniform_(math.log(0.1), math.log(10.0), generator=g1))
    X = (torch.randn(T, D, device=dev, generator=g1) * c).to(torch.bfloat16)
    counts = synth.zipf_counts()
    off = synth.offsets_from_counts(counts)
    idx = synth.routing_row_index(counts)
    W1 = (torch.randn(E, D, F2, device=dev, generator=g5) * 0.02).to(torch.bfloat16)
    W2 = (torch.randn(E, D, D, device=dev, generator=g5) * 0.02).to(torch.bfloat16)
    h = torch.randn(ROWS, D, device=dev, generator=g5).to(torch.bfloat16)
    dY1 = (torch.randn(ROWS, F2, device=dev, generator=g5) * 1e-3).to(torch.bfloat16)
    dY2 = (torch.randn(ROWS, D, device=dev, generator=g5) * 1e-3).to(torch.bfloat16)
    idx_d = torch.from_numpy(idx).to(dev)
    pad = (counts + 31) // 32 * 32
    poff = np.concatenate([[0], np.cumsum(pad)]).astype(np.int32)
    return dict(X=X, W1=W1, W2=W2, h=h, dY1=dY1, dY2=dY2, counts=counts,
                off=torch.from_numpy(off).to(dev), idx=idx_d,
                poff=torch.from_numpy(poff).to(dev), kp_used=int(poff[-1]))


class Step:
    """All buffers are allocated once; run() only launches kernels."""

    def __init__(self, torch, dev, inp):
        from mxfp4_precision_numerics_amd import mx
        self.mx, self.torch, self.inp = mx, torch, inp
        u8, bf, f32 = torch.uint8, torch.bfloat16, torch.float32
        z = lambda *s, dt=u8: torch.empty(*s, dtype=dt, device=dev)  # noqa: E731

        def zc(*s):
            # code rows padded to whole 128-byte lines (the GEMM reads each
            # operand row as whole lines); a view of the row's bytes
            return z(*s[:-1], (s[-1] + 127) // 128 * 128)[..., :s[-1]]

        self.kp = mx.padded_capacity(ROWS, E)
        self.mask = mx.rht_sign_mask(5)
        self.b = dict(
            w1c=zc(E, D, F2 // 2), w1s=z(E, D // 32, F2 // 32), w1tc=zc(E, F2, D // 2),
            w1ts=z(E, F2 // 32, D // 32),
            w2c=zc(E, D, D // 2), w2s=z(E, D // 32, D // 32), w2tc=zc(E, D, D // 2), w2ts=z(E, D // 32, D // 32),
            xc=zc(T, D // 2), xs=z(T, D // 32), hc=zc(ROWS, D // 2), hs=z(ROWS, D // 32),
            g2c=zc(ROWS, D // 2), g2s=z(ROWS, D // 32), g1c=zc(ROWS, F2 // 2), g1s=z(ROWS, F2 // 32),
            hTc=z(D, self.kp // 2), hTs=z(D, self.kp // 32), g2Tc=z(D, self.kp // 2), g2Ts=z(D, self.kp // 32),
            xTc=z(D, self.kp // 2), xTs=z(D, self.kp // 32), g1Tc=z(F2, self.kp // 2), g1Ts=z(F2, self.kp // 32),
            Y1=z(ROWS, F2, dt=bf), Y2=z(ROWS, D, dt=bf), dh=z(ROWS, D, dt=bf), dX=z(ROWS, D, dt=bf),
            dW2=z(E, D, D, dt=f32), dW1=z(E, D, F2, dt=f32),
        )
        self.events = None

    def _t(self, name, fn):
        if self.events is None:
            fn()
            return
        s = self.torch.cuda.Event(enable_timing=True)
        e = self.torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        self.events.append((name, s, e))

    def run(self):
        mx, b, i = self.mx, self.b, self.inp
        m = self.mask
        off, poff, idx = i["off"], i["poff"], i["idx"]
        self._t("q2d", lambda: mx.quantize_2d_into(i["W1"], b["w1c"], b["w1s"], b["w1tc"], b["w1ts"]))
        self._t("q2d", lambda: mx.quantize_2d_into(i["W2"], b["w2c"], b["w2s"], b["w2tc"], b["w2ts"]))
        self._t("q1d_row", lambda: mx.quantize_1d(i["X"], codes=b["xc"], scales=b["xs"]))
        self._t("gemm", lambda: mx.grouped_gemm(b["xc"], b["xs"], b["w1tc"], b["w1ts"], off, ROWS, F2, D,
                                                a_row_index=idx, b_scale_2d=True, out=b["Y1"]))
        self._t("q1d_row", lambda: mx.quantize_1d(i["h"], codes=b["hc"], scales=b["hs"]))
        self._t("gemm", lambda: mx.grouped_gemm(b["hc"], b["hs"], b["w2tc"], b["w2ts"], off, ROWS, D, D,
                                                b_scale_2d=True, out=b["Y2"]))
        self._t("q1d_row", lambda: mx.quantize_1d(i["dY2"], rnd=mx.SR, seed=5, stream_id=1,
                                                  codes=b["g2c"], scales=b["g2s"]))
        self._t("gemm", lambda: mx.grouped_gemm(b["g2c"], b["g2s"], b["w2c"], b["w2s"], off, ROWS, D, D,
                                                b_scale_2d=True, out=b["dh"]))
        self._t("q1d_row", lambda: mx.quantize_1d(i["dY1"], rnd=mx.SR, seed=5, stream_id=0,
                                                  codes=b["g1c"], scales=b["g1s"]))
        self._t("gemm", lambda: mx.grouped_gemm(b["g1c"], b["g1s"], b["w1c"], b["w1s"], off, ROWS, D, F2,
                                                b_scale_2d=True, out=b["dX"]))
        col = dict(block_axis=0, group_offsets=off, kp=self.kp, use_rht=True, sign_mask=m, rnd=mx.SR, seed=5)
        self._t("q1d_col", lambda: mx.quantize_1d(i["h"], stream_id=4, codes=b["hTc"], scales=b["hTs"], **col))
        self._t("q1d_col", lambda: mx.quantize_1d(i["dY2"], stream_id=5, codes=b["g2Tc"], scales=b["g2Ts"], **col))
        self._t("gemm_wgrad", lambda: mx.grouped_gemm(b["hTc"], b["hTs"], b["g2Tc"], b["g2Ts"], poff, D, D, self.kp,
                                                      group_dim_k=True, out=b["dW2"]))
        # X^T: the routed rows are gathered from the 16384-token X inside the
        # quantizer (no permuted copy)
        self._t("q1d_col", lambda: mx.quantize_1d(i["X"], stream_id=2, codes=b["xTc"], scales=b["xTs"],
                                                  row_index=idx, **col))
        self._t("q1d_col", lambda: mx.quantize_1d(i["dY1"], stream_id=3, codes=b["g1Tc"], scales=b["g1Ts"], **col))
        self._t("gemm_wgrad", lambda: mx.grouped_gemm(b["xTc"], b["xTs"], b["g1Tc"], b["g1Ts"], poff, D, F2, self.kp,
                                                      group_dim_k=True, out=b["dW1"]))


def work_model():
    """Algorithmic work per role in one step (bytes moved at minimum, or
    FLOPs): 1D quantize from bf16 = 2 + 1/2 + 1/32 B per element; 2D with both
    layouts = 2 + 1/2 + 1/2 + 2/1024 B per element; GEMM = 2 M N K with the
    real (unpadded) token count."""
    el_row = T * D + ROWS * D + ROWS * D + ROWS * F2
    el_col = ROWS * D * 3 + ROWS * F2
    el_2d = E * D * F2 + E * D * D
    return {
        "q1d_row": {"bytes": el_row * (2 + 0.5 + 1 / 32), "launches": 4},
        "q1d_col": {"bytes": el_col * (2 + 0.5 + 1 / 32), "launches": 4},
        "q2d": {"bytes": el_2d * (2 + 0.5 + 0.5 + 2 / 1024), "launches": 2},
        "gemm": {"flops": 2.0 * ROWS * (D * F2 + D * D + D * D + F2 * D), "launches": 4},
        "gemm_wgrad": {"flops": 2.0 * ROWS * (D * D + D * F2), "launches": 2},
    }


def kernel_source_hash():
    """sha256 over the sources the GEMM kernel is compiled from."""
    import hashlib
    h = hashlib.sha256()
    for rel in ("mxfp4_precision_numerics_amd/csrc/mx_gemm.hip",
                "mxfp4_precision_numerics_amd/csrc/mx_device.h", "include/mx.h"):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(role):
    """HBM bytes per launch (scaled FETCH_SIZE + WRITE_SIZE) recorded for this
    role's kernel, or None when no record exists or the kernel's sources have
    changed since the counters were taken."""
    if role not in ROLE_KERNEL or not os.path.exists(TRAFFIC_FILE):
        return None
    src, rec = None, {}
    for line in open(TRAFFIC_FILE):
        f = line.split()
        if len(f) >= 2 and f[0] == "source_sha256":
            src = f[1]
        elif len(f) >= 6 and f[0] == "kernel":
            calls = float(f[7]) if len(f) >= 8 and f[6] == "calls" else 1.0
            rec[f[1]] = (float(f[3]), float(f[5]), calls)
    # a role may launch several instantiations (e.g. with and without a row
    # gather): average over all of its dispatches
    names = [k for k in rec if k.startswith(ROLE_KERNEL[role]) and k.endswith(",false>")]
    if src != kernel_source_hash() or not names:
        return None
    n = sum(rec[k][2] for k in names)
    rd = sum(rec[k][0] * rec[k][2] for k in names) / n
    wr = sum(rec[k][1] * rec[k][2] for k in names) / n
    return {"read_bytes": rd, "write_bytes": wr, "bytes": rd + wr}


def fused_epilogue(torch, step, reps=5):
    """The quantizing epilogue on the second expert linear's forward GEMM
    (65536 x 2880 x 2880): its bf16 output quantized row-wise (1x32, RTNE) as
    the next MXFP4 GEMM's operand.  Times the GEMM followed by the 1D
    quantizer against the fused call, with and without the bf16 output.
    Measured after the timed steps, on the step's own buffers."""
    mx, b, i = step.mx, step.b, step.inp
    args = (b["hc"], b["hs"], b["w2tc"], b["w2ts"], i["off"], ROWS, D, D)
    runs = {
        "gemm_then_quantize_ms": lambda: (mx.grouped_gemm(*args, b_scale_2d=True, out=b["Y2"]),
                                          mx.quantize_1d(b["Y2"], codes=b["g2c"], scales=b["g2s"])),
        "fused_ms": lambda: mx.grouped_gemm_q(*args, b_scale_2d=True, out=b["Y2"], codes=b["g2c"],
                                              scales=b["g2s"]),
        "fused_mxfp4_only_ms": lambda: mx.grouped_gemm_q(*args, b_scale_2d=True, with_bf16=False,
                                                         codes=b["g2c"], scales=b["g2s"]),
    }
    res = {"shape": "%dx%dx%d" % (ROWS, D, D)}
    for name, fn in runs.items():
        for _ in range(2):
            fn()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        res[name] = s.elapsed_time(e) / reps
    return res


def cpu_baseline(gemm_seconds=8.0):
    """The oracle, untuned, on a bounded sample of the same step; its rate per
    role is extrapolated to the full step.  The quantizers run on fixed
    slices; the FP64 GEMM runs batches of sampled output rows (full N, full K)
    until about `gemm_seconds` have passed."""
    import oracle
    from mxfp4_precision_numerics_amd import synth
    threads = oracle.default_threads()
    rng = np.random.default_rng(0)
    rows = 4096
    xs = synth.channel_scaled_activations(rows=rows, cols=D, seed=1)
    gs = synth.normal_bf16((rows, F2), 1e-3, seed=5)
    w = work_model()
    per_el = 2 + 0.5 + 1 / 32
    timings = {}
    # row-wise RTNE and SR quantize: time per element
    t0 = time.perf_counter()
    oracle.quantize_1d(xs)
    oracle.quantize_1d(gs, rnd=oracle.SR, seed=5)
    dt = time.perf_counter() - t0
    timings["q1d_row"] = dt / (rows * (D + F2)) * (w["q1d_row"]["bytes"] / per_el)
    # column-wise RHT + SR over two ragged expert segments
    off = np.array([0, 1500, rows], dtype=np.int32)
    t0 = time.perf_counter()
    oracle.quantize_1d(gs, block_axis=0, group_offsets=off, use_rht=True, sign_mask=1, rnd=oracle.SR, seed=5)
    dt = time.perf_counter() - t0
    timings["q1d_col"] = dt / (rows * F2) * (w["q1d_col"]["bytes"] / per_el)
    # 2D, both layouts, on one full gate_up expert matrix
    wsl = synth.normal_bf16((1, D, F2), 0.02, seed=5)
    t0 = time.perf_counter()
    oracle.quantize_2d(wsl)
    dt = time.perf_counter() - t0
    timings["q2d"] = dt / wsl.size * (E * D * F2 + E * D * D)
    # GEMM: MAC rate on sampled output rows (full N, full K)
    ac, asc = oracle.quantize_1d(synth.channel_scaled_activations(rows=256, cols=D, seed=1))
    wb = synth.normal_bf16((1, F2, D), 0.02, seed=5)
    bc, bs, _, _ = oracle.quantize_2d(wb)
    done, dt = 0, 0.0
    while dt < gemm_seconds and done < 4096:
        sample_rows = [(0, int(m)) for m in rng.integers(0, 256, 2 * threads)]
        t0 = time.perf_counter()
        oracle.grouped_gemm(ac, asc, bc, bs, [0, 256], 256, F2, D, b_scale_2d=True, rows=sample_rows)
        dt += time.perf_counter() - t0
        done += len(sample_rows)
    mac_s = done * F2 * D / dt
    timings["gemm"] = w["gemm"]["flops"] / 2 / mac_s
    timings["gemm_wgrad"] = w["gemm_wgrad"]["flops"] / 2 / mac_s
    t_total = sum(timings.values())
    flops = w["gemm"]["flops"] + w["gemm_wgrad"]["flops"]
    return {
        "value": flops / t_total / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": ("row-wise quantize of 4096x2880 (RTNE) and 4096x5760 (SR), column-wise RHT+SR of "
                   "4096x5760 in two ragged segments, 2D (both layouts) of one 2880x5760 expert, FP64 "
                   "GEMM of %d sampled output rows x 5760 x 2880; per-role rates extrapolated to the "
                   "full step (%.0f s extrapolated)" % (done, t_total)),
        "extrapolated_step_s": t_total,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fused-epilogue", action="store_true",
                    help="skip the fused-epilogue comparison run after the timed steps (profiling runs)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device copy of this many bytes (3 launches), to "
                         "calibrate the HBM byte counters against a kernel of known traffic")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the path is data-parallel per expert and block, and this "
              "build runs no collectives; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    from mxfp4_precision_numerics_amd import mx
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_bytes:
        src = torch.empty(args.copy_bytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_bytes, "launches": 3}))
        return
    mx.lib()
    inp = build_inputs(torch, dev)
    step = Step(torch, dev, inp)
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()
    # timed region: K steps, per-launch events on the launch stream
    step.events = []
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for _ in range(args.steps):
        step.run()
    t_end.record()
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps
    per = {}
    for name, s, e in step.events:
        per.setdefault(name, []).append(s.elapsed_time(e))
    w = work_model()
    kernels = {}
    for name, times in per.items():
        avg = float(np.mean(times))
        launches = w[name]["launches"]
        ms_role = avg * launches
        k = {"launches_per_step": launches, "ms_per_step": ms_role, "avg_launch_ms": avg}
        if "bytes" in w[name]:
            gbs = w[name]["bytes"] / (ms_role / 1e3) / 1e9
            k.update({"GB/s": gbs, "frac_hbm": gbs / PEAK_HBM_GBS})
        else:
            tf = w[name]["flops"] / (ms_role / 1e3) / 1e12
            k.update({"TFLOP/s": tf, "frac_fp4": tf / PEAK_FP4_TFLOPS})
        kernels[name] = k
    total_flops = w["gemm"]["flops"] + w["gemm_wgrad"]["flops"]
    value = total_flops / (ms_step / 1e3) / 1e12
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    dk = kernels[dom]
    tr = measured_traffic(dom)
    if "TFLOP/s" in dk:
        roof = {"kernel": dom, "bound": "mfma", "achieved": dk["TFLOP/s"], "peak": PEAK_FP4_TFLOPS,
                "unit": "TFLOP/s", "frac": dk["TFLOP/s"] / PEAK_FP4_TFLOPS, "traffic": tr and tr["bytes"]}
    else:
        roof = {"kernel": dom, "bound": "hbm", "achieved": dk["GB/s"], "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": dk["GB/s"] / PEAK_HBM_GBS, "traffic": tr and tr["bytes"]}
    if tr:
        roof["traffic_read_write"] = [tr["read_bytes"], tr["write_bytes"]]
    quant_bytes = sum(w[k]["bytes"] for k in ("q1d_row", "q1d_col", "q2d"))
    quant_ms = sum(kernels[k]["ms_per_step"] for k in ("q1d_row", "q1d_col", "q2d"))
    gemm_ms = kernels["gemm"]["ms_per_step"] + kernels["gemm_wgrad"]["ms_per_step"]
    out = {
        "metric": "quantize GB/s + MXFP4 grouped-GEMM TFLOPS (fraction of HBM / FP4 roofline)",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4-e2m1/ue8m0 operands, fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": "quantized MoE expert step fwd+bwd: 32 experts, d_model 2880, ffn 2880 "
                               "(gate_up 5760), 16384 tokens top-4 Zipf(1.1)",
                   "experts": E, "d_model": D, "d_ff_gate_up": F2, "tokens": T, "top_k": TOPK},
        "quantize_GBps": quant_bytes / (quant_ms / 1e3) / 1e9,
        "quantize_frac_hbm": quant_bytes / (quant_ms / 1e3) / 1e9 / PEAK_HBM_GBS,
        "gemm_TFLOPs": total_flops / (gemm_ms / 1e3) / 1e12,
        "gemm_frac_fp4": total_flops / (gemm_ms / 1e3) / 1e12 / PEAK_FP4_TFLOPS,
        "kernels": kernels,
        "roofline": roof,
    }
    if not args.no_fused_epilogue:
        out["fused_epilogue"] = fused_epilogue(torch, step)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
