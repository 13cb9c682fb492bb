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
The metric is the pair quantize GB/s and grouped-GEMM TFLOP/s, each as a
fraction of its MI355X roofline; `value` is the whole step's algorithmic GEMM
FLOPs divided by the step time.

Every kernel instantiation is a role of its own, timed with HIP events on
the launch stream, and set against its binding roofline: HBM bytes / 8 TB/s
or FLOPs / 10.1 PFLOP/s, whichever floor is higher.  The line also carries
the stand-alone workloads (1x32 RTNE of a 256x512 fp32 outlier matrix; RHT
+ SR of 16384x2880 bf16 activations; 2D quantize and dequantize of 32 expert
weights 2880x5760; the grouped forward GEMM), with their round-trip error.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--config {1,2,3,4,5}]
                       [--no-cpu-baseline] [--no-standalone]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_FP4_TFLOPS = 10100.0      # MI355X dense FP4 MFMA, TFLOP/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_traffic.txt")
E, D, F2, T, TOPK = 32, 2880, 5760, 16384, 4
ROWS = T * TOPK
BPE_1D = 2 + 0.5 + 1 / 32      # bf16 in, codes + 1x32 scales out, per element
CS = 0.5 + 1 / 32              # 1x32 MXFP4 bytes per element
WS = 0.5 + 1 / 1024            # 32x32 MXFP4 bytes per element (one layout)

# role -> the kernel instantiation it launches (name without spaces)
ROLE_KERNEL = {
    "q2d": "q2d_kernel<true,false>",
    "q1d_row_rtne": "q1d_row_kernel_w<true,false,false>",
    "q1d_col": "q1d_col_kernel<true,true,true,0>",
    "q1d_dual_rtne": "q1d_col_kernel<true,true,true,1>",
    "q1d_dual_sr": "q1d_col_kernel<true,true,true,2>",
    "gemm_fwd_gather": "gemm_kernel<true,true,false,true,true,false,false>",
    "gemm_bf16": "gemm_kernel<true,true,false,false,true,false,true>",
    "gemm_wgrad": "gemm_kernel<false,false,true,false,false,false,true>",
}
QUANT_ROLES = ("q2d", "q1d_row_rtne", "q1d_col", "q1d_dual_rtne", "q1d_dual_sr")
GEMM_ROLES = ("gemm_fwd_gather", "gemm_bf16", "gemm_wgrad")


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
    # the weight gradient's K segments: each expert's tokens padded to 256, so
    # every K stage of its GEMM starts on whole 128-byte code lines
    pad = (counts + 255) // 256 * 256
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

        self.kp = mx.padded_capacity(ROWS, E, 256)
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
        # The step's GEMM operands carry their scales in the staged order
        # (include/mx.h, MX_SCALES_STAGED): A of the three data-path GEMMs
        # (row-wise, [ceil(K/256), rows, 8]) and both weight-gradient operands
        # (column-wise, [kp/256 + E, cols, 8]).  The row-major buffers above
        # serve the studies.
        st_r = lambda k: z((k + 255) // 256, ROWS, 8)          # noqa: E731
        st_c = lambda c: z(self.kp // 256 + E, c, 8)           # noqa: E731
        self.b.update(hs_st=st_r(D), g2s_st=st_r(D), g1s_st=st_r(F2), hTs_st=st_c(D), g2Ts_st=st_c(D),
                      xTs_st=st_c(D), g1Ts_st=st_c(F2))
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
        # h, dY2 and dY1 feed a row-wise GEMM operand and a column-wise
        # weight-gradient operand: one dual launch reads each tensor once and
        # writes both (mx_quantize_1d_dual).  X's row-wise operand is of the
        # 16,384 tokens, its column-wise one of the 65,536 routed rows, so it
        # keeps two launches.
        col = dict(block_axis=0, group_offsets=off, kp=self.kp, use_rht=True, sign_mask=m, rnd=mx.SR, seed=5,
                   group_pad=256)

        def dual(x, row_rnd, row_sid, col_sid, rc, rs, cc, cs):
            return mx.quantize_1d_dual(x, off, kp=self.kp, use_rht=True, sign_mask=m, col_rnd=mx.SR,
                                       col_stream_id=col_sid, row_rnd=row_rnd, row_stream_id=row_sid, seed=5,
                                       col_codes=b[cc], col_scales=b[cs], row_codes=b[rc], row_scales=b[rs],
                                       staged=True, group_pad=256)
        self._t("q2d", lambda: mx.quantize_2d_into(i["W1"], b["w1c"], b["w1s"], b["w1tc"], b["w1ts"]))
        self._t("q2d", lambda: mx.quantize_2d_into(i["W2"], b["w2c"], b["w2s"], b["w2tc"], b["w2ts"]))
        self._t("q1d_row_rtne", lambda: mx.quantize_1d(i["X"], codes=b["xc"], scales=b["xs"]))
        self._t("gemm_fwd_gather", lambda: mx.grouped_gemm(b["xc"], b["xs"], b["w1tc"], b["w1ts"], off, ROWS, F2,
                                                           D, a_row_index=idx, b_scale_2d=True, out=b["Y1"]))
        self._t("q1d_dual_rtne", lambda: dual(i["h"], mx.RNE, 0, 4, "hc", "hs_st", "hTc", "hTs_st"))
        self._t("gemm_bf16", lambda: mx.grouped_gemm(b["hc"], b["hs_st"], b["w2tc"], b["w2ts"], off, ROWS, D, D,
                                                     b_scale_2d=True, staged=True, out=b["Y2"]))
        self._t("q1d_dual_sr", lambda: dual(i["dY2"], mx.SR, 1, 5, "g2c", "g2s_st", "g2Tc", "g2Ts_st"))
        self._t("gemm_bf16", lambda: mx.grouped_gemm(b["g2c"], b["g2s_st"], b["w2c"], b["w2s"], off, ROWS, D, D,
                                                     b_scale_2d=True, staged=True, out=b["dh"]))
        self._t("gemm_wgrad", lambda: mx.grouped_gemm(b["hTc"], b["hTs_st"], b["g2Tc"], b["g2Ts_st"], poff, D, D,
                                                      self.kp, group_dim_k=True, staged=True, out=b["dW2"]))
        self._t("q1d_dual_sr", lambda: dual(i["dY1"], mx.SR, 0, 3, "g1c", "g1s_st", "g1Tc", "g1Ts_st"))
        self._t("gemm_bf16", lambda: mx.grouped_gemm(b["g1c"], b["g1s_st"], b["w1c"], b["w1s"], off, ROWS, D, F2,
                                                     b_scale_2d=True, staged=True, out=b["dX"]))
        # X^T: the routed rows are gathered from the 16384-token X inside the
        # quantizer (no permuted copy)
        self._t("q1d_col", lambda: mx.quantize_1d(i["X"], stream_id=2, codes=b["xTc"], scales=b["xTs_st"],
                                                  row_index=idx, staged=True, **col))
        self._t("gemm_wgrad", lambda: mx.grouped_gemm(b["xTc"], b["xTs_st"], b["g1Tc"], b["g1Ts_st"], poff, D, F2,
                                                      self.kp, group_dim_k=True, staged=True, out=b["dW1"]))


def work_model():
    """Algorithmic work per role in one step: each input read once, each
    output written once (padding and cache re-reads do not count), and
    2 M N K FLOPs over the real (unpadded) token rows.

    - 1D quantize from bf16: 2 B read + 0.5 + 1/32 B written per element;
      the gathered X of the weight gradient is read once (16,384 token rows)
      but written for every routed row (65,536).  Both 1x32 layouts of one
      tensor from one read (h, dY2, dY1): 2 B read + 2 x (0.5 + 1/32) B
      written per element.
    - 2D quantize, both layouts: 2 B read + 2 x (0.5 + 1/1024) B written.
    - GEMM: the A and B codes and scales read once, C written once (bf16, or
      fp32 for the weight gradient)."""
    gemm_fwd_gather = {
        "flops": 2.0 * ROWS * D * F2,
        "bytes": T * D * CS + E * F2 * D * WS + ROWS * F2 * 2,
    }
    # Y2 = h W2, dh = dY2 W2^T, dX = dY1 W1^T
    gemm_bf16 = {
        "flops": 2.0 * ROWS * (D * D + D * D + F2 * D),
        "bytes": (ROWS * D * CS + E * D * D * WS + ROWS * D * 2) * 2 + (ROWS * F2 * CS + E * D * F2 * WS + ROWS * D * 2),
    }
    # dW2 = h^T dY2, dW1 = X^T dY1
    gemm_wgrad = {
        "flops": 2.0 * ROWS * (D * D + D * F2),
        "bytes": (2 * ROWS * D * CS + E * D * D * 4) + (ROWS * D * CS + ROWS * F2 * CS + E * D * F2 * 4),
    }
    return {
        "q2d": {"bytes": (E * D * F2 + E * D * D) * (2 + 2 * WS), "launches": 2},
        "q1d_row_rtne": {"bytes": T * D * BPE_1D, "launches": 1},
        "q1d_col": {"bytes": T * D * 2 + ROWS * D * CS, "launches": 1},
        "q1d_dual_rtne": {"bytes": ROWS * D * (2 + 2 * CS), "launches": 1},
        "q1d_dual_sr": {"bytes": ROWS * (D + F2) * (2 + 2 * CS), "launches": 2},
        "gemm_fwd_gather": dict(gemm_fwd_gather, launches=1),
        "gemm_bf16": dict(gemm_bf16, launches=3),
        "gemm_wgrad": dict(gemm_wgrad, launches=2),
    }


def roof(work, ms):
    """The binding roofline of a kernel doing `work` in `ms`: the floor time
    at HBM peak (bytes) or FP4 MFMA peak (flops), whichever is longer, and
    the achieved rate in that roof's unit."""
    s = ms / 1e3
    t_hbm = work.get("bytes", 0.0) / (PEAK_HBM_GBS * 1e9)
    t_mfma = work.get("flops", 0.0) / (PEAK_FP4_TFLOPS * 1e12)
    if t_mfma >= t_hbm:
        ach = work["flops"] / s / 1e12
        return {"bound": "mfma", "achieved": ach, "peak": PEAK_FP4_TFLOPS, "unit": "TFLOP/s",
                "frac": ach / PEAK_FP4_TFLOPS}
    ach = work["bytes"] / s / 1e9
    return {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBS}


def kernel_source_hash():
    """sha256 over the device sources the GEMM kernel is compiled from."""
    import hashlib
    h = hashlib.sha256()
    for rel in ("mxfp4_precision_numerics_amd/csrc/mx_gemm.hip",
                "mxfp4_precision_numerics_amd/csrc/mx_device.h"):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(role):
    """HBM bytes per launch (scaled FETCH_SIZE + WRITE_SIZE) recorded for this
    role's kernel instantiation, or None when no record exists or the GEMM
    sources have changed since the counters were taken."""
    if role not in ROLE_KERNEL or not os.path.exists(TRAFFIC_FILE):
        return None
    src, rec = None, {}
    for line in open(TRAFFIC_FILE):
        f = line.split()
        if len(f) >= 2 and f[0] == "source_sha256":
            src = f[1]
        elif len(f) >= 6 and f[0] == "kernel":
            rec[f[1]] = (float(f[3]), float(f[5]))
    name = ROLE_KERNEL[role]
    if src != kernel_source_hash() or name not in rec:
        return None
    rd, wr = rec[name]
    return {"read_bytes": rd, "write_bytes": wr, "bytes": rd + wr}


def time_launches(torch, fns, reps, repeats=10):
    """Median over `repeats` of the mean time of `reps` back-to-back launches
    cycling through `fns` (ms per launch)."""
    for f in fns:
        f()
    torch.cuda.synchronize()
    out = []
    for _ in range(repeats):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for k in range(reps):
            fns[k % len(fns)]()
        e.record()
        torch.cuda.synchronize()
        out.append(s.elapsed_time(e) / reps)
    return float(np.median(out))


def rel_err(torch, x, y):
    """||x - y||_F / ||x||_F in float64 (round-trip error), and its SNR in dB."""
    num = den = 0.0
    for a, b in zip(x.reshape(-1).split(1 << 26), y.reshape(-1).split(1 << 26)):
        a64 = a.double()
        num += float(((a64 - b.double()) ** 2).sum())
        den += float((a64 ** 2).sum())
    r = math.sqrt(num / den)
    return {"rel_err": r, "snr_db": -20 * math.log10(r) if r > 0 else float("inf")}


# ---------------------------------------------------------------------------
# Stand-alone workloads
# ---------------------------------------------------------------------------
def config1(torch, dev):
    """1x32 RTNE of a 256x512 fp32 N(0,1) matrix with 131 entries (0.1%) x 50,
    then dequantize to fp32: launch-latency bound (0.59 MB)."""
    from mxfp4_precision_numerics_amd import mx
    g = torch.Generator(device=dev).manual_seed(0)
    x = torch.randn(256, 512, device=dev, generator=g)
    pos = torch.randperm(256 * 512, device=dev, generator=g)[:131]
    x.view(-1)[pos] *= 50.0
    c, s = mx.quantize_1d(x)
    y = mx.dequantize(c, s)
    tq = time_launches(torch, [lambda: mx.quantize_1d(x, codes=c, scales=s)], 200)
    td = time_launches(torch, [lambda: mx.dequantize(c, s, out=y)], 200)
    nbytes = 256 * 512 * (4 + CS)
    res = {"workload": "1x32 RTNE quantize + dequantize, fp32 256x512 N(0,1) with 0.1% outliers x50",
           "quantize_ms": tq, "quantize_GBps": nbytes / tq / 1e6, "dequantize_ms": td,
           "dequantize_GBps": nbytes / td / 1e6, "bound": "launch latency (0.59 MB)"}
    res.update(rel_err(torch, x, y))
    return res


def config2(torch, dev):
    """RHT + 1x32 SR of bf16 16384x2880 activations (N(0,1) x per-column
    log-uniform[0.1, 10]); sign mask from seed 1, SR key 2.  Five input/output
    sets (597 MB) rotate so the 256 MB Infinity Cache cannot hold the data."""
    from mxfp4_precision_numerics_amd import mx
    g = torch.Generator(device=dev).manual_seed(1)
    c = torch.exp(torch.empty(D, device=dev).uniform_(math.log(0.1), math.log(10.0), generator=g))
    sets = []
    for _ in range(5):
        x = (torch.randn(T, D, device=dev, generator=g) * c).to(torch.bfloat16)
        sets.append((x, torch.empty(T, D // 2, dtype=torch.uint8, device=dev),
                     torch.empty(T, D // 32, dtype=torch.uint8, device=dev)))
    mask = mx.rht_sign_mask(1)
    fns = [lambda s=s: mx.quantize_1d(s[0], use_rht=True, sign_mask=mask, rnd=mx.SR, seed=2,
                                      codes=s[1], scales=s[2]) for s in sets]
    t = time_launches(torch, fns, 50)
    nbytes = T * D * BPE_1D
    res = {"workload": "RHT + 1x32 SR quantize, bf16 16384x2880 activations (5 rotating sets, 597 MB)",
           "ms": t, "GBps": nbytes / t / 1e6, "roofline": roof({"bytes": nbytes}, t)}
    # round trip in the rotated basis: dequantized codes against RHT(x)
    x, cc, ss = sets[0]
    res.update(rel_err(torch, mx.rht(x, mask), mx.dequantize(cc, ss)))
    return res


def config3(torch, dev):
    """2D (32x32) RTNE quantize of 32 expert weights bf16 2880x5760 N(0, 0.02)
    (seed 3), both layouts, then dequantize the W layout to bf16."""
    from mxfp4_precision_numerics_amd import mx
    g = torch.Generator(device=dev).manual_seed(3)
    w = (torch.randn(E, D, F2, device=dev, generator=g) * 0.02).to(torch.bfloat16)
    c, s, ct, st = mx.quantize_2d(w)
    y = mx.dequantize(c, s, block_rows=32, out_dtype=torch.bfloat16)
    tq = time_launches(torch, [lambda: mx.quantize_2d_into(w, c, s, ct, st)], 5)
    td = time_launches(torch, [lambda: mx.dequantize(c, s, block_rows=32, out=y)], 5)
    n = E * D * F2
    qb, db = n * (2 + 2 * WS), n * (WS + 2)
    res = {"workload": "2D 32x32 RTNE quantize (both layouts) + bf16 dequantize, 32 x bf16 2880x5760 N(0,0.02)",
           "quantize_ms": tq, "quantize_GBps": qb / tq / 1e6, "quantize_roofline": roof({"bytes": qb}, tq),
           "dequantize_ms": td, "dequantize_GBps": db / td / 1e6, "dequantize_roofline": roof({"bytes": db}, td)}
    res.update(rel_err(torch, w, y))
    del w, c, s, ct, st, y
    return res


def fused_epilogue(torch, step, reps=5):
    """The quantizing epilogue on the second expert linear's forward GEMM
    (65536 x 2880 x 2880): its bf16 output quantized row-wise (1x32, RTNE) as
    the next MXFP4 GEMM's operand.  Times the GEMM followed by the 1D
    quantizer against the fused call, with and without the bf16 output, on
    the step's own buffers."""
    mx, b, i = step.mx, step.b, step.inp
    args = (b["hc"], b["hs_st"], b["w2tc"], b["w2ts"], i["off"], ROWS, D, D)
    runs = {
        "gemm_then_quantize_ms": lambda: (mx.grouped_gemm(*args, b_scale_2d=True, staged=True, out=b["Y2"]),
                                          mx.quantize_1d(b["Y2"], codes=b["g2c"], scales=b["g2s"])),
        "fused_ms": lambda: mx.grouped_gemm_q(*args, b_scale_2d=True, staged=True, out=b["Y2"], codes=b["g2c"],
                                              scales=b["g2s"]),
        "fused_mxfp4_only_ms": lambda: mx.grouped_gemm_q(*args, b_scale_2d=True, staged=True, with_bf16=False,
                                                         codes=b["g2c"], scales=b["g2s"]),
    }
    res = {"shape": "%dx%dx%d" % (ROWS, D, D)}
    for name, fn in runs.items():
        res[name] = time_launches(torch, [fn], reps, repeats=5)
    return res


def deosc_study(torch, dev, steps=10, sigma=1e-4, margins=(0, 4, 8, 16)):
    """Weight de-oscillation on a synthetic master-weight trajectory: 32
    expert weights fp32 2880x5760 N(0, 0.02) take `steps` zero-mean random
    steps of `sigma` per element (the converged, noise-dominated regime in
    which weights near a boundary oscillate).  The quantized state starts
    from the plain 2D quantization and is updated in place by
    mx_quantize_2d_deosc at each step.  Reports bin flips per step and the
    final round-trip error against the master weights for each margin, and
    the kernel's time and GB/s on this tensor."""
    from mxfp4_precision_numerics_amd import mx
    g = torch.Generator(device=dev).manual_seed(6)
    w0 = torch.randn(E, D, F2, device=dev, generator=g) * 0.02
    res = {"workload": "32 x fp32 2880x5760 master weights N(0,0.02), %d random-walk steps of %g" % (steps, sigma),
           "margins": {}}
    for m in margins:
        w = w0.clone()
        c, s, _, _ = mx.quantize_2d(w, transposed=False)
        gs = torch.Generator(device=dev).manual_seed(7)
        flips = []
        for _ in range(steps):
            w += torch.randn(w.shape, device=dev, generator=gs) * sigma
            _, _, _, _, fl = mx.quantize_2d_deosc(w, c, s, m, codes=c, scales=s, transposed=False)
            flips.append(int(fl.view(torch.int16).to(torch.int64).sum()))
        y = mx.dequantize(c, s, block_rows=32)
        r = rel_err(torch, w, y)
        res["margins"][str(m)] = {"flips_per_step": float(np.mean(flips)), "flip_rate": float(np.mean(flips)) / w.numel(),
                                  "rel_err": r["rel_err"], "snr_db": r["snr_db"]}
        del w, y
    # kernel time: fp32 master weights, both layouts, in place, margin 8
    c, s, ct, st = mx.quantize_2d(w0)
    t = time_launches(torch, [lambda: mx.quantize_2d_deosc(w0, c, s, 8, codes=c, scales=s, codes_t=ct,
                                                           scales_t=st)], 5)
    tp = time_launches(torch, [lambda: mx.quantize_2d_into(w0, c, s, ct, st)], 5)
    n = E * D * F2
    nbytes = n * (4 + WS + 2 * WS) + (n // 1024) * 2     # master weights, previous codes, both layouts, flips
    res.update({"deosc_ms": t, "deosc_GBps": nbytes / t / 1e6, "deosc_roofline": roof({"bytes": nbytes}, t),
                "plain_2d_fp32_ms": tp})
    del w0, c, s, ct, st
    return res


def snr_study(torch, dev):
    """Operator-level SNR (C26: -20 log10 of the relative Frobenius error) of
    outlier clipping and macro-block scaling on synthetic tensors, with and
    without the RHT, RTNE.  All quantization and decoding runs in the
    library's kernels (mx_quantize_1d_ex / mx_dequantize_1d_ex); the error
    sums are taken in float64 on the device."""
    from mxfp4_precision_numerics_amd import mx
    g = torch.Generator(device=dev).manual_seed(8)
    c = torch.exp(torch.empty(D, device=dev).uniform_(math.log(0.1), math.log(10.0), generator=g))
    act = (torch.randn(T, D, device=dev, generator=g) * c)
    out = act.clone().view(-1)
    pos = torch.randperm(out.numel(), device=dev, generator=g)[:out.numel() // 1000]
    out[pos] *= 50.0
    tensors = {
        "activations 16384x2880 (N(0,1) x log-uniform channel scale)": act.to(torch.bfloat16),
        "activations with 0.1% outliers x50": out.view(T, D).to(torch.bfloat16),
        "gradients 16384x2880 N(0, 1e-3)": (torch.randn(T, D, device=dev, generator=g) * 1e-3).to(torch.bfloat16),
        "heavy-tailed 16384x2880 (Student-t, 3 dof)": (torch.randn(T, D, device=dev, generator=g) / torch.sqrt(
            sum(torch.randn(T, D, device=dev, generator=g) ** 2 for _ in range(3)) / 3)).to(torch.bfloat16),
    }
    variants = [("plain", 1.0, 0), ("clip 0.875", 0.875, 0), ("clip 0.75", 0.75, 0), ("clip 0.5", 0.5, 0),
                ("clip search", 0.0, 0), ("macro 320", 1.0, 320), ("macro 2880 (row)", 1.0, 2880),
                ("macro 320 + clip search", 0.0, 320)]
    mask = mx.rht_sign_mask(1)
    res = {}
    for name, x in tensors.items():
        row = {}
        for use_rht in (False, True):
            ref = mx.rht(x, mask) if use_rht else x.float()
            for vname, clip, bm in variants:
                cc, ss, mr = mx.quantize_1d_ex(x, use_rht=use_rht, sign_mask=mask, clip_ratio=clip, macro_block=bm)
                y = mx.dequantize_1d_ex(cc, ss, mr, macro_block=bm)
                row[("RHT, " if use_rht else "") + vname] = round(rel_err(torch, ref, y)["snr_db"], 3)
        res[name] = row
    return res


def dual_vs_separate(torch, step, reps=5):
    """The dual quantizer (one read, row-wise and column-wise RHT+SR codes)
    against the two launches it replaces, on the step's buffers and layouts
    (staged scales, groups padded to 256 tokens): h (65536 x 2880, row RTNE),
    dY2 (65536 x 2880, row SR) and dY1 (65536 x 5760, row SR)."""
    mx, b, i = step.mx, step.b, step.inp
    off, m, kp = i["off"], step.mask, step.kp
    col = dict(block_axis=0, group_offsets=off, kp=kp, use_rht=True, sign_mask=m, rnd=mx.SR, seed=5,
               group_pad=256, staged=True)
    res = {}
    for name, x, rnd, rs, cs_, rc, rsc, cc, csc in (
            ("h_row_rtne", i["h"], mx.RNE, 0, 4, "hc", "hs_st", "hTc", "hTs_st"),
            ("dY2_row_sr", i["dY2"], mx.SR, 1, 5, "g2c", "g2s_st", "g2Tc", "g2Ts_st"),
            ("dY1_row_sr", i["dY1"], mx.SR, 0, 3, "g1c", "g1s_st", "g1Tc", "g1Ts_st")):
        sep = lambda: (mx.quantize_1d(x, rnd=rnd, seed=5, stream_id=rs, codes=b[rc], scales=b[rsc],  # noqa
                                      staged=True),
                       mx.quantize_1d(x, stream_id=cs_, codes=b[cc], scales=b[csc], **col))
        dual = lambda: mx.quantize_1d_dual(x, off, kp=kp, use_rht=True, sign_mask=m, col_rnd=mx.SR,  # noqa
                                           col_stream_id=cs_, row_rnd=rnd, row_stream_id=rs, seed=5,
                                           col_codes=b[cc], col_scales=b[csc], row_codes=b[rc], row_scales=b[rsc],
                                           staged=True, group_pad=256)
        res[name] = {"shape": "%dx%d" % tuple(x.shape), "separate_ms": time_launches(torch, [sep], reps, repeats=5),
                     "dual_ms": time_launches(torch, [dual], reps, repeats=5)}
    return res


def cpu_baseline_config(k, gemm_seconds=8.0):
    """The oracle on config k itself (configs 1-3 run whole; config 4 on
    sampled output rows, extrapolated)."""
    import oracle
    from mxfp4_precision_numerics_amd import synth
    threads = oracle.default_threads()
    if k == 1:
        x, _ = synth.outlier_matrix()
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < 2.0:
            c, s = oracle.quantize_1d(x)
            oracle.dequantize(c, s)
            reps += 1
        dt = (time.perf_counter() - t0) / reps
        return {"value": 256 * 512 * (4 + CS) / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
                "sample": "the whole 256x512 config, quantize + dequantize, %d repeats" % reps}
    if k == 2:
        x = synth.channel_scaled_activations()
        t0 = time.perf_counter()
        oracle.quantize_1d(x, use_rht=True, sign_mask=oracle.rht_sign_mask(1), rnd=oracle.SR, seed=2)
        dt = time.perf_counter() - t0
        return {"value": T * D * BPE_1D / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
                "sample": "the whole 16384x2880 config"}
    if k == 3:
        w = synth.normal_bf16((8, D, F2), 0.02, seed=3)
        t0 = time.perf_counter()
        oracle.quantize_2d(w)
        dt = time.perf_counter() - t0
        return {"value": w.size * (2 + 2 * WS) / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
                "sample": "8 of the 32 experts (2880x5760 each), both layouts"}
    base = cpu_baseline(gemm_seconds)
    return {"value": base["gemm_TFLOPs"], "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": base["gemm_sample"]}


def cpu_baseline(gemm_seconds=8.0, single_thread=True):
    """The oracle, untuned, on a bounded sample of the same step; its rate per
    role is extrapolated to the full step.  The quantizers run on fixed
    slices; the FP64 GEMM runs batches of sampled output rows (full N, full K)
    until about `gemm_seconds` have passed.  With single_thread, a quarter of
    the quantizer sample and 2 s of GEMM rows run again on one thread."""
    import oracle
    from mxfp4_precision_numerics_amd import synth
    threads = oracle.default_threads()
    rng = np.random.default_rng(0)
    w = work_model()

    def quant_rate(rows, nthreads):
        """seconds per element of each quantizer role, on `rows` token rows"""
        xs = synth.channel_scaled_activations(rows=rows, cols=D, seed=1)
        gs = synth.normal_bf16((rows, F2), 1e-3, seed=5)
        out = {}
        t0 = time.perf_counter()
        oracle.quantize_1d(xs, threads=nthreads)
        out["q1d_row_rtne"] = (time.perf_counter() - t0) / (rows * D)
        t0 = time.perf_counter()
        oracle.quantize_1d(gs, rnd=oracle.SR, seed=5, threads=nthreads)
        out["q1d_row_sr"] = (time.perf_counter() - t0) / (rows * F2)
        off = np.array([0, rows * 3 // 8, rows], dtype=np.int32)
        t0 = time.perf_counter()
        oracle.quantize_1d(gs, block_axis=0, group_offsets=off, use_rht=True, sign_mask=1, rnd=oracle.SR,
                           seed=5, threads=nthreads)
        out["q1d_col"] = (time.perf_counter() - t0) / (rows * F2)
        wrows = D if rows >= 4096 else max(32, rows // 4 // 32 * 32)
        wsl = synth.normal_bf16((1, wrows, F2), 0.02, seed=5)
        t0 = time.perf_counter()
        oracle.quantize_2d(wsl, threads=nthreads)
        out["q2d"] = (time.perf_counter() - t0) / wsl.size
        return out

    def gemm_rate(seconds, nthreads):
        ac, asc = oracle.quantize_1d(synth.channel_scaled_activations(rows=256, cols=D, seed=1))
        wb = synth.normal_bf16((1, F2, D), 0.02, seed=5)
        bc, bs, _, _ = oracle.quantize_2d(wb)
        done, dt = 0, 0.0
        while dt < seconds and done < 4096:
            sample_rows = [(0, int(m)) for m in rng.integers(0, 256, 2 * nthreads)]
            t0 = time.perf_counter()
            oracle.grouped_gemm(ac, asc, bc, bs, [0, 256], 256, F2, D, b_scale_2d=True, rows=sample_rows,
                                threads=nthreads)
            dt += time.perf_counter() - t0
            done += len(sample_rows)
        return done * F2 * D / dt, done

    def step_seconds(qr, mac_s):
        el = {"q1d_row_rtne": T * D + ROWS * D, "q1d_row_sr": ROWS * D + ROWS * F2,
              "q1d_col": 3 * ROWS * D + ROWS * F2, "q2d": E * D * F2 + E * D * D}   # (the oracle runs each layout)
        t = {k: qr[k] * el[k] for k in el}
        t["gemm"] = sum(w[r]["flops"] for r in GEMM_ROLES) / 2 / mac_s
        return t

    qr = quant_rate(4096, threads)
    mac_s, done = gemm_rate(gemm_seconds, threads)
    t = step_seconds(qr, mac_s)
    t_total = sum(t.values())
    flops = sum(w[r]["flops"] for r in GEMM_ROLES)
    res = {
        "value": flops / t_total / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": ("row-wise quantize of 4096x2880 (RTNE) and 4096x5760 (SR), column-wise RHT+SR of "
                   "4096x5760 in two ragged segments, 2D (both layouts) of one 2880x5760 expert, FP64 "
                   "GEMM of %d sampled output rows x 5760 x 2880; per-role rates extrapolated to the "
                   "full step (%.0f s extrapolated)" % (done, t_total)),
        "extrapolated_step_s": t_total,
        "gemm_TFLOPs": 2 * mac_s / 1e12,
        "gemm_sample": "FP64 GEMM of %d sampled output rows x 5760 x 2880" % done,
    }
    if single_thread:
        qr1 = quant_rate(1024, 1)
        mac1, done1 = gemm_rate(2.0, 1)
        t1 = sum(step_seconds(qr1, mac1).values())
        res["single_thread"] = {"value": flops / t1 / 1e12, "unit": "TFLOP/s", "extrapolated_step_s": t1,
                                "sample": "a quarter of the quantizer sample and %d GEMM rows, one thread"
                                          % done1}
    return res


def run_step(torch, dev, args):
    inp = build_inputs(torch, dev)
    step = Step(torch, dev, inp)
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()
    # timed region: K steps and nothing else on the launch stream
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for _ in range(args.steps):
        step.run()
    t_end.record()
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    # K more steps with an event pair around every launch, for the per-kernel
    # times (the events cost about 0.1 ms per step, so they stay out of the
    # timed region above)
    step.events = []
    for _ in range(args.steps):
        step.run()
    torch.cuda.synchronize()
    # per role: its launches' summed time in each step (launches of one role
    # may differ in size), then the median over the steps
    n = len(step.events) // args.steps
    per = {}
    for k in range(args.steps):
        tot = {}
        for name, s, e in step.events[k * n:(k + 1) * n]:
            tot[name] = tot.get(name, 0.0) + s.elapsed_time(e)
        for name, v in tot.items():
            per.setdefault(name, []).append(v)
    return step, inp, ms_step, per


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=5, choices=[1, 2, 3, 4, 5],
                    help="5 (default): the full expert step; 1-4: one stand-alone workload per line")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-standalone", action="store_true",
                    help="skip the stand-alone workloads after the timed steps (profiling runs)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device copy of this many bytes (3 launches), to "
                         "calibrate the HBM byte counters against a kernel of known traffic")
    ap.add_argument("--hbm-ceiling", action="store_true",
                    help="only run the HBM-rate probe (the quantizers' access patterns without "
                         "arithmetic; one JSON line per pattern)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the path is data-parallel per expert and block, and this "
              "build runs no collectives; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.hbm_ceiling:
        # a child process of its own, started before this one touches the GPU
        probe = os.path.join(ROOT, "mxfp4_precision_numerics_amd", "hbm_probe")
        if not os.path.exists(probe):
            sys.exit("hbm_probe is not built; run python -m mxfp4_precision_numerics_amd.build")
        sys.exit(subprocess.run([probe]).returncode)
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
    common = {"n_gpus": 1, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
              "data": "synthetic"}
    if args.config in (1, 2, 3):
        res = {1: config1, 2: config2, 3: config3}[args.config](torch, dev)
        r = res.get("roofline") or res.get("quantize_roofline") or roof({"bytes": 256 * 512 * (4 + CS)},
                                                                       res["quantize_ms"])
        out = dict(metric="quantize GB/s + MXFP4 grouped-GEMM TFLOPS (fraction of HBM / FP4 roofline)",
                   value=r["achieved"], unit="GB/s", steps=10, warmup=1, ms_per_step=res.get("ms", res.get(
                       "quantize_ms")), dtype="bf16 in, fp4-e2m1/ue8m0 out" if args.config > 1 else
                   "fp32 in, fp4-e2m1/ue8m0 out", config={"workload": res["workload"]}, roofline=r, result=res,
                   **common)
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline_config(args.config)
        print(json.dumps(out))
        return
    step, inp, ms_step, per = run_step(torch, dev, args)
    w = work_model()
    kernels = {}
    for name, times in per.items():
        ms_role = float(np.median(times))
        launches = w[name]["launches"]
        k = {"instantiation": ROLE_KERNEL[name], "launches_per_step": launches, "ms_per_step": ms_role,
             "avg_launch_ms": ms_role / launches, "roofline": roof(w[name], ms_role)}
        if "flops" in w[name]:
            tf = w[name]["flops"] / (ms_role / 1e3) / 1e12
            k.update({"TFLOP/s": tf, "frac_fp4": tf / PEAK_FP4_TFLOPS})
        gbs = w[name]["bytes"] / (ms_role / 1e3) / 1e9
        k.update({"GB/s": gbs, "frac_hbm": gbs / PEAK_HBM_GBS})
        kernels[name] = k
    total_flops = sum(w[r]["flops"] for r in GEMM_ROLES)
    value = total_flops / (ms_step / 1e3) / 1e12
    if args.config == 4:
        k = kernels["gemm_fwd_gather"]
        out = dict(metric="quantize GB/s + MXFP4 grouped-GEMM TFLOPS (fraction of HBM / FP4 roofline)",
                   value=k["TFLOP/s"], unit="TFLOP/s", steps=args.steps, warmup=args.warmup,
                   ms_per_step=k["ms_per_step"], dtype="fp4-e2m1/ue8m0 operands, fp32 accumulate, bf16 out",
                   config={"workload": "grouped MXFP4 GEMM forward, 32 experts, 65536 Zipf-routed rows gathered "
                                       "from 16384 tokens, K 2880, N 5760"},
                   roofline=dict(k["roofline"], kernel=k["instantiation"]), **common)
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline_config(4)
        print(json.dumps(out))
        return
    dom = max(kernels, key=lambda r: kernels[r]["ms_per_step"])
    dk = kernels[dom]
    rf = dict(dk["roofline"], kernel=dk["instantiation"], role=dom)
    tr = measured_traffic(dom)
    rf["traffic"] = tr and tr["bytes"]
    if tr:
        rf["traffic_read_write"] = [tr["read_bytes"], tr["write_bytes"]]
        rf["algorithmic_bytes_per_launch"] = w[dom]["bytes"] / w[dom]["launches"]
    if "flops" in w[dom]:
        rf["mfma_frac"] = dk["frac_fp4"]
    quant_bytes = sum(w[k]["bytes"] for k in QUANT_ROLES)
    quant_ms = sum(kernels[k]["ms_per_step"] for k in QUANT_ROLES)
    gemm_ms = sum(kernels[k]["ms_per_step"] for k in GEMM_ROLES)
    out = {
        "metric": "quantize GB/s + MXFP4 grouped-GEMM TFLOPS (fraction of HBM / FP4 roofline)",
        "value": value,
        "unit": "TFLOP/s",
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "dtype": "fp4-e2m1/ue8m0 operands, fp32 accumulate",
        "config": {"workload": "quantized MoE expert step fwd+bwd: 32 experts, d_model 2880, ffn 2880 "
                               "(gate_up 5760), 16384 tokens top-4 Zipf(1.1)",
                   "experts": E, "d_model": D, "d_ff_gate_up": F2, "tokens": T, "top_k": TOPK},
        "quantize_ms_per_step": quant_ms,
        "quantize_GB_per_step": quant_bytes / 1e9,
        "quantize_GBps": quant_bytes / (quant_ms / 1e3) / 1e9,
        "quantize_frac_hbm": quant_bytes / (quant_ms / 1e3) / 1e9 / PEAK_HBM_GBS,
        "gemm_ms_per_step": gemm_ms,
        "gemm_TFLOPs": total_flops / (gemm_ms / 1e3) / 1e12,
        "gemm_frac_fp4": total_flops / (gemm_ms / 1e3) / 1e12 / PEAK_FP4_TFLOPS,
        "kernels": kernels,
        "roofline": rf,
        **common,
    }
    if not args.no_standalone:
        out["fused_epilogue"] = fused_epilogue(torch, step)
        out["dual_quantize"] = dual_vs_separate(torch, step)
        del step, inp
        torch.cuda.empty_cache()
        out["deosc_study"] = deosc_study(torch, dev)
        torch.cuda.empty_cache()
        out["snr_study"] = snr_study(torch, dev)
        torch.cuda.empty_cache()
        out["standalone"] = {"config1": config1(torch, dev), "config2": config2(torch, dev),
                             "config3": config3(torch, dev),
                             "config4": {"workload": "grouped forward GEMM 65536x5760x2880 (the step's Y1 launch)",
                                         **{k: kernels["gemm_fwd_gather"][k] for k in
                                            ("avg_launch_ms", "TFLOP/s", "frac_fp4", "roofline")}}}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
