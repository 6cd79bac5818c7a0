"""Benchmark of the Fibonacci-offset sparse attention forward on one MI355X.

Workload (timed step): the long-context shape B=1, H=32, N=131072, D=64, bf16, W=12,
Fibonacci base up to 987, alpha = 1.5 (layer 15 of the staggered-linear schedule), integer
offsets, forward. One step = one call of fib_sparse_attn_fwd over the whole batch (offset
table, RoPE, window + offset gather, softmax, output and LSE). Inputs are seeded N(0, 1)
draws already resident in HBM. The other rows of the path (interpolated forward, integer and
interpolated backward) are timed on the same inputs and reported under "components".

Printed: one JSON line with metric, value (tokens/s = B*H*N / step time), a roofline object
for the forward kernel (algorithmic bytes / HIP-event time vs 8 TB/s) and the fp64 CPU
oracle's throughput on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
D = 64


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# device sources of the timed kernel (the ring forward): the stored HBM byte counts hold
# only while these are unchanged
TIMED_KERNEL_SOURCES = ("fwd_ring.hip", "ring_common.h", "fib_common.h")


def kernel_sources_sha() -> str:
    csrc = os.path.join(ROOT, "fibonacci_offset_dilated_amd", "csrc")
    h = hashlib.sha256()
    for f in TIMED_KERNEL_SOURCES:
        h.update(f.encode())
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on
    the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(f"{kernel}|{workload}")
    except Exception:
        return None
    if not rec or rec.get("sources_sha") != kernel_sources_sha():
        return None
    return rec.get("bytes_per_launch")


def make_inputs(B, H, N, seed, with_dout, dev):
    import torch

    from fibonacci_offset_dilated_amd.synthetic import normal_inputs

    arrs = normal_inputs(seed, (B, H, N, D), with_dout=with_dout)
    outs = []
    for a in arrs:
        # fp32 -> bf16 round-to-nearest-even (torch's cast); the draws are finite
        outs.append(torch.from_numpy(a).to(dev).to(torch.bfloat16))
        del a
    return outs, arrs


def time_calls(fn, steps, warmup, stream):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps  # ms


def cpu_baseline(arrs, B, H, N, W, alpha, base, mode, budget_s):
    """fp64 oracle on a bounded sample: as many whole heads as fit the time budget, run in a
    process pool over all host cores of this process's affinity mask."""
    import oracle as O
    from fibonacci_offset_dilated_amd.synthetic import bf16_bits_to_f32, f32_to_bf16_bits

    cores = len(os.sched_getaffinity(0))
    # probe: one head-chunk of rows to estimate the per-query cost
    q = bf16_bits_to_f32(f32_to_bf16_bits(arrs[0][0, 0])).astype(np.float64)
    k = bf16_bits_to_f32(f32_to_bf16_bits(arrs[1][0, 0])).astype(np.float64)
    v = bf16_bits_to_f32(f32_to_bf16_bits(arrs[2][0, 0])).astype(np.float64)
    rows = np.arange(0, min(N, 8192))
    t = time.perf_counter()
    O.forward_rows(q, k, v, rows, W, alpha, base, 10000.0, mode)
    per_q = (time.perf_counter() - t) / len(rows)
    heads = int(max(1, min(B * H, (budget_s * cores) / max(per_q * N, 1e-9))))
    heads = max(min(heads, B * H), 1)
    heads = min(B * H, max(heads - heads % max(1, min(cores, heads)), 1))
    sel = [(i // H, i % H) for i in range(heads)]

    def conv(x):
        return np.stack([bf16_bits_to_f32(f32_to_bf16_bits(x[b, h])).astype(np.float64) for b, h in sel])[None]

    qs, ks, vs = conv(arrs[0]), conv(arrs[1]), conv(arrs[2])
    workers = min(cores, heads)
    t = time.perf_counter()
    O.forward(qs, ks, vs, W, alpha, base, 10000.0, mode, workers=workers)
    dt = time.perf_counter() - t
    out = {"value": heads * N / dt, "unit": "tokens/s", "cores": workers, "kind": "oracle",
           "sample": f"{heads} of {B * H} heads x N={N} (fp64 NumPy forward, integer mode, process pool)",
           "seconds": round(dt, 3), "cpu_model": cpu_model(), "numpy": np.__version__}
    # backward of the oracle on a bounded sample: one head's sampled rows, timed the same way
    do = bf16_bits_to_f32(f32_to_bf16_bits(arrs[3][0, 0])).astype(np.float64)
    rows_b = np.arange(0, min(N, 2048))
    t = time.perf_counter()
    O.backward(q[None, None], k[None, None], v[None, None], do[None, None], W, alpha, base, 10000.0, mode, rows=rows_b)
    dtb = time.perf_counter() - t
    out["backward"] = {"value": len(rows_b) / dtb, "unit": "tokens/s", "cores": 1,
                       "sample": f"{len(rows_b)} query rows of one head (fp64 NumPy backward, one process)"}
    return out


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def small_configs(dev, stream, args):
    """The smaller measured workloads, timed the same way (launch- and tail-bound at these sizes):
    the 4x-extrapolation shape B4 H8 N4096 (integer forward, 16 coprime-schedule layers), and
    the training shape B8 H8 N1024 (integer forward at the linear schedule's layers,
    interpolated forward and backward at the learned-dilation alphas)."""
    import torch

    import fibonacci_offset_dilated_amd as F
    from fibonacci_offset_dilated_amd.synthetic import seed_for, uniform_alphas
    from fibonacci_offset_dilated_amd.workloads import (BY_CONFIG, FIB_BASE, INT, INTERP, UNIFORM_ALPHA_RANGE,
                                                        UNIFORM_ALPHA_SEED)

    def per_layer_us(make, layers):
        calls = [make(l) for l in layers]
        for c in calls:
            c()
        reps = max(5, args.steps // 5)
        ms = time_calls(lambda: [c() for c in calls], reps, 2, stream)
        return ms * 1e3 / len(calls)

    out = {}
    # the single-head fp32 workload (B1 H1 N1024, W 12, alpha 1, integer offsets): 16 calls
    # back to back, per-call time
    w1 = BY_CONFIG[1]
    q1, k1, v1 = (torch.randn((w1.B, w1.H, w1.N, D), generator=torch.Generator(device=dev).manual_seed(seed_for(1)),
                              device=dev, dtype=torch.float32) for _ in range(3))
    o1 = torch.empty_like(q1)
    l1 = torch.empty((w1.B, w1.H, w1.N), dtype=torch.float32, device=dev)
    us1 = per_layer_us(lambda l: (lambda: F.fwd(q1, k1, v1, 12, np.float32(1.0), FIB_BASE, 10000.0, INT, out=o1,
                                                lse=l1)), range(16))
    rows1 = w1.B * w1.H * w1.N
    out["c1_fp32_fwd_int_us"] = round(us1, 2)
    out["c1_fp32_fwd_int_hbm_frac"] = round(rows1 * (4 * D * 4 + 4) / (us1 * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    del q1, k1, v1, o1, l1

    w4 = BY_CONFIG[4]
    (q, k, v), _ = make_inputs(w4.B, w4.H, w4.N, seed_for(4, 0, 12, 0), False, dev)
    o = torch.empty_like(q)
    lse = torch.empty((w4.B, w4.H, w4.N), dtype=torch.float32, device=dev)
    al4 = [F.schedule_alpha(F.SCHED_COPRIME, l, 16) for l in range(16)]
    us = per_layer_us(lambda l: (lambda: F.fwd(q, k, v, 12, al4[l], FIB_BASE, 10000.0, INT, out=o, lse=lse)), range(16))
    rows4 = w4.B * w4.H * w4.N
    out["c4_fwd_int_us_per_layer"] = round(us, 2)
    out["c4_fwd_int_hbm_frac"] = round(rows4 * (4 * D * 2 + 4) / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    del q, k, v, o, lse

    w2 = BY_CONFIG[3]
    (q, k, v, do), _ = make_inputs(w2.B, w2.H, w2.N, seed_for(3, 0, 12, 0), True, dev)
    o = torch.empty_like(q)
    lse = torch.empty((w2.B, w2.H, w2.N), dtype=torch.float32, device=dev)
    al2 = [F.schedule_alpha(F.SCHED_LINEAR, l, 16) for l in range(16)]
    al3 = uniform_alphas(UNIFORM_ALPHA_SEED, 16, *UNIFORM_ALPHA_RANGE)
    us_int = per_layer_us(lambda l: (lambda: F.fwd(q, k, v, 12, al2[l], FIB_BASE, 10000.0, INT, out=o, lse=lse)),
                          range(16))
    us_interp = per_layer_us(lambda l: (lambda: F.fwd(q, k, v, 12, al3[l], FIB_BASE, 10000.0, INTERP, out=o,
                                                      lse=lse)), range(16))
    outs = [F.fwd(q, k, v, 12, al3[l], FIB_BASE, 10000.0, INTERP) for l in range(16)]
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    dal = torch.empty(1, dtype=torch.float32, device=dev)
    ws = torch.empty(F.bwd_workspace_size(w2.B, w2.H, w2.N, D, F.BF16, INTERP), dtype=torch.uint8, device=dev)
    us_bwd = per_layer_us(lambda l: (lambda: F.bwd(q, k, v, outs[l][0], outs[l][1], do, 12, al3[l], FIB_BASE, 10000.0,
                                                   INTERP, dq=dq, dk=dk, dv=dv, dalpha=dal, workspace=ws)), range(16))
    rows2 = w2.B * w2.H * w2.N
    out["b8h8n1024_fwd_int_us_per_layer"] = round(us_int, 2)
    out["b8h8n1024_fwd_interp_us_per_layer"] = round(us_interp, 2)
    out["b8h8n1024_interp_over_int"] = round(us_interp / us_int, 3)
    out["b8h8n1024_bwd_interp_us_per_layer"] = round(us_bwd, 2)
    out["b8h8n1024_fwd_int_hbm_frac"] = round(rows2 * (4 * D * 2 + 4) / (us_int * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    del q, k, v, do, o, lse, outs, dq, dk, dv, ws

    # decode: one new query per (batch, head) against a cache at the pages' evaluation length
    # (B8 H8, N = 4096), integer offsets at the linear schedule's layers vs interpolated at the
    # learned-dilation alphas (the comparison of Results 2)
    (qc, kc, vc), _ = make_inputs(8, 8, 4096, seed_for(3, 0, 12, 1), False, dev)
    qd = qc[:, :, -1, :].contiguous()
    od = torch.empty_like(qd)
    ld = torch.empty((8, 8), dtype=torch.float32, device=dev)
    us_di = per_layer_us(lambda l: (lambda: F.decode(qd, kc, vc, 12, al2[l], FIB_BASE, 10000.0, INT, out=od, lse=ld)),
                         range(16))
    us_dp = per_layer_us(lambda l: (lambda: F.decode(qd, kc, vc, 12, al3[l], FIB_BASE, 10000.0, INTERP, out=od,
                                                     lse=ld)), range(16))
    out["decode_b8h8n4096_int_us_per_layer"] = round(us_di, 2)
    out["decode_b8h8n4096_interp_us_per_layer"] = round(us_dp, 2)
    out["decode_b8h8n4096_interp_over_int"] = round(us_dp / us_di, 3)
    del qc, kc, vc, qd, od, ld

    # a 16-layer stack in one call (fwd_layers / bwd_layers: [16, B, H, N, D] inputs, distinct
    # per layer, so no layer's rows are cache-resident: 0.8 GB of Q, K, V at B4 H8 N4096) vs
    # 16 single-layer calls over the same stack; N(0, 1) draws made on the device
    out.update(layer_stacks(dev, stream, args, al4, al2, al3))
    out.update(dropped_mass_diag(dev, stream, args))
    return out


def dropped_mass_diag(dev, stream, args):
    """The dropped-attention-mass diagnostic at the 4x-extrapolation shape (B4 H8 N4096, alpha 1):
    the dense causal LSE kernel (bf16 MFMA, causal half of Q K^T) timed alone, and the mean
    dropped mass of the Fibonacci and power-of-two bases."""
    import torch

    import fibonacci_offset_dilated_amd as F
    from fibonacci_offset_dilated_amd.synthetic import seed_for
    from fibonacci_offset_dilated_amd.workloads import BY_CONFIG, FIB_BASE, POW2_BASE

    w = BY_CONFIG[4]
    (q, k, v), _ = make_inputs(w.B, w.H, w.N, seed_for(4, 0, 12, 0), False, dev)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    ws = torch.empty(int(F.lib().fib_dense_lse_workspace_size(w.B, w.H, w.N, D, F.BF16)), dtype=torch.uint8,
                     device=dev)
    reps = max(5, args.steps // 5)
    ms = time_calls(lambda: F.dense_lse(q, k, 10000.0, lse=lse, workspace=ws), reps, 2, stream)
    logits = w.B * w.H * (w.N * (w.N + 1) / 2)
    flops = logits * D * 2
    # VALU floor of the online log-sum-exp: per logit a max, an FMA and an add at full rate and
    # one exp2 at quarter rate = 7 full-rate lane operations; 256 CUs x 4 SIMDs x 16 lanes x
    # 2.4 GHz = 39.3e12 lane operations/s (no packed fp32 math)
    valu_floor_s = logits * 7 / (256 * 4 * 16 * 2.4e9)
    out = {"dense_lse_b4h8n4096_us": round(ms * 1e3, 2),
           "dense_lse_b4h8n4096_tflops": round(flops / (ms * 1e-3) / 1e12, 1),
           "dense_lse_b4h8n4096_mfma_frac": round(flops / (ms * 1e-3) / 1e12 / 2500.0, 4),
           "dense_lse_b4h8n4096_valu_floor_us": round(valu_floor_s * 1e6, 1),
           "dense_lse_b4h8n4096_valu_frac": round(valu_floor_s / (ms * 1e-3), 4)}
    for name, base in (("fib", FIB_BASE), ("pow2", POW2_BASE)):
        dm = F.dropped_mass(q, k, v, 12, 1.0, base)
        out[f"dropped_mass_b4h8n4096_{name}_mean"] = round(float(dm.mean().item()), 4)
    return out


def layer_stacks(dev, stream, args, al4, al2, al3):
    import torch

    import fibonacci_offset_dilated_amd as F
    from fibonacci_offset_dilated_amd.synthetic import seed_for
    from fibonacci_offset_dilated_amd.workloads import BY_CONFIG, FIB_BASE, INT, INTERP

    reps = max(5, args.steps // 5)
    # each timing warms up for 10 calls of its own (a 16-layer call is 0.2-1 ms of work: fewer
    # leave the clocks ramping and favour whichever variant is timed later)
    warm = 10
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed_for(4, 0, 12, 16))
    L = 16

    def stack(w, n):
        return [torch.randn((L, w.B, w.H, w.N, D), generator=gen, device=dev).to(torch.bfloat16) for _ in range(n)]

    out = {}
    plan = torch.empty(F.layers_plan_bytes(L), dtype=torch.uint8, device=dev)
    w4 = BY_CONFIG[4]
    q, k, v = stack(w4, 3)
    o = torch.empty_like(q)
    lse = torch.empty((L, w4.B, w4.H, w4.N), dtype=torch.float32, device=dev)
    a4 = np.array(al4, dtype=np.float32)
    us_f = time_calls(lambda: F.fwd_layers(q, k, v, 12, a4, FIB_BASE, 10000.0, INT, out=o, lse=lse, plan=plan),
                      reps, warm, stream) * 1e3 / L
    us_s = time_calls(lambda: [F.fwd(q[l], k[l], v[l], 12, a4[l], FIB_BASE, 10000.0, INT, out=o[l], lse=lse[l])
                               for l in range(L)], reps, warm, stream) * 1e3 / L
    rows4 = w4.B * w4.H * w4.N
    out["c4_stack16_fwd_int_us_per_layer"] = round(us_f, 2)
    out["c4_stack16_fwd_int_hbm_frac"] = round(rows4 * (4 * D * 2 + 4) / (us_f * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    out["c4_stack16_separate_calls_us_per_layer"] = round(us_s, 2)
    del q, k, v, o, lse

    w2 = BY_CONFIG[3]
    q, k, v, do = stack(w2, 4)
    o = torch.empty_like(q)
    lse = torch.empty((L, w2.B, w2.H, w2.N), dtype=torch.float32, device=dev)
    a2 = np.array(al2, dtype=np.float32)
    a3 = np.asarray(al3, dtype=np.float32)
    us_fi = time_calls(lambda: F.fwd_layers(q, k, v, 12, a2, FIB_BASE, 10000.0, INT, out=o, lse=lse, plan=plan),
                       reps, warm, stream) * 1e3 / L
    us_si = time_calls(lambda: [F.fwd(q[l], k[l], v[l], 12, a2[l], FIB_BASE, 10000.0, INT, out=o[l], lse=lse[l])
                                for l in range(L)], reps, warm, stream) * 1e3 / L
    us_fp = time_calls(lambda: F.fwd_layers(q, k, v, 12, a3, FIB_BASE, 10000.0, INTERP, out=o, lse=lse, plan=plan),
                       reps, warm, stream) * 1e3 / L
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    us_fb = us_sb = None
    if args.bwd_stacks:
        # (off by default: a GPU memory fault was first seen at a layer-stack backward test
        # case, and its cause is not yet shown)
        dal = torch.empty(L, dtype=torch.float32, device=dev)
        ws = torch.empty(F.bwd_workspace_size(L * w2.B, w2.H, w2.N, D, F.BF16, INTERP), dtype=torch.uint8,
                         device=dev)
        us_fb = time_calls(lambda: F.bwd_layers(q, k, v, o, lse, do, 12, a3, FIB_BASE, 10000.0, INTERP, dq=dq, dk=dk,
                                                dv=dv, dalpha=dal, workspace=ws, plan=plan), reps, warm,
                           stream) * 1e3 / L
        ws1 = torch.empty(F.bwd_workspace_size(w2.B, w2.H, w2.N, D, F.BF16, INTERP), dtype=torch.uint8, device=dev)
        dal1 = torch.empty(1, dtype=torch.float32, device=dev)
        us_sb = time_calls(lambda: [F.bwd(q[l], k[l], v[l], o[l], lse[l], do[l], 12, a3[l], FIB_BASE, 10000.0,
                                          INTERP, dq=dq[l], dk=dk[l], dv=dv[l], dalpha=dal1, workspace=ws1)
                                    for l in range(L)], reps, warm, stream) * 1e3 / L
        del ws
    rows2 = w2.B * w2.H * w2.N
    out["b8h8n1024_stack16_fwd_int_us_per_layer"] = round(us_fi, 2)
    out["b8h8n1024_stack16_fwd_int_hbm_frac"] = round(rows2 * (4 * D * 2 + 4) / (us_fi * 1e-6) / 1e9 / HBM_PEAK_GBS,
                                                      4)
    out["b8h8n1024_stack16_separate_calls_fwd_int_us_per_layer"] = round(us_si, 2)
    out["b8h8n1024_stack16_fwd_interp_us_per_layer"] = round(us_fp, 2)
    if us_fb is not None:
        out["b8h8n1024_stack16_bwd_interp_us_per_layer"] = round(us_fb, 2)
        out["b8h8n1024_stack16_separate_calls_bwd_interp_us_per_layer"] = round(us_sb, 2)
    del q, k, v, do, o, lse, dq, dk, dv

    # decode over a 16-layer cache stack at B8 H8 N4096 in one launch
    kc, vc = [torch.randn((L, 8, 8, 4096, D), generator=gen, device=dev).to(torch.bfloat16) for _ in range(2)]
    qd = torch.randn((L, 8, 8, D), generator=gen, device=dev).to(torch.bfloat16)
    od = torch.empty_like(qd)
    ld = torch.empty((L, 8, 8), dtype=torch.float32, device=dev)
    for mode, a, name in ((INT, a2, "int"), (INTERP, a3, "interp")):
        us_d = time_calls(lambda: F.decode_layers(qd, kc, vc, 12, a, FIB_BASE, 10000.0, mode, out=od, lse=ld,
                                                  plan=plan), reps, warm, stream) * 1e3 / L
        out[f"decode_b8h8n4096_stack16_{name}_us_per_layer"] = round(us_d, 2)
    return out


def sweep(path, dev, stream, reps):
    """One JSONL record per (workload, base, W, mode, pass, layer): GPU time per call from HIP
    events around each call, tokens/s (B*H*N per layer), algorithmic GB/s and % of the 8 TB/s
    peak, and the table size. Each layer has its own N(0, 1) inputs drawn on the device (seeded
    by the workload recipe), so a 16-layer stack exceeds the 256 MB Infinity Cache and every
    call reads cold data; the layers are called in turn, `reps` times."""
    import torch

    import fibonacci_offset_dilated_amd as F
    from fibonacci_offset_dilated_amd.synthetic import seed_for, uniform_alphas
    from fibonacci_offset_dilated_amd.workloads import (INT, INTERP, UNIFORM_ALPHA_RANGE, UNIFORM_ALPHA_SEED,
                                                        WORKLOADS)

    def alpha_for(w, l):
        if w.schedule == "fixed1":
            return F.schedule_alpha(F.SCHED_FIXED, l, 16)
        if w.schedule == "linear":
            return F.schedule_alpha(F.SCHED_LINEAR, l, 16)
        if w.schedule == "coprime":
            return F.schedule_alpha(F.SCHED_COPRIME, l, 16)
        if w.schedule == "layer15_linear":
            return F.schedule_alpha(F.SCHED_LINEAR, 15, 16)
        return uniform_alphas(UNIFORM_ALPHA_SEED, 16, *UNIFORM_ALPHA_RANGE)[l]

    out = open(path, "w")
    summary = []
    for w in WORKLOADS:
        dt = torch.float32 if w.dtype == F.F32 else torch.bfloat16
        esize = 4 if w.dtype == F.F32 else 2
        for base_id, base in w.bases:
            inputs = {}
            for l in w.layers:
                g = torch.Generator(device=dev)
                g.manual_seed(seed_for(w.config, base_id, 0, l))
                inputs[l] = [torch.randn((w.B, w.H, w.N, D), generator=g, device=dev).to(dt)
                             for _ in range(4 if w.backward else 3)]
            for W in w.windows:
                for mode in (w.mode,) + tuple(w.extra_modes):
                    passes = ("fwd", "bwd") if w.backward else ("fwd",)
                    fw = {}
                    for l in w.layers:
                        q, k, v = inputs[l][:3]
                        fw[l] = F.fwd(q, k, v, W, alpha_for(w, l), base, w.theta, mode)
                    for ps in passes:
                        ws = None
                        if ps == "bwd":
                            ws = torch.empty(F.bwd_workspace_size(w.B, w.H, w.N, D, w.dtype, mode), dtype=torch.uint8,
                                             device=dev)
                            grads = [torch.empty_like(inputs[w.layers[0]][0]) for _ in range(3)]
                            dal = torch.empty(1, dtype=torch.float32, device=dev)

                        def call(l):
                            q, k, v = inputs[l][:3]
                            o, lse = fw[l]
                            if ps == "fwd":
                                F.fwd(q, k, v, W, alpha_for(w, l), base, w.theta, mode, out=o, lse=lse)
                            else:
                                F.bwd(q, k, v, o, lse, inputs[l][3], W, alpha_for(w, l), base, w.theta, mode,
                                      dq=grads[0], dk=grads[1], dv=grads[2], dalpha=dal, workspace=ws)

                        for _ in range(max(3, -(-20 // len(w.layers)))):  # >= 20 warm-up calls (clocks)
                            for l in w.layers:
                                call(l)
                        ev = {l: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                                  for _ in range(reps)] for l in w.layers}
                        torch.cuda.synchronize()
                        for r in range(reps):
                            for l in w.layers:
                                ev[l][r][0].record(stream)
                                call(l)
                                ev[l][r][1].record(stream)
                        torch.cuda.synchronize()
                        per = []
                        for l in w.layers:
                            us = 1e3 * sum(a.elapsed_time(b) for a, b in ev[l]) / reps
                            rows = w.B * w.H * w.N
                            nbytes = rows * ((4 if ps == "fwd" else 8) * D * esize + 4)
                            gbs = nbytes / (us * 1e-6) / 1e9
                            n_tab = len(F.offset_table(alpha_for(w, l), base, W, mode)[0])
                            rec = {"workload": w.name, "config": w.config, "base": "fibonacci" if base_id == 0 else
                                   "power_of_two", "W": W, "mode": "integer" if mode == INT else "interpolated",
                                   "pass": ps, "layer": l, "alpha": float(alpha_for(w, l)), "table_entries": n_tab,
                                   "us_per_call": round(us, 3), "tokens_per_s": rows / (us * 1e-6),
                                   "algorithmic_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                                   "dtype": "f32" if w.dtype == F.F32 else "bf16",
                                   "seed": seed_for(w.config, base_id, 0, l), "reps": reps}
                            out.write(json.dumps(rec) + "\n")
                            per.append(us)
                        line = (f"{w.name} base={base_id} W={W} mode={mode} {ps}: us/call mean {sum(per) / len(per):.1f} "
                                f"min {min(per):.1f} max {max(per):.1f}; hbm frac mean "
                                f"{nbytes / (sum(per) / len(per) * 1e-6) / 1e9 / HBM_PEAK_GBS:.3f}")
                        summary.append(line)
                        log(line)
            del inputs, fw
            torch.cuda.empty_cache()
    out.close()
    return summary


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20, help="untimed steps first (the GPU clocks ramp up)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-components", action="store_true")
    ap.add_argument("--bwd-stacks", action="store_true",
                    help="also time the 16-layer backward stack (held off by default: a GPU memory fault was "
                         "first seen at a layer-stack backward test case)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="run one 1 GiB device-to-device copy first (reference for HBM byte counters)")
    ap.add_argument("--sweep", metavar="JSONL",
                    help="measurement aid: time every workload's layers, windows, bases, modes and passes "
                         "(one JSONL record each) instead of the bench line")
    ap.add_argument("--bwd-only", action="store_true",
                    help="profiling aid: one forward, then only backward calls (--warmup untimed, --steps "
                         "timed); prints their time, not the bench line")
    ap.add_argument("--bwd-mode", choices=("int", "interp"), default="int",
                    help="offset mode of the --bwd-only calls")
    ap.add_argument("--memprobe", action="store_true",
                    help="measurement aid: run the memory-delivery probe (the long-context forward's loads and "
                         "stores without its arithmetic, in several lane layouts and far distances); prints "
                         "one JSON line per variant instead of the bench line")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path. Heads (B*H) are "
              "independent, so the op would shard over them with no communication, plus one "
              "d(alpha) all-reduce per layer in the backward. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.memprobe:
        # a child process of its own (built by fibonacci_offset_dilated_amd.build)
        import subprocess
        exe = os.path.join(ROOT, "fibonacci_offset_dilated_amd", "probe", "memprobe")
        if not os.path.exists(exe):
            raise SystemExit(f"{exe} is missing: build first (python -m fibonacci_offset_dilated_amd.build)")
        sys.exit(subprocess.run([exe]).returncode)

    import torch

    import fibonacci_offset_dilated_amd as F
    from fibonacci_offset_dilated_amd.synthetic import seed_for
    from fibonacci_offset_dilated_amd.workloads import BY_CONFIG, FIB_BASE, INT, INTERP

    w = BY_CONFIG[5]
    B, H, N, W = w.B, w.H, w.N, 12
    alpha = F.schedule_alpha(F.SCHED_LINEAR, 15, 16)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    F.lib()
    if args.sweep:
        sweep(args.sweep, dev, torch.cuda.current_stream(), max(3, args.steps // 10))
        return
    log(f"inputs B={B} H={H} N={N} D={D} bf16 (seeded)")
    (q, k, v, do), arrs = make_inputs(B, H, N, seed_for(5, 0, 12, 15), True, dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    if args.calibration_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def fwd_int():
        F.fwd(q, k, v, W, alpha, FIB_BASE, 10000.0, INT, out=o, lse=lse)

    if args.bwd_only:
        bmode = INT if args.bwd_mode == "int" else INTERP
        F.fwd(q, k, v, W, alpha, FIB_BASE, 10000.0, bmode, out=o, lse=lse)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        dal = torch.empty(1, dtype=torch.float32, device=dev)
        ws = torch.empty(F.bwd_workspace_size(B, H, N, D, F.BF16, bmode, W, alpha, FIB_BASE), dtype=torch.uint8,
                         device=dev)
        log(f"timing {args.bwd_mode} backward only")
        ms_b = time_calls(lambda: F.bwd(q, k, v, o, lse, do, W, alpha, FIB_BASE, 10000.0, bmode, dq=dq, dk=dk, dv=dv,
                                        dalpha=dal, workspace=ws), args.steps, args.warmup, stream)
        print(json.dumps({"profiling_aid": f"bwd_{args.bwd_mode}",
                          "workload": "long_context_b1h32_n131072_bf16_w12_fib987_alpha1.5",
                          "ms_per_call": ms_b, "steps": args.steps, "warmup": args.warmup}), flush=True)
        return

    log("timing integer forward")
    ms = time_calls(fwd_int, args.steps, args.warmup, stream)
    rows = B * H * N
    bytes_per_launch = rows * (4 * D * 2 + 4)  # read Q, K, V; write O (bf16) and LSE (fp32)
    achieved = bytes_per_launch / (ms * 1e-3) / 1e9
    workload = "long_context_b1h32_n131072_bf16_w12_fib987_alpha1.5"
    traffic = measured_traffic("fwd_int", workload)

    components = None
    if not args.no_components:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        dal = torch.empty(1, dtype=torch.float32, device=dev)
        ws = torch.empty(F.bwd_workspace_size(B, H, N, D, F.BF16, INTERP), dtype=torch.uint8, device=dev)
        o2 = torch.empty_like(q)
        lse2 = torch.empty_like(lse)

        def fwd_interp():
            F.fwd(q, k, v, W, alpha, FIB_BASE, 10000.0, INTERP, out=o2, lse=lse2)

        def bwd(mode, oo, ll):
            return lambda: F.bwd(q, k, v, oo, ll, do, W, alpha, FIB_BASE, 10000.0, mode, dq=dq, dk=dk, dv=dv,
                                 dalpha=dal, workspace=ws)

        log("timing interpolated forward and both backwards")
        fwd_interp()
        ms_interp = time_calls(fwd_interp, args.steps, args.warmup, stream)
        ms_bwd_int = time_calls(bwd(INT, o, lse), 5, 2, stream)
        ms_bwd_interp = time_calls(bwd(INTERP, o2, lse2), 5, 2, stream)
        bwd_bytes = rows * (8 * D * 2 + 4)
        components = {
            "fwd_int_ms": round(ms, 4),
            "fwd_interp_ms": round(ms_interp, 4),
            "interp_over_int": round(ms_interp / ms, 3),
            "bwd_int_ms": round(ms_bwd_int, 4),
            "bwd_interp_ms": round(ms_bwd_interp, 4),
            "fwd_interp_hbm_frac": round(bytes_per_launch / (ms_interp * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "bwd_int_hbm_frac": round(bwd_bytes / (ms_bwd_int * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "bwd_interp_hbm_frac": round(bwd_bytes / (ms_bwd_interp * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        }

    if not args.no_components:
        components["small_configs"] = small_configs(dev, stream, args)

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(arrs, B, H, N, W, alpha, FIB_BASE, INT, args.cpu_budget)

    out = {
        "metric": "sparse-attn fwd tokens/s per layer (B*H*N)",
        "value": rows / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload, "B": B, "H": H, "N": N, "D": D, "W": W, "alpha": float(alpha),
                   "base": "fibonacci 1..987", "mode": "integer", "rope_theta": 10000.0},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "bytes_per_launch": bytes_per_launch},
        "cpu_baseline": cpu,
        # each (b, h, i) is one query vector: B*H*N per call (= value); B*N sequence positions
        "queries_per_s": rows / (ms * 1e-3),
        "positions_per_s": B * N / (ms * 1e-3),
        "components": components,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
