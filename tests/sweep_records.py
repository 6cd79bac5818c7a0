"""Results records of the measured workloads, with their parity.

Runs bench.py's per-layer timing sweep (one record per workload, base, W, mode, pass and
layer) and extends each record with its parity against the fp64 oracle on the same
configuration:

* ``max_abs_err_o`` and ``max_abs_err_lse`` (forward records): over sampled query rows
  (128 evenly spaced rows and the last 16) of two heads, the first and the last;
* ``max_abs_err_dq`` (backward records): over the same rows; ``max_abs_err_dk`` and
  ``max_abs_err_dv`` over the whole first head where N <= 4096 (the oracle's dK and dV of a
  row need every query that reads it); ``dalpha_err_over_bound`` where the oracle's dalpha is
  computed over all heads (N <= 4096);
* ``index_set_match``: the device export of the attended rows (fib_sparse_attn_index_set)
  equals the oracle's index_sets exactly;
* ``oracle_tokens_per_s`` (N <= 4096): the fp64 oracle's rate on the same layer call (the
  whole forward, or the whole backward), timed with time.perf_counter on the host cores of
  the same box, one worker process per core (``oracle_cores``), median of 3 runs.

The parity inputs follow the workload recipe (seeded N(0, 1) draws rounded to the workload
dtype, one set per layer); the timing inputs are drawn on the device, as in the sweep.

Usage (one GPU): python tests/sweep_records.py OUT.jsonl [--reps 3]
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
for p in (ROOT, HERE):
    if p not in sys.path:
        sys.path.insert(0, p)

import bench  # noqa: E402
import oracle as O  # noqa: E402
from gpu_util import dalpha_bound, host, to_device  # noqa: E402


def sample_rows(N):
    rows = np.unique(np.concatenate([np.linspace(0, N - 1, 128).astype(np.int64), np.arange(max(0, N - 16), N)]))
    return rows


def parity(w, base_id, base, layer, alpha_of, modes, say):
    """Parity fields per (W, mode, pass) for one layer's inputs."""
    import fibonacci_offset_dilated_amd as F
    from fibonacci_offset_dilated_amd.synthetic import normal_inputs, seed_for

    shape = (w.B, w.H, w.N, w.D)
    arrs = normal_inputs(seed_for(w.config, base_id, 0, layer), shape, with_dout=w.backward)
    dev = [to_device(a, w.dtype) for a in arrs]
    del arrs
    heads = [(0, 0), (w.B - 1, w.H - 1)]
    rows = sample_rows(w.N)
    alpha = alpha_of(w, layer)
    workers = min(16, len(os.sched_getaffinity(0)))
    tokens = w.B * w.H * w.N

    def oracle_rate(fn):
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return {"oracle_tokens_per_s": tokens / statistics.median(ts), "oracle_cores": workers}

    out = {}
    for W in w.windows:
        for mode in modes:
            (q, q64), (k, k64), (v, v64) = dev[:3]
            o, lse = F.fwd(q, k, v, W, alpha, base, w.theta, mode)
            oh, lh = host(o), host(lse)
            eo = el = 0.0
            for b, h in heads:
                ro, rl = O.forward_rows(q64[b, h], k64[b, h], v64[b, h], rows, W, alpha, base, w.theta, mode)
                eo = max(eo, float(np.abs(oh[b, h][rows] - ro).max()))
                el = max(el, float(np.abs(lh[b, h][rows] - rl).max()))
            ix = host(F.index_set(w.N, W, alpha, base, mode))
            match = bool(np.array_equal(ix, O.index_sets(w.N, W, alpha, base, mode)))
            rec = {"max_abs_err_o": eo, "max_abs_err_lse": el, "index_set_match": match,
                   "parity_sample": f"rows {len(rows)} of heads {heads}"}
            if w.N <= 4096:
                rec.update(oracle_rate(lambda: O.forward(q64, k64, v64, W, alpha, base, w.theta, mode,
                                                         workers=workers)))
            out[(W, mode, "fwd")] = rec
            say(f"  {w.name} base {base_id} layer {layer} W {W} mode {mode} fwd: O {eo:.2e} LSE {el:.2e} "
                f"index set {'match' if match else 'MISMATCH'}")
            if w.backward:
                (do, d64) = dev[3]
                dq, dk, dv, da = F.bwd(q, k, v, o, lse, do, W, alpha, base, w.theta, mode)
                dqh = host(dq)
                edq = 0.0
                for b, h in heads:
                    rq, _, _, _ = O.backward(q64[b, h][None, None], k64[b, h][None, None], v64[b, h][None, None],
                                             d64[b, h][None, None], W, alpha, base, w.theta, mode, rows=rows)
                    edq = max(edq, float(np.abs(dqh[b, h][rows] - rq[0, 0][rows]).max()))
                brec = {"max_abs_err_dq": edq, "index_set_match": match,
                        "parity_sample": f"dQ rows {len(rows)} of heads {heads}"}
                if w.N <= 4096:
                    rq, rk, rv, ra, rsc = O.backward(q64, k64, v64, d64, W, alpha, base, w.theta, mode,
                                                     workers=workers, return_scale=True)
                    brec.update(oracle_rate(lambda: O.backward(q64, k64, v64, d64, W, alpha, base, w.theta, mode,
                                                               workers=workers)))
                    brec["max_abs_err_dq"] = float(np.abs(dqh - rq).max())
                    brec["max_abs_err_dk"] = float(np.abs(host(dk) - rk).max())
                    brec["max_abs_err_dv"] = float(np.abs(host(dv) - rv).max())
                    brec["parity_sample"] = "every row of every head"
                    if mode == F.INTERP:
                        err = abs(float(da.item()) - ra)
                        brec["dalpha"] = float(da.item())
                        brec["dalpha_ref"] = float(ra)
                        brec["dalpha_err_over_bound"] = err / max(dalpha_bound(rsc, w.dtype), 1e-30)
                out[(W, mode, "bwd")] = brec
                say(f"  {w.name} base {base_id} layer {layer} W {W} mode {mode} bwd: "
                    + ", ".join(f"{k2} {v2:.2e}" for k2, v2 in brec.items() if isinstance(v2, float)))
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("out")
    ap.add_argument("--reps", type=int, default=3)
    args = ap.parse_args()

    import torch

    import fibonacci_offset_dilated_amd as F
    from fibonacci_offset_dilated_amd.synthetic import uniform_alphas
    from fibonacci_offset_dilated_amd.workloads import UNIFORM_ALPHA_RANGE, UNIFORM_ALPHA_SEED, WORKLOADS

    def say(*a):
        print(*a, flush=True)

    def alpha_of(w, l):
        if w.schedule == "fixed1":
            return F.schedule_alpha(F.SCHED_FIXED, l, 16)
        if w.schedule == "linear":
            return F.schedule_alpha(F.SCHED_LINEAR, l, 16)
        if w.schedule == "coprime":
            return F.schedule_alpha(F.SCHED_COPRIME, l, 16)
        if w.schedule == "layer15_linear":
            return F.schedule_alpha(F.SCHED_LINEAR, 15, 16)
        return np.float32(uniform_alphas(UNIFORM_ALPHA_SEED, 16, *UNIFORM_ALPHA_RANGE)[l])

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    timing_path = args.out + ".timing"
    say("timing sweep")
    bench.sweep(timing_path, dev, torch.cuda.current_stream(), args.reps)
    records = [json.loads(line) for line in open(timing_path)]
    os.remove(timing_path)

    par = {}
    for w in WORKLOADS:
        modes = (w.mode,) + tuple(w.extra_modes)
        for base_id, base in w.bases:
            for layer in w.layers:
                for (W, mode, ps), rec in parity(w, base_id, base, layer, alpha_of, modes, say).items():
                    par[(w.name, base_id, W, mode, ps, layer)] = rec
                torch.cuda.empty_cache()
    with open(args.out, "w") as f:
        for r in records:
            key = (r["workload"], 0 if r["base"] == "fibonacci" else 1, r["W"],
                   F.INT if r["mode"] == "integer" else F.INTERP, r["pass"], r["layer"])
            r.update(par.get(key, {}))
            f.write(json.dumps(r) + "\n")
    say(f"wrote {len(records)} records to {args.out}")


if __name__ == "__main__":
    main()
