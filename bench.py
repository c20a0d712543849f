#!/usr/bin/env python3
"""Benchmark of the exact causal attention backward (attn_bwd) on one MI355X.

One step = one attn_bwd over the whole workload: the preprocess (D), the
dK/dV kernel and the dQ kernel, launched back to back by the C ABI entry
point on torch's current stream.  Inputs, O and L (from attn_fwd_lse) are
resident in HBM before the timed region starts.  A second timed region runs
the same steps through the three stage entry points with HIP events between
the kernels, for the per-stage times and the roofline.

Prints one JSON line.  `value` is attn_bwd TFLOP/s with FLOPs counted as
10 * d * (kept pairs), kept pairs = B*H*N(N+1)/2 causal, over the first
region's wall time.  `roofline` covers the dominant kernel (dK/dV): its
algorithmic FLOPs (8 * d * pairs: S, dP, dV, dK) over its mean duration from
the HIP events recorded around it on the launch stream in the second region,
against the bf16 dense MFMA peak.  `cpu_baseline` times the
fp64 oracle on whole (batch, head) slices of the same workload on the host
cores (a bounded sample of about CPU_BASELINE_SECONDS).

Other workloads (--workload) time other steps the same way: the backward of
the backward (op "bob", 24 * d algorithmic FLOPs per kept pair: S, dP, G as
two, A, then hQ, hK and hdO as two each and hV; the 44 * d its three passes
execute, recomputation included, is reported beside it; its one call as the
roofline) and the forward alone (op "fwd", 4 * d per kept pair: S and P V,
its one kernel as the roofline, the oracle's forward as the CPU baseline).

Secondary denominators, measured after the timed region on the same GPU:
`denominators.copy_gbs` (a 1 GiB cast copy, bytes read + written per second)
and `denominators.gemm_bf16_tflops` (plain 8192^3 bf16 matrix products through
torch, which runs the vendor GEMM library), both sustained over back-to-back
calls, with the backward's value as a fraction of each.  `device_mem_delta_bytes` is the drop in free device
memory across one synchronised backward step (no N x N buffer: 0 expected).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "causal attention bwd TFLOP/s and % of bf16 MFMA peak at N=16K, d=128"
PEAK = {"bf16": 2516.6, "f32": 157.3}          # dense MFMA TFLOP/s, MI355X spec
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "dkdv_c5_long_traffic.json")
# the dominant kernel at the bench workload and the sources it is built from
DOMINANT_KERNEL = "bwd_dkdv_bf16_kernel"
KERNEL_SOURCES = ("exact_softmax_attention_attn_amd/csrc/attn_bwd_pipe.hip",
                  "exact_softmax_attention_attn_amd/csrc/common.h")
CPU_BASELINE_SECONDS = 12.0    # the oracle runs whole heads until this much time has passed


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def pairs(B, H, N, causal=True, block_mask=None, mask_block=128):
    """Kept (query, key) pairs: causal or full, within the kept blocks of a
    shared block mask if one is given."""
    if block_mask is None:
        return B * H * (N * (N + 1) // 2 if causal else N * N)
    total = 0
    for r, c in zip(*block_mask.nonzero()):
        rows = min(mask_block, N - r * mask_block)
        cols = min(mask_block, N - c * mask_block)
        if not causal or c < r:
            total += rows * cols
        elif c == r:
            total += rows * (rows + 1) // 2
    return B * H * total


def traffic_record():
    """HBM bytes per dK/dV launch from committed rocprofv3 counters, if still valid."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w, x, bm=None, cot=None, op="bwd"):
    """The oracle as it stands, on whole (batch, head) slices of the workload.

    Heads run one after another until CPU_BASELINE_SECONDS have passed (at
    least one), so the sample stays bounded; the rate is scaled by the FLOPs
    of the heads actually run.
    """
    import numpy as np
    from oracle import attn_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()
                       if p.get("user_api") == "blas"] or [os.cpu_count()])
    except Exception:  # pragma: no cover - threadpoolctl missing
        threads = os.cpu_count()
    done, spent = 0, 0.0
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    for b, h in heads:
        q, k, v, do = (x[n][b:b + 1, :, h:h + 1].astype(np.float64) for n in ("q", "k", "v", "do"))
        t0 = time.perf_counter()
        if op == "fwd":
            orc.attn_fwd(q, k, v, w.scale, w.causal, bm)
        elif cot is None:
            orc.attn_bwd(q, k, v, do, w.scale, w.causal, bm)
        else:
            gq, gk, gv = (cot[n][b:b + 1, :, h:h + 1].astype(np.float64) for n in ("gq", "gk", "gv"))
            orc.attn_bwd_bwd(q, k, v, do, gq, gk, gv, w.scale, w.causal, bm)
        spent += time.perf_counter() - t0
        done += 1
        if spent >= CPU_BASELINE_SECONDS:
            break
    per = 4 if op == "fwd" else (10 if cot is None else 24)
    fn = "attn_fwd" if op == "fwd" else ("attn_bwd" if cot is None else "attn_bwd_bwd")
    flops = per * w.d * pairs(1, 1, w.N, w.causal, bm) * done
    return {"value": round(flops / spent / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} of {len(heads)} (batch, head) slices of {w.name} (N={w.N}, d={w.d}, "
                      f"{'causal' if w.causal else 'full'}), fp64 numpy oracle {fn}, "
                      f"{spent:.1f} s; TFLOP/s from {per}*d*pairs of the slices run"}


def summarize_pmc(fetch_dirs, write_dirs, calib_mib):
    """HBM bytes per dK/dV launch from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs.

    Each counter is read in KiB per dispatch.  The run's calibration kernel (a
    dtype-cast copy of calib_mib MiB in, calib_mib MiB out, the largest
    'copy' dispatch of the run) gives the factor from counter KiB to bytes.
    """
    import csv
    import glob

    def per_dispatch(dirs, counter):
        rows = {}
        for d in dirs:
            for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
                for r in csv.DictReader(open(f)):
                    if r["Counter_Name"] != counter:
                        continue
                    key = (f, r["Dispatch_Id"])
                    rows[key] = (r["Kernel_Name"], float(r["Counter_Value"]))
        return list(rows.values())

    out = {}
    for counter, dirs in (("FETCH_SIZE", fetch_dirs), ("WRITE_SIZE", write_dirs)):
        rows = per_dispatch(dirs, counter)
        dk = [v for n, v in rows if DOMINANT_KERNEL in n]
        cp = [v for n, v in rows if "copy" in n.lower()]
        if not dk or not cp:
            raise SystemExit(f"{counter}: no {DOMINANT_KERNEL} or copy dispatch found")
        factor = calib_mib * (1 << 20) / max(cp)          # bytes per counter unit
        out[counter] = {"kernel_kib_mean": sum(dk) / len(dk), "dispatches": len(dk),
                        "copy_kib": max(cp), "bytes_per_unit": factor,
                        "bytes_per_launch": sum(dk) / len(dk) * factor}
    rec = {"kernel": DOMINANT_KERNEL, "kernel_source_sha256": kernel_source_hash(),
           "calibration_copy_mib": calib_mib,
           "fetch_bytes_per_launch": round(out["FETCH_SIZE"]["bytes_per_launch"]),
           "write_bytes_per_launch": round(out["WRITE_SIZE"]["bytes_per_launch"]),
           "counters": out}
    rec["bytes_per_launch"] = rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    return rec


def measure_denominators(torch, dev):
    """Measured copy bandwidth and library GEMM rate on this GPU, sustained: the
    median over 3 rounds of the mean time per call of 20 back-to-back calls."""
    import numpy as np
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(fn, calls=20, rounds=3):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        t = []
        for _ in range(rounds):
            ev[0].record()
            for _ in range(calls):
                fn()
            ev[1].record()
            torch.cuda.synchronize()
            t.append(ev[0].elapsed_time(ev[1]) / calls)
        return float(np.median(t)) * 1e-3

    n = (1 << 30) // 4
    a = torch.ones(n, dtype=torch.float32, device=dev)
    b = torch.empty(n, dtype=torch.int32, device=dev)
    copy_s = timed(lambda: b.copy_(a))           # a cast copy runs as a kernel
    del a, b
    m = 8192
    x = torch.randn(m, m, device=dev).to(torch.bfloat16).contiguous()
    y = torch.randn(m, m, device=dev).to(torch.bfloat16).contiguous()
    gemm_s = timed(lambda: torch.matmul(x, y))
    del x, y
    torch.cuda.synchronize()
    return {"copy_gbs": round(2 * (1 << 30) / copy_s / 1e9, 1),
            "gemm_bf16_tflops": round(2 * m ** 3 / gemm_s / 1e12, 1),
            "gemm_shape": f"{m}x{m}x{m} bf16, torch.matmul (vendor library), 20 calls back to back"}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c5_long")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one plain copy of this many MiB (counter calibration runs)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the dK/dV traffic record from two rocprofv3 --pmc output dirs "
                         "(FETCH_SIZE run, WRITE_SIZE run, both with --copy-calibration-mib)")
    args = ap.parse_args(argv)

    if args.summarize_pmc:
        rec = summarize_pmc([args.summarize_pmc[0]], [args.summarize_pmc[1]],
                            args.copy_calibration_mib or 1024)
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec))
        return 0

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: this build "
              "runs on a single GPU (every (batch, head) is independent, so heads would shard "
              "across GPUs with no communication, one process per GPU)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from exact_softmax_attention_attn_amd import binding, workloads

    binding.load()
    w = workloads.get(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] {w.name}: inputs", file=sys.stderr, flush=True)
    x = workloads.make_inputs(w, seed=0)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q, k, v, do = (torch.from_numpy(x[n]).to(dev).to(tdt) for n in ("q", "k", "v", "do"))
    bm = workloads.workload_mask(w)               # block-sparse workloads: a shared mask
    mask = None if bm is None else torch.from_numpy(bm).to(dev)

    def forward(o=None, lse=None):
        if mask is None:
            return binding.attn_fwd_lse(q, k, v, causal=w.causal, scale=w.scale, o=o, lse=lse)
        return binding.attn_fwd_lse_masked(q, k, v, mask, causal=w.causal, scale=w.scale, o=o,
                                           lse=lse)

    o, lse = forward()                            # the backward's O and L
    # the forward's own timed calls write into buffers of their own, allocated here
    o_f, lse_f = torch.empty_like(o), torch.empty_like(lse)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = binding.new_workspace(w.B, w.H, w.N, dev)
    cot = None
    if w.op == "bob":
        # the backward of the backward: cotangents of dQ, dK, dV in, hQ, hK, hV, hdO out
        cot = workloads.make_cotangents(w.B, w.H, w.N, w.d, w.dtype, seed=0)
        gq, gk, gv = (torch.from_numpy(cot[n]).to(dev).to(tdt) for n in ("gq", "gk", "gv"))
        hq, hdo = torch.empty_like(q), torch.empty_like(q)
        ws = torch.empty((4, w.B, w.H, w.N), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step_bob(ev=None):
        if ev is not None:
            ev[0].record()
            ev[1].record()
            ev[2].record()
        binding.attn_bwd_bwd(q, k, v, o, do, lse, gq, gk, gv, causal=w.causal, scale=w.scale,
                             hq=hq, hk=dk, hv=dv, hdo=hdo, workspace=ws)
        if ev is not None:
            ev[3].record()

    def step_fwd(ev=None):
        if ev is not None:
            ev[0].record()
            ev[1].record()
            ev[2].record()
        forward(o_f, lse_f)
        if ev is not None:
            ev[3].record()

    def step(ev=None):
        if w.op == "bob":
            return step_bob(ev)
        if w.op == "fwd":
            return step_fwd(ev)
        if ev is not None:
            ev[0].record()
        binding.attn_bwd_preprocess(o, do, lse, ws)
        if ev is not None:
            ev[1].record()
        if mask is None:
            binding.attn_bwd_dkdv(q, k, v, do, ws, dk, dv, causal=w.causal, scale=w.scale)
        else:
            binding.attn_bwd_dkdv_masked(q, k, v, do, ws, dk, dv, mask, causal=w.causal,
                                         scale=w.scale)
        if ev is not None:
            ev[2].record()
        if mask is None:
            binding.attn_bwd_dq(q, k, v, do, ws, dq, causal=w.causal, scale=w.scale)
        else:
            binding.attn_bwd_dq_masked(q, k, v, do, ws, dq, mask, causal=w.causal, scale=w.scale)
        if ev is not None:
            ev[3].record()

    def call():
        # one step as a user makes it: the operation's own entry point (the
        # backward's three kernels go out back to back from one C call)
        if w.op == "bob":
            return step_bob()
        if w.op == "fwd":
            return forward(o_f, lse_f)
        if mask is None:
            binding.attn_bwd(q, k, v, o, do, lse, causal=w.causal, scale=w.scale, dq=dq, dk=dk,
                             dv=dv, workspace=ws)
        else:
            binding.attn_bwd_masked(q, k, v, o, do, lse, mask, causal=w.causal, scale=w.scale,
                                    dq=dq, dk=dk, dv=dv, workspace=ws)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()

    # timed region 1 (value, ms_per_step): K steps of the entry point
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # timed region 2 (stages, roofline): the same K steps through the stage
    # entry points, HIP events between the kernels on the launch stream
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()

    pre = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    dkdv = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    dqk = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
    ms = wall / args.steps * 1e3
    P = pairs(w.B, w.H, w.N, w.causal, bm)
    # algorithmic FLOPs per kept pair, recomputation excluded: the backward's
    # five contractions (10 d); the backward of the backward's twelve (S, dP,
    # G as two, A, then hQ, hK, hdO as two each and hV: 24 d); the forward's
    # two (S and P V: 4 d).  The backward of the backward's three passes
    # execute 22 products (44 d), reported as executed work beside it.
    per_pair = {"bob": 24 * w.d, "fwd": 4 * w.d}.get(w.op, 10 * w.d)
    flops = per_pair * P
    value = flops / (ms * 1e-3) / 1e12
    if w.op in ("bob", "fwd"):
        # one call: the roofline covers all of it (the forward is one kernel)
        achieved = flops / (dqk * 1e-3) / 1e12
    else:
        dkdv_flops = 8 * w.d * P
        achieved = dkdv_flops / (dkdv * 1e-3) / 1e12
    peak = PEAK[w.dtype]

    # the forward (the step that supplies O and L), timed on its own after the
    # backward's timed region: 4 d FLOPs per kept pair (S and P V)
    fev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    forward(o_f, lse_f)
    torch.cuda.synchronize()
    fwd_runs = 5
    fev[0].record()
    for _ in range(fwd_runs):
        forward(o_f, lse_f)
    fev[1].record()
    torch.cuda.synchronize()
    fwd_ms = fev[0].elapsed_time(fev[1]) / fwd_runs

    # no-N^2 evidence: free device memory across one backward step
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info(dev)[0]
    step()
    torch.cuda.synchronize()
    mem_delta = free0 - torch.cuda.mem_get_info(dev)[0]

    denominators = measure_denominators(torch, dev)

    if args.copy_calibration_mib:
        # a cast copy runs as a kernel (a same-type copy may go to a DMA engine):
        # it reads and writes exactly n * 4 bytes
        n = args.copy_calibration_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty(n, dtype=torch.int32, device=dev)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    # the dK/dV kernel that ran: the pipelined one serves bf16 with d = 64 or 128
    dkdv_kernel = DOMINANT_KERNEL if (w.dtype == "bf16" and w.d in (64, 128)) else "bwd_dkdv_kernel"
    if w.op == "bob":
        dkdv_kernel = "attn_bwd_bwd (preprocess + bob_q_kernel x2 + bob_kv_kernel)"
    if w.op == "fwd":
        dkdv_kernel = ("fwd_bf16_pipe_kernel" if (w.dtype == "bf16" and w.d in (64, 128))
                       else "fwd_lse_kernel")
    esz = 2 if w.dtype == "bf16" else 4
    if w.op == "fwd":   # Q, K, V read, O and L written
        alg_bytes = 4 * w.B * w.N * w.H * w.d * esz + 4 * w.B * w.H * w.N
    else:
        alg_bytes = 8 * w.B * w.N * w.H * w.d * esz + 4 * w.B * w.H * w.N
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "scale": w.scale, "layout": "[B,N,H,d]",
                   "parallelism": "single GPU", "op": w.op, "flops_per_pair": per_pair,
                   **({"flops_per_pair_executed": 44 * w.d} if w.op == "bob" else {}),
                   **({"block_mask": w.mask, "kept_pairs": P} if bm is not None else {})},
        "pct_of_peak": round(100 * value / peak, 2),
        "stages_ms": ({"bwd_bwd": round(dqk, 4)} if w.op == "bob" else
                      {"fwd_lse": round(dqk, 4)} if w.op == "fwd" else
                      {"preprocess": round(pre, 4), "dkdv": round(dkdv, 4), "dq": round(dqk, 4)}),
        "hbm_gbs_algorithmic": round(alg_bytes / (ms * 1e-3) / 1e9, 1),
        "fwd_lse": {"ms": round(fwd_ms, 4),
                    "tflops": round(4 * w.d * P / (fwd_ms * 1e-3) / 1e12, 3)},
        "device_mem_delta_bytes": int(mem_delta),
        "denominators": dict(denominators,
                             value_over_gemm=round(value / denominators["gemm_bf16_tflops"], 4),
                             hbm_over_copy=round(alg_bytes / (ms * 1e-3) / 1e9
                                                 / denominators["copy_gbs"], 4)),
        "roofline": {"kernel": dkdv_kernel, "bound": "mfma", "achieved": round(achieved, 3),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic_record() if w.name == "c5_long" else None,
                     **({"executed_tflops": round(44 * w.d * P / (dqk * 1e-3) / 1e12, 3)}
                        if w.op == "bob" else {})},
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle, whole heads, bounded)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w, x, bm, cot if w.op == "bob" else None, w.op)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
