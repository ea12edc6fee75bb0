#!/usr/bin/env python3
"""Benchmark of the pair-biased attention library on one MI355X.

One step = triangle attention around the starting node followed by the
ending node (separate weight sets) over the seeded synthetic pair tensor
Z[1536, 1536, 128] (bf16, no mask, H=4, d=32): every stage of the path --
LayerNorm, the fused projections, logits + pair bias, online softmax, P.V,
gate and output projection, for both orientations -- runs inside the timed
region, with the inputs already resident in device memory.

Prints one JSON line (the last line of stdout):
  value    = module TFLOP/s (algorithmic flops of both orientations / time)
  roofline = the attention kernel's algorithmic flops per launch / its mean
             launch time measured with HIP events on its own stream,
             against the 2516.6 TFLOP/s dense 16-bit MFMA peak
  cpu_baseline = the fp64 oracle timed on a bounded sample of the same
             workload on this host's cores

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--extra]
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

METRIC = "triangle-attn bf16 TFLOP/s + pair-rows/s at I=1536; % of MFMA peak"
PEAK_MFMA_16BIT_TFLOPS = 2516.6          # 256 CU x 4096 flop/clk x 2.4 GHz (bf16 = fp16 dense)
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_kernel_tri_bf16_i1536_traffic.json")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------
# algorithmic flop counts (no tiling or padding counted)
# ----------------------------------------------------------------------------
def tri_module_flops(R: int, I: int, c: int, H: int, d: int, with_bias: bool = True) -> dict:
    """Per orientation for R attention rows of length I."""
    hd = H * d
    f = {
        "attention": 4.0 * R * I * I * H * d,          # Q K^T and P V
        "projections": 2.0 * R * I * c * 4 * hd,       # q, k, v, g
        "bias": 2.0 * I * I * c * H if with_bias else 0.0,
        "out_proj": 2.0 * R * I * hd * c,
    }
    f["total"] = sum(f.values())
    return f


def msa_module_flops(S: int, I: int, c_m: int, c_z: int, H: int, d: int) -> dict:
    hd = H * d
    f = {
        "attention": 4.0 * S * I * I * H * d,
        "projections": 2.0 * S * I * c_m * 4 * hd,
        "bias": 2.0 * I * I * c_z * H,
        "out_proj": 2.0 * S * I * hd * c_m,
    }
    f["total"] = sum(f.values())
    return f


def attn_kernel_flops(R: int, I: int, c: int, H: int, d: int) -> float:
    """Work of one attention-kernel launch: QK^T + PV + the output projection."""
    return 4.0 * R * I * I * H * d + 2.0 * R * I * H * d * c


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in ("pa_kernels_bf16.hip", "pa_device.h"):
        with open(os.path.join(ROOT, "pair_representation_attention_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_entry(per_launch_flops_bytes=None):
    """HBM bytes per attention launch from the committed counter summary, if
    it was taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


# ----------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample
# ----------------------------------------------------------------------------
def cpu_baseline(case, H: int, d: int, rows: int) -> dict:
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([x.get("num_threads", 1) for x in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    I, c = case.I, case.c
    sel = np.linspace(0, I - 1, rows).astype(np.int64)
    p = case.params_start.as_dict()
    t0 = time.perf_counter()
    oracle.tri_start(case.z, None, p, H, rows=sel)
    dt = time.perf_counter() - t0
    f = tri_module_flops(rows, I, c, H, d)["total"]
    return {
        "value": f / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"starting-node rows {sel.tolist()} of Z[{I},{I},{c}] (all queries, pair bias over all "
                  f"{I}x{I} pairs), fp64 numpy; {dt:.1f} s; flops counted as for the GPU",
        "seconds": dt,
    }


# ----------------------------------------------------------------------------
def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=3, help="oracle sample size (rows)")
    ap.add_argument("--extra", action="store_true", help="also time MSA row attention and the row block")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (no collectives); "
              "run with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from pair_representation_attention_amd import device, inputs, lib

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    lib.load()
    torch.cuda.set_device(0)
    cfg = inputs.CONFIGS["tri_bf16_i1536"]
    I, c, H, d = cfg["I"], cfg["c"], cfg["H"], cfg["d"]
    log(f"generating Z[{I},{I},{c}] seed={cfg['seed']}")
    case = inputs.make_tri_case(I=I, c=c, H=H, d=d, dtype=cfg["dtype"], mask=cfg["mask"], seed=cfg["seed"])
    start = device.TriRunner(case.z, None, case.params_start, H, "bf16")
    end = device.TriRunner(case.z, None, case.params_end, H, "bf16")
    end.z = start.z   # one resident copy of Z feeds both orientations
    stream = torch.cuda.current_stream()

    def step():
        start(lib.PAIRATTN_START, stream)
        end(lib.PAIRATTN_END, stream)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region; per-kernel HIP events on the same stream
    lib.pairattn_timing_enable(True)
    stage_ms = {}
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        start(lib.PAIRATTN_START, stream)
        for name, ms in lib.pairattn_timing_read():
            stage_ms.setdefault("start_" + name, []).append(ms)
        end(lib.PAIRATTN_END, stream)
        for name, ms in lib.pairattn_timing_read():
            stage_ms.setdefault("end_" + name, []).append(ms)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    lib.pairattn_timing_enable(False)
    ms_step = ev0.elapsed_time(ev1) / args.steps
    log(f"timed {args.steps} steps: {ms_step:.3f} ms/step (host wall {wall / args.steps * 1e3:.3f} ms/step)")

    f = tri_module_flops(I, I, c, H, d)
    step_flops = 2 * f["total"]
    tflops = step_flops / (ms_step * 1e-3) / 1e12
    pair_rows = 2 * I / (ms_step * 1e-3)

    attn_ms = float(np.mean(stage_ms["start_attention"] + stage_ms["end_attention"]))
    attn_flops = attn_kernel_flops(I, I, c, H, d)
    achieved = attn_flops / (attn_ms * 1e-3) / 1e12
    traffic = traffic_entry()
    roof = {
        "kernel": "attn_kernel<4,128,4> (tri, bf16 I/O, fp16 MFMA operands)",
        "bound": "mfma",
        "achieved": achieved,
        "peak": PEAK_MFMA_16BIT_TFLOPS,
        "unit": "TFLOP/s",
        "frac": achieved / PEAK_MFMA_16BIT_TFLOPS,
        "traffic": traffic,
        "flops_per_launch": attn_flops,
        "mean_launch_ms": attn_ms,
    }
    kernels = {k: float(np.mean(v)) for k, v in sorted(stage_ms.items())}

    result = {
        "metric": METRIC,
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "tri_bf16_i1536", "I": I, "c_z": c, "H": H, "d": d, "mask": "none",
                   "orientations": ["start", "end"], "seed": cfg["seed"]},
        "pair_rows_per_s": pair_rows,
        "frac_of_peak": tflops / PEAK_MFMA_16BIT_TFLOPS,
        "step_flops": step_flops,
        "kernels_ms": kernels,
        "roofline": roof,
    }

    if args.extra:
        result["extra"] = extra_workloads(args, device, inputs, lib, torch, np)

    del start, end
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on {args.cpu_rows} rows")
        result["cpu_baseline"] = cpu_baseline(case, H, d, args.cpu_rows)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


def _time(fn, steps, warmup, torch):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def extra_workloads(args, device, inputs, lib, torch, np) -> dict:
    out = {}
    cfg = inputs.CONFIGS["msa_bf16_s512_i384"]
    log("extra: MSA row attention S=512 I=384")
    case = inputs.make_msa_case(S=cfg["S"], I=cfg["I"], c_m=cfg["c_m"], c_z=cfg["c_z"], H=cfg["H"], d=cfg["d"],
                                dtype=cfg["dtype"], mask=cfg["mask"], seed=cfg["seed"])
    run = device.MsaRunner(case.m, case.z, case.mask, case.params, cfg["H"], "bf16")
    ms = _time(run, max(3, args.steps), 2, torch)
    f = msa_module_flops(cfg["S"], cfg["I"], cfg["c_m"], cfg["c_z"], cfg["H"], cfg["d"])["total"]
    out["msa_bf16_s512_i384"] = {"ms": ms, "tflops": f / (ms * 1e-3) / 1e12, "rows_per_s": cfg["S"] / (ms * 1e-3)}
    del run
    torch.cuda.empty_cache()
    return out


if __name__ == "__main__":
    sys.exit(main())
