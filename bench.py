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
       python bench.py --copy-probe MIB ...   (adds a plain device copy of
           MIB MiB after the timed region: the reference kernel for scaling
           the FETCH_SIZE / WRITE_SIZE counters of a rocprofv3 --pmc run)
       python bench.py --traffic-from FETCH_CSV WRITE_CSV --copy-mib MIB
           (no GPU: turns the counter CSVs of two such runs into the HBM
           traffic summary that later bench lines report)
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
PEAK_MFMA_FP32_TFLOPS = 157.3           # dense fp32 matrix peak
# exp2 issue ceiling at the nominal clock: 1024 SIMDs x 64 lanes per 8 cycles x 2.4 GHz
PEAK_EXP2_PER_S = 1024 * 64 / 8 * 2.4e9
# what the path computes in: bf16 in and out, every matrix product on fp16
# operands with fp32 accumulation, LayerNorm and softmax in fp32
DTYPE_LABEL = "bf16 I/O, fp16 MFMA operands, fp32 accumulation and softmax"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_tri_bf16_i1536.json")
CSRC = os.path.join(ROOT, "pair_representation_attention_amd", "csrc")
# source files each kernel is compiled from (a counter summary is valid for one source state)
KERNEL_SOURCES = {
    "attention": ("pa_attn.hip", "pa_device.h"),
    "projection": ("pa_kernels_bf16.hip", "pa_device.h"),
}
KERNEL_SYMBOLS = {"attention": "attn_kernel", "projection": "proj_kernel"}


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


def proj_kernel_bytes(R: int, I: int, c: int, H: int, d: int, with_bias: bool = True) -> float:
    """Algorithmic HBM bytes of one projection launch (bf16 in, fp16 out):
    read the R x I positions of x once, write q, k, v, g and the pair bias."""
    hd = H * d
    return 2.0 * R * I * c + 4 * 2.0 * R * I * hd + (2.0 * H * I * I if with_bias else 0.0)


def softmax_elements(R: int, I: int, H: int) -> float:
    """exp2 evaluations of one attention launch: one per (row, head, query, key)."""
    return float(R) * I * I * H


def stream_rates(R: int, I: int, c: int, H: int, d: int, attn_ms: float, proj_ms: float) -> dict:
    """Bytes and rates of the pair-bias and gate streams (bf16 path, one
    orientation): the projection writes both once; the attention reads the
    gate once and copies the bias tiles of its query blocks into LDS for
    every block of 2 rows (from L2 and the last-level cache: the bias is
    19 MB at I = 1536), i.e. I/2 times over."""
    Pp = (I + 31) // 32 * 32
    bias = 2.0 * H * Pp * Pp                  # fp16, padded, log2 units
    gate = 2.0 * R * Pp * H * d               # fp16, layout of q
    bias_lds = bias * ((R + 1) // 2)          # every 2-row workgroup group sweeps all key blocks
    return {
        "bias": {"bytes": bias, "written_gbs_over_projection": bias / (proj_ms * 1e-3) / 1e9,
                 "copied_to_lds_bytes_per_attention_launch": bias_lds,
                 "copied_to_lds_gbs": bias_lds / (attn_ms * 1e-3) / 1e9},
        "gate": {"bytes": gate, "written_gbs_over_projection": gate / (proj_ms * 1e-3) / 1e9,
                 "read_gbs_over_attention": gate / (attn_ms * 1e-3) / 1e9},
    }


def per_kernel_pass(lib, torch, stream, step, steps: int, prefixes) -> dict:
    """Run `steps` steps with the library's per-kernel events on; each step
    makes len(prefixes) calls.  Returns {prefix + stage: [ms per launch]}
    and the step time of this pass under "_step_ms"."""
    lib.pairattn_timing_enable(True)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    marks = lib.pairattn_timing_read()
    torch.cuda.synchronize()
    lib.pairattn_timing_enable(False)
    out = {"_step_ms": e0.elapsed_time(e1) / steps}
    # each call's marks start with "pack"; calls alternate over the prefixes
    call = -1
    for name, ms in marks:
        if name == "pack":
            call += 1
        out.setdefault(prefixes[call % len(prefixes)] + name, []).append(ms)
    return out


def calibrate_exp2(lib, torch, stream, iters: int = 4096, reps: int = 3) -> dict:
    """The device's exp2 throughput (pairattn_calibrate_exp2), timed with
    events on the launch stream: the ceiling of the softmax's exp2 issue."""
    out = torch.empty(2048 * 256, dtype=torch.float32, device="cuda")
    lib.pairattn_calibrate_exp2(out, iters, stream)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        lib.pairattn_calibrate_exp2(out, iters, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    n = 2048 * 256 * 8 * iters
    return {"exp2_per_launch": n, "ms": ms, "exp2_per_s": n / (ms * 1e-3),
            "cycles_per_wave_exp2_at_2.4GHz": 1024 * 64 * 2.4e9 / (n / (ms * 1e-3))}


def copy_probe(torch, mib: float) -> None:
    """Plain device copies and fills of `mib` MiB, outside any timed region:
    the reference kernels whose FETCH_SIZE / WRITE_SIZE scale the counters of
    a rocprofv3 --pmc run, and (in a kernel trace) this device's read+write
    and write-only HBM rates."""
    n = int(mib * 1024 * 1024)
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    for _ in range(2):
        dst.fill_(3)
    torch.cuda.synchronize()
    log(f"copy probe: {mib} MiB copied x 2, filled x 2")
    del src, dst


def cpu_info() -> dict:
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        aff = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        aff = None
    return {"cpu_model": model, "logical_cpus": os.cpu_count(), "affinity_cpus": aff}


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_entry(kernel: str):
    """Measured HBM bytes per launch of `kernel` from the committed counter
    summary, if it was taken on the kernel's current source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    k = t.get("kernels", {}).get(kernel)
    if not k or k.get("source_hash") != kernel_source_hash(kernel):
        return None
    return k.get("hbm_bytes_per_launch")


def _read_counter_csv(path: str, counter: str) -> dict:
    """{kernel name: [value per dispatch]} for one counter of a rocprofv3 CSV."""
    import csv
    out = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            out.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return out


def traffic_from(fetch_csv: str, write_csv: str, copy_mib: float, commands) -> dict:
    """Scale FETCH_SIZE / WRITE_SIZE (KiB per dispatch) by what the same
    counters read for the plain copy of copy_mib MiB, per kernel."""
    fetch = _read_counter_csv(fetch_csv, "FETCH_SIZE")
    write = _read_counter_csv(write_csv, "WRITE_SIZE")

    def copy_value(tab):
        vals = [v for name, vs in tab.items() if "copyBuffer" in name for v in vs]
        if not vals:
            raise SystemExit("no copy dispatch in the counter file (run bench.py with --copy-probe)")
        return max(vals)

    known_kib = copy_mib * 1024.0
    f_fetch = known_kib / copy_value(fetch)
    f_write = known_kib / copy_value(write)
    res = {"copy_mib": copy_mib, "fetch_scale": f_fetch, "write_scale": f_write, "commands": commands,
           "kernels": {}}
    for kernel, sym in KERNEL_SYMBOLS.items():
        fv = [v for name, vs in fetch.items() if sym in name for v in vs]
        wv = [v for name, vs in write.items() if sym in name for v in vs]
        if not fv or not wv:
            continue
        fb = sum(fv) / len(fv) * 1024.0 * f_fetch
        wb = sum(wv) / len(wv) * 1024.0 * f_write
        res["kernels"][kernel] = {"source_hash": kernel_source_hash(kernel), "dispatches": len(fv),
                                  "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
                                  "hbm_bytes_per_launch": fb + wb}
    return res


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
        **cpu_info(),
    }


# ----------------------------------------------------------------------------
def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=24, help="oracle sample size (rows, about 0.35-1.4 s each by host)")
    ap.add_argument("--extra", action="store_true",
                    help="also time the fp32 I=64 and padded I=384 triangle configurations, the padded I=1536 "
                         "module, MSA row attention, the row block and the extra-MSA fp32 workload")
    ap.add_argument("--workload", choices=["tri_bf16_i1536", "msa_bf16_s512_i384", "msa_fp32_s5120_i384",
                                           "tri_bf16_i16384_chunked", "ring_fp32_i1536_grid2x2",
                                           "ring_bf16_i1536_grid2x2", "tri_bf16_i384_pad", "tri_fp32_i64",
                                           "rows_bf16_i4096_r512"],
                    default="tri_bf16_i1536",
                    help="time only the fp32 extra-MSA workload, or chunked triangle attention at I = 16384 "
                         "(one JSON line)")
    ap.add_argument("--copy-probe", type=float, default=0.0, metavar="MIB",
                    help="after timing, run a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the traffic summary from two rocprofv3 --pmc counter CSVs and exit")
    ap.add_argument("--copy-mib", type=float, default=1024.0, help="copy size used in the --pmc runs")
    ap.add_argument("--command", action="append", default=[], help="command lines recorded with --traffic-from")
    args = ap.parse_args()

    if args.traffic_from:
        res = traffic_from(args.traffic_from[0], args.traffic_from[1], args.copy_mib, args.command)
        os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(res, f, indent=1)
        print(json.dumps(res, indent=1))
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (no collectives); "
              "run with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from pair_representation_attention_amd import device, inputs, lib

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    lib.load()
    if args.workload != "tri_bf16_i1536":
        fn = {"msa_fp32_s5120_i384": msa_fp32_workload, "tri_bf16_i16384_chunked": chunked_workload,
              "ring_fp32_i1536_grid2x2": ring_workload, "ring_bf16_i1536_grid2x2": ring_workload,
              "msa_bf16_s512_i384": msa_bf16_workload, "rows_bf16_i4096_r512": rows_workload,
              "tri_bf16_i384_pad": lambda *a: tri_config_workload("tri_bf16_i384_pad", *a, np=np),
              "tri_fp32_i64": lambda *a: tri_config_workload("tri_fp32_i64", *a, np=np, orientations=(0,))}[
            args.workload]
        res = fn(args, device, inputs, lib, torch)
        if args.copy_probe > 0:
            copy_probe(torch, args.copy_probe)
        print(json.dumps({"workload": args.workload, **res}), flush=True)
        return 0
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

    # timed region: K steps, nothing recorded between them
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_step = ev0.elapsed_time(ev1) / args.steps
    log(f"timed {args.steps} steps: {ms_step:.3f} ms/step (host wall {wall / args.steps * 1e3:.3f} ms/step)")

    # per-kernel pass: the same K steps again with HIP events recorded by the
    # library on the launch stream after each kernel (no host wait until the
    # end), for the kernels' launch times
    stage_ms = per_kernel_pass(lib, torch, stream, step, args.steps, ("start_", "end_"))
    ms_step_marked = stage_ms.pop("_step_ms")
    log(f"per-kernel pass: {ms_step_marked:.3f} ms/step")

    f = tri_module_flops(I, I, c, H, d)
    step_flops = 2 * f["total"]
    tflops = step_flops / (ms_step * 1e-3) / 1e12
    pair_rows = 2 * I / (ms_step * 1e-3)

    attn_ms = float(np.mean(stage_ms["start_attention"] + stage_ms["end_attention"]))
    attn_flops = attn_kernel_flops(I, I, c, H, d)
    achieved = attn_flops / (attn_ms * 1e-3) / 1e12
    roof = {
        "kernel": "attn_kernel<4,128> (tri, bf16 I/O, fp16 MFMA operands)",
        "bound": "mfma",
        "achieved": achieved,
        "peak": PEAK_MFMA_16BIT_TFLOPS,
        "unit": "TFLOP/s",
        "frac": achieved / PEAK_MFMA_16BIT_TFLOPS,
        "traffic": traffic_entry("attention"),
        "flops_per_launch": attn_flops,
        "mean_launch_ms": attn_ms,
    }
    proj_ms = float(np.mean(stage_ms["start_projection"] + stage_ms["end_projection"]))
    proj_bytes = proj_kernel_bytes(I, I, c, H, d)
    proj_gbs = proj_bytes / (proj_ms * 1e-3) / 1e9
    roof_proj = {
        "kernel": "proj_kernel<128,128,512,1,2> (LayerNorm + q|k|v|g + pair bias)",
        "bound": "hbm",
        "achieved": proj_gbs,
        "peak": PEAK_HBM_GBS,
        "unit": "GB/s",
        "frac": proj_gbs / PEAK_HBM_GBS,
        "traffic": traffic_entry("projection"),
        "bytes_per_launch": proj_bytes,
        "mean_launch_ms": proj_ms,
    }
    kernels = {k: float(np.mean(v)) for k, v in sorted(stage_ms.items())}

    # second roof: one exp2 per logit against the device's measured exp2 rate
    exp_cal = calibrate_exp2(lib, torch, stream)
    exps = softmax_elements(I, I, H)
    exp_rate = exps / (attn_ms * 1e-3)
    roof_exp = {
        "kernel": roof["kernel"],
        "bound": "exp2 issue",
        "achieved": exp_rate / 1e12,
        "peak": exp_cal["exp2_per_s"] / 1e12,
        "peak_nominal": PEAK_EXP2_PER_S / 1e12,
        "unit": "Texp2/s",
        "frac": exp_rate / exp_cal["exp2_per_s"],
        "exp2_per_launch": exps,
        "calibration": exp_cal,
    }
    streams = stream_rates(I, I, c, H, d, attn_ms, proj_ms)

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
        "dtype": DTYPE_LABEL,
        "data": "synthetic",
        "config": {"workload": "tri_bf16_i1536", "I": I, "c_z": c, "H": H, "d": d, "mask": "none",
                   "orientations": ["start", "end"], "seed": cfg["seed"]},
        "pair_rows_per_s": pair_rows,
        "frac_of_peak": tflops / PEAK_MFMA_16BIT_TFLOPS,
        "step_flops": step_flops,
        "ms_per_step_per_kernel_pass": ms_step_marked,
        "kernels_ms": kernels,
        "roofline": roof,
        "roofline_second": roof_exp,
        "roofline_projection": roof_proj,
        "streams": streams,
    }

    if args.extra:
        result["extra"] = extra_workloads(args, device, inputs, lib, torch, np)

    if args.copy_probe > 0:
        copy_probe(torch, args.copy_probe)

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


def tri_config_workload(name, args, device, inputs, lib, torch, np, orientations=(0, 1), mask_override=None):
    """One triangle-attention configuration: module time of the given
    orientations back to back (uninstrumented), the per-kernel split from a
    second pass, TFLOP/s and pair-rows/s."""
    cfg = inputs.CONFIGS[name]
    I, c, H, d, dt = cfg["I"], cfg["c"], cfg["H"], cfg["d"], cfg["dtype"]
    mask = cfg["mask"] if mask_override is None else mask_override
    log(f"extra: {name} mask={mask} orientations={list(orientations)}")
    case = inputs.make_tri_case(I=I, c=c, H=H, d=d, dtype=dt, mask=mask, seed=cfg["seed"])
    runs = [device.TriRunner(case.z, case.mask, case.params_start if o == 0 else case.params_end, H, dt)
            for o in orientations]
    for r in runs[1:]:
        r.z, r.mask = runs[0].z, runs[0].mask
    stream = torch.cuda.current_stream()

    def step():
        for o, r in zip(orientations, runs):
            r(o, stream)

    steps = max(3, args.steps)
    ms = _time(step, steps, 2, torch)
    st = per_kernel_pass(lib, torch, stream, step, steps, tuple(f"o{o}_" for o in orientations))
    st.pop("_step_ms")
    f = tri_module_flops(I, I, c, H, d)["total"] * len(orientations)
    res = {"I": I, "dtype": dt, "mask": mask, "orientations": list(orientations), "ms": ms,
           "tflops": f / (ms * 1e-3) / 1e12, "pair_rows_per_s": I * len(orientations) / (ms * 1e-3),
           "kernels_ms": {k: float(np.mean(v)) for k, v in sorted(st.items())}}
    att = [v for k, v in st.items() if k.endswith("attention")]
    if att:
        a_ms = float(np.mean([x for v in att for x in v]))
        res["attention_tflops"] = attn_kernel_flops(I, I, c, H, d) / (a_ms * 1e-3) / 1e12
    del runs, case
    torch.cuda.empty_cache()
    return res


def msa_bf16_workload(args, device, inputs, lib, torch) -> dict:
    """MSA row attention with pair bias, bf16: M[512,384,256], Z[384,384,128],
    H = 8, Bernoulli(0.95) keys: whole-call time and the per-kernel split."""
    import numpy as np
    cfg = inputs.CONFIGS["msa_bf16_s512_i384"]
    log("MSA row attention S=512 I=384 bf16")
    case = inputs.make_msa_case(S=cfg["S"], I=cfg["I"], c_m=cfg["c_m"], c_z=cfg["c_z"], H=cfg["H"], d=cfg["d"],
                                dtype=cfg["dtype"], mask=cfg["mask"], seed=cfg["seed"])
    run = device.MsaRunner(case.m, case.z, case.mask, case.params, cfg["H"], "bf16")
    stream = torch.cuda.current_stream()
    steps = max(3, args.steps)
    ms = _time(run, steps, 2, torch)
    st = per_kernel_pass(lib, torch, stream, lambda: run(stream), steps, ("",))
    st.pop("_step_ms")
    f = msa_module_flops(cfg["S"], cfg["I"], cfg["c_m"], cfg["c_z"], cfg["H"], cfg["d"])["total"]
    fa = attn_kernel_flops(cfg["S"], cfg["I"], cfg["c_m"], cfg["H"], cfg["d"])
    kern = {k: float(np.mean(v)) for k, v in sorted(st.items())}
    res = {"ms": ms, "tflops": f / (ms * 1e-3) / 1e12, "rows_per_s": cfg["S"] / (ms * 1e-3), "kernels_ms": kern,
           "attention_tflops": fa / (kern["attention"] * 1e-3) / 1e12}
    del run, case
    torch.cuda.empty_cache()
    return res


def rows_workload(args, device, inputs, lib, torch) -> dict:
    """Row block: 512 starting-node rows of Z[4096,4096,128] (a 171-residue
    block tiled 24 times plus noise), the bias from the whole Z
    (pairattn_tri_bias), then the rows (pairattn_tri_rows_fwd)."""
    import numpy as np
    cfg = inputs.CONFIGS["rows_bf16_i4096_r512"]
    I, R, c, H, d = cfg["I"], cfg["R"], cfg["c"], cfg["H"], cfg["d"]
    log(f"row block, {R} rows of Z[{I},{I},{c}]")
    case = inputs.make_rows_case(I=I, R=R, c=c, H=H, d=d, asu=cfg["asu"], noise=cfg["noise"], seed=cfg["seed"])
    zf = torch.from_numpy(case.zbits.view(np.int16)).to("cuda").view(torch.bfloat16)
    rr = device.RowsRunner(zf, zf[case.r0:case.r0 + R], None, case.params, H, "bf16")
    del case
    steps = max(3, args.steps)
    ms_bias = _time(rr.compute_bias, steps, 2, torch)
    ms_rows = _time(rr.rows, steps, 2, torch)
    ms = _time(rr, steps, 2, torch)
    f = tri_module_flops(R, I, c, H, d, with_bias=True)["total"]
    res = {"ms": ms, "ms_bias": ms_bias, "ms_rows": ms_rows, "tflops": f / (ms * 1e-3) / 1e12,
           "rows_per_s": R / (ms * 1e-3)}
    del rr, zf
    torch.cuda.empty_cache()
    return res


def extra_workloads(args, device, inputs, lib, torch, np) -> dict:
    out = {}
    # the other triangle configurations: fp32 I = 64 (starting node) and the
    # padded bf16 I = 384 (both orientations); the module of I = 1536 under
    # the padding mask of the I = 384 configuration (last 10% of residues)
    out["tri_fp32_i64"] = tri_config_workload("tri_fp32_i64", args, device, inputs, lib, torch, np, (0,))
    out["tri_bf16_i384_pad"] = tri_config_workload("tri_bf16_i384_pad", args, device, inputs, lib, torch, np)
    out["tri_bf16_i1536_pad"] = tri_config_workload("tri_bf16_i1536", args, device, inputs, lib, torch, np,
                                                    mask_override="pad")
    out["msa_bf16_s512_i384"] = msa_bf16_workload(args, device, inputs, lib, torch)

    out["rows_bf16_i4096_r512"] = rows_workload(args, device, inputs, lib, torch)

    out["msa_fp32_s5120_i384"] = msa_fp32_workload(args, device, inputs, lib, torch)
    return out


def msa_fp32_workload(args, device, inputs, lib, torch) -> dict:
    """Extra-MSA row attention, fp32 end to end (fp16-pair operands on the
    matrix cores): whole-call time and the per-kernel split."""
    cfg = inputs.CONFIGS["msa_fp32_s5120_i384"]
    log(f"extra: fp32 extra-MSA row attention S={cfg['S']} I={cfg['I']} c_m={cfg['c_m']}")
    case = inputs.make_msa_case(S=cfg["S"], I=cfg["I"], c_m=cfg["c_m"], c_z=cfg["c_z"], H=cfg["H"], d=cfg["d"],
                                dtype=cfg["dtype"], mask=cfg["mask"], seed=cfg["seed"])
    run = device.MsaRunner(case.m, case.z, case.mask, case.params, cfg["H"], "f32")
    del case
    steps = max(3, args.steps)
    ms = _time(run, steps, 2, torch)
    stages = {}
    lib.pairattn_timing_enable(True)
    for _ in range(steps):
        run()
        for name, t in lib.pairattn_timing_read():
            stages[name] = stages.get(name, 0.0) + t / steps
    lib.pairattn_timing_enable(False)
    f = msa_module_flops(cfg["S"], cfg["I"], cfg["c_m"], cfg["c_z"], cfg["H"], cfg["d"])
    fa = attn_kernel_flops(cfg["S"], cfg["I"], cfg["c_m"], cfg["H"], cfg["d"])
    a_tf = fa / (stages["attention"] * 1e-3) / 1e12
    res = {
        "ms": ms, "tflops": f["total"] / (ms * 1e-3) / 1e12, "rows_per_s": cfg["S"] / (ms * 1e-3),
        "kernels_ms": stages,
        # every product is three f16 MFMA products: fp32 accuracy, measured
        # against the fp32 matrix peak, with the f16 pipe's own load beside it
        "attention_roofline": {"bound": "mfma", "achieved": a_tf, "peak": PEAK_MFMA_FP32_TFLOPS, "unit": "TFLOP/s",
                               "frac": a_tf / PEAK_MFMA_FP32_TFLOPS,
                               "f16_pipe_frac": 3.0 * a_tf / PEAK_MFMA_16BIT_TFLOPS},
    }
    # projection: read M once, write q, k, v as fp16 pairs and the gate as fp32
    pb = 4.0 * cfg["S"] * cfg["I"] * cfg["c_m"] + 16.0 * cfg["S"] * cfg["I"] * cfg["H"] * cfg["d"]
    p_gbs = pb / (stages["projection"] * 1e-3) / 1e9
    res["projection_roofline"] = {"bound": "hbm", "achieved": p_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                  "frac": p_gbs / PEAK_HBM_GBS, "bytes_per_launch": pb}
    del run
    torch.cuda.empty_cache()
    return res


def chunked_workload(args, device, inputs, lib, torch) -> dict:
    """Starting-node triangle attention of Z[16384, 16384, 128] bf16 in blocks
    of 1024 rows (pairattn_tri_chunked_fwd): the one-pass workspace would not
    fit beside Z and the update.  One call per step; Z drawn on the device."""
    cfg = inputs.CONFIGS["tri_bf16_i16384_chunked"]
    I, c, H, d, block = cfg["I"], cfg["c"], cfg["H"], cfg["d"], cfg["block"]
    log(f"chunked: generating Z[{I},{I},{c}] on the device")
    z = inputs.make_z_device(I, c, cfg["seed"])
    p = inputs.make_chunked_params(c, H, d, cfg["seed"])
    run = device.TriChunkedRunner(z, None, p, H, "bf16", block)
    steps = max(1, min(args.steps, 3))
    ms = _time(lambda: run(lib.PAIRATTN_START), steps, 1, torch)
    stages = {}
    lib.pairattn_timing_enable(True)
    run(lib.PAIRATTN_START)
    for name, t in lib.pairattn_timing_read():
        stages[name] = t
    lib.pairattn_timing_enable(False)
    f = tri_module_flops(I, I, c, H, d, with_bias=True)["total"]
    res = {"ms": ms, "tflops": f / (ms * 1e-3) / 1e12, "rows_per_s": I / (ms * 1e-3), "block": block,
           "stages_ms": stages, "workspace_bytes": run.workspace_bytes,
           "one_pass_workspace_bytes": lib.pairattn_tri_workspace_bytes(I, c, H, d, lib.PAIRATTN_BF16),
           "z_bytes": I * I * c * 2, "frac_of_peak": f / (ms * 1e-3) / 1e12 / PEAK_MFMA_16BIT_TFLOPS}
    del run, z
    torch.cuda.empty_cache()
    return res


def ring_workload(args, device, inputs, lib, torch) -> dict:
    """One device's share of starting-node attention of Z[1536, 1536, 128]
    (fp32 or bf16) on a 2 x 2 grid: its 768 rows x 768 query columns against
    the two 768-column key shards in ring order (partial, partial merged,
    finish), beside the one-pass call on the same 768 rows (all 1536
    queries, i.e. twice the queries) for the rate comparison.  The attention
    kernel of the partial calls is timed with HIP events on its launch
    stream (a second pass, after the timed steps)."""
    import numpy as np

    dt = "bf16" if "bf16" in args.workload else "f32"
    code = device.dtype_code(dt)
    I, c, H, d, half = 1536, 128, 4, 32, 768
    log(f"ring: generating Z[1536,1536,128] {dt} on the device")
    z = inputs.make_z_device(I, c, 11, dtype=dt)
    p = inputs.make_chunked_params(c, H, d, 11, dtype=dt)
    zq = z[:half, :half].contiguous()                   # this device's pairs: rows A, columns B
    shards = [zq, z[:half, half:].contiguous()]         # its own shard is its query pairs
    bias = torch.empty((H, I, I), dtype=torch.float32, device="cuda")
    pr = device.make_params(p, dt)
    lib.pairattn_tri_bias(z, pr, bias, I, c, H, lib.PAIRATTN_START)
    btiles = [bias[:, :half, :half].contiguous(), bias[:, :half, half:].contiguous()]
    n = max(lib.pairattn_tri_partial_workspace_bytes(half, half, half, c, H, d, code),
            lib.pairattn_tri_partial_finish_workspace_bytes(half, half, c, H, d, code))
    prm = device.make_params(p, dt, n)
    o = torch.empty((half, half, H * d), dtype=torch.float32, device="cuda")
    lse = torch.empty((half, H, half), dtype=torch.float32, device="cuda")
    out = torch.empty((half, half, c), dtype=device.torch_dtype(dt), device="cuda")
    stages = {}

    def step(record=False):
        for sidx in range(2):
            # later shards merge, and reuse the packed weights and the projected q of the query pairs
            flags = 0 if sidx == 0 else lib.PAIRATTN_PARTIAL_MERGE | lib.PAIRATTN_PARTIAL_Q_READY
            lib.pairattn_tri_partial_fwd(zq, shards[sidx], btiles[sidx], None, prm, o, lse, flags, half, half,
                                         half, c, H, d)
            if record:
                for name, ms in lib.pairattn_timing_read():
                    stages.setdefault(name, []).append(ms)
        lib.pairattn_tri_partial_finish(zq, o, prm, out, half, half, c, H, d)
        if record:
            for name, ms in lib.pairattn_timing_read():
                stages.setdefault("finish_" + name, []).append(ms)

    steps = max(3, args.steps)
    ms = _time(step, steps, 2, torch)
    lib.pairattn_timing_enable(True)
    for _ in range(steps):
        step(True)
    lib.pairattn_timing_enable(False)
    f = 4.0 * half * half * I * H * d + 2.0 * half * half * H * d * c     # attention + output projection
    f_shard = 4.0 * half * half * half * H * d                              # one partial attention launch
    attn_ms = float(np.mean(stages["attention"]))
    rows = device.RowsRunner(z, z[:half].contiguous(), None, p, H, dt)
    rows.compute_bias()
    ms_rows = _time(rows.rows, steps, 2, torch)
    f_rows = 4.0 * half * I * I * H * d + 2.0 * half * I * H * d * c
    res = {"dtype": dt, "ms": ms, "tflops": f / (ms * 1e-3) / 1e12, "rows": half, "queries": half, "keys": I,
           "shards": 2, "shard_attention_ms": attn_ms, "shard_attention_tflops": f_shard / (attn_ms * 1e-3) / 1e12,
           "stage_ms": {k: float(np.mean(v)) for k, v in stages.items()},
           "one_pass_rows_ms": ms_rows, "one_pass_rows_tflops": f_rows / (ms_rows * 1e-3) / 1e12}
    del rows, z, shards, bias, o, lse, out
    torch.cuda.empty_cache()
    return res


if __name__ == "__main__":
    sys.exit(main())
