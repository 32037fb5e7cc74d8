"""Throughput of exact attention forward + backward on one MI355X.

Workload: GPT-2-medium-shaped causal attention, B=64 H=16 T=1024 hd=64,
bfloat16 inputs drawn N(0, 1) (seeded, synthetic), float32 accumulation and
outputs, P and dS rounded to bfloat16 for their matrix products.

One step = fa_forward, then the two backward stages (fa_backward_dq_delta,
fa_backward_dkv -- exactly what fa_backward runs), with every input already
resident in HBM.  W untimed warm-up steps, then K timed steps
between two device synchronisations; HIP events on the launch stream time each
kernel inside the timed region.

The metric counts 14*hd flops per (query, visible key) pair, B*H*T^2/2 pairs
for the causal mask.  The roofline object describes the kernel with the
largest share of the step; its algorithmic flops are the products it must
execute (forward 4*hd, dQ kernel 6*hd, dK/dV kernel 8*hd per pair; the dQ
kernel's 2*hd flops per row for D are not counted).

The CPU baseline times the float64 oracle on the host cores over a bounded
sample of the same workload (whole heads), and compares those heads of the
GPU outputs with it.

``--counters`` runs a minimal program for rocprofv3 --pmc: a float32 copy of
known size (the calibration kernel), then a few steps (of the bench workload,
or of each workload ``--workloads`` lists).

``--configs`` reports every workload instead (tiny, ragged, GPT-2-medium
float32, bfloat16 and IEEE half, long context): parity of sampled heads against the
float64 oracle first, then forward, backward and forward+backward each timed
over 9 runs after one warm-up (median and min, HIP events on the launch
stream, after ~50 ms of untimed steps to settle the clock), and the oracle's
time on one head extrapolated to the whole workload.  One JSON line per
workload, then a summary line.

``--lab`` runs the lab of the fused-attention lesson instead: one head, no
mask, float32 inputs uniform in [-2, 2), N in {256, ..., 4096}, d in {16, 64};
for the fused forward, the unfused three-kernel forward, the no-rescale
control and the split-key forward (128 keys per split) it times 9 runs after
one warm-up (HIP events around each run, the
unfused kernels' three dispatches in one timed run) and prints one JSON line
with the median milliseconds and the unfused/fused ratio.  Parity of these
kernels against the float64 reference with the lesson's error bound is checked
by tests/test_gpu_lab.py.  ``--lab --counters`` instead runs the calibration
copy and then each (N, d, kind) once, for rocprofv3 --pmc.

``--ramp N`` times each of the first N steps of the bench workload from the
first call of the process (HIP events between consecutive steps), then 20
steps after 200 ms of idle, and the mean over the window that --warmup W
--steps K would time: how the step time settles while the clock does.

``--split`` times the split-key forward against the plain forward on causal
workloads with few (batch, head) pairs and long sequences (B1 H4 T8192 hd128,
B1 H8 T16384 hd64, B1 H2 T32768 hd128 in bfloat16, B1 H4 T8192 hd64 in
float32; seeded N(0, 1) inputs): the plain forward and 2, 4, 8, 16 and 32
splits, each the median of 9 runs after one warm-up (merge included), with the
largest difference of O and L between the split and the plain results.  Parity
of the split forward against the oracle is checked by tests/test_gpu_splitkv.py
and tests/test_gpu_fp16.py.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "attention fwd+bwd TFLOP/s (% MFMA peak), causal B64 H16 T1024 hd64, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
STAGES = ("fwd", "dq", "dkv")
KERNEL_NAMES = {"fwd": "fwd64_kernel", "dq": "dq32_kernel", "dkv": "dkv64_kernel"}
COPY_BYTES = 1 << 30


def _code_only(text: str) -> str:
    """C/C++ source without comments, whitespace runs collapsed (string literals kept)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            i = text.find("\n", i)
            i = n if i < 0 else i
        elif text.startswith("/*", i):
            i = text.find("*/", i + 2)
            i = n if i < 0 else i + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code (comments and layout do not change it)."""
    h = hashlib.sha256()
    for p in sorted((ROOT / "exact_attention_forward_amd" / "csrc").glob("*")):
        h.update(p.name.encode())
        h.update(_code_only(p.read_text()).encode())
    return h.hexdigest()[:16]


def measured_traffic(stage: str):
    """HBM bytes per launch from the committed counter summary, if it matches the current kernels."""
    p = ROOT / "profiles" / "traffic.json"
    if not p.exists():
        return None
    rec = json.loads(p.read_text())
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    k = rec.get("kernels", {}).get(KERNEL_NAMES[stage])
    return None if k is None else k.get("hbm_bytes_per_launch")


def hbm_summary(per_ms: dict, ms_step: float):
    """HBM bytes of one step (the counter record's bytes per launch of each kernel) against the step time
    and each kernel's time, as a fraction of the 8 TB/s peak; None unless every kernel has a record
    that matches the current kernel sources."""
    got = {s: measured_traffic(s) for s in STAGES}
    if any(b is None for b in got.values()):
        return None
    total = sum(got.values())
    gbs = total / (ms_step * 1e-3) / 1e9
    return {"bytes_per_step": total, "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "kernels": {KERNEL_NAMES[s]: {"bytes": b, "achieved": round(b / (per_ms[s] * 1e-3) / 1e9, 1)}
                        for s, b in got.items()}}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed steps first; about 50 ms of work brings the GPU clock to its steady level")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle time budget for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--counters", action="store_true", help="minimal run for rocprofv3 counter collection")
    ap.add_argument("--workloads", default="C3",
                    help="with --counters: comma-separated workloads to step (C2 f32, C3 bf16, C4 long bf16)")
    ap.add_argument("--lab", action="store_true", help="fused vs unfused lab of the lesson (one head, float32)")
    ap.add_argument("--configs", action="store_true", help="time and check every workload, not only the bench one")
    ap.add_argument("--split", action="store_true",
                    help="split-key forward against the plain forward on few-head long-sequence workloads")
    ap.add_argument("--ramp", type=int, default=0, metavar="N",
                    help="time each of the first N steps of a fresh process, and 20 more after 200 ms idle")
    return ap.parse_args()


def main() -> int:
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1).",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import exact_attention_forward_amd as fa
    from exact_attention_forward_amd import inputs as I

    if args.lab:
        return lab(args)
    if args.configs:
        return configs(args)
    if args.split:
        return split(args)

    case = I.gpt2m_case(I.BF16)
    B, H, T, hd = case.B, case.H, case.T, case.hd
    prec = fa.FA_PREC_BF16
    dev = torch.device("cuda:0")

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v, do = (up(getattr(case, n)) for n in ("q", "k", "v", "do"))
    f32 = lambda *s: torch.empty(s, device=dev, dtype=torch.float32)
    o, lse = f32(B, T, H, hd), f32(B, H, T)
    dq, dk, dv, delta = f32(B, T, H, hd), f32(B, T, H, hd), f32(B, T, H, hd), f32(B, H, T)
    stream = torch.cuda.current_stream(dev)
    sc, dt = case.scale, fa.FA_BF16

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        fa.check(fa.fa_forward(q, k, v, o, lse, B, H, T, hd, sc, 1, dt, prec, stream))
        if ev is not None:
            ev[1].record(stream)
        fa.check(fa.fa_backward_dq_delta(q, k, v, o, lse, do, dq, delta, B, H, T, hd, sc, 1, dt, prec, stream))
        if ev is not None:
            ev[2].record(stream)
        fa.check(fa.fa_backward_dkv(q, k, v, lse, do, delta, dk, dv, B, H, T, hd, sc, 1, dt, prec, stream))
        if ev is not None:
            ev[3].record(stream)

    if args.ramp:
        return ramp(args.ramp, step, stream, args)

    if args.counters:
        x = torch.ones(COPY_BYTES // 4, device=dev, dtype=torch.float32)
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        del x, y
        names = [w.strip() for w in args.workloads.split(",") if w.strip()]
        for name in names:
            if name == "C3":
                for _ in range(3):
                    step()
                torch.cuda.synchronize()
            else:
                counter_steps(name)
        print(json.dumps({"counters_run": "done", "copy_bytes": COPY_BYTES, "workloads": names}), flush=True)
        return 0

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(STAGES) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    ms_step = (t1 - t0) * 1e3 / args.steps
    per = {s: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / args.steps for j, s in enumerate(STAGES)}
    pairs = B * H * T * T / 2
    counted = 14 * hd * pairs
    algo_flops = {"fwd": 4 * hd * pairs, "dq": 6 * hd * pairs, "dkv": 8 * hd * pairs}
    value = counted / (ms_step * 1e-3) / 1e12

    dom = max(("fwd", "dq", "dkv"), key=lambda s: per[s])
    achieved = algo_flops[dom] / (per[dom] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(dom),
                "kernel": KERNEL_NAMES[dom]}

    kernels = {KERNEL_NAMES[s]: {"ms": round(per[s], 4),
                                 "tflops": round(algo_flops[s] / (per[s] * 1e-3) / 1e12, 2) if algo_flops[s] else None}
               for s in STAGES}

    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1) bf16 inputs)",
        "config": {"workload": "causal attention fwd+bwd B64 H16 T1024 hd64 bf16 (P, dS bf16 operands)",
                   "B": B, "H": H, "T": T, "hd": hd, "causal": True, "precision": "FA_PREC_BF16"},
        "frac_of_mfma_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "roofline": roofline, "hbm": hbm_summary(per, ms_step), "kernels": kernels,
        "device": torch.cuda.get_device_name(dev),
    }

    if not args.no_cpu_baseline:
        rec["cpu_baseline"], rec["parity_sample"] = cpu_baseline(case, dict(O=o, L=lse, dQ=dq, dK=dk, dV=dv),
                                                                 args.cpu_seconds)
    print(json.dumps(rec), flush=True)
    return 0


def ramp(n: int, step, stream, args) -> int:
    """Per-step times (HIP events between consecutive steps) from the first call of a fresh process.

    Also reports the mean over the window a run with --warmup W --steps K would time, and 20 steps
    after 200 ms of idle, so that the settling of the clock under this load can be read off.
    """
    import torch

    def timed(count):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(count + 1)]
        ev[0].record(stream)
        for i in range(count):
            step()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        return [round(ev[i].elapsed_time(ev[i + 1]), 4) for i in range(count)]

    torch.cuda.synchronize()
    first = timed(n)
    time.sleep(0.2)
    again = timed(20)
    w, k = args.warmup, args.steps
    window = first[w:w + k]
    print(json.dumps({"ramp_steps_ms": first, "after_idle_200ms_ms": again, "warmup": w, "steps": k,
                      "window_mean_ms": round(sum(window) / len(window), 4) if len(window) == k else None,
                      "last_20_mean_ms": round(sum(first[-20:]) / 20, 4) if n >= 20 else None}), flush=True)
    return 0


def lab(args) -> int:
    """Median times of the fused, unfused and no-rescale forwards over the lesson's lab grid."""
    import torch

    import exact_attention_forward_amd as fa
    from exact_attention_forward_amd import inputs as I

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    if args.counters:
        x = torch.ones(COPY_BYTES // 4, device=dev, dtype=torch.float32)
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
    rows = []
    for d in I.LAB_WIDTHS:
        for N in I.LAB_SIZES:
            c = I.lab_case(N, d)
            q, k, v = (torch.from_numpy(getattr(c, n)).to(dev) for n in ("q", "k", "v"))
            o = torch.empty((1, N, 1, d), device=dev)
            lse = torch.empty((1, 1, N), device=dev)
            s = torch.empty((1, 1, N, N), device=dev)
            nsplit = min(64, max(1, N // 128))  # 128 keys per split
            ws = torch.empty((nsplit * (N * d + N),), device=dev)
            runs = {
                "fused": lambda: fa.check(fa.fa_forward(q, k, v, o, lse, 1, 1, N, d, c.scale, 0, fa.FA_F32, 0, stream)),
                # the plain fused kernel: no key split (fa_forward splits by itself here)
                "plain": lambda: fa.check(fa.fa_forward_splitkv(q, k, v, o, lse, None, 1, 1, N, d, c.scale, 0, 1,
                                                                fa.FA_F32, 0, stream)),
                "unfused": lambda: fa.check(fa.fa_forward_unfused(q, k, v, o, s, 1, 1, N, d, c.scale, 0, fa.FA_F32,
                                                                  stream)),
                "broken": lambda: fa.check(fa.fa_forward_norescale(q, k, v, o, lse, 1, 1, N, d, c.scale, 0, fa.FA_F32,
                                                                   stream)),
                "split": lambda: fa.check(fa.fa_forward_splitkv(q, k, v, o, lse, ws, 1, 1, N, d, c.scale, 0, nsplit,
                                                                fa.FA_F32, 0, stream)),
            }
            row = {"N": N, "d": d, "nsplit": nsplit,
                   "auto_nsplit": fa.fa_forward_auto_splits(1, 1, N, d, 0, fa.FA_F32, 0)}
            for kind, fn in runs.items():
                if args.counters:
                    fn()
                    torch.cuda.synchronize()
                    continue
                fn()  # warm-up
                torch.cuda.synchronize()
                ts = []
                for _ in range(9):
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    fn()
                    e1.record(stream)
                    torch.cuda.synchronize()
                    ts.append(e0.elapsed_time(e1))
                row[kind + "_ms"] = round(sorted(ts)[len(ts) // 2], 5)
            if not args.counters:
                row["unfused_over_fused"] = round(row["unfused_ms"] / row["fused_ms"], 3)
                row["unfused_over_plain"] = round(row["unfused_ms"] / row["plain_ms"], 3)
                row["unfused_over_split"] = round(row["unfused_ms"] / row["split_ms"], 3)
                row["score_bytes_saved"] = 16 * N * N
            rows.append(row)
    print(json.dumps({"lab": "fused vs unfused attention forward, one head, no mask, float32", "reps": 9,
                      "warmup": 1, "statistic": "median ms (HIP events)", "device": torch.cuda.get_device_name(dev),
                      "rows": rows} if not args.counters else {"lab_counters_run": "done"}), flush=True)
    return 0


PEAK_F32_MATRIX_TFLOPS = 157.3  # MI355X dense float32 MFMA

# Few (batch, head) pairs and long sequences, causal: one workgroup per query
# tile leaves most of the 256 CUs idle, which the key split is for.
# (B, H, T, hd, dtype, seed)
SPLIT_WORKLOADS = ((1, 4, 8192, 128, "bf16", 21), (1, 8, 16384, 64, "bf16", 22), (1, 2, 32768, 128, "bf16", 23),
                   (1, 4, 8192, 64, "f32", 24))
SPLIT_COUNTS = (2, 4, 8, 16, 32)


def split(args) -> int:
    """Split-key forward against the plain forward: median times and the largest
    differences of O and L between the two (the merge is exact up to rounding)."""
    import numpy as np
    import torch

    import exact_attention_forward_amd as fa
    from exact_attention_forward_amd import inputs as I

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    def median_ms(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(9):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return sorted(ts)[4]

    rows = []
    for B, H, T, hd, dts, seed in SPLIT_WORKLOADS:
        dtype = {"bf16": I.BF16, "f32": I.F32}[dts]
        case = I.make_case(f"split_B{B}H{H}T{T}hd{hd}_{dts}", B, H, T, hd, dtype, True, seed)
        if dtype == I.BF16:
            up = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        else:
            up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        q, k, v = (up(getattr(case, n)) for n in ("q", "k", "v"))
        dt = fa.FA_BF16 if dtype == I.BF16 else fa.FA_F32
        prec = fa.FA_PREC_BF16 if dtype == I.BF16 else fa.FA_PREC_DEFAULT
        o = torch.empty((B, T, H, hd), device=dev)
        lse = torch.empty((B, H, T), device=dev)
        n, nr = B * T * H * hd, B * H * T
        plain = lambda: fa.check(fa.fa_forward(q, k, v, o, lse, B, H, T, hd, case.scale, 1, dt, prec, stream))
        t_end = time.perf_counter() + 0.05  # settle the clock
        while time.perf_counter() < t_end:
            plain()
            torch.cuda.synchronize()
        t_plain = median_ms(plain)
        o_ref, l_ref = o.clone(), lse.clone()
        flops = 4 * hd * B * H * T * T / 2
        row = {"workload": case.name, "B": B, "H": H, "T": T, "hd": hd, "dtype": dts, "causal": True,
               "precision": int(prec), "plain_ms": round(t_plain, 5),
               "plain_tflops": round(flops / (t_plain * 1e-3) / 1e12, 2), "splits": []}
        ws = torch.empty((max(SPLIT_COUNTS) * (n + nr),), device=dev)
        for ns in SPLIT_COUNTS:
            o.fill_(float("nan"))
            lse.fill_(float("nan"))
            fn = lambda: fa.check(fa.fa_forward_splitkv(q, k, v, o, lse, ws, B, H, T, hd, case.scale, 1, ns, dt,
                                                        prec, stream))
            t = median_ms(fn)
            row["splits"].append({"nsplit": ns, "ms": round(t, 5), "speedup": round(t_plain / t, 3),
                                  "tflops": round(flops / (t * 1e-3) / 1e12, 2),
                                  "max_abs_diff_O": float(f"{float((o - o_ref).abs().max()):.3e}"),
                                  "max_abs_diff_L": float(f"{float((lse - l_ref).abs().max()):.3e}")})
        print(json.dumps(row), flush=True)
        rows.append(row)
        del q, k, v, o, lse, ws, o_ref, l_ref, case
        torch.cuda.empty_cache()
    print(json.dumps({"split_workloads": len(rows), "reps": 9, "warmup": 1,
                      "statistic": "median ms (HIP events, merge included)", **device_label(dev)}), flush=True)
    return 0


def counter_steps(name: str, steps: int = 2) -> None:
    """A few forward + backward steps of workload C2 (float32) or C4 (long context) for a counter run."""
    import numpy as np
    import torch

    import exact_attention_forward_amd as fa
    from exact_attention_forward_amd import inputs as I

    case, prec = {"C2": (lambda: I.gpt2m_case(I.F32), fa.FA_PREC_DEFAULT),
                  "C4": (I.long_case, fa.FA_PREC_BF16X2)}[name]
    case = case()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    B, H, T, hd = case.B, case.H, case.T, case.hd
    up = (lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)) \
        if case.dtype == I.BF16 else (lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev))
    dt = fa.FA_BF16 if case.dtype == I.BF16 else fa.FA_F32
    q, k, v, do = (up(getattr(case, n)) for n in ("q", "k", "v", "do"))
    f32 = lambda *s: torch.empty(s, device=dev, dtype=torch.float32)
    o, lse, dq, dk, dv, delta = f32(B, T, H, hd), f32(B, H, T), f32(B, T, H, hd), f32(B, T, H, hd), \
        f32(B, T, H, hd), f32(B, H, T)
    for _ in range(steps):
        fa.check(fa.fa_forward(q, k, v, o, lse, B, H, T, hd, case.scale, 1, dt, prec, stream))
        fa.check(fa.fa_backward_dq_delta(q, k, v, o, lse, do, dq, delta, B, H, T, hd, case.scale, 1, dt, prec,
                                         stream))
        fa.check(fa.fa_backward_dkv(q, k, v, lse, do, delta, dk, dv, B, H, T, hd, case.scale, 1, dt, prec, stream))
    torch.cuda.synchronize()


def host_label() -> dict:
    """Host CPU model, logical cores and the BLAS thread count the oracle runs with."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:  # pragma: no cover
        pass
    try:
        import numpy  # noqa: F401  (loads the BLAS library the oracle's products use)
        from threadpoolctl import threadpool_info

        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = None
    return {"cpu_model": model, "cpu_count": os.cpu_count(), "blas_threads": blas}


def device_label(dev) -> dict:
    """Device name, architecture, HIP version and the peak engine clock HIP reports."""
    import ctypes

    import torch

    prop = torch.cuda.get_device_properties(dev)
    clock_khz = None
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        v = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(v), 5, dev.index or 0) == 0:  # hipDeviceAttributeClockRate
            clock_khz = v.value
    except OSError:  # pragma: no cover
        pass
    return {"device": prop.name, "arch": prop.gcnArchName, "hip": torch.version.hip, "cus": prop.multi_processor_count,
            "peak_clock_mhz": clock_khz / 1000 if clock_khz else None}


def configs(args) -> int:
    """Every workload: sampled parity, then forward / backward / total times and the oracle's time."""
    import numpy as np
    import torch

    import exact_attention_forward_amd as fa
    from exact_attention_forward_amd import api
    from exact_attention_forward_amd import inputs as I

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    work = [("C0", I.tiny_case(False), fa.FA_PREC_DEFAULT), ("C0", I.tiny_case(True), fa.FA_PREC_DEFAULT)]
    work += [("C1", c, fa.FA_PREC_DEFAULT) for c in I.ragged_cases()]
    work += [("C2", lambda: I.gpt2m_case(I.F32), fa.FA_PREC_DEFAULT),
             ("C3", lambda: I.gpt2m_case(I.BF16), fa.FA_PREC_BF16),
             ("C3-split", lambda: I.gpt2m_case(I.BF16), fa.FA_PREC_BF16X2),
             ("C3-f16", lambda: I.gpt2m_case(I.F16), fa.FA_PREC_DEFAULT),
             ("C4", I.long_case, fa.FA_PREC_BF16X2),
             ("C4-single", I.long_case, fa.FA_PREC_BF16)]
    # outputs graded against the bar: with P and dS rounded once to bfloat16 the
    # long-context gradients exceed 2e-2 (reported, not graded; that workload
    # runs with split operands)
    graded = {"C4-single": ("O", "L")}
    label = device_label(dev)
    summary = []
    for cfg, case, prec in work:
        if callable(case):
            case = case()
        B, H, T, hd = case.B, case.H, case.T, case.hd
        t16 = {I.BF16: torch.bfloat16, I.F16: torch.float16}.get(case.dtype)
        up = (lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(t16).to(dev)) \
            if t16 is not None else (lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev))
        q, k, v, do = (up(getattr(case, n)) for n in ("q", "k", "v", "do"))
        o, lse = api.forward(q, k, v, case.scale, case.causal, prec)
        dq, dk, dv, delta = api.backward(q, k, v, o, lse, do, case.scale, case.causal, prec)
        torch.cuda.synchronize()
        # parity of sampled heads (every head of the small workloads), timing the oracle on the first
        heads = [(b, h) for b in range(B) for h in range(H)]
        if len(heads) > 4:
            heads = [heads[0], heads[len(heads) // 3], heads[2 * len(heads) // 3], heads[-1]]
        worst, t_oracle = cpu_baseline_heads(case, dict(O=o, L=lse, dQ=dq, dK=dk, dV=dv), heads)
        tol = 2e-5 if case.dtype == I.F32 else 2e-2
        names = graded.get(cfg, ("O", "L", "dQ", "dK", "dV"))
        ok = all(worst[n] <= tol for n in names)
        dt = {I.F32: fa.FA_F32, I.BF16: fa.FA_BF16, I.F16: fa.FA_F16}[case.dtype]

        def fwd():
            fa.check(fa.fa_forward(q, k, v, o, lse, B, H, T, hd, case.scale, int(case.causal),
                                   dt, prec, stream))

        def bwd():
            fa.check(fa.fa_backward(q, k, v, o, lse, do, dq, dk, dv, delta, B, H, T, hd, case.scale,
                                    int(case.causal), dt, prec, stream))

        def both():
            fwd()
            bwd()

        t_end = time.perf_counter() + 0.05  # settle the clock
        while time.perf_counter() < t_end:
            both()
            torch.cuda.synchronize()
        times = {}
        for name, fn in (("fwd", fwd), ("bwd", bwd), ("total", both)):
            fn()  # warm-up
            torch.cuda.synchronize()
            ts = []
            for _ in range(9):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            ts.sort()
            times[name] = {"median_ms": round(ts[4], 5), "min_ms": round(ts[0], 5)}
        pairs = B * H * (T * T / 2 if case.causal else T * T)
        counted = 14 * hd * pairs
        tflops = counted / (times["total"]["median_ms"] * 1e-3) / 1e12
        peak = PEAK_F32_MATRIX_TFLOPS if case.dtype == I.F32 else PEAK_BF16_TFLOPS  # fp16 dense = bf16 dense
        rec = {"config": cfg, "workload": case.name, "B": B, "H": H, "T": T, "hd": hd, "dtype": case.dtype,
               "causal": bool(case.causal), "precision": int(prec), "counted_gflop": round(counted / 1e9, 6),
               "times": times, "tflops": round(tflops, 3), "frac_of_peak": round(tflops / peak, 4),
               "peak_tflops": peak, "parity": {"heads": len(heads), "tol": tol, "ok": ok, "graded": list(names),
                                               "max_abs_err": {n: float(f"{e:.3e}") for n, e in worst.items()}},
               "oracle_s_per_head": round(t_oracle, 4), "oracle_s_est": round(t_oracle * B * H, 2)}
        print(json.dumps(rec), flush=True)
        summary.append(rec)
        del q, k, v, do, o, lse, dq, dk, dv, delta, case
        torch.cuda.empty_cache()
    print(json.dumps({"configs": len(summary), "all_parity_ok": all(r["parity"]["ok"] for r in summary),
                      "reps": 9, "warmup": 1, "statistic": "median and min ms (HIP events)",
                      "oracle_threads": host_label()["blas_threads"], "host": host_label(), **label}), flush=True)
    return 0 if all(r["parity"]["ok"] for r in summary) else 1


def _host_outputs(out):
    """The GPU outputs copied to host float64 once, outside every timed region."""
    import numpy as np

    return {n: t.cpu().numpy().astype(np.float64) for n, t in out.items()}


def _head_errors(host, b, h, ref, worst):
    import numpy as np

    for n, r in zip(("O", "L", "dQ", "dK", "dV"), ref):
        g = host[n][b, h] if n == "L" else host[n][b, :, h]
        worst[n] = max(worst.get(n, 0.0), float(np.abs(g - r).max()))


def _oracle_head(case, b, h):
    """(seconds, (O, L, dQ, dK, dV)) of the float64 oracle on one head; the timer covers only the oracle calls."""
    from oracle import attention as oracle

    qh, kh, vh, dh = (case.head_f64(n, b, h) for n in ("q", "k", "v", "do"))
    t0 = time.perf_counter()
    O, L, _ = oracle.head_forward(qh, kh, vh, case.scale, case.causal)
    dQ, dK, dV, _ = oracle.head_backward(qh, kh, vh, dh, case.scale, case.causal)
    return time.perf_counter() - t0, (O, L, dQ, dK, dV)


def cpu_baseline_heads(case, out, heads):
    """The oracle on the given heads: worst error of each output against it, and the
    oracle's time for the first head (the CPU baseline of one workload)."""
    host = _host_outputs(out)
    worst, t_first = {}, None
    for b, h in heads:
        t, ref = _oracle_head(case, b, h)
        t_first = t if t_first is None else t_first
        _head_errors(host, b, h, ref, worst)
    return worst, t_first


def cpu_baseline(case, out, budget_s: float):
    """Time the float64 oracle on whole heads of the workload until `budget_s` of oracle time is spent.

    Only the oracle's own calls are timed: the GPU outputs are copied to the
    host before, and each head is compared with them after, its timed calls.
    """
    import numpy as np

    host_info = host_label()
    threads = host_info["blas_threads"] or host_info["cpu_count"] or 1
    host = _host_outputs(out)
    heads = [(b, h) for b in range(case.B) for h in range(case.H)]
    order = np.random.default_rng(0).permutation(len(heads))
    done, worst, el = 0, {}, 0.0
    for idx in order:
        b, h = heads[idx]
        t, ref = _oracle_head(case, b, h)
        el += t
        done += 1
        _head_errors(host, b, h, ref, worst)
        if el >= budget_s:
            break
    flops = 14 * case.hd * case.T * case.T / 2 * done
    base = {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} of {case.B * case.H} heads (float64 NumPy, fwd+bwd per head), {el:.1f} s of oracle time",
            "cpu_model": host_info["cpu_model"], "cpu_count": host_info["cpu_count"],
            "blas_threads": host_info["blas_threads"]}
    parity = {"heads": done, "max_abs_err": {k: float(f"{v:.3e}") for k, v in worst.items()}, "tol": 2e-2,
              "ok": all(v <= 2e-2 for v in worst.values())}
    return base, parity


if __name__ == "__main__":
    sys.exit(main())
