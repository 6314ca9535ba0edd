"""Throughput of the fp16 tiled GEMM on one MI355X.

One step = one C = A*B call (the whole hot path) on the headline workload,
8192^3 with B stored N x K, seeded synthetic inputs already resident in HBM.
Prints ONE JSON line (rank 0):

  value      2*M*N*K*steps / wall time of the timed region, in TFLOPS
  roofline   the GEMM kernel against the dense fp16 matrix-core peak:
             achieved = 2*M*N*K / mean per-launch time (HIP events recorded
             on the launch stream between consecutive launches)
  launch_ms  mean, median, min and p90 of the per-launch times
  roofline.ceiling  the matrix-core ceiling probe in the same process (the
             GEMM's instruction stream without synchronization, tile changes or
             C stores, on the workload's A values, and on zeros) with its
             average clock; roofline.frac_of_ceiling = achieved / ceiling
  cold_cache variant B: up to 50 launches, each after a 512 MiB write that
             evicts the L2s and the Infinity Cache (events around the GEMM only)
  cpu_baseline  the CPU oracle (fp64, all OpenMP threads) timed on a bounded
             block of whole output rows of the same workload

Usage: python bench.py [--gpus 1] [--steps 200] [--warmup 100] [--workload NAME]
                       [--ab f16|bf16] [--out f16|bf16|f32] [--epilogue] [--tune]

The defaults time the headline line (binary16 in and out, tgemm_f16). --ab,
--out and --epilogue time the typed entry point (tgemm_gemm) on the same
workload: bfloat16 operands drawn from the same seeded values, a bfloat16 or
fp32 C, and the epilogue alpha = 0.5, a seeded fp32 bias, rectifier.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fp16 GEMM TFLOPS (2MNK/s) at 8192³ on 1 MI355X; % of MFMA peak"
PEAK_F16_TFLOPS = 2516.6      # 256 CUs x 2.4 GHz x 4096 dense fp16 flop/clk/CU (bfloat16 the same)
PEAK_F32_TFLOPS = 157.3       # dense fp32 matrix rate (256 flop/clk/CU)
KERNEL_SOURCES = ("dense_tiled_gemm_tgemm_amd/csrc/tgemm_kernels.h", "dense_tiled_gemm_tgemm_amd/csrc/tgemm_inst.hip",
                  "dense_tiled_gemm_tgemm_amd/csrc/tgemm.hip", "dense_tiled_gemm_tgemm_amd/csrc/tgemm_plan.h")
EPI_ALPHA = 0.5
COLD_FLUSH_BYTES = 512 << 20   # written between cold-cache launches (> 8 x 4 MiB L2 + 256 MiB Infinity Cache)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def code_text(src: str) -> str:
    """C++ source without comments and whitespace: what the compiler sees
    (the sources hold no string literal with // or /* in it)."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return re.sub(r"\s+", "", src)


def kernel_source_hash() -> str:
    """Hash of the kernel and planning sources' code (comments ignored): the
    recorded HBM traffic applies while this matches the hash it was taken with."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


def variant_tag(ab: str, out: str, epilogue: bool) -> str:
    """"" for the headline variant, else e.g. "_bf16_f32_epi"."""
    if ab == "f16" and out == "f16" and not epilogue:
        return ""
    return f"_{ab}_{out}" + ("_epi" if epilogue else "")


def traffic_from_profiles(workload: str, tag: str = ""):
    """Per-launch HBM bytes from committed rocprofv3 counter summaries, when they
    were taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"tgemm_{workload}{tag}_hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(A, B, w, got, target_s: float = 12.0, ab="f16", out="f16", alpha=1.0, bias=None, act="none"):
    """Time the oracle on whole output rows 0..R-1 (all N columns, full K)."""
    import oracle

    plain = ab == "f16" and out == "f16" and bias is None and alpha == 1.0 and act == "none"

    def run(rows):
        t0 = time.perf_counter()
        if plain:
            ref, tol = oracle.gemm(A[:rows], B, w.b_layout)
        else:
            ref, tol = oracle.gemm_ex(A[:rows], B, w.b_layout, ab, alpha, bias, act)
        return time.perf_counter() - t0, ref, tol

    # two-point calibration: the fixed cost (decoding all of B) drops out
    t_a, _, _ = run(16)
    t_b, _, _ = run(64)
    per_row = max((t_b - t_a) / 48, 1e-6)
    fixed = max(t_a - 16 * per_row, 0.0)
    rows = int(min(w.M, max(16, (target_s - fixed) / per_row)))
    dt, ref, tol = run(rows)
    res = oracle.check(got[:rows], ref, tol) if plain else oracle.check_ex(got[:rows], out, ref, tol)
    flops = 2.0 * rows * w.N * w.K
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOPS",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"output rows 0..{rows - 1} (all {w.N} columns, K={w.K}) of {w.name}; "
                  f"{dt:.1f} s for {flops / 1e9:.0f} GFLOP",
        "parity_rows_checked": rows,
        "parity_fail": res["nfail"],
        "host_cpus": len(os.sched_getaffinity(0)),
        "cpu_model": cpu_model(),
    }


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _read_csv(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _short(name: str) -> str:
    """Kernel name without its argument list ("void tg::k<...>(tg::Args)" -> "tg::k<...>")."""
    name = name.strip()
    if name.startswith("void "):
        name = name[5:]
    return name.split("(")[0]


def trace_summary(csv_path: str, bench_json: str) -> str:
    """Markdown summary of a rocprofv3 kernel trace of one bench.py run: the
    GEMM dispatches of the timed region only (after the run's warm-up
    launches, as many as its timed steps), against the run's own JSON line."""
    import numpy as np

    with open(bench_json) as f:
        rec = json.loads([l for l in f.read().splitlines() if l.startswith("{")][-1])
    rows = _read_csv(csv_path)
    if not rows or "Kernel_Name" not in rows[0]:
        raise SystemExit(f"{csv_path}: not a rocprofv3 kernel trace")
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    by = {}
    for r in rows:
        by.setdefault(_short(r["Kernel_Name"]), []).append(r)
    gemm = max((k for k in by if "tgemm_" in k and "probe" not in k and "ceiling" not in k),
               key=lambda k: len(by[k]))
    d = by[gemm]
    n_warm, steps = rec["warmup_launches"], rec["steps"]
    timed = d[n_warm:n_warm + steps]
    if len(timed) != steps:
        raise SystemExit(f"{len(d)} dispatches of {gemm}, expected at least {n_warm} + {steps}")
    dur = np.array([(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6 for r in timed])   # ms
    flops = 2.0 * rec["config"]["M"] * rec["config"]["N"] * rec["config"]["K"]
    peak = rec["roofline"]["peak"]
    mean, med = float(dur.mean()), float(np.median(dur))
    lines = [f"| kernel | dispatches in trace | timed dispatches | mean ms | median ms | min ms | p90 ms |",
             "|---|---|---|---|---|---|---|",
             f"| {gemm} | {len(d)} | {len(timed)} (#{n_warm}..#{n_warm + steps - 1}) | {mean:.5f} | {med:.5f} | "
             f"{dur.min():.5f} | {np.percentile(dur, 90):.5f} |", "",
             f"2MNK / mean = {flops / mean / 1e9:.1f} TFLOP/s = {flops / mean / 1e9 / peak:.4f} of {peak}; "
             f"2MNK / median = {flops / med / 1e9:.1f} TFLOP/s = {flops / med / 1e9 / peak:.4f}.",
             f"Same run's JSON line: value {rec['value']} TFLOP/s, ms_per_step {rec['ms_per_step']}, "
             f"roofline.frac {rec['roofline']['frac']} (HIP events between consecutive launches, so "
             f"the dispatch time is at most the per-step time: {mean:.5f} <= {rec['ms_per_step']})."]
    ceil = rec["roofline"].get("ceiling")
    if ceil:
        lines.append(f"Matrix-core ceiling probe, same process: {ceil['tflops']} TFLOP/s at "
                     f"{ceil['clock_ghz']} GHz (zero operands {ceil['tflops_zero_operands']} at "
                     f"{ceil['clock_ghz_zero_operands']} GHz); GEMM (trace mean) at "
                     f"{flops / mean / 1e9 / ceil['tflops']:.3f} of it.")
    return "\n".join(lines)


def counter_summary(csv_paths) -> str:
    """Markdown table of rocprofv3 --pmc runs (counter_collection CSVs): per
    kernel, the median over its dispatches of each counter, with the derived
    clock (GRBM_GUI_ACTIVE per die over the dispatch duration) and matrix-core
    occupancy (SQ_VALU_MFMA_BUSY_CYCLES over 1024 SIMDs x active cycles per die)."""
    import numpy as np

    per = {}      # (kernel, dispatch) -> {counter: value, "_ns": duration}
    for path in csv_paths:
        for r in _read_csv(path):
            key = (_short(r["Kernel_Name"]), path, r["Dispatch_Id"])
            d = per.setdefault(key, {})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            if "Start_Timestamp" in r and "End_Timestamp" in r:
                d["_ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    kern = {}
    for (k, _, _), d in per.items():
        kern.setdefault(k, []).append(d)
    out = []
    for k, ds in sorted(kern.items(), key=lambda kv: -len(kv[1])):
        if "tgemm_" not in k and "copyBuffer" not in k and "Cijk" not in k:
            continue
        names = sorted({c for d in ds for c in d if not c.startswith("_")})
        med = {c: float(np.median([d[c] for d in ds if c in d])) for c in names}
        row = [f"{c} {med[c]:,.0f}" for c in names]
        if "GRBM_GUI_ACTIVE" in med:
            clk = [d["GRBM_GUI_ACTIVE"] / 8 / d["_ns"] for d in ds if "_ns" in d and d["_ns"] > 0
                   and "GRBM_GUI_ACTIVE" in d]
            if clk:
                row.append(f"clock {np.median(clk):.3f} GHz")
            if "SQ_VALU_MFMA_BUSY_CYCLES" in med:
                occ = [d["SQ_VALU_MFMA_BUSY_CYCLES"] / (d["GRBM_GUI_ACTIVE"] / 8 * 1024) for d in ds
                       if "SQ_VALU_MFMA_BUSY_CYCLES" in d and "GRBM_GUI_ACTIVE" in d]
                row.append(f"MFMA occupancy {100 * np.median(occ):.1f}%")
        if "SQ_WAIT_ANY" in med and "SQ_WAVE_CYCLES" in med:
            row.append(f"waiting {100 * med['SQ_WAIT_ANY'] / med['SQ_WAVE_CYCLES']:.1f}% of wave-cycles")
        if "SQ_LDS_BANK_CONFLICT" in med and "SQ_LDS_IDX_ACTIVE" in med:
            row.append(f"LDS conflict cycles {100 * med['SQ_LDS_BANK_CONFLICT'] / max(med['SQ_LDS_IDX_ACTIVE'], 1):.2f}% "
                       f"of LDS active cycles")
        out.append(f"| {k} | {len(ds)} | " + "; ".join(row) + " |")
    return "\n".join(["| kernel | dispatches | medians per dispatch |", "|---|---|---|"] + out)


def traffic_summary(fetch_csv, write_csv, fetch_copy_csv, write_copy_csv, workload: str, copy_mib: int) -> dict:
    """HBM-side bytes per GEMM launch from rocprofv3 --pmc FETCH_SIZE and
    WRITE_SIZE runs (KiB per dispatch, medians over the GEMM kernel's
    dispatches), each scaled by what the same counter reads for device copies
    of copy_mib MiB (bench.py --copy-calibration): the record bench.py reports
    as roofline.traffic while the kernel sources hash to the stored value."""
    import numpy as np
    from dense_tiled_gemm_tgemm_amd import inputs

    def med(path, counter, pick):
        by = {}
        for r in _read_csv(path):
            if r["Counter_Name"] != counter:
                continue
            key = (_short(r["Kernel_Name"]), r["Dispatch_Id"])
            by[key] = by.get(key, 0.0) + float(r["Counter_Value"])
        names = {k for k, _ in by}
        kern = [n for n in names if pick(n)]
        if len(kern) != 1:
            raise SystemExit(f"{path}: expected one {counter} kernel to pick, found {sorted(names)}")
        vals = [v for (k, _), v in by.items() if k == kern[0]]
        return kern[0], float(np.median(vals)), len(vals)

    gemm = lambda n: "tgemm_" in n and "probe" not in n and "ceiling" not in n
    copy = lambda n: "copyBuffer" in n or "copy" in n.lower()
    kern, fetch, nf = med(fetch_csv, "FETCH_SIZE", gemm)
    _, write, nw = med(write_csv, "WRITE_SIZE", gemm)
    _, cfetch, _ = med(fetch_copy_csv, "FETCH_SIZE", copy)
    _, cwrite, _ = med(write_copy_csv, "WRITE_SIZE", copy)
    nbytes = copy_mib << 20
    fs, ws = nbytes / (cfetch * 1024), nbytes / (cwrite * 1024)
    w = inputs.WORKLOADS[workload]
    return {"workload": workload, "kernel": kern, "kernel_source_hash": kernel_source_hash(),
            "fetch_size_kib_per_launch": fetch, "write_size_kib_per_launch": write, "dispatches": [nf, nw],
            "copy_calibration": {"bytes_copied": nbytes, "fetch_size_kib": cfetch, "write_size_kib": cwrite,
                                 "fetch_scale": fs, "write_scale": ws},
            "hbm_bytes_per_launch": int(round(fetch * 1024 * fs + write * 1024 * ws)),
            "compulsory_bytes": int(2 * (w.M * w.K + w.N * w.K + w.M * w.N))}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the board's clock settles under sustained MFMA load over ~40 launches of
    # this size: 100 warmup launches (~80 ms) reach the steady state
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--warmup-seconds", type=float, default=0.3,
                    help="after --warmup launches, keep launching until this much time has passed: the board's "
                         "power-limited clock settles over tens of milliseconds of sustained load, which a fixed "
                         "launch count does not give small problems")
    ap.add_argument("--ab", choices=("f16", "bf16", "f32"), default="f16", help="operand type")
    ap.add_argument("--out", choices=("f16", "bf16", "f32"), default="f16", help="output type")
    ap.add_argument("--epilogue", action="store_true", help="alpha = 0.5, seeded fp32 bias, rectifier")
    ap.add_argument("--tune", action="store_true",
                    help="run the runtime tuner on the workload first; the timed launches use its choice")
    ap.add_argument("--k-step", type=int, default=0, help="launch choice (tgemm_gemm_config): K step 32 or 64")
    ap.add_argument("--stages", type=int, default=0, help="launch choice: LDS ring depth")
    ap.add_argument("--tile-m", type=int, default=0, help="launch choice: tile rows 256, 128 or 64")
    ap.add_argument("--producers", type=int, default=0, help="launch choice: 4 = producer/consumer workgroups")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache launches (512 MiB written before each) reported beside the headline")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the matrix-core ceiling probe reported in roofline.ceiling")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="instead of the GEMM, time the matrix-core ceiling probe (the GEMM's "
                         "instruction stream on the workload's values, without synchronization, "
                         "tile changes or C stores) and print its TFLOP/s")
    ap.add_argument("--stream-probes", metavar="KINDS",
                    help="instead of the GEMM, time the instruction-stream probes (comma-separated kinds of "
                         "include/tgemm_probe.h in lower case without the TGEMM_STREAM_ prefix, or 'all') on "
                         "the workload's A values and on zeros; one JSON line each")
    ap.add_argument("--torch-matmul", action="store_true",
                    help="instead of this library's GEMM, time torch.matmul (the vendor BLAS) on "
                         "the same inputs and print its TFLOP/s (context, not the headline)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the GEMM, run device-to-device copies of MIB MiB; used to "
                         "scale the HBM byte counters (FETCH_SIZE / WRITE_SIZE) of a profiler run")
    ap.add_argument("--trace-summary", metavar="CSV",
                    help="print a markdown summary of a rocprofv3 kernel trace of a bench.py run (its timed "
                         "dispatches only) and exit; needs --bench-json")
    ap.add_argument("--bench-json", metavar="FILE", help="the JSON line printed by the traced run")
    ap.add_argument("--counter-summary", metavar="CSV", nargs="+",
                    help="print a markdown table of rocprofv3 --pmc counter CSVs and exit")
    ap.add_argument("--traffic-summary", metavar="CSV", nargs=4,
                    help="FETCH_SIZE and WRITE_SIZE counter CSVs of the GEMM, then of --copy-calibration runs: "
                         "print the HBM traffic record (JSON) for --workload and exit")
    ap.add_argument("--copy-mib", type=int, default=1024, help="MiB per copy of the calibration runs")
    args = ap.parse_args()

    if args.traffic_summary:
        print(json.dumps(traffic_summary(*args.traffic_summary, args.workload or "sq8192_nt", args.copy_mib),
                         indent=1))
        return
    if args.trace_summary:
        print(trace_summary(args.trace_summary, args.bench_json))
        return
    if args.counter_summary:
        print(counter_summary(args.counter_summary))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {args.warmup + args.steps} copies of {n} bytes")
        return

    import dense_tiled_gemm_tgemm_amd as tg
    from dense_tiled_gemm_tgemm_amd import inputs

    def warm_up(fn):
        """args.warmup launches, then more until args.warmup_seconds have passed
        (the board's power-limited clock settles over the first fraction of a
        second of sustained matrix work)."""
        t_w = time.perf_counter()
        n = 0
        for _ in range(args.warmup):
            fn()
            n += 1
        torch.cuda.synchronize()
        while time.perf_counter() - t_w < args.warmup_seconds:
            for _ in range(16):
                fn()
                n += 1
            torch.cuda.synchronize()
        return n, time.perf_counter() - t_w

    def probe_data(A16):
        """The workload's A as probe operands: its first 64 MiB (a power of two
        of at least 1 MiB, the values repeated for a smaller A)."""
        a16 = np.ascontiguousarray(A16).view(np.uint16).reshape(-1)
        if a16.nbytes < (1 << 20):                    # the probes read at least 1 MiB: repeat the values
            a16 = np.resize(a16, (1 << 20) // 2)
        nbytes = 1 << min(26, int(a16.nbytes).bit_length() - 1)
        return torch.from_numpy(a16[: nbytes // 2].view(np.int16).copy()).to("cuda:0"), nbytes

    def probe_time(launch, wg, steps):
        """Mean ms per launch of a probe (after the warm-up) and its average
        clock in GHz (one more launch records each workgroup's shader cycles
        and 100 MHz reference ticks)."""
        stream = torch.cuda.current_stream()
        clk = torch.zeros(2 * wg, dtype=torch.int64, device="cuda:0")
        warm_up(launch)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(steps):
            launch()
        ev[1].record(stream)
        launch(clk.data_ptr())
        torch.cuda.synchronize()
        c = clk.cpu().numpy().reshape(wg, 2).astype(np.float64)
        return ev[0].elapsed_time(ev[1]) / steps, float(c[:, 0].sum() / c[:, 1].sum() / 10.0)

    def mfma_ceiling(A16, name, steps):
        """The matrix-core ceiling probe (libtgemm_probe.so): the GEMM's
        instruction stream without synchronization, tile changes or C stores,
        on the workload's own A values (the operands' switching activity sets
        the power-limited clock), and on zeros (the same instructions with
        operands that never toggle). TFLOP/s and the probe's average clock."""
        from dense_tiled_gemm_tgemm_amd import probe
        probe.load()
        data, nbytes = probe_data(A16)
        stream = torch.cuda.current_stream()
        wg, iters = 256, 400
        out = torch.empty(wg * 256, dtype=torch.float32, device="cuda:0")
        flops = wg * 4 * iters * 128 * 2.0 * 16 * 16 * 32

        def probe_ms(buf):
            def one(c=None):
                probe.mfma_issue_probe(wg, iters, buf.data_ptr(), nbytes, out.data_ptr(), c, stream.cuda_stream)
            return probe_time(one, wg, steps)

        ms, ghz = probe_ms(data)
        ms0, ghz0 = probe_ms(torch.zeros_like(data))
        return {"data": f"{name} A, first {nbytes >> 20} MiB", "workgroups": wg, "iters": iters,
                "ms": round(ms, 5), "tflops": round(flops / ms / 1e9, 1), "clock_ghz": round(ghz, 3),
                "tflops_zero_operands": round(flops / ms0 / 1e9, 1), "clock_ghz_zero_operands": round(ghz0, 3)}

    if args.stream_probes:
        # the GEMM's instruction stream taken apart (libtgemm_probe.so): per
        # kind and operand set, TFLOP/s, average clock, and matrix-core issue
        # efficiency = TFLOP/s over the dense peak scaled to that clock
        from dense_tiled_gemm_tgemm_amd import probe
        probe.load()
        name = args.workload or inputs.HEADLINE
        A, _ = inputs.make_inputs(inputs.WORKLOADS[name])
        data, nbytes = probe_data(A)
        zeros = torch.zeros_like(data)
        stream = torch.cuda.current_stream()
        wg, iters = 256, 200
        out = torch.empty(wg * 512, dtype=torch.float32, device="cuda:0")
        kinds = args.stream_probes.split(",") if args.stream_probes != "all" else list(probe.STREAM_KINDS)
        for kind in kinds:
            _, _, fpr = probe.STREAM_KINDS[kind]
            peak = PEAK_F32_TFLOPS if kind.startswith("f32") else PEAK_F16_TFLOPS
            for tag, buf in (("workload", data), ("zeros", zeros)):
                def one(c=None, buf=buf, kind=kind):
                    probe.mfma_stream_probe(kind, wg, iters, buf.data_ptr(), nbytes, out.data_ptr(), c,
                                            stream.cuda_stream)
                ms, ghz = probe_time(one, wg, args.steps)
                tf = wg * iters * float(fpr) / ms / 1e9
                print(json.dumps({"probe": "stream", "kind": kind, "operands": tag, "data": f"{name} A",
                                  "ms": round(ms, 5), "tflops": round(tf, 1), "clock_ghz": round(ghz, 3),
                                  "issue_efficiency": round(tf / (peak * ghz / 2.4), 4)}), flush=True)
        return

    if args.mfma_ceiling:
        tg.load()
        name = args.workload or inputs.HEADLINE
        A, _ = inputs.make_inputs(inputs.WORKLOADS[name])
        rec = {"probe": "mfma_ceiling", **mfma_ceiling(A, name, args.steps), "peak": PEAK_F16_TFLOPS}
        print(json.dumps(rec), flush=True)
        return

    name = args.workload or inputs.HEADLINE
    w = inputs.WORKLOADS[name]
    tag = variant_tag(args.ab, args.out, args.epilogue)
    log(f"bench: workload {name} M={w.M} N={w.N} K={w.K} B {w.b_layout} {args.ab}->{args.out}"
        f"{' epilogue' if args.epilogue else ''}")
    tg.load()
    dev = torch.device("cuda:0")
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}
    A, B = inputs.make_inputs(w, args.ab)
    if args.ab == "f32":
        Ad = torch.from_numpy(A).to(dev)
        Bd = torch.from_numpy(B).to(dev)
    else:
        A = A.view(np.uint16)
        B = B.view(np.uint16)
        Ad = torch.from_numpy(A.view(np.int16)).to(dev).view(tdt[args.ab])
        Bd = torch.from_numpy(B.view(np.int16)).to(dev).view(tdt[args.ab])
    Cd = torch.empty((w.M, w.N), dtype=tdt[args.out], device=dev)
    alpha, bias_np, act = 1.0, None, "none"
    if args.epilogue:
        alpha, act = EPI_ALPHA, "relu"
        bias_np = inputs.random_bias(w.N, w.seed + 77)
    bias_d = torch.from_numpy(bias_np).to(dev) if bias_np is not None else None
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream
    lda, ldb, ldc = w.K, B.shape[1], w.N

    if args.torch_matmul:
        Bt = Bd.t() if w.b_layout == "NxK" else Bd

        def vendor():
            torch.matmul(Ad, Bt, out=Cd)

        warm_up(vendor)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        for _ in range(args.steps):
            vendor()
        ev[1].record(stream)
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / args.steps
        print(json.dumps({"vendor": "torch.matmul", "workload": name, "ms": round(ms, 5),
                          "tflops": round(float(w.flops) / ms / 1e9, 1)}), flush=True)
        return

    launch = dict(k_step=args.k_step, stages=args.stages, tile_m=args.tile_m, producers=args.producers)
    explicit = any(launch.values())
    if tag == "" and not explicit:
        def step():
            rc = tg.tgemm_f16(w.M, w.N, w.K, Ad.data_ptr(), lda, Bd.data_ptr(), ldb, w.b_layout,
                              Cd.data_ptr(), ldc, sptr)
            if rc != tg.TGEMM_OK:
                raise tg.TgemmError(rc)
    else:
        bptr = bias_d.data_ptr() if bias_d is not None else None

        def step():
            rc = tg.tgemm_gemm_config(w.M, w.N, w.K, args.ab, Ad.data_ptr(), lda, Bd.data_ptr(), ldb, w.b_layout,
                                      args.out, Cd.data_ptr(), ldc, alpha, bptr, act, sptr, **launch)
            if rc != tg.TGEMM_OK:
                raise tg.TgemmError(rc)

    tuned = None
    if args.tune:
        warm_up(step)                                 # tune on a settled clock
        rc, tuned = tg.tgemm_tune_gemm(w.M, w.N, w.K, args.ab, Ad.data_ptr(), lda, Bd.data_ptr(), ldb, w.b_layout,
                                       args.out, Cd.data_ptr(), ldc, alpha,
                                       bias_d.data_ptr() if bias_d is not None else None, act, sptr, 5)
        if rc != tg.TGEMM_OK:
            raise tg.TgemmError(rc, "tune")
        log(f"bench: tuned choice {tuned}")

    n_warm, t_warm = warm_up(step)
    log(f"bench: {n_warm} warm-up launches in {t_warm:.3f} s")

    # events recorded on the launch stream between consecutive launches
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_launch_ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    region_ms = ev[0].elapsed_time(ev[-1])

    flops = float(w.flops)
    value = flops * args.steps / (region_ms / 1e3) / 1e12
    mean_ms = float(np.mean(per_launch_ms))
    achieved = flops / (mean_ms / 1e3) / 1e12
    peak = PEAK_F32_TFLOPS if args.ab == "f32" else PEAK_F16_TFLOPS
    log(f"bench: {args.steps} steps, region {region_ms:.3f} ms (host wall {wall * 1e3:.3f} ms), "
        f"per launch mean {mean_ms:.4f} min {min(per_launch_ms):.4f} max {max(per_launch_ms):.4f} ms")

    def stats(ms):
        q = np.percentile(ms, [50, 90])
        return {"mean": round(float(np.mean(ms)), 5), "median": round(float(q[0]), 5),
                "min": round(float(np.min(ms)), 5), "p90": round(float(q[1]), 5)}

    cold = None
    if not args.no_cold:
        # variant B: a 512 MiB write between launches evicts every L2 and the
        # 256 MiB Infinity Cache, so each launch reads its operands from HBM;
        # events bracket the GEMM launches only
        flush = torch.empty(COLD_FLUSH_BYTES, dtype=torch.uint8, device=dev)
        n_cold = min(args.steps, 50)
        ev_c = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n_cold)]
        torch.cuda.synchronize()
        for i in range(n_cold):
            flush.fill_(i & 255)
            ev_c[2 * i].record(stream)
            step()
            ev_c[2 * i + 1].record(stream)
        torch.cuda.synchronize()
        cold_ms = [ev_c[2 * i].elapsed_time(ev_c[2 * i + 1]) for i in range(n_cold)]
        del flush
        cs = stats(cold_ms)
        cold = {"flush_bytes": COLD_FLUSH_BYTES, "launches": n_cold, "launch_ms": cs,
                "tflops_at_median": round(flops / (cs["median"] / 1e3) / 1e12, 2)}
        log(f"bench: cold-cache launches (512 MiB written before each): median {cs['median']:.4f} ms, "
            f"{cold['tflops_at_median']:.1f} TFLOP/s")

    ceiling = None
    if not args.no_ceiling and args.ab == "f16":       # the probe runs binary16 MFMAs
        # same process, same board, after the timed region: the matrix-core
        # ceiling of this instruction mix on the workload's values
        ceiling = mfma_ceiling(A, name, min(args.steps, 100))
        log(f"bench: ceiling probe {ceiling['tflops']} TFLOP/s at {ceiling['clock_ghz']} GHz "
            f"(zero operands {ceiling['tflops_zero_operands']} at {ceiling['clock_ghz_zero_operands']} GHz); "
            f"GEMM at {achieved / ceiling['tflops']:.3f} of it")

    metric = METRIC if (tag == "" and name == inputs.HEADLINE) else (
        f"GEMM TFLOPS (2MNK/s) at {w.M}x{w.N}x{w.K}, {args.ab} in, {args.out} out"
        f"{', alpha/bias/relu epilogue' if args.epilogue else ''} on 1 MI355X")
    rec = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_launches": n_warm,
        "ms_per_step": round(region_ms / args.steps, 5),
        "launch_ms": stats(per_launch_ms),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.ab,
        "data": "synthetic",
        "config": {"workload": name, "M": w.M, "N": w.N, "K": w.K, "b_layout": w.b_layout,
                   "seed": w.seed, "accumulate": "f32", "output": args.out,
                   "epilogue": (f"alpha={EPI_ALPHA}, bias, relu" if args.epilogue else "none"),
                   "launch": ({k: tuned[k] for k in ("k_step", "stages", "group_m", "num_xcd", "tile_m",
                                                     "producers")} if tuned
                              else ({k: v for k, v in launch.items() if v} if explicit else "default"))},
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": traffic_from_profiles(name, tag),
        },
    }
    if ceiling is not None:
        rec["roofline"]["ceiling"] = ceiling
        rec["roofline"]["frac_of_ceiling"] = round(achieved / ceiling["tflops"], 4)
    if cold is not None:
        rec["cold_cache"] = cold
    if not args.no_cpu_baseline:
        torch.cuda.synchronize()
        got = Cd.cpu().numpy() if args.out == "f32" else Cd.view(torch.int16).cpu().numpy().view(np.uint16)
        rec["cpu_baseline"] = cpu_baseline(A, B, w, got, ab=args.ab, out=args.out, alpha=alpha, bias=bias_np,
                                           act=act)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
