"""Throughput of the fp16 tiled GEMM on one MI355X.

One step = one C = A*B call (the whole hot path) on the headline workload,
8192^3 with B stored N x K, seeded synthetic inputs already resident in HBM.
Prints ONE JSON line (rank 0):

  value      2*M*N*K*steps / wall time of the timed region, in TFLOPS
  roofline   the GEMM kernel against the dense fp16 matrix-core peak:
             achieved = 2*M*N*K / mean per-launch time (HIP events recorded
             on the launch stream between consecutive launches)
  cpu_baseline  the CPU oracle (fp64, all OpenMP threads) timed on a bounded
             block of whole output rows of the same workload

Usage: python bench.py [--gpus 1] [--steps 200] [--warmup 100] [--workload NAME]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fp16 GEMM TFLOPS (2MNK/s) at 8192³ on 1 MI355X; % of MFMA peak"
PEAK_F16_TFLOPS = 2516.6      # 256 CUs x 2.4 GHz x 4096 dense fp16 flop/clk/CU
KERNEL_SOURCES = ("dense_tiled_gemm_tgemm_amd/csrc/tgemm.hip", "dense_tiled_gemm_tgemm_amd/csrc/tgemm_plan.h")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str):
    """Per-launch HBM bytes from committed rocprofv3 counter summaries, when they
    were taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"tgemm_{workload}_hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(A, B, w, got, target_s: float = 12.0):
    """Time the oracle on whole output rows 0..R-1 (all N columns, full K)."""
    import numpy as np
    import oracle

    def run(rows):
        t0 = time.perf_counter()
        ref, ab = oracle.gemm(A[:rows], B, w.b_layout)
        return time.perf_counter() - t0, ref, ab

    # two-point calibration: the fixed cost (decoding all of B) drops out
    t_a, _, _ = run(16)
    t_b, _, _ = run(64)
    per_row = max((t_b - t_a) / 48, 1e-6)
    fixed = max(t_a - 16 * per_row, 0.0)
    rows = int(min(w.M, max(16, (target_s - fixed) / per_row)))
    dt, ref, ab = run(rows)
    res = oracle.check(got[:rows], ref, ab)
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
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the board's clock settles under sustained MFMA load over ~40 launches of
    # this size: 100 warmup launches (~80 ms) reach the steady state
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="instead of the GEMM, time the matrix-core ceiling probe (the GEMM's "
                         "instruction stream on the workload's values, without synchronization, "
                         "tile changes or C stores) and print its TFLOP/s")
    ap.add_argument("--torch-matmul", action="store_true",
                    help="instead of this library's GEMM, time torch.matmul (the vendor BLAS) on "
                         "the same inputs and print its TFLOP/s (context, not the headline)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the GEMM, run device-to-device copies of MIB MiB; used to "
                         "scale the HBM byte counters (FETCH_SIZE / WRITE_SIZE) of a profiler run")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
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

    if args.mfma_ceiling:
        # the GEMM's instruction stream without synchronization, tile changes or
        # C stores, on the workload's own A values (the operands' switching
        # activity sets the power-limited clock)
        tg.load()
        name = args.workload or inputs.HEADLINE
        w = inputs.WORKLOADS[name]
        A, _ = inputs.make_inputs(w)
        nbytes = 1 << min(26, int(A.nbytes).bit_length() - 1)
        data = torch.from_numpy(A.reshape(-1)[: nbytes // 2].copy()).to("cuda:0")
        stream = torch.cuda.current_stream()
        wg, iters = 256, 400
        out = torch.empty(wg * 256, dtype=torch.float32, device="cuda:0")
        flops = wg * 4 * iters * 128 * 2.0 * 16 * 16 * 32

        def probe_ms(buf):
            for _ in range(args.warmup):
                tg.mfma_issue_probe(wg, iters, buf.data_ptr(), nbytes, out.data_ptr(), stream.cuda_stream)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record(stream)
            for _ in range(args.steps):
                tg.mfma_issue_probe(wg, iters, buf.data_ptr(), nbytes, out.data_ptr(), stream.cuda_stream)
            ev[1].record(stream)
            torch.cuda.synchronize()
            return ev[0].elapsed_time(ev[1]) / args.steps

        ms = probe_ms(data)
        ms0 = probe_ms(torch.zeros_like(data))      # same instructions, operands that never toggle
        print(json.dumps({"probe": "mfma_ceiling", "data": f"{name} A, first {nbytes >> 20} MiB",
                          "workgroups": wg, "iters": iters, "ms": round(ms, 5),
                          "tflops": round(flops / ms / 1e9, 1),
                          "tflops_zero_operands": round(flops / ms0 / 1e9, 1),
                          "peak": PEAK_F16_TFLOPS}), flush=True)
        return

    name = args.workload or inputs.HEADLINE
    w = inputs.WORKLOADS[name]
    log(f"bench: workload {name} M={w.M} N={w.N} K={w.K} B {w.b_layout}")
    tg.load()
    dev = torch.device("cuda:0")
    A, B = inputs.make_inputs(w)
    Ad = torch.from_numpy(A).to(dev)
    Bd = torch.from_numpy(B).to(dev)
    Cd = torch.empty((w.M, w.N), dtype=torch.float16, device=dev)
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream
    lda, ldb, ldc = w.K, B.shape[1], w.N

    if args.torch_matmul:
        Bt = Bd.t() if w.b_layout == "NxK" else Bd

        def vendor():
            torch.matmul(Ad, Bt, out=Cd)

        for _ in range(args.warmup):
            vendor()
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

    def step():
        rc = tg.tgemm_f16(w.M, w.N, w.K, Ad.data_ptr(), lda, Bd.data_ptr(), ldb, w.b_layout,
                          Cd.data_ptr(), ldc, sptr)
        if rc != tg.TGEMM_OK:
            raise tg.TgemmError(rc)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

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
    log(f"bench: {args.steps} steps, region {region_ms:.3f} ms (host wall {wall * 1e3:.3f} ms), "
        f"per launch mean {mean_ms:.4f} min {min(per_launch_ms):.4f} max {max(per_launch_ms):.4f} ms")

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(region_ms / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": name, "M": w.M, "N": w.N, "K": w.K, "b_layout": w.b_layout,
                   "seed": w.seed, "accumulate": "f32", "output": "f16"},
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_F16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_F16_TFLOPS, 4),
            "traffic": traffic_from_profiles(name),
        },
    }
    if not args.no_cpu_baseline:
        torch.cuda.synchronize()
        got = Cd.cpu().numpy()
        rec["cpu_baseline"] = cpu_baseline(A, B, w, got)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
