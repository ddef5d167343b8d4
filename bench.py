#!/usr/bin/env python3
"""Benchmark of the flash-attention backward on one MI355X.

Workload (default): the long-cache causal-tail case, N=2048 query rows against an M=75520
cache, H=24 query heads over Hkv=4 KV heads (GQA 6), D=Dv=256, q8_0 K/V, F32 Q/dO drawn
N(0,1), F16 causal-tail mask (query i sees keys j <= M-N+i), scale 1/16, seed 0.

A step is one fa_back_run (every kernel of the backward) on inputs already resident in HBM.
W warmup steps, then K timed steps between device synchronisations. Each timed step goes
through fa_back_run_timed, which records HIP events on the launch stream between the
library's kernels, so the dominant kernel's average duration is measured live over the
timed region. Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c4|c4q4|c4n16|c3|...]
                  [--mask stored|implicit] [--saved]

--mask implicit passes the workload's causal-tail mask as the storage-free mask type (the
library forms it from the row and key indices) instead of the stored F16 mask; the metric's
workload is the stored mask. --saved times fa_back_run_saved (forward-saved LSE and O; walk 1
and the merge are not run) with the LSE that fa_back_run itself produces on the same inputs
and a synthetic F32 O drawn N(0,1) (its values only set delta and the dS bound); its work is
counted as 2*V*(3D + 4Dv) (walk 2 and the key side).
"""
import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attn-backward TFLOP/s + ms/call, q8_0 H24/Hkv4/D256 N2048 M75520"
PEAK_MFMA_F16_TFLOPS = 2500.0      # MI355X dense fp16/bf16 MFMA
PEAK_HBM_GBS = 8000.0

# matrix-product work per visible (row, key, head) triple, per phase (D = Dv)
PHASE_FLOPS_PER_PAIR_PER_D = {"walk1": 4, "walk2": 6, "kvpass": 8}
# the kernels a phase may run (the plan picks one), as name prefixes of their instantiations
# ("walk2" is the dQ phase: walk 2, or the dQ pass from the key side's stored dS)
KERNEL_PREFIXES = {"walk1": ("walk1_rows_kernel<D>", "walk1_keys_kernel<D>", "qpass_kernel<D, false"),
                   "walk2": ("qpass_kernel<D, true", "dq_stored_kernel<D>"), "kvpass": ("kvpass_kernel<D",)}
# the dQ phase with stored dS forms only dS K: 2 * D flops per visible triple
DQ_STORED_FLOPS_PER_PAIR_PER_D = 2


def phase_bytes(p, phase):
    """Algorithmic HBM bytes of one launch of a phase's kernel: what it must read and write once.
    Every phase reads the K/V cache (stored types) and the fp16 q and dO rows (2 bytes a value,
    each row once); walk 1 and walk 2 also read the stored mask and write 8 bytes of statistics a
    row, walk 2 writes dQ (F32), the key side reads 8 bytes of statistics a row and writes dK and
    dV (F32). When the plan stores dS (2 bytes per (row, key, head)), the key side also writes
    it, and the dQ phase reads it, K, the statistics, and writes dQ."""
    import fa_inputs
    import flash_attention_backward_amd as fab
    stored = bool(fab.fa_back_layout_query(fab.fa_back.describe(p)).plan_flags & fab.fa_back.FLAG_DS_STORE)
    ds = 2 * p.N * p.H * p.M if stored else 0
    kv = fa_inputs.storage_bytes(p.k) + fa_inputs.storage_bytes(p.v)
    rows = p.N * p.H
    qd = 2 * 2 * rows * p.D
    mask = 0 if p.mask is None or p.mask_type == "causal_tail" else fa_inputs.storage_bytes(p.mask)
    if phase == "kvpass":
        return kv + qd + 8 * rows + 4 * 2 * p.Hkv * p.M * p.D + ds
    if phase == "walk2":
        if stored:
            return fa_inputs.storage_bytes(p.k) + ds + 8 * rows + 4 * rows * p.D
        return kv + qd + mask + 8 * rows + 4 * rows * p.D
    return kv + qd + mask + 8 * rows


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash():
    """sha256 over the HIP sources of the library (the kernels whose counters were taken)."""
    import hashlib
    csrc = os.path.join(ROOT, "flash_attention_backward_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".h", ".hip")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(prefixes, workload):
    """(kernel name, HBM bytes per launch) of the kernel whose name starts with one of `prefixes`
    in the committed FETCH_SIZE / WRITE_SIZE summary of `workload`, or (None, None) when that
    summary was taken on other kernel sources (or is absent)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None, None
    if rec.get("source_sha256") != kernel_source_hash():
        return None, None
    for name, k in rec.get("kernels", {}).get(workload, {}).items():
        if name.startswith(prefixes):
            return name, k.get("hbm_bytes_per_launch")
    return None, None


def copy_calibration(mib: int, reps: int = 3):
    """A plain device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copy calibration: {reps} copies of {mib} MiB (read {mib} MiB + write {mib} MiB each)")
    del a, b
    torch.cuda.empty_cache()


def copy_rate_gbs(mib: int = 1024, reps: int = 5) -> float:
    """Read + write GB/s of a plain device copy of `mib` MiB (torch copy_, timed with events on the
    current stream after two untimed copies): what a streaming kernel reaches on this chip."""
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(2):
        b.copy_(a)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    torch.cuda.empty_cache()
    return 2 * mib * (1 << 20) / (ms * 1e-3) / 1e9


def describe_workload(p):
    mask = "none" if p.mask is None else (
        "causal-tail implicit" if p.mask_type == "causal_tail" else f"causal-tail {p.mask_type}")
    return (f"{p.name}: N{p.N} M{p.M} H{p.H} Hkv{p.Hkv} D{p.D} K {p.k_type} V {p.v_type} "
            f"Q/dO {p.q_type} mask {mask}")


def cpu_baseline(workload: str, rows: int):
    """Time the float64 oracle on a bounded sample of the same workload: its last `rows`
    query rows of every head (all of them when it has no more) against the whole cache (same
    draws, same mask rows)."""
    import numpy as np
    import fa_inputs
    from oracle import fa_back_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    s = fa_inputs.make(workload)
    if rows < s.N:
        s.name = f"{workload} last {rows} rows"
        s.q = np.ascontiguousarray(s.q[:, s.N - rows:, :])
        s.d = np.ascontiguousarray(s.d[s.N - rows:, :, :])
        if s.mask is not None:
            s.mask = np.ascontiguousarray(s.mask[:, s.N - rows:, :])
        s.N = rows
    f = fa_inputs.flop_count(s)
    log(f"cpu baseline: oracle on {s.name} ({f['full'] / 1e9:.1f} GFLOP counted), {threads} BLAS threads")
    t0 = time.perf_counter()
    O.run_problem(s)
    dt = time.perf_counter() - t0
    log(f"cpu baseline: {dt:.2f} s")
    return {"value": f["full"] / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "seconds": dt,
            "sample": f"float64 numpy oracle on the last {s.N} query rows of all {s.H} heads against "
                      f"the full M={s.M} cache (same inputs and mask rows); value = that sample's "
                      f"counted FLOPs / oracle wall time"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c4")
    ap.add_argument("--mask", choices=("stored", "implicit"), default="stored")
    ap.add_argument("--saved", action="store_true", help="time the saved-statistics entry")
    ap.add_argument("--cpu-rows", type=int, default=768, help="query rows in the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after timing, run plain device copies of this size (counter scaling)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this implementation runs on one GPU; multi-GPU runs are not supported "
              f"(got --gpus {args.gpus}, WORLD_SIZE {world})", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import fa_inputs
    import flash_attention_backward_amd as fab

    log(f"generating {args.workload} inputs")
    p = fa_inputs.make(args.workload)
    if args.mask == "implicit":
        p = fa_inputs.implicit_causal(p)
    flops = fa_inputs.flop_count(p)
    log(f"{describe_workload(p)}; visible pairs {flops['visible']:,}; {flops['full'] / 1e12:.3f} TFLOP")
    dev = torch.device("cuda:0")
    dp = fab.DeviceProblem(p, dev, poison=False)
    stream = torch.cuda.current_stream(dev)
    F = fab.fa_back
    pf = dict(PHASE_FLOPS_PER_PAIR_PER_D)
    stored_ds = bool(dp.layout.plan_flags & F.FLAG_DS_STORE)
    if stored_ds:
        pf["walk2"] = DQ_STORED_FLOPS_PER_PAIR_PER_D
    plan = [n for n, b in (("walk1_keys", F.FLAG_WALK1_KEYS), ("walk1_rows", F.FLAG_WALK1_ROWS),
                            ("kv_image", F.FLAG_KV_IMAGE), ("kv_inline", F.FLAG_KV_INLINE),
                            ("ds_store", F.FLAG_DS_STORE), ("ds_recompute", F.FLAG_DS_RECOMPUTE))
            if dp.layout.plan_flags & b]
    if args.saved:
        # the LSE of the full operator on the same inputs, and a synthetic O
        dp.run()
        torch.cuda.synchronize()
        lse_t = torch.from_numpy(np.ascontiguousarray(dp.outputs()["lse"], dtype=np.float32)).to(dev)
        gen = torch.Generator(device="cpu").manual_seed(p.seed + 1)
        o_t = torch.randn((p.H, p.N, p.Dv), generator=gen, dtype=torch.float32).to(dev)
        run = lambda: dp.run_saved(lse_t, o_t, stream)
        run_timed = lambda: dp.run_saved(lse_t, o_t, stream, timed=True)
        flops["full"] = 2 * flops["visible"] * (3 * p.D + 4 * p.Dv)
    else:
        run = dp.run
        run_timed = lambda: dp.run_timed(stream)
    log(f"warmup x{args.warmup}")
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    log(f"timing x{args.steps}")
    phases = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        phases.append(run_timed())
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    mean_phase = {n: statistics.fmean(ph[k] for ph in phases) for k, n in enumerate(fab.fa_back.PHASES)}
    # per-call device time: the sum of the call's phase intervals (HIP events on the stream)
    per_call = sorted(sum(ph) for ph in phases)
    call_stats = {"median": round(statistics.median(per_call), 4), "min": round(per_call[0], 4),
                  "p90": round(per_call[min(len(per_call) - 1, int(0.9 * len(per_call)))], 4),
                  "source": "HIP events on the launch stream, per call"}
    log("phase ms: " + " ".join(f"{k}={v:.3f}" for k, v in mean_phase.items()))

    dom = max(pf, key=lambda n: mean_phase[n])
    prefixes = tuple(k.replace("D", str(p.D), 1) for k in KERNEL_PREFIXES[dom])
    nbytes = fa_inputs.min_bytes(p)
    intensity = flops["full"] / nbytes["total"]
    kname, traffic = (measured_traffic(prefixes, args.workload) if args.mask == "stored" and not args.saved
                      else (None, None))
    if kname is None:
        kname = " | ".join(prefixes)   # the phase's kernel, as far as the record can tell
    if intensity >= PEAK_MFMA_F16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        dom_flops = pf[dom] * p.D * flops["visible"]
        achieved = dom_flops / (mean_phase[dom] * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_MFMA_F16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / PEAK_MFMA_F16_TFLOPS, 4), "traffic": traffic,
                    "kernel": kname, "phase": dom,
                    "flops_per_launch": dom_flops, "avg_launch_ms": round(mean_phase[dom], 4)}
    else:
        dom_bytes = phase_bytes(p, dom)
        achieved = dom_bytes / (mean_phase[dom] * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                    "kernel": kname, "phase": dom,
                    "bytes_per_launch": dom_bytes, "avg_launch_ms": round(mean_phase[dom], 4),
                    "call": {"min_bytes": nbytes["total"],
                             "gbs": round(nbytes["total"] / (statistics.median(per_call) * 1e-3) / 1e9, 1)}}
    if roofline["bound"] == "hbm":
        # the nominal 8 TB/s stays the peak; a plain device copy (read + write) measured in the
        # same process shows what streaming traffic reaches on this chip
        copy = copy_rate_gbs()
        roofline["copy_reference"] = {"gbs": round(copy, 1), "frac_of_copy": round(achieved / copy, 4),
                                      "what": "plain 1 GiB device copy, read + write bytes / time"}
    value = flops["full"] / (ms * 1e-3) / 1e12
    executed = sum(pf[k] for k in pf if not (args.saved and k == "walk1")) * p.D * flops["visible"]
    rec = {
        "metric": (METRIC if args.workload == "c4" and args.mask == "stored" and not args.saved
                   else f"attn-backward TFLOP/s + ms/call, {args.workload} mask {args.mask}"
                        + (" saved LSE/O" if args.saved else "")),
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "ms_per_call": call_stats,
        "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": describe_workload(p), "N": p.N, "M": p.M, "H": p.H, "Hkv": p.Hkv,
                   "D": p.D, "Dv": p.Dv, "q_type": p.q_type, "k_type": p.k_type, "v_type": p.v_type,
                   "mask": p.mask_type, "seed": p.seed},
        "flops": {"count": ("2*V*(3D+4Dv)" if args.saved else "2*V*(5D+4Dv)") +
                           ", V = visible (row, key, head) triples",
                  "visible": flops["visible"], "full": flops["full"], "five_gemm": flops["five"],
                  "tflops_five_gemm": round(flops["five"] / (ms * 1e-3) / 1e12, 3),
                  "executed": executed, "tflops_executed": round(executed / (ms * 1e-3) / 1e12, 3),
                  "executed_note": "matrix flops this plan runs (walk 1 skipped by the saved entry; "
                                   "dQ from stored dS runs 2*D*V instead of walk 2's 6*D*V)"},
        "plan": plan,
        "phase_ms": {k: round(v, 4) for k, v in mean_phase.items()},
        "roofline": roofline,
    }
    dp.close()
    del dp
    torch.cuda.empty_cache()
    if args.copy_calibration > 0:
        copy_calibration(args.copy_calibration)
    if not args.no_cpu_baseline and args.mask == "stored" and not args.saved:
        rec["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_rows)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
