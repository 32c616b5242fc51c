"""Throughput of the exact attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3]

A step is one fa_fwd launch over the whole workload (every step of the
method runs inside that one kernel).  Inputs are generated once, copied to
HBM, and stay resident; the timed region holds exactly K launches bracketed
by device synchronisation, timed both by the host clock and by HIP events
recorded on the stream the kernel is launched on.  Prints one JSON line.

Default workload: B=2, H=32, N_q=N_kv=8192, d=128, bf16, non-causal.
FLOPs per step = 4*B*Hq*N_q*N_kv*d, halved for causal.

The CPU baseline times the fp64 oracle on the host cores on a bounded
sample (whole heads of the same workload, about 10 s of CPU work) and scales
its rate to the same FLOP count; the heads it computed are then compared with
the GPU's output of the timed launches (``parity_sample``).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_FP8_TFLOPS = 5033.2    # 256 CU x 2.4 GHz x 8192 dense fp8 FLOP/clk/CU
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
METRIC = "attn fwd TFLOP/s and % of MI355X bf16 MFMA peak (N=8k/32k, d=128)"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # about 50 ms of untimed launches of the default workload: from an idle GPU the first
    # 20 or so launches run ~1% slower while the clock settles
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", type=int, default=3,
                    help="named workload index (1-7; 7 is the E4M3 variant of 3)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="approximate CPU time budget of the oracle baseline (0 disables)")
    ap.add_argument("--path", choices=["auto", "fwd", "splitkv"], default="auto",
                    help="entry point to time: fa_fwd_stream, or fa_fwd_splitkv (auto: split-KV "
                         "for the decoding workload 6, fa_fwd otherwise)")
    ap.add_argument("--backward", action="store_true",
                    help="time fa_bwd (gradients of the workload's forward) instead of the forward")
    ap.add_argument("--splits", type=int, default=0,
                    help="split count for the split-KV path (0: fa_splitkv_default_splits)")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the context measurements (library GEMM and zero-input run)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="instead of attention, run 3 plain device-to-device copies of this "
                         "many MiB (calibrates the HBM byte counters of a profiler)")
    return ap.parse_args()


def copy_calibration(mib: int):
    import torch
    n = mib * (1 << 20)
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}), flush=True)


def measured_traffic(workload_name: str):
    """HBM bytes per launch recorded under profiles/ for this workload, or None.

    The profile summary stores the FETCH_SIZE + WRITE_SIZE bytes (scaled by a
    plain-copy calibration) together with the sha256 of the kernel sources it
    was taken with (kernel_source_sha); a changed kernel makes the figure
    stale, so it is dropped.
    """
    path = os.path.join(ROOT, "profiles", f"attn_fwd_{workload_name}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.startswith("traffic_"):
            key, val = line.split(":", 1)
            fields[key.strip()] = val.strip()
    if "traffic_bytes_per_launch" not in fields:
        return None
    if fields.get("traffic_kernel_source_sha256") != kernel_source_sha():
        return None
    return float(fields["traffic_bytes_per_launch"])


def kernel_source_sha() -> str:
    """sha256 over the kernel sources: fa_fwd.hip and the generators of its 64-row bodies."""
    import hashlib
    h = hashlib.sha256()
    for name in ("fa_fwd.hip", "gen_fwd_w64.py", "gen_fwd_w64_fp8.py"):
        with open(os.path.join(ROOT, "exact_io_aware_37_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def power_context(fa, w, qd, kd, vd, o, lse, scale, stream, dcode, fp8_descales=None):
    """Context for the roofline fraction, measured on the same GPU in the same process.

    MI355X lowers its clock under sustained dense MFMA load on random operands, so the
    published peak is not reachable with such data.  Two reference points show by how
    much: a library bf16 GEMM (torch.mm, 8192^3, the same N(0,1) values as the workload)
    and the attention kernel itself on all-zero inputs (same instructions, little
    switching activity), each next to its own zero/random counterpart.
    """
    import torch

    def timed(fn, n):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    g = torch.Generator(device="cpu").manual_seed(7)
    a = torch.randn(8192, 8192, generator=g).to(device=qd.device, dtype=torch.bfloat16)
    b = torch.randn(8192, 8192, generator=g).to(device=qd.device, dtype=torch.bfloat16)
    c = torch.empty_like(a)
    gemm_flops = 2.0 * 8192 ** 3
    with torch.cuda.stream(stream):
        ms_rand = timed(lambda: torch.mm(a, b, out=c), 40)
        a.zero_()
        b.zero_()
        ms_zero = timed(lambda: torch.mm(a, b, out=c), 40)
    del a, b, c
    zdt = torch.uint8 if fp8_descales is not None else qd.dtype   # E4M3 code 0 is +0.0
    zq, zk, zv = (torch.zeros(x.shape, dtype=zdt, device=x.device) for x in (qd, kd, vd))
    o, lse = torch.empty_like(o), torch.empty_like(lse)   # keep the benchmarked outputs intact

    def attn_zero():
        if fp8_descales is not None:
            st = fa.fa_fwd_fp8(zq, zk, zv, o, lse, w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, scale,
                               w.causal, *fp8_descales, stream)
        else:
            st = fa.fa_fwd_stream(zq, zk, zv, o, lse, w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, scale,
                                  w.causal, dcode, stream)
        if st != 0:
            raise RuntimeError(fa.fa_status_string(st))
    ms_attn_zero = timed(attn_zero, 20)
    return {
        "library_gemm_bf16_8192_random_tflops": round(gemm_flops / ms_rand / 1e9, 1),
        "library_gemm_bf16_8192_zero_tflops": round(gemm_flops / ms_zero / 1e9, 1),
        "this_kernel_zero_inputs_tflops": round(w.flops() / ms_attn_zero / 1e9, 1),
        "note": "same GPU, same process; random operands draw more power and lower the clock",
    }


def cpu_baseline(w, q, k, v, budget_s, hbm_bound=False, fp8_descales=None, o_gpu=None,
                 lse_gpu=None, scale=None):
    """Time the oracle on whole (b, h) heads until ~budget_s of wall time.

    The rate is in the benchmark's unit: FLOPs of the heads done (TFLOP/s), or
    for the HBM-bound decoding workload their share of the compulsory bytes
    (GB/s).  For an E4M3 workload the oracle is the exact attention of the
    dequantised codes.

    Outside the timed calls, the heads the oracle computed are compared with
    the GPU's output of the benchmarked launches (o_gpu, lse_gpu): max-abs
    errors, and for E4M3 the worst ratio to the oracle's tolerance model."""
    import numpy as np
    import workloads
    from oracle import attention_fp64, attention_fp8_fp64, dequantize_e4m3, fp8_tolerances
    from oracle.attention_ref import _default_threads
    cores = _default_threads()
    heads = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    rng = np.random.default_rng(0)
    order = rng.permutation(len(heads))
    g = w.Hq // w.Hkv
    done, t_total, flops = 0, 0.0, 0.0
    per_head = (w.io_bytes() if hbm_bound else w.flops()) / (w.B * w.Hq)
    o_cpu = None if o_gpu is None else o_gpu.cpu()
    l_cpu = None if lse_gpu is None else lse_gpu.cpu()
    err_o, err_l, worst = 0.0, 0.0, 0.0
    for i in order:
        b, h = heads[i]
        sl = (slice(b, b + 1), slice(h, h + 1))
        skv = (slice(b, b + 1), slice(h // g, h // g + 1))
        if fp8_descales is not None:
            qh, kh, vh = (workloads.codes_of(x[s_]) for x, s_ in ((q, sl), (k, skv), (v, skv)))
            t0 = time.perf_counter()
            ro, rl = attention_fp8_fp64(qh, kh, vh, *fp8_descales, w.scale, w.causal)
        else:
            qh, kh, vh = (workloads.to_f64(x[s_]) for x, s_ in ((q, sl), (k, skv), (v, skv)))
            t0 = time.perf_counter()
            ro, rl = attention_fp64(qh, kh, vh, w.scale, w.causal)
        t_total += time.perf_counter() - t0
        flops += per_head
        done += 1
        if o_cpu is not None:
            eo = np.abs(workloads.to_f64(o_cpu[sl]) - ro)
            el = np.abs(l_cpu[sl].double().numpy() - rl)
            err_o, err_l = max(err_o, float(eo.max())), max(err_l, float(el.max()))
            if fp8_descales is not None:
                # the tolerance model on the 16 rows with the largest errors of this head
                pick = np.argsort(-eo.max(axis=(0, 1, 3)))[:16]
                deq = [dequantize_e4m3(x, s_) for x, s_ in zip((qh, kh, vh), fp8_descales)]
                to, tl = fp8_tolerances(*deq, w.scale, w.causal, rows=pick)
                worst = max(worst, float(np.max(eo[:, :, pick] / to)),
                            float(np.max(el[:, :, pick] / tl)))
        if t_total >= budget_s:
            break
    scale_, unit = (1e9, "GB/s") if hbm_bound else (1e12, "TFLOP/s")
    parity = None
    if o_cpu is not None:
        parity = {"heads_checked": done, "rows_per_head": w.Nq, "max_abs_err_O": err_o,
                  "max_abs_err_lse": err_l}
        if fp8_descales is not None:
            parity["worst_err_over_tolerance"] = worst
            parity["tolerance_rows"] = "the 16 rows of largest error per head"
    return {"value": flops / t_total / scale_, "unit": unit, "cores": cores,
            "kind": "oracle",
            "sample": f"{done} of {len(heads)} (b,h) heads of the same workload, all "
                      f"{w.Nq} rows each, fp64 numpy, {t_total:.2f} s",
            "seconds": t_total, "parity": parity}


def main():
    args = parse()
    if args.copy_mib > 0:
        copy_calibration(args.copy_mib)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has "
              "no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import exact_io_aware_37_amd as fa
    import workloads

    w = workloads.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    fp8 = w.dtype == "e4m3"
    descales = None
    if fp8:
        (q, k, v), descales, scale = workloads.workload_inputs_fp8(w)
    else:
        q, k, v, scale = workloads.workload_inputs(w)
    paged = None
    if w.block_size > 0:
        # the same keys, held in a paged cache (block tables in device memory)
        kc, vc, tab, sl = workloads.paginate(k, v, [w.Nkv] * w.B, w.block_size, seed=w.seed)
        paged = tuple(x.to(dev) for x in (kc, vc, tab, sl))
        del kc, vc
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    o = torch.empty(qd.shape, dtype=torch.bfloat16 if fp8 else qd.dtype, device=dev)
    lse = torch.empty(qd.shape[:3], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    dcode = None if fp8 else fa.dtype_code(qd.dtype)
    fa.load_library()

    path = args.path if args.path != "auto" else ("splitkv" if w.index == 6 else "fwd")
    if args.backward:
        path = "bwd"
    if paged is not None:
        if path not in ("fwd", "paged"):
            print("the paged workload has the paged split-KV entry point only", file=sys.stderr)
            sys.exit(2)
        path = "paged"
        del kd, vd
    if fp8:
        if path != "fwd":
            print("the E4M3 workload has a forward entry point only", file=sys.stderr)
            sys.exit(2)
        path = "fp8"
    splits = None
    if path == "paged":
        kcd, vcd, tbd, sld = paged
        nb, bs = kcd.shape[0], kcd.shape[1]
        mbps = tbd.shape[1]
        splits = args.splits or fa.fa_splitkv_default_splits(w.B, w.Hq, w.Hkv, w.Nq, mbps * bs, w.D,
                                                              dcode)
        ws_bytes = fa.fa_splitkv_workspace_bytes(w.B, w.Hq, w.Nq, w.D, splits)
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

        def step():
            st = fa.fa_fwd_paged(qd, kcd, vcd, tbd, sld, o, lse, w.B, w.Hq, w.Hkv, w.Nq, w.D, nb, bs,
                                 mbps, scale, w.causal, dcode, splits, workspace, ws_bytes, stream)
            if st != 0:
                raise RuntimeError(fa.fa_status_string(st))
    elif path == "splitkv":
        splits = args.splits or fa.fa_splitkv_default_splits(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D,
                                                              dcode)
        ws_bytes = fa.fa_splitkv_workspace_bytes(w.B, w.Hq, w.Nq, w.D, splits)
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

        def step():
            st = fa.fa_fwd_splitkv(qd, kd, vd, o, lse, w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, scale,
                                   w.causal, dcode, splits, workspace, ws_bytes, stream)
            if st != 0:
                raise RuntimeError(fa.fa_status_string(st))
    elif path == "bwd":
        # The forward's outputs and a seeded dO are inputs of every timed step.
        st = fa.fa_fwd_stream(qd, kd, vd, o, lse, w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, scale,
                              w.causal, dcode, stream)
        if st != 0:
            raise RuntimeError(fa.fa_status_string(st))
        dod = workloads.make_inputs(w.B, w.Hq, w.Hq, w.Nq, 1, w.D, w.dtype, w.seed + 100)[0].to(dev)
        dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
        ws_bytes = fa.fa_bwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D)
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

        def step():
            st = fa.fa_bwd(qd, kd, vd, o, lse, dod, dq, dk, dv, w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D,
                           scale, w.causal, dcode, workspace, ws_bytes, stream)
            if st != 0:
                raise RuntimeError(fa.fa_status_string(st))
    elif path == "fp8":
        def step():
            st = fa.fa_fwd_fp8(qd, kd, vd, o, lse, w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, scale,
                               w.causal, *descales, stream)
            if st != 0:
                raise RuntimeError(fa.fa_status_string(st))
    else:
        def step():
            st = fa.fa_fwd_stream(qd, kd, vd, o, lse, w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, scale,
                                  w.causal, dcode, stream)
            if st != 0:
                raise RuntimeError(fa.fa_status_string(st))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # One event before every launch and one after the last: the launches stay
    # back to back, and each launch's duration is the gap between its events.
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i].record(stream)
        step()
    evs[-1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_launch = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    kernel_ms = evs[0].elapsed_time(evs[-1]) / args.steps
    median_ms = per_launch[len(per_launch) // 2]
    wall_ms = wall * 1e3 / args.steps

    # Backward: the algorithmic count is 2.5x the forward's (dV, dP, dQ, dK and
    # the recomputed S: 10*N_q*N_kv*d per head, against 4 for the forward).
    flops = w.flops() * (2.5 if path == "bwd" else 1.0)
    hbm_bound = path in ("splitkv", "paged")
    if hbm_bound:
        # Decoding reads the whole K/V cache for one query row per head: HBM-bound.
        work, unit, peak, bound = w.io_bytes() / 1e9, "GB/s", PEAK_HBM_GBS, "hbm"
        metric = "decode attention HBM GB/s (split-KV, compulsory bytes)"
        if path == "paged":
            metric = "decode attention HBM GB/s (split-KV over a paged cache, compulsory bytes)"
    else:
        work, unit, bound = flops / 1e12, "TFLOP/s", "mfma"
        peak = {"f32": PEAK_F32_TFLOPS, "e4m3": PEAK_FP8_TFLOPS}.get(w.dtype, PEAK_BF16_TFLOPS)
        metric = METRIC
        if path == "bwd":
            metric = "attn backward TFLOP/s (2.5x forward FLOPs) and % of MI355X bf16 MFMA peak"
        elif path == "fp8":
            metric = "attn fwd TFLOP/s with E4M3 inputs and % of MI355X fp8 MFMA peak (N=8k, d=128)"
    value = work / (wall_ms * 1e-3)
    achieved = work / (kernel_ms * 1e-3)
    print(f"[bench] {w.name} ({path}): kernel {kernel_ms:.4f} ms/step (events), wall "
          f"{wall_ms:.4f} ms/step -> {achieved:.1f} {unit} = {100 * achieved / peak:.1f}% of "
          f"{peak} peak", file=sys.stderr, flush=True)

    context = None
    if not args.no_context and w.dtype != "f32" and not hbm_bound and path in ("fwd", "fp8"):
        context = power_context(fa, w, qd, kd, vd, o, lse, scale, stream, dcode, descales)

    cpu = None
    if args.cpu_seconds > 0 and path != "bwd":
        cpu = cpu_baseline(w, q, k, v, args.cpu_seconds, hbm_bound, descales, o, lse, scale)

    if path == "bwd":
        launch = {"entry": "fa_bwd", "note": "three launches per step: row pass, dK/dV, dQ",
                  "keys_per_block_dkdv": 256, "rows_per_block_dq": 256}
    elif path == "paged":
        launch = {"entry": "fa_fwd_paged", "num_splits": splits, "block_size": w.block_size,
                  "keys_per_tile": 32, "rows_per_wave": 32, "waves_per_block": 8,
                  "note": "two launches per step: chunk kernel over the block tables, then combine"}
    elif path == "splitkv":
        launch = {"entry": "fa_fwd_splitkv", "num_splits": splits, "keys_per_tile": 32,
                  "rows_per_wave": 32, "waves_per_block": 8,
                  "note": "two launches per step: chunk kernel, then combine"}
    elif path == "fp8":
        # d = 128: the 64-row E4M3 body, 4 waves of 64 rows; d = 64: 8 waves of 32 rows
        launch = {"entry": "fa_fwd_fp8", "rows_per_block": 256, "keys_per_tile": 64,
                  "threads_per_block": 256 if w.D == 128 else 512,
                  "lds_bytes": 65536 if w.D == 128 else 131072 * w.D // 128,
                  "blocks": w.B * w.Hq * ((w.Nq + 255) // 256),
                  "descales": list(descales)}
    else:
        launch = fa.fa_launch_info(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, w.causal, dcode)[1]
    line = {
        "metric": metric,
        "value": round(value, 3),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N_q": w.Nq,
                   "N_kv": w.Nkv, "d": w.D, "causal": w.causal, "seed": w.seed,
                   "flops_per_step": flops, "launch": launch},
        "pct_of_peak": round(100 * value / peak, 2),
        "roofline": {"bound": bound, "achieved": round(achieved, 3), "peak": peak,
                     "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": measured_traffic(w.name), "kernel_ms": round(kernel_ms, 5),
                     "kernel_ms_median": round(median_ms, 5),
                     "kernel_ms_min": round(per_launch[0], 5)},
        "context": context,
        "cpu_baseline": None if cpu is None else {k_: cpu[k_] for k_ in
                                                  ("value", "unit", "cores", "kind", "sample")},
        "parity_sample": None if cpu is None else cpu["parity"],
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
