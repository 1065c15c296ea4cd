#!/usr/bin/env python3
"""LiteLA forward benchmark on one MI355X.

One step = one full forward of the Sana-1600M 4096px self-attention shape
(B=1, N=16384 tokens, H=70 heads, D=32, bf16 q/k/v, fp32 out as the reference
returns it, eps=1e-15): one sana_linattn_fwd call, which enqueues the state,
merge and apply kernels on torch's current stream.  Inputs are
seeded synthetic tensors (workloads.py), resident in HBM before timing starts;
three input/output sets rotate so the 367 MB per step streams from HBM rather
than from the 256 MB Infinity Cache.

Prints ONE JSON line on stdout (everything else goes to stderr):
  value        algorithmic GB/s = (read q, k, v + write out) bytes / time per step
  roofline     the dominant kernel's algorithmic bytes per launch / its average
               duration (HIP events on the launch stream), against 8 TB/s
  cpu_baseline the fp64 oracle on the host cores, same workload, GB/s
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LiteLA fwd GB/s & tokens*heads/s at N=16384,H=70,D=32; % of HBM peak"
HBM_PEAK_GBPS = 8000.0
# the forward kernels and the headers they include
KERNEL_SRC = [os.path.join(ROOT, "diffusion_transformer_relu_amd", "csrc", f)
              for f in ("linattn_kernels.hip", "linattn_device.h", "linattn_internal.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SRC:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str, out_dtype: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none for this kernel or the kernel source has changed
    since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    ent = data.get(f"{kernel}|{workload}|{out_dtype}")
    if not ent or ent.get("kernel_src_sha") != kernel_source_sha():
        return None
    return ent.get("bytes_per_launch")


def summarize_traffic(fetch_csv: str, write_csv: str, out_dtype: str = "f32") -> int:
    """Per-dispatch HBM bytes of the forward's kernels from two rocprofv3 --pmc
    runs of this script (`--no-extras --calibration-copy --cpu-seconds 0`).
    Each counter is scaled by what it reads for the device-to-device copy of
    known size in the same run (the copy's FETCH and WRITE should each equal its
    size)."""
    import csv
    import statistics

    import workloads
    w = workloads.HEADLINE
    out_bytes = 4 if out_dtype == "f32" else 2
    copy_bytes = w.algorithmic_bytes(out_bytes) // 2     # bytes read (and written) by the copy

    def per_kernel(path, counter):
        vals = {}
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                vals.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]) * 1024.0)
        return vals

    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")

    def calib(vals):
        # the calibration copy is the largest copy of the run (input clones are
        # smaller); the counters may see only part of the chip's traffic, which
        # is exactly what the scale corrects
        copies = [x for name, xs in vals.items() if "copyBuffer" in name for x in xs]
        if not copies:
            raise SystemExit("no calibration copy dispatch found in the counter file")
        top = max(copies)
        return copy_bytes / statistics.median([x for x in copies if x >= 0.95 * top])

    sf, sw = calib(fetch), calib(write)
    # bf16 inputs, head dim 32: the state kernel's template arguments are
    # F16 = false and the head dim; the apply kernel's the input and output
    # element types and the head dim
    apply_tag = "k_apply_mfma<unsigned short, " + ("float" if out_dtype == "f32" else "unsigned short") + ", 32>"
    kernels = {"k_state_partial_mfma": lambda n: "k_state_partial_mfma<false, 32>" in n,
               "k_merge": lambda n: "k_merge" in n,
               "k_apply_mfma": lambda n: apply_tag in n}
    algo = {"k_state_partial_mfma": w.token_heads * w.D * 4,
            "k_merge": None,
            "k_apply_mfma": w.token_heads * w.D * (2 + out_bytes)}
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        data = {}
    sha = kernel_source_sha()
    lines = [f"calibration: copy of {copy_bytes} B per direction; FETCH scale {sf:.4f}, WRITE scale {sw:.4f}"]
    for kname, match in kernels.items():
        fv = [x for n, xs in fetch.items() if match(n) for x in xs]
        wv = [x for n, xs in write.items() if match(n) for x in xs]
        if not fv or not wv:
            continue
        fb, wb = statistics.median(fv) * sf, statistics.median(wv) * sw
        ent = {"fetch_bytes": round(fb), "write_bytes": round(wb), "bytes_per_launch": round(fb + wb),
               "dispatches": [len(fv), len(wv)], "scale_fetch": round(sf, 5), "scale_write": round(sw, 5),
               "algorithmic_bytes": algo[kname], "kernel_src_sha": sha}
        data[f"{kname}|{w.name}|{out_dtype}"] = ent
        ratio = f"{(fb + wb) / algo[kname]:.3f} x algorithmic" if algo[kname] else "(workspace only)"
        lines.append(f"{kname:22s} fetch {fb / 1e6:9.3f} MB  write {wb / 1e6:9.3f} MB  {ratio}")
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    print("\n".join(lines))
    return 0


def short_kernel_name(name: str) -> str:
    """'void ns::(anonymous namespace)::k<a, b>(args)' -> 'k<a, b>'."""
    head = name.split("(unsigned", 1)[0].split("(float", 1)[0]
    head = head.replace("(anonymous namespace)::", "").replace("void ", "")
    return head.split("::")[-1] if "<" not in head else head[head.rfind("::", 0, head.find("<")) + 2:]


def summarize_trace(stats_csv: str) -> int:
    """Markdown table of a rocprofv3 --kernel-trace --stats run_kernel_stats.csv;
    with the run_kernel_trace.csv beside it, also each kernel's longest run of
    back-to-back launches (the per-kernel loop this script times with HIP
    events) and the whole forwards (state, merge, apply in sequence)."""
    import csv
    import statistics
    rows = list(csv.DictReader(open(stats_csv)))
    print("| kernel | calls | avg µs | min µs | max µs | share % |")
    print("|---|---|---|---|---|---|")
    for r in rows:
        print(f"| `{short_kernel_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
              f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |")
    trace_csv = os.path.join(os.path.dirname(stats_csv), os.path.basename(stats_csv).replace("kernel_stats",
                                                                                             "kernel_trace"))
    if not os.path.exists(trace_csv):
        return 0
    ev = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), short_kernel_name(r["Kernel_Name"]))
                for r in csv.DictReader(open(trace_csv)))
    runs = {}
    i = 0
    while i < len(ev):
        j = i
        while j + 1 < len(ev) and ev[j + 1][2] == ev[i][2]:
            j += 1
        if j - i + 1 > len(runs.get(ev[i][2], [])):
            runs[ev[i][2]] = [(e - s) / 1e3 for s, e, _ in ev[i:j + 1]]
        i = j + 1
    print()
    print("Longest run of back-to-back launches of each kernel:")
    print()
    print("| kernel | launches | mean µs | median µs |")
    print("|---|---|---|---|")
    for name, d in sorted(runs.items(), key=lambda kv: -len(kv[1])):
        if len(d) >= 10:
            print(f"| `{name}` | {len(d)} | {statistics.mean(d):.2f} | {statistics.median(d):.2f} |")
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--out-dtype", choices=("f32", "bf16"), default="f32")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall time budget of the oracle CPU baseline (0 skips it)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the other-out-dtype, block-causal, fp16-input, backward and JVP timings")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="with --no-extras, still run the device-to-device copy (counter calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU run: turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, "
                         "WRITE_SIZE) of a profiled bench run into profiles/traffic.json")
    ap.add_argument("--trace-from", metavar="STATS_CSV",
                    help="no GPU run: print a rocprofv3 --kernel-trace --stats run_kernel_stats.csv as a "
                         "markdown table")
    args = ap.parse_args()
    if args.trace_from:
        return summarize_trace(args.trace_from)
    if args.traffic_from:
        return summarize_traffic(*args.traffic_from, out_dtype=args.out_dtype)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: LiteLA is independent per (batch, head), and this "
              f"build has no multi-GPU path (asked for --gpus {args.gpus}, WORLD_SIZE {world}).",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import diffusion_transformer_relu_amd as sana
    import workloads

    w = workloads.HEADLINE
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    out_t = torch.float32 if args.out_dtype == "f32" else torch.bfloat16
    out_bytes = 4 if args.out_dtype == "f32" else 2
    B, N, H, D = w.B, w.N, w.H, w.D

    log(f"bench: generating {w.name}")
    q_np, k_np, v_np = workloads.make_inputs(w)

    def up(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    NSETS = 3
    base = [up(q_np), up(k_np), up(v_np)]
    sets = [base] + [[t.clone() for t in base] for _ in range(NSETS - 1)]
    outs = [torch.empty((B, N, H, D), dtype=out_t, device=dev) for _ in range(NSETS)]
    ws = torch.empty(sana.sana_linattn_workspace_bytes(B, H, N, D, 0), dtype=torch.uint8, device=dev)
    plan = sana.sana_linattn_plan_info(sana.SANA_DT_BF16, B, H, N, D, 0)
    stream = torch.cuda.current_stream()
    stages = (sana.SANA_STAGE_STATE, sana.SANA_STAGE_MERGE, sana.SANA_STAGE_APPLY)

    def step(i):
        q, k, v = sets[i % NSETS]
        sana.sana_linattn_fwd(q, k, v, outs[i % NSETS], ws, eps=w.eps, stream=stream)

    def stage_loop(st, n):
        for i in range(n):
            q, k, v = sets[i % NSETS]
            sana.sana_linattn_fwd_stages(q, k, v, outs[i % NSETS], ws, st, eps=w.eps, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: K whole forwards, one C-ABI call each.
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    # Per-kernel durations: each kernel launched K times back to back on the
    # launch stream (state, then merge, then apply, so each reads what the one
    # before left in the workspace), bracketed by two HIP events.
    per_kernel_ms = {}
    for name, st in zip(("state", "merge", "apply"), stages):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        stage_loop(st, args.steps)
        e1.record(stream)
        torch.cuda.synchronize()
        per_kernel_ms[name] = e0.elapsed_time(e1) / args.steps
    # the timed forwards' output is recomputed once, for the parity check below
    step(args.steps - 1)
    torch.cuda.synchronize()

    alg_bytes = w.algorithmic_bytes(out_bytes)
    gbps = alg_bytes / (ms_per_step * 1e-3) / 1e9
    th_per_s = w.token_heads / (ms_per_step * 1e-3)

    # Dominant kernel and its algorithmic bytes per launch.
    kernel_bytes = {
        "state": w.token_heads * D * 2 * 2,            # read k and v (bf16)
        "apply": w.token_heads * D * (2 + out_bytes),  # read q, write out
    }
    kernel_names = {"state": "k_state_partial_mfma", "apply": "k_apply_mfma"}
    dom = max(kernel_bytes, key=lambda n: per_kernel_ms[n])
    achieved = kernel_bytes[dom] / (per_kernel_ms[dom] * 1e-3) / 1e9
    traffic = measured_traffic(kernel_names[dom], w.name, args.out_dtype)

    # Parity of what was timed, against the oracle (also the first CPU-baseline run).
    import oracle
    torch.cuda.synchronize()
    got = outs[(args.steps - 1) % NSETS].float().cpu().double().numpy()
    tc0 = time.perf_counter()
    want = oracle.linattn_fwd(q_np, k_np, v_np, eps=w.eps)
    oracle_s = [time.perf_counter() - tc0]
    ref = want if out_t == torch.float32 else torch.from_numpy(want).float().to(torch.bfloat16).double().numpy()
    rel_l2 = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    max_abs = float(np.max(np.abs(got - ref)))
    vmax = float(np.max(np.abs((v_np.astype(np.uint32) << np.uint32(16)).view(np.float32))))
    parity_ok = rel_l2 <= 1e-4 and max_abs <= 2e-3 * vmax
    log(f"bench: parity rel_l2={rel_l2:.3e} max_abs={max_abs:.3e} ok={parity_ok}")

    cpu = None
    if args.cpu_seconds > 0:
        while sum(oracle_s) < args.cpu_seconds and len(oracle_s) < 200:
            tc0 = time.perf_counter()
            oracle.linattn_fwd(q_np, k_np, v_np, eps=w.eps)
            oracle_s.append(time.perf_counter() - tc0)
        cpu = {
            "value": round(alg_bytes * len(oracle_s) / sum(oracle_s) / 1e9, 4),
            "unit": "GB/s",
            "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"the whole {w.name} workload (fp64 C oracle, OpenMP over the {B * H} (b,h) pairs), "
                      f"run {len(oracle_s)} times in {sum(oracle_s):.1f} s; input generation excluded",
        }

    extra = {}

    def timed(fn, n):
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        a = time.perf_counter()
        for i in range(n):
            fn(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - a) * 1e3 / n

    if not args.no_extras or args.calibration_copy:
        # device-to-device copy of the same byte count: a practical HBM ceiling,
        # and the known-size kernel that calibrates the byte counters
        src = torch.empty(alg_bytes // 2, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        ms = timed(lambda i: dst.copy_(src), args.steps)
        extra["device_copy"] = {"bytes_moved": 2 * src.numel(), "ms": round(ms, 5),
                                "GBps": round(2 * src.numel() / ms / 1e6, 1)}
        extra["pct_of_device_copy"] = round(100 * gbps / extra["device_copy"]["GBps"], 2)
        del src, dst

    if not args.no_extras:
        other_t = torch.bfloat16 if out_t == torch.float32 else torch.float32
        other_bytes = 2 if other_t == torch.bfloat16 else 4
        outs2 = [torch.empty((B, N, H, D), dtype=other_t, device=dev) for _ in range(NSETS)]

        def fused2(i):
            q, k, v = sets[i % NSETS]
            sana.sana_linattn_fwd(q, k, v, outs2[i % NSETS], ws, eps=w.eps, stream=stream)
        ms = timed(fused2, args.steps)
        b2 = w.algorithmic_bytes(other_bytes)
        extra[("bf16" if other_t == torch.bfloat16 else "f32") + "_out"] = {
            "ms_per_step": round(ms, 5), "GBps": round(b2 / ms / 1e6, 1),
            "pct_hbm_peak": round(100 * b2 / ms / 1e6 / HBM_PEAK_GBPS, 2)}

        L = workloads.BLOCK_CAUSAL.block_len
        ws_bc = torch.empty(sana.sana_linattn_workspace_bytes(B, H, N, D, L), dtype=torch.uint8, device=dev)

        def bc(i):
            q, k, v = sets[i % NSETS]
            sana.sana_linattn_blockcausal_fwd(q, k, v, outs[i % NSETS], ws_bc, L, eps=w.eps, stream=stream)
        ms = timed(bc, args.steps)
        extra["blockcausal_16x1024_" + args.out_dtype + "out"] = {
            "ms_per_step": round(ms, 5), "GBps": round(alg_bytes / ms / 1e6, 1),
            "pct_hbm_peak": round(100 * alg_bytes / ms / 1e6 / HBM_PEAK_GBPS, 2),
            "note": "same-shape buffers as the non-causal run, block_len 1024"}
        del outs2, ws_bc

        # streaming block-causal: the same sequence in 4 calls of 4096 tokens,
        # the state carried between them (block_len 1024)
        C = N // 4
        ws_st = torch.empty(sana.sana_linattn_workspace_bytes(B, H, C, D, L), dtype=torch.uint8, device=dev)
        carried = torch.empty((B, H, D, D + 1), dtype=torch.float32, device=dev)
        chunks = [[[t[:, c * C:(c + 1) * C].contiguous() for t in st] for c in range(4)] for st in sets]
        couts = [torch.empty((B, C, H, D), dtype=out_t, device=dev) for _ in range(4)]

        def stream4(i):
            for c in range(4):
                q, k, v = chunks[i % NSETS][c]
                sana.sana_linattn_blockcausal_stream_fwd(q, k, v, couts[c], ws_st, L,
                                                         state_in=carried if c else None, state_out=carried,
                                                         eps=w.eps, stream=stream)
        ms = timed(stream4, args.steps)
        extra["stream_4x4096_bc1024_" + args.out_dtype + "out"] = {
            "ms_per_step": round(ms, 5), "GBps": round(alg_bytes / ms / 1e6, 1),
            "pct_hbm_peak": round(100 * alg_bytes / ms / 1e6 / HBM_PEAK_GBPS, 2),
            "note": "the headline sequence as 4 chained calls of 4096 tokens with the state carried "
                    "(block_len 1024); ms per whole sequence"}
        del chunks, couts, ws_st, carried

        # q, k, v as strided views of one fused [B, N, 3, H, D] projection output
        fused = [torch.stack(st, dim=2) for st in sets]

        def strided(i):
            f = fused[i % NSETS]
            sana.sana_linattn_fwd_strided(f[:, :, 0], f[:, :, 1], f[:, :, 2], outs[i % NSETS], ws, eps=w.eps,
                                          stream=stream)
        ms = timed(strided, args.steps)
        extra["fused_qkv_strided_" + args.out_dtype + "out"] = {
            "ms_per_step": round(ms, 5), "GBps": round(alg_bytes / ms / 1e6, 1),
            "pct_hbm_peak": round(100 * alg_bytes / ms / 1e6 / HBM_PEAK_GBPS, 2),
            "note": "q, k, v read in place from one [B, N, 3, H, D] buffer (token stride 3 H D)"}
        del fused

        # fp16 inputs (the same values, converted on the device), fp32 out
        sets16 = [[t.to(torch.float16) for t in st] for st in sets]

        def f16(i):
            q, k, v = sets16[i % NSETS]
            sana.sana_linattn_fwd(q, k, v, outs[i % NSETS], ws, eps=w.eps, stream=stream)
        ms = timed(f16, args.steps)
        extra["f16_in_" + args.out_dtype + "out"] = {
            "ms_per_step": round(ms, 5), "GBps": round(alg_bytes / ms / 1e6, 1),
            "pct_hbm_peak": round(100 * alg_bytes / ms / 1e6 / HBM_PEAK_GBPS, 2),
            "note": "the headline inputs converted to fp16 on the device"}
        del sets16

        # fp32 inputs (the same values widened on the device), same out dtype:
        # 12 bytes more per token-head of input
        sets32 = [[t.float() for t in st] for st in sets]

        def f32(i):
            q, k, v = sets32[i % NSETS]
            sana.sana_linattn_fwd(q, k, v, outs[i % NSETS], ws, eps=w.eps, stream=stream)
        ms = timed(f32, args.steps)
        bytes32 = w.token_heads * D * (3 * 4 + out_bytes)
        extra["f32_in_" + args.out_dtype + "out"] = {
            "ms_per_step": round(ms, 5), "GBps": round(bytes32 / ms / 1e6, 1),
            "pct_hbm_peak": round(100 * bytes32 / ms / 1e6 / HBM_PEAK_GBPS, 2),
            "note": "the headline inputs widened to fp32 on the device; algorithmic bytes with 4-byte inputs"}

        # fp32 backward: fp32 q, k, v, dout -> fp32 gradients
        grads32 = [torch.empty((B, N, H, D), dtype=torch.float32, device=dev) for _ in range(3)]
        ws_b32 = torch.empty(sana.sana_linattn_bwd_workspace_bytes(B, H, N, D, 0), dtype=torch.uint8, device=dev)

        def bwd32(i):
            q, k, v = sets32[i % NSETS]
            sana.sana_linattn_bwd(q, k, v, sets32[(i + 1) % NSETS][0], *grads32, ws_b32, eps=w.eps, stream=stream)
        ms = timed(bwd32, args.steps)
        b32 = w.token_heads * D * 4 * 7
        extra["backward_f32"] = {
            "ms_per_step": round(ms, 5), "GBps": round(b32 / ms / 1e6, 1),
            "pct_hbm_peak": round(100 * b32 / ms / 1e6 / HBM_PEAK_GBPS, 2),
            "note": "sana_linattn_bwd, fp32 q/k/v/dout/gradients (the headline inputs widened); "
                    "algorithmic bytes = 7 tensors"}
        del grads32, ws_b32

        # fp32 forward-mode derivative: fp32 q, k, v and tangents -> fp32 out and out_t
        outs_j32 = [torch.empty((B, N, H, D), dtype=torch.float32, device=dev) for _ in range(2)]
        ws_j32 = torch.empty(sana.sana_linattn_jvp_workspace_bytes(B, H, N, D, 0), dtype=torch.uint8, device=dev)

        def jvp32(i):
            q, k, v = sets32[i % NSETS]
            qt, kt, vt = sets32[(i + 1) % NSETS]
            sana.sana_linattn_jvp(q, k, v, qt, kt, vt, *outs_j32, ws_j32, eps=w.eps, stream=stream)
        ms = timed(jvp32, args.steps)
        j32 = w.token_heads * D * 4 * 8
        extra["jvp_f32"] = {
            "ms_per_step": round(ms, 5), "GBps": round(j32 / ms / 1e6, 1),
            "pct_hbm_peak": round(100 * j32 / ms / 1e6 / HBM_PEAK_GBPS, 2),
            "note": "sana_linattn_jvp, fp32 inputs, tangents and outputs (the headline inputs widened); "
                    "algorithmic bytes = 6 inputs + 2 outputs"}
        del sets32, outs_j32, ws_j32

        # other head dims at the same byte count: the headline buffers viewed as
        # 35 heads of 64 and as 140 heads of 16
        for Hx, Dx in ((H // 2, 2 * D), (2 * H, D // 2)):
            wsx = torch.empty(sana.sana_linattn_workspace_bytes(B, Hx, N, Dx, 0), dtype=torch.uint8, device=dev)
            setsx = [[t.view(B, N, Hx, Dx) for t in st] for st in sets]
            outsx = [o.view(B, N, Hx, Dx) for o in outs]

            def hdx(i):
                q, k, v = setsx[i % NSETS]
                sana.sana_linattn_fwd(q, k, v, outsx[i % NSETS], wsx, eps=w.eps, stream=stream)
            ms = timed(hdx, args.steps)
            extra[f"d{Dx}_h{Hx}_" + args.out_dtype + "out"] = {
                "ms_per_step": round(ms, 5), "GBps": round(alg_bytes / ms / 1e6, 1),
                "pct_hbm_peak": round(100 * alg_bytes / ms / 1e6 / HBM_PEAK_GBPS, 2),
                "note": f"head dim {Dx}: the headline buffers viewed as B=1, N=16384, H={Hx}, D={Dx}, bf16 in"}

            # and its backward: bf16 q, k, v, dout (another input set) -> bf16 gradients
            gx = [torch.empty((B, N, Hx, Dx), dtype=torch.bfloat16, device=dev) for _ in range(3)]
            wsb = torch.empty(sana.sana_linattn_bwd_workspace_bytes(B, Hx, N, Dx, 0), dtype=torch.uint8, device=dev)

            def hdx_bwd(i):
                q, k, v = setsx[i % NSETS]
                sana.sana_linattn_bwd(q, k, v, setsx[(i + 1) % NSETS][0], *gx, wsb, eps=w.eps, stream=stream)
            ms = timed(hdx_bwd, args.steps)
            bxb = w.token_heads * D * 2 * 7
            extra[f"backward_d{Dx}_h{Hx}_bf16"] = {
                "ms_per_step": round(ms, 5), "GBps": round(bxb / ms / 1e6, 1),
                "pct_hbm_peak": round(100 * bxb / ms / 1e6 / HBM_PEAK_GBPS, 2),
                "note": f"sana_linattn_bwd at head dim {Dx} (H={Hx}), bf16; algorithmic bytes = 7 tensors"}
            del setsx, outsx, wsx, gx, wsb

        # backward (dq, dk, dv) of the same forward: bf16 q, k, v, dout -> bf16 gradients
        grads = [[torch.empty((B, N, H, D), dtype=torch.bfloat16, device=dev) for _ in range(3)]
                 for _ in range(NSETS)]
        ws_bw = torch.empty(sana.sana_linattn_bwd_workspace_bytes(B, H, N, D, 0), dtype=torch.uint8, device=dev)

        def bwd(i):
            q, k, v = sets[i % NSETS]
            dq, dk, dv = grads[i % NSETS]
            sana.sana_linattn_bwd(q, k, v, sets[(i + 1) % NSETS][0], dq, dk, dv, ws_bw, eps=w.eps, stream=stream)
        ms = timed(bwd, args.steps)
        bw_bytes = w.token_heads * D * 2 * 7    # read q, k, v, dout; write dq, dk, dv (bf16)
        extra["backward_bf16"] = {
            "ms_per_step": round(ms, 5), "GBps": round(bw_bytes / ms / 1e6, 1),
            "pct_hbm_peak": round(100 * bw_bytes / ms / 1e6 / HBM_PEAK_GBPS, 2),
            "note": "sana_linattn_bwd, bf16 q/k/v/dout/gradients; dout is another input set; "
                    "algorithmic bytes = 7 tensors"}
        del grads, ws_bw

        # forward-mode derivative: bf16 q, k, v and tangents -> out and out_t in the bench's out dtype
        tangents = [torch.empty((B, N, H, D), dtype=out_t, device=dev) for _ in range(NSETS)]
        ws_jv = torch.empty(sana.sana_linattn_jvp_workspace_bytes(B, H, N, D, 0), dtype=torch.uint8, device=dev)

        def jvp(i):
            q, k, v = sets[i % NSETS]
            qt, kt, vt = sets[(i + 1) % NSETS]
            sana.sana_linattn_jvp(q, k, v, qt, kt, vt, outs[i % NSETS], tangents[i % NSETS], ws_jv, eps=w.eps,
                                  stream=stream)
        ms = timed(jvp, args.steps)
        jv_bytes = w.token_heads * D * (6 * 2 + 2 * out_bytes)   # read 6 bf16 tensors, write out and out_t
        extra["jvp_bf16_" + args.out_dtype + "out"] = {
            "ms_per_step": round(ms, 5), "GBps": round(jv_bytes / ms / 1e6, 1),
            "pct_hbm_peak": round(100 * jv_bytes / ms / 1e6 / HBM_PEAK_GBPS, 2),
            "note": "sana_linattn_jvp; tangents are another input set; algorithmic bytes = 6 inputs + 2 outputs"}
        del tangents, ws_jv

    line = {
        "metric": METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "N": N, "H": H, "D": D, "in_dtype": "bf16",
                   "out_dtype": args.out_dtype, "accumulate": "f32", "eps": w.eps, "block_len": None,
                   "rotating_sets": NSETS, "plan": plan},
        "tokens_heads_per_s": round(th_per_s, 1),
        "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "per_kernel_ms": {k: round(v, 5) for k, v in per_kernel_ms.items()},
        "roofline": {"bound": "hbm", "kernel": kernel_names[dom], "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "alg_bytes_per_launch": kernel_bytes[dom],
                     "avg_launch_ms": round(per_kernel_ms[dom], 5)},
        "cpu_baseline": cpu,
        "parity": {"rel_l2": rel_l2, "max_abs": max_abs, "max_abs_bar": 2e-3 * vmax, "ok": parity_ok},
        "extra": extra,
    }
    print(json.dumps(line), flush=True)
    return 0 if parity_ok else 1


if __name__ == "__main__":
    sys.exit(main())
