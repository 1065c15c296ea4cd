#!/usr/bin/env python3
"""LiteLA forward benchmark on one MI355X.

One step = one full forward of the Sana-1600M 4096px self-attention shape
(B=1, N=16384 tokens, H=70 heads, D=32, bf16 q/k/v, fp32 out as the reference
returns it, eps=1e-15): the state kernel, the merge kernel and the apply
kernel, enqueued through the C ABI on torch's current stream.  Inputs are
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
KERNEL_SRC = os.path.join(ROOT, "diffusion_transformer_relu_amd", "csrc", "linattn_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


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


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--out-dtype", choices=("f32", "bf16"), default="f32")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall time budget of the oracle CPU baseline (0 skips it)")
    ap.add_argument("--no-extras", action="store_true", help="skip the bf16-out and block-causal timings")
    args = ap.parse_args()

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

    def step(i, events=None):
        q, k, v = sets[i % NSETS]
        o = outs[i % NSETS]
        for s, st in enumerate(stages):
            if events is not None:
                events[s].record(stream)
            sana.sana_linattn_fwd_stages(q, k, v, o, ws, st, eps=w.eps, stream=stream)
        if events is not None:
            events[3].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    per_kernel_ms = {
        name: float(np.mean([e[s].elapsed_time(e[s + 1]) for e in evs]))
        for s, name in enumerate(("state", "merge", "apply"))
    }
    step_ms_events = float(np.mean([e[0].elapsed_time(e[3]) for e in evs]))

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
    if not args.no_extras:
        def timed(fn, n):
            for i in range(3):
                fn(i)
            torch.cuda.synchronize()
            a = time.perf_counter()
            for i in range(n):
                fn(i)
            torch.cuda.synchronize()
            return (time.perf_counter() - a) * 1e3 / n

        # the one-call entry point on the same buffers
        def fused(i):
            q, k, v = sets[i % NSETS]
            sana.sana_linattn_fwd(q, k, v, outs[i % NSETS], ws, eps=w.eps, stream=stream)
        ms = timed(fused, args.steps)
        extra["fused_call_f32out" if out_t == torch.float32 else "fused_call_bf16out"] = {
            "ms_per_step": round(ms, 5), "GBps": round(alg_bytes / ms / 1e6, 1)}

        other_t = torch.bfloat16 if out_t == torch.float32 else torch.float32
        other_bytes = 2 if other_t == torch.bfloat16 else 4
        outs2 = [torch.empty((B, N, H, D), dtype=other_t, device=dev) for _ in range(NSETS)]

        def fused2(i):
            q, k, v = sets[i % NSETS]
            sana.sana_linattn_fwd(q, k, v, outs2[i % NSETS], ws, eps=w.eps, stream=stream)
        ms = timed(fused2, args.steps)
        b2 = w.algorithmic_bytes(other_bytes)
        extra["fused_call_" + ("bf16out" if other_t == torch.bfloat16 else "f32out")] = {
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
        "step_ms_events": round(step_ms_events, 5),
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
