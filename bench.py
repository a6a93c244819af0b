"""Benchmark of the GDN sublayer hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Headline (``value``): the fused decode step of 64 sequences x 1 token, bf16
activations, fp32 state [64, 48, 128, 128] updated in place -> state-updates/s
(one update = one sequence-token across all 48 value heads).  Three state sets
(604 MB) are rotated so the 201 MB state never sits in the 256 MB Infinity
Cache between steps.

Also measured in the same run and reported under ``prefill``: the 4096-token
prefill (conv -> chunk-wise delta rule -> gated norm, bf16 inputs, random fp32
initial state) in tokens/s.

Every timed launch is a library call on torch's current stream, timed with
events on that stream.  ``cpu_baseline`` runs the fp64 oracle (test
infrastructure) on the host cores over a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import gated_deltanet_causal_amd as gdn  # noqa: E402
import gdn_inputs as gi  # noqa: E402

HK, HV, D = gi.HK, gi.HV, gi.DK
PEAK_HBM_GBS = 8000.0
METRIC = "GDN prefill tokens/s + decode state-updates/s; % MFMA / HBM roofline"

# Algorithmic bytes of one decode sequence-update (each input / output moved once):
# state read + write, conv state read + write, x, z, g, beta, out.
DECODE_BYTES_PER_UPDATE = (2 * HV * D * D * 4 + 2 * 3 * gi.conv_channels() * 2 + gi.conv_channels() * 2
                           + HV * D * 2 + 2 * HV * 4 + HV * D * 2)
# Algorithmic bytes of one prefill token through conv -> chunk -> norm, fused minimum:
# x, z, g, beta in; out (bf16) out.  The 2 x 3 MiB per-sequence state is added per call.
PREFILL_BYTES_PER_TOKEN = gi.conv_channels() * 2 + HV * D * 2 + 2 * HV * 4 + HV * D * 2
STATE_BYTES = HV * D * D * 4


def t_dev(a, bf16=False):
    x = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    return x.to(torch.bfloat16) if bf16 else x


def time_launches(fn, n_sets, steps, warmup):
    """Run fn(i) warmup + steps times; time the steps with events on the current stream.
    Returns (total_ms, per-launch ms list)."""
    for i in range(warmup):
        fn(i % n_sets)
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record()
    for i in range(steps):
        fn(i % n_sets)
        evs[i + 1].record()
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    return evs[0].elapsed_time(evs[-1]), per


def bench_decode(steps, warmup, batch=64):
    d = gi.gen_decode(1002, batch)
    cfg = gdn.config()
    n_sets = 3
    x, w, g, beta, z, nw = (t_dev(d["x"], True), t_dev(d["conv_w"]), t_dev(d["g"]), t_dev(d["beta"]),
                            t_dev(d["z"], True), t_dev(d["norm_w"]))
    states = [t_dev(d["state"]) for _ in range(n_sets)]
    convs = [t_dev(d["conv_state"], True) for _ in range(n_sets)]
    out = torch.empty((batch, HV, D), dtype=torch.bfloat16, device="cuda")

    def step(i):
        gdn.decode_step(x, w, convs[i], g, beta, z, nw, states[i], out=out, cfg=cfg)

    total_ms, per = time_launches(step, n_sets, steps, warmup)
    ms = total_ms / steps
    achieved = DECODE_BYTES_PER_UPDATE * batch / (ms * 1e-3) / 1e9
    return dict(ms=ms, per=per, updates_per_s=batch / (ms * 1e-3), achieved_gbs=achieved)


def bench_prefill(steps, warmup, T=4096):
    d = gi.gen_prefill(1003, [T], bf16=True, init_state=True)
    cfg = gdn.config()
    cu_np = d["cu"]
    cu = torch.from_numpy(cu_np).cuda()
    x, w, g, beta, z, nw = (t_dev(d["x"], True), t_dev(d["conv_w"]), t_dev(d["g"]), t_dev(d["beta"]),
                            t_dev(d["z"], True), t_dev(d["norm_w"]))
    s_in = t_dev(d["state_in"])
    s_out = torch.empty_like(s_in)
    y = torch.empty((T, gi.conv_channels()), dtype=torch.bfloat16, device="cuda")
    o = torch.empty((T, HV, D), dtype=torch.float32, device="cuda")
    out = torch.empty((T, HV, D), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(gdn.chunk_prefill_workspace_size(1, T, cfg), dtype=torch.uint8, device="cuda")
    marks = {}

    def step(_):
        gdn.conv1d_prefill(x, w, cu, cu_host=cu_np, y=y, cfg=cfg)
        gdn.chunk_prefill(y[:, : HK * D], y[:, HK * D: 2 * HK * D], y[:, 2 * HK * D:], g, beta, cu,
                          cu_host=cu_np, initial_state=s_in, out=o, final_state=s_out, workspace=ws, cfg=cfg)
        gdn.gated_rmsnorm(o, z, nw, out=out, cfg=cfg)

    total_ms, per = time_launches(step, 1, steps, warmup)
    ms = total_ms / steps
    # one instrumented pass: time of each library call
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    evs[0].record()
    gdn.conv1d_prefill(x, w, cu, cu_host=cu_np, y=y, cfg=cfg)
    evs[1].record()
    gdn.chunk_prefill(y[:, : HK * D], y[:, HK * D: 2 * HK * D], y[:, 2 * HK * D:], g, beta, cu,
                      cu_host=cu_np, initial_state=s_in, out=o, final_state=s_out, workspace=ws, cfg=cfg)
    evs[2].record()
    gdn.gated_rmsnorm(o, z, nw, out=out, cfg=cfg)
    evs[3].record()
    torch.cuda.synchronize()
    marks = dict(conv_ms=evs[0].elapsed_time(evs[1]), chunk_ms=evs[1].elapsed_time(evs[2]),
                 norm_ms=evs[2].elapsed_time(evs[3]))
    bytes_alg = PREFILL_BYTES_PER_TOKEN * T + 2 * STATE_BYTES
    return dict(ms=ms, per=per, tokens_per_s=T / (ms * 1e-3), achieved_gbs=bytes_alg / (ms * 1e-3) / 1e9,
                roofline_ms=bytes_alg / (PEAK_HBM_GBS * 1e9) * 1e3, **marks)


def cpu_baseline_decode(target_s=10.0):
    import oracle
    orc = oracle.Oracle()
    d = gi.gen_decode(1002, 64)
    reps, t0 = 0, time.perf_counter()
    state, cs = d["state"], d["conv_state"]
    while True:
        _, cs, state = orc.decode_step(d["x"], d["conv_w"], cs, d["g"], d["beta"], d["z"], d["norm_w"], state,
                                       Hk=HK, Hv=HV, dk=D, dv=D)
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s or reps >= 200:
            break
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return dict(value=64 * reps / el, unit="state-updates/s", cores=threads, kind="oracle",
                sample=f"{reps} decode steps of the 64-sequence batch, fp64, {el:.1f} s")


def cpu_baseline_prefill(tokens=512):
    import oracle
    orc = oracle.Oracle()
    d = gi.gen_prefill(1003, [tokens], bf16=True, init_state=True)
    t0 = time.perf_counter()
    orc.prefill(d["x"], d["conv_w"], d["cu"], d["g"], d["beta"], d["z"], d["norm_w"], Hk=HK, Hv=HV, dk=D, dv=D,
                state_in=d["state_in"], round_y_bf16=True)
    el = time.perf_counter() - t0
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return dict(value=tokens / el, unit="tokens/s", cores=threads, kind="oracle",
                sample=f"first {tokens} tokens of the 4096-token prefill, all 48 heads, fp64, {el:.1f} s")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this build has no "
              f"multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    dec = bench_decode(args.steps, args.warmup)
    pre = bench_prefill(max(10, args.steps // 10), max(3, args.warmup // 4))
    per = np.array(dec["per"])
    line = {
        "metric": METRIC,
        "value": dec["updates_per_s"],
        "unit": "state-updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dec["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "decode_b64_bf16", "batch": 64, "k_heads": HK, "v_heads": HV, "head_dim": D,
                   "activations": "bf16", "state": "f32 [64,48,128,128] x3 rotated"},
        "p10_ms": float(np.percentile(per, 10)),
        "p90_ms": float(np.percentile(per, 90)),
        "head_updates_per_s": dec["updates_per_s"] * HV,
        "roofline": {"bound": "hbm", "achieved": dec["achieved_gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": dec["achieved_gbs"] / PEAK_HBM_GBS, "traffic": None,
                     "kernel": "decode_step_kernel", "bytes_per_update": DECODE_BYTES_PER_UPDATE},
        "prefill": {"workload": "prefill_s4096_bf16", "tokens_per_s": pre["tokens_per_s"], "ms": pre["ms"],
                    "conv_ms": pre["conv_ms"], "chunk_ms": pre["chunk_ms"], "norm_ms": pre["norm_ms"],
                    "roofline": {"bound": "hbm", "achieved": pre["achieved_gbs"], "peak": PEAK_HBM_GBS,
                                 "unit": "GB/s", "frac": pre["achieved_gbs"] / PEAK_HBM_GBS,
                                 "roofline_ms": pre["roofline_ms"]}},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_decode()
        line["prefill"]["cpu_baseline"] = cpu_baseline_prefill()
    print(json.dumps(line))


if __name__ == "__main__":
    main()
