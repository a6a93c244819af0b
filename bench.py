"""Benchmark of the GDN sublayer hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload all|decode|prefill|varlen|kda]
                    [--no-cpu-baseline] [--calibration-copy]

Headline (``value``, ``ms_per_step``, ``roofline``): the fused decode step of
64 sequences x 1 token (bf16 activations, fp32 state [64, 48, 128, 128]
updated in place) in state-updates/s; one update = one sequence-token across
all 48 value heads.  Three state sets (604 MB) rotate so the 201 MB state
never sits in the 256 MB Infinity Cache between steps.

Also measured in the same run (``workloads``):
  prefill_s4096_bf16  one 4096-token sequence, conv -> chunk -> gated norm in one gdn_prefill call,
                      random initial state
  varlen8_33k_bf16    8 packed sequences (63, 64, 65 + five lengths up to 8192), same call
  kda_h64_s16384_bf16 per-key-channel decay, 64 heads, 16384 tokens, the chunk call alone
  kda_decode_b64_h64_bf16  the per-key-channel decode step, 64 sequences x 64 heads
  decode_b64_ab_bf16  the decode step with g, beta derived from the a / b projections
  verify_k4_b64_bf16  a speculative transaction: verify 4 rows x 64 sequences, commit all 4
  decode_b64_h16_bf16 the decode step with the recurrent state stored in fp16
each in tokens/s (state-updates/s for the decode) with its roofline fraction (algorithmic HBM
bytes / time / 8 TB/s).

Every workload rotates three copies of its inputs, states and outputs and times
at least 20 calls.  Every launch is a library call on torch's current stream
(the stream the library enqueues on), timed with events on that stream: the
mean from one event pair around all timed calls, median / p10 / p90 from a
second pass with an event after each call.  The prefill-side workloads also
report an ``mfma`` block (the method's algorithmic flops against the dense bf16 / fp16
peak).  ``cpu_baseline`` runs the fp64 oracle (test infrastructure) over a
bounded sample of the same workload, on every host core and on one thread.
``--calibration-copy`` only runs 256 MiB device copies (the known-size
reference for the HBM traffic counters).
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
CC = gi.conv_channels()
PEAK_HBM_GBS = 8000.0
METRIC = "GDN prefill tokens/s + decode state-updates/s; % MFMA / HBM roofline"
STATE_BYTES = HV * D * D * 4          # one sequence's fp32 state, 48 heads

# Algorithmic bytes (each input / output moved once):
# decode, per sequence-update: state read + write, conv state read + write, x, z, g, beta, out
DECODE_BYTES_PER_UPDATE = 2 * STATE_BYTES + 2 * 3 * CC * 2 + CC * 2 + HV * D * 2 + 2 * HV * 4 + HV * D * 2
# prefill pipeline, per token: x, z, g, beta in; gated output out (bf16); plus 2 states per sequence
PREFILL_BYTES_PER_TOKEN = CC * 2 + HV * D * 2 + 2 * HV * 4 + HV * D * 2
# per-key-channel chunk call, 64 heads, per token: q, k, v, g [64,128] fp32, beta, out (bf16)
KDA_H = 64
KDA_BYTES_PER_TOKEN = 3 * KDA_H * D * 2 + KDA_H * D * 4 + KDA_H * 4 + KDA_H * D * 2
KDA_STATE_BYTES = KDA_H * D * D * 4
# per-key-channel decode at 64 heads, per sequence-update: state read + write, conv state read + write,
# x, z, g [64,128] fp32, beta, out
KDA_CC = 3 * KDA_H * D
KDA_DECODE_BYTES_PER_UPDATE = (2 * KDA_STATE_BYTES + 2 * 3 * KDA_CC * 2 + KDA_CC * 2 + KDA_H * D * 2 +
                               KDA_H * D * 4 + KDA_H * 4 + KDA_H * D * 2)


def t_dev(a, bf16=False):
    x = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    return x.to(torch.bfloat16) if bf16 else x


def time_calls(fn, n_sets, steps, warmup):
    """Run fn(i) warmup + steps times, rotating over n_sets input sets; time the steps with
    events on the current stream (the stream every library call enqueues on).  Returns
    (mean ms, per-step ms list): the mean from one event pair around all steps (nothing
    recorded between launches), the per-step times from a second pass with an event after
    every step."""
    for i in range(warmup):
        fn(i % n_sets)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        fn(i % n_sets)
    e1.record()
    torch.cuda.synchronize()
    mean = e0.elapsed_time(e1) / steps
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record()
    for i in range(steps):
        fn(i % n_sets)
        evs[i + 1].record()
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    return mean, per


def spread(per):
    """Median, p10 and p90 of per-step times (ms)."""
    a = np.asarray(per)
    return {"median_ms": float(np.median(a)), "p10_ms": float(np.percentile(a, 10)),
            "p90_ms": float(np.percentile(a, 90)), "timed_calls": int(a.size)}


def rotated(tensors, n_sets):
    """n_sets device copies of each tensor (None stays None): the timed calls rotate over
    them, so no call finds its inputs or state left in the 256 MB Infinity Cache by the
    call before."""
    return [[None if t is None else t.clone() for t in tensors] for _ in range(n_sets)]


# HBM bytes per launch measured with the FETCH_SIZE / WRITE_SIZE counters, scaled by a known-size
# copy (profiles/hbm_traffic_pmc.txt); valid for the kernels as they stand when it was taken.
DECODE_TRAFFIC_BYTES = 213.9e6 + 206.1e6          # both launches of a step
PREFILL_S4096_TRAFFIC_BYTES = 366.1e6 + 278.0e6    # gdn_prefill, all its kernels
VARLEN_TRAFFIC_BYTES = 2843.8e6 + 1758.4e6
KDA_TRAFFIC_BYTES = 2430.6e6 + 1287.7e6


def roofline(bytes_alg, ms, traffic=None):
    achieved = bytes_alg / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS, "traffic": traffic}


# Algorithmic flops of the chunk-wise rule per token and value head (64-token chunks, d = 128;
# triangles counted as triangles): K K^T, W and U strictly lower (C(C-1)/2 d MACs each),
# Q K^T and P V lower with the diagonal (C(C+1)/2 d), three full C d^2 products (the state
# read for the rows, the state read for the output, the state update), and the unit-lower
# solve (C^3 / 3 flops); divided by C.
CHUNK_C = 64
RULE_FLOPS_PER_TOKEN_HEAD = (3 * CHUNK_C * (CHUNK_C - 1) * D + 2 * CHUNK_C * (CHUNK_C + 1) * D
                             + 3 * 2 * CHUNK_C * D * D + CHUNK_C ** 3 / 3) / CHUNK_C
# the pipeline adds per token: the width-4 conv (2 flops per tap and channel), the q / k L2
# norms (2 per element) and the gated norm (5 per output element: square-add, three scalings)
PIPE_EXTRA_FLOPS_PER_TOKEN = 2 * 4 * CC + 2 * 2 * HK * D + 5 * HV * D
PREFILL_FLOPS_PER_TOKEN = HV * RULE_FLOPS_PER_TOKEN_HEAD + PIPE_EXTRA_FLOPS_PER_TOKEN
KDA_FLOPS_PER_TOKEN = KDA_H * RULE_FLOPS_PER_TOKEN_HEAD
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 and fp16 MFMA (the same rate)


def mfma_block(flops, ms):
    """Achieved matrix throughput from algorithmic flops (the spines' contractions are
    issued on fp16 MFMA, the intra kernels' Gram products on bf16 MFMA) against the dense
    bf16 / fp16 peak."""
    achieved = flops / (ms * 1e-3) / 1e12
    return {"achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
            "flops_per_call": flops}


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

def bench_decode(steps, warmup, batch=64, per_channel=False, derived_gates=False, state_f16=False):
    """64 sequences of one token; per_channel: the per-key-channel decode at 64 heads (ratio 1);
    derived_gates: g and beta derived in the kernel from the a / b projections (gdn_decode_step_ab)."""
    if per_channel:
        geo = gi.Geometry(hk=KDA_H, hv=KDA_H)
        d = gi.gen_decode(1006, batch, geo, per_channel=True)
        cfg = gdn.config(num_k_heads=KDA_H, num_v_heads=KDA_H, decay_per_key_channel=1)
        hv, bytes_per, traffic = KDA_H, KDA_DECODE_BYTES_PER_UPDATE, None
    else:
        d = gi.gen_decode(1002, batch)
        cfg = gdn.config()
        hv, bytes_per, traffic = HV, DECODE_BYTES_PER_UPDATE, DECODE_TRAFFIC_BYTES
    ab = None
    if derived_gates:
        r = gi.gen_gate_projections(1102, batch)
        ab = (t_dev(r["a"], True), t_dev(r["b"], True), t_dev(r["A_log"]), t_dev(r["dt_bias"]))
        bytes_per, traffic = bytes_per - 2 * hv * 4 + 2 * hv * 2, None   # a, b bf16 in place of g, beta fp32
    if state_f16:   # the fp16 state: half the state bytes
        bytes_per, traffic = bytes_per - hv * D * D * 4, None
    n_sets = 3
    x, w, g, beta, z, nw = (t_dev(d["x"], True), t_dev(d["conv_w"]), t_dev(d["g"]), t_dev(d["beta"]),
                            t_dev(d["z"], True), t_dev(d["norm_w"]))
    states = [t_dev(d["state"]).to(torch.float16 if state_f16 else torch.float32) for _ in range(n_sets)]
    convs = [t_dev(d["conv_state"], True) for _ in range(n_sets)]
    out = torch.empty((batch, hv, D), dtype=torch.bfloat16, device="cuda")

    def step(i):
        if ab is None:
            gdn.decode_step(x, w, convs[i], g, beta, z, nw, states[i], out=out, cfg=cfg)
        else:
            gdn.decode_step(x, w, convs[i], None, None, z, nw, states[i], out=out, cfg=cfg, ab=ab)

    ms, per = time_calls(step, n_sets, steps, warmup)
    return dict(ms=ms, per=per, updates_per_s=batch / (ms * 1e-3),
                roofline=roofline(bytes_per * batch, ms, traffic), **spread(per))


def bench_verify(steps, warmup, batch=64, K=4):
    """One speculative transaction per step: gdn_verify of K rows for every sequence, then
    gdn_verify_commit accepting all K (the commit's largest write)."""
    steps_in = [gi.gen_decode(2400 + t, batch) for t in range(K)]
    d = steps_in[0]
    cfg = gdn.config()
    x = t_dev(np.stack([st["x"] for st in steps_in], 1), True)
    g = t_dev(np.stack([st["g"] for st in steps_in], 1))
    beta = t_dev(np.stack([st["beta"] for st in steps_in], 1))
    z = t_dev(np.stack([st["z"] for st in steps_in], 1), True)
    w, nw = t_dev(d["conv_w"]), t_dev(d["norm_w"])
    n_sets = 3
    states = [t_dev(d["state"]) for _ in range(n_sets)]
    convs = [t_dev(d["conv_state"], True) for _ in range(n_sets)]
    out = torch.empty((batch, K, HV, D), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(gdn.verify_workspace_size(batch, K, cfg), dtype=torch.uint8, device="cuda")
    accepted = torch.full((batch,), K, dtype=torch.int32, device="cuda")

    def step(i):
        gdn.verify(x, w, convs[i], g, beta, z, nw, states[i], out=out, workspace=ws, cfg=cfg)
        gdn.verify_commit(accepted, x, g, convs[i], states[i], ws, cfg=cfg)

    ms, per = time_calls(step, n_sets, steps, warmup)
    stats = spread(per)
    rec = K * (HV * D + HK * D) * 4
    # per sequence: state read by the verify, read + written by the commit; conv state read
    # by each and written by the commit; x, z, g, beta and out of the K rows; the records
    # written and read back
    per_seq = (3 * STATE_BYTES + 3 * 3 * CC * 2 + K * (2 * CC * 2 + HV * D * 2 + 3 * HV * 4 + HV * D * 2)
               + 2 * rec)
    return dict(ms=ms, rows_per_s=batch * K / (ms * 1e-3), roofline=roofline(per_seq * batch, ms, None),
                bytes_per_transaction=per_seq * batch, **stats)


def _oracle():
    import oracle
    return oracle.Oracle()


def cpu_baseline_decode(target_s=10.0, single_s=5.0):
    """The oracle's fused decode step of the 64-sequence batch, repeated for about target_s on
    every host core, then about single_s on one thread."""
    orc = _oracle()
    d = gi.gen_decode(1002, 64)

    def run(limit_s):
        reps, t0 = 0, time.perf_counter()
        state, cs = d["state"], d["conv_state"]
        while True:
            _, cs, state = orc.decode_step(d["x"], d["conv_w"], cs, d["g"], d["beta"], d["z"], d["norm_w"],
                                           state, Hk=HK, Hv=HV, dk=D, dv=D)
            reps += 1
            el = time.perf_counter() - t0
            if el >= limit_s or reps >= 400:
                return reps, el

    cores = orc.max_threads()
    reps, el = run(target_s)
    orc.set_threads(1)
    reps1, el1 = run(single_s)
    orc.set_threads(cores)
    return dict(value=64 * reps / el, unit="state-updates/s", cores=cores, kind="oracle",
                sample=f"{reps} fused decode steps of the 64-sequence batch, fp64, {el:.1f} s",
                single_thread=dict(value=64 * reps1 / el1, cores=1,
                                   sample=f"{reps1} steps of the same batch on one thread, {el1:.1f} s"))


# ---------------------------------------------------------------------------
# prefill pipelines (conv -> chunk -> gated norm)
# ---------------------------------------------------------------------------

def bench_pipeline(lengths, seed, steps, warmup, n_sets=3):
    """A step is one gdn_prefill call (conv -> chunk -> gated norm) on one of n_sets rotated
    copies of the inputs, states and outputs.  The same work as three separate calls (conv,
    chunk with an fp32 output, norm) is timed per call for the split."""
    d = gi.gen_prefill(seed, lengths, bf16=True, init_state=True)
    cfg = gdn.config()
    T, N = int(sum(lengths)), len(lengths)
    cu_np = d["cu"]
    cu = torch.from_numpy(cu_np).cuda()
    base = (t_dev(d["x"], True), t_dev(d["g"]), t_dev(d["beta"]), t_dev(d["z"], True), t_dev(d["state_in"]),
            torch.empty((N, HV, D, D), dtype=torch.float32, device="cuda"),
            torch.empty((T, HV, D), dtype=torch.bfloat16, device="cuda"))
    w, nw = t_dev(d["conv_w"]), t_dev(d["norm_w"])
    del d
    sets = rotated(base, n_sets)
    del base
    y = torch.empty((T, CC), dtype=torch.bfloat16, device="cuda")
    o = torch.empty((T, HV, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(gdn.chunk_prefill_workspace_size(N, T, cfg), dtype=torch.uint8, device="cuda")
    ws_one = torch.empty(gdn.prefill_workspace_size(N, T, torch.bfloat16, cfg), dtype=torch.uint8, device="cuda")

    def one_call(i):
        x, g, beta, z, s_in, s_out, out = sets[i]
        gdn.prefill(x, w, cu, g, beta, z, nw, cu_host=cu_np, initial_state=s_in, out=out, final_state=s_out,
                    workspace=ws_one, cfg=cfg)

    def conv(i):
        gdn.conv1d_prefill(sets[i][0], w, cu, cu_host=cu_np, y=y, cfg=cfg)

    def chunk(i):
        x, g, beta, z, s_in, s_out, out = sets[i]
        gdn.chunk_prefill(y[:, : HK * D], y[:, HK * D: 2 * HK * D], y[:, 2 * HK * D:], g, beta, cu,
                          cu_host=cu_np, initial_state=s_in, out=o, final_state=s_out, workspace=ws, cfg=cfg)

    def norm(i):
        gdn.gated_rmsnorm(o, sets[i][3], nw, out=sets[i][6], cfg=cfg)

    ms, per = time_calls(one_call, n_sets, steps, warmup)
    # the separate calls, each timed, over a few passes
    split = {"conv_ms": 0.0, "chunk_ms": 0.0, "norm_ms": 0.0}
    reps = 3
    conv(0)   # first launches of these kernel variants load their code, untimed
    chunk(0)
    norm(0)
    torch.cuda.synchronize()
    for r in range(reps):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        evs[0].record()
        conv(r % n_sets)
        evs[1].record()
        chunk(r % n_sets)
        evs[2].record()
        norm(r % n_sets)
        evs[3].record()
        torch.cuda.synchronize()
        for i, key in enumerate(split):
            split[key] += evs[i].elapsed_time(evs[i + 1]) / reps
    bytes_alg = PREFILL_BYTES_PER_TOKEN * T + 2 * STATE_BYTES * N
    traffic = {(4096,): PREFILL_S4096_TRAFFIC_BYTES,
               tuple(gi.varlen_lengths()[0]): VARLEN_TRAFFIC_BYTES}.get(tuple(lengths))
    # the latency floor: the longest sequence's chunks are a serial chain
    serial = max((n + CHUNK_C - 1) // CHUNK_C for n in lengths)
    return dict(ms=ms, tokens=T, tokens_per_s=T / (ms * 1e-3), roofline=roofline(bytes_alg, ms, traffic),
                mfma=mfma_block(PREFILL_FLOPS_PER_TOKEN * T, ms),
                roofline_ms=bytes_alg / (PEAK_HBM_GBS * 1e9) * 1e3, separate_calls=split,
                serial_chunk_steps=serial, chunk_call_us_per_serial_step=split["chunk_ms"] * 1e3 / serial,
                **spread(per))


def _head_of(lengths, max_tokens):
    take, total = [], 0
    for n in lengths:
        if total + n > max_tokens:
            take.append(max_tokens - total)
            break
        take.append(n)
        total += n
    return [n for n in take if n > 0]


def _repeat(run, limit_s):
    """Call run() (which returns its own seconds) until limit_s have passed; returns (calls, s)."""
    n, el = 0, 0.0
    while el < limit_s:
        el += run()
        n += 1
    return n, el


def cpu_baseline_pipeline(lengths, seed, max_tokens, single_tokens=1024, target_s=10.0, single_s=5.0):
    """The oracle's conv -> rule -> norm over the first sequences of the workload (up to
    max_tokens tokens), repeated for about target_s on every host core, then over up to
    single_tokens repeated for about single_s on one thread."""
    orc = _oracle()

    def sample(limit):
        take = _head_of(lengths, limit)
        d = gi.gen_prefill(seed, take, bf16=True, init_state=True)

        def run():
            t0 = time.perf_counter()
            orc.prefill(d["x"], d["conv_w"], d["cu"], d["g"], d["beta"], d["z"], d["norm_w"], Hk=HK, Hv=HV, dk=D,
                        dv=D, state_in=d["state_in"], round_y_bf16=True)
            return time.perf_counter() - t0
        return take, run

    cores = orc.max_threads()
    take, run = sample(max_tokens)
    n, el = _repeat(run, target_s)
    orc.set_threads(1)
    take1, run1 = sample(single_tokens)
    n1, el1 = _repeat(run1, single_s)
    orc.set_threads(cores)
    T, T1 = int(sum(take)), int(sum(take1))
    return dict(value=n * T / el, unit="tokens/s", cores=cores, kind="oracle",
                sample=f"{n} passes over {T} tokens (sequence lengths {take}) of the workload, all 48 heads, fp64, "
                       f"{el:.1f} s",
                single_thread=dict(value=n1 * T1 / el1, cores=1,
                                   sample=f"{n1} passes over {T1} tokens (lengths {take1}) on one thread, {el1:.1f} s"))


# ---------------------------------------------------------------------------
# per-key-channel decay, chunk call alone
# ---------------------------------------------------------------------------

def bench_kda(steps, warmup, T=16384, n_sets=3):
    """The per-key-channel chunk call on n_sets rotated copies of its inputs (1.4 GB each)."""
    geo = gi.Geometry(hk=KDA_H, hv=KDA_H)
    d = gi.gen_qkv(1005, [T], geo, per_channel=True)
    cfg = gdn.config(num_k_heads=KDA_H, num_v_heads=KDA_H, decay_per_key_channel=1)
    cu_np = d["cu"]
    cu = torch.from_numpy(cu_np).cuda()
    base = (t_dev(d["q"], True), t_dev(d["k"], True), t_dev(d["v"], True), t_dev(d["g"]), t_dev(d["beta"]),
            t_dev(d["state_in"]), torch.empty((1, KDA_H, D, D), dtype=torch.float32, device="cuda"),
            torch.empty((T, KDA_H, D), dtype=torch.bfloat16, device="cuda"))
    del d
    sets = rotated(base, n_sets)
    del base
    ws = torch.empty(gdn.chunk_prefill_workspace_size(1, T, cfg), dtype=torch.uint8, device="cuda")

    def step(i):
        q, k, v, g, beta, s_in, s_out, out = sets[i]
        gdn.chunk_prefill(q, k, v, g, beta, cu, cu_host=cu_np, initial_state=s_in, out=out, final_state=s_out,
                          workspace=ws, cfg=cfg)

    ms, per = time_calls(step, n_sets, steps, warmup)
    bytes_alg = KDA_BYTES_PER_TOKEN * T + 2 * KDA_STATE_BYTES
    return dict(ms=ms, tokens=T, tokens_per_s=T / (ms * 1e-3), roofline=roofline(bytes_alg, ms, KDA_TRAFFIC_BYTES),
                mfma=mfma_block(KDA_FLOPS_PER_TOKEN * T, ms),
                roofline_ms=bytes_alg / (PEAK_HBM_GBS * 1e9) * 1e3, **spread(per))


def cpu_baseline_kda(tokens=2048, single_tokens=256, target_s=10.0, single_s=5.0):
    """The oracle's per-key-channel rule over the first tokens of the workload, repeated for
    about target_s on every host core and single_s on one thread."""
    orc = _oracle()
    geo = gi.Geometry(hk=KDA_H, hv=KDA_H)

    def sample(n):
        d = gi.gen_qkv(1005, [n], geo, per_channel=True)

        def run():
            t0 = time.perf_counter()
            orc.delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"], d["state_in"])
            return time.perf_counter() - t0
        return run

    cores = orc.max_threads()
    n, el = _repeat(sample(tokens), target_s)
    orc.set_threads(1)
    n1, el1 = _repeat(sample(single_tokens), single_s)
    orc.set_threads(cores)
    return dict(value=n * tokens / el, unit="tokens/s", cores=cores, kind="oracle",
                sample=f"{n} passes over the first {tokens} tokens of the 16384-token per-key-channel workload, "
                       f"64 heads, fp64, {el:.1f} s",
                single_thread=dict(value=n1 * single_tokens / el1, cores=1,
                                   sample=f"{n1} passes over the first {single_tokens} tokens on one thread, "
                                          f"{el1:.1f} s"))


def calibration_copy(steps):
    n = 256 * 1024 * 1024 // 4
    a = torch.randn(n, device="cuda")
    b = torch.empty_like(a)
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="all",
                    choices=["all", "decode", "prefill", "varlen", "kda", "kda_decode", "decode_ab", "verify",
                             "decode_h16"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibration-copy", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the library has no "
              f"multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    if args.calibration_copy:
        calibration_copy(args.steps)
        print(json.dumps({"calibration_copy_bytes": 2 * 256 * 1024 * 1024, "copies": args.steps}))
        return
    wl = args.workload
    cpu = not args.no_cpu_baseline
    # the other workloads: at least 100 timed calls after at least 10 untimed (15 ms to 0.2 s
    # of GPU time each); the clocks settle over the first calls
    small_steps, small_warm = max(100, args.steps // 2), max(10, args.warmup)
    line = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "data": "synthetic"}
    workloads = {}
    if wl in ("all", "decode"):
        dec = bench_decode(args.steps, args.warmup)
        line.update({
            "value": dec["updates_per_s"], "unit": "state-updates/s", "ms_per_step": dec["ms"],
            "dtype": "f32",
            "config": {"workload": "decode_b64_bf16", "batch": 64, "k_heads": HK, "v_heads": HV, "head_dim": D,
                       "activations": "bf16", "state": "f32 [64,48,128,128], 3 sets rotated"},
            "median_ms": dec["median_ms"], "p10_ms": dec["p10_ms"], "p90_ms": dec["p90_ms"],
            "input_sets": 3, "head_updates_per_s": dec["updates_per_s"] * HV,
            "roofline": dict(dec["roofline"], kernel="decode_step_kernel + conv_shift_kernel (the two launches of one step, timed together)",
                             bytes_per_update=DECODE_BYTES_PER_UPDATE),
        })
        if cpu:
            line["cpu_baseline"] = cpu_baseline_decode()
    if wl in ("all", "prefill"):
        pre = bench_pipeline([4096], 1003, small_steps, small_warm)
        workloads["prefill_s4096_bf16"] = dict(
            metric="tokens/s", value=pre["tokens_per_s"], ms=pre["ms"], call="gdn_prefill",
            separate_calls=pre["separate_calls"], roofline=pre["roofline"], mfma=pre["mfma"],
            roofline_ms=pre["roofline_ms"], dtype="bf16 storage; fp16-operand MFMA (bf16 in the intra Gram products), f32 accumulate and state",
            input_sets=3, **{k: pre[k] for k in ("median_ms", "p10_ms", "p90_ms", "timed_calls",
                                                  "serial_chunk_steps", "chunk_call_us_per_serial_step")})
        if cpu:
            workloads["prefill_s4096_bf16"]["cpu_baseline"] = cpu_baseline_pipeline([4096], 1003, 4096)
    if wl in ("all", "varlen"):
        lengths, _ = gi.varlen_lengths()
        var = bench_pipeline(lengths, 1004, small_steps, small_warm)
        workloads["varlen8_33k_bf16"] = dict(
            metric="tokens/s", value=var["tokens_per_s"], ms=var["ms"], tokens=var["tokens"], lengths=lengths,
            call="gdn_prefill", separate_calls=var["separate_calls"], roofline=var["roofline"], mfma=var["mfma"],
            roofline_ms=var["roofline_ms"], input_sets=3,
            **{k: var[k] for k in ("median_ms", "p10_ms", "p90_ms", "timed_calls",
                                   "serial_chunk_steps", "chunk_call_us_per_serial_step")})
        if cpu:
            workloads["varlen8_33k_bf16"]["cpu_baseline"] = cpu_baseline_pipeline(lengths, 1004, 4096)
    if wl in ("all", "kda"):
        kda = bench_kda(small_steps, 10)
        workloads["kda_h64_s16384_bf16"] = dict(
            metric="tokens/s", value=kda["tokens_per_s"], ms=kda["ms"], roofline=kda["roofline"], mfma=kda["mfma"],
            roofline_ms=kda["roofline_ms"], call="gdn_chunk_prefill, decay per key channel", input_sets=3,
            **{k: kda[k] for k in ("median_ms", "p10_ms", "p90_ms", "timed_calls")})
        if cpu:
            workloads["kda_h64_s16384_bf16"]["cpu_baseline"] = cpu_baseline_kda()
    if wl in ("all", "decode_h16"):
        dh = bench_decode(small_steps, small_warm, state_f16=True)
        workloads["decode_b64_h16_bf16"] = dict(
            metric="state-updates/s", value=dh["updates_per_s"], ms=dh["ms"], roofline=dh["roofline"],
            median_ms=dh["median_ms"], p10_ms=dh["p10_ms"], p90_ms=dh["p90_ms"],
            call="gdn_decode_step_h16: the recurrent state stored in fp16 (rounded once per token)")
    if wl in ("all", "verify"):
        ver = bench_verify(small_steps, small_warm)
        workloads["verify_k4_b64_bf16"] = dict(
            metric="state-updates/s", value=ver["rows_per_s"], ms=ver["ms"], roofline=ver["roofline"],
            median_ms=ver["median_ms"], p10_ms=ver["p10_ms"], p90_ms=ver["p90_ms"],
            bytes_per_transaction=ver["bytes_per_transaction"],
            call="gdn_verify (64 sequences x 4 rows) + gdn_verify_commit accepting all 4; one update = one row")
    if wl in ("all", "decode_ab"):
        dab = bench_decode(small_steps, small_warm, derived_gates=True)
        workloads["decode_b64_ab_bf16"] = dict(
            metric="state-updates/s", value=dab["updates_per_s"], ms=dab["ms"], roofline=dab["roofline"],
            median_ms=dab["median_ms"], p10_ms=dab["p10_ms"], p90_ms=dab["p90_ms"],
            call="gdn_decode_step_ab: g, beta derived in the kernel from the a / b projections")
    if wl in ("all", "kda_decode"):
        kdd = bench_decode(small_steps, small_warm, per_channel=True)
        workloads["kda_decode_b64_h64_bf16"] = dict(
            metric="state-updates/s", value=kdd["updates_per_s"], ms=kdd["ms"], roofline=kdd["roofline"],
            median_ms=kdd["median_ms"], p10_ms=kdd["p10_ms"], p90_ms=kdd["p90_ms"],
            bytes_per_update=KDA_DECODE_BYTES_PER_UPDATE,
            call="gdn_decode_step, decay per key channel, 64 heads, state f32 [64,64,128,128], 3 sets rotated")
    if wl != "decode" and "value" not in line:
        # a single prefill-side workload was requested: it is the headline
        name, obj = next(iter(workloads.items()))
        line.update({"value": obj["value"], "unit": obj["metric"], "ms_per_step": obj["ms"], "dtype": "bf16",
                     "config": {"workload": name}, "roofline": obj["roofline"]})
        for key in ("mfma", "median_ms", "p10_ms", "p90_ms"):
            if key in obj:
                line[key] = obj[key]
        if "cpu_baseline" in obj:
            line["cpu_baseline"] = obj["cpu_baseline"]
    if workloads:
        line["workloads"] = workloads
    print(json.dumps(line))


if __name__ == "__main__":
    main()
