#!/usr/bin/env python3
"""Benchmark of the gated delta rule on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--skip-decode]
                    [--skip-batched] [--no-cpu-baseline]

One "step" is one chunked prefill of the 16K-token layer workload
(B=1, H=16, T=16384, dk=dv=128, bf16 q/k/v/o, fp32 gates and state, keys in a
narrow cone, 10 short- / 6 long-horizon heads).  `value` is its throughput in
tokens/s with inputs resident in HBM.  The same JSON line also carries the
decode step at B=64 (dk=128 and the channel-pruned dk=64) and B=1, and the
batched prefill B=8, T=4096 at dk=128 vs 64, each with its own roofline.

Timing: W untimed steps, continued until at least 0.1 s of back-to-back load
has passed (the GPU's clocks take ~30 ms of sustained load to settle, so every
leg is timed in steady state); then K steps launched eagerly with HIP events
around each phase (the per-kernel durations, recorded on the stream the
kernels are launched on: torch's current stream, which the binding passes to
libgdn); then the timed K steps, bracketed by device synchronisation, as
replays of a HIP graph that holds one step.
Decode timing captures 512 steps x 18 state sets (one per GDN layer of a
Qwen3.5-0.8B-sized model) in one HIP graph, so consecutive launches touch
different 64 MiB states and the state streams from HBM rather than the
256 MB last-level cache.

The fp64 oracle is timed on the host cores first (before the GPU is
initialised) as a reported baseline; it is not the target.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import multiprocessing as mp
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from workloads import gdn_inputs as gi  # noqa: E402

HBM_PEAK = 8.0e12           # B/s, MI355X HBM3E
MFMA_BF16_PEAK = 2.5e15     # flop/s, dense bf16
C = 64                      # tokens per chunk


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic traffic and executed MFMA work
# ---------------------------------------------------------------------------

def prefill_bytes(B, T, H, dk, dv, io_bytes=2, with_S0=False):
    """q, k, v read + o written (io dtype), alpha/beta read (fp32), final
    state written (fp32), initial state read if given."""
    per_tok = io_bytes * (2 * dk + 2 * dv) + 8
    state = 4 * dv * dk * (2 if with_S0 else 1)
    return B * H * (T * per_tok + state)


def decode_bytes(B, H, dk, dv, io_bytes=2):
    """State read + written once (fp32), q, k, v read, o written, gates."""
    return B * H * (8 * dv * dk + io_bytes * (2 * dk + 2 * dv) + 8)


def prefill_mfma_flops(B, T, H, dk, dv, nseg, seg_chunks):
    """bf16 MFMA flops the prefill kernels execute (bf16 in / bf16 out), from
    their structure; one v_mfma_f32_16x16x32_bf16 = 16384 flops.
      prepare: per chunk and head, 10 lower tiles of K K^T and of Q K^T,
               dk/32 k-steps each.
      scan:    per chunk and 16-row wave: K S^T 4 x dk/32 x 2 (split state),
               Q S^T 4 x dk/32, T Z 6 k-blocks x 3, P U 6, state update
               dk/16 tiles x 2 k-blocks x 2; transition rows (dk per head)
               run for the chunks of segments >= 1.
      combine: per later segment and 16-row wave: dk/16 x dk/32 x 3.
      correct: per chunk of later segments and 16-row wave: 4 x dk/32."""
    nch = -(-T // C)
    nkb, ndt = dk // 32, dk // 16
    f = 16 * 16 * 32 * 2
    prep = B * H * nch * 20 * nkb
    per_wave_chunk = 4 * nkb * 2 + 4 * nkb + 6 * 3 + 6 + ndt * 2 * 2
    later = nch - seg_chunks if nseg > 1 else 0
    scan = B * H * (dv // 16 * nch + dk // 16 * later) * per_wave_chunk
    comb = B * H * (nseg - 1) * (dv // 16) * ndt * nkb * 3
    corr = B * H * later * (dv // 16) * 4 * nkb
    return prep * f, (scan + comb + corr) * f


def prefill_algorithmic_flops(B, T, H, dk, dv):
    """Chunked-form flops per token-head: 6 C dk + 4 C dv + 6 dk dv."""
    return B * H * T * (6 * C * dk + 4 * C * dv + 6 * dk * dv)


# Sustained load this long before any timed region.  Measured on MI355X: from
# an idle GPU the scan kernel of the 16K step takes ~145 us, rises to ~170 us
# within 4 ms and settles at ~132 us after ~30 ms of back-to-back steps (the
# clocks settle under load); after 50 ms idle the same ramp repeats.
SETTLE_S = 0.1


def settle(torch, fn, min_calls):
    """Untimed warm-up: call fn() at least min_calls times and until SETTLE_S
    seconds of back-to-back work have passed; returns the number of calls."""
    calls, t0 = 0, time.perf_counter()
    while calls < min_calls or time.perf_counter() - t0 < SETTLE_S:
        fn()
        calls += 1
        if calls % 16 == 0:
            torch.cuda.synchronize()      # keep the host at most 16 calls ahead
    torch.cuda.synchronize()
    return calls


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_deltanet_recurrent_delta_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch from committed rocprofv3 counter runs
    (profiles/traffic.json), or None if absent or taken on other sources."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("source_hash") != kernel_source_hash():
        return None
    e = d.get("kernels", {}).get(kernel)
    return None if e is None else e.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on the host cores (before GPU init)
# ---------------------------------------------------------------------------

def _oracle_head(args):
    q, k, v, a, b = args
    from oracle import gdn_oracle as orc
    orc.gdn_head(q, k, v, a, b, None)
    return q.shape[0]


def cpu_baseline(x, T_sample):
    """Oracle over all heads of the prefill workload, first T_sample tokens,
    one worker process per head (fork pool; the GPU is not initialised)."""
    H = x.q.shape[2]
    jobs = [(x.q[0, :T_sample, h], x.k[0, :T_sample, h], x.v[0, :T_sample, h],
             x.alpha[0, :T_sample, h], x.beta[0, :T_sample, h]) for h in range(H)]
    ncpu = len(os.sched_getaffinity(0))
    workers = max(1, min(ncpu, H, 16))
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(workers) as pool:
        toks = sum(pool.map(_oracle_head, jobs))
    dt = time.perf_counter() - t0
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": T_sample / dt, "unit": "tokens/s", "cores": workers,
            "kind": "oracle",
            "sample": f"fp64 numpy token-by-token oracle, all {H} heads of the "
                      f"prefill workload, first {T_sample} tokens "
                      f"({toks} token-heads), one process per head; "
                      f"{dt:.2f} s wall on {workers} of {ncpu} host cores ({model})",
            "seconds": dt}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=512)
    ap.add_argument("--decode-batch", type=int, nargs="+", default=[64, 1],
                    help="decode batch sizes to measure (each at d_k 128 and 64)")
    ap.add_argument("--layers", type=int, default=18)
    ap.add_argument("--skip-prefill", action="store_true",
                    help="omit the 16K prefill step (for per-leg profiling; "
                         "value is then null)")
    ap.add_argument("--skip-decode", action="store_true")
    ap.add_argument("--skip-batched", action="store_true")
    ap.add_argument("--eager-decode", action="store_true",
                    help="launch the decode steps one by one instead of "
                         "replaying a HIP graph (for counter collection)")
    ap.add_argument("--skip-truncated", action="store_true",
                    help="skip the segment-truncated prefill leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=16384)
    a = ap.parse_args(argv)

    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the gated delta rule's heads "
              "are independent, so a multi-GPU run is B/H sharding of this "
              "same kernel with no exchange; --gpus must be 1.",
              file=sys.stderr)
        return 2

    rank = int(os.environ.get("RANK", "0"))
    log("generating the 16K-token prefill workload ...")
    x2 = gi.prefill_16k()
    cpu = None
    if not a.no_cpu_baseline and rank == 0:
        log("timing the fp64 oracle on the host cores ...")
        cpu = cpu_baseline(x2, min(a.cpu_tokens, x2.q.shape[1]))
        log(f"  oracle: {cpu['value']:.0f} tokens/s ({cpu['sample']})")

    import torch
    from gated_deltanet_recurrent_delta_amd import binding as gdn

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    def up(xx):
        dt = torch.bfloat16 if xx.dtype == "bf16" else torch.float32
        return [torch.from_numpy(getattr(xx, n)).to(dev).to(dt).contiguous()
                for n in ("q", "k", "v")] + \
               [torch.from_numpy(getattr(xx, n)).to(dev).contiguous()
                for n in ("alpha", "beta")]

    # ---------------- prefill, 16K tokens (the step) ----------------
    B, T, H, dk = x2.q.shape
    dv = x2.v.shape[-1]
    value = ms_per_step = None
    prefill_info, roof = {}, None
    if not a.skip_prefill:
        q, k, v, al, be = up(x2)
        del x2
        o = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
        ST = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
        ws = torch.empty(gdn.prefill_workspace_bytes(B, T, H, dk, dv),
                         dtype=torch.uint8, device=dev)

        def prefill_step(evs=None):
            if evs is not None:
                evs[0].record(stream)
            gdn.prefill_prepare(q, k, al, be, dv, ws, out_dtype=o.dtype)
            if evs is not None:
                evs[1].record(stream)
            gdn.prefill_scan(q, k, v, None, o, ST, ws)
            if evs is not None:
                evs[2].record(stream)

        warm_calls = settle(torch, prefill_step, a.warmup)
        # per-phase kernel times: eager steps bracketed by events
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
               for _ in range(a.steps)]
        t0 = time.perf_counter()
        for i in range(a.steps):
            prefill_step(evs[i])
        torch.cuda.synchronize()
        eager_wall = time.perf_counter() - t0
        # the timed steps: one step (prepare + scan) captured in a HIP graph,
        # replayed K times
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            prefill_step()
        settle(torch, g.replay, 1)
        t0 = time.perf_counter()
        for i in range(a.steps):
            g.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        del g
        prep_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
        scan_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
        call_ms = prep_ms + scan_ms
        ms_per_step = wall * 1e3 / a.steps
        tokens = B * T
        value = tokens * a.steps / wall
        pbytes = prefill_bytes(B, T, H, dk, dv)
        nseg, seg_chunks = gdn.prefill_segments(B, T, H, dk, dv)
        f_prep, f_scan = prefill_mfma_flops(B, T, H, dk, dv, nseg, seg_chunks)
        log(f"prefill 16K: {ms_per_step * 1e3:.1f} us/step wall (HIP graph), "
            f"{eager_wall * 1e6 / a.steps:.1f} us launched eagerly; events: prepare "
            f"{prep_ms * 1e3:.1f} us, scan {scan_ms * 1e3:.1f} us; "
            f"{value / 1e6:.1f} M tokens/s")
        prefill_info = {
            "timed": "K replays of a HIP graph holding one step (prepare + scan)",
            "untimed_warmup_steps": warm_calls,
            "eager_us_per_step": eager_wall * 1e6 / a.steps,
            "segments": {"per_head": nseg, "chunks_per_segment": seg_chunks},
            "kernels_us": {"prepare_kernel": prep_ms * 1e3,
                           "scan (scan_wide_kernel + segment_combine_kernel + segment_correct_kernel)": scan_ms * 1e3},
            "mfma": {"executed_flops": f_prep + f_scan,
                     "achieved_tflops": (f_prep + f_scan) / (call_ms * 1e-3) / 1e12,
                     "frac_of_bf16_peak": (f_prep + f_scan) / (call_ms * 1e-3) / MFMA_BF16_PEAK,
                     "scan_frac": f_scan / (scan_ms * 1e-3) / MFMA_BF16_PEAK,
                     "prepare_kernel_frac": f_prep / (prep_ms * 1e-3) / MFMA_BF16_PEAK,
                     "algorithmic_flops": prefill_algorithmic_flops(B, T, H, dk, dv)},
        }
        roof = {"bound": "hbm", "kernel": "gdn_prefill (prepare_kernel + scan)",
                "achieved": pbytes / (call_ms * 1e-3) / 1e9,
                "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                "frac": pbytes / (call_ms * 1e-3) / HBM_PEAK,
                "traffic": measured_traffic("prefill"),
                "algorithmic_bytes": pbytes,
                "launch_us": call_ms * 1e3}
        del q, k, v, al, be, o, ws

    # ---------------- decode, B=64 (dk 128, 64) and B=1 ----------------
    decode = {}
    if not a.skip_decode:
        for Bd, dkd in [(bb, dd) for bb in a.decode_batch for dd in (128, 64)]:
            decode[f"B{Bd}_dk{dkd}"] = bench_decode(
                torch, gdn, dev, stream, Bd, dkd, a.decode_steps, a.layers, up,
                eager=a.eager_decode)
    # ---------------- batched prefill, dk 128 vs 64 ----------------
    batched = {}
    if not a.skip_batched:
        for dkb in (128, 64):
            batched[f"dk{dkb}"] = bench_batched(torch, gdn, dev, stream, dkb,
                                                max(3, a.steps // 2), a.warmup, up)
        batched["speedup_dk64_vs_dk128"] = (batched["dk128"]["us_per_call"] /
                                            batched["dk64"]["us_per_call"])
    for bb in a.decode_batch:
        if f"B{bb}_dk128" in decode and f"B{bb}_dk64" in decode:
            decode[f"speedup_dk64_vs_dk128_B{bb}"] = (decode[f"B{bb}_dk128"]["us_per_step"] /
                                                     decode[f"B{bb}_dk64"]["us_per_step"])

    # ---------------- segment-truncated prefill, r in {1, 4, 12, 32} ----------
    truncated = {}
    if not a.skip_truncated:
        truncated = bench_truncated(torch, gdn, dev, stream, up)

    copy_bw = copy_bandwidth(torch, dev, stream)
    log(f"device copy (512 MiB): {copy_bw / 1e9:.0f} GB/s read+write")
    out = {
        "metric": "GDN layer tokens/s (prefill T=16K; decode B=64) + % HBM/MFMA peak",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; no weights or datasets)",
        "config": {"workload": "GDN layer prefill, Qwen3.5-0.8B-shaped: B=1, H=16, "
                               "T=16384, dk=dv=128, bf16 q/k/v/o, fp32 gates/state, "
                               "narrow-cone keys, 10 short / 6 long horizon heads",
                   "B": B, "T": T, "H": H, "dk": dk, "dv": dv, "chunk": C},
        "roofline": roof,
        "prefill": prefill_info,
        "decode": decode,
        "batched_prefill": batched,
        "truncated_prefill": truncated,
        "cpu_baseline": cpu,
        "copy_bandwidth_GBps": copy_bw / 1e9,
        "host": platform.node(),
    }
    if cpu is not None:
        out["cpu_baseline"] = {kk: vv for kk, vv in cpu.items() if kk != "seconds"}
    if rank == 0:
        print(json.dumps(out), flush=True)
    return 0


def copy_bandwidth(torch, dev, stream, nbytes=512 << 20, reps=20):
    """Read + write bytes per second of a plain device-to-device copy
    (torch's copy kernel) of `nbytes`: the achievable streaming rate that
    the HBM-bound kernels are compared with."""
    x = torch.empty(nbytes // 4, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    x.fill_(1.0)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        y.copy_(x)
    e1.record(stream)
    torch.cuda.synchronize()
    return 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3)


def bench_decode(torch, gdn, dev, stream, B, dk, n_steps, layers, up,
                 eager=False):
    """512 decode steps x `layers` state sets, captured in one HIP graph
    (or launched one by one with `eager`, which then times launch gaps
    too)."""
    H, dv = 16, 128
    log(f"decode B={B} dk={dk}: prompt prefill (2048 tokens) ...")
    pr = gi.decode_prompt(B=B, dk=dk)
    q, k, v, al, be = up(pr)
    del pr
    _, S = gdn.prefill(q, k, v, al, be)
    del q, k, v, al, be
    st = gi.decode_steps(B=B, n_steps=n_steps, dk=dk)
    qs, ks, vs, als, bes = [t.transpose(0, 1).contiguous() for t in up(st)]
    del st
    states = [S.clone() for _ in range(layers)]
    o = torch.empty((B, H, dv), dtype=torch.bfloat16, device=dev)

    def one(t, l):
        gdn.decode_step(qs[t], ks[t], vs[t], als[t], bes[t], states[l],
                        S_out=states[l], o=o)

    # warm up (also compiles nothing; checks the path eagerly)
    for l in range(layers):
        one(0, l)
    torch.cuda.synchronize()

    def all_steps():
        for t in range(n_steps):
            for l in range(layers):
                one(t, l)

    if eager:
        replay = all_steps
    else:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            all_steps()
        replay = g.replay
    torch.cuda.synchronize()
    settle(torch, replay, 1)         # untimed passes
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    launches = n_steps * layers
    us = ms * 1e3 / launches
    nbytes = decode_bytes(B, H, dk, dv)
    res = {"us_per_step": us, "tokens_per_s": B / (us * 1e-6),
           "launches_timed": launches, "state_sets": layers,
           "graph": not eager,
           "roofline": {"bound": "hbm", "kernel": "decode_kernel",
                        "achieved": nbytes / (us * 1e-6) / 1e9,
                        "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                        "frac": nbytes / (us * 1e-6) / HBM_PEAK,
                        "traffic": measured_traffic(f"decode_B{B}_dk{dk}"),
                        "algorithmic_bytes": nbytes}}
    log(f"  decode B={B} dk={dk}: {us:.2f} us/step, "
        f"{res['roofline']['achieved']:.0f} GB/s ({100 * res['roofline']['frac']:.1f} % of HBM)")
    del replay, states, qs, ks, vs, als, bes, S
    torch.cuda.empty_cache()
    return res


def bench_batched(torch, gdn, dev, stream, dk, steps, warmup, up):
    x = gi.batched_prefill(dk=dk)
    B, T, H, _ = x.q.shape
    dv = x.v.shape[-1]
    q, k, v, al, be = up(x)
    del x
    o = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
    ST = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    ws = torch.empty(gdn.prefill_workspace_bytes(B, T, H, dk, dv),
                     dtype=torch.uint8, device=dev)
    settle(torch, lambda: gdn.prefill(q, k, v, al, be, o=o, ST=ST, workspace=ws),
           warmup)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        gdn.prefill(q, k, v, al, be, o=o, ST=ST, workspace=ws)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    nbytes = prefill_bytes(B, T, H, dk, dv)
    res = {"us_per_call": us, "tokens_per_s": B * T / (us * 1e-6),
           "roofline": {"bound": "hbm", "achieved": nbytes / (us * 1e-6) / 1e9,
                        "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                        "frac": nbytes / (us * 1e-6) / HBM_PEAK,
                        "traffic": measured_traffic(f"batched_dk{dk}"),
                        "algorithmic_bytes": nbytes}}
    log(f"batched prefill B=8 T=4096 dk={dk}: {us:.1f} us, "
        f"{res['tokens_per_s'] / 1e6:.1f} M tokens/s")
    del q, k, v, al, be, o, ST, ws
    torch.cuda.empty_cache()
    return res


def bench_truncated(torch, gdn, dev, stream, up, ranks=(1, 4, 12, 32),
                    segment=256):
    """Segment-truncated prefill: B=1, H=16, T=16384, dk=dv=128; at each of
    the 63 boundaries between 256-token segments every head's state is
    projected onto its top-r left singular directions.  Each r's whole pass
    (64 prefill calls + 63 truncations) is captured in one HIP graph and
    replayed; r = 128 is the untruncated control.  The truncation alone is
    also timed on the 16 states met at the first boundary."""
    x = gi.truncated_prefill()
    B, T, H, dk = x.q.shape
    dv = x.v.shape[-1]
    q, k, v, al, be = up(x)
    del x
    _, S_b1 = gdn.prefill(q[:, :segment], k[:, :segment], v[:, :segment],
                          al[:, :segment], be[:, :segment])
    ws = torch.empty(gdn.truncate_workspace_bytes(B * H, dv, dk),
                     dtype=torch.uint8, device=dev)
    res = {"workload": f"B={B}, H={H}, T={T}, dk=dv={dk}, bf16 in/out, "
                       f"truncation every {segment} tokens",
           "boundaries": (T - 1) // segment}
    for r in (*ranks, min(dk, dv)):
        def run():
            return gdn.prefill_truncated(q, k, v, al, be, r, segment=segment)
        run()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            _, _, er = run()
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        erv = er.float().cpu().numpy().reshape(-1)
        item = {"ms_per_pass": ms, "tokens_per_s": B * T / (ms * 1e-3),
                "stable_rank_at_T": {"mean": float(np.mean(erv)),
                                     "min": float(np.min(erv)),
                                     "max": float(np.max(erv)),
                                     "per_head": [round(float(e), 3) for e in erv]}}
        if r < min(dk, dv):
            times = []
            for _ in range(5):
                Sx = S_b1.clone()
                torch.cuda.synchronize()
                e0.record(stream)
                gdn.truncate_rank(Sx, r, stable_rank=False, workspace=ws)
                e1.record(stream)
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1))
            item["one_boundary_truncate_us"] = float(np.median(times)) * 1e3
        res[f"r{r}"] = item
        log(f"truncated prefill r={r}: {ms:.2f} ms/pass, er(S_T) mean "
            f"{np.mean(erv):.2f}" + (f", one boundary {item['one_boundary_truncate_us']:.0f} us"
                                     if "one_boundary_truncate_us" in item else ""))
        del g, er
    base = res[f"r{min(dk, dv)}"]["ms_per_pass"]
    for r in ranks:
        res[f"r{r}"]["truncation_ms"] = res[f"r{r}"]["ms_per_pass"] - base
    del q, k, v, al, be, S_b1, ws
    torch.cuda.empty_cache()
    return res


if __name__ == "__main__":
    sys.exit(main())
