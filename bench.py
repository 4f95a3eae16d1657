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

def prefill_bytes(B, T, H, dk, dv, io_bytes=2, with_S0=False, dk_in=None):
    """q, k, v read + o written (io dtype), alpha/beta read (fp32), final
    state written (fp32), initial state read if given.  dk_in: width of the
    raw q/k rows the fused input path reads, default dk."""
    dk_in = dk if dk_in is None else dk_in
    per_tok = io_bytes * (2 * dk_in + 2 * dv) + 8
    state = 4 * dv * dk * (2 if with_S0 else 1)
    return B * H * (T * per_tok + state)


def decode_bytes(B, H, dk, dv, io_bytes=2, dk_in=None):
    """State read + written once (fp32), q, k, v read, o written, gates.
    dk_in: width of the raw q/k rows the fused input path reads (a random
    channel subset touches every cache line of the row), default dk."""
    dk_in = dk if dk_in is None else dk_in
    return B * H * (8 * dv * dk + io_bytes * (2 * dk_in + 2 * dv) + 8)


def prefill_mfma_flops(B, T, H, dk, dv, nseg, seg_chunks):
    """bf16 MFMA flops the prefill kernels execute (bf16 in / bf16 out), from
    their structure; one v_mfma_f32_16x16x32_bf16 = 16384 flops.
      prepare: per chunk and head, 10 lower tiles of K K^T and of Q K^T,
               dk/32 k-steps each (segmented: K K^T only).
      scan:    per chunk and 16-row wave: K S^T 4 x dk/32 x 2 (split state),
               Q S^T 4 x dk/32, T Z 6 k-blocks x 3, P U 6, state update
               dk/16 tiles x 2 k-blocks x 2; transition rows (dk per head)
               run for the chunks of segments >= 1; segmented, the 10
               lower tiles of Q K^T per chunk and head-segment as well.
      combine: per later segment and 16-row wave: dk/16 x dk/32 x 3.
      correct: per chunk of later segments and 16-row wave: 4 x dk/32."""
    nch = -(-T // C)
    nkb, ndt = dk // 32, dk // 16
    f = 16 * 16 * 32 * 2
    prep = B * H * nch * (10 if nseg > 1 else 20) * nkb
    per_wave_chunk = 4 * nkb * 2 + 4 * nkb + 6 * 3 + 6 + ndt * 2 * 2
    later = nch - seg_chunks if nseg > 1 else 0
    scan = B * H * (dv // 16 * nch + dk // 16 * later) * per_wave_chunk
    if nseg > 1:
        scan += B * H * nch * 10 * nkb
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


# Host-only sources (argument checks and dispatch, the host channel
# selection) do not change what a kernel moves; every other source file in
# csrc/ is hashed.
HOST_ONLY_SOURCES = ("gdn_api.hip", "gdn_select.hip")


def kernel_source_hash():
    """Hash of the GPU kernel sources (and their launch code): the counter
    traffic stored in profiles/traffic.json is valid while it is unchanged."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_deltanet_recurrent_delta_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f in HOST_ONLY_SOURCES:
            continue
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
# HBM traffic from rocprofv3 counters (FETCH_SIZE, WRITE_SIZE)
# ---------------------------------------------------------------------------

# Which dispatches belong to which measured launch: kernel name, first
# template argument (d_k), the gather flag where the kernel has one, and the
# grid size (work-items) at the benchmark's shapes.  Kernels of the decode
# prompts (prefills of B=64 or B=1) have other grids and are not counted.
COUNTER_LEGS = {
    # (kernel, d_k, last template argument or None, grid): the last template
    # argument is prepare_kernel's gather flag (0, 1; its third template
    # argument: the segmented prefill's instance, which leaves P to the
    # scan, has a grid of its own), decode_kernel's
    # input-path mode (0 none, 1 norm + scale, 2 channel subset + norm + scale)
    # and scan_kernel's state-storing flag (1 in the backward pass)
    # 16 heads x 16 segments: scan_wide 512 threads per head-segment,
    # combine 8 row groups x 9 waves per head, correction 15 segments x 10
    # waves per head (a B=1 decode prompt's combine has the same grid: count
    # the B=1 decode legs in a run of their own)
    "prefill": [("prepare_kernel", 128, 0, 256 * 16 * 64),
                ("scan_wide_kernel", 128, None, 16 * 16 * 512),
                ("segment_combine_kernel", 128, None, 16 * 8 * 576),
                ("segment_correct_kernel", 128, None, 16 * 15 * 640)],
    "decode_B64_dk128": [("decode_kernel", 128, 0, 64 * 16 * 32 * 64)],
    "decode_B64_dk64": [("decode_kernel", 64, 0, 64 * 16 * 4 * 64)],
    "decode_B1_dk128": [("decode_kernel", 128, 0, 16 * 32 * 64)],
    "decode_B1_dk64": [("decode_kernel", 64, 0, 16 * 32 * 64)],
    "batched_dk128": [("prepare_kernel", 128, 0, 64 * 16 * 8 * 64),
                      ("scan_kernel", 128, 0, 8 * 16 * 2 * 256)],
    "batched_dk64": [("prepare_kernel", 64, 0, 64 * 16 * 8 * 64),
                     ("scan_kernel", 64, 0, 8 * 16 * 2 * 256)],
    "batched_qk_dk64": [("prepare_kernel", 64, 1, 64 * 16 * 8 * 64),
                        ("scan_kernel", 64, 0, 8 * 16 * 2 * 256)],
    "decode_qk_B64_dk64": [("decode_kernel", 64, 2, 64 * 16 * 4 * 64)],
    "batched_qk_norm_dk64": [("prepare_kernel", 64, 0, 64 * 16 * 8 * 64),
                             ("scan_kernel", 64, 0, 8 * 16 * 2 * 256)],
    "decode_qk_norm_B64_dk64": [("decode_kernel", 64, 1, 64 * 16 * 4 * 64)],
    # generalised gates: the recurrent decode (B=64; 8 rows per wave at
    # d_k=128, 32 at d_k=64); the sequence at B=8 in chunked form (prepare: one 256-thread workgroup per
    # (b, h, chunk); scan: one per (b, h, 64 state rows)) and, for
    # comparison, in recurrent form (16 rows per wave)
    "gated_decode_B64_dk128": [("gated_recurrent_kernel", 128, None, 64 * 16 * 16 * 64)],
    "gated_decode_B64_dk64": [("gated_recurrent_kernel", 64, None, 64 * 16 * 4 * 64)],
    "gated_prefill_B8_T4096_dk64": [("gated_prepare_kernel", 64, 0, 8 * 16 * 64 * 256),
                                    ("gated_scan_kernel", 64, None, 8 * 16 * 2 * 256)],
    "gated_recurrent_B8_T4096_dk64": [("gated_recurrent_kernel", 64, None, 8 * 16 * 8 * 64)],
    # backward pass at B=8, T=4096, H=16, d_v=128 in chunked form: the
    # prefill's prepare (same grid as the batched prefill's: count them in
    # runs of their own), the state-storing scan, the reverse chain (64 rows
    # per workgroup) and the chunk kernel (8 waves per (b, h, chunk))
    "backward_B8_T4096_dk128": [("prepare_kernel", 128, 0, 64 * 16 * 8 * 64),
                                ("scan_kernel", 128, 1, 8 * 16 * 2 * 256),
                                ("bwd_chain_kernel", 128, None, 8 * 16 * 2 * 256),
                                ("bwd_chunk_kernel", 128, None, 8 * 16 * 64 * 512)],
    "backward_B8_T4096_dk64": [("prepare_kernel", 64, 0, 64 * 16 * 8 * 64),
                               ("scan_kernel", 64, 1, 8 * 16 * 2 * 256),
                               ("bwd_chain_kernel", 64, None, 8 * 16 * 2 * 256),
                               ("bwd_chunk_kernel", 64, None, 8 * 16 * 64 * 512)],
}


def _legs_in_run(a):
    """The legs a run with these flags times, in the order it runs them."""
    legs = []
    if not a.skip_prefill:
        legs.append("prefill")
    if not a.skip_decode:
        legs += [f"decode_B{b}_dk{d}" for b in a.decode_batch for d in (128, 64)]
    if not a.skip_batched:
        legs += ["batched_dk128", "batched_dk64"]
    if not a.skip_qk:
        legs.append("batched_qk_dk64")
        if not a.qk_gather_only:
            legs.append("batched_qk_norm_dk64")
        if 64 in a.decode_batch:
            legs.append("decode_qk_B64_dk64")
            if not a.qk_gather_only:
                legs.append("decode_qk_norm_B64_dk64")
    if not a.skip_gated:
        if 64 in a.decode_batch:
            legs += ["gated_decode_B64_dk128", "gated_decode_B64_dk64"]
        legs += ["gated_prefill_B8_T4096_dk64", "gated_recurrent_B8_T4096_dk64"]
    if not a.skip_backward:
        legs += ["backward_B8_T4096_dk128", "backward_B8_T4096_dk64"]
    return legs


def _kernel_key(name):
    """(base name, first template int, last template argument as an int, or
    None) of a kernel name as rocprofv3 reports it: demangled ('void
    gdn::prepare_kernel<128, __bf16, true>(...)') or, where its demangler
    gives up, mangled ('_ZN3gdn14prepare_kernelILi128EDF16bLb1EEEv...')."""
    import re
    mm = re.match(r"_ZN3gdn(\d+)", name)
    if mm:
        n = int(mm.group(1))
        base = name[mm.end():mm.end() + n]
        rest = name[mm.end() + n:]
        tmpl = rest.split("EEv", 1)[0] + "E"
        di = re.match(r"ILi(\d+)E", rest)
        last = re.findall(r"L[bi](\d+)E", tmpl)
        if base == "prepare_kernel" and len(last) > 2:
            return base, int(last[0]), int(last[1])      # <dk, type, gather, no-P>
        return (base, int(di.group(1)) if di else None,
                int(last[-1]) if len(last) > 1 or (last and not di) else None)
    m = re.search(r"(\w+)<([^>]*)>", name)
    if not m:
        return re.sub(r"\(.*", "", name).split("::")[-1].strip(), None, None
    args = [x.strip() for x in m.group(2).split(",")]
    dk = int(args[0]) if args and args[0].lstrip("-").isdigit() else None
    tail = args[-1] if len(args) > 1 else ""
    if m.group(1) == "prepare_kernel" and len(args) > 3:
        tail = args[2]                                   # the gather flag
    flag = {"true": 1, "false": 0}.get(tail, int(tail) if tail.isdigit() else None)
    return m.group(1), dk, flag


def _read_counters(path, counter):
    """{dispatch id: (kernel name, grid size, value)} from a rocprofv3
    counter_collection.csv (values of one dispatch summed over its rows)."""
    import csv
    out = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter:
                continue
            d = int(row["Dispatch_Id"])
            name, grid, val = row["Kernel_Name"], int(row["Grid_Size"]), float(row["Counter_Value"])
            if d in out:
                val += out[d][2]
            out[d] = (name, grid, val)
    return out


def summarize_counters(a, fetch_csv, write_csv, out_path=None):
    fetch = _read_counters(fetch_csv, "FETCH_SIZE")
    write = _read_counters(write_csv, "WRITE_SIZE")
    # calibration: the 3 + 20 device copies of 512 MiB that copy_bandwidth()
    # makes at the end of every run (the last 23 copy dispatches; earlier
    # ones are uploads and state clones of other sizes)
    copy_bytes = 512 << 20
    cf = [fetch[d][2] for d in sorted(fetch) if "copyBuffer" in fetch[d][0]][-23:]
    cw = [write[d][2] for d in sorted(write) if "copyBuffer" in write[d][0]][-23:]
    if not cf or not cw:
        raise SystemExit("no device-copy dispatches found for the calibration")
    ffac = copy_bytes / 1024 / float(np.mean(cf))
    wfac = copy_bytes / 1024 / float(np.mean(cw))
    legs = _legs_in_run(a)
    # every (name, dk, flag, grid) key must belong to one leg of this run
    owner = {}
    for leg in legs:
        for spec in COUNTER_LEGS[leg]:
            for other, ospec in owner.items():
                if ospec[0] == spec[0] and ospec[1] == spec[1] and \
                        (spec[2] is None or ospec[2] is None or ospec[2] == spec[2]) and \
                        (spec[3] is None or ospec[3] is None or ospec[3] == spec[3]):
                    raise SystemExit(f"{leg} and {other[0]} share kernel {spec}: run them apart")
            owner[(leg, spec)] = spec

    def match(spec, name, grid):
        base, dk, flag = _kernel_key(name)
        # a flag the demangler garbled (None) matches either value: the
        # legs of one run never differ in the flag alone
        return (base == spec[0] and dk == spec[1] and
                (spec[2] is None or flag is None or flag == spec[2]) and
                (spec[3] is None or grid == spec[3]))

    tpath = out_path or os.path.join(ROOT, "profiles", "traffic.json")
    src = kernel_source_hash()
    data = {}
    if os.path.exists(tpath):
        with open(tpath) as f:
            data = json.load(f)
    if data.get("source_hash") != src:
        data = {"source_hash": src, "kernels": {}}
    data["calibration"] = {"copy_bytes": copy_bytes, "fetch_factor": ffac,
                           "write_factor": wfac, "copy_fetch_kib": float(np.mean(cf)),
                           "copy_write_kib": float(np.mean(cw)),
                           "copy_dispatches": len(cf)}
    for leg in legs:
        parts, total = {}, 0.0
        for spec in COUNTER_LEGS[leg]:
            fv = [v for n, g, v in fetch.values() if match(spec, n, g)]
            wv = [v for n, g, v in write.values() if match(spec, n, g)]
            if not fv or not wv:
                raise SystemExit(f"{leg}: no dispatches of {spec}")
            b = float(np.mean(fv)) * 1024 * ffac + float(np.mean(wv)) * 1024 * wfac
            parts[spec[0]] = {"fetch_kib": float(np.mean(fv)), "write_kib": float(np.mean(wv)),
                              "dispatches": len(fv), "bytes": b}
            total += b
        data["kernels"][leg] = {"hbm_bytes_per_launch": total, "parts": parts}
        log(f"{leg}: {total / 1e6:.1f} MB per launch " +
            ", ".join(f"{k} {v['bytes'] / 1e6:.1f} MB" for k, v in parts.items()))
    with open(tpath, "w") as f:
        json.dump(data, f, indent=1)
    log(f"wrote {tpath} (fetch factor {ffac:.4f}, write factor {wfac:.4f}, sources {src})")
    return 0


def summarize_trace(a, db, last=20):
    """Kernel durations per leg from a rocprofv3 kernel-trace database: for
    every kernel of every selected leg, the number of dispatches, the mean
    over all of them and over the last `last` (the timed region, after the
    warm-up), and the minimum, in microseconds."""
    import sqlite3
    con = sqlite3.connect(db)
    # mangled names from the symbol table (the demangled ones can be garbled)
    rows = con.execute(
        "select s.kernel_name, d.grid_size_x * d.grid_size_y * d.grid_size_z, d.start, d.end "
        "from rocpd_kernel_dispatch d join rocpd_info_kernel_symbol s on d.kernel_id = s.id "
        "order by d.start").fetchall()
    print("| leg | kernel | grid (work-items) | dispatches | mean us | mean of last "
          f"{last} us | min us |")
    print("|---|---|---|---|---|---|---|")
    legs = _legs_in_run(a)

    def matches(spec):
        out = []
        for name, grid, t0, t1 in rows:
            base, dk, flag = _kernel_key(name)
            if (base == spec[0] and dk == spec[1] and
                    (spec[2] is None or flag is None or flag == spec[2]) and
                    (spec[3] is None or grid == spec[3])):
                out.append((t0, t1))
        return out

    for leg in legs:
        for spec in COUNTER_LEGS[leg]:
            d = matches(spec)
            # legs of this run that launch the same kernel at the same grid
            # run one after the other, seconds apart (input generation):
            # split the dispatches at the largest gaps, in leg order
            sharing = [l for l in legs if spec in COUNTER_LEGS[l]]
            if len(sharing) > 1 and len(d) > len(sharing):
                gaps = sorted(range(1, len(d)), key=lambda i: d[i][0] - d[i - 1][1])
                cuts = sorted(gaps[-(len(sharing) - 1):])
                bounds = [0] + cuts + [len(d)]
                i = sharing.index(leg)
                d = d[bounds[i]:bounds[i + 1]]
            d = [(t1 - t0) / 1e3 for t0, t1 in d]
            if not d:
                continue
            g = spec[3] if spec[3] is not None else "-"
            print(f"| {leg} | {spec[0]}<{spec[1]}{'' if spec[2] is None else f', {spec[2]}'}> "
                  f"| {g} | {len(d)} | {np.mean(d):.2f} | {np.mean(d[-last:]):.2f} | {np.min(d):.2f} |")
    return 0


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on the host cores (before GPU init)
# ---------------------------------------------------------------------------

def _oracle_head(args):
    q, k, v, a, b = args
    from oracle import gdn_oracle as orc
    orc.gdn_head(q, k, v, a, b, None)
    return q.shape[0]


def _one_core_oracle(args):
    """Runs in a fresh process with one BLAS/OpenMP thread, pinned to one
    core: the oracle on the given heads, token by token."""
    jobs, core = args
    try:
        os.sched_setaffinity(0, {core})
    except OSError:
        pass
    t0 = time.perf_counter()
    toks = sum(_oracle_head(j) for j in jobs)
    return toks, time.perf_counter() - t0


def cpu_baseline_one_core(x, T_sample, heads=2):
    """The oracle on ONE host core (OPENBLAS_NUM_THREADS = OMP_NUM_THREADS =
    1, a spawned process pinned to one core): `heads` heads of the prefill
    workload, first T_sample tokens; scaled to layer tokens/s (all H heads)."""
    H = x.q.shape[2]
    jobs = [(x.q[0, :T_sample, h], x.k[0, :T_sample, h], x.v[0, :T_sample, h],
             x.alpha[0, :T_sample, h], x.beta[0, :T_sample, h]) for h in range(heads)]
    saved = {kk: os.environ.get(kk) for kk in ("OPENBLAS_NUM_THREADS", "OMP_NUM_THREADS",
                                               "MKL_NUM_THREADS")}
    for kk in saved:
        os.environ[kk] = "1"
    try:
        core = sorted(os.sched_getaffinity(0))[0]
        with mp.get_context("spawn").Pool(1) as pool:
            toks, dt = pool.map(_one_core_oracle, [(jobs, core)])[0]
    finally:
        for kk, vv in saved.items():
            if vv is None:
                os.environ.pop(kk, None)
            else:
                os.environ[kk] = vv
    return {"value": toks / H / dt, "unit": "tokens/s", "cores": 1,
            "token_heads_per_s": toks / dt,
            "sample": f"{heads} of {H} heads, first {T_sample} tokens ({toks} "
                      f"token-heads), one process pinned to one core, "
                      f"OPENBLAS_NUM_THREADS = OMP_NUM_THREADS = 1; {dt:.2f} s; "
                      f"value = token-heads/s / {H} heads",
            "seconds": dt}


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
    ap.add_argument("--skip-qk", action="store_true",
                    help="skip the fused input-path legs (channel subset + "
                         "L2 norm + query scale inside the kernels)")
    ap.add_argument("--skip-gated", action="store_true",
                    help="skip the generalised-gate legs (per-key-channel "
                         "retention, split erase/write gates; recurrent form)")
    ap.add_argument("--qk-gather-only", action="store_true",
                    help="of the fused input-path legs run only those with a "
                         "channel subset (for counter collection: the others "
                         "launch the same kernels at the same grids)")
    ap.add_argument("--skip-backward", action="store_true",
                    help="skip the backward pass leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=16384)
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no benchmark: turn the counter_collection.csv files of "
                         "two rocprofv3 runs of this script (--pmc FETCH_SIZE, "
                         "--pmc WRITE_SIZE; same leg options) into per-launch HBM "
                         "bytes, merged into profiles/traffic.json")
    ap.add_argument("--summarize-trace", metavar="RESULTS_DB",
                    help="no benchmark: print, per measured launch of the legs "
                         "selected by the same options, the kernel durations of a "
                         "rocprofv3 --kernel-trace run of this script (its "
                         "*_results.db) as a markdown table")
    a = ap.parse_args(argv)
    if a.summarize_counters:
        return summarize_counters(a, *a.summarize_counters)
    if a.summarize_trace:
        return summarize_trace(a, a.summarize_trace)

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
        one = cpu_baseline_one_core(x2, min(4096, x2.q.shape[1]))
        log(f"  oracle, one core: {one['value']:.0f} tokens/s ({one['sample']})")
        cpu["one_core"] = {kk: vv for kk, vv in one.items() if kk != "seconds"}

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
                     "algorithmic_flops": prefill_algorithmic_flops(B, T, H, dk, dv),
                     "frac_of_peak_algorithmic": prefill_algorithmic_flops(B, T, H, dk, dv) /
                                                 (call_ms * 1e-3) / MFMA_BF16_PEAK},
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

    # ---------------- the fused input path (raw 128-wide q/k) ----------------
    qk = {}
    if not a.skip_qk:
        variants = ((True,) if a.qk_gather_only else (True, False))
        for name, gth in (("batched_dk64_from128", True), ("batched_dk64_norm", False)):
            if gth not in variants:
                continue
            qk[name] = bench_batched_qk(torch, gdn, dev, stream, max(3, a.steps // 2),
                                        a.warmup, up, gather=gth)
            if "dk64" in batched:
                qk[name]["time_vs_plain_dk64"] = (qk[name]["us_per_call"] /
                                                  batched["dk64"]["us_per_call"])
        if 64 in a.decode_batch:
            for name, gth in (("decode_B64_dk64_from128", True), ("decode_B64_dk64_norm", False)):
                if gth not in variants:
                    continue
                qk[name] = bench_decode(torch, gdn, dev, stream, 64, 64, a.decode_steps,
                                        a.layers, up, eager=a.eager_decode, fused=True,
                                        gather=gth)
                if "B64_dk64" in decode:
                    qk[name]["time_vs_plain_dk64"] = (qk[name]["us_per_step"] /
                                                      decode["B64_dk64"]["us_per_step"])

    # ---------------- generalised gates (chunked and recurrent forms) --------
    gated = {}
    if not a.skip_gated:
        if 64 in a.decode_batch:
            for dkg in (128, 64):
                gated[f"decode_B64_dk{dkg}"] = bench_gated_decode(
                    torch, gdn, dev, stream, 64, dkg, min(a.decode_steps, 64), a.layers, up)
        gated["prefill_B8_T4096_dk64"] = bench_gated_prefill(torch, gdn, dev, stream, up)
        if "dk64" in batched:             # the plain chunked prefill at the same shape
            gated["prefill_B8_T4096_dk64"]["time_vs_plain_chunked"] = (
                gated["prefill_B8_T4096_dk64"]["us_per_call"] / batched["dk64"]["us_per_call"])

    # ---------------- backward pass (chunked form) ----------------
    backward = {}
    if not a.skip_backward:
        for dkb in (128, 64):
            backward[f"B8_T4096_dk{dkb}"] = bench_backward(torch, gdn, dev, stream, up, dk=dkb)
        backward["time_dk64_vs_dk128"] = (backward["B8_T4096_dk64"]["us_per_call"] /
                                          backward["B8_T4096_dk128"]["us_per_call"])
        for dkb in (128, 64):
            if f"dk{dkb}" in batched:       # the forward prefill at the same shape
                backward[f"B8_T4096_dk{dkb}"]["time_vs_forward"] = (
                    backward[f"B8_T4096_dk{dkb}"]["us_per_call"] /
                    batched[f"dk{dkb}"]["us_per_call"])

    # ---------------- segment-truncated prefill, r in {1, 4, 12, 32} ----------
    truncated = {}
    if not a.skip_truncated:
        truncated = bench_truncated(torch, gdn, dev, stream, up)

    # ---------------- DRRQR channel selection (host, calibration time) ----------
    selection = bench_drrqr(gdn)

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
        "fused_input_path": qk,
        "generalised_gates": gated,
        "backward": backward,
        "truncated_prefill": truncated,
        "channel_selection": selection,
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
                 eager=False, fused=False, gather=True):
    """512 decode steps x `layers` state sets, captured in one HIP graph
    (or launched one by one with `eager`, which then times launch gaps
    too).  fused: q/k are raw rows that the kernel normalises (over the
    layer's per-head channel subset of 128-wide rows with `gather`, else
    over the dk-wide rows) before it scales q."""
    H, dv = 16, 128
    tag = f"decode B={B} dk={dk}" + ((" (fused input path, from 128)" if gather else
                                      " (fused input path, norm + scale)") if fused else "")
    log(f"{tag}: prompt prefill (2048 tokens) ...")
    if fused:
        chn = gi.pruning_subsets(3, H, 128, dk) if gather else None
        ch = torch.from_numpy(chn).to(dev) if gather else None
        wid = 128 if gather else dk
        pr = gi.raw_qk(B, 2048, H, wid, dv, gi.seed_for(3, 5), "bf16", channel_idx=chn)
        q, k, v, al, be = up(pr)
        del pr
        _, S = gdn.prefill_qk(q, k, v, al, be, channels=ch, q_scale=dk ** -0.5)
        st = gi.raw_qk(B, n_steps, H, wid, dv, gi.seed_for(3, 6), "bf16", channel_idx=chn)
    else:
        pr = gi.decode_prompt(B=B, dk=dk)
        q, k, v, al, be = up(pr)
        del pr
        _, S = gdn.prefill(q, k, v, al, be)
        st = gi.decode_steps(B=B, n_steps=n_steps, dk=dk)
    del q, k, v, al, be
    qs, ks, vs, als, bes = [t.transpose(0, 1).contiguous() for t in up(st)]
    del st
    states = [S.clone() for _ in range(layers)]
    o = torch.empty((B, H, dv), dtype=torch.bfloat16, device=dev)

    def one(t, l):
        if fused:
            gdn.decode_step_qk(qs[t], ks[t], vs[t], als[t], bes[t], states[l],
                               S_out=states[l], o=o, channels=ch,
                               q_scale=dk ** -0.5, validate=False)
        else:
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
    nbytes = decode_bytes(B, H, dk, dv, dk_in=128 if fused and gather else dk)
    key = (f"decode_qk_B{B}_dk{dk}" if gather else None) if fused else f"decode_B{B}_dk{dk}"
    res = {"us_per_step": us, "tokens_per_s": B / (us * 1e-6),
           "launches_timed": launches, "state_sets": layers,
           "graph": not eager,
           "roofline": {"bound": "hbm", "kernel": "decode_kernel",
                        "achieved": nbytes / (us * 1e-6) / 1e9,
                        "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                        "frac": nbytes / (us * 1e-6) / HBM_PEAK,
                        "traffic": measured_traffic(key) if key else None,
                        "algorithmic_bytes": nbytes}}
    log(f"  {tag}: {us:.2f} us/step, "
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


def bench_batched_qk(torch, gdn, dev, stream, steps, warmup, up, gather=True):
    """The batched prefill (B=8, H=16, T=4096, dv=128) at dk=64 from raw,
    unnormalised q/k rows.  gather: the rows are 128 wide and the prepare
    kernel keeps each head's channel subset (the scan reads the gathered
    copy it writes); else the rows are the 64 kept channels already (the
    projection weights permuted offline).  Either way the kernels normalise
    over the kept channels and fold the norms and a 1/sqrt(64) query scale
    into the chunk products."""
    H, dk = 16, 64
    ch_np = gi.pruning_subsets(4, H, 128, dk) if gather else None
    x = gi.raw_qk(8, 4096, H, 128 if gather else dk, 128, gi.seed_for(4, 5), "bf16",
                  channel_idx=ch_np)
    B, T, _, dk_in = x.q.shape
    dv = x.v.shape[-1]
    q, k, v, al, be = up(x)
    del x
    ch = torch.from_numpy(ch_np).to(dev) if gather else None
    o = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
    ST = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    ws = torch.empty(gdn.prefill_qk_workspace_bytes(B, T, H, dk, dv, torch.bfloat16, gather),
                     dtype=torch.uint8, device=dev)

    def call():
        gdn.prefill_qk(q, k, v, al, be, channels=ch, q_scale=dk ** -0.5, o=o, ST=ST,
                       workspace=ws, validate=False)
    settle(torch, call, warmup)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    nbytes = prefill_bytes(B, T, H, dk, dv, dk_in=dk_in)
    res = {"us_per_call": us, "tokens_per_s": B * T / (us * 1e-6),
           "inputs": (f"raw bf16 q/k [8, 4096, 16, {dk_in}]; "
                      + ("per-head 64-channel subset, " if gather else "")
                      + "L2 norm over the kept channels and q scale 1/8 inside the kernels"),
           "roofline": {"bound": "hbm", "achieved": nbytes / (us * 1e-6) / 1e9,
                        "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                        "frac": nbytes / (us * 1e-6) / HBM_PEAK,
                        "traffic": measured_traffic("batched_qk_dk64") if gather else None,
                        "algorithmic_bytes": nbytes}}
    log(f"batched prefill B=8 T=4096 dk=64 from raw {dk_in}-wide q/k (fused input path"
        f"{', gather' if gather else ', norm + scale'}): "
        f"{us:.1f} us, {res['tokens_per_s'] / 1e6:.1f} M tokens/s")
    del q, k, v, al, be, o, ST, ws
    torch.cuda.empty_cache()
    return res


def bench_drrqr(gdn, n_tokens=8192, d=128, k=64, f=1.1, heads=4):
    """The library's host DRRQR on the calibration matrix of each of `heads`
    heads: raw key and query projections of n_tokens seeded tokens stacked
    ([2 n_tokens, d] fp64), keeping k channels."""
    x = gi.raw_qk(1, n_tokens, heads, d, 8, gi.seed_for(4, 6))
    times, swaps = [], []
    for h in range(heads):
        M = np.concatenate([x.k[0, :, h], x.q[0, :, h]], axis=0).astype(np.float64)
        t0 = time.perf_counter()
        _, sw, rho = gdn.drrqr_select(M, k, f)
        times.append(time.perf_counter() - t0)
        swaps.append(sw)
    res = {"ms_per_head": 1e3 * float(np.median(times)), "swaps": swaps,
           "matrix": f"[{2 * n_tokens}, {d}] fp64 (K and Q samples of one head), k={k}, f={f}",
           "where": "host code in libgdn (calibration time, not a per-token kernel)"}
    log(f"DRRQR channel selection: {res['ms_per_head']:.0f} ms per head ({res['matrix']}), "
        f"trades {swaps}")
    return res


def gated_decode_bytes(B, H, dk, dv, io_bytes=2):
    """State read + written (fp32); q, k, v read and o written (io dtype);
    the per-channel gates alpha, b (fp32, dk each) and w (fp32, dv)."""
    return B * H * (8 * dv * dk + io_bytes * (2 * dk + 2 * dv) + 4 * (2 * dk + dv))


def bench_gated_decode(torch, gdn, dev, stream, B, dk, n_steps, layers, up):
    """Decode steps (T = 1) of the generalised gates over `layers` rotating
    state sets, captured in one HIP graph, like the plain decode leg."""
    H, dv = 16, 128
    x = gi.generic(B, n_steps, H, dk, dv, gi.seed_for(3, 7), "bf16")
    al, bg, wg = gi.gate_vectors(B, n_steps, H, dk, dv, gi.seed_for(3, 8))
    q, k, v, _, _ = [t.transpose(0, 1).contiguous()[:, :, None] for t in up(x)]
    f32 = lambda z: torch.from_numpy(z).to(dev).transpose(0, 1).contiguous()[:, :, None]
    al, bg, wg = f32(al), f32(bg), f32(wg)          # [steps, B, 1, H, *]
    del x
    g0 = torch.Generator(device="cpu").manual_seed(gi.seed_for(3, 9))
    S_init = (0.1 * torch.randn((B, H, dv, dk), generator=g0)).to(dev)
    states = [S_init.clone() for _ in range(layers)]
    del S_init
    o = torch.empty((B, 1, H, dv), dtype=torch.bfloat16, device=dev)

    def one(t, l):
        gdn.gated_recurrent(q[t], k[t], v[t], al[t], bg[t], wg[t], states[l], o=o,
                            ST=states[l])

    for l in range(layers):
        one(0, l)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t in range(n_steps):
            for l in range(layers):
                one(t, l)
    settle(torch, g.replay, 1)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (n_steps * layers)
    nbytes = gated_decode_bytes(B, H, dk, dv)
    res = {"us_per_step": us, "tokens_per_s": B / (us * 1e-6),
           "launches_timed": n_steps * layers, "state_sets": layers, "graph": True,
           "roofline": {"bound": "hbm", "kernel": "gated_recurrent_kernel (T=1)",
                        "achieved": nbytes / (us * 1e-6) / 1e9,
                        "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                        "frac": nbytes / (us * 1e-6) / HBM_PEAK,
                        "traffic": measured_traffic(f"gated_decode_B{B}_dk{dk}"),
                        "algorithmic_bytes": nbytes}}
    log(f"  generalised-gate decode B={B} dk={dk}: {us:.2f} us/step, "
        f"{res['roofline']['achieved']:.0f} GB/s ({100 * res['roofline']['frac']:.1f} % of HBM)")
    del g, states, q, k, v, al, bg, wg
    torch.cuda.empty_cache()
    return res


def bench_gated_prefill(torch, gdn, dev, stream, up, B=8, T=4096, H=16, dk=64, dv=128,
                        calls=3):
    """The generalised gates over whole sequences at the batched prefill's
    shape (dk = 64): the chunked form (gdn_gated_prefill: prepare, then the
    scan) and, for comparison, the recurrent form (gdn_gated_recurrent).
    Reported as time, tokens/s and the HBM rate of the chunked form's
    algorithmic bytes (q, k, v read and o written in bf16; the three gate
    tensors read in fp32; the final state written)."""
    x = gi.generic(B, T, H, dk, dv, gi.seed_for(4, 7), "bf16")
    al, bg, wg = gi.gate_vectors(B, T, H, dk, dv, gi.seed_for(4, 8))
    q, k, v, _, _ = up(x)
    del x
    al, bg, wg = (torch.from_numpy(z).to(dev) for z in (al, bg, wg))
    o = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
    ST = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    ws = torch.empty(gdn.gated_prefill_workspace_bytes(B, T, H, dk, dv), dtype=torch.uint8,
                     device=dev)

    def timed(call):
        settle(torch, call, 1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(calls):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / calls

    us = timed(lambda: gdn.gated_prefill(q, k, v, al, bg, wg, o=o, ST=ST, workspace=ws))
    us_rec = timed(lambda: gdn.gated_recurrent(q, k, v, al, bg, wg, o=o, ST=ST))
    ntok = B * T * H
    nbytes = ntok * (2 * (2 * dk + 2 * dv) + 4 * (2 * dk + dv)) + B * H * dv * dk * 4
    res = {"workload": f"B={B}, T={T}, H={H}, dk={dk}, dv={dv}, bf16 q/k/v/o, fp32 "
                       "per-key-channel retention and erase gate, per-value-channel write gate",
           "form": "chunked (gdn_gated_prefill, bf16 inputs)",
           "us_per_call": us, "tokens_per_s": B * T / (us * 1e-6),
           "algorithmic_bytes": nbytes, "hbm_frac": nbytes / (us * 1e-6) / HBM_PEAK,
           "workspace_bytes": ws.numel(),
           "recurrent_us_per_call": us_rec,
           "speedup_vs_recurrent": us_rec / us,
           "traffic": measured_traffic("gated_prefill_B8_T4096_dk64")}
    log(f"generalised-gate prefill B={B} T={T} dk={dk}: chunked {us:.0f} us "
        f"({res['tokens_per_s'] / 1e6:.2f} M tokens/s, {100 * res['hbm_frac']:.1f} % of HBM), "
        f"recurrent {us_rec:.0f} us")
    del q, k, v, al, bg, wg, o, ST, ws
    torch.cuda.empty_cache()
    return res


def bench_backward(torch, gdn, dev, stream, up, B=8, T=4096, H=16, dk=128, dv=128,
                   calls=3):
    """The backward pass (gradients of q, k, v, alpha, beta and S_0) at the
    batched prefill's shape (d_k = 128, or the pruned 64), bf16 inputs and
    d_o, fp32 gradients, in chunked form (prepare, forward sweep storing
    the chunk-start states, reverse chain of the state gradients, chunk-
    parallel gradients).  Reported as time, tokens/s and the HBM rate of
    its algorithmic bytes (inputs, d_o, dST and S_0 read once; gradients
    written once)."""
    x = gi.generic(B, T, H, dk, dv, gi.seed_for(4, 9), "bf16", S0_scale=0.3)
    d_o, dST = gi.cotangents(B, T, H, dk, dv, gi.seed_for(4, 10), "bf16")
    q, k, v, al, be = up(x)
    S0 = torch.from_numpy(x.S0).to(dev)
    del x
    d_o = torch.from_numpy(d_o).to(dev).to(torch.bfloat16)
    dST = torch.from_numpy(dST).to(dev)
    ws = torch.empty(gdn.backward_workspace_bytes(B, T, H, dk, dv), dtype=torch.uint8,
                     device=dev)
    out = {}

    def call():
        return gdn.backward(q, k, v, al, be, S0, d_o, dST, out=out, workspace=ws)
    out.update(call())
    settle(torch, call, 1)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(calls):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / calls
    ntok = B * T * H
    nbytes = (ntok * (2 * dk + 2 * dv) * 2 + ntok * 8 +        # q, k, v, d_o; alpha, beta
              2 * B * H * dv * dk * 4 +                         # S_0, dST
              ntok * (2 * dk + dv + 2) * 4 + B * H * dv * dk * 4)   # gradients, dS_0
    res = {"workload": f"B={B}, T={T}, H={H}, dk={dk}, dv={dv}, bf16 q/k/v/d_o, "
                       "fp32 gates, S_0, dS_T and gradients",
           "us_per_call": us, "tokens_per_s": B * T / (us * 1e-6),
           "us_per_token_step": us / T, "algorithmic_bytes": nbytes,
           "hbm_frac": nbytes / (us * 1e-6) / HBM_PEAK,
           "workspace_bytes": ws.numel(),
           "form": "chunked (bf16 inputs)",
           "bound": "the two sequential sweeps over the chunks and the chunk kernel's "
                    "split-bf16 MFMA work; the per-chunk states it stores and reads "
                    "back are most of its HBM traffic"}
    # HBM bytes per call from the committed counter runs (the stored chunk
    # states and state gradients included), and the rate they are moved at
    tr = measured_traffic(f"backward_B8_T4096_dk{dk}")
    res["traffic"] = tr
    res["traffic_GBps"] = None if tr is None else tr / (us * 1e-6) / 1e9
    log(f"backward B={B} T={T} H={H} dk={dk} (chunked form): {us:.0f} us, "
        f"{res['tokens_per_s'] / 1e6:.2f} M tokens/s, {us / T * 1e3:.0f} ns per token step, "
        f"{100 * res['hbm_frac']:.1f} % of HBM for its algorithmic bytes")
    del q, k, v, al, be, S0, d_o, dST, ws, out
    torch.cuda.empty_cache()
    return res


def bench_truncated(torch, gdn, dev, stream, up, ranks=(1, 4, 12, 32),
                    segment=256):
    """Segment-truncated prefill: B=1, H=16, T=16384, dk=dv=128; at each of
    the 63 boundaries between 256-token segments every head's state is
    projected onto its top-r left singular directions.  Each r's whole pass
    (64 prefill calls + 63 truncations) is captured in one HIP graph and
    replayed; r = 128 is the untruncated control.  The truncation alone is
    also timed on the 16 states met at the first boundary.

    The workload's inputs have the tiny case's distributions (per-token
    log alpha ~ -U(0.001, 0.1): a horizon of about 20 tokens, so the state
    at T is rebuilt from the last few hundred tokens whatever r is).  The
    same pass is also run on the 16K benchmark step's inputs, whose six
    long-horizon heads (log alpha ~ -U(1e-4, 1e-3)) carry the truncated
    directions across boundaries: there the ranks at T depend on r."""
    res = _truncated_pass(torch, gdn, dev, stream, up, gi.truncated_prefill(), ranks,
                          segment, "tiny-case distributions")
    res["c2_inputs"] = _truncated_pass(
        torch, gdn, dev, stream, up, gi.prefill_16k(), ranks, segment,
        "the 16K benchmark step's inputs (cone keys, 10 short- and 6 long-horizon heads)",
        time_boundary=False)
    return res


def _truncated_pass(torch, gdn, dev, stream, up, x, ranks, segment, inputs,
                    time_boundary=True):
    B, T, H, dk = x.q.shape
    dv = x.v.shape[-1]
    q, k, v, al, be = up(x)
    del x
    ws = None
    if time_boundary:
        _, S_b1 = gdn.prefill(q[:, :segment], k[:, :segment], v[:, :segment],
                              al[:, :segment], be[:, :segment])
        ws = torch.empty(gdn.truncate_workspace_bytes(B * H, dv, dk),
                         dtype=torch.uint8, device=dev)
    res = {"workload": f"B={B}, H={H}, T={T}, dk=dv={dk}, bf16 in/out, "
                       f"truncation every {segment} tokens; {inputs}",
           "boundaries": (T - 1) // segment}
    for r in (*ranks, min(dk, dv)):
        def run():
            return gdn.prefill_truncated(q, k, v, al, be, r, segment=segment)
        run()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            _, S_T, er = run()
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
        # secondary columns of the same final states, from their singular
        # values (host fp64 SVD of the GPU's S_T): the entropy effective rank
        # exp(-sum p log p), p = sigma / sum sigma, and the numerical rank
        # #{sigma_i > sigma_1 * 128 * 2^-23} ("How much of its state does
        # Gated DeltaNet use?", §1)
        sv = np.linalg.svd(S_T.double().cpu().numpy().reshape(-1, dv, dk), compute_uv=False)
        p = sv / np.maximum(sv.sum(axis=1, keepdims=True), 1e-300)
        ent = np.exp(-np.sum(np.where(p > 0, p * np.log(np.where(p > 0, p, 1.0)), 0.0), axis=1))
        nrank = np.sum(sv > sv[:, :1] * 128.0 * 2.0 ** -23, axis=1)

        def stats(x, nd=3):
            return {"mean": float(np.mean(x)), "min": float(np.min(x)),
                    "max": float(np.max(x)), "per_head": [round(float(e), nd) for e in x]}

        item = {"ms_per_pass": ms, "tokens_per_s": B * T / (ms * 1e-3),
                "stable_rank_at_T": stats(erv),
                "entropy_erank_at_T": stats(ent),
                "numerical_rank_at_T": stats(nrank, 0),
                "rank_columns": "stable rank from gdn_truncate_rank's er_out (the "
                                "primary figure); entropy erank and numerical rank "
                                "from a host fp64 SVD of the same S_T"}
        if time_boundary and r < min(dk, dv):
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
        log(f"truncated prefill ({inputs.split(' (')[0]}) r={r}: {ms:.2f} ms/pass, "
            f"er(S_T) mean {np.mean(erv):.2f}, entropy erank {np.mean(ent):.1f}" +
            (f", one boundary {item['one_boundary_truncate_us']:.0f} us"
             if "one_boundary_truncate_us" in item else ""))
        del g, er, S_T
    base = res[f"r{min(dk, dv)}"]["ms_per_pass"]
    for r in ranks:
        res[f"r{r}"]["truncation_ms"] = res[f"r{r}"]["ms_per_pass"] - base
    del q, k, v, al, be, ws
    if time_boundary:
        del S_b1
    torch.cuda.empty_cache()
    return res


if __name__ == "__main__":
    sys.exit(main())
