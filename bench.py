#!/usr/bin/env python3
"""Benchmark of the chunked gated-delta-rule forward pass on one MI355X.

One step = one gdn_chunk_fwd call over the main workload (B=4, H=16, T=8192,
d_k=d_v=128, C=64, bf16 q/k/v, fp32 gates, zero initial state, fp32 final
state), inputs resident in HBM before the timed region.  Prints ONE JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                  [--no-decode] [--no-long] [--no-loop] [--no-gla] [--no-vecgate] [--no-routes]
                  [--pmc-pass]
  python bench.py --summarize-pmc FETCH_DIR WRITE_DIR   (writes the HBM-traffic
                  summary under profiles/ from two rocprofv3 --pmc runs)

Roofline: the dominant (only) kernel of a step is chunk_fwd_pipe_kernel; its
algorithmic bytes per launch are the minimal HBM traffic: read q, k, v
(bf16), alpha, beta (fp32) once, write o (bf16) and the final state (fp32)
once.  Each launch is bracketed by HIP events recorded on the stream the
kernel is launched on; the JSON line gives their mean (used for the
roofline), median, p10 and p90 over the timed launches (default: 10 warm-up
and 100 timed launches).
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MAIN = dict(B=4, H=16, T=8192, d=128, C=64, seed=3)
SETTLE_MS = 60.0
PMC_LAUNCHES = 10   # chunk launches after the clock settling in a --pmc-pass run
DECODE = dict(N=256, H=16, d=128, steps=64, seed=5)
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_chunk_fwd_main.txt")
# Sources whose text identifies a measured kernel: whole files, or
# "file:function" for one function of a file (a kernel's launch code).
KERNEL_SOURCES = ["gdn_common.hpp", "chunk_fwd_pipe.hpp", "gdn_api.hip:launch_chunk_pipe", "gdn_api.hip:seq_map"]
DECODE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_recurrent_step_decode.txt")
DECODE_SOURCES = ["gdn_common.hpp", "recurrent_step.hpp", "gdn_api.hip:launch_step"]


def alg_bytes_main(B, H, T, d):
    tok = B * H * T
    return tok * d * 2 * 3 + tok * 4 * 2 + tok * d * 2 + B * H * d * d * 4


def alg_flops_main(B, H, T, d, C):
    # full C x C tiles: 10*C*d + 6*d^2 per token-head
    return B * H * T * (10 * C * d + 6 * d * d)


def alg_bytes_decode(N, H, d):
    heads = N * H
    return 2 * heads * d * d * 4 + heads * (3 * d * 2 + 2 * 4 + d * 2)


def source_text(entry, read=None):
    """Text of a KERNEL_SOURCES entry: a whole file, or for "file:function"
    the function's definition (from its first line at column 0 to the first
    closing brace at column 0)."""
    f, _, fn = entry.partition(":")
    if read is None:
        with open(os.path.join(ROOT, "gated_deltanet_sequence_amd", "csrc", f), encoding="utf-8") as fh:
            text = fh.read()
    else:
        text = read(f)
    if not fn:
        return text
    m = re.search(r"^\S[^\n]*\b%s\(" % re.escape(fn), text, re.M)
    if m is None:
        raise ValueError("no definition of %s in %s" % (fn, f))
    end = text.index("\n}\n", m.start())
    return text[m.start():end + 3]


def code_only(text):
    """Source text without comments and with whitespace runs collapsed, so
    that a measurement stays tied to the code, not to its comments."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(sources=None, read=None):
    h = hashlib.sha256()
    for e in (sources or KERNEL_SOURCES):
        h.update(code_only(source_text(e, read)).encode("utf-8"))
    return h.hexdigest()[:16]


def read_summary(path, key, sources=None):
    """A value from a committed rocprofv3 --pmc summary, or None when the file
    is missing or was taken on different kernel sources."""
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path, encoding="utf-8") as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.split("(")[0].strip()
    if vals.get("kernel_source_hash") != kernel_source_hash(sources):
        return None
    try:
        return float(vals[key])
    except (KeyError, ValueError):
        return None


def read_traffic(path=None, sources=None):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary (by
    default the main kernel's), or None (see read_summary)."""
    v = read_summary(path or TRAFFIC_FILE, "hbm_bytes_per_launch", sources)
    return None if v is None else int(v)


def main_inputs(torch, dev):
    from gated_deltanet_sequence_amd import inputs
    x = inputs.make_fwd_inputs(MAIN["B"], MAIN["H"], MAIN["T"], MAIN["d"], "bf16",
                               seed=MAIN["seed"], init_state=False)
    xd = {k: (v.to(dev) if v is not None else None) for k, v in x.items()}
    return x, xd


def settle_clocks(torch, step, settle_ms=SETTLE_MS):
    """Run `step` back to back for `settle_ms` of wall time, untimed.

    Coming out of idle, the GPU needs about 20 ms of sustained load before its
    clocks settle: the first 60-80 launches of the main workload run 20-50 %
    slower than the steady state (measured with per-launch HIP events).  The
    steps timed afterwards therefore measure sustained throughput.  Returns
    the number of launches made."""
    n = 0
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < settle_ms:
        for _ in range(10):
            step()
        n += 10
        torch.cuda.synchronize()
    return n


def time_chunk(torch, xd, steps, warmup, settle_ms=SETTLE_MS, spread=True):
    """Settle the clocks, run `warmup` steps, then (with `spread`) `steps`
    launches each bracketed by its own pair of HIP events, for the spread of
    launch times, and finally the timed region: `steps` launches back to back
    between one pair of HIP events.  Per-launch events add a few microseconds
    of stream work between launches, so the timed region has none.  Returns
    the timed region's wall seconds, its event time per launch (ms), the
    per-launch event times (ms) and the outputs."""
    from gated_deltanet_sequence_amd.binding import gdn_chunk_fwd
    B, H, T, d = xd["q"].shape
    o = torch.empty_like(xd["v"])
    sT = torch.empty((B, H, d, d), dtype=torch.float32, device=xd["q"].device)
    stream = torch.cuda.current_stream()

    def step():
        gdn_chunk_fwd(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], None, MAIN["C"],
                      o=o, final_state=sT, stream=stream)

    settle = settle_clocks(torch, step, settle_ms) if settle_ms > 0 else 0
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    kms = []
    if spread:
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        for i in range(steps):
            starts[i].record(stream)
            step()
            ends[i].record(stream)
        torch.cuda.synchronize()
        kms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    time_chunk.settle_launches = settle
    return wall, e0.elapsed_time(e1) / steps, kms, o, sT


LONG = dict(B=1, H=16, T=131072, d=128, seed=4, init_state=True,
            workload="long context: B=1, H=16, T=131072, d_k=d_v=128, C=64, bf16 q/k/v, "
                     "fp32 gates, S0 ~ N(0,0.1)")
LOOP = dict(B=1, H=4, T=8192, d=64, seed=2, init_state=False,
            workload="the pages' loop case: B=1, H=4, T=8192, d_k=d_v=64, C=64, bf16 q/k/v, "
                     "fp32 gates, zero S0")


def time_split(torch, dev, cfg, launches=10):
    """A few-sequence workload through the sequence-split entry point and, for
    comparison, the plain one; mean of `launches` back-to-back launches
    between two events, each after settling the clocks on that entry point."""
    from gated_deltanet_sequence_amd import inputs
    from gated_deltanet_sequence_amd.binding import (gdn_chunk_fwd, gdn_chunk_fwd_split,
                                                     gdn_chunk_fwd_split_workspace)
    B, H, T, d = cfg["B"], cfg["H"], cfg["T"], cfg["d"]
    x = inputs.make_fwd_inputs(B, H, T, d, "bf16", seed=cfg["seed"], init_state=cfg["init_state"])
    xd = {k: (v.to(dev) if v is not None else None) for k, v in x.items()}
    o = torch.empty_like(xd["v"])
    sT = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    need = gdn_chunk_fwd_split_workspace(B, H, T, d, d, 64, torch.bfloat16)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    args = (xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], xd.get("s0"), 64)
    runs = {
        "split": lambda: gdn_chunk_fwd_split(*args, o=o, final_state=sT, workspace=ws, stream=stream),
        "plain": lambda: gdn_chunk_fwd(*args, o=o, final_state=sT, stream=stream),
    }
    alg = B * H * T * (3 * d * 2 + 8 + d * 2) + (2 if cfg["init_state"] else 1) * B * H * d * d * 4
    res = {"workload": cfg["workload"], "alg_bytes": alg, "split_workspace_bytes": need}
    for name, f in runs.items():
        settle_clocks(torch, f)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(launches):
            f()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / launches
        res[name + "_ms"] = ms
        res[name + "_tokens_per_s"] = B * T / (ms * 1e-3)
        res[name + "_hbm_frac"] = alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS
    return res


def time_gla(torch, xd, launches=50):
    """Gated linear attention without the delta rule (gla_chunk_fwd) on the
    main workload's inputs: mean launch time over `launches` back-to-back
    launches between two events, and its HBM-roofline fraction (same
    algorithmic bytes as the main path)."""
    from gated_deltanet_sequence_amd.binding import gla_chunk_fwd
    B, H, T, d = xd["q"].shape
    o = torch.empty_like(xd["v"])
    sT = torch.empty((B, H, d, d), dtype=torch.float32, device=xd["q"].device)
    stream = torch.cuda.current_stream()
    f = lambda: gla_chunk_fwd(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], None, 64,
                              o=o, final_state=sT, stream=stream)
    settle_clocks(torch, f)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(launches):
        f()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / launches
    alg = alg_bytes_main(B, H, T, d)
    return {"workload": "gated linear attention (no delta rule) on the main workload's inputs",
            "ms": ms, "tokens_per_s": B * T / (ms * 1e-3),
            "hbm_frac": alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


def time_vecgate(torch, xd, launches=10):
    """The chunked per-dimension-gate routes on the main workload's q, k, v,
    beta with a gate drawn per token and key dimension (the workloads' gate
    law): mean times of the two-pass route (gdn_chunk_fwd_vecgate_2pass, the
    reported one, with its HBM-roofline fraction; its algorithmic bytes count
    the [B,H,T,d_k] fp32 gate), the single-pass route and the scan route."""
    from gated_deltanet_sequence_amd import inputs
    from gated_deltanet_sequence_amd.binding import (gdn_chunk_fwd_vecgate, gdn_chunk_fwd_vecgate_2pass,
                                                     gdn_chunk_fwd_vecgate_2pass_workspace, gdn_scan_fwd_vecgate,
                                                     gdn_scan_fwd_workspace)
    B, H, T, d = xd["q"].shape
    av = inputs.make_vec_alpha(B, H, T, d, seed=MAIN["seed"] + 200).to(xd["q"].device)
    o = torch.empty_like(xd["v"])
    sT = torch.empty((B, H, d, d), dtype=torch.float32, device=xd["q"].device)
    ws = torch.empty(gdn_scan_fwd_workspace(B, H, T, d, d, torch.bfloat16), dtype=torch.uint8, device=xd["q"].device)
    n2 = gdn_chunk_fwd_vecgate_2pass_workspace(B, H, T, d, d, 32, torch.bfloat16)
    ws2 = torch.empty(n2, dtype=torch.uint8, device=xd["q"].device)
    stream = torch.cuda.current_stream()
    times = {}
    for name, f in (("two_pass", lambda: gdn_chunk_fwd_vecgate_2pass(xd["q"], xd["k"], xd["v"], av, xd["beta"],
                                                                     None, o=o, final_state=sT, workspace=ws2,
                                                                     stream=stream)),
                    ("chunked", lambda: gdn_chunk_fwd_vecgate(xd["q"], xd["k"], xd["v"], av, xd["beta"], None,
                                                              o=o, final_state=sT, stream=stream)),
                    ("scan", lambda: gdn_scan_fwd_vecgate(xd["q"], xd["k"], xd["v"], av, xd["beta"], None,
                                                          o=o, final_state=sT, workspace=ws, stream=stream))):
        settle_clocks(torch, f)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(launches):
            f()
        e1.record(stream)
        torch.cuda.synchronize()
        times[name] = e0.elapsed_time(e1) / launches
    ms = times["two_pass"]
    alg = alg_bytes_main(B, H, T, d) + B * H * T * (d - 1) * 4  # the gate is d_k floats per token, not one
    del av, ws, ws2
    return {"workload": "per-dimension gate, two-pass chunked route (32-token chunks), on the main workload's "
                        "shape: B=4, H=16, T=8192, d_k=d_v=128, bf16 q/k/v, fp32 alpha [B,H,T,d_k]",
            "ms": ms, "tokens_per_s": B * T / (ms * 1e-3), "alg_bytes": alg,
            "hbm_frac": alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "workspace_bytes": n2,
            "single_pass_ms": times["chunked"], "scan_route_ms": times["scan"]}


ROUTES = dict(B=1, H=8, T=16384, d=64, seed=6)


def time_routes(torch, dev, launches=5):
    """The pages' route comparison shape (d=64, 8 heads, 16384 tokens, batch
    1, bf16): the chunked pass (plain and sequence-split), the blocked
    parallel-scan route, and the per-token route (one decode-step launch per
    token).  Mean times."""
    from gated_deltanet_sequence_amd import inputs
    from gated_deltanet_sequence_amd.binding import (gdn_chunk_fwd, gdn_chunk_fwd_split,
                                                     gdn_chunk_fwd_split_workspace, gdn_chunk_fwd_vecgate,
                                                     gdn_chunk_fwd_vecgate_2pass,
                                                     gdn_chunk_fwd_vecgate_2pass_workspace,
                                                     gdn_chunk_fwd_vecgate_split,
                                                     gdn_chunk_fwd_vecgate_split_workspace,
                                                     gdn_recurrent_fwd, gdn_recurrent_step, gdn_scan_fwd,
                                                     gdn_scan_fwd_vecgate, gdn_scan_fwd_workspace)
    B, H, T, d = ROUTES["B"], ROUTES["H"], ROUTES["T"], ROUTES["d"]
    x = inputs.make_fwd_inputs(B, H, T, d, "bf16", seed=ROUTES["seed"])
    xd = {k: (v.to(dev) if v is not None else None) for k, v in x.items()}
    ws = torch.empty(gdn_scan_fwd_workspace(B, H, T, d, d, torch.bfloat16), dtype=torch.uint8, device=dev)
    wsp = torch.empty(max(gdn_chunk_fwd_split_workspace(B, H, T, d, d, 64, torch.bfloat16), 16),
                      dtype=torch.uint8, device=dev)
    wsv = torch.empty(max(gdn_chunk_fwd_vecgate_split_workspace(B, H, T, d, d, 32, torch.bfloat16), 16),
                      dtype=torch.uint8, device=dev)
    ws2 = torch.empty(gdn_chunk_fwd_vecgate_2pass_workspace(B, H, T, d, d, 32, torch.bfloat16),
                      dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    a = (xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], None)
    # the same gates repeated over the key dimension, for the per-dimension-gate routes,
    # and a gate drawn per key dimension (the same law) for the chunked one
    av = xd["alpha"][..., None].expand(-1, -1, -1, d).contiguous()
    avd = inputs.make_vec_alpha(B, H, T, d, seed=ROUTES["seed"] + 100).to(dev)
    res = {"workload": "route comparison: B=1, H=8, T=16384, d_k=d_v=64, bf16 q/k/v, fp32 gates, zero S0"}
    for name, f in (("chunked", lambda: gdn_chunk_fwd(*a, 64, stream=stream)),
                    ("chunked_split", lambda: gdn_chunk_fwd_split(*a, 64, workspace=wsp, stream=stream)),
                    ("scan", lambda: gdn_scan_fwd(*a, workspace=ws, stream=stream)),
                    ("scan_vecgate", lambda: gdn_scan_fwd_vecgate(xd["q"], xd["k"], xd["v"], av, xd["beta"],
                                                                  None, workspace=ws, stream=stream)),
                    ("chunked_vecgate", lambda: gdn_chunk_fwd_vecgate(xd["q"], xd["k"], xd["v"], av, xd["beta"],
                                                                      None, stream=stream)),
                    ("chunked_vecgate_percolumn", lambda: gdn_chunk_fwd_vecgate(xd["q"], xd["k"], xd["v"], avd,
                                                                                xd["beta"], None, stream=stream)),
                    ("chunked_vecgate_split", lambda: gdn_chunk_fwd_vecgate_split(xd["q"], xd["k"], xd["v"], avd,
                                                                                  xd["beta"], None, workspace=wsv,
                                                                                  stream=stream)),
                    ("chunked_vecgate_2pass", lambda: gdn_chunk_fwd_vecgate_2pass(xd["q"], xd["k"], xd["v"], avd,
                                                                                  xd["beta"], None, workspace=ws2,
                                                                                  stream=stream)),
                    # the token loop in one launch, the state in registers
                    ("recurrent_fwd", lambda: gdn_recurrent_fwd(*a, stream=stream))):
        settle_clocks(torch, f)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(launches):
            f()
        e1.record(stream)
        torch.cuda.synchronize()
        res[name + "_ms"] = e0.elapsed_time(e1) / launches
    # per-token route: T launches of the decode step over the B*H heads (token_loop_ms)
    n = B * H
    cols = {nm: [xd[nm][:, :, t].reshape(n, 1, -1).contiguous() for t in range(T)] for nm in ("q", "k", "v")}
    gates = {nm: [xd[nm][:, :, t].reshape(n, 1).contiguous() for t in range(T)] for nm in ("alpha", "beta")}
    state = torch.zeros(n, 1, d, d, dtype=torch.float32, device=dev)
    outs = torch.empty(T, n, 1, d, dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for t in range(T):
        gdn_recurrent_step(cols["q"][t], cols["k"][t], cols["v"][t], gates["alpha"][t], gates["beta"][t],
                           state, o=outs[t], stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    res["token_loop_ms"] = e0.elapsed_time(e1)
    return res


def time_decode(torch, dev, steps_override=None):
    from gated_deltanet_sequence_amd import inputs
    from gated_deltanet_sequence_amd.binding import gdn_recurrent_step
    N, H, d, steps = DECODE["N"], DECODE["H"], DECODE["d"], DECODE["steps"]
    # first, so that the timed decode steps below are the last scalar-gate
    # steps of this shape in a kernel trace
    few = time_few_new_tokens(torch, dev) if steps_override is None else None
    x = inputs.make_decode_inputs(N, H, d, steps, "bf16", seed=DECODE["seed"])
    if steps_override is not None:
        steps = min(steps, steps_override)
    state = x["s0"].to(dev)
    qs = [t.to(dev) for t in x["q"]]
    ks = [t.to(dev) for t in x["k"]]
    vs = [t.to(dev) for t in x["v"]]
    als = [t.to(dev) for t in x["alpha"]]
    bes = [t.to(dev) for t in x["beta"]]
    o = torch.empty((N, H, d), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    # warm-up on a scratch copy, long enough for the clocks to settle, so the
    # timed 64 steps start from S0 on a GPU under sustained load
    scratch = state.clone()
    it = [0]

    def warm():
        t = it[0] % steps
        it[0] += 1
        gdn_recurrent_step(qs[t], ks[t], vs[t], als[t], bes[t], scratch, o=o, stream=stream)

    settle_clocks(torch, warm)
    del scratch
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for t in range(steps):
        gdn_recurrent_step(qs[t], ks[t], vs[t], als[t], bes[t], state, o=o, stream=stream)
        ev[t + 1].record(stream)
    torch.cuda.synchronize()
    per = [ev[t].elapsed_time(ev[t + 1]) for t in range(steps)]
    avg_ms = ev[0].elapsed_time(ev[steps]) / steps
    byts = alg_bytes_decode(N, H, d)
    variants = {} if steps_override is not None else time_decode_variants(torch, dev, x, qs, ks, vs, bes, o)
    if few is not None:
        variants["few_new_tokens"] = few
    return {"workload": "decode: 256 sequences x H=16, d_k=d_v=128, fp32 state [256,16,128,128] "
                        "updated in place, bf16 q/k/v, 64 consecutive steps",
            "tokens_per_s": N / (avg_ms * 1e-3), "ms_per_step": avg_ms,
            "step_ms_median": sorted(per)[steps // 2],
            "alg_bytes_per_step": byts, "achieved_GBs": byts / (avg_ms * 1e-3) / 1e9,
            "hbm_frac": byts / (avg_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            # DRAM bytes per step from the committed rocprofv3 --pmc summary (null when
            # it is missing or was taken on other kernel sources)
            "traffic": read_traffic(DECODE_TRAFFIC_FILE, DECODE_SOURCES),
            **variants}


def time_few_new_tokens(torch, dev, T=8, launches=20):
    """Eight new tokens for each of the decode workload's 256 x 16 sequences
    (a state ~ N(0, 0.1)): the token-by-token pass (gdn_recurrent_fwd), the
    chunked pass and eight decode steps.  Mean times."""
    from gated_deltanet_sequence_amd import inputs
    from gated_deltanet_sequence_amd.binding import gdn_chunk_fwd, gdn_recurrent_fwd, gdn_recurrent_step
    N, H, d = DECODE["N"], DECODE["H"], DECODE["d"]
    x = inputs.make_fwd_inputs_on_device(N, H, T, d, seed=DECODE["seed"] + 200, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(DECODE["seed"] + 201)
    s0 = 0.1 * torch.randn((N, H, d, d), generator=g, device=dev, dtype=torch.float32)
    o = torch.empty_like(x["v"])
    sT = torch.empty_like(s0)
    stream = torch.cuda.current_stream()
    a = (x["q"], x["k"], x["v"], x["alpha"], x["beta"], s0)
    cols = [{nm: x[nm][:, :, t].contiguous() for nm in ("q", "k", "v", "alpha", "beta")} for t in range(T)]
    state = s0.clone()
    ob = torch.empty((N, H, d), dtype=torch.bfloat16, device=dev)

    def steps():
        for c in cols:
            gdn_recurrent_step(c["q"], c["k"], c["v"], c["alpha"], c["beta"], state, o=ob, stream=stream)
    res = {"workload": "%d new tokens for each of 256 sequences x H=16, d_k=d_v=128, bf16 q/k/v, fp32 state "
                       "~ N(0, 0.1)" % T}
    for name, f in (("recurrent_fwd", lambda: gdn_recurrent_fwd(*a, o=o, final_state=sT, stream=stream)),
                    ("chunked", lambda: gdn_chunk_fwd(*a, 64, o=o, final_state=sT, stream=stream)),
                    ("decode_steps", steps)):
        settle_clocks(torch, f)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(launches):
            f()
        e1.record(stream)
        torch.cuda.synchronize()
        res[name + "_ms"] = e0.elapsed_time(e1) / launches
    # the state read and written once, the tokens' q, k, v, alpha, beta read and o written once
    byts = 2 * N * H * d * d * 4 + N * H * T * (3 * d * 2 + 2 * 4 + d * 2)
    res["alg_bytes"] = byts
    res["recurrent_fwd_hbm_frac"] = byts / (res["recurrent_fwd_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS
    return res


def time_decode_variants(torch, dev, x, qs, ks, vs, bes, o, launches=64):
    """The decode steps with a per-dimension gate and without the delta rule on
    the decode workload's shape, each over 64 steps on a copy of S0 (eight
    per-dimension gates drawn once and cycled; the scalar gates of the
    workload)."""
    from gated_deltanet_sequence_amd import inputs
    from gated_deltanet_sequence_amd.binding import gdn_recurrent_step_vecgate, gla_recurrent_step
    N, H, d, steps = DECODE["N"], DECODE["H"], DECODE["d"], DECODE["steps"]
    av = inputs.make_vec_alpha(N, H, 8, d, seed=DECODE["seed"] + 100).to(dev)
    avs = [av[:, :, t].contiguous() for t in range(8)]
    als = [t.to(dev) for t in x["alpha"]]
    stream = torch.cuda.current_stream()
    res = {}
    for name, fn, alphas, gate_bytes in (("vecgate", gdn_recurrent_step_vecgate, avs, N * H * (d - 1) * 4),
                                         ("gla", gla_recurrent_step, als, 0)):
        state = x["s0"].to(dev)
        for t in range(4):
            fn(qs[t], ks[t], vs[t], alphas[t % len(alphas)], bes[t], state, o=o, stream=stream)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(launches):
            t = i % steps
            fn(qs[t], ks[t], vs[t], alphas[t % len(alphas)], bes[t], state, o=o, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / launches
        byts = alg_bytes_decode(N, H, d) + gate_bytes
        res[name + "_step"] = {"ms_per_step": ms, "tokens_per_s": N / (ms * 1e-3),
                               "hbm_frac": byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        del state
    return res


def host_info():
    """The host the CPU figures come from: logical CPUs the OS reports, the CPUs
    this process may run on, and the CPU model name."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {"nproc": os.cpu_count(), "affinity_cpus": affinity, "cpu_model": model}


def cpu_baseline(x, o_gpu, sT_gpu):
    """The fp64 oracle on the host cores over the whole main workload, plus
    the parity of this run's GPU output against it."""
    import numpy as np

    import oracle
    from gated_deltanet_sequence_amd import inputs
    f = inputs.to_f32_numpy
    q, k, v = f(x["q"]), f(x["k"]), f(x["v"])
    a, b = x["alpha"].numpy(), x["beta"].numpy()
    chains = MAIN["B"] * MAIN["H"]
    # the oracle's OpenMP loop runs over the independent sequences
    threads = min(oracle.num_threads(), chains)
    t0 = time.perf_counter()
    ro, rs = oracle.oracle_fwd(q, k, v, a, b, None)
    dt = time.perf_counter() - t0
    go = o_gpu.float().cpu().numpy()
    gs = sT_gpu.cpu().numpy()
    eo = float(np.max(np.abs(go - ro)) / np.max(np.abs(ro)))
    es = float(np.max(np.abs(gs - rs)) / np.max(np.abs(rs)))
    tokens = MAIN["B"] * MAIN["T"]
    res = {"value": tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": "the whole main workload (B=4,H=16,T=8192,d=128: 64 sequences x 8192 "
                     "tokens), fp64 token loop, %.2f s" % dt,
           "seconds": dt}
    res.update(host_info())
    return (res, {"max_rel_err_o": eo, "max_rel_err_final_state": es, "tol": 2e-2,
                  "pass": bool(eo <= 2e-2 and es <= 2e-2)})


def cpu_configs():
    """The oracle timed on the host cores over the other workloads (the pages'
    loop case, the long context and the 64 decode steps; the tiny workload
    too): seconds, tokens/s and the threads its OpenMP loop used."""
    import oracle
    from gated_deltanet_sequence_amd import inputs
    f = inputs.to_f32_numpy
    out = {"host": host_info()}
    for name, cfg, dtype in (("tiny", dict(B=1, H=1, T=256, d=64, seed=1, init_state=False), "f32"),
                             ("loop_case", LOOP, "bf16"), ("long_context", LONG, "bf16")):
        x = inputs.make_fwd_inputs(cfg["B"], cfg["H"], cfg["T"], cfg["d"], dtype, seed=cfg["seed"],
                                   init_state=cfg["init_state"])
        args = (f(x["q"]), f(x["k"]), f(x["v"]), x["alpha"].numpy(), x["beta"].numpy(),
                x["s0"].numpy() if x.get("s0") is not None else None)
        del x
        t0 = time.perf_counter()
        oracle.oracle_fwd(*args)
        dt = time.perf_counter() - t0
        out[name] = {"seconds": dt, "tokens_per_s": cfg["B"] * cfg["T"] / dt,
                     "threads": min(oracle.num_threads(), cfg["B"] * cfg["H"])}
        del args
    N, H, d, steps = DECODE["N"], DECODE["H"], DECODE["d"], DECODE["steps"]
    x = inputs.make_decode_inputs(N, H, d, steps, "bf16", seed=DECODE["seed"])
    state = x["s0"].numpy().astype("float64")
    cols = [(f(x["q"][t]), f(x["k"][t]), f(x["v"][t]), x["alpha"][t].numpy(), x["beta"][t].numpy())
            for t in range(steps)]
    del x
    t0 = time.perf_counter()
    for c in cols:
        oracle.oracle_step(*c, state)
    dt = time.perf_counter() - t0
    out["decode"] = {"seconds": dt, "seconds_per_step": dt / steps, "tokens_per_s": N * steps / dt,
                     "threads": min(oracle.num_threads(), N * H)}
    return out


PMC_TARGETS = {
    # which: (kernel-name test, summary file, kernel sources, title, algorithmic bytes)
    "main": (lambda n: "chunk_fwd" in n, "TRAFFIC_FILE", KERNEL_SOURCES,
             "chunk_fwd_pipe_kernel, main workload (B=4,H=16,T=8192,d=128,C=64, bf16)",
             lambda: alg_bytes_main(MAIN["B"], MAIN["H"], MAIN["T"], MAIN["d"])),
    "decode": (lambda n: "recurrent_step" in n, "DECODE_TRAFFIC_FILE", DECODE_SOURCES,
               "recurrent_step_kernel, decode step (256 sequences x H=16, d=128, fp32 state in place)",
               lambda: alg_bytes_decode(DECODE["N"], DECODE["H"], DECODE["d"])),
}


def summarize_pmc(fetch_dir, write_dir, which="main"):
    """Write the traffic summary of one kernel from two rocprofv3 --pmc runs of
    `bench.py --pmc-pass WHICH` (FETCH_SIZE, then WRITE_SIZE; KiB per
    dispatch).  Each counter is calibrated by what it reads for the plain
    512 MiB device copy the pass makes first."""
    import csv
    is_kernel, out_var, sources, title, alg_fn = PMC_TARGETS[which]
    out_file = globals()[out_var]

    def read(d, counter):
        rows = []
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path, newline="") as fh:
                for r in csv.DictReader(fh):
                    if r.get("Counter_Name") == counter:
                        rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
        rows.sort()
        return [(n, v) for _, n, v in rows]

    out = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = read(d, counter)
        copy = [v for n, v in rows if "gdn::" not in n and v > 100000]
        # the last launches of the pass, after the clocks have settled
        kern = [v for n, v in rows if "gdn::" in n and is_kernel(n)][-PMC_LAUNCHES:]
        if not copy or not kern:
            raise SystemExit("no %s rows for the copy and the %s kernel in %s" % (counter, which, d))
        out[counter] = (max(copy), sum(kern) / len(kern))
    copy_kib = (1 << 29) / 1024.0  # the copy kernel moves 512 MiB each way
    f_fetch = copy_kib / out["FETCH_SIZE"][0]
    f_write = copy_kib / out["WRITE_SIZE"][0]
    fetch_b = out["FETCH_SIZE"][1] * 1024 * f_fetch
    write_b = out["WRITE_SIZE"][1] * 1024 * f_write
    alg = alg_fn()
    lines = [
        "# HBM traffic of %s" % title,
        "# from two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch):",
        "#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d %s -- python3 bench.py --pmc-pass %s" % (fetch_dir, which),
        "#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d %s -- python3 bench.py --pmc-pass %s" % (write_dir, which),
        "# (each pass runs the kernel for %.0f ms to settle the clocks, then %d more launches;" % (SETTLE_MS, PMC_LAUNCHES),
        "#  the figures below average those last %d launches)" % PMC_LAUNCHES,
        "#   python3 bench.py --summarize-pmc %s %s --pmc-kernel %s" % (fetch_dir, write_dir, which),
        "# Each counter is scaled by (512 MiB / what it reads for a plain 512 MiB device copy",
        "# in the same run).",
        "copy_fetch_kib = %.1f" % out["FETCH_SIZE"][0],
        "copy_write_kib = %.1f" % out["WRITE_SIZE"][0],
        "fetch_scale = %.4f" % f_fetch,
        "write_scale = %.4f" % f_write,
        "kernel_fetch_kib = %.1f" % out["FETCH_SIZE"][1],
        "kernel_write_kib = %.1f" % out["WRITE_SIZE"][1],
        "hbm_fetch_bytes = %d" % fetch_b,
        "hbm_write_bytes = %d" % write_b,
        "hbm_bytes_per_launch = %d" % (fetch_b + write_b),
        "algorithmic_bytes_per_launch = %d" % alg,
        "traffic_over_algorithmic = %.3f" % ((fetch_b + write_b) / alg),
        "# kernel_source_hash: sha256 (first 16 hex digits) of the code (comments and whitespace runs removed) of %s"
        % ", ".join(sources),
        "kernel_source_hash = %s" % kernel_source_hash(sources),
    ]
    with open(out_file, "w", encoding="utf-8") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# Instruction counters of the main chunk kernel, one rocprofv3 --pmc run per
# group (each group within one pass's hardware counter limits).
ACTIVITY_GROUPS = (("MfmaUtil", "MfmaFlopsBF16"),
                   ("SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE"))
ACTIVITY_FILE = os.path.join(ROOT, "profiles", "activity_chunk_fwd_main.txt")


def summarize_activity(dirs):
    """Write the MFMA and LDS activity summary of the main chunk kernel from
    rocprofv3 --pmc runs of `bench.py --pmc-pass main`, one per group of
    ACTIVITY_GROUPS: each counter averaged over the last launches of the pass."""
    import csv
    vals = {}
    for d in dirs:
        rows = []
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path, newline="") as fh:
                for r in csv.DictReader(fh):
                    if "gdn::" in r["Kernel_Name"] and "chunk_fwd" in r["Kernel_Name"]:
                        rows.append((int(r["Dispatch_Id"]), r["Counter_Name"], float(r["Counter_Value"])))
        by = {}
        for disp, name, v in rows:
            by.setdefault(name, {}).setdefault(disp, 0.0)
            by[name][disp] += v
        for name, per in by.items():
            last = [per[k] for k in sorted(per)][-PMC_LAUNCHES:]
            vals[name] = sum(last) / len(last)
    missing = [c for g in ACTIVITY_GROUPS for c in g if c not in vals]
    if missing:
        raise SystemExit("no rows for %s in %s" % (", ".join(missing), " ".join(dirs)))
    B, H, T, d, C = MAIN["B"], MAIN["H"], MAIN["T"], MAIN["d"], MAIN["C"]
    alg_f = alg_flops_main(B, H, T, d, C)
    lines = ["# MFMA and LDS activity of chunk_fwd_pipe_kernel, main workload (B=4,H=16,T=8192,d=128,C=64, bf16)",
             "# from rocprofv3 --pmc runs of bench.py --pmc-pass main (the kernel for %.0f ms to settle" % SETTLE_MS,
             "# the clocks, then %d more launches; each figure is the mean over those last launches):" % PMC_LAUNCHES]
    for g, d_ in zip(ACTIVITY_GROUPS, dirs):
        lines.append("#   rocprofv3 --pmc %s --output-format csv -d %s -- python3 bench.py --pmc-pass main"
                     % (" ".join(g), d_))
    lines.append("#   python3 bench.py --summarize-activity %s" % " ".join(dirs))
    for g in ACTIVITY_GROUPS:
        for c in g:
            lines.append("%s = %.1f" % (c, vals[c]))
    lines += [
        "# derived",
        "mfma_bf16_flops_per_launch = %d" % vals["MfmaFlopsBF16"],
        "algorithmic_flops_per_launch = %d  (full C x C tiles)" % alg_f,
        "mfma_flops_over_algorithmic = %.3f" % (vals["MfmaFlopsBF16"] / alg_f),
        "mfma_busy_percent_of_simd_cycles = %.1f  (MfmaUtil)" % vals["MfmaUtil"],
        "flops_per_mfma_instruction = %.0f" % (vals["MfmaFlopsBF16"] / vals["SQ_INSTS_MFMA"]),
        "valu_instructions_per_mfma = %.2f  (SQ_INSTS_VALU counts MFMAs too)"
        % (vals["SQ_INSTS_VALU"] / vals["SQ_INSTS_MFMA"]),
        "lds_bank_conflict_cycles_over_lds_active = %.3f" % (vals["SQ_LDS_BANK_CONFLICT"] / vals["SQ_LDS_IDX_ACTIVE"]),
        "# kernel_source_hash: sha256 (first 16 hex digits) of the code (comments and whitespace runs removed) of %s"
        % ", ".join(KERNEL_SOURCES),
        "kernel_source_hash = %s" % kernel_source_hash(KERNEL_SOURCES),
    ]
    with open(ACTIVITY_FILE, "w", encoding="utf-8") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_trace(trace_dir, out_name, command, note="", tail=100):
    """Write profiles/OUT_NAME.txt from a rocprofv3 --kernel-trace run: for every
    kernel of the library and launch shape, the number of launches and the
    mean, min and max duration, and the mean over the last `tail` launches
    (the timed ones, when the run is bench.py's).  For the main chunk kernel
    (256 workgroups) and the decode kernel it adds the fraction of the 8 TB/s
    HBM peak that their algorithmic bytes give at that mean."""
    import collections
    import csv
    paths = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not paths:
        raise SystemExit("no *kernel_trace.csv under %s" % trace_dir)
    rows = []
    for p in paths:
        with open(p, newline="") as fh:
            rows += list(csv.DictReader(fh))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    groups = collections.OrderedDict()
    for r in rows:
        name = r["Kernel_Name"]
        if "gdn::" not in name:
            continue
        short = name.split("(")[0].replace("void ", "")
        wg = int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"])
        key = (short, wg, int(r["Workgroup_Size_X"]))
        groups.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    out = ["# rocprofv3 kernel-trace summary (one MI355X); repository root as $REPO:",
           "#   %s" % command,
           "#   python3 bench.py --summarize-trace <that -d directory> %s --trace-cmd '<the command above>'%s"
           % (out_name, (" --tail %d" % tail) if tail != 100 else "")]
    out += ["# " + line for line in note.splitlines() if line.strip()]
    out.append("# per kernel and launch shape: launches, mean, min and max duration, and the mean of")
    out.append("# the last %d launches of that shape (us)" % tail)
    out.append("%-72s %6s %7s %8s %10s %10s %10s %10s" % ("kernel", "wgs", "threads", "launches",
                                                        "mean_us", "min_us", "max_us", "tail_us"))
    derived = []
    for (k, wg, th), v in groups.items():
        t = v[-tail:]
        tmean = sum(t) / len(t)
        out.append("%-72s %6d %7d %8d %10.2f %10.2f %10.2f %10.2f" % (
            k[:72], wg, th, len(v), sum(v) / len(v) / 1e3, min(v) / 1e3, max(v) / 1e3, tmean / 1e3))
        alg = None
        if "chunk_fwd_pipe_kernel<false, true, 4>" in k and wg == 256:
            alg, what = alg_bytes_main(MAIN["B"], MAIN["H"], MAIN["T"], MAIN["d"]), "main workload"
        elif "recurrent_step_kernel" in k and wg == DECODE["N"] * DECODE["H"]:
            # the last template argument is the gate kind: 0 scalar, 1 per
            # dimension (dk - 1 more gate floats per head), 2 no delta rule
            alg, what = alg_bytes_decode(DECODE["N"], DECODE["H"], DECODE["d"]), "decode step"
            if k.endswith(", 1>"):
                alg += DECODE["N"] * DECODE["H"] * (DECODE["d"] - 1) * 4
                what = "decode step, per-dimension gate"
            elif k.endswith(", 2>"):
                what = "decode step, gated linear attention"
        if alg is not None:
            derived += ["roofline of %s (%s, %d wgs): tail_average_ns = %d" % (k, what, wg, tmean),
                        "  algorithmic_bytes_per_launch = %d" % alg,
                        "  algorithmic_GBps_at_tail_average = %.1f" % (alg / tmean),
                        "  fraction_of_8000_GBps = %.4f" % (alg / tmean / 8000.0)]
    out += derived
    path = os.path.join(ROOT, "profiles", out_name + ".txt")
    with open(path, "w", encoding="utf-8") as fh:
        fh.write("\n".join(out) + "\n")
    print("\n".join(out))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the long-context (sequence-split) report")
    ap.add_argument("--no-loop", action="store_true",
                    help="skip the loop-case (sequence-split) report")
    ap.add_argument("--no-gla", action="store_true",
                    help="skip the gated-linear-attention report")
    ap.add_argument("--no-vecgate", action="store_true",
                    help="skip the per-dimension-gate route on the main workload's shape")
    ap.add_argument("--no-routes", action="store_true",
                    help="skip the chunked / scan / per-token route comparison")
    ap.add_argument("--pmc-pass", nargs="?", const="main", choices=sorted(PMC_TARGETS),
                    help="one 512 MiB copy, then the kernel (main chunk kernel, or the decode "
                         "step) for the settling time and %d more launches, for rocprofv3 --pmc "
                         "runs" % PMC_LAUNCHES)
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--pmc-kernel", default="main", choices=sorted(PMC_TARGETS))
    ap.add_argument("--summarize-activity", nargs=len(ACTIVITY_GROUPS), metavar="PMC_DIR",
                    help="write the MFMA / LDS activity summary from one --pmc run per counter group")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "OUT_NAME"),
                    help="write profiles/OUT_NAME.txt from a rocprofv3 --kernel-trace run")
    ap.add_argument("--trace-cmd", default="", help="the profiling command, for the summary header")
    ap.add_argument("--trace-note", default="", help="extra header lines for the summary")
    ap.add_argument("--tail", type=int, default=100, help="launches averaged per shape (--summarize-trace)")
    ap.add_argument("--cpu-configs", action="store_true",
                    help="also time the oracle on the other workloads (loop case, long context, decode)")
    args = ap.parse_args()

    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, which=args.pmc_kernel)
        return
    if args.summarize_activity:
        summarize_activity(args.summarize_activity)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace, command=args.trace_cmd, note=args.trace_note,
                        tail=args.tail)
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: there is no multi-GPU path here "
              "(each (batch, head) sequence is independent, so the work would shard by sequence)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    x, xd = main_inputs(torch, dev)

    if args.pmc_pass:
        src = torch.empty(1 << 28, dtype=torch.float16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        del src, dst
        if args.pmc_pass == "main":
            time_chunk(torch, xd, steps=PMC_LAUNCHES, warmup=0, spread=False)
        else:
            time_decode(torch, dev, steps_override=PMC_LAUNCHES)
        torch.cuda.synchronize()
        print("pmc pass done", flush=True)
        return

    wall, avg_k, kms, o, sT = time_chunk(torch, xd, args.steps, args.warmup)
    B, H, T, d, C = MAIN["B"], MAIN["H"], MAIN["T"], MAIN["d"], MAIN["C"]
    tokens = B * T
    ms_per_step = wall * 1e3 / args.steps
    ks = sorted(kms)

    def pct(q):
        return ks[min(len(ks) - 1, int(round(q * (len(ks) - 1))))]
    alg_b = alg_bytes_main(B, H, T, d)
    alg_f = alg_flops_main(B, H, T, d, C)
    achieved = alg_b / (avg_k * 1e-3) / 1e9
    res = {
        "metric": "tokens/s chunked GDN fwd (H16,d128,T8K) + % MFMA/HBM roofline",
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded: q,k ~N(0,1) L2-normalised, v ~N(0,1), "
                "alpha=exp(-softplus(N(0,1))), beta=sigmoid(N(0,1)))",
        "config": {"workload": "main: B=4, H=16, T=8192, d_k=d_v=128, C=64, bf16 q/k/v, "
                               "fp32 alpha/beta, zero initial state, fp32 final state",
                   "B": B, "H": H, "T": T, "d": d, "chunk_size": C},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": read_traffic(),
                     "kernel": "chunk_fwd_pipe_kernel", "alg_bytes_per_launch": alg_b,
                     # event time of the timed region per launch (back to back)
                     "avg_launch_ms": avg_k, "timed_launches": args.steps,
                     # spread: the same number of launches, each between its own events
                     "launch_ms_median": pct(0.5), "launch_ms_p10": pct(0.1),
                     "launch_ms_p90": pct(0.9), "launch_ms_mean": sum(kms) / len(kms),
                     "mfma_achieved_TFLOPs": alg_f / (avg_k * 1e-3) / 1e12,
                     "mfma_frac": alg_f / (avg_k * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                     # rocprofv3 counters (profiles/activity_chunk_fwd_main.txt; None once the
                     # kernel sources differ from those the counters were taken on)
                     "mfma_busy_pct_counter": read_summary(ACTIVITY_FILE, "mfma_busy_percent_of_simd_cycles"),
                     "mfma_bf16_flops_counter": read_summary(ACTIVITY_FILE, "mfma_bf16_flops_per_launch")},
        "token_heads_per_s": B * H * T / (ms_per_step * 1e-3),
    }
    if not args.no_decode:
        res["decode"] = time_decode(torch, dev)
    if not args.no_long:
        res["long_context"] = time_split(torch, dev, LONG)
    if not args.no_loop:
        res["loop_case"] = time_split(torch, dev, LOOP, launches=100)
    if not args.no_gla:
        res["gla"] = time_gla(torch, xd)
    if not args.no_vecgate:
        res["vecgate"] = time_vecgate(torch, xd)
    if not args.no_routes:
        res["routes"] = time_routes(torch, dev)
    if not args.no_cpu_baseline:
        res["cpu_baseline"], res["parity"] = cpu_baseline(x, o, sT)
    if args.cpu_configs:
        res["cpu_oracle_other_workloads"] = cpu_configs()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
