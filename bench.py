"""Benchmark: loop-query tokens/s of loop-aware attention on one MI355X.

Default workload: the largest single-GPU configuration, Ouro-shaped paged decode with
split-K (32 sequences, 24 core layers x 4 loops, 16 heads x 128, bf16, context 8192,
16-token pages behind shuffled block tables, 8 splits merged by log-sum-exp; all 96
(layer, loop) planes resident, 206 GB).  One step runs every core layer at every loop
as its own attention call, loop-major, as a looped model's sequential loops require;
it yields batch * q * loops loop-query tokens.  Inputs are resident in HBM before
timing starts.  Without --workload the same run then times the Huginn-shaped RIPE
decode (the other configuration with a bandwidth target) and reports it under
"secondary".

Prints one JSON line with the throughput, the roofline of the attention kernel
(algorithmic bytes per launch / mean launch time from HIP events recorded
around each launch on the launch stream) and the fp64 oracle's throughput on a
bounded sample of the same workload on the host cores.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload W] [--policy full|ripe] [--also W,...]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "loop-query tokens/s + achieved HBM GB/s (% of MI355X peak), looped-KV attention"
# Sources of each workload's timed attention kernel (with the shared device headers): the
# counter summary in profiles/ holds their hash, together with the compiler flags, and is
# ignored once any of them changes.
_CSRC = "verify_attention_loop_amd/csrc/"
_COMMON = [_CSRC + "device.hpp", _CSRC + "params.hpp"]
KERNEL_SOURCES = {
    "tiny": [_CSRC + "decode.hip", _CSRC + "attn_common.hpp"] + _COMMON,
    "huginn_ripe": [_CSRC + "decode.hip", _CSRC + "attn_common.hpp"] + _COMMON,
    "ouro_splitk": [_CSRC + "decode.hip", _CSRC + "attn_common.hpp"] + _COMMON,
    "huginn_verify": [_CSRC + "verify.hip"] + _COMMON,
    "huginn_draft": [_CSRC + "decode.hip", _CSRC + "attn_common.hpp"] + _COMMON,
    "loopkv_cells": [_CSRC + "cell.hip", _CSRC + "attn_common.hpp"] + _COMMON,
    "raven_ripe": [_CSRC + "gqa.hip", _CSRC + "attn_common.hpp"] + _COMMON,
    "dory_lastloop": [_CSRC + "gqa.hip", _CSRC + "attn_common.hpp"] + _COMMON,
}
# The timed attention kernel of each workload (rocprofv3 kernel name prefix).
KERNEL_NAME = {"tiny": "decode_kernel", "huginn_ripe": "decode_kernel", "ouro_splitk": "decode_kernel", "huginn_verify": "verify_kernel",
               "huginn_draft": "decode_kernel",
               "loopkv_cells": "cell_kernel", "raven_ripe": "gqa_decode_kernel", "dory_lastloop": "gqa_decode_kernel"}


def kernel_hash(workload: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[workload]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    from verify_attention_loop_amd import build as _build  # flags only; compiles nothing
    flags = [f for f in _build.flags() if f != "-I" and not os.path.isabs(f)]  # no include paths
    h.update(" ".join(flags).encode())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None,
                    choices=["huginn_ripe", "ouro_splitk", "huginn_verify", "huginn_draft", "loopkv_cells",
                             "raven_ripe", "dory_lastloop", "tiny"])
    ap.add_argument("--split-k", type=int, default=-1, help="splits per row (-1: the workload's, 0: library's)")
    ap.add_argument("--waves", type=int, default=0, help="waves per workgroup (0: the library's choice)")
    ap.add_argument("--policy", choices=["default", "full", "ripe"], default="default",
                    help="cache policy of a plain workload (default: the workload's own; the verify configuration "
                         "names both the full-depth cache and the RIPE window)")
    ap.add_argument("--layers", type=int, default=0, help="distinct layers held in HBM (0: all)")
    ap.add_argument("--batch", type=int, default=0,
                    help="sequences per call (0: the workload's); other batches report no traffic figure")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true", help="skip the streaming-read probe")
    ap.add_argument("--event-every", type=int, default=8,
                    help="record HIP events around one launch in this many (rotating over the calls, so every "
                         "(layer, loop) call is sampled); event markers on every launch add ~7%% to the step time")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--v-rule", choices=["fixed", "running"], default="fixed",
                    help="quantised cells: the workload's fixed hot rule (s >= m0 - 4) or the running-maximum rule")
    ap.add_argument("--v-tau", type=float, default=14.0, help="tau of the running-maximum rule")
    ap.add_argument("--v-offset", type=float, default=4.0,
                    help="fixed rule's offset: a far token is hot iff its score >= m0 - offset (the workload: 4.0)")
    ap.add_argument("--ripen", choices=["workload", "paper"], default="workload",
                    help="ripening planes (Huginn-shaped workloads): the workload's noise 0.88^(R-1-r) on plane r, or "
                         "0.88^(r+1), the RIPE page's direction (values only: no byte count or plane read changes)")
    ap.add_argument("--also", default="auto",
                    help="workloads timed after the first one in the same run, reported under 'secondary' "
                         "(comma-separated; 'auto': huginn_ripe when no --workload is given, else none; 'none')")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration under rocprofv3)")
    return ap.parse_args()


def build_workload(w, args):
    import harness
    layers = list(range(w.n_layers if args.layers <= 0 else min(args.layers, w.n_layers)))
    # the draft workload's cache takes blocks of draft_passes + 1 tokens (the verify block)
    max_block = w.extra["draft_passes"] + 1 if "draft_passes" in w.extra else None
    built = harness.build_plain(w, layers=layers, max_block=max_block)
    return built, layers


def host_info() -> str:
    """The host CPU the oracle ran on: model name and logical CPUs visible to this process."""
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return f"{model}; {len(os.sched_getaffinity(0))} logical CPUs available"


def cpu_baseline(w, seconds: float):
    """The fp64 oracle, as it stands, on a bounded sample of the workload: rows of (seq, layer 0, loop,
    head) with their own and deepest planes regenerated on the host; the sample repeats until `seconds`
    of oracle time accumulate.  Input generation is not timed."""
    import numpy as np

    import harness
    import oracle
    import synth

    R = w.n_loops
    pol = oracle.RIPE if w.policy == "ripe" else oracle.FULL
    rng = np.random.default_rng(0)
    n_rows = 24
    draft = "draft_passes" in w.extra
    # a draft row (the middle pass, 4 draft tokens): cached positions through the draft window, the block from
    # the draft streams
    dl = 4 if draft else 0
    window = w.extra["draft_window"] if draft else w.window
    L = w.length + dl
    q = np.empty((n_rows, w.head_dim))
    ko = np.empty((n_rows, L, w.head_dim))
    vo, kd, vd = np.empty_like(ko), np.empty_like(ko), np.empty_like(ko)
    loops = np.empty(n_rows, dtype=np.int32)
    for i in range(n_rows):
        b, h = int(rng.integers(w.batch)), int(rng.integers(w.n_heads))
        r = int(rng.integers(w.extra["draft_loops"] if draft else R))
        hk = h // (w.n_heads // w.hkv)  # the query head's KV head
        loops[i] = r
        ko[i] = harness.cpu_values(w, synth.T_K, b, 0, r, hk, L)
        vo[i] = harness.cpu_values(w, synth.T_V, b, 0, r, hk, L)
        if pol == oracle.RIPE and r != R - 1:
            kd[i] = harness.cpu_values(w, synth.T_K, b, 0, R - 1, hk, L)
            vd[i] = harness.cpu_values(w, synth.T_V, b, 0, R - 1, hk, L)
        else:
            kd[i], vd[i] = ko[i], vo[i]
        if draft:
            ko[i, w.length:] = harness.cpu_draft_values(w, synth.T_DRAFTK, b, 0, r, hk, w.length, dl)
            vo[i, w.length:] = harness.cpu_draft_values(w, synth.T_DRAFTV, b, 0, r, hk, w.length, dl)
        q[i] = harness.cpu_query(w, b, 0, r, h, L - 1)
    t = np.full(n_rows, L - 1, dtype=np.int32)
    t0 = np.full(n_rows, L - 1 - (dl - 1 if draft else 0), dtype=np.int32)
    done, elapsed = 0, 0.0
    while elapsed < seconds:
        t1 = time.perf_counter()
        oracle.attend_rows(q, ko, vo, kd, vd, t, t0, loops, pol, R, window)
        elapsed += time.perf_counter() - t1
        done += n_rows
    rows_per_s = done / elapsed
    cores = oracle.threads()
    # the same rows on one core, for about a fifth of the time
    prev = oracle.set_threads(1)
    done1, elapsed1 = 0, 0.0
    try:
        while elapsed1 < seconds / 5:
            t1 = time.perf_counter()
            oracle.attend_rows(q, ko, vo, kd, vd, t, t0, loops, pol, R, window)
            elapsed1 += time.perf_counter() - t1
            done1 += n_rows
    finally:
        oracle.set_threads(prev)
    rows_per_token = w.n_layers * w.n_heads  # one loop-query token = every layer and head of one (seq, loop)
    return {"value": rows_per_s / rows_per_token, "unit": "loop-query tokens/s", "cores": cores,
            "kind": "oracle", "host": host_info(),
            "one_core": {"value": done1 / elapsed1 / rows_per_token, "seconds": round(elapsed1, 1),
                         "row_ms": round(1e3 * elapsed1 / done1, 3)},
            "sample": f"{done} rows ({n_rows} distinct (seq, layer 0, loop, head) rows of the {w.name} workload, "
                      f"L={L}, d={w.head_dim}, repeated) in {elapsed:.1f} s of fp64 oracle time; "
                      f"{rows_per_token} rows = 1 loop-query token"}


def probe_regions(nbytes: int, total: int, chunk: int):
    """(n, m): launches of n bytes (nbytes rounded down to the chunk, at least one chunk, at most half the
    buffer) over m regions of the buffer (m n <= total), with m n >= 768 MB where 64 regions allow it."""
    n = min(total // 2, max(chunk, nbytes // chunk * chunk))
    m = min(total // n, max(2, -(-(768 << 20) // n)), 64)
    return n, m


class ReadProbe:
    """Achievable HBM read rate of a launch of n bytes: the library's streaming-read probe (lkv_probe_read:
    16-byte nontemporal loads, as the page streams use), timed with the same launch-stamped events as the
    sampled attention launches.  The probe buffer (8 GiB) is allocated before the workload, as a fresh
    allocation, so its placement does not depend on what the workload allocated and freed.  Launch i reads
    region i mod m of the buffer, with m regions spanning at least 768 MB where n allows, so no launch finds
    its bytes in the 256 MB Infinity Cache."""

    TOTAL = 8 << 30

    def __init__(self):
        import torch

        self.buf = torch.empty(self.TOTAL, dtype=torch.uint8, device="cuda")
        self.sink = torch.zeros(1, dtype=torch.int32, device="cuda")

    def rate(self, nbytes: int, reps: int = 15):
        """(bytes per launch, GB/s) for launches of about nbytes (rounded down to the probe's chunk), from the
        median launch."""
        import numpy as np
        import torch

        import verify_attention_loop_amd as vla

        n, m = probe_regions(nbytes, self.TOTAL, vla.PROBE_CHUNK)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in evs:
            a.record()  # torch creates the underlying HIP event on its first record
            b.record()
        for i in range(m + 1):  # every region once before timing
            vla.lkv_probe_read(self.buf[i % m * n:], n, self.sink)
        for i, (a, b) in enumerate(evs):
            vla.lkv_probe_read(self.buf[(i + m + 1) % m * n:], n, self.sink, a.cuda_event, b.cuda_event)
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b) for a, b in evs]))
        return n, n / (ms / 1e3) / 1e9

    def close(self):
        del self.buf


def read_traffic(workload: str, khash: str):
    """HBM bytes per launch of the attention kernel from the rocprofv3 counter summary of this workload
    (profiles/traffic_<workload>.txt: FETCH_SIZE + WRITE_SIZE per dispatch, scaled by the same counters
    read on a plain device copy of known size).  None when absent or taken on other kernel sources."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(p):
        return None
    kv = {}
    with open(p) as fh:
        for line in fh:
            m = re.match(r"^\s*([a-z_]+)\s*:\s*(\S+)", line)
            if m:
                kv[m.group(1)] = m.group(2)
    if kv.get("kernel_hash") != khash or "bytes_per_launch" not in kv:
        return None
    return int(float(kv["bytes_per_launch"]))


def cpu_baseline_cells(bc, seconds: float, v_rule: str = "fixed", v_offset: float = 4.0, v_tau: float = 14.0,
                       n_splits: int = 1):
    """The fp64 oracle's cell routine, as it stands, on a bounded sample of the quantised-cell workload:
    rows (seq, layer 0, loop, head) of every loop with inputs regenerated on the host (not timed), repeated
    until `seconds` of wall time pass, under the timed V-precision rule (the fixed rule at m0 - v_offset, or
    the page's running rule at v_tau over the call's n_splits far splits).  The routine computes one row per
    call, so the rows go to as many host threads as the oracle's plain row loop uses (each call releases the
    interpreter lock); the same rows on one thread, for about a fifth of the time, give the one-core rate."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import harness
    import oracle

    w = bc.w
    rng = np.random.default_rng(0)
    rows = []
    for i in range(8):
        b, h, r = int(rng.integers(w.batch)), int(rng.integers(w.n_heads)), i % w.n_loops
        rows.append(harness.cell_inputs(bc, b, 0, r, h))

    def row(a):
        args = (a["q"], a["k_near"], a["v_near"], a["kc"], a["ks"], a["kz"], a["vc"], a["vs"], a["vz"], a["sink"],
                a["tail"], a["kind"])
        if v_rule == "running":
            oracle.cell_row_running(*args, v_tau, n_splits)
        else:
            oracle.cell_row(*args, v_offset)

    done1, elapsed1 = 0, 0.0
    while elapsed1 < seconds / 5:
        t1 = time.perf_counter()
        row(rows[done1 % len(rows)])
        elapsed1 += time.perf_counter() - t1
        done1 += 1
    cores = oracle.threads()
    t_start = time.perf_counter()
    t_end = t_start + seconds

    def worker(k):
        n = 0
        while n == 0 or time.perf_counter() < t_end:
            row(rows[(k + n) % len(rows)])
            n += 1
        return n

    with ThreadPoolExecutor(cores) as ex:
        done = sum(ex.map(worker, range(cores)))
    elapsed = time.perf_counter() - t_start
    rows_per_token = w.n_layers * w.n_heads
    return {"value": done / elapsed / rows_per_token, "unit": "loop-query tokens/s", "cores": cores, "kind": "oracle",
            "host": host_info(),
            "one_core": {"value": done1 / elapsed1 / rows_per_token, "seconds": round(elapsed1, 1),
                         "row_ms": round(1e3 * elapsed1 / done1, 3)},
            "sample": f"{done} cell rows ({len(rows)} distinct (seq, layer 0, loop, head) rows of the {w.name} "
                      f"workload, L={w.length}, repeated, "
                      + (f"running rule at tau {v_tau} over {n_splits} far splits" if v_rule == "running"
                         else f"fixed rule at m0 - {v_offset}")
                      + f") in {elapsed:.1f} s of fp64 oracle time on {cores} threads; "
                      f"{rows_per_token} rows = 1 loop-query token"}


def run_workload(args, workload: str, prober, with_cpu: bool) -> dict:
    """Build one workload in HBM, time it, and return its bench line (a dict)."""
    import dataclasses

    import numpy as np
    import torch

    import harness
    import synth
    import verify_attention_loop_amd as vla

    w = synth.WORKLOADS[workload]
    import dataclasses
    if args.batch > 0:
        w = dataclasses.replace(w, batch=args.batch)
    if args.policy != "default" and not w.quant and args.policy != w.policy:
        w = dataclasses.replace(w, policy=args.policy, window=w.window if args.policy == "ripe" else 0)
    if args.ripen == "paper" and w.mode == synth.MODE_RIPEN:
        w = dataclasses.replace(w, mode=synth.MODE_RIPEN_PAPER)
    t_setup = time.perf_counter()
    R, B, q_len = w.n_loops, w.batch, w.q_len
    split = w.split_k if args.split_k < 0 else args.split_k
    layers = list(range(w.n_layers if args.layers <= 0 else min(args.layers, w.n_layers)))
    draft = "draft_passes" in w.extra
    if w.quant:
        built = harness.build_cells(w, layers=layers)
        mode = vla.MODE_DECODE
    else:
        built, layers = build_workload(w, args)
        mode = vla.MODE_DRAFT if draft else (vla.MODE_VERIFY if q_len > 1 else vla.MODE_DECODE)
    kernel = KERNEL_NAME[w.name]
    cache = built.cache
    n_layers_step = w.n_layers
    # Every call of a step, (layer, loop, g), in the model's order: every core layer at every loop, loop-major;
    # the draft workload repeats that over its first loops for passes g = 1 .. draft_passes (draft block of g
    # tokens).  Queries, outputs and draft scratch of every call are resident in HBM.
    if draft:
        passes, d_loops = w.extra["draft_passes"], w.extra["draft_loops"]
        calls = [(layer, loop, g) for g in range(1, passes + 1) for loop in range(d_loops)
                 for layer in range(n_layers_step)]
    else:
        calls = [(layer, loop, 0) for loop in range(R) for layer in range(n_layers_step)]
    qs, outs, call_kw = {}, {}, {}
    for c in calls:
        layer, loop, g = c
        src_layer = layers[layer % len(layers)]
        if draft:
            qs[c] = harness.gpu_queries(built, src_layer, loop, 1, t0s=[L + g - 1 for L in built.lengths])
            dk, dv = harness.gpu_draft_kv(w, built.rows, src_layer, loop, built.lengths, g)
            call_kw[c] = dict(window=w.extra["draft_window"], draft_k=dk, draft_v=dv, draft_len=g)
        else:
            qs[c] = harness.gpu_queries(built, src_layer, loop, q_len)
            call_kw[c] = {}
        outs[c] = torch.empty_like(qs[c])
    ws_bytes = cache.lkv_workspace_bytes(0, 0, built.seqs, q_len=q_len, mode=mode, split_k=split)
    ws = torch.empty(max(4, ws_bytes), dtype=torch.uint8, device="cuda")
    extra = {}
    if w.quant:
        extra = {"v_thresh_offset": args.v_offset}
        if args.v_rule == "running":
            extra = {"v_rule": vla.VRULE_RUNNING, "v_tau": args.v_tau}
    if args.waves > 0:
        extra["waves"] = args.waves

    # Algorithmic bytes of each call.  Quantised cells skip the V lo plane of cold tokens, so one untimed
    # pass with the hot-mask trace counts them first.
    if w.quant:
        n_far = [L - w.sink - w.tail for L in built.lengths]
        words = (max(n_far) + 31) // 32
        mask = torch.empty((len(built.seqs), w.n_heads, words), dtype=torch.int32, device="cuda")
        valid = torch.zeros((len(built.seqs), 1, words * 32), dtype=torch.bool)
        for b, nf in enumerate(n_far):
            valid[b, 0, :nf] = True
        call_bytes = []
        cold_total, masked_total = 0, 0  # cold far token-heads of the cells that test hotness
        for c in calls:
            layer, loop, _ = c
            src_layer = layers[layer % len(layers)]
            cache.lkv_attend(src_layer, loop, built.seqs, qs[c], outs[c], split_k=split, workspace=ws,
                             mask_trace=mask, **extra)
            bits = np.unpackbits(mask.cpu().numpy().view(np.uint8), bitorder="little").reshape(
                len(built.seqs), w.n_heads, words * 32).astype(bool)
            n_cold = int((~bits & valid.numpy()).sum())
            call_bytes.append(harness.cell_bytes_per_call(built, src_layer, loop, n_cold))
            if built.plan[src_layer, loop] != synth.CELL_INT2:
                cold_total += n_cold
                masked_total += int(valid.numpy().sum()) * w.n_heads
    elif draft:  # the cached positions and the g draft tokens, once per (seq, KV head)
        call_bytes = [harness.algorithmic_bytes_per_call(w, [L + g for L in built.lengths], 1) for (_, _, g) in calls]
    else:
        call_bytes = [harness.algorithmic_bytes_per_call(w, built.lengths, q_len)] * len(calls)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    every = max(1, args.event_every)

    def step(events=None, k=0):
        for n, c in enumerate(calls):
            layer, loop, _ = c
            kw = dict(extra, **call_kw[c])
            if events is not None and (n + k) % every == 0:
                kw.update(ev_begin=events[2 * n].cuda_event, ev_end=events[2 * n + 1].cuda_event)
            cache.lkv_attend(layers[layer % len(layers)], loop, built.seqs, qs[c], outs[c], q_len=q_len, mode=mode,
                             split_k=split, workspace=ws, **kw)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * len(calls))] for _ in range(args.steps)]
    for e in ev:
        for x in e:
            x.record()  # torch creates the underlying HIP event on its first record
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for k in range(args.steps):
        step(ev[k], k)
    end.record()
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(end)
    ms_per_step = ms_total / args.steps
    # sampled launches: (step k, call n) with (n + k) % every == 0
    sampled = [(k, n) for k in range(args.steps) for n in range(len(calls)) if (n + k) % every == 0]
    kern = np.array([ev[k][2 * n].elapsed_time(ev[k][2 * n + 1]) for (k, n) in sampled])
    mean_launch_ms = float(kern.mean())
    for o in outs.values():
        assert torch.isfinite(o.float()).all(), "non-finite attention output"

    tokens_per_step = B * passes * d_loops if draft else B * q_len * R
    value = tokens_per_step / (ms_per_step / 1e3)
    alg_bytes = float(np.mean(call_bytes))
    # achieved = algorithmic bytes of the sampled launches / their summed duration
    achieved = float(sum(call_bytes[n] for (_, n) in sampled)) / (kern.sum() / 1e3) / 1e9
    khash = kernel_hash(workload)
    # the counters were taken on the workload as defined: its batch, splits and resident layers and, for
    # cells, the fixed rule at m0 - 4.0 (profiles/traffic_loopkv_cells.txt) or the page's running rule at
    # tau 14 (traffic_loopkv_cells_running.txt)
    as_profiled = (args.batch <= 0 and args.split_k < 0 and args.layers <= 0 and args.waves <= 0 and
                   (not w.quant or (args.v_rule == "fixed" and args.v_offset == 4.0) or
                    (args.v_rule == "running" and args.v_tau == 14.0)))
    policy_tag = "" if w.policy == synth.WORKLOADS[workload].policy else "_" + w.policy
    rule_tag = "_running" if w.quant and args.v_rule == "running" else ""
    traffic = read_traffic(workload + policy_tag + rule_tag, khash) if as_profiled else None

    if args.calibrate_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)  # device-to-device blit: reads 1 GiB, writes 1 GiB
        af, bf = a.view(torch.float32), b.view(torch.float32)
        for _ in range(3):
            torch.mul(af, 1.0, out=bf)  # elementwise kernel: reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()

    probe = None
    if prober is not None:
        # the same byte count as the attention launch (none for latency-bound launches under 16 MB, whose
        # time is the launch itself), and the large-read asymptote
        # (the 4 GiB reads first: they also bring the clocks back up after the host-side work above)
        r4 = prober.rate(4 << 30)[1]
        probe = {"bytes": None, "GBps": None, "frac": None}
        if alg_bytes >= 16e6:
            pb, pr = prober.rate(int(alg_bytes))
            probe = {"bytes": pb, "GBps": round(pr, 1), "frac": round(achieved / pr, 4)}
        probe.update(GBps_4GiB=round(r4, 1))

    cpu = None
    if with_cpu and not args.no_cpu_baseline:
        if w.quant:
            # the call's far splits (the running rule's runs), read back from the workspace size
            # [rows][S + 1][d + 1] fp32
            n_far_splits = ws_bytes // (B * w.n_heads * (w.head_dim + 1) * 4) - 1
            cpu = cpu_baseline_cells(built, args.cpu_seconds, args.v_rule, args.v_offset, args.v_tau, n_far_splits)
        else:
            cpu = cpu_baseline(w, args.cpu_seconds)

    if w.quant:
        dtype = "int4/int2 codes + bf16 near, fp32 accumulate"
        data = "synthetic (seeded counter-hash generator: binomial codes, fp16 metadata, seeded cell plan)"
    else:
        dtype = "bf16" if w.dtype == synth.DT_BF16 else "f32"
        data = ("synthetic (seeded counter-hash generator; Huginn-shaped ripening planes)" if w.mode == synth.MODE_RIPEN
                else "synthetic (seeded counter-hash generator; ripening planes in the RIPE page's direction)"
                if w.mode == synth.MODE_RIPEN_PAPER else "synthetic (seeded counter-hash generator)")
    cfg = {"workload": w.name, "batch": B, "core_layers": w.n_layers, "loops": R, "heads": w.n_heads,
           "kv_heads": w.hkv,
           "head_dim": w.head_dim, "context": w.length, "q_len": q_len, "policy": w.policy, "window": w.window,
           "page_tokens": 32 if w.quant else 16, "split_k": split, "calls_per_step": len(calls),
           "layers_resident": len(layers), "setup_s": round(setup_s, 1)}
    if args.waves > 0:
        cfg["waves"] = args.waves
    if draft:
        cfg.update(draft_passes=passes, draft_loops=d_loops, draft_window=w.extra["draft_window"],
                   draft_block="1..%d tokens from scratch" % passes)
    if w.quant:
        cfg.update(sink=w.sink, tail=w.tail, cold_fraction=round(cold_total / max(1, masked_total), 4),
                   v_thresh=f"m0 - {args.v_offset}" if args.v_rule == "fixed" else f"max(m, m0) - {args.v_tau} ln 2 (running)",
                   plan={k: int((built.plan == v).sum()) for k, v in (("int4", synth.CELL_INT4),
                                                                      ("int2", synth.CELL_INT2),
                                                                      ("shared", synth.CELL_SHARED))})
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "loop-query tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": data,
        "config": cfg,
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": kernel,
            "algorithmic_bytes_per_launch": int(alg_bytes), "mean_launch_us": round(mean_launch_ms * 1e3, 2),
            "launches_timed": len(sampled),
            # whole-step rate: every call's algorithmic bytes over the wall time of the step (launch gaps, merge
            # launches and host issue included), a lower bound of the kernels' own rate
            "step_GBps": round(float(sum(call_bytes)) / (ms_per_step / 1e3) / 1e9, 1),
            # the sampled launches' event durations scaled to a step; the launch-stamped events run ~1 us per launch
            # longer than the kernel trace (rocprofv3), so for back-to-back launches this can exceed ms_per_step
            "event_ms_per_step": round(mean_launch_ms * len(calls), 4),
            "kernel_hash": khash,
            "read_probe": probe,
        },
        "cpu_baseline": cpu,
    }
    return line


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (--gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    import verify_attention_loop_amd as vla

    vla.load()
    torch.cuda.set_device(0)
    prober = None if args.no_probe else ReadProbe()
    # Without --workload: the largest single-GPU configuration (Ouro-shaped split-K, all layers resident), then
    # the other configuration with a bandwidth target (Huginn-shaped RIPE decode), timed in the same run after
    # the first workload's memory is released and reported in a compact block.
    also = args.also
    if also == "auto":
        also = "huginn_ripe" if args.workload is None else "none"
    workload = args.workload or "ouro_splitk"
    line = run_workload(args, workload, prober, with_cpu=True)
    if also != "none":
        import gc
        gc.collect()
        torch.cuda.empty_cache()
        line["secondary"] = []
        for wl in also.split(","):
            sub = run_workload(args, wl, prober, with_cpu=False)
            r = sub["roofline"]
            line["secondary"].append({
                "workload": wl, "value": sub["value"], "unit": sub["unit"], "ms_per_step": sub["ms_per_step"],
                "steps": sub["steps"], "config": sub["config"],
                "roofline": {k: r[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic", "kernel",
                                               "algorithmic_bytes_per_launch", "mean_launch_us", "launches_timed",
                                               "step_GBps", "kernel_hash", "read_probe")}})
            gc.collect()
            torch.cuda.empty_cache()
    if prober is not None:
        prober.close()
    print(json.dumps(line))


if __name__ == "__main__":
    main()
