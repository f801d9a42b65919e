"""Benchmark of the chunkwise gated delta-rule forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

One step = one gdn_chunk_fwd call over the whole workload (gate scan, Gram tiles,
triangular solve, WY factors, state pass and output for every chunk of every
chain), on inputs already resident in HBM.  The default workload is the
Sykra-shaped layer (B=8, T=2048, H=12, d=64, chunk 64, bf16 q/k/v);
``--workload sykra_layer_bf16_prologue`` runs the same layer from raw inputs
through gdn_chunk_fwd_prologue (q, k normalised and the gates formed from their
logits on the device; ``long_context_bf16_prologue``, ``deltaphase_c64_prologue``
and ``single_head_f32_prologue`` do the same for the other shapes).  To keep
the 256 MB Infinity Cache from serving a step's inputs, the timed loop cycles
through enough independent copies of the inputs (>= 1 GiB in total) that each
step reads data not touched for several steps.

Prints ONE JSON line on stdout.  `value` is tokens/s (B*T tokens per step) from
the wall time of the K timed steps; `roofline.achieved` is the kernel's
algorithmic bytes per launch divided by its average launch duration, measured
with HIP events on the stream the kernel runs on.  `cpu_baseline` times the
fp64 CPU oracle on the host cores over the same workload (and, for the small
fp32 head and the default layer, on one thread as well).

`context` holds figures that are not the metric:
* `cold`: the cold protocol -- before each of `--cold` further calls an untimed
  pass over a 1 GiB scratch buffer evicts the Infinity Cache and the L2s, and
  each call is bracketed by its own event pair; median and min per call, once
  with a writing flush and once with a reading one.
* `measured_peaks`: a 1 GiB streaming read and device copy, and the
  matrix-core / vector throughput loops of libgdn_peak.so, with the kernel's
  fraction of the measured figures beside the published one.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
METRIC = "tokens/sec gated-delta chunk fwd (H=12,d=64,T=2048,C=64); % of roofline"
PROFILES = os.path.join(ROOT, "profiles")
_CSRC = "linear_attention_sequence_gated_amd/csrc/"
# Sources each measured kernel is compiled from; a counter summary is used only
# while the hash of these files matches the one recorded with it.
KERNEL_SOURCES = {
    "chunk_two": [_CSRC + "chunk_two.hip", _CSRC + "gdn_pipe.hpp", _CSRC + "gdn_device.hpp"],
    "chunk_pipe3_kernel": [_CSRC + "chunk_pipe.hip", _CSRC + "gdn_pipe.hpp", _CSRC + "gdn_device.hpp"],
    "chunk_fwd_kernel": [_CSRC + "chunk_fwd.hip", _CSRC + "gdn_device.hpp"],
    "cx_prep_scan_out": [_CSRC + "chunk_cx.hip", _CSRC + "gdn_device.hpp"],
    "decode_kernel": [_CSRC + "decode.hip", _CSRC + "gdn_device.hpp"],
    "bwd_kernel": [_CSRC + "chunk_bwd.hip", _CSRC + "gdn_lane.hpp", _CSRC + "gdn_device.hpp"],
    "tok_bwd": [_CSRC + "tok_bwd.hip", _CSRC + "gdn_lane.hpp", _CSRC + "gdn_device.hpp"],
    "channel_decay_kernel": [_CSRC + "channel_decay.hip", _CSRC + "gdn_lane.hpp", _CSRC + "gdn_device.hpp"],
    "channel_chunk_kernel": [_CSRC + "channel_chunk.hip", _CSRC + "gdn_pipe.hpp", _CSRC + "gdn_device.hpp"],
    "channel_decay_c64_kernel": [_CSRC + "channel_decay.hip", _CSRC + "gdn_lane.hpp", _CSRC + "gdn_device.hpp"],
    "chunk_grad": [_CSRC + "chunk_grad.hip", _CSRC + "chunk_two.hip", _CSRC + "gdn_pipe.hpp", _CSRC + "gdn_lane.hpp",
                   _CSRC + "gdn_device.hpp"],
}
FLUSH_BYTES = 1 << 30  # the cold protocol's cache-evicting fill


def algorithmic_bytes(w, with_s0: bool) -> int:
    """Bytes the method must move per call: q, k, v, alpha, beta, o, S0 (if given), S_final."""
    eb = {"bf16": 2, "f32": 4, "c64": 8}[w.dtype]
    sb = 8 if w.dtype == "c64" else 4
    tok = w.B * w.T * w.H
    b = tok * (2 * w.dk + 2 * w.dv) * eb + tok * 2 * 4 + w.B * w.H * w.dk * w.dv * sb
    if with_s0:
        b += w.B * w.H * w.dk * w.dv * sb
    return b


FP32_MFMA_PEAK_TFS = 157.3  # MI355X dense fp32 matrix, published


def algorithmic_flops(w) -> float:
    """Triangular-aware flops of one call: 3C dk + 2C dv + 6 dk dv + C^2/3 per token-head, x4 for complex."""
    C = w.chunk
    per = 3 * C * w.dk + 2 * C * w.dv + 6 * w.dk * w.dv + C * C / 3
    return per * (4 if w.dtype == "c64" else 1) * w.B * w.T * w.H


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; otherwise None."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_b = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    m_h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    if not m_b or not m_h or m_h.group(1) != kernel_source_hash(kernel):
        return None
    return float(m_b.group(1))


def timed_region(step, args, stream):
    """W untimed warm-up calls, then K back-to-back calls bracketed by one event pair on the launch
    stream (and by synchronisation on both sides for the wall clock).  Returns (wall s, avg ms/call)."""
    import torch
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    return time.perf_counter() - t0, ev0.elapsed_time(ev1) / args.steps


_PEAK = None


def peak_lib():
    """libgdn_peak.so: the matrix-core / vector throughput loops and the streaming read (include/gdn_peak.h)."""
    global _PEAK
    if _PEAK is None:
        import ctypes
        from linear_attention_sequence_gated_amd import build as gbuild
        if not os.path.exists(gbuild.PEAK_LIB):
            raise RuntimeError(f"{gbuild.PEAK_LIB} is missing; run python -m linear_attention_sequence_gated_amd.build")
        lib = ctypes.CDLL(gbuild.PEAK_LIB)
        lib.gdn_peak_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        lib.gdn_peak_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                      ctypes.c_void_p]
        _PEAK = lib
    return _PEAK


READ_BLOCKS = 4096  # 16 workgroups per CU for the streaming read


def cold_calls(step, first: int, n: int, stream, dev):
    """The cold protocol: before each call an untimed pass over a 1 GiB scratch buffer on the same stream
    evicts the 256 MB Infinity Cache and the L2s; every call has its own event pair.  Two flushes:
    `write` fills the buffer (the protocol as specified; it leaves dirty lines whose write-back can fall
    inside the timed call) and `read` streams it once (clean lines only)."""
    import torch
    if n <= 0:
        return None
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    flush.fill_(3)
    sink = torch.empty(READ_BLOCKS * 256, dtype=torch.float32, device=dev)
    lib = peak_lib()
    res = {"calls": n, "flush_bytes_before_each_call": FLUSH_BYTES}
    for mode in ("write", "read"):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        torch.cuda.synchronize()
        for j, (a, b) in enumerate(evs):
            if mode == "write":
                flush.fill_(j & 0x7F)
            elif lib.gdn_peak_read(flush.data_ptr(), FLUSH_BYTES, READ_BLOCKS, sink.data_ptr(), stream.cuda_stream):
                raise RuntimeError("gdn_peak_read failed")
            a.record(stream)
            step(first + j)
            b.record(stream)
        torch.cuda.synchronize()
        us = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
        res[f"{mode}_flush"] = {"median_us": float(np.median(us)), "min_us": us[0], "max_us": us[-1]}
        first += n
    return res


def measured_peaks(dev):
    """A 1 GiB streaming read and device copy, and the bf16 / fp32 matrix-core and fp32 vector loops of
    libgdn_peak.so, timed with events."""
    import torch
    out = {}
    lib = peak_lib()
    stream = torch.cuda.current_stream(dev)
    src = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    sink = torch.empty(max(READ_BLOCKS, 256 * 8) * 256, dtype=torch.float32, device=dev)
    src.fill_(1)
    dst.copy_(src)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(5):
        dst.copy_(src)
    ev1.record(stream)
    torch.cuda.synchronize()
    out["copy_GBs"] = 2 * FLUSH_BYTES * 5 / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
    ev0.record(stream)
    for i in range(5):  # alternate buffers so no pass reads what the previous one left in the caches
        if lib.gdn_peak_read((src if i % 2 else dst).data_ptr(), FLUSH_BYTES, READ_BLOCKS, sink.data_ptr(),
                             stream.cuda_stream):
            raise RuntimeError("gdn_peak_read failed")
    ev1.record(stream)
    torch.cuda.synchronize()
    out["read_GBs"] = FLUSH_BYTES * 5 / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
    del src, dst
    blocks, iters = 256 * 8, 2000
    for kind, name, per in ((0, "mfma_bf16_TFs", 16384), (1, "mfma_f32_TFs", 2048), (2, "valu_fma_f32_TFs", 128)):
        if lib.gdn_peak_mfma_loop(kind, iters, blocks, sink.data_ptr(), stream.cuda_stream) != 0:
            raise RuntimeError("gdn_peak_mfma_loop failed")
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(3):
            lib.gdn_peak_mfma_loop(kind, iters, blocks, sink.data_ptr(), stream.cuda_stream)
        ev1.record(stream)
        torch.cuda.synchronize()
        out[name] = 3.0 * blocks * 4 * iters * 8 * per / (ev0.elapsed_time(ev1) * 1e-3) / 1e12
    return out


def add_context(result, args, step, stream, dev, key: str, before: int):
    """The cold protocol and the measured peaks, with the kernel's fraction of the measured figures.
    `calls` records the order of the calls in this process (for reading a kernel trace of it): `before`
    untimed calls (argument checks through the torch helper, warm-up), the K timed ones, then the cold
    ones, write-flushed first."""
    ctx = {"calls": {"kernel_key": key, "before_timed": before + args.warmup, "timed": args.steps,
                     "cold": 2 * max(args.cold, 0)}}
    cold = cold_calls(step, args.warmup + args.steps, args.cold, stream, dev)
    if cold:
        ctx["cold"] = cold
    if not args.no_peaks:
        pk = measured_peaks(dev)
        rf = result["roofline"]
        if rf["unit"] == "GB/s":
            keys = ("read_GBs", "copy_GBs")
        elif rf["bound"] == "alu":
            keys = ("valu_fma_f32_TFs",)
        else:
            keys = ("mfma_bf16_TFs",) if result["dtype"] == "bf16" else ("mfma_f32_TFs",)
        pk["kernel_frac_of_measured"] = {k: rf["achieved"] / pk[k] for k in keys}
        ctx["measured_peaks"] = pk
    result["context"] = ctx


def decode_bytes(w) -> int:
    """Bytes one decode step must move: S read and written (fp32), q, k, v, o (bf16), alpha, beta."""
    eb = {"bf16": 2, "f32": 4, "c64": 8}[w.dtype]
    sb = 8 if w.dtype == "c64" else 4
    return w.N * (2 * w.dk * w.dv * sb + (2 * w.dk + 2 * w.dv) * eb + 2 * 4)


def cpu_baseline(inp, w, budget_s: float = 12.0):
    """Time the fp64 oracle (as it stands) on the host over the full workload.  For raw
    layer inputs that is the oracle's input transforms followed by its token loop."""
    import oracle
    from oracle import prologue as oracle_prologue
    q, k, v = (np.asarray(inp[x], dtype=np.float64) for x in ("q", "k", "v"))
    s0 = None if inp.get("S0") is None else np.asarray(inp["S0"], np.float64)
    threads = os.cpu_count() or 1
    reps, t0 = 0, time.perf_counter()
    used = threads
    while True:
        if w.kind == "prologue":
            qh, kh, a, b = oracle_prologue.prologue(q, k, inp["a_logit"], inp["b_logit"], w.beta_scale)
        else:
            qh, kh, a, b = q, k, np.asarray(inp["alpha"], np.float64), np.asarray(inp["beta"], np.float64)
        _, _, used = oracle.recurrent_fwd(qh, kh, v, a, b, s0, threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 400:
            break
    tokens = w.B * w.T * reps
    res = {"value": tokens / el, "unit": "tokens/s", "cores": int(used), "kind": "oracle",
           "sample": f"whole workload ({w.B}x{w.T} tokens x {w.H} heads, "
                     f"{'fp64 NumPy input transforms, ' if w.kind == 'prologue' else ''}fp64 C token loop, "
                     f"OpenMP over {w.B * w.H} chains) repeated {reps}x in {el:.1f} s"}
    if w.name in ("single_head_f32", "sykra_layer_bf16"):
        # The same token loop on one thread, over the whole workload.
        reps1, t0 = 0, time.perf_counter()
        while True:
            oracle.recurrent_fwd(q, k, v, np.asarray(inp["alpha"], np.float64), np.asarray(inp["beta"], np.float64),
                                 s0, threads=1)
            reps1 += 1
            el1 = time.perf_counter() - t0
            if el1 >= budget_s / 2 or reps1 >= 400:
                break
        res["single_thread"] = {"value": w.B * w.T * reps1 / el1, "unit": "tokens/s", "cores": 1,
                                "sample": f"whole workload, fp64 C token loop on one thread, repeated {reps1}x "
                                          f"in {el1:.1f} s"}
    return res


def summarize(path: str) -> None:
    """Print a markdown summary of rocprofv3 CSV output under `path` (kernel stats and/or
    FETCH_SIZE / WRITE_SIZE counters, scaled by the copy kernel recorded in the same run)."""
    import csv
    import glob
    stats = glob.glob(os.path.join(path, "**", "*kernel_stats.csv"), recursive=True)
    for f in stats:
        print(f"kernel stats ({os.path.relpath(f, path)}):\n")
        print("| kernel | calls | avg us | min us | max us | total % |")
        print("|---|---|---|---|---|---|")
        for r in csv.DictReader(open(f)):
            name = r["Name"]
            short = name if len(name) < 70 else name[:67] + "..."
            print(f"| {short} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                  f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |")
        print()
    counters = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    for f in counters:
        per = {}
        for r in csv.DictReader(open(f)):
            key = (r["Kernel_Name"], r["Counter_Name"])
            per.setdefault(key, []).append(float(r["Counter_Value"]))
        print(f"counters ({os.path.relpath(f, path)}), mean per dispatch:\n")
        print("| kernel | counter | dispatches | mean per dispatch |")
        print("|---|---|---|---|")
        for (k, cn), vals in sorted(per.items()):
            short = k if len(k) < 70 else k[:67] + "..."
            print(f"| {short} | {cn} | {len(vals)} | {np.mean(vals):.1f} |")
        print()


COUNTER_ARGS = "--steps 5 --warmup 1 --no-cpu --no-peaks --cold 0"
STALL_COUNTERS = ("SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_VMEM SQ_ACTIVE_INST_LDS SQ_INSTS_VMEM_RD "
                  "SQ_INSTS_LDS SQ_BUSY_CYCLES TA_TA_BUSY_sum TA_ADDR_STALLED_BY_TC_CYCLES_sum "
                  "TCP_TCC_READ_REQ_LATENCY_sum TCP_TCC_READ_REQ_sum GRBM_GUI_ACTIVE")
# One rocprofv3 run per pass; {d} is the output folder, {w} the workload.  The trace pass is the benchmark
# command itself (its JSON line goes to {d}/bench.json); the counter passes cut it to a few calls.
PROFILE_PASSES = {
    "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d {d}/trace -o run -- "
             "python3 -u bench.py --workload {w}",
    "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d}/fetch -o run -- "
             "python3 -u bench.py --workload {w} " + COUNTER_ARGS + " --calibrate-copy",
    "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d}/write -o run -- "
             "python3 -u bench.py --workload {w} " + COUNTER_ARGS + " --calibrate-copy",
    "util": "rocprofv3 --pmc MfmaUtil LdsUtil LdsBankConflict VALUBusy --output-format csv -d {d}/util -o run -- "
            "python3 -u bench.py --workload {w} " + COUNTER_ARGS,
    "stall": "rocprofv3 --pmc " + STALL_COUNTERS + " --output-format csv -d {d}/stall -o run -- "
             "python3 -u bench.py --workload {w} " + COUNTER_ARGS,
}


def run_profiles(root: str, workload: str, passes) -> int:
    """Run the named PROFILE_PASSES for one workload, one child process at a time, from the repository root with
    TMPDIR=/tmp, each under a 240 s limit (the whole process group is killed past it); output under
    root/<workload>.  Returns the first non-zero status, else 0."""
    import shlex
    import signal
    import subprocess
    d = os.path.join(root, workload)
    os.makedirs(d, exist_ok=True)
    env = dict(os.environ, TMPDIR="/tmp")
    for name in passes:
        cmd = PROFILE_PASSES[name].format(d=d, w=workload)
        out = os.path.join(d, "bench.json" if name == "trace" else name + ".out")
        err = os.path.join(d, name + ".err")
        print(f"[profile] {workload} {name}: {cmd}", flush=True)
        t0 = time.time()
        with open(out, "w") as fo, open(err, "w") as fe:
            p = subprocess.Popen(shlex.split(cmd), stdin=subprocess.DEVNULL, stdout=fo, stderr=fe, cwd=ROOT, env=env,
                                 start_new_session=True)
            try:
                rc = p.wait(timeout=240)
            except subprocess.TimeoutExpired:
                os.killpg(p.pid, signal.SIGKILL)
                p.wait()
                rc = 124
        print(f"[profile] {workload} {name}: status {rc} after {time.time() - t0:.0f} s", flush=True)
        if rc != 0:
            print(open(err).read()[-2000:], flush=True)
            return rc
    return 0


def _csv_rows(path, pattern):
    import csv
    import glob
    files = glob.glob(os.path.join(path, "**", pattern), recursive=True)
    return [r for f in files for r in csv.DictReader(open(f))]


def _demangle(names):
    """Itanium-mangled kernel names (counter passes report them so) -> readable, through c++filt."""
    import subprocess
    names = sorted(set(names))
    # c++filt predates the bf16 builtin type's code (DF16b); spell it as a vendor type it knows.
    r = subprocess.run(["c++filt"], input="\n".join(n.replace("DF16b", "u6__bf16") for n in names),
                       capture_output=True, text=True, check=True)
    return dict(zip(names, r.stdout.splitlines()))


def _counters(path):
    """{(dispatch id, kernel name, counter): value summed over dimensions} of a counter pass."""
    rows = _csv_rows(path, "*counter_collection.csv")
    dm = _demangle(r["Kernel_Name"] for r in rows)
    per = {}
    for r in rows:
        key = (int(r["Dispatch_Id"]), dm[r["Kernel_Name"]], r["Counter_Name"])
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    return per


def _short(name: str) -> str:
    name = re.sub(r"\(.*\)$", "", name)
    return name.replace("void ", "")


def write_profile(workload: str, d: str) -> str:
    """Summarise the rocprofv3 passes of PROFILE_PASSES for one workload (run from the repository root with
    their output under `d`) into profiles/<kernel>_<workload>.md; returns the path."""
    bench = json.loads(open(os.path.join(d, "bench.json")).read().strip().splitlines()[-1])
    rf, calls = bench["roofline"], bench["context"]["calls"]
    key = calls["kernel_key"]
    alg = rf.get("algorithmic_bytes_per_launch", rf.get("algorithmic_bytes_per_call"))
    lines = [f"# {rf['kernel']} -- workload {workload}", ""]
    cfg = ", ".join(f"{k}={v}" for k, v in bench["config"].items() if k != "workload")
    lines += [f"Configuration: {cfg}; dtype {bench['dtype']}.", "",
              "Commands, from the repository root on one MI355X, after `cd /tmp && export TMPDIR=/tmp` "
              "(the trace pass writes the benchmark's JSON line to bench.json in its folder; each counter pass "
              "runs alone):", ""]
    dd = os.path.relpath(os.path.abspath(d), ROOT)
    for name, cmd in PROFILE_PASSES.items():
        if name == "stall" and not os.path.isdir(os.path.join(d, "stall")):
            continue
        extra = f" > {dd}/bench.json" if name == "trace" else ""
        lines.append("    timeout -s KILL 240 " + cmd.format(d=dd, w=workload) + extra)
    lines += ["", f"(`python3 bench.py --run-profiles {os.path.dirname(dd)} --workload {workload}` runs the same passes "
              "in turn.)", ""]

    # Kernel trace.
    tr = [r for r in _csv_rows(os.path.join(d, "trace"), "*kernel_trace.csv")]
    dm = _demangle(r["Kernel_Name"] for r in tr)
    for r in tr:
        r["Kernel_Name"] = dm[r["Kernel_Name"]]
    tr.sort(key=lambda r: int(r["Start_Timestamp"]))
    gk = [r for r in tr if "gdn::" in r["Kernel_Name"]]
    ncalls = calls["before_timed"] + calls["timed"] + calls["cold"]
    per_call = len(gk) // ncalls if ncalls else 0
    lines += ["## Kernel trace", ""]
    if per_call * ncalls != len(gk):
        lines += [f"(the trace holds {len(gk)} dispatches of this library for {ncalls} calls: not a whole number "
                  f"per call, so the per-call split below is skipped)", ""]
    lines += ["| kernel | dispatches | avg us | min us | max us |", "|---|---|---|---|---|"]
    byname = {}
    for r in gk:
        byname.setdefault(_short(r["Kernel_Name"]), []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    for n, v in byname.items():
        lines.append(f"| {n} | {len(v)} | {np.mean(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
    lines.append("")
    if per_call and per_call * ncalls == len(gk):
        grp = [gk[i * per_call:(i + 1) * per_call] for i in range(ncalls)]
        b0, k = calls["before_timed"], calls["timed"]
        timed = grp[b0:b0 + k]
        busy = [sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in g) / 1e3 for g in timed]
        span = (int(timed[-1][-1]["End_Timestamp"]) - int(timed[0][0]["Start_Timestamp"])) / 1e3 / k
        lines += [f"The {k} timed calls ({per_call} launch{'es' if per_call > 1 else ''} each), from the trace:",
                  f"- kernel time per call, mean {np.mean(busy):.2f} us (min {min(busy):.2f}, max {max(busy):.2f});",
                  f"- first start to last end over {k} calls: {span:.2f} us per call;",
                  f"- the benchmark's own figure from HIP events on the launch stream (same run): "
                  f"{rf['kernel_avg_ms'] * 1e3:.2f} us per call; {bench['ms_per_step'] * 1e3:.2f} us per step "
                  f"by the wall clock."]
        nc = calls["cold"] // 2
        if nc:
            for j, mode in enumerate(("write", "read")):
                g = grp[b0 + k + j * nc:b0 + k + (j + 1) * nc]
                cb = [sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in x) / 1e3 for x in g]
                lines.append(f"- {nc} cold calls after a 1 GiB {mode} flush: kernel time median "
                             f"{np.median(cb):.2f} us (min {min(cb):.2f}).")
        lines.append("")
    seen = set()
    lines += ["| kernel | grid | workgroup | LDS B | VGPR | AGPR | SGPR | scratch |", "|---|---|---|---|---|---|---|---|"]
    for r in gk:
        n = _short(r["Kernel_Name"])
        sig = (n, r["Grid_Size_X"])
        if sig in seen:
            continue
        seen.add(sig)
        lines.append(f"| {n} | {r['Grid_Size_X']} | {r['Workgroup_Size_X']} | {r['LDS_Block_Size']} | "
                     f"{r['VGPR_Count']} | {r['Accum_VGPR_Count']} | {r['SGPR_Count']} | {r['Scratch_Size']} |")
    lines.append("")

    # HBM traffic.
    traffic = None
    if os.path.isdir(os.path.join(d, "fetch")) and os.path.isdir(os.path.join(d, "write")):
        lines += ["## HBM traffic (FETCH_SIZE, WRITE_SIZE)", "",
                  "`--calibrate-copy` ends each counter run with five plain 256 MiB device-to-device copies; "
                  "they give the scale from each counter to bytes.", ""]
        tot = {}
        lines += ["| counter | copy KiB/dispatch | true KiB | scale |", "|---|---|---|---|"]
        rows = []
        for cn, sub in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
            per = _counters(os.path.join(d, sub))
            copies = sorted((di, v) for (di, n, c), v in per.items() if c == cn and "copyBuffer" in n)[-5:]
            scale = 262144.0 / np.mean([v for _, v in copies])
            lines.append(f"| {cn} | {np.mean([v for _, v in copies]):.1f} | 262144 | {scale:.5f} |")
            mine = {}
            for (di, n, c), v in per.items():
                if c == cn and "gdn::" in n:
                    mine.setdefault(_short(n), []).append(v)
            ncall = min(len(v) for v in mine.values())
            tot[cn] = sum(sum(v) for v in mine.values()) * 1024 * scale / ncall
            for n, v in mine.items():
                rows.append(f"| {n} | {cn} | {len(v)} | {np.mean(v):.1f} | {np.mean(v) * 1024 * scale:,.0f} |")
        lines += ["", "| kernel | counter | dispatches | raw KiB/dispatch | bytes/dispatch |", "|---|---|---|---|---|"]
        lines += rows
        traffic = tot["FETCH_SIZE"] + tot["WRITE_SIZE"]
        lines += ["", f"Per call: {tot['FETCH_SIZE']:,.0f} B fetched + {tot['WRITE_SIZE']:,.0f} B written = "
                  f"{traffic:,.0f} B, {traffic / alg:.3f}x the algorithmic {alg:,} B.", "",
                  f"traffic_bytes_per_launch: {traffic:.0f}", f"algorithmic_bytes_per_launch: {alg}",
                  f"kernel_source_sha256_16: {kernel_source_hash(key)}", "",
                  "The hash covers " + ", ".join(KERNEL_SOURCES[key]) + " as of these runs; the benchmark "
                  "reports the traffic figure only while it matches.", ""]

    # Utilisation and stalls.
    for sub, title in (("util", "Utilisation (derived counters, mean per dispatch)"),
                       ("stall", "Wave states and memory pipeline (raw counters, mean per dispatch)")):
        if not os.path.isdir(os.path.join(d, sub)):
            continue
        per = _counters(os.path.join(d, sub))
        mine = {}
        for (di, n, c), v in per.items():
            if "gdn::" in n:
                mine.setdefault((_short(n), c), []).append(v)
        names = sorted({c for _, c in mine})
        kern = sorted({n for n, _ in mine})
        lines += [f"## {title}", "", "| kernel | " + " | ".join(names) + " |", "|---" * (len(names) + 1) + "|"]
        for n in kern:
            lines.append(f"| {n} | " + " | ".join(f"{np.mean(mine[(n, c)]):.4g}" if (n, c) in mine else "-"
                                                   for c in names) + " |")
        if sub == "stall":
            lines += ["", "Ratios (SQ wave counters are in quad-cycles; GRBM_GUI_ACTIVE in cycles):", ""]
            for n in kern:
                g = lambda c: np.mean(mine.get((n, c), [np.nan]))  # noqa: E731
                lines.append(
                    f"- {n}: waiting on anything {g('SQ_WAIT_ANY') / g('SQ_WAVE_CYCLES'):.2f} of wave time, "
                    f"waiting to issue {g('SQ_WAIT_INST_ANY') / g('SQ_WAVE_CYCLES'):.2f}; "
                    f"vector-memory instructions {g('SQ_INSTS_VMEM_RD'):.3g} reads; "
                    f"TA busy {g('TA_TA_BUSY_sum') / (g('GRBM_GUI_ACTIVE') * 256):.2f} of the time per TA; "
                    f"TA address stalled by the L1 {g('TA_ADDR_STALLED_BY_TC_CYCLES_sum') / max(g('TA_TA_BUSY_sum'), 1):.2f}"
                    f" of TA busy cycles; mean L1->L2 read latency "
                    f"{g('TCP_TCC_READ_REQ_LATENCY_sum') / max(g('TCP_TCC_READ_REQ_sum'), 1):.0f} cycles.")
        lines.append("")
    path = os.path.join(PROFILES, f"{key}_{workload}.md")
    with open(path, "w") as f:
        f.write("\n".join(lines))
    return path


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="sykra_layer_bf16")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copies", type=int, default=0, help="input copies to cycle (0 = enough for >= 1 GiB)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB device copy 5 times (reference for HBM byte counters)")
    ap.add_argument("--summarize", metavar="DIR", help="summarise rocprofv3 CSV output under DIR and exit")
    ap.add_argument("--cold", type=int, default=20, help="calls timed one by one after a 1 GiB cache flush (0 = none)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured copy / matrix-core peak loops")
    ap.add_argument("--profile-commands", metavar="ROOT",
                    help="print the rocprofv3 passes for --workload, writing under ROOT/<workload>")
    ap.add_argument("--run-profiles", metavar="ROOT",
                    help="run the rocprofv3 passes named by --passes for --workload, writing under ROOT/<workload>")
    ap.add_argument("--passes", default=",".join(PROFILE_PASSES), help="comma-separated passes for --run-profiles")
    ap.add_argument("--write-profile", metavar="DIR",
                    help="summarise the rocprofv3 passes under DIR into profiles/<kernel>_<workload>.md")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize)
        return
    if args.profile_commands:
        d = os.path.join(args.profile_commands, args.workload)
        for name, cmd in PROFILE_PASSES.items():
            print(name + "\t" + cmd.format(d=d, w=args.workload) + (f" > {d}/bench.json" if name == "trace" else ""))
        return
    if args.run_profiles:
        sys.exit(run_profiles(args.run_profiles, args.workload, [p for p in args.passes.split(",") if p]))
    if args.write_profile:
        print(write_profile(args.workload, args.write_profile))
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (chains are independent, so a "
              f"multi-GPU run would shard batch x heads with no communication).", file=sys.stderr)
        sys.exit(2)

    import torch

    import linear_attention_sequence_gated_amd as gdn
    from gdn_inputs import WORKLOADS, gen_workload

    w = WORKLOADS[args.workload]
    gdn.load()
    dev = torch.device("cuda:0")
    if w.kind == "decode":
        return bench_decode(args, w, dev)
    if w.kind == "backward":
        return bench_backward(args, w, dev)
    if w.kind == "channel":
        return bench_channel(args, w, dev)
    inp = gen_workload(w)
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32, "c64": torch.complex64}[w.dtype]
    wbytes = algorithmic_bytes(w, inp["S0"] is not None)
    ncopies = args.copies or max(2, int(np.ceil((1 << 30) / wbytes)))

    pro = w.kind == "prologue"  # raw q, k and gate logits through gdn_chunk_fwd_prologue
    gates = ("a_logit", "b_logit") if pro else ("alpha", "beta")

    def upload():
        d = {x: torch.from_numpy(inp[x]).to(dev) for x in ("q", "k", "v") + gates}
        for x in ("q", "k", "v"):
            d[x] = d[x].to(tdt)
        d["S0"] = None if inp["S0"] is None else torch.from_numpy(inp["S0"]).to(dev)
        d["out"] = torch.empty((w.B, w.T, w.H, w.dv), dtype=tdt, device=dev)
        d["S"] = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.complex64 if w.dtype == "c64" else torch.float32,
                             device=dev)
        return d

    sets = [upload() for _ in range(ncopies)]
    stream = torch.cuda.current_stream(dev)
    # The torch helper validates its arguments once (first warm-up call); the
    # timed steps then call the C ABI directly with the prepared pointers, as a
    # serving loop would, so host-side checks do not open gaps between launches.
    code = {"bf16": gdn.GDN_BF16, "f32": gdn.GDN_F32, "c64": gdn.GDN_C64}[w.dtype]
    lib = gdn.load()
    ws_query = gdn.gdn_chunk_fwd_prologue_workspace_bytes if pro else gdn.gdn_chunk_fwd_workspace_bytes
    ws_bytes = ws_query(w.B, w.T, w.H, w.dk, w.dv, w.chunk, code)
    # One workspace serves every copy: the calls are ordered on one stream.
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    ws_ptr = ws.data_ptr() if ws_bytes else None
    calls = []
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    for d in sets:
        if pro:
            gdn.chunk_fwd_prologue(d["q"], d["k"], d["v"], d["a_logit"], d["b_logit"], w.beta_scale, d["S0"],
                                   out=d["out"], S_final=d["S"], stream=stream.cuda_stream)
            calls.append((ptr(d["q"]), ptr(d["k"]), ptr(d["v"]), ptr(d["a_logit"]), ptr(d["b_logit"]), w.beta_scale,
                          ptr(d["S0"]), w.chunk, ptr(d["out"]), ptr(d["S"]), w.B, w.T, w.H, w.dk, w.dv, code,
                          ws_ptr, ws_bytes, stream.cuda_stream))
        else:
            gdn.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], out=d["out"], S_final=d["S"],
                          stream=stream.cuda_stream)
            calls.append((ptr(d["q"]), ptr(d["k"]), ptr(d["v"]), ptr(d["alpha"]), ptr(d["beta"]), ptr(d["S0"]),
                          w.chunk, ptr(d["out"]), ptr(d["S"]), w.B, w.T, w.H, w.dk, w.dv, code, ws_ptr, ws_bytes,
                          stream.cuda_stream))
    entry = lib.gdn_chunk_fwd_prologue if pro else lib.gdn_chunk_fwd

    def step(i):
        s = entry(*calls[i % ncopies])
        if s != 0:  # GDN_OK
            raise gdn.GdnError(s)

    # One event pair brackets the K back-to-back launches on the launch stream;
    # their average duration (gaps between launches included) prices the roofline.
    wall, avg_ms = timed_region(step, args, stream)

    tokens = w.B * w.T
    value = tokens * args.steps / wall
    achieved = wbytes / (avg_ms * 1e-3) / 1e9
    # bf16 calls that need a workspace run the two-launch path (a factor pass and a state pass, segmented
    # for long sequences with few chains): d = 128, and d = 64 when the chains alone cannot fill the CUs.
    # Other bf16 d = 64 calls, with or without the prologue, run the three-stage kernel; fp32 the fused
    # kernel.  The fp32 and complex64 prologues add a pass over the rows ahead of the forward.
    two = w.dtype == "bf16" and ws_bytes > 0
    if w.dtype == "c64":
        kernel, qual = "cx_prep_scan_out", "gdn::cx::"
    elif two:
        kernel, qual = "chunk_two", "gdn::two::"
    elif w.dtype == "bf16" and w.dk == 64:
        kernel, qual = "chunk_pipe3_kernel", "gdn::pipe3::"
    else:
        kernel, qual = "chunk_fwd_kernel", "gdn::"
    traffic = measured_traffic(kernel, args.workload)
    result = {
        "metric": METRIC if args.workload == "sykra_layer_bf16" else f"tokens/sec gated-delta chunk fwd ({w.name})",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": (("synthetic (seeded; raw q/k rows of unit phasors x U(0.25,4), complex normal v, "
                  if w.dtype == "c64" else "synthetic (seeded; raw q/k rows N(0,1) x U(0.25,4), N(0,1) v, ")
                 + f"logits b ~ N(0,1), a ~ N({w.alpha_mu:g},1); normalisation and gates on the device)" if pro else
                 "synthetic (seeded; unit-norm q/k, N(0,1) v, sigmoid beta, exp(-softplus) alpha)"),
        "config": {"workload": w.name, "B": w.B, "T": w.T, "H": w.H, "dk": w.dk, "dv": w.dv, "chunk": w.chunk,
                   "S0": inp["S0"] is not None, "input_copies_cycled": ncopies},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": wbytes, "kernel_avg_ms": avg_ms,
                     "kernel": qual + kernel},
    }
    if two:
        # The factor pass and the state pass of one call are priced together: achieved is the call's
        # algorithmic bytes over the call's average duration (both launches and the gap between them).
        result["roofline"]["kernel"] = "gdn::two::factor_kernel + state_kernel (one call)"
    if w.dtype == "c64":
        # Complex products run on fp32 matrix cores, which bind before HBM does.  The three
        # launches of one call (prep, state scan, output) are priced together.
        flops = algorithmic_flops(w)
        tfs = flops / (avg_ms * 1e-3) / 1e12
        result["roofline"] = {"bound": "mfma", "achieved": tfs, "peak": FP32_MFMA_PEAK_TFS, "unit": "TFLOP/s",
                              "frac": tfs / FP32_MFMA_PEAK_TFS, "traffic": traffic,
                              "algorithmic_flops_per_call": flops, "algorithmic_bytes_per_call": wbytes,
                              "hbm_achieved_GBs": achieved, "kernel_avg_ms": avg_ms,
                              "kernel": "gdn::cx::cx_prep_kernel + cx_scan_kernel + cx_out_kernel"}
    add_context(result, args, step, stream, dev, kernel, ncopies)
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(inp, w)
    if args.calibrate_copy:
        calibrate_copy(dev)
    print(json.dumps(result), flush=True)


def calibrate_copy(dev):
    """A plain device-to-device copy of 256 MiB, five times: its FETCH_SIZE / WRITE_SIZE
    counters give the scale between counter units and bytes on this machine."""
    import torch
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()


def bench_decode(args, w, dev):
    """One step = one gdn_recurrent_step over all N states (one token each).  The timed loop
    cycles through independent state sets (>= 1 GiB in total) so a step's state is not
    served from the Infinity Cache."""
    import torch

    import linear_attention_sequence_gated_amd as gdn
    from gdn_inputs import gen_decode_workload
    inp = gen_decode_workload(w, steps=8)
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32, "c64": torch.complex64}[w.dtype]
    sbytes = decode_bytes(w)
    state_bytes = inp["S"].nbytes
    ncopies = args.copies or max(2, int(np.ceil((1 << 30) / state_bytes)))
    S = [torch.from_numpy(inp["S"]).to(dev) for _ in range(ncopies)]
    toks = []
    for t in range(inp["q"].shape[0]):
        d = {x: torch.from_numpy(inp[x][t]).to(dev) for x in ("q", "k", "v", "alpha", "beta")}
        for x in ("q", "k", "v"):
            d[x] = d[x].to(tdt)
        toks.append(d)
    out = torch.empty((w.N, w.dv), dtype=tdt, device=dev)
    stream = torch.cuda.current_stream(dev)
    # Validate once through the torch helper, then time direct C ABI calls.
    d0 = toks[0]
    gdn.recurrent_step(d0["q"], d0["k"], d0["v"], d0["alpha"], d0["beta"], S[0], out=out, stream=stream.cuda_stream)
    code = {"bf16": gdn.GDN_BF16, "f32": gdn.GDN_F32, "c64": gdn.GDN_C64}[w.dtype]
    lib = gdn.load()
    tok_ptrs = [tuple(d[x].data_ptr() for x in ("q", "k", "v", "alpha", "beta")) for d in toks]
    s_ptrs = [t.data_ptr() for t in S]
    tail = (out.data_ptr(), w.N, w.dk, w.dv, code, stream.cuda_stream)

    def step(i):
        s = lib.gdn_recurrent_step(*tok_ptrs[i % len(tok_ptrs)], s_ptrs[i % ncopies], *tail)
        if s != 0:  # GDN_OK
            raise gdn.GdnError(s)

    wall, avg_ms = timed_region(step, args, stream)
    achieved = sbytes / (avg_ms * 1e-3) / 1e9
    result = {
        "metric": f"state-steps/sec gated-delta decode step ({w.name})", "value": w.N * args.steps / wall,
        "unit": "state-steps/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded)",
        "config": {"workload": w.name, "N": w.N, "dk": w.dk, "dv": w.dv, "state_copies_cycled": ncopies},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic("decode_kernel", w.name),
                     "algorithmic_bytes_per_launch": sbytes, "kernel_avg_ms": avg_ms, "kernel": "gdn::decode_kernel"},
    }
    add_context(result, args, step, stream, dev, "decode_kernel", 1)
    if args.calibrate_copy:
        calibrate_copy(dev)
    print(json.dumps(result), flush=True)


FP32_VALU_PEAK_TFS = 157.3  # MI355X fp32 vector, published (256 CUs at 2.4 GHz)


def backward_flops(w) -> float:
    """Vector flops of the backward per call: one forward recompute (u = S^T k and the rank-one update,
    5 d^2 per token-head) and the reverse step (D, u, w, <D, S>, the two row sums and the carried
    gradient, 17 d^2), i.e. 22 d^2 per token-head.  The checkpoint pass's second forward is not counted."""
    return 22.0 * w.dk * w.dv * w.B * w.T * w.H * (4 if w.dtype == "c64" else 1)


def bench_backward(args, w, dev):
    """One step = one gdn_chunk_bwd over the whole layer (all chains): forward checkpoints, recompute and the
    reverse pass.  Two input sets are cycled."""
    import torch

    import linear_attention_sequence_gated_amd as gdn
    from gdn_inputs import bf16_round, gen_upstream_grads, gen_workload
    inp = gen_workload(w)
    cx = w.dtype == "c64"
    dO, dS = gen_upstream_grads(w.B, w.T, w.H, w.dk, w.dv, seed=w.seed, with_dS=True, dtype="c64" if cx else "f32")
    if w.dtype == "bf16":
        dO = bf16_round(dO)
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32, "c64": torch.complex64}[w.dtype]
    code = {"bf16": gdn.GDN_BF16, "f32": gdn.GDN_F32, "c64": gdn.GDN_C64}[w.dtype]
    ncopies = args.copies or 2
    f32 = dict(dtype=torch.complex64 if cx else torch.float32, device=dev)
    g32 = dict(dtype=torch.float32, device=dev)
    sets = []
    for _ in range(ncopies):
        d = {x: torch.from_numpy(inp[x]).to(dev).to(tdt) for x in ("q", "k", "v")}
        d.update({x: torch.from_numpy(inp[x]).to(dev) for x in ("alpha", "beta")})
        d["dO"], d["dS"] = torch.from_numpy(dO).to(dev).to(tdt), torch.from_numpy(dS).to(dev)
        sets.append(d)
    outs = [torch.empty((w.B, w.T, w.H, w.dk), **f32), torch.empty((w.B, w.T, w.H, w.dk), **f32),
            torch.empty((w.B, w.T, w.H, w.dv), **f32), torch.empty((w.B, w.T, w.H), **g32),
            torch.empty((w.B, w.T, w.H), **g32), torch.empty((w.B, w.H, w.dk, w.dv), **f32)]
    ws_bytes = gdn.gdn_chunk_bwd_workspace_bytes(w.B, w.T, w.H, w.dk, w.dv, code)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    d0 = sets[0]
    gdn.chunk_bwd(d0["q"], d0["k"], d0["v"], d0["alpha"], d0["beta"], d0["dO"], None, d0["dS"],
                  stream=stream.cuda_stream)  # validates once through the torch helper
    lib = gdn.load()
    calls = [tuple(d[x].data_ptr() for x in ("q", "k", "v", "alpha", "beta")) + (None, d["dO"].data_ptr(),
             d["dS"].data_ptr()) + tuple(o.data_ptr() for o in outs)
             + (w.B, w.T, w.H, w.dk, w.dv, code, ws.data_ptr(), ws_bytes, stream.cuda_stream) for d in sets]

    def step(i):
        s = lib.gdn_chunk_bwd(*calls[i % ncopies])
        if s != 0:  # GDN_OK
            raise gdn.GdnError(s)

    wall, avg_ms = timed_region(step, args, stream)
    flops = backward_flops(w)
    tfs = flops / (avg_ms * 1e-3) / 1e12
    tok = w.B * w.T * w.H
    # q, k, v, dO in; alpha, beta in; dq, dk, dv (fp32) and dalpha, dbeta out; dS_T in and dS0 out
    eb = {"bf16": 2, "f32": 4, "c64": 8}[w.dtype]
    gb = 8 if cx else 4
    hbm_bytes = (tok * (2 * w.dk * eb + 2 * w.dv * eb + 8) + tok * (2 * w.dk + w.dv) * gb + tok * 8
                 + 2 * w.B * w.H * w.dk * w.dv * gb)
    result = {
        "metric": f"tokens/sec gated-delta chunk bwd ({w.name})", "value": w.B * w.T * args.steps / wall,
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype,
        "data": ("synthetic (seeded; inputs as deltaphase_c64, complex normal upstream gradients)" if cx else
                 "synthetic (seeded; inputs as the forward workload, upstream gradients N(0,1))"),
        "config": {"workload": w.name, "B": w.B, "T": w.T, "H": w.H, "dk": w.dk, "dv": w.dv,
                   "input_copies_cycled": ncopies, "workspace_bytes": ws_bytes},
        "roofline": {"bound": "alu", "achieved": tfs, "peak": FP32_VALU_PEAK_TFS, "unit": "TFLOP/s",
                     "frac": tfs / FP32_VALU_PEAK_TFS, "traffic": measured_traffic("tok_bwd", w.name),
                     "algorithmic_flops_per_launch": flops,
                     "algorithmic_bytes_per_launch": hbm_bytes,
                     "hbm_achieved_GBs": hbm_bytes / (avg_ms * 1e-3) / 1e9, "kernel_avg_ms": avg_ms,
                     "kernel": "gdn::tbwd::tok_bwd_kernel + tok_bwd_sum_kernel (one call)"},
    }
    key = "tok_bwd"
    if w.dtype == "bf16":
        # bf16 runs the chunk form on the matrix cores, four launches per call (the forward's factor and
        # state passes, the adjoint scan, the chunk-parallel gradients): priced on its HBM bytes.
        key = "chunk_grad"
        achieved = hbm_bytes / (avg_ms * 1e-3) / 1e9
        result["roofline"] = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(key, w.name),
                              "algorithmic_bytes_per_launch": hbm_bytes, "kernel_avg_ms": avg_ms,
                              "kernel": "gdn::two::factor_kernel + state_kernel + gdn::grad::adj_kernel + "
                                        + ("grad_kernel" if w.dk == 64 else "grad_cols_kernel + grad_rows_kernel")
                                        + " (one call)"}
    add_context(result, args, step, stream, dev, key, 1)
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline_backward(inp, dO, dS, w)
    if args.calibrate_copy:
        calibrate_copy(dev)
    print(json.dumps(result), flush=True)


def cpu_baseline_backward(inp, dO, dS, w, budget_s: float = 12.0):
    """The oracle's reverse-mode gradients (NumPy fp64, as they stand) on a sample of chains (and, for long
    sequences, of their first 2048 tokens: the oracle keeps every state)."""
    from oracle.backward import recurrent_bwd
    chains = [(0, 0), (w.B - 1, w.H - 1)]
    tt = min(w.T, 2048)
    sub = {x: np.stack([inp[x][b, :tt, h] for b, h in chains], axis=1)[None] for x in ("q", "k", "v", "alpha", "beta")}
    dO_s = np.stack([dO[b, :tt, h] for b, h in chains], axis=1)[None]
    dS_s = np.stack([dS[b, h] for b, h in chains])[None]
    reps, t0 = 0, time.perf_counter()
    while True:
        recurrent_bwd(sub["q"], sub["k"], sub["v"], sub["alpha"], sub["beta"], None, dO_s, dS_s)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 50:
            break
    tokens = reps * tt * len(chains) / w.H  # a token is all H heads of one position
    return {"value": tokens / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(chains)} of {w.B * w.H} chains x {tt} tokens, NumPy fp64 token loop (one thread), "
                      f"repeated {reps}x in {el:.1f} s; tokens counted as chains x T / H"}


def bench_channel(args, w, dev):
    """One step = one gdn_fwd_channel_decay over the whole layer.  Input copies are cycled over >= 1 GiB."""
    import torch

    import linear_attention_sequence_gated_amd as gdn
    from gdn_inputs import gen_workload
    inp = gen_workload(w)
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32, "c64": torch.complex64}[w.dtype]
    sdt = torch.complex64 if w.dtype == "c64" else torch.float32
    code = {"bf16": gdn.GDN_BF16, "f32": gdn.GDN_F32, "c64": gdn.GDN_C64}[w.dtype]
    eb = {"bf16": 2, "f32": 4, "c64": 8}[w.dtype]
    sb = 8 if w.dtype == "c64" else 4
    tok = w.B * w.T * w.H
    wbytes = tok * ((2 * w.dk + 2 * w.dv) * eb + w.dv * 4 + 4) + w.B * w.H * w.dk * w.dv * sb
    ncopies = args.copies or max(2, int(np.ceil((1 << 30) / wbytes)))
    sets = []
    for _ in range(ncopies):
        d = {x: torch.from_numpy(inp[x]).to(dev).to(tdt) for x in ("q", "k", "v")}
        d.update({x: torch.from_numpy(inp[x]).to(dev) for x in ("r", "beta")})
        d["out"] = torch.empty((w.B, w.T, w.H, w.dv), dtype=tdt, device=dev)
        d["S"] = torch.empty((w.B, w.H, w.dk, w.dv), dtype=sdt, device=dev)
        sets.append(d)
    stream = torch.cuda.current_stream(dev)
    d0 = sets[0]
    gdn.fwd_channel_decay(d0["q"], d0["k"], d0["v"], d0["r"], d0["beta"], None, out=d0["out"], S_final=d0["S"],
                          stream=stream.cuda_stream)  # validates once through the torch helper
    lib = gdn.load()
    calls = [tuple(d[x].data_ptr() for x in ("q", "k", "v", "r", "beta")) + (None, d["out"].data_ptr(),
             d["S"].data_ptr(), w.B, w.T, w.H, w.dk, w.dv, code, stream.cuda_stream) for d in sets]

    def step(i):
        s = lib.gdn_fwd_channel_decay(*calls[i % ncopies])
        if s != 0:  # GDN_OK
            raise gdn.GdnError(s)

    wall, avg_ms = timed_region(step, args, stream)
    achieved = wbytes / (avg_ms * 1e-3) / 1e9
    # bf16: the chunk form; fp32 and complex64: the token loops.
    kernel, qual = {"bf16": ("channel_chunk_kernel", "gdn::chc::"), "f32": ("channel_decay_kernel", "gdn::chd::"),
                    "c64": ("channel_decay_c64_kernel", "gdn::chd::")}[w.dtype]
    result = {
        "metric": f"tokens/sec gated-delta forward, per-channel decay ({w.name})",
        "value": w.B * w.T * args.steps / wall, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": ("synthetic (seeded; phasor q, k = e^{i theta} e^{-U(0,0.5)} / sqrt(d), complex N(0,1) v, sigmoid "
                 "beta, r = exp(-softplus) per token and channel)" if w.dtype == "c64" else
                 "synthetic (seeded; unit-norm q/k, N(0,1) v, sigmoid beta, r = exp(-softplus) per token and channel)"),
        "config": {"workload": w.name, "B": w.B, "T": w.T, "H": w.H, "dk": w.dk, "dv": w.dv,
                   "input_copies_cycled": ncopies},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(kernel, w.name),
                     "algorithmic_bytes_per_launch": wbytes, "kernel_avg_ms": avg_ms, "kernel": qual + kernel},
    }
    add_context(result, args, step, stream, dev, kernel, 1)
    if not args.no_cpu:
        from oracle.channel_decay import channel_decay_fwd
        chains = [(0, 0), (3, 7)]
        sub = {x: np.stack([inp[x][b, :, h] for b, h in chains], axis=1)[None] for x in ("q", "k", "v", "r", "beta")}
        reps, t0 = 0, time.perf_counter()
        while True:
            channel_decay_fwd(sub["q"], sub["k"], sub["v"], sub["r"], sub["beta"], None)
            reps += 1
            el = time.perf_counter() - t0
            if el >= 12.0 or reps >= 100:
                break
        result["cpu_baseline"] = {
            "value": reps * w.T * len(chains) / w.H / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(chains)} of {w.B * w.H} chains x {w.T} tokens, NumPy fp64 token loop (one thread), "
                      f"repeated {reps}x in {el:.1f} s; tokens counted as chains x T / H"}
    if args.calibrate_copy:
        calibrate_copy(dev)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
