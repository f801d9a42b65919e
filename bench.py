"""Benchmark of the chunkwise gated delta-rule forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

One step = one gdn_chunk_fwd call over the whole workload (gate scan, Gram tiles,
triangular solve, WY factors, state pass and output for every chunk of every
chain), on inputs already resident in HBM.  The default workload is the
Sykra-shaped layer (B=8, T=2048, H=12, d=64, chunk 64, bf16 q/k/v);
``--workload sykra_layer_bf16_prologue`` runs the same layer from raw inputs
through gdn_chunk_fwd_prologue (q, k normalised and the gates formed from their
logits inside the kernel).  To keep
the 256 MB Infinity Cache from serving a step's inputs, the timed loop cycles
through enough independent copies of the inputs (>= 1 GiB in total) that each
step reads data not touched for several steps.

Prints ONE JSON line on stdout.  `value` is tokens/s (B*T tokens per step) from
the wall time of the K timed steps; `roofline.achieved` is the kernel's
algorithmic bytes per launch divided by its average launch duration, measured
with HIP events on the stream the kernel runs on.  `cpu_baseline` times the
fp64 CPU oracle on the host cores over the same workload.
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
    "channel_decay_kernel": [_CSRC + "channel_decay.hip", _CSRC + "gdn_lane.hpp", _CSRC + "gdn_device.hpp"],
    "channel_chunk_kernel": [_CSRC + "channel_chunk.hip", _CSRC + "gdn_pipe.hpp", _CSRC + "gdn_device.hpp"],
}


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
    path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_b = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    m_h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    if not m_b or not m_h or m_h.group(1) != kernel_source_hash(kernel):
        return None
    return float(m_b.group(1))


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
    return {"value": tokens / el, "unit": "tokens/s", "cores": int(used), "kind": "oracle",
            "sample": f"whole workload ({w.B}x{w.T} tokens x {w.H} heads, "
                      f"{'fp64 NumPy input transforms, ' if w.kind == 'prologue' else ''}fp64 C token loop, "
                      f"OpenMP over {w.B * w.H} chains) repeated {reps}x in {el:.1f} s"}


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
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize)
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
    ws_bytes = gdn.gdn_chunk_fwd_workspace_bytes(w.B, w.T, w.H, w.dk, w.dv, w.chunk, code)
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
                          stream.cuda_stream))
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

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # One event pair brackets the K back-to-back launches on the launch stream;
    # their average duration (gaps between launches included) prices the roofline.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg_ms = ev0.elapsed_time(ev1) / args.steps

    tokens = w.B * w.T
    value = tokens * args.steps / wall
    achieved = wbytes / (avg_ms * 1e-3) / 1e9
    # bf16 calls that need a workspace run the two-launch path (a factor pass and a state pass, segmented
    # for long sequences with few chains): d = 128, and d = 64 when the chains alone cannot fill the CUs.
    # Other bf16 d = 64 calls and the fused prologue run the three-stage kernel; fp32 the fused kernel.
    two = w.dtype == "bf16" and not pro and ws_bytes > 0
    if w.dtype == "c64":
        kernel, qual = "cx_prep_scan_out", "gdn::cx::"
    elif two:
        kernel, qual = "chunk_two", "gdn::two::"
    elif pro or (w.dtype == "bf16" and w.dk == 64):
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
        "data": ("synthetic (seeded; raw q/k rows N(0,1) x U(0.25,4), N(0,1) v, logits b ~ N(0,1), a ~ N(-4,1); "
                 "normalisation and gates inside the kernel)" if pro else
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
    wall = time.perf_counter() - t0
    avg_ms = ev0.elapsed_time(ev1) / args.steps
    achieved = sbytes / (avg_ms * 1e-3) / 1e9
    result = {
        "metric": f"state-steps/sec gated-delta decode step ({w.name})", "value": w.N * args.steps / wall,
        "unit": "state-steps/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded)",
        "config": {"workload": w.name, "N": w.N, "dk": w.dk, "dv": w.dv, "state_copies_cycled": ncopies},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None, "algorithmic_bytes_per_launch": sbytes,
                     "kernel_avg_ms": avg_ms, "kernel": "gdn::decode_kernel"},
    }
    print(json.dumps(result), flush=True)


FP32_VALU_PEAK_TFS = 157.3  # MI355X fp32 vector, published (256 CUs at 2.4 GHz)


def backward_flops(w) -> float:
    """Vector flops of the backward per call: one forward recompute (u = S^T k and the rank-one update,
    5 d^2 per token-head) and the reverse step (D, u, w, <D, S>, the two row sums and the carried
    gradient, 17 d^2), i.e. 22 d^2 per token-head.  The checkpoint pass's second forward is not counted."""
    return 22.0 * w.dk * w.dv * w.B * w.T * w.H


def bench_backward(args, w, dev):
    """One step = one gdn_chunk_bwd over the whole layer (all chains): forward checkpoints, recompute and the
    reverse pass.  Two input sets are cycled."""
    import torch

    import linear_attention_sequence_gated_amd as gdn
    from gdn_inputs import bf16_round, gen_upstream_grads, gen_workload
    inp = gen_workload(w)
    dO, dS = gen_upstream_grads(w.B, w.T, w.H, w.dk, w.dv, seed=w.seed, with_dS=True)
    dO = bf16_round(dO)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    code = gdn.GDN_BF16 if w.dtype == "bf16" else gdn.GDN_F32
    ncopies = args.copies or 2
    f32 = dict(dtype=torch.float32, device=dev)
    sets = []
    for _ in range(ncopies):
        d = {x: torch.from_numpy(inp[x]).to(dev).to(tdt) for x in ("q", "k", "v")}
        d.update({x: torch.from_numpy(inp[x]).to(dev) for x in ("alpha", "beta")})
        d["dO"], d["dS"] = torch.from_numpy(dO).to(dev).to(tdt), torch.from_numpy(dS).to(dev)
        sets.append(d)
    outs = [torch.empty((w.B, w.T, w.H, w.dk), **f32), torch.empty((w.B, w.T, w.H, w.dk), **f32),
            torch.empty((w.B, w.T, w.H, w.dv), **f32), torch.empty((w.B, w.T, w.H), **f32),
            torch.empty((w.B, w.T, w.H), **f32), torch.empty((w.B, w.H, w.dk, w.dv), **f32)]
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
    wall = time.perf_counter() - t0
    avg_ms = ev0.elapsed_time(ev1) / args.steps
    flops = backward_flops(w)
    tfs = flops / (avg_ms * 1e-3) / 1e12
    tok = w.B * w.T * w.H
    hbm_bytes = tok * (3 * w.dk * 2 + w.dv * 2 + 8) + tok * (2 * w.dk + w.dv) * 4 + tok * 8 + 2 * w.B * w.H * w.dk * w.dv * 4
    result = {
        "metric": f"tokens/sec gated-delta chunk bwd ({w.name})", "value": w.B * w.T * args.steps / wall,
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded; inputs as sykra_layer_bf16, upstream gradients N(0,1))",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "H": w.H, "dk": w.dk, "dv": w.dv,
                   "input_copies_cycled": ncopies, "workspace_bytes": ws_bytes},
        "roofline": {"bound": "alu", "achieved": tfs, "peak": FP32_VALU_PEAK_TFS, "unit": "TFLOP/s",
                     "frac": tfs / FP32_VALU_PEAK_TFS, "traffic": None, "algorithmic_flops_per_launch": flops,
                     "algorithmic_bytes_per_launch": hbm_bytes,
                     "hbm_achieved_GBs": hbm_bytes / (avg_ms * 1e-3) / 1e9, "kernel_avg_ms": avg_ms,
                     "kernel": "gdn::bwd::bwd_kernel"},
    }
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline_backward(inp, dO, dS, w)
    print(json.dumps(result), flush=True)


def cpu_baseline_backward(inp, dO, dS, w, budget_s: float = 12.0):
    """The oracle's reverse-mode gradients (NumPy fp64, as they stand) on a sample of chains."""
    from oracle.backward import recurrent_bwd
    chains = [(0, 0), (3, 7)]
    sub = {x: np.stack([inp[x][b, :, h] for b, h in chains], axis=1)[None] for x in ("q", "k", "v", "alpha", "beta")}
    dO_s = np.stack([dO[b, :, h] for b, h in chains], axis=1)[None]
    dS_s = np.stack([dS[b, h] for b, h in chains])[None]
    reps, t0 = 0, time.perf_counter()
    while True:
        recurrent_bwd(sub["q"], sub["k"], sub["v"], sub["alpha"], sub["beta"], None, dO_s, dS_s)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 50:
            break
    tokens = reps * w.T * len(chains) / w.H  # a token is all H heads of one position
    return {"value": tokens / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(chains)} of {w.B * w.H} chains x {w.T} tokens, NumPy fp64 token loop (one thread), "
                      f"repeated {reps}x in {el:.1f} s; tokens counted as chains x T / H"}


def bench_channel(args, w, dev):
    """One step = one gdn_fwd_channel_decay over the whole layer.  Input copies are cycled over >= 1 GiB."""
    import torch

    import linear_attention_sequence_gated_amd as gdn
    from gdn_inputs import gen_workload
    inp = gen_workload(w)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    code = gdn.GDN_BF16 if w.dtype == "bf16" else gdn.GDN_F32
    eb = 2 if w.dtype == "bf16" else 4
    tok = w.B * w.T * w.H
    wbytes = tok * ((2 * w.dk + 2 * w.dv) * eb + w.dv * 4 + 4) + w.B * w.H * w.dk * w.dv * 4
    ncopies = args.copies or max(2, int(np.ceil((1 << 30) / wbytes)))
    sets = []
    for _ in range(ncopies):
        d = {x: torch.from_numpy(inp[x]).to(dev).to(tdt) for x in ("q", "k", "v")}
        d.update({x: torch.from_numpy(inp[x]).to(dev) for x in ("r", "beta")})
        d["out"] = torch.empty((w.B, w.T, w.H, w.dv), dtype=tdt, device=dev)
        d["S"] = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
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
    wall = time.perf_counter() - t0
    avg_ms = ev0.elapsed_time(ev1) / args.steps
    achieved = wbytes / (avg_ms * 1e-3) / 1e9
    result = {
        "metric": f"tokens/sec gated-delta forward, per-channel decay ({w.name})",
        "value": w.B * w.T * args.steps / wall, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded; unit-norm q/k, N(0,1) v, sigmoid beta, r = exp(-softplus) per token and channel)",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "H": w.H, "dk": w.dk, "dv": w.dv,
                   "input_copies_cycled": ncopies},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None, "algorithmic_bytes_per_launch": wbytes,
                     "kernel_avg_ms": avg_ms,
                     "kernel": "gdn::chc::channel_chunk_kernel" if w.dtype == "bf16" else "gdn::chd::channel_decay_kernel"},
    }
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
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
