#!/usr/bin/env python3
"""Throughput of the AuT encoder forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload wide]

A step is one whole forward (plan, plan upload, conv stem, conv_out +
positions + pack, every encoder layer, final LayerNorm and projector) over the
same synthetic batch, with features and parameters already resident in HBM.
Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth_inputs as si  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 matrix/vector peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

# HBM traffic of the layer GEMMs, from rocprofv3 FETCH_SIZE / WRITE_SIZE runs
# scaled by a copy of known size; valid only for the kernel sources it was
# taken with (their SHA-256 is stored beside the figures).
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_wide_hbm_traffic.md")
GEMM_SOURCES = ("packed_windowed_attention_amd/csrc/k_gemm256.hip",
                "packed_windowed_attention_amd/csrc/device_common.h",
                "packed_windowed_attention_amd/csrc/aut_internal.h")
LAYER_GEMM_RE = r"gemm(8w|256)_kernel<\d+, 0, \d+(, \d+)?>"

METRIC = "encoder tokens/s and audio-sec/s on 1 MI355X; % of bf16 MFMA peak"

DESCR = {
    "tiny": "1 request x 8 s, 1 layer, d_model 1280, 20 heads, FFN 5120, conv 128 ch, fp32",
    "rag": "4 requests x (3, 8, 17.37, 30) s, 18 layers, d_model 1024, 16 heads, FFN 4096, conv 128 ch",
    "wide": "64 requests x U[5, 30] s (seeded), 24 layers, d_model 1280, 20 heads x 64, FFN 5120, "
            "conv 480 ch, conv_out 7680->1280, projector 1280->1280->2048",
    "long": "1 request x 1200 s, 24 layers, d_model 1280, 20 heads, FFN 5120, conv 480 ch",
    "conc": "512 requests x lognormal(median 7 s, sigma 0.6) in [0.5, 35] s, 24 layers, d_model 1280",
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def gemm_source_sha():
    import hashlib
    h = hashlib.sha256()
    for rel in GEMM_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stored_traffic(workload):
    """Bytes per layer-GEMM launch from the stored counter summary, or None
    when it is missing, for another workload, or for other kernel sources."""
    try:
        text = open(TRAFFIC_FILE).read()
        blob = text.split("```json", 1)[1].split("```", 1)[0]
        rec = json.loads(blob)
    except (OSError, IndexError, ValueError):
        return None
    if rec.get("workload") != workload or rec.get("source_sha256") != gemm_source_sha():
        return None
    return rec["bytes_per_launch"]


def traffic_summary(fetch_csv, write_csv, cal_fetch_csv, cal_write_csv, cal_mib, cmds):
    """Writes the HBM-traffic summary of the layer GEMMs from rocprofv3 counter
    CSVs: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of one bench step, each
    scaled by bytes / counter of a device copy of cal_mib MiB."""
    import csv
    import re

    def rows(path):
        with open(path) as f:
            return list(csv.DictReader(f))

    def factor(path):
        vals = [float(r["Counter_Value"]) for r in rows(path) if "copyBuffer" in r["Kernel_Name"]]
        vals = [v for v in vals if v > 0.5 * max(vals)]
        return cal_mib * 1024.0 / (sum(vals) / len(vals))

    ff, fw = factor(cal_fetch_csv), factor(cal_write_csv)
    fr, wr = rows(fetch_csv), rows(write_csv)
    assert len(fr) == len(wr)
    per = {}
    for a, b in zip(fr, wr):
        assert a["Kernel_Name"] == b["Kernel_Name"]
        name = a["Kernel_Name"]
        m = re.search(LAYER_GEMM_RE, name)
        if not m:
            continue
        key = m.group(0)
        e = per.setdefault(key, [0, 0.0, 0.0])
        e[0] += 1
        e[1] += float(a["Counter_Value"]) * 1024.0 * ff
        e[2] += float(b["Counter_Value"]) * 1024.0 * fw
    n = sum(e[0] for e in per.values())
    tot = sum(e[1] + e[2] for e in per.values())
    rec = {"workload": "wide", "kernel": "layer GEMMs (qkv, out_proj, fc1, fc2, proj1, proj2)",
           "launches": n, "bytes_per_launch": tot / n,
           "fetch_factor": ff, "write_factor": fw, "source_sha256": gemm_source_sha()}
    out = ["# HBM traffic of the layer GEMMs: wide workload, bf16, one forward step", "",
           "Counters FETCH_SIZE and WRITE_SIZE (KiB per dispatch) from two rocprofv3 runs, each",
           f"scaled by what the same counter reads for a {cal_mib} MiB device-to-device copy",
           f"(bytes / counter: fetch {ff:.3f}, write {fw:.3f}).", "", "Commands (from /tmp, TMPDIR=/tmp):", "", "```"]
    out += cmds + ["```", "",
                   "| kernel | launches | fetch MB / launch | write MB / launch |", "|---|---|---|---|"]
    for k, (c, f, w) in sorted(per.items()):
        out.append(f"| `{k}` | {c} | {f / c / 1e6:.1f} | {w / c / 1e6:.1f} |")
    out += ["", f"All layer GEMMs: {n} launches, {tot / n / 1e6:.1f} MB per launch.", "",
            "```json", json.dumps(rec, indent=1), "```", ""]
    with open(TRAFFIC_FILE, "w") as f:
        f.write("\n".join(out))
    print("\n".join(out))


def logmel_rate(aut, torch, frame_lens, reps=10):
    """The step before the encoder: the same batch's audio (16 kHz, 160 samples
    per frame; seeded speech-like stand-in) to log-mel on the GPU
    (aut_logmel). Algorithmic flops: the windowed DFT as a [frames x 400] x
    [400 x 416] product plus the [frames x 208] x [208 x 128] filterbank, fp32
    on the matrix cores (peak 157.3 TFLOP/s)."""
    n = np.asarray(frame_lens, dtype=np.int64) * 160
    audio = torch.from_numpy(si.audio_samples(n, seed=8)).cuda()
    tables = aut.logmel_tables()
    T_max = (int(max(n)) // 160 + 3) // 4 * 4
    feats = torch.empty((len(n), 128, T_max), dtype=torch.float32, device="cuda")
    ws = torch.empty(1 << 16, dtype=torch.uint8, device="cuda")
    aut.logmel(audio, n, tables, feats, ws=ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        aut.logmel(audio, n, tables, feats, ws=ws)
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0) / reps
    frames = float(np.sum(n // 160))
    flops = frames * (2.0 * 400 * 416 + 2.0 * 208 * 128)
    return {"frames": int(frames), "audio_seconds": frames / 100.0, "ms": ms,
            "audio_s_per_s": frames / 100.0 / (ms * 1e-3), "tflops": flops / (ms * 1e-3) / 1e12,
            "peak_tflops": PEAK_FP32_TFLOPS, "frac": flops / (ms * 1e-3) / 1e12 / PEAK_FP32_TFLOPS,
            "note": "wall time per call over back-to-back calls, incl. the length upload"}


def inject_rate(aut, torch, out, reps=20):
    """The step after the encoder: the batch's [T, 2048] fp32 output rows into
    a bf16 decoder sequence of T + 512 rows at placeholder positions
    (aut_inject_audio). Algorithmic bytes: fp32 rows read, bf16 rows written,
    row indices read."""
    T, D = out.shape
    S = T + 512
    rng = np.random.default_rng(3)
    rows = torch.from_numpy(np.sort(rng.choice(S, size=T, replace=False)).astype(np.int32)).cuda()
    dst = torch.zeros((S, D), dtype=torch.bfloat16, device="cuda")
    aut.inject_audio(out, rows, dst, "bf16")
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        aut.inject_audio(out, rows, dst, "bf16")
    e1.record()
    torch.cuda.synchronize()
    us = 1e3 * e0.elapsed_time(e1) / reps
    nbytes = T * D * 4 + T * D * 2 + T * 4
    return {"rows": int(T), "dim": int(D), "us": us, "gbs": nbytes / (us * 1e-6) / 1e9,
            "peak_gbs": PEAK_HBM_GBS, "frac": nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS}


def graph_rate(aut, torch, cfg, pl, fd, packed, dtype, eager_out, steps, audio_s):
    """The planned forward as a HIP graph: the plan is built and uploaded once,
    outside; aut_encode_planned (kernels only) is captured once and replayed
    `steps` times between two synchronisations. The replay's output is checked
    bit for bit against the eager forward's."""
    ws = aut.workspace(cfg, pl, dtype)
    out = torch.full_like(eager_out, float("nan"))
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        aut.plan_upload(pl, ws, stream=side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        aut.encode_planned(cfg, pl, fd, packed, dtype, out, ws, stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    same = bool(torch.equal(out, eager_out))
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000.0 / steps
    T = pl.total_tokens
    del g, ws
    return {"ms_per_step": ms, "tokens_per_s": T / (ms / 1e3), "audio_s_per_s": audio_s / (ms / 1e3),
            "replays": steps, "bit_identical_to_eager": same,
            "note": "aut_encode_planned captured once in a HIP graph, plan built and uploaded once "
                    "outside; wall time per replay between two synchronisations"}


def workload_rate(aut, torch, name, steps):
    """Another full-size workload of the same model (long: one 1200 s request;
    conc: 512 log-normal requests), its own seeded inputs and parameters:
    eager aut_encode steps (plan, upload, kernels) and the forward captured
    once in a HIP graph with the plan built and uploaded once outside (the
    fixed-plan replay), each timed between two synchronisations."""
    cfg_d, lens, feats, P = si.workload(name)
    cfg_d = dict(cfg_d, conv_chunksize=max(cfg_d["conv_chunksize"], 4096))
    dtype = cfg_d["dtype"]
    cfg = aut.config(cfg_d)
    dev = {k: torch.from_numpy(v).cuda() for k, v in P.items()}
    packed = aut.weights_pack(cfg, dev, dtype)
    del dev
    fd = torch.from_numpy(feats).cuda()
    pl = aut.plan(cfg, lens)
    T = pl.total_tokens
    audio_s = float(np.sum(lens)) / 100.0
    ws = aut.workspace(cfg, pl, dtype)
    out = torch.empty((T, cfg.output_dim), dtype=torch.float32, device="cuda")
    for _ in range(2):
        aut.encode(cfg, fd, lens, packed, dtype, out=out, ws=ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        aut.encode(cfg, fd, lens, packed, dtype, out=out, ws=ws)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000.0 / steps
    del ws
    res = {"workload": f"{name}: {DESCR[name]}", "requests": int(len(lens)), "total_tokens": int(T),
           "audio_seconds": audio_s, "n_windows": int(pl.n_windows), "steps": steps,
           "ms_per_step": ms, "tokens_per_s": T / (ms / 1e3), "audio_s_per_s": audio_s / (ms / 1e3),
           "dtype": dtype}
    res["graph_replay"] = graph_rate(aut, torch, cfg, pl, fd, packed, dtype, out, steps, audio_s)
    del out, packed, fd
    torch.cuda.empty_cache()
    return res


def stream_latency(aut, torch, cfg, packed, dtype, feats, steps, append=100):
    """Incremental encode of one live request (the workload's first request's
    mel, repeated as needed) receiving `append` frames per step: each step
    re-encodes from the first non-final window (aut_encode_stream). Reports the
    per-step latency; not part of `value`."""
    mel = np.ascontiguousarray(np.nan_to_num(feats[0], nan=-4.0))
    total = steps * append
    reps = -(-total // mel.shape[1])
    full = np.tile(mel, (1, reps))[:, :total]
    fdev = torch.from_numpy(np.ascontiguousarray(full)).cuda()
    rows_max = aut.stream_plan(cfg, total, 0)["rows"]
    out = torch.empty((rows_max, cfg.output_dim), dtype=torch.float32, device="cuda")
    ws = aut.stream_workspace(cfg, total, dtype)
    times = []
    wf = 0
    for k in range(1, steps + 1):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        wf = aut.encode_stream(cfg, fdev, k * append, wf, packed, dtype, out, ws)
        torch.cuda.synchronize()
        times.append(1e3 * (time.perf_counter() - t0))
    t = np.array(times[1:])
    return {"append_frames": append, "steps": steps, "request_seconds": total / 100.0,
            "step_ms_p50": float(np.percentile(t, 50)), "step_ms_p95": float(np.percentile(t, 95)),
            "rtf_p50": float(np.percentile(t, 50)) / (1e3 * append / 100.0),
            "note": "wall time per step from an idle stream to its end, incl. the plan upload; one "
                    "request, re-encodes at most one 8 s window plus the new chunks"}


PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 (MX-fp8) matrix peak


def fp8_rate(aut, torch, cfg_d, P, fd, lens, steps, mask):
    """The same workload under AUT_FP8 with the products of `mask` on MX-fp8
    operands: ms per step and the fp8 products' rate against the fp8 peak."""
    cfg = aut.config(dict(cfg_d, fp8_gemms=mask))
    dev = {k: torch.from_numpy(v).cuda() for k, v in P.items()}
    packed = aut.weights_pack(cfg, dev, "fp8")
    del dev
    pl = aut.plan(cfg, lens)
    T = pl.total_tokens
    ws = aut.workspace(cfg, pl, "fp8")
    out = torch.empty((T, cfg.output_dim), dtype=torch.float32, device="cuda")
    for _ in range(2):
        aut.encode(cfg, fd, lens, packed, "fp8", out=out, ws=ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        aut.encode(cfg, fd, lens, packed, "fp8", out=out, ws=ws)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / steps
    # per-kernel durations from a second, instrumented pass
    aut.profile_collect()
    aut.profile_enable(True)
    for _ in range(steps):
        aut.encode(cfg, fd, lens, packed, "fp8", out=out, ws=ws)
    torch.cuda.synchronize()
    aut.profile_enable(False)
    st = aut.profile_collect()
    g8 = st["gemm_fp8"]
    res = {"fp8_gemms": mask, "ms_per_step": ms, "tokens_per_s": T / (ms / 1e3),
           "audio_s_per_s": float(np.sum(lens)) / 100.0 / (ms / 1e3)}
    if g8["launches"]:
        sec = g8["total_ms"] / 1e3
        res.update(gemm_fp8_tflops=g8["flops"] / sec / 1e12, gemm_fp8_peak=PEAK_FP8_TFLOPS,
                   gemm_fp8_frac=g8["flops"] / sec / 1e12 / PEAK_FP8_TFLOPS,
                   gemm_fp8_ms_per_step=g8["total_ms"] / steps,
                   gemm_fp8_avg_us=1e3 * g8["total_ms"] / g8["launches"])
    if st["gemm"]["launches"]:
        res["gemm_bf16_ms_per_step"] = st["gemm"]["total_ms"] / steps
    res["ms_per_step_by_class"] = {c: v["total_ms"] / steps for c, v in st.items() if v["launches"]}
    del ws, packed, out
    return res


def cpu_baseline(name, cfg_d, lens, feats, P, n_windows):
    """The float64 oracle on a bounded sample of the same workload's windows."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    pl = oracle.plan(lens, cfg_d)
    nw = len(pl["window_lengths"])
    rng = np.random.default_rng(1000 + si.workload_seed(name))
    wins = sorted({0} | set(int(w) for w in rng.choice(nw, size=min(nw, n_windows) - 1, replace=False)))
    ntok = sum(pl["window_lengths"][w] for w in wins)
    t0 = time.perf_counter()
    oracle.forward_windows(feats, lens, P, cfg_d, wins)
    dt = time.perf_counter() - t0
    res = {
        "value": ntok / dt,
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{len(wins)} windows ({ntok} tokens) of the {name} workload, windows {wins}: "
                  f"conv stem, conv_out, {cfg_d['encoder_layers']} layers and projector in float64 numpy; "
                  f"{dt:.1f} s wall",
        "audio_s_per_s": ntok / 13.0 / dt,
        "cpu_model": cpu_model(),
    }
    # the same oracle on one thread, over the first sampled window only
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:
        return res
    w1 = wins[:1]
    n1 = sum(pl["window_lengths"][w] for w in w1)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        oracle.forward_windows(feats, lens, P, cfg_d, w1)
        d1 = time.perf_counter() - t0
    res["one_thread"] = {"value": n1 / d1, "unit": "tokens/s",
                         "sample": f"window {w1[0]} ({n1} tokens), {d1:.1f} s wall"}
    return res


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="wide", choices=list(si.WORKLOADS))
    ap.add_argument("--cpu-windows", type=int, default=24)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fp8-steps", type=int, default=5,
                    help="steps of the AUT_FP8 legs (0: skip them)")
    ap.add_argument("--stream-steps", type=int, default=30,
                    help="1 s appends timed for the incremental-encode latency (0: skip)")
    ap.add_argument("--graph-steps", type=int, default=10,
                    help="replays of the forward captured in a HIP graph (0: skip)")
    ap.add_argument("--other-steps", type=int, default=5,
                    help="steps of the long and conc workloads, eager and as a fixed-plan graph replay (0: skip)")
    ap.add_argument("--no-kernel-events", action="store_true",
                    help="time the steps without per-launch HIP events (no roofline)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run 10 device-to-device copies of MIB MiB (the known-size kernel "
                         "that scales the FETCH_SIZE / WRITE_SIZE counters) and exit")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "CAL_FETCH_CSV", "CAL_WRITE_CSV"),
                    help="write the layer-GEMM HBM traffic summary from rocprofv3 counter CSVs and exit")
    ap.add_argument("--calibrate-mib", type=int, default=512)
    args = ap.parse_args()
    if args.traffic_summary:
        cmds = [f"rocprofv3 --pmc {c} -f csv -d <out> -o wide -- python <repo>/bench.py --steps 1 --warmup 0 "
                "--no-cpu-baseline --no-kernel-events --fp8-steps 0 --stream-steps 0 --other-steps 0"
                for c in ("FETCH_SIZE", "WRITE_SIZE")]
        cmds += [f"rocprofv3 --pmc {c} -f csv -d <out> -o copy -- python <repo>/bench.py --calibrate-copy "
                 f"{args.calibrate_mib}" for c in ("FETCH_SIZE", "WRITE_SIZE")]
        cmds += ["python <repo>/bench.py --traffic-summary <fetch csv> <write csv> <copy fetch csv> <copy write csv>"]
        traffic_summary(*args.traffic_summary, args.calibrate_mib, cmds)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the forward pass has no cross-GPU step here "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from packed_windowed_attention_amd import aut

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {args.calibrate_copy} MiB x 10")
        return
    name = args.workload
    log(f"generating workload {name}")
    cfg_d, lens, feats, P = si.workload(name)
    # conv-stem batch: as many chunks per launch as the kernels' 32-bit buffer
    # offsets allow (the library caps it); a memory knob with no effect on the
    # results, and fewer, fuller launches
    cfg_d = dict(cfg_d, conv_chunksize=max(cfg_d["conv_chunksize"], 4096))
    dtype = cfg_d["dtype"]
    cfg = aut.config(cfg_d)
    dev = {k: torch.from_numpy(v).cuda() for k, v in P.items()}
    packed = aut.weights_pack(cfg, dev, dtype)
    del dev
    fd = torch.from_numpy(feats).cuda()
    pl = aut.plan(cfg, lens)
    T = pl.total_tokens
    audio_s = float(np.sum(lens)) / 100.0
    ws = aut.workspace(cfg, pl, dtype)
    out = torch.empty((T, cfg.output_dim), dtype=torch.float32, device="cuda")
    log(f"T={T} tokens, {pl.n_windows} windows, {pl.n_chunks} chunks, workspace {ws.numel() / 2**30:.2f} GiB")

    def step():
        aut.encode(cfg, fd, lens, packed, dtype, out=out, ws=ws)

    for i in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done")

    events = not args.no_kernel_events
    stream = torch.cuda.current_stream()

    def timed(profiled):
        """args.steps steps between two synchronisations; per-step events on
        the stream; with `profiled`, also an event pair around every launch
        (the per-kernel durations; the markers add ~10 us between kernels, so
        the step time of that pass is not the one reported as `value`)."""
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        if profiled:
            aut.profile_collect()
            aut.profile_enable(True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            ev[k][0].record(stream)
            step()
            ev[k][1].record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        st = None
        if profiled:
            aut.profile_enable(False)
            st = aut.profile_collect()
        return (t1 - t0) * 1000.0 / args.steps, np.array([a.elapsed_time(b) for a, b in ev]), st

    ms_per_step, step_ms, _ = timed(False)
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step")
    if events:
        ms_instr, _, stats = timed(True)
        log(f"timed {args.steps} more steps with per-launch events: {ms_instr:.3f} ms/step")

    res = {
        "metric": METRIC,
        "value": T / (ms_per_step / 1000.0),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{name}: {DESCR[name]}",
            "requests": int(len(lens)),
            "total_tokens": int(T),
            "audio_seconds": audio_s,
            "n_windows": int(pl.n_windows),
            "n_chunks": int(pl.n_chunks),
            "parallelism": "single GPU",
        },
        "audio_s_per_s": audio_s / (ms_per_step / 1000.0),
        "latency_ms": {q: float(np.percentile(step_ms, p)) for q, p in (("p50", 50), ("p95", 95), ("p99", 99))},
    }
    if events:
        peak = PEAK_BF16_TFLOPS if dtype == "bf16" else PEAK_FP32_TFLOPS
        kern = {}
        for cls, s in stats.items():
            if s["launches"] == 0:
                continue
            sec = s["total_ms"] / 1e3
            kern[cls] = {"launches": s["launches"], "ms_per_step": s["total_ms"] / args.steps,
                         "avg_us": 1e3 * s["total_ms"] / s["launches"],
                         "tflops": s["flops"] / sec / 1e12 if sec else None,
                         "gbs": s["bytes"] / sec / 1e9 if sec else None}
        res["kernels"] = kern
        res["ms_per_step_with_launch_events"] = ms_instr
        g = stats["gemm"]
        a = stats["attention"]
        g_sec = g["total_ms"] / 1e3
        res["roofline"] = {
            "kernel": "gemm (qkv, out_proj, fc1, fc2, proj1, proj2)",
            "bound": "mfma",
            "achieved": g["flops"] / g_sec / 1e12,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": g["flops"] / g_sec / 1e12 / peak,
            "traffic": stored_traffic(name),
            "flops_per_launch": g["flops"] / g["launches"],
            "algorithmic_bytes_per_launch": g["bytes"] / g["launches"],
            "avg_launch_us": 1e6 * g_sec / g["launches"],
        }
        mf = [stats[c] for c in ("gemm", "attention")]
        res["mfma_frac_gemm_attn"] = (sum(s["flops"] for s in mf) / (sum(s["total_ms"] for s in mf) / 1e3)
                                      / 1e12 / peak)
        allf = sum(s["flops"] for c, s in stats.items() if c != "layernorm" and c != "gemm_fp8")
        res["mfma_frac_step"] = allf / args.steps / (ms_per_step / 1e3) / 1e12 / peak
        res["attention_gbs"] = a["bytes"] / (a["total_ms"] / 1e3) / 1e9 if a["total_ms"] else None
    if args.graph_steps > 0:
        res["graph_replay"] = graph_rate(aut, torch, cfg, pl, fd, packed, dtype, out, args.graph_steps, audio_s)
        log(f"graph replay: {res['graph_replay']['ms_per_step']:.3f} ms/step, "
            f"bit-identical to eager: {res['graph_replay']['bit_identical_to_eager']}")
    if args.other_steps > 0 and name == "wide":
        res["other_workloads"] = []
        for other in ("long", "conc"):
            r = workload_rate(aut, torch, other, args.other_steps)
            res["other_workloads"].append(r)
            log(f"{other}: {r['ms_per_step']:.2f} ms/step eager, {r['graph_replay']['ms_per_step']:.2f} ms "
                f"graph replay, {r['graph_replay']['tokens_per_s'] / 1e3:.0f} k tokens/s")
    res["logmel"] = logmel_rate(aut, torch, lens)
    log(f"logmel: {res['logmel']['ms']:.3f} ms for {res['logmel']['audio_seconds']:.0f} s of audio")
    res["inject"] = inject_rate(aut, torch, out)
    log(f"inject: {res['inject']['us']:.1f} us, {res['inject']['gbs']:.0f} GB/s")
    if args.stream_steps > 0:
        res["stream"] = stream_latency(aut, torch, cfg, packed, dtype, feats, args.stream_steps)
        log(f"stream: {res['stream']['step_ms_p50']:.3f} ms per 1 s append (p50)")
    if args.fp8_steps > 0 and dtype == "bf16":
        # the conv stem on MX-fp8 (the one product class whose quantisation
        # keeps every token's cosine to the unquantised encoder above the
        # pages' 0.999 at 24 layers), then every product on MX-fp8 (conv stem,
        # layers, projector: the fastest, below that bar)
        res["fp8"] = [fp8_rate(aut, torch, cfg_d, P, fd, lens, args.fp8_steps, m) for m in (32, 63)]
        for r in res["fp8"]:
            r["per_token_cosine_above_0.999"] = r["fp8_gemms"] == 32
            log(f"fp8 mask {r['fp8_gemms']}: {r['ms_per_step']:.3f} ms/step, "
                f"fp8 products {r.get('gemm_fp8_tflops', 0):.0f} TFLOP/s")
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on sampled windows)")
        res["cpu_baseline"] = cpu_baseline(name, cfg_d, lens, feats, P, args.cpu_windows)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
