#!/usr/bin/env python3
"""Throughput of the fused mel-spectrogram forward pass on one MI355X.

A step is one fm_forward launch over one whole batch of the chosen workload
(default: 8 x 480000 float32 samples, n_fft 400, hop 160, 128 HTK mels, the
Whisper-shaped case).  Inputs are resident in HBM before timing starts.  To
keep the 256 MB Infinity Cache from serving the data, the steps rotate over
enough input/output buffer sets to exceed 2 x 256 MB.

With --backward a step is one fm_backward launch instead (the gradient of
sum(grad_out * mel(x)) with respect to the float32 signal), over the same
rotation of buffer sets (signal, output gradient, signal gradient); its
algorithmic bytes are the signal and the output gradient read plus the
signal gradient written.

Prints ONE JSON line (rank 0, N = 1):
  value        mel frames per second over the K timed steps (events around
               the whole timed region, torch's current stream);
  roofline     achieved HBM GB/s of the kernel: algorithmic bytes (input +
               output) / the average launch duration over the timed region
               (events on the launch stream around K back-to-back launches),
               against 8 TB/s;
  cpu_baseline the f64 oracle timed on this host on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from stft_mel_spectrogram_amd import workloads as W  # noqa: E402

HBM_PEAK_GBPS = 8000.0
METRIC = "mel frames/sec and achieved HBM GB/s (% roofline), 8×480000 n_fft=400 128 mels"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="whisper", choices=sorted(W.WORKLOADS))
    ap.add_argument("--sets", type=int, default=0, help="rotating buffer sets (0: enough for 512 MB)")
    ap.add_argument("--out-dtype", default="f32", choices=["f32", "f16"],
                    help="output element type (f16: the f32 result rounded at the store)")
    ap.add_argument("--backward", action="store_true",
                    help="time fm_backward (gradient w.r.t. the signal) instead of the forward")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-copy-probe", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle sample")
    ap.add_argument("--oracle-table", action="store_true",
                    help="time only the oracle, on each of the five benchmark workloads (median "
                         "of 3 bounded samples each); one JSON line per workload, no GPU use")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="measured HBM bytes per launch (from rocprofv3 --pmc), if present")
    return ap.parse_args()


def host_cpu() -> dict:
    """The host the oracle runs on: logical CPUs, CPU model, BLAS threads."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max([i.get("num_threads", 1) for i in blas] or [1])
        lib = ",".join(sorted({f"{i.get('internal_api')} {i.get('version')}" for i in blas})) or None
    except Exception:  # pragma: no cover
        threads, lib = 1, None
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):  # pragma: no cover
        affinity = None
    return {"cpu_count": os.cpu_count(), "cpu_affinity": affinity, "cpu_model": model,
            "blas_threads": int(threads), "blas": lib}


def cpu_baseline(cfg: dict, budget_s: float, backward: bool = False) -> dict:
    """The oracle as it stands, on whole signals of the workload, repeated
    until about `budget_s` seconds of CPU work; frames/s (with `backward`,
    the oracle's vector-Jacobian product).  `cores` is the number of BLAS
    threads the oracle's products run on (the rest of it is one thread)."""
    from oracle import mel_oracle as O
    host = host_cpu()
    threads = host["blas_threads"]
    targs = W.transform_args(cfg)
    x = W.make_signal(W.workload(cfg["name"], batch=1))
    if backward:
        T = O.frame_count(x.shape[-1], targs["n_fft"], targs["hop_length"], targs.get("center", True),
                          targs.get("pad", 0))
        u = np.random.default_rng(1).standard_normal((1, targs["n_mels"], T))
    t0 = time.perf_counter()
    frames = 0
    runs = 0
    while True:
        if backward:
            O.mel_spectrogram_vjp(x, u, **targs)
            frames += T
        else:
            y = O.mel_spectrogram(x, **targs)
            frames += y.shape[0] * y.shape[-1]
        runs += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": frames / dt, "unit": "frames/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{runs} x one {cfg['length']}-sample signal of the {cfg['name']} workload "
                      f"({'backward, ' if backward else ''}"
                      f"{frames} frames, {dt:.1f} s, numpy f64 with BLAS threads)",
            **host}


def oracle_table(budget_s: float) -> None:
    """The oracle's forward rate on each of the five benchmark workloads:
    three bounded samples each (whole signals, about `budget_s` seconds per
    sample), the median printed as one JSON line per workload."""
    for name in ("tiny", "whisper", "int16", "pow2", "large"):
        cfg = W.workload(name)
        runs = [cpu_baseline(cfg, budget_s) for _ in range(3)]
        vals = sorted(r["value"] for r in runs)
        print(json.dumps({"workload": name, "oracle_frames_per_s_median": vals[1],
                          "runs": vals, "sample": runs[1]["sample"],
                          **{k: runs[0][k] for k in ("cores", "cpu_count", "cpu_affinity",
                                                      "cpu_model", "blas_threads", "blas")}}),
              flush=True)


def copy_probe(torch, dev, nbytes: int, reps: int = 50) -> dict:
    """Device-to-device copy of a known size (torch's copy kernel), rotating
    over buffers larger than the Infinity Cache: the measured copy peak, and
    the reference kernel for scaling HBM byte counters."""
    n = nbytes // 4
    sets = max(2, int(np.ceil(2 * 256e6 / (2 * nbytes))) + 1)
    src = [torch.ones(n, device=dev) for _ in range(sets)]
    dst = [torch.empty(n, device=dev) for _ in range(sets)]
    for i in range(5):
        dst[i % sets].copy_(src[i % sets])
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(reps):
        dst[i % sets].copy_(src[i % sets])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return {"bytes_read": n * 4, "bytes_written": n * 4, "ms": ms,
            "gbps": 2 * n * 4 / (ms * 1e-3) / 1e9}


def kernel_sources_hash() -> str:
    """sha256[:16] of the library sources with comments and whitespace
    removed, so that only a change of code invalidates measured counters."""
    import glob
    import hashlib
    import re
    m = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "stft_mel_spectrogram_amd", "csrc", "*"))):
        src = open(f, encoding="utf-8", errors="replace").read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)       # block comments
        src = re.sub(r"//[^\n]*", " ", src)                       # line comments
        m.update(os.path.basename(f).encode())
        m.update(" ".join(src.split()).encode())
    return m.hexdigest()[:16]


def sleep_rate(torch) -> float:
    """Cycles of torch.cuda._sleep per millisecond on this device."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    torch.cuda._sleep(2_000_000)
    e1.record()
    torch.cuda.synchronize()
    return 2_000_000 / max(e0.elapsed_time(e1), 1e-3)


def main():
    args = parse()
    if args.oracle_table:
        oracle_table(args.cpu_seconds)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(frames are independent: a batch would shard across GPUs with no exchange).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from stft_mel_spectrogram_amd import MelSpectrogram

    cfg = W.workload(args.workload)
    x_np = W.make_signal(cfg)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    out_dt = torch.float16 if args.out_dtype == "f16" else torch.float32
    mel = MelSpectrogram(device=dev, out_dtype=out_dt, **W.transform_args(cfg))
    B, L = x_np.shape
    T = mel.out_frames(L)
    in_bytes = x_np.nbytes
    out_bytes = B * cfg["n_mels"] * T * (2 if args.out_dtype == "f16" else 4)
    if args.backward:
        if x_np.dtype != np.float32 or args.out_dtype != "f32":
            print("--backward needs a float32 workload and f32 gradients", file=sys.stderr)
            sys.exit(2)
        algo_bytes = in_bytes + out_bytes + in_bytes   # x, grad_out read; grad_x written
    else:
        algo_bytes = in_bytes + out_bytes
    frames = B * T

    sets = args.sets or max(2, int(np.ceil(2 * 256e6 / algo_bytes)) + 1)
    x0 = torch.from_numpy(x_np).to(dev)
    xs = [x0] + [x0.clone() for _ in range(sets - 1)]
    ys = [torch.empty((B, cfg["n_mels"], T), dtype=out_dt, device=dev) for _ in range(sets)]
    if args.backward:
        g0 = torch.from_numpy(np.random.default_rng(11).standard_normal((B, cfg["n_mels"], T))
                              .astype(np.float32)).to(dev)
        for y in ys:
            y.copy_(g0)            # the output gradients
        dxs = [torch.empty((B, L), dtype=torch.float32, device=dev) for _ in range(sets)]

        def step(i):
            mel.backward(xs[i % sets], ys[i % sets], out=dxs[i % sets])
    else:
        def step(i):
            mel(xs[i % sets], out=ys[i % sets])
    stream = torch.cuda.current_stream(dev)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # The launches are queued behind a GPU sleep, so the device runs them
    # back to back however long the host takes to enqueue them; the events
    # then time device execution, not Python call overhead.
    cyc_per_ms = sleep_rate(torch)

    def queued(fn, n_launch):
        est_host_ms = 0.08 * n_launch + 5.0
        torch.cuda._sleep(int(cyc_per_ms * est_host_ms))
        t_host = time.perf_counter()
        fn()
        t_host = (time.perf_counter() - t_host) * 1e3
        torch.cuda.synchronize()
        return t_host, est_host_ms

    # (1) throughput: events around the whole timed region
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)

    def timed_steps():
        ev0.record(stream)
        for i in range(args.steps):
            step(i)
        ev1.record(stream)

    torch.cuda.synchronize()
    host_ms, budget_ms = queued(timed_steps, args.steps)
    total_ms = ev0.elapsed_time(ev1)
    ms_per_step = total_ms / args.steps
    queued_ok = host_ms < budget_ms

    # (2) per-launch kernel duration: an event pair around every launch
    n_k = min(args.steps, 200)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n_k)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n_k)]

    def timed_each():
        for i in range(n_k):
            starts[i].record(stream)
            step(i)
            ends[i].record(stream)

    torch.cuda.synchronize()
    queued(timed_each, n_k)
    durs = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
    pair_ms = float(np.mean(durs))
    # The kernel's average launch duration: the timed region over K queued,
    # back-to-back launches (event pairs around single launches add the
    # markers' own cost and are reported alongside).
    kern_ms = ms_per_step
    achieved = algo_bytes / (kern_ms * 1e-3) / 1e9

    # (3) for reference: the same steps driven from the host with no queue
    torch.cuda.synchronize()
    t = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    host_loop_ms = (time.perf_counter() - t) * 1e3 / args.steps

    # Measured HBM bytes per launch (rocprofv3 FETCH_SIZE/WRITE_SIZE, scaled
    # by a copy kernel of known size), valid only for the kernel sources
    # they were taken from.
    traffic = None
    if os.path.exists(args.traffic_json):
        try:
            for t in json.load(open(args.traffic_json)).get("entries", []):
                if (t.get("workload") == cfg["name"] and t.get("out_dtype", "f32") == args.out_dtype
                        and bool(t.get("backward", False)) == args.backward
                        and t.get("kernel_sources_sha256_16") == kernel_sources_hash()):
                    traffic = t.get("bytes_per_launch")
        except Exception:
            traffic = None

    res = {
        "metric": ("backward (gradient w.r.t. the signal): " + METRIC) if args.backward else METRIC,
        "value": frames / (ms_per_step * 1e-3),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",   # arithmetic type of the path; input/output types are in config
        "data": "synthetic (seeded; see workloads.py)",
        "config": {"workload": f"{cfg['name']}: {B}x{L} {cfg['dtype']}, n_fft={cfg['n_fft']} "
                               f"hop={cfg['hop_length']} {cfg['n_mels']} mels, power={cfg['power']}, "
                               f"{args.out_dtype} out" + (", backward" if args.backward else ""),
                   "batch": B, "length": L, "n_frames": T, "buffer_sets": sets,
                   "in_dtype": cfg["dtype"], "out_dtype": args.out_dtype,
                   "parallelism": "single GPU"},
        "hbm_gbps_step": algo_bytes / (ms_per_step * 1e-3) / 1e9,
        "kernel_ms_mean": kern_ms,
        "kernel_ms_event_pairs": pair_ms,
        "host_loop_ms_per_step": host_loop_ms,
        "launches_queued_ahead": bool(queued_ok),
        "kernel_ms_median": float(np.median(durs)),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "algorithmic_bytes": algo_bytes},
    }
    if not args.no_copy_probe:
        res["copy_probe"] = copy_probe(torch, dev, in_bytes)
        res["copy_probe_large"] = copy_probe(torch, dev, 512 << 20, reps=20)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds, args.backward)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
