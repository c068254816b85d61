#!/usr/bin/env python3
"""Throughput of the 128-bin log-mel front end on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2|c4|c3|c1|p3]
                    [--in-rate R]  (c2 made at R Hz, resampled to 16 kHz in the step)

Prints one JSON line. A step is one logmel_compute over one batch of
synthetic input already resident in HBM: framing, window, rFFT, power, mel
and log for every frame of the batch (frame offsets are computed once, on
the host, before the timed region). The default workload is the offline
batch of 64 speech-like 30 s clips (64 x 480000 fp32 samples); the timed
loop rotates over 5 copies of input and output buffers (1.1 GB) so that
successive steps do not hit in the 256 MB Infinity Cache.

``dtype`` names the arithmetic of the path: the window and the transform in fp64 (the filterbank
and the log in fp32). ``value`` is audio-seconds per second (sum of samples / 16000 per step,
divided by the wall time per step, measured between device synchronisations
around exactly K steps). ``roofline`` is the HBM roofline the target is set
against: ``achieved`` is the algorithmic HBM bytes per launch (4 B per input
sample + 512 B per output frame + the offsets) divided by the kernel's average
launch duration, the timed region's time per launch from one pair of HIP events
around all the back-to-back launches on the stream it runs on (the profiler's
kernel trace of the same run agrees), against 8 TB/s; pairs around every 8th
launch (--event-every) add the per-launch median and minimum and read a few
microseconds higher (they also time the dispatch and their own packets). ``traffic`` is
the measured HBM bytes per launch from the
committed counter summary; the vector-ALU figures (this implementation's
algorithmic flops per launch against the 78.6 TFLOP/s vector peak) ride along
as ``alu_*`` keys. The default run also times the ragged long batch (200
clips, 0.5 s to 87 min) and reports it as the nested ``c4`` record.
``cpu_baseline`` times the fp64 oracle on the host cores over the same clips
(a bounded sample: repeated passes for about --cpu-seconds seconds).
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# MI355X vector ALU: 256 CUs x 4 SIMDs x 16 lanes x 2 flops (FMA) x 2.4 GHz.
# fp64 FMA runs at this rate, as does fp32 without packed instructions.
ALU_PEAK_TFLOPS = 78.6
# Algorithmic floating-point work per frame of this implementation (FMA = 2):
# fp64: window 400, 16 real-input 25-point DFTs 16 x 264, 26 8-point DFTs
# (two of them on real input) 2 x 702, even/odd combine and power 2 x 1100
# -> 8228; fp32: filterbank 664, log scaling 124 -> 788.
FLOPS_PER_FRAME = 8228 + 788
FS = 16000


TILES_SOURCES = ("logmel_kernels.hip", "logmel_tile.h", "logmel_frame.h", "logmel_launch.h",
                 "gen_tables.py")
# the resampler's counters also depend on its geometry and taps, built in
# the C-ABI layer
RESAMPLE_SOURCES = ("logmel_resample.hip", "logmel_resample_launch.h", "logmel_api.cpp")


def kernel_source_hash(files=TILES_SOURCES):
    """Hash of the kernel sources with comments and blank space removed, so
    that a comment edit does not invalidate a counter summary."""
    import re
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "log_mel_spectrogram_amd", "csrc", f)) as fh:
            text = fh.read()
        if f.endswith(".py"):
            text = re.sub(r"#[^\n]*", "", text)
            text = re.sub(r'"""(.|\n)*?"""', "", text)
        else:
            text = re.sub(r"/\*(.|\n)*?\*/", "", text)
            text = re.sub(r"//[^\n]*", "", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(profile, files=TILES_SOURCES):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    profiles/<profile>_pmc.md, if it was taken on the current kernel source;
    else None."""
    path = os.path.join(ROOT, "profiles", f"{profile}_pmc.md")
    if not os.path.exists(path):
        return None
    rec = None
    for line in open(path):
        if line.startswith("TRAFFIC_JSON "):
            rec = json.loads(line[len("TRAFFIC_JSON "):])
    if not rec or rec.get("kernel_source_hash") != kernel_source_hash(files):
        return None
    return rec.get("hbm_bytes_per_launch")


# ------------------------------------------------------------ CPU baseline

def _oracle_worker(args):
    import numpy as np
    x, reps = args
    from oracle import logmel_clip
    for _ in range(reps):
        logmel_clip(x)
    return 0


def host_cores():
    """(cores to use, cores in the affinity mask). The GPU machine gives each GPU
    a share of the host's cores and states it in OMP_NUM_THREADS (16 for one
    GPU); the affinity mask may list more, which belong to other shares.
    Every core of the share is used."""
    aff = len(os.sched_getaffinity(0))
    share = os.environ.get("OMP_NUM_THREADS", "")
    n = min(aff, int(share)) if share.isdigit() and int(share) > 0 else aff
    return n, aff


def cpu_baseline(clips, seconds):
    """fp64 oracle over the given clips (list of numpy fp32 arrays) on a
    process pool of the host cores of this GPU's share, one BLAS thread each."""
    import multiprocessing as mp
    cores, aff = host_cores()
    for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[v] = "1"
    ctx = mp.get_context("spawn")
    audio_per_pass = sum(c.size for c in clips) / FS
    with ctx.Pool(cores) as pool:
        pool.map(_oracle_worker, [(clips[i % len(clips)], 1) for i in range(cores)])  # warm
        # calibrate on a few passes (one pass is too short against the pool's overhead)
        t0 = time.perf_counter()
        pool.map(_oracle_worker, [(c, 4) for c in clips])
        one = (time.perf_counter() - t0) / 4
        reps = max(1, int(seconds / max(one, 1e-3)))
        t0 = time.perf_counter()
        pool.map(_oracle_worker, [(c, reps) for c in clips])
        dt = time.perf_counter() - t0
    # one core, in this process, for about 2 s
    from oracle import logmel_clip
    done, k = 0.0, 0
    t1 = time.perf_counter()
    while True:
        c = clips[k % len(clips)]
        logmel_clip(c)
        done += c.size / FS
        k += 1
        if time.perf_counter() - t1 > 2.0:
            break
    dt1 = time.perf_counter() - t1
    return {
        "value": audio_per_pass * reps / dt,
        "unit": "audio-seconds/s",
        "cores": cores,
        "affinity_cores": aff,
        "kind": "oracle",
        "sample": f"{len(clips)} clips of the workload ({audio_per_pass:.0f} audio-s), "
                  f"{reps} passes, {dt:.1f} s wall",
        "one_core_value": done / dt1,
        "one_core_sample": f"{k} clips, {dt1:.1f} s",
        "cpu_model": _cpu_model(),
    }


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def copy_bandwidth(torch, dev, nbytes=1 << 30, reps=5):
    """Device-to-device copy of nbytes (read + write) timed with HIP events:
    the bandwidth a plain streaming kernel reaches on this GPU, in GB/s."""
    a = torch.empty(nbytes // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    a.fill_(1.0)
    b.copy_(a)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) / 1e3)
    del a, b
    torch.cuda.empty_cache()
    return 2 * nbytes / sorted(ts)[len(ts) // 2] / 1e9


# ---------------------------------------------------------------- workloads

def make_workload(name, device):
    import logmel_synth as S
    if name == "c2":
        x, so = S.config2(device=device)
        desc = "offline batch: 64 speech-like clips x 30 s (480000 fp32 samples each), packed"
    elif name == "c1":
        x, so = S.config1(device=device)
        desc = "1 speech-like clip, 30 s (480000 fp32 samples)"
    elif name == "p3":
        # the shape of the transcribe.cpp page's timing: one 11-s clip
        x, so = S.pack([176000], lambda i, v: S.speech_like(7, 176000, device, out=v), device)
        desc = "1 speech-like clip, 11 s (176000 fp32 samples, 1098 frames)"
    elif name == "c4":
        x, so = S.config4(device=device)
        desc = ("ragged long batch: 200 speech-like clips, log-uniform 0.5 s..87 min, "
                "packed with int64 offsets")
    else:
        raise ValueError(name)
    return x, so, desc


def bench_offline(args, lm, plan, torch):
    import numpy as np
    dev = torch.device("cuda", 0)
    x, so, desc = make_workload(args.workload, dev)
    fo = lm.logmel_frame_offsets(so)
    total = int(fo[-1])
    n_samples = int(so[-1])
    so_d = torch.from_numpy(so).to(dev)
    fo_d = torch.from_numpy(fo).to(dev)
    chunked = args.layout == "chunked"
    in_i16 = args.in_dtype == "i16"
    out_f16 = args.out_dtype == "f16"
    if in_i16:
        # int16 PCM of the same signal (s / 32768 is what the kernel computes on)
        x = torch.clamp(torch.round(x * 32768.0), -32768, 32767).to(torch.int16)
        desc += "; int16 PCM input"
    if out_f16:
        desc += "; fp16 output"
    out_dtype = torch.float16 if out_f16 else torch.float32
    if chunked:
        co = lm.logmel_chunk_offsets(so)
        n_chunks = int(co[-1])
        co_d = torch.from_numpy(co).to(dev)
        out_rows = n_chunks * lm.CHUNK_FRAMES
        desc += "; 30-s chunk layout [chunks, 3000, 128]"
    else:
        out_rows = total
    set_bytes = (2 if in_i16 else 4) * n_samples + (256 if out_f16 else 512) * out_rows
    n_sets = max(1, min(5, int(math.ceil(1.1e9 / set_bytes)))) if args.workload != "c4" else 1
    if args.workload == "p3":
        n_sets = 1   # a latency run: the one clip, resident
    xs = [x] + [x.clone() for _ in range(n_sets - 1)]
    if chunked:
        outs = [torch.empty((n_chunks, lm.CHUNK_FRAMES, 128), dtype=out_dtype, device=dev)
                for _ in range(n_sets)]
    else:
        outs = [torch.empty((total, 128), dtype=out_dtype, device=dev) for _ in range(n_sets)]
    stream = torch.cuda.current_stream(dev)
    general = in_i16 or out_f16

    def step(k):
        if general:
            lm.logmel_compute_ex(plan, xs[k], so_d, fo_d, total,
                                 chunk_offsets=co_d if chunked else None,
                                 total_chunks=n_chunks if chunked else 0, out=outs[k],
                                 stream=stream)
        elif chunked:
            lm.logmel_compute_chunked(plan, xs[k], so_d, fo_d, co_d, total, n_chunks, out=outs[k],
                                      stream=stream)
        else:
            lm.logmel_compute(plan, xs[k], so_d, fo_d, total, out=outs[k], stream=stream)

    for i in range(args.warmup):
        step(i % n_sets)
    torch.cuda.synchronize()
    # Events recorded around a launch put their own packets between the
    # kernels and lengthen the step (about 8 us per step on the batch of 64
    # clips), so only every event_every-th launch of a long run carries a
    # pair; one more pair brackets the whole timed region.
    every = args.event_every if args.steps >= 2 * args.event_every else 1
    timed = [i for i in range(args.steps) if i % every == 0]
    starts = {i: torch.cuda.Event(enable_timing=True) for i in timed}
    ends = {i: torch.cuda.Event(enable_timing=True) for i in timed}
    region = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    region[0].record(stream)
    for i in range(args.steps):
        if i in starts:
            starts[i].record(stream)
        step(i % n_sets)
        if i in ends:
            ends[i].record(stream)
    region[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [starts[i].elapsed_time(ends[i]) for i in timed]
    stream_us_per_launch = region[0].elapsed_time(region[1]) * 1e3 / args.steps
    # The kernel's average launch duration: the timed region's time per
    # launch (one event pair around all the back-to-back launches, which the
    # profiler's kernel trace matches); the pairs around single launches also
    # time the command processor's dispatch and their own packets, and read a
    # few microseconds higher (reported beside it).
    sampled_avg_s = sum(kern_ms) / len(kern_ms) / 1e3
    kern_avg_s = stream_us_per_launch / 1e6
    kern_sorted = sorted(kern_ms)
    kern_med_s = kern_sorted[len(kern_sorted) // 2] / 1e3
    kern_min_s = kern_sorted[0] / 1e3
    copy_gbs = copy_bandwidth(torch, dev) if args.workload != "p3" else None
    algo_bytes = set_bytes + 8 * 2 * (len(so))
    ms_per_step = wall / args.steps * 1e3
    audio_s = n_samples / FS
    achieved_gbs = algo_bytes / kern_avg_s / 1e9
    achieved_tflops = FLOPS_PER_FRAME * total / kern_avg_s / 1e12
    traffic = measured_traffic(f"logmel_tiles_{args.workload}") if not (chunked or general) else None
    rec = {
        "metric": "audio-seconds/sec of 128-bin log-mel on 1 MI355X + % of HBM roofline",
        "value": audio_s / (ms_per_step / 1e3),
        "unit": "audio-seconds/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        # The only page number for this stage is the transcribe.cpp page's mel
        # time for 11 s of audio on an Apple M4 Max (best: 43 ms, 256 audio-s/s,
        # Vulkan): a ratio only for that workload's shape, as context.
        "vs_baseline": (audio_s / (ms_per_step / 1e3)) / (11.0 / 0.043) if args.workload == "p3" else None,
        "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": desc, "clips": len(so) - 1, "samples": n_samples,
                   "frames": total, "output_rows": out_rows, "buffer_sets": n_sets},
        "frames_per_s": total / (ms_per_step / 1e3),
        # The HBM roofline of the target; the vector-ALU figures ride along.
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved_gbs / HBM_PEAK_GBS,
                     "traffic": traffic,
                     "kernel": (("logmel_chunk_pad_kernel + " if chunked else "")
                                + {(0, 0): "logmel_tiles_kernel", (1, 0): "logmel_tiles_i16_kernel",
                                   (0, 1): "logmel_tiles_f16out_kernel",
                                   (1, 1): "logmel_tiles_i16_f16out_kernel"}[(in_i16, out_f16)]),
                     "kernel_avg_us": kern_avg_s * 1e6,
                     # event pairs around single launches (every event_every-th)
                     "kernel_sampled_avg_us": sampled_avg_s * 1e6,
                     "kernel_median_us": kern_med_s * 1e6,
                     "kernel_min_us": kern_min_s * 1e6,
                     "launches_timed": len(timed),
                     # the stream's time per launch over the whole timed region
                     "stream_us_per_launch": stream_us_per_launch,
                     "algorithmic_bytes_per_launch": algo_bytes,
                     "hbm_achieved_gbs": achieved_gbs,
                     "hbm_frac": achieved_gbs / HBM_PEAK_GBS,
                     "alu_achieved_tflops": achieved_tflops,
                     "alu_peak_tflops": ALU_PEAK_TFLOPS,
                     "alu_frac": achieved_tflops / ALU_PEAK_TFLOPS,
                     "algorithmic_flops_per_launch": FLOPS_PER_FRAME * total,
                     # a 1 GiB device-to-device copy in the same run: what a
                     # plain streaming kernel reaches here
                     "copy_gbs": copy_gbs,
                     "hbm_frac_of_copy": achieved_gbs / copy_gbs if copy_gbs else None},
    }
    clips_host = None
    if not args.no_cpu_baseline:
        xh = x.cpu().numpy()
        if xh.dtype == np.int16:
            xh = xh.astype(np.float32) / np.float32(32768.0)
        nclip = min(len(so) - 1, 64)
        if args.workload == "c4":
            # the shortest clips of the ragged batch would skew nothing; take
            # a contiguous 60 s slice of each of the first clips instead
            clips_host = [xh[so[i]:min(so[i + 1], so[i] + 960000)] for i in range(16)]
        else:
            clips_host = [xh[so[i]:so[i + 1]] for i in range(nclip)]
    return rec, clips_host


# fp32 vector peak as published (packed FP32); without packed instructions,
# which this build does not emit, the ceiling is half of it.
FP32_PEAK_TFLOPS = 157.3


def _resample_worker(args):
    x, rate, reps = args
    from oracle import logmel_clip, resample_clip
    for _ in range(reps):
        y, _ = resample_clip(x, rate)
        logmel_clip(y.astype("float32"))
    return 0


def bench_resampled(args, lm, plan, torch):
    """One step = the 64 x 30 s batch made at --in-rate, resampled to 16 kHz
    (logmel_resample) and then turned into log-mel (logmel_compute): two
    launches on one stream, each timed with its own HIP events (on every
    --event-every-th step)."""
    import logmel_synth as S
    import numpy as np
    import multiprocessing as mp
    dev = torch.device("cuda", 0)
    rate = args.in_rate
    x, so = S.config2_at(rate, device=dev)
    r = lm.logmel_resampler_create(plan, rate)
    L, T = lm.logmel_resampler_info(r)
    oo = lm.logmel_resample_offsets(so, rate)
    fo = lm.logmel_frame_offsets(oo)
    n_out, total = int(oo[-1]), int(fo[-1])
    n_in = int(so[-1])
    so_d, oo_d, fo_d = (torch.from_numpy(a).to(dev) for a in (so, oo, fo))
    n_sets = 3
    xs = [x] + [x.clone() for _ in range(n_sets - 1)]
    ys = [torch.empty(n_out, dtype=torch.float32, device=dev) for _ in range(n_sets)]
    outs = [torch.empty((total, 128), dtype=torch.float32, device=dev) for _ in range(n_sets)]
    stream = torch.cuda.current_stream(dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]

    def step(k, e=None):
        if e: e[0].record(stream)
        lm.logmel_resample(r, xs[k], so_d, oo_d, n_out, out=ys[k], stream=stream)
        if e: e[1].record(stream)
        lm.logmel_compute(plan, ys[k], oo_d, fo_d, total, out=outs[k], stream=stream)
        if e: e[2].record(stream)

    for i in range(args.warmup):
        step(i % n_sets)
    torch.cuda.synchronize()
    # events on every event_every-th step only (their packets lengthen a step)
    every = args.event_every if args.steps >= 2 * args.event_every else 1
    timed = [i for i in range(args.steps) if i % every == 0]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i % n_sets, ev[i] if i % every == 0 else None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    rs_s = sum(ev[i][0].elapsed_time(ev[i][1]) for i in timed) / len(timed) / 1e3
    lm_s = sum(ev[i][1].elapsed_time(ev[i][2]) for i in timed) / len(timed) / 1e3
    ms_per_step = wall / args.steps * 1e3
    # taps inside the kernel's support per output: 2 H on average
    H = 24 * rate / (0.96 * min(rate, FS))
    rs_flops = 2 * (2 * H) * n_out
    rs_bytes = 4 * n_in + 4 * n_out + 16 * len(so)
    rs_tflops = rs_flops / rs_s / 1e12
    rec = {
        "metric": "audio-seconds/sec of 128-bin log-mel on 1 MI355X + % of HBM roofline",
        "value": (n_in / rate) / (ms_per_step / 1e3),
        "unit": "audio-seconds/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32+f64", "data": "synthetic",
        "config": {"workload": f"offline batch: 64 speech-like clips x 30 s made at {rate} Hz "
                               f"({30 * rate} fp32 samples each), resampled to 16 kHz, then log-mel",
                   "clips": len(so) - 1, "in_rate": rate, "samples_in": n_in,
                   "samples_16k": n_out, "frames": total, "phases": L, "taps_per_phase": T,
                   "buffer_sets": n_sets},
        "frames_per_s": total / (ms_per_step / 1e3),
        "resample_kernel_avg_us": rs_s * 1e6,
        "logmel_kernel_avg_us": lm_s * 1e6,
        "roofline": {"bound": "mfma", "achieved": rs_tflops, "peak": FP32_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": rs_tflops / FP32_PEAK_TFLOPS,
                     "traffic": measured_traffic("logmel_resample_c2_44k", RESAMPLE_SOURCES)
                     if rate == 44100 else None,
                     "kernel": "logmel_resample" + (" (instance logmel_resample2_wide_8w_kernel)"
                                                    if rate == 44100 else
                                                    " (the instance the launcher picks for this rate)"),
                     "kernel_avg_us": rs_s * 1e6,
                     "algorithmic_flops_per_launch": rs_flops,
                     "algorithmic_bytes_per_launch": rs_bytes,
                     "hbm_achieved_gbs": rs_bytes / rs_s / 1e9,
                     "hbm_frac": rs_bytes / rs_s / 1e9 / HBM_PEAK_GBS},
    }
    if not args.no_cpu_baseline:
        xh = x.cpu().numpy()
        clips = [xh[so[i]:so[i + 1]] for i in range(16)]
        cores, _ = host_cores()
        for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
            os.environ[v] = "1"
        with mp.get_context("spawn").Pool(cores) as pool:
            t0 = time.perf_counter()
            pool.map(_resample_worker, [(c, rate, 1) for c in clips])
            dt = time.perf_counter() - t0
        audio = sum(c.size for c in clips) / rate
        rec["cpu_baseline"] = {"value": audio / dt, "unit": "audio-seconds/s", "cores": cores,
                               "kind": "oracle",
                               "sample": f"16 clips of the workload ({audio:.0f} audio-s): "
                                         f"oracle resampling then oracle log-mel, one pass, "
                                         f"{dt:.1f} s wall"}
    else:
        rec["cpu_baseline"] = None
    r.close()
    return rec


def bench_stream(args, lm, plan, torch):
    """One step = every 30 s stream of 512 pushed through in pushes of the
    audio clock (80 ms: 375 pushes of 1280 samples; 120 ms: 250 of 1920;
    160 ms: 187 of 2560 and one of 1280). With --in-rate R the streams are
    made at R Hz, pushed in pushes of the clock at R Hz, resampled on the
    device, and each step ends with a flush."""
    import logmel_synth as S
    import numpy as np
    dev = torch.device("cuda", 0)
    rate = args.in_rate
    n, N = 512, 30 * rate
    P = args.clock_ms * rate // 1000
    streams = (S.config3_streams(device=dev) if rate == FS
               else S.config3_streams_at(rate, device=dev))
    lens = [min(P, N - a) for a in range(0, N, P)]
    pushes = len(lens)
    chunks = [streams[:, a:a + L].contiguous().reshape(-1) for a, L in zip(range(0, N, P), lens)]
    s = lm.logmel_stream_create(plan, n, P, rate)
    pls = [np.full(n, L, dtype=np.int64) for L in lens]
    out = torch.empty((n * (args.clock_ms * FS // 1000 // 160 + 2), 128), dtype=torch.float32,
                      device=dev)
    flush_out = torch.empty((n * 4, 128), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def one_pass():
        lm.logmel_stream_reset(s)
        for c in range(pushes):
            # out has room for the largest push; the push writes its first rows
            lm.logmel_stream_push(s, chunks[c], pls[c], out=out, stream=stream)
        if rate != FS:
            fo = lm.logmel_stream_frames_for_flush(s)
            lm.logmel_stream_flush(s, out=flush_out[:int(fo[-1])], stream=stream)

    for _ in range(args.warmup):
        one_pass()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        one_pass()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / args.steps * 1e3
    audio_s = n * N / rate
    frames = n * 2998
    rec = {
        "metric": "audio-seconds/sec of 128-bin log-mel on 1 MI355X + % of HBM roofline",
        "value": audio_s / (ms_per_step / 1e3),
        "unit": "audio-seconds/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f64", "data": "synthetic",
        "config": {"workload": f"streaming: 512 streams x 30 s in pushes of {P} samples "
                               f"({args.clock_ms} ms audio clock, {pushes} pushes)"
                               + ("" if rate == FS else
                                  f" made at {rate} Hz, resampled to 16 kHz in each push, "
                                  "then a flush"),
                   "streams": n, "pushes": pushes, "push_samples": P, "in_rate": rate},
        "frames_per_s": frames / (ms_per_step / 1e3),
        "push_latency_us": ms_per_step * 1e3 / pushes,
    }
    s.close()
    return rec, None


def nested_c4(args, lm, plan, torch):
    """The ragged long batch (200 clips, 0.5 s to 87 min) timed in the same
    run as the headline: a few launches, kernel time from HIP events."""
    import argparse as _ap
    sub = _ap.Namespace(**vars(args))
    sub.workload, sub.steps, sub.warmup = "c4", 5, 2
    sub.no_cpu_baseline = True
    r, _ = bench_offline(sub, lm, plan, torch)
    torch.cuda.empty_cache()
    rf = r["roofline"]
    return {"config": r["config"], "value": r["value"], "unit": r["unit"],
            "steps": sub.steps, "warmup": sub.warmup, "ms_per_step": r["ms_per_step"],
            "frames_per_s": r["frames_per_s"], "kernel": rf["kernel"],
            "kernel_avg_us": rf["kernel_avg_us"], "kernel_sampled_avg_us": rf["kernel_sampled_avg_us"],
            "kernel_min_us": rf["kernel_min_us"],
            "algorithmic_bytes_per_launch": rf["algorithmic_bytes_per_launch"],
            "hbm_achieved_gbs": rf["hbm_achieved_gbs"], "hbm_frac": rf["hbm_frac"],
            "traffic": rf["traffic"], "alu_frac": rf["alu_frac"]}


def counter_pass(args, lm, plan, torch):
    """The run that hardware-counter summaries are taken over: three launches
    on the workload's buffers, then a 1 GiB fill and three 1 GiB
    device-to-device copies whose counter readings calibrate bytes."""
    dev = torch.device("cuda", 0)
    x, so, _ = make_workload(args.workload, dev)
    fo = lm.logmel_frame_offsets(so)
    total = int(fo[-1])
    so_d = torch.from_numpy(so).to(dev)
    fo_d = torch.from_numpy(fo).to(dev)
    out = torch.empty((total, 128), dtype=torch.float32, device=dev)
    for _ in range(3):
        lm.logmel_compute(plan, x, so_d, fo_d, total, out=out)
    a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    b = torch.ones_like(a)
    for _ in range(3):
        a.copy_(b)
    torch.cuda.synchronize()
    print(json.dumps({"counter_pass": args.workload, "frames": total}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="c2", choices=["c2", "c1", "c4", "c3", "p3"])
    ap.add_argument("--clock-ms", type=int, default=80, choices=[80, 120, 160],
                    help="audio clock of the streaming workload (c3)")
    ap.add_argument("--in-dtype", default="f32", choices=["f32", "i16"],
                    help="sample type: fp32, or int16 PCM (the workload quantised to 16 bits)")
    ap.add_argument("--out-dtype", default="f32", choices=["f32", "f16"],
                    help="output type: fp32 or fp16")
    ap.add_argument("--layout", default="frames", choices=["frames", "chunked"],
                    help="output layout: [frames, 128] or 30-s chunks [chunks, 3000, 128]")
    ap.add_argument("--in-rate", type=int, default=16000,
                    help="make the c2 batch at this rate and resample it to 16 kHz in the step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-c4", action="store_true",
                    help="skip the nested ragged-long-batch record of the default run")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--event-every", type=int, default=8,
                    help="record HIP events around every N-th timed launch (all of them in "
                         "runs of fewer than 2N steps)")
    ap.add_argument("--counter-pass", action="store_true",
                    help="run three launches and a 1 GiB copy for hardware counters; no timing")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(frames are independent, so several GPUs would each run this same kernel "
              "on their own share of the batch)", file=sys.stderr)
        sys.exit(2)
    defaults = {"c2": (200, 20), "c1": (500, 50), "c4": (5, 2), "c3": (3, 1), "p3": (500, 50)}
    if args.in_rate != FS:
        defaults["c2"] = (50, 5)
    if args.steps is None:
        args.steps = defaults[args.workload][0]
    if args.warmup is None:
        args.warmup = defaults[args.workload][1]

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    import log_mel_spectrogram_amd as lm
    plan = lm.logmel_plan_create(0)
    if args.counter_pass:
        counter_pass(args, lm, plan, torch)
        return
    if args.in_rate != FS and args.workload not in ("c2", "c3"):
        print("bench.py: --in-rate applies to the c2 and c3 workloads", file=sys.stderr)
        sys.exit(2)
    if args.in_rate != FS and args.workload == "c2":
        print(json.dumps(bench_resampled(args, lm, plan, torch)), flush=True)
        return
    if args.workload == "c3":
        rec, clips = bench_stream(args, lm, plan, torch)
    else:
        rec, clips = bench_offline(args, lm, plan, torch)
    if args.workload == "c2" and not args.no_c4 and args.layout == "frames" \
            and args.in_dtype == "f32" and args.out_dtype == "f32":
        rec["c4"] = nested_c4(args, lm, plan, torch)
    if clips is not None:
        rec["cpu_baseline"] = cpu_baseline(clips, args.cpu_seconds)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
