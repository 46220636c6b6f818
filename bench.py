#!/usr/bin/env python3
"""Benchmark of the BigVGAN decode path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c3]
    python bench.py --path encode [--workload e3]

A step is one full decode (dec_in_proj -> conv_pre -> 7 x (transposed conv
+ averaged AMP blocks) -> activation_post + conv_post + clamp) of one batch
of seeded synthetic latents already resident in HBM. Prints one JSON line.

The metric is decoded audio-seconds per second: B * N / 40 / seconds per
step (40 latents per second of 32 kHz audio). The default workload is two
30 s items (B=2, N=1200) with the default MiniMax-H3 decoder and seeded
random weights. `--workload c4` times the stage-1 AMP set alone on
(2, 256, 30000).

`roofline` covers the dominant kernel, the AMP dilated convolution of the
wide stages (conv_kernel on the packed activated input; by default its
products run as three fp16 piece products per fp32 product on the fp16
matrix cores with fp32 accumulation, fp32-accurate), whose kernel durations
come from HIP events the library records on the decode stream around every
AMP conv launch of the last timed step (other launches are not bracketed
there; a second, untimed pass with every launch bracketed gives the
per-class breakdown). `achieved` counts the method's FLOPs (2 C_out C_in k
per output); `peak` is the dense peak of the matrix instruction the kernel
issues (fp16 / bf16, 2500 TFLOP/s; fp32 with --fp32-matrix), so `frac` is at
most 1 / products. The named extras give the matrix pipe's occupancy
counting every piece product, and the ratio to the fp32 matrix peak.
`cpu_baseline` times the CPU oracle (numpy, fp64 inside each op) on a
bounded sample: the first 320 latents of item 0, decoded in full.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

FP32_MFMA_PEAK_TFLOPS = 157.3   # MI355X dense fp32 matrix, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published
SPLIT_PRODUCTS = 6              # bf16 piece products per fp32 product (matrix_form SPLIT)
F16_PRODUCTS = 3                # fp16 piece products per fp32 product (the default form)
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
LATENTS_PER_SECOND = 40         # 32 kHz / hop 800
SAMPLE_RATE = 32000

WORKLOADS = {
    # name: (batch, frames, flags, description); c4 is (batch, channels, length) of the AMP stage-1 set
    "c1": (1, 4, 0, "B=1 x N=4 latents (0.1 s)"),
    "c2": (2, 200, 1, "B=2 x N=200 latents (5 s/item), de-normalized latents"),
    "c3": (2, 1200, 0, "B=2 x N=1200 latents (30 s/item)"),
    "c4": (2, 256, 30000, "stage-1 AMP set alone on (2, 256, 30000): three blocks k 3/7/11, d 1/3/5, averaged"),
    "c5": (16, 401, 0, "B=16 x N=401 latents (10.025 s/item)"),
}
# encoder workloads (--path encode): name: (batch, samples, description)
ENC_WORKLOADS = {
    "e3": (2, 960000, "B=2 x 960000 samples (30 s/item at 32 kHz)"),
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--path", default="decode", choices=("decode", "encode"),
                    help="decode: the BigVGAN decoder (default); encode: the encoder's convolution stack")
    ap.add_argument("--workload", default=None, choices=sorted(WORKLOADS) + sorted(ENC_WORKLOADS))
    ap.add_argument("--bf16", action="store_true", help="bf16-split matrix-core operands (MH3A_FLAG_BF16_MFMA)")
    ap.add_argument("--fp32-matrix", action="store_true",
                    help="build the decoder (or encoder) with matrix_form = MH3A_MATRIX_FP32 (fp32 matrix cores throughout)")
    ap.add_argument("--bf16x6", action="store_true",
                    help="build the decoder (or encoder) with matrix_form = MH3A_MATRIX_SPLIT (six bf16 piece products)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="also time K replays of one decode captured in a HIP graph (graph_ms_per_step)")
    ap.add_argument("--cpu-latents", type=int, default=320, help="latents in the oracle's timed sample")
    ap.add_argument("--cpu-samples", type=int, default=128000, help="samples in the oracle's timed encode sample")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES (calibrates HBM byte counters)")
    return ap.parse_args()


def copy_probe(nbytes):
    """One plain device copy of nbytes: the reference the HBM read/write
    counters of the decode kernels are scaled by."""
    import torch
    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n * 4}), flush=True)
    return 0


def sources_digest():
    """sha256 over the library's sources (csrc/* and include/mh3a.h, sorted
    by path): a counter record holds for the build it was taken on."""
    import glob
    import hashlib
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "neural_audio_vae_amd", "csrc", "*")))
    files.append(os.path.join(ROOT, "include", "mh3a.h"))
    for f in files:
        h.update(os.path.relpath(f, ROOT).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload, form):
    """HBM bytes per launch of the roofline kernel from the committed
    rocprofv3 counter runs (profiles/amp_conv_c3_traffic.json for the
    decode's AMP convs, profiles/enc_unit_conv_e3_traffic.json for the
    encoder's k7 convs), or None when the library's sources changed since
    the counters were taken, or the workload or matrix form differs."""
    files = {"c3": "amp_conv_c3_traffic.json", "e3": "enc_unit_conv_e3_traffic.json"}
    if workload not in files:
        return None
    path = os.path.join(ROOT, "profiles", files[workload])
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("form") != form or rec.get("source_sha256") != sources_digest():
        return None
    return rec["traffic_bytes_per_launch"]


def _blas_threads():
    try:
        import threadpoolctl
        return max((p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()), default=1)
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline(params, n_latents):
    """The oracle, as it stands, on the first n latents of item 0 of the
    workload (a full decode of that short clip)."""
    import numpy as np
    import oracle as O
    from neural_audio_vae_amd import synth
    threads = _blas_threads()
    z = synth.make_latents(2, 1200)[:1, :, :n_latents]
    t0 = time.perf_counter()
    y = O.decode(params, np.ascontiguousarray(z))
    dt = time.perf_counter() - t0
    assert y.shape == (1, 1, 800 * n_latents)
    return {
        "value": (n_latents / LATENTS_PER_SECOND) / dt,
        "unit": "audio-s/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"numpy oracle (fp64 inside each op; its per-tap matmuls on {threads} BLAS threads, the "
                  f"resampling and SnakeBeta steps on one thread): full decode of latents [0, {n_latents}) of "
                  f"item 0 of the workload ({n_latents / LATENTS_PER_SECOND:.1f} s of audio, a bounded sample) "
                  f"in {dt:.1f} s",
    }


def roofline_entry(kernel, stats, form):
    """The roofline record of the matrix-core kernel from its HIP-event
    stats: `form` is "f16x3" (three fp16 piece products, the default),
    "split" (six bf16 piece products), "bf16x3" (three bf16 piece products)
    or "fp32" (fp32 matrix cores)."""
    products = {"f16x3": F16_PRODUCTS, "split": SPLIT_PRODUCTS, "bf16x3": 3, "fp32": 1}[form]
    peak = FP32_MFMA_PEAK_TFLOPS if form == "fp32" else BF16_MFMA_PEAK_TFLOPS
    achieved = stats["flops"] / (stats["ms"] / 1e3) / 1e12 if stats["ms"] > 0 else 0.0
    return {
        "kernel": kernel,
        "bound": "mfma",
        "achieved": round(achieved, 2),
        "peak": peak,
        "peak_basis": {"fp32": "dense fp32 matrix peak (v_mfma_f32_32x32x2f32)",
                       "f16x3": "dense fp16 matrix peak (v_mfma_f32_32x32x16_f16, the instruction issued)"}.get(
                           form, "dense bf16 matrix peak (v_mfma_f32_32x32x16_bf16, the instruction issued)"),
        "unit": "TFLOP/s",
        "frac": round(achieved / peak, 4),
        "achieved_counts": "the method's FLOPs, 2 C_out C_in k per output",
        "products_per_fp32_product": products,
        "matrix_pipe_occupancy": round(achieved * products / peak, 4),
        "vs_fp32_matrix_peak": round(achieved / FP32_MFMA_PEAK_TFLOPS, 4),
        "launches_timed": stats["launches"],
        "avg_launch_us": round(1e3 * stats["ms"] / max(1, stats["launches"]), 2),
        "flops_per_launch": stats["flops"] / max(1, stats["launches"]),
    }


def _per_step(kernels, steps):
    return {
        name: {
            "launches_per_step": k["launches"] / steps,
            "ms_per_step": round(k["ms"] / steps, 4),
            "tflops": round(k["flops"] / (k["ms"] / 1e3) / 1e12, 2) if k["ms"] > 0 else None,
            "gbs_compulsory": round(k["bytes"] / (k["ms"] / 1e3) / 1e9, 1) if k["ms"] > 0 else None,
        }
        for name, k in kernels.items()
    }


def main():
    args = parse()
    if args.copy_probe:
        return copy_probe(args.copy_probe)
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the decode and encode paths run on a single GPU; see the sharding notes).", file=sys.stderr)
        return 2
    import torch
    from neural_audio_vae_amd import Decoder, _lib, synth

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        return 2
    if args.path == "encode":
        return main_encode(args)
    args.workload = args.workload or "c3"
    if args.workload not in WORKLOADS:
        print(f"--workload {args.workload} is an encoder workload (use --path encode)", file=sys.stderr)
        return 2
    stage_bench = args.workload == "c4"
    if stage_bench:
        batch, channels, length, desc = WORKLOADS["c4"]
        flags = 0
    else:
        batch, frames, flags, desc = WORKLOADS[args.workload]
    if args.bf16:
        flags |= 0x2
    form = "fp32" if args.fp32_matrix else ("bf16x3" if args.bf16 else ("split" if args.bf16x6 else "f16x3"))
    params = synth.make_params()
    mean, std = synth.make_denorm()
    cfg = ({"matrix_form": _lib.MH3A_MATRIX_FP32} if args.fp32_matrix else
           {"matrix_form": _lib.MH3A_MATRIX_SPLIT} if args.bf16x6 else None)
    dec = Decoder(params, cfg, latents_mean=mean, latents_std=std)
    stream = torch.cuda.current_stream()
    if stage_bench:
        x = torch.from_numpy(synth.make_signal((batch, channels, length), seed=0)).cuda()
        out = torch.empty_like(x)

        def step():
            dec.amp_stage(1, x, flags=flags, out=out, stream=stream)
    else:
        z = torch.from_numpy(synth.make_latents(batch, frames)).cuda()
        out = torch.empty((batch, 1, 800 * frames), dtype=torch.float32, device="cuda")

        def step():
            dec.decode(z, flags=flags, out=out, stream=stream)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K steps. In the last one the library brackets each AMP
    # conv launch (the roofline kernel) with HIP events on the decode stream
    # (events on every step would add their own cost, ~2%, to every step).
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        if i == args.steps - 1:
            dec.timing(_lib.MH3A_TIMING_AMP_CONV)
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_total = start.elapsed_time(stop)
    amp_only = dec.timing_read()
    # Per-class breakdown from a second, untimed pass with every launch
    # bracketed (the events add ~2% when on every launch).
    dec.timing(_lib.MH3A_TIMING_ALL)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kernels = dec.timing_read()
    dec.timing(_lib.MH3A_TIMING_OFF)

    ms_step = ms_total / args.steps
    amp = amp_only.get("amp_conv", {"launches": 0, "ms": 0.0, "flops": 0.0, "bytes": 0.0})
    total_flops = sum(k["flops"] for k in kernels.values()) / args.steps
    if stage_bench:
        metric, unit = "AMP stage-1 set TFLOP/s (c4, fp32)", "TFLOP/s"
        value = total_flops / (ms_step / 1e3) / 1e12
        config = {"workload": f"AMP residual-block set of stage 1 of the MiniMax-H3 audio-VAE decoder, {desc}, "
                              "seeded random weights", "batch": batch, "channels": channels, "length": length}
    else:
        metric = ("decoded audio-sec/s (B=2, 30 s clips, fp32)" if args.workload == "c3" else
                  f"decoded audio-sec/s ({args.workload})")
        unit = "audio-s/s"
        value = batch * frames / LATENTS_PER_SECOND / (ms_step / 1e3)
        config = {
            "workload": f"BigVGAN decode of the MiniMax-H3 audio VAE, {desc}, default decoder "
                        "(32->2048 proj, conv_pre 2048->1024, 7 upsampling stages 1024->8 ch, AMP k 3/7/11 "
                        "d 1/3/5), seeded random weights, 32 kHz mono output",
            "batch": batch,
            "frames": frames,
            "samples_per_item": 800 * frames,
            "flags": flags,
        }
    kernel_desc = ("conv_kernel, AMP dilated convs of the 64-512 channel stages (packed activated input; " +
                   {"f16x3": "three fp16 piece products per fp32 product (two pieces per operand, weights "
                             "scaled by 2^e) on v_mfma_f32_32x32x16_f16, fp32 accumulation)",
                    "split": "six bf16 piece products per fp32 product on v_mfma_f32_32x32x16_bf16, fp32 "
                             "accumulation)",
                    "bf16x3": "three bf16 piece products (two-piece split) on v_mfma_f32_32x32x16_bf16)",
                    "fp32": "fp32 matrix cores)"}[form])
    line = {
        "metric": metric,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f16x3": "f32", "split": "f32", "bf16x3": "bf16x3", "fp32": "f32"}[form],
        "data": "synthetic",
        "config": config,
        "algorithmic_tflops": round(total_flops / (ms_step / 1e3) / 1e12, 2),
        "roofline": dict(roofline_entry(kernel_desc, amp, form),
                         traffic=measured_traffic(args.workload, form)),
        "kernels": _per_step(kernels, args.steps),
        "wall_s_timed": round(wall, 4),
    }
    if args.graph and not stage_bench:
        # one decode captured on a side stream (after a warm-up call there),
        # then K replays between synchronizations: the launch overhead of the
        # ~130 kernels goes away, which matters for the small workloads
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            dec.decode(z, flags=flags, out=out, stream=s)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            dec.decode(z, flags=flags, out=out, stream=s)
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        line["graph_ms_per_step"] = round((time.perf_counter() - t0) / args.steps * 1e3, 4)
    if not args.no_cpu_baseline and not stage_bench:
        line["cpu_baseline"] = cpu_baseline(params, args.cpu_latents)
    print(json.dumps(line), flush=True)
    dec.close()
    return 0


def cpu_baseline_encode(params, n_samples):
    """The oracle's encode (stack, attention projection, mean_proj), as it
    stands, on the first n samples of item 0 of the workload."""
    import numpy as np
    import oracle as O
    from neural_audio_vae_amd import synth
    threads = _blas_threads()
    wave = synth.make_waveform(1, n_samples, seed=0)
    t0 = time.perf_counter()
    h = O.encode(params, wave)
    dt = time.perf_counter() - t0
    assert h.shape[-1] == -(-n_samples // 800)
    return {
        "value": (n_samples / SAMPLE_RATE) / dt,
        "unit": "audio-s/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"numpy oracle (fp64 inside each op; per-tap matmuls on {threads} BLAS threads, the Snake "
                  f"steps on one thread): encode of a {n_samples}-sample waveform ({n_samples / SAMPLE_RATE:.2f} s "
                  f"of audio, a bounded sample) in {dt:.1f} s",
    }


def main_encode(args):
    """A step is one whole encode to the posterior mean: the convolution
    stack (k7 conv, five strided blocks of Snake residual units, final Snake
    + k3 conv), the causal attention projection and mean_proj, over a batch
    of seeded synthetic waveforms resident in HBM."""
    import torch
    from neural_audio_vae_amd import Encoder, _lib, synth

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        return 2
    args.workload = args.workload or "e3"
    if args.workload not in ENC_WORKLOADS:
        print(f"--workload {args.workload} is a decoder workload (use --path decode)", file=sys.stderr)
        return 2
    batch, samples, desc = ENC_WORKLOADS[args.workload]
    params = dict(synth.make_encoder_params(seed=0), **synth.make_pre_block_params(seed=0))
    form = "fp32" if args.fp32_matrix else ("split" if args.bf16x6 else "f16x3")
    enc = Encoder(params, {"matrix_form": _lib.MH3A_MATRIX_FP32} if args.fp32_matrix else
                  {"matrix_form": _lib.MH3A_MATRIX_SPLIT} if args.bf16x6 else None)
    x = torch.from_numpy(synth.make_waveform(batch, samples, seed=0)).cuda()
    out = torch.empty((batch, enc.latent_channels, enc.frames(samples)), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        enc.encode_mean(x, out=out, stream=stream)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        if i == args.steps - 1:
            enc.timing(_lib.MH3A_TIMING_AMP_CONV)  # the residual units' k7 convs only
        enc.encode_mean(x, out=out, stream=stream)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_total = start.elapsed_time(stop)
    unit_only = enc.timing_read()
    enc.timing(_lib.MH3A_TIMING_ALL)
    for _ in range(args.steps):
        enc.encode_mean(x, out=out, stream=stream)
    torch.cuda.synchronize()
    kernels = enc.timing_read()
    enc.timing(_lib.MH3A_TIMING_OFF)
    ms_step = ms_total / args.steps
    value = batch * samples / SAMPLE_RATE / (ms_step / 1e3)
    k7 = unit_only.get("enc_unit_conv", {"launches": 0, "ms": 0.0, "flops": 0.0, "bytes": 0.0})
    total_flops = sum(k["flops"] for k in kernels.values()) / args.steps
    line = {
        "metric": f"encoded audio-sec/s ({args.workload}, fp32)",
        "value": round(value, 2),
        "unit": "audio-s/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"encoder of the MiniMax-H3 audio VAE to the posterior mean, {desc}: convolution stack "
                        "(encoder_dim 64, rates (2, 4, 4, 5, 5), hidden 2048), causal attention projection (8 heads, "
                        "32 streams, GeGLU 128) and mean_proj, seeded random weights",
            "batch": batch,
            "samples_per_item": samples,
        },
        "algorithmic_tflops": round(total_flops / (ms_step / 1e3) / 1e12, 2),
        "roofline": dict(roofline_entry(
            "conv_kernel, the residual units' k7 dilated convs (split-product packed input; "
            + {"f16x3": "three fp16 piece products per fp32 product (two pieces per operand, weights scaled by "
                        "2^e) on v_mfma_f32_32x32x16_f16, fp32 accumulation)",
               "split": "six bf16 piece products per fp32 product on v_mfma_f32_32x32x16_bf16)",
               "fp32": "fp32 matrix cores)"}[form], k7, form), traffic=measured_traffic(args.workload, form)),
        "kernels": _per_step(kernels, args.steps),
        "wall_s_timed": round(wall, 4),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_encode(params, args.cpu_samples)
    print(json.dumps(line), flush=True)
    enc.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
