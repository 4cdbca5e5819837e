#!/usr/bin/env python3
"""Throughput of the DAC-style waveform decoder on one MI355X.

One step = one full decode (conv_in, 4 upsampling blocks with 3 residual
units each, head) of one batch of synthetic latents, with the latent, the
weights and the output buffer already resident in HBM.  For the windowed
workload one step is one vocoder_decode_windows call: every window of the
song decoded as one batch and stitched into planar output.  For the
streaming workload one step is one pass of every stream through the clip:
a reset, then the clip's latent frames in fixed-size chunks.  For the encode
workload one step is one vocoder_encode of the audio batch.

Prints ONE JSON line: audio-seconds decoded per second (value), whole-decode
TFLOP/s, the roofline of the dominant kernel measured live with HIP events
recorded on the decode stream by the library's per-launch profiler around
that kernel's launches in the timed steps (the per-kind table comes from a
separate profiled pass that times every launch), what this device delivers
beside the published peaks (a copy and matrix-core loops, measured after the
timed steps), and the CPU oracle timed on a bounded sample of the same
workload (cpu_baseline).
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "audio-seconds decoded/sec (44.1 kHz stereo) + TFLOP/s as % of MFMA peak"
PEAK_TFLOPS = {"f32": 157.3, "bf16": 2500.0}   # MI355X dense MFMA
PEAK_HBM_GBS = 8000.0
KIND_NAMES = ["conv_in", "convt", "res_k7", "res_k1", "head", "import", "export", "res_fused",
              "in_proj", "enc_down", "enc_out", "af_snake", "snake", "col2im", "tanh"]
HBM_KINDS = ("head", "af_snake", "snake", "col2im", "tanh")   # stream / stencil kernels: priced against HBM bandwidth
KERNEL_SOURCES = ["dac_vocoder_decoding_amd/csrc/conv_gemm.hip",
                  "dac_vocoder_decoding_amd/csrc/fused_ru.hip",
                  "dac_vocoder_decoding_amd/csrc/stream_kernels.hip",
                  "dac_vocoder_decoding_amd/csrc/gemm_common.h",
                  "dac_vocoder_decoding_amd/csrc/device_math.h",
                  "dac_vocoder_decoding_amd/csrc/internal.h"]


def kernel_source_sha() -> str:
    """Hash of the kernel sources' code: comments and layout are dropped, so
    stored counter readings stay attached to the code they were taken on."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            text = re.sub(r"//[^\n]*", "", f.read())
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def workload_name(cfg: dict) -> str:
    lat = f"[{cfg['batch']},{cfg['latent_channels']},{cfg['frames']}]"
    w = "/".join(str(x) for x in cfg["widths"])
    s = ",".join(str(x) for x in cfg["strides"])
    tile = f", time tiles of {cfg['tile_frames']} frames" if cfg["tile_frames"] else ""
    proj = f"dec_in_proj {cfg['latent_channels']}->{cfg['in_proj']}, " if cfg.get("in_proj") else ""
    if cfg.get("chunk"):
        lat += f" streamed in chunks of {cfg['chunk']} frames, causal"
    if cfg.get("windows"):
        lat = (f"{cfg['windows']} windows [{cfg['batch']},{cfg['latent_channels']},{cfg['frames']}] "
               f"(last {cfg['last_frames']} frames), crops {cfg['crop'][0]}/{cfg['crop'][1]}, stitched")
    if cfg.get("encode"):
        ew = "/".join(str(x) for x in cfg["enc_widths"])
        es = ",".join(str(x) for x in reversed(cfg["strides"]))
        return (f"{cfg['name']}: audio [{cfg['batch']},1,{cfg['frames'] * cfg['hop']}] -> latent {lat} "
                f"{cfg['dtype']}, encoder widths {ew}, strides {es}, conv_out k=3, projection to "
                f"{cfg['latent_channels']}, {cfg['act']}")
    af = ", alias-free Snake (2x up / Snake / 2x down)" if cfg.get("af_snake") else ""
    out = ", 2 output channels" if cfg.get("out_channels", 1) == 2 else ""
    terms = ", two-term bf16 operands" if cfg.get("operand_terms", 0) == 2 else ""
    return (f"{cfg['name']}: latent {lat} {cfg['dtype']}{terms}, {proj}widths {w}, strides {s}, "
            f"{cfg['act']}{af}{out}{tile}")


def traffic_for(workload_key: str, kind: str):
    """HBM bytes per launch of the dominant kernel from committed rocprofv3
    --pmc FETCH_SIZE / WRITE_SIZE runs, scaled by a copy-kernel calibration;
    None when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    ent = rec.get(workload_key, {}).get(kind)
    if not ent or ent.get("kernel_source_sha") != kernel_source_sha():
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(cfg: dict, tensors: dict, latent, target_s: float = 15.0,
                 kept_frac: float = 1.0) -> dict:
    """The oracle (fp64 direct loops, OpenMP) on a bounded time slice of the
    same workload: one stereo pair (or one mono row) of the first frames (of
    the first window, for the windowed workload, whose rate is then scaled by
    the fraction of decoded frames the stitching keeps)."""
    from dac_vocoder_decoding_amd import inputs as I
    from oracle import oracle as O
    rows = 2 if cfg["stereo"] and cfg.get("out_channels", 1) == 1 else 1
    hop = cfg["hop"]
    if cfg.get("encode"):   # `latent` is the audio [B, 1, T*hop]
        enc = O.Encoder(cfg, tensors)
        run = lambda n: enc.encode(latent[:rows, :, :n * hop])   # noqa: E731
    else:
        model = O.Model(cfg, tensors)
        run = lambda n: model.decode(latent[:rows, :, :n])       # noqa: E731
    t0 = time.perf_counter()
    run(4)
    t4 = time.perf_counter() - t0
    frames = int(max(4, min(cfg["frames"], round(4 * target_s / max(t4, 1e-3)))))
    t0 = time.perf_counter()
    run(frames)
    wall = time.perf_counter() - t0
    secs = I.audio_seconds(cfg, rows, frames)
    flops = I.encode_flops(cfg, rows, frames) if cfg.get("encode") else I.algorithmic_flops(cfg, rows, frames)
    note = "" if kept_frac == 1.0 else (f"; rate x {kept_frac:.4f}, the share of decoded window "
                                        "frames that the stitching keeps")
    return {"value": secs / wall * kept_frac, "unit": "audio-s/s", "cores": O.num_threads(),
            "kind": "oracle", "gflops_fp64": flops / wall / 1e9,
            "sample": f"{rows} row(s) x {frames} latent frames of the same input "
                      f"({secs:.3f} audio-s) decoded by the fp64 oracle in {wall:.2f} s{note}"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=1,
                    help="synthetic workload index (default 1: full-width stereo window)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile", action="store_true",
                    help="skip the per-launch event profiler (roofline becomes null)")
    ap.add_argument("--operand-terms", type=int, default=1, choices=(1, 2),
                    help="2: two-term bf16 matrix-core operands (bf16 workloads)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="before the decode, run the library's plain copy kernel 3 times "
                         "over MIB MiB (a known byte count for HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this decoder shards rows and time tiles "
              "across GPUs with no exchange, and only the single-GPU path is built; "
              "run with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    from dac_vocoder_decoding_amd import inputs as I
    from dac_vocoder_decoding_amd import vocoder as V

    cfg = I.config(args.config)
    if args.operand_terms == 2:
        if cfg["dtype"] != "bf16":
            print("--operand-terms 2 applies to the bf16 workloads", file=sys.stderr)
            return 2
        cfg = dict(cfg, name=cfg["name"] + "_two_term", operand_terms=2)
    tensors = I.make_weights(cfg)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    ctx = V.open_context(cfg, tensors, device=0)
    stream = torch.cuda.current_stream()
    nout = cfg.get("out_channels", 1)
    sides = 2 if cfg["stereo"] and nout == 1 else 1
    if cfg.get("encode"):
        audio_np = I.make_audio(cfg)
        B, T = cfg["batch"], cfg["frames"]
        latent_np = audio_np                       # the CPU-baseline sample (audio)
        audio = torch.from_numpy(audio_np).to(dev)
        pcm = torch.empty(B, cfg["latent_channels"], T, device=dev)
        secs = I.audio_seconds(cfg, B, T)
        flops = I.encode_flops(cfg, B, T)
        kept_frac = 1.0

        def step():
            V.check(V.vocoder_encode(ctx, audio, B, T, pcm, stream), ctx)
    elif cfg.get("windows"):
        win_np = I.make_windows(cfg)
        n, L, last, (cl, cr) = cfg["windows"], cfg["frames"], cfg["last_frames"], cfg["crop"]
        latent_np = win_np[0].reshape(sides, cfg["latent_channels"], L)  # CPU-baseline sample
        latent = torch.from_numpy(win_np).to(dev)
        N = V.vocoder_windows_output_length(ctx, n, L, last, cl, cr)
        pcm = torch.empty(sides * nout, N, device=dev)
        B, T = n * sides, L
        secs = N / cfg["sample_rate"]
        kept_frac = N / (cfg["hop"] * (L * (n - 1) + last))
        flops = sum(I.algorithmic_flops(cfg, sides, L if k < n - 1 else last) for k in range(n))

        def step():
            V.check(V.vocoder_decode_windows(ctx, latent, n, sides, L, last, cl, cr, pcm, stream), ctx)
    elif cfg.get("chunk"):
        latent_np = I.make_latent(cfg)
        B, _, T = latent_np.shape
        ck = cfg["chunk"]
        assert T % ck == 0
        chunks = [torch.from_numpy(np.ascontiguousarray(latent_np[:, :, k:k + ck])).to(dev)
                  for k in range(0, T, ck)]
        outs = [torch.empty(B, nout, V.vocoder_output_length(ctx, ck), device=dev) for _ in chunks]
        pcm = outs[-1]
        secs = I.audio_seconds(cfg, B, T)
        flops = I.algorithmic_flops(cfg, B, T)   # the clip's own work (context re-decodes excluded)
        kept_frac = 1.0

        def step():
            V.check(V.vocoder_stream_reset(ctx, B), ctx)
            for x, y in zip(chunks, outs):
                V.check(V.vocoder_stream_decode(ctx, x, ck, y, stream), ctx)
    else:
        latent_np = I.make_latent(cfg)
        latent = torch.from_numpy(latent_np).to(dev)
        B, _, T = latent.shape
        pcm = torch.empty(B, nout, V.vocoder_output_length(ctx, T), device=dev)
        secs = I.audio_seconds(cfg, B, T)
        flops = I.algorithmic_flops(cfg, B, T)
        kept_frac = 1.0

        def step():
            V.check(V.vocoder_decode(ctx, latent, B, T, pcm, stream), ctx)

    if args.calibrate_copy:
        nbytes = args.calibrate_copy * (1 << 20)
        src = torch.ones(nbytes // 4, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            V.check(V.voc_dbg_copy(dst, src, nbytes, stream))
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    def read_stats():
        out = {}
        for k, name in enumerate(KIND_NAMES):
            st, s = V.vocoder_profile_read(ctx, k)
            V.check(st, ctx)
            if s["launches"]:
                out[name] = s
        return out

    # Per-kind table from a profiled pass of its own (every launch timed),
    # which also names the dominant kernel kind.
    profile = not args.no_profile
    diag, dom = {}, None
    diag_steps = max(2, min(args.steps, 5))
    if profile:
        V.check(V.vocoder_profile_reset(ctx), ctx)
        V.check(V.vocoder_profile_enable(ctx, True), ctx)
        for _ in range(diag_steps):
            step()
        torch.cuda.synchronize()
        V.check(V.vocoder_profile_enable(ctx, False), ctx)
        diag = read_stats()
        dom = max((n for n in diag if n not in ("import", "export")), key=lambda n: diag[n]["ms"])
        # Timed region: events only around the dominant kind's launches
        # (events between every launch would lengthen the kernel gaps).
        V.check(V.vocoder_profile_reset(ctx), ctx)
        V.check(V.vocoder_profile_select(ctx, 1 << KIND_NAMES.index(dom)), ctx)
        V.check(V.vocoder_profile_enable(ctx, True), ctx)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    kernels = {}
    if profile:
        V.check(V.vocoder_profile_enable(ctx, False), ctx)
        V.check(V.vocoder_profile_select(ctx, 0), ctx)
        kernels = read_stats()

    value = secs / (ms_per_step / 1e3)
    tflops = flops / (ms_per_step / 1e3) / 1e12
    peak = PEAK_TFLOPS[cfg["dtype"]]
    ok = bool(torch.isfinite(pcm).all().item()) and (cfg.get("encode") or float(pcm.abs().max()) <= 1.0)

    roofline = None
    per_kernel = {}
    if profile:
        total_ms = sum(x["ms"] for x in diag.values())
        for name, s in diag.items():
            avg_ms = s["ms"] / s["launches"]
            per_kernel[name] = {
                "launches_per_step": s["launches"] / diag_steps,
                "avg_us": round(1e3 * avg_ms, 3),
                "share": round(s["ms"] / total_ms, 4),
                "tflops": round(s["flops"] / (s["ms"] / 1e3) / 1e12, 3),
                "alg_gbs": round(s["bytes"] / (s["ms"] / 1e3) / 1e9, 1),
            }
        s = kernels[dom]  # the dominant kind, timed over the timed steps
        if dom in HBM_KINDS:
            achieved = s["bytes"] / (s["ms"] / 1e3) / 1e9
            roofline = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS}
        else:
            achieved = s["flops"] / (s["ms"] / 1e3) / 1e12
            roofline = {"bound": "mfma", "achieved": achieved, "peak": peak,
                        "unit": "TFLOP/s", "frac": achieved / peak}
        roofline.update({
            "kernel": dom,
            "avg_launch_us": 1e3 * s["ms"] / s["launches"],
            "launches_timed": s["launches"],
            "alg_flops_per_launch": s["flops"] / s["launches"],
            "alg_bytes_per_launch": s["bytes"] / s["launches"],
            "traffic": traffic_for(cfg["name"], dom),
        })

    # Achievable peaks, measured after the timed steps: a 1 GiB copy and the
    # matrix-core loops of both operand dtypes.
    achievable = None
    if profile:
        st0, gbs = V.voc_dbg_peak(0, 1 << 30, stream)
        loops = [V.voc_dbg_peak(w, n, stream) for w, n in ((1, 2000), (3, 1000), (2, 20000), (4, 10000))]
        if st0 == V.VOC_OK and all(st == V.VOC_OK for st, _ in loops):
            tf32 = max(loops[0][1], loops[1][1])
            tbf16 = max(loops[2][1], loops[3][1])
            achievable = {"hbm_copy_gbs": gbs, "mfma_f32_tflops": tf32, "mfma_bf16_tflops": tbf16,
                          "mfma_loops_tflops": {"f32_16x16x4": loops[0][1], "f32_32x32x2": loops[1][1],
                                                "bf16_16x16x32": loops[2][1], "bf16_32x32x16": loops[3][1]},
                          "note": "plain copy of 1 GiB (bytes read + written) and loops of independent "
                                  "MFMA chains (the faster shape per dtype), measured in this run"}
            meas = gbs if roofline["bound"] == "hbm" else (tf32 if cfg["dtype"] == "f32" else tbf16)
            roofline["frac_of_measured_peak"] = roofline["achieved"] / meas

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, tensors, latent_np, kept_frac=kept_frac)

    rec = {
        "metric": METRIC,
        "value": value,
        "unit": ("audio-s/s" if cfg["sample_rate"] == 44100 else
                 f"audio-s/s (stereo {cfg['sample_rate'] / 1000:g} kHz)") if cfg["stereo"]
                else "audio-s/s (mono 24 kHz)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"],
        "data": "synthetic (seeded latents and random-init weights of the stated shapes)",
        "config": {"workload": workload_name(cfg), "rows": B, "latent_frames": T,
                   "audio_seconds_per_step": secs, "parallelism": "single GPU"},
        "tflops": tflops,
        "mfma_peak_frac": tflops / peak,
        "output_ok": ok,
        "host_wall_s": wall,
        "kernels": per_kernel,
        "kernels_note": f"per-kind table from a separate pass of {diag_steps} decodes timing every launch",
        "roofline": roofline,
        "achievable": achievable,
        "cpu_baseline": cpu,
    }
    V.vocoder_destroy(ctx)
    print(json.dumps(rec))
    return 0


if __name__ == "__main__":
    sys.exit(main())
