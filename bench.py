#!/usr/bin/env python3
"""Frame-step benchmark of the MI355X Moshi/PersonaPlex library.

One "step" is one full frame of the hot path for every live session: the
17-channel embedding, the 4096-d / 32-layer temporal transformer over a
3000-frame ring (prefilled full, N(0,1) K/V), the 32000-way text head, and the
16 depformer substeps (1024-d / 6 layers, per-substep weights) with a greedy
argmax on every head. Weights are N(0, 0.02) bf16 drawn from a fixed seed;
frames are uniform random codes (synthetic stand-ins for live Mimi streams).

Timed region: K device-resident steps (frames already in HBM, outputs written
to HBM) bracketed by torch.cuda.synchronize(). Printed: one JSON line with
frames/s at B=1, the real-time factor (step time / 80 ms), the fraction of the
HBM roofline for the whole step, the roofline of the dominant kernel (HIP
events around each launch), and the fp64 CPU oracle timed on a bounded sample.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "frames/sec (80 ms frames) at B=1 and B=16; % HBM roofline; real-time factor"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
FRAME_MS = 80.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--timing-steps", type=int, default=3,
                    help="eager steps with HIP events around every kernel")
    ap.add_argument("--cpu-frames", type=int, default=2,
                    help="full-size frames the CPU oracle runs for its baseline")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--b16", type=int, default=1, help="also measure B=16 (elastic fills)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (the reference "
                         "dispatch that scales HBM byte counters)")
    return ap.parse_args()


def make_engine(M, shape, weights, B, stream):
    cfg = M.make_config(dim=shape.dim, n_layers=shape.n_layers, n_heads=shape.n_heads,
                        ffn_hidden=shape.ffn, window=shape.window, dep_dim=shape.dep_dim,
                        dep_layers=shape.dep_layers, dep_heads=shape.dep_heads,
                        dep_ffn_hidden=shape.dep_ffn, n_substeps=shape.n_substeps,
                        text_vocab=shape.text_vocab, audio_card=shape.audio_card,
                        rope_theta=shape.rope_theta, norm_eps=shape.norm_eps,
                        dtype=shape.dtype, max_sessions=B)
    return M.moshi_create(cfg, weights, hip_stream=stream.cuda_stream)


def timed_steps(M, torch, ctx, stream, d_frames, d_text, d_codes, warmup, steps):
    B = ctx.B
    for k in range(warmup):
        M.moshi_step_enqueue(ctx, d_frames[k % d_frames.shape[0]].data_ptr())
    M.moshi_sync(ctx)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for k in range(steps):
        M.moshi_step_enqueue(ctx, d_frames[(warmup + k) % d_frames.shape[0]].data_ptr(),
                             d_text[k % d_text.shape[0]].data_ptr(),
                             d_codes[k % d_codes.shape[0]].data_ptr())
    ev1.record(stream)
    M.moshi_sync(ctx)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall * 1000.0 / steps, ev0.elapsed_time(ev1) / steps, B


def kernel_table(M, ctx, frames_host, n):
    t = M.moshi_time_kernels(ctx, frames_host, n)
    out = {}
    for name, v in t.items():
        if v["launches"] == 0:
            continue
        ms = v["ms"] / n
        by = v["bytes"] / n
        out[name] = {"ms_per_step": round(ms, 4), "launches_per_step": v["launches"] // n,
                     "bytes_per_step": by,
                     "GBps": round(by / (ms * 1e6), 1) if ms > 0 else None}
    return out


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.txt")
KERNEL_SRCS = [os.path.join(ROOT, "full_duplex_speech_amd", "csrc", f)
               for f in ("dev.h", "kernels.h", "kernels.hip", "step.hip")]


def kernel_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for p in KERNEL_SRCS:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter runs
    (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy), or None when the kernel
    sources have changed since they were taken."""
    try:
        sha = kernel_sources_sha256()
        with open(TRAFFIC_FILE) as f:
            for line in f:
                kv = dict(x.split("=", 1) for x in line.split() if "=" in x)
                if kv.get("kernel") == kernel and kv.get("sources_sha256") == sha:
                    return float(kv["fetch_bytes"]) + float(kv["write_bytes"])
    except OSError:
        pass
    return None


def cpu_baseline(shape, weights, k, v, frames, n):
    import oracle
    om = oracle.Model(shape, weights)
    s = oracle.Session(om)
    s.prefill(k, v)
    t0 = time.perf_counter()
    for t in range(n):
        s.step(frames[t], want_logits=False)
    dt = time.perf_counter() - t0
    return n / dt, dt


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (sessions would shard "
              "one engine per GPU with no exchange); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import full_duplex_speech_amd as M
    from synth import spec, workloads as wl

    shape = spec.PERSONAPLEX
    W = shape.window
    t0 = time.perf_counter()
    weights = wl.make_weights(shape, wl.MODEL_SEEDS["personaplex"], threads=16)
    log(f"weights generated in {time.perf_counter() - t0:.1f}s")
    stream = torch.cuda.Stream()

    # ---------------- B = 1: the headline workload ----------------
    ctx = make_engine(M, shape, weights, 1, stream)
    slot = M.moshi_session_join(ctx)
    wk = wl.WORKLOADS[2]
    k, v = wl.prefill_kv(shape, wk.seed("prefill"), 0, W, threads=16)
    M.moshi_session_prefill_kv(ctx, slot, k, v)
    nfr = args.warmup + args.steps
    frames = wl.frames(shape, wk.seed("frames"), 0, 0, nfr)
    d_frames = torch.from_numpy(frames.reshape(nfr, 1, -1)).to("cuda")
    d_text = torch.zeros((args.steps, 1), dtype=torch.int32, device="cuda")
    d_codes = torch.zeros((args.steps, 1, shape.n_substeps), dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    log("B=1 engine ready")
    ms_wall, ms_gpu, _ = timed_steps(M, torch, ctx, stream, d_frames, d_text, d_codes,
                                     args.warmup, args.steps)
    fps = 1000.0 / ms_wall
    log(f"B=1: {ms_wall:.3f} ms/step wall, {ms_gpu:.3f} ms/step events, {fps:.1f} frames/s")

    # host-synchronous step (frames from host, tokens back to host every step)
    t1 = time.perf_counter()
    nsync = 20
    for i in range(nsync):
        M.moshi_step(ctx, frames[i % nfr][None, :])
    ms_sync = (time.perf_counter() - t1) * 1000.0 / nsync

    kt = kernel_table(M, ctx, frames[0][None, :], args.timing_steps)
    bytes_step = sum(x["bytes_per_step"] for x in kt.values())
    if M.moshi_uses_step_kernel(ctx):
        # the whole step is one persistent kernel: its launch duration is the
        # event-timed step (one launch per step, back to back on the stream)
        dname = "step_kernel"
        d_bytes, d_ms = bytes_step, ms_gpu
    else:
        # the temporal gate/up projection, the largest weight stream of the
        # step (184.5 MB per launch, 32 launches)
        dname = "temporal_gateup"
        d = kt[dname]
        d_bytes = d["bytes_per_step"] / d["launches_per_step"]
        d_ms = d["ms_per_step"] / d["launches_per_step"]
    achieved = d_bytes / (d_ms * 1e6)  # GB/s
    roofline = {"bound": "hbm", "kernel": dname, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(dname), "bytes_per_launch": d_bytes,
                "ms_per_launch": round(d_ms, 5)}
    step_gbs = bytes_step / (ms_wall * 1e6)
    log(f"dominant kernel {dname}: {achieved:.0f} GB/s; step {step_gbs:.0f} GB/s")
    M.moshi_destroy(ctx)
    del ctx

    if args.copy_mib > 0:
        n = args.copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: {args.copy_mib} MiB read + {args.copy_mib} MiB written")
        del src, dst

    # ---------------- B = 16: elastic fills ----------------
    b16 = None
    if args.b16:
        w4 = wl.WORKLOADS[4]
        initial, _ = wl.churn_schedule(w4)
        ctx = make_engine(M, shape, weights, 16, stream)
        for sid, fill in initial:
            s = M.moshi_session_join(ctx)
            kk, vv = wl.prefill_kv(shape, w4.seed("prefill"), sid, fill, threads=16)
            M.moshi_session_prefill_kv(ctx, s, kk, vv)
        del kk, vv
        n16 = 60
        fr16 = np.stack([wl.frames(shape, w4.seed("frames"), sid, 0, n16 + 5)
                         for sid, _ in initial], axis=1)  # [T, 16, 17]
        d16 = torch.from_numpy(np.ascontiguousarray(fr16)).to("cuda")
        t16 = torch.zeros((n16, 16), dtype=torch.int32, device="cuda")
        c16 = torch.zeros((n16, 16, shape.n_substeps), dtype=torch.int32, device="cuda")
        ms16, ms16g, _ = timed_steps(M, torch, ctx, stream, d16, t16, c16, 5, n16)
        kt16 = kernel_table(M, ctx, fr16[0], 1)
        by16 = sum(x["bytes_per_step"] for x in kt16.values())
        b16 = {"frames_per_s": round(16 * 1000.0 / ms16, 1), "ms_per_step": round(ms16, 4),
               "rtf": round(ms16 / FRAME_MS, 5), "bytes_per_step": by16,
               "hbm_frac_step": round(by16 / (ms16 * 1e6) / HBM_PEAK_GBS, 4),
               "fills": "U{0..3000} per slot (workload 4 at t=0)", "steps": n16,
               "kernels": kt16}
        log(f"B=16: {ms16:.3f} ms/step, {b16['frames_per_s']} frames/s")
        M.moshi_destroy(ctx)
        del ctx

    # ---------------- CPU oracle baseline ----------------
    cpu = None
    if not args.no_cpu and args.cpu_frames > 0:
        fps_cpu, dt = cpu_baseline(shape, weights, k, v, frames, args.cpu_frames)
        cpu = {"value": round(fps_cpu, 5), "unit": "frames/s", "cores": 1, "kind": "oracle",
               "sample": f"{args.cpu_frames} full-size frames (B=1, ring 3000, temporal + 16 "
                         f"depformer substeps) of the same workload, fp64, single thread, "
                         f"{dt:.1f}s"}
        log(f"CPU oracle: {fps_cpu:.4f} frames/s")

    rec = {
        "metric": METRIC, "value": round(fps, 2), "unit": "frames/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_wall, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f64",
        "storage": "bf16 weights, embeddings, K/V rings and projection inputs",
        "data": "synthetic",
        "config": {"workload": "full frame step, B=1: temporal 4096-d/32L/32h, F 11264, ring "
                               "prefilled to the 3000-frame window; text head 32000; depformer "
                               "1024-d/6L/16h, F 2816, 16 substeps with per-substep weights",
                   "batch": 1, "ring_fill": W, "parallelism": "none (one GPU)"},
        "rtf": round(ms_wall / FRAME_MS, 5),
        "ms_per_step_events": round(ms_gpu, 4),
        "ms_per_step_host_sync": round(ms_sync, 4),
        "bytes_per_step": bytes_step,
        "hbm_frac_step": round(step_gbs / HBM_PEAK_GBS, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "b16": b16,
        "kernels": kt,
    }
    print(json.dumps(rec), flush=True)
    # every context is destroyed: unload the library now, so that its HIP
    # module teardown does not run among the exit handlers (after a profiler
    # attached to the process may have finalised)
    M.unload()


if __name__ == "__main__":
    main()
