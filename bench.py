#!/usr/bin/env python3
"""Frame-step benchmark of the MI355X Moshi/PersonaPlex library.

One "step" is one full frame of the hot path for every live session: the
17-channel embedding, the 4096-d / 32-layer temporal transformer over a
3000-frame ring (prefilled full, N(0,1) K/V), the 32000-way text head, and the
16 depformer substeps (1024-d / 6 layers, per-substep weights) with a greedy
argmax on every head. Weights are N(0, 0.02) bf16 drawn from a fixed seed;
frames are uniform random codes (synthetic stand-ins for live Mimi streams).

Timed region: K device-resident steps (frames already in HBM, outputs written
to HBM) bracketed by torch.cuda.synchronize(), with a HIP event after every
step on the engine's stream (per-tick median / p90 / max). Printed: one JSON
line with frames/s at B=1 (the headline `value`), the real-time factor (step
time / 80 ms), the fraction of the HBM roofline for the whole step, the
roofline of the dominant kernel, the fp64 CPU oracle timed on a bounded
sample, and one line per other workload under "lines": the tiny fp32 model,
the temporal and depformer steps alone, 16 sessions (elastic fills) and 64
sessions (full rings), the 8-substep depformer reading and a 64-frame prefill.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "frames/sec (80 ms frames) at B=1 and B=16; % HBM roofline; real-time factor"
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, 8 TB/s
FP64_MFMA_PEAK_TFS = 78.6  # MI355X dense fp64 matrix peak
FRAME_MS = 80.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--timing-steps", type=int, default=3,
                    help="steps of the per-operation timing hook")
    ap.add_argument("--cpu-frames", type=int, default=2,
                    help="full-size frames the CPU oracle runs for its B=1 baseline")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--b1", type=int, default=1,
                    help="measure the B=1 headline workload (0: only the other workloads, "
                         "e.g. for counter runs; value is then null)")
    ap.add_argument("--b16", type=int, default=1, help="also measure B=16 (elastic fills)")
    ap.add_argument("--b64", type=int, default=1, help="also measure B=64 (full rings)")
    ap.add_argument("--extra", type=int, default=1,
                    help="also measure the tiny model, the temporal / depformer steps alone, "
                         "dep_q = 8 and the 64-frame prefill")
    ap.add_argument("--profile-b16", type=int, default=0,
                    help="only run this many host-synchronous steps of the B=16 workload "
                         "through the library's own stream, without torch (for hardware "
                         "counter runs: rocprofv3's SQ counters have crashed processes "
                         "that run torch), and exit")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (the reference "
                         "dispatch that scales HBM byte counters)")
    return ap.parse_args()


def make_engine(M, shape, weights, B, stream, flags=0):
    cfg = M.make_config(dim=shape.dim, n_layers=shape.n_layers, n_heads=shape.n_heads,
                        ffn_hidden=shape.ffn, window=shape.window, dep_dim=shape.dep_dim,
                        dep_layers=shape.dep_layers, dep_heads=shape.dep_heads,
                        dep_ffn_hidden=shape.dep_ffn, n_substeps=shape.n_substeps,
                        text_vocab=shape.text_vocab, audio_card=shape.audio_card,
                        rope_theta=shape.rope_theta, norm_eps=shape.norm_eps,
                        dtype=shape.dtype, max_sessions=B, flags=flags, dep_q=shape.dep_q)
    return M.moshi_create(cfg, weights, hip_stream=stream.cuda_stream)


def rnd(x, n):
    return None if x is None else round(x, n)


def ticks_stats(ticks):
    import numpy as np
    t = np.asarray(ticks)
    return {"median": round(float(np.median(t)), 4), "p90": round(float(np.percentile(t, 90)), 4),
            "max": round(float(t.max()), 4)}


def timed_steps(M, torch, ctx, stream, d_frames, d_text, d_codes, warmup, steps):
    """(wall ms/step, event ms/step, per-tick ms list)."""
    for k in range(warmup):
        M.moshi_step_enqueue(ctx, d_frames[k % d_frames.shape[0]].data_ptr())
    M.moshi_sync(ctx)
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    evs[0].record(stream)
    for k in range(steps):
        M.moshi_step_enqueue(ctx, d_frames[(warmup + k) % d_frames.shape[0]].data_ptr(),
                             d_text[k % d_text.shape[0]].data_ptr(),
                             d_codes[k % d_codes.shape[0]].data_ptr())
        evs[k + 1].record(stream)
    M.moshi_sync(ctx)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ticks = [evs[k].elapsed_time(evs[k + 1]) for k in range(steps)]
    return wall * 1000.0 / steps, evs[0].elapsed_time(evs[steps]) / steps, ticks


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


TEMPORAL_CLASSES = ("embed", "temporal_qkv", "temporal_attn", "temporal_o", "temporal_gateup",
                    "temporal_down", "text_head", "temporal_attn_combine")
DEPFORMER_CLASSES = ("dep_inproj", "dep_entry", "dep_qkv", "dep_attn", "dep_o", "dep_gateup",
                     "dep_down", "dep_head")


def phase(kt, classes):
    ms = sum(kt[c]["ms_per_step"] for c in classes if c in kt)
    by = sum(kt[c]["bytes_per_step"] for c in classes if c in kt)
    return ms, by


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


def cpu_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count()
    return {"nproc": os.cpu_count(), "cores_available": avail, "cpu_model": model}


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


def cpu_baseline_b16(shape, weights, w4, initial, threads):
    """The oracle on 16 sessions of the B=16 workload (their fills), one
    thread per session, one frame each."""
    import threading
    import oracle
    from synth import workloads as wl
    om = oracle.Model(shape, weights)
    sess = []
    for sid, fill in initial:
        o = oracle.Session(om)
        kk, vv = wl.prefill_kv(shape, w4.seed("prefill"), sid, fill, threads=16)
        o.prefill(kk, vv)
        sess.append((o, wl.frames(shape, w4.seed("frames"), sid, 0, 1)[0]))
    del kk, vv
    th = [threading.Thread(target=lambda o=o, f=f: o.step(f, want_logits=False))
          for o, f in sess[:threads]]
    t0 = time.perf_counter()
    for t in th:
        t.start()
    for t in th:
        t.join()
    dt = time.perf_counter() - t0
    return len(th) / dt, dt


def profile_b16(n):
    """n host-synchronous steps of the B=16 workload (workload 4's initial
    fills), library only: no torch in the process."""
    import numpy as np

    import full_duplex_speech_amd as M
    from synth import spec, workloads as wl

    shape = spec.PERSONAPLEX
    weights = wl.make_weights(shape, wl.MODEL_SEEDS["personaplex"], threads=16)
    cfg = M.make_config(dim=shape.dim, n_layers=shape.n_layers, n_heads=shape.n_heads,
                        ffn_hidden=shape.ffn, window=shape.window, dep_dim=shape.dep_dim,
                        dep_layers=shape.dep_layers, dep_heads=shape.dep_heads,
                        dep_ffn_hidden=shape.dep_ffn, n_substeps=shape.n_substeps,
                        text_vocab=shape.text_vocab, audio_card=shape.audio_card,
                        rope_theta=shape.rope_theta, norm_eps=shape.norm_eps,
                        dtype=shape.dtype, max_sessions=16)
    ctx = M.moshi_create(cfg, weights)
    w4 = wl.WORKLOADS[4]
    initial, _ = wl.churn_schedule(w4)
    for sid, fill in initial:
        s = M.moshi_session_join(ctx)
        kk, vv = wl.prefill_kv(shape, w4.seed("prefill"), sid, fill, threads=16)
        M.moshi_session_prefill_kv(ctx, s, kk, vv)
    fr = np.stack([wl.frames(shape, w4.seed("frames"), sid, 0, n) for sid, _ in initial], axis=1)
    t0 = time.perf_counter()
    for t in range(n):
        M.moshi_step(ctx, fr[t])
    ms = (time.perf_counter() - t0) * 1000.0 / max(n, 1)
    print(json.dumps({"profile_b16_steps": n, "ms_per_step_host_sync": round(ms, 3),
                      "dep_kernel": M.moshi_uses_dep_kernel(ctx)}), flush=True)
    M.moshi_destroy(ctx)
    M.unload()


def main():
    args = parse()
    if args.profile_b16 > 0:
        profile_b16(args.profile_b16)
        return
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
    lines = {}

    # ---------------- B = 1: the headline workload ----------------
    wk = wl.WORKLOADS[2]
    k, v = wl.prefill_kv(shape, wk.seed("prefill"), 0, W, threads=16)
    nfr = args.warmup + args.steps
    frames = wl.frames(shape, wk.seed("frames"), 0, 0, nfr)
    fps = ms_wall = ms_gpu = ms_sync = bytes_step = step_gbs = None
    ticks1, roofline, kt = None, None, {}
    if args.b1:
        ctx = make_engine(M, shape, weights, 1, stream)
        slot = M.moshi_session_join(ctx)
        M.moshi_session_prefill_kv(ctx, slot, k, v)
        d_frames = torch.from_numpy(frames.reshape(nfr, 1, -1)).to("cuda")
        d_text = torch.zeros((args.steps, 1), dtype=torch.int32, device="cuda")
        d_codes = torch.zeros((args.steps, 1, shape.n_substeps), dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        log("B=1 engine ready")
        ms_wall, ms_gpu, ticks1 = timed_steps(M, torch, ctx, stream, d_frames, d_text, d_codes,
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

        if args.extra:
            # workload 2 (temporal alone) and 3 (depformer alone): their phases
            # inside the step kernel (per-operation timestamps), and the
            # temporal-only / depformer-only entry points (per-operation kernels,
            # host-synchronous)
            tms, tby = phase(kt, TEMPORAL_CLASSES)
            dms, dby = phase(kt, DEPFORMER_CLASSES)
            t1 = time.perf_counter()
            for i in range(10):
                M.moshi_temporal_step(ctx, frames[i % nfr][None, :])
            t_entry = (time.perf_counter() - t1) * 100.0
            w3 = wl.WORKLOADS[3]
            hids, toks = wl.dep_inputs(shape, w3.seed("dep"), 0, 10)
            t1 = time.perf_counter()
            for i in range(10):
                M.moshi_depformer_step(ctx, hids[i][None, :], toks[i:i + 1])
            d_entry = (time.perf_counter() - t1) * 100.0
            lines["temporal_b1"] = {
                "workload": "temporal step alone, B=1, ring full at 3000 (workload 2)",
                "ms_in_step_kernel": round(tms, 4), "frames_per_s": round(1000.0 / tms, 1),
                "bytes_per_frame": tby, "hbm_frac": round(tby / (tms * 1e6) / HBM_PEAK_GBS, 4),
                "ms_temporal_entry_host_sync": round(t_entry, 4)}
            lines["depformer_b1"] = {
                "workload": "16 depformer substeps alone, B=1 (workload 3)",
                "ms_in_step_kernel": round(dms, 4), "frames_per_s": round(1000.0 / dms, 1),
                "bytes_per_frame": dby, "hbm_frac": round(dby / (dms * 1e6) / HBM_PEAK_GBS, 4),
                "ms_depformer_entry_host_sync": round(d_entry, 4)}
            log(f"temporal phase {tms:.3f} ms, depformer phase {dms:.3f} ms")

            # 64 frames prefilled at once after the full ring (MFMA columns)
            M.moshi_session_leave(ctx, slot)
            slot = M.moshi_session_join(ctx)
            M.moshi_session_prefill_kv(ctx, slot, k, v)
            pf = wl.frames(shape, wk.seed("frames") + 100, 0, 0, 64)
            M.moshi_session_prefill_frames(ctx, slot, pf)  # workspace + warm-up
            reps = 3
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            for _ in range(reps):
                M.moshi_session_leave(ctx, slot)
                slot = M.moshi_session_join(ctx)
                M.moshi_session_prefill_frames(ctx, slot, pf)
            ms_pf = (time.perf_counter() - t1) * 1000.0 / reps
            D, F, L = shape.dim, shape.ffn, shape.n_layers
            flops = 64 * (2.0 * (4 * D * D + 3 * F * D) * L + 2.0 * shape.text_vocab * D)
            tfs = flops / (ms_pf * 1e9)
            lines["b1_prefill_64"] = {
                "workload": "64 frames of one session prefilled at once (positions 0..63; "
                            "the projections as fp64 MFMA products over 64 columns)",
                "ms_per_call": round(ms_pf, 4), "frames_per_s": round(64 * 1000.0 / ms_pf, 1),
                "roofline": {"bound": "mfma", "achieved": round(tfs, 2),
                             "peak": FP64_MFMA_PEAK_TFS, "unit": "TFLOP/s",
                             "frac": round(tfs / FP64_MFMA_PEAK_TFS, 4)},
                "flops_per_call": flops}
            log(f"prefill 64 frames: {ms_pf:.2f} ms ({tfs:.1f} TFLOP/s)")
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

    if args.extra and args.b1:
        # the 8-substep depformer reading (dep_q = 8), B=1, full ring
        sh8 = shape.replace(dep_q=8)
        ctx = make_engine(M, sh8, weights, 1, stream)
        s8 = M.moshi_session_join(ctx)
        M.moshi_session_prefill_kv(ctx, s8, k, v)
        n8 = 50
        ms8, _, ticks8 = timed_steps(M, torch, ctx, stream, d_frames, d_text, d_codes, 5, n8)
        kt8 = kernel_table(M, ctx, frames[0][None, :], 1)
        by8 = sum(x["bytes_per_step"] for x in kt8.values())
        lines["b1_dep_q8"] = {
            "workload": "full step, B=1, ring full, depformer runs 8 substeps (dep_q = 8)",
            "ms_per_step": round(ms8, 4), "frames_per_s": round(1000.0 / ms8, 1),
            "rtf": round(ms8 / FRAME_MS, 5), "bytes_per_step": by8,
            "hbm_frac": round(by8 / (ms8 * 1e6) / HBM_PEAK_GBS, 4), "ticks_ms": ticks_stats(ticks8)}
        log(f"B=1 dep_q=8: {ms8:.3f} ms/step")
        M.moshi_destroy(ctx)
        del ctx

        # workload 1: the tiny fp32 model, B=1, 100 frames from an empty ring
        tiny = spec.TINY
        tw = wl.make_weights(tiny, wl.MODEL_SEEDS["tiny"])
        ctx = make_engine(M, tiny, tw, 1, stream)
        M.moshi_session_join(ctx)
        w1 = wl.WORKLOADS[1]
        tfr = torch.from_numpy(wl.frames(tiny, w1.seed("frames"), 0, 0, 110).reshape(110, 1, -1)).to("cuda")
        tt = torch.zeros((100, 1), dtype=torch.int32, device="cuda")
        tc = torch.zeros((100, 1, tiny.n_substeps), dtype=torch.int32, device="cuda")
        mst, _, tickst = timed_steps(M, torch, ctx, stream, tfr, tt, tc, 10, 100)
        lines["tiny_fp32_b1"] = {
            "workload": "tiny fp32 model (256-d/2L, depformer 128-d/2L), B=1, 100 frames, "
                        "ring wraps at 64 (workload 1; launch-latency bound)",
            "ms_per_step": round(mst, 4), "frames_per_s": round(1000.0 / mst, 1),
            "ticks_ms": ticks_stats(tickst)}
        log(f"tiny fp32: {mst:.3f} ms/step")
        M.moshi_destroy(ctx)
        del ctx, tw

    # ---------------- B = 16: elastic fills ----------------
    b16 = None
    w4 = wl.WORKLOADS[4]
    initial, _ = wl.churn_schedule(w4)
    if args.b16:
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
        ms16, ms16g, ticks16 = timed_steps(M, torch, ctx, stream, d16, t16, c16, 5, n16)
        kt16 = kernel_table(M, ctx, fr16[0], 1)
        by16 = sum(x["bytes_per_step"] for x in kt16.values())
        b16 = {"frames_per_s": round(16 * 1000.0 / ms16, 1), "ms_per_step": round(ms16, 4),
               "rtf": round(ms16 / FRAME_MS, 5), "bytes_per_step": by16,
               "hbm_frac_step": round(by16 / (ms16 * 1e6) / HBM_PEAK_GBS, 4),
               "fills": "U{0..3000} per slot (workload 4 at t=0)", "steps": n16,
               "ticks_ms": ticks_stats(ticks16), "kernels": kt16}
        log(f"B=16: {ms16:.3f} ms/step, {b16['frames_per_s']} frames/s")
        M.moshi_destroy(ctx)
        del ctx, d16

    # ---------------- B = 64: every ring full ----------------
    if args.b64:
        ctx = make_engine(M, shape, weights, 64, stream)
        for sid in range(64):
            s = M.moshi_session_join(ctx)
            # every ring holds the same 3000 prefilled positions (the bytes
            # each step streams do not depend on their values)
            M.moshi_session_prefill_kv(ctx, s, k, v)
        w5 = wl.WORKLOADS[5]
        n64 = 20
        fr64 = np.stack([wl.frames(shape, w5.seed("frames"), sid, 0, n64 + 3)
                         for sid in range(64)], axis=1)
        d64 = torch.from_numpy(np.ascontiguousarray(fr64)).to("cuda")
        t64 = torch.zeros((n64, 64), dtype=torch.int32, device="cuda")
        c64 = torch.zeros((n64, 64, shape.n_substeps), dtype=torch.int32, device="cuda")
        ms64, _, ticks64 = timed_steps(M, torch, ctx, stream, d64, t64, c64, 3, n64)
        kt64 = kernel_table(M, ctx, fr64[0], 1)
        by64 = sum(x["bytes_per_step"] for x in kt64.values())
        lines["b64_full_rings"] = {
            "workload": "full step, B=64, every ring full at 3000 (workload 5)",
            "ms_per_step": round(ms64, 4), "frames_per_s": round(64 * 1000.0 / ms64, 1),
            "rtf": round(ms64 / FRAME_MS, 5), "bytes_per_step": by64,
            "hbm_frac": round(by64 / (ms64 * 1e6) / HBM_PEAK_GBS, 4),
            "ticks_ms": ticks_stats(ticks64), "kernels": kt64}
        log(f"B=64: {ms64:.3f} ms/step, {64 * 1000.0 / ms64:.1f} frames/s")
        M.moshi_destroy(ctx)
        del ctx, d64

    # ---------------- B = 4: every ring full (context) ----------------
    # the pages' one multi-session figure is four concurrent sessions at
    # ~70-74 ms per tick on an H20-class GPU (whole serving loop, other
    # hardware): context only
    if args.extra:
        ctx = make_engine(M, shape, weights, 4, stream)
        for sid in range(4):
            s = M.moshi_session_join(ctx)
            M.moshi_session_prefill_kv(ctx, s, k, v)
        w5 = wl.WORKLOADS[5]
        n4 = 40
        fr4 = np.stack([wl.frames(shape, w5.seed("frames"), sid, 0, n4 + 3)
                        for sid in range(4)], axis=1)
        d4 = torch.from_numpy(np.ascontiguousarray(fr4)).to("cuda")
        t4 = torch.zeros((n4, 4), dtype=torch.int32, device="cuda")
        c4 = torch.zeros((n4, 4, shape.n_substeps), dtype=torch.int32, device="cuda")
        ms4, _, ticks4 = timed_steps(M, torch, ctx, stream, d4, t4, c4, 3, n4)
        kt4 = kernel_table(M, ctx, fr4[0], 1)
        by4 = sum(x["bytes_per_step"] for x in kt4.values())
        lines["b4_full_rings"] = {
            "workload": "full step, B=4, every ring full at 3000 (the B=64 workload's "
                        "first 4 sessions)",
            "ms_per_step": round(ms4, 4), "frames_per_s": round(4 * 1000.0 / ms4, 1),
            "rtf": round(ms4 / FRAME_MS, 5), "bytes_per_step": by4,
            "hbm_frac": round(by4 / (ms4 * 1e6) / HBM_PEAK_GBS, 4),
            "ticks_ms": ticks_stats(ticks4), "kernels": kt4}
        log(f"B=4: {ms4:.3f} ms/step, {4 * 1000.0 / ms4:.1f} frames/s")
        M.moshi_destroy(ctx)
        del ctx, d4

    # ---------------- CPU oracle baseline ----------------
    cpu = None
    if not args.no_cpu and args.cpu_frames > 0:
        info = cpu_info()
        fps_cpu, dt = cpu_baseline(shape, weights, k, v, frames, args.cpu_frames)
        cpu = {"value": round(fps_cpu, 5), "unit": "frames/s", "cores": 1, "kind": "oracle",
               "sample": f"{args.cpu_frames} full-size frames (B=1, ring 3000, temporal + 16 "
                         f"depformer substeps) of the same workload, fp64, single thread, "
                         f"{dt:.1f}s", **info}
        log(f"CPU oracle: {fps_cpu:.4f} frames/s")
        if args.b16:
            nth = min(16, info["cores_available"] or 1)
            fps16, dt16 = cpu_baseline_b16(shape, weights, w4, initial, nth)
            cpu["b16"] = {"value": round(fps16, 4), "unit": "frames/s", "cores": nth,
                          "sample": f"one frame of each of {nth} sessions of the B=16 workload "
                                    f"(their fills), one thread per session, {dt16:.1f}s"}
            log(f"CPU oracle B=16: {fps16:.4f} frames/s on {nth} threads")

    rec = {
        "metric": METRIC, "value": rnd(fps, 2), "unit": "frames/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": rnd(ms_wall, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f64",
        "storage": "bf16 weights, embeddings, K/V rings and projection inputs",
        "data": "synthetic",
        "config": {"workload": "full frame step, B=1: temporal 4096-d/32L/32h, F 11264, ring "
                               "prefilled to the 3000-frame window; text head 32000; depformer "
                               "1024-d/6L/16h, F 2816, 16 substeps with per-substep weights",
                   "batch": 1, "ring_fill": W, "parallelism": "none (one GPU)"},
        "rtf": rnd(ms_wall / FRAME_MS if ms_wall else None, 5),
        "ms_per_step_events": rnd(ms_gpu, 4),
        "ms_per_step_host_sync": rnd(ms_sync, 4),
        "ticks_ms": ticks_stats(ticks1) if ticks1 else None,
        "bytes_per_step": bytes_step,
        "hbm_frac_step": rnd(step_gbs / HBM_PEAK_GBS if step_gbs else None, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "b16": b16,
        "lines": lines,
        "kernels": kt,
    }
    print(json.dumps(rec), flush=True)
    # every context is destroyed: unload the library now, so that its HIP
    # module teardown does not run among the exit handlers
    M.unload()


if __name__ == "__main__":
    main()
