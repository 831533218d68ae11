"""GPU parity at the full PersonaPlex shape (4096-d / 32 layers, window 3000;
depformer 1024-d / 6 layers, 16 substeps), in the launch configuration the
benchmark times, on the four full-size workloads.

The oracle takes seconds per full-size frame, so it checks sampled frames:
* frames computed straight from the seeded prefill (the first frames of a
  session, or of a session that just joined);
* later frames, by loading the GPU's ring for that slot into an oracle
  session (the GPU's K/V of earlier positions) and stepping the oracle from
  there; at B=1 these segments are spread over the whole run, and the K/V
  rows the oracle writes are compared with the rows the GPU wrote;
* every depformer-only frame is independent, so any frame can be sampled.
Bit-exact isolation (a session replayed alone in a fresh engine) and the ring
bookkeeping are checked on every frame.
"""
import threading

import numpy as np
import pytest

import full_duplex_speech_amd as M
import oracle
from synth import spec, workloads as wl
from gpu_util import Stats, cfg_of, compare_frame, log

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

SHAPE = spec.PERSONAPLEX


@pytest.fixture(scope="module")
def weights():
    log("generating full-size weights (16.7 GB)")
    w = wl.make_weights(SHAPE, wl.MODEL_SEEDS["personaplex"], threads=16)
    log("weights ready")
    return w


@pytest.fixture(scope="module")
def omodel(weights):
    return oracle.Model(SHAPE, weights)


def _parallel(jobs):
    """Run oracle jobs (callables) in threads; the C oracle releases the GIL."""
    out = [None] * len(jobs)
    err = []

    def run(i, f):
        try:
            out[i] = f()
        except BaseException as e:  # re-raised below
            err.append(e)

    th = [threading.Thread(target=run, args=(i, f)) for i, f in enumerate(jobs)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    if err:
        raise err[0]
    return out


def _oracle_from_prefill(om, k, v, frame, tok, codes):
    s = oracle.Session(om)
    s.prefill(k, v)
    return s.step(frame, forced_text=int(tok), forced_codes=codes)


def _oracle_from_ring(om, pos, k, v, frame, tok, codes):
    s = oracle.Session(om)
    s.load_ring(pos, k, v)
    return s.step(frame, forced_text=int(tok), forced_codes=codes)


@pytest.fixture(scope="module")
def b1(weights):
    ctx = M.moshi_create(cfg_of(SHAPE, 1), weights)
    log("B=1 engine created")
    yield ctx
    M.moshi_destroy(ctx)


def _kv_rows_match(tag, gk, gv, ok_, ov_, slots):
    """The K/V rows of ring slots `slots` written by the GPU equal the oracle's:
    every element within one bf16 step (both sides round an fp64 value, so
    they differ only where that value lies within rounding error of a bf16
    midpoint); the count of non-identical elements is reported."""
    diff = 0
    for a, b in ((gk, ok_), (gv, ov_)):
        x = a[:, slots].astype(np.int32)
        y = b[:, slots].astype(np.int32)
        ne = x != y
        diff += int(ne.sum())
        if ne.any():  # adjacent bf16 values of the same sign differ by 1 in their bits
            assert np.max(np.abs(x[ne] - y[ne])) == 1 and np.all((x[ne] ^ y[ne]) < 0x8000), \
                f"{tag}: K/V rows differ by more than one bf16 step"
    n = 2 * gk.shape[0] * len(slots) * gk.shape[2]
    log(f"{tag}: K/V rows of slots {slots}: {n - diff}/{n} bit-identical")
    assert diff <= n // 100000, f"{tag}: {diff} K/V elements off by one bf16 step"


def _segment_check(tag, omodel, pos, rk0, rv0, frames, outs, rk1, rv1, temporal_only, stats):
    """From the GPU's ring before frame t0 (rk0, rv0 at position pos), the
    oracle steps the same frames (teacher-forced on the GPU's tokens): logits
    and tokens match, and the K/V rows it writes equal the GPU's (rk1, rv1,
    read after those frames)."""
    o = oracle.Session(omodel)
    o.load_ring(pos, rk0, rv0)
    for i, (fr, out) in enumerate(zip(frames, outs)):
        if temporal_only:
            tok, tl = out
            r = o.temporal(fr)
            compare_frame(SHAPE, stats, f"{tag} +{i}", tok, None, tl, None, r)
        else:
            tok, codes, tl, al = out
            r = o.step(fr, forced_text=int(tok), forced_codes=codes)
            compare_frame(SHAPE, stats, f"{tag} +{i}", tok, codes, tl, al, r)
    ok_, ov_ = o.read_ring()
    W = SHAPE.window
    _kv_rows_match(tag, rk1, rv1, ok_, ov_, [(pos + i) % W for i in range(len(frames))])
    return True


SEG_STARTS = (2, 60, 131, 197)  # each segment: 2 frames checked from the GPU's ring


def _run_b1_with_segments(ctx, omodel, temporal_only):
    """200 frames of workload 2 at B=1 (ring full at 3000). Frames 0, 1 are
    checked against the oracle stepped from the seeded prefill (with the K/V
    rows it writes); each segment of SEG_STARTS from the GPU's own ring just
    before it. Oracle work runs in threads after the GPU run."""
    w2 = wl.WORKLOADS[2]
    slot = M.moshi_session_join(ctx)
    k, v = wl.prefill_kv(SHAPE, w2.seed("prefill"), 0, SHAPE.window, threads=16)
    M.moshi_session_prefill_kv(ctx, slot, k, v)
    n = w2.frames
    frames = wl.frames(SHAPE, w2.seed("frames"), 0, 0, n)
    outs, segs = [], []
    pending = None
    for t in range(n):
        if t in SEG_STARTS:
            pos = M.moshi_session_info(ctx, slot)[0]
            rk0, rv0 = M.moshi_session_read_kv(ctx, slot)
            pending = (t, pos, rk0, rv0)
        if temporal_only:
            tok = M.moshi_temporal_step(ctx, frames[t][None, :])
            tl, _ = M.moshi_read_logits(ctx, audio=False)
            outs.append((int(tok[0]), tl[0].copy()))
        else:
            tok, codes = M.moshi_step(ctx, frames[t][None, :])
            tl, al = M.moshi_read_logits(ctx)
            outs.append((int(tok[0]), codes[0].copy(), tl[0].copy(), al[0].copy()))
        if t == 1 or (pending is not None and t == pending[0] + 1):
            rk1, rv1 = M.moshi_session_read_kv(ctx, slot)
            if t == 1:
                segs.append(("from prefill", None, None, None, 0, rk1, rv1))
            else:
                t0, pos, rk0, rv0 = pending
                segs.append((f"t={t0}", pos, rk0, rv0, t0, rk1, rv1))
                pending = None
    assert M.moshi_session_info(ctx, slot) == (SHAPE.window + n, SHAPE.window, n % SHAPE.window)
    M.moshi_session_leave(ctx, slot)
    log(f"B=1 GPU run done ({'temporal' if temporal_only else 'full step'}); "
        f"{len(segs)} segments to check")
    stats = Stats()

    def job(seg):
        tag, pos, rk0, rv0, t0, rk1, rv1 = seg
        if pos is None:
            o = oracle.Session(omodel)
            o.prefill(k, v)
            rk0, rv0 = o.read_ring()
            pos = SHAPE.window
        return _segment_check(tag, omodel, pos, rk0, rv0, frames[t0:t0 + 2], outs[t0:t0 + 2],
                              rk1, rv1, temporal_only, stats)

    _parallel([lambda s=s: job(s) for s in segs])
    log(f"B=1 segments ok {stats}")


def test_w2_temporal_b1(b1, omodel):
    """Workload 2: temporal step, ring full at 3000, 200 frames; oracle-checked
    segments spread over the run, with the K/V rows the GPU writes."""
    _run_b1_with_segments(b1, omodel, temporal_only=True)


def test_w3_depformer_b1(b1, omodel):
    """Workload 3: depformer alone from N(0,1) hidden states, 1000 frames;
    every frame is independent, so sampled frames are checked directly."""
    ctx = b1
    slot = M.moshi_session_join(ctx)
    w3 = wl.WORKLOADS[3]
    sample = {0, 1, 500, 999}
    hids, toks = wl.dep_inputs(SHAPE, w3.seed("dep"), 0, w3.frames)
    stats = Stats()
    jobs = []
    from synth.rng import bf16_to_f32
    for t in range(w3.frames):
        codes = M.moshi_depformer_step(ctx, hids[t][None, :], toks[t:t + 1])
        if t in sample:
            _, al = M.moshi_read_logits(ctx, text=False)
            hid64 = bf16_to_f32(hids[t]).astype(np.float64)
            jobs.append((t, codes[0].copy(), al[0].copy(),
                         (lambda h=hid64, tt=int(toks[t]), c=codes[0].copy():
                          omodel.depformer(h, tt, forced=c))))
    res = _parallel([j[3] for j in jobs])
    for (t, codes, al, _), r in zip(jobs, res):
        r["text_margin"], r["text_token"] = np.inf, 0
        compare_frame(SHAPE, stats, f"w3 t={t}", 0, codes, None, al, r)
    log(f"w3 done {stats}")
    M.moshi_session_leave(ctx, slot)


def test_full_step_b1(b1, omodel):
    """Temporal + depformer at B=1 with a full ring (the benchmark's step):
    oracle-checked segments spread over 200 frames, with the K/V rows."""
    log(f"full step B=1: step kernel {M.moshi_uses_step_kernel(b1)}")
    _run_b1_with_segments(b1, omodel, temporal_only=False)


def _elastic_run(weights, B, w, bank, plan_initial, events, T, want_ring_at=None,
                 sample_sid=None):
    """Run an elastic workload; returns per-session outputs, joins, ring dumps."""
    ctx = M.moshi_create(cfg_of(SHAPE, B), weights)
    slot_of, t_of, outs, joined_at, rings = {}, {}, {}, {}, {}
    fill_of = {}

    def join(sid, fill):
        s = M.moshi_session_join(ctx)
        slot_of[sid] = s
        kk, vv = wl.prefill_from_bank(bank, sid, fill)
        M.moshi_session_prefill_kv(ctx, s, kk, vv)
        t_of[sid] = 0
        fill_of[sid] = fill

    for sid, fill in plan_initial:
        join(sid, fill)
    for t in range(T):
        for act in events.get(t, []):
            if act[0] == "leave":
                M.moshi_session_leave(ctx, slot_of.pop(act[1]))
            else:
                join(act[1], act[2])
                joined_at[act[1]] = t
        if want_ring_at is not None and t == want_ring_at:
            for sid in sample_sid or []:
                if sid in slot_of:
                    rk, rv = M.moshi_session_read_kv(ctx, slot_of[sid])
                    rings[sid] = (M.moshi_session_info(ctx, slot_of[sid])[0], rk, rv)
        f = np.zeros((B, SHAPE.n_channels), np.int32)
        for sid, s in slot_of.items():
            f[s] = wl.frames(SHAPE, w.seed("frames"), sid, t_of[sid], 1)[0]
        tok, codes = M.moshi_step(ctx, f)
        need_logits = (t == 0) or (t == want_ring_at) or any(joined_at.get(sid) == t
                                                              for sid in slot_of)
        tl = al = None
        if need_logits:
            tl, al = M.moshi_read_logits(ctx)
        for sid, s in slot_of.items():
            rec = (int(tok[s]), codes[s].copy(), f[s].copy(),
                   None if tl is None else tl[s].copy(), None if al is None else al[s].copy())
            outs.setdefault(sid, []).append(rec)
            t_of[sid] += 1
    M.moshi_destroy(ctx)
    return outs, joined_at, rings, fill_of


def test_w4_elastic_b16(weights, omodel):
    """Workload 4: 16 slots with fills U{0..3000}, 2 leave and 2 join every 50
    frames, 500 frames; sampled oracle checks + bit-exact isolation."""
    w = wl.WORKLOADS[4]
    bank = wl.prefill_bank(SHAPE, w.seed("prefill"), threads=16)
    initial, events = wl.churn_schedule(w)
    last = w.frames - 1
    stay = [sid for sid, _ in initial
            if not any(a[0] == "leave" and a[1] == sid for acts in events.values() for a in acts)]
    ring_sids = stay[:2]
    outs, joined_at, rings, fill_of = _elastic_run(weights, 16, w, bank, initial, events, w.frames,
                                                   want_ring_at=last, sample_sid=ring_sids)
    log("w4 GPU run done")
    stats = Stats()
    jobs, meta = [], []
    for sid, fill in initial[:3]:                         # tick 0, from the seeded prefill
        tok, codes, fr, tl, al = outs[sid][0]
        kk, vv = wl.prefill_from_bank(bank, sid, fill)
        jobs.append(lambda kk=kk, vv=vv, fr=fr, tok=tok, codes=codes:
                    _oracle_from_prefill(omodel, kk, vv, fr, tok, codes))
        meta.append((f"w4 sid={sid} t=0", tok, codes, tl, al))
    for sid, t0 in sorted(joined_at.items())[-2:]:          # the last joiners' first frame
        tok, codes, fr, tl, al = outs[sid][0]
        kk, vv = wl.prefill_from_bank(bank, sid, fill_of[sid])
        jobs.append(lambda kk=kk, vv=vv, fr=fr, tok=tok, codes=codes:
                    _oracle_from_prefill(omodel, kk, vv, fr, tok, codes))
        meta.append((f"w4 sid={sid} joined t={t0}", tok, codes, tl, al))
    for sid, (pos, rk, rv) in rings.items():                # the last frame, from the GPU ring
        tok, codes, fr, tl, al = outs[sid][-1]
        jobs.append(lambda pos=pos, rk=rk, rv=rv, fr=fr, tok=tok, codes=codes:
                    _oracle_from_ring(omodel, pos, rk, rv, fr, tok, codes))
        meta.append((f"w4 sid={sid} t={last} (from ring)", tok, codes, tl, al))
    res = _parallel(jobs)
    for (tag, tok, codes, tl, al), r in zip(meta, res):
        compare_frame(SHAPE, stats, tag, tok, codes, tl, al, r)
    log(f"w4 oracle samples ok {stats}")
    del rings
    # isolation: one session that stays all along, replayed alone in a fresh engine
    sid = stay[0]
    fill = dict(initial)[sid]
    alone, _, _, _ = _elastic_run(weights, 16, w, bank, [(sid, fill)], {}, w.frames)
    for t, (a, b) in enumerate(zip(alone[sid], outs[sid])):
        assert a[0] == b[0] and np.array_equal(a[1], b[1]), f"isolation broken at t={t}"
    log("w4 isolation bit-exact over 500 frames")


def test_w5_b64_full_rings(weights, omodel):
    """Workload 5: 64 slots, every ring at the full 3000-frame window, 300 frames."""
    w = wl.WORKLOADS[5]
    bank = wl.prefill_bank(SHAPE, w.seed("prefill"), threads=16)
    initial = [(sid, SHAPE.window) for sid in range(64)]
    last = w.frames - 1
    outs, _, rings, _ = _elastic_run(weights, 64, w, bank, initial, {}, w.frames,
                                     want_ring_at=last, sample_sid=[63])
    log("w5 GPU run done")
    stats = Stats()
    jobs, meta = [], []
    for sid in (0, 37):
        tok, codes, fr, tl, al = outs[sid][0]
        kk, vv = wl.prefill_from_bank(bank, sid, SHAPE.window)
        jobs.append(lambda kk=kk, vv=vv, fr=fr, tok=tok, codes=codes:
                    _oracle_from_prefill(omodel, kk, vv, fr, tok, codes))
        meta.append((f"w5 sid={sid} t=0", tok, codes, tl, al))
    pos, rk, rv = rings[63]
    tok, codes, fr, tl, al = outs[63][-1]
    jobs.append(lambda: _oracle_from_ring(omodel, pos, rk, rv, fr, tok, codes))
    meta.append((f"w5 sid=63 t={last} (from ring)", tok, codes, tl, al))
    res = _parallel(jobs)
    for (tag, tok, codes, tl, al), r in zip(meta, res):
        compare_frame(SHAPE, stats, tag, tok, codes, tl, al, r)
    log(f"w5 oracle samples ok {stats}")


def test_prefill_frames_b1_full_ring(b1, omodel):
    """64 frames prefilled at once after the full 3000-frame ring (positions
    3000..3063, one MFMA chunk): frames 0 and 1 against the oracle stepped
    from the seeded prefill, frame 63 against the oracle stepped from the
    GPU's ring after the call, with the K/V rows of those positions."""
    ctx = b1
    w2 = wl.WORKLOADS[2]
    slot = M.moshi_session_join(ctx)
    k, v = wl.prefill_kv(SHAPE, w2.seed("prefill"), 0, SHAPE.window, threads=16)
    M.moshi_session_prefill_kv(ctx, slot, k, v)
    n = 64
    frames = wl.frames(SHAPE, w2.seed("frames") + 100, 0, 0, n)
    tok, tl = M.moshi_session_prefill_frames(ctx, slot, frames, want_logits=True)
    assert M.moshi_session_info(ctx, slot)[0] == SHAPE.window + n
    rk, rv = M.moshi_session_read_kv(ctx, slot)
    M.moshi_session_leave(ctx, slot)
    log("prefill of 64 frames done on the GPU")
    stats = Stats()

    def first_frames():
        o = oracle.Session(omodel)
        o.prefill(k, v)
        out = [o.temporal(frames[j]) for j in range(2)]
        return out, o.read_ring()

    def last_frame():
        o = oracle.Session(omodel)
        o.load_ring(SHAPE.window + n - 1, rk, rv)
        r = o.temporal(frames[n - 1])
        return r, o.read_ring()

    (firsts, ring_a), (last, ring_b) = _parallel([first_frames, last_frame])
    for j, r in enumerate(firsts):
        compare_frame(SHAPE, stats, f"prefill frame {j}", int(tok[j]), None, tl[j], None, r)
    compare_frame(SHAPE, stats, f"prefill frame {n - 1}", int(tok[n - 1]), None, tl[n - 1], None,
                  last)
    _kv_rows_match("prefill frames 0-1", rk, rv, ring_a[0], ring_a[1], [0, 1])
    _kv_rows_match("prefill frame 63", rk, rv, ring_b[0], ring_b[1], [(SHAPE.window + n - 1) % SHAPE.window])
    log(f"prefill 64 frames: {stats}")


def test_dep_q8_full_step_b1(weights):
    """The 8-substep depformer reading (dep_q = 8) at full size through the
    step kernel: the first frames from the seeded prefill against the oracle
    of the same reading; codes of substeps 8..15 are -1."""
    shape = SHAPE.replace(dep_q=8)
    ctx = M.moshi_create(cfg_of(shape, 1), weights)
    assert M.moshi_uses_step_kernel(ctx)
    om = oracle.Model(shape, weights)
    w2 = wl.WORKLOADS[2]
    slot = M.moshi_session_join(ctx)
    k, v = wl.prefill_kv(shape, w2.seed("prefill"), 0, shape.window, threads=16)
    M.moshi_session_prefill_kv(ctx, slot, k, v)
    frames = wl.frames(shape, w2.seed("frames"), 0, 0, 3)
    o = oracle.Session(om)
    o.prefill(k, v)
    stats = Stats()
    n = shape.dep_steps
    for t in range(3):
        tok, codes = M.moshi_step(ctx, frames[t][None, :])
        tl, al = M.moshi_read_logits(ctx)
        assert (codes[0][n:] == -1).all()
        r = o.step(frames[t], forced_text=int(tok[0]), forced_codes=codes[0])
        r2 = dict(r, audio_logits=r["audio_logits"][:n], codes=r["codes"][:n],
                  audio_margins=r["audio_margins"][:n])
        compare_frame(shape.replace(n_substeps=n), stats, f"dep_q8 t={t}", int(tok[0]),
                      codes[0][:n], tl[0], al[0][:n], r2)
    M.moshi_destroy(ctx)
    log(f"dep_q=8 full step: {stats}")


def test_b3_full_size_valu_tiles(weights, omodel):
    """Three slots, so the temporal projections run on the fp64 VALU tiles of
    two to four sessions (among them the 11264-wide down projection, whose
    last batch is partial), with rings at 3000, 1000 and 7: the first frame
    of every slot from its prefill, and the third frame of the full-ring slot
    from the GPU's ring, against the oracle."""
    w = wl.WORKLOADS[5]
    bank = wl.prefill_bank(SHAPE, w.seed("prefill"), threads=16)
    initial = [(0, SHAPE.window), (1, 1000), (2, 7)]
    T = 3
    outs, _, rings, _ = _elastic_run(weights, 3, w, bank, initial, {}, T, want_ring_at=T - 1,
                                     sample_sid=[0])
    log("B=3 GPU run done")
    stats = Stats()
    jobs, meta = [], []
    for sid, fill in initial:
        tok, codes, fr, tl, al = outs[sid][0]
        kk, vv = wl.prefill_from_bank(bank, sid, fill)
        jobs.append(lambda kk=kk, vv=vv, fr=fr, tok=tok, codes=codes:
                    _oracle_from_prefill(omodel, kk, vv, fr, tok, codes))
        meta.append((f"B=3 sid={sid} fill={fill} t=0", tok, codes, tl, al))
    pos, rk, rv = rings[0]
    tok, codes, fr, tl, al = outs[0][-1]
    jobs.append(lambda: _oracle_from_ring(omodel, pos, rk, rv, fr, tok, codes))
    meta.append((f"B=3 sid=0 t={T - 1} (from ring)", tok, codes, tl, al))
    res = _parallel(jobs)
    for (tag, tok, codes, tl, al), r in zip(meta, res):
        compare_frame(SHAPE, stats, tag, tok, codes, tl, al, r)
    log(f"B=3 oracle samples ok {stats}")
