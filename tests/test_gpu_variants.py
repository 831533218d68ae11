"""GPU parity of the step's options against the fp64 oracle at small sizes:
teacher forcing (moshi_step_forced), the depformer readings (dep_q, the ring
reading, the final norm), the device-resident step with sessions joining and
leaving between enqueued steps, and the step kernel's bounded-wait failure
path (forced from the host by a tiny spin limit: every workgroup exits)."""
import os

import numpy as np
import pytest

import full_duplex_speech_amd as M
import oracle
from synth import spec, workloads as wl
from gpu_util import DevBuf, Stats, compare_frame, frames_matrix, log, new_engine

pytestmark = pytest.mark.gpu


def _forced_pattern(shape, B, t, live, seed):
    """Forced tokens of tick t: some text tokens and some codes forced, -1 elsewhere."""
    g = np.random.default_rng(seed * 1000 + t)
    f = np.full((B, shape.n_channels), -1, np.int32)
    for b in live:
        if g.random() < 0.4:
            f[b, 0] = g.integers(0, shape.text_vocab)
        for s in range(shape.n_substeps):
            if g.random() < 0.3:
                f[b, 1 + s] = g.integers(0, shape.audio_card)
    return f


def _run_forced(shape, weights, B, T, fills, seed=3, step_kernel=None):
    """B sessions (prefilled to `fills`) stepped T ticks with forcing; every
    session-frame checked against the oracle forced with the same tokens."""
    old = os.environ.get("MOSHI_STEP_KERNEL")
    if step_kernel is not None:
        os.environ["MOSHI_STEP_KERNEL"] = "1" if step_kernel else "0"
    try:
        ctx = new_engine(shape, weights, B)
    finally:
        if old is None:
            os.environ.pop("MOSHI_STEP_KERNEL", None)
        else:
            os.environ["MOSHI_STEP_KERNEL"] = old
    om = oracle.Model(shape, weights)
    orc, outs = [], []
    for b in range(len(fills)):
        assert M.moshi_session_join(ctx) == b
        o = oracle.Session(om)
        if fills[b]:
            k, v = wl.prefill_kv(shape, seed + 1, b, fills[b])
            M.moshi_session_prefill_kv(ctx, b, k, v)
            o.prefill(k, v)
        orc.append(o)
    stats = Stats()
    n = shape.dep_steps
    for t in range(T):
        fr = frames_matrix(shape, B, {b: wl.frames(shape, seed, b, t, 1)[0] for b in range(len(fills))})
        fc = _forced_pattern(shape, B, t, range(len(fills)), seed)
        tok, codes = M.moshi_step_forced(ctx, fr, fc)
        tl, al = M.moshi_read_logits(ctx)
        outs.append((tok.copy(), codes.copy(), tl.copy(), al.copy()))
        for b, o in enumerate(orc):
            # forced positions come back as given; the rest are the model's
            for s in range(shape.n_substeps):
                if s >= n:
                    assert codes[b, s] == -1
                elif fc[b, 1 + s] >= 0:
                    assert codes[b, s] == fc[b, 1 + s]
            if fc[b, 0] >= 0:
                assert tok[b] == fc[b, 0]
            # the oracle fed the same tokens; its own argmax is compared where
            # nothing was forced
            r = o.step(fr[b], forced_text=int(tok[b]), forced_codes=codes[b])
            ftok = int(tok[b]) if fc[b, 0] < 0 else r["text_token"]
            fcodes = codes[b].copy()
            for s in range(n):
                if fc[b, 1 + s] >= 0:
                    fcodes[s] = r["codes"][s]
            r2 = dict(r)
            r2["audio_logits"] = r["audio_logits"][:n]
            r2["codes"] = r["codes"][:n]
            r2["audio_margins"] = r["audio_margins"][:n]
            compare_frame(shape.replace(n_substeps=n), stats, f"t={t} b={b}", ftok, fcodes[:n],
                          tl[b], al[b][:n], r2)
            assert M.moshi_session_info(ctx, b) == o.info()
    used = M.moshi_uses_step_kernel(ctx)
    M.moshi_destroy(ctx)
    return outs, stats, used


@pytest.mark.parametrize("case", ["tiny_fp32_b1", "ragged_bf16_b3"])
def test_forced_step_parity(case):
    """Teacher forcing through the C ABI: forced tokens are fed on and
    returned; logits and the unforced tokens match the oracle."""
    if case == "tiny_fp32_b1":
        shape, B, fills, T = spec.TINY, 1, [0], 12
    else:
        shape, B, fills, T = spec.RAGGED, 3, [0, 20, 37], 12
    weights = wl.make_weights(shape, 71, gains="random")
    _, stats, used = _run_forced(shape, weights, B, T, fills)
    log(f"forced {case}: step kernel {used}; {stats}")


VARIANTS = {
    "dep_q8": dict(dep_q=8),
    "ref_ring": dict(dep_ref_ring=True),
    "final_norm": dict(dep_final_norm=True),
    "all_three": dict(dep_q=8, dep_ref_ring=True, dep_final_norm=True),
}


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_depformer_variants_parity(variant):
    """Each depformer reading: the step kernel (tiny fp32, B=1) and the
    per-operation kernels give bit-identical outputs, both match the oracle;
    the ragged bf16 model at B=3 (MFMA path) matches the oracle."""
    kw = VARIANTS[variant]
    shape = spec.TINY.replace(window=9, **kw)
    weights = wl.make_weights(shape, 73, gains="random")
    a, sa, used_a = _run_forced(shape, weights, 1, 12, [5], step_kernel=True)
    b, sb, used_b = _run_forced(shape, weights, 1, 12, [5], step_kernel=False)
    assert used_a and not used_b
    for t, (x, y) in enumerate(zip(a, b)):
        for u, v in zip(x, y):
            assert np.array_equal(u, v), f"{variant}: step kernel differs from per-op at t={t}"
    shape_r = spec.RAGGED.replace(**kw)
    weights_r = wl.make_weights(shape_r, 74, gains="random")
    _, sr, _ = _run_forced(shape_r, weights_r, 3, 8, [0, 11, 37])
    log(f"{variant}: tiny {sa}; ragged {sr}")


@pytest.mark.parametrize("case", ["tiny_fp32_b1", "ragged_bf16_b3"])
def test_enqueue_with_churn_matches_step(case):
    """Device-resident steps enqueued back to back while sessions join,
    prefill and leave between them (the metadata of an earlier step must not
    be overwritten before it runs), then one sync: tokens, codes and slot
    bookkeeping equal the same sequence run through moshi_step."""
    if case == "tiny_fp32_b1":
        shape, B = spec.TINY, 1
        plan = [("join", 0), ("step",), ("step",), ("leave", 0), ("step",), ("join", 1),
                ("prefill", 1, 7), ("step",), ("step",)]
    else:
        shape, B = spec.RAGGED, 3
        plan = [("join", 0), ("step",), ("join", 1), ("prefill", 1, 20), ("step",), ("join", 2),
                ("step",), ("leave", 0), ("step",), ("join", 3), ("step",), ("leave", 2),
                ("prefill", 1, 3), ("step",)]
    weights = wl.make_weights(shape, 77, gains="random")
    # the frames of every step, from the plan (joins take the lowest free slot)
    step_frames, slot_of, t_of = [], {}, {}
    for act in plan:
        if act[0] == "join":
            slot_of[act[1]] = min(set(range(B)) - set(slot_of.values()))
            t_of[act[1]] = 0
        elif act[0] == "leave":
            slot_of.pop(act[1])
        elif act[0] == "step":
            step_frames.append(frames_matrix(shape, B, {
                s: wl.frames(shape, 9, sid, t_of[sid], 1)[0] for sid, s in slot_of.items()}))
            for sid in slot_of:
                t_of[sid] += 1
    # every device buffer is ready before the first enqueue (no allocation or
    # copy between enqueued steps that could wait for them to finish)
    dev = [(DevBuf(fr), DevBuf(np.full(B, -7, np.int32)),
            DevBuf(np.full((B, shape.n_substeps), -7, np.int32))) for fr in step_frames]
    results = []
    for mode in ("enqueue", "sync"):
        ctx = new_engine(shape, weights, B)
        slot_of, outs, infos, k = {}, [], [], 0
        frames_of_step = []
        for act in plan:
            if act[0] == "join":
                slot_of[act[1]] = M.moshi_session_join(ctx)
            elif act[0] == "leave":
                M.moshi_session_leave(ctx, slot_of.pop(act[1]))
            elif act[0] == "prefill":
                kk, vv = wl.prefill_kv(shape, 5, act[1], act[2])
                M.moshi_session_prefill_kv(ctx, slot_of[act[1]], kk, vv)
            else:
                fr = step_frames[k]
                frames_of_step.append(fr)
                if mode == "sync":
                    tok, codes = M.moshi_step(ctx, fr)
                    outs.append((tok.copy(), codes.copy()))
                else:
                    d_fr, d_tok, d_codes = dev[k]
                    M.moshi_step_enqueue(ctx, d_fr.ptr, d_tok.ptr, d_codes.ptr)
                k += 1
                infos.append({sid: M.moshi_session_info(ctx, s) for sid, s in slot_of.items()})
        if mode == "enqueue":
            M.moshi_sync(ctx)
            outs = [(t.read(), c.read()) for _, t, c in dev]
        results.append((outs, infos, frames_of_step))
        M.moshi_destroy(ctx)
    (oe, ie, _), (os_, is_, _) = results
    assert ie == is_
    for i, ((t1, c1), (t2, c2)) in enumerate(zip(oe, os_)):
        assert np.array_equal(t1, t2) and np.array_equal(c1, c2), f"{case}: step {i} differs"


def test_step_kernel_wait_limit_fails_cleanly():
    """With the step kernel's waits limited to one poll, a launch gives up at
    its first wait that is not already satisfied: every workgroup leaves, the
    call reports a device error, the context stays failed, and a new context
    on the same GPU works."""
    shape = spec.TINY
    weights = wl.make_weights(shape, 79, gains="random")
    ctx = new_engine(shape, weights, 1)
    assert M.moshi_uses_step_kernel(ctx)
    slot = M.moshi_session_join(ctx)
    f = wl.frames(shape, 3, 0, 0, 2)
    M.moshi_step(ctx, f[0][None, :])  # a normal step first
    M.moshi_test_set_spin_limit(ctx, 1)
    with pytest.raises(M.MoshiError) as e:
        M.moshi_step(ctx, f[1][None, :])
    assert e.value.status == M.MOSHI_E_DEVICE
    with pytest.raises(M.MoshiError) as e:
        M.moshi_step(ctx, f[1][None, :])
    assert e.value.status == M.MOSHI_E_DEVICE
    M.moshi_destroy(ctx)
    # the GPU is fine: a fresh context steps and matches the oracle
    ctx = new_engine(shape, weights, 1)
    slot = M.moshi_session_join(ctx)
    o = oracle.Session(oracle.Model(shape, weights))
    tok, codes = M.moshi_step(ctx, f[0][None, :])
    tl, al = M.moshi_read_logits(ctx)
    r = o.step(f[0], forced_text=int(tok[slot]), forced_codes=codes[slot])
    compare_frame(shape, Stats(), "after abort", int(tok[slot]), codes[slot], tl[slot], al[slot], r)
    M.moshi_destroy(ctx)
