"""GPU parity of the multi-frame prefill (moshi_session_prefill_frames:
the temporal transformer over n frames of one session at once, 64 frames per
MFMA chunk) against the oracle stepping the same frames one at a time:
per-frame text logits and greedy tokens, the ring contents afterwards, and
the next regular steps. Cases: the ring wrapping inside one call (70 frames,
window 64), a chunk wider than the window (50 frames, window 37), the
masked-oldest reading, a one-frame call, and other live sessions in the
batch that must not be disturbed."""
import numpy as np
import pytest

import full_duplex_speech_amd as M
import oracle
from synth import spec, workloads as wl
from gpu_util import Stats, compare_frame, frames_matrix, log, new_engine

pytestmark = pytest.mark.gpu


def _check_prefill(shape, ctx, slot, o, frames, stats, tag):
    tok, tl = M.moshi_session_prefill_frames(ctx, slot, frames, want_logits=True)
    for j, fr in enumerate(frames):
        r = o.temporal(fr)
        compare_frame(shape, stats, f"{tag} frame {j}", int(tok[j]), None, tl[j], None, r)
    assert M.moshi_session_info(ctx, slot) == o.info()


def _check_ring(shape, ctx, slot, o, tag):
    gk, gv = M.moshi_session_read_kv(ctx, slot)
    ok_, ov_ = o.read_ring()
    pos = o.info()[0]
    rows = sorted({p % shape.window for p in range(max(0, pos - shape.window), pos)})
    for a, b in ((gk, ok_), (gv, ov_)):
        if shape.dtype == "bf16":
            x, y = a[:, rows].astype(np.int32), b[:, rows].astype(np.int32)
            assert np.max(np.abs(x - y)) <= 1, f"{tag}: K/V rows differ by more than one bf16 step"
        else:
            assert np.allclose(a[:, rows], b[:, rows], rtol=1e-5, atol=1e-6), f"{tag}: K/V rows"


@pytest.mark.parametrize("case", ["tiny_fp32_wrap", "ragged_bf16_wide", "mask_oldest", "one_frame"])
def test_prefill_parity(case):
    if case == "tiny_fp32_wrap":
        shape, fill, pieces = spec.TINY, 0, [70]
    elif case == "ragged_bf16_wide":
        shape, fill, pieces = spec.RAGGED, 30, [20, 50]
    elif case == "mask_oldest":
        shape, fill, pieces = spec.RAGGED.replace(window=9, mask_oldest=True), 4, [12, 3]
    else:
        shape, fill, pieces = spec.RAGGED, 10, [1, 1]
    weights = wl.make_weights(shape, 87, gains="random")
    ctx = new_engine(shape, weights, 1)
    slot = M.moshi_session_join(ctx)
    o = oracle.Session(oracle.Model(shape, weights))
    if fill:
        k, v = wl.prefill_kv(shape, 88, 0, fill)
        M.moshi_session_prefill_kv(ctx, slot, k, v)
        o.prefill(k, v)
    stats = Stats()
    t = 0
    for n in pieces:
        frames = wl.frames(shape, 89, 0, t, n)
        _check_prefill(shape, ctx, slot, o, frames, stats, case)
        t += n
    _check_ring(shape, ctx, slot, o, case)
    # regular steps continue from the prefilled state
    for j in range(3):
        f = wl.frames(shape, 89, 0, t + j, 1)
        tok, codes = M.moshi_step(ctx, f)
        tl, al = M.moshi_read_logits(ctx)
        r = o.step(f[0], forced_text=int(tok[slot]), forced_codes=codes[slot])
        compare_frame(shape, stats, f"{case} step {j}", int(tok[slot]), codes[slot], tl[slot],
                      al[slot], r)
    M.moshi_destroy(ctx)
    log(f"prefill {case}: {stats}")


def test_prefill_leaves_other_slots_alone():
    """Capacity 3: slot 1 is prefilled with 40 frames while slots 0 and 2
    hold sessions; then every session steps and matches its oracle."""
    shape = spec.RAGGED
    weights = wl.make_weights(shape, 90, gains="random")
    om = oracle.Model(shape, weights)
    ctx = new_engine(shape, weights, 3)
    orc = []
    for b, fill in enumerate((5, 0, 37)):
        assert M.moshi_session_join(ctx) == b
        o = oracle.Session(om)
        if fill:
            k, v = wl.prefill_kv(shape, 91, b, fill)
            M.moshi_session_prefill_kv(ctx, b, k, v)
            o.prefill(k, v)
        orc.append(o)
    stats = Stats()
    f0 = np.stack([wl.frames(shape, 92, b, 0, 1)[0] for b in range(3)])
    tok, codes = M.moshi_step(ctx, f0)
    for b in range(3):
        orc[b].step(f0[b], forced_text=int(tok[b]), forced_codes=codes[b])
    _check_prefill(shape, ctx, 1, orc[1], wl.frames(shape, 93, 1, 0, 40), stats, "slot 1")
    for t in range(3):
        f = np.stack([wl.frames(shape, 92, b, 1 + t, 1)[0] for b in range(3)])
        tok, codes = M.moshi_step(ctx, f)
        tl, al = M.moshi_read_logits(ctx)
        for b in range(3):
            r = orc[b].step(f[b], forced_text=int(tok[b]), forced_codes=codes[b])
            compare_frame(shape, stats, f"after prefill t={t} b={b}", int(tok[b]), codes[b], tl[b],
                          al[b], r)
            assert M.moshi_session_info(ctx, b) == orc[b].info()
    M.moshi_destroy(ctx)
    log(f"prefill with others live: {stats}")
