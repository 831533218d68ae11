"""GPU parity of the library's delayed-stream wrapper (moshi_stream_*, host
C++ over moshi_step_forced) against the oracle's own bookkeeping
(oracle/stream.py) over an oracle session.

A priming-like schedule (mobius PR #368, the persona/voice commit: voice
prompt, silence, persona text, silence, then the conversation): agent audio
forced from a synthetic "voice" code sequence, then a fixed "silence" code,
then forced text tokens, then silence, then free running; random user codes
throughout. The oracle wrapper runs its session teacher-forced on the GPU's
raw step tokens, so both sides feed back the same tokens: the frames the two
wrappers return must be identical, the logits within tolerance, and the
oracle's own argmax must equal the GPU's token wherever nothing was forced
and the margin is clear."""
import numpy as np
import pytest

import full_duplex_speech_amd as M
import oracle
from oracle.stream import DelayedStream
from synth import spec, workloads as wl
from gpu_util import Stats, compare_frame, log, new_engine

pytestmark = pytest.mark.gpu


def _schedule(shape, A, T, seed):
    """forced [T, 1 + A] (-1 = free) of a priming-like schedule."""
    g = np.random.default_rng(seed)
    f = np.full((T, 1 + A), -1, np.int32)
    voice = g.integers(0, shape.audio_card, (5, A))
    silence = g.integers(0, shape.audio_card, A)
    f[0:5, 1:] = voice                                   # voice prompt: agent audio
    f[5:7, 1:] = silence                                 # silence
    f[7:10, 0] = g.integers(0, shape.text_vocab, 3)      # persona text
    f[10:12, 1:] = silence                               # silence
    return f


@pytest.mark.parametrize("case", ["tiny_fp32_b1", "ragged_bf16_b2_dep8"])
def test_stream_wrapper_parity(case):
    if case == "tiny_fp32_b1":
        shape, B = spec.TINY.replace(window=16), 1
    else:
        shape, B = spec.RAGGED.replace(dep_q=8), 2
    A, S, T = 8, shape.n_substeps, 20
    weights = wl.make_weights(shape, 81, gains="random")
    ctx = new_engine(shape, weights, B)
    st = M.moshi_stream_create(ctx, A)
    om = oracle.Model(shape, weights)
    sess, wraps, gpu_raw = [], [], {}
    for b in range(B):
        assert M.moshi_session_join(ctx) == b
        M.moshi_stream_reset(st, b)
        o = oracle.Session(om)
        sess.append(o)

        def fn(frame, ft, fc, b=b, o=o):
            # teacher-forced on the GPU's raw tokens of this step
            tok, codes = gpu_raw[b]
            r = o.step(np.asarray(frame, np.int32), forced_text=int(tok),
                       forced_codes=np.asarray(codes, np.int32))
            gpu_raw[b] = (tok, codes, r)
            return tok, codes
        wraps.append(DelayedStream(fn, S, A, shape.text_vocab, shape.audio_card))
    sched = [_schedule(shape, A, T, 90 + b) for b in range(B)]
    users = [np.random.default_rng(95 + b).integers(0, shape.audio_card, (T, S - A)) for b in range(B)]
    stats = Stats()
    n = shape.dep_steps
    n_frames = 0
    for t in range(T):
        forced = np.stack([sched[b][t] for b in range(B)])
        fr, ready, tt, tc = M.moshi_stream_step(st, np.stack([users[b][t] for b in range(B)]), forced)
        tl, al = M.moshi_read_logits(ctx)
        for b in range(B):
            gpu_raw[b] = (int(tt[b]), tc[b].copy())
            out = wraps[b].step(users[b][t], forced[b])
            _, _, r = gpu_raw[b]
            # forced heads return the forced token; the rest are the model's
            if forced[b, 0] >= 0:
                assert tt[b] == forced[b, 0]
            for k in range(1, A + 1):
                if forced[b, k] >= 0:
                    assert tc[b, k - 1] == forced[b, k]
            ftok = int(tt[b]) if forced[b, 0] < 0 else r["text_token"]
            fcodes = tc[b][:n].copy()
            for k in range(1, A + 1):
                if forced[b, k] >= 0:
                    fcodes[k - 1] = r["codes"][k - 1]
            r2 = dict(r, audio_logits=r["audio_logits"][:n], codes=r["codes"][:n],
                      audio_margins=r["audio_margins"][:n])
            compare_frame(shape.replace(n_substeps=n), stats, f"{case} t={t} b={b}", ftok, fcodes,
                          tl[b], al[b][:n], r2)
            # the input frame the GPU wrapper fed equals the oracle wrapper's
            # (checked through the logits above) and the returned frame matches
            if out is None:
                assert ready[b] == 0 and (fr[b] == -1).all()
            else:
                assert ready[b] == 1 and list(fr[b]) == out, f"{case} t={t} b={b}: frame"
                n_frames += 1
    assert n_frames == B * (T - 1)
    # a slot that joins without a reset is refused
    if B > 1:
        M.moshi_session_leave(ctx, 1)
        assert M.moshi_session_join(ctx) == 1
        with pytest.raises(M.MoshiError) as e:
            M.moshi_stream_step(st, np.zeros((B, S - A), np.int32))
        assert e.value.status == M.MOSHI_E_INVALID
    M.moshi_stream_destroy(st)
    M.moshi_destroy(ctx)
    log(f"stream {case}: {n_frames} frames identical; {stats}")
