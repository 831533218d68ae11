"""CPU pins of the oracle's delayed-stream bookkeeping (oracle/stream.py),
each against something other than the class itself: the frame count, the
un-delaying of the outputs (a fake model that generates a known acoustic
sequence), the placement of user codes and initial tokens in the input
columns (written out from the definition), and forcing (with the model's own
choices it changes nothing; forced tokens come out in the right frames)."""
import numpy as np
import pytest

import oracle
from oracle.stream import DelayedStream, default_delays, oracle_step_fn
from synth import spec, workloads as wl

S, A, VT, CARD = 16, 8, 50, 40


def _fake(seed=0):
    """A deterministic fake model: tokens from a hash of the input frame."""
    def fn(frame, ft, fc):
        h = hash((tuple(frame), seed))
        text = h % VT
        codes = np.array([(h >> (3 * i)) % CARD for i in range(S)], np.int32)
        return text, codes
    return fn


def test_default_delays_are_the_pages():
    assert default_delays(16, 8) == [0, 0, 1, 1, 1, 1, 1, 1, 1, 0, 1, 1, 1, 1, 1, 1, 1]


@pytest.mark.parametrize("delays", [None, [0] * 17, [0, 0, 2, 1, 1, 1, 1, 1, 1, 0, 1, 2, 1, 1, 1, 1, 1]])
def test_frame_count(delays):
    """n steps return n - max(d) frames (5 -> 4 with the pages' delays)."""
    st = DelayedStream(_fake(), S, A, VT, CARD, delays)
    g = np.random.default_rng(1)
    out = [st.step(g.integers(0, CARD, S - A)) for _ in range(5)]
    D = max(default_delays(S, A) if delays is None else delays)
    assert sum(o is not None for o in out) == 5 - D
    assert all(o is None for o in out[:D])


@pytest.mark.parametrize("delays", [None, [0, 0, 2, 1, 1, 1, 1, 1, 1, 0, 1, 2, 1, 1, 1, 1, 1]])
def test_outputs_are_undelayed(delays):
    """A fake model that, at step t, generates for channel k the token of a
    known acoustic sequence at frame t + 1 - d_k: the returned frame tau is
    exactly that sequence's frame tau."""
    d = default_delays(S, A) if delays is None else delays
    g = np.random.default_rng(2)
    T = 12
    seq = g.integers(0, CARD, (T + 3, A + 1))
    seq[:, 0] = g.integers(0, VT, T + 3)
    t_box = [0]

    def fn(frame, ft, fc):
        t = t_box[0]
        t_box[0] += 1
        codes = np.zeros(S, np.int32)
        for k in range(1, A + 1):
            codes[k - 1] = seq[t + 1 - d[k], k] if t + 1 - d[k] >= 0 else 0
        return int(seq[t + 1, 0]), codes

    st = DelayedStream(fn, S, A, VT, CARD, d)
    D = max(d)
    for t in range(T):
        out = st.step(g.integers(0, CARD, S - A))
        tau = t + 1 - D
        if tau >= 1:
            assert out == [int(seq[tau, k]) for k in range(A + 1)], f"frame {tau}"


def test_input_columns_by_definition():
    """Input frame t, channel by channel: user channel k gets the user's
    frame t - d_k (initial before that); a generated channel gets what step
    t - 1 generated for it (initial at t = 0 and while t < d_k)."""
    d = default_delays(S, A)
    g = np.random.default_rng(3)
    T = 6
    users = g.integers(0, CARD, (T, S - A))
    st = DelayedStream(_fake(4), S, A, VT, CARD)
    gen = []  # (text, codes) generated at each step
    orig = st.step_fn

    def rec(frame, ft, fc):
        r = orig(frame, ft, fc)
        gen.append(r)
        return r
    st.step_fn = rec
    for t in range(T):
        st.step(users[t])
    for t, frame in enumerate(st.inputs):
        assert frame[0] == (VT if t == 0 else gen[t - 1][0])
        for k in range(1, A + 1):
            want = CARD if (t == 0 or t < d[k]) else int(gen[t - 1][1][k - 1])
            assert frame[k] == want, (t, k)
        for k in range(A + 1, S + 1):
            want = CARD if t < d[k] else int(users[t - d[k]][k - A - 1])
            assert frame[k] == want, (t, k)


def _tiny_session():
    shape = spec.TINY.replace(window=8)
    w = wl.make_weights(shape, 5, gains="random", std=0.25)
    return shape, oracle.Model(shape, w)


def test_forcing_own_choices_is_a_noop():
    shape, om = _tiny_session()
    g = np.random.default_rng(6)
    users = g.integers(0, shape.audio_card, (7, 8))
    free = DelayedStream(oracle_step_fn(oracle.Session(om)), 16, 8, shape.text_vocab,
                         shape.audio_card)
    outs_free = [free.step(u) for u in users]
    forced = DelayedStream(oracle_step_fn(oracle.Session(om)), 16, 8, shape.text_vocab,
                           shape.audio_card)
    outs_forced = []
    for t, u in enumerate(users):
        f = [free.cols[0][t + 1]] + [free.cols[k][t + 1] for k in range(1, 9)]
        outs_forced.append(forced.step(u, f))
    assert outs_free == outs_forced
    assert free.inputs == forced.inputs


def test_forced_tokens_come_out_in_their_frames():
    """A token forced at step t for column t+1 of channel k is channel k of
    acoustic frame t + 1 - d_k."""
    d = default_delays(S, A)
    st = DelayedStream(_fake(7), S, A, VT, CARD)
    g = np.random.default_rng(8)
    T = 8
    forced = np.full((T, A + 1), -1)
    forced[3, 0] = 11        # text of frame 4
    forced[3, 1] = 12        # agent codebook 1 (delay 0): frame 4
    forced[3, 2] = 13        # agent codebook 2 (delay 1): frame 3
    outs = {}
    for t in range(T):
        o = st.step(g.integers(0, CARD, S - A), forced[t])
        if o is not None:
            outs[t + 1 - max(d)] = o
    assert outs[4][0] == 11 and outs[4][1] == 12 and outs[3][2] == 13
