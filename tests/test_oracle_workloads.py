"""The oracle on the small named workloads (CPU only)."""
import numpy as np

import oracle
from synth import spec, workloads as wl


def test_tiny_workload_runs_and_wraps():
    w = wl.WORKLOADS[1]
    m = w.shape()
    W = wl.make_weights(m, wl.MODEL_SEEDS["tiny"])
    M = oracle.Model(m, W)
    s = oracle.Session(M)
    fr = wl.frames(m, w.seed("frames"), 0, 0, w.frames)
    toks = []
    for t in range(w.frames):
        o = s.step(fr[t])
        toks.append(o["text_token"])
        assert 0 <= o["text_token"] < m.text_vocab
        assert o["codes"].min() >= 0 and o["codes"].max() < m.audio_card
        assert np.isfinite(o["text_logits"]).all() and np.isfinite(o["audio_logits"]).all()
    pos, fill, wi = s.info()
    assert (pos, fill, wi) == (100, 64, 100 % 64)
    assert len(set(toks)) > 10


def test_oracle_rejects_bad_codes():
    m = spec.RAGGED
    M = oracle.Model(m, wl.make_weights(m, 3))
    s = oracle.Session(M)
    bad = np.zeros(17, np.int32)
    bad[5] = m.audio_card + 1
    try:
        s.step(bad)
        raise AssertionError("expected rejection")
    except ValueError:
        pass
    assert s.info()[0] == 0
    ok = np.zeros(17, np.int32)
    ok[0] = m.text_vocab          # the "initial token" row is a valid code
    ok[1:] = m.audio_card
    s.step(ok)
    assert s.info()[0] == 1
