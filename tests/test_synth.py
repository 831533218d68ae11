"""The seeded input generators: determinism, slicing, ranges and moments."""
import numpy as np

from synth import rng, spec, workloads as wl


def test_normal_deterministic_and_sliceable():
    a = rng.normal(5, 3, 10000, 1.0, dtype="f64")
    b = rng.normal(5, 3, 10000, 1.0, dtype="f64")
    assert np.array_equal(a, b)
    c = rng.normal(5, 3, 500, 1.0, offset=1234, dtype="f64")
    assert np.array_equal(a[1234:1734], c)
    d = rng.normal(5, 4, 10000, 1.0, dtype="f64")
    assert not np.allclose(a, d)


def test_normal_threads_match_single_thread():
    a = rng.normal(9, 1, 400001, 0.02, dtype="bf16", threads=1)
    b = rng.normal(9, 1, 400001, 0.02, dtype="bf16", threads=7)
    assert np.array_equal(a, b)
    f = rng.normal(9, 1, 400001, 0.02, dtype="f32", threads=5)
    assert np.array_equal(rng.f32_to_bf16(f), a)


def test_normal_moments():
    x = rng.normal(11, 0, 1 << 20, 2.0, dtype="f64")
    assert abs(x.mean()) < 0.01 and abs(x.std() - 2.0) < 0.01
    # fraction beyond 2 sigma of a normal: 4.55%
    assert abs(np.mean(np.abs(x) > 4.0) - 0.0455) < 0.002


def test_uniform_int_ranges():
    m = spec.PERSONAPLEX
    f = wl.frames(m, 2021, 3, 0, 4000)
    assert f.shape == (4000, 17)
    assert f[:, 0].min() >= 0 and f[:, 0].max() < m.text_vocab
    assert f[:, 1:].min() >= 0 and f[:, 1:].max() < m.audio_card
    assert abs(f[:, 1:].mean() - (m.audio_card - 1) / 2) < 10
    g = wl.frames(m, 2021, 3, 100, 10)
    assert np.array_equal(f[100:110], g)


def test_bf16_helpers_roundtrip():
    x = np.array([1.0, -2.5, 1.00390625, 1.01171875, 3.14159], np.float32)
    b = rng.f32_to_bf16(x)
    y = rng.bf16_to_f32(b)
    assert y[0] == 1.0 and y[1] == -2.5 and y[2] == 1.0 and y[3] == 1.015625
    assert abs(y[4] - 3.140625) < 1e-7


def test_prefill_independent_of_fill():
    m = spec.RAGGED
    k1, v1 = wl.prefill_kv(m, 7, 2, 10)
    k2, v2 = wl.prefill_kv(m, 7, 2, 20)
    assert np.array_equal(k1, k2[:, :10]) and np.array_equal(v1, v2[:, :10])
    assert not np.array_equal(k1, v1)


def test_churn_schedule_shape():
    w = wl.WORKLOADS[4]
    initial, events = wl.churn_schedule(w)
    assert len(initial) == 16 and all(0 <= f <= 3000 for _, f in initial)
    assert sorted(events) == list(range(50, 500, 50))
    live = {sid for sid, _ in initial}
    for t in sorted(events):
        for a in events[t]:
            if a[0] == "leave":
                live.remove(a[1])
            else:
                assert a[1] not in live
                live.add(a[1])
        assert len(live) == 16


def test_tensor_list_counts():
    for m in (spec.TINY, spec.PERSONAPLEX, spec.RAGGED):
        S, L, Ld = m.n_substeps, m.n_layers, m.dep_layers
        assert spec.n_tensors(m) == 1 + S + 6 * L + 2 + S + S + 2 * Ld + 4 * S * Ld + S
    # full-size weight bytes: temporal + depformer matrices (bf16)
    assert spec.weight_bytes(spec.PERSONAPLEX) > 16e9
