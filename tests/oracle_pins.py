"""Pin checks of the CPU oracle against things other than itself.

Each check returns None on success and raises AssertionError otherwise. They
are collected by ``test_oracle_pins.py`` and re-run against deliberately
broken copies of the oracle by ``test_oracle_mutations.py`` (which expects at
least one of them to fail for every planted mistake).

What pins what:
* bf16 rounding            -- torch's float64 -> bfloat16 conversion (library).
* RMSNorm                  -- closed form on constant vectors; scale invariance.
* RoPE                     -- identity at p = 0; complex rotation e^{i p theta_i}
                              (the standard rotary convention); relative-position
                              invariance of q.k.
* one attention head       -- torch's scaled_dot_product_attention (library);
                              single key gives v; equal keys give mean(v).
* SiLU / argmax            -- torch.nn.functional.silu; numpy argmax (first max);
                              constructed ties.
* embedding                -- one-hot tables (zero layers): hidden = norm(row).
* ring + window + positions-- full-history recompute with a window mask
                              (fullseq_ref.temporal_fullseq), W in {1,2,4,7,64},
                              T up to 3W, wrap-around, prefill + decode, and the
                              mask-oldest reading.
* depformer                -- all-substeps-at-once recompute with a causal mask
                              (fullseq_ref.depformer_fullseq), teacher-forced.
* sizes                    -- K/V bytes per frame printed on the pages.
"""
import numpy as np
import torch

import oracle
from synth import spec, workloads as wl, rng
import fullseq_ref as ref

TOL = 1e-10


def mini(dtype="f32", window=8, mask_oldest=False, n_layers=2):
    return spec.ModelShape(dim=64, n_layers=n_layers, n_heads=2, ffn=96, window=window,
                           dep_dim=32, dep_layers=2, dep_heads=2, dep_ffn=48, n_substeps=16,
                           text_vocab=50, audio_card=40, dtype=dtype, mask_oldest=mask_oldest)


def _model(shape, seed=7, std=0.25):
    w = wl.make_weights(shape, seed, gains="random", std=std)
    return w, oracle.Model(shape, w)


# ------------------------------------------------------------ primitives

def check_bf16_round():
    g = np.random.default_rng(1)
    x = np.concatenate([g.normal(0, 1, 2000), g.normal(0, 1e-3, 500), g.normal(0, 50, 500),
                        [0.0, 1.0, -1.0, 1.00390625, 1.01171875, 1.005859375, 3.0e-39, -2.5]])
    want = torch.tensor(x, dtype=torch.float64).to(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_round(v) for v in x])
    assert np.array_equal(got, want), "bf16 rounding differs from torch"


def check_rmsnorm():
    eps = 1e-8
    for c in (0.5, -3.0, 1e-3):
        g = np.linspace(0.5, 2.0, 16)
        got = oracle.rmsnorm(np.full(16, c), g, eps)
        want = np.sign(c) * g * abs(c) / np.sqrt(c * c + eps)
        assert np.allclose(got, want, rtol=1e-13, atol=0), "rmsnorm closed form"
    x = np.random.default_rng(2).normal(size=33)
    g = np.random.default_rng(3).normal(size=33)
    a = oracle.rmsnorm(x, g, 0.0)
    b = oracle.rmsnorm(7.5 * x, g, 0.0)
    assert np.allclose(a, b, rtol=1e-12), "rmsnorm scale invariance"


def check_rope():
    hd, H = 16, 3
    v = np.random.default_rng(4).normal(size=H * hd)
    assert np.array_equal(oracle.rope(v, H, hd, 0), v), "rope at p=0 must be the identity"
    for p in (1, 5, 123, 3000):
        got = oracle.rope(v, H, hd, p).reshape(H, hd // 2, 2)
        z = v.reshape(H, hd // 2, 2)
        zc = (z[..., 0] + 1j * z[..., 1]) * np.exp(1j * p * 1e4 ** (-2.0 * np.arange(hd // 2) / hd))
        assert np.allclose(got[..., 0], zc.real, atol=1e-12) and \
            np.allclose(got[..., 1], zc.imag, atol=1e-12), "rope != complex rotation"
    q = np.random.default_rng(5).normal(size=hd)
    k = np.random.default_rng(6).normal(size=hd)
    base = oracle.rope(q, 1, hd, 10) @ oracle.rope(k, 1, hd, 3)
    for d in (1, 17, 400):
        sh = oracle.rope(q, 1, hd, 10 + d) @ oracle.rope(k, 1, hd, 3 + d)
        assert abs(sh - base) < 1e-10, "rope relative-position invariance"


def check_attend():
    g = np.random.default_rng(8)
    hd = 24
    for n in (1, 2, 9, 40):
        q = g.normal(size=hd)
        K = g.normal(size=(n, hd))
        V = g.normal(size=(n, hd))
        got = oracle.attend(q, K, V)
        want = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(q)[None, None, None, :], torch.tensor(K)[None, None],
            torch.tensor(V)[None, None]).numpy().reshape(-1)
        assert np.allclose(got, want, atol=1e-12), "attention != torch sdpa"
    V = g.normal(size=(1, hd))
    assert np.allclose(oracle.attend(g.normal(size=hd), g.normal(size=(1, hd)), V), V[0]), \
        "single key must return its value"
    K = np.tile(g.normal(size=(1, hd)), (6, 1))
    V = g.normal(size=(6, hd))
    assert np.allclose(oracle.attend(g.normal(size=hd), K, V), V.mean(0), atol=1e-13), \
        "equal keys must average the values"


def check_silu_argmax():
    z = np.linspace(-30, 30, 121)
    got = np.array([oracle.silu(v) for v in z])
    want = torch.nn.functional.silu(torch.tensor(z)).numpy()
    assert np.allclose(got, want, rtol=1e-14, atol=1e-300) and oracle.silu(0.0) == 0.0
    v = np.random.default_rng(9).normal(size=1000)
    i, m = oracle.argmax(v)
    srt = np.sort(v)
    assert i == int(np.argmax(v)) and abs(m - (srt[-1] - srt[-2])) < 1e-15
    t = np.zeros(10)
    t[[3, 7]] = 2.0
    assert oracle.argmax(t) == (3, 0.0), "ties go to the lowest index"


# ------------------------------------------------------------ model pins

def check_embedding_onehot():
    s = mini(n_layers=0)
    w = [np.zeros_like(a) if nm.startswith("emb.") else a
         for a, (nm, _, _) in zip(wl.make_weights(s, 11, gains="random", std=0.25),
                                  spec.tensor_list(s))]
    names = [t[0] for t in spec.tensor_list(s)]
    row = np.random.default_rng(12).normal(size=s.dim).astype(np.float32)
    frame = np.array([4] + [1] * s.n_substeps, np.int32)
    w[names.index("emb.audio.5")].reshape(s.audio_card + 1, s.dim)[1] = row
    M = oracle.Model(s, w)
    out = oracle.Session(M).temporal(frame)
    g = w[names.index("out_norm")].astype(np.float64)
    want = oracle.rmsnorm(row.astype(np.float64), g, s.norm_eps)
    assert np.allclose(out["hidden"], want, atol=1e-12), "one-hot embedding"
    # linearity: a second channel adds its own row
    row2 = np.random.default_rng(13).normal(size=s.dim).astype(np.float32)
    w[names.index("emb.text")].reshape(s.text_vocab + 1, s.dim)[4] = row2
    M = oracle.Model(s, w)
    out = oracle.Session(M).temporal(frame)
    want = oracle.rmsnorm(row.astype(np.float64) + row2, g, s.norm_eps)
    assert np.allclose(out["hidden"], want, atol=1e-12), "embedding sum"


def _ring_case(shape, T, n_prefill, seed=21):
    w, M = _model(shape, seed)
    W64 = ref.Weights(shape, w)
    fr = wl.frames(shape, 99, 0, 0, T)
    sess = oracle.Session(M)
    pre = None
    if n_prefill:
        k, v = wl.prefill_kv(shape, 98, 0, n_prefill)
        sess.prefill(k, v)
        pre = (ref.to_f64(k, shape.dtype), ref.to_f64(v, shape.dtype))
    hid_ref, log_ref = ref.temporal_fullseq(W64, fr, pre)
    for t in range(T):
        o = sess.temporal(fr[t])
        assert np.max(np.abs(o["hidden"] - hid_ref[t])) < TOL, \
            f"hidden mismatch at t={t} (W={shape.window}, prefill={n_prefill})"
        assert np.max(np.abs(o["text_logits"] - log_ref[t])) < TOL, f"logits mismatch t={t}"
        assert o["text_token"] == int(np.argmax(log_ref[t]))
        pos, fill, wi = sess.info()
        assert pos == n_prefill + t + 1 and wi == pos % shape.window
        assert fill == min(pos, shape.window)


def check_ring_window_fp32():
    for W in (1, 2, 4, 7):
        _ring_case(mini("f32", window=W), T=3 * W + 2, n_prefill=0)
    _ring_case(mini("f32", window=7), T=12, n_prefill=5)
    _ring_case(mini("f32", window=7), T=9, n_prefill=7)


def check_ring_window_mask_oldest():
    for W in (2, 5):
        _ring_case(mini("f32", window=W, mask_oldest=True), T=3 * W, n_prefill=0)
    _ring_case(mini("f32", window=6, mask_oldest=True), T=8, n_prefill=6)


def check_incremental_equals_fullseq_bf16():
    _ring_case(mini("bf16", window=64), T=20, n_prefill=0)
    _ring_case(mini("bf16", window=4), T=11, n_prefill=3)


def check_depformer_fullseq():
    for dt in ("f32", "bf16"):
        s = mini(dt)
        w, M = _model(s, 31)
        W64 = ref.Weights(s, w)
        g = np.random.default_rng(32)
        hid = g.normal(size=s.dim)
        if dt == "bf16":
            hid = ref.bf_round(hid)
        text_in = 17
        out = M.depformer(hid, text_in)
        want = ref.depformer_fullseq(W64, hid, text_in, out["codes"])
        assert np.max(np.abs(out["audio_logits"] - want)) < TOL, f"depformer ({dt})"
        forced = g.integers(0, s.audio_card, size=s.n_substeps).astype(np.int32)
        out = M.depformer(hid, text_in, forced=forced)
        want = ref.depformer_fullseq(W64, hid, text_in, forced)
        assert np.max(np.abs(out["audio_logits"] - want)) < TOL, f"forced depformer ({dt})"
        assert np.array_equal(out["codes"], np.argmax(want, axis=1))


def check_step_composition():
    """orc_step = temporal then depformer on the temporal hidden and token."""
    s = mini("bf16", window=5)
    w, M = _model(s, 41)
    fr = wl.frames(s, 42, 0, 0, 3)
    a, b = oracle.Session(M), oracle.Session(M)
    for t in range(3):
        full = a.step(fr[t])
        tp = b.temporal(fr[t])
        dp = M.depformer(tp["hidden"], tp["text_token"])
        assert full["text_token"] == tp["text_token"]
        assert np.array_equal(full["codes"], dp["codes"])
        assert np.array_equal(full["audio_logits"], dp["audio_logits"])
        # teacher forcing with the oracle's own choices changes nothing
        c = oracle.Session(M)
        for u in range(t):
            c.temporal(fr[u])
        forced = c.step(fr[t], forced_text=full["text_token"], forced_codes=full["codes"])
        assert np.array_equal(forced["audio_logits"], full["audio_logits"])


def check_sizes():
    """K/V per frame and per 3.1k positions, as printed on the pages."""
    import json, os
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_sizes.json")))
    m = spec.PERSONAPLEX
    assert spec.kv_bytes_per_frame(m) == gold["kv_bytes_per_frame_bf16"]["value"]
    gib = 3100 * spec.kv_bytes_per_frame(m) / 2 ** 30
    assert abs(gib - gold["kv_gib_at_3100_positions"]["value"]) < 0.05
    assert m.window * gold["frame_ms"]["value"] / 1000 / 60 == gold["window_minutes"]["value"]


def check_ring_transfer():
    """read_ring -> load_ring into a fresh session continues bit-identically
    (the state transfer the full-size GPU checks rely on): after T frames that
    wrap the ring, and after a prefill. The bf16 ring is stored as bf16, so the
    transfer is lossless; the fp32 model's oracle ring holds fp64 values and
    the transfer rounds them to fp32, so there it is checked to 1e-6 relative."""
    for dt, W, T, pre in (("f32", 5, 12, 0), ("bf16", 7, 4, 6), ("bf16", 4, 9, 3),
                          ("bf16", 5, 13, 0)):
        s = mini(dt, window=W)
        w, M = _model(s, 51)
        fr = wl.frames(s, 52, 0, 0, T + 2)
        a = oracle.Session(M)
        if pre:
            k, v = wl.prefill_kv(s, 53, 0, pre)
            a.prefill(k, v)
        for t in range(T):
            a.step(fr[t])
        rk, rv = a.read_ring()
        b = oracle.Session(M)
        b.load_ring(a.info()[0], rk, rv)
        assert b.info() == a.info(), "ring transfer: bookkeeping"
        for t in range(T, T + 2):
            x = a.step(fr[t])
            y = b.step(fr[t], forced_text=x["text_token"], forced_codes=x["codes"])
            for key in ("text_logits", "audio_logits", "hidden"):
                if dt == "bf16":
                    ok = np.array_equal(x[key], y[key])
                else:
                    ok = np.max(np.abs(x[key] - y[key])) < 1e-6 * max(1.0, np.max(np.abs(x[key])))
                assert ok, f"ring transfer: {key} differs ({dt}, W={W})"
        # both sessions wrote the same rows since (bf16: lossless transfer)
        if dt == "bf16":
            k2, v2 = b.read_ring()
            k1, v1 = a.read_ring()
            assert np.array_equal(k2, k1) and np.array_equal(v2, v1), "ring transfer: rows"


def check_depformer_variants():
    """dep_q, the ring reading and the final-norm reading, each against the
    full-sequence form and an invariant of its own."""
    base = mini("f32")
    g = np.random.default_rng(61)
    hid = g.normal(size=base.dim)
    forced = g.integers(0, base.audio_card, size=base.n_substeps).astype(np.int32)
    w0, M0 = _model(base, 62)
    full = M0.depformer(hid, 9, forced=forced)
    for shape in (base.replace(dep_q=8), base.replace(dep_ref_ring=True),
                  base.replace(dep_q=8, dep_ref_ring=True), base.replace(dep_q=2, dep_ref_ring=True),
                  base.replace(dep_final_norm=True), base.replace(dep_q=5, dep_final_norm=True),
                  mini("bf16").replace(dep_q=8, dep_ref_ring=True, dep_final_norm=True)):
        w, M = _model(shape, 62)
        n = shape.dep_steps
        out = M.depformer(hid if shape.dtype == "f32" else ref.bf_round(hid), 9, forced=forced)
        want = ref.depformer_fullseq(ref.Weights(shape, w),
                                     hid if shape.dtype == "f32" else ref.bf_round(hid), 9, forced)
        assert np.max(np.abs(out["audio_logits"][:n] - want)) < TOL, f"variant {shape}"
        assert (out["codes"][n:] == -1).all() and np.isinf(out["audio_margins"][n:]).all(), \
            "substeps past dep_q must not run"
        assert np.array_equal(out["codes"][:n], np.argmax(want, axis=1))
    # dep_q: the substeps that run are those of the full depformer (a prefix)
    w, M = _model(base.replace(dep_q=5), 62)
    part = M.depformer(hid, 9, forced=forced)
    assert np.array_equal(part["audio_logits"][:5], full["audio_logits"][:5]), "dep_q prefix"
    # ring reading with 2 substeps: substep 1 attends itself only, so substep
    # 0's attention weights cannot reach it; without the reading they do
    for ring in (True, False):
        shp = base.replace(dep_q=2, dep_ref_ring=ring)
        w, M = _model(shp, 63)
        a = M.depformer(hid, 9, forced=forced)["audio_logits"][1]
        names = [t[0] for t in spec.tensor_list(shp)]
        w2 = [x.copy() for x in w]
        w2[names.index("dep.0.layer.0.qkv")] *= 3.0
        b = oracle.Model(shp, w2).depformer(hid, 9, forced=forced)["audio_logits"][1]
        assert np.array_equal(a, b) == ring, f"ring reading (on={ring}): substep 1 and entry 0"
    # final norm: doubling its gain doubles every head's logits exactly
    shp = mini("bf16").replace(dep_final_norm=True)
    w, M = _model(shp, 64)
    names = [t[0] for t in spec.tensor_list(shp)]
    h16 = ref.bf_round(hid)
    a = M.depformer(h16, 9, forced=forced)
    w2 = [x.copy() for x in w]
    gi = names.index("dep.out_norm")
    w2[gi] = rng.f32_to_bf16(rng.bf16_to_f32(w2[gi]) * 2.0)
    b = oracle.Model(shp, w2).depformer(h16, 9, forced=forced)
    assert np.array_equal(b["audio_logits"], 2.0 * a["audio_logits"]), "final norm gain"


def check_splitmix64_published():
    """The counter generator behind the sampling draws is splitmix64: its
    published first outputs for seed 0 (tests/golden/splitmix64_seed0.json)."""
    import json, os
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "splitmix64_seed0.json")))
    got = [oracle.splitmix64(0, n) for n in range(1, 5)]
    assert got == [int(h, 16) for h in gold["outputs_hex"]], "splitmix64 outputs"


def check_uniform_draws():
    """Draws lie in [0, 1), look uniform (mean, variance, a 10-bin histogram
    over 20000 positions), and the streams of one seed and the same stream
    of two seeds differ."""
    u = np.array([oracle.uniform(7, 0, p) for p in range(20000)])
    assert u.min() >= 0.0 and u.max() < 1.0
    assert abs(u.mean() - 0.5) < 0.01 and abs(u.var() - 1 / 12) < 0.005
    h = np.histogram(u, bins=10, range=(0, 1))[0]
    assert np.all(np.abs(h - 2000) < 200), "uniform histogram"
    a = [oracle.uniform(7, 1, p) for p in range(50)]
    b = [oracle.uniform(7, 2, p) for p in range(50)]
    c = [oracle.uniform(8, 1, p) for p in range(50)]
    assert len(set(a) & set(b)) == 0 and len(set(a) & set(c)) == 0
    assert oracle.uniform(7, 1, 3) == oracle.uniform(7, 1, 3)


def check_sampling():
    """Temperature + top-k draws against numpy: on a grid of u the number of
    grid points that choose each token is N * p within one, p the softmax of
    logits / T over the top k (ties at the boundary to the lower index);
    top-k 1 is the argmax; doubling the logits and the temperature changes
    nothing; the draw is decided on the fp32 values."""
    g = np.random.default_rng(71)
    N = 4000
    for n, T, k in ((37, 0.7, 5), (300, 0.8, 250), (60, 1.3, -1), (50, 0.5, 50)):
        lg = g.normal(0, 1.5, n)
        l32 = lg.astype(np.float32).astype(np.float64)
        order = sorted(range(n), key=lambda i: (-l32[i], i))
        kk = n if (k <= 0 or k >= n) else k
        members = np.zeros(n, bool)
        members[order[:kk]] = True
        w = np.where(members, np.exp((l32 - l32.max()) / T), 0.0)
        p = w / w.sum()
        counts = np.zeros(n)
        for j in range(N):
            i, _ = oracle.sample(lg, T, k, (j + 0.5) / N)
            counts[i] += 1
        assert np.all(np.abs(counts - N * p) <= 1.0 + 1e-9), f"sampling distribution n={n} k={k}"
        assert counts[~members].sum() == 0, "a token outside the top k was drawn"
        for u in (0.0, 0.3, 0.999):
            a = oracle.sample(lg, T, k, u)
            b = oracle.sample(2.0 * lg, 2.0 * T, k, u)
            assert a == b, "temperature must divide the logit differences"
        i1, _ = oracle.sample(lg, T, 1, 0.77)
        assert i1 == order[0], "top-k 1 is the argmax"
    # ties at the top-k boundary: the lower indices are the candidates
    lg = np.array([1.0, 3.0, 3.0, 3.0, 0.0])
    picks = {oracle.sample(lg, 1.0, 2, u)[0] for u in np.linspace(0.01, 0.99, 30)}
    assert picks == {1, 2}, f"boundary ties: {picks}"
    # decided on fp32: logits that round to the same fp32 values draw the same
    lg = g.normal(0, 1, 40)
    l2 = lg.astype(np.float32).astype(np.float64) + 1e-12 * g.normal(size=40)
    assert all(oracle.sample(lg, 0.9, 7, u)[0] == oracle.sample(l2, 0.9, 7, u)[0]
               for u in np.linspace(0.05, 0.95, 19))
    # ... where fp32 rounding matters: 1e8 + 3 and 1e8 + 2 round to 1e8
    # (fp32 spacing 8 there), so the three tokens weigh the same and u = 0.34
    # draws token 1; in fp64 their weights e^{3/4}, e^{2/4}, 1 would draw token 0
    lg = np.array([1e8 + 3, 1e8 + 2, 1e8])
    assert oracle.sample(lg, 4.0, -1, 0.34)[0] == 1, "decided on the fp32 values"
    assert oracle.sample(lg, 4.0, -1, 0.30)[0] == 0 and oracle.sample(lg, 4.0, -1, 0.7)[0] == 2


ALL = [check_bf16_round, check_rmsnorm, check_rope, check_attend, check_silu_argmax,
       check_embedding_onehot, check_ring_window_fp32, check_ring_window_mask_oldest,
       check_incremental_equals_fullseq_bf16, check_depformer_fullseq, check_step_composition,
       check_sizes, check_ring_transfer, check_depformer_variants, check_splitmix64_published,
       check_uniform_draws, check_sampling]
