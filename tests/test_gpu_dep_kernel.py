"""The persistent multi-session depformer kernel (capacity 2..64) against the
per-operation kernels (MOSHI_DEP_MULTI=0): every output a step returns is
bit-identical, at capacities whose projection tiles take 8 waves (B <= 32)
and 4 (B > 32), from the smallest capacity (2) to the first with 4 waves
(33) and beyond, with free slots, teacher forcing, the depformer readings
(dep_q, the ring reading, the final norm) and a down projection split over
K into segments; a few session-frames are also
checked against the oracle; and its bounded-wait failure path (forced from
the host by a tiny spin limit: every workgroup exits)."""
import os

import numpy as np
import pytest

import full_duplex_speech_amd as M
import oracle
from synth import spec, workloads as wl
from gpu_util import Stats, compare_frame, frames_matrix, log, new_engine

pytestmark = pytest.mark.gpu


def _engine(shape, weights, B, multi):
    old = os.environ.get("MOSHI_DEP_MULTI")
    os.environ["MOSHI_DEP_MULTI"] = "1" if multi else "0"
    try:
        ctx = new_engine(shape, weights, B)
    finally:
        if old is None:
            os.environ.pop("MOSHI_DEP_MULTI", None)
        else:
            os.environ["MOSHI_DEP_MULTI"] = old
    assert M.moshi_uses_dep_kernel(ctx) == multi
    return ctx


def _forced(shape, B, t, live, seed):
    g = np.random.default_rng(seed * 7919 + t)
    f = np.full((B, shape.n_channels), -1, np.int32)
    for b in live:
        if g.random() < 0.3:
            f[b, 0] = g.integers(0, shape.text_vocab)
        for s in range(shape.n_substeps):
            if g.random() < 0.2:
                f[b, 1 + s] = g.integers(0, shape.audio_card)
    return f


def _run(shape, weights, B, free, T, seed, multi, force, check_oracle=()):
    """B slots joined, prefilled to varied fills, the slots in `free` left;
    T ticks (forced when `force`); per tick the tokens, codes and logits.
    Slots in check_oracle are compared with the teacher-forced oracle."""
    ctx = _engine(shape, weights, B, multi)
    om = oracle.Model(shape, weights) if check_oracle else None
    orc = {}
    for b in range(B):
        assert M.moshi_session_join(ctx) == b
        n = (b * 7) % (shape.window + 1)
        if n:
            k, v = wl.prefill_kv(shape, seed + 1, b, n)
            M.moshi_session_prefill_kv(ctx, b, k, v)
            if b in check_oracle:
                orc[b] = oracle.Session(om)
                orc[b].prefill(k, v)
        elif b in check_oracle:
            orc[b] = oracle.Session(om)
    for b in free:
        M.moshi_session_leave(ctx, b)
    live = [b for b in range(B) if b not in free]
    stats, outs = Stats(), []
    for t in range(T):
        fr = frames_matrix(shape, B, {b: wl.frames(shape, seed, b, t, 1)[0] for b in live})
        fc = _forced(shape, B, t, live, seed) if force else None
        if force:
            tok, codes = M.moshi_step_forced(ctx, fr, fc)
        else:
            tok, codes = M.moshi_step(ctx, fr)
        tl, al = M.moshi_read_logits(ctx)
        n = shape.dep_steps
        # logits of free slots and of substeps not run are never written
        outs.append((tok.copy(), codes.copy(), tl[live].copy(), al[live][:, :n].copy()))
        for b, o in orc.items():
            r = o.step(fr[b], forced_text=int(tok[b]), forced_codes=codes[b])
            r2 = dict(r)
            r2["audio_logits"] = r["audio_logits"][:n]
            r2["codes"] = r["codes"][:n]
            r2["audio_margins"] = r["audio_margins"][:n]
            # where a token was forced the oracle's own choice stands in (the
            # oracle was fed the forced token; its argmax is not compared)
            ftok = int(tok[b]) if fc is None or fc[b, 0] < 0 else r["text_token"]
            fcodes = codes[b].copy()
            if fc is not None:
                for s in range(n):
                    if fc[b, 1 + s] >= 0:
                        fcodes[s] = r["codes"][s]
            compare_frame(shape.replace(n_substeps=n), stats, f"t={t} b={b}",
                          ftok, fcodes[:n], tl[b], al[b][:n], r2)
    M.moshi_destroy(ctx)
    return outs, stats


def _assert_same(a, b, tag):
    assert len(a) == len(b)
    for t, (x, y) in enumerate(zip(a, b)):
        for name, u, v in zip(("text", "codes", "text logits", "audio logits"), x, y):
            assert np.array_equal(u, v), f"{tag}: {name} differ at t={t}"


CASES = {
    # (shape, capacity, free slots, ticks, forcing, oracle-checked slots)
    "tiny_fp32_b2": (spec.TINY.replace(window=9), 2, [], 4, True, [1]),  # the smallest capacity
    "tiny_fp32_b3": (spec.TINY.replace(window=9), 3, [1], 6, True, [0]),
    "ragged_bf16_b5_variants": (spec.RAGGED.replace(dep_q=8, dep_ref_ring=True,
                                                    dep_final_norm=True), 5, [3], 4, True, [4]),
    "ragged_bf16_b17": (spec.RAGGED, 17, [0, 16], 3, False, [5]),
    "ragged_bf16_b33": (spec.RAGGED, 33, [32], 2, False, [31]),  # the first with 4 waves per tile
    "ragged_bf16_b40": (spec.RAGGED, 40, [2, 33, 39], 3, True, [1]),
    "ragged_bf16_b36_variants": (spec.RAGGED.replace(dep_q=8, dep_ref_ring=True,
                                                     dep_final_norm=True), 36, [0, 20], 2, True,
                                 [35]),
    # a down projection long enough to be split over K (4 segments up to 32
    # sessions), its K (2104) not a multiple of the 32-element k-step
    "ksplit_bf16_b5": (spec.RAGGED.replace(dep_ffn=2104), 5, [1], 3, True, [0]),
    "ksplit_bf16_b17": (spec.RAGGED.replace(dep_ffn=2104), 17, [3, 16], 2, False, [2]),
}


@pytest.mark.parametrize("case", list(CASES))
def test_dep_kernel_matches_per_op(case):
    shape, B, free, T, force, chk = CASES[case]
    weights = wl.make_weights(shape, 83, gains="random")
    log(f"dep kernel {case}: B={B} free={free} T={T}")
    a, sa = _run(shape, weights, B, free, T, 11, True, force, check_oracle=chk)
    b, _ = _run(shape, weights, B, free, T, 11, False, force)
    _assert_same(a, b, case)
    log(f"dep kernel {case}: bit-identical to per-op; oracle {sa}")


def test_dep_kernel_not_used_with_sampling():
    shape = spec.TINY
    cfg = M.make_config(**{**_cfg_kwargs(shape), "max_sessions": 3,
                           "flags": M.MOSHI_FLAG_SAMPLING})
    ctx = M.moshi_create(cfg, wl.make_weights(shape, 85, gains="random"))
    assert not M.moshi_uses_dep_kernel(ctx)
    M.moshi_destroy(ctx)


def _cfg_kwargs(shape):
    return dict(dim=shape.dim, n_layers=shape.n_layers, n_heads=shape.n_heads,
                ffn_hidden=shape.ffn, window=shape.window, dep_dim=shape.dep_dim,
                dep_layers=shape.dep_layers, dep_heads=shape.dep_heads,
                dep_ffn_hidden=shape.dep_ffn, n_substeps=shape.n_substeps,
                text_vocab=shape.text_vocab, audio_card=shape.audio_card,
                rope_theta=shape.rope_theta, norm_eps=shape.norm_eps, dtype=shape.dtype)


def test_dep_kernel_wait_limit_fails_cleanly():
    """Waits limited to one poll: the depformer kernel gives up at its first
    wait that is not already satisfied, every workgroup leaves, the call
    reports a device error and the context stays failed; a new context on the
    same GPU works."""
    shape = spec.TINY
    weights = wl.make_weights(shape, 87, gains="random")
    ctx = _engine(shape, weights, 3, True)
    for _ in range(2):
        M.moshi_session_join(ctx)
    f = wl.frames(shape, 3, 0, 0, 2)
    fr = [frames_matrix(shape, 3, {0: f[i], 1: f[i]}) for i in range(2)]
    M.moshi_step(ctx, fr[0])
    M.moshi_test_set_spin_limit(ctx, 1)
    for _ in range(2):
        with pytest.raises(M.MoshiError) as e:
            M.moshi_step(ctx, fr[1])
        assert e.value.status == M.MOSHI_E_DEVICE
    M.moshi_destroy(ctx)
    ctx = _engine(shape, weights, 3, True)
    slot = M.moshi_session_join(ctx)
    o = oracle.Session(oracle.Model(shape, weights))
    tok, codes = M.moshi_step(ctx, frames_matrix(shape, 3, {slot: f[0]}))
    tl, al = M.moshi_read_logits(ctx)
    r = o.step(f[0], forced_text=int(tok[slot]), forced_codes=codes[slot])
    compare_frame(shape, Stats(), "after abort", int(tok[slot]), codes[slot], tl[slot], al[slot], r)
    M.moshi_destroy(ctx)
