"""GPU test of moshi_step_enqueue_noalloc (the step with its kernel scratch in
the library's static device array): on two calls in a row -- the first on a
larger model, the second on a smaller one, so the second finds the first's
contents in the shared array -- and then over several frames of each
context, the outputs equal moshi_step_enqueue's on an identical context
(same kernel: bit-identical), and the slot bookkeeping matches."""
import numpy as np
import pytest

import full_duplex_speech_amd as M
from synth import spec, workloads as wl
from gpu_util import DevBuf, log, new_engine

pytestmark = pytest.mark.gpu


def _pair(shape, seed, fill):
    weights = wl.make_weights(shape, seed, gains="random")
    ctxs = []
    for _ in range(2):
        ctx = new_engine(shape, weights, 1)
        assert M.moshi_uses_step_kernel(ctx)
        slot = M.moshi_session_join(ctx)
        if fill:
            k, v = wl.prefill_kv(shape, seed + 1, 0, fill)
            M.moshi_session_prefill_kv(ctx, slot, k, v)
        ctxs.append(ctx)
    return ctxs


def _bufs(shape, frames):
    return [(DevBuf(f[None, :]), DevBuf(np.full(1, -7, np.int32)),
             DevBuf(np.full((1, shape.n_substeps), -7, np.int32))) for f in frames]


def test_noalloc_matches_enqueue():
    big, small = spec.RAGGED.replace(window=150), spec.TINY  # bf16 then a smaller fp32 model
    a_ref, a_na = _pair(big, 91, 140)
    b_ref, b_na = _pair(small, 92, 0)
    T = 6
    fa = wl.frames(big, 93, 0, 0, T)
    fb = wl.frames(small, 94, 0, 0, T)
    ba_ref, ba_na, bb_ref, bb_na = _bufs(big, fa), _bufs(big, fa), _bufs(small, fb), _bufs(small, fb)
    # two calls in a row: the larger model, then the smaller one
    for t in range(T):
        M.moshi_step_enqueue_noalloc(a_na, *(x.ptr for x in ba_na[t]))
        M.moshi_step_enqueue_noalloc(b_na, *(x.ptr for x in bb_na[t]))
        M.moshi_step_enqueue(a_ref, *(x.ptr for x in ba_ref[t]))
        M.moshi_step_enqueue(b_ref, *(x.ptr for x in bb_ref[t]))
    for ctx in (a_ref, a_na, b_ref, b_na):
        M.moshi_sync(ctx)
    for name, ref, na in (("ragged bf16", ba_ref, ba_na), ("tiny fp32", bb_ref, bb_na)):
        for t in range(T):
            assert np.array_equal(ref[t][1].read(), na[t][1].read()), f"{name} t={t}: text token"
            assert np.array_equal(ref[t][2].read(), na[t][2].read()), f"{name} t={t}: codes"
    assert M.moshi_session_info(a_ref, 0) == M.moshi_session_info(a_na, 0)
    assert M.moshi_session_info(b_ref, 0) == M.moshi_session_info(b_na, 0)
    tl_r, al_r = M.moshi_read_logits(b_ref)
    tl_n, al_n = M.moshi_read_logits(b_na)
    assert np.array_equal(tl_r, tl_n) and np.array_equal(al_r, al_n)
    for ctx in (a_ref, a_na, b_ref, b_na):
        M.moshi_destroy(ctx)
    log("no-alloc step: bit-identical to moshi_step_enqueue on both models")


def test_noalloc_rejects_what_does_not_fit():
    """A context without the one-session step kernel (capacity 2) is refused
    with a clear error; nothing is launched."""
    shape = spec.TINY
    ctx = new_engine(shape, wl.make_weights(shape, 95), 2)
    M.moshi_session_join(ctx)
    d = DevBuf(np.zeros((2, shape.n_channels), np.int32))
    with pytest.raises(M.MoshiError) as e:
        M.moshi_step_enqueue_noalloc(ctx, d.ptr)
    assert e.value.status == M.MOSHI_E_INVALID and "step kernel" in str(e.value)
    M.moshi_destroy(ctx)


def test_noalloc_after_a_call_that_launches_nothing():
    """A call with no live session launches no step kernel (its outputs read
    -1); the barrier counter sets alternate per launch on the device, not per
    call, so the launches after it still find a cleared set: several frames
    then equal moshi_step_enqueue's bit for bit."""
    shape = spec.TINY
    weights = wl.make_weights(shape, 96, gains="random")
    ref, na = new_engine(shape, weights, 1), new_engine(shape, weights, 1)
    T = 5
    fr = wl.frames(shape, 97, 0, 0, T)
    empty_ref, empty_na = _bufs(shape, fr[:1]), _bufs(shape, fr[:1])
    M.moshi_step_enqueue(ref, *(x.ptr for x in empty_ref[0]))
    M.moshi_step_enqueue_noalloc(na, *(x.ptr for x in empty_na[0]))
    M.moshi_sync(na)
    assert empty_na[0][1].read()[0] == -1 and np.all(empty_na[0][2].read() == -1)
    for ctx in (ref, na):
        assert M.moshi_session_join(ctx) == 0
    b_ref, b_na = _bufs(shape, fr), _bufs(shape, fr)
    for t in range(T):
        M.moshi_step_enqueue(ref, *(x.ptr for x in b_ref[t]))
        M.moshi_step_enqueue_noalloc(na, *(x.ptr for x in b_na[t]))
    for ctx in (ref, na):
        M.moshi_sync(ctx)
    for t in range(T):
        assert np.array_equal(b_ref[t][1].read(), b_na[t][1].read()), f"t={t}: text token"
        assert np.array_equal(b_ref[t][2].read(), b_na[t][2].read()), f"t={t}: codes"
    assert M.moshi_session_info(ref, 0) == M.moshi_session_info(na, 0)
    for ctx in (ref, na):
        M.moshi_destroy(ctx)
    log("no-alloc step after a call that launched nothing: bit-identical")
