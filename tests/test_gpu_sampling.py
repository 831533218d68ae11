"""GPU parity of temperature + top-k sampling (MOSHI_FLAG_SAMPLING) against
the oracle's sampler: every drawn token equals the oracle's draw from the
GPU's own fp32 logits with the same counter-based uniform (splitmix64 child
stream of the session seed at the session's frame position) -- exact except
where the draw lies within 1e-12 of a neighbour's running sum; the logits
themselves match the oracle (teacher-forced on the GPU's tokens); greedy
sessions in the same batch stay greedy; forced heads return the forced token;
a session's draws do not depend on its slot or on the other sessions."""
import numpy as np
import pytest

import full_duplex_speech_amd as M
import oracle
from synth import spec, workloads as wl
from gpu_util import Stats, cfg_of, compare_frame, frames_matrix, log

pytestmark = pytest.mark.gpu

PARAMS = {  # sid -> (text T, text k, audio T, audio k, seed) or None = greedy
    0: None,
    1: (0.7, 25, 0.8, 250, 11),
    2: (1.0, -1, 0.9, 5, 12),
    3: (0.7, 25, 0.0, 0, 13),   # text draws, greedy codes
}


def _run(shape, weights, B, plan, T, check=True, forcing=True):
    cfg = cfg_of(shape, B)
    cfg.flags |= M.MOSHI_FLAG_SAMPLING
    ctx = M.moshi_create(cfg, weights)
    assert not M.moshi_uses_step_kernel(ctx)
    om = oracle.Model(shape, weights)
    slot_of, orc, t_of = {}, {}, {}
    stats = Stats()
    n_drawn = n_excused = 0
    outs = {}
    n = shape.dep_steps
    for t in range(T):
        for act in plan.get(t, []):
            if act[0] == "leave":
                M.moshi_session_leave(ctx, slot_of.pop(act[1]))
                continue
            sid, fill = act[1], act[2]
            s = M.moshi_session_join(ctx)
            slot_of[sid] = s
            o = oracle.Session(om)
            if fill:
                k, v = wl.prefill_kv(shape, 41, sid, fill)
                M.moshi_session_prefill_kv(ctx, s, k, v)
                o.prefill(k, v)
            p = PARAMS[sid % len(PARAMS)]
            if p is not None:
                M.moshi_session_set_sampling(ctx, s, *p)
            orc[sid] = o
            t_of[sid] = 0
        rows = {slot_of[sid]: wl.frames(shape, 43, sid, t_of[sid], 1)[0] for sid in slot_of}
        fr = frames_matrix(shape, B, rows)
        fc = np.full((B, shape.n_channels), -1, np.int32)
        if forcing and t % 3 == 1:
            for sid, s in slot_of.items():
                fc[s, 2] = (sid * 7 + t) % shape.audio_card  # code 1 forced
        pos_before = {sid: M.moshi_session_info(ctx, s)[0] for sid, s in slot_of.items()}
        tok, codes = M.moshi_step_forced(ctx, fr, fc)
        tl, al = M.moshi_read_logits(ctx)
        for sid, s in slot_of.items():
            outs.setdefault(sid, []).append((int(tok[s]), codes[s].copy()))
            t_of[sid] += 1
            if not check:
                continue
            p = PARAMS[sid % len(PARAMS)]
            r = orc[sid].step(fr[s], forced_text=int(tok[s]), forced_codes=codes[s])
            # heads: (is text, index, gpu token, logits row, temperature, top k, stream, forced)
            heads = [(True, 0, int(tok[s]), tl[s], p[0] if p else 0.0, p[1] if p else 0, 0, -1)]
            for q in range(n):
                heads.append((False, q, int(codes[s][q]), al[s][q], p[2] if p else 0.0,
                              p[3] if p else 0, 1 + q, int(fc[s, 1 + q])))
            greedy_text, greedy_codes = int(tok[s]), codes[s][:n].copy()
            for is_text, q, g, lrow, temp, kk, stream, forced in heads:
                if forced >= 0:
                    assert g == forced
                    if not is_text:
                        greedy_codes[q] = r["codes"][q]
                    continue
                if temp > 0:
                    u = oracle.uniform(p[4], stream, pos_before[sid])
                    want, margin = oracle.sample(lrow.astype(np.float64), temp, kk, u)
                    n_drawn += 1
                    if margin < 1e-12:
                        n_excused += 1
                    else:
                        assert g == want, f"t={t} sid={sid} stream={stream}: drew {g}, oracle {want}"
                    # the comparison below is for greedy heads only
                    if is_text:
                        greedy_text = r["text_token"]
                    else:
                        greedy_codes[q] = r["codes"][q]
            r2 = dict(r, audio_logits=r["audio_logits"][:n], codes=r["codes"][:n],
                      audio_margins=r["audio_margins"][:n])
            compare_frame(shape.replace(n_substeps=n), stats, f"t={t} sid={sid}", greedy_text,
                          greedy_codes, tl[s], al[s][:n], r2)
    M.moshi_destroy(ctx)
    return outs, stats, n_drawn, n_excused


@pytest.mark.parametrize("case", ["tiny_fp32_b1", "ragged_bf16_b4", "ragged_bf16_b17"])
def test_sampling_parity(case):
    if case == "tiny_fp32_b1":
        shape, B = spec.TINY.replace(window=16), 1
        plan = {0: [("join", 1, 0)]}
        T = 10
    elif case == "ragged_bf16_b17":
        # two 16-column MFMA blocks per projection tile, with churn
        shape, B = spec.RAGGED, 17
        plan = {0: [("join", i, (5 * i) % 38) for i in range(16)],
                2: [("join", 16, 3)],
                4: [("leave", 2)],
                5: [("join", 17, 0)]}
        T = 7
    else:
        shape, B = spec.RAGGED, 4
        plan = {0: [("join", 0, 0), ("join", 1, 12), ("join", 2, 37)],
                3: [("join", 3, 5)],
                6: [("leave", 0)],
                7: [("join", 5, 2)]}  # sid 5 samples like sid 1 (seed 11)
        T = 10
    weights = wl.make_weights(shape, 85, gains="random")
    _, stats, nd, ne = _run(shape, weights, B, plan, T)
    assert nd > 0
    log(f"sampling {case}: {nd} draws checked ({ne} within 1e-12 of a boundary); greedy {stats}")


def test_sampling_isolation():
    """A sampling session's tokens are bit-identical alone in slot 0 and
    batched in slot 2 with other sessions."""
    shape = spec.RAGGED
    weights = wl.make_weights(shape, 86, gains="random")
    batched, _, _, _ = _run(shape, weights, 4, {0: [("join", 0, 3), ("join", 2, 0),
                                                     ("join", 1, 9)]}, 8, check=False, forcing=False)
    alone, _, _, _ = _run(shape, weights, 4, {0: [("join", 1, 9)]}, 8, check=False, forcing=False)
    for t, (a, b) in enumerate(zip(alone[1], batched[1])):
        assert a[0] == b[0] and np.array_equal(a[1], b[1]), f"isolation broken at t={t}"
