"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the pins catch every one of them.

Each mutation is a textual edit of ``oracle/moshi_oracle.c``; the broken copy
is compiled into a temporary library and the pin checks of ``oracle_pins.py``
run against it in a child process (a mutant that reads out of bounds may crash,
which also counts as caught). A mutation that no pin catches fails this test.
"""
import os
import subprocess
import sys

import pytest

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "moshi_oracle.c")

# (id, text to replace, replacement, which occurrence (0-based))
MUTATIONS = [
    ("rope_sign", "x[2 * i] = a * c - b * s;", "x[2 * i] = a * c + b * s;", 0),
    ("rope_second", "x[2 * i + 1] = a * s + b * c;", "x[2 * i + 1] = a * s - b * c;", 0),
    ("rope_freq", "pow(theta, -2.0 * i / head_dim)", "pow(theta, -1.0 * i / head_dim)", 0),
    ("rope_position_ring_index", "orc_rope(k, H, hd, p, c->rope_theta);",
     "orc_rope(k, H, hd, p % W, c->rope_theta);", 0),
    ("window_off_by_one", "int64_t first = p - W + 1;", "int64_t first = p - W;", 0),
    ("window_too_short", "int64_t first = p - W + 1;", "int64_t first = p - W + 2;", 0),
    ("mask_oldest_ignored", "first = p - W + 2;", "first = p - W + 1;", 0),
    ("ring_slot", "int64_t slot = (first + j) % W;", "int64_t slot = (first + j + 1) % W;", 0),
    ("ring_write_slot", "ring_put(s, s->k_ring, l, p % W, k);",
     "ring_put(s, s->k_ring, l, (p + 1) % W, k);", 0),
    ("prefill_position", "s->pos = n;", "s->pos = n - (n > 0);", 0),
    ("attn_residual_dropped", "for (int i = 0; i < D; ++i) x[i] += y[i];",
     "for (int i = 0; i < D; ++i) x[i] = y[i];", 0),
    ("mlp_residual_dropped", "for (int i = 0; i < D; ++i) x[i] += y[i];",
     "for (int i = 0; i < D; ++i) x[i] = y[i];", 1),
    ("norm_gain_dropped", "gd[i] = wget(m, g, i);", "gd[i] = 1.0;", 0),
    ("norm_eps_dropped", "sqrt(ss / n + eps)", "sqrt(ss / n)", 0),
    ("swiglu_swapped", "a[i] = rnd(m, orc_silu(gu[i]) * gu[F + i]);",
     "a[i] = rnd(m, orc_silu(gu[F + i]) * gu[i]);", 0),
    ("attn_scale", "1.0 / sqrt((double)hd)", "1.0 / (double)hd", 0),
    ("attn_o_unrounded", "for (int i = 0; i < D; ++i) o[i] = rnd(m, o[i]);",
     "for (int i = 0; i < D; ++i) o[i] = o[i];", 0),
    ("embed_channel_shift", "(size_t)frame[1 + k] * D", "(size_t)frame[k] * D", 0),
    ("final_norm_gain", "rmsnorm_w(m, x, m->out_norm, D, h);",
     "rmsnorm_w(m, x, m->mlp_norm[c->n_layers - 1], D, h);", 0),
    ("dep_forcing_ignored", "prev = (forced && forced[s] >= 0) ? forced[s] : code;",
     "prev = code;", 0),
    ("dep_self_excluded", "hh * hdd, s + 1 - first, hdd", "hh * hdd, s > first ? s - first : 1, hdd",
     0),
    ("dep_q_ignored", "int S_run = dep_run(c);", "int S_run = S;", 0),
    ("dep_ring_reading_ignored", "int first = (c->dep_ref_ring && s == S_run - 1) ? 1 : 0;",
     "int first = 0;", 0),
    ("dep_ring_reading_wrong_step", "int first = (c->dep_ref_ring && s == S_run - 1) ? 1 : 0;",
     "int first = (c->dep_ref_ring && s == S_run - 2) ? 1 : 0;", 0),
    ("dep_final_norm_skipped", "if (c->dep_final_norm) {", "if (0) {", 0),
    ("dep_final_norm_wrong_gain", "rmsnorm_w(m, y, m->dep_out_norm, Dd, h);",
     "rmsnorm_w(m, y, m->dep_mlp_norm[Ld - 1], Dd, h);", 0),
    ("load_ring_row_shift", "ring_put(s, s->k_ring, l, j, kv);",
     "ring_put(s, s->k_ring, l, (j + 1) % W, kv);", 0),
    ("load_ring_position", "  s->pos = pos;\n", "  s->pos = pos + 1;\n", 0),
    ("splitmix_constant", "0xBF58476D1CE4E5B9ULL", "0xBF58476D1CE4E5B7ULL", 0),
    ("uniform_bits", "(double)(orc_splitmix64(child, (uint64_t)pos + 1) >> 11)",
     "(double)(orc_splitmix64(child, (uint64_t)pos + 1) >> 12)", 0),
    ("sample_topk_short", "for (int j = 0; j < k; ++j) member[c[j].i] = 1;",
     "for (int j = 0; j + 1 < k; ++j) member[c[j].i] = 1;", 0),
    ("sample_temperature_total", "total += exp(((double)(float)logits[i] - lmax) / temperature);",
     "total += exp(((double)(float)logits[i] - lmax));", 0),
    ("sample_temperature_run", "run += exp(((double)(float)logits[i] - lmax) / temperature);",
     "run += exp(((double)(float)logits[i] - lmax) * temperature);", 0),
    ("sample_tie_order", "return x->i < y->i ? -1 : (x->i > y->i);",
     "return x->i > y->i ? -1 : (x->i < y->i);", 0),
    ("sample_order_reversed", "if (kx != ky) return kx > ky ? -1 : 1;",
     "if (kx != ky) return kx < ky ? -1 : 1;", 0),
    ("sample_fp64_weights", "run += exp(((double)(float)logits[i] - lmax) / temperature);",
     "run += exp((logits[i] - lmax) / temperature);", 0),
    ("dep_inproj_shared", "linear(m, m->dep_in[s], Dd, D, hid_r, y);",
     "linear(m, m->dep_in[0], Dd, D, hid_r, y);", 0),
    ("dep_embedding_shared", "wget(m, m->dep_emb[s], (size_t)prev * Dd + i)",
     "wget(m, m->dep_emb[s > 0 ? 1 : 0], (size_t)prev * Dd + i)", 0),
    ("dep_head_input_unrounded", "for (int i = 0; i < Dd; ++i) h[i] = rnd(m, y[i]);",
     "for (int i = 0; i < Dd; ++i) h[i] = y[i];", 0),
    ("dep_layer_weights_shared", "int wi = s * Ld + l;", "int wi = l;", 0),
    ("argmax_last_tie", "if (v[i] > v[best]) best = i;", "if (v[i] >= v[best]) best = i;", 0),
    ("bf16_ties_away", "return ldexp(nearbyint(ldexp(mant, 8)), e - 8);",
     "return ldexp(round(ldexp(mant, 8)), e - 8);", 0),
]


def _mutate(text, old, new, occ):
    start = -1
    for _ in range(occ + 1):
        start = text.index(old, start + 1)
    return text[:start] + new + text[start + len(old):]


@pytest.mark.parametrize("mid,old,new,occ", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(tmp_path, mid, old, new, occ):
    text = open(SRC).read()
    assert text.count(old) > occ, f"mutation anchor not found: {old!r}"
    src = tmp_path / "mutant.c"
    src.write_text(_mutate(text, old, new, occ))
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
                           "-ffp-contract=off", "-o", str(so), str(src), "-lm"])
    r = subprocess.run([sys.executable, os.path.join(os.path.dirname(__file__), "run_pins.py"),
                        str(so)], capture_output=True, text=True, timeout=600)
    assert r.returncode != 3, f"no pin caught mutation {mid}:\n{r.stdout}{r.stderr}"
    assert r.returncode != 0 or "CAUGHT" in r.stdout, r.stdout + r.stderr
