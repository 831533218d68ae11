"""Full-sequence recompute of the Moshi frame step, for pinning the oracle.

This is a second, differently organised formulation of the same model, used
only by the oracle's CPU pin tests:
* the temporal transformer runs all T frames of a session at once, keeps the
  whole K/V history (no ring) and applies the sliding window as a mask matrix;
* RoPE is a complex multiplication by exp(i * p * theta^(-2i/hd)) on
  interleaved pairs, not a per-pair rotation loop;
* the depformer runs all 16 substeps of a frame at once, teacher-forced, with a
  causal mask instead of a growing K/V list.
The oracle steps one frame (and one substep) at a time through a ring cache.
Agreement to ~1e-10 pins the ring bookkeeping, the window, the position
origin and the layer composition (the repository's design notes list which
pin covers what).
"""
import numpy as np

from synth import rng


def to_f64(w, dtype):
    if dtype == "bf16":
        return rng.bf16_to_f32(w).astype(np.float64)
    return np.asarray(w, np.float32).astype(np.float64)


def bf_round(x, on=True):
    """Nearest bf16 value, ties to even (vectorised frexp/ldexp form)."""
    if not on:
        return x
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.round(np.ldexp(m, 8)), e - 8)


class Weights:
    """Named fp64 views of a weight list (list order of synth.spec)."""

    def __init__(self, shape, weights):
        from synth import spec
        self.s = shape
        self.t = {}
        for (name, shp, _), w in zip(spec.tensor_list(shape), weights):
            self.t[name] = to_f64(w, shape.dtype).reshape(shp)

    def __getitem__(self, k):
        return self.t[k]


def _rms(x, g, eps):
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def _rope_complex(x, pos, hd, theta):
    """x [T, H*hd] at positions pos [T] -> rotated copy (complex form)."""
    T = x.shape[0]
    z = x.reshape(T, -1, hd // 2, 2)
    zc = z[..., 0] + 1j * z[..., 1]
    inv = theta ** (-2.0 * np.arange(hd // 2) / hd)
    rot = np.exp(1j * pos[:, None].astype(np.float64) * inv[None, :])  # [T, hd/2]
    zc = zc * rot[:, None, :]
    out = np.stack([zc.real, zc.imag], axis=-1)
    return out.reshape(T, -1)


def window_mask(q_pos, k_pos, W, mask_oldest):
    """True where query position q may attend key position k."""
    qp = q_pos[:, None]
    kp = k_pos[None, :]
    first = qp - W + 1
    if mask_oldest:
        first = np.where(qp >= W - 1, qp - W + 2, first)
    first = np.maximum(first, 0)
    return (kp <= qp) & (kp >= first)


def temporal_fullseq(w: Weights, frames, prefill=None):
    """Hidden states [T, D] and text logits [T, Vt] of T consecutive frames of
    one session that starts with ``prefill`` = (k, v) [L][n][D] fp64 (post-RoPE)
    at positions 0..n-1 (or nothing)."""
    s = w.s
    bf = s.dtype == "bf16"
    D, H, hd, F = s.dim, s.n_heads, s.head_dim, s.ffn
    frames = np.asarray(frames)
    T = frames.shape[0]
    n0 = 0 if prefill is None else prefill[0].shape[1]
    pos = n0 + np.arange(T)
    x = w["emb.text"][frames[:, 0]].copy()
    for k in range(s.n_substeps):
        x = x + w[f"emb.audio.{k}"][frames[:, 1 + k]]
    for l in range(s.n_layers):
        h = bf_round(_rms(x, w[f"layer.{l}.attn_norm"], s.norm_eps), bf)
        qkv = h @ w[f"layer.{l}.qkv"].T
        q, k, v = qkv[:, :D], qkv[:, D:2 * D], qkv[:, 2 * D:]
        q = _rope_complex(q, pos, hd, s.rope_theta)
        k = bf_round(_rope_complex(k, pos, hd, s.rope_theta), bf)
        v = bf_round(v, bf)
        if n0:
            k = np.concatenate([prefill[0][l], k], 0)
            v = np.concatenate([prefill[1][l], v], 0)
        kpos = np.arange(n0 + T)
        mask = window_mask(pos, kpos, s.window, s.mask_oldest)
        qh = q.reshape(T, H, hd).transpose(1, 0, 2)
        kh = k.reshape(-1, H, hd).transpose(1, 0, 2)
        vh = v.reshape(-1, H, hd).transpose(1, 0, 2)
        sc = qh @ kh.transpose(0, 2, 1) / np.sqrt(hd)
        sc = np.where(mask[None], sc, -np.inf)
        sc = sc - sc.max(-1, keepdims=True)
        p = np.exp(sc)
        p = p / p.sum(-1, keepdims=True)
        o = (p @ vh).transpose(1, 0, 2).reshape(T, D)
        o = bf_round(o, bf)
        x = x + o @ w[f"layer.{l}.o"].T
        h = bf_round(_rms(x, w[f"layer.{l}.mlp_norm"], s.norm_eps), bf)
        gu = h @ w[f"layer.{l}.gate_up"].T
        g, u = gu[:, :F], gu[:, F:]
        a = bf_round(g / (1.0 + np.exp(-g)) * u, bf)
        x = x + a @ w[f"layer.{l}.down"].T
    hid = bf_round(_rms(x, w["out_norm"], s.norm_eps), bf)
    return hid, hid @ w["text_head"].T


def depformer_fullseq(w: Weights, hidden, text_in, tokens):
    """Logits [S_run, Va] of the substeps run in one frame (S_run = dep_q or
    all), teacher-forced: the input token of substep s is text_in for s = 0
    and tokens[s-1] after. The depformer variants of the shape are applied as
    a mask (ring reading: the last row also excludes column 0) and as a norm
    on the head input (final-norm reading)."""
    s = w.s
    bf = s.dtype == "bf16"
    S, Dd, Hd, hdd, Fd = s.dep_steps, s.dep_dim, s.dep_heads, s.dep_head_dim, s.dep_ffn
    hid = bf_round(np.asarray(hidden, np.float64), bf)
    prev = [int(text_in)] + [int(t) for t in tokens[:S - 1]]
    Win = np.stack([w[f"dep.in.{i}"] for i in range(S)])               # [S, Dd, D]
    y = np.einsum("sod,d->so", Win, hid)
    y = y + np.stack([w[f"dep.emb.{i}"][prev[i]] for i in range(S)])
    causal = np.tril(np.ones((S, S), bool))
    if s.dep_ref_ring:
        causal[S - 1, 0] = False
    for l in range(s.dep_layers):
        Wqkv = np.stack([w[f"dep.{i}.layer.{l}.qkv"] for i in range(S)])
        Wo = np.stack([w[f"dep.{i}.layer.{l}.o"] for i in range(S)])
        Wgu = np.stack([w[f"dep.{i}.layer.{l}.gate_up"] for i in range(S)])
        Wdn = np.stack([w[f"dep.{i}.layer.{l}.down"] for i in range(S)])
        h = bf_round(_rms(y, w[f"dep.layer.{l}.attn_norm"], s.norm_eps), bf)
        qkv = np.einsum("sod,sd->so", Wqkv, h)
        q, k, v = qkv[:, :Dd], bf_round(qkv[:, Dd:2 * Dd], bf), bf_round(qkv[:, 2 * Dd:], bf)
        qh = q.reshape(S, Hd, hdd).transpose(1, 0, 2)
        kh = k.reshape(S, Hd, hdd).transpose(1, 0, 2)
        vh = v.reshape(S, Hd, hdd).transpose(1, 0, 2)
        sc = qh @ kh.transpose(0, 2, 1) / np.sqrt(hdd)
        sc = np.where(causal[None], sc, -np.inf)
        sc = sc - sc.max(-1, keepdims=True)
        p = np.exp(sc)
        p = p / p.sum(-1, keepdims=True)
        o = bf_round((p @ vh).transpose(1, 0, 2).reshape(S, Dd), bf)
        y = y + np.einsum("sod,sd->so", Wo, o)
        h = bf_round(_rms(y, w[f"dep.layer.{l}.mlp_norm"], s.norm_eps), bf)
        gu = np.einsum("sod,sd->so", Wgu, h)
        g, u = gu[:, :Fd], gu[:, Fd:]
        a = bf_round(g / (1.0 + np.exp(-g)) * u, bf)
        y = y + np.einsum("sod,sd->so", Wdn, a)
    Whd = np.stack([w[f"dep.head.{i}"] for i in range(S)])
    if s.dep_final_norm:
        y = _rms(y, w["dep.out_norm"], s.norm_eps)
    return np.einsum("sod,sd->so", Whd, bf_round(y, bf))
