"""The named synthetic workloads and their seeded inputs.

Inputs stand in for live conversations (the pages measure live audio only, no
public suite): uniform random codes with the token column's shape and ranges,
N(0, 0.02) weights, N(0, 1) K/V prefill standing in for minutes of context.

Seeds: the tiny model's weights use seed 1001, the PersonaPlex-shape model's
weights seed 1002 (shared by the four full-size workloads), the ragged test
model seed 1003. Workload w (1..5) draws frames from seed 2000+10w+1, prefill
K/V from 2000+10w+2, churn from 2000+10w+3, depformer-only inputs from
2000+10w+4. The multi-session full-size workloads (4, 5) build every session's
prefill from one shared bank of W positions, rotated per session
(prefill_from_bank), so that 64 sessions do not need 100 GB of fresh draws.
"""
from dataclasses import dataclass, field

import numpy as np

from . import rng, spec

MODEL_SEEDS = {"tiny": 1001, "personaplex": 1002, "ragged": 1003}
WEIGHT_STD = 0.02


def make_weights(m: spec.ModelShape, seed: int, gains: str = "ones", threads=None,
                 std: float = WEIGHT_STD):
    """All weight tensors of ``m`` in list order, as flat numpy arrays.

    Matrices and embeddings are N(0, std) draws of stream (seed, tensor id),
    std = 0.02 unless a test asks for another.
    RMSNorm gains are 1.0 ("ones") or 1 + 0.25 N(0, 1) ("random", used by unit
    tests so that a dropped gain changes the result). bf16 models get uint16 bf16
    bit patterns; fp32 models get float32.
    """
    out = []
    for tid, (name, shape, kind) in enumerate(spec.tensor_list(m)):
        n = int(np.prod(shape))
        if kind == "gain":
            if gains == "ones":
                g = np.ones(n, np.float32)
            else:
                g = (1.0 + 0.25 * rng.normal(seed, tid, n, 1.0, dtype="f64")).astype(np.float32)
            out.append(rng.f32_to_bf16(g) if m.dtype == "bf16" else g)
        else:
            out.append(rng.normal(seed, tid, n, std, dtype=m.dtype, threads=threads))
    return out


def frame_bounds(m: spec.ModelShape):
    return [m.text_vocab] + [m.audio_card] * m.n_substeps


def frames(m: spec.ModelShape, seed: int, session: int, t0: int, count: int) -> np.ndarray:
    """Token columns of frames t0..t0+count-1 of a session: int32 [count, 17].

    Column 0 (text) is uniform in [0, text_vocab), columns 1..16 (audio codes)
    uniform in [0, audio_card).
    """
    C = m.n_channels
    a = rng.uniform_int(seed, session, count * C, frame_bounds(m), offset=t0 * C)
    return a.reshape(count, C)


def prefill_kv(m: spec.ModelShape, seed: int, session: int, n: int, threads=None):
    """N(0, 1) K and V for positions 0..n-1 of a session, layout [L][n][H][hd].

    Element (l, j, h, d) is draw ((l*W + j)*H + h)*hd + d of stream
    (seed, 2*session) for K and (seed, 2*session+1) for V, so a session's values
    do not depend on n. Returned in the model's storage type.
    """
    L, W, D = m.n_layers, m.window, m.dim
    dt = m.dtype
    k = np.empty((L, n, D), np.uint16 if dt == "bf16" else np.float32)
    v = np.empty_like(k)
    if n == 0:
        return k, v
    for l in range(L):
        off = l * W * D
        rng.normal(seed, 2 * session, n * D, 1.0, offset=off, dtype=dt, threads=threads,
                   out=k[l].reshape(-1))
        rng.normal(seed, 2 * session + 1, n * D, 1.0, offset=off, dtype=dt, threads=threads,
                   out=v[l].reshape(-1))
    return k, v


def prefill_bank(m: spec.ModelShape, seed: int, threads=None):
    """A shared bank of N(0, 1) K and V for all W positions ([L][W][D], bank
    session id 0). Large workloads build each session's prefill from it."""
    return prefill_kv(m, seed, 0, m.window, threads=threads)


def prefill_from_bank(bank, session: int, n: int, stride: int = 47):
    """Session `session`'s prefill of n positions: the bank rotated by
    stride*session positions, then cut to n (distinct content per session
    without drawing W*D*2*L fresh values for every one of them)."""
    k, v = bank
    W = k.shape[1]
    idx = (np.arange(n) + stride * session) % W
    return np.ascontiguousarray(k[:, idx]), np.ascontiguousarray(v[:, idx])


def dep_inputs(m: spec.ModelShape, seed: int, t0: int, count: int):
    """Depformer-only inputs: hidden N(0,1) [count, D] (model storage type) and a
    text token uniform in [0, text_vocab) per frame."""
    D = m.dim
    hid = np.empty((count, D), np.uint16 if m.dtype == "bf16" else np.float32)
    for i in range(count):
        rng.normal(seed, 1 << 20, D, 1.0, offset=(t0 + i) * D, dtype=m.dtype,
                   out=hid[i].reshape(-1))
    tok = rng.uniform_int(seed, (1 << 20) + 1, count, [m.text_vocab], offset=t0)
    return hid, tok


@dataclass
class Workload:
    idx: int
    name: str
    model: str
    batch: int
    frames: int
    prefill: str            # "none", "full", "uniform"
    churn_every: int = 0
    churn_n: int = 0
    depformer_only: bool = False
    temporal_only: bool = False
    notes: str = ""
    seeds: dict = field(default_factory=dict)

    def shape(self):
        return {"tiny": spec.TINY, "personaplex": spec.PERSONAPLEX, "ragged": spec.RAGGED}[self.model]

    def seed(self, what):
        base = 2000 + 10 * self.idx
        return base + {"frames": 1, "prefill": 2, "churn": 3, "dep": 4}[what]


WORKLOADS = {
    1: Workload(1, "tiny_fp32_b1", "tiny", 1, 100, "none",
                notes="tiny fp32 model, empty ring, W=64 wraps at frame 64"),
    2: Workload(2, "temporal_bf16_b1", "personaplex", 1, 200, "full", temporal_only=True,
                notes="temporal step alone, ring prefilled to 3000 positions"),
    3: Workload(3, "depformer_bf16_b1", "personaplex", 1, 1000, "none", depformer_only=True,
                notes="depformer alone, hidden N(0,1), text token uniform"),
    4: Workload(4, "elastic_bf16_b16", "personaplex", 16, 500, "uniform", churn_every=50,
                churn_n=2, notes="fills U{0..3000}; 2 leave and 2 join every 50 frames"),
    5: Workload(5, "full_bf16_b64", "personaplex", 64, 300, "full",
                notes="all rings at the full 3000-frame window"),
}


def churn_schedule(w: Workload):
    """Session plan of an elastic workload.

    Returns (initial, events): ``initial`` is a list of (session_id, fill) for
    sessions live at tick 0 (one per slot); ``events`` maps a tick to a list of
    ("leave", session_id) and ("join", session_id, fill) actions applied before
    that tick's step. Leavers are a seeded uniform choice among live sessions;
    each joiner gets a fresh fill uniform in {0..W} (prefill of that many
    positions) and the lowest free slot.
    """
    m = w.shape()
    g = np.random.Generator(np.random.PCG64(w.seed("churn")))
    W = m.window
    if w.prefill == "full":
        fills = [W] * w.batch
    elif w.prefill == "uniform":
        fills = [int(x) for x in g.integers(0, W + 1, size=w.batch)]
    else:
        fills = [0] * w.batch
    initial = [(sid, fills[sid]) for sid in range(w.batch)]
    live = [sid for sid, _ in initial]
    nxt = w.batch
    events = {}
    if w.churn_every:
        for t in range(w.churn_every, w.frames, w.churn_every):
            acts = []
            leave = sorted(int(x) for x in g.choice(live, size=w.churn_n, replace=False))
            for sid in leave:
                acts.append(("leave", sid))
                live.remove(sid)
            for _ in range(w.churn_n):
                acts.append(("join", nxt, int(g.integers(0, W + 1))))
                live.append(nxt)
                nxt += 1
            events[t] = acts
    return initial, events
