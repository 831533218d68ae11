"""TEST INFRASTRUCTURE ONLY -- ctypes front end of the fp64 CPU oracle.

The oracle (``moshi_oracle.c``) is a plain, slow, single-threaded fp64
reference of one Moshi/PersonaPlex frame step. Only ``tests/``, the smoke check
in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import it.
It shares no code with the HIP library; both read the same host arrays from
``synth``.

Calls into the C library release the GIL, so independent sessions can run in
parallel Python threads (one session per thread).
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moshi_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math: IEEE fp64 throughout)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
                               "-ffp-contract=off", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "dim", "n_layers", "n_heads", "ffn_hidden", "window",
        "dep_dim", "dep_layers", "dep_heads", "dep_ffn_hidden", "n_substeps",
        "text_vocab", "audio_card")] + [
        ("rope_theta", ctypes.c_double), ("norm_eps", ctypes.c_double),
        ("bf16", ctypes.c_int32), ("mask_oldest", ctypes.c_int32), ("dep_q", ctypes.c_int32),
        ("dep_final_norm", ctypes.c_int32), ("dep_ref_ring", ctypes.c_int32)]


def _p(a):
    return None if a is None else a.ctypes.data


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


class using:
    """Context manager: route every oracle call to another build of the oracle
    (the mutation tests load deliberately broken copies this way)."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = lib()
        _lib = _bind(ctypes.CDLL(self.path))
        return _lib

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _bind(L):
    vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    L.orc_bf16_round.argtypes = [dbl]
    L.orc_bf16_round.restype = dbl
    L.orc_rmsnorm.argtypes = [vp, vp, ctypes.c_int, dbl, vp]
    L.orc_rmsnorm.restype = None
    L.orc_rope.argtypes = [vp, ctypes.c_int, ctypes.c_int, i64, dbl]
    L.orc_rope.restype = None
    L.orc_attend.argtypes = [vp, vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
    L.orc_attend.restype = None
    L.orc_silu.argtypes = [dbl]
    L.orc_silu.restype = dbl
    L.orc_argmax.argtypes = [vp, ctypes.c_int, vp]
    L.orc_argmax.restype = i32
    L.orc_splitmix64.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
    L.orc_splitmix64.restype = ctypes.c_uint64
    L.orc_uniform.argtypes = [ctypes.c_uint64, i32, i64]
    L.orc_uniform.restype = dbl
    L.orc_sample.argtypes = [vp, ctypes.c_int, dbl, ctypes.c_int, dbl, vp]
    L.orc_sample.restype = i32
    L.orc_n_tensors.argtypes = [ctypes.POINTER(Config)]
    L.orc_n_tensors.restype = i32
    L.orc_model_new.argtypes = [ctypes.POINTER(Config), vp, i32]
    L.orc_model_new.restype = vp
    L.orc_model_free.argtypes = [vp]
    L.orc_model_free.restype = None
    L.orc_session_new.argtypes = [vp]
    L.orc_session_new.restype = vp
    L.orc_session_free.argtypes = [vp]
    L.orc_session_free.restype = None
    L.orc_session_reset.argtypes = [vp]
    L.orc_session_reset.restype = None
    L.orc_session_prefill.argtypes = [vp, i32, vp, vp]
    L.orc_session_prefill.restype = ctypes.c_int
    L.orc_session_load_ring.argtypes = [vp, i64, vp, vp]
    L.orc_session_load_ring.restype = ctypes.c_int
    L.orc_session_read_ring.argtypes = [vp, vp, vp]
    L.orc_session_read_ring.restype = None
    L.orc_session_info.argtypes = [vp, vp, vp, vp]
    L.orc_session_info.restype = None
    L.orc_temporal.argtypes = [vp, vp, vp, vp, vp, vp]
    L.orc_temporal.restype = ctypes.c_int
    L.orc_depformer.argtypes = [vp, vp, i32, vp, vp, vp, vp]
    L.orc_depformer.restype = ctypes.c_int
    L.orc_step.argtypes = [vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    L.orc_step.restype = ctypes.c_int
    return L


# ---------------------------------------------------------------- primitives

def bf16_round(x: float) -> float:
    return lib().orc_bf16_round(float(x))


def rmsnorm(x, g, eps):
    x = np.ascontiguousarray(x, np.float64)
    g = np.ascontiguousarray(g, np.float64)
    out = np.empty_like(x)
    lib().orc_rmsnorm(_p(x), _p(g), x.size, eps, _p(out))
    return out


def rope(v, n_heads, head_dim, pos, theta=1e4):
    v = np.array(v, np.float64, copy=True).reshape(-1)
    lib().orc_rope(_p(v), n_heads, head_dim, int(pos), theta)
    return v


def attend(q, keys, vals):
    q = np.ascontiguousarray(q, np.float64)
    keys = np.ascontiguousarray(keys, np.float64)
    vals = np.ascontiguousarray(vals, np.float64)
    n, hd = keys.shape
    o = np.empty(hd, np.float64)
    lib().orc_attend(_p(q), _p(keys), _p(vals), n, hd, hd, _p(o))
    return o


def silu(z: float) -> float:
    return lib().orc_silu(float(z))


def argmax(v):
    v = np.ascontiguousarray(v, np.float64)
    m = np.zeros(1, np.float64)
    i = lib().orc_argmax(_p(v), v.size, _p(m))
    return int(i), float(m[0])


def splitmix64(seed: int, n: int) -> int:
    return int(lib().orc_splitmix64(seed & (2**64 - 1), n))


def uniform(seed: int, stream: int, pos: int) -> float:
    """The session's draw in [0, 1) for a stream (0 text, 1+s substep s) at a position."""
    return float(lib().orc_uniform(seed & (2**64 - 1), int(stream), int(pos)))


def sample(logits, temperature: float, top_k: int, u: float):
    """Temperature + top-k draw (decided on the fp32 values of the logits);
    returns (index, margin)."""
    v = np.ascontiguousarray(logits, np.float64)
    m = np.zeros(1, np.float64)
    i = lib().orc_sample(_p(v), v.size, float(temperature), int(top_k), float(u), _p(m))
    return int(i), float(m[0])


# ---------------------------------------------------------------- model

def make_config(shape) -> Config:
    c = Config()
    c.dim, c.n_layers, c.n_heads = shape.dim, shape.n_layers, shape.n_heads
    c.ffn_hidden, c.window = shape.ffn, shape.window
    c.dep_dim, c.dep_layers, c.dep_heads = shape.dep_dim, shape.dep_layers, shape.dep_heads
    c.dep_ffn_hidden, c.n_substeps = shape.dep_ffn, shape.n_substeps
    c.text_vocab, c.audio_card = shape.text_vocab, shape.audio_card
    c.rope_theta, c.norm_eps = shape.rope_theta, shape.norm_eps
    c.bf16 = 1 if shape.dtype == "bf16" else 0
    c.mask_oldest = 1 if shape.mask_oldest else 0
    c.dep_q = shape.dep_q
    c.dep_final_norm = 1 if shape.dep_final_norm else 0
    c.dep_ref_ring = 1 if shape.dep_ref_ring else 0
    return c


class Model:
    """Oracle model bound to host weight arrays (kept alive here)."""

    def __init__(self, shape, weights):
        self.shape = shape
        self.cfg = make_config(shape)
        want = np.uint16 if shape.dtype == "bf16" else np.float32
        self._w = [np.ascontiguousarray(w, want) for w in weights]
        self._ptrs = (ctypes.c_void_p * len(self._w))(*[w.ctypes.data for w in self._w])
        self._L = lib()
        self.h = self._L.orc_model_new(ctypes.byref(self.cfg), self._ptrs, len(self._w))
        if not self.h:
            raise ValueError("oracle rejected the model config / tensor count")

    def __del__(self):
        if getattr(self, "h", None):
            self._L.orc_model_free(self.h)
            self.h = None

    def depformer(self, hidden, text_in, forced=None, want_logits=True):
        """Depformer substeps from a hidden state (fp64 values) and a text token."""
        s = self.shape
        hid = np.ascontiguousarray(hidden, np.float64)
        fc = None if forced is None else np.ascontiguousarray(forced, np.int32)
        lg = np.empty((s.n_substeps, s.audio_card), np.float64) if want_logits else None
        codes = np.empty(s.n_substeps, np.int32)
        mg = np.empty(s.n_substeps, np.float64)
        rc = self._L.orc_depformer(self.h, _p(hid), int(text_in), _p(fc), _p(lg), _p(codes), _p(mg))
        if rc:
            raise ValueError("oracle rejected depformer inputs")
        return {"codes": codes, "audio_logits": lg, "audio_margins": mg}


class Session:
    def __init__(self, model: Model):
        self.model = model
        self._L = model._L
        self.h = self._L.orc_session_new(model.h)
        if not self.h:
            raise MemoryError("oracle session allocation failed")

    def __del__(self):
        if getattr(self, "h", None):
            self._L.orc_session_free(self.h)
            self.h = None

    def reset(self):
        self._L.orc_session_reset(self.h)

    def prefill(self, k, v):
        n = k.shape[1] if k.ndim == 3 else 0
        k = np.ascontiguousarray(k)
        v = np.ascontiguousarray(v)
        if self._L.orc_session_prefill(self.h, n, _p(k), _p(v)):
            raise ValueError("prefill length outside [0, window]")

    def load_ring(self, pos, k, v):
        """Replace the ring (k, v [L][W][D], model storage type, row j = ring
        slot j) and set the position (state transfer for tests)."""
        k = np.ascontiguousarray(k)
        v = np.ascontiguousarray(v)
        if self._L.orc_session_load_ring(self.h, int(pos), _p(k), _p(v)):
            raise ValueError("negative position")

    def read_ring(self):
        """The ring (k, v [L][W][D], model storage type, row j = ring slot j)."""
        s = self.model.shape
        dt = np.uint16 if s.dtype == "bf16" else np.float32
        k = np.empty((s.n_layers, s.window, s.dim), dt)
        v = np.empty_like(k)
        self._L.orc_session_read_ring(self.h, _p(k), _p(v))
        return k, v

    def info(self):
        pos = np.zeros(1, np.int64)
        fill = np.zeros(1, np.int32)
        wi = np.zeros(1, np.int32)
        self._L.orc_session_info(self.h, _p(pos), _p(fill), _p(wi))
        return int(pos[0]), int(fill[0]), int(wi[0])

    def temporal(self, frame, want_logits=True):
        s = self.model.shape
        f = np.ascontiguousarray(frame, np.int32)
        hid = np.empty(s.dim, np.float64)
        lg = np.empty(s.text_vocab, np.float64) if want_logits else None
        tok = np.zeros(1, np.int32)
        mg = np.zeros(1, np.float64)
        if self._L.orc_temporal(self.h, _p(f), _p(hid), _p(lg), _p(tok), _p(mg)):
            raise ValueError("oracle rejected the frame")
        return {"text_token": int(tok[0]), "text_margin": float(mg[0]), "text_logits": lg,
                "hidden": hid}

    def step(self, frame, forced_text=-1, forced_codes=None, want_logits=True):
        s = self.model.shape
        f = np.ascontiguousarray(frame, np.int32)
        fc = None if forced_codes is None else np.ascontiguousarray(forced_codes, np.int32)
        tok = np.zeros(1, np.int32)
        codes = np.empty(s.n_substeps, np.int32)
        tl = np.empty(s.text_vocab, np.float64) if want_logits else None
        al = np.empty((s.n_substeps, s.audio_card), np.float64) if want_logits else None
        tm = np.zeros(1, np.float64)
        am = np.empty(s.n_substeps, np.float64)
        hid = np.empty(s.dim, np.float64)
        rc = self._L.orc_step(self.h, _p(f), int(forced_text), _p(fc), _p(tok), _p(codes), _p(tl),
                            _p(al), _p(tm), _p(am), _p(hid))
        if rc:
            raise ValueError("oracle rejected the frame")
        return {"text_token": int(tok[0]), "codes": codes, "text_logits": tl, "audio_logits": al,
                "text_margin": float(tm[0]), "audio_margins": am, "hidden": hid}
