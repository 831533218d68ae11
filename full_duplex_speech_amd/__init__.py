"""MI355X-native Moshi/PersonaPlex frame step.

A thin ctypes binding of ``libmoshi.so`` (the C ABI in ``include/moshi.h``):
argument marshalling only, with the same function names. Every step of the
path runs in the library's HIP kernels; if the library is not built this
module raises instead of falling back to anything else.

Typical use::

    import full_duplex_speech_amd as m
    cfg = m.make_config(dim=4096, n_layers=32, ..., dtype="bf16", max_sessions=1)
    ctx = m.moshi_create(cfg, weights)          # list of host numpy arrays
    slot = m.moshi_session_join(ctx)
    text, codes = m.moshi_step(ctx, frames)     # frames int32 [B, 17]
    m.moshi_destroy(ctx)
"""
import ctypes
import os
import subprocess
import weakref

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)
LIB_PATH = os.path.join(_HERE, "libmoshi.so")
_CSRC = os.path.join(_HERE, "csrc")
_SOURCES = [os.path.join(_CSRC, "kernels.hip"), os.path.join(_CSRC, "step.hip"),
            os.path.join(_CSRC, "static_step.hip"), os.path.join(_CSRC, "engine.cpp"),
            os.path.join(_CSRC, "stream.cpp")]
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
               # no packed-fp32 instructions in any kernel
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", os.path.join(_ROOT, "include")]

MOSHI_OK, MOSHI_E_INVALID, MOSHI_E_FULL, MOSHI_E_NOSESSION, MOSHI_E_DEVICE, MOSHI_E_OOM = \
    0, -1, -2, -3, -4, -5
MOSHI_F32, MOSHI_BF16 = 0, 1
MOSHI_FLAG_MASK_OLDEST = 1
MOSHI_FLAG_DEP_FINAL_NORM = 2
MOSHI_FLAG_DEP_REF_RING = 4
MOSHI_FLAG_SAMPLING = 8

_lib = None
_live_ctx = weakref.WeakSet()


def build(verbose=False) -> str:
    """Compile libmoshi.so for gfx950 with hipcc (in-tree)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [hipcc] + HIPCC_FLAGS + _SOURCES + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stdout + r.stderr)
    if verbose:
        print(r.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


class MoshiError(RuntimeError):
    def __init__(self, status, msg=""):
        super().__init__(f"{moshi_strerror(status)} ({status}){': ' + msg if msg else ''}")
        self.status = status


class moshi_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "dim", "n_layers", "n_heads", "ffn_hidden", "window",
        "dep_dim", "dep_layers", "dep_heads", "dep_ffn_hidden", "n_substeps",
        "text_vocab", "audio_card")] + [
        ("rope_theta", ctypes.c_double), ("norm_eps", ctypes.c_double),
        ("dtype", ctypes.c_int32), ("max_sessions", ctypes.c_int32), ("flags", ctypes.c_uint32),
        ("dep_q", ctypes.c_int32)]


class moshi_sampling(ctypes.Structure):
    _fields_ = [("text_temperature", ctypes.c_double), ("text_top_k", ctypes.c_int32),
                ("audio_temperature", ctypes.c_double), ("audio_top_k", ctypes.c_int32),
                ("seed", ctypes.c_uint64)]


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first (__graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        cfgp = ctypes.POINTER(moshi_config)
        sig = {
            "moshi_n_tensors": ([cfgp], i32),
            "moshi_create": ([cfgp, vp, i32, vp, ctypes.POINTER(vp)], ctypes.c_int),
            "moshi_destroy": ([vp], ctypes.c_int),
            "moshi_get_config": ([vp, cfgp], ctypes.c_int),
            "moshi_stream_create": ([vp, i32, vp, ctypes.POINTER(vp)], ctypes.c_int),
            "moshi_stream_destroy": ([vp], ctypes.c_int),
            "moshi_stream_reset": ([vp, i32], ctypes.c_int),
            "moshi_stream_step": ([vp, vp, vp, vp, vp, vp, vp], ctypes.c_int),
            "moshi_stream_last_error": ([vp], ctypes.c_char_p),
            "moshi_session_join": ([vp, ctypes.POINTER(i32)], ctypes.c_int),
            "moshi_session_leave": ([vp, i32], ctypes.c_int),
            "moshi_session_set_sampling": ([vp, i32, ctypes.POINTER(moshi_sampling)], ctypes.c_int),
            "moshi_step": ([vp, vp, vp, vp], ctypes.c_int),
            "moshi_step_forced": ([vp, vp, vp, vp, vp], ctypes.c_int),
            "moshi_test_set_spin_limit": ([vp, i32], ctypes.c_int),
            "moshi_temporal_step": ([vp, vp, vp], ctypes.c_int),
            "moshi_step_enqueue": ([vp, vp, vp, vp], ctypes.c_int),
            "moshi_step_enqueue_noalloc": ([vp, vp, vp, vp], ctypes.c_int),
            "moshi_sync": ([vp], ctypes.c_int),
            "moshi_depformer_step": ([vp, vp, vp, vp], ctypes.c_int),
            "moshi_session_prefill_kv": ([vp, i32, i32, vp, vp], ctypes.c_int),
            "moshi_session_info": ([vp, i32, vp, vp, vp], ctypes.c_int),
            "moshi_session_read_kv": ([vp, i32, vp, vp], ctypes.c_int),
            "moshi_session_prefill_frames": ([vp, i32, i32, vp, vp, vp], ctypes.c_int),
            "moshi_read_logits": ([vp, vp, vp], ctypes.c_int),
            "moshi_read_hidden": ([vp, vp], ctypes.c_int),
            "moshi_time_kernels": ([vp, vp, i32, vp, vp, vp, i32], ctypes.c_int),
            "moshi_kernel_class_name": ([i32], ctypes.c_char_p),
            "moshi_uses_step_kernel": ([vp], i32),
            "moshi_uses_dep_kernel": ([vp], i32),
            "moshi_strerror": ([ctypes.c_int], ctypes.c_char_p),
            "moshi_last_error": ([vp], ctypes.c_char_p),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def unload():
    """Unloads libmoshi.so (after every context has been destroyed), so that
    its HIP module teardown runs now, while the GPU runtime is fully alive,
    rather than among the process's exit handlers."""
    global _lib
    if _lib is None:
        return
    alive = [c for c in _live_ctx if c.h]
    if alive:
        raise RuntimeError(f"{len(alive)} moshi context(s) still alive: destroy them first")
    import _ctypes
    h = _lib._handle
    _lib = None
    _ctypes.dlclose(h)


def _p(a):
    return None if a is None else a.ctypes.data


def _check(status, ctx=None):
    if status < 0:
        msg = ""
        if ctx is not None:
            msg = lib().moshi_last_error(ctx.h).decode()
        raise MoshiError(status, msg)
    return status


def make_config(dim, n_layers, n_heads, ffn_hidden, window, dep_dim, dep_layers, dep_heads,
                dep_ffn_hidden, n_substeps, text_vocab, audio_card, rope_theta=1e4,
                norm_eps=1e-8, dtype="bf16", max_sessions=1, flags=0, dep_q=0) -> moshi_config:
    c = moshi_config()
    c.dim, c.n_layers, c.n_heads, c.ffn_hidden, c.window = dim, n_layers, n_heads, ffn_hidden, window
    c.dep_dim, c.dep_layers, c.dep_heads = dep_dim, dep_layers, dep_heads
    c.dep_ffn_hidden, c.n_substeps = dep_ffn_hidden, n_substeps
    c.text_vocab, c.audio_card = text_vocab, audio_card
    c.rope_theta, c.norm_eps = rope_theta, norm_eps
    c.dtype = MOSHI_BF16 if dtype in ("bf16", MOSHI_BF16) else MOSHI_F32
    c.max_sessions, c.flags, c.dep_q = max_sessions, flags, dep_q
    return c


class Ctx:
    """Owning handle of a moshi_ctx (destroyed on moshi_destroy or GC)."""

    def __init__(self, h, cfg):
        self.h = h
        self.cfg = cfg
        self.B = cfg.max_sessions
        self.S = cfg.n_substeps
        self.D = cfg.dim
        self.esz = 2 if cfg.dtype == MOSHI_BF16 else 4

    def __del__(self):
        if getattr(self, "h", None) and _lib is not None:
            _lib.moshi_destroy(self.h)
            self.h = None


def moshi_strerror(status) -> str:
    return lib().moshi_strerror(int(status)).decode()


def moshi_n_tensors(cfg) -> int:
    return int(lib().moshi_n_tensors(ctypes.byref(cfg)))


def moshi_create(cfg, tensors, hip_stream=None) -> Ctx:
    """tensors: host arrays in the weight-list order (uint16 bf16 bits or float32)."""
    arrs = [np.ascontiguousarray(t) for t in tensors]
    ptrs = (ctypes.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])
    out = ctypes.c_void_p()
    st = _check(lib().moshi_create(ctypes.byref(cfg), ptrs, len(arrs), hip_stream,
                                   ctypes.byref(out)))
    del st
    ctx = Ctx(out.value, cfg)
    _live_ctx.add(ctx)
    return ctx


def moshi_destroy(ctx: Ctx):
    if ctx.h:
        lib().moshi_destroy(ctx.h)
        ctx.h = None


def moshi_session_join(ctx: Ctx) -> int:
    slot = ctypes.c_int32()
    _check(lib().moshi_session_join(ctx.h, ctypes.byref(slot)), ctx)
    return slot.value


def moshi_session_leave(ctx: Ctx, slot: int):
    _check(lib().moshi_session_leave(ctx.h, int(slot)), ctx)


def moshi_session_set_sampling(ctx: Ctx, slot: int, text_temperature=0.0, text_top_k=0,
                               audio_temperature=0.0, audio_top_k=0, seed=0, greedy=False):
    """Temperature + top-k draws for one session (greedy=True: back to greedy)."""
    if greedy:
        _check(lib().moshi_session_set_sampling(ctx.h, int(slot), None), ctx)
        return
    p = moshi_sampling(float(text_temperature), int(text_top_k), float(audio_temperature),
                       int(audio_top_k), int(seed) & (2**64 - 1))
    _check(lib().moshi_session_set_sampling(ctx.h, int(slot), ctypes.byref(p)), ctx)


def moshi_step(ctx: Ctx, frames):
    """frames int32 [B, 1+S] -> (text_token [B], audio_codes [B, S]); -1 for free slots."""
    f = np.ascontiguousarray(frames, np.int32).reshape(ctx.B, ctx.S + 1)
    tok = np.empty(ctx.B, np.int32)
    codes = np.empty((ctx.B, ctx.S), np.int32)
    _check(lib().moshi_step(ctx.h, _p(f), _p(tok), _p(codes)), ctx)
    return tok, codes


def moshi_step_forced(ctx: Ctx, frames, forced=None):
    """frames int32 [B, 1+S]; forced int32 [B, 1+S] (-1 = not forced) or None
    -> (text_token [B], audio_codes [B, S])."""
    f = np.ascontiguousarray(frames, np.int32).reshape(ctx.B, ctx.S + 1)
    fc = None if forced is None else np.ascontiguousarray(forced, np.int32).reshape(ctx.B, ctx.S + 1)
    tok = np.empty(ctx.B, np.int32)
    codes = np.empty((ctx.B, ctx.S), np.int32)
    _check(lib().moshi_step_forced(ctx.h, _p(f), _p(fc), _p(tok), _p(codes)), ctx)
    return tok, codes


def moshi_test_set_spin_limit(ctx: Ctx, limit: int):
    _check(lib().moshi_test_set_spin_limit(ctx.h, int(limit)), ctx)


def moshi_step_enqueue(ctx: Ctx, d_frames: int, d_text_token: int = None,
                       d_audio_codes: int = None):
    """Device-resident step: the arguments are DEVICE addresses (ints), e.g.
    ``tensor.data_ptr()`` of int32 device tensors. Returns without waiting."""
    for p in (d_frames, d_text_token, d_audio_codes):
        if p is not None and not isinstance(p, int):
            raise TypeError("device addresses must be ints")
    _check(lib().moshi_step_enqueue(ctx.h, d_frames, d_text_token, d_audio_codes), ctx)


def moshi_step_enqueue_noalloc(ctx: Ctx, d_frames: int, d_text_token: int = None,
                               d_audio_codes: int = None):
    """moshi_step_enqueue whose kernel scratch is the library's static device
    array (allocates nothing); device addresses as ints."""
    for p in (d_frames, d_text_token, d_audio_codes):
        if p is not None and not isinstance(p, int):
            raise TypeError("device addresses must be ints")
    _check(lib().moshi_step_enqueue_noalloc(ctx.h, d_frames, d_text_token, d_audio_codes), ctx)


def moshi_sync(ctx: Ctx):
    _check(lib().moshi_sync(ctx.h), ctx)


def moshi_temporal_step(ctx: Ctx, frames):
    f = np.ascontiguousarray(frames, np.int32).reshape(ctx.B, ctx.S + 1)
    tok = np.empty(ctx.B, np.int32)
    _check(lib().moshi_temporal_step(ctx.h, _p(f), _p(tok)), ctx)
    return tok


def moshi_depformer_step(ctx: Ctx, hidden, text_in):
    """hidden [B, D] in the model dtype (uint16 bf16 bits or float32); text_in [B]."""
    dt = np.uint16 if ctx.esz == 2 else np.float32
    h = np.ascontiguousarray(hidden, dt).reshape(ctx.B, ctx.D)
    t = np.ascontiguousarray(text_in, np.int32).reshape(ctx.B)
    codes = np.empty((ctx.B, ctx.S), np.int32)
    _check(lib().moshi_depformer_step(ctx.h, _p(h), _p(t), _p(codes)), ctx)
    return codes


def moshi_session_prefill_kv(ctx: Ctx, slot: int, k, v):
    """k, v: [L][n][D] in the model dtype."""
    n = int(k.shape[1]) if k is not None and k.ndim == 3 else 0
    k = None if n == 0 else np.ascontiguousarray(k)
    v = None if n == 0 else np.ascontiguousarray(v)
    _check(lib().moshi_session_prefill_kv(ctx.h, int(slot), n, _p(k), _p(v)), ctx)


def moshi_session_prefill_frames(ctx: Ctx, slot: int, frames, want_logits=False):
    """frames int32 [n, 1+S] of one session -> (text_tokens [n], text_logits
    [n, Vt] or None); the temporal transformer over all n frames at once."""
    f = np.ascontiguousarray(frames, np.int32).reshape(-1, ctx.S + 1)
    n = f.shape[0]
    tok = np.empty(n, np.int32)
    tl = np.empty((n, ctx.cfg.text_vocab), np.float32) if want_logits else None
    _check(lib().moshi_session_prefill_frames(ctx.h, int(slot), n, _p(f), _p(tok), _p(tl)), ctx)
    return tok, tl


def moshi_session_read_kv(ctx: Ctx, slot: int):
    """The slot's ring: (k, v) [L][W][D] in the model dtype (ring-slot order)."""
    c = ctx.cfg
    dt = np.uint16 if ctx.esz == 2 else np.float32
    k = np.empty((c.n_layers, c.window, c.dim), dt)
    v = np.empty_like(k)
    _check(lib().moshi_session_read_kv(ctx.h, int(slot), _p(k), _p(v)), ctx)
    return k, v


def moshi_session_info(ctx: Ctx, slot: int):
    pos = np.zeros(1, np.int64)
    fill = np.zeros(1, np.int32)
    wi = np.zeros(1, np.int32)
    _check(lib().moshi_session_info(ctx.h, int(slot), _p(pos), _p(fill), _p(wi)), ctx)
    return int(pos[0]), int(fill[0]), int(wi[0])


def moshi_read_logits(ctx: Ctx, text=True, audio=True):
    c = ctx.cfg
    tl = np.empty((ctx.B, c.text_vocab), np.float32) if text else None
    al = np.empty((ctx.B, ctx.S, c.audio_card), np.float32) if audio else None
    _check(lib().moshi_read_logits(ctx.h, _p(tl), _p(al)), ctx)
    return tl, al


def moshi_read_hidden(ctx: Ctx):
    h = np.empty((ctx.B, ctx.D), np.float32)
    _check(lib().moshi_read_hidden(ctx.h, _p(h)), ctx)
    return h


def moshi_uses_step_kernel(ctx: Ctx) -> bool:
    """True when a step runs as one persistent kernel (see include/moshi.h)."""
    return _check(lib().moshi_uses_step_kernel(ctx.h), ctx) == 1


def moshi_uses_dep_kernel(ctx: Ctx) -> bool:
    """True if the depformer runs as one persistent kernel for all slots."""
    return _check(lib().moshi_uses_dep_kernel(ctx.h), ctx) == 1


def moshi_kernel_class_name(c: int) -> str:
    return lib().moshi_kernel_class_name(int(c)).decode()


def moshi_time_kernels(ctx: Ctx, frames, n_steps: int, n_classes: int = 32):
    """Per-kernel-class device time (ms), launch count and algorithmic bytes over
    n_steps eager steps bracketed by HIP events."""
    f = np.ascontiguousarray(frames, np.int32).reshape(ctx.B, ctx.S + 1)
    ms = np.zeros(n_classes, np.float64)
    nl = np.zeros(n_classes, np.int64)
    by = np.zeros(n_classes, np.float64)
    n = _check(lib().moshi_time_kernels(ctx.h, _p(f), int(n_steps), _p(ms), _p(nl), _p(by),
                                        n_classes), ctx)
    return {moshi_kernel_class_name(i): {"ms": float(ms[i]), "launches": int(nl[i]),
                                         "bytes": float(by[i])} for i in range(min(n, n_classes))}


def moshi_last_error(ctx: Ctx) -> str:
    return lib().moshi_last_error(ctx.h).decode()


class Stream:
    """Owning handle of a moshi_stream (the delayed-stream wrapper)."""

    def __init__(self, h, ctx, n_agent):
        self.h = h
        self.ctx = ctx
        self.A = n_agent

    def __del__(self):
        if getattr(self, "h", None) and _lib is not None:
            _lib.moshi_stream_destroy(self.h)
            self.h = None


def _check_stream(status, st):
    if status < 0:
        raise MoshiError(status, lib().moshi_stream_last_error(st.h).decode())
    return status


def moshi_get_config(ctx: Ctx) -> moshi_config:
    c = moshi_config()
    _check(lib().moshi_get_config(ctx.h, ctypes.byref(c)), ctx)
    return c


def moshi_stream_create(ctx: Ctx, n_agent: int, delays=None) -> Stream:
    d = None if delays is None else np.ascontiguousarray(delays, np.int32)
    out = ctypes.c_void_p()
    _check(lib().moshi_stream_create(ctx.h, int(n_agent), _p(d), ctypes.byref(out)), ctx)
    return Stream(out.value, ctx, n_agent)


def moshi_stream_destroy(st: Stream):
    if st.h:
        lib().moshi_stream_destroy(st.h)
        st.h = None


def moshi_stream_reset(st: Stream, slot: int):
    _check_stream(lib().moshi_stream_reset(st.h, int(slot)), st)


def moshi_stream_step(st: Stream, user, forced=None):
    """user int32 [B, S-A]; forced int32 [B, 1+A] or None -> (frames [B, 1+A],
    ready [B], step_text [B], step_codes [B, S])."""
    B, S, A = st.ctx.B, st.ctx.S, st.A
    u = np.ascontiguousarray(user, np.int32).reshape(B, S - A)
    f = None if forced is None else np.ascontiguousarray(forced, np.int32).reshape(B, 1 + A)
    fr = np.empty((B, 1 + A), np.int32)
    ready = np.empty(B, np.int32)
    tt = np.empty(B, np.int32)
    tc = np.empty((B, S), np.int32)
    _check_stream(lib().moshi_stream_step(st.h, _p(u), _p(f), _p(fr), _p(ready), _p(tt), _p(tc)), st)
    return fr, ready, tt, tc
