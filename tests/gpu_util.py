"""Shared helpers of the GPU parity tests (HIP library vs the fp64 oracle).

Compare rule (teacher-forced): the oracle runs every frame with the GPU's own
text token and codes as the next-substep inputs, so every head is compared
even after a legitimate low-margin flip.
* logits: max |gpu - oracle| <= 2e-2 (bf16 model) or 1e-4 (fp32 model);
* tokens and codes: equal wherever the oracle's top-2 margin exceeds
  min(1e-2, 2 * logit tolerance) -- past that margin no logit error within the
  tolerance can reorder the top two;
* ring bookkeeping (pos, fill, write index): always equal.
"""
import sys

import numpy as np

import full_duplex_speech_amd as M
import oracle
from synth import spec, workloads as wl


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def cfg_of(shape: spec.ModelShape, B: int):
    flags = (M.MOSHI_FLAG_MASK_OLDEST if shape.mask_oldest else 0) | \
        (M.MOSHI_FLAG_DEP_FINAL_NORM if shape.dep_final_norm else 0) | \
        (M.MOSHI_FLAG_DEP_REF_RING if shape.dep_ref_ring else 0)
    return M.make_config(dim=shape.dim, n_layers=shape.n_layers, n_heads=shape.n_heads,
                         ffn_hidden=shape.ffn, window=shape.window, dep_dim=shape.dep_dim,
                         dep_layers=shape.dep_layers, dep_heads=shape.dep_heads,
                         dep_ffn_hidden=shape.dep_ffn, n_substeps=shape.n_substeps,
                         text_vocab=shape.text_vocab, audio_card=shape.audio_card,
                         rope_theta=shape.rope_theta, norm_eps=shape.norm_eps,
                         dtype=shape.dtype, max_sessions=B, flags=flags, dep_q=shape.dep_q)


def tolerances(shape):
    tol = 2e-2 if shape.dtype == "bf16" else 1e-4
    return tol, min(1e-2, 2 * tol)


class Stats:
    def __init__(self):
        self.heads = 0
        self.excused = 0
        self.max_text_err = 0.0
        self.max_audio_err = 0.0

    def __repr__(self):
        return (f"heads={self.heads} excused={self.excused} "
                f"max_text_err={self.max_text_err:.3g} max_audio_err={self.max_audio_err:.3g}")


def compare_frame(shape, stats, tag, gpu_tok, gpu_codes, gpu_tl, gpu_al, orc):
    """Check one session-frame of the GPU against the teacher-forced oracle."""
    tol, mtol = tolerances(shape)
    if gpu_tl is not None and orc.get("text_logits") is not None:
        e = float(np.max(np.abs(gpu_tl.astype(np.float64) - orc["text_logits"])))
        stats.max_text_err = max(stats.max_text_err, e)
        assert e <= tol, f"{tag}: text logits err {e:.3g} > {tol}"
    stats.heads += 1
    if orc["text_margin"] > mtol:
        assert gpu_tok == orc["text_token"], \
            f"{tag}: text token {gpu_tok} != oracle {orc['text_token']} (margin {orc['text_margin']:.3g})"
    else:
        stats.excused += 1
    if gpu_codes is None:
        return
    if gpu_al is not None and orc.get("audio_logits") is not None:
        e = float(np.max(np.abs(gpu_al.astype(np.float64) - orc["audio_logits"])))
        stats.max_audio_err = max(stats.max_audio_err, e)
        assert e <= tol, f"{tag}: audio logits err {e:.3g} > {tol}"
    for s in range(shape.n_substeps):
        stats.heads += 1
        if orc["audio_margins"][s] > mtol:
            assert gpu_codes[s] == orc["codes"][s], \
                f"{tag}: code {s}: {gpu_codes[s]} != oracle {orc['codes'][s]} " \
                f"(margin {orc['audio_margins'][s]:.3g})"
        else:
            stats.excused += 1


def new_engine(shape, weights, B):
    return M.moshi_create(cfg_of(shape, B), weights)


def frames_matrix(shape, B, rows):
    """[B, 17] int32 with `rows` {slot: frame}; other rows zero."""
    f = np.zeros((B, shape.n_channels), np.int32)
    for slot, fr in rows.items():
        f[slot] = fr
    return f


class DevBuf:
    """A device buffer from the HIP runtime libmoshi.so itself uses (loaded
    through ctypes), for tests of the device-resident entry points. (torch
    would bring up its own copy of the runtime, which cannot start once
    libmoshi's has.)"""
    _hip = None

    @classmethod
    def hip(cls):
        if cls._hip is None:
            import ctypes
            M.lib()  # the runtime libmoshi.so links against is loaded now
            h = ctypes.CDLL("libamdhip64.so.7")
            h.hipMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t]
            h.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
            h.hipFree.argtypes = [ctypes.c_void_p]
            cls._hip = h
        return cls._hip

    def __init__(self, host: np.ndarray):
        import ctypes
        self.shape, self.dtype = host.shape, host.dtype
        self.nbytes = host.nbytes
        p = ctypes.c_void_p()
        assert self.hip().hipMalloc(ctypes.byref(p), self.nbytes) == 0, "hipMalloc failed"
        self.ptr = p.value
        self.write(host)

    def write(self, host):
        a = np.ascontiguousarray(host, self.dtype)
        assert self.hip().hipMemcpy(self.ptr, a.ctypes.data, self.nbytes, 1) == 0  # H2D

    def read(self):
        a = np.empty(self.shape, self.dtype)
        assert self.hip().hipMemcpy(a.ctypes.data, self.ptr, self.nbytes, 2) == 0  # D2H
        return a

    def __del__(self):
        if getattr(self, "ptr", None):
            self.hip().hipFree(self.ptr)
            self.ptr = None
