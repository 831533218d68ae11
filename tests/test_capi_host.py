"""Host-only checks of the C-ABI library (no GPU work): it loads, exports every
entry point the header declares, and rejects bad arguments before touching a
device."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

import full_duplex_speech_amd as M
from synth import spec

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moshi.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moshi_[a-z_]+)\s*\(", text)))


def _lib():
    if not os.path.exists(M.LIB_PATH):
        pytest.skip("libmoshi.so not built")
    return M.lib()


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("moshi_create", "moshi_destroy", "moshi_session_join", "moshi_session_leave",
              "moshi_step"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = _lib()
    missing = [n for n in _declared() if not hasattr(L, n)]
    assert not missing, missing
    out = subprocess.run(["nm", "-D", "--defined-only", M.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r"\bT (moshi_[a-z_]+)", out))
    assert set(_declared()) <= exported


def _cfg(shape=spec.PERSONAPLEX, B=1, **kw):
    from gpu_util import cfg_of
    c = cfg_of(shape, B)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_n_tensors_matches_the_weight_list():
    _lib()
    for shape in (spec.PERSONAPLEX, spec.TINY, spec.RAGGED):
        assert M.moshi_n_tensors(_cfg(shape)) == spec.n_tensors(shape)


@pytest.mark.parametrize("field,value", [
    ("n_heads", 3), ("dim", 0), ("dep_heads", 5), ("window", 0), ("max_sessions", 0),
    ("max_sessions", 65), ("dtype", 7), ("ffn_hidden", 1001), ("text_vocab", 1), ("flags", 16),
    ("n_substeps", 0), ("n_layers", 0), ("rope_theta", 0.0), ("dep_q", 17), ("dep_q", -1),
])
def test_bad_configs_are_rejected(field, value):
    _lib()
    c = _cfg(**{field: value})
    assert M.moshi_n_tensors(c) == M.MOSHI_E_INVALID
    out = ctypes.c_void_p()
    ptrs = (ctypes.c_void_p * 1)()
    rc = M.lib().moshi_create(ctypes.byref(c), ptrs, 1, None, ctypes.byref(out))
    assert rc == M.MOSHI_E_INVALID and not out.value


def test_sampling_vocabulary_limit():
    _lib()
    c = _cfg(spec.PERSONAPLEX, flags=M.MOSHI_FLAG_SAMPLING)
    assert M.moshi_n_tensors(c) == spec.n_tensors(spec.PERSONAPLEX)
    c = _cfg(spec.PERSONAPLEX.replace(text_vocab=40000), flags=M.MOSHI_FLAG_SAMPLING)
    assert M.moshi_n_tensors(c) == M.MOSHI_E_INVALID


def test_null_and_count_errors_need_no_device():
    L = _lib()
    c = _cfg(spec.TINY)
    out = ctypes.c_void_p()
    assert L.moshi_create(ctypes.byref(c), None, 0, None, ctypes.byref(out)) == M.MOSHI_E_INVALID
    ptrs = (ctypes.c_void_p * 3)()
    assert L.moshi_create(ctypes.byref(c), ptrs, 3, None, ctypes.byref(out)) == M.MOSHI_E_INVALID
    assert L.moshi_create(ctypes.byref(c), ptrs, 3, None, None) == M.MOSHI_E_INVALID
    for fn, args in (("moshi_session_join", (None, None)), ("moshi_session_leave", (None, 0)),
                     ("moshi_step", (None, None, None, None)),
                     ("moshi_session_info", (None, 0, None, None, None))):
        assert getattr(L, fn)(*args) == M.MOSHI_E_INVALID
    assert L.moshi_destroy(None) == 0
    assert M.moshi_strerror(M.MOSHI_E_FULL) == "all session slots are taken"


def test_create_without_a_gpu_reports_device_error():
    """On a machine with no GPU a valid config fails cleanly with E_DEVICE."""
    _lib()
    code = (
        "import sys; sys.path.insert(0, %r); sys.path.insert(0, %r)\n"
        "import numpy as np, full_duplex_speech_amd as M\n"
        "from synth import spec, workloads as wl\n"
        "from gpu_util import cfg_of\n"
        "import ctypes\n"
        "s = spec.RAGGED\n"
        "w = wl.make_weights(s, 1)\n"
        "try:\n"
        "    M.moshi_create(cfg_of(s, 1), w)\n"
        "    print('CREATED')\n"
        "except M.MoshiError as e:\n"
        "    print('STATUS', e.status)\n" % (ROOT, os.path.join(ROOT, "tests")))
    env = dict(os.environ)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120,
                       env=env)
    if "CREATED" in r.stdout:
        pytest.skip("a GPU is present")
    assert "STATUS -4" in r.stdout, r.stdout + r.stderr
