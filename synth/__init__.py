"""Seeded synthetic inputs for the Moshi frame step.

This package draws numbers and lays them out; it holds none of the model's
arithmetic. The CPU oracle (``oracle/``) and the HIP library
(``full_duplex_speech_amd``) both read the host arrays built here, and neither
imports the other.

* ``synth.spec``      -- the model shapes and the ordered weight-tensor list
                         (the layout contract of the weight pointer array).
* ``synth.workloads`` -- the five named workloads (weights seed, frames,
                         prefill K/V, session churn).
* ``synth.rng``       -- ctypes front end of ``synth.c`` (counter-based
                         splitmix64 + Box-Muller draws).
"""
from . import rng, spec, workloads  # noqa: F401
