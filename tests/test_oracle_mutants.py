"""Planted mistakes in the oracle must fail at least one pin (CPU only).

Each mutant is a textual edit of ``oracle/kda_oracle.c`` (a plausible slip in
reading or coding the recurrence), compiled into a temporary library that
replaces the oracle's for the duration of one run of the pin tests.  Every
mutant keeps all memory accesses in bounds.
"""
import ctypes
import inspect
import os
import subprocess
import tempfile

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")

DECAY = "for (long j = 0; j < w; ++j) S[i * w + j] *= a[i];"
WRITE = "for (long j = 0; j < w; ++j) S[i * w + j] += bt * kt[i] * e[j];"
ERR_INIT = "for (long j = 0; j < w; ++j) e[j] = vt[j0 + j];"

MUTANTS = {
    # forget gate applied after the delta write instead of before it
    "decay_after_write": [(DECAY, ""),
                          (WRITE, WRITE + "\n            for (long i2 = 0; i2 < dk; ++i2)"
                                  " for (long j = 0; j < w; ++j) S[i2 * w + j] *= a[i2];")],
    # the error is measured on the undecayed state
    "error_on_undecayed_state": [(DECAY, ""),
                                 ("/* delta write: S = S' + beta_t k_t e^T */",
                                  "for (long i2 = 0; i2 < dk; ++i2) for (long j = 0; j < w; ++j)"
                                  " S[i2 * w + j] *= a[i2];")],
    # output read before the write
    "read_before_write": [("/* delta write: S = S' + beta_t k_t e^T */",
                           "double *ot0 = o + tok * dv; for (long j = 0; j < w; ++j) {"
                           " double acc = 0.0; for (long i = 0; i < dk; ++i)"
                           " acc += S[i * w + j] * qt[i]; ot0[j0 + j] = acc; }"),
                          ("ot[j0 + j] = acc;", "(void)acc; (void)ot;")],
    # sign of the error flipped
    "error_sign": [("e[j] -= S[i * w + j] * kt[i];", "e[j] += S[i * w + j] * kt[i];")],
    # beta applied twice
    "beta_squared": [("+= bt * kt[i] * e[j];", "+= bt * bt * kt[i] * e[j];")],
    # value term dropped from the error
    "error_without_value": [(ERR_INIT, "for (long j = 0; j < w; ++j) e[j] = 0.0;")],
    # decay not exponentiated (uses alpha = 1 + log alpha)
    "linear_gate": [("a[i] = exp(clamp_log_alpha(lat[i]));",
                     "a[i] = 1.0 + clamp_log_alpha(lat[i]);")],
    # lower clamp missing
    "no_lower_clamp": [("if (x < KDA_ORACLE_LOG_ALPHA_MIN) return KDA_ORACLE_LOG_ALPHA_MIN;",
                        "")],
    # upper clamp missing
    "no_upper_clamp": [("if (x > KDA_ORACLE_LOG_ALPHA_MAX) return KDA_ORACLE_LOG_ALPHA_MAX;",
                        "")],
    # gate applied along the value axis (index wrapped to stay in bounds)
    "gate_on_value_axis": [(DECAY, "for (long j = 0; j < w; ++j) S[i * w + j] *= a[(j0 + j) % dk];")],
    # query and key swapped in the read
    "read_with_key": [("acc += S[i * w + j] * qt[i];", "acc += S[i * w + j] * kt[i];")],
    # token rows indexed as [B, H, T] instead of [B, T, H]
    "token_layout": [("const long tok = (b * T + t) * H + h;",
                      "const long tok = (b * H + h) * T + t;")],
}


def _pin_functions():
    out = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_") or name == "test_pages_decay_constants":
            continue
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        if params:
            argnames, values = params[0].args[0], params[0].args[1]
            argnames = [a.strip() for a in argnames.split(",")] if isinstance(argnames, str) else argnames
            for val in values:
                val = val if isinstance(val, tuple) else (val,)
                out.append((name, fn, dict(zip(argnames, val))))
        else:
            out.append((name, fn, {}))
    return out


def _build_mutant(edits, tmpdir, tag):
    src = open(SRC).read()
    for old, new in edits:
        assert old in src, f"mutant {tag}: pattern not found: {old!r}"
        src = src.replace(old, new)
    cpath = os.path.join(tmpdir, f"{tag}.c")
    lpath = os.path.join(tmpdir, f"lib{tag}.so")
    with open(cpath, "w") as f:
        f.write(src)
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-w",
                           "-o", lpath, cpath, "-lm"])
    return lpath


def test_unmodified_source_passes_all_pins():
    oracle._load()
    for name, fn, kw in _pin_functions():
        fn(**kw)


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_mutant_is_caught(mutant, monkeypatch):
    real = oracle._load()
    with tempfile.TemporaryDirectory() as td:
        lib = ctypes.CDLL(_build_mutant(MUTANTS[mutant], td, mutant))
        lib.kda_oracle_prefill.argtypes = real.kda_oracle_prefill.argtypes
        lib.kda_oracle_prefill.restype = ctypes.c_int
        monkeypatch.setattr(oracle, "_lib", lib)
        caught = []
        for name, fn, kw in _pin_functions():
            try:
                fn(**kw)
            except AssertionError:
                caught.append(name)
        monkeypatch.setattr(oracle, "_lib", real)
    assert caught, f"no pin catches the mutant {mutant}"
