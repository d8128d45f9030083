"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case copies oracle/kda_oracle.c, plants one plausible slip (a dropped
term, a wrong sign, a transposed state, read-out before the update, beta or
the gate in the wrong place, a wrong sequence offset, ...), builds the copy
with gcc into a temporary library and runs every pin of tests/test_oracle.py
against it.  At least one pin has to fail for every planted slip; the
unmodified source has to pass them all.
"""
import ctypes
import os
import subprocess
import tempfile

import pytest

import oracle
from tests import test_oracle as pins

SRC = open(os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")).read()

READOUT = """    /* read-out o = S^T qn */
    double* ot = out + row * V;
    for (int64_t j = 0; j < V; ++j) ot[j] = 0.0;
    for (int64_t i = 0; i < K; ++i)
      for (int64_t j = 0; j < V; ++j) ot[j] += S[i * V + j] * qn[i];
"""
DECAY = "    /* decay: S <- diag(exp(a)) S */\n"


def _readout_first(s):
    assert s.count(READOUT) == 1 and s.count(DECAY) == 1
    s = s.replace(READOUT, "")
    return s.replace(DECAY, READOUT + DECAY)


MUTANTS = {
    "correction_sign": [("S[i * V + j] += c * r[j]", "S[i * V + j] -= c * r[j]")],
    "residual_drops_state": [("r[j] -= S[i * V + j] * kn[i]", "r[j] -= 0.0 * kn[i]")],
    "beta_on_output": [("const double c = bt * kn[i];", "const double c = kn[i];"),
                       ("ot[j] += S[i * V + j] * qn[i];", "ot[j] += bt * S[i * V + j] * qn[i];")],
    "state_store_transposed": [("s_out[j * K + i] = S[i * V + j]", "s_out[i * V + j] = S[i * V + j]")],
    "state_load_transposed": [("s_in[j * K + i]", "s_in[i * V + j]")],
    "dt_bias_sign": [("(g + dt_bias)", "(g - dt_bias)")],
    "A_log_not_exponentiated": [("exp(A_log) * (g + dt_bias)", "A_log * (g + dt_bias)")],
    "gate_sign": [("return lower_bound * sigmoid(", "return -0.1 * lower_bound * sigmoid(")],
    "gate_on_value_axis": [("const double d = exp(a[i]);\n      for (int64_t j = 0; j < V; ++j) S[i * V + j] *= d;",
                            "for (int64_t j = 0; j < V; ++j) S[i * V + j] *= exp(a[j]);")],
    "no_key_norm": [("const double rk = 1.0 / sqrt(sk + KDA_ORACLE_EPS);", "const double rk = 1.0;")],
    "no_scale": [("const double rq = scale / sqrt(", "const double rq = 1.0 / sqrt(")],
    "no_beta_sigmoid": [("const double bt = sigmoid(bf16_to_f64(beta[row]));",
                         "const double bt = bf16_to_f64(beta[row]);")],
    "varlen_start_offset": [("const int64_t t0 = cu_seqlens ? cu_seqlens[n] : 0;",
                             "const int64_t t0 = cu_seqlens ? (n > 0 ? cu_seqlens[n] - 1 : 0) : 0;")],
    "bf16_decode_shift": [("(uint32_t)b << 16", "(uint32_t)b << 15")],
    "readout_before_update": _readout_first,
}

PINS = [getattr(pins, n) for n in dir(pins) if n.startswith("test_") and callable(getattr(pins, n))]
PARAM_PINS = {"test_oracle_matches_chunked_form"}


def _run_pins(lib):
    """Number of pins that fail with `lib` swapped in as the oracle library."""
    saved = oracle._lib
    oracle._lib = lib
    failed = 0
    try:
        for fn in PINS:
            cases = [()]
            if fn.__name__ in PARAM_PINS:
                mark = [m for m in fn.pytestmark if m.name == "parametrize"][0]
                cases = mark.args[1]
            for args in cases:
                try:
                    fn(*args)
                except (AssertionError, ValueError, FloatingPointError):
                    failed += 1
    finally:
        oracle._lib = saved
    return failed


def _build(src, tmp):
    c = os.path.join(tmp, "m.c")
    so = os.path.join(tmp, "m.so")
    open(c, "w").write(src)
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", c, "-o", so, "-lm"], check=True)
    lib = ctypes.CDLL(so)
    ref = oracle._load()
    lib.kda_oracle_fwd.argtypes = ref.kda_oracle_fwd.argtypes
    lib.kda_oracle_fwd.restype = ctypes.c_int
    lib.kda_oracle_max_threads.restype = ctypes.c_int
    return lib


def test_unmodified_source_passes_all_pins():
    with tempfile.TemporaryDirectory() as tmp:
        assert _run_pins(_build(SRC, tmp)) == 0


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    m = MUTANTS[name]
    if callable(m):
        src = m(SRC)
    else:
        src = SRC
        for old, new in m:
            assert src.count(old) == 1, (name, old)
            src = src.replace(old, new)
    with tempfile.TemporaryDirectory() as tmp:
        assert _run_pins(_build(src, tmp)) > 0, name
