"""The stored expected values under tests/golden/ (written by
tests/golden/make_golden.py from the fp64 oracle) against the oracle as it
stands and, for the K = V = 128 case, against the HIP path.

They pin the oracle and the seeded generator against unnoticed change: a
change to either that moves these numbers must come with regenerated files
and a reason."""
import json
import os

import numpy as np
import pytest

import oracle
from gated_delta_rule_prep_amd.inputs import make_inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def hexbits(xs, shape):
    return np.array([int(x, 16) for x in xs], dtype=np.uint16).reshape(shape)


def test_tiny_worked_example_reproduces():
    d = load("kda_tiny_K4V4.json")
    s = d["shape"]
    B, T, H, K, V, N = s["B"], s["T"], s["H"], s["K"], s["V"], s["N"]
    q, k, g = (hexbits(d[n], (B, T, H, K)) for n in ("q", "k", "g"))
    v = hexbits(d["v"], (B, T, H, V))
    beta = hexbits(d["beta"], (B, T, H))
    A_log = np.array(d["A_log"], dtype=np.float32)
    dt_bias = np.array(d["dt_bias"], dtype=np.float32).reshape(H, K)
    s0 = np.array(d["initial_state"], dtype=np.float64).reshape(N, H, V, K)
    cu = np.array(d["cu_seqlens"], dtype=np.int64)
    out, fin = oracle.kda_fwd(q, k, v, g, beta, d["scale"], A_log, dt_bias, d["lower_bound"], initial_state=s0,
                              cu_seqlens=cu)
    np.testing.assert_allclose(out.ravel(), d["out"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(fin.ravel(), d["final_state"], rtol=1e-12, atol=1e-14)
    # the seeded generator still draws the stored inputs
    inp = make_inputs(**d["args"])
    assert np.array_equal(inp.q, q) and np.array_equal(inp.k, k) and np.array_equal(inp.v, v)
    assert np.array_equal(inp.g, g) and np.array_equal(inp.beta, beta)
    assert np.array_equal(inp.A_log, A_log) and np.array_equal(inp.dt_bias, dt_bias)
    assert np.array_equal(inp.initial_state.astype(np.float64), s0)


def _small_oracle():
    d = load("kda_small_K128.json")
    inp = make_inputs(**d["args"])
    out, fin = oracle.kda_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, inp.A_log, inp.dt_bias,
                              inp.lower_bound, initial_state=inp.initial_state_f64(),
                              cu_seqlens=inp.cu_seqlens)
    return d, inp, out, fin


def test_small_case_reproduces():
    d, _, out, fin = _small_oracle()
    assert list(out.shape) == d["out_shape"] and list(fin.shape) == d["final_state_shape"]
    np.testing.assert_allclose(out.ravel()[d["out_index"]], d["out_value"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(fin.ravel()[d["final_index"]], d["final_value"], rtol=1e-12, atol=1e-14)
    for y, sm in ((out, d["out_summary"]), (fin, d["final_summary"])):
        assert np.sqrt(np.mean(y * y)) == pytest.approx(sm["rms"], rel=1e-12)
        assert y.sum() == pytest.approx(sm["sum"], rel=1e-10, abs=1e-10)
        assert (y * y).sum() == pytest.approx(sm["sumsq"], rel=1e-12)


def _check_samples(x, idx, vals, rms, what, dtype_ulp):
    x = x.ravel()[idx]
    y = np.asarray(vals, dtype=np.float64)
    # the parity bound of the GPU tests, per sampled element: 2e-2 of the
    # tensor's RMS plus half an ulp of the stored type
    bound = 2e-2 * rms + 0.5 * dtype_ulp(y)
    bad = np.abs(x - y) > bound
    assert not bad.any(), "%s: %d of %d samples off, worst |x - y| / RMS = %.3g" % (
        what, bad.sum(), len(y), float(np.max(np.abs(x - y)) / rms))


@pytest.mark.gpu
@pytest.mark.parametrize("path", ["split", "fused", None])
def test_small_case_on_the_gpu(path):
    from tests.kda_gpu import run_gpu, say, to_f64
    d = load("kda_small_K128.json")
    inp = make_inputs(**d["args"])
    say("case golden small K128 path=%s" % path)
    out, fin = run_gpu(inp, path=path)

    def bf16_ulp(y):
        e = np.floor(np.log2(np.maximum(np.abs(y), 1e-30)))
        return np.exp2(e - 7)

    _check_samples(to_f64(out), d["out_index"], d["out_value"], d["out_summary"]["rms"], "out", bf16_ulp)
    _check_samples(to_f64(fin), d["final_index"], d["final_value"], d["final_summary"]["rms"], "final_state",
                   bf16_ulp)
