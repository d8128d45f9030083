"""Seeded random sweep of the forward's arguments against the fp64 oracle:
sequence lengths (zero-length and ragged ones included), head counts, state
dtypes, lower bounds, gate scales, and every path / chunk size / part count,
all small enough that the oracle checks every element."""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_prep_amd.inputs import make_inputs
from tests.kda_gpu import assert_close, run_gpu, say, to_f64

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

N_CASES = 120


def draw(i):
    rng = np.random.default_rng(5000 + i)
    H = int(rng.choice([1, 2, 3, 5, 8]))
    if rng.random() < 0.5:   # B sequences of T tokens
        B, T, lens = int(rng.integers(1, 4)), int(rng.integers(0, 200)), None
    else:                    # one batch of ragged sequences through cu_seqlens
        n = int(rng.integers(1, 7))
        lens = [int(x) for x in rng.choice([0, 1, 15, 16, 17, 31, 32, 33, int(rng.integers(1, 150))], size=n)]
        B, T = 1, sum(lens)
    state = str(rng.choice(["bf16", "fp32", "none"]))
    form = str(rng.choice(["auto", "split16", "fused16", "split32", "parts"]))
    lb = float(rng.choice([-5.0, -3.0, -1.0, 0.0]))
    g_std = float(rng.choice([0.5, 1.0, 2.0]))
    return dict(B=B, T=T, H=H, lens=lens, state=state, form=form, lb=lb, g_std=g_std, seed=6000 + i)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    c = draw(i)
    say("case random%d %s" % (i, c))
    inp = make_inputs(c["B"], c["T"], c["H"], seed=c["seed"], lower_bound=c["lb"], g_std=c["g_std"],
                      state_dtype=None if c["state"] == "none" else c["state"],
                      initial_state=c["state"] != "none", seq_lens=c["lens"])
    kw = dict(auto={}, split16=dict(path="split", chunk=16), fused16=dict(path="fused", chunk=16),
              split32=dict(path="split", chunk=32), parts=dict(path="split", chunk=16, parts=3))[c["form"]]
    out, fin = run_gpu(inp, **kw)
    torch.cuda.synchronize()
    ref_o, ref_f = oracle.kda_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, inp.A_log, inp.dt_bias,
                                  inp.lower_bound, initial_state=inp.initial_state_f64(),
                                  output_final_state=inp.output_final_state, cu_seqlens=inp.cu_seqlens)
    if inp.B * inp.T > 0:
        assert_close(to_f64(out), ref_o, "out")
    if inp.output_final_state:
        assert_close(to_f64(fin), ref_f, "final_state", inp.state_dtype)


# Shapes where the workgroups' waves meet through LDS flags: the recurrence's
# 64-column tiles with a CU each (65 .. 128 pairs), its 128-column tiles (more
# than 128 pairs of equal length), and the fused kernel at both tile widths.
N_FLAG_CASES = 48


def draw_flag(i):
    rng = np.random.default_rng(7000 + i)
    kind = int(rng.integers(0, 3))
    if kind == 0:
        N = int(rng.integers(1, 5))
        H = int(rng.integers(max(17, 65 // N), 128 // N + 1))
        lens = [int(x) for x in rng.integers(0, 120, size=N)]
        if sum(lens) == 0:
            lens[0] = 5
        B, T = 1, sum(lens)
    elif kind == 1:
        B = int(rng.integers(2, 5))
        H = int(rng.integers(129 // B + 1, 129 // B + 30))
        T, lens = int(rng.integers(1, 100)), None
    else:
        N = int(rng.integers(1, 6))
        H = int(rng.integers(8, 70))
        lens = [int(x) for x in rng.integers(1, 90, size=N)]
        B, T = 1, sum(lens)
    path = ("split", "split", "fused")[kind] if rng.random() < 0.8 else None
    state = str(rng.choice(["bf16", "fp32", "none"]))
    lb = float(rng.choice([-5.0, -2.0, 0.0]))
    return dict(B=B, T=T, H=H, lens=lens, path=path, state=state, lb=lb, seed=8000 + i)


@pytest.mark.parametrize("i", range(N_FLAG_CASES))
def test_random_flag_case(i):
    c = draw_flag(i)
    say("case flag%d %s" % (i, c))
    inp = make_inputs(c["B"], c["T"], c["H"], seed=c["seed"], lower_bound=c["lb"],
                      state_dtype=None if c["state"] == "none" else c["state"],
                      initial_state=c["state"] != "none", seq_lens=c["lens"])
    out, fin = run_gpu(inp, path=c["path"], chunk=16 if c["path"] else None)
    torch.cuda.synchronize()
    ref_o, ref_f = oracle.kda_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, inp.A_log, inp.dt_bias,
                                  inp.lower_bound, initial_state=inp.initial_state_f64(),
                                  output_final_state=inp.output_final_state, cu_seqlens=inp.cu_seqlens)
    if inp.B * inp.T > 0:
        assert_close(to_f64(out), ref_o, "out")
    if inp.output_final_state:
        assert_close(to_f64(fin), ref_f, "final_state", inp.state_dtype)


# 64-token chunks (split path, one or more parts): lengths around the chunk and
# its 16- and 32-token blocks, so partial chunks end inside every block.
N_C64_CASES = 32


def draw_c64(i):
    rng = np.random.default_rng(9000 + i)
    H = int(rng.choice([1, 2, 3, 4, 6]))
    if rng.random() < 0.4:
        B, T, lens = int(rng.integers(1, 4)), int(rng.integers(0, 300)), None
    else:
        n = int(rng.integers(1, 7))
        lens = [int(x) for x in rng.choice([0, 1, 16, 17, 31, 32, 33, 48, 63, 64, 65, 127, 128, 129,
                                            int(rng.integers(1, 260))], size=n)]
        B, T = 1, sum(lens)
    state = str(rng.choice(["bf16", "fp32", "none"]))
    parts = int(rng.choice([1, 1, 1, 2, 3]))
    lb = float(rng.choice([-5.0, -3.0, -1.0, 0.0]))
    g_std = float(rng.choice([0.5, 1.0, 2.0]))
    return dict(B=B, T=T, H=H, lens=lens, state=state, parts=parts, lb=lb, g_std=g_std, seed=10000 + i)


@pytest.mark.parametrize("i", range(N_C64_CASES))
def test_random_chunk64_case(i):
    c = draw_c64(i)
    say("case c64-%d %s" % (i, c))
    inp = make_inputs(c["B"], c["T"], c["H"], seed=c["seed"], lower_bound=c["lb"], g_std=c["g_std"],
                      state_dtype=None if c["state"] == "none" else c["state"],
                      initial_state=c["state"] != "none", seq_lens=c["lens"])
    out, fin = run_gpu(inp, path="split", chunk=64, parts=c["parts"])
    torch.cuda.synchronize()
    ref_o, ref_f = oracle.kda_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, inp.A_log, inp.dt_bias,
                                  inp.lower_bound, initial_state=inp.initial_state_f64(),
                                  output_final_state=inp.output_final_state, cu_seqlens=inp.cu_seqlens)
    if inp.B * inp.T > 0:
        assert_close(to_f64(out), ref_o, "out")
    if inp.output_final_state:
        assert_close(to_f64(fin), ref_f, "final_state", inp.state_dtype)
