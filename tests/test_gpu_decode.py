"""GPU parity of the single-token step (kda_decode) against the fp64 oracle:
one token per sequence is the oracle's recurrence with B = N, T = 1.  Also
checked: the step equals kda_fwd on the same one-token batch within the same
tolerance, in-place state update, no states, and repeated steps chained
through the state against the oracle run over all the steps at once."""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_prep_amd.inputs import make_inputs
from tests.kda_gpu import assert_close, bf16_tensor, device_inputs, run_gpu, say, state_torch_dtype, to_f64

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def oracle_run(inp, heads=None):
    hs = list(range(inp.H)) if heads is None else heads
    sl = lambda x: np.ascontiguousarray(x[:, :, hs])
    s0 = inp.initial_state_f64()
    return oracle.kda_fwd(sl(inp.q), sl(inp.k), sl(inp.v), sl(inp.g), sl(inp.beta), inp.scale,
                          inp.A_log[hs].copy(), inp.dt_bias[hs].copy(), inp.lower_bound,
                          initial_state=None if s0 is None else np.ascontiguousarray(s0[:, hs]),
                          output_final_state=True)


def run_decode(inp, d=None, inplace=False):
    from gated_delta_rule_prep_amd import kda
    d = d or device_inputs(inp)
    N, H = inp.B, inp.H
    out = torch.full((N, 1, H, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    fin = None
    if inp.output_final_state:
        fin = d["initial_state"] if inplace else torch.full((N, H, 128, 128), float("nan"),
                                                            dtype=state_torch_dtype(inp), device="cuda")
    kda.decode(d["q"], d["k"], d["v"], d["g"], d["beta"], inp.scale, out, d["A_log"], d["dt_bias"],
               inp.lower_bound, initial_state=d["initial_state"], final_state=fin)
    return out, fin


CASES = [
    dict(B=1, T=1, H=1, state_dtype="fp32", seed=500),
    dict(B=7, T=1, H=3, state_dtype="bf16", seed=501),
    dict(B=33, T=1, H=4, state_dtype="fp32", seed=502, lower_bound=-0.5, g_std=2.0),
    dict(B=5, T=1, H=2, state_dtype="fp32", initial_state=False, seed=503),
    dict(B=4, T=1, H=2, state_dtype=None, seed=504),
    dict(B=16, T=1, H=96, state_dtype="bf16", seed=505),
]


@pytest.mark.parametrize("i", range(len(CASES)))
def test_decode_parity(i):
    inp = make_inputs(**CASES[i])
    say("case decode%d N=%d H=%d state=%s" % (i, inp.B, inp.H, inp.state_dtype))
    out, fin = run_decode(inp)
    torch.cuda.synchronize()
    ref_o, ref_f = oracle_run(inp)
    assert_close(to_f64(out), ref_o, "out")
    if inp.output_final_state:
        assert_close(to_f64(fin), ref_f, "final_state", inp.state_dtype)


def test_decode_inplace_and_matches_chunked_path():
    inp = make_inputs(12, 1, 3, seed=506, state_dtype="fp32")
    say("case decode in-place vs kda_fwd")
    d = device_inputs(inp)
    o_c, f_c = run_gpu(inp, d=d)              # the chunked path on the same one-token batch
    s0 = d["initial_state"].clone()
    out, fin = run_decode(inp, d=d, inplace=True)
    torch.cuda.synchronize()
    assert fin.data_ptr() == d["initial_state"].data_ptr()
    assert not torch.equal(fin, s0)
    ref_o, ref_f = oracle_run(inp)
    assert_close(to_f64(out), ref_o, "out")
    assert_close(to_f64(fin), ref_f, "final_state", "fp32")
    assert_close(to_f64(o_c), ref_o, "out(chunked)")


def test_decode_steps_chain_like_one_sequence():
    """Ten decode steps, the state fed back each time, equal the oracle over
    the ten tokens as one sequence per batch row."""
    from gated_delta_rule_prep_amd import kda
    T, N, H = 10, 6, 2
    inp = make_inputs(N, T, H, seed=507, state_dtype="fp32")
    say("case decode chain T=%d N=%d H=%d" % (T, N, H))
    d = device_inputs(inp)
    st = d["initial_state"].clone()
    outs = []
    for t in range(T):
        tok = lambda x: x[:, t:t + 1].contiguous()
        o = torch.empty((N, 1, H, 128), dtype=torch.bfloat16, device="cuda")
        kda.decode(tok(d["q"]), tok(d["k"]), tok(d["v"]), tok(d["g"]), tok(d["beta"]), inp.scale, o, d["A_log"],
                   d["dt_bias"], inp.lower_bound, initial_state=st, final_state=st)
        outs.append(o)
    torch.cuda.synchronize()
    ref_o, ref_f = oracle_run(inp)
    assert_close(np.concatenate([to_f64(o) for o in outs], axis=1), ref_o, "out(chain)")
    assert_close(to_f64(st), ref_f, "final(chain)", "fp32")


def test_decode_large_batch_sampled_heads():
    """N = 256 sequences, H = 96 (a serving batch); the oracle on 4 heads."""
    inp = make_inputs(256, 1, 96, seed=508, state_dtype="bf16")
    say("case decode N=256 H=96")
    out, fin = run_decode(inp)
    torch.cuda.synchronize()
    hs = [0, 1, 47, 95]
    ref_o, ref_f = oracle_run(inp, hs)
    assert_close(to_f64(out)[:, :, hs], ref_o, "out")
    assert_close(to_f64(fin)[:, hs], ref_f, "final_state", "bf16")
