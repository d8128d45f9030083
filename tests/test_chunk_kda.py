"""The chunk_kda-shaped entry point: flag checks on the host (no GPU), and on
the GPU the same bits as kda.fwd for the pages' call (README mirror, section
"依赖要求", step 2)."""
import numpy as np
import pytest
import torch

kda = pytest.importorskip("gated_delta_rule_prep_amd.kda")
from gated_delta_rule_prep_amd.chunk_kda import chunk_kda  # noqa: E402

FLAGS = dict(use_gate_in_kernel=True, use_qk_l2norm_in_kernel=True, use_beta_sigmoid_in_kernel=True,
             safe_gate=True, transpose_state_layout=True)


def cpu_args(T=8, H=2):
    z = lambda *s: torch.zeros(*s, dtype=torch.bfloat16)
    return dict(q=z(1, T, H, 128), k=z(1, T, H, 128), v=z(1, T, H, 128), g=z(1, T, H, 128), beta=z(1, T, H),
                A_log=torch.zeros(H), dt_bias=torch.zeros(H, 128), lower_bound=-5.0)


@pytest.mark.parametrize("flag", sorted(FLAGS))
def test_each_unsupported_flag_is_rejected_by_name(flag):
    kw = dict(FLAGS)
    kw[flag] = False
    with pytest.raises(ValueError, match="rejected: %s=False" % flag):
        chunk_kda(**cpu_args(), **kw)


def test_missing_gate_parameters_are_rejected():
    a = cpu_args()
    for drop, what in (("A_log", "A_log"), ("dt_bias", "dt_bias"), ("lower_bound", "lower_bound")):
        kw = dict(a)
        kw[drop] = None
        with pytest.raises(ValueError, match=what):
            chunk_kda(**kw, **FLAGS)


def test_cpu_tensors_reach_the_binding_checks():
    # the supported flag set passes the facade and stops at the binding's device check
    with pytest.raises(ValueError, match="HIP device"):
        chunk_kda(**cpu_args(), **FLAGS)


@pytest.mark.gpu
@pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")
@pytest.mark.parametrize("state", [None, "bf16", "fp32"])
def test_same_bits_as_kda_fwd(state):
    from gated_delta_rule_prep_amd.inputs import make_inputs
    from tests.kda_gpu import device_inputs, run_gpu, say
    lens = [5, 40, 100, 16]
    inp = make_inputs(1, sum(lens), 3, seed=400, state_dtype=state or "fp32", seq_lens=lens,
                      initial_state=state is not None)
    say("case chunk_kda state=%s lens=%s" % (state, lens))
    d = device_inputs(inp)
    with torch.inference_mode():
        out, fin = chunk_kda(q=d["q"], k=d["k"], v=d["v"], g=d["g"], beta=d["beta"], scale=inp.scale,
                             initial_state=d["initial_state"], output_final_state=True, A_log=d["A_log"],
                             dt_bias=d["dt_bias"], lower_bound=inp.lower_bound, cu_seqlens=d["cu_seqlens"],
                             **FLAGS)
    ref_o, ref_f = run_gpu(inp, d=d)
    torch.cuda.synchronize()
    assert fin.dtype == (torch.bfloat16 if state == "bf16" else torch.float32)
    assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16))
    assert torch.equal(fin.view(torch.int16) if fin.dtype == torch.bfloat16 else fin,
                       ref_f.view(torch.int16) if ref_f.dtype == torch.bfloat16 else ref_f)


@pytest.mark.gpu
@pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")
@pytest.mark.parametrize("varlen", [False, True])
def test_against_the_oracle(varlen):
    """chunk_kda with the pages' flags and the default scale (K^-1/2) against
    the fp64 oracle, every head: the facade maps the call onto the kernels'
    arguments without changing what is computed."""
    import oracle
    from gated_delta_rule_prep_amd.inputs import make_inputs
    from tests.kda_gpu import assert_close, device_inputs, say, to_f64
    lens = [33, 1, 90, 16] if varlen else None
    inp = make_inputs(1 if varlen else 2, 140 if varlen else 70, 3, seed=401, state_dtype="bf16", seq_lens=lens)
    inp.scale = 128 ** -0.5
    say("case chunk_kda vs oracle varlen=%s" % varlen)
    d = device_inputs(inp)
    out, fin = chunk_kda(q=d["q"], k=d["k"], v=d["v"], g=d["g"], beta=d["beta"], initial_state=d["initial_state"],
                         output_final_state=True, A_log=d["A_log"], dt_bias=d["dt_bias"],
                         lower_bound=inp.lower_bound, cu_seqlens=d["cu_seqlens"], **FLAGS)
    torch.cuda.synchronize()
    ref_o, ref_f = oracle.kda_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, inp.A_log, inp.dt_bias,
                                  inp.lower_bound, initial_state=inp.initial_state_f64(),
                                  output_final_state=True, cu_seqlens=inp.cu_seqlens)
    assert_close(to_f64(out), ref_o, "out")
    assert_close(to_f64(fin), ref_f, "final_state", "bf16")
