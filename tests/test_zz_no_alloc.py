"""kda_fwd_fused_noalloc (the fused path on the library's static per-GPU
scratch, for callers that cannot allocate) against kda_fwd_ex on the fused
path with a caller workspace: the same kernels, so the outputs and final
states must agree bit for bit.  Two calls in a row, the second smaller, so
the second runs on tables the first left in the shared scratch."""
import numpy as np
import pytest
import torch

from gated_delta_rule_prep_amd.inputs import make_inputs
from tests.kda_gpu import device_inputs, say, state_torch_dtype

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def _buffers(inp):
    out = torch.full((inp.B, inp.T, inp.H, inp.V), float("nan"), dtype=torch.bfloat16, device="cuda")
    fin = torch.full((inp.N, inp.H, inp.V, inp.K), float("nan"), dtype=state_torch_dtype(inp), device="cuda")
    return out, fin


def _both(inp):
    from gated_delta_rule_prep_amd import kda
    d = device_inputs(inp)
    o1, f1 = _buffers(inp)
    kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], inp.scale, o1, d["A_log"], d["dt_bias"], inp.lower_bound,
            initial_state=d["initial_state"], final_state=f1, cu_seqlens=d["cu_seqlens"], path="fused")
    o2, f2 = _buffers(inp)
    kda.fwd_fused_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], inp.scale, o2, d["A_log"], d["dt_bias"],
                          inp.lower_bound, initial_state=d["initial_state"], final_state=f2,
                          cu_seqlens=d["cu_seqlens"])
    torch.cuda.synchronize()
    return (o1, f1), (o2, f2)


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_noalloc_matches_the_fused_path_on_two_calls_the_second_smaller():
    big = make_inputs(1, 700, 4, seed=900, state_dtype="fp32", seq_lens=[300, 1, 17, 382])
    small = make_inputs(2, 45, 2, seed=901, state_dtype="bf16")
    for inp in (big, small):
        say("case noalloc B=%d T=%d H=%d N=%d state=%s" % (inp.B, inp.T, inp.H, inp.N, inp.state_dtype))
        (o1, f1), (o2, f2) = _both(inp)
        assert not torch.isnan(o1.float()).any() and not torch.isnan(f1.float()).any()
        assert torch.equal(_bits(o1), _bits(o2)), "out differs from kda_fwd_ex(fused)"
        assert torch.equal(_bits(f1), _bits(f2)), "final_state differs from kda_fwd_ex(fused)"


def test_noalloc_rejects_more_sequences_than_the_scratch_holds():
    from gated_delta_rule_prep_amd import kda
    N, H = 16385, 1
    say("case noalloc N=%d (over the limit)" % N)
    z = torch.zeros(1, N, H, 128, dtype=torch.bfloat16, device="cuda")
    beta = torch.zeros(1, N, H, dtype=torch.bfloat16, device="cuda")
    A_log = torch.zeros(H, dtype=torch.float32, device="cuda")
    dt_bias = torch.zeros(H, 128, dtype=torch.float32, device="cuda")
    cu = torch.arange(N + 1, dtype=torch.int64, device="cuda")
    out = torch.full_like(z, 5.0)
    with pytest.raises(kda.KDAValueError):
        kda.fwd_fused_noalloc(z, z, z, z, beta, 1.0, out, A_log, dt_bias, -5.0, cu_seqlens=cu)
    torch.cuda.synchronize()
    assert bool((out == 5.0).all())


def test_noalloc_bad_cu_seqlens_touches_nothing():
    from gated_delta_rule_prep_amd import kda
    inp = make_inputs(1, 64, 2, seed=902, state_dtype="fp32", seq_lens=[30, 34])
    d = device_inputs(inp)
    say("case noalloc bad cu_seqlens")
    cu = torch.tensor([0, 40, 30], dtype=torch.int64, device="cuda")
    out = torch.full((1, 64, 2, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    fin = torch.full((2, 2, 128, 128), 7.0, dtype=torch.float32, device="cuda")
    kda.fwd_fused_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], inp.scale, out, d["A_log"], d["dt_bias"],
                          inp.lower_bound, initial_state=d["initial_state"], final_state=fin, cu_seqlens=cu)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all()) and bool((fin == 7.0).all())
