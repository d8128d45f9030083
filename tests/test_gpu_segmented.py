"""GPU parity of kda_fwd_segmented (every sequence cut into segments joined by
their affine state maps) against the fp64 oracle of the uncut recurrence.

The oracle knows nothing of segments: a correct composition must reproduce the
one-chain result within the same tolerance as kda_fwd.
"""
import pytest
import torch

from gated_delta_rule_prep_amd.inputs import configs, make_inputs, ragged_lengths
from tests.kda_gpu import assert_close, device_inputs, run_gpu, say, state_torch_dtype, to_f64
from tests.test_gpu_parity import oracle_run

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def run_seg(inp, segments, d=None, workspace=None, out=None, final=None):
    from gated_delta_rule_prep_amd import kda
    if d is None:
        d = device_inputs(inp)
    B, T, H, V = inp.B, inp.T, inp.H, inp.V
    if out is None:
        out = torch.full((B, T, H, V), float("nan"), dtype=torch.bfloat16, device="cuda")
    if final is None and inp.output_final_state:
        final = torch.full((inp.N, H, V, inp.K), float("nan"), dtype=state_torch_dtype(inp), device="cuda")
    kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], inp.scale, out, d["A_log"], d["dt_bias"],
            inp.lower_bound, initial_state=d["initial_state"], final_state=final, cu_seqlens=d["cu_seqlens"],
            workspace=workspace, segments=segments)
    return out, final


def check_seg(inp, segments, heads=None, tag=""):
    say("case %s B=%d T=%d H=%d N=%d state=%s segments=%d" % (
        tag, inp.B, inp.T, inp.H, inp.N, inp.state_dtype, segments))
    out, fin = run_seg(inp, segments)
    torch.cuda.synchronize()
    ref_o, ref_f = oracle_run(inp, heads)
    hs = list(range(inp.H)) if heads is None else heads
    assert_close(to_f64(out)[:, :, hs], ref_o, "out")
    if inp.output_final_state:
        assert_close(to_f64(fin)[:, hs], ref_f, "final_state", inp.state_dtype)


SEG_CASES = [
    (dict(B=1, T=37, H=2, state_dtype=None, lower_bound=-5.0, seed=400), 4),   # last segment empty
    (dict(B=1, T=300, H=2, state_dtype="fp32", lower_bound=-5.0, seed=401), 3),
    (dict(B=2, T=100, H=3, state_dtype="bf16", lower_bound=-5.0, seed=402), 2),
    (dict(B=1, T=257, H=2, state_dtype="fp32", lower_bound=-0.5, seed=403, g_std=2.0), 8),
    (dict(B=1, T=300, H=3, state_dtype="bf16", lower_bound=-5.0, seed=404, seq_lens=ragged_lengths(300, 7)), 8),
    (dict(B=1, T=113, H=2, state_dtype="fp32", lower_bound=-2.0, seed=405, seq_lens=[1, 15, 17, 0, 40, 16, 24]),
     3),
    (dict(B=1, T=1024, H=1, state_dtype="fp32", lower_bound=-5.0, seed=406), 64),   # 16 tokens per segment
]


@pytest.mark.parametrize("i", range(len(SEG_CASES)))
def test_segmented_small_parity(i):
    kw, S = SEG_CASES[i]
    check_seg(make_inputs(**kw), S, tag="seg%d" % i)


@pytest.mark.parametrize("ci,S", [(1, 8), (2, 4), (4, 16)])
def test_segmented_config_parity(ci, S):
    cfg = configs()[ci]
    inp = cfg.make()
    heads = sorted({0, 1, inp.H // 2, inp.H - 1})
    check_seg(inp, S, heads, tag="config%d %s" % (ci, cfg.name))


@pytest.mark.parametrize("S", [8, 0])
def test_segmented_few_heads_long_sequence(S):
    """The case the cut is for: one long sequence and few heads (S = 0: the
    library's count, 16 here)."""
    from gated_delta_rule_prep_amd import kda
    inp = make_inputs(1, 8192, 4, seed=407, state_dtype="fp32")
    assert kda.segments_for(1, 8192, 4) == 16
    check_seg(inp, S, tag="T8192 H4")


def test_segmented_one_segment_is_kda_fwd_bitwise():
    inp = make_inputs(1, 300, 3, seed=408, state_dtype="bf16", seq_lens=ragged_lengths(300, 5))
    say("case segments=1 vs kda_fwd")
    d = device_inputs(inp)
    o1, f1 = run_seg(inp, 1, d=d)
    o2, f2 = run_gpu(inp, d=d)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(f1.view(torch.int16), f2.view(torch.int16))


def test_segmented_deterministic_and_inplace_state():
    inp = make_inputs(1, 500, 2, seed=409, state_dtype="fp32", seq_lens=[200, 300])
    say("case segmented in-place state")
    d = device_inputs(inp)
    o1, f1 = run_seg(inp, 3, d=d)
    o2, f2 = run_seg(inp, 3, d=d)
    st = d["initial_state"].clone()
    o3, _ = run_seg(inp, 3, d=dict(d, initial_state=st), final=st)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(f1, f2)
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16)) and torch.equal(st, f1)


def test_segmented_zero_tokens_passes_state_through():
    inp = make_inputs(1, 0, 3, seed=410, state_dtype="fp32")
    say("case segmented T=0")
    out, fin = run_seg(inp, 4)
    torch.cuda.synchronize()
    assert torch.equal(fin.cpu(), torch.from_numpy(inp.initial_state))


def test_segmented_bad_cu_seqlens_sets_status_and_touches_nothing():
    from gated_delta_rule_prep_amd import kda
    inp = make_inputs(1, 64, 2, seed=411, state_dtype="fp32", seq_lens=[30, 34])
    d = device_inputs(inp)
    for bad in ([0, 40, 30], [1, 30, 64], [0, 30, 63]):
        say("case segmented bad cu_seqlens %s" % bad)
        cu = torch.tensor(bad, dtype=torch.int64, device="cuda")
        out = torch.zeros(1, 64, 2, 128, dtype=torch.bfloat16, device="cuda")
        fin = torch.zeros(2, 2, 128, 128, dtype=torch.float32, device="cuda")
        ws = torch.empty(kda.segmented_workspace_bytes(1, 64, 2, 2, True, 3), dtype=torch.uint8, device="cuda")
        run_seg(inp, 3, d=dict(d, cu_seqlens=cu), workspace=ws, out=out, final=fin)
        assert kda.check_status(ws) == kda.KDA_STATUS_BAD_CU_SEQLENS
        assert torch.count_nonzero(out.view(torch.int16)) == 0
        assert torch.count_nonzero(fin) == 0
    ws = torch.empty(kda.segmented_workspace_bytes(1, 64, 2, 2, True, 3), dtype=torch.uint8, device="cuda")
    run_seg(inp, 3, d=d, workspace=ws)
    assert kda.check_status(ws) == kda.KDA_STATUS_OK


def test_kda_fwd_takes_the_segmented_form_when_the_workspace_allows():
    """Without cu_seqlens and with few heads, kda_fwd runs kda_fwd_segmented
    with the library's count (bitwise the same result); with a workspace sized
    only for the uncut call it runs uncut (bitwise kda_fwd_ex's library choice)."""
    from gated_delta_rule_prep_amd import kda
    inp = make_inputs(1, 8192, 4, seed=412, state_dtype="fp32")
    say("case kda_fwd cut / uncut, T8192 H4")
    d = device_inputs(inp)
    o_fwd, f_fwd = run_gpu(inp, d=d)                      # kda_fwd, all-paths workspace
    o_seg, f_seg = run_seg(inp, kda.segments_for(1, 8192, 4), d=d)
    small = kda.alloc_workspace(1, 8192, 4, 1, False, "cuda", None, None, "auto")
    o_unc, f_unc = run_gpu(inp, d=d, workspace=small)     # kda_fwd, too small to cut
    o_ex, f_ex = run_gpu(inp, d=d, path="auto")           # kda_fwd_ex, the library's path
    torch.cuda.synchronize()
    assert torch.equal(o_fwd.view(torch.int16), o_seg.view(torch.int16)) and torch.equal(f_fwd, f_seg)
    assert torch.equal(o_unc.view(torch.int16), o_ex.view(torch.int16)) and torch.equal(f_unc, f_ex)
    ref_o, ref_f = oracle_run(inp)
    assert_close(to_f64(o_fwd), ref_o, "out")
    assert_close(to_f64(f_fwd), ref_f, "final_state", "fp32")
