"""The forward captured in a HIP graph (torch.cuda.graph over the library's
stream-ordered launches) and replayed: every replay must give the eager
call's bits.

The library only enqueues kernels (no memsets, copies or host waits), so a
captured call is the same kernels with the same arguments.  Between replays
the outputs are refilled with NaN by eager work and the device is
synchronised, so each replay is checked on its own.
"""
import pytest
import torch

from gated_delta_rule_prep_amd.inputs import make_inputs, ragged_lengths
from tests.kda_gpu import device_inputs, say, state_torch_dtype

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

REPLAYS = 3


def make_call(inp, d, kind, out, fin):
    from gated_delta_rule_prep_amd import kda
    has_cu = inp.cu_seqlens is not None
    if kind == "decode":
        def call():
            kda.decode(d["q"], d["k"], d["v"], d["g"], d["beta"], inp.scale, out, d["A_log"], d["dt_bias"],
                       inp.lower_bound, initial_state=d["initial_state"], final_state=fin)
        return call
    kw = {}
    if kind == "segmented":
        kw["segments"] = 4
        nbytes = kda.segmented_workspace_bytes(inp.B, inp.T, inp.H, inp.N, has_cu, 4)
    else:
        path = {"auto": None, "split_flags": "split", "fused_wide": "fused", "split64": "split"}.get(kind, kind)
        kw["path"] = path
        chunk = 64 if kind == "split64" else None
        if chunk:
            kw["chunk"] = chunk
        nbytes = kda.workspace_bytes(inp.B, inp.T, inp.H, inp.N, has_cu, chunk, None, path)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    def call():
        kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], inp.scale, out, d["A_log"], d["dt_bias"],
                inp.lower_bound, initial_state=d["initial_state"], final_state=fin,
                cu_seqlens=d["cu_seqlens"], workspace=ws, **kw)
    return call


CASES = {
    "auto": dict(B=1, T=300, H=3, state_dtype="fp32", seed=700, seq_lens=ragged_lengths(300, 5)),
    "split": dict(B=2, T=200, H=2, state_dtype="bf16", seed=701),
    "fused": dict(B=1, T=300, H=3, state_dtype="bf16", seed=702, seq_lens=ragged_lengths(300, 5)),
    # 80 pairs: 64-column recurrence tiles whose waves meet through LDS flags
    "split_flags": dict(B=1, T=160, H=80, state_dtype="fp32", seed=705),
    # 150 pairs: the fused kernel's 128-column workgroups
    "fused_wide": dict(B=1, T=120, H=50, state_dtype="bf16", seed=706, seq_lens=[40, 50, 30]),
    # 64-token chunks on a varlen batch
    "split64": dict(B=1, T=300, H=3, state_dtype="fp32", seed=707, seq_lens=ragged_lengths(300, 5)),
    "segmented": dict(B=1, T=2048, H=2, state_dtype="fp32", seed=703),
    "decode": dict(B=64, T=1, H=4, state_dtype="bf16", seed=704),
}


@pytest.mark.parametrize("kind", list(CASES))
def test_graph_replays_match_eager_bitwise(kind):
    inp = make_inputs(**CASES[kind])
    say("case graph %s B=%d T=%d H=%d" % (kind, inp.B, inp.T, inp.H))
    d = device_inputs(inp)
    shape = (inp.B, inp.T, inp.H, inp.V) if kind != "decode" else (inp.B, 1, inp.H, inp.V)
    out = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    fin = torch.full((inp.N, inp.H, inp.V, inp.K), float("nan"), dtype=state_torch_dtype(inp), device="cuda")
    call = make_call(inp, d, kind, out, fin)

    call()   # eager
    torch.cuda.synchronize()
    ref_o, ref_f = out.clone(), fin.clone()
    assert bool(torch.isfinite(ref_o).all()) and bool(torch.isfinite(ref_f).all())

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()   # a call on the capture's stream before capturing
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for rep in range(REPLAYS):
        out.fill_(float("nan"))
        fin.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16)), "replay %d: out" % rep
        assert torch.equal(fin.view(torch.int16) if fin.dtype == torch.bfloat16 else fin,
                           ref_f.view(torch.int16) if fin.dtype == torch.bfloat16 else ref_f), "replay %d: state" % rep
