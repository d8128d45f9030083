"""The precision study of kda_fwd_precision against the fp64 oracle: the
library's arithmetic next to the alternatives the FlashKDA blog post weighs in
§二 2.1 and 2.3 (the state stored in bf16 between chunk updates; the inverse stage
E = T R in bf16 instead of fp16; the state products in bf16; the 16 x 16 inverse
as the fp16 Neumann product the pages describe instead of fp32 substitution).

The default variant must equal the split path bitwise and meet the contract's
tolerance, and so must the pages' fp16 Neumann inverse (the study found it as
accurate).  The other alternatives are measurements, not contracts: each is
checked to be finite, and its scores are printed for the table of the study.
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_prep_amd.inputs import configs, make_inputs
from tests.kda_gpu import (assert_close, device_inputs, run_gpu, say, score,
                           state_torch_dtype, to_f64)
from tests.test_gpu_parity import oracle_run

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

VARIANTS = {0: "default (fp32 state, fp16 operands)", 1: "bf16 state between updates", 2: "bf16 inverse stage",
            4: "bf16 state products", 3: "state + inverse", 5: "state + products", 6: "inverse + products",
            7: "all three", 8: "fp16 Neumann inverse (the pages')", 9: "Neumann inverse + bf16 state"}


def run_variant(inp, d, variant):
    from gated_delta_rule_prep_amd import kda
    out = torch.full((inp.B, inp.T, inp.H, inp.V), float("nan"), dtype=torch.bfloat16, device="cuda")
    fin = torch.full((inp.N, inp.H, inp.V, inp.K), float("nan"), dtype=state_torch_dtype(inp), device="cuda")
    kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], inp.scale, out, d["A_log"], d["dt_bias"], inp.lower_bound,
            initial_state=d["initial_state"], final_state=fin, cu_seqlens=d["cu_seqlens"], precision=variant)
    return out, fin


CASES = [("small T300 H2 fp32", lambda: make_inputs(1, 300, 2, seed=500, state_dtype="fp32")),
         ("small T257 H2 lb-0.5 g2", lambda: make_inputs(1, 257, 2, seed=501, state_dtype="fp32",
                                                         lower_bound=-0.5, g_std=2.0))] + \
        [(c.name, c.make) for c in configs()]


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_precision_variants(ci):
    name, make = CASES[ci]
    inp = make()
    heads = None if inp.H <= 4 else sorted({0, 1, inp.H // 2, inp.H - 1})
    hs = list(range(inp.H)) if heads is None else heads
    d = device_inputs(inp)
    ref_o, ref_f = oracle_run(inp, heads)
    base_o, base_f = run_gpu(inp, d=d, path="split", chunk=16)
    for v, label in VARIANTS.items():
        say("case %s variant %d (%s)" % (name, v, label))
        o, f = run_variant(inp, d, v)
        torch.cuda.synchronize()
        so = score(to_f64(o)[:, :, hs], ref_o)
        sf = score(to_f64(f)[:, hs], ref_f, inp.state_dtype)
        say("  study %-40s | %-28s | out max/RMS %.3e mean rel %.3e | state max/RMS %.3e mean rel %.3e" % (
            name, label, so["adj_max_over_rms"], so["mean_rel"], sf["adj_max_over_rms"], sf["mean_rel"]))
        if v == 0:
            assert torch.equal(o.view(torch.int16), base_o.view(torch.int16))
            assert torch.equal(f.view(torch.int16) if f.dtype == torch.bfloat16 else f,
                               base_f.view(torch.int16) if f.dtype == torch.bfloat16 else base_f)
            assert_close(to_f64(o)[:, :, hs], ref_o, "out")
            assert_close(to_f64(f)[:, hs], ref_f, "final_state", inp.state_dtype)
        if v == 8:   # the pages' fp16 Neumann inverse: as accurate as the library's substitution
            assert_close(to_f64(o)[:, :, hs], ref_o, "out")
            assert_close(to_f64(f)[:, hs], ref_f, "final_state", inp.state_dtype)
        for s in (so, sf):
            assert s["finite"]
