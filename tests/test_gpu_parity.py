"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Every case compares every output element and every final-state element with
the oracle, the five full-size workloads included (all heads); a few other
large cases run the oracle on a sample of heads (heads never interact, so
slicing the inputs along H gives the oracle's exact values for those heads).
"""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_prep_amd.inputs import bf16_bits_to_f32, configs, make_inputs, ragged_lengths, f32_to_bf16_bits
from tests.kda_gpu import VARIANT_IDS, VARIANTS, assert_close, device_inputs, run_gpu, say, to_f64

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def oracle_run(inp, heads=None):
    if heads is None:
        heads = list(range(inp.H))
    sl = lambda x: np.ascontiguousarray(x[:, :, heads])
    s0 = inp.initial_state_f64()
    return oracle.kda_fwd(sl(inp.q), sl(inp.k), sl(inp.v), sl(inp.g), sl(inp.beta), inp.scale,
                          inp.A_log[heads].copy(), inp.dt_bias[heads].copy(), inp.lower_bound,
                          initial_state=None if s0 is None else np.ascontiguousarray(s0[:, heads]),
                          output_final_state=True, cu_seqlens=inp.cu_seqlens)


_ORACLE_CACHE = {}


def config_oracle(ci, inp):
    """The oracle's out and final state of workload ci, every head; the last
    workload's are kept, since the tests of one workload run one after another."""
    if ci not in _ORACLE_CACHE:
        _ORACLE_CACHE.clear()
        _ORACLE_CACHE[ci] = oracle_run(inp)
    return _ORACLE_CACHE[ci]


def check(inp, heads=None, tag="", chunk=None, path=None, ref=None):
    say("case %s B=%d T=%d H=%d N=%d state=%s lb=%g path=%s chunk=%s" % (
        tag or inp.name, inp.B, inp.T, inp.H, inp.N, inp.state_dtype, inp.lower_bound, path, chunk))
    out, fin = run_gpu(inp, chunk=chunk, path=path)
    torch.cuda.synchronize()
    ref_o, ref_f = oracle_run(inp, heads) if ref is None else ref
    hs = list(range(inp.H)) if heads is None else heads
    x = to_f64(out)[:, :, hs]
    assert_close(x, ref_o, "out")
    if inp.output_final_state:
        assert_close(to_f64(fin)[:, hs], ref_f, "final_state", inp.state_dtype)
    return out, fin


SMALL = [
    dict(B=1, T=37, H=2, state_dtype=None, lower_bound=-5.0, seed=100),
    dict(B=1, T=64, H=1, state_dtype="fp32", initial_state=False, lower_bound=-5.0, seed=101),
    dict(B=2, T=100, H=3, state_dtype="fp32", lower_bound=-5.0, seed=102),
    dict(B=1, T=300, H=2, state_dtype="bf16", lower_bound=-5.0, seed=103),
    dict(B=1, T=257, H=4, state_dtype="fp32", lower_bound=-0.5, seed=104, g_std=2.0),
    dict(B=3, T=16, H=2, state_dtype="bf16", lower_bound=0.0, seed=105),
    dict(B=1, T=1, H=5, state_dtype="fp32", lower_bound=-5.0, seed=106),
    dict(B=1, T=113, H=2, state_dtype="fp32", lower_bound=-2.0, seed=107, seq_lens=[1, 15, 17, 0, 40, 16, 24]),
    dict(B=1, T=300, H=3, state_dtype="bf16", lower_bound=-5.0, seed=108, seq_lens=ragged_lengths(300, 7)),
]


@pytest.mark.parametrize("path,chunk", VARIANTS, ids=VARIANT_IDS)
@pytest.mark.parametrize("i", range(len(SMALL)))
def test_small_parity(i, path, chunk):
    kw = dict(SMALL[i])
    inp = make_inputs(**kw)
    check(inp, tag="small%d" % i, chunk=chunk, path=path)


@pytest.mark.parametrize("path,chunk", VARIANTS, ids=VARIANT_IDS)
@pytest.mark.parametrize("ci", range(5))
def test_config_parity(ci, path, chunk):
    """The five workloads at full size on every path and chunk size, every
    head against the oracle."""
    cfg = configs()[ci]
    inp = cfg.make()
    check(inp, None, tag="config%d %s" % (ci, cfg.name), chunk=chunk, path=path, ref=config_oracle(ci, inp))


@pytest.mark.parametrize("ci", range(5))
def test_config_parity_library_choice(ci):
    """The five workloads as bench.py times them: kda_fwd_ex with the library's
    path choice (the fixed 8192-token headline runs the split path, the 8 x 1024
    varlen batch the fused kernel), every head against the oracle."""
    from gated_delta_rule_prep_amd import kda
    cfg = configs()[ci]
    inp = cfg.make()
    say("case config%d %s path=auto" % (ci, cfg.name))
    ws = kda.alloc_workspace(inp.B, inp.T, inp.H, inp.N, inp.cu_seqlens is not None, "cuda", None, None, "auto")
    out, fin = run_gpu(inp, workspace=ws, path="auto")
    torch.cuda.synchronize()
    taken = kda.path_taken(ws)
    assert taken in ("split", "fused")
    if ci in (2, 3):
        assert taken == ("split" if ci == 2 else "fused")
    ref_o, ref_f = config_oracle(ci, inp)
    assert_close(to_f64(out), ref_o, "out")
    assert_close(to_f64(fin), ref_f, "final_state", inp.state_dtype)


def test_fused_many_pairs_parity():
    """More (sequence, head) pairs than two 64-column tiles each can place on
    the 256 CUs at once: the fused path then runs one workgroup per pair
    with 128 columns; checked on sampled heads of a varlen batch."""
    lens = [5, 300, 16, 77, 1, 130, 64, 33]
    inp = make_inputs(1, sum(lens), 40, seed=110, state_dtype="bf16", seq_lens=lens)
    assert 2 * inp.N * inp.H > 512
    check(inp, [0, 7, 21, 39], tag="many-pairs", path="fused")


@pytest.mark.parametrize("lens,H,expect", [([2048], 8, "split"), ([512] * 8, 64, "fused")],
                         ids=["one-long", "many-short"])
def test_library_choice_picks_a_path_and_matches_it_bitwise(lens, H, expect):
    """The library's path choice from the chunk counts (on the host for the
    one fixed-length sequence, by the scheduler kernel with cu_seqlens): a
    single long sequence runs the split path, many short ones the fused kernel;
    the result is bit for bit the chosen path's."""
    from gated_delta_rule_prep_amd import kda
    inp = make_inputs(1, sum(lens), H, seed=111, state_dtype="bf16", seq_lens=lens if len(lens) > 1 else None)
    d = device_inputs(inp)
    say("case library choice lens=%s H=%d (expect %s)" % (lens[:2], H, expect))
    ws = kda.alloc_workspace(1, inp.T, H, inp.N, inp.cu_seqlens is not None, "cuda", None, None, "auto")
    out, fin = run_gpu(inp, d=d, workspace=ws)
    assert kda.path_taken(ws) == expect
    o2, f2 = run_gpu(inp, d=d, path=expect)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(fin.view(torch.int16), f2.view(torch.int16))
    hs = [0, H // 2, H - 1]
    ref_o, ref_f = oracle_run(inp, hs)
    assert_close(to_f64(out)[:, :, hs], ref_o, "out")
    assert_close(to_f64(fin)[:, hs], ref_f, "final_state", "bf16")


def test_host_choice_for_fixed_lengths_picks_fused_for_many_short():
    """B sequences of T tokens: the host evaluates the path estimate itself and
    enqueues only the chosen path; 8 x 512 tokens at H = 64 runs the fused
    kernel, bit for bit as kda_fwd_ex(fused)."""
    from gated_delta_rule_prep_amd import kda
    inp = make_inputs(8, 512, 64, seed=112, state_dtype="bf16")
    d = device_inputs(inp)
    say("case host choice B=8 T=512 H=64 (expect fused)")
    ws = kda.alloc_workspace(8, 512, 64, 8, False, "cuda", None, None, "auto")
    out, fin = run_gpu(inp, d=d, workspace=ws, path="auto")
    assert kda.path_taken(ws) == "fused"
    o2, f2 = run_gpu(inp, d=d, path="fused")
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(fin.view(torch.int16), f2.view(torch.int16))
    hs = [0, 63]
    ref_o, ref_f = oracle_run(inp, hs)
    assert_close(to_f64(out)[:, :, hs], ref_o, "out")
    assert_close(to_f64(fin)[:, hs], ref_f, "final_state", "bf16")


@pytest.mark.parametrize("path,chunk", VARIANTS, ids=VARIANT_IDS)
def test_deterministic_bitwise(path, chunk):
    inp = make_inputs(1, 500, 4, seed=200, state_dtype="fp32")
    say("case determinism T=500 H=4 path=%s chunk=%d" % (path, chunk))
    o1, f1 = run_gpu(inp, chunk=chunk, path=path)
    o2, f2 = run_gpu(inp, chunk=chunk, path=path)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(f1, f2)


@pytest.mark.parametrize("path,chunk", VARIANTS, ids=VARIANT_IDS)
def test_varlen_equals_separate_calls_bitwise(path, chunk):
    lens = [1, 15, 17, 33, 130, 60]
    inp = make_inputs(1, sum(lens), 3, seed=201, state_dtype="bf16", seq_lens=lens)
    say("case varlen-vs-separate lens=%s path=%s chunk=%d" % (lens, path, chunk))
    out, fin = run_gpu(inp, chunk=chunk, path=path)
    cu = inp.cu_seqlens
    for n in range(len(lens)):
        a, b = int(cu[n]), int(cu[n + 1])
        sub = make_inputs(1, b - a, 3, seed=201, state_dtype="bf16")
        for f in ("q", "k", "v", "g", "beta"):
            setattr(sub, f, np.ascontiguousarray(getattr(inp, f)[:, a:b]))
        sub.A_log, sub.dt_bias = inp.A_log, inp.dt_bias
        sub.initial_state = np.ascontiguousarray(inp.initial_state[n:n + 1])
        o, f = run_gpu(sub, chunk=chunk, path=path)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), out[:, a:b].view(torch.int16)), n
        assert torch.equal(f[0].view(torch.int16), fin[n].view(torch.int16)), n


def test_resume_split_matches_one_call():
    inp = make_inputs(1, 400, 2, seed=202, state_dtype="fp32")
    say("case resume T=400 split at 163")
    out, fin = run_gpu(inp)
    t1 = 163
    d = device_inputs(inp)
    from gated_delta_rule_prep_amd import kda
    o = torch.empty_like(out)
    mid = torch.empty_like(fin)
    f2 = torch.empty_like(fin)
    sl = lambda t, a, b: t[:, a:b].contiguous()
    kda.fwd(sl(d["q"], 0, t1), sl(d["k"], 0, t1), sl(d["v"], 0, t1), sl(d["g"], 0, t1), sl(d["beta"], 0, t1),
            inp.scale, o[:, :t1], d["A_log"], d["dt_bias"], inp.lower_bound, initial_state=d["initial_state"],
            final_state=mid)
    o2 = torch.empty_like(out[:, t1:])
    kda.fwd(sl(d["q"], t1, 400), sl(d["k"], t1, 400), sl(d["v"], t1, 400), sl(d["g"], t1, 400),
            sl(d["beta"], t1, 400), inp.scale, o2, d["A_log"], d["dt_bias"], inp.lower_bound,
            initial_state=mid, final_state=f2)
    torch.cuda.synchronize()
    ref_o, ref_f = oracle_run(inp)
    assert_close(np.concatenate([to_f64(o[:, :t1]), to_f64(o2)], axis=1), ref_o, "out(split)")
    assert_close(to_f64(f2), ref_f, "final(split)", "fp32")


def test_inplace_state():
    inp = make_inputs(1, 90, 2, seed=203, state_dtype="fp32")
    say("case in-place state")
    d = device_inputs(inp)
    out = torch.empty(1, 90, 2, 128, dtype=torch.bfloat16, device="cuda")
    st = d["initial_state"].clone()
    from gated_delta_rule_prep_amd import kda
    kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], inp.scale, out, d["A_log"], d["dt_bias"],
            inp.lower_bound, initial_state=st, final_state=st)
    o_ref, f_ref = run_gpu(inp, d=d)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(st, f_ref)


def test_identity_lower_bound_zero_beta_zero():
    inp = make_inputs(1, 50, 2, seed=204, state_dtype="fp32", lower_bound=0.0)
    inp.beta[:] = f32_to_bf16_bits(np.array([-1e4], np.float32))[0]
    say("case identity lb=0 beta=0")
    out, fin = run_gpu(inp)
    torch.cuda.synchronize()
    assert torch.equal(fin.cpu(), torch.from_numpy(inp.initial_state))
    ref_o, _ = oracle_run(inp)
    assert_close(to_f64(out), ref_o, "out")


def test_zero_tokens_passes_state_through():
    inp = make_inputs(1, 0, 3, seed=205, state_dtype="bf16")
    say("case T=0")
    out, fin = run_gpu(inp)
    torch.cuda.synchronize()
    assert torch.equal(fin.cpu().view(torch.int16), torch.from_numpy(inp.initial_state.view(np.int16)))


@pytest.mark.parametrize("path,chunk,parts", [("auto", None, None), ("split", 16, None), ("fused", 16, None),
                                               ("split", 32, None), ("split", 16, 3), ("split", 32, 2),
                                               ("split", 64, None), ("split", 64, 2)])
def test_bad_cu_seqlens_sets_status_and_touches_nothing(path, chunk, parts):
    """A rejected cu_seqlens leaves out and final_state exactly as they were
    (both filled with a sentinel first), on every path."""
    from gated_delta_rule_prep_amd import kda
    inp = make_inputs(1, 64, 2, seed=206, state_dtype="fp32", seq_lens=[30, 34])
    d = device_inputs(inp)
    for bad in ([0, 40, 30], [1, 30, 64], [0, 30, 63]):
        say("case bad cu_seqlens %s path %s chunk %s parts %s" % (bad, path, chunk, parts))
        cu = torch.tensor(bad, dtype=torch.int64, device="cuda")
        out = torch.full((1, 64, 2, 128), 3.0, dtype=torch.bfloat16, device="cuda")
        fin = torch.full((2, 2, 128, 128), 7.0, dtype=torch.float32, device="cuda")
        ws = kda.alloc_workspace(1, 64, 2, 2, True, "cuda", chunk=chunk, parts=parts, path=path)
        kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], inp.scale, out, d["A_log"], d["dt_bias"],
                inp.lower_bound, initial_state=d["initial_state"], final_state=fin, cu_seqlens=cu, workspace=ws,
                chunk=chunk, parts=parts, path=path)
        assert kda.check_status(ws) == kda.KDA_STATUS_BAD_CU_SEQLENS
        assert bool((out == 3.0).all()), "out was written"
        assert bool((fin == 7.0).all()), "final_state was written"
    ws = kda.alloc_workspace(1, 64, 2, 2, True, "cuda", chunk=chunk, parts=parts, path=path)
    run_gpu(inp, d=d, workspace=ws, chunk=chunk, parts=parts, path=path)
    assert kda.check_status(ws) == kda.KDA_STATUS_OK


def _scaled(inp, v_scale, state_scale):
    """The same inputs with v and the initial state multiplied (v rounded
    back to bf16)."""
    inp.v = f32_to_bf16_bits(bf16_bits_to_f32(inp.v) * np.float32(v_scale))
    if inp.initial_state is not None:
        if inp.state_dtype == "bf16":
            inp.initial_state = f32_to_bf16_bits(bf16_bits_to_f32(inp.initial_state) * np.float32(state_scale))
        else:
            inp.initial_state = (inp.initial_state * np.float32(state_scale)).astype(np.float32)
    return inp


@pytest.mark.parametrize("path,chunk", VARIANTS, ids=VARIANT_IDS)
def test_large_magnitude_inside_the_fp16_range(path, chunk):
    """v and the initial state scaled by 1000 (the top of the activation scale
    the numerical-range note in include/kda.h covers): the state and the
    per-chunk residuals stay inside the fp16 operand range, the result meets
    the tolerance relative to its own RMS, and the status word is OK."""
    from gated_delta_rule_prep_amd import kda
    inp = _scaled(make_inputs(1, 300, 3, seed=210, state_dtype="fp32", seq_lens=[1, 120, 179]), 1000.0, 1000.0)
    say("case large magnitude x1000 path=%s chunk=%s" % (path, chunk))
    ws = kda.alloc_workspace(1, inp.T, inp.H, inp.N, True, "cuda", chunk, None, path)
    out, fin = run_gpu(inp, workspace=ws, chunk=chunk, path=path)
    assert kda.check_status(ws) == kda.KDA_STATUS_OK
    ref_o, ref_f = oracle_run(inp)
    assert float(np.abs(ref_f).max()) < 65504.0
    assert_close(to_f64(out), ref_o, "out")
    assert_close(to_f64(fin), ref_f, "final_state", "fp32")


@pytest.mark.parametrize("form", ["fused16", "split16", "split32", "split64", "parts3", "segments4"])
def test_beyond_the_fp16_range_is_reported(form):
    """v scaled by 1e6: the residuals leave the fp16 operand range, the state
    ends non-finite, and every path reports KDA_STATUS_OVERFLOW in the status
    word; the next in-range call on the same workspace reports OK again."""
    from gated_delta_rule_prep_amd import kda
    kw = dict(fused16=dict(path="fused", chunk=16), split16=dict(path="split", chunk=16),
              split32=dict(path="split", chunk=32), split64=dict(path="split", chunk=64),
              parts3=dict(path="split", chunk=16, parts=3), segments4=dict(segments=4))[form]
    for scale, expect in ((1e6, kda.KDA_STATUS_OVERFLOW), (1.0, kda.KDA_STATUS_OK)):
        inp = _scaled(make_inputs(1, 256, 2, seed=211, state_dtype="fp32"), scale, 1.0)
        say("case beyond fp16 range form=%s v x %g" % (form, scale))
        d = device_inputs(inp)
        if "segments" in kw:
            n = kda.segmented_workspace_bytes(1, 256, 2, 1, False, kw["segments"])
        else:
            n = kda.workspace_bytes(1, 256, 2, 1, False, kw["chunk"], kw.get("parts"), kw["path"])
        if scale != 1.0:
            ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        out = torch.empty(1, 256, 2, 128, dtype=torch.bfloat16, device="cuda")
        fin = torch.empty(1, 2, 128, 128, dtype=torch.float32, device="cuda")
        kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], inp.scale, out, d["A_log"], d["dt_bias"],
                inp.lower_bound, initial_state=d["initial_state"], final_state=fin, workspace=ws, **kw)
        st = kda.check_status(ws)
        assert st == expect, (form, scale, st)
        if expect == kda.KDA_STATUS_OVERFLOW:
            assert not bool(torch.isfinite(fin).all())


def test_fixed_length_call_rewrites_a_stale_header():
    """B sequences of T tokens on the split path run without the scheduler
    kernel; the prep kernel writes the header itself, so a workspace that a
    previous call left marked bad (rejected cu_seqlens) or overflowed reports
    OK and the split path after a good fixed-length call, with the right result."""
    from gated_delta_rule_prep_amd import kda
    inp = make_inputs(2, 40, 2, seed=212, state_dtype="fp32")
    d = device_inputs(inp)
    n = max(kda.workspace_bytes(1, 80, 2, 2, True), kda.workspace_bytes(2, 40, 2, 2, False, 16, None, "split"))
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    say("case stale header: a rejected cu_seqlens call, then a fixed-length call")
    bad = make_inputs(1, 80, 2, seed=213, state_dtype="fp32", seq_lens=[40, 40])
    db = device_inputs(bad)
    cu = torch.tensor([0, 50, 40], dtype=torch.int64, device="cuda")
    o = torch.empty(1, 80, 2, 128, dtype=torch.bfloat16, device="cuda")
    f = torch.empty(2, 2, 128, 128, dtype=torch.float32, device="cuda")
    kda.fwd(db["q"], db["k"], db["v"], db["g"], db["beta"], bad.scale, o, db["A_log"], db["dt_bias"],
            bad.lower_bound, initial_state=db["initial_state"], final_state=f, cu_seqlens=cu, workspace=ws)
    assert kda.check_status(ws) == kda.KDA_STATUS_BAD_CU_SEQLENS
    out, fin = run_gpu(inp, d=d, workspace=ws, path="split", chunk=16)
    assert kda.check_status(ws) == kda.KDA_STATUS_OK
    assert kda.path_taken(ws) == "split"
    ref_o, ref_f = oracle_run(inp)
    assert_close(to_f64(out), ref_o, "out")
    assert_close(to_f64(fin), ref_f, "final_state", "fp32")
    say("case stale header: an overflowing fixed-length call, then a good one")
    big = _scaled(make_inputs(2, 40, 2, seed=212, state_dtype="fp32"), 1e6, 1.0)
    run_gpu(big, workspace=ws, path="split", chunk=16)
    assert kda.check_status(ws) == kda.KDA_STATUS_OVERFLOW
    run_gpu(inp, d=d, workspace=ws, path="split", chunk=16)
    assert kda.check_status(ws) == kda.KDA_STATUS_OK


@pytest.mark.parametrize("path", ["split", "fused"])
@pytest.mark.parametrize("B", [1, 2])
def test_wave_sync_timeout_is_reported(B, path):
    """The waits between the waves of a recurrence or fused workgroup are
    bounded.  With the bound forced to zero polls from the host, every such
    wait gives up at once: the kernels still finish and the status word
    reports the time-out.  With the default bound restored, the same call is
    clean and gives the same result as before.  Split path -- B = 1: 96 pairs,
    64-column recurrence tiles with a CU each; B = 2: 192 equal pairs,
    128-column tiles; 10 chunks, more than the ring's slots, so the loaders
    wait too.  Fused path -- B = 1: 64-column workgroups, B = 2: 128-column."""
    from gated_delta_rule_prep_amd import kda
    inp = make_inputs(B, 160, 96, seed=230 + B, state_dtype="fp32")
    d = device_inputs(inp)
    ws = torch.empty(kda.workspace_bytes(B, 160, 96, B, False, 16, None, path), dtype=torch.uint8,
                     device="cuda")
    say("case sync timeout B=%d T=160 H=96 %s: default bound" % (B, path))
    ref_out, ref_fin = run_gpu(inp, d=d, workspace=ws, path=path, chunk=16)
    assert kda.check_status(ws) == kda.KDA_STATUS_OK
    say("case sync timeout B=%d %s: bound of zero polls" % (B, path))
    try:
        kda.debug_set_spin_limit(0)
        run_gpu(inp, d=d, workspace=ws, path=path, chunk=16)
        st = kda.check_status(ws)
    finally:
        kda.debug_set_spin_limit(-1)
    assert st & kda.KDA_STATUS_SYNC_TIMEOUT
    say("case sync timeout B=%d %s: default bound again" % (B, path))
    out, fin = run_gpu(inp, d=d, workspace=ws, path=path, chunk=16)
    assert kda.check_status(ws) == kda.KDA_STATUS_OK
    assert torch.equal(out, ref_out) and torch.equal(fin, ref_fin)
    ref_o, ref_f = oracle_run(inp)
    assert_close(to_f64(out), ref_o, "out")
    assert_close(to_f64(fin), ref_f, "final_state", "fp32")


# Launch shapes at the boundaries of the tiling rules (kda_internal.h): value
# tiles per (sequence, head) in the recurrence (4 while 4 pairs <= 256 CUs,
# else 2, or 1 for equal lengths past 128 pairs), two recurrence workgroups
# per CU past 256 workgroups, and the fused kernel's 64- or 128-column tiles
# (64 while 2 pairs <= 256).
TILING_CASES = [
    dict(B=1, T=37, H=64, seq_lens=[37], seed=220),               # 64 pairs: 4 tiles, 256 workgroups
    dict(B=1, T=37, H=65, seq_lens=[37], seed=221),               # 65 pairs: 2 tiles
    dict(B=1, T=37, H=64, seq_lens=[20, 17], seed=222),           # 128 pairs: 2 tiles, 256 workgroups; fused 64
    dict(B=1, T=37, H=43, seq_lens=[10, 20, 7], seed=223),        # 129 pairs: 2 tiles, two per CU; fused 128
    dict(B=43, T=37, H=3, seed=224),                              # 129 equal pairs: 1 tile of 128 columns
    dict(B=64, T=20, H=2, seed=225),                              # 128 equal pairs: 2 tiles
]


@pytest.mark.parametrize("path,chunk", VARIANTS, ids=VARIANT_IDS)
@pytest.mark.parametrize("i", range(len(TILING_CASES)))
def test_tiling_boundaries(i, path, chunk):
    kw = dict(TILING_CASES[i])
    inp = make_inputs(state_dtype="bf16", **kw)
    check(inp, tag="tiling%d" % i, chunk=chunk, path=path)


_MANY = [int(x) for x in np.random.default_rng(305).integers(0, 13, size=1100)]
PART_CASES = [
    dict(B=2, T=300, H=3, state_dtype="fp32", lower_bound=-5.0, seed=300),
    dict(B=1, T=513, H=2, state_dtype="bf16", lower_bound=-5.0, seed=301, seq_lens=ragged_lengths(513, 9)),
    dict(B=1, T=200, H=2, state_dtype="fp32", lower_bound=-1.0, seed=302, seq_lens=[0, 3, 0, 150, 1, 46, 0]),
    dict(B=1, T=40, H=4, state_dtype=None, lower_bound=-5.0, seed=303),
    # more sequences than one scheduler scan tile (1024): the parts' bounds from the written table
    dict(B=1, T=sum(_MANY), H=1, state_dtype="fp32", lower_bound=-3.0, seed=305, seq_lens=_MANY),
]


@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("i", range(len(PART_CASES)))
def test_parts_bitwise_equal_one_part(i, chunk):
    """Cutting the rows into parts (prep of part p + 1 overlapped with the
    recurrence of part p, the state handed over in fp32) changes no bit of
    the result; part boundaries fall inside chunks, between sequences and
    inside empty sequences."""
    inp = make_inputs(**PART_CASES[i])
    d = device_inputs(inp)
    say("case parts%d B=%d T=%d H=%d N=%d chunk=%d" % (i, inp.B, inp.T, inp.H, inp.N, chunk))
    o1, f1 = run_gpu(inp, d=d, parts=1, chunk=chunk, path="split")
    torch.cuda.synchronize()
    ref_o, ref_f = oracle_run(inp)
    assert_close(to_f64(o1), ref_o, "out")
    if inp.output_final_state:
        assert_close(to_f64(f1), ref_f, "final_state", inp.state_dtype)
    for P in (2, 3, 5, 8):
        say("  parts=%d" % P)
        o, f = run_gpu(inp, d=d, parts=P, chunk=chunk, path="split")
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o1.view(torch.int16)), P
        if inp.output_final_state:
            assert torch.equal(f.view(torch.int16) if f.dtype == torch.bfloat16 else f,
                               f1.view(torch.int16) if f1.dtype == torch.bfloat16 else f1), P


def test_parts_inplace_state_and_events():
    """In-place state (initial_state is final_state) with parts, and the
    per-kernel events of kda_fwd_ex (2 + 4 P of them) all complete in order."""
    from gated_delta_rule_prep_amd import kda
    inp = make_inputs(1, 700, 2, seed=304, state_dtype="fp32")
    d = device_inputs(inp)
    say("case parts in-place + events")
    o_ref, f_ref = run_gpu(inp, d=d, parts=1, path="split")
    st = d["initial_state"].clone()
    out = torch.empty_like(o_ref)
    P = kda.parts(1, 700, 4)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 + 4 * P)]
    for e in ev:
        e.record()
    torch.cuda.synchronize()
    kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], inp.scale, out, d["A_log"], d["dt_bias"],
            inp.lower_bound, initial_state=st, final_state=st, workspace=None, events=ev, parts=4)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(st, f_ref)
    for p in range(P):
        assert ev[2 + 2 * p].elapsed_time(ev[3 + 2 * p]) >= 0
        assert ev[2 + 2 * P + 2 * p].elapsed_time(ev[3 + 2 * P + 2 * p]) >= 0
        # the recurrence of part p starts after the prep of part p ended
        assert ev[3 + 2 * p].elapsed_time(ev[2 + 2 * P + 2 * p]) >= 0
