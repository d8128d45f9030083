"""Pins of the fp64 oracle against closed forms, invariants and a second
implementation (CPU only).

Page key: P1 = blog post "FlashKDA：月之暗面开源的 Kimi Delta Attention 高性能内核";
P2 = FlashKDA README mirror, section "内核 API" (Kernel API).

The pages print no worked numerical example, so every pin here is a closed
form derived by hand, an exact invariant, a library special case, or a
brute-force second implementation (tests/chunked_ref.py).  Each is chosen so a
plausible slip in the oracle (a dropped term, a wrong sign or index, a
transposed state, read-out before the update, beta on the wrong factor, the
gate on the wrong axis) fails at least one of them.
"""
import math

import numpy as np
import pytest

import oracle
from gated_delta_rule_prep_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits, make_inputs, ragged_lengths
from tests import chunked_ref

EPS = 1e-6


def bits(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def run(inp, **kw):
    return oracle.kda_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, inp.A_log, inp.dt_bias,
                          inp.lower_bound, initial_state=inp.initial_state_f64(),
                          output_final_state=True, cu_seqlens=inp.cu_seqlens, **kw)


def rel(x, y):
    return np.abs(x - y).max() / max(np.abs(y).max(), 1e-300)


def blank(T, H=1, K=8, V=8, B=1):
    """All-zero bit patterns of the right shapes, to be filled by a test."""
    return dict(q=np.zeros((B, T, H, K), np.uint16), k=np.zeros((B, T, H, K), np.uint16),
                v=np.zeros((B, T, H, V), np.uint16), g=np.zeros((B, T, H, K), np.uint16),
                beta=np.zeros((B, T, H), np.uint16), A_log=np.zeros(H, np.float32),
                dt_bias=np.zeros((H, K), np.float32))


def call(d, scale, lb, s0=None, cu=None):
    return oracle.kda_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale, d["A_log"], d["dt_bias"], lb,
                          initial_state=s0, output_final_state=True, cu_seqlens=cu)


# ---------------------------------------------------------------- decoding
def test_bf16_decode_known_patterns():
    pats = np.array([0x3F80, 0xC000, 0x7F7F, 0x0001, 0x8000, 0x4049], dtype=np.uint16)
    want = [1.0, -2.0, (2 - 2 ** -7) * 2.0 ** 127, 2.0 ** -133, -0.0, 3.140625]
    got = oracle.bf16_bits_to_f64(pats)
    assert list(got) == want
    # round-to-nearest-even encode used by the input generator
    assert list(bits([1.0, 1.00390625, 1.01171875, -2.0])) == [0x3F80, 0x3F80, 0x3F82, 0xC000]


# ---------------------------------------------------------------- closed forms
def test_single_token_closed_form():
    """T = 1, no initial state: S = beta kn v^T, o = beta <kn, qn> v (read-out after update)."""
    d = blank(1)
    q = np.zeros(8); q[0], q[1] = 3.0, 4.0           # |q| = 5
    k = np.zeros(8); k[0] = 2.0                      # |k| = 2
    v = np.arange(1, 9, dtype=np.float64) * 0.25     # exact in bf16
    d["q"][0, 0, 0] = bits(q); d["k"][0, 0, 0] = bits(k); d["v"][0, 0, 0] = bits(v)
    d["beta"][0, 0, 0] = bits([0.0])[0]                 # sigmoid(0) = 1/2
    scale = 0.5
    out, fin = call(d, scale, -5.0)
    kq = (3.0 * 2.0) / (math.sqrt(25 + EPS) * math.sqrt(4 + EPS))
    np.testing.assert_allclose(out[0, 0, 0], scale * 0.5 * kq * v, rtol=1e-14)
    want_fin = np.zeros((8, 8))
    want_fin[:, 0] = 0.5 * (2.0 / math.sqrt(4 + EPS)) * v   # stored [v, k]
    np.testing.assert_allclose(fin[0, 0], want_fin, rtol=1e-14, atol=0)


def test_pure_decay_closed_form():
    """beta -> 0: S_t = diag(e^{a_t}) S_{t-1}; special gates with hand-known values.

    channel 0,4: g = +1e4  -> a = lower_bound
    channel 1,5: g = -1e4  -> a = 0
    channel 2,6: g = 0     -> a = lower_bound / 2   (sigmoid(0) = 1/2)
    channel 3,7: g = 1, A = ln 3 -> a = 3/4 lower_bound (sigmoid(ln 3) = 3/4)
    (channel 7 instead takes g = 0 and dt_bias = 1: the bias adds to g.)
    """
    T, lb = 5, -1.5
    d = blank(T)
    gch = np.array([1e4, -1e4, 0.0, 1.0, 1e4, -1e4, 0.0, 0.0])
    d["g"][0, :, 0, :] = bits(gch)[None, :]
    d["dt_bias"][0, 7] = 1.0
    d["A_log"][0] = np.float32(math.log(math.log(3.0)))
    A = float(np.exp(np.float64(d["A_log"][0])))
    d["beta"][0, :, 0] = bits([-1e4])[0]
    act = np.array([lb, 0.0, lb / 2, lb / (1 + 3.0 ** -(A / math.log(3.0))), lb, 0.0, lb / 2,
                    lb / (1 + 3.0 ** -(A / math.log(3.0)))])
    # A is ln 3 up to fp32 rounding of A_log; the closed form uses the rounded A
    rng = np.random.default_rng(7)
    s0 = rng.standard_normal((1, 1, 8, 8))
    for t in range(T):
        d["q"][0, t, 0] = bits(np.eye(8)[t % 8] * 2.0)    # one-hot query on channel t
    scale = 0.75
    out, fin = call(d, scale, lb, s0=s0)
    want_fin = s0[0, 0] * np.exp(T * act)[None, :]
    np.testing.assert_allclose(fin[0, 0], want_fin, rtol=1e-13)
    for t in range(T):
        m = t % 8
        want_o = scale * 2.0 / math.sqrt(4.0 + EPS) * s0[0, 0, :, m] * math.exp((t + 1) * act[m])
        np.testing.assert_allclose(out[0, t, 0], want_o, rtol=1e-13)


def test_identity_lower_bound_zero_beta_zero():
    """lower_bound = 0 and beta -> 0 leave the state unchanged bitwise; o_t = S0^T qn_t."""
    inp = make_inputs(1, 37, 2, K=16, V=8, seed=3, state_dtype="fp32", lower_bound=0.0)
    inp.beta[:] = bits([-1e4])[0]
    out, fin = run(inp)
    s0 = inp.initial_state_f64()
    assert np.array_equal(fin, s0)
    qf = bf16_bits_to_f32(inp.q).astype(np.float64)
    qn = inp.scale * qf / np.sqrt((qf * qf).sum(-1, keepdims=True) + EPS)
    want = np.einsum("bthk,hvk->bthv", qn, s0[0])
    np.testing.assert_allclose(out, want, rtol=1e-13, atol=1e-15)


def test_delta_rule_retrieval_and_overwrite():
    """beta = 1, no decay, orthonormal keys: reading key j returns v_j; a key
    written twice keeps only the later value (the textbook delta-rule property)."""
    K = V = 8
    T = 6
    d = blank(T, K=K, V=V)
    rng = np.random.default_rng(11)
    vals = np.round(rng.standard_normal((T, V)) * 8) / 8
    keys = [0, 1, 2, 1, 3, 0]      # key 1 and key 0 rewritten later
    for t in range(T):
        d["k"][0, t, 0] = bits(np.eye(K)[keys[t]])
        d["v"][0, t, 0] = bits(vals[t])
        d["beta"][0, t, 0] = bits([1e4])[0]               # sigmoid -> 1
        d["q"][0, t, 0] = bits(np.eye(K)[keys[t]])     # read the key just written
    out, fin = call(d, 1.0, 0.0)
    for t in range(T):
        np.testing.assert_allclose(out[0, t, 0], vals[t], rtol=0, atol=1e-5)
    # final state: column k holds the last value written with key k
    last = {}
    for t in range(T):
        last[keys[t]] = vals[t]
    for kk, val in last.items():
        np.testing.assert_allclose(fin[0, 0, :, kk], val, rtol=0, atol=1e-5)
    # a key never written reads back zero
    assert np.all(fin[0, 0, :, 5] == 0)


def test_two_token_closed_form():
    """S1 = b1 k1 v1^T;  r = v2 - b1 <k2, e^{a2} k1> v1;  S2 = diag(e^{a2}) S1 + b2 k2 r^T;  o2 = S2^T q2."""
    inp = make_inputs(1, 2, 1, K=8, V=8, seed=5, lower_bound=-3.0)
    out, fin = run(inp)
    f = lambda x: bf16_bits_to_f32(x).astype(np.float64)
    q, k, v, g, b = f(inp.q)[0, :, 0], f(inp.k)[0, :, 0], f(inp.v)[0, :, 0], f(inp.g)[0, :, 0], f(inp.beta)[0, :, 0]
    A = math.exp(float(inp.A_log[0]))
    dt = inp.dt_bias[0].astype(np.float64)
    a = inp.lower_bound / (1 + np.exp(-A * (g + dt)))
    bt = 1 / (1 + np.exp(-b))
    kn = k / np.sqrt((k * k).sum(-1, keepdims=True) + EPS)
    qn = inp.scale * q / np.sqrt((q * q).sum(-1, keepdims=True) + EPS)
    e2 = np.exp(a[1])
    S1 = bt[0] * np.outer(kn[0], v[0])                   # zero initial state
    r = v[1] - bt[0] * np.dot(kn[1], e2 * kn[0]) * v[0]
    S2 = e2[:, None] * S1 + bt[1] * np.outer(kn[1], r)
    np.testing.assert_allclose(out[0, 0, 0], S1.T @ qn[0], rtol=1e-13)
    np.testing.assert_allclose(out[0, 1, 0], S2.T @ qn[1], rtol=1e-13)
    np.testing.assert_allclose(fin[0, 0], S2.T, rtol=1e-13)


def test_gate_range_and_claimed_bf16_headroom():
    """Every activated gate lies in [lower_bound, 0] (checked through the state
    with beta -> 0), and the range argument of P1 §二 2.1 holds: 16 tokens at
    lower_bound = -5 decay by at most e^-80, and e^80 is below the largest bf16."""
    inp = make_inputs(1, 16, 3, K=16, V=4, seed=9, g_std=30.0, lower_bound=-5.0, state_dtype="fp32")
    inp.beta[:] = bits([-1e4])[0]
    inp.initial_state[:] = 1.0
    _, fin = run(inp)
    assert np.all(fin <= 1.0) and np.all(fin >= math.exp(-80.0) * (1 - 1e-12))
    bf16_max = (2 - 2 ** -7) * 2.0 ** 127
    assert math.exp(80.0) < bf16_max


# ---------------------------------------------------------------- second implementation
@pytest.mark.parametrize("K,V,T,C,lb,state,seed", [
    (8, 8, 1, 16, -5.0, None, 0),
    (8, 8, 15, 3, -5.0, "fp32", 1),
    (8, 8, 17, 16, -2.0, "fp32", 2),
    (8, 8, 37, 1, -5.0, "bf16", 3),
    (16, 8, 300, 16, -5.0, "fp32", 4),
    (128, 128, 37, 16, -5.0, "bf16", 5),
    (128, 128, 300, 16, -0.5, "fp32", 6),
    (128, 128, 64, 32, -2.0, "fp32", 7),
    (128, 128, 150, 64, -5.0, "fp32", 8),
])
def test_oracle_matches_chunked_form(K, V, T, C, lb, state, seed):
    inp = make_inputs(1, T, 2, K=K, V=V, seed=seed, lower_bound=lb, state_dtype=state)
    out, fin = run(inp)
    o2, f2 = chunked_ref.chunked_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, inp.A_log,
                                     inp.dt_bias, inp.lower_bound, inp.initial_state_f64(), C=C)
    assert rel(out, o2) < 1e-12
    if state is not None:
        assert rel(fin, f2) < 1e-12


def test_oracle_matches_chunked_form_varlen():
    lens = [1, 15, 17, 40, 0, 23]
    inp = make_inputs(1, sum(lens), 2, K=16, V=16, seed=12, state_dtype="fp32", seq_lens=lens)
    out, fin = run(inp)
    o2, f2 = chunked_ref.chunked_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, inp.A_log,
                                     inp.dt_bias, inp.lower_bound, inp.initial_state_f64(),
                                     cu_seqlens=inp.cu_seqlens, C=16)
    assert rel(out, o2) < 1e-12 and rel(fin, f2) < 1e-12
    # a zero-length sequence passes its state through unchanged
    assert np.array_equal(fin[4], inp.initial_state_f64()[4])


# ---------------------------------------------------------------- inverse claims (P1 §二 2.1, 2.3)
def test_neumann_product_is_exact_inverse_and_bounded():
    inp = make_inputs(1, 16 * 24, 2, K=128, V=8, seed=21, lower_bound=-5.0)
    f = lambda x: bf16_bits_to_f32(x).astype(np.float64)
    worst = 0.0
    for h in range(2):
        for c in range(24):
            sl = slice(16 * c, 16 * c + 16)
            q, k, g, b = f(inp.q)[0, sl, h], f(inp.k)[0, sl, h], f(inp.g)[0, sl, h], f(inp.beta)[0, sl, h]
            A = math.exp(float(inp.A_log[h]))
            a = inp.lower_bound / (1 + np.exp(-A * (g + inp.dt_bias[h].astype(np.float64))))
            kn = k / np.sqrt((k * k).sum(-1, keepdims=True) + EPS)
            qn = q / np.sqrt((q * q).sum(-1, keepdims=True) + EPS)
            P = chunked_ref.chunk_pieces(qn, kn, a, 1 / (1 + np.exp(-b)))
            L = P["L"]
            assert np.all(np.triu(L) == 0)
            assert np.all(np.linalg.matrix_power(L, 16) == 0)         # nilpotent, exactly
            inv = np.linalg.inv(np.eye(16) + L)
            neu = chunked_ref.neumann_inverse(L)
            assert np.abs(neu - inv).max() < 1e-12
            worst = max(worst, np.abs(inv).max())
            assert np.all(np.abs(P["T"]) <= 1.0 + 1e-12)
    assert worst <= 1.0 + 1e-12


# ---------------------------------------------------------------- invariants
def test_resume_split_equals_one_call_bitwise():
    inp = make_inputs(1, 100, 3, K=16, V=16, seed=31, state_dtype="fp32")
    out, fin = run(inp)
    t1 = 37
    sub = lambda x, a, b: np.ascontiguousarray(x[:, a:b])
    o1, f1 = oracle.kda_fwd(sub(inp.q, 0, t1), sub(inp.k, 0, t1), sub(inp.v, 0, t1), sub(inp.g, 0, t1),
                            sub(inp.beta, 0, t1), inp.scale, inp.A_log, inp.dt_bias, inp.lower_bound,
                            initial_state=inp.initial_state_f64())
    o2, f2 = oracle.kda_fwd(sub(inp.q, t1, 100), sub(inp.k, t1, 100), sub(inp.v, t1, 100), sub(inp.g, t1, 100),
                            sub(inp.beta, t1, 100), inp.scale, inp.A_log, inp.dt_bias, inp.lower_bound,
                            initial_state=f1)
    assert np.array_equal(np.concatenate([o1, o2], axis=1), out)
    assert np.array_equal(f2, fin)


def test_varlen_equals_separate_calls_bitwise():
    lens = ragged_lengths(total=300, seed=5)
    inp = make_inputs(1, 300, 2, K=16, V=16, seed=41, state_dtype="fp32", seq_lens=lens)
    out, fin = run(inp)
    cu = inp.cu_seqlens
    for n in range(len(lens)):
        a, b = int(cu[n]), int(cu[n + 1])
        sub = lambda x: np.ascontiguousarray(x[:, a:b])
        o, f = oracle.kda_fwd(sub(inp.q), sub(inp.k), sub(inp.v), sub(inp.g), sub(inp.beta), inp.scale,
                              inp.A_log, inp.dt_bias, inp.lower_bound,
                              initial_state=inp.initial_state_f64()[n:n + 1])
        assert np.array_equal(o, out[:, a:b])
        assert np.array_equal(f[0], fin[n])


def test_batch_rows_are_independent_sequences():
    inp = make_inputs(3, 20, 2, K=16, V=8, seed=43, state_dtype="fp32")
    out, fin = run(inp)
    for b in range(3):
        sub = lambda x: np.ascontiguousarray(x[b:b + 1])
        o, f = oracle.kda_fwd(sub(inp.q), sub(inp.k), sub(inp.v), sub(inp.g), sub(inp.beta), inp.scale,
                              inp.A_log, inp.dt_bias, inp.lower_bound,
                              initial_state=inp.initial_state_f64()[b:b + 1])
        assert np.array_equal(o, out[b:b + 1]) and np.array_equal(f[0], fin[b])


def test_linearity_in_values_and_state_exact():
    """(v, S0) -> (out, final) is linear; doubling is exact in binary floating point."""
    inp = make_inputs(1, 50, 2, K=16, V=16, seed=51, state_dtype="fp32")
    out, fin = run(inp)
    s0 = inp.initial_state_f64()
    v2 = bits(2.0 * bf16_bits_to_f32(inp.v))
    o2, f2 = oracle.kda_fwd(inp.q, inp.k, v2, inp.g, inp.beta, inp.scale, inp.A_log, inp.dt_bias,
                            inp.lower_bound, initial_state=2.0 * s0)
    assert np.array_equal(o2, 2.0 * out) and np.array_equal(f2, 2.0 * fin)
    # scale multiplies the output only; the final state does not depend on q or scale
    o3, f3 = oracle.kda_fwd(inp.q[:, :, :, ::-1].copy(), inp.k, inp.v, inp.g, inp.beta, 2.0 * inp.scale,
                            inp.A_log, inp.dt_bias, inp.lower_bound, initial_state=s0)
    assert np.array_equal(f3, fin)
    o4, _ = oracle.kda_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta, 2.0 * inp.scale, inp.A_log, inp.dt_bias,
                           inp.lower_bound, initial_state=s0)
    assert np.array_equal(o4, 2.0 * out)


def test_head_and_value_permutations():
    inp = make_inputs(1, 30, 3, K=16, V=16, seed=61, state_dtype="fp32")
    out, fin = run(inp)
    s0 = inp.initial_state_f64()
    ph = [2, 0, 1]
    o, f = oracle.kda_fwd(inp.q[:, :, ph].copy(), inp.k[:, :, ph].copy(), inp.v[:, :, ph].copy(),
                          inp.g[:, :, ph].copy(), inp.beta[:, :, ph].copy(), inp.scale, inp.A_log[ph].copy(),
                          inp.dt_bias[ph].copy(), inp.lower_bound, initial_state=s0[:, ph].copy())
    assert np.array_equal(o, out[:, :, ph]) and np.array_equal(f, fin[:, ph])
    pv = np.random.default_rng(0).permutation(16)
    o, f = oracle.kda_fwd(inp.q, inp.k, inp.v[..., pv].copy(), inp.g, inp.beta, inp.scale, inp.A_log,
                          inp.dt_bias, inp.lower_bound, initial_state=s0[:, :, pv].copy())
    assert np.array_equal(o, out[..., pv]) and np.array_equal(f, fin[:, :, pv])


def test_empty_sequence_and_zero_tokens():
    inp = make_inputs(1, 0, 2, K=16, V=16, seed=71, state_dtype="fp32")
    out, fin = run(inp)
    assert out.shape == (1, 0, 2, 16)
    assert np.array_equal(fin, inp.initial_state_f64())


def test_threads_do_not_change_results():
    inp = make_inputs(1, 64, 4, K=32, V=32, seed=81, state_dtype="fp32")
    o1, f1 = run(inp, threads=1)
    o2, f2 = run(inp, threads=4)
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2)
