"""GPU unit test of the scheduler and chunk-prep kernels alone, for 16-, 32-
and 64-token chunks: the chunk table and every chunk record are decoded from the
workspace and compared with the fp64 chunked-form intermediates of
tests/chunked_ref.py."""
import numpy as np
import pytest
import torch

from gated_delta_rule_prep_amd.inputs import make_inputs
from tests import chunked_ref
from tests.kda_gpu import device_inputs, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

EPS = 1e-6
# stored gamma slot of channel c = 64 r + 16 a + 4 b + i (record layout in include/kda.h)
GAM_SLOT = np.array([2 * (16 * ((c >> 2) & 3) + 4 * ((c >> 4) & 3) + (c & 3)) + (c >> 6) for c in range(128)])


def perm_ch(p):
    j, g = p % 8, p // 8
    return 4 * g + j if j < 4 else 16 + 4 * g + j - 4


PERM = np.array([(p // 32) * 32 + perm_ch(p % 32) for p in range(128)])
PERM32 = np.array([perm_ch(p) for p in range(32)])


def unpermute(x, perm=PERM):
    y = np.empty_like(x)
    y[..., perm] = x
    return y


def decode_record(rec, C):
    """Record fields as natural-order float64 arrays (layouts in include/kda.h)."""
    f16 = lambda o, shape: rec[o:o + 2 * int(np.prod(shape))].view(np.float16).astype(np.float64).reshape(shape)
    gam = lambda o: rec[o:o + 512].view(np.float32).astype(np.float64)[GAM_SLOT]
    if C == 16:   # the 16-token record holds -Khat (the recurrence forms T (V - Khat Z))
        return dict(Qh=unpermute(f16(0, (16, 128))), Kh=-unpermute(f16(4096, (16, 128))), Kb=f16(8192, (16, 128)),
                    T=f16(12288, (16, 16)).T, M=f16(12800, (16, 16)).T, gamma=gam(13312))
    if C == 32:
        return dict(Qh=unpermute(f16(0, (32, 128))), W=-unpermute(f16(8192, (32, 128))), Kb=f16(16384, (32, 128)),
                    T=unpermute(f16(24576, (32, 32)), PERM32), M=unpermute(f16(26624, (32, 32)), PERM32),
                    gamma=gam(28672))

    def blocked(o):   # 8 blocks of 16 rows x 32 token columns (kPermCh order), block (t, u) at (2t + u) KB
        m = np.empty((64, 64))
        for t in range(4):
            for u in range(2):
                m[16 * t:16 * t + 16, 32 * u:32 * u + 32] = unpermute(f16(o + (2 * t + u) * 1024, (16, 32)), PERM32)
        return m
    return dict(Qh=unpermute(f16(0, (64, 128))), W=-unpermute(f16(16384, (64, 128))), Kb=f16(32768, (64, 128)),
                T=blocked(49152), M=blocked(57344), gamma=gam(65536))


def check_tables(buf, lay, lens, cu, C):
    """The scheduler's chunk table, sequence table and work order, exactly;
    returns the chunk table's entries."""
    hdr = buf[:8].view(np.int32)
    nch = sum((l + C - 1) // C for l in lens)
    assert hdr[1] == nch
    table = buf[lay["chunk_table"]:lay["chunk_table"] + 12 * nch].view(np.int32).reshape(nch, 3)
    want = []
    for n, l in enumerate(lens):
        for c in range(0, l, C):
            want.append((n, int(cu[n]) + c, min(C, l - c)))
    assert [tuple(r) for r in table] == want
    seqs = buf[lay["seq_table"]:lay["seq_table"] + 16 * len(lens)].view(np.int32).reshape(-1, 4)
    order = buf[lay["order"]:lay["order"] + 4 * len(lens)].view(np.int32)
    assert list(seqs[:, 1]) == [(l + C - 1) // C for l in lens]
    assert list(seqs[:, 2]) == [int(x) for x in cu[:-1]] and list(seqs[:, 3]) == list(lens)
    assert list(seqs[:, 0]) == [sum((l + C - 1) // C for l in lens[:n]) for n in range(len(lens))]
    assert sorted(order) == list(range(len(lens)))
    counts = [seqs[n, 1] for n in order]
    assert counts == sorted(counts, reverse=True)               # longest first
    if len(lens) <= 2048:                                        # ties in index order
        keyed = [(-seqs[n, 1], n) for n in order]
        assert keyed == sorted(keyed)
    return want


@pytest.mark.parametrize("N", [40, 300, 1300])
def test_scheduler_tables_many_sequences(N):
    """The scheduler's tables for one wave's worth of sequences, one block's
    and more than one scan tile (1024 sequences per tile), with empty
    sequences among them."""
    from gated_delta_rule_prep_amd import kda
    rng = np.random.default_rng(320 + N)
    lens = [int(x) for x in rng.integers(0, 40, size=N)]
    T = sum(lens)
    inp = make_inputs(1, T, 1, seed=321, lower_bound=-5.0, seq_lens=lens)
    say("case scheduler tables N=%d T=%d" % (N, T))
    d = device_inputs(inp)
    ws = kda.debug_prep(d["q"], d["k"], d["g"], d["beta"], inp.scale, d["A_log"], d["dt_bias"], inp.lower_bound,
                        cu_seqlens=d["cu_seqlens"], chunk=16)
    torch.cuda.synchronize()
    lay = kda.workspace_layout(1, T, 1, N, True, chunk=16)
    buf = ws.cpu().numpy()
    assert buf[:4].view(np.int32)[0] == kda.KDA_STATUS_OK
    check_tables(buf, lay, lens, inp.cu_seqlens, 16)


@pytest.mark.parametrize("C", [16, 32, 64])
def test_chunk_table_and_records_match_chunked_form(C):
    from gated_delta_rule_prep_amd import kda
    lens = [1, 15, 17, 40, 0, 33, 64] + ([50, 130] if C == 64 else [])
    T = sum(lens)
    H = 3
    inp = make_inputs(1, T, H, seed=300, lower_bound=-5.0, seq_lens=lens)
    say("case prep records C=%d lens=%s H=%d" % (C, lens, H))
    d = device_inputs(inp)
    ws = kda.debug_prep(d["q"], d["k"], d["g"], d["beta"], inp.scale, d["A_log"], d["dt_bias"], inp.lower_bound,
                        cu_seqlens=d["cu_seqlens"], chunk=C)
    torch.cuda.synchronize()
    lay = kda.workspace_layout(1, T, H, len(lens), True, chunk=C)
    assert lay["rec_bytes"] == {16: 13824, 32: 29184, 64: 66048}[C]
    buf = ws.cpu().numpy()
    hdr = buf[:8].view(np.int32)
    assert hdr[0] == kda.KDA_STATUS_OK
    cu = inp.cu_seqlens
    want = check_tables(buf, lay, lens, cu, C)

    f = chunked_ref.decode_bf16
    qf, kf, gf, bf = f(inp.q)[0], f(inp.k)[0], f(inp.g)[0], f(inp.beta)[0]
    R = lay["rec_bytes"]
    worst = {}
    for h in range(H):
        A = np.exp(np.float64(inp.A_log[h]))
        for ci, (n, r0, ln) in enumerate(want):
            sl = slice(r0, r0 + ln)
            a = inp.lower_bound / (1 + np.exp(-A * (gf[sl, h] + inp.dt_bias[h].astype(np.float64))))
            kk, qq = kf[sl, h], qf[sl, h]
            kn = kk / np.sqrt((kk * kk).sum(-1, keepdims=True) + EPS)
            qn = inp.scale * qq / np.sqrt((qq * qq).sum(-1, keepdims=True) + EPS)
            P = chunked_ref.chunk_pieces(qn, kn, a, 1 / (1 + np.exp(-bf[sl, h])))
            off = lay["records"] + (ci * H + h) * R   # chunk-major
            full = decode_record(buf[off:off + R], C)
            got = {k: (v if k == "gamma" else v[:ln, :ln] if k in ("T", "M") else v[:ln]) for k, v in full.items()}
            ref = dict(Qh=P["Qh"], Kb=P["Kb"], T=P["T"], M=P["M"], gamma=P["gamma"])
            if C == 16:
                ref["Kh"] = P["Kh"]
            else:
                ref["W"] = P["T"] @ P["Kh"]
            # padded rows / columns of a partial chunk are exactly zero
            for key in ("Qh", "Kh" if C == 16 else "W", "Kb", "T", "M"):
                assert np.all(full[key][ln:] == 0), key
            assert np.all(full["T"][:, ln:] == 0) and np.all(full["M"][:, ln:] == 0)
            # structure: T lower triangular, Mqk lower triangular incl. diagonal
            assert np.all(np.triu(got["T"], 1) == 0) and np.all(np.triu(got["M"], 1) == 0)
            for key in ref:
                e = np.abs(got[key] - ref[key]).max() / max(np.abs(ref[key]).max(), 1e-30)
                worst[key] = max(worst.get(key, 0.0), e)
    say("  worst relative max error per record field: %s" % {k: "%.2e" % v for k, v in worst.items()})
    assert worst["Qh"] < 2e-3 and worst["Kb"] < 2e-3 and worst["gamma"] < 1e-5
    assert worst["T"] < 1e-2 and worst["M"] < 1e-2
    assert worst["Kh"] < 2e-3 if C == 16 else worst["W"] < 1e-2
