"""GPU parity past 4 GiB: one varlen batch whose token tensors (q, k, v, g,
out: 180 224 tokens x 96 heads x 128 bf16 = 4.43 GB each) and chunk records
(about 15 GB) reach past byte offset 2^32, so every address the kernels form
has to be 64-bit.

Sequences: 300 tokens, then one long sequence of 179 624 tokens, then 300
tokens that end at the last row.  Rows [0, 600) and the last 300 rows come
from the seeded input generator (a 900-token batch of three 300-token
sequences); the rest is seeded GPU noise of the same distribution.  An output
at step t of a sequence depends only on the sequence's tokens up to t, so the
oracle run on the 900-token batch gives the exact values of the first
sequence, the first 300 outputs of the long one and the whole last sequence
(with the final states of the first and last); these are compared on four
heads, and everything else must be finite.
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_prep_amd.inputs import make_inputs
from tests.kda_gpu import VARIANT_IDS, VARIANTS, assert_close, bf16_tensor, say, to_f64
from tests.test_gpu_parity import oracle_run

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

H = 96
T_BIG = 180224   # 11 x 16384 tokens
EDGE = 300
HEADS = [0, 1, 47, 95]


@pytest.fixture(scope="module")
def big_batch():
    small = make_inputs(1, 3 * EDGE, H, seed=600, state_dtype="fp32", seq_lens=[EDGE] * 3)
    T = T_BIG
    assert T * H * 128 * 2 > 2 ** 32
    gen = torch.Generator(device="cuda")
    gen.manual_seed(601)

    def token_tensor(bits, shape):
        x = torch.empty(shape, dtype=torch.bfloat16, device="cuda").normal_(generator=gen)
        x[0, :2 * EDGE] = bf16_tensor(bits[0, :2 * EDGE], "cuda")
        x[0, T - EDGE:] = bf16_tensor(bits[0, 2 * EDGE:], "cuda")
        return x

    d = dict(q=token_tensor(small.q, (1, T, H, 128)), k=token_tensor(small.k, (1, T, H, 128)),
             v=token_tensor(small.v, (1, T, H, 128)), g=token_tensor(small.g, (1, T, H, 128)),
             beta=token_tensor(small.beta, (1, T, H)),
             A_log=torch.from_numpy(small.A_log).cuda(), dt_bias=torch.from_numpy(small.dt_bias).cuda(),
             initial_state=torch.from_numpy(small.initial_state).cuda(),
             cu_seqlens=torch.tensor([0, EDGE, T - EDGE, T], dtype=torch.int64, device="cuda"))
    ref_o, ref_f = oracle_run(small, HEADS)
    yield small, d, ref_o, ref_f
    del d
    torch.cuda.empty_cache()


@pytest.mark.parametrize("path,chunk", VARIANTS, ids=VARIANT_IDS)
def test_offsets_past_4gib(big_batch, path, chunk):
    from gated_delta_rule_prep_amd import kda
    small, d, ref_o, ref_f = big_batch
    T = T_BIG
    say("case past 4 GiB: T=%d H=%d N=3 path=%s chunk=%d" % (T, H, path, chunk))
    out = torch.full((1, T, H, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    fin = torch.full((3, H, 128, 128), float("nan"), dtype=torch.float32, device="cuda")
    kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], small.scale, out, d["A_log"], d["dt_bias"],
            small.lower_bound, initial_state=d["initial_state"], final_state=fin, cu_seqlens=d["cu_seqlens"],
            path=path, chunk=chunk)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(fin).all())
    got = np.concatenate([to_f64(out[:, :2 * EDGE, HEADS]), to_f64(out[:, T - EDGE:, HEADS])], axis=1)
    assert_close(got, ref_o, "out (first 600 and last 300 rows)")
    assert_close(to_f64(fin[[0, 2]][:, HEADS]), ref_f[[0, 2]], "final_state (first and last sequence)", "fp32")
    del out, fin
