"""Write the stored expected values under tests/golden/ (run from the
repository root: python -m tests.golden.make_golden).

Every expected value here comes from the fp64 oracle (oracle/, the token-by-
token gated delta rule that the FlashKDA README mirror's "内核 API" section
specifies the call of, with the state update of the FlashKDA blog post §一);
the inputs come from the seeded generator.  Nothing else is called.

  kda_tiny_K4V4.json  -- a worked example small enough to read: K = V = 4,
      two sequences (2 and 4 tokens, cu_seqlens), one head, an fp32 initial
      state; every input and every output is stored.
  kda_small_K128.json -- K = V = 128 (the shape the library takes), two heads,
      two sequences of 21 and 16 tokens, a bf16 initial state; the inputs are
      the generator's (arguments stored), the outputs are stored as fixed
      samples plus whole-tensor RMS, sum and sum of squares.
"""
import json
import os

import numpy as np

import oracle
from gated_delta_rule_prep_amd.inputs import make_inputs

HERE = os.path.dirname(os.path.abspath(__file__))

TINY = dict(B=1, T=6, H=1, K=4, V=4, seed=7, state_dtype="fp32", seq_lens=[2, 4])
SMALL = dict(B=1, T=37, H=2, seed=11, state_dtype="bf16", seq_lens=[21, 16])
N_SAMPLES = 96


def run(inp):
    return oracle.kda_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, inp.A_log, inp.dt_bias,
                          inp.lower_bound, initial_state=inp.initial_state_f64(),
                          output_final_state=inp.output_final_state, cu_seqlens=inp.cu_seqlens)


def bits(a):
    return ["%04x" % int(x) for x in np.asarray(a, dtype=np.uint16).ravel()]


def floats(a):
    return [float(x) for x in np.asarray(a, dtype=np.float64).ravel()]


def sample_indices(shape, n, seed):
    rng = np.random.default_rng(seed)
    size = int(np.prod(shape))
    return sorted(int(i) for i in rng.choice(size, size=min(n, size), replace=False))


def summary(y):
    y = np.asarray(y, dtype=np.float64)
    return dict(rms=float(np.sqrt(np.mean(y * y))), sum=float(y.sum()), sumsq=float((y * y).sum()))


def tiny():
    inp = make_inputs(**TINY)
    out, fin = run(inp)
    return dict(
        about="K = V = 4, one head, cu_seqlens [0, 2, 6]; bf16 inputs as uint16 bit patterns (hex), "
              "fp32 A_log, dt_bias and initial state, fp64 outputs of the oracle",
        args=TINY, shape=dict(B=inp.B, T=inp.T, H=inp.H, K=inp.K, V=inp.V, N=inp.N),
        scale=inp.scale, lower_bound=inp.lower_bound, cu_seqlens=[int(x) for x in inp.cu_seqlens],
        q=bits(inp.q), k=bits(inp.k), v=bits(inp.v), g=bits(inp.g), beta=bits(inp.beta),
        A_log=floats(inp.A_log), dt_bias=floats(inp.dt_bias), initial_state=floats(inp.initial_state),
        out=floats(out), final_state=floats(fin))


def small():
    inp = make_inputs(**SMALL)
    out, fin = run(inp)
    io = sample_indices(out.shape, N_SAMPLES, 1)
    jf = sample_indices(fin.shape, N_SAMPLES, 2)
    return dict(
        about="inputs: gated_delta_rule_prep_amd.inputs.make_inputs(**args); out [B, T, H, V] and "
              "final_state [N, H, V, K] sampled at flat indices, with whole-tensor summaries",
        args=SMALL, out_shape=list(out.shape), final_state_shape=list(fin.shape),
        out_index=io, out_value=[float(out.ravel()[i]) for i in io], out_summary=summary(out),
        final_index=jf, final_value=[float(fin.ravel()[j]) for j in jf], final_summary=summary(fin))


def main():
    for name, make in (("kda_tiny_K4V4.json", tiny), ("kda_small_K128.json", small)):
        with open(os.path.join(HERE, name), "w") as f:
            json.dump(make(), f, indent=1)
            f.write("\n")
        print("wrote", name)


if __name__ == "__main__":
    main()
