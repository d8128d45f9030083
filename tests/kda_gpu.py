"""Helpers for the GPU parity tests: move seeded inputs to the device, run the
HIP path through the C ABI, and score a result against the fp64 oracle.

Tolerances (stated with the method's contract): for `out` and for the final
state, separately,
  max |x - y| <= 2e-2 * RMS(y)          (RMS over the whole tensor)
  sum |x - y| / sum |y| <= 5e-3
where y is the fp64 oracle (not rounded) and x the GPU result widened to fp64.

Reading of the max bound for a result stored in a 16-bit type: a correctly
rounded bf16 value is already up to half an ulp (|y| * 2^-9) away from y, and
on heavy-tailed outputs (|y| > 10 RMS) that alone exceeds 2e-2 * RMS.  So the
max bound is applied per element on top of half an ulp of the stored dtype:
  |x_i - y_i| <= 2e-2 * RMS(y) + ulp_dtype(y_i) / 2.
The unadjusted max |x - y| / RMS and the floor max |bf16(y) - y| / RMS (what a
correctly rounded result would score) are printed next to every check.
"""
import sys

import numpy as np
import torch

MAX_ABS_TOL = 2e-2
MEAN_REL_TOL = 5e-3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_tensor(bits: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def device_inputs(inp, device="cuda"):
    d = dict(q=bf16_tensor(inp.q, device), k=bf16_tensor(inp.k, device), v=bf16_tensor(inp.v, device),
             g=bf16_tensor(inp.g, device), beta=bf16_tensor(inp.beta, device),
             A_log=torch.from_numpy(inp.A_log).to(device), dt_bias=torch.from_numpy(inp.dt_bias).to(device))
    d["cu_seqlens"] = None if inp.cu_seqlens is None else torch.from_numpy(inp.cu_seqlens).to(device)
    s0 = None
    if inp.initial_state is not None:
        s0 = (bf16_tensor(inp.initial_state, device) if inp.state_dtype == "bf16"
              else torch.from_numpy(inp.initial_state).to(device))
    d["initial_state"] = s0
    return d


def state_torch_dtype(inp):
    return torch.bfloat16 if inp.state_dtype == "bf16" else torch.float32


# (path, chunk) variants of kda_fwd_ex that the parity tests cover
VARIANTS = [("fused", 16), ("split", 16), ("split", 32), ("split", 64)]
VARIANT_IDS = ["%s%d" % v for v in VARIANTS]


def run_gpu(inp, device="cuda", d=None, workspace=None, out=None, final=None, parts=None, chunk=None, path=None):
    from gated_delta_rule_prep_amd import kda
    if d is None:
        d = device_inputs(inp, device)
    B, T, H, V = inp.B, inp.T, inp.H, inp.V
    if out is None:
        out = torch.full((B, T, H, V), float("nan"), dtype=torch.bfloat16, device=device)
    if final is None and inp.output_final_state:
        final = torch.full((inp.N, H, V, inp.K), float("nan"), dtype=state_torch_dtype(inp), device=device)
    kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], inp.scale, out, d["A_log"], d["dt_bias"],
            inp.lower_bound, initial_state=d["initial_state"], final_state=final,
            cu_seqlens=d["cu_seqlens"], workspace=workspace, parts=parts, chunk=chunk, path=path)
    return out, final


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def bf16_round(y: np.ndarray) -> np.ndarray:
    return torch.from_numpy(y).to(torch.bfloat16).to(torch.float64).numpy()


def half_ulp(y: np.ndarray, dtype: str) -> np.ndarray:
    """Half the spacing of `dtype` ("bf16" or "fp32") at |y| (0 at y = 0)."""
    mbits = 8 if dtype == "bf16" else 24
    _, e = np.frexp(np.abs(y))          # |y| = m 2^e, m in [0.5, 1)
    return np.where(y == 0, 0.0, np.ldexp(1.0, e - 1 - mbits))


def score(x: np.ndarray, y: np.ndarray, dtype: str = "bf16") -> dict:
    err = np.abs(x - y)
    rms = float(np.sqrt(np.mean(y * y))) if y.size else 0.0
    fl = np.abs(bf16_round(y) - y)
    sy = float(np.abs(y).sum())
    adj = err - half_ulp(y, dtype)
    return dict(max_over_rms=float(err.max() / rms) if y.size and rms > 0 else 0.0,
                adj_max_over_rms=float(max(adj.max(), 0.0) / rms) if y.size and rms > 0 else 0.0,
                mean_rel=float(err.sum() / sy) if sy > 0 else float(err.sum()),
                floor_max_over_rms=float(fl.max() / rms) if y.size and rms > 0 else 0.0,
                floor_mean_rel=float(fl.sum() / sy) if sy > 0 else 0.0,
                finite=bool(np.all(np.isfinite(x))))


def assert_close(x, y, what, dtype="bf16"):
    s = score(x, y, dtype)
    say("  %-12s max|err|/RMS %.3e (beyond half-ulp %.3e; bf16 floor %.3e)  mean rel %.3e (floor %.3e)" % (
        what, s["max_over_rms"], s["adj_max_over_rms"], s["floor_max_over_rms"], s["mean_rel"],
        s["floor_mean_rel"]))
    assert s["finite"], "%s has non-finite values" % what
    assert s["adj_max_over_rms"] <= MAX_ABS_TOL, (what, s)
    assert s["mean_rel"] <= MEAN_REL_TOL, (what, s)
    return s
