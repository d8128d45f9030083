"""``chunk_kda``-shaped entry point over ``kda.fwd`` (argument mapping only).

The FlashKDA README mirror (section "依赖要求", step 2) shows the call site
that models already have: flash-linear-attention's ``chunk_kda`` with the
flags ``use_gate_in_kernel``, ``use_qk_l2norm_in_kernel``,
``use_beta_sigmoid_in_kernel``, ``safe_gate`` and ``transpose_state_layout``
all set, ``A_log`` / ``dt_bias`` / ``lower_bound`` given, and the result
returned as ``(out, final_state)``.  This function accepts exactly that
configuration and runs it on the HIP kernels behind ``kda_fwd``.  There is no
dispatch: a flag value the kernels do not implement (the gate, the L2 norms or
the beta sigmoid computed outside, a gate other than the bounded one, the
state in [K, V] order) raises ``ValueError`` naming it, never a fallback to
another implementation.

What each flag means for the kernels:
  use_gate_in_kernel         g is the raw gate; the kernel applies
                             lower_bound * sigmoid(exp(A_log) * (g + dt_bias))
  safe_gate                  that bounded form (decay in [lower_bound, 0])
  use_qk_l2norm_in_kernel    q and k are L2-normalised in the kernel
  use_beta_sigmoid_in_kernel beta is the raw logit; the kernel applies sigmoid
  transpose_state_layout     states are [N, H, V, K] (K contiguous)
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import torch

from . import kda


def _reject(reason: str):
    raise kda.KDAValueError(kda.KDA_EINVAL, "chunk_kda rejected: " + reason)


def chunk_kda(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
              scale: Optional[float] = None, initial_state: Optional[torch.Tensor] = None,
              output_final_state: bool = False, use_gate_in_kernel: bool = False,
              use_qk_l2norm_in_kernel: bool = False, use_beta_sigmoid_in_kernel: bool = False,
              safe_gate: bool = False, A_log: Optional[torch.Tensor] = None,
              dt_bias: Optional[torch.Tensor] = None, lower_bound: Optional[float] = None,
              transpose_state_layout: bool = False, cu_seqlens: Optional[torch.Tensor] = None,
              final_state_dtype: Optional[torch.dtype] = None, chunk: Optional[int] = None
              ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Forward KDA in the ``chunk_kda`` calling convention.

    q, k, g: bf16 [B, T, H, 128]; v: bf16 [B, T, H, 128]; beta: bf16 [B, T, H];
    A_log: fp32 [H]; dt_bias: fp32 [H, 128]; lower_bound in [-5, 0];
    initial_state: None or bf16 / fp32 [N, H, V, K]; cu_seqlens: None or int64
    [N + 1] (then B == 1).  ``scale`` defaults to K^-1/2.  Returns ``(out,
    final_state)``: out bf16 [B, T, H, V]; final_state [N, H, V, K] in the
    dtype of initial_state (``final_state_dtype`` when there is none, fp32 by
    default) if ``output_final_state``, else None.  ``chunk``: None for the
    library's chunk size, or 16 / 32 / 64.  Runs on the current stream.
    """
    if not use_gate_in_kernel:
        _reject("use_gate_in_kernel=False (the kernels take the raw gate g)")
    if not safe_gate:
        _reject("safe_gate=False (the kernels implement the bounded gate only)")
    if not use_qk_l2norm_in_kernel:
        _reject("use_qk_l2norm_in_kernel=False (the kernels L2-normalise q and k)")
    if not use_beta_sigmoid_in_kernel:
        _reject("use_beta_sigmoid_in_kernel=False (the kernels take the beta logit)")
    if not transpose_state_layout:
        _reject("transpose_state_layout=False (states are [N, H, V, K])")
    if A_log is None or dt_bias is None:
        _reject("A_log and dt_bias are required with use_gate_in_kernel")
    if lower_bound is None:
        _reject("lower_bound is required with safe_gate")
    if q.dim() != 4:
        _reject("q must be [B, T, H, K]")
    B, T, H, K = q.shape
    V = v.shape[-1]
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    out = torch.empty((B, T, H, V), dtype=torch.bfloat16, device=q.device)
    final = None
    if output_final_state:
        if initial_state is not None:
            fdt = initial_state.dtype
        else:
            fdt = torch.float32 if final_state_dtype is None else final_state_dtype
        final = torch.empty((N, H, V, K), dtype=fdt, device=q.device)
    kda.fwd(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state=initial_state,
            final_state=final, cu_seqlens=cu_seqlens, chunk=chunk)
    return out, final
