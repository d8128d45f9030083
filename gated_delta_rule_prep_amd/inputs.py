"""Seeded synthetic inputs for the KDA forward pass.

This module holds no arithmetic of the method: it only draws random numbers,
rounds them to the storage dtypes the kernel API fixes and builds cu_seqlens.
Both the fp64 oracle (test infrastructure) and the HIP path are fed from here.

Shapes and dtypes follow the kernel API table of the FlashKDA README mirror
(section "内核 API"): q, k, g bf16 [B, T, H, K]; v bf16 [B, T, H, V]; beta bf16
[B, T, H]; A_log fp32 [H]; dt_bias fp32 [H, K]; states bf16 or fp32
[B|N, H, V, K]; cu_seqlens int64 [N + 1].

Draw recipe (one numpy PCG64 generator per input set, seeded by the caller):
  q, k, v, g, beta  : float32 standard normal x std (std 1; g may use another)
  A_log             : log(U[1, 16]) per head, fp32
  dt_bias           : 0.1 x standard normal, fp32 [H, K]
  initial state     : 0.05 x standard normal, rounded to the state dtype
drawn in exactly that order; bf16 values are fp32 rounded to nearest even and
kept as uint16 bit patterns.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

BF16 = "bf16"
FP32 = "fp32"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    r = (u + np.uint32(0x7FFF) + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class KDAInputs:
    q: np.ndarray            # uint16 bf16 bits [B, T, H, K]
    k: np.ndarray            # uint16 bf16 bits [B, T, H, K]
    v: np.ndarray            # uint16 bf16 bits [B, T, H, V]
    g: np.ndarray            # uint16 bf16 bits [B, T, H, K]
    beta: np.ndarray         # uint16 bf16 bits [B, T, H]
    A_log: np.ndarray        # float32 [H]
    dt_bias: np.ndarray      # float32 [H, K]
    scale: float
    lower_bound: float
    state_dtype: Optional[str]            # None, "bf16" or "fp32"
    initial_state: Optional[np.ndarray]   # uint16 bits or float32, [N, H, V, K]; None if absent
    output_final_state: bool
    cu_seqlens: Optional[np.ndarray]      # int64 [N + 1] or None
    name: str = ""

    @property
    def B(self) -> int:
        return self.q.shape[0]

    @property
    def T(self) -> int:
        return self.q.shape[1]

    @property
    def H(self) -> int:
        return self.q.shape[2]

    @property
    def K(self) -> int:
        return self.q.shape[3]

    @property
    def V(self) -> int:
        return self.v.shape[3]

    @property
    def N(self) -> int:
        return self.B if self.cu_seqlens is None else len(self.cu_seqlens) - 1

    def initial_state_f64(self) -> Optional[np.ndarray]:
        """The initial state widened (exactly) to fp64, or None."""
        if self.initial_state is None:
            return None
        if self.state_dtype == BF16:
            return bf16_bits_to_f32(self.initial_state).astype(np.float64)
        return self.initial_state.astype(np.float64)


def make_inputs(B: int, T: int, H: int, K: int = 128, V: int = 128, seed: int = 0,
                g_std: float = 1.0, lower_bound: float = -5.0, scale: Optional[float] = None,
                state_dtype: Optional[str] = None, initial_state: bool = True,
                output_final_state: bool = True, seq_lens: Optional[List[int]] = None,
                name: str = "") -> KDAInputs:
    """Draw one seeded input set (recipe in the module docstring).

    seq_lens: if given, B must be 1 and sum(seq_lens) == T; cu_seqlens is built
    from it.  state_dtype None means no state in or out.
    """
    rng = np.random.default_rng(seed)

    def draw(shape, std):
        return (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)

    q = f32_to_bf16_bits(draw((B, T, H, K), 1.0))
    k = f32_to_bf16_bits(draw((B, T, H, K), 1.0))
    v = f32_to_bf16_bits(draw((B, T, H, V), 1.0))
    g = f32_to_bf16_bits(draw((B, T, H, K), g_std))
    beta = f32_to_bf16_bits(draw((B, T, H), 1.0))
    A_log = np.log(rng.uniform(1.0, 16.0, size=H)).astype(np.float32)
    dt_bias = draw((H, K), 0.1)
    cu = None
    if seq_lens is not None:
        assert B == 1 and sum(seq_lens) == T
        cu = np.zeros(len(seq_lens) + 1, dtype=np.int64)
        cu[1:] = np.cumsum(np.asarray(seq_lens, dtype=np.int64))
    N = B if cu is None else len(cu) - 1
    s0 = None
    if state_dtype is not None and initial_state:
        x = draw((N, H, V, K), 0.05)
        s0 = f32_to_bf16_bits(x) if state_dtype == BF16 else x
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    return KDAInputs(q=q, k=k, v=v, g=g, beta=beta, A_log=A_log, dt_bias=dt_bias, scale=float(scale),
                     lower_bound=float(lower_bound), state_dtype=state_dtype, initial_state=s0,
                     output_final_state=(state_dtype is not None and output_final_state),
                     cu_seqlens=cu, name=name)


def ragged_lengths(total: int = 8192, seed: int = 1004) -> List[int]:
    """Twelve sequence lengths summing to `total`.

    [1, 15, 17] plus eight log-uniform draws over [1, 2048], shuffled, then a
    last length that makes the sum `total` (redrawn if it would be < 1).
    """
    rng = np.random.default_rng(seed)
    while True:
        draws = np.clip(np.floor(np.exp(rng.uniform(0.0, math.log(2048.0), size=8))), 1, 2048)
        lens = [1, 15, 17] + [int(x) for x in draws]
        rng.shuffle(lens)
        last = total - sum(lens)
        if last >= 1:
            return lens + [last]


@dataclass
class Config:
    index: int
    name: str
    B: int
    T: int
    H: int
    state_dtype: Optional[str]
    initial_state: bool
    lower_bound: float
    g_std: float
    seq_lens: Optional[List[int]] = field(default=None)

    def make(self, K: int = 128, V: int = 128) -> KDAInputs:
        return make_inputs(self.B, self.T, self.H, K=K, V=V, seed=self.index, g_std=self.g_std,
                           lower_bound=self.lower_bound, state_dtype=self.state_dtype,
                           initial_state=self.initial_state, seq_lens=self.seq_lens, name=self.name)

    @property
    def token_heads(self) -> int:
        return self.B * self.T * self.H


def configs() -> List[Config]:
    """The five workloads: a tiny one, two fixed-length and two varlen ones."""
    return [
        Config(0, "T64_H1_fixed_nostate_in", 1, 64, 1, FP32, False, -5.0, 1.0),
        Config(1, "T8192_H64_fixed_fp32state", 1, 8192, 64, FP32, True, -5.0, 1.0),
        Config(2, "T8192_H96_fixed_bf16state", 1, 8192, 96, BF16, True, -5.0, 1.0),
        Config(3, "T8192_H96_varlen8x1024_bf16state", 1, 8192, 96, BF16, True, -5.0, 1.0, [1024] * 8),
        Config(4, "T8192_H96_ragged12_fp32state_lb-2_gstd2", 1, 8192, 96, FP32, True, -2.0, 2.0,
               ragged_lengths()),
    ]
