"""fp64 CPU oracle for the KDA forward pass -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU product path
(``gated_delta_rule_prep_amd``) never imports it, and the two share no code:
the only thing both sides use is the seeded input generator, which holds none
of the method's arithmetic.

The arithmetic lives in ``kda_oracle.c`` (plain C, fp64, token by token); see
its header for what is computed and which passage of the pages each step
follows.  This module only builds that file with gcc and marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile kda_oracle.c with gcc (-O2, IEEE arithmetic, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
               "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.kda_oracle_fwd.argtypes = [p, p, p, p, p, ctypes.c_double, p, p, ctypes.c_double,
                                       p, p, p, p, i64, i64, i64, i64, i64, i64, ctypes.c_int]
        lib.kda_oracle_fwd.restype = ctypes.c_int
        lib.kda_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return _load().kda_oracle_max_threads()


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact decode of bf16 bit patterns (uint16) to fp64."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def kda_fwd(q, k, v, g, beta, scale, A_log, dt_bias, lower_bound, initial_state=None,
            output_final_state=True, cu_seqlens=None, threads: int = 0):
    """Run the oracle.

    q, k, g : uint16 bf16 bit patterns [B, T, H, K];  v : [B, T, H, V];
    beta : uint16 [B, T, H];  A_log : float32 [H];  dt_bias : float32 [H, K];
    initial_state : float64 [N, H, V, K] or None (zeros);
    cu_seqlens : int64 [N+1] or None.
    Returns (out float64 [B, T, H, V], final_state float64 [N, H, V, K] or None).
    """
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    g = np.ascontiguousarray(g, dtype=np.uint16)
    beta = np.ascontiguousarray(beta, dtype=np.uint16)
    A_log = np.ascontiguousarray(A_log, dtype=np.float32)
    dt_bias = np.ascontiguousarray(dt_bias, dtype=np.float32)
    B, T, H, K = q.shape
    V = v.shape[-1]
    assert k.shape == q.shape and g.shape == q.shape and v.shape == (B, T, H, V)
    assert beta.shape == (B, T, H) and A_log.shape == (H,) and dt_bias.shape == (H, K)
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
        N = cu.shape[0] - 1
        assert B == 1
    else:
        cu = None
        N = B
    s0 = None
    if initial_state is not None:
        s0 = np.ascontiguousarray(initial_state, dtype=np.float64)
        assert s0.shape == (N, H, V, K)
    out = np.zeros((B, T, H, V), dtype=np.float64)
    fin = np.zeros((N, H, V, K), dtype=np.float64) if output_final_state else None
    rc = lib.kda_oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale),
                            _ptr(A_log), _ptr(dt_bias), float(lower_bound), _ptr(s0), _ptr(out),
                            _ptr(fin), _ptr(cu), N, B, T, H, K, V, int(threads))
    if rc != 0:
        raise ValueError("kda_oracle_fwd failed with code %d" % rc)
    return out, fin
