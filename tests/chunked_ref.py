"""Brute-force chunked (WY-form) fp64 KDA forward, numpy, for small inputs.

A second, independent fp64 implementation used only to pin the token-by-token
oracle.  It reaches the same result by the chunk-parallel rewrite the pages
describe as the split between a token-parallel stage (gate activation, L2
norm, decay, the L / Mqk matrices and their inverse: P1 §二 2.2) and a
chunk-by-chunk recurrence (same section), with the chunk inverse taken by a
library solve instead of the Neumann product (P1 §二 2.1 says the 16 x 16
inverse needs no factorisation; the test of that claim is separate).

P1 = blog post "FlashKDA：月之暗面开源的 Kimi Delta Attention 高性能内核".

Per chunk of c tokens with chunk-start state Z (K x V), in fp64:
  Gam_r   = sum_{j<=r} a_j                       (per key channel)
  Qh = qn*e^Gam, Kh = kn*e^Gam, Kc = kn*e^-Gam, Kb = kn*e^(Gam_c - Gam)
  Lm = strict_lower(diag(beta) Kh Kc^T),  Mm = lower_incl(Qh Kc^T)
  Tm = (I + Lm)^-1 diag(beta),  W = Tm Kh,  U = Tm Vc
  E = U - W Z,  O = Qh Z + Mm E,  Z <- diag(e^Gam_c) Z + Kb^T E
"""
from __future__ import annotations

import numpy as np

EPS = 1e-6


def decode_bf16(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def chunk_pieces(qn, kn, a, beta):
    """Intermediates of one chunk (rows = tokens of the chunk)."""
    Gam = np.cumsum(a, axis=0)
    Qh = qn * np.exp(Gam)
    Kh = kn * np.exp(Gam)
    Kc = kn * np.exp(-Gam)
    Kb = kn * np.exp(Gam[-1][None, :] - Gam)
    Lm = np.tril(beta[:, None] * (Kh @ Kc.T), -1)
    Mm = np.tril(Qh @ Kc.T)
    c = qn.shape[0]
    Tm = np.linalg.solve(np.eye(c) + Lm, np.diag(beta))
    return dict(Gam=Gam, Qh=Qh, Kh=Kh, Kc=Kc, Kb=Kb, L=Lm, M=Mm, T=Tm, gamma=np.exp(Gam[-1]))


def chunked_fwd(q, k, v, g, beta, scale, A_log, dt_bias, lower_bound, initial_state=None,
                cu_seqlens=None, C=16, output_final_state=True):
    """Same argument conventions as the oracle (bf16 bit patterns in, fp64 out)."""
    qf, kf, vf, gf = decode_bf16(q), decode_bf16(k), decode_bf16(v), decode_bf16(g)
    bf = decode_bf16(beta)
    A_log = np.asarray(A_log, dtype=np.float32).astype(np.float64)
    dt_bias = np.asarray(dt_bias, dtype=np.float32).astype(np.float64)
    B, T, H, K = qf.shape
    V = vf.shape[-1]
    if cu_seqlens is None:
        segs = [(b, 0, T) for b in range(B)]
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        segs = [(0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]
    out = np.zeros((B, T, H, V))
    fin = np.zeros((len(segs), H, V, K))
    for n, (b, t0, t1) in enumerate(segs):
        for h in range(H):
            gg = gf[b, t0:t1, h, :]
            A = np.exp(A_log[h])
            a = lower_bound / (1.0 + np.exp(-A * (gg + dt_bias[h][None, :])))
            bt = 1.0 / (1.0 + np.exp(-bf[b, t0:t1, h]))
            kk = kf[b, t0:t1, h, :]
            qq = qf[b, t0:t1, h, :]
            kn = kk / np.sqrt((kk * kk).sum(-1, keepdims=True) + EPS)
            qn = scale * qq / np.sqrt((qq * qq).sum(-1, keepdims=True) + EPS)
            vv = vf[b, t0:t1, h, :]
            Z = np.zeros((K, V)) if initial_state is None else np.array(initial_state[n, h]).T.astype(np.float64)
            for c0 in range(0, t1 - t0, C):
                c1 = min(c0 + C, t1 - t0)
                P = chunk_pieces(qn[c0:c1], kn[c0:c1], a[c0:c1], bt[c0:c1])
                W = P["T"] @ P["Kh"]
                U = P["T"] @ vv[c0:c1]
                E = U - W @ Z
                out[b, t0 + c0:t0 + c1, h, :] = P["Qh"] @ Z + P["M"] @ E
                Z = P["gamma"][:, None] * Z + P["Kb"].T @ E
            fin[n, h] = Z.T
    return out, (fin if output_final_state else None)


def neumann_inverse(Lm: np.ndarray) -> np.ndarray:
    """(I + L)^-1 for strictly lower L of size c <= 16: (I - L)(I + L^2)(I + L^4)(I + L^8)."""
    c = Lm.shape[0]
    I = np.eye(c)
    Nm = -Lm
    R = I + Nm
    P = Nm
    span = 2
    while span < c:
        P = P @ P
        R = R @ (I + P)
        span *= 2
    return R
