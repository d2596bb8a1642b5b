"""fp64 NumPy statement of the chunkwise algorithm, used only by the tests.

It pins the chunk-level equations the HIP kernels implement to the oracle's
token recurrence: "Linear Attention, Visualized", section "Cost", states that
every valid chunk size C gives exact results (C = 1 is the recurrent form,
C = n the parallel form), so at any C this must match the oracle to rounding.

Per chunk r (local positions l, m = 1..C, incoming state S_r), following the
sections "Mamba-2: input-dependent scalar decay" (chunkwise form), "Chunkwise
algorithm" of DeltaNet (UT transform, incoming-state correction), the GDN
table of chunkwise read-out and state update, "Gated Linear Attention (GLA)"
(channelwise prefix products) and "Kimi Delta Attention (KDA)" (table of
channelwise quantities):

  G_l        = sum_{s<=l} g_s   (vector over key channels for a channel gate)
  <-q_l      = exp(G_l) * q_l,  <-k_l = exp(G_l) * k_l,  ->k_l = exp(G_C - G_l) * k_l
  A[l,m]     = sum_c q_lc exp(G_lc - G_mc) k_mc      (m <= l, else 0)
  L[l,m]     = sum_c k_lc exp(G_lc - G_mc) k_mc      (m <  l, else 0)
  add rule   : Z = V
  delta rule : T = (I + diag(beta) L)^-1, W = T diag(beta) <-K, U = T diag(beta) V,
               Z = U - W S_r
  O_r        = <-Q S_r + A Z
  S_{r+1}    = Diag(exp(G_C)) S_r + ->K^T Z
"""
from __future__ import annotations

import numpy as np


def chunk_forward(q, k, v, g, beta, s0, *, rule, gate, C):
    """One head: q,k [T,dk], v [T,dv], g [T]|[T,dk]|None, beta [T]|None, s0 [dk,dv]|None."""
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if s0 is None else np.array(s0, np.float64)
    if gate == "none":
        gg = np.zeros((T, dk))
    elif gate == "scalar":
        gg = np.repeat(np.asarray(g, np.float64)[:, None], dk, axis=1)
    else:
        gg = np.asarray(g, np.float64)
    o = np.zeros((T, dv))
    for c0 in range(0, T, C):
        c1 = min(T, c0 + C)
        n = c1 - c0
        Q, K, V = q[c0:c1], k[c0:c1], v[c0:c1]
        G = np.cumsum(gg[c0:c1], axis=0)                # [n, dk]
        decay = np.exp(G[:, None, :] - G[None, :, :])   # [l, m, c]
        A = np.einsum("lc,lmc,mc->lm", Q, decay, K) * np.tril(np.ones((n, n)))
        Qd = np.exp(G) * Q
        Kr = np.exp(G[-1][None, :] - G) * K
        if rule == "delta":
            bb = np.asarray(beta, np.float64)[c0:c1]
            L = np.einsum("lc,lmc,mc->lm", K, decay, K) * np.tril(np.ones((n, n)), -1)
            Tm = np.linalg.inv(np.eye(n) + bb[:, None] * L)
            W = Tm @ (bb[:, None] * (np.exp(G) * K))
            U = Tm @ (bb[:, None] * V)
            Z = U - W @ S
        else:
            Z = V
        o[c0:c1] = Qd @ S + A @ Z
        S = np.exp(G[-1])[:, None] * S + Kr.T @ Z
    return o, S
