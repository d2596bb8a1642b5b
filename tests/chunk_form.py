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


def chunk_backward(q, k, v, g, beta, s0, do, dsT, *, rule, gate, C):
    """Gradients of sum(do . o) + sum(dsT . S_T) in the chunk form, one head,
    written as the three passes the HIP backward runs:

      1. forward over the chunks, keeping the incoming state S_r of every chunk;
      2. backward over the chunks, newest first, carrying dS (the gradient with
         respect to the state leaving the chunk):
           dZ = A^T dO + ->K dS;  dR = Tb^T dZ (delta; dR = dZ for add)
           dS_r = Diag(exp(G_C)) dS + <-Q^T dO - <-K^T dR (the last term: delta only)
      3. per chunk, from S_r and dS_{r+1} alone, with Tb = T diag(beta),
         R = V - <-K S_r, Z = Tb R, D_c[l,m] = exp(G_lc - G_mc):
           dv = dR;  d<-Q = dO S_r^T;  d<-K = -dR S_r^T;  d->K = Z dS_{r+1}^T
           dA = (dO Z^T) masked;  dTb = dZ R^T;  dbeta_m = sum_l T[l,m] dTb[l,m]
           dM = -T^T dTb Tb^T (M = I + diag(beta) L);  dL = diag(beta) dM masked;
           dbeta_l += sum_m dM[l,m] L[l,m]
           dq_A[l,c] = sum_m dA[l,m] k_mc D_c[l,m];   dk_A[m,c] = sum_l dA[l,m] q_lc D_c[l,m]
           dk_L1[l,c] = sum_m dL[l,m] k_mc D_c[l,m];  dk_L2[m,c] = sum_l dL[l,m] k_lc D_c[l,m]
           dq = exp(G) d<-Q + dq_A
           dk = exp(G) d<-K + exp(G_C - G) d->K + dk_A + dk_L1 + dk_L2
           dG = q.exp(G).d<-Q + k.exp(G).d<-K - k.exp(G_C-G).d->K + q.dq_A - k.dk_A + k.dk_L1 - k.dk_L2
           dG_C += sum_l k_l.exp(G_C-G_l).d->K_l + exp(G_C) . (row sums of S_r . dS_{r+1})
           dg = reverse prefix sum of dG within the chunk (per channel).
    With a scalar gate every channel of G is the same and dg sums the channels;
    without a gate G = 0.  Returns dq, dk, dv, dg (None without a gate), dbeta
    (None for add), ds0."""
    q, k, v, do = (np.asarray(x, np.float64) for x in (q, k, v, do))
    T, dk = q.shape
    dv = v.shape[1]
    if gate == "none":
        gg = np.zeros((T, dk))
    elif gate == "scalar":
        gg = np.repeat(np.asarray(g, np.float64)[:, None], dk, axis=1)
    else:
        gg = np.asarray(g, np.float64)
    bb = np.asarray(beta, np.float64) if rule == "delta" else None
    starts = list(range(0, T, C))

    def local(c0):
        c1 = min(T, c0 + C)
        n = c1 - c0
        G = np.cumsum(gg[c0:c1], axis=0)                  # [n, dk]
        D = np.exp(G[:, None, :] - G[None, :, :])         # [l, m, c]
        Q, K, V = q[c0:c1], k[c0:c1], v[c0:c1]
        A = np.einsum("lc,lmc,mc->lm", Q, D, K) * np.tril(np.ones((n, n)))
        out = dict(n=n, G=G, D=D, Q=Q, K=K, V=V, A=A, Qd=np.exp(G) * Q, Kd=np.exp(G) * K,
                   Kr=np.exp(G[-1][None, :] - G) * K, gC=np.exp(G[-1]))
        if rule == "delta":
            b = bb[c0:c1]
            L = np.einsum("lc,lmc,mc->lm", K, D, K) * np.tril(np.ones((n, n)), -1)
            Tm = np.linalg.inv(np.eye(n) + b[:, None] * L)
            out.update(b=b, L=L, T=Tm, Tb=Tm * b[None, :])
        return out

    # pass 1: incoming states
    S = np.zeros((dk, dv)) if s0 is None else np.array(s0, np.float64)
    Sin = []
    for c0 in starts:
        x = local(c0)
        Sin.append(S.copy())
        Z = x["Tb"] @ (x["V"] - x["Kd"] @ S) if rule == "delta" else x["V"]
        S = x["gC"][:, None] * S + x["Kr"].T @ Z
    # pass 2: gradients of the outgoing states
    dS = np.zeros((dk, dv)) if dsT is None else np.array(dsT, np.float64)
    dSout = [None] * len(starts)
    for r in range(len(starts) - 1, -1, -1):
        x = local(starts[r])
        dSout[r] = dS.copy()
        dO = do[starts[r]:starts[r] + x["n"]]
        dZ = x["A"].T @ dO + x["Kr"] @ dS
        dSn = x["gC"][:, None] * dS + x["Qd"].T @ dO
        if rule == "delta":
            dSn = dSn - x["Kd"].T @ (x["Tb"].T @ dZ)
        dS = dSn
    ds0 = dS
    # pass 3: per chunk
    gq, gk, gv, gG = np.zeros((T, dk)), np.zeros((T, dk)), np.zeros((T, dv)), np.zeros((T, dk))
    gb = np.zeros(T) if rule == "delta" else None
    for r, c0 in enumerate(starts):
        x = local(c0)
        n = x["n"]
        Sr, dSn = Sin[r], dSout[r]
        dO = do[c0:c0 + n]
        if rule == "delta":
            R = x["V"] - x["Kd"] @ Sr
            Z = x["Tb"] @ R
        else:
            Z = x["V"]
        dZ = x["A"].T @ dO + x["Kr"] @ dSn
        dR = x["Tb"].T @ dZ if rule == "delta" else dZ
        gv[c0:c0 + n] = dR
        dQd = dO @ Sr.T
        dKr = Z @ dSn.T
        dKd = -dR @ Sr.T if rule == "delta" else np.zeros((n, dk))
        dA = (dO @ Z.T) * np.tril(np.ones((n, n)))
        D, G, Q, K = x["D"], x["G"], x["Q"], x["K"]
        eG, eR = np.exp(G), np.exp(G[-1][None, :] - G)
        dqA = np.einsum("lm,mc,lmc->lc", dA, K, D)
        dkA = np.einsum("lm,lc,lmc->mc", dA, Q, D)
        dq = eG * dQd + dqA
        dkk = eG * dKd + eR * dKr + dkA
        dG = Q * eG * dQd + K * eG * dKd - K * eR * dKr + Q * dqA - K * dkA
        dG[-1] += np.sum(K * eR * dKr, 0) + x["gC"] * np.sum(Sr * dSn, 1)
        if rule == "delta":
            dTb = (dZ @ R.T) * np.tril(np.ones((n, n)))
            db = np.sum(x["T"] * dTb, 0)
            dM = -x["T"].T @ dTb @ x["Tb"].T
            dL = x["b"][:, None] * dM * np.tril(np.ones((n, n)), -1)
            db = db + np.sum(dM * x["L"], 1)
            dkL1 = np.einsum("lm,mc,lmc->lc", dL, K, D)
            dkL2 = np.einsum("lm,lc,lmc->mc", dL, K, D)
            dkk = dkk + dkL1 + dkL2
            dG = dG + K * dkL1 - K * dkL2
            gb[c0:c0 + n] = db
        gq[c0:c0 + n], gk[c0:c0 + n] = dq, dkk
        gG[c0:c0 + n] = np.cumsum(dG[::-1], 0)[::-1]
    if gate == "none":
        gg_out = None
    elif gate == "scalar":
        gg_out = gG.sum(axis=1)
    else:
        gg_out = gG
    return gq, gk, gv, gg_out, gb, ds0
