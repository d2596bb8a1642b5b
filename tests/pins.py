"""Checks that pin the fp64 oracle to what the pages and the mathematics fix.

Each pin takes an oracle handle (``oracle.OracleLib``) and raises
AssertionError when the oracle disagrees.  None of them re-runs the oracle's
token loop: they use closed forms (the parallel/quadratic forms, a triangular
solve), invariants, brute-force dense transition matrices, and worked examples
from the pages (``tests/golden``).  ``test_oracle_mutants.py`` plants
plausible mistakes into copies of the oracle and checks that each one trips at
least one pin.

Page titles: [LAV] "Linear Attention, Visualized"; [BA] "Beyond attention";
[ASF] "All sorts of famous Attention Layers".
"""
from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TOL = 1e-11  # fp64 reassociation between the recurrence and a closed form


def rel_err(x, ref):
    x, ref = np.asarray(x, np.float64), np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def _softplus(x):
    return np.maximum(x, 0) + np.log1p(np.exp(-np.abs(x)))


def rand_case(rng, B, H, T, dk, dv, *, gate="scalar", gate_scale=0.3, unit_keys=True,
              s0=True):
    """Gaussian fp64 inputs; keys (and queries) unit-norm when asked."""
    q = rng.standard_normal((B, H, T, dk))
    k = rng.standard_normal((B, H, T, dk))
    if unit_keys:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((B, H, T, dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, H, T))))
    if gate == "channel":
        g = -_softplus(rng.standard_normal((B, H, T, dk))) * gate_scale
    elif gate == "scalar":
        g = -_softplus(rng.standard_normal((B, H, T))) * gate_scale
    else:
        g = None
    S0 = rng.standard_normal((B, H, dk, dv)) * 0.5 if s0 else None
    return q, k, v, g, beta, S0


def _Gc(g, gate, dk):
    """Prefix sums of the log-gate as a [T, dk] array (a scalar gate repeated)."""
    if gate == "none":
        return None
    G = np.cumsum(g, axis=0)
    if gate == "scalar":
        G = np.repeat(G[:, None], dk, axis=1)
    return G


# ---------------------------------------------------------------------------
# V1  add rule == (Q K^T . M) V with the inclusive causal mask M
#     [LAV] "Naive linear attention" (causal version, prefix products, state
#     S_t); [ASF] "The Prefill Problem" (masked .tril() attention in a chunk).
# ---------------------------------------------------------------------------
def pin_add_equals_masked_quadratic(orc):
    rng = np.random.default_rng(101)
    B, H, T, dk, dv = 2, 2, 37, 5, 3
    q, k, v, _, _, S0 = rand_case(rng, B, H, T, dk, dv, gate="none", unit_keys=False)
    for s0 in (None, S0):
        o, S = orc.recurrence(q, k, v, None, None, s0, rule="add", gate="none")
        for b in range(B):
            for h in range(H):
                Q, K, V = q[b, h], k[b, h], v[b, h]
                ref = np.tril(Q @ K.T) @ V
                Sref = K.T @ V
                if s0 is not None:
                    ref = ref + Q @ s0[b, h]
                    Sref = Sref + s0[b, h]
                assert rel_err(o[b, h], ref) < TOL, "add rule != masked quadratic form"
                assert rel_err(S[b, h], Sref) < TOL, "add rule final state != K^T V"


# ---------------------------------------------------------------------------
# V2  decay == (Q K^T . Gamma) V, Gamma[t,j] = prod_{s=j+1..t} a_s
#     [LAV] "RetNet: scalar decay" (parallel form), "Mamba-2" (parallel form,
#     inclusive-interval decay products), "Gated Linear Attention (GLA)"
#     (local score with channelwise decay).
# ---------------------------------------------------------------------------
def pin_decay_equals_gamma_form(orc):
    rng = np.random.default_rng(102)
    B, H, T, dk, dv = 1, 2, 41, 6, 4
    for gate in ("scalar", "channel"):
        q, k, v, g, _, S0 = rand_case(rng, B, H, T, dk, dv, gate=gate, unit_keys=False)
        o, S = orc.recurrence(q, k, v, g, None, S0, rule="add", gate=gate)
        for b in range(B):
            for h in range(H):
                Q, K, V, s0 = q[b, h], k[b, h], v[b, h], S0[b, h]
                G = _Gc(g[b, h], gate, dk)                       # [T, dk]
                dec = np.exp(G[:, None, :] - G[None, :, :])      # [t, j, c]
                score = np.einsum("tc,tjc,jc->tj", Q, dec, K) * np.tril(np.ones((T, T)))
                ref = score @ V + (np.exp(G) * Q) @ s0
                Sref = np.exp(G[-1])[:, None] * s0 + (np.exp(G[-1][None, :] - G) * K).T @ V
                assert rel_err(o[b, h], ref) < TOL, f"{gate} decay != Gamma-masked form"
                assert rel_err(S[b, h], Sref) < TOL, f"{gate} decay final state wrong"


# ---------------------------------------------------------------------------
# V2b RetNet worked fact: a write made s steps earlier carries weight gamma^s
#     ([LAV] "RetNet: scalar decay").  Golden fixture, exact numbers.
# ---------------------------------------------------------------------------
def pin_golden_retnet_weights(orc):
    fx = json.load(open(os.path.join(GOLDEN, "retnet_decay_weights.json")))
    T, d = fx["T"], fx["d"]
    q = np.zeros((1, 1, T, d)); k = np.zeros((1, 1, T, d)); v = np.zeros((1, 1, T, d))
    k[0, 0, 0, fx["write_channel"]] = 1.0
    v[0, 0, 0] = fx["value"]
    q[0, 0, :, fx["write_channel"]] = 1.0
    g = np.full((1, 1, T), np.log(fx["gamma"]))
    for rule in ("add", "delta"):
        beta = np.ones((1, 1, T))
        o, _ = orc.recurrence(q, k, v, g, beta, None, rule=rule, gate="scalar")
        ref = np.asarray(fx["expected_outputs"], np.float64)
        assert np.max(np.abs(o[0, 0] - ref)) < 1e-14, f"RetNet weights gamma^s wrong ({rule})"


# ---------------------------------------------------------------------------
# V3  g == 0 makes decay identical to the add rule (a_t = 1), bit for bit
#     ([LAV] "Optional: TTT interpretation" table: RetNet/Mamba-2 rows reduce
#     to the Naive row at gamma = a_t = 1; [BA] "Three ways to update").
# ---------------------------------------------------------------------------
def pin_zero_gate_is_add(orc):
    rng = np.random.default_rng(103)
    B, H, T, dk, dv = 1, 3, 29, 4, 5
    q, k, v, _, beta, S0 = rand_case(rng, B, H, T, dk, dv, gate="none")
    for rule in ("add", "delta"):
        ref = orc.recurrence(q, k, v, None, beta, S0, rule=rule, gate="none")
        for gate, gshape in (("scalar", (B, H, T)), ("channel", (B, H, T, dk))):
            got = orc.recurrence(q, k, v, np.zeros(gshape), beta, S0, rule=rule, gate=gate)
            assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1]), \
                f"zero {gate} gate differs from no gate ({rule})"


# ---------------------------------------------------------------------------
# V4  delta rule with beta == 0 writes nothing: S_t = lambda[1:t] S_0
#     ([LAV] "DeltaNet" recurrent form: the correction u_t is scaled by beta_t).
# ---------------------------------------------------------------------------
def pin_beta_zero_keeps_state(orc):
    rng = np.random.default_rng(104)
    B, H, T, dk, dv = 2, 1, 23, 5, 4
    for gate in ("none", "scalar", "channel"):
        q, k, v, g, _, S0 = rand_case(rng, B, H, T, dk, dv, gate=gate)
        beta = np.zeros((B, H, T))
        o, S = orc.recurrence(q, k, v, g, beta, S0, rule="delta", gate=gate)
        for b in range(B):
            for h in range(H):
                if gate == "none":
                    assert np.array_equal(S[b, h], S0[b, h]), "beta=0 changed the state"
                    ref = q[b, h] @ S0[b, h]
                    Sref = S0[b, h]
                else:
                    G = _Gc(g[b, h], gate, dk)
                    ref = (np.exp(G) * q[b, h]) @ S0[b, h]
                    Sref = np.exp(G[-1])[:, None] * S0[b, h]
                assert rel_err(o[b, h], ref) < TOL, f"beta=0 read-out wrong ({gate})"
                assert rel_err(S[b, h], Sref) < TOL, f"beta=0 state wrong ({gate})"


# ---------------------------------------------------------------------------
# V5  exact recall: beta = 1, no decay, orthonormal unit keys -> reading a key
#     returns the latest value written at it ([LAV] "DeltaNet", "An intuitive
#     example": with beta = 1 the new value replaces the old prediction).
#     Also the general unit-key identity k_t S_t = (1-beta_t) k_t S' + beta_t v_t.
# ---------------------------------------------------------------------------
def pin_orthonormal_exact_recall(orc):
    rng = np.random.default_rng(105)
    d, T = 8, 60
    basis, _ = np.linalg.qr(rng.standard_normal((d, d)))
    widx = rng.integers(0, d, T)
    ridx = rng.integers(0, d, T)
    k = basis[widx][None, None]
    q = basis[ridx][None, None]
    v = rng.standard_normal((1, 1, T, d))
    beta = np.ones((1, 1, T))
    o, _ = orc.recurrence(q, k, v, None, beta, None, rule="delta", gate="none")
    latest = {}
    for t in range(T):
        latest[int(widx[t])] = v[0, 0, t]
        ref = latest.get(int(ridx[t]), np.zeros(d))
        assert np.max(np.abs(o[0, 0, t] - ref)) < 1e-12, "orthonormal recall not exact"


def pin_unit_key_partial_correction(orc):
    rng = np.random.default_rng(106)
    N, H, dk, dv = 3, 2, 6, 5
    for gate in ("none", "scalar", "channel"):
        q, k, v, g, beta, S0 = rand_case(rng, N, H, 1, dk, dv, gate=gate)
        q, k, v, beta = q[:, :, 0], k[:, :, 0], v[:, :, 0], beta[:, :, 0]
        g = None if g is None else g[:, :, 0]
        _, S1 = orc.decode_step(q, k, v, g, beta, S0, rule="delta", gate=gate)
        for n in range(N):
            for h in range(H):
                if gate == "none":
                    Sp = S0[n, h]
                elif gate == "scalar":
                    Sp = np.exp(g[n, h]) * S0[n, h]
                else:
                    Sp = np.exp(g[n, h])[:, None] * S0[n, h]
                lhs = k[n, h] @ S1[n, h]
                rhs = (1 - beta[n, h]) * (k[n, h] @ Sp) + beta[n, h] * v[n, h]
                assert rel_err(lhs, rhs) < TOL, f"unit-key correction identity fails ({gate})"


# ---------------------------------------------------------------------------
# V5b golden: the Alice/Bob memory example ([LAV] "An intuitive example").
# ---------------------------------------------------------------------------
def pin_golden_alice_bob(orc):
    fx = json.load(open(os.path.join(GOLDEN, "alice_bob.json")))
    keys = {n: np.asarray(x, np.float64) for n, x in fx["keys"].items()}
    vals = {n: np.asarray(x, np.float64) for n, x in fx["values"].items()}
    d = len(next(iter(keys.values())))
    dv = len(next(iter(vals.values())))
    for case in fx["cases"]:
        writes, reads = case["writes"], case["reads"]
        T = len(writes) + len(reads)
        q = np.zeros((1, 1, T, d)); k = np.zeros((1, 1, T, d)); v = np.zeros((1, 1, T, dv))
        beta = np.zeros((1, 1, T))
        for t, (kn, vn, bt) in enumerate(writes):
            k[0, 0, t], v[0, 0, t], beta[0, 0, t] = keys[kn], vals[vn], bt
        for i, r in enumerate(reads):
            q[0, 0, len(writes) + i] = keys[r["key"]]
        o, _ = orc.recurrence(q, k, v, None, beta, None, rule="delta", gate="none")
        for i, r in enumerate(reads):
            got = o[0, 0, len(writes) + i]
            assert np.max(np.abs(got - np.asarray(r["expect"]))) < 1e-14, \
                f"Alice/Bob example, last beta={writes[-1][2]}, read {r['key']}"


# ---------------------------------------------------------------------------
# V6  the delta step is one gradient step on 1/2 ||k S - v||^2 with rate beta
#     ([LAV] "Optional: Test-time training (TTT) interpretation").  Weak pin:
#     an algebraic identity of the same update.
# ---------------------------------------------------------------------------
def pin_ttt_gradient_step(orc):
    rng = np.random.default_rng(107)
    N, H, dk, dv = 2, 2, 5, 3
    q, k, v, _, beta, S0 = rand_case(rng, N, H, 1, dk, dv, gate="none")
    q, k, v, beta = q[:, :, 0], k[:, :, 0], v[:, :, 0], beta[:, :, 0]
    _, S1 = orc.decode_step(q, k, v, None, beta, S0, rule="delta", gate="none")
    for n in range(N):
        for h in range(H):
            S, kk, vv = S0[n, h], k[n, h], v[n, h]
            grad = np.outer(kk, kk @ S - vv)     # d/dS of 1/2 ||k S - v||^2
            assert rel_err(S1[n, h], S - beta[n, h] * grad) < TOL, "delta != SGD step"


# ---------------------------------------------------------------------------
# V7  the full-sequence triangular form: (I + B L) U = B V, O = (Q K^T . Gamma) U
#     ([LAV] "The triangular correction system", "Parallel output", the GDN
#     chunkwise table and the KDA table of L for m < l), solved with LAPACK.
# ---------------------------------------------------------------------------
def pin_delta_triangular_system(orc):
    rng = np.random.default_rng(108)
    B, H, T, dk, dv = 1, 2, 53, 6, 4
    for gate in ("none", "scalar", "channel"):
        q, k, v, g, beta, _ = rand_case(rng, B, H, T, dk, dv, gate=gate)
        o, S = orc.recurrence(q, k, v, g, beta, None, rule="delta", gate=gate)
        for b in range(B):
            for h in range(H):
                Q, K, V, bb = q[b, h], k[b, h], v[b, h], beta[b, h]
                G = np.zeros((T, dk)) if gate == "none" else _Gc(g[b, h], gate, dk)
                dec = np.exp(G[:, None, :] - G[None, :, :])
                L = np.einsum("tc,tjc,jc->tj", K, dec, K) * np.tril(np.ones((T, T)), -1)
                U = np.linalg.solve(np.eye(T) + bb[:, None] * L, bb[:, None] * V)
                A = np.einsum("tc,tjc,jc->tj", Q, dec, K) * np.tril(np.ones((T, T)))
                assert rel_err(o[b, h], A @ U) < 1e-10, f"triangular form mismatch ({gate})"
                Sref = (np.exp(G[-1][None, :] - G) * K).T @ U
                assert rel_err(S[b, h], Sref) < 1e-10, f"triangular-form state ({gate})"


# ---------------------------------------------------------------------------
# V8  brute force with explicit dense transitions on tiny inputs:
#     S_t = (I - beta_t k_t^T k_t) D_t S_{t-1} + beta_t k_t^T v_t (delta),
#     S_t = D_t S_{t-1} + k_t^T v_t (add), D_t = I | a_t I | Diag(a_t)
#     ([LAV] "One chunk as an affine recurrence", "Gated DeltaNet (GDN)",
#     "Kimi Delta Attention (KDA)": decay channel by channel, then correct).
#     Rectangular d_k != d_v so that a transposed operand cannot pass.
# ---------------------------------------------------------------------------
def pin_brute_force_transitions(orc):
    rng = np.random.default_rng(109)
    for (dk, dv) in ((3, 4), (4, 2)):
        T = 7
        for rule in ("add", "delta"):
            for gate in ("none", "scalar", "channel"):
                q, k, v, g, beta, S0 = rand_case(rng, 1, 1, T, dk, dv, gate=gate,
                                                 gate_scale=0.7, unit_keys=False)
                o, S = orc.recurrence(q, k, v, g, beta, S0, rule=rule, gate=gate)
                St = S0[0, 0].copy()
                for t in range(T):
                    if gate == "none":
                        D = np.eye(dk)
                    elif gate == "scalar":
                        D = np.exp(g[0, 0, t]) * np.eye(dk)
                    else:
                        D = np.diag(np.exp(g[0, 0, t]))
                    kt = k[0, 0, t][:, None]           # column d_k x 1
                    vt = v[0, 0, t][None, :]           # row 1 x d_v
                    if rule == "delta":
                        bt = beta[0, 0, t]
                        M = (np.eye(dk) - bt * kt @ kt.T) @ D
                        St = M @ St + bt * kt @ vt
                    else:
                        St = D @ St + kt @ vt
                    ref = q[0, 0, t][None, :] @ St
                    assert rel_err(o[0, 0, t], ref[0]) < TOL, \
                        f"brute force mismatch ({rule}/{gate}, t={t}, dk={dk}, dv={dv})"
                assert rel_err(S[0, 0], St) < TOL, f"brute force final state ({rule}/{gate})"


# ---------------------------------------------------------------------------
# V9  a channel gate with all channels equal is the scalar gate
#     ([LAV] "Kimi Delta Attention (KDA)": with a_t = a_t * 1 it reduces
#     exactly to GDN; "Gated Linear Attention (GLA)" vs "Mamba-2").
# ---------------------------------------------------------------------------
def pin_equal_channels_is_scalar(orc):
    rng = np.random.default_rng(110)
    B, H, T, dk, dv = 2, 2, 31, 5, 3
    q, k, v, g, beta, S0 = rand_case(rng, B, H, T, dk, dv, gate="scalar")
    gc = np.repeat(g[..., None], dk, axis=-1)
    for rule in ("add", "delta"):
        a = orc.recurrence(q, k, v, g, beta, S0, rule=rule, gate="scalar")
        c = orc.recurrence(q, k, v, gc, beta, S0, rule=rule, gate="channel")
        assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1]), \
            f"equal-channel gate != scalar gate ({rule})"


# ---------------------------------------------------------------------------
# V10 the chunkwise algorithm at any chunk size equals the recurrence
#     ([LAV] "Cost": every valid C is exact; "Chunkwise algorithm" of DeltaNet:
#     the regrouping is exact).  Ragged last chunk, nonzero S_0, all rules.
# ---------------------------------------------------------------------------
def pin_chunk_form_any_C(orc):
    from chunk_form import chunk_forward
    rng = np.random.default_rng(111)
    B, H, T, dk, dv = 1, 2, 45, 6, 5
    for rule in ("add", "delta"):
        for gate in ("none", "scalar", "channel"):
            q, k, v, g, beta, S0 = rand_case(rng, B, H, T, dk, dv, gate=gate)
            o, S = orc.recurrence(q, k, v, g, beta, S0, rule=rule, gate=gate)
            for C in (1, 2, 16, T):
                for h in range(H):
                    oc, Sc = chunk_forward(q[0, h], k[0, h], v[0, h],
                                           None if g is None else g[0, h],
                                           beta[0, h], S0[0, h], rule=rule, gate=gate, C=C)
                    assert rel_err(o[0, h], oc) < 1e-10, f"chunk form C={C} ({rule}/{gate})"
                    assert rel_err(S[0, h], Sc) < 1e-10, f"chunk state C={C} ({rule}/{gate})"


# ---------------------------------------------------------------------------
# V11 T decode steps == one pass; resuming from the returned state == one pass
#     ([ASF] linear-attention layer returns its state; the chunk loop seeds S
#     from a cache; [LAV] "Update the state": chunk boundaries form a chain).
# ---------------------------------------------------------------------------
def pin_decode_and_resume(orc):
    rng = np.random.default_rng(112)
    B, H, T, dk, dv = 2, 2, 19, 4, 6
    for rule in ("add", "delta"):
        for gate in ("none", "scalar", "channel"):
            q, k, v, g, beta, S0 = rand_case(rng, B, H, T, dk, dv, gate=gate)
            o, S = orc.recurrence(q, k, v, g, beta, S0, rule=rule, gate=gate)
            st = S0.copy()
            for t in range(T):
                ot, st = orc.decode_step(q[:, :, t], k[:, :, t], v[:, :, t],
                                         None if g is None else g[:, :, t],
                                         beta[:, :, t], st, rule=rule, gate=gate)
                assert rel_err(ot, o[:, :, t]) < TOL, f"decode step {t} ({rule}/{gate})"
            assert rel_err(st, S) < TOL, f"decode final state ({rule}/{gate})"
            t1 = 7
            gs = (lambda a, s: None if a is None else a[:, :, s])
            o1, S1 = orc.recurrence(q[:, :, :t1], k[:, :, :t1], v[:, :, :t1], gs(g, slice(0, t1)),
                                    beta[:, :, :t1], S0, rule=rule, gate=gate)
            o2, S2 = orc.recurrence(q[:, :, t1:], k[:, :, t1:], v[:, :, t1:], gs(g, slice(t1, T)),
                                    beta[:, :, t1:], S1, rule=rule, gate=gate)
            assert rel_err(np.concatenate([o1, o2], axis=2), o) < TOL, "resume read-out"
            assert rel_err(S2, S) < TOL, "resume final state"


# ---------------------------------------------------------------------------
# V12 Gated DeltaProduct with one substep is Gated DeltaNet
#     ([LAV] "Gated Delta Product (GDP)": GDP replaces GDN's single transition
#     per token by a product of n_h of them; n_h = 1 is GDN itself).
# ---------------------------------------------------------------------------
def pin_deltaproduct_one_substep_is_gdn(orc):
    rng = np.random.default_rng(113)
    B, H, T, dk, dv = 2, 2, 23, 5, 4
    for gate in ("none", "scalar"):
        q, k, v, g, beta, S0 = rand_case(rng, B, H, T, dk, dv, gate=gate)
        a = orc.recurrence(q, k, v, g, beta, S0, rule="delta", gate=gate)
        b = orc.deltaproduct(q, k[:, :, :, None], v[:, :, :, None], g, beta[..., None], S0,
                             gate=gate)
        assert rel_err(b[0], a[0]) < TOL and rel_err(b[1], a[1]) < TOL, \
            f"GDP with n_h = 1 != GDN ({gate})"


def _gdp_case(rng, B, H, T, nh, dk, dv, gate):
    q = rng.standard_normal((B, H, T, dk))
    k = rng.standard_normal((B, H, T, nh, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, H, T, nh, dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, H, T, nh))))
    g = -_softplus(rng.standard_normal((B, H, T))) * 0.5 if gate == "scalar" else None
    S0 = rng.standard_normal((B, H, dk, dv)) * 0.5
    return q, k, v, g, beta, S0


# ---------------------------------------------------------------------------
# V13 Gated DeltaProduct as a product of dense transitions on tiny inputs:
#     S_t = H_{n_h} ... H_1 a_t S_{t-1} + sum_j H_{n_h} ... H_{j+1} beta_j k_j^T v_j,
#     H_j = I - beta_j k_j^T k_j  ([LAV] "Gated Delta Product (GDP)": the decay
#     before the first substep, the transitions in order, the query after the
#     last).  Rectangular d_k != d_v.
# ---------------------------------------------------------------------------
def pin_deltaproduct_dense_product(orc):
    rng = np.random.default_rng(114)
    for (nh, dk, dv) in ((2, 3, 4), (3, 4, 2)):
        T = 6
        for gate in ("none", "scalar"):
            q, k, v, g, beta, S0 = _gdp_case(rng, 1, 1, T, nh, dk, dv, gate)
            o, S = orc.deltaproduct(q, k, v, g, beta, S0, gate=gate)
            St = S0[0, 0].copy()
            for t in range(T):
                a = np.exp(g[0, 0, t]) if gate == "scalar" else 1.0
                Hs = [np.eye(dk) - beta[0, 0, t, j] * np.outer(k[0, 0, t, j], k[0, 0, t, j])
                      for j in range(nh)]
                P = np.eye(dk)
                for j in range(nh):
                    P = Hs[j] @ P                      # H_j ... H_1
                acc = P @ (a * St)
                for j in range(nh):
                    Pj = np.eye(dk)
                    for i in range(j + 1, nh):
                        Pj = Hs[i] @ Pj                # H_{n_h} ... H_{j+1}
                    acc = acc + beta[0, 0, t, j] * Pj @ np.outer(k[0, 0, t, j], v[0, 0, t, j])
                St = acc
                assert rel_err(o[0, 0, t], q[0, 0, t] @ St) < TOL, \
                    f"GDP dense product read-out (n_h={nh}, {gate}, t={t})"
            assert rel_err(S[0, 0], St) < TOL, f"GDP dense product state (n_h={nh}, {gate})"


# ---------------------------------------------------------------------------
# V14 Gated DeltaProduct is GDN over the virtual sequence of n_h T steps
#     ([LAV] "GDP as GDN over a virtual sequence": keys, values and correction
#     gates flattened in order, the decay on each token's first virtual step
#     and 1 elsewhere, the query on its last virtual step and 0 elsewhere,
#     every n_h-th output retained).
# ---------------------------------------------------------------------------
def pin_deltaproduct_virtual_sequence(orc):
    rng = np.random.default_rng(115)
    B, H, T, nh, dk, dv = 2, 2, 9, 3, 4, 5
    for gate in ("none", "scalar"):
        q, k, v, g, beta, S0 = _gdp_case(rng, B, H, T, nh, dk, dv, gate)
        o, S = orc.deltaproduct(q, k, v, g, beta, S0, gate=gate)
        qv = np.zeros((B, H, T, nh, dk))
        qv[:, :, :, nh - 1] = q
        gv = None
        if gate == "scalar":
            gv = np.zeros((B, H, T, nh))
            gv[:, :, :, 0] = g
            gv = gv.reshape(B, H, T * nh)
        ov, Sv = orc.recurrence(qv.reshape(B, H, T * nh, dk), k.reshape(B, H, T * nh, dk),
                                v.reshape(B, H, T * nh, dv), gv, beta.reshape(B, H, T * nh), S0,
                                rule="delta", gate=gate)
        assert rel_err(o, ov.reshape(B, H, T, nh, dv)[:, :, :, nh - 1]) < TOL, \
            f"GDP != GDN over the virtual sequence ({gate})"
        assert rel_err(S, Sv) < TOL, f"GDP state != virtual-sequence state ({gate})"


# ---------------------------------------------------------------------------
# V15 normalised linear attention == the masked, decay-weighted quadratic form
#     divided by its row sums: o_t = sum_j w_tj v_j / sum_j w_tj with
#     w_tj = (q_t . k_j) prod_{s=j+1..t} a_s for j <= t ([ASF] "Linear Magic":
#     the normaliser of the feature-map attention; [LAV] "Mamba-2": the decay
#     weights of the parallel form).  Carried states (S_0, z_0) enter as an
#     extra decayed term in numerator and denominator.
# ---------------------------------------------------------------------------
def _norm_case(rng, B, H, T, dk, dv, gate):
    q = np.abs(rng.standard_normal((B, H, T, dk))) + 0.1
    k = np.abs(rng.standard_normal((B, H, T, dk))) + 0.1
    v = rng.standard_normal((B, H, T, dv))
    g = None
    if gate == "scalar":
        g = -_softplus(rng.standard_normal((B, H, T))) * 0.3
    elif gate == "channel":
        g = -_softplus(rng.standard_normal((B, H, T, dk))) * 0.3
    S0 = np.abs(rng.standard_normal((B, H, dk, dv)))
    z0 = np.abs(rng.standard_normal((B, H, dk))) + 0.5
    return q, k, v, g, S0, z0


def pin_normalized_quadratic_form(orc):
    rng = np.random.default_rng(116)
    B, H, T, dk, dv = 1, 2, 13, 5, 3
    for gate in ("none", "scalar", "channel"):
        q, k, v, g, S0, z0 = _norm_case(rng, B, H, T, dk, dv, gate)
        o, S, z = orc.normalized(q, k, v, g, S0, z0, gate=gate)
        for h in range(H):
            G = _Gc(g[0, h], gate, dk) if gate != "none" else np.zeros((T, dk))
            # w_tj = sum_c q_tc k_jc exp(G_tc - G_jc), j <= t; carried states decay by exp(G_t)
            W = np.einsum("tc,jc,tjc->tj", q[0, h], k[0, h], np.exp(G[:, None, :] - G[None, :, :]))
            W = np.tril(W)
            lam = np.exp(G)                                # [T, dk]
            num = W @ v[0, h] + (q[0, h] * lam) @ S0[0, h]
            den = W.sum(axis=1) + (q[0, h] * lam) @ z0[0, h]
            assert rel_err(o[0, h], num / den[:, None]) < TOL, f"normalised LA quadratic form ({gate})"
            zT = lam[-1] * z0[0, h] + (np.exp(G[-1][None, :] - G) * k[0, h]).sum(axis=0)
            assert rel_err(z[0, h], zT) < TOL, f"normaliser state ({gate})"


# ---------------------------------------------------------------------------
# V16 normalisation invariants: a constant value vector comes back unchanged
#     (the weights sum to one) when the carried state holds that value too, and
#     scaling every query by c > 0 leaves the output unchanged.
# ---------------------------------------------------------------------------
def pin_normalized_invariants(orc):
    rng = np.random.default_rng(117)
    B, H, T, dk, dv = 2, 1, 17, 4, 3
    for gate in ("none", "scalar"):
        q, k, v, g, S0, z0 = _norm_case(rng, B, H, T, dk, dv, gate)
        c = rng.standard_normal(dv)
        vc = np.broadcast_to(c, v.shape).copy()
        Sc = z0[..., None] * c                           # S0 = z0^T c: the same constant
        oc, _, _ = orc.normalized(q, k, vc, g, Sc, z0, gate=gate)
        assert rel_err(oc, np.broadcast_to(c, oc.shape)) < TOL, f"constant value ({gate})"
        o1, _, _ = orc.normalized(q, k, v, g, S0, z0, gate=gate)
        o2, _, _ = orc.normalized(q * 3.7, k, v, g, S0, z0, gate=gate)
        assert rel_err(o2, o1) < TOL, f"query scale ({gate})"
        if gate == "scalar":
            # a channel gate with all channels equal is the scalar gate
            gc = np.repeat(g[..., None], dk, axis=-1)
            o3, S3, z3 = orc.normalized(q, k, v, gc, S0, z0, gate="channel")
            a = orc.normalized(q, k, v, g, S0, z0, gate="scalar")
            assert rel_err(o3, a[0]) < TOL and rel_err(S3, a[1]) < TOL and rel_err(z3, a[2]) < TOL, \
                "equal-channel gate != scalar gate (normalised)"


# ---------------------------------------------------------------------------
# Backward pass.  The gradients of loss = sum(do . o) + sum(dsT . S_T) with
# respect to q, k, v, g, beta and s0 ([LAV] "Optional: Linear attention as an
# RNN" and "Update the state": the states autograd keeps for the backward pass
# of the recurrent and the chunk form).
# ---------------------------------------------------------------------------
BWD_NAMES = (("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("beta", "dbeta"), ("s0", "ds0"))


def _bwd_case(rng, T, dk, dv, rule, gate, B=1, H=1):
    q, k, v, g, beta, S0 = rand_case(rng, B, H, T, dk, dv, gate=gate, gate_scale=0.7,
                                     unit_keys=False)
    do = rng.standard_normal((B, H, T, dv))
    dsT = rng.standard_normal((B, H, dk, dv))
    x = {"q": q, "k": k, "v": v, "g": g if gate != "none" else None,
         "beta": beta if rule == "delta" else None, "s0": S0}
    return x, do, dsT


def _loss(orc, x, do, dsT, rule, gate):
    o, S = orc.recurrence(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], rule=rule, gate=gate)
    return float(np.sum(o * do) + np.sum(S * dsT))


# ---------------------------------------------------------------------------
# V17  the backward pass against central differences of the (pinned) forward:
#      every entry of every input on tiny cases, for each rule and gate, with
#      d_k != d_v; and random directions on a case longer than the oracle's
#      replay segment (64 tokens).
# ---------------------------------------------------------------------------
def pin_bwd_finite_differences(orc):
    rng = np.random.default_rng(117)
    eps = 1e-6
    for rule in ("add", "delta"):
        for gate in ("none", "scalar", "channel"):
            x, do, dsT = _bwd_case(rng, 6, 3, 2, rule, gate)
            grads = orc.recurrence_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], do, dsT,
                                       rule=rule, gate=gate)
            for name, gname in BWD_NAMES:
                if x[name] is None:
                    assert grads[gname] is None, f"{gname} given for an absent input"
                    continue
                fd = np.zeros_like(x[name])
                for idx in np.ndindex(x[name].shape):
                    xp = dict(x); xp[name] = x[name].copy(); xp[name][idx] += eps
                    xm = dict(x); xm[name] = x[name].copy(); xm[name][idx] -= eps
                    fd[idx] = (_loss(orc, xp, do, dsT, rule, gate) - _loss(orc, xm, do, dsT, rule, gate)) / (2 * eps)
                err = np.max(np.abs(grads[gname] - fd)) / max(1.0, np.max(np.abs(fd)))
                assert err < 1e-7, f"{gname} vs central differences ({rule}/{gate}): {err:.2e}"
    # 150 tokens: three replay segments; directional derivatives
    for rule, gate in (("delta", "scalar"), ("add", "channel"), ("delta", "channel")):
        x, do, dsT = _bwd_case(rng, 150, 4, 3, rule, gate)
        x["q"] /= 2.0
        grads = orc.recurrence_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], do, dsT,
                                   rule=rule, gate=gate)
        for _ in range(3):
            dirs = {n: (None if x[n] is None else rng.standard_normal(x[n].shape)) for n, _g in BWD_NAMES}
            xp = {n: (None if x[n] is None else x[n] + eps * dirs[n]) for n in x}
            xm = {n: (None if x[n] is None else x[n] - eps * dirs[n]) for n in x}
            fd = (_loss(orc, xp, do, dsT, rule, gate) - _loss(orc, xm, do, dsT, rule, gate)) / (2 * eps)
            an = sum(float(np.sum(grads[gn] * dirs[n])) for n, gn in BWD_NAMES if x[n] is not None)
            assert abs(an - fd) < 1e-6 * max(1.0, abs(fd)), \
                f"directional derivative ({rule}/{gate}, T=150): {an} vs {fd}"


# ---------------------------------------------------------------------------
# V18  the backward pass against automatic differentiation (torch, fp64) of
#      the one-chunk parallel form: C = T, incoming state s0 (the special case
#      of the chunkwise equations in [LAV] "Chunkwise algorithm", the GDN and
#      KDA tables, which pin V10 ties to the recurrence).  A different formula,
#      differentiated by a library.
# ---------------------------------------------------------------------------
def _one_chunk_torch(q, k, v, g, beta, s0, rule, gate):
    import torch
    T, dk = q.shape
    if gate == "none":
        G = torch.zeros((T, dk), dtype=q.dtype)
    elif gate == "scalar":
        G = torch.cumsum(g, 0)[:, None].expand(T, dk)
    else:
        G = torch.cumsum(g, 0)
    dec = torch.exp(G[:, None, :] - G[None, :, :])               # [l, m, c]
    incl = torch.tril(torch.ones((T, T), dtype=q.dtype))
    A = torch.einsum("lc,lmc,mc->lm", q, dec, k) * incl
    Qd, Kd = torch.exp(G) * q, torch.exp(G) * k
    Kr = torch.exp(G[-1][None, :] - G) * k
    if rule == "delta":
        Lm = torch.einsum("lc,lmc,mc->lm", k, dec, k) * (incl - torch.eye(T, dtype=q.dtype))
        M = torch.eye(T, dtype=q.dtype) + beta[:, None] * Lm
        Z = torch.linalg.solve(M, beta[:, None] * (v - Kd @ s0))
    else:
        Z = v
    o = Qd @ s0 + A @ Z
    S = torch.exp(G[-1])[:, None] * s0 + Kr.T @ Z
    return o, S


def pin_bwd_autograd_one_chunk(orc):
    import torch
    rng = np.random.default_rng(118)
    for rule in ("add", "delta"):
        for gate in ("none", "scalar", "channel"):
            x, do, dsT = _bwd_case(rng, 37, 5, 4, rule, gate)
            grads = orc.recurrence_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], do, dsT,
                                       rule=rule, gate=gate)
            tx = {n: (None if a is None else torch.tensor(a[0, 0], requires_grad=True)) for n, a in x.items()}
            o, S = _one_chunk_torch(tx["q"], tx["k"], tx["v"], tx["g"], tx["beta"], tx["s0"], rule, gate)
            loss = (o * torch.tensor(do[0, 0])).sum() + (S * torch.tensor(dsT[0, 0])).sum()
            loss.backward()
            for name, gname in BWD_NAMES:
                if tx[name] is None:
                    continue
                assert rel_err(grads[gname][0, 0], tx[name].grad.numpy()) < 1e-10, \
                    f"{gname} vs autograd of the one-chunk form ({rule}/{gate})"


# ---------------------------------------------------------------------------
# V19  the Gated DeltaProduct backward against central differences of the
#      pinned GDP forward: every entry on tiny cases, n_h in {1, 2, 3}, gate
#      none and scalar; directional derivatives over 70 tokens (two replay
#      segments).  ([LAV] "Gated Delta Product (GDP)")
# ---------------------------------------------------------------------------
def _gdp_bwd_case(rng, T, nh, dk, dv, gate):
    q = rng.standard_normal((1, 1, T, dk))
    k = rng.standard_normal((1, 1, T, nh, dk)) / np.sqrt(dk)
    v = rng.standard_normal((1, 1, T, nh, dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((1, 1, T, nh))))
    g = -_softplus(rng.standard_normal((1, 1, T))) * 0.5 if gate == "scalar" else None
    s0 = rng.standard_normal((1, 1, dk, dv)) * 0.5
    do = rng.standard_normal((1, 1, T, dv))
    dsT = rng.standard_normal((1, 1, dk, dv))
    return {"q": q, "k": k, "v": v, "g": g, "beta": beta, "s0": s0}, do, dsT


def _gdp_loss(orc, x, do, dsT, gate):
    o, S = orc.deltaproduct(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], gate=gate)
    return float(np.sum(o * do) + np.sum(S * dsT))


def pin_deltaproduct_bwd_finite_differences(orc):
    rng = np.random.default_rng(119)
    eps = 1e-6
    for nh in (1, 2, 3):
        for gate in ("none", "scalar"):
            x, do, dsT = _gdp_bwd_case(rng, 5, nh, 3, 2, gate)
            gr = orc.deltaproduct_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], do, dsT, gate=gate)
            for name, gname in BWD_NAMES:
                if x[name] is None:
                    assert gr[gname] is None
                    continue
                fd = np.zeros_like(x[name])
                for idx in np.ndindex(x[name].shape):
                    xp = dict(x); xp[name] = x[name].copy(); xp[name][idx] += eps
                    xm = dict(x); xm[name] = x[name].copy(); xm[name][idx] -= eps
                    fd[idx] = (_gdp_loss(orc, xp, do, dsT, gate) - _gdp_loss(orc, xm, do, dsT, gate)) / (2 * eps)
                err = np.max(np.abs(gr[gname] - fd)) / max(1.0, np.max(np.abs(fd)))
                assert err < 1e-7, f"GDP {gname} vs central differences (nh={nh}, {gate}): {err:.2e}"
    x, do, dsT = _gdp_bwd_case(rng, 70, 2, 4, 3, "scalar")
    gr = orc.deltaproduct_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], do, dsT, gate="scalar")
    for _ in range(3):
        dirs = {n: rng.standard_normal(a.shape) for n, a in x.items()}
        xp = {n: a + eps * dirs[n] for n, a in x.items()}
        xm = {n: a - eps * dirs[n] for n, a in x.items()}
        fd = (_gdp_loss(orc, xp, do, dsT, "scalar") - _gdp_loss(orc, xm, do, dsT, "scalar")) / (2 * eps)
        an = sum(float(np.sum(gr[gn] * dirs[n])) for n, gn in BWD_NAMES)
        assert abs(an - fd) < 1e-6 * max(1.0, abs(fd)), f"GDP directional derivative: {an} vs {fd}"


# ---------------------------------------------------------------------------
# V20  the Gated DeltaProduct backward equals the Gated DeltaNet backward over
#      the virtual sequence of n_h T steps ([LAV] "GDP as GDN over a virtual
#      sequence"): the query sits on the last substep and the gate on the first,
#      so dq and dg are the virtual ones there; dk, dv, dbeta share the layout.
# ---------------------------------------------------------------------------
def pin_deltaproduct_bwd_virtual_sequence(orc):
    rng = np.random.default_rng(120)
    for nh, gate in ((1, "scalar"), (2, "scalar"), (3, "none")):
        T, dk, dv = 23, 5, 4
        x, do, dsT = _gdp_bwd_case(rng, T, nh, dk, dv, gate)
        gr = orc.deltaproduct_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], do, dsT, gate=gate)
        Tv = T * nh
        qv = np.zeros((1, 1, Tv, dk)); qv[0, 0, nh - 1::nh] = x["q"][0, 0]
        dov = np.zeros((1, 1, Tv, dv)); dov[0, 0, nh - 1::nh] = do[0, 0]
        gv = None
        if gate == "scalar":
            gv = np.zeros((1, 1, Tv)); gv[0, 0, 0::nh] = x["g"][0, 0]
        ref = orc.recurrence_bwd(qv, x["k"].reshape(1, 1, Tv, dk), x["v"].reshape(1, 1, Tv, dv), gv,
                                 x["beta"].reshape(1, 1, Tv), x["s0"], dov, dsT, rule="delta", gate=gate)
        assert rel_err(gr["dq"][0, 0], ref["dq"][0, 0, nh - 1::nh]) < 1e-10, f"GDP dq (nh={nh})"
        assert rel_err(gr["dk"].reshape(Tv, dk), ref["dk"][0, 0]) < 1e-10, f"GDP dk (nh={nh})"
        assert rel_err(gr["dv"].reshape(Tv, dv), ref["dv"][0, 0]) < 1e-10, f"GDP dv (nh={nh})"
        assert rel_err(gr["dbeta"].reshape(Tv), ref["dbeta"][0, 0]) < 1e-10, f"GDP dbeta (nh={nh})"
        assert rel_err(gr["ds0"], ref["ds0"]) < 1e-10, f"GDP ds0 (nh={nh})"
        if gate == "scalar":
            assert rel_err(gr["dg"][0, 0], ref["dg"][0, 0, 0::nh]) < 1e-10, f"GDP dg (nh={nh})"


PINS = [
    pin_add_equals_masked_quadratic,
    pin_decay_equals_gamma_form,
    pin_golden_retnet_weights,
    pin_zero_gate_is_add,
    pin_beta_zero_keeps_state,
    pin_orthonormal_exact_recall,
    pin_unit_key_partial_correction,
    pin_golden_alice_bob,
    pin_ttt_gradient_step,
    pin_delta_triangular_system,
    pin_brute_force_transitions,
    pin_equal_channels_is_scalar,
    pin_chunk_form_any_C,
    pin_decode_and_resume,
    pin_deltaproduct_one_substep_is_gdn,
    pin_deltaproduct_dense_product,
    pin_deltaproduct_virtual_sequence,
    pin_normalized_quadratic_form,
    pin_normalized_invariants,
    pin_bwd_finite_differences,
    pin_bwd_autograd_one_chunk,
    pin_deltaproduct_bwd_finite_differences,
    pin_deltaproduct_bwd_virtual_sequence,
]
