"""Seeded synthetic inputs for causal linear attention.

This module is shared by the HIP path's tests and benchmark and by the fp64
oracle: it draws random numbers and shapes them into the input distributions
of the workloads, and holds none of the method's arithmetic (no state update,
no read-out, no chunking).

Every case is drawn per (batch, head) from ``numpy.random.default_rng`` seeded
with ``[seed, case_id, b, h]``, so any subset of heads can be regenerated on
the host without drawing the rest.  Draw order inside a head is fixed:
q, k, v, beta-logits, gate-logits, initial state.  Draws are fp32; values are
shaped in fp32 and then rounded (round-to-nearest-even) to the token dtype, so
the arrays returned here hold exactly the values a kernel receives.

Distributions (per element unless stated):
  * q, k "l2":   N(0,1) then L2-normalised per token
  * q, k "elu1": elu(N(0,1)) + 1 (the positive feature map)
  * v:           N(0,1)
  * beta:        sigmoid(N(0,1)) per (b,h,t)
  * g (log of the forget gate alpha): -softplus(N(0,1)) * gate_scale, per
    (b,h,t) for a scalar gate or per (b,h,t,key channel) for a channel gate
  * initial state: N(0, s0_std^2) (only when s0_std > 0)
"""
from __future__ import annotations

import dataclasses
from typing import Iterable, Optional, Sequence

import numpy as np

SEED = 27


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "fp32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(f"unknown token dtype {dtype!r}")


def _l2(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / np.maximum(n, np.float32(1e-6))).astype(np.float32)


def _elu1(x: np.ndarray) -> np.ndarray:
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0))).astype(np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x))).astype(np.float32)


def _softplus(x: np.ndarray) -> np.ndarray:
    return (np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))).astype(np.float32)


@dataclasses.dataclass(frozen=True)
class Case:
    """One chunk-forward workload (shapes, update rule, gate kind, dtype, law)."""
    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    rule: str = "delta"          # "add" | "delta"
    gate: str = "scalar"         # "none" | "scalar" | "channel"
    dtype: str = "bf16"          # token dtype: "bf16" | "fp32"
    qk: str = "l2"               # "l2" | "elu1"
    chunk: int = 64
    gate_scale: float = 1.0      # g = -softplus(N(0,1)) * gate_scale
    beta_mode: str = "sigmoid"   # "sigmoid" | "zero" | "one"
    s0_std: float = 0.0          # 0 => no initial state
    case_id: int = 0

    def with_(self, **kw) -> "Case":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class DecodeCase:
    """A decode workload: N sequences x H heads, one token each per step."""
    name: str
    N: int
    H: int
    dk: int
    dv: int
    steps: int
    rule: str = "delta"
    gate: str = "scalar"
    dtype: str = "bf16"
    qk: str = "l2"
    state_std: float = 0.02
    gate_scale: float = 1.0
    beta_mode: str = "sigmoid"
    case_id: int = 5


# The five workloads (sizes, laws and chunk size as stated with the metric).
CFG1 = Case("gdn_fwd_B1_H2_T256_d64_fp32", 1, 2, 256, 64, 64, "delta", "scalar", "fp32",
            case_id=1)
CFG2 = Case("add_fwd_B4_H16_T4096_d128_bf16", 4, 16, 4096, 128, 128, "add", "none", "bf16",
            qk="elu1", case_id=2)
CFG3 = Case("gdn_fwd_B8_H16_T8192_d128_bf16", 8, 16, 8192, 128, 128, "delta", "scalar", "bf16",
            case_id=3)
CFG3B = Case("decay_add_fwd_B8_H16_T8192_d128_bf16", 8, 16, 8192, 128, 128, "add", "scalar",
             "bf16", case_id=33)
CFG4 = Case("kda_fwd_B1_H32_T262144_d128_bf16", 1, 32, 262144, 128, 128, "delta", "channel",
            "bf16", case_id=4)
CFG5 = DecodeCase("gdn_decode_N256_H32_d128_bf16_1000steps", 256, 32, 128, 128, 1000)

CONFIGS = {1: CFG1, 2: CFG2, 3: CFG3, "3b": CFG3B, 4: CFG4, 5: CFG5}


def _beta(rng, shape, mode):
    x = rng.standard_normal(shape, dtype=np.float32)
    if mode == "sigmoid":
        return _sigmoid(x)
    if mode == "zero":
        return np.zeros(shape, np.float32)
    if mode == "one":
        return np.ones(shape, np.float32)
    raise ValueError(mode)


def _qk(rng, shape, law):
    x = rng.standard_normal(shape, dtype=np.float32)
    if law == "l2":
        return _l2(x)
    if law == "elu1":
        return _elu1(x)
    if law == "gauss":
        return x
    raise ValueError(law)


def head_inputs(case: Case, b: int, h: int, seed: int = SEED) -> dict:
    """Inputs of one (b,h) head: q,k [T,dk], v [T,dv], g [T]|[T,dk]|None,
    beta [T]|None, s0 [dk,dv]|None, as fp32 arrays holding token-dtype values."""
    rng = np.random.default_rng([seed, case.case_id, b, h])
    T, dk, dv = case.T, case.dk, case.dv
    q = to_dtype(_qk(rng, (T, dk), case.qk), case.dtype)
    k = to_dtype(_qk(rng, (T, dk), case.qk), case.dtype)
    v = to_dtype(rng.standard_normal((T, dv), dtype=np.float32), case.dtype)
    beta = to_dtype(_beta(rng, (T,), case.beta_mode), case.dtype)
    gshape = (T, dk) if case.gate == "channel" else (T,)
    g = to_dtype(-_softplus(rng.standard_normal(gshape, dtype=np.float32))
                 * np.float32(case.gate_scale), case.dtype)
    s0 = None
    if case.s0_std > 0:
        s0 = (rng.standard_normal((dk, dv), dtype=np.float32)
              * np.float32(case.s0_std)).astype(np.float32)
    return {
        "q": q, "k": k, "v": v,
        "g": None if case.gate == "none" else g,
        "beta": beta if case.rule == "delta" else None,
        "s0": s0,
    }


def chunk_inputs(case: Case, heads: Optional[Sequence[tuple]] = None, seed: int = SEED) -> dict:
    """All heads ([B,H,...] arrays) or the listed (b,h) heads ([n,...] arrays)."""
    if heads is None:
        idx = [(b, h) for b in range(case.B) for h in range(case.H)]
    else:
        idx = list(heads)
    parts = [head_inputs(case, b, h, seed) for (b, h) in idx]
    out = {}
    for key in ("q", "k", "v", "g", "beta", "s0"):
        if parts[0][key] is None:
            out[key] = None
            continue
        arr = np.stack([p[key] for p in parts])
        if heads is None:
            arr = arr.reshape((case.B, case.H) + arr.shape[1:])
        out[key] = arr
    return out


def raw_inputs(case: Case, seed: int = SEED) -> dict:
    """Raw projections for the fused input preparation, all heads: q, k
    N(0,1) * 2 (not normalised), v N(0,1), beta logits N(0,1), gate logits
    N(0,1) * gate_scale ([B,H,T] scalar gate, [B,H,T,dk] per-channel gate),
    initial state as in ``head_inputs``; same draw order per (b,h) head."""
    parts = []
    for b in range(case.B):
        for h in range(case.H):
            rng = np.random.default_rng([seed, case.case_id, b, h])
            T, dk, dv = case.T, case.dk, case.dv
            q = to_dtype(rng.standard_normal((T, dk), dtype=np.float32) * np.float32(2), case.dtype)
            k = to_dtype(rng.standard_normal((T, dk), dtype=np.float32) * np.float32(2), case.dtype)
            v = to_dtype(rng.standard_normal((T, dv), dtype=np.float32), case.dtype)
            beta = to_dtype(rng.standard_normal((T,), dtype=np.float32), case.dtype)
            gshape = (T, dk) if case.gate == "channel" else (T,)
            g = to_dtype(rng.standard_normal(gshape, dtype=np.float32) * np.float32(case.gate_scale),
                         case.dtype)
            s0 = None
            if case.s0_std > 0:
                s0 = (rng.standard_normal((dk, dv), dtype=np.float32)
                      * np.float32(case.s0_std)).astype(np.float32)
            parts.append({"q": q, "k": k, "v": v, "beta": beta if case.rule == "delta" else None,
                          "g": None if case.gate == "none" else g, "s0": s0})
    out = {}
    for key in ("q", "k", "v", "g", "beta", "s0"):
        out[key] = None if parts[0][key] is None else \
            np.stack([p[key] for p in parts]).reshape((case.B, case.H) + parts[0][key].shape)
    return out


def grad_head_inputs(case: Case, b: int, h: int, seed: int = SEED) -> dict:
    """Upstream gradients of one head for the backward pass: do [T,dv] N(0,1)
    in the token dtype, dsT [dk,dv] N(0, 0.5^2) fp32 (its own stream,
    [seed, case_id, b, h, 1])."""
    rng = np.random.default_rng([seed, case.case_id, b, h, 1])
    do = to_dtype(rng.standard_normal((case.T, case.dv), dtype=np.float32), case.dtype)
    dsT = (rng.standard_normal((case.dk, case.dv), dtype=np.float32) * np.float32(0.5)).astype(np.float32)
    return {"do": do, "dsT": dsT}


def grad_inputs(case: Case, heads: Optional[Sequence[tuple]] = None, seed: int = SEED) -> dict:
    """All heads ([B,H,...]) or the listed (b,h) heads ([n,...]) of grad_head_inputs."""
    idx = [(b, h) for b in range(case.B) for h in range(case.H)] if heads is None else list(heads)
    parts = [grad_head_inputs(case, b, h, seed) for (b, h) in idx]
    out = {}
    for key in ("do", "dsT"):
        arr = np.stack([p[key] for p in parts])
        if heads is None:
            arr = arr.reshape((case.B, case.H) + arr.shape[1:])
        out[key] = arr
    return out


def iter_heads(case: Case, seed: int = SEED) -> Iterable[tuple]:
    """Yield ((b,h), inputs) one head at a time (for workloads too big to hold twice)."""
    for b in range(case.B):
        for h in range(case.H):
            yield (b, h), head_inputs(case, b, h, seed)


@dataclasses.dataclass(frozen=True)
class DeltaProductCase:
    """A Gated DeltaProduct workload: nh (key, value, beta) substeps per token."""
    name: str
    B: int
    H: int
    T: int
    nh: int
    dk: int
    dv: int
    gate: str = "scalar"         # "none" | "scalar"
    dtype: str = "bf16"
    gate_scale: float = 1.0
    s0_std: float = 0.0
    case_id: int = 6

    def with_(self, **kw) -> "DeltaProductCase":
        return dataclasses.replace(self, **kw)


# Gated DeltaProduct with two substeps at the GDN workload's head size
# (virtual length 2 T = 8192, the GDN workload's sequence length)
GDP2 = DeltaProductCase("gdp2_fwd_B8_H16_T4096_d128_bf16", 8, 16, 4096, 2, 128, 128, case_id=6)


def deltaproduct_head_inputs(case: DeltaProductCase, b: int, h: int, seed: int = SEED) -> dict:
    """Inputs of one head: q [T,dk]; k [T,nh,dk] and q L2-normalised per
    (token, substep); v [T,nh,dv] N(0,1); beta [T,nh] sigmoid(N(0,1));
    g [T] -softplus(N(0,1)) * gate_scale or None; s0 [dk,dv] or None.  Draw
    order q, k, v, beta-logits, gate-logits, initial state."""
    rng = np.random.default_rng([seed, case.case_id, b, h])
    T, nh, dk, dv = case.T, case.nh, case.dk, case.dv
    q = to_dtype(_qk(rng, (T, dk), "l2"), case.dtype)
    k = to_dtype(_qk(rng, (T, nh, dk), "l2"), case.dtype)
    v = to_dtype(rng.standard_normal((T, nh, dv), dtype=np.float32), case.dtype)
    beta = to_dtype(_beta(rng, (T, nh), "sigmoid"), case.dtype)
    g = to_dtype(-_softplus(rng.standard_normal((T,), dtype=np.float32))
                 * np.float32(case.gate_scale), case.dtype)
    s0 = None
    if case.s0_std > 0:
        s0 = (rng.standard_normal((dk, dv), dtype=np.float32)
              * np.float32(case.s0_std)).astype(np.float32)
    return {"q": q, "k": k, "v": v, "beta": beta,
            "g": None if case.gate == "none" else g, "s0": s0}


def deltaproduct_inputs(case: DeltaProductCase, heads: Optional[Sequence[tuple]] = None,
                        seed: int = SEED) -> dict:
    """All heads ([B,H,...] arrays) or the listed (b,h) heads ([n,...] arrays)."""
    idx = [(b, h) for b in range(case.B) for h in range(case.H)] if heads is None else list(heads)
    parts = [deltaproduct_head_inputs(case, b, h, seed) for (b, h) in idx]
    out = {}
    for key in ("q", "k", "v", "g", "beta", "s0"):
        if parts[0][key] is None:
            out[key] = None
            continue
        arr = np.stack([p[key] for p in parts])
        if heads is None:
            arr = arr.reshape((case.B, case.H) + arr.shape[1:])
        out[key] = arr
    return out


def deltaproduct_inputs_torch(case: DeltaProductCase, device, seed: int = SEED) -> dict:
    """The same laws drawn with torch's device generator (large workloads)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed * 1000 + case.case_id)
    dt = torch.bfloat16 if case.dtype == "bf16" else torch.float32
    shp = (case.B, case.H, case.T)
    rn = lambda *s: torch.randn(*s, generator=gen, device=device, dtype=torch.float32)
    out = {"q": _torch_laws(rn(*shp, case.dk), "l2").to(dt),
           "k": _torch_laws(rn(*shp, case.nh, case.dk), "l2").to(dt),
           "v": rn(*shp, case.nh, case.dv).to(dt),
           "beta": torch.sigmoid(rn(*shp, case.nh)).to(dt)}
    g = -torch.nn.functional.softplus(rn(*shp)) * case.gate_scale
    out["g"] = None if case.gate == "none" else g.to(dt)
    out["s0"] = None
    return out


def decode_state(case: DecodeCase, seed: int = SEED) -> np.ndarray:
    rng = np.random.default_rng([seed, case.case_id, 1 << 20])
    s = rng.standard_normal((case.N, case.H, case.dk, case.dv), dtype=np.float32)
    return (s * np.float32(case.state_std)).astype(np.float32)


def decode_tokens(case: DecodeCase, step: int, seed: int = SEED) -> dict:
    """Tokens of one decode step: q,k [N,H,dk], v [N,H,dv], g [N,H]|[N,H,dk], beta [N,H]."""
    rng = np.random.default_rng([seed, case.case_id, step])
    N, H, dk, dv = case.N, case.H, case.dk, case.dv
    q = to_dtype(_qk(rng, (N, H, dk), case.qk), case.dtype)
    k = to_dtype(_qk(rng, (N, H, dk), case.qk), case.dtype)
    v = to_dtype(rng.standard_normal((N, H, dv), dtype=np.float32), case.dtype)
    beta = to_dtype(_beta(rng, (N, H), case.beta_mode), case.dtype)
    gshape = (N, H, dk) if case.gate == "channel" else (N, H)
    g = to_dtype(-_softplus(rng.standard_normal(gshape, dtype=np.float32))
                 * np.float32(case.gate_scale), case.dtype)
    return {
        "q": q, "k": k, "v": v,
        "g": None if case.gate == "none" else g,
        "beta": beta if case.rule == "delta" else None,
    }


# ---------------------------------------------------------------------------
# Device-side generation for the benchmark (multi-GB inputs).  Same laws as
# above, drawn with torch's generator on the device; values differ from the
# numpy streams, which are the ones parity tests use.
# ---------------------------------------------------------------------------
def _torch_laws(t, law):
    import torch
    if law == "l2":
        return t / t.norm(dim=-1, keepdim=True).clamp_min(1e-6)
    if law == "elu1":
        return torch.nn.functional.elu(t) + 1.0
    return t


def chunk_inputs_torch(case: Case, device, seed: int = SEED) -> dict:
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed * 1000 + (case.case_id if isinstance(case.case_id, int) else 0))
    dt = torch.bfloat16 if case.dtype == "bf16" else torch.float32
    shp = (case.B, case.H, case.T)
    rn = lambda *s: torch.randn(*s, generator=gen, device=device, dtype=torch.float32)
    out = {"q": _torch_laws(rn(*shp, case.dk), case.qk).to(dt),
           "k": _torch_laws(rn(*shp, case.dk), case.qk).to(dt),
           "v": rn(*shp, case.dv).to(dt)}
    b = torch.sigmoid(rn(*shp))
    if case.beta_mode == "zero":
        b = torch.zeros_like(b)
    elif case.beta_mode == "one":
        b = torch.ones_like(b)
    out["beta"] = b.to(dt) if case.rule == "delta" else None
    gshape = shp + ((case.dk,) if case.gate == "channel" else ())
    g = -torch.nn.functional.softplus(rn(*gshape)) * case.gate_scale
    out["g"] = None if case.gate == "none" else g.to(dt)
    out["s0"] = None
    return out


def grad_inputs_torch(case: Case, device, seed: int = SEED) -> dict:
    """Upstream gradients drawn on the device: do [B,H,T,dv] N(0,1), dsT None."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed * 1000 + 500 + (case.case_id if isinstance(case.case_id, int) else 0))
    dt = torch.bfloat16 if case.dtype == "bf16" else torch.float32
    do = torch.randn(case.B, case.H, case.T, case.dv, generator=gen, device=device, dtype=torch.float32)
    return {"do": do.to(dt), "dsT": None}


def decode_tokens_torch(case: DecodeCase, steps: int, device, seed: int = SEED) -> dict:
    """Tokens for `steps` decode steps at once: q,k [steps,N,H,dk], v [steps,N,H,dv],
    g [steps,N,H] | [steps,N,H,dk], beta [steps,N,H]."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed * 1000 + case.case_id)
    dt = torch.bfloat16 if case.dtype == "bf16" else torch.float32
    shp = (steps, case.N, case.H)
    rn = lambda *s: torch.randn(*s, generator=gen, device=device, dtype=torch.float32)
    out = {"q": _torch_laws(rn(*shp, case.dk), case.qk).to(dt),
           "k": _torch_laws(rn(*shp, case.dk), case.qk).to(dt),
           "v": rn(*shp, case.dv).to(dt),
           "beta": torch.sigmoid(rn(*shp)).to(dt) if case.rule == "delta" else None}
    gshape = shp + ((case.dk,) if case.gate == "channel" else ())
    g = -torch.nn.functional.softplus(rn(*gshape)) * case.gate_scale
    out["g"] = None if case.gate == "none" else g.to(dt)
    return out


def decode_state_torch(case: DecodeCase, device, seed: int = SEED):
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed * 1000 + case.case_id + 7)
    return torch.randn(case.N, case.H, case.dk, case.dv, generator=gen, device=device,
                       dtype=torch.float32) * case.state_std
