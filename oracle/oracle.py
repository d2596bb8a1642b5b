"""Python face of the fp64 CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY.  The oracle is the checker for the HIP library: only
the tests, the smoke check and the benchmark's CPU-baseline leg may import it.
It imports nothing from the HIP package and the HIP package never imports it.

``recurrence`` runs the token-by-token recurrence of causal linear attention
(add rule, decay with a scalar or per-key-channel gate, delta rule) described
in ``oracle.c``; ``decode_step`` runs one token per (sequence, head) in place;
``deltaproduct`` runs the Gated DeltaProduct recurrence (n_h substeps per token);
``recurrence_bwd`` returns the recurrence's gradients (reverse mode, fp64).
Every input is widened to float64 exactly (bf16 and fp32 values are exact in
fp64), so the oracle sees the very values a GPU kernel received.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

RULES = {"add": 0, "delta": 1}
GATES = {"none": 0, "scalar": 1, "channel": 2}

_lock = threading.Lock()
_default = None


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # a CPU torch tensor (bf16 included): widen exactly
        import torch
        x = x.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile ``oracle.c`` (or another source, e.g. in a test) with gcc:
    fp64, no fast-math, no FMA contraction, OpenMP over heads."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
               "-ffp-contract=off", "-fno-fast-math", "-o", tmp, src, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


class OracleLib:
    """ctypes handle on one compiled oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        d = ctypes.POINTER(ctypes.c_double)
        i64, i32 = ctypes.c_int64, ctypes.c_int
        lib.oracle_recurrence.argtypes = [i64, i64, i64, i32, i32, i32, i32,
                                          d, d, d, d, d, d, d, d, i32]
        lib.oracle_recurrence.restype = i32
        lib.oracle_decode_step.argtypes = [i64, i64, i32, i32, i32, i32,
                                           d, d, d, d, d, d, d, i32]
        lib.oracle_decode_step.restype = i32
        lib.oracle_deltaproduct.argtypes = [i64, i64, i64, i32, i32, i32, i32,
                                            d, d, d, d, d, d, d, d, i32]
        lib.oracle_deltaproduct.restype = i32
        lib.oracle_normalized.argtypes = [i64, i64, i64, i32, i32, i32, d, d, d, d, d, d, d, d, d,
                                          i32]
        lib.oracle_normalized.restype = i32
        lib.oracle_recurrence_bwd.argtypes = [i64, i64, i64, i32, i32, i32, i32,
                                              d, d, d, d, d, d, d, d, d, d, d, d, d, d, i32]
        lib.oracle_recurrence_bwd.restype = i32
        lib.oracle_deltaproduct_bwd.argtypes = [i64, i64, i64, i32, i32, i32, i32,
                                                d, d, d, d, d, d, d, d, d, d, d, d, d, d, i32]
        lib.oracle_deltaproduct_bwd.restype = i32
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = i32
        self.lib = lib
        self.path = path

    def max_threads(self) -> int:
        return int(self.lib.oracle_max_threads())

    def recurrence(self, q, k, v, g=None, beta=None, s0=None, *, rule="delta", gate="scalar",
                   nthreads: int = 0):
        """fp64 token recurrence.  Shapes: q,k [B,H,T,dk]; v [B,H,T,dv];
        g [B,H,T] or [B,H,T,dk]; beta [B,H,T]; s0 [B,H,dk,dv].
        Returns (o [B,H,T,dv], S_T [B,H,dk,dv]) as float64 arrays."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        g, beta, s0 = _f64(g), _f64(beta), _f64(s0)
        B, H, T, dk = q.shape
        dv = v.shape[-1]
        if k.shape != (B, H, T, dk) or v.shape != (B, H, T, dv):
            raise ValueError("q/k/v shapes disagree")
        if gate == "scalar" and (g is None or g.shape != (B, H, T)):
            raise ValueError("scalar gate needs g of shape [B,H,T]")
        if gate == "channel" and (g is None or g.shape != (B, H, T, dk)):
            raise ValueError("channel gate needs g of shape [B,H,T,dk]")
        if rule == "delta" and (beta is None or beta.shape != (B, H, T)):
            raise ValueError("delta rule needs beta of shape [B,H,T]")
        if s0 is not None and s0.shape != (B, H, dk, dv):
            raise ValueError("s0 must be [B,H,dk,dv]")
        if gate == "none":
            g = None
        if rule == "add":
            beta = None
        o = np.empty((B, H, T, dv), dtype=np.float64)
        s = np.empty((B, H, dk, dv), dtype=np.float64)
        rc = self.lib.oracle_recurrence(B, H, T, dk, dv, RULES[rule], GATES[gate],
                                        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                        _ptr(s0), _ptr(o), _ptr(s), int(nthreads))
        if rc != 0:
            raise RuntimeError(f"oracle_recurrence failed with code {rc}")
        return o, s

    def decode_step(self, q, k, v, g, beta, state, *, rule="delta", gate="scalar",
                    nthreads: int = 0):
        """One recurrent step for N sequences x H heads.  Shapes: q,k [N,H,dk];
        v [N,H,dv]; g [N,H] or [N,H,dk]; beta [N,H]; state [N,H,dk,dv].
        Returns (o [N,H,dv], new_state) as float64; the input is not modified."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        g, beta = _f64(g), _f64(beta)
        st = np.array(_f64(state), dtype=np.float64, copy=True)
        N, H, dk = q.shape
        dv = v.shape[-1]
        if st.shape != (N, H, dk, dv):
            raise ValueError("state must be [N,H,dk,dv]")
        if gate == "none":
            g = None
        if rule == "add":
            beta = None
        o = np.empty((N, H, dv), dtype=np.float64)
        rc = self.lib.oracle_decode_step(N, H, dk, dv, RULES[rule], GATES[gate],
                                         _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                         _ptr(st), _ptr(o), int(nthreads))
        if rc != 0:
            raise RuntimeError(f"oracle_decode_step failed with code {rc}")
        return o, st


def _deltaproduct(self, q, k, v, g=None, beta=None, s0=None, *, gate="scalar", nthreads: int = 0):
    """fp64 Gated DeltaProduct recurrence (see ``oracle.c``).  Shapes: q [B,H,T,dk];
    k [B,H,T,nh,dk]; v [B,H,T,nh,dv]; beta [B,H,T,nh]; g [B,H,T] (scalar gate)
    or None; s0 [B,H,dk,dv].  Returns (o [B,H,T,dv], S_T [B,H,dk,dv])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    g, beta, s0 = _f64(g), _f64(beta), _f64(s0)
    B, H, T, dk = q.shape
    nh, dv = k.shape[3], v.shape[-1]
    if k.shape != (B, H, T, nh, dk) or v.shape != (B, H, T, nh, dv):
        raise ValueError("k/v must be [B,H,T,nh,d]")
    if beta is None or beta.shape != (B, H, T, nh):
        raise ValueError("beta must be [B,H,T,nh]")
    if gate == "scalar" and (g is None or g.shape != (B, H, T)):
        raise ValueError("scalar gate needs g of shape [B,H,T]")
    if gate not in ("none", "scalar"):
        raise ValueError("Gated DeltaProduct takes no gate or a scalar gate")
    if s0 is not None and s0.shape != (B, H, dk, dv):
        raise ValueError("s0 must be [B,H,dk,dv]")
    if gate == "none":
        g = None
    o = np.empty((B, H, T, dv), dtype=np.float64)
    s = np.empty((B, H, dk, dv), dtype=np.float64)
    rc = self.lib.oracle_deltaproduct(B, H, T, nh, dk, dv, GATES[gate], _ptr(q), _ptr(k), _ptr(v),
                                      _ptr(g), _ptr(beta), _ptr(s0), _ptr(o), _ptr(s),
                                      int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_deltaproduct failed with code {rc}")
    return o, s


OracleLib.deltaproduct = _deltaproduct


def _deltaproduct_bwd(self, q, k, v, g=None, beta=None, s0=None, do=None, dsT=None, *, gate="scalar",
                      nthreads: int = 0):
    """fp64 gradients of the Gated DeltaProduct recurrence for the loss
    sum(do * o) + sum(dsT * S_T).  Shapes as ``deltaproduct``; do [B,H,T,dv].
    Returns dq [B,H,T,dk], dk [B,H,T,nh,dk], dv [B,H,T,nh,dv], dg [B,H,T] (None
    without a gate), dbeta [B,H,T,nh], ds0 [B,H,dk,dv]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    g, beta, s0, do, dsT = _f64(g), _f64(beta), _f64(s0), _f64(do), _f64(dsT)
    B, H, T, dk = q.shape
    nh, dv = k.shape[3], v.shape[-1]
    if k.shape != (B, H, T, nh, dk) or v.shape != (B, H, T, nh, dv):
        raise ValueError("k/v must be [B,H,T,nh,d]")
    if beta is None or beta.shape != (B, H, T, nh):
        raise ValueError("beta must be [B,H,T,nh]")
    if do is None or do.shape != (B, H, T, dv):
        raise ValueError("do must be [B,H,T,dv]")
    if gate == "scalar" and (g is None or g.shape != (B, H, T)):
        raise ValueError("scalar gate needs g of shape [B,H,T]")
    if gate not in ("none", "scalar"):
        raise ValueError("Gated DeltaProduct takes no gate or a scalar gate")
    if gate == "none":
        g = None
    out = {"dq": np.empty((B, H, T, dk)), "dk": np.empty((B, H, T, nh, dk)),
           "dv": np.empty((B, H, T, nh, dv)), "dbeta": np.empty((B, H, T, nh)),
           "dg": None if g is None else np.empty((B, H, T)), "ds0": np.empty((B, H, dk, dv))}
    rc = self.lib.oracle_deltaproduct_bwd(B, H, T, nh, dk, dv, GATES[gate], _ptr(q), _ptr(k), _ptr(v),
                                          _ptr(g), _ptr(beta), _ptr(s0), _ptr(do), _ptr(dsT),
                                          _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                                          _ptr(out["dg"]), _ptr(out["dbeta"]), _ptr(out["ds0"]),
                                          int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_deltaproduct_bwd failed with code {rc}")
    return out


OracleLib.deltaproduct_bwd = _deltaproduct_bwd


def _recurrence_bwd(self, q, k, v, g=None, beta=None, s0=None, do=None, dsT=None, *, rule="delta",
                    gate="scalar", nthreads: int = 0):
    """fp64 gradients of the token recurrence (see ``oracle.c``) for the loss
    sum(do * o) + sum(dsT * S_T).  Shapes as ``recurrence``; do [B,H,T,dv];
    dsT [B,H,dk,dv] or None.  Returns a dict with dq, dk, dv, dg (None without a
    gate), dbeta (None for the add rule) and ds0, all float64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    g, beta, s0, do, dsT = _f64(g), _f64(beta), _f64(s0), _f64(do), _f64(dsT)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    if k.shape != (B, H, T, dk) or v.shape != (B, H, T, dv):
        raise ValueError("q/k/v shapes disagree")
    if do is None or do.shape != (B, H, T, dv):
        raise ValueError("do must be [B,H,T,dv]")
    if gate == "scalar" and (g is None or g.shape != (B, H, T)):
        raise ValueError("scalar gate needs g of shape [B,H,T]")
    if gate == "channel" and (g is None or g.shape != (B, H, T, dk)):
        raise ValueError("channel gate needs g of shape [B,H,T,dk]")
    if rule == "delta" and (beta is None or beta.shape != (B, H, T)):
        raise ValueError("delta rule needs beta of shape [B,H,T]")
    for name, a in (("s0", s0), ("dsT", dsT)):
        if a is not None and a.shape != (B, H, dk, dv):
            raise ValueError(f"{name} must be [B,H,dk,dv]")
    if gate == "none":
        g = None
    if rule == "add":
        beta = None
    out = {"dq": np.empty((B, H, T, dk)), "dk": np.empty((B, H, T, dk)),
           "dv": np.empty((B, H, T, dv)), "ds0": np.empty((B, H, dk, dv)),
           "dg": None if g is None else np.empty(g.shape),
           "dbeta": None if beta is None else np.empty((B, H, T))}
    rc = self.lib.oracle_recurrence_bwd(B, H, T, dk, dv, RULES[rule], GATES[gate], _ptr(q), _ptr(k),
                                        _ptr(v), _ptr(g), _ptr(beta), _ptr(s0), _ptr(do), _ptr(dsT),
                                        _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                                        _ptr(out["dg"]), _ptr(out["dbeta"]), _ptr(out["ds0"]),
                                        int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_recurrence_bwd failed with code {rc}")
    return out


OracleLib.recurrence_bwd = _recurrence_bwd


def _normalized(self, q, k, v, g=None, s0=None, z0=None, *, gate="none", nthreads: int = 0):
    """fp64 normalised linear attention (see ``oracle.c``).  Shapes: q, k
    [B,H,T,dk]; v [B,H,T,dv]; g [B,H,T] | [B,H,T,dk] | None; s0 [B,H,dk,dv];
    z0 [B,H,dk].
    Returns (o [B,H,T,dv], S_T [B,H,dk,dv], z_T [B,H,dk])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    g, s0, z0 = _f64(g), _f64(s0), _f64(z0)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    if k.shape != (B, H, T, dk) or v.shape != (B, H, T, dv):
        raise ValueError("q/k/v shapes disagree")
    if gate == "scalar" and (g is None or g.shape != (B, H, T)):
        raise ValueError("scalar gate needs g of shape [B,H,T]")
    if gate == "channel" and (g is None or g.shape != (B, H, T, dk)):
        raise ValueError("channel gate needs g of shape [B,H,T,dk]")
    if gate == "none":
        g = None
    o = np.empty((B, H, T, dv), dtype=np.float64)
    s = np.empty((B, H, dk, dv), dtype=np.float64)
    z = np.empty((B, H, dk), dtype=np.float64)
    rc = self.lib.oracle_normalized(B, H, T, dk, dv, GATES[gate], _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                    _ptr(s0), _ptr(z0), _ptr(o), _ptr(s), _ptr(z), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_normalized failed with code {rc}")
    return o, s, z


OracleLib.normalized = _normalized


# Input preparation from raw projections, fp64 ([ASF] "DeltaNet": keys and
# queries L2-normalised per token and the write strength beta a sigmoid;
# "Linear Magic": the positive feature map elu + 1; [LAV] "Mamba-2" and "Gated
# DeltaNet (GDN)": the forget gate alpha = exp(-softplus(x)) in (0, 1), so the
# log-gate is -softplus(x)).  L2 uses x / max(|x|, 1e-6).
QK_MAPS = ("identity", "l2", "elu1")
GATE_MAPS = ("log", "neg_softplus")
BETA_MAPS = ("identity", "sigmoid")
L2_EPS = 1e-6


def prepare_qk(x, qk_map):
    x = _f64(x)
    if qk_map == "identity":
        return x
    if qk_map == "l2":
        n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
        return x / np.maximum(n, L2_EPS)
    if qk_map == "elu1":
        return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))
    raise ValueError(f"unknown q/k map {qk_map!r}")


def prepare_gate(g, gate_map):
    g = _f64(g)
    if g is None or gate_map == "log":
        return g
    if gate_map == "neg_softplus":
        return -(np.maximum(g, 0.0) + np.log1p(np.exp(-np.abs(g))))
    raise ValueError(f"unknown gate map {gate_map!r}")


def prepare_beta(beta, beta_map):
    beta = _f64(beta)
    if beta is None or beta_map == "identity":
        return beta
    if beta_map == "sigmoid":
        return 1.0 / (1.0 + np.exp(-beta))
    raise ValueError(f"unknown beta map {beta_map!r}")


def default() -> OracleLib:
    """The oracle built from ``oracle.c`` in this directory."""
    global _default
    with _lock:
        if _default is None:
            if not os.path.exists(_LIB):
                build(force=False)
            _default = OracleLib(_LIB)
    return _default


def max_threads() -> int:
    return default().max_threads()


def recurrence(*args, **kw):
    """See :meth:`OracleLib.recurrence`."""
    return default().recurrence(*args, **kw)


def decode_step(*args, **kw):
    """See :meth:`OracleLib.decode_step`."""
    return default().decode_step(*args, **kw)


def deltaproduct(*args, **kw):
    """See :meth:`OracleLib.deltaproduct`."""
    return default().deltaproduct(*args, **kw)


def deltaproduct_bwd(*args, **kw):
    """See :meth:`OracleLib.deltaproduct_bwd`."""
    return default().deltaproduct_bwd(*args, **kw)


def recurrence_bwd(*args, **kw):
    """See :meth:`OracleLib.recurrence_bwd`."""
    return default().recurrence_bwd(*args, **kw)


def normalized(*args, **kw):
    """See :meth:`OracleLib.normalized`."""
    return default().normalized(*args, **kw)
